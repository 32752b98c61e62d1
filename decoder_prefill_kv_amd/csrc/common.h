// Shared device/host definitions for the dpk kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <type_traits>

#define DPK_DEV __device__ __forceinline__

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace dpk {

// Kernel-class timing.  While a profiling scope is open on this thread every
// launch takes its timestamps from the dispatch itself (hipExtLaunchKernel's
// start/stop events), so a class's duration excludes the gaps between
// kernels.  The first launch of a scope records start and stop, later ones
// only move stop.
struct LaunchTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchTiming g_timing;

template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, unsigned shmem, hipStream_t st, Args... args) {
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, g_timing.start, g_timing.stop, 0u, args...);
  g_timing.start = nullptr;
}

// One row of a forward call: the token it embeds, the position it occupies
// and the KV-cache slot (sequence) it belongs to.  A row attends to every
// cached key of its sequence at positions <= pos.
struct RowParam {
  int32_t token;
  int32_t pos;
  int32_t seq;
  int32_t pad;
};

// Weight formats of the linear layers.
enum WFmt : int { W_F32 = 0, W_BF16 = 1, W_Q4 = 2, W_I8 = 3, W_Q8 = 4, W_Q40 = 5 };

DPK_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
DPK_DEV float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
DPK_DEV float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// round-to-nearest-even fp32 -> bf16 bits (finite inputs)
DPK_DEV uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi); |x - hi - lo| <= 2^-17 |x|
DPK_DEV void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_bits(x);
  float r = x - __uint_as_float(hi << 16);
  lo = f32_to_bf16_bits(r);
}

DPK_DEV _Float16 f32_to_f16(float f) { return (_Float16)f; }

// ---------------------------------------------------------------- wave reductions
DPK_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DPK_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// (value, index) max with lowest index on ties
DPK_DEV void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, 64);
    int oi = __shfl_xor(i, o, 64);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

// Block-wide sum over blockDim.x threads (multiple of 64); red has >= 16 floats.
// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// accesses, not for its outstanding global loads (a __syncthreads() fence
// would also drain every load in flight, e.g. a weight prefetch).  Global
// data written before it is not made visible to the other waves.
DPK_DEV void lds_barrier() {
  asm volatile("" ::: "memory");       // no memory access moves across it in the compiler
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// block_sum with lds_barrier(): the sum of v over the workgroup
DPK_DEV float block_sum_lds(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = blockDim.x >> 6;
  lds_barrier();
  if (l == 0) red[w] = v;
  lds_barrier();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

DPK_DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = blockDim.x >> 6;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// threadIdx.x as a value the compiler cannot see through.  In a long
// persistent kernel, per-lane address terms derived from the thread index
// would otherwise be computed once, kept live across every phase and spilled
// to scratch; a phase that takes its index from here computes them itself.
DPK_DEV int opaque_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Device-coherent access (agent-scope relaxed atomics: sc1 loads/stores that
// bypass the non-coherent per-XCD L2 state) for data handed from one
// workgroup to another inside a launch.
DPK_DEV void coh_store(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DPK_DEV void coh_store(int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DPK_DEV float coh_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DPK_DEV int coh_load(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 8-byte device-coherent accesses (two floats; same sc1 policy)
DPK_DEV void coh_store2(float* p, float x, float y) {
  const uint64_t v = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DPK_DEV void coh_load2(const float* p, float& x, float& y) {
  const uint64_t v = __hip_atomic_load((uint64_t*)const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  x = __uint_as_float((uint32_t)v);
  y = __uint_as_float((uint32_t)(v >> 32));
}

// Device-coherent loads / stores without atomic semantics: buffer accesses
// with the same sc1 cache policy as the agent-scope atomics above, through a
// descriptor whose base must be uniform over the wave.  Being plain loads,
// the compiler batches them and waits only where a value is used (an atomic
// load waits for itself before the next memory operation).
constexpr int CPOL_SC1 = 16;
typedef __amdgpu_buffer_rsrc_t coh_buf;
DPK_DEV coh_buf coh_buffer(const void* base) {
  // raw buffer: stride 0, 2^31-1 bytes, the gfx9 data-format word
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
// (the builtins move 32-bit integers: the values are bit-cast, never converted)
DPK_DEV float cload(coh_buf r, uint32_t i) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, i * 4u, 0, CPOL_SC1));
}
DPK_DEV void cload2(coh_buf r, uint32_t i, float& x, float& y) {  // floats i, i+1, i % 2 == 0
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, i * 4u, 0, CPOL_SC1);
  x = __uint_as_float(v[0]);
  y = __uint_as_float(v[1]);
}
DPK_DEV f32x4 cload4(coh_buf r, uint32_t i) {  // floats i .. i+3, i % 4 == 0
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, i * 4u, 0, CPOL_SC1));
}
DPK_DEV void cstore2(coh_buf r, uint32_t i, float x, float y) {  // floats i, i+1, i % 2 == 0
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(x), __float_as_uint(y)}, r, i * 4u, 0, CPOL_SC1);
}
DPK_DEV void cstore(coh_buf r, uint32_t i, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, i * 4u, 0, CPOL_SC1);
}

// 16 bytes at byte offset 16 i (i.e. two 64-bit words 2 i, 2 i + 1), device-coherent
DPK_DEV u32x4 cload16(coh_buf r, uint32_t i) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, i * 16u, 0, CPOL_SC1));
}
DPK_DEV void cstore8z(coh_buf r, uint32_t i) {  // zero the 64-bit word i
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, r, i * 8u, 0, CPOL_SC1);
}

// Partial sums added by several workgroups with 64-bit integer atomics, in
// fixed point (value * 2^FX_BITS): integer adds are exact, so the sum does not
// depend on the order the workgroups arrive in.  A value that is not finite
// or not below 2^26 in magnitude is entered as FX_BAD; with at most 16 terms a
// total at or beyond FX_NAN in magnitude can only come from such a term and
// reads back as NaN.
constexpr int FX_BITS = 28;
constexpr long long FX_BAD = 1ll << 59, FX_NAN = 1ll << 58;
DPK_DEV long long to_fixed(float v) {
  if (!(fabsf(v) < 67108864.0f)) return FX_BAD;  // NaN included
  return __float2ll_rn(v * (float)(1 << FX_BITS));
}
DPK_DEV float from_fixed(long long x) {
  if (x >= FX_NAN || x <= -FX_NAN) return __builtin_nanf("");
  return __ll2float_rn(x) * (1.0f / (float)(1 << FX_BITS));
}
DPK_DEV long long fixed_word(uint32_t lo, uint32_t hi) { return (long long)(((uint64_t)hi << 32) | lo); }

// Last-arriving-workgroup election.  Every workgroup calls this once after
// writing the data it hands over with coh_store; exactly one (the last) gets
// true and may then read all of it with coh_load.  The counter is reset for
// the next launch.
//
// No release/acquire fences: on multi-XCD gfx950 those are whole-L2
// write-back / invalidate operations, far too slow to run once per workgroup.
// Instead the handed-over data never lives in a non-coherent cache (coh_*),
// each wave waits until its coherent stores have completed before the
// barrier, and only then does one thread count in.
DPK_DEV bool last_block_arrive(unsigned* counter, unsigned expected, int* smem_flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (prev == expected - 1);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *smem_flag = last;
  }
  __syncthreads();
  return *smem_flag != 0;
}

DPK_DEV float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace dpk
