// Decode attention over the resident KV cache (M <= a few rows, each with its
// own sequence and position).  Grouped-query: query head h reads KV head
// h / G, so one workgroup serves the G query heads of a KV head and reads each
// K/V byte once.  The context is split into chunks over workgroups (the keys-
// split-across-threads idea of the oxinfer docs' Whisper cross-attention, here
// across compute units); each chunk keeps an online softmax (running max, sum,
// weighted V) and the last chunk to finish merges the chunks by log-sum-exp.
#include "common.h"
#include "kernels.h"

namespace dpk {

namespace {

constexpr int THREADS = 256;
constexpr int SUB = 64;      // positions per sub-block
constexpr int MAXG = 8;      // query heads per KV head supported
constexpr float LOG2E = 1.4426950408889634f;

template <typename KT>
DPK_DEV float ld_kv(const KT* p) { return (float)*p; }

template <typename KT>
__global__ __launch_bounds__(THREADS) void attn_decode_kernel(AttnDecodeArgs a) {
  const int chunk_id = blockIdx.x, g = blockIdx.y, m = blockIdx.z;
  const RowParam rp = a.rows_param[m];
  const int ctx = rp.pos + 1;
  const int nch = (ctx + a.chunk - 1) / a.chunk;
  if (chunk_id >= nch) return;
  const int d = a.d;  // 64 or 128
  const int G = a.n_heads / a.n_kv;
  const int c0 = chunk_id * a.chunk;
  const int c1 = min(ctx, c0 + a.chunk);
  const int tid = threadIdx.x;

  __shared__ float qs[MAXG][128];
  __shared__ float sc[MAXG][SUB];
  __shared__ float mrun[MAXG], lrun[MAXG], alpha[MAXG];
  __shared__ float obuf[MAXG][128];
  __shared__ int flag;

  for (int i = tid; i < G * d; i += THREADS) {
    const int h = i / d, e = i % d;
    qs[h][e] = a.q[((size_t)m * a.n_heads + g * G + h) * d + e] * a.scale * LOG2E;
  }
  if (tid < MAXG) { mrun[tid] = -INFINITY; lrun[tid] = 0.f; }
  // V accumulation: thread -> (channel e, half): half covers SUB/2 positions
  const int e_ch = tid % 128, half = tid / 128;
  float acc[MAXG];
#pragma unroll
  for (int h = 0; h < MAXG; ++h) acc[h] = 0.f;
  __syncthreads();

  const KT* Kb = (const KT*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 0, g);
  const KT* Vb = (const KT*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 1, g);
  const int tpp = THREADS / SUB;      // 4 threads per position
  const int dq = d / tpp;             // channels per thread in the score phase

  for (int p0 = c0; p0 < c1; p0 += SUB) {
    // scores
    {
      const int pl = tid / tpp, qd = tid % tpp;
      const int p = p0 + pl;
      float s[MAXG];
#pragma unroll
      for (int h = 0; h < MAXG; ++h) s[h] = 0.f;
      if (p < c1) {
        const KT* kr = Kb + (size_t)p * d + qd * dq;
        for (int e = 0; e < dq; ++e) {
          const float kv = ld_kv(kr + e);
#pragma unroll
          for (int h = 0; h < MAXG; ++h)
            if (h < G) s[h] += qs[h][qd * dq + e] * kv;
        }
      }
#pragma unroll
      for (int h = 0; h < MAXG; ++h) {
        s[h] += __shfl_xor(s[h], 1, 64);
        s[h] += __shfl_xor(s[h], 2, 64);
      }
      if (qd == 0) {
#pragma unroll
        for (int h = 0; h < MAXG; ++h)
          if (h < G) sc[h][pl] = (p < c1) ? s[h] : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax update: wave w handles heads w, w+4
    {
      const int w = tid >> 6, l = tid & 63;
      for (int h = w; h < G; h += THREADS / 64) {
        const float v = sc[h][l];
        const float mx = wave_max(v);
        const float mnew = fmaxf(mrun[h], mx);
        const float pr = (v == -INFINITY) ? 0.f : exp2f(v - mnew);
        const float ps = wave_sum(pr);
        sc[h][l] = pr;
        if (l == 0) {
          const float al = (mrun[h] == -INFINITY) ? 0.f : exp2f(mrun[h] - mnew);
          alpha[h] = al;
          lrun[h] = lrun[h] * al + ps;
          mrun[h] = mnew;
        }
      }
    }
    __syncthreads();
    // o += p . V   (V^T rows: channel e, positions contiguous)
    if (e_ch < d) {
      const int pa = p0 + half * (SUB / 2);
      float part[MAXG];
#pragma unroll
      for (int h = 0; h < MAXG; ++h) part[h] = 0.f;
      const KT* vr = Vb + (size_t)e_ch * a.kv.max_seq;
      for (int j = 0; j < SUB / 2; ++j) {
        const int p = pa + j;
        if (p < c1) {
          const float vv = ld_kv(vr + p);
#pragma unroll
          for (int h = 0; h < MAXG; ++h)
            if (h < G) part[h] += sc[h][half * (SUB / 2) + j] * vv;
        }
      }
#pragma unroll
      for (int h = 0; h < MAXG; ++h)
        if (h < G) acc[h] = acc[h] * alpha[h] + part[h];
    }
    __syncthreads();
  }
  // combine the two halves
  if (half == 1 && e_ch < d) {
#pragma unroll
    for (int h = 0; h < MAXG; ++h)
      if (h < G) obuf[h][e_ch] = acc[h];
  }
  __syncthreads();
  if (half == 0 && e_ch < d) {
#pragma unroll
    for (int h = 0; h < MAXG; ++h)
      if (h < G) obuf[h][e_ch] += acc[h];
  }
  __syncthreads();

  if (nch == 1) {
    for (int i = tid; i < G * d; i += THREADS) {
      const int h = i / d, e = i % d;
      a.out[(size_t)m * a.n_heads * d + (size_t)(g * G + h) * d + e] = obuf[h][e] / lrun[h];
    }
    return;
  }
  // partial record per (row, head, chunk): [m_run, l_run, o[d]]
  const int rec = d + 2;
  for (int i = tid; i < G * rec; i += THREADS) {
    const int h = i / rec, j = i % rec;
    const float v = j == 0 ? mrun[h] : (j == 1 ? lrun[h] : obuf[h][j - 2]);
    a.part[(((size_t)m * a.n_heads + g * G + h) * a.max_chunks + chunk_id) * rec + j] = v;
  }
  if (!last_block_arrive(a.counters + m * a.n_kv + g, nch, &flag)) return;
  for (int i = tid; i < G * d; i += THREADS) {
    const int h = i / d, e = i % d;
    const float* base = a.part + (((size_t)m * a.n_heads + g * G + h) * a.max_chunks) * rec;
    float mx = -INFINITY;
    for (int c = 0; c < nch; ++c) mx = fmaxf(mx, base[(size_t)c * rec]);
    float num = 0.f, den = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float w = exp2f(base[(size_t)c * rec] - mx);
      den += w * base[(size_t)c * rec + 1];
      num += w * base[(size_t)c * rec + 2 + e];
    }
    a.out[(size_t)m * a.n_heads * d + (size_t)(g * G + h) * d + e] = num / den;
  }
}

}  // namespace

hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t stream) {
  if (a.d > 128 || a.n_heads / a.n_kv > MAXG || a.chunk % SUB != 0) return hipErrorInvalidValue;
  dim3 grid(a.max_chunks, a.n_kv, a.M);
  if (a.kv.is_f32)
    hipLaunchKernelGGL(attn_decode_kernel<float>, grid, dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_decode_kernel<_Float16>, grid, dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dpk
