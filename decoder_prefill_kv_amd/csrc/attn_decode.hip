// Decode attention over the resident KV cache (M rows, each with its own
// sequence slot and position; a row attends to cached positions 0..pos).
// Grouped-query: query head h reads KV head h / G, so one workgroup serves
// the G query heads of a KV head and reads each K/V byte once.  The context is
// split into chunks of 256 positions over workgroups (the keys-split-across-
// threads idea of the oxinfer docs' Whisper cross-attention, here across
// compute units); each chunk computes its softmax statistics (max, sum,
// weighted V) and the last chunk to finish merges them by log-sum-exp.
//
// Per chunk: thread t owns position c0 + t for the scores (one 16-byte vector
// load per 8 fp16 K values) and, for P.V, one channel over a slice of the
// positions (V is stored transposed, positions contiguous per channel).
#include "common.h"
#include "kernels.h"

namespace dpk {

namespace {

constexpr int THREADS = 256;
constexpr int CHUNK = 256;   // positions per workgroup (= threads)
constexpr int MAXG = 8;      // query heads per KV head supported
constexpr int MAXD = 128;
constexpr int MAXCH = 64;    // chunks merged through LDS statistics
constexpr float LOG2E = 1.4426950408889634f;

// 16-byte vector of cache elements -> floats
DPK_DEV void cvt8(const _Float16* p, float* o) {
  const f16x8 v = *(const f16x8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
}
DPK_DEV void cvt8(const float* p, float* o) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

template <typename KT, int D>
__global__ __launch_bounds__(THREADS) void attn_decode_kernel(AttnDecodeArgs a) {
  const int chunk_id = blockIdx.x, g = blockIdx.y, m = blockIdx.z;
  const RowParam rp = a.rows_param[m];
  const int ctx = rp.pos + 1;
  const int nch = (ctx + CHUNK - 1) / CHUNK;
  if (chunk_id >= nch) return;
  const int G = a.n_heads / a.n_kv;
  const int c0 = chunk_id * CHUNK;
  const int c1 = min(ctx, c0 + CHUNK);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  __shared__ float qs[MAXG][MAXD];
  __shared__ float pr[MAXG][CHUNK];
  __shared__ float red[4][MAXG];
  __shared__ float stat[2][MAXG];        // chunk max, chunk sum
  __shared__ float obuf[4][MAXG][MAXD];  // P.V partials of the position slices
  __shared__ float mw[MAXCH][MAXG];      // merge: chunk weights
  __shared__ int flag;

  for (int i = tid; i < G * D; i += THREADS) {
    const int h = i / D, e = i % D;
    qs[h][e] = a.q[((size_t)m * a.n_heads + g * G + h) * D + e] * a.scale * LOG2E;
  }
  __syncthreads();

  const KT* Kb = (const KT*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 0, g);
  const KT* Vb = (const KT*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 1, g);

  // ---- scores (log2 domain): thread t -> position c0 + t
  const int p = c0 + tid;
  float s[MAXG];
#pragma unroll
  for (int h = 0; h < MAXG; ++h) s[h] = 0.f;
  if (p < c1) {
    const KT* kr = Kb + (size_t)p * D;
#pragma unroll
    for (int e8 = 0; e8 < D; e8 += 8) {
      float kv[8];
      cvt8(kr + e8, kv);
#pragma unroll
      for (int h = 0; h < MAXG; ++h)
        if (h < G) {
#pragma unroll
          for (int i = 0; i < 8; ++i) s[h] += qs[h][e8 + i] * kv[i];
        }
    }
  }
  // chunk max per head
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
    if (h >= G) break;
    const float v = (p < c1) ? s[h] : -INFINITY;
    const float mx = wave_max(v);
    if (lane == 0) red[wave][h] = mx;
  }
  __syncthreads();
  if (tid < G) stat[0][tid] = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
  __syncthreads();
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
    if (h >= G) break;
    const float e = (p < c1) ? exp2f(s[h] - stat[0][h]) : 0.f;
    pr[h][tid] = e;
    const float sm = wave_sum(e);
    if (lane == 0) red[wave][h] = sm;
  }
  __syncthreads();
  if (tid < G) stat[1][tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];

  // ---- P.V: thread -> (channel e, slice of CHUNK / SL positions)
  constexpr int SL = THREADS / D;          // 2 slices for D = 128, 4 for D = 64
  constexpr int SPOS = CHUNK / SL;
  const int e = tid % D, sl = tid / D;
  float acc[MAXG];
#pragma unroll
  for (int h = 0; h < MAXG; ++h) acc[h] = 0.f;
  const int pa = c0 + sl * SPOS;
  const KT* vr = Vb + (size_t)e * a.kv.max_seq + pa;
  const int nvalid = min(SPOS, c1 - pa);  // may be <= 0
  for (int j8 = 0; j8 < SPOS; j8 += 8) {
    if (j8 >= nvalid) break;
    float vv[8];
    cvt8(vr + j8, vv);  // the slab row has max_seq (multiple of 64) entries
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (j8 + i >= nvalid) vv[i] = 0.f;  // beyond the context: may be uninitialised
#pragma unroll
      for (int h = 0; h < MAXG; ++h)
        if (h < G) acc[h] += pr[h][sl * SPOS + j8 + i] * vv[i];
    }
  }
#pragma unroll
  for (int h = 0; h < MAXG; ++h)
    if (h < G) obuf[sl][h][e] = acc[h];
  __syncthreads();

  if (nch == 1) {
    for (int i = tid; i < G * D; i += THREADS) {
      const int h = i / D, ee = i % D;
      float o = 0.f;
      for (int k = 0; k < SL; ++k) o += obuf[k][h][ee];
      a.out[(size_t)m * a.n_heads * D + (size_t)(g * G + h) * D + ee] = o / stat[1][h];
    }
    return;
  }
  // partial record per (row, head, chunk): [max, sum, o[D]] (unnormalised o)
  const int rec = D + 2;
  for (int i = tid; i < G * rec; i += THREADS) {
    const int h = i / rec, j = i % rec;
    float v;
    if (j < 2) {
      v = stat[j][h];
    } else {
      v = 0.f;
      for (int k = 0; k < SL; ++k) v += obuf[k][h][j - 2];
    }
    coh_store(a.part + (((size_t)m * a.n_heads + g * G + h) * a.max_chunks + chunk_id) * rec + j, v);
  }
  if (!last_block_arrive(a.counters + m * a.n_kv + g, nch, &flag)) return;
  // merge: weight of chunk c for head h = 2^(m_c - M) / sum_c' 2^(m_c' - M) l_c'
  // (all (max, sum) pairs are loaded in parallel, one per thread)
  __shared__ float ml[2][MAXCH][MAXG];
  for (int i = tid; i < G * nch; i += THREADS) {
    const int h = i % G, c = i / G;
    const float* base = a.part + ((((size_t)m * a.n_heads + g * G + h) * a.max_chunks) + c) * rec;
    ml[0][c][h] = coh_load(base);
    ml[1][c][h] = coh_load(base + 1);
  }
  __syncthreads();
  if (tid < G) {
    const int h = tid;
    float mx = -INFINITY;
    for (int c = 0; c < nch; ++c) mx = fmaxf(mx, ml[0][c][h]);
    float den = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float w = exp2f(ml[0][c][h] - mx);
      mw[c][h] = w;
      den += w * ml[1][c][h];
    }
    const float inv = 1.0f / den;
    for (int c = 0; c < nch; ++c) mw[c][h] *= inv;
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += THREADS) {
    const int h = i / D, ee = i % D;
    const float* base = a.part + (((size_t)m * a.n_heads + g * G + h) * a.max_chunks) * rec + 2 + ee;
    float o = 0.f;
    int c = 0;
    for (; c + 4 <= nch; c += 4) {
      const float o0 = coh_load(base + (size_t)c * rec), o1 = coh_load(base + (size_t)(c + 1) * rec);
      const float o2 = coh_load(base + (size_t)(c + 2) * rec), o3 = coh_load(base + (size_t)(c + 3) * rec);
      o += mw[c][h] * o0 + mw[c + 1][h] * o1 + mw[c + 2][h] * o2 + mw[c + 3][h] * o3;
    }
    for (; c < nch; ++c) o += mw[c][h] * coh_load(base + (size_t)c * rec);
    a.out[(size_t)m * a.n_heads * D + (size_t)(g * G + h) * D + ee] = o;
  }
}

}  // namespace

int attn_decode_chunk() { return CHUNK; }

hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t stream) {
  if (a.n_heads / a.n_kv > MAXG || a.max_chunks > MAXCH || a.kv.max_seq % 64) return hipErrorInvalidValue;
  dim3 grid(a.max_chunks, a.n_kv, a.M);
  if (a.kv.is_f32 && a.d == 64)
    hipLaunchKernelGGL((attn_decode_kernel<float, 64>), grid, dim3(THREADS), 0, stream, a);
  else if (a.kv.is_f32 && a.d == 128)
    hipLaunchKernelGGL((attn_decode_kernel<float, 128>), grid, dim3(THREADS), 0, stream, a);
  else if (!a.kv.is_f32 && a.d == 64)
    hipLaunchKernelGGL((attn_decode_kernel<_Float16, 64>), grid, dim3(THREADS), 0, stream, a);
  else if (!a.kv.is_f32 && a.d == 128)
    hipLaunchKernelGGL((attn_decode_kernel<_Float16, 128>), grid, dim3(THREADS), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dpk
