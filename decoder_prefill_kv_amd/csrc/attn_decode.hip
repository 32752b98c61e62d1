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

// 8 cache elements as raw bits (16 bytes of fp16 or 32 bytes of fp32)
template <typename KT>
struct Raw8 {
  u32x4 w[sizeof(KT) / 2];
};
template <typename KT>
DPK_DEV void ld8(Raw8<KT>& r, const KT* p) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(KT) / 2); ++i) r.w[i] = *(const u32x4*)((const char*)p + 16 * i);
}
DPK_DEV void cvt8(const Raw8<_Float16>& r, float* o) {
  const f16x8 v = __builtin_bit_cast(f16x8, r.w[0]);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
}
DPK_DEV void cvt8(const Raw8<float>& r, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i] = __uint_as_float(r.w[0][i]);
    o[4 + i] = __uint_as_float(r.w[1][i]);
  }
}

template <typename KT, int D, int G>
__global__ __launch_bounds__(THREADS) void attn_decode_kernel(AttnDecodeArgs a) {
  const int chunk_id = blockIdx.x, g = blockIdx.y, m = blockIdx.z;
  const RowParam rp = a.rows_param[m];
  const int ctx = rp.pos + 1;
  const int nch = (ctx + CHUNK - 1) / CHUNK;
  if (chunk_id >= nch) return;
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

  const KT* Kb = (const KT*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 0, g);
  const KT* Vb = (const KT*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 1, g);
  __shared__ float knew[MAXD], vnew[MAXD];
  const bool raw = a.qkv_raw != nullptr;
  const bool own = raw && rp.pos >= c0 && rp.pos < c1;  // this chunk holds the new position

  // all cache loads are issued before anything waits: the K row of this
  // thread's position and the V^T slice of its P.V channel
  constexpr int SL = THREADS / D;          // 2 slices for D = 128, 4 for D = 64
  constexpr int SPOS = CHUNK / SL;
  const int p = c0 + tid;
  const bool fresh = own && p == rp.pos;  // the new key is computed here, not loaded
  Raw8<KT> kreg[D / 8];
  if (p < c1 && !fresh) {
    const KT* kr = Kb + (size_t)p * D;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) ld8(kreg[i], kr + 8 * i);
  }
  const int e = tid % D, sl = tid / D;
  const int pa = c0 + sl * SPOS;
  const int nvalid = min(SPOS, c1 - pa);  // may be <= 0
  Raw8<KT> vreg[SPOS / 8];
  {
    // the slab row has max_seq (multiple of 64) entries, so 8-position loads
    // that start inside the context stay inside the row
    const KT* vr = Vb + (size_t)e * a.kv.max_seq + pa;
#pragma unroll
    for (int j = 0; j < SPOS / 8; ++j)
      if (8 * j < nvalid) ld8(vreg[j], vr + 8 * j);
  }
  if (!raw) {
    for (int i = tid; i < G * D; i += THREADS) {
      const int h = i / D, e = i % D;
      qs[h][e] = a.q[((size_t)m * a.n_heads + g * G + h) * D + e] * a.scale * LOG2E;
    }
  } else {
    // QK-norm (RMSNorm over head_dim with gain) and RoPE at the row's position
    // for the G query heads (and, in the owning chunk, the new key); wave w
    // handles heads w, w+4, ...; head index G is the key
    const float* src = a.qkv_raw + (size_t)m * a.ld_raw;
    const int nh = own ? G + 1 : G;
    for (int h = wave; h < nh; h += 4) {
      const float* x = (h < G) ? src + (size_t)(g * G + h) * D : src + (size_t)(a.n_heads + g) * D;
      const uint16_t* gn = (h < G) ? a.qn : a.kn;
      float ss = 0.f;
      for (int e = lane; e < D; e += 64) ss += x[e] * x[e];
      ss = wave_sum(ss);
      const float r = gn ? rsqrtf(ss / (float)D + a.eps) : 1.0f;
      for (int i = lane; i < D / 2; i += 64) {
        float x1 = x[i] * r, x2 = x[i + D / 2] * r;
        if (gn) {
          x1 *= bf16_to_f32(gn[i]);
          x2 *= bf16_to_f32(gn[i + D / 2]);
        }
        const float cs = a.rope_cos[(size_t)rp.pos * (D / 2) + i], sn = a.rope_sin[(size_t)rp.pos * (D / 2) + i];
        const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
        if (h < G) {
          qs[h][i] = y1 * a.scale * LOG2E;
          qs[h][i + D / 2] = y2 * a.scale * LOG2E;
        } else {
          knew[i] = y1;
          knew[i + D / 2] = y2;
        }
      }
    }
    if (own) {
      const float* vsrc = src + (size_t)(a.n_heads + a.n_kv + g) * D;
      for (int e = tid; e < D; e += THREADS) vnew[e] = vsrc[e];
    }
  }
  __syncthreads();
  if (own) {  // the cache keeps the new position for later steps
    for (int e = tid; e < D; e += THREADS) {
      kv_store(a.kv, kv_offset(a.kv, rp.seq, a.layer, 0, g, e, rp.pos), knew[e]);
      kv_store(a.kv, kv_offset(a.kv, rp.seq, a.layer, 1, g, e, rp.pos), vnew[e]);
    }
  }

  // ---- scores (log2 domain): thread t -> position c0 + t
  float s[MAXG];
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = 0.f;
  if (p < c1) {
#pragma unroll
    for (int e8 = 0; e8 < D; e8 += 8) {
      float kv[8];
      if (fresh) {
#pragma unroll
        for (int i = 0; i < 8; ++i) kv[i] = knew[e8 + i];
      } else {
        cvt8(kreg[e8 / 8], kv);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) s[h] += qs[h][e8 + i] * kv[i];
      }
    }
  }
  // chunk max per head
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float v = (p < c1) ? s[h] : -INFINITY;
    const float mx = wave_max(v);
    if (lane == 0) red[wave][h] = mx;
  }
  __syncthreads();
  if (tid < G) stat[0][tid] = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float e = (p < c1) ? exp2f(s[h] - stat[0][h]) : 0.f;
    pr[h][tid] = e;
    const float sm = wave_sum(e);
    if (lane == 0) red[wave][h] = sm;
  }
  __syncthreads();
  if (tid < G) stat[1][tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];

  // ---- P.V: thread -> (channel e, slice of SPOS positions)
  float acc[MAXG];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.f;
#pragma unroll
  for (int j = 0; j < SPOS / 8; ++j) {
    if (8 * j >= nvalid) break;
    float vv[8];
    cvt8(vreg[j], vv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (8 * j + i >= nvalid) vv[i] = 0.f;  // beyond the context: may be uninitialised
      if (own && pa + 8 * j + i == rp.pos) vv[i] = vnew[e];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] += pr[h][sl * SPOS + 8 * j + i] * vv[i];
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) obuf[sl][h][e] = acc[h];
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

template <typename KT, int D>
hipError_t launch_g(const AttnDecodeArgs& a, dim3 grid, hipStream_t stream) {
  switch (a.n_heads / a.n_kv) {
    case 1: launch((attn_decode_kernel<KT, D, 1>), grid, dim3(THREADS), 0, stream, a); break;
    case 2: launch((attn_decode_kernel<KT, D, 2>), grid, dim3(THREADS), 0, stream, a); break;
    case 4: launch((attn_decode_kernel<KT, D, 4>), grid, dim3(THREADS), 0, stream, a); break;
    case 8: launch((attn_decode_kernel<KT, D, 8>), grid, dim3(THREADS), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t stream) {
  if (a.n_heads % a.n_kv || a.max_chunks > MAXCH || a.kv.max_seq % 64) return hipErrorInvalidValue;
  dim3 grid(a.max_chunks, a.n_kv, a.M);
  if (a.kv.is_f32 && a.d == 64) return launch_g<float, 64>(a, grid, stream);
  if (a.kv.is_f32 && a.d == 128) return launch_g<float, 128>(a, grid, stream);
  if (!a.kv.is_f32 && a.d == 64) return launch_g<_Float16, 64>(a, grid, stream);
  if (!a.kv.is_f32 && a.d == 128) return launch_g<_Float16, 128>(a, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace dpk
