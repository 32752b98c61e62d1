// Decode attention on gfx950 matrix cores (fp16 KV cache).
//
// Same contract as attn_decode.hip (rows with their own slot and position,
// grouped-query heads, context split in chunks of 256 positions merged by
// log-sum-exp), but both products run on v_mfma_f32_16x16x32_f16 with the G
// query heads of a KV head as the MFMA columns:
//   S   = K Q^T     A = K rows (16 positions x 32 channels, straight from the
//                   cache), B = q (32 channels x 16 columns, G used)
//   O^T = V^T P^T   A = V^T rows (16 channels x 32 positions), B = P^T taken
//                   directly from the S accumulators
// q and p are split into fp16 hi + lo (two MFMAs each), so the only rounding
// is the fp16 cache itself.  Each wave owns 64 positions of the chunk; the
// four waves' softmax statistics are combined through LDS.
//
// MFMA 16x16x32 lane layout: A lane l holds row l%16, k = 8(l/16)..+7; B lane l
// holds column l%16, the same k; D lane l holds rows 4(l/16)+v, column l%16.
#include "common.h"
#include "kernels.h"

namespace dpk {

namespace {

constexpr int THREADS = 256;
constexpr int CHUNK = 256;   // positions per workgroup, 64 per wave
constexpr int MAXCH = 64;
constexpr float LOG2E = 1.4426950408889634f;

DPK_DEV void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

template <int D>
__global__ __launch_bounds__(THREADS) void attn_decode_mfma_kernel(AttnDecodeArgs a) {
  const int chunk_id = blockIdx.x, g = blockIdx.y, m = blockIdx.z;
  const RowParam rp = a.rows_param[m];
  const int ctx = rp.pos + 1;
  const int nch = (ctx + CHUNK - 1) / CHUNK;
  if (chunk_id >= nch) return;
  const int G = a.n_heads / a.n_kv;
  const int c0 = chunk_id * CHUNK;
  const int c1 = min(ctx, c0 + CHUNK);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, j4 = lane >> 4;
  const int wp0 = c0 + 64 * wave;  // this wave's first position

  __shared__ float qs[16][D];
  __shared__ float knew[D], vnew[D];
  __shared__ float wst[4][2][16];     // per wave: max, sum per column
  __shared__ float ow[4][D][16];      // per wave: O^T partial
  __shared__ float ml[2][MAXCH][16];
  __shared__ float mw[MAXCH][16];
  __shared__ int flag;

  const _Float16* Kb = (const _Float16*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 0, g);
  const _Float16* Vb = (const _Float16*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 1, g);
  const bool raw = a.qkv_raw != nullptr;
  const bool own = raw && rp.pos >= c0 && rp.pos < c1;

  // ---- cache loads first (independent of q): K fragments of 4 tiles x D/32
  // k-steps, V^T fragments of D/16 channel tiles x 2 position steps
  u32x4 kf[4][D / 32];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int p = wp0 + 16 * t + r16;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      kf[t][s] = u32x4{0u, 0u, 0u, 0u};
      if (p < c1) kf[t][s] = *(const u32x4*)(Kb + (size_t)p * D + 32 * s + 8 * j4);
    }
  }
  // position slots of k-group j4 in step ps: 32 ps + {4 j4..+3, 16 + 4 j4..+3}
  u32x2 vf[D / 16][2][2];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int ps = 0; ps < 2; ++ps)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int p = wp0 + 32 * ps + 16 * h + 4 * j4;
        vf[dt][ps][h] = u32x2{0u, 0u};
        // the 4-position group stays inside the slab row (max_seq % 64 == 0)
        if (p < c1) {
          vf[dt][ps][h] = *(const u32x2*)(Vb + (size_t)(dt * 16 + r16) * a.kv.max_seq + p);
          if (p + 4 > c1) {  // positions past the context may hold any bits (0 * NaN)
            f16x4 v4 = __builtin_bit_cast(f16x4, vf[dt][ps][h]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (p + e >= c1) v4[e] = (_Float16)0.f;
            vf[dt][ps][h] = __builtin_bit_cast(u32x2, v4);
          }
        }
      }

  // ---- q (and in raw mode the new key/value) -> LDS
  for (int i = tid; i < 16 * D; i += THREADS) (&qs[0][0])[i] = 0.f;
  __syncthreads();
  if (!raw) {
    for (int i = tid; i < G * D; i += THREADS) {
      const int h = i / D, e = i % D;
      qs[h][e] = a.q[((size_t)m * a.n_heads + g * G + h) * D + e] * a.scale * LOG2E;
    }
  } else {
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
  if (own) {
    for (int e = tid; e < D; e += THREADS) {
      kv_store(a.kv, kv_offset(a.kv, rp.seq, a.layer, 0, g, e, rp.pos), knew[e]);
      kv_store(a.kv, kv_offset(a.kv, rp.seq, a.layer, 1, g, e, rp.pos), vnew[e]);
    }
    // the new position inside this wave's fragments comes from knew / vnew
    const int off = rp.pos - wp0;
    if (off >= 0 && off < 64) {
      // compile-time fragment indices only (runtime ones would spill the arrays)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t == off / 16 && r16 == off % 16) {
#pragma unroll
          for (int s = 0; s < D / 32; ++s) {
            f16x8 k8;
#pragma unroll
            for (int i = 0; i < 8; ++i) k8[i] = (_Float16)knew[32 * s + 8 * j4 + i];
            kf[t][s] = __builtin_bit_cast(u32x4, k8);
          }
        }
      const int e4 = off % 4;
#pragma unroll
      for (int ps = 0; ps < 2; ++ps)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (ps == off / 32 && h == (off % 32) / 16 && j4 == (off % 16) / 4) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
              f16x4 v4 = __builtin_bit_cast(f16x4, vf[dt][ps][h]);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (e == e4) v4[e] = (_Float16)vnew[dt * 16 + r16];
              vf[dt][ps][h] = __builtin_bit_cast(u32x2, v4);
            }
          }
    }
  }

  // ---- S = K Q^T (log2 domain), 4 tiles of 16 positions
  f16x8 qh[D / 32], ql[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      _Float16 h, l;
      split_f16(qs[r16][32 * s + 8 * j4 + i], h, l);
      qh[s][i] = h;
      ql[s][i] = l;
    }
  f32x4 sc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const f16x8 A = __builtin_bit_cast(f16x8, kf[t][s]);
      sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qh[s], sc[t], 0, 0, 0);
      sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ql[s], sc[t], 0, 0, 0);
    }
  }
  // mask (positions 16 t + 4 j4 + v past the context), column max / sum
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (wp0 + 16 * t + 4 * j4 + v >= c1) sc[t][v] = -INFINITY;
      mx = fmaxf(mx, sc[t][v]);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float e = (sc[t][v] == -INFINITY) ? 0.f : exp2f(sc[t][v] - mx);
      sc[t][v] = e;
      sum += e;
    }
  sum += __shfl_xor(sum, 16, 64);
  sum += __shfl_xor(sum, 32, 64);

  // ---- O^T = V^T P^T: step ps uses tiles 2 ps (slots 0..3) and 2 ps + 1 (4..7)
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
    f16x8 ph, pl;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      _Float16 h0, l0, h1, l1;
      split_f16(sc[2 * ps][v], h0, l0);
      split_f16(sc[2 * ps + 1][v], h1, l1);
      ph[v] = h0;
      pl[v] = l0;
      ph[4 + v] = h1;
      pl[4 + v] = l1;
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u32x4 w = {vf[dt][ps][0].x, vf[dt][ps][0].y, vf[dt][ps][1].x, vf[dt][ps][1].y};
      const f16x8 A = __builtin_bit_cast(f16x8, w);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ph, o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pl, o[dt], 0, 0, 0);
    }
  }

  // ---- combine the four waves (per column = query head)
  if (j4 == 0) {
    wst[wave][0][r16] = mx;
    wst[wave][1][r16] = sum;
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int v = 0; v < 4; ++v) ow[wave][dt * 16 + 4 * j4 + v][r16] = o[dt][v];
  __syncthreads();
  // chunk statistics per column c: M = max_w m_w, L = sum_w 2^(m_w - M) l_w,
  // O = sum_w 2^(m_w - M) O_w
  const int rec = D + 2;
  for (int i = tid; i < G * D; i += THREADS) {
    const int c = i / D, e = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wst[w][0][c]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (wst[w][0][c] == -INFINITY) ? 0.f : exp2f(wst[w][0][c] - M);
      L += f * wst[w][1][c];
      O += f * ow[w][e][c];
    }
    if (nch == 1) {
      a.out[(size_t)m * a.n_heads * D + (size_t)(g * G + c) * D + e] = O / L;
    } else {
      float* r = a.part + (((size_t)m * a.n_heads + g * G + c) * a.max_chunks + chunk_id) * rec;
      coh_store(r + 2 + e, O);
      if (e == 0) {
        coh_store(r, M);
        coh_store(r + 1, L);
      }
    }
  }
  if (nch == 1) return;
  if (!last_block_arrive(a.counters + m * a.n_kv + g, nch, &flag)) return;
  for (int i = tid; i < G * nch; i += THREADS) {
    const int h = i % G, c = i / G;
    const float* base = a.part + ((((size_t)m * a.n_heads + g * G + h) * a.max_chunks) + c) * rec;
    ml[0][c][h] = coh_load(base);
    ml[1][c][h] = coh_load(base + 1);
  }
  __syncthreads();
  if (tid < G) {
    const int h = tid;
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, ml[0][c][h]);
    float den = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float w = exp2f(ml[0][c][h] - M);
      mw[c][h] = w;
      den += w * ml[1][c][h];
    }
    const float inv = 1.0f / den;
    for (int c = 0; c < nch; ++c) mw[c][h] *= inv;
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += THREADS) {
    const int h = i / D, e = i % D;
    const float* base = a.part + (((size_t)m * a.n_heads + g * G + h) * a.max_chunks) * rec + 2 + e;
    float O = 0.f;
    int c = 0;
    for (; c + 4 <= nch; c += 4) {
      const float o0 = coh_load(base + (size_t)c * rec), o1 = coh_load(base + (size_t)(c + 1) * rec);
      const float o2 = coh_load(base + (size_t)(c + 2) * rec), o3 = coh_load(base + (size_t)(c + 3) * rec);
      O += mw[c][h] * o0 + mw[c + 1][h] * o1 + mw[c + 2][h] * o2 + mw[c + 3][h] * o3;
    }
    for (; c < nch; ++c) O += mw[c][h] * coh_load(base + (size_t)c * rec);
    a.out[(size_t)m * a.n_heads * D + (size_t)(g * G + h) * D + e] = O;
  }
}

}  // namespace

hipError_t launch_attn_decode_mfma(const AttnDecodeArgs& a, hipStream_t stream) {
  if (a.kv.is_f32 || a.n_heads % a.n_kv || a.n_heads / a.n_kv > 16 || a.max_chunks > MAXCH || a.kv.max_seq % 64)
    return hipErrorInvalidValue;
  dim3 grid(a.max_chunks, a.n_kv, a.M);
  if (a.d == 128)
    launch(attn_decode_mfma_kernel<128>, grid, dim3(THREADS), 0, stream, a);
  else if (a.d == 64)
    launch(attn_decode_mfma_kernel<64>, grid, dim3(THREADS), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dpk
