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

// the fp16 of positions p + e >= c1 zeroed (a group of 8 from position p)
DPK_DEV u32x4 vmask(u32x4 v, int p, int c1) {
  const int n = c1 - p;
  auto m = [n](int e) { return n >= e + 2 ? 0xffffffffu : (n == e + 1 ? 0x0000ffffu : 0u); };
  return u32x4{v.x & m(0), v.y & m(2), v.z & m(4), v.w & m(6)};
}

template <int D, bool RAW>
__global__ __launch_bounds__(THREADS) void attn_decode_mfma_kernel(AttnDecodeArgs a) {
  const int chunk_id = blockIdx.x, g = blockIdx.y;
  // rows m .. m + R - 1 (one sequence when R > 1); column c = r G + head
  const int SH = a.share > 1 ? a.share : 1;
  const int m = blockIdx.z * SH;
  const int R = min(SH, a.M - m);
  const int G = a.n_heads / a.n_kv;
  const int RG = R * G;
  RowParam rp = a.rows_param[m];
  for (int r = 1; r < R; ++r) rp.pos = max(rp.pos, a.rows_param[m + r].pos);
  const int ctx = rp.pos + 1;  // the group's longest context
  const int nch = (ctx + CHUNK - 1) / CHUNK;
  if (chunk_id >= nch) return;
  const int c0 = chunk_id * CHUNK;
  const int c1 = min(ctx, c0 + CHUNK);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform over the wave
  const int r16 = lane & 15, j4 = lane >> 4;
  const int wp0 = c0 + 64 * wave;  // this wave's first position
  // end of this lane's column (its row's context) inside the chunk
  const int c1_col = (r16 < RG) ? min(a.rows_param[m + r16 / G].pos + 1, c1) : c1;

  __shared__ float qs[16][D];
  __shared__ float knew[D], vnew[D];
  __shared__ float wst[4][2][16];     // per wave: max, sum per column
  __shared__ float ow[4][D][16];      // per wave: O^T partial
  __shared__ float ml[2][MAXCH][16];
  __shared__ float mw[MAXCH][16];
  __shared__ int flag;

  const _Float16* Kb = (const _Float16*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 0, g);
  const _Float16* Vb = (const _Float16*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 1, g);
  constexpr bool raw = RAW;  // a.qkv_raw != nullptr
  const bool own = raw && rp.pos >= c0 && rp.pos < c1;

  // ---- this workgroup's inputs other than the cache are loaded before it,
  // so that waiting for them leaves the cache loads in flight (loads complete
  // in issue order).  Not raw: q of the RG columns.  Raw: the row's projected
  // heads that this wave normalises and rotates (query heads wave, wave + 4,
  // ..., then the KV head's key when own), their gains, the rotation of the
  // position and the new value; clamped indices, no branches.
  constexpr int QPT = 16 * D / THREADS;
  constexpr int HD = D / 2;
  constexpr int NIT = (16 + 1 + 3) / 4;  // G + 1 <= 17 heads over 4 waves
  const int nh = own ? G + 1 : G;
  const int li = lane % HD;
  float qv[QPT];
  float xr[NIT][2], rc = 0.f, rsn = 0.f, vv = 0.f;
  uint16_t gr[NIT][2];
  if constexpr (!raw) {
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int i = tid + j * THREADS, c = i / D, e = i % D, cc = min(c, RG - 1);
      qv[j] = a.q[((size_t)(m + cc / G) * a.n_heads + g * G + cc % G) * D + e];  // columns >= RG: zeroed later
    }
  } else {
    const float* src = a.qkv_raw + (size_t)m * a.ld_raw;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int h = min(wave + 4 * it, nh - 1);
      const float* x = (h < G) ? src + (size_t)(g * G + h) * D : src + (size_t)(a.n_heads + g) * D;
      xr[it][0] = x[li];
      xr[it][1] = x[li + HD];
      const uint16_t* gn = (h < G) ? a.qn : a.kn;
      // no gain: read a valid dummy address (no branch), use 1
      const uint16_t* gp = gn ? gn : (const uint16_t*)a.rope_cos;
      gr[it][0] = gp[li];  // converted where used
      gr[it][1] = gp[li + HD];
    }
    rc = a.rope_cos[(size_t)rp.pos * HD + li];
    rsn = a.rope_sin[(size_t)rp.pos * HD + li];
    vv = src[(size_t)(a.n_heads + a.n_kv + g) * D + tid % D];
  }

  // ---- cache loads (independent of q), unconditional: positions past the
  // context read the last one's address (K rows are masked in S, V groups at
  // the product).  K fragments of 4 tiles x D/32 k-steps, V^T fragments of
  // D/16 channel tiles x 2 position steps.
  // Row r of K tile t is position kpos(t, r) = 32 (t / 2) + 8 (r / 4) + 4 (t % 2)
  // + r % 4 of the wave's 64: the S accumulators of tiles 2 ps and 2 ps + 1 then
  // give lane group j4 the positions 32 ps + 8 j4 .. + 7, which is the k range
  // of P^T that lane group takes in the P V product, so V^T is read as one
  // contiguous 8-position (16-byte) group per lane.
  u32x4 kf[4][D / 32];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int p = min(wp0 + 32 * (t >> 1) + 8 * (r16 >> 2) + 4 * (t & 1) + (r16 & 3), c1 - 1);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) kf[t][s] = *(const u32x4*)(Kb + (size_t)p * D + 32 * s + 8 * j4);
  }
  // V^T: channel row dt * 16 + r16, positions 32 ps + 8 j4 .. + 7 (an 8-position
  // group stays inside the slab row: max_seq % 64 == 0)
  u32x4 vf[D / 16][2];
  const int vlast = (c1 - 1) & ~7;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int p = min(wp0 + 32 * ps + 8 * j4, vlast);
      vf[dt][ps] = *(const u32x4*)(Vb + (size_t)(dt * 16 + r16) * a.kv.max_seq + p);
    }
  const bool vfull = wp0 + 64 <= c1;  // no V group of this wave reaches past the context

  // ---- q (and in raw mode the new key/value) -> LDS
  if constexpr (!raw) {
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int i = tid + j * THREADS;
      // (a multiply, not a select: a load used on one side of a select gets
      // sunk past the cache loads and then waits for them)
      (&qs[0][0])[i] = qv[j] * ((i / D < RG) ? a.scale * LOG2E : 0.f);
    }
  } else {
    for (int i = G * D + tid; i < 16 * D; i += THREADS) (&qs[0][0])[i] = 0.f;  // unused columns
    const bool qk = a.qn != nullptr;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int h = wave + 4 * it;
      if (h >= nh) break;
      const bool on = lane < HD;
      float ss = on ? xr[it][0] * xr[it][0] + xr[it][1] * xr[it][1] : 0.f;
      ss = wave_sum(ss);
      const bool normed = (h < G) ? qk : (a.kn != nullptr);
      const float r = normed ? rsqrtf(ss / (float)D + a.eps) : 1.0f;
      if (on) {
        const float g0 = normed ? bf16_to_f32(gr[it][0]) : 1.0f, g1 = normed ? bf16_to_f32(gr[it][1]) : 1.0f;
        const float x1 = xr[it][0] * r * g0, x2 = xr[it][1] * r * g1;
        const float y1 = x1 * rc - x2 * rsn, y2 = x2 * rc + x1 * rsn;
        if (h < G) {
          qs[h][lane] = y1 * a.scale * LOG2E;
          qs[h][lane + HD] = y2 * a.scale * LOG2E;
        } else {
          knew[lane] = y1;
          knew[lane + HD] = y2;
        }
      }
    }
    if (own && tid < D) vnew[tid] = vv;
  }
  lds_barrier();  // an LDS-only barrier: the cache loads stay in flight
  if (own) {
    for (int e = tid; e < D; e += THREADS) {
      kv_store(a.kv, kv_offset(a.kv, rp.seq, a.layer, 0, g, e, rp.pos), knew[e]);
      kv_store(a.kv, kv_offset(a.kv, rp.seq, a.layer, 1, g, e, rp.pos), vnew[e]);
    }
    // the new position inside this wave's fragments comes from knew / vnew
    const int off = rp.pos - wp0;
    if (off >= 0 && off < 64) {
      // compile-time fragment indices only (runtime ones would spill the arrays)
      const int kt = 2 * (off / 32) + (off % 8) / 4, kr = 4 * ((off % 32) / 8) + off % 4;  // kpos^-1
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t == kt && r16 == kr) {
#pragma unroll
          for (int s = 0; s < D / 32; ++s) {
            f16x8 k8;
#pragma unroll
            for (int i = 0; i < 8; ++i) k8[i] = (_Float16)knew[32 * s + 8 * j4 + i];
            kf[t][s] = __builtin_bit_cast(u32x4, k8);
          }
        }
      const int e8 = off % 8;
#pragma unroll
      for (int ps = 0; ps < 2; ++ps)
        if (ps == off / 32 && j4 == (off % 32) / 8) {
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            f16x8 v8 = __builtin_bit_cast(f16x8, vf[dt][ps]);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e == e8) v8[e] = (_Float16)vnew[dt * 16 + r16];
            vf[dt][ps] = __builtin_bit_cast(u32x4, v8);
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
      if (wp0 + 32 * (t >> 1) + 8 * j4 + 4 * (t & 1) + v >= c1_col) sc[t][v] = -INFINITY;
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
      u32x4 w = vf[dt][ps];
      if (!vfull) w = vmask(w, wp0 + 32 * ps + 8 * j4, c1);  // past the context: any bits (0 * NaN)
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
  for (int i = tid; i < RG * D; i += THREADS) {
    const int c = i / D, e = i % D;
    const size_t mh = (size_t)(m + c / G) * a.n_heads + g * G + c % G;  // (row, head)
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
    if (nch == 1 && !a.merge) {
      a.out[mh * D + e] = O / L;
    } else {
      float* r = a.part + (mh * a.max_chunks + chunk_id) * rec;
      coh_store(r + 2 + e, O);
      if (e == 0) {
        coh_store(r, M);
        coh_store(r + 1, L);
      }
    }
  }
  if (nch == 1 || a.merge) return;
  if (!last_block_arrive(a.counters + blockIdx.z * a.n_kv + g, nch, &flag)) return;
  // the other workgroups' partials: device-coherent plain loads (batched,
  // unlike atomic loads, which wait for themselves one by one)
  const coh_buf pb = coh_buffer(a.part);
  for (int i = tid; i < RG * nch; i += THREADS) {
    const int h = i % RG, c = i / RG;  // h: column
    const size_t mh = (size_t)(m + h / G) * a.n_heads + g * G + h % G;
    const uint32_t base = (uint32_t)((mh * a.max_chunks + c) * rec);
    ml[0][c][h] = cload(pb, base);
    ml[1][c][h] = cload(pb, base + 1);
  }
  __syncthreads();
  if (tid < RG) {
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
  for (int i = tid; i < RG * D; i += THREADS) {
    const int h = i / D, e = i % D;
    const size_t mh = (size_t)(m + h / G) * a.n_heads + g * G + h % G;
    const uint32_t base = (uint32_t)((mh * a.max_chunks) * rec + 2 + e);
    float O = 0.f;
    int c = 0;
    for (; c + 8 <= nch; c += 8) {
      float o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = cload(pb, base + (uint32_t)((c + u) * rec));
#pragma unroll
      for (int u = 0; u < 8; ++u) O += mw[c + u][h] * o[u];
    }
    for (; c < nch; ++c) O += mw[c][h] * cload(pb, base + (uint32_t)(c * rec));
    a.out[mh * D + e] = O;
  }
}

// Log-sum-exp merge of the chunk partials [M][n_heads][max_chunks][D + 2]
// (max, sum, O[D]); grid (n_heads, M), one thread per channel, the chunks
// taken 16 at a time with a running maximum.  A row uses the chunks that hold
// its own positions (later chunks of its row group hold nothing of it).
template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(AttnDecodeArgs a) {
  constexpr int B = 16;
  const int head = blockIdx.x, m = blockIdx.y, e = threadIdx.x;
  const int nch = (a.rows_param[m].pos + 1 + CHUNK - 1) / CHUNK;
  const int rec = D + 2;
  const float* base = a.part + ((size_t)m * a.n_heads + head) * a.max_chunks * rec;
  float mx = -INFINITY, den = 0.f, O = 0.f;
  for (int c0 = 0; c0 < nch; c0 += B) {
    float w[B], l[B], o[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {  // clamped, all issued before any use
      const int c = min(c0 + u, nch - 1);
      w[u] = base[(size_t)c * rec];
      l[u] = base[(size_t)c * rec + 1];
      o[u] = base[(size_t)c * rec + 2 + e];
    }
    float bm = mx;
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (c0 + u < nch) bm = fmaxf(bm, w[u]);
    const float f0 = (mx == -INFINITY) ? 0.f : exp2f(mx - bm);
    den *= f0;
    O *= f0;
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const float f = (c0 + u >= nch || w[u] == -INFINITY) ? 0.f : exp2f(w[u] - bm);
      den += f * l[u];
      O += f * o[u];
    }
    mx = bm;
  }
  const float y = O / den;
  const size_t oi = ((size_t)m * a.n_heads + head) * D + e;
  if (a.out_hi) {
    uint32_t h16, l16;
    split_bf16(y, h16, l16);
    const size_t xi = xg_index(m, head * D + e);
    a.out_hi[xi] = (uint16_t)h16;
    a.out_lo[xi] = (uint16_t)l16;
  } else {
    a.out[oi] = y;
  }
}

}  // namespace

hipError_t launch_attn_decode_mfma(const AttnDecodeArgs& a, hipStream_t stream) {
  if (a.kv.is_f32 || a.n_heads % a.n_kv || a.n_heads / a.n_kv > 16 || a.max_chunks > MAXCH || a.kv.max_seq % 64)
    return hipErrorInvalidValue;
  const int sh = a.share > 1 ? a.share : 1;
  if (sh > 1 && (a.qkv_raw || sh * (a.n_heads / a.n_kv) > 16)) return hipErrorInvalidValue;
  dim3 grid(a.max_chunks, a.n_kv, (a.M + sh - 1) / sh);
  const bool raw = a.qkv_raw != nullptr;
  if (a.d == 128) {
    if (raw)
      launch(attn_decode_mfma_kernel<128, true>, grid, dim3(THREADS), 0, stream, a);
    else
      launch(attn_decode_mfma_kernel<128, false>, grid, dim3(THREADS), 0, stream, a);
    if (a.merge) launch(attn_merge_kernel<128>, dim3(a.n_heads, a.M), dim3(128), 0, stream, a);
  } else if (a.d == 64) {
    if (raw)
      launch(attn_decode_mfma_kernel<64, true>, grid, dim3(THREADS), 0, stream, a);
    else
      launch(attn_decode_mfma_kernel<64, false>, grid, dim3(THREADS), 0, stream, a);
    if (a.merge) launch(attn_merge_kernel<64>, dim3(a.n_heads, a.M), dim3(64), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dpk
