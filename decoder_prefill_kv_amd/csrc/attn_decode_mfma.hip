// Decode attention on gfx950 matrix cores (fp16 KV cache).
//
// Same contract as attn_decode.hip (rows with their own slot and position,
// grouped-query heads, context split in chunks merged by log-sum-exp), with
// both products on v_mfma_f32_16x16x32_f16 and the G query heads of a KV head
// as the MFMA columns:
//   S   = K Q^T     A = K rows (16 positions x 32 channels, straight from the
//                   cache), B = q (32 channels x 16 columns, G used)
//   O^T = V^T P^T   A = V^T rows (16 channels x 32 positions), B = P^T taken
//                   directly from the S accumulators
// q and p are split into fp16 hi + lo (two MFMAs each), so the only rounding
// is the fp16 cache itself.
//
// Streaming: a workgroup (8 waves) walks a chunk of a.chunk positions in
// steps of 256 (32 per wave) with an online softmax, the next step's cache
// loads in flight while the current one is computed, so the memory system
// stays busy instead of every workgroup loading, then computing, then exiting
// at once.  The host sizes the chunk to give about one workgroup per CU.  The
// chunks' (max, sum, O) records are merged by attn_merge_kernel.
//
// MFMA 16x16x32 lane layout: A lane l holds row l%16, k = 8(l/16)..+7; B lane l
// holds column l%16, the same k; D lane l holds rows 4(l/16)+v, column l%16.
//
// int8 cache (KV8): each position's K and V head vectors are int8 codes with
// one fp32 scale.  The codes enter the MFMAs as the fp16 integers 1152 + q (the
// byte q ^ 0x80 under the high byte 0x64); S starts from -1152 sum_d q_c per
// column and is then multiplied by the key's scale; each value's scale is
// folded into P (P'), and 1152 sum_p P' per column, carried with the online
// rescale, comes off O at the end.
#include "common.h"
#include "kernels.h"

namespace dpk {

namespace {

constexpr int NW = 8;              // waves per workgroup
constexpr int THREADS = 64 * NW;
constexpr int STEP = 32 * NW;      // positions per step (32 per wave)
constexpr int MAXCH = 64;
constexpr float LOG2E = 1.4426950408889634f;

DPK_DEV void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

template <int D, bool RAW, bool KV8>
__global__ __launch_bounds__(THREADS) void attn_decode_mfma_kernel(AttnDecodeArgs a) {
  static_assert(!KV8 || D == 128, "int8 cache: head_dim 128");
  using Frag = typename std::conditional<KV8, u32x2, u32x4>::type;  // 8 cache elements
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
  const int CH = a.chunk;
  const int nch = (ctx + CH - 1) / CH;
  if (chunk_id >= nch) return;
  const int c0 = chunk_id * CH;
  const int c1 = min(ctx, c0 + CH);
  const int nsteps = (c1 - c0 + STEP - 1) / STEP;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform over the wave
  const int r16 = lane & 15, j4 = lane >> 4;
  // end of this lane's column (its row's context) inside the chunk
  const int c1_col = (r16 < RG) ? min(a.rows_param[m + r16 / G].pos + 1, c1) : c1;

  __shared__ float qs[16][D];
  __shared__ __attribute__((aligned(16))) _Float16 qh16[16][D], ql16[16][D];
  __shared__ float knew[D], vnew[D];
  __shared__ float wst[NW][2][16];     // per wave: max, sum per column
  __shared__ float ow[NW][D][16];      // per wave: O^T partial
  __shared__ float qsum[16];           // int8 cache: sum of q hi + lo per column
  __shared__ __attribute__((aligned(16))) int8_t knew8[KV8 ? D : 16], vnew8[KV8 ? D : 16];
  __shared__ float newsc[2];           // int8 cache: scales of the own position's key / value

  // (element pointers: fp16, or int8 codes with per-position scales)
  using Elt = typename std::conditional<KV8, int8_t, _Float16>::type;
  const Elt* Kb = (const Elt*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 0, g);
  const Elt* Vb = (const Elt*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 1, g);
  const float* Ksc = KV8 ? a.kv.scales + kv_scale_slab(a.kv, rp.seq, a.layer, 0, g) : nullptr;
  const float* Vsc = KV8 ? a.kv.scales + kv_scale_slab(a.kv, rp.seq, a.layer, 1, g) : nullptr;
  constexpr bool raw = RAW;  // a.qkv_raw != nullptr
  const bool own = raw && rp.pos >= c0 && rp.pos < c1;

  // ---- this workgroup's inputs other than the cache are loaded before it,
  // so that waiting for them leaves the cache loads in flight (loads complete
  // in issue order).  Not raw: q of the RG columns.  Raw: the row's projected
  // heads that this wave normalises and rotates (query heads wave, wave + NW,
  // ..., then the KV head's key when own), their gains, the rotation of the
  // position and the new value; clamped indices, no branches.
  constexpr int QPT = 16 * D / THREADS;
  constexpr int HD = D / 2;
  constexpr int NIT = (16 + 1 + NW - 1) / NW;  // G + 1 <= 17 heads over NW waves
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
      const int h = min(wave + NW * it, nh - 1);
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

  // ---- cache fragments of one step for this wave, unconditional loads:
  // positions past the context read the last one's address (K rows are masked
  // in S, V groups where they are used).  K tile t row r is position
  // 8 (r / 4) + 4 t + r % 4 of the wave's 32, so the S accumulators give lane
  // group j4 positions 8 j4 .. + 7 (its k range of P^T in the P V product)
  // and V^T is read as one 8-position (16-byte) group per lane; an 8-position
  // group stays inside the slab row (max_seq % 64 == 0).
  // int8 cache: the scales of the lane's 8 positions sp + 8 j4 .. + 7 (the
  // same group as its V fragment; a group past the context reads the last
  // whole group's, and those positions are masked)
  auto load = [&](Frag (&kf)[2][D / 32], Frag (&vf)[D / 16], f32x4 (&sc8)[4], int s) {
    const int sp = c0 + s * STEP + 32 * wave;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int p = min(sp + 8 * (r16 >> 2) + 4 * t + (r16 & 3), c1 - 1);
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) kf[t][ks] = *(const Frag*)(Kb + (size_t)p * D + 32 * ks + 8 * j4);
    }
    const int p8 = min(sp + 8 * j4, (c1 - 1) & ~7);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) vf[dt] = *(const Frag*)(Vb + (size_t)(dt * 16 + r16) * a.kv.max_seq + p8);
    if constexpr (KV8) {
      sc8[0] = *(const f32x4*)(Ksc + p8);
      sc8[1] = *(const f32x4*)(Ksc + p8 + 4);
      sc8[2] = *(const f32x4*)(Vsc + p8);
      sc8[3] = *(const f32x4*)(Vsc + p8 + 4);
    }
  };
  Frag kA[2][D / 32], vA[D / 16], kB[2][D / 32], vB[D / 16];
  f32x4 sA[4], sB[4];
  load(kA, vA, sA, 0);
  if (nsteps > 1) load(kB, vB, sB, 1);

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
      const int h = wave + NW * it;
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
    if constexpr (KV8) {  // wave 0: codes and scales of the new key and value, to the cache and LDS
      if (wave == 0) {
        float q0, q1;
        float sk = kv_quant_i8(knew[lane], knew[lane + 64], q0, q1);
        knew8[lane] = (int8_t)q0;
        knew8[lane + 64] = (int8_t)q1;
        int8_t* kb = (int8_t*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 0, g) + (size_t)rp.pos * D;
        kb[lane] = (int8_t)q0;
        kb[lane + 64] = (int8_t)q1;
        const float sv = kv_quant_i8(vnew[lane], vnew[lane + 64], q0, q1);
        vnew8[lane] = (int8_t)q0;
        vnew8[lane + 64] = (int8_t)q1;
        int8_t* vb = (int8_t*)a.kv.base + kv_slab(a.kv, rp.seq, a.layer, 1, g);
        vb[(size_t)lane * a.kv.max_seq + rp.pos] = (int8_t)q0;
        vb[(size_t)(lane + 64) * a.kv.max_seq + rp.pos] = (int8_t)q1;
        if (lane == 0) {
          newsc[0] = sk;
          newsc[1] = sv;
          a.kv.scales[kv_scale_slab(a.kv, rp.seq, a.layer, 0, g) + rp.pos] = sk;
          a.kv.scales[kv_scale_slab(a.kv, rp.seq, a.layer, 1, g) + rp.pos] = sv;
        }
      }
    } else {
      for (int e = tid; e < D; e += THREADS) {
        kv_store(a.kv, kv_offset(a.kv, rp.seq, a.layer, 0, g, e, rp.pos), knew[e]);
        kv_store(a.kv, kv_offset(a.kv, rp.seq, a.layer, 1, g, e, rp.pos), vnew[e]);
      }
    }
  }

  // q as fp16 hi + lo, kept in LDS (the B fragments are re-read every step:
  // registers are what the two steps of cache fragments in flight need)
  for (int i = tid; i < 16 * D; i += THREADS) {
    _Float16 h, l;
    split_f16((&qs[0][0])[i], h, l);
    (&qh16[0][0])[i] = h;
    (&ql16[0][0])[i] = l;
  }
  lds_barrier();
  if constexpr (KV8) {  // per column, the sum of the q parts the MFMAs multiply (waves 0 .. 7: columns 2w, 2w + 1)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int col = 2 * wave + cc;
      float qs2 = (float)qh16[col][lane] + (float)ql16[col][lane] + (float)qh16[col][lane + 64] +
                  (float)ql16[col][lane + 64];
      qs2 = wave_sum(qs2);
      if (lane == 0) qsum[col] = qs2;
    }
    lds_barrier();
  }
  const float cq = KV8 ? -1152.0f * qsum[r16] : 0.f;  // the S accumulator's start (int8 cache)
  float corr = 0.f;  // int8 cache: 1152 sum_p P' of the lane's column, online-rescaled

  // ---- the steps, online softmax per column (log2 domain)
  float mrun = -INFINITY, lrun = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](Frag (&kf)[2][D / 32], Frag (&vf)[D / 16], f32x4 (&sc8)[4], int s) {
    const int sp = c0 + s * STEP + 32 * wave;
    float sk[8], sv[8];  // int8 cache: scales of the lane's positions sp + 8 j4 + i (values past the context: 0)
    if constexpr (KV8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sk[i] = sc8[i >> 2][i & 3];
        sv[i] = (sp + 8 * j4 + i < c1) ? sc8[2 + (i >> 2)][i & 3] : 0.f;
      }
    }
    if constexpr (KV8) {  // int8 cache: the new position's codes and scales come from LDS
      const int off = rp.pos - sp;
      if (own && off >= 0 && off < 32) {
        const int kt = (off % 8) / 4, kr = 4 * (off / 8) + off % 4;
#pragma unroll
        for (int t = 0; t < 2; ++t)
          if (t == kt && r16 == kr) {
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) kf[t][ks] = *(const Frag*)&knew8[32 * ks + 8 * j4];
          }
        const int e8 = off % 8;
        if (j4 == off / 8) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (i == e8) {
              sk[i] = newsc[0];
              sv[i] = newsc[1];
            }
          const uint32_t sh = 8u * (e8 & 3), keep = ~(0xFFu << sh);
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            const uint32_t b = (uint32_t)(uint8_t)vnew8[dt * 16 + r16] << sh;
            if (e8 < 4)
              vf[dt].x = (vf[dt].x & keep) | b;
            else
              vf[dt].y = (vf[dt].y & keep) | b;
          }
        }
      }
    } else {  // the new position inside this wave's fragments comes from knew / vnew
      const int off = rp.pos - sp;
      if (own && off >= 0 && off < 32) {
        // compile-time fragment indices only (runtime ones would spill the arrays)
        const int kt = (off % 8) / 4, kr = 4 * (off / 8) + off % 4;
#pragma unroll
        for (int t = 0; t < 2; ++t)
          if (t == kt && r16 == kr) {
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
              f16x8 k8;
#pragma unroll
              for (int i = 0; i < 8; ++i) k8[i] = (_Float16)knew[32 * ks + 8 * j4 + i];
              kf[t][ks] = __builtin_bit_cast(u32x4, k8);
            }
          }
        const int e8 = off % 8;
        if (j4 == off / 8) {
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            f16x8 v8 = __builtin_bit_cast(f16x8, vf[dt]);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e == e8) v8[e] = (_Float16)vnew[dt * 16 + r16];
            vf[dt] = __builtin_bit_cast(u32x4, v8);
          }
        }
      }
    }
    f32x4 sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sc[t] = f32x4{cq, cq, cq, cq};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        f16x8 A;
        if constexpr (KV8)
          A = __builtin_bit_cast(f16x8, kv_codes_f16(kf[t][ks]));
        else
          A = __builtin_bit_cast(f16x8, kf[t][ks]);
        const f16x8 qh = *(const f16x8*)&qh16[r16][32 * ks + 8 * j4];
        const f16x8 ql = *(const f16x8*)&ql16[r16][32 * ks + 8 * j4];
        sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qh, sc[t], 0, 0, 0);
        sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ql, sc[t], 0, 0, 0);
      }
      if constexpr (KV8) {  // the keys' scales (lane rows 4 j4 + v of tile t: positions 8 j4 + 4 t + v)
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[t][v] *= sk[4 * t + v];
      }
    }
    // mask (positions sp + 8 j4 + 4 t + v past the column's context), step max
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (sp + 8 * j4 + 4 * t + v >= c1_col) sc[t][v] = -INFINITY;
        mx = fmaxf(mx, sc[t][v]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(mrun, mx);
    const float alpha = (mrun == -INFINITY) ? 0.f : exp2f(mrun - mnew);
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float e = (sc[t][v] == -INFINITY) ? 0.f : exp2f(sc[t][v] - mnew);
        sc[t][v] = e;
        sum += e;
      }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    lrun = lrun * alpha + sum;
    mrun = mnew;
    if constexpr (KV8) {  // P' = P times the value's scale
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[t][v] *= sv[4 * t + v];
    }
    // O^T = alpha O^T + V^T P^T (k slots 0..3 from tile 0, 4..7 from tile 1)
    f16x8 ph, pl;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      _Float16 h0, l0, h1, l1;
      split_f16(sc[0][v], h0, l0);
      split_f16(sc[1][v], h1, l1);
      ph[v] = h0;
      pl[v] = l0;
      ph[4 + v] = h1;
      pl[4 + v] = l1;
    }
    if constexpr (KV8) {  // 1152 sum_p P' of the column (the parts the MFMAs take)
      float cs = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) cs += (float)ph[i] + (float)pl[i];
      cs += __shfl_xor(cs, 16, 64);
      cs += __shfl_xor(cs, 32, 64);
      corr = corr * alpha + 1152.0f * cs;
    }
    // V positions past the context may hold any bits (0 * NaN): masked with
    // ANDs (no branch, so the wait counts stay exact); int8 codes are always
    // finite as fp16 and meet P' = 0 there
    const int nv = c1 - sp - 8 * j4;
    auto mk = [nv](int e) { return nv >= e + 2 ? 0xffffffffu : (nv == e + 1 ? 0x0000ffffu : 0u); };
    const u32x4 vm = {mk(0), mk(2), mk(4), mk(6)};
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      u32x4 w;
      if constexpr (KV8)
        w = kv_codes_f16(vf[dt]);
      else
        w = vf[dt] & vm;
      const f16x8 A = __builtin_bit_cast(f16x8, w);
#pragma unroll
      for (int v = 0; v < 4; ++v) o[dt][v] *= alpha;
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ph, o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pl, o[dt], 0, 0, 0);
    }
  };
  for (int s = 0; s < nsteps; s += 2) {
    step(kA, vA, sA, s);
    if (s + 2 < nsteps) load(kA, vA, sA, s + 2);
    if (s + 1 < nsteps) {
      step(kB, vB, sB, s + 1);
      if (s + 3 < nsteps) load(kB, vB, sB, s + 3);
    }
  }
  if constexpr (KV8) {  // the code offset of the values (lane: column r16 of every O^T tile)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[dt][v] -= corr;
  }

  // ---- combine the waves (per column = query head)
  if (j4 == 0) {
    wst[wave][0][r16] = mrun;
    wst[wave][1][r16] = lrun;
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
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wst[w][0][c]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = (wst[w][0][c] == -INFINITY) ? 0.f : exp2f(wst[w][0][c] - M);
      L += f * wst[w][1][c];
      O += f * ow[w][e][c];
    }
    if (!a.merge) {  // one chunk: the result
      a.out[mh * D + e] = O / L;
    } else {
      float* r = a.part + (mh * a.max_chunks + chunk_id) * rec;
      r[2 + e] = O;
      if (e == 0) {
        r[0] = M;
        r[1] = L;
      }
    }
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
  const int nch = (a.rows_param[m].pos + 1 + a.chunk - 1) / a.chunk;
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

int attn_decode_mfma_chunk(int max_ctx, int units, int n_cu) {
  // about one workgroup per CU: chunks per (row group, KV head) unit
  const int per = units >= n_cu ? 1 : n_cu / units;
  int ch = (max_ctx + per - 1) / per;
  ch = (ch + STEP - 1) / STEP * STEP;
  while ((max_ctx + ch - 1) / ch > MAXCH) ch += STEP;
  return ch;
}

hipError_t launch_attn_decode_mfma(const AttnDecodeArgs& a, hipStream_t stream) {
  if (a.kv.is_f32 || (a.kv.i8 && a.d != 128) || a.n_heads % a.n_kv || a.n_heads / a.n_kv > 16 ||
      a.max_chunks > MAXCH || a.kv.max_seq % 64 ||
      a.chunk < STEP || a.chunk % STEP || (a.max_chunks > 1 && !a.merge))
    return hipErrorInvalidValue;
  const int sh = a.share > 1 ? a.share : 1;
  if (sh > 1 && (a.qkv_raw || sh * (a.n_heads / a.n_kv) > 16)) return hipErrorInvalidValue;
  dim3 grid(a.max_chunks, a.n_kv, (a.M + sh - 1) / sh);
  const bool raw = a.qkv_raw != nullptr;
  if (a.d == 128 && a.kv.i8) {
    if (raw)
      launch(attn_decode_mfma_kernel<128, true, true>, grid, dim3(THREADS), 0, stream, a);
    else
      launch(attn_decode_mfma_kernel<128, false, true>, grid, dim3(THREADS), 0, stream, a);
    if (a.merge) launch(attn_merge_kernel<128>, dim3(a.n_heads, a.M), dim3(128), 0, stream, a);
  } else if (a.d == 128) {
    if (raw)
      launch(attn_decode_mfma_kernel<128, true, false>, grid, dim3(THREADS), 0, stream, a);
    else
      launch(attn_decode_mfma_kernel<128, false, false>, grid, dim3(THREADS), 0, stream, a);
    if (a.merge) launch(attn_merge_kernel<128>, dim3(a.n_heads, a.M), dim3(128), 0, stream, a);
  } else if (a.d == 64) {
    if (raw)
      launch(attn_decode_mfma_kernel<64, true, false>, grid, dim3(THREADS), 0, stream, a);
    else
      launch(attn_decode_mfma_kernel<64, false, false>, grid, dim3(THREADS), 0, stream, a);
    if (a.merge) launch(attn_merge_kernel<64>, dim3(a.n_heads, a.M), dim3(64), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dpk
