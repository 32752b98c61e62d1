// Weight-streaming GEMV body for decode steps (few activation rows, the whole
// K in one workgroup), gfx950 matrix cores.
//
//   y[m][n] = sum_k W[n][k] * x'[m][k],   x'[m][k] = x[m][k] * rs[m] * g[k]
//
// A decode step reads every weight once (oxinfer docs, "Performance"), so
// this is an HBM stream.  W is the A operand of v_mfma_f32_16x16x32_bf16
// straight from memory, x' the B operand from LDS, split into bf16 hi + lo so
// that the activations keep fp32 precision.  4-bit MLX weights (w = s*c + b per
// 64 inputs; oxinfer docs, "MLX checkpoints") become the exact bf16 value
// 128 + c in registers and are rescaled per group:
//   sum_k w x = s * sum (128 + c) x + (b - 128 s) * sum x.
//
// Weights are read from a copy re-tiled at load time into MFMA fragment order
// (one 1 KB block = the A operand of one 16-row x 32-column step, lane order),
// so every wave reads one contiguous stream.  A workgroup stages x' once and
// then walks its row tiles; its waves split K and are summed through LDS, and
// the next tile's first weights are already loading while the current tile's
// epilogue runs.  No partial sums leave a workgroup; the only grid-wide step
// is the lm_head's argmax.  The RMSNorm scale of the input rows is rebuilt in
// the prologue from per-tile sums of squares written by the producer.
//
// Used by gemv.hip (one launch per GEMV) and decode_step.hip (all GEMVs of a
// decode step inside one persistent launch).
#pragma once

#include "common.h"
#include "kernels.h"

namespace dpk {
namespace gemv_detail {

// p as a global-memory pointer.  Arguments that a persistent caller stages in
// LDS hold their pointers as plain values the compiler cannot trace to global
// memory; without this it would use flat accesses, which also count against
// the LDS wait counter.
template <typename T>
DPK_DEV __attribute__((address_space(1))) T* gmem(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

__host__ __device__ inline int gemv_lds_layout(int M, int K, int RB, int fmt, int WAVES, int* xs_off,
                                                int* xsum_off, int* red_off, int* misc_off) {
  const int kq = K / WAVES, xstride = kq + 8;
  int off = 0;
  *xs_off = off;  // per wave: hi and lo of M rows x K/WAVES (+8 pad) bf16
  off += WAVES * 2 * M * xstride * 2;
  off = (off + 15) & ~15;
  *xsum_off = off;
  off += (fmt == W_Q4 ? M * (K / 64) * 4 : fmt == W_Q40 ? M * (K / 32) * 4 : 0);
  off = (off + 15) & ~15;
  *red_off = off;
  off += WAVES * M * RB * 4;
  *misc_off = off;
  off += (64 + 16 * WAVES) * 4;
  return off;
}

// One GEMV of M rows over all of a's row tiles (a.M is not read), run by
// workgroup wg of nwg (tiles wg, wg + nwg, ...).  pre(issue) runs once per
// workgroup before x is read and must call issue() once, which starts the
// first tile's weight loads (they do not depend on x): a persistent caller
// waits there for the producer of x and lets the loads fly during the wait; a
// plain launch just calls issue().  COH: x, the norm sums and the outputs are
// accessed with device-coherent loads / stores, for a producer or consumer in
// the same launch.  Barriers inside are LDS-only (lds_barrier), so weight
// loads in flight are never drained by them.
//
// XG: the activations come ready-made from global memory as bf16 hi / lo
// rows (a.xb_hi / a.xb_lo in the xg_index layout, norm gain already applied)
// instead of being staged in LDS, so M is not limited by LDS (bf16 weights).
// KI: columns a wave reduces per iteration (0: the default for T; 128 lets
// eight waves split rows of 1024, 2048, 3072 ... columns).
//
// PF (bf16): the first tile's third iteration of weights is loaded straight
// into LDS (pf + wave * T * U KB, this wave's slot) together with its first
// two, so three iterations are in flight while the caller waits at its
// barrier; the loop reads that iteration from LDS.  pf_ready: the caller has
// already loaded it (gemv_pf_first).
// ACC (COH): a.xacc / a.racc may be set (the persistent step's fixed-point O
// sums); without it they are ignored.
// 16-row tile index (inside its segment, seg) of 16-row tile t of row tile
// `tile` (RB = 16 T rows)
template <int T>
DPK_DEV size_t gemv_tile_rt(const GemvArgs& a, int tile, int t, int& seg) {
  constexpr int RB = 16 * T;
  int rt;
  if (a.swiglu) {  // RB/2 gate rows then RB/2 up rows, both at rows tile * RB/2
    seg = t / (T / 2 > 0 ? T / 2 : 1);
    rt = tile * (T / 2) + t % (T / 2 > 0 ? T / 2 : 1);
  } else {
    const int n = tile * RB + t * 16;
    seg = 0;
    int base = 0;
    while (seg < 2 && n >= a.seg_end[seg]) { base = a.seg_end[seg]; ++seg; }
    rt = (n - base) / 16;
  }
  return (size_t)rt;
}

// (bf16, staged x) k-steps of 32 columns a wave reduces per iteration
template <int T, int KI>
constexpr int gemv_bf16_u() {
  return KI ? KI / 32 : 8 / T;
}

// The LDS-prefetched iteration of workgroup wg's first row tile -- what
// gemv_body (PF) loads when its barrier is passed -- issued earlier by a
// persistent caller whose prefetch slots are free sooner; gemv_body is then
// called with pf_ready.  Returns whether anything was issued.
template <int T, int WAVES, int KI>
DPK_DEV bool gemv_pf_first(const GemvArgs& a, int wg, unsigned char* pf) {
  constexpr int U = gemv_bf16_u<T, KI>();
  const int K = a.K, KF = a.kfull ? a.kfull : K, KO = a.kofs;
  const int kq = K / WAVES, nit = kq / (32 * U);
  const int rows = a.swiglu ? 2 * a.N : a.N;
  if (wg >= rows / (16 * T) || nit <= 2) return false;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  unsigned char* const slot = pf + (size_t)wave * (T * U * 1024);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    int seg;
    const size_t rt = gemv_tile_rt<T>(a, wg, t, seg);
    const unsigned char* wp =
        (const unsigned char*)a.w[seg] + (rt * (KF / 32) + (KO + wave * kq) / 32) * 1024 + lane * 16;
#pragma unroll
    for (int u = 0; u < U; ++u)
      __builtin_amdgcn_global_load_lds(gmem((const void*)(wp + (size_t)(2 * U + u) * 1024)),
                                       (__attribute__((address_space(3))) void*)(slot + (t * U + u) * 1024), 16, 0,
                                       2 /* nt */);
  }
  return true;
}

template <int FMT, int T, int WAVES, bool COH, bool XG = false, int KI = 0, bool PF = false, bool ACC = false,
          typename Pre>
DPK_DEV void gemv_body(const GemvArgs& a, const int M, unsigned char* lds, const int wg, const int nwg, Pre&& pre,
                       unsigned char* pf = nullptr, bool pf_ready = false) {
  static_assert(!PF || (FMT == W_BF16 && !XG), "LDS prefetch is for staged-x bf16 GEMVs");
  static_assert(!XG || FMT == W_BF16, "ready-made activations are for bf16 weights");
  static_assert((FMT != W_Q40 && FMT != W_Q8) || KI == 0, "Q4_0 / Q8: whole blocks per iteration");
  constexpr int RB = 16 * T;
  constexpr int THREADS = 64 * WAVES;
  const int K = a.K;                      // columns this call reduces over
  const int KF = a.kfull ? a.kfull : K;   // full row length (layout stride, norm mean)
  const int KO = a.kofs;                  // first column of this call
  const int kq = K / WAVES, xstride = kq + 8, ng = K / 64;
  int xs_off, xsum_off, red_off, misc_off;
  if constexpr (XG) {  // no staged x: red and misc only
    xs_off = xsum_off = red_off = 0;
    misc_off = WAVES * M * RB * 4;
  } else {
    gemv_lds_layout(M, K, RB, FMT, WAVES, &xs_off, &xsum_off, &red_off, &misc_off);
  }
  const int tid = COH ? opaque_tid() : (int)threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint16_t* xs_hi = (uint16_t*)(lds + xs_off) + (size_t)wave * 2 * M * xstride;
  uint16_t* xs_lo = xs_hi + M * xstride;
  float* xsum = (float*)(lds + xsum_off);
  float* red = (float*)(lds + red_off);
  float* misc = (float*)(lds + misc_off);
  const int k0 = wave * kq;
  const int r16 = lane & 15, j4 = lane >> 4;
  const bool col_on = r16 < M;
  const int rows = a.swiglu ? 2 * a.N : a.N;
  const int n_tiles = rows / RB;

  auto tile_rt = [&](int tile, int t, int& seg) -> size_t { return gemv_tile_rt<T>(a, tile, t, seg); };

  // bf16: k-steps of 32 per iteration (XG holds its activations in registers
  // as well: a one-tile XG wave loads half as much per iteration, a two-tile
  // one a quarter -- measured faster for the 16-row QKV and lm_head GEMVs, and
  // it leaves the 8-wave variant without register spills)
  constexpr int U = (XG && T == 1 && !KI) ? 4 : (XG && T == 2 && !KI) ? 2 : gemv_bf16_u<T, KI>();
  // 4-bit: groups of 64 per iteration; int8 on eight waves: blocks of 64
  // columns, twice the 4-bit count (the same bytes per iteration)
  constexpr int GU = KI ? KI / 64 : (FMT == W_I8 && WAVES == 8) ? 8 / T : 4 / T > 0 ? 4 / T : 1;
  static_assert(KI % 64 == 0, "whole 4-bit groups per iteration");
  // Q4_0: QH halves of 128 columns (4 blocks of 32 each) per tile and
  // iteration, 4 KB of codes per wave and iteration
  constexpr int QH = 4 / T > 0 ? 4 / T : 1;
  // Q8: NG8 groups of 64 columns (2 blocks of 32 each) per tile and iteration,
  // 4 KB of codes per wave and iteration
  constexpr int NG8 = 4 / T > 0 ? 4 / T : 1;
  const int nit = (FMT == W_BF16) ? kq / (32 * U)
                  : (FMT == W_Q40) ? kq / (128 * QH)
                  : (FMT == W_Q8)  ? kq / (64 * NG8)
                                   : kq / (64 * GU);
  const unsigned char* wp[T];   // this wave's stream inside each 16-row tile
  const unsigned char* sbp[T];  // 4-bit: scale/bias stream; int8: the tile's row scales (bf16)
  uint32_t rsc[T][2];           // int8: bf16 scales of rows 4 j4 .. 4 j4 + 3 of each tile
  auto set_tile = [&](int tile) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      int seg;
      const size_t rt = tile_rt(tile, t, seg);
      if (FMT == W_BF16) {
        // block (rt, s) at ((rt * K/32) + s) * 1024; this wave starts at s = k0/32
        wp[t] = (const unsigned char*)a.w[seg] + (rt * (KF / 32) + (KO + k0) / 32) * 1024 + lane * 16;
      } else if (FMT == W_I8) {
        // int8 codes block (rt, g) (16 rows x 64 columns) at ((rt * K/64) + g) * 1024,
        // lane l's 16 bytes: MFMA k-steps 2g and 2g + 1 of row l % 16
        wp[t] = (const unsigned char*)a.w[seg] + (rt * (KF / 64) + (KO + k0) / 64) * 1024 + lane * 16;
        sbp[t] = (const unsigned char*)a.sb[seg] + (rt * 16 + 4 * j4) * 2;
      } else if (FMT == W_Q8) {
        // Q8 codes: block (rt, g) (16 rows x 64 columns) at ((rt * K/64) + g) * 1024, lane
        // l's 16 bytes: codes 32 h + 8 (l / 16) .. + 7 of row l % 16 (h = 0, 1); the blocks'
        // fp32 scales as for Q4_0 (row r's 8 of 256 columns at 32 r of the chunk's 512 bytes)
        wp[t] = (const unsigned char*)a.w[seg] + (rt * (KF / 64) + (KO + k0) / 64) * 1024 + lane * 16;
        sbp[t] = (const unsigned char*)a.sb[seg] + ((rt * (KF / 256) + (KO + k0) / 256) * 16 + r16) * 32;
      } else if (FMT == W_Q40) {
        // Q4_0 codes of chunk (rt, c) (16 rows x 256 columns) at ((rt * K/256) + c) * 2048,
        // lane l's 16 bytes at l * 16 of each 1 KB half (blocks 0-3, then 4-7); the
        // blocks' scales (fp16) of row r at ((rt * K/256 + c) * 16 + r) * 16
        const size_t ch = rt * (KF / 256) + (KO + k0) / 256;
        wp[t] = (const unsigned char*)a.w[seg] + ch * 2048 + lane * 16;
        sbp[t] = (const unsigned char*)a.sb[seg] + (ch * 16 + r16) * 16;
      } else {
        // codes block (rt, g) at ((rt * K/64) + g) * 512; scales (rt, g) at * 64
        wp[t] = (const unsigned char*)a.w[seg] + (rt * (KF / 64) + (KO + k0) / 64) * 512 + lane * 8;
        sbp[t] = (const unsigned char*)a.sb[seg] + (rt * (KF / 64) + (KO + k0) / 64) * 64 + j4 * 16;
      }
    }
  };
  u32x4 b0[T][U], b1[T][U];
  u32x2 c0[T][GU], c1[T][GU];
  u32x4 s0[T][GU], s1[T][GU];
  u32x4 qc0[T][QH], qc1[T][QH];      // Q4_0: the halves' codes (4 blocks each)
  u32x2 qs0[T][QH], qs1[T][QH];      //   and lane row r16's 4 block scales of each (fp16)
  u32x4 g8c0[T][NG8], g8c1[T][NG8];  // Q8: the groups' codes (2 blocks each)
  u32x2 g8s0[T][NG8], g8s1[T][NG8];  //   and lane row r16's 2 block scales of each (fp32 bits)
  // XG: each iteration's activation fragments are loaded with its weights, so
  // one wait covers both and the next iteration's loads stay in flight.  Rows
  // past M read row M - 1 (their results are never stored).
  constexpr int UX = XG ? U : 1;
  u32x4 xh0[UX], xl0[UX], xh1[UX], xl1[UX];
  size_t xrow = 0;
  if constexpr (XG) xrow = xg_index(a.xrow0 + (r16 < M ? r16 : M - 1), KO + k0 + 8 * j4);
  auto load_bf = [&](u32x4 (&b)[T][U], u32x4 (&xh)[UX], u32x4 (&xl)[UX], int it) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int u = 0; u < U; ++u)
        b[t][u] = __builtin_nontemporal_load(gmem((const u32x4*)(wp[t] + (size_t)(it * U + u) * 1024)));
    if constexpr (XG) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        xh[u] = *(const u32x4*)(a.xb_hi + xrow + ((size_t)(it * U + u) << 9));  // next 32-column block
        xl[u] = *(const u32x4*)(a.xb_lo + xrow + ((size_t)(it * U + u) << 9));
      }
    }
  };
  // int8: GU blocks of 64 columns per iteration, into the u32x4 buffers
  auto load_i8 = [&](u32x4 (&q)[T][GU], int it) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int u = 0; u < GU; ++u)
        q[t][u] = __builtin_nontemporal_load(gmem((const u32x4*)(wp[t] + (size_t)(it * GU + u) * 1024)));
  };
  // (half gh of the wave's part: chunk gh / 2, 1 KB half gh % 2 of its codes,
  // 8 bytes of the row's scales)
  auto load_q40 = [&](u32x4 (&q)[T][QH], u32x2 (&z)[T][QH], int it) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int h = 0; h < QH; ++h) {
        const int gh = it * QH + h;
        q[t][h] = __builtin_nontemporal_load(gmem((const u32x4*)(wp[t] + (size_t)(gh >> 1) * 2048 + (gh & 1) * 1024)));
        z[t][h] = __builtin_nontemporal_load(gmem((const u32x2*)(sbp[t] + (size_t)(gh >> 1) * 256 + (gh & 1) * 8)));
      }
  };
  // (group gg of the wave's part: codes at gg KB, scales of chunk gg / 4 at 8 (gg % 4))
  auto load_q8 = [&](u32x4 (&q)[T][NG8], u32x2 (&z)[T][NG8], int it) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int u = 0; u < NG8; ++u) {
        const int gg = it * NG8 + u;
        q[t][u] = __builtin_nontemporal_load(gmem((const u32x4*)(wp[t] + (size_t)gg * 1024)));
        z[t][u] = __builtin_nontemporal_load(gmem((const u32x2*)(sbp[t] + (size_t)(gg >> 2) * 512 + (gg & 3) * 8)));
      }
  };
  auto load_q4 = [&](u32x2 (&c)[T][GU], u32x4 (&sv)[T][GU], int it) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        c[t][u] = __builtin_nontemporal_load(gmem((const u32x2*)(wp[t] + (size_t)(it * GU + u) * 512)));
        sv[t][u] = __builtin_nontemporal_load(gmem((const u32x4*)(sbp[t] + (size_t)(it * GU + u) * 64)));
      }
  };

  // ---- first tile's first two iterations of weights, before x is read
  int tile = wg;
  bool two = false;  // iterations 0 and 1 of the current tile are already loading
  bool in_pf = false;  // iteration 2 of the current tile is in this wave's LDS slot
  unsigned char* const pf_slot = PF ? pf + (size_t)__builtin_amdgcn_readfirstlane(wave) * (T * U * 1024) : nullptr;
  auto pf_issue = [&]() {
    if constexpr (PF) {
      if (nit > 2) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int u = 0; u < U; ++u)
            __builtin_amdgcn_global_load_lds(gmem((const void*)(wp[t] + (size_t)(2 * U + u) * 1024)),
                                             (__attribute__((address_space(3))) void*)(pf_slot + (t * U + u) * 1024),
                                             16, 0, 2 /* nt */);
        in_pf = true;
      }
    }
  };
  // residual epilogue: element tid of the tile's h (final before this GEMV
  // starts: only the workgroup that owns a tile writes it) is loaded with the
  // tile's first weights, so the epilogue does not wait for it
  const bool h_early = a.epi == EPI_RESID && M * RB <= THREADS;
  float h_tile = 0.f;
  uint32_t r_lo = 0, r_hi = 0;  // racc word of the same element (COH)
  auto load_h = [&](int t) {
    if (h_early && tid < M * RB) {
      const uint32_t hi = (uint32_t)((tid / RB) * a.ldo + t * RB + tid % RB);
      h_tile = COH ? cload(coh_buffer(a.out), hi) : gmem(a.out)[hi];
      if (COH && ACC && a.racc) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(coh_buffer(a.racc), hi * 8u, 0, CPOL_SC1);
        r_lo = w[0];
        r_hi = w[1];
      }
    }
  };
  auto first_loads = [&]() {
    if constexpr (FMT == W_BF16) {
      load_bf(b0, xh0, xl0, 0);
      if (nit > 1) load_bf(b1, xh1, xl1, 1);
    } else if constexpr (FMT == W_Q40) {
      load_q40(qc0, qs0, 0);
      if (nit > 1) load_q40(qc1, qs1, 1);
    } else if constexpr (FMT == W_Q8) {
      load_q8(g8c0, g8s0, 0);
      if (nit > 1) load_q8(g8c1, g8s1, 1);
    } else if constexpr (FMT == W_I8) {
      load_i8(s0, 0);
      if (nit > 1) load_i8(s1, 1);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const u32x2 r = *gmem((const u32x2*)sbp[t]);
        rsc[t][0] = r[0];
        rsc[t][1] = r[1];
      }
    } else {
      load_q4(c0, s0, 0);
      if (nit > 1) load_q4(c1, s1, 1);
    }
    two = true;
  };
  pre([&] {
    if (tile < n_tiles) {
      set_tile(tile);
      first_loads();
      if (pf_ready)  // (gemv_pf_first issued it)
        in_pf = PF && nit > 2;
      else
        pf_issue();
      load_h(tile);
    }
  });
  // no row tile here: nothing to stage or finish (the head's argmax needs
  // every workgroup's candidates, and it has more tiles than workgroups)
  if (tile >= n_tiles && a.epi != EPI_HEAD) return;

  // ---- row norm scales from the producer's per-tile sums of squares (each
  // wave computes them itself, so no barrier separates them from x's loads;
  // XG applies wave 0's copy to the reduced outputs).  own_rs (persistent
  // step, whole rows here): the scale comes from x itself instead -- each
  // wave's part of every row's sum of squares goes to misc and the reduced
  // outputs are scaled -- so x is the only thing this GEMV waits for.
  float* rsw = misc + 64 + 16 * wave;
  const bool own_rs = COH && !XG && a.sq_in && KO == 0 && KF == K;
  if (XG && a.sq_in) {  // rows spread over the waves, one shared copy
    for (int m = wave; m < M; m += WAVES) {
      float s = 0.f;
      for (int b = lane; b < a.sq_nb; b += 64) s += a.sq_in[m * a.sq_nb + b];
      s = wave_sum(s);
      if (lane == 0) misc[64 + m] = rsqrtf(s / (float)KF + a.eps);
    }
  } else if (a.sq_in && !own_rs) {
    for (int m = 0; m < M; ++m) {
      float s = 0.f;
      for (int b = lane; b < a.sq_nb; b += 64)
        s += COH ? cload(coh_buffer(a.sq_in), m * a.sq_nb + b) : a.sq_in[m * a.sq_nb + b];
      s = wave_sum(s);
      if (lane == 0) rsw[m] = rsqrtf(s / (float)KF + a.eps);
    }
  }
  if constexpr (!XG) {
  // ---- prologue: this wave's K part of x' -> bf16 hi/lo (once per workgroup);
  // stage(m, kl) does columns kl .. kl + 7 of row m and returns their sum of
  // squares (before the gain)
  auto stage = [&](const int m, const int kl) -> float {
    const float* xp = a.x + (size_t)m * a.ldx + KO + k0 + kl;
    float v[8];
    if constexpr (COH) {
      const uint32_t xi = (uint32_t)(m * a.ldx + KO + k0 + kl);
      const f32x4 v0 = cload4(coh_buffer(a.x), xi), v1 = cload4(coh_buffer(a.x), xi + 4);
      v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
      v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
      if (ACC && a.xacc) {  // x + the fixed-point sums (8 words = 4 x 16 bytes)
        const coh_buf ab = coh_buffer(a.xacc);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 w = cload16(ab, xi / 2 + q);
          v[2 * q] = v[2 * q] + from_fixed(fixed_word(w[0], w[1]));
          v[2 * q + 1] = v[2 * q + 1] + from_fixed(fixed_word(w[2], w[3]));
        }
      }
    } else {
      const float4 v0 = *(const float4*)xp, v1 = *(const float4*)(xp + 4);
      v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
      v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
    const float r = (a.sq_in && !own_rs) ? rsw[m] : 1.0f;
    if (a.gain) {
      const u32x4 g = *gmem((const u32x4*)(a.gain + KO + k0 + kl));
      const uint32_t gw[4] = {g[0], g[1], g[2], g[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] *= r * bf16lo_to_f32(gw[e]);
        v[2 * e + 1] *= r * bf16hi_to_f32(gw[e]);
      }
    } else if (a.sq_in && !own_rs) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= r;
    }
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // 4-bit codes pair nibble p with p+4 in a dword: slots (0,4,1,5,2,6,3,7)
      const int src = (FMT == W_Q4) ? ((e & 1) ? (e >> 1) + 4 : (e >> 1)) : e;
      split_bf16(v[src], hi[e], lo[e]);
    }
    uint4 H, L;
    H.x = hi[0] | (hi[1] << 16); H.y = hi[2] | (hi[3] << 16); H.z = hi[4] | (hi[5] << 16); H.w = hi[6] | (hi[7] << 16);
    L.x = lo[0] | (lo[1] << 16); L.y = lo[2] | (lo[3] << 16); L.z = lo[4] | (lo[5] << 16); L.w = lo[6] | (lo[7] << 16);
    *(uint4*)(xs_hi + m * xstride + kl) = H;
    *(uint4*)(xs_lo + m * xstride + kl) = L;
    if (FMT == W_Q4) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[e];
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 4, 64);
      if ((kl & 63) == 0) xsum[m * ng + (k0 + kl) / 64] = s;
    } else if (FMT == W_Q40) {
      // per block of 32 (four lanes' 8 columns), the sum of the hi + lo parts
      // the MFMAs multiply, so that the code offset cancels exactly
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += __uint_as_float(hi[e] << 16) + __uint_as_float(lo[e] << 16);
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      if ((kl & 31) == 0) xsum[m * (K / 32) + (k0 + kl) / 32] = s;
    }
    return ss;
  };
  if (own_rs) {  // this wave's part of row m's sum of squares -> misc[64 + m * WAVES + wave]
    for (int m = 0; m < M; ++m) {
      float ss = 0.f;
      for (int j = lane; j < kq / 8; j += 64) ss += stage(m, 8 * j);
      ss = wave_sum(ss);
      if (lane == 0) misc[64 + m * WAVES + wave] = ss;
    }
  } else {
    for (int i = lane; i < M * (kq / 8); i += 64) (void)stage(i / (kq / 8), (i % (kq / 8)) * 8);
  }
  lds_barrier();
  }

  auto compute_bf = [&](f32x4 (&acc)[T], const u32x4 (&b)[T][U], const u32x4 (&xh)[UX], const u32x4 (&xl)[UX],
                        int it) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x4 bh = {0u, 0u, 0u, 0u}, bl = {0u, 0u, 0u, 0u};
      if constexpr (XG) {
        bh = xh[u];
        bl = xl[u];
      } else if (col_on) {
        const int kl = (it * U + u) * 32 + 8 * j4;
        bh = *(const u32x4*)(xs_hi + r16 * xstride + kl);
        bl = *(const u32x4*)(xs_lo + r16 * xstride + kl);
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const bf16x8 A = __builtin_bit_cast(bf16x8, b[t][u]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bh), acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bl), acc[t], 0, 0, 0);
      }
    }
  };
  // 4-bit: lane (row r16, k group j4) holds the codes of 64 g + 16 j4 .. +15;
  // MFMA step t2 uses codes 8 t2 .. 8 t2 + 7.  sv holds (s, b) bf16 pairs of
  // rows 4 j4 .. 4 j4 + 3 of the 16-row tile.
  auto compute_q4 = [&](f32x4 (&acc)[T], const u32x2 (&c)[T][GU], const u32x4 (&sv)[T][GU], int it) {
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int gl = it * GU + u;  // group inside this wave's K part
      f32x4 ag[T];
#pragma unroll
      for (int t = 0; t < T; ++t) ag[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        u32x4 bh = {0u, 0u, 0u, 0u}, bl = {0u, 0u, 0u, 0u};
        const int koff = gl * 64 + 16 * j4 + 8 * t2;
        if (col_on) {
          bh = *(const u32x4*)(xs_hi + r16 * xstride + koff);
          bl = *(const u32x4*)(xs_lo + r16 * xstride + koff);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint32_t w = c[t][u][t2];
          u32x4 av;
          av.x = 0x43004300u | (w & 0x000F000Fu);
          av.y = 0x43004300u | ((w >> 4) & 0x000F000Fu);
          av.z = 0x43004300u | ((w >> 8) & 0x000F000Fu);
          av.w = 0x43004300u | ((w >> 12) & 0x000F000Fu);
          const bf16x8 A = __builtin_bit_cast(bf16x8, av);
          ag[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bh), ag[t], 0, 0, 0);
          ag[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bl), ag[t], 0, 0, 0);
        }
      }
      const float sx = col_on ? xsum[r16 * ng + k0 / 64 + gl] : 0.f;
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t p = sv[t][u][v];  // (s, b) of row 4 j4 + v
          const float s = bf16lo_to_f32(p), b = bf16hi_to_f32(p);
          acc[t][v] += s * ag[t][v] + (b - 128.0f * s) * sx;
        }
    }
  };

  // Q4_0 (blocks of 32 four-bit codes c around 8 with one scale s each:
  // w = s (c - 8)): the activations are the MFMA's A operand and the codes its
  // B operand, so D lane l holds activation rows 4 j4 + v of weight row r16 and
  // takes one block scale.  Lane (r16, j4) of block b holds the codes of
  // columns 32 b + 8 j4 .. + 7 (nibble slots 0-3: even elements, 4-7: odd),
  // which enter as the exact bf16 values 128 + c; the block's MFMAs start
  // from -136 times the sum of the same hi + lo activation parts, so the
  // offset cancels up to the fp32 accumulation, leaving one scale FMA per
  // block (for one activation row, only D row 0 is kept).
  auto compute_q40 = [&](f32x4 (&acc)[T], const u32x4 (&q)[T][QH], const u32x2 (&z)[T][QH], int it) {
#pragma unroll
    for (int hb = 0; hb < 4 * QH; ++hb) {
      const int h = hb >> 2, b = hb & 3;  // block b of half it * QH + h
      u32x4 xh = {0u, 0u, 0u, 0u}, xl = {0u, 0u, 0u, 0u};
      const int kl = (it * QH + h) * 128 + 32 * b + 8 * j4;
      if (col_on) {
        xh = *(const u32x4*)(xs_hi + r16 * xstride + kl);
        xl = *(const u32x4*)(xs_lo + r16 * xstride + kl);
      }
      const bf16x8 Ah = __builtin_bit_cast(bf16x8, xh), Al = __builtin_bit_cast(bf16x8, xl);
      const int xb = (k0 + (it * QH + h) * 128) / 32 + b;  // the block's index in xsum rows
      f32x4 init = {0.f, 0.f, 0.f, 0.f};
      if (M == 1) {
        const float x0 = xsum[xb];
        init[0] = j4 == 0 ? -136.0f * x0 : 0.f;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 4 * j4 + v;
          init[v] = m < M ? -136.0f * xsum[m * (K / 32) + xb] : 0.f;
        }
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t w = q[t][h][b];
        const u32x4 bv = {0x43004300u | (w & 0x000F000Fu), 0x43004300u | ((w >> 4) & 0x000F000Fu),
                          0x43004300u | ((w >> 8) & 0x000F000Fu), 0x43004300u | ((w >> 12) & 0x000F000Fu)};
        const bf16x8 B = __builtin_bit_cast(bf16x8, bv);
        f32x4 ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, B, init, 0, 0, 0);
        ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, B, ag, 0, 0, 0);
        const uint32_t zw = z[t][h][b >> 1];
        const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)((b & 1) ? (zw >> 16) : (zw & 0xFFFFu)));
        if (M == 1) {  // (one activation row: only D row 0 is used)
          acc[t][0] += sc * ag[0];
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[t][v] += sc * ag[v];
        }
      }
    }
  };

  // Q8 (blocks of 32 int8 codes q with one fp32 scale s each: w = s q): the
  // same transposed roles as Q4_0; each lane's 8 codes of a block become exact
  // bf16 values (an integer of at most 8 bits is exact in fp32 and in the
  // upper half of its bits), and one FMA per block applies the scale.
  auto compute_q8 = [&](f32x4 (&acc)[T], const u32x4 (&q)[T][NG8], const u32x2 (&z)[T][NG8], int it) {
#pragma unroll
    for (int u = 0; u < NG8; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 xh = {0u, 0u, 0u, 0u}, xl = {0u, 0u, 0u, 0u};
        const int kl = (it * NG8 + u) * 64 + 32 * h + 8 * j4;
        if (col_on) {
          xh = *(const u32x4*)(xs_hi + r16 * xstride + kl);
          xl = *(const u32x4*)(xs_lo + r16 * xstride + kl);
        }
        const bf16x8 Ah = __builtin_bit_cast(bf16x8, xh), Al = __builtin_bit_cast(bf16x8, xl);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint32_t w0 = h ? q[t][u][2] : q[t][u][0], w1 = h ? q[t][u][3] : q[t][u][1];
          uint32_t f[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            f[e] = __float_as_uint((float)(int)(int8_t)(((e < 4 ? w0 : w1) >> (8 * (e & 3))) & 0xFFu));
          const u32x4 bv = {__builtin_amdgcn_perm(f[1], f[0], 0x07060302u), __builtin_amdgcn_perm(f[3], f[2], 0x07060302u),
                            __builtin_amdgcn_perm(f[5], f[4], 0x07060302u), __builtin_amdgcn_perm(f[7], f[6], 0x07060302u)};
          const bf16x8 B = __builtin_bit_cast(bf16x8, bv);
          f32x4 ag = {0.f, 0.f, 0.f, 0.f};
          ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, B, ag, 0, 0, 0);
          ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, B, ag, 0, 0, 0);
          const float sc = __uint_as_float(z[t][u][h]);
          if (M == 1) {  // (one activation row: only D row 0 is used)
            acc[t][0] += sc * ag[0];
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[t][v] += sc * ag[v];
          }
        }
      }
    }
  };

  // int8: lane (row r16, k group j4) holds codes 32 h + 8 j4 .. + 7 of each
  // 64-column block (h = 0, 1); each becomes the exact bf16 value q (an
  // integer of at most 8 bits is exact in fp32 and in the upper half of its
  // bits), the row scale multiplies the finished tile
  auto compute_i8 = [&](f32x4 (&acc)[T], const u32x4 (&q)[T][GU], int it) {
#pragma unroll
    for (int u = 0; u < GU; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 bh = {0u, 0u, 0u, 0u}, bl = {0u, 0u, 0u, 0u};
        const int kl = (it * GU + u) * 64 + 32 * h + 8 * j4;
        if (col_on) {
          bh = *(const u32x4*)(xs_hi + r16 * xstride + kl);
          bl = *(const u32x4*)(xs_lo + r16 * xstride + kl);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint32_t w0 = h ? q[t][u][2] : q[t][u][0], w1 = h ? q[t][u][3] : q[t][u][1];
          uint32_t f[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            f[e] = __float_as_uint((float)(int)(int8_t)(((e < 4 ? w0 : w1) >> (8 * (e & 3))) & 0xFFu));
          const u32x4 av = {__builtin_amdgcn_perm(f[1], f[0], 0x07060302u), __builtin_amdgcn_perm(f[3], f[2], 0x07060302u),
                            __builtin_amdgcn_perm(f[5], f[4], 0x07060302u), __builtin_amdgcn_perm(f[7], f[6], 0x07060302u)};
          const bf16x8 A = __builtin_bit_cast(bf16x8, av);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bh), acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bl), acc[t], 0, 0, 0);
        }
      }
    }
  };

  const int nb = nwg;
  float best_v[16];
  int best_i[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    best_v[m] = -INFINITY;
    best_i[m] = 0x7fffffff;
  }
  // sum of WAVES consecutive floats of LDS (16-byte aligned)
  auto lds_sum = [&](const float* p) -> float {
    if constexpr (WAVES % 4 == 0) {
      f32x4 s4 = *(const f32x4*)p;
#pragma unroll
      for (int w = 4; w < WAVES; w += 4) s4 += *(const f32x4*)(p + w);
      return (s4[0] + s4[1]) + (s4[2] + s4[3]);
    } else {
      float s1 = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) s1 += p[w];
      return s1;
    }
  };
  auto finish_tile = [&](const int tile, const f32x4 (&acc)[T], const float h_pre, const long long r_pre) {
    // ---- the waves' K parts go to red[(m * RB + r) * WAVES + wave] (D[n][m]
    // lane layout: rows 4 j4 + v, column r16), so one output's parts are
    // adjacent and the thread that sums them finishes that output itself
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if constexpr (FMT == W_Q40 || FMT == W_Q8) {  // (D lane: activation row 4 j4 + v, weight row r16)
          if (4 * j4 + v < M) red[((4 * j4 + v) * RB + t * 16 + r16) * WAVES + wave] = acc[t][v];
        } else if (col_on) {
          red[(r16 * RB + t * 16 + 4 * j4 + v) * WAVES + wave] = acc[t][v];
        }
      }
    lds_barrier();
    auto result = [&](const int i) -> float {
      float v = lds_sum(red + i * WAVES);
      if constexpr (XG) {
        if (a.sq_in) v *= misc[64 + i / RB];  // the row's norm scale
      } else if (own_rs) {
        v *= rsqrtf(lds_sum(misc + 64 + (i / RB) * WAVES) / (float)KF + a.eps);
      }
      return v;
    };

    if (a.epi == EPI_STORE) {
      for (int i = tid; i < M * RB; i += THREADS) {
        const int m = i / RB, n = tile * RB + i % RB;
        const float y = result(i);
        if constexpr (COH)
          cstore(coh_buffer(a.out), (uint32_t)(m * a.ldo + n), y);
        else
          gmem(a.out)[(size_t)m * a.ldo + n] = y;
      }
    } else if (a.epi == EPI_SWIGLU) {
      constexpr int HR = RB / 2;
      for (int i = tid; i < M * HR; i += THREADS) {
        const int m = i / HR, r = i % HR;
        const float y = silu(result(m * RB + r)) * result(m * RB + HR + r);
        if (a.xo_hi) {  // the next GEMV's activations, bf16 hi / lo
          uint32_t h16, l16;
          split_bf16(y, h16, l16);
          const size_t o = xg_index(m, tile * HR + r);
          gmem(a.xo_hi)[o] = (uint16_t)h16;
          gmem(a.xo_lo)[o] = (uint16_t)l16;
        } else if constexpr (COH)
          cstore(coh_buffer(a.out), (uint32_t)(m * a.ldo + tile * HR + r), y);
        else
          gmem(a.out)[(size_t)m * a.ldo + tile * HR + r] = y;
      }
    } else if (a.epi == EPI_RESID) {
      // h += y; the per-row sum of squares of the new h over the tile (the
      // next GEMV's norm) by shuffles: a row's RB outputs are RB adjacent
      // lanes of one wave
      for (int i = tid; i < M * RB; i += THREADS) {
        const int m = i / RB, n = tile * RB + i % RB;
        const uint32_t hi = (uint32_t)(m * a.ldo + n);
        float h0 = h_early ? h_pre : COH ? cload(coh_buffer(a.out), hi) : gmem(a.out)[hi];
        if (COH && ACC && a.racc) {  // h after the O projection, exactly as the gate/up GEMV staged it
          long long r = r_pre;
          if (!h_early) {
            const auto w = __builtin_amdgcn_raw_buffer_load_b64(coh_buffer(a.racc), hi * 8u, 0, CPOL_SC1);
            r = fixed_word(w[0], w[1]);
          }
          h0 = h0 + from_fixed(r);
          cstore8z(coh_buffer(a.racc), hi);
        }
        const float h = h0 + result(i);
        if constexpr (COH)
          cstore(coh_buffer(a.out), hi, h);
        else
          gmem(a.out)[hi] = h;
        if (a.xo_hi) {  // h * gain as the next GEMV's bf16 hi / lo activations
          uint32_t h16, l16;
          split_bf16(a.xo_gain ? h * bf16_to_f32(gmem(a.xo_gain)[n]) : h, h16, l16);
          gmem(a.xo_hi)[xg_index(m, n)] = (uint16_t)h16;
          gmem(a.xo_lo)[xg_index(m, n)] = (uint16_t)l16;
        }
        float sq = h * h;
#pragma unroll
        for (int o = 1; o < RB; o <<= 1) sq += __shfl_xor(sq, o, 64);
        if (i % RB == 0) {
          if constexpr (COH)
            cstore(coh_buffer(a.sq_out), (uint32_t)(m * n_tiles + tile), sq);
          else
            a.sq_out[m * n_tiles + tile] = sq;
        }
      }
    } else if (a.epi == EPI_HEAD) {
      // logits; running (max, lowest index) per row for this workgroup
      for (int i = tid; i < M * RB; i += THREADS) {
        const int m = i / RB, n = tile * RB + i % RB;
        const float v = result(i);
        gmem(a.out)[(size_t)m * a.ldo + n] = v;
#pragma unroll
        for (int mm = 0; mm < 16; ++mm)
          if (mm == m && (v > best_v[mm] || (v == best_v[mm] && n < best_i[mm]))) {
            best_v[mm] = v;
            best_i[mm] = n;
          }
      }
    }
    if (tile + nwg < n_tiles) lds_barrier();  // red is rewritten by the next tile
  };

  for (; tile < n_tiles; tile += nwg) {
    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (FMT == W_BF16) {
      for (int it = 0; it < nit; it += 2) {
        if (it + 1 < nit && !(two && it == 0)) load_bf(b1, xh1, xl1, it + 1);
        compute_bf(acc, b0, xh0, xl0, it);
        if (it + 2 < nit) {
          if (PF && in_pf && it == 0) {
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
              for (int u = 0; u < U; ++u) b0[t][u] = *(const u32x4*)(pf_slot + (t * U + u) * 1024 + lane * 16);
          } else {
            load_bf(b0, xh0, xl0, it + 2);
          }
        }
        if (it + 1 < nit) compute_bf(acc, b1, xh1, xl1, it + 1);
      }
      in_pf = false;
    } else if constexpr (FMT == W_Q40) {
      for (int it = 0; it < nit; it += 2) {
        if (it + 1 < nit && !(two && it == 0)) load_q40(qc1, qs1, it + 1);
        compute_q40(acc, qc0, qs0, it);
        if (it + 2 < nit) load_q40(qc0, qs0, it + 2);
        if (it + 1 < nit) compute_q40(acc, qc1, qs1, it + 1);
      }
    } else if constexpr (FMT == W_Q8) {
      for (int it = 0; it < nit; it += 2) {
        if (it + 1 < nit && !(two && it == 0)) load_q8(g8c1, g8s1, it + 1);
        compute_q8(acc, g8c0, g8s0, it);
        if (it + 2 < nit) load_q8(g8c0, g8s0, it + 2);
        if (it + 1 < nit) compute_q8(acc, g8c1, g8s1, it + 1);
      }
    } else if constexpr (FMT == W_I8) {
      for (int it = 0; it < nit; it += 2) {
        if (it + 1 < nit && !(two && it == 0)) load_i8(s1, it + 1);
        compute_i8(acc, s0, it);
        if (it + 2 < nit) load_i8(s0, it + 2);
        if (it + 1 < nit) compute_i8(acc, s1, it + 1);
      }
      // the tile's row scales (lane rows 4 j4 + v), before the next tile's loads replace them
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] *= (v & 1) ? bf16hi_to_f32(rsc[t][v >> 1]) : bf16lo_to_f32(rsc[t][v >> 1]);
    } else {
      for (int it = 0; it < nit; it += 2) {
        if (it + 1 < nit && !(two && it == 0)) load_q4(c1, s1, it + 1);
        compute_q4(acc, c0, s0, it);
        if (it + 2 < nit) load_q4(c0, s0, it + 2);
        if (it + 1 < nit) compute_q4(acc, c1, s1, it + 1);
      }
    }
    two = false;
    // the next tile's first weights load while this tile is finished
    const int next = tile + nwg;
    const float h_cur = h_tile;
    const long long r_cur = fixed_word(r_lo, r_hi);
    if (next < n_tiles) {
      set_tile(next);
      first_loads();
      load_h(next);
    }
    finish_tile(tile, acc, h_cur, r_cur);
  }

  if (a.epi != EPI_HEAD) return;
  // ---- greedy argmax: per-workgroup candidates, the last workgroup reduces
  int* flag = (int*)(misc + 48);
  for (int m = 0; m < M; ++m) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int mm = 0; mm < 16; ++mm)
      if (mm == m) {
        bv = best_v[mm];
        bi = best_i[mm];
      }
    wave_argmax(bv, bi);
    if (lane == 0) {
      misc[32 + wave] = bv;
      ((int*)misc)[40 + wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < WAVES; ++w) {
        const float v = misc[32 + w];
        const int ix = ((int*)misc)[40 + w];
        if (v > bv || (v == bv && ix < bi)) { bv = v; bi = ix; }
      }
      coh_store(a.cand_val + m * nb + wg, bv);
      coh_store(a.cand_idx + m * nb + wg, bi);
    }
    __syncthreads();
  }
  if (!last_block_arrive(a.counters, nb, flag)) return;
  for (int m = wave; m < M; m += WAVES) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int b0i = 0; b0i < nb; b0i += 512) {
      float v[8];
      int ix[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int b = b0i + lane + 64 * u;
        v[u] = b < nb ? coh_load(a.cand_val + m * nb + b) : -INFINITY;
        ix[u] = b < nb ? coh_load(a.cand_idx + m * nb + b) : 0x7fffffff;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (v[u] > bv || (v[u] == bv && ix[u] < bi)) { bv = v[u]; bi = ix[u]; }
    }
    wave_argmax(bv, bi);
    if (lane == 0 && a.argmax_out) a.argmax_out[m] = bi;
  }
}

}  // namespace gemv_detail
}  // namespace dpk
