// A whole decode step in one persistent launch (gfx950, bf16 or MLX 4-bit
// weights).
//
// The step is the single-token decode order of the Butter architecture notes
// ("SINGLE-TOKEN DECODE": gather, then per layer norm / q,k,v / rope at the
// cache length / cache append / attention / o / add / norm / gate, up /
// silu-mul / down / add, then final norm, lm_head and the greedy token).
// Every weight is read once per step, so the step is an HBM stream; what
// keeps a stream of ~180 dependent kernels from reaching the bandwidth is the
// gap at each kernel boundary, where the next weights only start to load
// after the previous kernel has drained.
//
// Here one workgroup per CU runs all phases in order, separated by grid-wide
// barriers, and each workgroup issues the first weight loads of its next
// phase *before* it waits at the barrier (weights do not depend on the
// activations), so the barrier's latency overlaps the weight stream.  Data
// handed between phases (activations, norm sums, attention records) is
// written and read with device-coherent accesses, which is what makes it
// visible across the XCDs' separate L2 caches inside one launch.
//
// Phases: embedding (h), then per layer the QKV GEMV, attention (with
// QK-norm, RoPE and the KV write), the O GEMV with the residual add, the
// gate/up GEMV with SwiGLU and the down GEMV with the residual add; then the
// lm_head GEMV with the greedy argmax.  The GEMVs are gemv_body.h's (each
// takes its input row's norm scale from the row it stages); attention splits
// the context into 256-position chunks, one per workgroup item (32 positions
// per wave), merged by the last chunk to finish.
//
// LDS: the phases' own scratch from offset 0; after the largest of those, the
// current layer's argument table entry, the lm_head's arguments and the rows'
// parameters (copied in once, so no phase re-reads them from device memory
// while its weight loads are in flight); then, for bf16, each wave's slot for
// the LDS-prefetched weight iteration of the next GEMV.
//
// The launch is cooperative (all workgroups resident), and every barrier wait
// is bounded: a workgroup that waits too long raises an abort flag, after
// which every barrier passes at once and the host sees the error flag.
#include "gemv_body.h"

namespace dpk {

namespace {

constexpr int MT = 512;        // threads per workgroup (8 waves)
constexpr int AW = MT / 64;    // attention: waves per workgroup
constexpr int ACH = 32 * AW;   // attention: positions per workgroup item
constexpr int D = 128;         // head dim
constexpr float LOG2E = 1.4426950408889634f;
constexpr unsigned SPIN_LIMIT = 200000;

// Grid barrier in two levels: workgroup wg counts in on the counter of group
// wg % 8 (its own 256-byte line; with round-robin dispatch that is the
// workgroups of one XCD), the last of a group counts the group in on the top
// counter, and every workgroup polls the top counter.  Counters only grow
// within a launch (phase p completes at p * group size, p * 8).
struct Barrier {
  unsigned* ctr;         // [0] top, [64 * (1 + g)] group g
  unsigned* abort_flag;
  unsigned nwg;
  unsigned phase;
};

// All of the workgroup's stores are complete before it counts in; prefetch()
// (loads of the next phase that do not depend on other workgroups) is issued
// after counting in and before the wait, so those loads fly while the barrier
// completes.  Only wave 0 waits on memory for the barrier itself, and its
// waits also cover its own prefetch loads (vector memory returns in order);
// the other waves leave theirs in flight.
template <typename F>
DPK_DEV void grid_sync(Barrier& b, F&& prefetch) {
  ++b.phase;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
  __syncthreads();
  const unsigned ngrp = b.nwg < 8u ? b.nwg : 8u;
  if (threadIdx.x == 0) {
    const unsigned grp = blockIdx.x & 7u;
    const unsigned gsize = (b.nwg - grp + 7u) / 8u;
    const unsigned prev =
        __hip_atomic_fetch_add(b.ctr + 64 * (1 + grp), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == b.phase * gsize - 1u) __hip_atomic_fetch_add(b.ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  prefetch();
  if (threadIdx.x == 0) {
    const unsigned target = b.phase * ngrp;
    for (unsigned spin = 0;; ++spin) {
      if (__hip_atomic_load(b.ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
      if (__hip_atomic_load(b.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
      if (spin >= SPIN_LIMIT) {
        __hip_atomic_store(b.abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  // execution order only: what other workgroups handed over is read with
  // device-coherent loads issued after this, and a __syncthreads here would
  // make every wave wait for its whole prefetch before it could even issue
  // the loads of its input
  lds_barrier();
}

// After the last barrier: the last workgroup out resets the arrival counters
// (and the attention chunk counters) for the next launch (no workgroup waits
// on them any more) and turns an abort into bit 1 of the error word the host
// reads.
DPK_DEV void grid_exit(Barrier& b, unsigned* exit_ctr, int* err, unsigned* attn_ctr, int n_attn_ctr) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(exit_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == b.nwg - 1) {
      if (__hip_atomic_load(b.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
        atomicOr(err, 2);
        __hip_atomic_store(b.abort_flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      for (int g = 0; g <= 8; ++g) __hip_atomic_store(b.ctr + 64 * g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // (the fused attention's chunk counters grow over the step)
      for (int i = 0; i < n_attn_ctr; ++i)
        __hip_atomic_store(attn_ctr + i * MEGA_CTR_STRIDE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(exit_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// h[m] = E[token m] and its sums of squares per 16-column tile (the first
// layer's norm input, in the same layout the residual epilogues write).
DPK_DEV void embed_phase(const MegaArgs& a, const RowParam* rows, int wg, int nwg) {
  const int tid = threadIdx.x;
  const int ntile = a.H / 16;
  for (int n = wg; n < ntile; n += nwg) {
    if (tid < 16) {
      for (int m = 0; m < a.M; ++m) {
        int tok = a.ids_dev ? a.ids_dev[m] : rows[m].token;
        if (tok < 0 || tok >= a.vocab) {
          if (tid == 0) atomicOr(a.err, 1);
          tok = 0;
        }
        const int col = n * 16 + tid;
        float v;
        if (a.fmt == W_Q4) {  // MLX 4-bit: w = s * c + b per 64 columns
          const uint32_t word = ((const uint32_t*)a.emb)[(size_t)tok * (a.H / 8) + col / 8];
          const size_t gi = (size_t)tok * (a.H / 64) + col / 64;
          v = bf16_to_f32(a.emb_sc[gi]) * (float)((word >> (4 * (col & 7))) & 0xFu) + bf16_to_f32(a.emb_bi[gi]);
        } else if (a.fmt == W_I8) {  // int8 with one bf16 scale per row
          v = bf16_to_f32(a.emb_sc[tok]) * (float)((const int8_t*)a.emb)[(size_t)tok * a.H + col];
        } else if (a.fmt == W_Q8) {  // int8 in blocks of 32 with an fp32 scale each
          v = ((const float*)a.emb_sc)[(size_t)tok * (a.H / 32) + col / 32] *
              (float)((const int8_t*)a.emb)[(size_t)tok * a.H + col];
        } else if (a.fmt == W_Q40) {  // blocks of 32 codes around 8, fp16 scale; byte j: codes j, j + 16
          const int i = col & 31;
          const uint8_t b = ((const uint8_t*)a.emb)[(size_t)tok * (a.H / 2) + (col / 32) * 16 + (i & 15)];
          const int c = i < 16 ? (b & 0xF) : (b >> 4);
          v = (float)__builtin_bit_cast(_Float16, a.emb_sc[(size_t)tok * (a.H / 32) + col / 32]) * (float)(c - 8);
        } else {
          v = bf16_to_f32(((const uint16_t*)a.emb)[(size_t)tok * a.H + col]);
        }
        cstore(coh_buffer(a.h), (uint32_t)(m * a.H + col), v);
        float ss = v * v;
        ss += __shfl_xor(ss, 1, 64);
        ss += __shfl_xor(ss, 2, 64);
        ss += __shfl_xor(ss, 4, 64);
        ss += __shfl_xor(ss, 8, 64);
        if (tid == 0) cstore(coh_buffer(a.sq), (uint32_t)(m * ntile + n), ss);
      }
    }
  }
}

DPK_DEV void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

// Attention of one layer for all rows.  Item = (row m, KV head g, chunk of
// ACH positions); wave w of the item takes positions c0 + 32 w .. + 31.
//   S   = K Q^T   on v_mfma_f32_16x16x32_f16, A = K rows from the cache, B = q
//                 (the G query heads of g are the MFMA columns), q as fp16
//                 hi + lo;
//   O^T = V^T P^T with P^T straight from the S accumulators (hi + lo).
// The waves' softmax statistics are combined in LDS; with more than one chunk
// each chunk writes a record (max, sum, O) and the last chunk of (m, g) to
// finish merges them (log-sum-exp weights).  QK-norm, RoPE and the new
// position's K/V come from the raw QKV projection of the previous phase.
//
// FO (bf16, a.oacc set): the O projection runs in the same phase, split by
// KV head, on the workgroups attention does not use (o_phase).  Every chunk
// writes its record and counts in on the (m, g) counter: there is no merge
// step and no grid barrier after attention.
// The O projection of the fused phase.  Item j = (block j / n_kv of 16 * o_rt
// output rows, KV head g = j % n_kv) multiplies those rows of W_o,
// restricted to g's G * d columns, by g's attention outputs and adds the
// product to a.oacc in fixed point (the n_kv items of a row block are summed
// there, exactly and in any order).  Wave w takes 16-row tile w / WPT of the
// block over k-steps (32 columns) (w % WPT) * KW .. + KW, its weight blocks
// in registers.
//
// The items run on the workgroups that attention does not use: workgroup ow
// of n_ow (a multiple of n_kv) takes items ow, ow + n_ow, ... -- all of KV
// head g = ow % n_kv, so one wait on g's chunk counters and one merge of g's
// records (running maximum, log-sum-exp weights) serve them.  The weights
// of its first two items load when the QKV barrier is passed, while
// attention runs; a further item (a grid of fewer than half as many
// workgroups as items) loads after the two.
struct OItem {
  int RT, WPT, KW, n_o;
};
template <int G>
DPK_DEV OItem o_shape(const MegaArgs& a) {
  OItem o;
  o.RT = a.o_rt;
  o.WPT = 8 / o.RT;
  o.KW = (G * D / 32) / o.WPT;
  o.n_o = (a.H / (16 * o.RT)) * a.n_kv;
  return o;
}
constexpr int O_KWMAX = 16;  // k-steps per wave: G * D / 32 with G <= 4
template <int G>
DPK_DEV void o_load(const MegaArgs& a, const GemvArgs* Lo, const OItem& o, int j, u32x4 (&wr)[O_KWMAX]) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int g = j % a.n_kv;
  const size_t rt = (size_t)(j / a.n_kv) * o.RT + wave / o.WPT;
  const unsigned char* src = (const unsigned char*)Lo->w[0] +
                             (rt * (Lo->K / 32) + g * (G * D / 32) + (wave % o.WPT) * o.KW) * 1024 + lane * 16;
#pragma unroll
  for (int k = 0; k < O_KWMAX; ++k)
    if (k < o.KW) wr[k] = __builtin_nontemporal_load(gemv_detail::gmem((const u32x4*)(src + (size_t)k * 1024)));
}

// This wave's products of up to two items over KW k-steps, x' from LDS (row
// stride xst bf16): with PACK (at most 8 rows) one MFMA takes hi and lo
// together -- B column m is row m's hi part, column m + 8 its lo part, added
// with a lane shuffle; otherwise hi and lo are two MFMAs.  Columns past the
// rows read row M - 1: they are never used (an MFMA column depends on its
// own B column only).
template <int KW, bool PACK, bool TWO>
DPK_DEV void o_products(const u32x4 (&w0)[O_KWMAX], const u32x4 (&w1)[O_KWMAX], const uint16_t* xs_hi,
                        const uint16_t* xs_lo, int xst, int M, int ksw, f32x4& y0, f32x4& y1) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, j4 = lane >> 4;
  const int mrow = min(PACK ? (r16 & 7) : r16, M - 1);
  const uint16_t* xa = ((PACK && r16 >= 8) ? xs_lo : xs_hi) + mrow * xst + ksw * 32 + 8 * j4;
  const uint16_t* xb = xs_lo + mrow * xst + ksw * 32 + 8 * j4;
  f32x4 a0[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}}, a1[2] = {a0[0], a0[0]};
  constexpr int KB = KW < 4 ? KW : 4;  // x fragments read in batches of KB k-steps
#pragma unroll
  for (int k0 = 0; k0 < KW; k0 += KB) {
    u32x4 xh[KB], xl[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      xh[u] = *(const u32x4*)(xa + 32 * (k0 + u));
      if (!PACK) xl[u] = *(const u32x4*)(xb + 32 * (k0 + u));
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int k = k0 + u;
      const bf16x8 H = __builtin_bit_cast(bf16x8, xh[u]);
      a0[k & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w0[k]), H, a0[k & 1], 0, 0, 0);
      if (TWO)
        a1[k & 1] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w1[k]), H, a1[k & 1], 0, 0, 0);
      if (!PACK) {
        const bf16x8 L = __builtin_bit_cast(bf16x8, xl[u]);
        a0[k & 1] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w0[k]), L, a0[k & 1], 0, 0, 0);
        if (TWO)
          a1[k & 1] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w1[k]), L, a1[k & 1], 0, 0, 0);
      }
    }
  }
  y0 = a0[0] + a0[1];
  y1 = a1[0] + a1[1];
  if (PACK) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      y0[v] += __shfl_down(y0[v], 8, 16);
      if (TWO) y1[v] += __shfl_down(y1[v], 8, 16);
    }
  }
}
template <int KW>
DPK_DEV void o_products_kw(bool pack, bool two, const u32x4 (&w0)[O_KWMAX], const u32x4 (&w1)[O_KWMAX],
                           const uint16_t* xs_hi, const uint16_t* xs_lo, int xst, int M, int ksw, f32x4& y0,
                           f32x4& y1) {
  if (pack) {
    if (two) o_products<KW, true, true>(w0, w1, xs_hi, xs_lo, xst, M, ksw, y0, y1);
    else o_products<KW, true, false>(w0, w1, xs_hi, xs_lo, xst, M, ksw, y0, y1);
  } else {
    if (two) o_products<KW, false, true>(w0, w1, xs_hi, xs_lo, xst, M, ksw, y0, y1);
    else o_products<KW, false, false>(w0, w1, xs_hi, xs_lo, xst, M, ksw, y0, y1);
  }
}

//
// Its prefetch slots are free during this phase, so it also loads the
// gate/up GEMV's LDS-prefetched iteration (gemv_pf_first) when the QKV
// barrier is passed; returns whether it did.
template <int G, int KI, typename Sync>
DPK_DEV bool o_phase(const MegaArgs& a, const RowParam* rows, int layer, const GemvArgs* Lo, const GemvArgs* Lgu,
                     unsigned char* lds, unsigned char* pf, const Barrier& bar, int wg, int ow, int n_ow,
                     Sync&& sync) {
  const int tid = opaque_tid(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, j4 = lane >> 4;
  const OItem o = o_shape<G>(a);
  const int g = ow % a.n_kv, rtw = wave / o.WPT, ksw = (wave % o.WPT) * o.KW;
  const int rec = D + 2;
  constexpr int GD = G * D, XST = GD + 8;  // x' row stride (bf16)
  uint16_t* xs_hi = (uint16_t*)lds;        // [M][XST] attention outputs of g, bf16 hi
  uint16_t* xs_lo = xs_hi + a.M * XST;     //   and lo
  float* red = (float*)(lds + ((4 * a.M * XST + 15) & ~15));  // [8 waves][64 lanes][4]

  u32x4 w0[O_KWMAX], w1[O_KWMAX];  // this wave's blocks of items ow and ow + n_ow
  const int j0 = ow, j1 = ow + n_ow;
  bool gu_pf = false;
  sync([&] {  // the QKV projection of every row is complete after this
    if (j0 < o.n_o) o_load<G>(a, Lo, o, j0, w0);
    if (j1 < o.n_o) o_load<G>(a, Lo, o, j1, w1);
    gu_pf = gemv_detail::gemv_pf_first<2, 8, KI>(*Lgu, wg, pf);
  });
  if (j0 >= o.n_o) return gu_pf;  // uniform over the workgroup

  // every row's chunks of g have stored their records
  if (tid == 0) {
    for (int m = 0; m < a.M; ++m) {
      const unsigned target = (unsigned)(layer + 1) * (unsigned)((rows[m].pos + ACH) / ACH);
      for (unsigned spin = 0;; ++spin) {
        if (__hip_atomic_load(a.attn_counters + (m * a.n_kv + g) * MEGA_CTR_STRIDE, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT) >= target)
          break;
        if (__hip_atomic_load(bar.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
        if (spin >= SPIN_LIMIT) {
          __hip_atomic_store(bar.abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  }
  lds_barrier();
  // x'[m][c * D + e] = query head g * G + c of row m, as bf16 hi + lo.  Waves
  // 0 .. 3 take blocks of 64 outputs (one (m, c), half of e) two at a time;
  // lane u loads chunk u's (max, sum), broadcast with readlane, and every
  // load of both blocks is issued before the first is used.
  const coh_buf pb = coh_buffer(a.part);
  if (wave < 4) {
    const int nblk = a.M * G * 2;
    for (int b0 = wave; b0 < nblk; b0 += 8) {
      float mvl[2], lvl[2], ov[2][16];
      int nchb[2];
      uint32_t bse[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b = min(b0 + 4 * h, nblk - 1);
        const int m = b / (2 * G), c = (b / 2) % G, e = (b % 2) * 64 + lane;
        nchb[h] = (rows[m].pos + ACH) / ACH;
        bse[h] = (uint32_t)(((m * a.n_heads + g * G + c) * a.max_chunks) * rec);
        const uint32_t rl = bse[h] + (uint32_t)min(lane, nchb[h] - 1) * rec;
        mvl[h] = cload(pb, rl);
        lvl[h] = cload(pb, rl + 1);
#pragma unroll
        for (int u = 0; u < 16; ++u) ov[h][u] = cload(pb, bse[h] + (uint32_t)min(u, nchb[h] - 1) * rec + 2 + e);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b = b0 + 4 * h;
        if (b >= nblk) break;
        const int m = b / (2 * G), c = (b / 2) % G, e = (b % 2) * 64 + lane;
        float Mx = -INFINITY, den = 0.f, O = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (u < nchb[h]) {
            const float mu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mvl[h]), u));
            const float lu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lvl[h]), u));
            const float mn = fmaxf(Mx, mu);
            const float fa = __builtin_amdgcn_exp2f(Mx - mn), fb = __builtin_amdgcn_exp2f(mu - mn);
            den = den * fa + lu * fb;
            O = O * fa + ov[h][u] * fb;
            Mx = mn;
          }
        // chunks past 16 (contexts beyond 16 * 256 positions), one at a time
        for (int u = 16; u < nchb[h]; ++u) {
          const uint32_t r = bse[h] + (uint32_t)u * rec;
          const float mu = cload(pb, r), lu = cload(pb, r + 1), ou = cload(pb, r + 2 + e);
          const float mn = fmaxf(Mx, mu);
          const float fa = __builtin_amdgcn_exp2f(Mx - mn), fb = __builtin_amdgcn_exp2f(mu - mn);
          den = den * fa + lu * fb;
          O = O * fa + ou * fb;
          Mx = mn;
        }
        uint32_t h16, l16;
        split_bf16(O / den, h16, l16);
        xs_hi[m * XST + c * D + e] = (uint16_t)h16;
        xs_lo[m * XST + c * D + e] = (uint16_t)l16;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's weight blocks are in registers
  __syncthreads();

  // the WPT waves of a row tile are summed in wave order, then the first adds
  // rows 4 j4 .. + 3 of column r16 (= row m) to oacc
  const bool pack = a.M <= 8;
  auto finish = [&](int j, f32x4 acc) {
    if (o.WPT > 1) {
      *(f32x4*)(red + (wave * 64 + lane) * 4) = acc;
      lds_barrier();
      if (wave % o.WPT == 0)
        for (int q = 1; q < o.WPT; ++q) acc += *(const f32x4*)(red + ((wave + q) * 64 + lane) * 4);
      lds_barrier();  // red is rewritten next
    }
    if (wave % o.WPT == 0 && r16 < a.M && (!pack || r16 < 8)) {
      const size_t n0 = (size_t)r16 * a.H + (size_t)((j / a.n_kv) * o.RT + rtw) * 16 + 4 * j4;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        __hip_atomic_fetch_add(a.oacc + n0 + v, to_fixed(acc[v]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  for (int j = j0; j < o.n_o; j += 2 * n_ow) {
    const int jb = j + n_ow;
    const bool two = jb < o.n_o;
    if (j != j0) {  // items past the first two, loaded now
      o_load<G>(a, Lo, o, j, w0);
      if (two) o_load<G>(a, Lo, o, jb, w1);
      __builtin_amdgcn_s_waitcnt(0);
    }
    f32x4 y0, y1;
    switch (o.KW) {
      case 1: o_products_kw<1>(pack, two, w0, w1, xs_hi, xs_lo, XST, a.M, ksw, y0, y1); break;
      case 2: o_products_kw<2>(pack, two, w0, w1, xs_hi, xs_lo, XST, a.M, ksw, y0, y1); break;
      case 4: o_products_kw<4>(pack, two, w0, w1, xs_hi, xs_lo, XST, a.M, ksw, y0, y1); break;
      case 8: o_products_kw<8>(pack, two, w0, w1, xs_hi, xs_lo, XST, a.M, ksw, y0, y1); break;
      default: o_products_kw<16>(pack, two, w0, w1, xs_hi, xs_lo, XST, a.M, ksw, y0, y1); break;
    }
    finish(j, y0);
    if (two) finish(jb, y1);
  }
  lds_barrier();  // x' and red are rewritten by the next phase
  return gu_pf;
}

// Returns whether the gate/up GEMV's LDS-prefetched iteration was loaded
// here (FO: o_phase).
// KV8: the cache holds int8 codes with one fp32 scale per position and head
// vector.  The codes enter the MFMAs as the fp16 integers 1152 + q; S starts
// from -1152 times the column's sum of the q parts and is multiplied by the
// keys' scales; the values' scales are folded into P (P'), and 1152 times the
// column's sum of P' comes off O at the end.  The new position is quantized
// here (per head vector, as the cache stores it) and attended in that form.
template <int G, bool FO, int KI, bool KV8, typename Sync>
DPK_DEV bool attn_phase(const MegaArgs& a, const RowParam* rows, int layer, const uint16_t* qn, const uint16_t* kn,
                        const GemvArgs* Lo, const GemvArgs* Lgu, unsigned char* lds, unsigned char* pf,
                        const Barrier& bar, int wg, int nwg, Sync&& sync) {
  // q (log2 domain) as fp16 hi + lo and the new position's K / V in cache
  // precision, all in MFMA fragment order (8 consecutive d per 16 bytes)
  _Float16* qh16 = (_Float16*)lds;      // [G][D]
  _Float16* ql16 = qh16 + G * D;        // [G][D]
  _Float16* kn16 = ql16 + G * D;        // [D]
  _Float16* vn16 = kn16 + D;            // [D]
  float* wst = (float*)lds + G * D + 2 * D;  // [AW][2][G]
  float* ow = wst + AW * 2 * G;         // [AW][D][G]
  int* flag = (int*)(ow + AW * D * G);
  // KV8, in the 4 D bytes between vn16 and wst: the new position's codes,
  // the columns' q sums and the new key's / value's scales
  int8_t* knew8 = (int8_t*)(vn16 + D);  // [D]
  int8_t* vnew8 = knew8 + D;            // [D]
  float* qsum = (float*)(vnew8 + D);    // [16]
  float* newsc = qsum + 16;             // [2]
  using Frag = typename std::conditional<KV8, u32x2, u32x4>::type;  // 8 cache elements
  using Elt = typename std::conditional<KV8, int8_t, _Float16>::type;

  const int tid = opaque_tid(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform over the wave
  const int r16 = lane & 15, j4 = lane >> 4;
  const int n_items = a.M * a.n_kv * a.max_chunks;
  const int rec = D + 2;

  // K tile t row r is position 8 (r / 4) + 4 t + r % 4 of the wave's 32, so the
  // S accumulators give lane group j4 positions 8 j4 .. + 7 (its k range of P^T
  // in the P V product) and V^T is read as one 8-position group per lane
  Frag kf[2][D / 32];
  Frag vf[D / 16];
  f32x4 sc8[4];  // KV8: scales of the lane's 8 positions (its V group): keys, then values
  float cs = 0.f, sn = 0.f;  // this wave's RoPE values
  uint16_t gr0 = 0, gr1 = 0;  // and its QK-norm gains (bf16)

  // K / V^T fragments of the item's positions for this wave, and the RoPE /
  // QK-norm constants of the row (none of it depends on the previous phase)
  RowParam rp_it{};  // the row parameters of the prefetched item
  auto prefetch = [&](int it) {
    const int chunk = it % a.max_chunks, g = (it / a.max_chunks) % a.n_kv, m = it / (a.max_chunks * a.n_kv);
    rp_it = rows[m];
    const RowParam rp = rp_it;
    const int ctx = rp.pos + 1;
    const int c0 = chunk * ACH, c1 = min(ctx, c0 + ACH);
    const int wp0 = c0 + 32 * wave;
    const Elt* Kb = (const Elt*)a.kv.base + kv_slab(a.kv, rp.seq, layer, 0, g);
    const Elt* Vb = (const Elt*)a.kv.base + kv_slab(a.kv, rp.seq, layer, 1, g);
    // unconditional loads: positions past the context read the last one's
    // address (K rows are masked in S, V groups where they are used); an
    // 8-position group stays inside the slab row (max_seq % 64 == 0)
    const int plast = max(c1 - 1, 0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int p = min(wp0 + 8 * (r16 >> 2) + 4 * t + (r16 & 3), plast);
#pragma unroll
      for (int s = 0; s < D / 32; ++s) kf[t][s] = *(const Frag*)(Kb + (size_t)p * D + 32 * s + 8 * j4);
    }
    const int p8 = min(wp0 + 8 * j4, plast & ~7);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) vf[dt] = *(const Frag*)(Vb + (size_t)(dt * 16 + r16) * a.kv.max_seq + p8);
    if constexpr (KV8) {  // (a group past the context reads the last whole group's scales: masked)
      const float* Ksc = a.kv.scales + kv_scale_slab(a.kv, rp.seq, layer, 0, g);
      const float* Vsc = a.kv.scales + kv_scale_slab(a.kv, rp.seq, layer, 1, g);
      sc8[0] = *(const f32x4*)(Ksc + p8);
      sc8[1] = *(const f32x4*)(Ksc + p8 + 4);
      sc8[2] = *(const f32x4*)(Vsc + p8);
      sc8[3] = *(const f32x4*)(Vsc + p8 + 4);
    }
    // (unconditional too: a gain that does not exist reads a dummy address,
    // and the values are converted where they are used)
    cs = a.rope_cos[(size_t)rp.pos * (D / 2) + lane];
    sn = a.rope_sin[(size_t)rp.pos * (D / 2) + lane];
    const uint16_t* gn = wave < G ? qn : kn;
    const uint16_t* gp = gn ? gn : (const uint16_t*)a.rope_cos;
    gr0 = gemv_detail::gmem(gp)[lane];
    gr1 = gemv_detail::gmem(gp)[lane + 64];
  };

  // FO: workgroups [0, n_aw) run the attention items and the other n_ow (a
  // multiple of n_kv, at least half the grid) the O projection (o_phase)
  int n_aw = nwg;
  if constexpr (FO) {
    const int n_ow = ((nwg - min(n_items, nwg / 2)) / a.n_kv) * a.n_kv;
    n_aw = nwg - n_ow;
    if (wg >= n_aw) return o_phase<G, KI>(a, rows, layer, Lo, Lgu, lds, pf, bar, wg, wg - n_aw, n_ow, sync);
  }
  int it = wg;
  sync([&] {  // the QKV projection of every row is complete after this
    if (it < n_items) prefetch(it);
  });
  for (; it < n_items; it += n_aw) {
    if (it != wg) prefetch(it);
    const int chunk = it % a.max_chunks, g = (it / a.max_chunks) % a.n_kv, m = it / (a.max_chunks * a.n_kv);
    const RowParam rp = rp_it;
    const int ctx = rp.pos + 1;
    const int nch = (ctx + ACH - 1) / ACH;
    if (chunk >= nch) continue;  // uniform over the workgroup
    const int c0 = chunk * ACH, c1 = min(ctx, c0 + ACH);
    const int wp0 = c0 + 32 * wave;
    const bool own = rp.pos >= c0 && rp.pos < c1;

    // ---- q heads (waves < G), the new key (wave G) and value (wave G + 1)
    // from the raw projection
    const coh_buf q0 = coh_buffer(a.qkv);
    const uint32_t row = (uint32_t)(m * a.ld_qkv);
    if (wave <= G && (wave < G || own)) {
      const uint32_t x = row + (uint32_t)((wave < G ? g * G + wave : a.n_heads + g) * D);
      const float xa = cload(q0, x + lane);
      const float xb = cload(q0, x + lane + 64);
      const bool norm = (wave < G ? qn : kn) != nullptr;
      const float ss = wave_sum(xa * xa + xb * xb);
      const float r = norm ? rsqrtf(ss / (float)D + a.eps) : 1.0f;
      const float g0 = norm ? bf16_to_f32(gr0) : 1.0f, g1 = norm ? bf16_to_f32(gr1) : 1.0f;
      const float x1 = xa * r * g0, x2 = xb * r * g1;
      const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
      if (wave < G) {
        _Float16 h, l, h2, l2;
        split_f16(y1 * a.scale * LOG2E, h, l);
        qh16[wave * D + lane] = h;
        ql16[wave * D + lane] = l;
        split_f16(y2 * a.scale * LOG2E, h2, l2);
        qh16[wave * D + lane + 64] = h2;
        ql16[wave * D + lane + 64] = l2;
        if constexpr (KV8) {  // the column's sum of the q parts the MFMAs multiply
          const float qs = wave_sum((float)h + (float)l + (float)h2 + (float)l2);
          if (lane == 0) qsum[wave] = qs;
        }
      } else if constexpr (KV8) {  // the new key's codes and scale: to the cache and LDS
        float c0, c1;
        const float sk = kv_quant_i8(y1, y2, c0, c1);
        knew8[lane] = (int8_t)c0;
        knew8[lane + 64] = (int8_t)c1;
        int8_t* kb = (int8_t*)a.kv.base + kv_slab(a.kv, rp.seq, layer, 0, g) + (size_t)rp.pos * D;
        kb[lane] = (int8_t)c0;
        kb[lane + 64] = (int8_t)c1;
        if (lane == 0) {
          newsc[0] = sk;
          a.kv.scales[kv_scale_slab(a.kv, rp.seq, layer, 0, g) + rp.pos] = sk;
        }
      } else {
        kn16[lane] = (_Float16)y1;
        kn16[lane + 64] = (_Float16)y2;
      }
    } else if (wave == G + 1 && own) {
      const uint32_t v = row + (uint32_t)((a.n_heads + a.n_kv + g) * D);
      if constexpr (KV8) {  // the new value's codes and scale: to the cache and LDS
        float c0, c1;
        const float sv = kv_quant_i8(cload(q0, v + lane), cload(q0, v + lane + 64), c0, c1);
        vnew8[lane] = (int8_t)c0;
        vnew8[lane + 64] = (int8_t)c1;
        int8_t* vb = (int8_t*)a.kv.base + kv_slab(a.kv, rp.seq, layer, 1, g);
        vb[(size_t)lane * a.kv.max_seq + rp.pos] = (int8_t)c0;
        vb[(size_t)(lane + 64) * a.kv.max_seq + rp.pos] = (int8_t)c1;
        if (lane == 0) {
          newsc[1] = sv;
          a.kv.scales[kv_scale_slab(a.kv, rp.seq, layer, 1, g) + rp.pos] = sv;
        }
      } else {
        vn16[lane] = (_Float16)cload(q0, v + lane);
        vn16[lane + 64] = (_Float16)cload(q0, v + lane + 64);
      }
    }
    __syncthreads();
    // KV8: the scales of the lane's positions wp0 + 8 j4 + i (values past the
    // context: 0, so P' is 0 there)
    float sk[KV8 ? 8 : 1], sv[KV8 ? 8 : 1];
    if constexpr (KV8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sk[i] = sc8[i >> 2][i & 3];
        sv[i] = (wp0 + 8 * j4 + i < c1) ? sc8[2 + (i >> 2)][i & 3] : 0.f;
      }
      if (own) {
        // the new position inside this wave's fragments: its codes and scales
        // from LDS (compile-time fragment indices only)
        const int off = rp.pos - wp0;
        if (off >= 0 && off < 32) {
          const int kt = (off % 8) / 4, kr = 4 * (off / 8) + off % 4;
          if (r16 == kr) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
              if (t == kt) {
#pragma unroll
                for (int s = 0; s < D / 32; ++s) kf[t][s] = *(const Frag*)(knew8 + 32 * s + 8 * j4);
              }
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
      }
    } else if (own) {
      for (int e = tid; e < D; e += MT) {
        kv_store(a.kv, kv_offset(a.kv, rp.seq, layer, 0, g, e, rp.pos), (float)kn16[e]);
        kv_store(a.kv, kv_offset(a.kv, rp.seq, layer, 1, g, e, rp.pos), (float)vn16[e]);
      }
      // the new position inside this wave's fragments comes from kn16 / vn16
      const int off = rp.pos - wp0;
      if (off >= 0 && off < 32) {
        // compile-time fragment indices only (runtime ones would spill the arrays)
        const int kt = (off % 8) / 4, kr = 4 * (off / 8) + off % 4;  // the row holding position off
        if (r16 == kr) {
          u32x4 k4[D / 32];
#pragma unroll
          for (int s = 0; s < D / 32; ++s) k4[s] = *(const u32x4*)(kn16 + 32 * s + 8 * j4);
#pragma unroll
          for (int t = 0; t < 2; ++t)
            if (t == kt) {
#pragma unroll
              for (int s = 0; s < D / 32; ++s) kf[t][s] = k4[s];
            }
        }
        const int e8 = off % 8;
        if (j4 == off / 8) {
          _Float16 vv[D / 16];
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) vv[dt] = vn16[dt * 16 + r16];
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            f16x8 v8 = __builtin_bit_cast(f16x8, vf[dt]);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e == e8) v8[e] = vv[dt];
            vf[dt] = __builtin_bit_cast(u32x4, v8);
          }
        }
      }
    }

    // ---- S = K Q^T (log2 domain), 2 tiles of 16 positions.  Columns past G
    // read head G - 1: they are never used, and an MFMA column depends on its
    // own B column only.
    f16x8 qh[D / 32], ql[D / 32];
    {
      const int qc = r16 < G ? r16 : G - 1;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        qh[s] = *(const f16x8*)(qh16 + qc * D + 32 * s + 8 * j4);
        ql[s] = *(const f16x8*)(ql16 + qc * D + 32 * s + 8 * j4);
      }
    }
    const float cq = KV8 ? -1152.0f * qsum[r16 < G ? r16 : G - 1] : 0.f;  // S's start (int8 cache)
    f32x4 sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sc[t] = f32x4{cq, cq, cq, cq};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        f16x8 A;
        if constexpr (KV8)
          A = __builtin_bit_cast(f16x8, kv_codes_f16(kf[t][s]));
        else
          A = __builtin_bit_cast(f16x8, kf[t][s]);
        sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qh[s], sc[t], 0, 0, 0);
        sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ql[s], sc[t], 0, 0, 0);
      }
      if constexpr (KV8) {  // the keys' scales (lane rows 4 j4 + v of tile t: positions 8 j4 + 4 t + v)
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[t][v] *= sk[4 * t + v];
      }
    }
    // mask (positions 8 j4 + 4 t + v past the context), column max / sum
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (wp0 + 8 * j4 + 4 * t + v >= c1) sc[t][v] = -INFINITY;
        mx = fmaxf(mx, sc[t][v]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float e = (sc[t][v] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[t][v] - mx);
        sc[t][v] = e;
        sum += e;
      }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    if constexpr (KV8) {  // P' = P times the value's scale
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[t][v] *= sv[4 * t + v];
    }

    // ---- O^T = V^T P^T over the 32 positions (k slots 0..3 from tile 0, 4..7 from tile 1)
    f32x4 o[D / 16];
    {
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
      // KV8: 1152 times the column's sum of P' (the parts the MFMAs take)
      float corr = 0.f;
      if constexpr (KV8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) corr += (float)ph[i] + (float)pl[i];
        corr += __shfl_xor(corr, 16, 64);
        corr += __shfl_xor(corr, 32, 64);
        corr *= 1152.0f;
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 w;
        if constexpr (KV8) {  // (int8 codes are finite as fp16 and meet P' = 0 past the context)
          w = kv_codes_f16(vf[dt]);
        } else {
          w = vf[dt];
          if (wp0 + 32 > c1) {  // positions past the context may hold any bits (0 * NaN)
            const int n = c1 - wp0 - 8 * j4;
            auto mk = [n](int e) { return n >= e + 2 ? 0xffffffffu : (n == e + 1 ? 0x0000ffffu : 0u); };
            w = u32x4{w.x & mk(0), w.y & mk(2), w.z & mk(4), w.w & mk(6)};
          }
        }
        const f16x8 A = __builtin_bit_cast(f16x8, w);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ph, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pl, o[dt], 0, 0, 0);
        if constexpr (KV8) {  // the values' code offset (lane: column r16)
#pragma unroll
          for (int v = 0; v < 4; ++v) o[dt][v] -= corr;
        }
      }
    }


    // ---- combine the waves (per column = query head)
    if (r16 < G) {
      if (j4 == 0) {
        wst[(wave * 2 + 0) * G + r16] = mx;
        wst[(wave * 2 + 1) * G + r16] = sum;
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int v = 0; v < 4; ++v) ow[(wave * D + dt * 16 + 4 * j4 + v) * G + r16] = o[dt][v];
    }
    __syncthreads();
    // chunk statistics per column c: Mc = max_w m_w, Lc = sum_w 2^(m_w - Mc) l_w,
    // Oc = sum_w 2^(m_w - Mc) O_w
    const coh_buf ob = coh_buffer(a.attn_out), pb = coh_buffer(a.part);
    const uint32_t outp = (uint32_t)((m * a.n_heads + g * G) * D);
    for (int i = tid; i < G * D; i += MT) {
      const int c = i / D, e = i % D;
      float Mc = -INFINITY;
#pragma unroll
      for (int w = 0; w < AW; ++w) Mc = fmaxf(Mc, wst[(w * 2) * G + c]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < AW; ++w) {
        const float mwv = wst[(w * 2) * G + c];
        const float f = (mwv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mwv - Mc);
        L += f * wst[(w * 2 + 1) * G + c];
        O += f * ow[(w * D + e) * G + c];
      }
      if (nch == 1 && !FO) {
        cstore(ob, outp + c * D + e, O / L);
      } else {
        const uint32_t r = (uint32_t)(((m * a.n_heads + g * G + c) * a.max_chunks + chunk) * rec);
        cstore(pb, r + 2 + e, O);
        if (e == 0) {
          cstore(pb, r, Mc);
          cstore(pb, r + 1, L);
        }
      }
    }
    if (FO) {
      // count in once the records are stored; the counter grows over the
      // step's layers
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0)
        __hip_atomic_fetch_add(a.attn_counters + (m * a.n_kv + g) * MEGA_CTR_STRIDE, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else if (nch > 1 && last_block_arrive(a.attn_counters + m * a.n_kv + g, nch, flag)) {
      // output (c, e) of every query head of g: the (max, sum, O[e]) records
      // of up to 16 chunks are loaded at once and folded in with a running
      // maximum (log-sum-exp weights)
      for (int i = tid; i < G * D; i += MT) {
        const int c = i / D, e = i % D;
        const uint32_t base = (uint32_t)(((m * a.n_heads + g * G + c) * a.max_chunks) * rec);
        float Mx = -INFINITY, den = 0.f, O = 0.f;
        for (int ch0 = 0; ch0 < nch; ch0 += 16) {
          float mv[16], lv[16], ov[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const uint32_t r = base + (uint32_t)min(ch0 + u, nch - 1) * rec;
            mv[u] = cload(pb, r);
            lv[u] = cload(pb, r + 1);
            ov[u] = cload(pb, r + 2 + e);
          }
#pragma unroll
          for (int u = 0; u < 16; ++u)
            if (ch0 + u < nch) {
              const float mn = fmaxf(Mx, mv[u]);
              const float fa = __builtin_amdgcn_exp2f(Mx - mn), fb = __builtin_amdgcn_exp2f(mv[u] - mn);
              den = den * fa + lv[u] * fb;
              O = O * fa + ov[u] * fb;
              Mx = mn;
            }
        }
        cstore(ob, outp + c * D + e, O / den);
      }
    }
    __syncthreads();  // LDS is rewritten by the next item
  }
  return false;
}

// FMT: weight format of every GEMV.  SMALL: each wave reduces 128 columns per
// iteration (so rows of 1024, 2048, 3072 ... columns split over eight waves)
// and the QKV projection goes in 16-row tiles, which gives a narrow model's
// QKV about one tile per workgroup.
//
// FO (bf16, a.oacc set): attention and the O projection are one phase (see
// attn_phase), and gate/up and down fold the fixed-point O sums into h.
// KV8: the KV cache holds int8 codes with per-vector scales (a.kv.i8).
template <int G, int FMT, bool SMALL, bool FO, bool KV8>
__global__ __launch_bounds__(MT, 1) void decode_step_kernel(MegaArgs a) {
  // (the lm_head of a narrow model goes in 32-row tiles: one 128-column
  // iteration per 16 rows would leave a wave a single 4 KB load in flight)
  constexpr int KI = SMALL ? 128 : 0, TQ = SMALL ? 1 : 2, TH = mega_head_tiles(FMT, SMALL), TGU = mega_gu_tiles(FMT);
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int wg = blockIdx.x, nwg = gridDim.x;
  Barrier bar{a.bar, a.bar + MEGA_BAR_ABORT, (unsigned)nwg, 0u};
  // phase tracing (workgroup 0, thread 0): ticks from one barrier release to
  // the next go to the phase the barrier closes
  const bool tr = a.trace && wg == 0 && threadIdx.x == 0;
  unsigned long long t_prev = tr ? wall_clock64() : 0ull;
  int closing = MP_EMBED;
  auto mark = [&](int phase) {
    if (tr) {
      const unsigned long long t = wall_clock64();
      a.trace[phase] += t - t_prev;
      t_prev = t;
    }
  };
  auto sync = [&](auto&& prefetch) {
    grid_sync(bar, prefetch);
    mark(closing);
  };
  using gemv_detail::gemv_body;
  // The layer's table entry (and at the end the lm_head's arguments) is
  // copied into LDS before its first phase: the phases then read their
  // arguments from LDS, where a read never waits for the weight loads in
  // flight (a reload from device memory would wait for every vector load
  // issued before it).  The copy overwrites the previous layer's entry only
  // after every wave has finished that layer (the barrier below).
  // The rows' parameters (constant over the step) are staged there too, so
  // the attention prefetch computes its cache addresses without a round trip.
  MegaLayer* const Ls = (MegaLayer*)(lds + a.lds_args);
  GemvArgs* const Hs = (GemvArgs*)(Ls + 1);
  RowParam* const Rs = (RowParam*)(Hs + 1);
  // bf16: the GEMVs' LDS prefetch slots (8 waves x 8 KB), after the staged
  // arguments, used by nothing else
  constexpr bool PF = FMT == W_BF16;
  unsigned char* const pf = lds + a.lds_args + MEGA_ARGS_LDS;
  auto stage = [&](void* dst, const void* src, int bytes) {
    __syncthreads();
    for (int i = threadIdx.x; i < bytes / 4; i += MT) ((uint32_t*)dst)[i] = ((const uint32_t*)src)[i];
    __syncthreads();
  };
  __syncthreads();
  if (threadIdx.x == 0) {  // from the kernel arguments (compile-time indices)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < a.M) Rs[i] = a.rows[i];
  }
  __syncthreads();
  embed_phase(a, Rs, wg, nwg);
  for (int l = 0; l < a.n_layers; ++l) {
    stage(Ls, a.layers + l, (int)sizeof(MegaLayer));
    const MegaLayer& L = *Ls;
    gemv_body<FMT, TQ, 8, true, false, KI, PF>(L.qkv, a.M, lds, wg, nwg, sync, pf);
    closing = MP_QKV;
    const bool gu_pf = attn_phase<G, FO, KI, KV8>(a, Rs, l, L.qn, L.kn, &L.o, &L.gu, lds, pf, bar, wg, nwg, sync);
    closing = MP_ATTN;
    if constexpr (!FO) {
      gemv_body<FMT, 1, 8, true, false, KI, PF>(L.o, a.M, lds, wg, nwg, sync, pf);
      closing = MP_O;
    }
    gemv_body<FMT, TGU, 8, true, false, KI, PF, FO>(L.gu, a.M, lds, wg, nwg, sync, pf, gu_pf);
    closing = MP_GATEUP;
    gemv_body<FMT, 1, 8, true, false, KI, PF, FO>(L.down, a.M, lds, wg, nwg, sync, pf);
    closing = MP_DOWN;
  }
  stage(Hs, &a.head, (int)sizeof(GemvArgs));
  gemv_body<FMT, TH, 8, true, false, KI>(*Hs, a.M, lds, wg, nwg, sync);
  grid_exit(bar, a.bar + MEGA_BAR_EXIT, a.err, a.attn_counters, FO ? a.M * a.n_kv : 0);
  if (tr) {
    mark(MP_HEAD);
    a.trace[MP_STEPS] += 1;
  }
}

#ifdef DPK_DECODE_STEP_KV8_TU
}  // namespace

// The variants over an int8 KV cache: at 256 columns per iteration bf16 with
// the fused O projection, int8 weights (one scale per row), Q8 and Q4_0
// weights, G = 1, 2, 4; at 128 columns bf16 and MLX 4-bit, G = 2, 4.
const void* mega_kernel_kv8(int G, int fmt, bool small, bool fo) {
  if (small) {  // 128 columns per iteration: bf16 and MLX 4-bit, G = 2, 4, the O projection a GEMV
    if (fo) return nullptr;
    if (fmt == W_BF16 && G == 2) return (const void*)decode_step_kernel<2, W_BF16, true, false, true>;
    if (fmt == W_BF16 && G == 4) return (const void*)decode_step_kernel<4, W_BF16, true, false, true>;
    if (fmt == W_Q4 && G == 2) return (const void*)decode_step_kernel<2, W_Q4, true, false, true>;
    if (fmt == W_Q4 && G == 4) return (const void*)decode_step_kernel<4, W_Q4, true, false, true>;
    return nullptr;
  }
  if (fmt == W_BF16 && fo) {
    if (G == 1) return (const void*)decode_step_kernel<1, W_BF16, false, true, true>;
    if (G == 2) return (const void*)decode_step_kernel<2, W_BF16, false, true, true>;
    if (G == 4) return (const void*)decode_step_kernel<4, W_BF16, false, true, true>;
  } else if (fmt == W_I8 && !fo) {
    if (G == 1) return (const void*)decode_step_kernel<1, W_I8, false, false, true>;
    if (G == 2) return (const void*)decode_step_kernel<2, W_I8, false, false, true>;
    if (G == 4) return (const void*)decode_step_kernel<4, W_I8, false, false, true>;
  } else if (fmt == W_Q40 && !fo) {
    if (G == 1) return (const void*)decode_step_kernel<1, W_Q40, false, false, true>;
    if (G == 2) return (const void*)decode_step_kernel<2, W_Q40, false, false, true>;
    if (G == 4) return (const void*)decode_step_kernel<4, W_Q40, false, false, true>;
  } else if (fmt == W_Q8 && !fo) {
    if (G == 1) return (const void*)decode_step_kernel<1, W_Q8, false, false, true>;
    if (G == 2) return (const void*)decode_step_kernel<2, W_Q8, false, false, true>;
    if (G == 4) return (const void*)decode_step_kernel<4, W_Q8, false, false, true>;
  }
  return nullptr;
}

}  // namespace dpk
#else
// Built variants (fp16 KV cache): bf16, int8 (one scale per row), Q8 and Q4_0
// at 256 columns per iteration for G = 1, 2, 4; bf16 and 4-bit at 128 columns for
// G = 2, 4; bf16 with and without the fused O projection.  The int8-cache
// variants are built in a translation unit of their own (mega_kernel_kv8).
template <bool FO>
const void* mega_kernel_fo(int G, int fmt, bool small) {
  if (fmt == W_BF16 && !small) {
    switch (G) {
      case 1: return (const void*)decode_step_kernel<1, W_BF16, false, FO, false>;
      case 2: return (const void*)decode_step_kernel<2, W_BF16, false, FO, false>;
      case 4: return (const void*)decode_step_kernel<4, W_BF16, false, FO, false>;
      default: return nullptr;
    }
  }
  if (fmt == W_I8 && !small && !FO) {  // int8 codes, one scale per row: the 256-column variant only
    if (G == 1) return (const void*)decode_step_kernel<1, W_I8, false, false, false>;
    if (G == 2) return (const void*)decode_step_kernel<2, W_I8, false, false, false>;
    if (G == 4) return (const void*)decode_step_kernel<4, W_I8, false, false, false>;
    return nullptr;
  }
  if (fmt == W_Q40 && !small && !FO) {  // Q4_0 blocks: 256-column chunks
    if (G == 1) return (const void*)decode_step_kernel<1, W_Q40, false, false, false>;
    if (G == 2) return (const void*)decode_step_kernel<2, W_Q40, false, false, false>;
    if (G == 4) return (const void*)decode_step_kernel<4, W_Q40, false, false, false>;
    return nullptr;
  }
  if (fmt == W_Q8 && !small && !FO) {  // Q8 blocks: 256-column chunks of scales
    if (G == 1) return (const void*)decode_step_kernel<1, W_Q8, false, false, false>;
    if (G == 2) return (const void*)decode_step_kernel<2, W_Q8, false, false, false>;
    if (G == 4) return (const void*)decode_step_kernel<4, W_Q8, false, false, false>;
    return nullptr;
  }
  if (!small) return nullptr;
  if (fmt == W_BF16) {
    if (G == 2) return (const void*)decode_step_kernel<2, W_BF16, true, FO, false>;
    if (G == 4) return (const void*)decode_step_kernel<4, W_BF16, true, FO, false>;
  } else if (fmt == W_Q4 && !FO) {
    if (G == 2) return (const void*)decode_step_kernel<2, W_Q4, true, false, false>;
    if (G == 4) return (const void*)decode_step_kernel<4, W_Q4, true, false, false>;
  }
  return nullptr;
}

}  // namespace

const void* mega_kernel_kv8(int G, int fmt, bool small, bool fo);

namespace {
const void* mega_kernel_for(int G, int fmt, bool small, bool fo, bool kv8) {
  if (kv8) return mega_kernel_kv8(G, fmt, small, fo);
  return fo ? mega_kernel_fo<true>(G, fmt, small) : mega_kernel_fo<false>(G, fmt, small);
}

}  // namespace

size_t mega_o_lds_bytes(int M, int G, int rt) {
  if (rt != 1 && rt != 2 && rt != 4 && rt != 8) return 0;
  const int KS = G * D / 32, WPT = 8 / rt;
  if (KS % WPT || KS / WPT > O_KWMAX) return 0;
  return ((4 * (size_t)M * (G * D + 8) + 15) & ~(size_t)15) + 8 * 64 * 4 * 4;
}

size_t mega_attn_lds_bytes(int G) {
  return ((size_t)G * D + 2 * D + AW * 2 * G + AW * D * G + 4) * 4;
}

int mega_threads() { return MT; }
int mega_attn_chunk() { return ACH; }

// Workgroups per CU the kernel can keep resident with lds bytes of LDS (0 if
// the kernel does not exist for G, fmt, small, fo, kv8).
int mega_occupancy(int G, int fmt, bool small, bool fo, bool kv8, size_t lds) {
  const void* k = mega_kernel_for(G, fmt, small, fo, kv8);
  if (!k) return 0;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k, MT, lds) != hipSuccess) return 0;
  return nb;
}

hipError_t launch_decode_step(const MegaArgs& a, int G, int n_wg, size_t lds, hipStream_t stream) {
  const void* k = mega_kernel_for(G, a.fmt, a.small != 0, a.oacc != nullptr, a.kv.i8 != 0);
  if (!k || n_wg < 1 || a.M < 1 || a.M > 16) return hipErrorInvalidValue;
  MegaArgs copy = a;
  void* args[] = {&copy};
  hipEvent_t start = g_timing.start, stop = g_timing.stop;
  if (start) (void)hipEventRecord(start, stream);
  const hipError_t e = hipLaunchCooperativeKernel(k, dim3(n_wg), dim3(MT), args, (unsigned)lds, stream);
  if (stop) (void)hipEventRecord(stop, stream);
  g_timing.start = nullptr;
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace dpk
#endif
