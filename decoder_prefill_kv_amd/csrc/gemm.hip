// Prefill GEMM on gfx950 matrix cores: C[m][n] = sum_k A[m][k] * B[n][k]
// with A = activations [M][K] and B = weights [N][K] (the [out, in] layout),
// both fp16 and K-contiguous, fp32 accumulation.
//
// Prefill is compute bound (the whole prompt goes through every weight at
// once, "LLMs on the ANE", opening section); this kernel is where its FLOPs go.
// The operands are fp16 rather than bf16: every weight of the bf16 model is
// exactly representable in fp16 (magnitudes >= 2^-24; smaller ones round with
// an absolute error below 2^-25), and fp16 activations carry three more
// mantissa bits, which the logits tolerance needs on deep models.  Where that
// is still not enough (the QKV projection), A is given as [A_hi | A_lo] with
// K = 2 Kb and B is read twice, which computes (A_hi + A_lo) B^T.
//
// Tile 256 x 256 x 64, 4 waves in a 2 x 2 layout, each wave 128 x 128 from
// 4 x 4 v_mfma_f32_32x32x16_f16 blocks (256 fp32 accumulators per lane, in
// AGPRs).  One wave per SIMD, so latency is hidden inside the wave:
//  * fragments are double-buffered in registers: the LDS reads of k-step
//    s+1 are interleaved with the 16 MFMAs of step s;
//  * the next k-tile's global loads are issued a whole k-tile ahead into
//    staging registers and written to the other LDS stage between the MFMAs
//    of the third k-step;
//  * the one barrier per k-tile sits before the last k-step, whose operands
//    are already in registers, so the first LDS reads of the next tile
//    overlap its MFMAs.
//
// QKV epilogue: a wave's 128 columns are exactly one head (tiles start at
// multiples of 256, heads at multiples of 128), and each of its rows is held
// by 32 lanes of one half-wave, four columns per lane with column c and
// c + 64 in the same lane.  So the per-head QK-norm ("LLMs on the ANE",
// "Correctness": RMSNorm of q and k per head before RoPE) is a 32-lane sum of
// squares and the RoPE rotation of the pair (c, c + 64) is lane-local; q goes
// out as fp16 hi / lo, k and v straight into the fp16 KV cache, so the fp32
// projection never reaches memory.
//
// Split-K: when the (M, N) tiles cannot fill the chip (N = 4096 at M = 2048
// gives 128 tiles for 256 CUs), blockIdx.z takes a contiguous 1/S of the
// k-tiles.  Each split writes its partial tile to a workspace with device-
// coherent stores; the last split to arrive adds the partials in split order
// (so the result does not depend on arrival order) and runs the epilogue.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dpk {

namespace {

constexpr int BM = 256, BN = 256, BK = 64, THREADS = 256;
constexpr int LDS_STRIDE = BK + 8;  // halfs per LDS row (pad against bank conflicts)

// instruction classes for __builtin_amdgcn_sched_group_barrier
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200;

// BNT: tile columns, 256, or 128 (whole-K STORE / ADD GEMMs whose 256-wide
// tiles would leave CUs idle: each wave then holds 128 x 64 of C).
template <int EPI, bool SPLIT, int BNT = BN>
__global__ __launch_bounds__(THREADS, 1) void gemm_kernel(GemmArgs a) {
  static_assert(BNT == BN || (BNT == BN / 2 && EPI != GEMM_SWIGLU_F16 && EPI != GEMM_QKV_F16 && !SPLIT),
                "narrow tiles: whole K, no SwiGLU, no QKV epilogue");
  constexpr int JB = BNT / 64;  // 32-column blocks per wave
  __shared__ __attribute__((aligned(16))) _Float16 As[2][BM][LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][BNT][LDS_STRIDE];
  __shared__ int s_last;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  // tile (bx, by) and split bz of this workgroup.  xcd_blocks: consecutive
  // workgroups go to the 8 XCDs in turn, so workgroup L runs on XCD L % 8;
  // XCD k then takes the 4 x 4 tile block k with all its splits, which its
  // L2 shares (A rows across the block's columns, B rows across its rows).
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if (a.xcd_blocks) {
    // blocks of 4 tile rows x BW tile columns (4 x 4 wide tiles, 4 x 8 narrow
    // ones: 1024 A rows and 1024 B rows per XCD either way)
    constexpr int BW = (BNT == BN) ? 4 : 8;
    const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int k = L & 7, s = L >> 3, gx = gridDim.x / BW;
    bz = s % gridDim.z;
    bx = BW * (k % gx) + (s / gridDim.z) % BW;
    by = 4 * (k / gx) + s / (gridDim.z * BW);
  }
  const int m0 = by * BM;
  // SWIGLU: the tile's B rows are 128 gate rows then the same 128 up rows
  const int n0 = (EPI == GEMM_SWIGLU_F16) ? bx * (BN / 2) : bx * BNT;
  const int nk_all = a.K / BK;
  const int nks = SPLIT ? nk_all / a.splits : nk_all;
  const int kt0 = SPLIT ? bz * nks : 0;

  // global load assignment: 8 threads per 64-half row, 32 rows per pass.
  // Row block i of a pass is a uniform offset from the thread's first row,
  // so each load is (uniform base, one per-thread 32-bit offset).  The A
  // buffer holds whole 256-row tiles: rows past M are read but their results
  // are never stored.
  const int lrow = tid >> 3, lk = (tid & 7) * 8;
  const uint32_t a_off = (uint32_t)(lrow * a.lda + lk), b_off = (uint32_t)(lrow * a.ldb + lk);
  const _Float16* A0 = a.A + (size_t)m0 * a.lda;
  const _Float16* B0 = a.B + (size_t)n0 * a.ldb;
  const _Float16* B20 = (EPI == GEMM_SWIGLU_F16) ? a.B2 + (size_t)n0 * a.ldb : nullptr;

  f32x16 acc[4][JB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // two staging sets: tile t+1 waits in one while tile t+2 is in flight into
  // the other (global loads are issued two k-tiles ahead of their LDS write).
  // Staging register r < 8 holds A row block r, r >= 8 B row block r - 8.
  u32x4 ra[2][BM / 32], rb[2][BNT / 32];
  const int Kb = a.Kb ? a.Kb : a.K;
  // global loads of staging registers [R0, R1) of set SET for k-tile kt
  auto gload = [&](auto set_c, int kt, auto r0_c, auto r1_c) {
    constexpr int SET = decltype(set_c)::value, R0 = decltype(r0_c)::value, R1 = decltype(r1_c)::value;
    const int ko = kt * BK;
    const int kob = ko < Kb ? ko : ko - Kb;  // B is read twice when A = [hi | lo]
    const _Float16* Ak = A0 + ko;
#pragma unroll
    for (int r = R0; r < R1; ++r) {
      if (r < BM / 32) {
        ra[SET][r] = *(const u32x4*)(Ak + (size_t)r * 32 * a.lda + a_off);
      } else {
        const int i = r - BM / 32;
        // SWIGLU: B rows 0..127 of the tile are gate rows, 128..255 the same up rows
        const _Float16* Bk = (EPI == GEMM_SWIGLU_F16 && i >= BN / 64) ? B20 + (size_t)(i - BN / 64) * 32 * a.ldb
                                                                      : B0 + (size_t)i * 32 * a.ldb;
        rb[SET][i] = *(const u32x4*)(Bk + kob + b_off);
      }
    }
  };
  auto lstore = [&](auto set_c, int st, auto r0_c, auto r1_c) {
    constexpr int SET = decltype(set_c)::value, R0 = decltype(r0_c)::value, R1 = decltype(r1_c)::value;
#pragma unroll
    for (int r = R0; r < R1; ++r) {
      if (r < BM / 32)
        *(u32x4*)&As[st][lrow + 32 * r][lk] = ra[SET][r];
      else
        *(u32x4*)&Bs[st][lrow + 32 * (r - BM / 32)][lk] = rb[SET][r - BM / 32];
    }
  };
  // the staging registers written out / reloaded in k-steps 0, 1, 2
  constexpr int NR = BM / 32 + BNT / 32;
  using R0_ = std::integral_constant<int, 0>;
  using R6_ = std::integral_constant<int, NR == 16 ? 6 : 4>;
  using R11_ = std::integral_constant<int, NR == 16 ? 11 : 8>;
  using R16_ = std::integral_constant<int, NR>;

  // B rows of this wave inside the LDS tile
  int brow[JB];
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    if (EPI == GEMM_SWIGLU_F16)
      brow[j] = (j < 2 ? 0 : BN / 2) + wn * 64 + (j & 1) * 32;
    else
      brow[j] = wn * (BNT / 2) + j * 32;
  }

  const int r32 = lane & 31, k8 = (lane >> 5) * 8;
  f16x8 fa0[4], fb0[JB], fa1[4], fb1[JB];
  auto frag_load = [&](f16x8 (&fa)[4], f16x8 (&fb)[JB], int st, int kk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *(const f16x8*)&As[st][wm * 128 + i * 32 + r32][kk + k8];
#pragma unroll
    for (int j = 0; j < JB; ++j) fb[j] = *(const f16x8*)&Bs[st][brow[j] + r32][kk + k8];
  };
  auto mfma16 = [&](const f16x8 (&fa)[4], const f16x8 (&fb)[JB]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  // 4 JB MFMAs with the 4 + JB fragment reads of the next step spread between them
  auto interleave_reads = [&]() {
    if constexpr (JB == 4) {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      }
    } else {
#pragma unroll
      for (int x = 0; x < 6; ++x) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
    }
  };

  // One k-tile t of parity PAR (the staging set of tile t+1 is PAR ^ 1).
  // Tile t+1 goes into the other LDS stage during k-steps 0-2 (that stage
  // is free since the previous barrier), and each staging register is
  // reloaded with tile t+3 right after it is written out, so LDS writes and
  // global loads are spread over three k-steps.  Past the last tile the loads
  // repeat the last tile (clamped index, results unused), so the body has no
  // branches: it is one basic block, which the instruction-group
  // interleaving needs.
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  const int kt_last = kt0 + nks - 1;
  // 4 JB MFMAs with 4 + JB fragment reads, up to 2 JB LDS writes and 2 JB
  // global loads
  auto interleave_all = [&]() {
#pragma unroll
    for (int x = 0; x < 2 * JB; ++x) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
    }
    if constexpr (JB == 2) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
  };
  auto ktile = [&](int t, auto par_c) {
    constexpr int PAR = decltype(par_c)::value;
    using NSET = std::integral_constant<int, PAR ^ 1>;
    const int st = t & 1;
    const int kt3 = min(kt0 + t + 3, kt_last);
    // k-step 0 (operands fa0/fb0), reads for step 1
    frag_load(fa1, fb1, st, 16);
    mfma16(fa0, fb0);
    lstore(NSET{}, st ^ 1, R0_{}, R6_{});
    gload(NSET{}, kt3, R0_{}, R6_{});
    interleave_all();
    __builtin_amdgcn_sched_barrier(0);
    // k-step 1, reads for step 2
    frag_load(fa0, fb0, st, 32);
    mfma16(fa1, fb1);
    lstore(NSET{}, st ^ 1, R6_{}, R11_{});
    gload(NSET{}, kt3, R6_{}, R11_{});
    interleave_all();
    __builtin_amdgcn_sched_barrier(0);
    // k-step 2, reads for step 3
    frag_load(fa1, fb1, st, 48);
    mfma16(fa0, fb0);
    lstore(NSET{}, st ^ 1, R11_{}, R16_{});
    gload(NSET{}, kt3, R11_{}, R16_{});
    interleave_all();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // k-step 3 (operands already in registers), first reads of the next tile
    frag_load(fa0, fb0, st ^ 1, 0);
    mfma16(fa1, fb1);
    interleave_reads();
    __builtin_amdgcn_sched_barrier(0);
  };

  gload(P0{}, kt0, R0_{}, R16_{});
  lstore(P0{}, 0, R0_{}, R16_{});
  __syncthreads();
  frag_load(fa0, fb0, 0, 0);
  gload(P1{}, min(kt0 + 1, kt_last), R0_{}, R16_{});
  gload(P0{}, min(kt0 + 2, kt_last), R0_{}, R16_{});
  int t = 0;
  for (; t + 1 < nks; t += 2) {
    ktile(t, P0{});
    ktile(t + 1, P1{});
  }
  if (t < nks) ktile(t, P0{});

  if constexpr (SPLIT) {
    // partial tile: value pair (v, v+1) of block (i, j) of thread tid sits at
    // float offset ((((i * 4 + j) * 8 + v / 2) * THREADS + tid) * 2, so each
    // 8-byte coherent store or load of a wave covers 512 contiguous bytes
    const int tile = by * gridDim.x + bx;
    const int S = a.splits;
    float* wsp = a.ws + (size_t)tile * S * (BM * BN);
    const coh_buf wsb = coh_buffer(wsp);
    const uint32_t own = (uint32_t)(bz * (BM * BN) + tid * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; v += 2)
          cstore2(wsb, own + (uint32_t)((((i * 4 + j) * 8 + v / 2) * THREADS) * 2), acc[i][j][v], acc[i][j][v + 1]);
    if (!last_block_arrive(a.counters + tile, (unsigned)S, &s_last)) return;
    // the last split re-reads every partial, its own included, and adds them
    // in split order (device-coherent buffer loads: batched, unlike atomic
    // loads, which wait for themselves one by one)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          float x, y;
          cload2(wsb, (uint32_t)((((i * 4 + j) * 8 + v / 2) * THREADS + tid) * 2), x, y);
          acc[i][j][v] = x;
          acc[i][j][v + 1] = y;
        }
      }
      for (int p = 1; p < S; ++p) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            float x, y;
            cload2(wsb, (uint32_t)(p * (BM * BN) + (((i * 4 + j) * 8 + v / 2) * THREADS + tid) * 2), x, y);
            acc[i][j][v] += x;
            acc[i][j][v + 1] += y;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // int8 codes as B: each column times its weight row's scale
  if (a.rs[0]) {
    const int c32 = lane & 31;
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      float sc;
      if constexpr (EPI == GEMM_SWIGLU_F16) {  // blocks 0, 1 gate, 2, 3 up, at the same rows
        sc = bf16_to_f32(a.rs[j >> 1][n0 + wn * 64 + (j & 1) * 32 + c32]);
      } else {
        const int n = n0 + wn * (BNT / 2) + j * 32 + c32;
        const int sg = (n >= a.rs_end[0]) + (n >= a.rs_end[1]);
        sc = bf16_to_f32(a.rs[sg][n - (sg == 0 ? 0 : a.rs_end[sg - 1])]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] *= sc;
    }
  }

  // epilogue: lane holds C[row][col], col = lane % 32,
  // row = 8 * (v / 4) + 4 * (lane / 32) + v % 4 inside each 32 x 32 block
  const int hi4 = (lane >> 5) * 4;
  if constexpr (EPI == GEMM_QKV_F16) {
    constexpr int D = 128, HD = 64, VT = 132;  // VT: halfs per transposed row in LDS (8-byte aligned rows)
    const int hh = (n0 + wn * 128) / D;  // this wave's head
    const bool is_q = hh < a.n_heads, is_v = hh >= a.n_heads + a.n_kv;
    __syncthreads();  // every wave is done with the tiles in LDS
    if (is_v) {
      // V^T rows (a channel's positions are contiguous in the cache): the
      // wave's 128 x 128 block goes through LDS transposed (waves 0, 1 in As,
      // 2, 3 in Bs), then each store covers consecutive positions
      _Float16* vt = (wave < 2 ? &As[0][0][0] : &Bs[0][0][0]) + (wave & 1) * (D * VT);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            vt[(j * 32 + r32) * VT + i * 32 + 8 * (v / 4) + hi4 + (v % 4)] = (_Float16)acc[i][j][v];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done (lgkmcnt(0))
      _Float16* const vb = (_Float16*)a.kv.base + kv_slab(a.kv, a.seq, a.layer, 1, hh - a.n_heads - a.n_kv);
      if ((a.start & 3) == 0) {
        // 4 positions per lane, two channels per store round (8-byte stores)
        const int r = 4 * (lane & 31), mr = m0 + wm * 128 + r;
        _Float16* const col = vb + (size_t)(lane >> 5) * a.kv.max_seq + a.start + mr;
        for (int c = 0; c < D; c += 2) {
          const u32x2 four = *(const u32x2*)&vt[(c + (lane >> 5)) * VT + r];
          _Float16* dst = col + (size_t)c * a.kv.max_seq;
          if (mr + 3 < a.M) {
            *(u32x2*)dst = four;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (mr + e < a.M) dst[e] = __builtin_bit_cast(_Float16, (uint16_t)((e < 2 ? four.x : four.y) >> (16 * (e & 1))));
          }
        }
      } else {
        const int r = 2 * lane, mr = m0 + wm * 128 + r;  // rows r, r + 1 of the block
        for (int c = 0; c < D; ++c) {
          const uint32_t two = *(const uint32_t*)&vt[c * VT + r];
          _Float16* dst = vb + (size_t)c * a.kv.max_seq + a.start + mr;
          if (mr < a.M) dst[0] = __builtin_bit_cast(_Float16, (uint16_t)(two & 0xFFFFu));
          if (mr + 1 < a.M) dst[1] = __builtin_bit_cast(_Float16, (uint16_t)(two >> 16));
        }
      }
      return;
    }
    const uint16_t* g = is_q ? a.qn : a.kn;
    float gj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) gj[j] = (g && !is_v) ? bf16_to_f32(g[j * 32 + r32]) : 1.f;
    _Float16* const qh = a.q16;
    _Float16* const ql = a.q16 + (size_t)a.M * a.n_heads * D;
    _Float16* const kb = is_q ? nullptr : (_Float16*)a.kv.base + kv_slab(a.kv, a.seq, a.layer, 0, hh - a.n_heads);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the RoPE values of this block's 16 rows first, all loads in flight together
      float c0[16], s0[16], c1[16], s1[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 128 + i * 32 + 8 * (v / 4) + hi4 + (v % 4);
        const size_t t = (size_t)(a.start + (m < a.M ? m : a.M - 1)) * HD;
        c0[v] = a.rope_cos[t + r32];
        s0[v] = a.rope_sin[t + r32];
        c1[v] = a.rope_cos[t + 32 + r32];
        s1[v] = a.rope_sin[t + 32 + r32];
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 128 + i * 32 + 8 * (v / 4) + hi4 + (v % 4);
        const bool ok = m < a.M;
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = acc[i][j][v];
        // every lane of the half-wave holding this row takes part (rows past M included)
        float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
        const float r = g ? rsqrtf(ss / (float)D + a.eps) : 1.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] *= r * gj[j];
        // rotate (c, c + 64) for c = r32 and c = 32 + r32 by pos * theta^(-2c/d)
        float y[4];
        y[0] = x[0] * c0[v] - x[2] * s0[v];
        y[2] = x[2] * c0[v] + x[0] * s0[v];
        y[1] = x[1] * c1[v] - x[3] * s1[v];
        y[3] = x[3] * c1[v] + x[1] * s1[v];
        // neighbour lanes swap so that each lane owns two adjacent columns:
        // an even lane (columns 2k of each block j) takes blocks 0 and 2, an odd
        // lane blocks 1 and 3; each lane then stores 4-byte pairs
        const bool even = (r32 & 1) == 0;
        const float t0 = __shfl_xor(even ? y[1] : y[0], 1, 64);
        const float t1 = __shfl_xor(even ? y[3] : y[2], 1, 64);
        float p[4];  // (first, second) of the two pairs
        p[0] = even ? y[0] : t0;
        p[1] = even ? t0 : y[1];
        p[2] = even ? y[2] : t1;
        p[3] = even ? t1 : y[3];
        const int cb = (r32 & ~1) + (even ? 0 : 32);  // first column of this lane's first pair
        if (!ok) continue;
        if (is_q) {
          const size_t o = ((size_t)m * a.n_heads + hh) * D + cb;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const _Float16 h0 = (_Float16)p[2 * u], h1 = (_Float16)p[2 * u + 1];
            const f16x2 hv = {h0, h1};
            const f16x2 lv = {(_Float16)(p[2 * u] - (float)h0), (_Float16)(p[2 * u + 1] - (float)h1)};
            *(f16x2*)(qh + o + 64 * u) = hv;
            *(f16x2*)(ql + o + 64 * u) = lv;
          }
        } else {
          _Float16* kr = kb + (size_t)(a.start + m) * D + cb;
#pragma unroll
          for (int u = 0; u < 2; ++u) *(f16x2*)(kr + 64 * u) = f16x2{(_Float16)p[2 * u], (_Float16)p[2 * u + 1]};
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * 128 + i * 32 + 8 * (v / 4) + hi4 + (v % 4);
      if (m >= a.M) continue;
      if constexpr (EPI == GEMM_SWIGLU_F16) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + wn * 64 + j * 32 + r32;
          const float g = acc[i][j][v], u = acc[i][j + 2][v];
          a.C16[(size_t)m * a.ldc16 + n] = (_Float16)(silu(g) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          const int n = n0 + wn * (BNT / 2) + j * 32 + r32;
          float* c = a.C + (size_t)m * a.ldc + n;
          if (EPI == GEMM_ADD_F32)
            *c += acc[i][j][v];
          else
            *c = acc[i][j][v];
        }
      }
    }
  }
}

template <int EPI>
void launch_epi(const GemmArgs& a, dim3 grid, bool narrow, hipStream_t stream) {
  if (a.splits > 1) {
    launch(gemm_kernel<EPI, true>, grid, dim3(THREADS), 0, stream, a);
  } else if constexpr (EPI != GEMM_SWIGLU_F16 && EPI != GEMM_QKV_F16) {
    if (narrow)
      launch(gemm_kernel<EPI, false, BN / 2>, grid, dim3(THREADS), 0, stream, a);
    else
      launch(gemm_kernel<EPI, false>, grid, dim3(THREADS), 0, stream, a);
  } else {
    launch(gemm_kernel<EPI, false>, grid, dim3(THREADS), 0, stream, a);
  }
}

// 256 x 128 tiles (no split) when 256 x 256 tiles leave CUs idle and the
// narrow ones still fit one round: the N = 4096 projections of a 2048-row
// prefill get 256 tiles instead of 128 split in two along K.
bool gemm_narrow(int M, int N, int epi, int n_cu) {
  if (epi == GEMM_SWIGLU_F16 || epi == GEMM_QKV_F16 || N % (BN / 2)) return false;
  const int mt = (M + BM - 1) / BM;
  return (N / BN) * mt < n_cu && (N / (BN / 2)) * mt <= n_cu;
}

int device_cus() {  // compute units of the current device (cached per device)
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace

bool gemm_prefers_narrow(int M, int N, int n_cu) { return gemm_narrow(M, N, GEMM_STORE_F32, n_cu); }

int gemm_choose_splits(int M, int N, int K, int epi, int n_cu) {
  if (K % BK) return 1;
  if (gemm_narrow(M, N, epi, n_cu)) return 1;
  const int ntile = (epi == GEMM_SWIGLU_F16) ? BN / 2 : BN;
  const int tiles = (N / ntile) * ((M + BM - 1) / BM);
  const int nk = K / BK;
  int best = 1;
  double best_t = 1e30;
  // the partial exchange costs about a quarter of a round, so a split must
  // save more than that
  for (int S = 1; S <= GEMM_MAX_SPLITS; S *= 2) {
    if (nk % S || nk / S < 4) break;
    if (S > 1 && (size_t)tiles * S > GEMM_WS_TILES) break;
    const int rounds = (tiles * S + n_cu - 1) / n_cu;
    const double t = (double)rounds / S + (S > 1 ? 0.25 : 0.0);
    if (t < best_t - 1e-9) {
      best_t = t;
      best = S;
    }
  }
  return best;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.K % BK || a.M < 1) return hipErrorInvalidValue;
  if (a.Kb && (a.Kb % BK || (a.K != a.Kb && a.K != 2 * a.Kb))) return hipErrorInvalidValue;
  const int S = a.splits < 1 ? 1 : a.splits;
  const bool narrow = S == 1 && gemm_narrow(a.M, a.N, a.epi, device_cus());
  const int ntile = (a.epi == GEMM_SWIGLU_F16 || narrow) ? BN / 2 : BN;
  if (a.N % ntile) return hipErrorInvalidValue;
  dim3 grid(a.N / ntile, (a.M + BM - 1) / BM, S);
  if (S > 1) {
    if (!a.ws || !a.counters || (a.K / BK) % S || (size_t)grid.x * grid.y * S > GEMM_WS_TILES)
      return hipErrorInvalidValue;
  }
  GemmArgs b = a;
  // one round of exactly 8 blocks of 4 x 4 tiles (with all their splits), or
  // of 4 x 8 narrow tiles
  const int bw = narrow ? 8 : 4;
  b.xcd_blocks = (grid.x % bw == 0 && grid.y % 4 == 0 && (grid.x / bw) * (grid.y / 4) == 8) ? 1 : 0;
  switch (a.epi) {
    case GEMM_STORE_F32: launch_epi<GEMM_STORE_F32>(b, grid, narrow, stream); break;
    case GEMM_ADD_F32: launch_epi<GEMM_ADD_F32>(b, grid, narrow, stream); break;
    case GEMM_SWIGLU_F16: launch_epi<GEMM_SWIGLU_F16>(b, grid, false, stream); break;
    case GEMM_QKV_F16:
      if (a.kv.is_f32 || a.kv.d != 128 || !a.q16 || !a.rope_cos || !a.rope_sin) return hipErrorInvalidValue;
      launch_epi<GEMM_QKV_F16>(b, grid, false, stream);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dpk
