// Weight-streaming GEMV for M <= 16 activation rows (decode, batched decode,
// speculative verify) on gfx950 matrix cores.
//
//   y[m][n] = sum_k W[n][k] * x'[m][k],   x'[m][k] = x[m][k] * rs[m] * g[k]
//
// Decode is memory bound: each weight byte is read once per step (oxinfer docs,
// "Performance": a generated token streams every dense weight once).  The
// weights are the MFMA A operand straight from HBM (16 rows x 32 k per
// v_mfma_f32_16x16x32_bf16); the activations are the B operand from LDS.  To
// keep fp32 activation precision, x' is split into bf16 hi + lo parts and both
// are multiplied (two MFMAs per weight fragment): the matrix cores have more
// than ten times the throughput that the HBM stream needs at M <= 16.
//
// 4-bit weights (MLX affine, group 64, w = s*c + b; oxinfer docs, "MLX
// checkpoints") are expanded in registers to the exact bf16 value 128 + c
// (bit pattern 0x4300 | c) and accumulated per group:
//   sum_k w x = s * sum (128+c) x + (b - 128 s) * sum x.
//
// int8 codes (one scale per output row, w = s * q; or blocks of 32 with an
// fp32 scale per block, oxinfer docs, "Build and run": the q8 format) go into
// fp16 MFMAs without a conversion: the byte q + 128 under the high byte 0x64
// is the fp16 integer 1152 + q.  The activations are fp16 hi + lo of x' times
// a power of two per row (its largest magnitude in the chunk brought to
// [2^14, 2^15), undone on the sums), and sum (1152 + q) x - 1152 sum x gives
// sum q x.  The row scale multiplies the finished sum; a block scale
// multiplies each MFMA k-step's sum (one k-step is one block):
//   acc += s_b * (sum_{k in b} (1152 + q) x - 1152 sum_{k in b} x),
// the block's MFMAs starting from the staged - 1152 sum x.  GGUF-style
// 4-bit blocks (Q4_0: w = d (c - 8), 32 codes per fp16 d; oxinfer docs, "Build
// and run": the q4 flag) take the same path with fp16 1024 + c (a nibble
// under 0x640) and the offset 1032.
//
// Grid: x = row blocks, y = K splits.  The workgroup that finishes a row block
// last sums the K-split partials in a fixed order (deterministic) and runs the
// fused epilogue; the last row block to finish runs the grid-wide tail
// (row norm scale, final argmax).
#include "common.h"
#include "kernels.h"

namespace dpk {

namespace {

constexpr int WAVES = 4;
constexpr int THREADS = WAVES * 64;
constexpr int KSTEP = 256;  // k per main-loop iteration (8 MFMA k-steps)

struct SkinnyLds {
  // offsets in bytes inside dynamic LDS
  int xs_hi, xs_lo, xsum, xsc, qsc, qbi, fin, misc;
  int xstride;  // elements per activation row in LDS (kchunk + 8)
  int total;
};

__host__ __device__ inline SkinnyLds skinny_lds_layout(int M, int kchunk, int rows, int fmt) {
  SkinnyLds L;
  L.xstride = kchunk + 8;
  int off = 0;
  L.xs_hi = off; off += M * L.xstride * 2;
  L.xs_lo = off; off += M * L.xstride * 2;
  off = (off + 15) & ~15;
  int ng = kchunk / 64;
  const bool i8f = fmt == W_I8 || fmt == W_Q8 || fmt == W_Q40;
  // q4: [M][kchunk/64] sums of x'; int8 codes: [kchunk/32][16] sums of the
  // scaled x' per block of 32, then 16 row maxima and 16 row unscales
  L.xsum = off; off += (fmt == W_Q4 ? M * ng * 4 : i8f ? (kchunk / 32) * 16 * 4 : 0);
  L.xsc = off; off += (i8f ? 32 * 4 : 0);
  L.qsc = off;  // fp32 s
  off += (fmt == W_Q4 ? rows * ng * 4 : fmt == W_I8 ? rows * 4 : 0);
  L.qbi = off; off += (fmt == W_Q4 ? rows * ng * 4 : 0);  // fp32 b - 128 s
  off = (off + 15) & ~15;
  L.fin = off; off += M * rows * 4;
  L.misc = off; off += 64 * 4;
  L.total = off;
  return L;
}

// map (block, local row) -> (segment, row inside segment) for each epilogue
DPK_DEV void map_row(const SkinnyArgs& a, int block, int lrow, int& seg, int& srow) {
  if (a.epi == EPI_SWIGLU) {
    const int half = a.rows_per_wg / 2;
    seg = lrow / half;
    srow = block * half + (lrow % half);
    return;
  }
  int n = block * a.rows_per_wg + lrow;
  seg = 0;
  int base = 0;
  while (seg < 2 && n >= a.seg_end[seg]) {
    base = a.seg_end[seg];
    ++seg;
  }
  srow = n - base;
}

template <int FMT, int T>
__global__ __launch_bounds__(THREADS) void skinny_kernel(SkinnyArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int M = a.M;
  const int rows = a.rows_per_wg;  // = WAVES * T * 16
  const int block = blockIdx.x;
  const int ks = blockIdx.y;
  const int k0 = ks * a.kchunk;
  const int kchunk = a.kchunk;
  const SkinnyLds L = skinny_lds_layout(M, kchunk, rows, FMT);
  uint16_t* xs_hi = (uint16_t*)(lds + L.xs_hi);
  uint16_t* xs_lo = (uint16_t*)(lds + L.xs_lo);
  float* xsum = (float*)(lds + L.xsum);
  float* qsc = (float*)(lds + L.qsc);
  float* qbi = (float*)(lds + L.qbi);
  float* fin = (float*)(lds + L.fin);
  int* misc = (int*)(lds + L.misc);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int ng = kchunk / 64;

  constexpr bool I8F = FMT == W_I8 || FMT == W_Q8 || FMT == W_Q40;  // integer codes
  constexpr bool BLK = FMT == W_Q8 || FMT == W_Q40;                   // a scale per 32 columns
  constexpr int TB = FMT == W_Q40 ? 2048 : 4096;  // code bytes per 16-row tile and 256 columns
  constexpr float OFF = FMT == W_Q40 ? 1032.0f : 1152.0f;  // the codes' fp16 value minus the weight's code
  constexpr int SB = FMT == W_Q40 ? 2 : 4;  // bytes per block scale in the fragment-order copy
  const int nbk = kchunk / 32;  // int8 formats: blocks of 32 columns in the chunk
  const int r16 = lane & 15;    // A row / B column / D column
  const int j4 = lane >> 4;     // k group of 8
  const bool col_on = r16 < M;
  // Activation column r16 of the MFMA B operand: rows past M read row 0
  // (their outputs are never stored), so the reads need no branch.
  const int xrow = col_on ? r16 : 0;

  const unsigned char* wrow[T];
  const unsigned char* srow_sf[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    int seg, srow;
    map_row(a, block, (wave * T + t) * 16 + r16, seg, srow);
    if (FMT == W_Q4)
      wrow[t] = (const unsigned char*)a.w[seg] + (size_t)srow * (a.K / 2) + k0 / 2;
    else if (I8F) {  // fragment-order codes: this tile's 4 / 2 KB per 256 columns, this lane's 16 bytes
      wrow[t] = (const unsigned char*)a.w[seg] + ((size_t)(srow >> 4) * (a.K / 256) + k0 / 256) * TB + lane * 16;
      if (BLK)  // fragment-order block scales per tile and 256 columns, row r16's 8: Q8 fp32 (512 bytes,
                // at r16 * 32), Q4_0 fp16 (256 bytes, at r16 * 16)
        srow_sf[t] = (const unsigned char*)a.sf[seg] + ((size_t)(srow >> 4) * (a.K / 256) + k0 / 256) * (SB * 128) +
                     r16 * (SB * 8);
    } else
      wrow[t] = (const unsigned char*)a.w[seg] + (size_t)srow * a.K * 2 + (size_t)k0 * 2;
  }
  // integer codes: two register buffers of 256 columns (a wave reads 1 KB in
  // one 16-byte-per-lane load: two k-steps of int8 codes, four of 4-bit ones);
  // the first is requested before the prologue, the next while the current
  // one is multiplied (block formats: with the 8 scales of the lane's row)
  u32x4 wqa[T][4], wqb[T][4], sqa[T][2], sqb[T][2];
  auto load = [&](u32x4 (&wq)[T][4], u32x4 (&sq)[T][2], int kk) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int p = 0; p < TB / 1024; ++p)
        wq[t][p] = __builtin_nontemporal_load((const u32x4*)(wrow[t] + kk * (TB / 256) + p * 1024));
      if constexpr (BLK) {
        sq[t][0] = __builtin_nontemporal_load((const u32x4*)(srow_sf[t] + kk * SB / 2));
        if constexpr (SB == 4) sq[t][1] = __builtin_nontemporal_load((const u32x4*)(srow_sf[t] + kk * 2 + 16));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of what follows
  };
  if constexpr (I8F) load(wqa, sqa, 0);

  // x'[m][k8 .. k8 + 8) of this chunk (x * rs * g in fp32)
  auto xprime = [&](int m, int k8, float (&v)[8]) {
    const float* xp = a.x + (size_t)m * a.ldx + k0 + k8;
    const float4 v0 = *(const float4*)xp, v1 = *(const float4*)(xp + 4);
    v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
    v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    const float r = a.rs ? a.rs[m] : 1.0f;
    if (a.gain) {
      const uint4 g = *(const uint4*)(a.gain + k0 + k8);
      const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] *= r * bf16lo_to_f32(gw[e]);
        v[2 * e + 1] *= r * bf16hi_to_f32(gw[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= r;
    }
  };

  if constexpr (I8F) {
    // ---- prologue (int8 codes): x' scaled by a power of two per row so that
    // its largest magnitude in the chunk lies in [2^14, 2^15), then split
    // into fp16 hi + lo; per block of 32 columns the sum of hi + lo, which
    // the code offset needs (the codes enter the MFMA as fp16 1152 + q).
    unsigned* rmax = (unsigned*)(lds + L.xsc);
    float* xunscale = (float*)(lds + L.xsc) + 16;
    if (tid < 16) {
      rmax[tid] = 0u;
      xunscale[tid] = 1.0f;
    }
    __syncthreads();
    for (int i = tid; i < M * (kchunk / 8); i += THREADS) {
      const int m = i / (kchunk / 8), k8 = (i % (kchunk / 8)) * 8;
      float v[8];
      xprime(m, k8, v);
      float mx = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
      if (mx != mx) mx = __uint_as_float(0x7fc00000u);  // a NaN wins the maximum
      atomicMax(&rmax[m], __float_as_uint(mx));  // non-negative floats order as their bits
    }
    __syncthreads();
    for (int i = tid; i < M * (kchunk / 8); i += THREADS) {
      const int m = i / (kchunk / 8), k8 = (i % (kchunk / 8)) * 8;
      float v[8];
      xprime(m, k8, v);
      const float mx = __uint_as_float(rmax[m]);
      int ex = 0;
      if (mx > 0.f && mx <= 3.0e38f) frexpf(mx, &ex);  // mx = f 2^ex, f in [0.5, 1)
      const int sh = min(max(15 - ex, -100), 100);
      const float sc = ldexpf(1.0f, sh);
      uint32_t hl[8], ll[8];
      float bs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = v[e] * sc;
        const _Float16 h = (_Float16)x;
        const _Float16 l = (_Float16)(x - (float)h);
        bs += (float)h + (float)l;
        hl[e] = __builtin_bit_cast(uint16_t, h);
        ll[e] = __builtin_bit_cast(uint16_t, l);
      }
      *(uint4*)(xs_hi + m * L.xstride + k8) =
          uint4{hl[0] | (hl[1] << 16), hl[2] | (hl[3] << 16), hl[4] | (hl[5] << 16), hl[6] | (hl[7] << 16)};
      *(uint4*)(xs_lo + m * L.xstride + k8) =
          uint4{ll[0] | (ll[1] << 16), ll[2] | (ll[3] << 16), ll[4] | (ll[5] << 16), ll[6] | (ll[7] << 16)};
      // 4 consecutive threads cover one block of 32 (kchunk / 8 is a multiple of 32)
      bs += __shfl_xor(bs, 1, 64);
      bs += __shfl_xor(bs, 2, 64);
      // (block formats keep - o * sum, the accumulator a block's MFMAs start from)
      if ((k8 & 31) == 0) xsum[(k8 / 32) * 16 + m] = BLK ? -OFF * bs : bs;
      if (k8 == 0) xunscale[m] = ldexpf(1.0f, -sh);
    }
  } else {
    // ---- prologue: x'[m][k0 .. k0+kchunk) -> bf16 hi/lo in LDS
    for (int i = tid; i < M * (kchunk / 8); i += THREADS) {
      const int m = i / (kchunk / 8);
      const int k8 = (i % (kchunk / 8)) * 8;
      float v[8];
      xprime(m, k8, v);
      // q4 codes pair nibble p with nibble p+4 inside a packed dword, so the
      // activation slots are permuted the same way: (0,4,1,5,2,6,3,7)
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int src = (FMT == W_Q4) ? ((e & 1) ? (e >> 1) + 4 : (e >> 1)) : e;
        split_bf16(v[src], hi[e], lo[e]);
      }
      uint4 H, Lo;
      H.x = hi[0] | (hi[1] << 16); H.y = hi[2] | (hi[3] << 16);
      H.z = hi[4] | (hi[5] << 16); H.w = hi[6] | (hi[7] << 16);
      Lo.x = lo[0] | (lo[1] << 16); Lo.y = lo[2] | (lo[3] << 16);
      Lo.z = lo[4] | (lo[5] << 16); Lo.w = lo[6] | (lo[7] << 16);
      *(uint4*)(xs_hi + m * L.xstride + k8) = H;
      *(uint4*)(xs_lo + m * L.xstride + k8) = Lo;
      if (FMT == W_Q4) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s += v[e];
        // 8 consecutive threads cover one group of 64: reduce over them
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64);
        if ((k8 & 63) == 0) xsum[m * ng + k8 / 64] = s;
      }
    }
  }
  if (FMT == W_Q4) {
    // per-row scale s and offset b - 128 s for this workgroup's rows
    for (int i = tid; i < rows * ng; i += THREADS) {
      const int lr = i / ng, g = i % ng;
      int seg, srow;
      map_row(a, block, lr, seg, srow);
      const size_t gi = (size_t)srow * (a.K / 64) + (k0 / 64) + g;
      const float s = bf16_to_f32(a.sc[seg][gi]);
      const float b = bf16_to_f32(a.bi[seg][gi]);
      qsc[lr * ng + g] = s;
      qbi[lr * ng + g] = b - 128.0f * s;
    }
  }
  if (FMT == W_I8) {  // the workgroup's row scales
    for (int i = tid; i < rows; i += THREADS) {
      int seg, srow;
      map_row(a, block, i, seg, srow);
      qsc[i] = bf16_to_f32(a.sc[seg][srow]);
    }
  }
  __syncthreads();

  // ---- main loop: each wave owns T row tiles of 16 rows
  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (FMT == W_BF16) {
    for (int kk = 0; kk < kchunk; kk += KSTEP) {
      u32x4 wa[T][8];
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int s = 0; s < 8; ++s)
          wa[t][s] = __builtin_nontemporal_load((const u32x4*)(wrow[t] + (size_t)(kk + 32 * s + 8 * j4) * 2));
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        u32x4 bh = {0u, 0u, 0u, 0u}, bl = {0u, 0u, 0u, 0u};
        if (col_on) {
          bh = *(const u32x4*)(xs_hi + r16 * L.xstride + kk + 32 * s + 8 * j4);
          bl = *(const u32x4*)(xs_lo + r16 * L.xstride + kk + 32 * s + 8 * j4);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const bf16x8 A = __builtin_bit_cast(bf16x8, wa[t][s]);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bh), acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bl), acc[t], 0, 0, 0);
        }
      }
    }
  } else if (I8F) {
    // Codes as fp16 without a conversion: byte q ^ 0x80 = q + 128 becomes the
    // low byte of an fp16 whose high byte is 0x64, i.e. 1024 + q + 128 (fp16
    // integers are exact up to 2048), so the MFMA sums (1152 + q) x and
    // 1152 * sum x is subtracted.  One v_perm places two codes.  The
    // activations are the A operand and the codes the B operand, so a lane's
    // four results share one weight row (r16 of the tile) and one scale:
    // D[m = 4 j4 + v][n = r16].
    auto mul = [&](const u32x4 (&wq)[T][4], const u32x4 (&sq)[T][2], int kk) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const f16x8 Xh = __builtin_bit_cast(f16x8, *(const u32x4*)(xs_hi + xrow * L.xstride + kk + 32 * s + 8 * j4));
        const f16x8 Xl = __builtin_bit_cast(f16x8, *(const u32x4*)(xs_lo + xrow * L.xstride + kk + 32 * s + 8 * j4));
        // block formats: - o sum x of rows 4 j4 .. + 3 over block kk / 32 + s
        const f32x4 c0 = BLK ? *(const f32x4*)(xsum + (kk / 32 + s) * 16 + 4 * j4) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < T; ++t) {
          // this lane's codes of k-step s: weight row r16, columns 32 s + 8 j4 .. + 7
          u32x4 bv;
          if constexpr (FMT == W_Q40) {
            // 4-bit: one dword, nibble n holding element 2n (n < 4) or
            // 2 (n - 4) + 1, so each shift and mask gives elements 2p, 2p + 1
            // as fp16 1024 + c
            const uint32_t w = wq[t][s >> 2][s & 3];
            bv = u32x4{0x64006400u | (w & 0x000F000Fu), 0x64006400u | ((w >> 4) & 0x000F000Fu),
                       0x64006400u | ((w >> 8) & 0x000F000Fu), 0x64006400u | ((w >> 12) & 0x000F000Fu)};
          } else {
            const uint32_t u0 = ((s & 1) ? wq[t][s >> 1].z : wq[t][s >> 1].x) ^ 0x80808080u;
            const uint32_t u1 = ((s & 1) ? wq[t][s >> 1].w : wq[t][s >> 1].y) ^ 0x80808080u;
            bv = u32x4{__builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u),
                       __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u),
                       __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u),
                       __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)};
          }
          const f16x8 B = __builtin_bit_cast(f16x8, bv);
          if constexpr (BLK) {
            // the block's sum of (o + q) x started from - o sum x (o = 1152
            // for int8 codes, 1032 for 4-bit codes around 8, staged per row
            // and block), so the offset leaves inside the block sum; then the
            // block scale of the lane's weight row
            f32x4 ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(Xh, B, c0, 0, 0, 0);
            ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(Xl, B, ag, 0, 0, 0);
            float sb;
            if constexpr (SB == 4) {
              sb = __uint_as_float(sq[t][s >> 2][s & 3]);
            } else {  // (fp16: half s % 2 of word s / 2)
              const uint32_t wd = sq[t][0][s >> 1];
              sb = (float)__builtin_bit_cast(_Float16, (uint16_t)((s & 1) ? (wd >> 16) : (wd & 0xFFFFu)));
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[t][v] += sb * ag[v];
          } else {
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Xh, B, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Xl, B, acc[t], 0, 0, 0);
          }
        }
      }
    };
    // (loads stay outside branches inside the loop, so that each wait
    // counts only the loads of the buffer it needs)
    int kk = 0;
    for (; kk + 2 * KSTEP < kchunk; kk += 2 * KSTEP) {
      load(wqb, sqb, kk + KSTEP);
      mul(wqa, sqa, kk);
      load(wqa, sqa, kk + 2 * KSTEP);
      mul(wqb, sqb, kk + KSTEP);
    }
    if (kk + KSTEP < kchunk) {  // two passes left (kchunk is a multiple of 256)
      load(wqb, sqb, kk + KSTEP);
      mul(wqa, sqa, kk);
      mul(wqb, sqb, kk + KSTEP);
    } else {
      mul(wqa, sqa, kk);
    }
    // activation row m = 4 j4 + v: undo its power of two; i8: the code offset
    // and the weight row's scale
    const float* xunscale = (const float*)(lds + L.xsc) + 16;
    float sx[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (FMT == W_I8) {
      // sum x of rows 4 j4 + v over the chunk: the 16 lanes of a j4 group
      // take every 16th block, then a butterfly over them (fixed order)
      for (int b = r16; b < nbk; b += 16) {
        const float4 xs4 = *(const float4*)(xsum + b * 16 + 4 * j4);
        sx[0] += xs4.x; sx[1] += xs4.y; sx[2] += xs4.z; sx[3] += xs4.w;
      }
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) sx[v] += __shfl_xor(sx[v], o, 64);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * j4 + v;
      const float us = xunscale[m];
      if constexpr (FMT == W_I8) {
        const float c = 1152.0f * sx[v];
#pragma unroll
        for (int t = 0; t < T; ++t) acc[t][v] = (acc[t][v] - c) * qsc[(wave * T + t) * 16 + r16] * us;
      } else {
#pragma unroll
        for (int t = 0; t < T; ++t) acc[t][v] *= us;
      }
    }
  } else {  // W_Q4: per group of 64: lane k range 64g + 16 j4 + 8 t2 + e, t2 in {0,1}
    for (int kk = 0; kk < kchunk; kk += KSTEP) {
      u32x2 wc[T][4];
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          wc[t][g] = __builtin_nontemporal_load((const u32x2*)(wrow[t] + (size_t)(kk + 64 * g + 16 * j4) / 2));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gi = (kk >> 6) + g;
        f32x4 ag[T];
#pragma unroll
        for (int t = 0; t < T; ++t) ag[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          u32x4 bh = {0u, 0u, 0u, 0u}, bl = {0u, 0u, 0u, 0u};
          const int koff = kk + 64 * g + 16 * j4 + 8 * t2;
          if (col_on) {
            bh = *(const u32x4*)(xs_hi + r16 * L.xstride + koff);
            bl = *(const u32x4*)(xs_lo + r16 * L.xstride + koff);
          }
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const uint32_t w = wc[t][g][t2];
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
        const float sx = col_on ? xsum[r16 * ng + gi] : 0.f;
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int lr = (wave * T + t) * 16 + 4 * j4 + v;
            acc[t][v] += qsc[lr * ng + gi] * ag[t][v] + qbi[lr * ng + gi] * sx;
          }
        }
      }
    }
  }

  // ---- D[n][m]: lane holds rows 4*j4+v of each tile, column m = r16 (int8
  // codes: activation rows m = 4*j4+v, weight row r16 of each tile)
  const int nb = gridDim.x;
  auto res_m = [&](int v) { return I8F ? 4 * j4 + v : r16; };
  auto res_n = [&](int t, int v) { return (wave * T + t) * 16 + (I8F ? r16 : 4 * j4 + v); };
  if (a.ksplit == 1) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (res_m(v) < M) fin[res_m(v) * rows + res_n(t, v)] = acc[t][v];
    __syncthreads();
  } else {
    // partials [ks][M][nb*rows]
    const size_t ldp = (size_t)nb * rows;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (res_m(v) < M)
          coh_store(a.part + ((size_t)ks * M + res_m(v)) * ldp + (size_t)block * rows + res_n(t, v), acc[t][v]);
    if (!last_block_arrive(a.counters + 1 + block, a.ksplit, misc)) return;
    for (int i = tid; i < M * rows; i += THREADS) {
      const int m = i / rows, lr = i % rows;
      const float* src = a.part + (size_t)m * ldp + (size_t)block * rows + lr;
      const size_t kstride = (size_t)M * ldp;
      // independent loads first (fixed summation order k2 = 0..ksplit-1)
      float v[16];
#pragma unroll
      for (int k2 = 0; k2 < 16; ++k2) v[k2] = (k2 < a.ksplit) ? coh_load(src + k2 * kstride) : 0.f;
      float s = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < 16; ++k2) s += v[k2];
      fin[m * rows + lr] = s;
    }
    __syncthreads();
  }

  // ---- fused epilogues
  if (a.epi == EPI_STORE) {
    for (int i = tid; i < M * rows; i += THREADS) {
      const int m = i / rows, lr = i % rows;
      const int n = block * rows + lr;
      if (n < a.N) a.out[(size_t)m * a.ldo + n] = fin[i];
    }
    return;
  }
  if (a.epi == EPI_RESID) {
    // h += y; per-row partial sum of squares of the new h for the next norm
    float* red = (float*)misc;
    for (int m = 0; m < M; ++m) {
      float sq = 0.f;
      for (int lr = tid; lr < rows; lr += THREADS) {
        const int n = block * rows + lr;
        float h = a.out[(size_t)m * a.ldo + n] + fin[m * rows + lr];
        a.out[(size_t)m * a.ldo + n] = h;
        sq += h * h;
      }
      sq = block_sum(sq, red + 16);
      if (tid == 0) coh_store(a.sq + m * nb + block, sq);
    }
    if (!last_block_arrive(a.counters, nb, misc)) return;
    // rs[m] = rsqrt(sum_b sq[m][b] / N + eps): one wave per row, lanes stride
    // the blocks with independent loads, fixed-order wave reduction
    for (int m = wave; m < M; m += WAVES) {
      float s = 0.f;
      for (int b0 = 0; b0 < nb; b0 += 256) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int b = b0 + lane + 64 * u;
          v[u] = b < nb ? coh_load(a.sq + m * nb + b) : 0.f;
        }
        s += (v[0] + v[1]) + (v[2] + v[3]);
      }
      s = wave_sum(s);
      if (lane == 0) a.rs_out[m] = rsqrtf(s / (float)a.N + a.eps);
    }
    return;
  }
  if (a.epi == EPI_SWIGLU) {
    const int half = rows / 2;
    for (int i = tid; i < M * half; i += THREADS) {
      const int m = i / half, r = i % half;
      const float g = fin[m * rows + r], u = fin[m * rows + half + r];
      a.out[(size_t)m * a.ldo + block * half + r] = silu(g) * u;
    }
    return;
  }
  if (a.epi == EPI_QKV) {
    // this block is one head (rows == head_dim): q / k heads get RMSNorm over
    // head_dim and RoPE; k and v go into the KV cache at the row's position
    const int d = rows, hd2 = d / 2;
    const int n0 = block * rows;
    int seg = 0, base = 0;
    while (seg < 2 && n0 >= a.seg_end[seg]) { base = a.seg_end[seg]; ++seg; }
    const int head = (n0 - base) / d;
    float* red = (float*)misc;
    for (int m = 0; m < M; ++m) {
      const RowParam rp = a.rows_param[m];
      const float* f = fin + m * rows;
      if (seg == 2) {  // v: V^T layout [d][max_seq]
        if (a.kv.i8) {  // int8 cache (d == 128): wave 0 quantizes the vector
          if (tid < 64) kv_put_i8(a.kv, rp.seq, a.layer, 1, head, rp.pos, f[tid], f[tid + 64], tid);
          continue;
        }
        for (int e = tid; e < d; e += THREADS) {
          const size_t off = kv_offset(a.kv, rp.seq, a.layer, 1, head, e, rp.pos);
          kv_store(a.kv, off, f[e]);
        }
        continue;
      }
      float ss = 0.f;
      for (int e = tid; e < d; e += THREADS) ss += f[e] * f[e];
      ss = block_sum(ss, red + 16);
      const float r = rsqrtf(ss / (float)d + a.eps);
      const uint16_t* gn = (seg == 0) ? a.qn : a.kn;
      for (int e = tid; e < hd2; e += THREADS) {
        float x1 = f[e] * r, x2 = f[e + hd2] * r;
        if (gn) {
          x1 *= bf16_to_f32(gn[e]);
          x2 *= bf16_to_f32(gn[e + hd2]);
        }
        const float c = a.rope_cos[(size_t)rp.pos * hd2 + e];
        const float s = a.rope_sin[(size_t)rp.pos * hd2 + e];
        const float y1 = x1 * c - x2 * s, y2 = x2 * c + x1 * s;
        if (seg == 0) {
          float* q = a.qout + ((size_t)m * a.n_heads + head) * d;
          q[e] = y1;
          q[e + hd2] = y2;
        } else if (a.kv.i8) {  // (d == 128: wave 0, one element pair per lane)
          kv_put_i8(a.kv, rp.seq, a.layer, 0, head, rp.pos, y1, y2, tid);
        } else {
          kv_store(a.kv, kv_offset(a.kv, rp.seq, a.layer, 0, head, 0, rp.pos) + e, y1);
          kv_store(a.kv, kv_offset(a.kv, rp.seq, a.layer, 0, head, 0, rp.pos) + e + hd2, y2);
        }
      }
    }
    return;
  }
  if (a.epi == EPI_HEAD) {
    // logits + per-block (max, lowest index) candidates; last block: argmax
    for (int m = 0; m < M; ++m) {
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int lr = tid; lr < rows; lr += THREADS) {
        const int n = block * rows + lr;
        if (n < a.N) {
          const float v = fin[m * rows + lr];
          a.out[(size_t)m * a.ldo + n] = v;
          if (v > best || (v == best && n < bi)) { best = v; bi = n; }
        }
      }
      wave_argmax(best, bi);
      float* rv = (float*)misc;
      int* ri = misc + 8;
      __syncthreads();
      if (lane == 0) { rv[wave] = best; ri[wave] = bi; }
      __syncthreads();
      if (tid == 0) {
        float bv = rv[0];
        int bx = ri[0];
        for (int w = 1; w < WAVES; ++w)
          if (rv[w] > bv || (rv[w] == bv && ri[w] < bx)) { bv = rv[w]; bx = ri[w]; }
        coh_store(a.cand_val + m * nb + block, bv);
        coh_store(a.cand_idx + m * nb + block, bx);
      }
      __syncthreads();
    }
    if (!last_block_arrive(a.counters, nb, misc + 32)) return;
    for (int m = wave; m < M; m += WAVES) {
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int b0 = 0; b0 < nb; b0 += 512) {
        float v[8];
        int ix[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int b = b0 + lane + 64 * u;
          v[u] = b < nb ? coh_load(a.cand_val + m * nb + b) : -INFINITY;
          ix[u] = b < nb ? coh_load(a.cand_idx + m * nb + b) : 0x7fffffff;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (v[u] > best || (v[u] == best && ix[u] < bi)) { best = v[u]; bi = ix[u]; }
      }
      wave_argmax(best, bi);
      if (lane == 0 && a.argmax_out) a.argmax_out[m] = bi;
    }
    return;
  }
}

}  // namespace

size_t skinny_lds_bytes(int M, int kchunk, int rows, int fmt) {
  return (size_t)skinny_lds_layout(M, kchunk, rows, fmt).total;
}

hipError_t launch_skinny(const SkinnyArgs& a, hipStream_t stream) {
  const int tiles = a.rows_per_wg / (WAVES * 16);
  dim3 grid(a.n_blocks, a.ksplit), block(THREADS);
  const size_t lds = skinny_lds_bytes(a.M, a.kchunk, a.rows_per_wg, a.fmt);
  if (a.fmt == W_BF16 && tiles == 1) launch((skinny_kernel<W_BF16, 1>), grid, block, lds, stream, a);
  else if (a.fmt == W_BF16 && tiles == 2) launch((skinny_kernel<W_BF16, 2>), grid, block, lds, stream, a);
  else if (a.fmt == W_Q4 && tiles == 1) launch((skinny_kernel<W_Q4, 1>), grid, block, lds, stream, a);
  else if (a.fmt == W_Q4 && tiles == 2) launch((skinny_kernel<W_Q4, 2>), grid, block, lds, stream, a);
  else if (a.fmt == W_I8 && tiles == 1) launch((skinny_kernel<W_I8, 1>), grid, block, lds, stream, a);
  else if (a.fmt == W_I8 && tiles == 2) launch((skinny_kernel<W_I8, 2>), grid, block, lds, stream, a);
  else if (a.fmt == W_Q8 && tiles == 1) launch((skinny_kernel<W_Q8, 1>), grid, block, lds, stream, a);
  else if (a.fmt == W_Q8 && tiles == 2) launch((skinny_kernel<W_Q8, 2>), grid, block, lds, stream, a);
  else if (a.fmt == W_Q40 && tiles == 1) launch((skinny_kernel<W_Q40, 1>), grid, block, lds, stream, a);
  else if (a.fmt == W_Q40 && tiles == 2) launch((skinny_kernel<W_Q40, 2>), grid, block, lds, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dpk
