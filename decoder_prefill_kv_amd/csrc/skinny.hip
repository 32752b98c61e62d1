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
// int8 weights with one scale per output row (w = s * q) become the exact
// bf16 value q in registers; the row scale multiplies the accumulated sum.
// int8 weights in blocks of 32 with an fp32 scale per block (oxinfer docs,
// "Build and run": the q8 format) take the same registers; one MFMA k-step
// is one block, so each block's sum is scaled as it is added:
//   acc += s_b * sum_{k in b} q x.
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
  int xs_hi, xs_lo, xsum, qsc, qbi, fin, misc;
  int xstride;  // elements per activation row in LDS (kchunk + 8)
  int sstride;  // q8: floats per block of the transposed scale table (rows + 4)
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
  L.xsum = off; off += (fmt == W_Q4 ? M * ng * 4 : 0);
  // q8: scales [kchunk/32][rows + 4], so that a lane's four rows are one
  // 16-byte read and the staging writes spread over the banks
  L.sstride = rows + 4;
  L.qsc = off;  // fp32 s
  off += (fmt == W_Q4 ? rows * ng * 4 : fmt == W_I8 ? rows * 4 : fmt == W_Q8 ? (kchunk / 32) * L.sstride * 4 : 0);
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

  // ---- prologue: x'[m][k0 .. k0+kchunk) -> bf16 hi/lo in LDS
  for (int i = tid; i < M * (kchunk / 8); i += THREADS) {
    const int m = i / (kchunk / 8);
    const int k8 = (i % (kchunk / 8)) * 8;
    const float* xp = a.x + (size_t)m * a.ldx + k0 + k8;
    float4 v0 = *(const float4*)xp, v1 = *(const float4*)(xp + 4);
    float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
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
  if (FMT == W_Q8) {  // the block scales of this K chunk, transposed
    const int nbk = kchunk / 32;
    for (int i = tid; i < rows * nbk; i += THREADS) {
      const int lr = i / nbk, b = i % nbk;
      int seg, srow;
      map_row(a, block, lr, seg, srow);
      qsc[b * L.sstride + lr] = a.sf[seg][(size_t)srow * (a.K / 32) + k0 / 32 + b];
    }
  }
  __syncthreads();

  // ---- main loop: each wave owns T row tiles of 16 rows
  const int r16 = lane & 15;  // A row / B column / D column
  const int j4 = lane >> 4;   // k group of 8
  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool col_on = r16 < M;

  const unsigned char* wrow[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    int seg, srow;
    map_row(a, block, (wave * T + t) * 16 + r16, seg, srow);
    if (FMT == W_Q4)
      wrow[t] = (const unsigned char*)a.w[seg] + (size_t)srow * (a.K / 2) + k0 / 2;
    else if (FMT == W_I8 || FMT == W_Q8)
      wrow[t] = (const unsigned char*)a.w[seg] + (size_t)srow * a.K + k0;
    else
      wrow[t] = (const unsigned char*)a.w[seg] + (size_t)srow * a.K * 2 + (size_t)k0 * 2;
  }

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
  } else if (FMT == W_I8 || FMT == W_Q8) {
    // Activation column r16 of the MFMA B operand: rows past M read row 0
    // (their outputs are never stored), so the reads need no branch.
    const int xrow = col_on ? r16 : 0;
    // Two register buffers: the weights of the next 256 k are loaded while
    // this 256 k is multiplied.
    u32x2 wqa[T][8], wqb[T][8];
    auto load = [&](u32x2 (&wq)[T][8], int kk) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int s = 0; s < 8; ++s)
          wq[t][s] = __builtin_nontemporal_load((const u32x2*)(wrow[t] + kk + 32 * s + 8 * j4));
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the multiplies
    };
    auto mul = [&](const u32x2 (&wq)[T][8], int kk) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x4 bh = *(const u32x4*)(xs_hi + xrow * L.xstride + kk + 32 * s + 8 * j4);
        const u32x4 bl = *(const u32x4*)(xs_lo + xrow * L.xstride + kk + 32 * s + 8 * j4);
        f32x4 ag[T];
#pragma unroll
        for (int t = 0; t < T; ++t) ag[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < T; ++t) {
          // 8 int8 codes -> 8 exact bf16 values: an integer of at most 8 bits
          // is exact in fp32 and in the upper half of its fp32 bit pattern;
          // v_perm packs the upper halves of two values into one dword.
          uint32_t f[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t word = e < 4 ? wq[t][s].x : wq[t][s].y;
            f[e] = __float_as_uint((float)(int)(int8_t)((word >> (8 * (e & 3))) & 0xFFu));
          }
          const u32x4 av = {__builtin_amdgcn_perm(f[1], f[0], 0x07060302u), __builtin_amdgcn_perm(f[3], f[2], 0x07060302u),
                            __builtin_amdgcn_perm(f[5], f[4], 0x07060302u), __builtin_amdgcn_perm(f[7], f[6], 0x07060302u)};
          const bf16x8 A = __builtin_bit_cast(bf16x8, av);
          f32x4& d = (FMT == W_Q8) ? ag[t] : acc[t];
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bh), d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bl), d, 0, 0, 0);
        }
        if (FMT == W_Q8) {  // k-step s is block (kk / 32 + s): lane holds rows 4 j4 + v
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const float4 sb = *(const float4*)(qsc + (kk / 32 + s) * L.sstride + (wave * T + t) * 16 + 4 * j4);
            acc[t][0] += sb.x * ag[t][0];
            acc[t][1] += sb.y * ag[t][1];
            acc[t][2] += sb.z * ag[t][2];
            acc[t][3] += sb.w * ag[t][3];
          }
        }
      }
    };
    // (loads stay outside branches inside the loop, so that each wait
    // counts only the loads of the buffer it needs)
    load(wqa, 0);
    int kk = 0;
    for (; kk + 2 * KSTEP < kchunk; kk += 2 * KSTEP) {
      load(wqb, kk + KSTEP);
      mul(wqa, kk);
      load(wqa, kk + 2 * KSTEP);
      mul(wqb, kk + KSTEP);
    }
    if (kk + KSTEP < kchunk) {  // two passes left (kchunk is a multiple of 256)
      load(wqb, kk + KSTEP);
      mul(wqa, kk);
      mul(wqb, kk + KSTEP);
    } else {
      mul(wqa, kk);
    }
    if (FMT == W_I8) {  // row scales: lane holds rows 4 j4 + v of each tile
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] *= qsc[(wave * T + t) * 16 + 4 * j4 + v];
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

  // ---- D[n][m]: lane holds rows 4*j4+v of each tile, column m = r16
  const int nb = gridDim.x;
  if (a.ksplit == 1) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (col_on) fin[r16 * rows + (wave * T + t) * 16 + 4 * j4 + v] = acc[t][v];
    __syncthreads();
  } else {
    // partials [ks][M][nb*rows]
    const size_t ldp = (size_t)nb * rows;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (col_on)
          coh_store(a.part + ((size_t)ks * M + r16) * ldp + (size_t)block * rows + (wave * T + t) * 16 + 4 * j4 + v,
                    acc[t][v]);
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
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dpk
