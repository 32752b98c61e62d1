// Weight-streaming GEMV for decode steps (few activation rows, the whole K in
// one workgroup), gfx950 matrix cores.
//
//   y[m][n] = sum_k W[n][k] * x'[m][k],   x'[m][k] = x[m][k] * rs[m] * g[k]
//
// A decode step reads every weight once (oxinfer docs, "Performance"), so
// this kernel is an HBM stream: W is the A operand of v_mfma_f32_16x16x32_bf16
// straight from memory (16-byte loads, double buffered), x' the B operand from
// LDS, split into bf16 hi + lo so that activations keep fp32 precision.  4-bit
// MLX weights (w = s*c + b per 64 inputs; oxinfer docs, "MLX checkpoints")
// become the exact bf16 value 128 + c in registers and are rescaled per group:
//   sum_k w x = s * sum (128 + c) x + (b - 128 s) * sum x.
//
// A workgroup owns RB = 16 T rows; its four waves take a quarter of K each and
// are summed through LDS, so no partial sums leave the workgroup and the
// launch needs no cross-workgroup synchronisation (except the grid-wide
// argmax of the lm_head).  The RMSNorm scale of the input rows is rebuilt in
// the prologue from per-workgroup sums of squares written by the producer.
#include "common.h"
#include "kernels.h"

namespace dpk {

namespace {

constexpr int WAVES = 4;
constexpr int THREADS = 256;

__host__ __device__ inline int gemv_lds_layout(int M, int K, int RB, int fmt, int* xs_off, int* xsum_off,
                                                int* q_off, int* red_off, int* misc_off) {
  // per wave: hi and lo of M rows x K/4 (+8 pad) bf16
  const int kq = K / WAVES, xstride = kq + 8;
  int off = 0;
  *xs_off = off;
  off += WAVES * 2 * M * xstride * 2;
  off = (off + 15) & ~15;
  *xsum_off = off;
  off += (fmt == W_Q4 ? M * (K / 64) * 4 : 0);
  *q_off = off;
  off += (fmt == W_Q4 ? 2 * RB * (K / 64) * 4 : 0);
  off = (off + 15) & ~15;
  *red_off = off;
  off += WAVES * M * RB * 4;
  *misc_off = off;
  off += (64 + 16 * WAVES) * 4;
  return off;
}

template <int FMT, int T>
__global__ __launch_bounds__(THREADS) void gemv_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  constexpr int RB = 16 * T;
  const int M = a.M, K = a.K;
  const int kq = K / WAVES, xstride = kq + 8, ng = K / 64;
  int xs_off, xsum_off, q_off, red_off, misc_off;
  gemv_lds_layout(M, K, RB, FMT, &xs_off, &xsum_off, &q_off, &red_off, &misc_off);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int block = blockIdx.x;
  uint16_t* xs_hi = (uint16_t*)(lds + xs_off) + (size_t)wave * 2 * M * xstride;
  uint16_t* xs_lo = xs_hi + M * xstride;
  float* xsum = (float*)(lds + xsum_off);
  float* qsc = (float*)(lds + q_off);
  float* qbi = qsc + RB * ng;
  float* red = (float*)(lds + red_off);
  float* misc = (float*)(lds + misc_off);

  // row of segment `seg` that local row lr maps to
  auto seg_row = [&](int lr, int& seg, int& srow) {
    if (a.swiglu) {  // rows 0..RB/2-1 gate, RB/2..RB-1 up, both at block*RB/2 + r
      seg = lr / (RB / 2);
      srow = block * (RB / 2) + lr % (RB / 2);
      return;
    }
    const int n = block * RB + lr;
    seg = 0;
    int base = 0;
    while (seg < 2 && n >= a.seg_end[seg]) { base = a.seg_end[seg]; ++seg; }
    srow = n - base;
  };

  // ---- weight rows and the first weight loads: they do not depend on x, so
  // they are in flight while the prologue below builds the activations
  const int k0 = wave * kq;
  const int r16 = lane & 15, j4 = lane >> 4;
  const bool col_on = r16 < M;
  const unsigned char* wrow[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    int seg, srow;
    seg_row(t * 16 + r16, seg, srow);
    if (srow >= a.seg_rows[seg]) srow = a.seg_rows[seg] - 1;  // ragged tail: load a valid row
    wrow[t] = (const unsigned char*)a.w[seg] + (FMT == W_Q4 ? (size_t)srow * (K / 2) + k0 / 2
                                                              : ((size_t)srow * K + k0) * 2);
  }
  constexpr int U = 8 / T;  // bf16: k-steps of 32 per iteration (8 fragments per buffer)
  constexpr int KI = 32 * U;
  constexpr int GU = 4 / T > 0 ? 4 / T : 1;  // 4-bit: groups of 64 per iteration
  u32x4 b0[T][U], b1[T][U];
  u32x2 c0[T][GU], c1[T][GU];
  auto load_bf = [&](u32x4 (&b)[T][U], int it) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int u = 0; u < U; ++u)
        b[t][u] = __builtin_nontemporal_load((const u32x4*)(wrow[t] + (size_t)(it * KI + 32 * u + 8 * j4) * 2));
  };
  // 4-bit: per group of 64, lane (row r16, k group j4) reads the 16 codes
  // 64 g + 16 j4 .. +15 (8 bytes); MFMA step t2 uses codes 8 t2 .. 8 t2 + 7
  auto load_q4 = [&](u32x2 (&c)[T][GU], int it) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int u = 0; u < GU; ++u)
        c[t][u] = __builtin_nontemporal_load((const u32x2*)(wrow[t] + (size_t)((it * GU + u) * 64 + 16 * j4) / 2));
  };
  if constexpr (FMT == W_BF16)
    load_bf(b0, 0);
  else
    load_q4(c0, 0);

  // ---- row norm scales from the producer's per-workgroup sums of squares
  // (every wave computes them itself: no barrier between these loads and the
  // activation loads below)
  float* rsw = misc + 64 + 16 * wave;
  if (a.sq_in) {
    for (int m = 0; m < M; ++m) {
      float s = 0.f;
      for (int b = lane; b < a.sq_nb; b += 64) s += a.sq_in[m * a.sq_nb + b];
      s = wave_sum(s);
      if (lane == 0) rsw[m] = rsqrtf(s / (float)K + a.eps);
    }
  }

  // ---- prologue: this wave's K quarter of x' -> bf16 hi/lo
  for (int i = lane; i < M * (kq / 8); i += 64) {
    const int m = i / (kq / 8);
    const int kl = (i % (kq / 8)) * 8;
    const float* xp = a.x + (size_t)m * a.ldx + k0 + kl;
    const float4 v0 = *(const float4*)xp, v1 = *(const float4*)(xp + 4);
    float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    const float r = a.sq_in ? rsw[m] : 1.0f;
    if (a.gain) {
      const uint4 g = *(const uint4*)(a.gain + k0 + kl);
      const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] *= r * bf16lo_to_f32(gw[e]);
        v[2 * e + 1] *= r * bf16hi_to_f32(gw[e]);
      }
    } else if (a.sq_in) {
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
    }
  }
  if (FMT == W_Q4) {
    for (int i = tid; i < RB * ng; i += THREADS) {
      const int lr = i / ng, g = i % ng;
      int seg, srow;
      seg_row(lr, seg, srow);
      if (srow >= a.seg_rows[seg]) srow = a.seg_rows[seg] - 1;
      const size_t gi = (size_t)srow * ng + g;
      const float s = bf16_to_f32(a.sc[seg][gi]);
      qsc[lr * ng + g] = s;
      qbi[lr * ng + g] = bf16_to_f32(a.bi[seg][gi]) - 128.0f * s;
    }
  }
  __syncthreads();

  // ---- main loop over this wave's K quarter
  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (FMT == W_BF16) {
    const int nit = kq / KI;
    auto compute = [&](const u32x4 (&b)[T][U], int it) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        u32x4 bh = {0u, 0u, 0u, 0u}, bl = {0u, 0u, 0u, 0u};
        if (col_on) {
          bh = *(const u32x4*)(xs_hi + r16 * xstride + it * KI + 32 * u + 8 * j4);
          bl = *(const u32x4*)(xs_lo + r16 * xstride + it * KI + 32 * u + 8 * j4);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const bf16x8 A = __builtin_bit_cast(bf16x8, b[t][u]);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bh), acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bl), acc[t], 0, 0, 0);
        }
      }
    };
    for (int it = 0; it < nit; it += 2) {
      if (it + 1 < nit) load_bf(b1, it + 1);
      compute(b0, it);
      if (it + 2 < nit) load_bf(b0, it + 2);
      if (it + 1 < nit) compute(b1, it + 1);
    }
  } else {
    const int nit = kq / (64 * GU);
    auto compute = [&](const u32x2 (&c)[T][GU], int it) {
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        const int gl = it * GU + u;            // group inside this wave's quarter
        const int gg = k0 / 64 + gl;           // group inside the row
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
        const float sx = col_on ? xsum[r16 * ng + gg] : 0.f;
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int lr = t * 16 + 4 * j4 + v;
            acc[t][v] += qsc[lr * ng + gg] * ag[t][v] + qbi[lr * ng + gg] * sx;
          }
      }
    };
    for (int it = 0; it < nit; it += 2) {
      if (it + 1 < nit) load_q4(c1, it + 1);
      compute(c0, it);
      if (it + 2 < nit) load_q4(c0, it + 2);
      if (it + 1 < nit) compute(c1, it + 1);
    }
  }

  // ---- sum the four K quarters: D[n][m] lane layout rows 4 j4 + v, column r16
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (col_on) red[(wave * M + r16) * RB + t * 16 + 4 * j4 + v] = acc[t][v];
  __syncthreads();
  float* fin = red;  // reduced in place into the wave-0 slice
  for (int i = tid; i < M * RB; i += THREADS)
    fin[i] = ((red[i] + red[M * RB + i]) + red[2 * M * RB + i]) + red[3 * M * RB + i];
  __syncthreads();

  // ---- epilogues
  const int nb = gridDim.x;
  if (a.epi == EPI_STORE) {
    for (int i = tid; i < M * RB; i += THREADS) {
      const int m = i / RB, n = block * RB + i % RB;
      if (n < a.N) a.out[(size_t)m * a.ldo + n] = fin[i];
    }
    return;
  }
  if (a.epi == EPI_SWIGLU) {
    constexpr int HR = RB / 2;
    for (int i = tid; i < M * HR; i += THREADS) {
      const int m = i / HR, r = i % HR;
      const int n = block * HR + r;
      if (n < a.N) a.out[(size_t)m * a.ldo + n] = silu(fin[m * RB + r]) * fin[m * RB + HR + r];
    }
    return;
  }
  if (a.epi == EPI_RESID) {
    // h += y; per-workgroup sum of squares of the new h (the next kernel's norm)
    for (int m = 0; m < M; ++m) {
      float sq = 0.f;
      for (int r = tid; r < RB; r += THREADS) {
        const int n = block * RB + r;
        float* hp = a.out + (size_t)m * a.ldo + n;
        const float h = *hp + fin[m * RB + r];
        *hp = h;
        sq += h * h;
      }
      sq = block_sum(sq, misc + 16);
      if (tid == 0) a.sq_out[m * nb + block] = sq;
    }
    return;
  }
  if (a.epi == EPI_HEAD) {
    // logits + per-block (max, lowest index); the last block reduces them
    int* flag = (int*)(misc + 48);
    for (int m = 0; m < M; ++m) {
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int r = tid; r < RB; r += THREADS) {
        const int n = block * RB + r;
        if (n < a.N) {
          const float v = fin[m * RB + r];
          a.out[(size_t)m * a.ldo + n] = v;
          if (v > best) { best = v; bi = n; }
        }
      }
      wave_argmax(best, bi);
      __syncthreads();
      if (lane == 0) { misc[32 + wave] = best; ((int*)misc)[40 + wave] = bi; }
      __syncthreads();
      if (tid == 0) {
        for (int w = 1; w < WAVES; ++w) {
          const float v = misc[32 + w];
          const int ix = ((int*)misc)[40 + w];
          if (v > best || (v == best && ix < bi)) { best = v; bi = ix; }
        }
        coh_store(a.cand_val + m * nb + block, best);
        coh_store(a.cand_idx + m * nb + block, bi);
      }
    }
    if (!last_block_arrive(a.counters, nb, flag)) return;
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

size_t gemv_lds_bytes(int M, int K, int tiles, int fmt) {
  int a, b, c, d, e;
  return (size_t)gemv_lds_layout(M, K, 16 * tiles, fmt, &a, &b, &c, &d, &e);
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  const int RB = 16 * a.tiles;
  if (a.K % (WAVES * 256) || a.M < 1 || a.M > 16) return hipErrorInvalidValue;
  const size_t lds = gemv_lds_bytes(a.M, a.K, a.tiles, a.fmt);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  const int rows = a.swiglu ? 2 * a.N : a.N;
  dim3 grid((rows + RB - 1) / RB);
#define DPK_GEMV_CASE(F, T)                                                                \
  if (a.fmt == F && a.tiles == T) {                                                         \
    hipLaunchKernelGGL((gemv_kernel<F, T>), grid, dim3(THREADS), lds, stream, a);          \
    return hipGetLastError();                                                               \
  }
  DPK_GEMV_CASE(W_BF16, 1)
  DPK_GEMV_CASE(W_BF16, 2)
  DPK_GEMV_CASE(W_BF16, 4)
  DPK_GEMV_CASE(W_Q4, 1)
  DPK_GEMV_CASE(W_Q4, 2)
  DPK_GEMV_CASE(W_Q4, 4)
#undef DPK_GEMV_CASE
  return hipErrorInvalidValue;
}

}  // namespace dpk
