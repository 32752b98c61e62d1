// Weight-streaming GEMV for decode steps (few activation rows, the whole K in
// one workgroup), gfx950 matrix cores.
//
//   y[m][n] = sum_k W[n][k] * x'[m][k],   x'[m][k] = x[m][k] * rs[m] * g[k]
//
// A decode step reads every weight once (oxinfer docs, "Performance"), so
// this kernel is an HBM stream.  W is the A operand of
// v_mfma_f32_16x16x32_bf16 straight from memory, x' the B operand from LDS,
// split into bf16 hi + lo so that the activations keep fp32 precision.  4-bit
// MLX weights (w = s*c + b per 64 inputs; oxinfer docs, "MLX checkpoints")
// become the exact bf16 value 128 + c in registers and are rescaled per group:
//   sum_k w x = s * sum (128 + c) x + (b - 128 s) * sum x.
//
// Weights are read from a copy re-tiled at load time into MFMA fragment order
// (one 1 KB block = the A operand of one 16-row x 32-column step, lane order),
// so every wave reads one contiguous stream.  A workgroup stages x' once and
// then walks row tiles blockIdx.x, blockIdx.x + gridDim.x, ...; its waves
// split K and are summed through LDS, and the next tile's first weights are
// already loading while the current tile's epilogue runs.  No partial sums
// leave a workgroup; the only grid-wide step is the lm_head's argmax.  The
// RMSNorm scale of the input rows is rebuilt in the prologue from per-tile
// sums of squares written by the producer.
#include "common.h"
#include "kernels.h"

namespace dpk {

namespace {

__host__ __device__ inline int gemv_lds_layout(int M, int K, int RB, int fmt, int WAVES, int* xs_off,
                                                int* xsum_off, int* red_off, int* misc_off) {
  const int kq = K / WAVES, xstride = kq + 8;
  int off = 0;
  *xs_off = off;  // per wave: hi and lo of M rows x K/WAVES (+8 pad) bf16
  off += WAVES * 2 * M * xstride * 2;
  off = (off + 15) & ~15;
  *xsum_off = off;
  off += (fmt == W_Q4 ? M * (K / 64) * 4 : 0);
  off = (off + 15) & ~15;
  *red_off = off;
  off += WAVES * M * RB * 4;
  *misc_off = off;
  off += (64 + 16 * WAVES) * 4;
  return off;
}

template <int FMT, int T, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  constexpr int RB = 16 * T;
  constexpr int THREADS = 64 * WAVES;
  const int M = a.M, K = a.K;
  const int kq = K / WAVES, xstride = kq + 8, ng = K / 64;
  int xs_off, xsum_off, red_off, misc_off;
  gemv_lds_layout(M, K, RB, FMT, WAVES, &xs_off, &xsum_off, &red_off, &misc_off);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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

  // 16-row tile index (inside its segment) of tile t of row tile `tile`
  auto tile_rt = [&](int tile, int t, int& seg) -> size_t {
    int rt;
    if (a.swiglu) {  // RB/2 gate rows then RB/2 up rows, both at rows tile * RB/2
      seg = t / (T / 2);
      rt = tile * (T / 2) + t % (T / 2);
    } else {
      const int n = tile * RB + t * 16;
      seg = 0;
      int base = 0;
      while (seg < 2 && n >= a.seg_end[seg]) { base = a.seg_end[seg]; ++seg; }
      rt = (n - base) / 16;
    }
    return (size_t)rt;
  };

  constexpr int U = 8 / T;                   // bf16: k-steps of 32 per iteration
  constexpr int GU = 4 / T > 0 ? 4 / T : 1;  // 4-bit: groups of 64 per iteration
  const int nit = (FMT == W_BF16) ? kq / (32 * U) : kq / (64 * GU);
  const unsigned char* wp[T];   // this wave's stream inside each 16-row tile
  const unsigned char* sbp[T];  // 4-bit: scale/bias stream
  auto set_tile = [&](int tile) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      int seg;
      const size_t rt = tile_rt(tile, t, seg);
      if (FMT == W_BF16) {
        // block (rt, s) at ((rt * K/32) + s) * 1024; this wave starts at s = k0/32
        wp[t] = (const unsigned char*)a.w[seg] + (rt * (K / 32) + k0 / 32) * 1024 + lane * 16;
      } else {
        // codes block (rt, g) at ((rt * K/64) + g) * 512; scales (rt, g) at * 64
        wp[t] = (const unsigned char*)a.w[seg] + (rt * ng + k0 / 64) * 512 + lane * 8;
        sbp[t] = (const unsigned char*)a.sb[seg] + (rt * ng + k0 / 64) * 64 + j4 * 16;
      }
    }
  };
  u32x4 b0[T][U], b1[T][U];
  u32x2 c0[T][GU], c1[T][GU];
  u32x4 s0[T][GU], s1[T][GU];
  auto load_bf = [&](u32x4 (&b)[T][U], int it) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int u = 0; u < U; ++u)
        b[t][u] = __builtin_nontemporal_load((const u32x4*)(wp[t] + (size_t)(it * U + u) * 1024));
  };
  auto load_q4 = [&](u32x2 (&c)[T][GU], u32x4 (&sv)[T][GU], int it) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        c[t][u] = __builtin_nontemporal_load((const u32x2*)(wp[t] + (size_t)(it * GU + u) * 512));
        sv[t][u] = __builtin_nontemporal_load((const u32x4*)(sbp[t] + (size_t)(it * GU + u) * 64));
      }
  };

  // ---- first tile's first weights, before the prologue
  int tile = blockIdx.x;
  if (tile < n_tiles) {
    set_tile(tile);
    if constexpr (FMT == W_BF16)
      load_bf(b0, 0);
    else
      load_q4(c0, s0, 0);
  }

  // ---- row norm scales from the producer's per-tile sums of squares (each
  // wave computes them itself, so no barrier separates them from x's loads)
  float* rsw = misc + 64 + 16 * wave;
  if (a.sq_in) {
    for (int m = 0; m < M; ++m) {
      float s = 0.f;
      for (int b = lane; b < a.sq_nb; b += 64) s += a.sq_in[m * a.sq_nb + b];
      s = wave_sum(s);
      if (lane == 0) rsw[m] = rsqrtf(s / (float)K + a.eps);
    }
  }
  // ---- prologue: this wave's K part of x' -> bf16 hi/lo (once per workgroup)
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
  __syncthreads();

  auto compute_bf = [&](f32x4 (&acc)[T], const u32x4 (&b)[T][U], int it) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x4 bh = {0u, 0u, 0u, 0u}, bl = {0u, 0u, 0u, 0u};
      const int kl = (it * U + u) * 32 + 8 * j4;
      if (col_on) {
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

  const int nb = gridDim.x;
  float best_v[16];
  int best_i[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    best_v[m] = -INFINITY;
    best_i[m] = 0x7fffffff;
  }
  for (; tile < n_tiles; tile += nb) {
    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (FMT == W_BF16) {
      for (int it = 0; it < nit; it += 2) {
        if (it + 1 < nit) load_bf(b1, it + 1);
        compute_bf(acc, b0, it);
        if (it + 2 < nit) load_bf(b0, it + 2);
        if (it + 1 < nit) compute_bf(acc, b1, it + 1);
      }
    } else {
      for (int it = 0; it < nit; it += 2) {
        if (it + 1 < nit) load_q4(c1, s1, it + 1);
        compute_q4(acc, c0, s0, it);
        if (it + 2 < nit) load_q4(c0, s0, it + 2);
        if (it + 1 < nit) compute_q4(acc, c1, s1, it + 1);
      }
    }
    // the next tile's first weights load while this tile is finished
    const int next = tile + nb;
    if (next < n_tiles) {
      set_tile(next);
      if constexpr (FMT == W_BF16)
        load_bf(b0, 0);
      else
        load_q4(c0, s0, 0);
    }

    // ---- sum the waves' K parts: D[n][m] lane layout rows 4 j4 + v, column r16
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (col_on) red[(wave * M + r16) * RB + t * 16 + 4 * j4 + v] = acc[t][v];
    __syncthreads();
    for (int i = tid; i < M * RB; i += THREADS) {
      float v = red[i];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) v += red[w * M * RB + i];
      red[i] = v;  // wave 0's slice holds the result (each i touched by one thread)
    }
    __syncthreads();

    // ---- epilogues on red[m * RB + r]
    if (a.epi == EPI_STORE) {
      for (int i = tid; i < M * RB; i += THREADS) {
        const int m = i / RB, n = tile * RB + i % RB;
        a.out[(size_t)m * a.ldo + n] = red[i];
      }
    } else if (a.epi == EPI_SWIGLU) {
      constexpr int HR = RB / 2;
      for (int i = tid; i < M * HR; i += THREADS) {
        const int m = i / HR, r = i % HR;
        a.out[(size_t)m * a.ldo + tile * HR + r] = silu(red[m * RB + r]) * red[m * RB + HR + r];
      }
    } else if (a.epi == EPI_RESID) {
      // h += y; per-tile sum of squares of the new h (the next kernel's norm)
      for (int m = 0; m < M; ++m) {
        float sq = 0.f;
        for (int r = tid; r < RB; r += THREADS) {
          float* hp = a.out + (size_t)m * a.ldo + tile * RB + r;
          const float h = *hp + red[m * RB + r];
          *hp = h;
          sq += h * h;
        }
        sq = block_sum(sq, misc + 16);
        if (tid == 0) a.sq_out[m * n_tiles + tile] = sq;
      }
    } else if (a.epi == EPI_HEAD) {
      // logits; running (max, lowest index) per row for this workgroup
      for (int i = tid; i < M * RB; i += THREADS) {
        const int m = i / RB, n = tile * RB + i % RB;
        const float v = red[i];
        a.out[(size_t)m * a.ldo + n] = v;
#pragma unroll
        for (int mm = 0; mm < 16; ++mm)
          if (mm == m && (v > best_v[mm] || (v == best_v[mm] && n < best_i[mm]))) {
            best_v[mm] = v;
            best_i[mm] = n;
          }
      }
    }
    __syncthreads();  // red is rewritten by the next tile
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
      coh_store(a.cand_val + m * nb + blockIdx.x, bv);
      coh_store(a.cand_idx + m * nb + blockIdx.x, bi);
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

// ---- load-time re-tiling into fragment order
__global__ void tile_bf16_kernel(const uint16_t* src, uint16_t* dst, int N, int K) {
  // dst block (rt, s) = 64 lanes x 8 elements: lane l -> row 16 rt + l%16,
  // columns 32 s + 8 (l/16) .. +7
  const size_t nblk = (size_t)(N / 16) * (K / 32);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < nblk * 64; i += (size_t)gridDim.x * blockDim.x) {
    const size_t blk = i / 64;
    const int l = (int)(i % 64);
    const size_t rt = blk / (K / 32), s = blk % (K / 32);
    const uint4 v = *(const uint4*)(src + (16 * rt + (l & 15)) * (size_t)K + 32 * s + 8 * (l >> 4));
    *(uint4*)(dst + i * 8) = v;
  }
}

__global__ void tile_q4_kernel(const uint32_t* codes, const uint16_t* sc, const uint16_t* bi, uint32_t* dst_c,
                               uint32_t* dst_sb, int N, int K) {
  // codes block (rt, g) = 64 lanes x 2 words: lane l -> row 16 rt + l%16,
  // inputs 64 g + 16 (l/16) .. +15; scales block (rt, g) = 16 rows x (s, b)
  const int ng = K / 64;
  const size_t nblk = (size_t)(N / 16) * ng;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < nblk * 64; i += (size_t)gridDim.x * blockDim.x) {
    const size_t blk = i / 64;
    const int l = (int)(i % 64);
    const size_t rt = blk / ng, g = blk % ng;
    const size_t row = 16 * rt + (l & 15);
    const uint32_t* s = codes + row * (K / 8) + 8 * g + 2 * (l >> 4);
    dst_c[2 * i] = s[0];
    dst_c[2 * i + 1] = s[1];
    if (l < 16) {
      const size_t r2 = 16 * rt + l;
      dst_sb[blk * 16 + l] = (uint32_t)sc[r2 * ng + g] | ((uint32_t)bi[r2 * ng + g] << 16);
    }
  }
}

}  // namespace

// Waves per workgroup: 8 when K splits into eight parts of whole iterations,
// else 4.
int gemv_waves(int K, int tiles, int fmt) {
  const int per_iter = (fmt == W_Q4) ? 64 * (4 / tiles > 0 ? 4 / tiles : 1) : 32 * (8 / tiles);
  return (K % (8 * per_iter) == 0 && K / 8 >= per_iter) ? 8 : 4;
}

size_t gemv_lds_bytes(int M, int K, int tiles, int fmt) {
  int a, b, c, d;
  return (size_t)gemv_lds_layout(M, K, 16 * tiles, fmt, gemv_waves(K, tiles, fmt), &a, &b, &c, &d);
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  const int RB = 16 * a.tiles;
  if (a.K % 1024 || a.M < 1 || a.M > 16 || a.grid < 1) return hipErrorInvalidValue;
  const int rows = a.swiglu ? 2 * a.N : a.N;
  if (rows % RB || (a.swiglu && a.tiles < 2)) return hipErrorInvalidValue;
  for (int i = 0; i < 3; ++i)
    if (a.seg_rows[i] % 16) return hipErrorInvalidValue;
  const size_t lds = gemv_lds_bytes(a.M, a.K, a.tiles, a.fmt);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  const int W = gemv_waves(a.K, a.tiles, a.fmt);
  const int n_tiles = rows / RB;
  dim3 grid(a.grid < n_tiles ? a.grid : n_tiles);
#define DPK_GEMV_CASE(F, T, WV)                                                            \
  if (a.fmt == F && a.tiles == T && W == WV) {                                            \
    launch((gemv_kernel<F, T, WV>), grid, dim3(64 * WV), lds, stream, a);    \
    return hipGetLastError();                                                             \
  }
  DPK_GEMV_CASE(W_BF16, 1, 4)
  DPK_GEMV_CASE(W_BF16, 2, 4)
  DPK_GEMV_CASE(W_BF16, 4, 4)
  DPK_GEMV_CASE(W_Q4, 1, 4)
  DPK_GEMV_CASE(W_Q4, 2, 4)
  DPK_GEMV_CASE(W_Q4, 4, 4)
  DPK_GEMV_CASE(W_BF16, 1, 8)
  DPK_GEMV_CASE(W_BF16, 2, 8)
  DPK_GEMV_CASE(W_BF16, 4, 8)
  DPK_GEMV_CASE(W_Q4, 1, 8)
  DPK_GEMV_CASE(W_Q4, 2, 8)
  DPK_GEMV_CASE(W_Q4, 4, 8)
#undef DPK_GEMV_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_tile_bf16(const uint16_t* src, uint16_t* dst, int N, int K, hipStream_t stream) {
  if (N % 16 || K % 32) return hipErrorInvalidValue;
  const size_t n = (size_t)N / 16 * (K / 32) * 64;
  const int blocks = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  launch(tile_bf16_kernel, dim3(blocks), dim3(256), 0, stream, src, dst, N, K);
  return hipGetLastError();
}

hipError_t launch_tile_q4(const uint32_t* codes, const uint16_t* sc, const uint16_t* bi, uint32_t* dst_c,
                          uint32_t* dst_sb, int N, int K, hipStream_t stream) {
  if (N % 16 || K % 64) return hipErrorInvalidValue;
  const size_t n = (size_t)N / 16 * (K / 64) * 64;
  const int blocks = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  launch(tile_q4_kernel, dim3(blocks), dim3(256), 0, stream, codes, sc, bi, dst_c, dst_sb, N, K);
  return hipGetLastError();
}

}  // namespace dpk
