// Decode GEMV launches (one kernel per GEMV) and the load-time re-tiling of
// the weights into the fragment order the GEMV body reads (gemv_body.h).
#include "gemv_body.h"

namespace dpk {

namespace {

using gemv_detail::gemv_lds_layout;

template <int FMT, int T, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  gemv_detail::gemv_body<FMT, T, WAVES, false>(a, a.M, lds, blockIdx.x, gridDim.x, [](auto&& issue) { issue(); });
}

// bf16 weights with ready-made bf16 hi / lo activation rows (any M <= 16)
template <int T, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_xg_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  gemv_detail::gemv_body<W_BF16, T, WAVES, false, true>(a, a.M, lds, blockIdx.x, gridDim.x,
                                                        [](auto&& issue) { issue(); });
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
  if (fmt == W_I8) return K % (8 * 64 * (8 / tiles)) == 0 ? 8 : 4;  // 64 (8/T) columns per iteration on 8 waves
  const int per_iter = (fmt == W_Q4) ? 64 * (4 / tiles > 0 ? 4 / tiles : 1) : 32 * (8 / tiles);
  return (K % (8 * per_iter) == 0 && K / 8 >= per_iter) ? 8 : 4;
}

size_t gemv_lds_bytes_waves(int M, int K, int tiles, int fmt, int waves) {
  int a, b, c, d;
  return (size_t)gemv_lds_layout(M, K, 16 * tiles, fmt, waves, &a, &b, &c, &d);
}

size_t gemv_lds_bytes(int M, int K, int tiles, int fmt) {
  return gemv_lds_bytes_waves(M, K, tiles, fmt, gemv_waves(K, tiles, fmt));
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  const int RB = 16 * a.tiles;
  if (a.K % 1024 || a.M < 1 || a.M > 16 || a.grid < 1) return hipErrorInvalidValue;
  const int rows = a.swiglu ? 2 * a.N : a.N;
  if (rows % RB || (a.swiglu && a.tiles < 2)) return hipErrorInvalidValue;
  for (int i = 0; i < 3; ++i)
    if (a.seg_rows[i] % 16) return hipErrorInvalidValue;
  const int n_tiles = rows / RB;
  dim3 grid(a.grid < n_tiles ? a.grid : n_tiles);
  if (a.xb_hi) {
    // 4 waves by default (measured a little faster than 8 at every layer
    // shape); each wave's K part must hold whole 128-column iterations
    const int W = a.waves ? a.waves : 4;
    if ((W != 4 && W != 8) || a.K % (W * 128)) return hipErrorInvalidValue;
    if (a.fmt != W_BF16 || !a.xb_lo || a.xrow0 < 0 || a.xrow0 + a.M > 16 || (a.kofs + a.K) % 32)
      return hipErrorInvalidValue;
    const size_t lds_xg = (size_t)W * a.M * RB * 4 + (64 + 16 * W) * 4;
#define DPK_GEMV_XG_CASE(T, WV)                                                  \
  if (a.tiles == T && W == WV) {                                               \
    launch((gemv_xg_kernel<T, WV>), grid, dim3(64 * WV), lds_xg, stream, a);   \
    return hipGetLastError();                                                  \
  }
    DPK_GEMV_XG_CASE(1, 4)
    DPK_GEMV_XG_CASE(2, 4)
    DPK_GEMV_XG_CASE(1, 8)
    DPK_GEMV_XG_CASE(2, 8)
#undef DPK_GEMV_XG_CASE
    return hipErrorInvalidValue;
  }
  const int W = gemv_waves(a.K, a.tiles, a.fmt);
  const size_t lds = gemv_lds_bytes(a.M, a.K, a.tiles, a.fmt);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  if (a.fmt != W_BF16) {  // each wave's K part must hold whole iterations (64 GU columns, as gemv_body sets GU)
    const int gu = (a.fmt == W_I8 && W == 8) ? 8 / a.tiles : (4 / a.tiles > 0 ? 4 / a.tiles : 1);
    if ((a.K / W) % (64 * gu) != 0 || a.K / W < 64 * gu) return hipErrorInvalidValue;
  }
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
  DPK_GEMV_CASE(W_I8, 1, 4)
  DPK_GEMV_CASE(W_I8, 2, 4)
  DPK_GEMV_CASE(W_I8, 4, 4)
  DPK_GEMV_CASE(W_I8, 1, 8)
  DPK_GEMV_CASE(W_I8, 2, 8)
  DPK_GEMV_CASE(W_I8, 4, 8)
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
