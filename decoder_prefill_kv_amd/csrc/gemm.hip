// Prefill GEMM on gfx950 matrix cores: C[m][n] = sum_k A[m][k] * B[n][k]
// with A = activations [M][K] and B = weights [N][K] (the [out, in] layout),
// both fp16 and K-contiguous, fp32 accumulation.
//
// Prefill is compute bound (the whole prompt goes through every weight at
// once, "LLMs on the ANE", opening section); this kernel is where its FLOPs go.
// The operands are fp16 rather than bf16: every weight of the bf16 model is
// exactly representable in fp16 (magnitudes >= 2^-17; smaller ones round with
// an absolute error below 2^-25), and fp16 activations carry three more
// mantissa bits, which the logits tolerance needs on deep models.  Where that
// is still not enough (the QKV projection), A is given as [A_hi | A_lo] with
// K = 2 Kb and B is read twice, which computes (A_hi + A_lo) B^T.
//
// Tile 256 x 256 x 64, 4 waves in a 2 x 2 layout, each wave 128 x 128 from
// 4 x 4 v_mfma_f32_32x32x16_f16 blocks (256 fp32 accumulators per lane).
// Global -> registers -> LDS double buffer, one barrier per k-tile.
#include "common.h"
#include "kernels.h"

namespace dpk {

namespace {

constexpr int BM = 256, BN = 256, BK = 64, THREADS = 256;
constexpr int LDS_STRIDE = BK + 8;  // halfs per LDS row (pad against bank conflicts)

template <int EPI>
__global__ __launch_bounds__(THREADS, 1) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][BM][LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][BN][LDS_STRIDE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  // SWIGLU: the tile's B rows are 128 gate rows then the same 128 up rows
  const int n0 = (EPI == GEMM_SWIGLU_F16) ? blockIdx.x * (BN / 2) : blockIdx.x * BN;

  // global load assignment: 8 threads per 64-half row, 32 rows per pass
  const int lrow = tid >> 3, lk = (tid & 7) * 8;
  const _Float16* Ag[BM / 32];
  const _Float16* Bg[BN / 32];
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) {
    int r = m0 + lrow + 32 * i;
    r = r < a.M ? r : a.M - 1;  // clamp the M tail (rows discarded at the store)
    Ag[i] = a.A + (size_t)r * a.lda + lk;
  }
#pragma unroll
  for (int i = 0; i < BN / 32; ++i) {
    const int rr = lrow + 32 * i;
    if (EPI == GEMM_SWIGLU_F16)
      Bg[i] = (rr < BN / 2 ? a.B + (size_t)(n0 + rr) * a.ldb : a.B2 + (size_t)(n0 + rr - BN / 2) * a.ldb) + lk;
    else
      Bg[i] = a.B + (size_t)(n0 + rr) * a.ldb + lk;
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  u32x4 ra[BM / 32], rb[BN / 32];
  const int Kb = a.Kb ? a.Kb : a.K;
  auto gload = [&](int kt) {
    const int ko = kt * BK;
    const int kob = ko < Kb ? ko : ko - Kb;  // B is read twice when A = [hi | lo]
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) ra[i] = *(const u32x4*)(Ag[i] + ko);
#pragma unroll
    for (int i = 0; i < BN / 32; ++i) rb[i] = *(const u32x4*)(Bg[i] + kob);
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) *(u32x4*)&As[st][lrow + 32 * i][lk] = ra[i];
#pragma unroll
    for (int i = 0; i < BN / 32; ++i) *(u32x4*)&Bs[st][lrow + 32 * i][lk] = rb[i];
  };

  // B rows of this wave inside the LDS tile
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (EPI == GEMM_SWIGLU_F16)
      brow[j] = (j < 2 ? 0 : BN / 2) + wn * 64 + (j & 1) * 32;
    else
      brow[j] = wn * 128 + j * 32;
  }

  const int nk = a.K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int r32 = lane & 31, k8 = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      f16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const f16x8*)&As[st][wm * 128 + i * 32 + r32][kk + k8];
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = *(const f16x8*)&Bs[st][brow[j] + r32][kk + k8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[row][col], col = lane % 32,
  // row = 8 * (v / 4) + 4 * (lane / 32) + v % 4 inside each 32 x 32 block
  const int hi4 = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * 128 + i * 32 + 8 * (v / 4) + hi4 + (v % 4);
      if (m >= a.M) continue;
      if (EPI == GEMM_SWIGLU_F16) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + wn * 64 + j * 32 + r32;
          const float g = acc[i][j][v], u = acc[i][j + 2][v];
          a.C16[(size_t)m * a.ldc16 + n] = (_Float16)(silu(g) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 128 + j * 32 + r32;
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

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.K % BK || a.M < 1) return hipErrorInvalidValue;
  if (a.Kb && (a.Kb % BK || (a.K != a.Kb && a.K != 2 * a.Kb))) return hipErrorInvalidValue;
  const int ntile = (a.epi == GEMM_SWIGLU_F16) ? BN / 2 : BN;
  if (a.N % ntile) return hipErrorInvalidValue;
  dim3 grid(a.N / ntile, (a.M + BM - 1) / BM);
  switch (a.epi) {
    case GEMM_STORE_F32: launch(gemm_kernel<GEMM_STORE_F32>, grid, dim3(THREADS), 0, stream, a); break;
    case GEMM_ADD_F32: launch(gemm_kernel<GEMM_ADD_F32>, grid, dim3(THREADS), 0, stream, a); break;
    case GEMM_SWIGLU_F16: launch(gemm_kernel<GEMM_SWIGLU_F16>, grid, dim3(THREADS), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dpk
