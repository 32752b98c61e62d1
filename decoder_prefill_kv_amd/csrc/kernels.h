// Kernel launch interface of the dpk library (internal; not part of the C ABI).
#pragma once
#include "common.h"

namespace dpk {

// KV cache: one slab per (sequence, layer, K|V, kv head).
//   K   [max_seq][head_dim]   (row per position)
//   V^T [head_dim][max_seq]   (row per channel, positions contiguous)
// Element type fp16 (bf16/q4 models) or fp32 (fp32 models).
struct KVDesc {
  void* base;
  int is_f32;
  int n_layers, n_kv, max_seq, d;
  int i8;         // int8 codes at base (same element layout), one fp32 scale per position in scales
  float* scales;  // int8 cache: [seq][layer][K|V][head][max_seq]
};

__host__ __device__ inline size_t kv_slab(const KVDesc& kv, int seq, int layer, int which, int head) {
  return ((((size_t)seq * kv.n_layers + layer) * 2 + which) * kv.n_kv + head) * (size_t)kv.max_seq * kv.d;
}
// which = 0: K element (pos, e); which = 1: V element (pos, e)
__host__ __device__ inline size_t kv_offset(const KVDesc& kv, int seq, int layer, int which, int head,
                                            int e, int pos) {
  const size_t s = kv_slab(kv, seq, layer, which, head);
  return which == 0 ? s + (size_t)pos * kv.d + e : s + (size_t)e * kv.max_seq + pos;
}
__host__ __device__ inline size_t kv_scale_slab(const KVDesc& kv, int seq, int layer, int which, int head) {
  return ((((size_t)seq * kv.n_layers + layer) * 2 + which) * kv.n_kv + head) * (size_t)kv.max_seq;
}
// int8 cache: one position's head vector (d == 128) held by a wave, elements
// lane and lane + 64, quantized to codes round(x / s), s = max |x| / 127
// (clipped to +-127; s = 0 stores zeros), codes and scale stored
DPK_DEV float kv_quant_i8(float x0, float x1, float& q0, float& q1) {  // returns s (wave-uniform)
  const float m = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float s = m / 127.0f;
  q0 = s > 0.f ? fminf(fmaxf(rintf(x0 / s), -127.f), 127.f) : 0.f;
  q1 = s > 0.f ? fminf(fmaxf(rintf(x1 / s), -127.f), 127.f) : 0.f;
  return s;
}
// 8 int8 cache codes -> the fp16 integers 1152 + q (exact: the byte q ^ 0x80
// under the high byte 0x64), the form the attention MFMAs take them in
DPK_DEV u32x4 kv_codes_f16(u32x2 w) {
  const uint32_t u0 = w.x ^ 0x80808080u, u1 = w.y ^ 0x80808080u;
  return u32x4{__builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u), __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u),
               __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u), __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)};
}
DPK_DEV void kv_put_i8(const KVDesc& kv, int seq, int layer, int which, int head, int pos, float x0, float x1,
                       int lane) {
  float q0, q1;
  const float s = kv_quant_i8(x0, x1, q0, q1);
  int8_t* b = (int8_t*)kv.base + kv_slab(kv, seq, layer, which, head);
  if (which == 0) {
    b[(size_t)pos * 128 + lane] = (int8_t)q0;
    b[(size_t)pos * 128 + lane + 64] = (int8_t)q1;
  } else {
    b[(size_t)lane * kv.max_seq + pos] = (int8_t)q0;
    b[(size_t)(lane + 64) * kv.max_seq + pos] = (int8_t)q1;
  }
  if (lane == 0) kv.scales[kv_scale_slab(kv, seq, layer, which, head) + pos] = s;
}
DPK_DEV void kv_store(const KVDesc& kv, size_t off, float v) {
  if (kv.is_f32)
    ((float*)kv.base)[off] = v;
  else
    ((_Float16*)kv.base)[off] = (_Float16)v;
}

enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_QKV = 3, EPI_HEAD = 4 };

struct SkinnyArgs {
  int M, K, N;  // activation rows (<=16), input dim, output rows
  int fmt;      // W_BF16 | W_Q4 | W_I8 | W_Q8
  const void* w[3];         // bf16 [rows][K], q4 codes uint32 [rows][K/8], int8: launch_tile_i8 order
  const uint16_t* sc[3];    // q4 scales bf16 [rows][K/64]; int8: row scales bf16 [rows]
  const uint16_t* bi[3];    // q4 biases bf16 [rows][K/64]
  const float* sf[3];       // q8: block scales fp32 in launch_tile_q8s order
  int seg_end[3];           // cumulative row ends of the stacked segments
  int seg_rows[3];          // rows of each segment (load clamp)
  const float* x;
  int ldx;
  const float* rs;          // [M] row norm scale or null
  const uint16_t* gain;     // bf16 [K] or null
  int ksplit, kchunk, rows_per_wg, n_blocks;
  float* part;              // [ksplit][M][n_blocks*rows]
  unsigned* counters;       // [1 + n_blocks], zero between launches
  int epi;
  float* out;               // STORE/RESID/SWIGLU/HEAD target
  int ldo;
  float* sq;                // RESID: [M][n_blocks]
  float* rs_out;            // RESID: [M]
  float eps;
  // QKV epilogue
  const RowParam* rows_param;
  const uint16_t* qn;       // bf16 [d] or null
  const uint16_t* kn;
  const float* rope_cos;    // [max_seq][d/2]
  const float* rope_sin;
  float* qout;              // [M][n_heads][d]
  int n_heads, layer;
  KVDesc kv;
  // HEAD epilogue
  float* cand_val;          // [M][n_blocks]
  int* cand_idx;
  int* argmax_out;          // [M]
};

size_t skinny_lds_bytes(int M, int kchunk, int rows, int fmt);
// 16-row tiles per lm_head tile of the persistent step with int8 weights
// (measured, 8B: 1 / 2 / 4 -> head phase 130.4 / 112.6 / 110.7 us)
constexpr int MEGA_HEAD_I8_TILES = 2;
// Block formats (Q8, Q4_0) in the persistent step: 16-row tiles per gate / up
// tile and per lm_head tile (the head's 64-row tiles stream four iterations
// deep; 96-row gate / up tiles, one per compute unit at 2 x 12288 rows, spill
// registers)
constexpr int MEGA_GU_BLK_TILES = 2, MEGA_HEAD_BLK_TILES = 4;
// 16-row tiles per gate / up and lm_head tile of the persistent step
constexpr int mega_gu_tiles(int fmt) { return (fmt == W_Q40 || fmt == W_Q8) ? MEGA_GU_BLK_TILES : 2; }
constexpr int mega_head_tiles(int fmt, bool small) {
  return small ? 2 : fmt == W_I8 ? MEGA_HEAD_I8_TILES : (fmt == W_Q40 || fmt == W_Q8) ? MEGA_HEAD_BLK_TILES : 1;
}

// ---- decode GEMV with the whole K in one workgroup (gemv.hip)
// Weights are given in the re-tiled fragment layout (launch_tile_bf16 /
// launch_tile_q4): w = tiled bf16 or tiled 4-bit codes, sb = tiled 4-bit
// (scale, bias) pairs.  Every segment has a multiple of 16 rows.
// Layout of ready-made GEMV activations: blocks of 32 columns, each holding
// 16 rows x 32 columns (1 KB of bf16), so that one wave's MFMA B fragment
// (row = lane % 16, columns 8 (lane / 16) .. + 7 of a 32-column step) is one
// contiguous 1 KB read.  Holds 16 rows; column counts are multiples of 32.
__host__ __device__ inline size_t xg_index(int m, int k) {
  return ((size_t)(k >> 5) << 9) + ((size_t)m << 5) + (k & 31);
}

struct GemvArgs {
  int M, K, N;              // rows (<=16), input dim, output rows (per matrix for swiglu)
  int fmt, tiles, swiglu, epi;
  int grid;                 // workgroups (they loop over row tiles)
  int waves;                // ready-made-activation mode: 4 or 8 waves per workgroup, 0: by K
  int kofs, kfull;          // reduce over columns [kofs, kofs + K) of rows of kfull (0: K) columns
  const uint16_t* xb_hi;    // non-null: activations as bf16 hi / lo in the xg_index layout (bf16
  const uint16_t* xb_lo;    //   weights; x is not read), rows xrow0 .. xrow0 + M - 1.  Any gain
  int xrow0;                //   is already applied; with sq_in the outputs are scaled by each
                            //   row's rsqrt(mean + eps)
  uint16_t* xo_hi;          // non-null (EPI_RESID / EPI_SWIGLU): also write the result as the
  uint16_t* xo_lo;          //   next GEMV's bf16 hi / lo activations (xg_index layout), times
  const uint16_t* xo_gain;  //   xo_gain[n] if given (RESID); SWIGLU then skips out
  const void* w[3];
  const void* sb[3];
  int seg_end[3];
  int seg_rows[3];
  const float* x;
  int ldx;
  const float* sq_in;       // [M][sq_nb] sums of squares of x's rows, or null (no norm)
  int sq_nb;
  const uint16_t* gain;     // bf16 [K] or null
  float eps;
  float* out;
  int ldo;
  float* sq_out;            // RESID: [M][row tiles]
  unsigned* counters;       // HEAD
  float* cand_val;          // HEAD: [M][grid]
  int* cand_idx;
  int* argmax_out;
  // persistent step, O projection by KV head (fixed-point partial sums, see
  // to_fixed): xacc [M][ldx] is added to x as it is staged; RESID with racc
  // [M][ldo]: h = (h + racc) + y, and racc is cleared
  const long long* xacc;
  long long* racc;
};
size_t gemv_lds_bytes(int M, int K, int tiles, int fmt);
size_t gemv_lds_bytes_waves(int M, int K, int tiles, int fmt, int waves);
int gemv_waves(int K, int tiles, int fmt);
hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream);
// fragment-order copies of [N][K] weights for launch_gemv
hipError_t launch_tile_bf16(const uint16_t* src, uint16_t* dst, int N, int K, hipStream_t stream);
hipError_t launch_tile_q4(const uint32_t* codes, const uint16_t* sc, const uint16_t* bi, uint32_t* dst_c,
                          uint32_t* dst_sb, int N, int K, hipStream_t stream);
hipError_t launch_skinny(const SkinnyArgs& a, hipStream_t stream);
// fragment-order copy of int8 codes [N][K] for the int8 skinny GEMV: per 16-row
// tile and 256 columns, 4 KB in which lane l of a wave finds its 16 bytes of
// MFMA k-steps 2p and 2p+1 at p * 1024 + l * 16 (N % 16 == 0, K % 256 == 0)
hipError_t launch_tile_i8(const int8_t* src, int8_t* dst, int N, int K, hipStream_t stream);
// fragment-order copy of q8 block scales [N][K/32]: per 16-row tile and 256
// columns, 512 bytes holding row r's 8 scales at r * 32
hipError_t launch_tile_q8s(const float* src, float* dst, int N, int K, hipStream_t stream);
// the same layout for Q4_0's fp16 scales, kept fp16: 256 bytes per tile and 256
// columns, row r's 8 at r * 16
hipError_t launch_tile_q40s(const uint16_t* src, uint16_t* dst, int N, int K, hipStream_t stream);
// fragment-order copy of Q4_0 codes (GGUF blocks: byte j of a block's 16 holds
// codes j and j + 16): per 16-row tile and 256 columns 2 KB, lane l's dword of
// k-step s at (s / 4) * 1024 + l * 16 + (s % 4) * 4, its nibble n holding
// element 2n (n < 4) or 2 (n - 4) + 1 of columns 32 s + 8 (l / 16) .. + 7
hipError_t launch_tile_q40(const uint8_t* src, uint32_t* dst, int N, int K, hipStream_t stream);
// lo: the residual w - fp16(w) of each weight instead of fp16(w) (likewise below)
hipError_t launch_q40_to_f16(const uint8_t* q, const uint16_t* d, int rows, int K, _Float16* dst, hipStream_t stream,
                             bool lo = false);

// ---- decode attention (split-K over the context, merged in-kernel)
struct AttnDecodeArgs {
  int M;                      // rows
  int n_heads, n_kv, d;
  const RowParam* rows_param;
  const float* q;             // [M][n_heads][d] (normed, roped)
  KVDesc kv;
  int layer;
  int chunk;                  // positions per workgroup (attn_decode_chunk() / attn_decode_mfma_chunk())
  int max_chunks;             // grid.x
  float* part;                // [M][n_heads][max_chunks][d + 2]
  unsigned* counters;         // [M * n_kv]
  float* out;                 // [M][n_heads*d] fp32
  float scale;                // 1/sqrt(d)
  // share (mfma kernel, 0 or 1: off): consecutive groups of `share` rows of one
  // sequence (each its own position) run in one workgroup per chunk and KV
  // head, their share * G query heads as the MFMA columns (share * G <= 16),
  // so each chunk of the cache is read once per group; not with raw mode
  int share;
  // merge (mfma kernel): 1 = the chunks' partials are always written and a
  // second launch (attn_merge_kernel) combines them, one thread per output
  // element, instead of the last-arriving workgroup of each row and KV head
  int merge;
  uint16_t* out_hi;           // with merge: if non-null, the output goes here as bf16 hi / lo
  uint16_t* out_lo;           //   (a GEMV's activations, xg_index layout) instead of to out
  // raw mode (qkv_raw != null): q is taken from the raw projection
  // [M][ld_raw] (q heads, k heads, v heads) and gets QK-norm + RoPE here; the
  // workgroup whose chunk holds the row's position computes that position's
  // k and v, stores them in the cache and uses them.  Each row's sequence
  // must have exactly one new position (a decode step).
  const float* qkv_raw;
  int ld_raw;
  const uint16_t* qn;         // bf16 gains or null
  const uint16_t* kn;
  const float* rope_cos;
  const float* rope_sin;
  float eps;
};
hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t stream);
int attn_decode_chunk();  // positions per decode-attention workgroup
// same contract on matrix cores, fp16 caches only (attn_decode_mfma.hip):
// a.chunk from attn_decode_mfma_chunk (a multiple of 256), a.merge set
// whenever a.max_chunks > 1
hipError_t launch_attn_decode_mfma(const AttnDecodeArgs& a, hipStream_t stream);
// positions per workgroup for max_ctx over `units` (row group, KV head) pairs
int attn_decode_mfma_chunk(int max_ctx, int units, int n_cu);

// ---- misc
hipError_t launch_rope_table(float* cos_t, float* sin_t, int max_seq, int d, double theta,
                             hipStream_t stream);
// h[m] = E[token_m] (fp32 / bf16 / q4 table); rs[m] = rsqrt(mean(h^2)+eps) if rs != null;
// sq[m] = sum(h^2) if sq != null
// sc: bf16 scales (q4 groups, i8 rows), fp32 block scales (q8) or fp16 ones (q4_0)
hipError_t launch_embed(int M, int H, int fmt, const void* table, const void* sc, const uint16_t* bi,
                        const RowParam* rp, const int32_t* ids_dev, int vocab, float* h, float* rs,
                        float eps, int* err_flag, hipStream_t stream, float* sq = nullptr);
// y[m] = x[m] * rsqrt(mean(x^2)+eps) * g; y_is_f16: 0 fp32, 1 fp16, 2 fp16 hi
// in columns [0, H) and fp16 lo (= y - hi) in [H, 2H); g is fp32 or bf16
hipError_t launch_rmsnorm_rows(int M, int H, const float* x, int ldx, const void* g, int g_is_f32,
                               float eps, void* y, int y_is_f16, int ldy, hipStream_t stream);
// prefill: qkv fp32 [M][(Hq+2Hkv)d] -> q (q_is_f16 0: fp32 [M][Hq][d]; 1: fp16; 2: fp16 hi plane
// then lo plane), K/V into the cache
hipError_t launch_qk_rope_kv(int M, const float* qkv, int n_heads, int n_kv, int d, int qk_norm,
                             const void* qn, const void* kn, int g_is_f32, float eps,
                             const float* rope_cos, const float* rope_sin, const RowParam* rp,
                             void* q_out, int q_is_f16, KVDesc kv, int layer, hipStream_t stream);
// fp32-weight GEMV / small GEMM for any M (VALU): out[m][n] (=|+=) sum_k W[n][k] x[m][k]
// mode 0 store, 1 add, 2 swiglu (gate=W, up=W2)
hipError_t launch_gemv_f32(int M, int N, int K, const float* W, const float* W2, const float* x, int ldx,
                           float* out, int ldo, int mode, hipStream_t stream);
// argmax per row over [M][N] logits (lowest index on ties)
hipError_t launch_argmax_rows(int M, int N, const float* logits, int ld, int* out, hipStream_t stream);
// x'[m][k] = x[m][k] * rs[m] * g[k] as bf16 hi + lo in the xg_index layout
// (M <= 16, K % 32 == 0); rs[m] from the sums of squares sq_in[m][0..nb)
// over K (null: 1), g bf16 [K] or null
hipError_t launch_xprep(int M, int K, const float* x, int ldx, const float* sq_in, int nb, const uint16_t* g,
                        float eps, uint16_t* hi, uint16_t* lo, hipStream_t stream);
// residual add out += in
hipError_t launch_add(int n, const float* in, float* out, hipStream_t stream);
// bf16 -> fp16 / q4 -> fp16 weight conversion for the prefill GEMM operands
hipError_t launch_bf16_to_f16(const uint16_t* src, _Float16* dst, size_t n, hipStream_t stream);
hipError_t launch_i8_to_f16(const int8_t* q, const uint16_t* sc, int rows, int K, _Float16* dst,
                            hipStream_t stream);
hipError_t launch_q8_to_f16(const int8_t* q, const float* sf, int rows, int K, _Float16* dst, hipStream_t stream,
                            bool lo = false);
hipError_t launch_q4_to_f16(const uint32_t* codes, const uint16_t* sc, const uint16_t* bi, int rows, int K,
                            _Float16* dst, hipStream_t stream, bool lo = false);
hipError_t launch_f32_to_f16(const float* src, _Float16* dst, size_t n, hipStream_t stream);

// ---- prefill GEMM (fp16 MFMA): C[m][n] = sum_k A[m][k] B[n][k]
// GEMM_QKV_F16: the QKV projection's epilogue (head_dim 128): per-head
// QK-norm and RoPE of the q and k heads, q written as fp16 hi / lo planes for
// the prefill attention, k and v written into the KV cache (v transposed).
enum GemmEpi : int { GEMM_STORE_F32 = 0, GEMM_ADD_F32 = 1, GEMM_SWIGLU_F16 = 2, GEMM_QKV_F16 = 3 };
struct GemmArgs {
  int M, N, K;
  int Kb;                         // K of B (0: = K); K = 2 Kb multiplies [A_hi | A_lo] by [B | B]
  const _Float16* A; int lda;
  const _Float16* B; int ldb;     // [N][K]; for SWIGLU rows [0,N) gate, B2 up
  const _Float16* B2;
  int epi;
  float* C; int ldc;              // STORE/ADD
  _Float16* C16; int ldc16;       // SWIGLU
  int splits;                     // split-K factor (<= 1: none)
  int xcd_blocks;                 // set by launch_gemm: workgroups remapped so each of the 8 XCDs
                                  //   (workgroup i runs on XCD i % 8) takes a 4 x 4 tile block
  float* ws;                      // split-K partial tiles [tiles][splits][256 * 256]
  unsigned* counters;             // split-K arrival counters [tiles], zero between launches
  // QKV epilogue: rows are positions start.. of sequence seq; columns are the
  // n_heads q heads, then the n_kv k heads, then the n_kv v heads (128 each)
  int n_heads, n_kv, start, seq, layer;
  const uint16_t* qn;             // q / k RMSNorm gains (bf16 [128]) or null
  const uint16_t* kn;
  float eps;
  const float* rope_cos;          // [max_seq][64]
  const float* rope_sin;
  _Float16* q16;                  // hi plane [M][n_heads][128], then the lo plane
  KVDesc kv;
  // int8 weights with one scale per output row: B (and B2) hold the codes
  // themselves (exact in fp16) and each product column is multiplied by its
  // row's bf16 scale before the epilogue: rows [0, rs_end[0]) of B take rs[0],
  // then rs[1] up to rs_end[1], then rs[2]; SWIGLU: rs[0] gate, rs[1] up.
  // rs[0] null: no scaling.
  const uint16_t* rs[3];
  int rs_end[2];
};
constexpr int GEMM_MAX_SPLITS = 2;
constexpr size_t GEMM_WS_TILES = 768;             // partial tiles the workspace holds
constexpr size_t GEMM_TILE_FLOATS = 256 * 256;
// split-K factor that best fills n_cu CUs with (M, N) tiles
int gemm_choose_splits(int M, int N, int K, int epi, int n_cu);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
// Whether a plain store GEMM of this shape runs on 256 x 128 tiles.
bool gemm_prefers_narrow(int M, int N, int n_cu);

// ---- prefill attention (fp16 MFMA, causal over the cache)
struct AttnPrefillArgs {
  int M;               // query rows, at positions start..start+M-1 of sequence seq
  int start, seq;
  int n_heads, n_kv, d;
  const _Float16* q;   // [2][M][n_heads][d]: fp16 hi plane, then the lo plane (q - hi)
  KVDesc kv;
  int layer;
  _Float16* out;       // [M][2][n_heads*d]: per row the fp16 hi half, then the lo half (o - hi)
  float scale;
};
hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t stream);

// ---- whole decode step in one persistent (cooperative) launch, bf16 weights
constexpr int MEGA_ATTN_MAXCH = 64;  // attention chunks per row (256 positions each)
constexpr int MEGA_CTR_STRIDE = 64;  // words between the fused step's attention counters (own 256-byte line)
struct MegaLayer {                   // device-resident, one per layer
  GemvArgs qkv;                      // the QKV projection, whole K: 32-row tiles (measured faster
                                     //   than 16-row tiles and than K splits that balance the tiles),
                                     //   16-row tiles in the 128-column variant
  GemvArgs o, gu, down;              // M is set per launch
  const uint16_t* qn;                // QK-norm gains (bf16) or null
  const uint16_t* kn;
};
struct MegaArgs {
  int M, n_layers, H, vocab;
  const MegaLayer* layers;
  GemvArgs head;
  int fmt;                           // W_BF16, W_Q4, W_I8, W_Q8 or W_Q40 (every linear, the embedding included)
  int small;                         // GEMVs reduce 128 columns per wave and iteration (rows of 1024 k)
  const void* emb;                   // bf16 [vocab][H], MLX 4-bit codes [vocab][H / 8] words, int8 / Q8
                                     //   codes [vocab][H], or Q4_0 codes [vocab][H / 2] bytes
  const uint16_t* emb_sc;            // MLX 4-bit: per-64 scales / biases [vocab][H / 64]; int8: the
                                     //   bf16 row scales; Q4_0: the fp16 block scales [vocab][H / 32];
                                     //   Q8: the fp32 block scales [vocab][H / 32]
  const uint16_t* emb_bi;
  RowParam rows[16];                 // the rows' token / position / slot (by value: no upload per step)
  const int32_t* ids_dev;            // token ids, or null: rp[m].token
  float* h;                          // [M][H] residual
  float* sq;                         // [M][H/16] per-tile sums of squares
  int* err;                          // bit 0: token out of range
  int n_heads, n_kv;
  KVDesc kv;
  const float* qkv;                  // [M][ld_qkv] raw projection
  int ld_qkv;
  const float* rope_cos;
  const float* rope_sin;
  float eps, scale;
  int max_chunks;
  float* part;                       // [M][n_heads][max_chunks][d + 2]
  unsigned* attn_counters;           // [M * n_kv] (fused O: one per MEGA_CTR_STRIDE words)
  float* attn_out;                   // [M][n_heads * d]
  long long* oacc;                   // [M][H] fixed-point O-projection sums, or null: the O projection is a
                                     //   GEMV after attention (see attn_phase)
  int o_rt;                          // 16-row tiles per O item (1, 2, 4 or 8) when oacc is set
  unsigned* bar;                     // MEGA_BAR_WORDS zeroed words: barrier counters, exit count, abort flag
  unsigned long long* trace;         // null, or MEGA_TRACE_WORDS accumulators (see below)
  int lds_args;                      // byte offset of the staged arguments (MEGA_ARGS_LDS bytes) and,
                                     //   for bf16, the GEMVs' prefetch slots (MEGA_PF_LDS bytes)
};
// Phase tracing: workgroup 0 adds the wall-clock ticks from one barrier
// release to the next to trace[phase] and counts steps in trace[0].
enum MegaPhase : int { MP_STEPS = 0, MP_EMBED, MP_QKV, MP_ATTN, MP_O, MP_GATEUP, MP_DOWN, MP_HEAD, MEGA_TRACE_WORDS };
constexpr int MEGA_BAR_EXIT = 64 * 9, MEGA_BAR_ABORT = 64 * 10, MEGA_BAR_WORDS = 64 * 11;
// LDS after the phases' own use: the staged layer / head arguments and row
// parameters (MEGA_ARGS_LDS bytes), then (bf16) the GEMVs' prefetch slots
constexpr int MEGA_ARGS_LDS = (int)((sizeof(MegaLayer) + sizeof(GemvArgs) + 16 * sizeof(RowParam) + 15) / 16 * 16);
constexpr int MEGA_PF_LDS = 8 * 8 * 1024;
size_t mega_attn_lds_bytes(int G);
// LDS of the fused attention + O phase below the staged arguments (the
// weights not held in the prefetch slots, x, reduction), 0 if the shape does
// not fit it
size_t mega_o_lds_bytes(int M, int G, int rt);
int mega_threads();
int mega_attn_chunk();
int mega_occupancy(int G, int fmt, bool small, bool fo, bool kv8, size_t lds);
hipError_t launch_decode_step(const MegaArgs& a, int G, int n_wg, size_t lds, hipStream_t stream);

// ---------------------------------------------------------------- sampling (sample.hip)
// Temperature / top-k / top-p sampling of `rows` logit rows, one token each
// drawn with the row's uniform u[r]; T == 0 is greedy.
hipError_t launch_sample(const float* logits, long long ld, int rows, int V, float T, int top_k, float top_p,
                         const float* u, int* out, hipStream_t stream);
// Bytes of the per-row distribution records speculative acceptance of K
// drafts keeps in its workspace.
size_t spec_dist_bytes(int K);
// The allocation-free acceptance's workspace: the device address of a
// file-scope array on the current device (looked up once per device), and
// the most drafts one call may have.
hipError_t spec_noalloc_scratch(void** ptr);
int spec_noalloc_max_k();
// Speculative-sampling acceptance of K drafts: out[0] = accepted count,
// out[1] = next token (residual or bonus draw).
hipError_t launch_spec_accept(const float* target, const float* draft, long long ld, int V, int K, float T,
                              int top_k, float top_p, const int* drafts, const float* r, const float* u, void* ws,
                              int* out, hipStream_t stream);

}  // namespace dpk
