// C-ABI runtime: configuration and weight validation, workspace carving and
// the per-call launch sequences of prefill, decode and verify.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <string>
#include <vector>

#include "../../include/dpk.h"
#include "common.h"
#include "kernels.h"

namespace dpk {
thread_local LaunchTiming g_timing;
}

using namespace dpk;

namespace {

thread_local std::string g_err;

dpk_status fail(dpk_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

constexpr int SKINNY_MAX = 16;  // rows handled by the weight-streaming path
constexpr int KSPLIT_MAX = 16;  // K splits of one weight-streaming launch
constexpr int ALIGN = 256;

struct LinearW {
  const void* w = nullptr;        // bf16 / f32 data or q4 codes
  const uint16_t* sc = nullptr;   // q4
  const uint16_t* bi = nullptr;   // q4
  const float* sf = nullptr;      // q8 block scales [rows][cols/32] (q4_0: fp16 bits)
  int rows = 0, cols = 0;
  // decode copy in fragment order (prep buffer): bf16 or q4 codes, q4 (s, b)
  const void* wt = nullptr;
  const void* sbt = nullptr;       // q4: tiled (s, b); q8: tiled block scales
};

struct LayerW {
  LinearW q, k, v, o, gate, up, down;
  const void* in_norm = nullptr;
  const void* post_norm = nullptr;
  const void* q_norm = nullptr;
  const void* k_norm = nullptr;
  // prefill operands (fp16, in the prep buffer)
  _Float16 *qkv16 = nullptr, *o16 = nullptr, *gate16 = nullptr, *up16 = nullptr, *down16 = nullptr;
  _Float16* kvlo16 = nullptr;  // block formats over an int8 cache: w - fp16(w) of the K and V rows
};

}  // namespace

struct dpk_model {
  dpk_config cfg;
  int fmt = 0;
  int Nqkv = 0;
  std::vector<LayerW> layers;
  LinearW embed, head;
  const void* final_norm = nullptr;
  bool bound = false, loaded = false, failed = false;
  // caller buffers
  void* kv = nullptr;
  void* scratch = nullptr;
  void* prep = nullptr;
  KVDesc kvd{};
  // carved scratch
  float *rope_cos = nullptr, *rope_sin = nullptr;
  RowParam* rows_dev = nullptr;
  float *h = nullptr, *rs = nullptr, *qkv = nullptr, *y32 = nullptr, *qbuf = nullptr, *attn_o = nullptr,
        *act = nullptr, *part = nullptr, *sink = nullptr, *sq = nullptr, *cand_val = nullptr, *attn_part = nullptr;
  int* cand_idx = nullptr;
  _Float16 *y16 = nullptr, *q16 = nullptr, *o16 = nullptr, *act16 = nullptr;
  unsigned *counters = nullptr, *attn_counters = nullptr, *gemm_counters = nullptr;
  long long* oacc = nullptr;  // [SKINNY_MAX][hidden] fixed-point O-projection sums of the persistent step
  float* gemm_ws = nullptr;
  // whole-step persistent decode kernel
  MegaLayer* mega_layers = nullptr;  // device table (in scratch)
  unsigned* mega_bar = nullptr;      // barrier words (in scratch)
  unsigned long long* mega_trace = nullptr;  // phase-time accumulators (in scratch)
  // batch GEMV activations: two sets of bf16 (hi, lo) rows [16][xb_w]
  uint16_t* xb[2][2] = {};
  int xb_w = 0;
  int mega_G = 0;                    // query heads per KV head, 0: not available
  size_t mega_lds = 0;
  bool mega_table = false;           // table written for the loaded weights
  int* err_flag = nullptr;
  int* argmax_sink = nullptr;
  int* spec_ids = nullptr;  // 64 device ints: tokens of the speculative loop
  int rows_f32 = 0;       // rows of the fp32 activation buffers
  int n_cu = 256;         // compute units of the bound device
  int lds_max = 64 * 1024;  // LDS bytes one workgroup may allocate on it
  int attn_chunks_cap = 0;
  size_t part_floats = 0;
  // pinned staging for row parameters
  static constexpr int NSTAGE = 4;
  RowParam* stage[NSTAGE] = {};
  hipEvent_t stage_ev[NSTAGE] = {};
  bool stage_used[NSTAGE] = {};
  int stage_next = 0;
  int32_t* acc_host = nullptr;  // pinned readback for verify
  std::vector<int32_t> seq_len;
  // optional per-launch timing (dpk_profile_begin / dpk_profile_end)
  struct ProfRec {
    int cls;
    double bytes, flops;
  };
  bool prof = false;
  int prof_max = 0;
  std::vector<hipEvent_t> prof_ev;
  std::vector<ProfRec> prof_rec;
  long prof_dropped = 0;
  double prof_step_kv = 0;  // persistent steps while profiling: cached positions their attention read
};

namespace {

size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// the attention chunk counters (the persistent step's fused O projection
// keeps each on its own line)
size_t attn_counter_bytes(const dpk_model* md) {
  const bool f32 = md->fmt == DPK_FMT_F32;
  return (size_t)(f32 ? md->cfg.max_rows : SKINNY_MAX) * md->cfg.n_kv_heads * 4 * (f32 ? 1 : MEGA_CTR_STRIDE);
}

struct ScratchLayout {
  size_t rope_cos, rope_sin, rows, h, rs, qkv, y32, qbuf, attn_o, act, part, sink, sq, cand_val, cand_idx, attn_part,
      y16, q16, o16, act16, counters, attn_counters, err, argmax_sink, spec_ids, gemm_ws, gemm_counters, mega_layers,
      mega_bar, mega_trace, xb, oacc, total;
  size_t xb_w;
  int rows_f32, attn_chunks_cap;
  size_t part_floats;
};

// Most workgroups (row blocks) any one GEMV reports per-row argmax
// candidates or per-tile sums for: every row-block count, and at least the
// lm_head's grid on ready-made activations (up to two workgroups per compute
// unit; MAX_HEAD_WG covers 512 units).
constexpr int MAX_HEAD_WG = 1024;
int nblocks_max(const dpk_config& c) {
  const int Nqkv = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  int nb = MAX_HEAD_WG;
  for (int n : {Nqkv / 64, c.hidden / 64, c.intermediate / 32, (c.vocab + 63) / 64}) nb = n > nb ? n : nb;
  return nb;
}

ScratchLayout scratch_layout(const dpk_config& c) {
  ScratchLayout L{};
  const size_t R = c.max_rows, H = c.hidden, I = c.intermediate, d = c.head_dim;
  const size_t Nqkv = (c.n_heads + 2 * c.n_kv_heads) * d, Qd = (size_t)c.n_heads * d;
  const bool f32 = c.weight_format == DPK_FMT_F32;
  const size_t Rf = f32 ? R : SKINNY_MAX;
  L.rows_f32 = (int)Rf;
  L.attn_chunks_cap = (c.max_seq + 63) / 64;
  const size_t nbm = nblocks_max(c);
  size_t nmax = Nqkv;
  if (2 * I > nmax) nmax = 2 * I;
  if (H > nmax) nmax = H;
  if ((size_t)c.vocab > nmax) nmax = c.vocab;
  L.part_floats = (size_t)KSPLIT_MAX * SKINNY_MAX * nmax;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = up(o + bytes);
    return at;
  };
  L.rope_cos = take((size_t)c.max_seq * d / 2 * 4);
  L.rope_sin = take((size_t)c.max_seq * d / 2 * 4);
  L.rows = take(R * sizeof(RowParam));
  L.h = take(R * H * 4);
  L.rs = take(R * 4);
  L.qkv = take(R * Nqkv * 4);
  L.y32 = take(Rf * H * 4);
  L.qbuf = take(Rf * Qd * 4);
  L.attn_o = take(Rf * Qd * 4);
  L.act = take(Rf * I * 4);
  L.part = take(L.part_floats * 4);
  L.sink = take((size_t)SKINNY_MAX * c.vocab * 4);
  L.sq = take(SKINNY_MAX * nbm * 4);
  L.cand_val = take(SKINNY_MAX * nbm * 4);
  L.cand_idx = take(SKINNY_MAX * nbm * 4);
  L.attn_part = take((size_t)(f32 ? R : SKINNY_MAX) * c.n_heads * L.attn_chunks_cap * (d + 2) * 4);
  // GEMM A operands hold whole 256-row tiles (rows past M are read, never stored)
  const size_t Rg = (R + 255) / 256 * 256;
  L.y16 = take(f32 ? 0 : Rg * H * 2 * 2);
  L.q16 = take(f32 ? 0 : R * Qd * 2 * 2);   // hi and lo planes
  L.o16 = take(f32 ? 0 : Rg * Qd * 2 * 2);  // per row hi then lo
  L.act16 = take(f32 ? 0 : Rg * I * 2);
  L.counters = take((1 + nbm) * 4);
  L.attn_counters = take((size_t)(f32 ? R : SKINNY_MAX) * c.n_kv_heads * 4 * (f32 ? 1 : MEGA_CTR_STRIDE));
  L.err = take(4);
  L.argmax_sink = take(SKINNY_MAX * 4);
  L.spec_ids = take(64 * 4);
  const bool gemm_path = !f32 && R > SKINNY_MAX;
  L.gemm_ws = take(gemm_path ? GEMM_WS_TILES * GEMM_TILE_FLOATS * 4 : 0);
  L.gemm_counters = take(gemm_path ? GEMM_WS_TILES * 4 : 0);
  L.mega_layers = take(f32 ? 0 : (size_t)c.n_layers * sizeof(MegaLayer));
  L.mega_bar = take(MEGA_BAR_WORDS * 4);
  L.mega_trace = take(MEGA_TRACE_WORDS * 8);
  L.xb_w = H > Qd ? H : Qd;
  if (I > L.xb_w) L.xb_w = I;
  L.xb = take(f32 ? 0 : 4 * SKINNY_MAX * L.xb_w * 2);
  L.oacc = take(f32 ? 0 : SKINNY_MAX * H * 8);
  L.total = o;
  return L;
}

// bytes of the fragment-order decode copy of one [rows][cols] linear layer
size_t tiled_bytes(const dpk_config& c, size_t rows, size_t cols) {
  if (c.weight_format == DPK_FMT_I8) return up(rows * cols);  // int8 codes
  if (c.weight_format == DPK_FMT_Q8) return up(rows * cols) + up(rows * (cols / 32) * 4);  // codes + block scales
  if (c.weight_format == DPK_FMT_Q40) return up(rows * cols / 2) + up(rows * (cols / 32) * 2);  // + fp16 scales
  if (c.weight_format == DPK_FMT_BF16) return up(rows * cols * 2);
  return up(rows * cols / 2) + up(rows * (cols / 64) * 4);  // codes + (s, b) pairs
}

// Block-scaled weights (MLX 4-bit, Q8, Q4_0) whose prefill copy rounds each
// weight to fp16, over an int8 KV cache: the K and V projections also get the
// rounding residual, so the keys and values the cache quantizes come from the
// exact weights (the rounding of the copy alone moved enough of them across a
// code boundary to take an 8B-shaped Q4_0 prefill to 0.03 from the exact
// logits, against 0.006 over the fp16 cache).
bool kv_lo_copy(const dpk_config& c) {
  return (c.flags & DPK_FLAG_KV_I8) &&
         (c.weight_format == DPK_FMT_Q4G64 || c.weight_format == DPK_FMT_Q8 || c.weight_format == DPK_FMT_Q40);
}

size_t prep_bytes(const dpk_config& c) {
  if (c.weight_format == DPK_FMT_F32) return 0;
  const size_t H = c.hidden, I = c.intermediate, d = c.head_dim;
  const size_t Nqkv = (c.n_heads + 2 * c.n_kv_heads) * d, Qd = (size_t)c.n_heads * d, KVd = (size_t)c.n_kv_heads * d;
  // fp16 prefill operands
  size_t per = up(Nqkv * H * 2) + up(H * Qd * 2) + 2 * up(I * H * 2) + up(H * I * 2);
  if (kv_lo_copy(c)) per += up(2 * KVd * H * 2);
  // decode copies
  per += tiled_bytes(c, Qd, H) + 2 * tiled_bytes(c, KVd, H) + tiled_bytes(c, H, Qd) + 2 * tiled_bytes(c, I, H) +
         tiled_bytes(c, H, I);
  return per * c.n_layers + tiled_bytes(c, c.vocab, H);
}

// positions per KV slab row: max_seq rounded up to a multiple of 64 so that
// 64-key tiles never leave a row
int kv_seq(const dpk_config& c) { return (c.max_seq + 63) / 64 * 64; }

// int8 cache: codes, then at a 256-byte boundary one fp32 scale per position and slab
size_t kv_code_bytes(const dpk_config& c) {
  const size_t elt = c.weight_format == DPK_FMT_F32 ? 4 : (c.flags & DPK_FLAG_KV_I8) ? 1 : 2;
  return (size_t)c.max_batch * c.n_layers * 2 * c.n_kv_heads * kv_seq(c) * c.head_dim * elt;
}

size_t kv_bytes(const dpk_config& c) {
  const size_t codes = kv_code_bytes(c);
  if (!(c.flags & DPK_FLAG_KV_I8)) return codes;
  return up(codes) + (size_t)c.max_batch * c.n_layers * 2 * c.n_kv_heads * kv_seq(c) * 4;
}

#define HIP_TRY(expr)                                                                  \
  do {                                                                                 \
    hipError_t _e = (expr);                                                            \
    if (_e != hipSuccess) {                                                            \
      md->failed = true;                                                               \
      return fail(DPK_EHIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(_e), __FILE__, __LINE__); \
    }                                                                                  \
  } while (0)

#define HIP_TRY_M(model, expr)                                                         \
  do {                                                                                 \
    hipError_t _e = (expr);                                                            \
    if (_e != hipSuccess) {                                                            \
      (model)->failed = true;                                                          \
      return fail(DPK_EHIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(_e), __FILE__, __LINE__); \
    }                                                                                  \
  } while (0)

enum KClass : int {
  K_GEMV_QKV, K_GEMV_O, K_GEMV_GATEUP, K_GEMV_DOWN, K_GEMV_HEAD, K_ATTN_DECODE, K_EMBED, K_GEMM_QKV, K_GEMM_O,
  K_GEMM_GATEUP, K_GEMM_DOWN, K_ATTN_PREFILL, K_QK_ROPE_KV, K_RMSNORM, K_GEMV_F32, K_DECODE_STEP, K_STEP_EMBED, K_STEP_QKV,
  K_STEP_ATTN, K_STEP_O, K_STEP_GATEUP, K_STEP_DOWN, K_STEP_HEAD, K_XPREP, K_OTHER, K_NCLASS
};
const char* const kclass_name[K_NCLASS] = {
    "gemv.qkv", "gemv.o", "gemv.gate_up", "gemv.down", "gemv.head", "attn.decode", "embed", "gemm.qkv", "gemm.o",
    "gemm.gate_up", "gemm.down", "attn.prefill", "qk_rope_kv", "rmsnorm", "gemv.f32", "decode.step", "step.embed", "step.qkv",
    "step.attn", "step.o", "step.gate_up", "step.down", "step.head", "xprep", "other"};

// Start/stop events of the launches of one kernel class when profiling is on.
struct ProfScope {
  dpk_model* md;
  hipStream_t st;
  int idx = -1;
  ProfScope(dpk_model* m, hipStream_t s, int cls, double bytes, double flops) : md(m), st(s) {
    if (!md->prof) return;
    if ((int)md->prof_rec.size() >= md->prof_max) {
      ++md->prof_dropped;
      return;
    }
    idx = (int)md->prof_rec.size();
    md->prof_rec.push_back({cls, bytes, flops});
    g_timing.start = md->prof_ev[2 * idx];
    g_timing.stop = md->prof_ev[2 * idx + 1];
  }
  ~ProfScope() { g_timing = LaunchTiming{}; }
};

double wbytes_per_elem(int fmt) {
  return fmt == DPK_FMT_F32 ? 4.0 : fmt == DPK_FMT_BF16 ? 2.0 : fmt == DPK_FMT_I8 ? 1.0 :
         fmt == DPK_FMT_Q8 ? 1.0 + 4.0 / 32.0 : fmt == DPK_FMT_Q40 ? 0.5 + 2.0 / 32.0 : 0.5 + 4.0 / 64.0;
}

// Kernel weight format of the model's linear layers (bf16 / q4 / i8 / q8 / q4_0 models).
int wfmt(const dpk_model* md) {
  switch (md->fmt) {
    case DPK_FMT_Q4G64: return W_Q4;
    case DPK_FMT_I8: return W_I8;
    case DPK_FMT_Q8: return W_Q8;
    case DPK_FMT_Q40: return W_Q40;
    default: return W_BF16;
  }
}

bool int_code_fmt(int fmt) { return fmt == DPK_FMT_I8 || fmt == DPK_FMT_Q8 || fmt == DPK_FMT_Q40; }

// Scales the embedding gather takes: fp32 (q8) or fp16 (q4_0) block scales, or bf16 ones.
const void* embed_scales(const dpk_model* md) {
  return (md->fmt == DPK_FMT_Q8 || md->fmt == DPK_FMT_Q40) ? (const void*)md->embed.sf : (const void*)md->embed.sc;
}

dpk_status check_ready(const dpk_model* md) {
  if (!md) return fail(DPK_EINVAL, "null model");
  if (md->failed) return fail(DPK_ESTATE, "model is in a failed state after an earlier HIP error");
  if (!md->bound) return fail(DPK_ESTATE, "workspace not bound (call dpk_bind_workspace)");
  if (!md->loaded) return fail(DPK_ESTATE, "weights not loaded (call dpk_load_weights)");
  return DPK_OK;
}

// Stage row parameters into pinned memory and enqueue the upload.
dpk_status upload_rows(dpk_model* md, const RowParam* rows, int n, hipStream_t st) {
  int s = md->stage_next;
  md->stage_next = (s + 1) % dpk_model::NSTAGE;
  if (md->stage_used[s]) HIP_TRY(hipEventSynchronize(md->stage_ev[s]));
  memcpy(md->stage[s], rows, sizeof(RowParam) * n);
  HIP_TRY(hipMemcpyAsync(md->rows_dev, md->stage[s], sizeof(RowParam) * n, hipMemcpyHostToDevice, st));
  HIP_TRY(hipEventRecord(md->stage_ev[s], st));
  md->stage_used[s] = true;
  return DPK_OK;
}

#ifndef SKINNY_I8_WG_TARGET
#define SKINNY_I8_WG_TARGET 256
#endif
// Smallest K split that fits the activation chunk in 64 KB of LDS, grown until
// the launch has ~1024 workgroups (4 per compute unit).  The int8-code GEMV
// stops at ~256: its workgroups pay a longer prologue (two passes over x),
// and fewer, longer ones measured faster (8B shapes, 256 / 512 / 1024 / 2048 /
// 4096 workgroups: gate/up 21.8 / 21.8 / 23.0 / 25.5 / 37.2 us).
int choose_ksplit(int K, int nblocks, int M, int rows, int fmt) {
  const long target = (fmt == W_I8 || fmt == W_Q8 || fmt == W_Q40) ? SKINNY_I8_WG_TARGET : 1024;
  int best = 0;
  for (int ks = 1; ks <= KSPLIT_MAX; ks *= 2) {
    if (K % (ks * 256) != 0) break;
    const int kchunk = K / ks;
    if (skinny_lds_bytes(M, kchunk, rows, fmt) > 64 * 1024) continue;
    best = ks;
    if ((long)nblocks * ks >= target) break;
  }
  return best;
}

// One weight-streaming GEMV launch (M <= 16).
dpk_status skinny(dpk_model* md, int cls, int M, const float* x, int ldx, const float* rs, const void* gain,
                  const LinearW* segs, int nseg, int epi, float* out, int ldo, hipStream_t st,
                  int layer = 0) {
  const dpk_config& c = md->cfg;
  SkinnyArgs a{};
  a.M = M;
  a.K = segs[0].cols;
  a.fmt = wfmt(md);
  int n = 0;
  for (int i = 0; i < 3; ++i) {
    const LinearW& s = segs[i < nseg ? i : nseg - 1];
    a.w[i] = int_code_fmt(md->fmt) ? s.wt : s.w;
    a.sc[i] = s.sc;
    a.bi[i] = s.bi;
    a.sf[i] = (const float*)s.sbt;
    if (i < nseg) n += s.rows;
    a.seg_end[i] = n;
    a.seg_rows[i] = s.rows;
  }
  a.N = (epi == EPI_SWIGLU) ? segs[0].rows : n;
  a.rows_per_wg = (epi == EPI_QKV) ? c.head_dim : 64;
  const int rows_total = (epi == EPI_SWIGLU) ? 2 * segs[0].rows : n;
  a.n_blocks = (rows_total + a.rows_per_wg - 1) / a.rows_per_wg;
  if (rows_total % a.rows_per_wg != 0)
    return fail(DPK_EINVAL, "output rows %d not a multiple of %d", rows_total, a.rows_per_wg);
  a.ksplit = choose_ksplit(a.K, a.n_blocks, M, a.rows_per_wg, a.fmt);
  if (a.ksplit == 0) return fail(DPK_EINVAL, "no K split for K=%d M=%d", a.K, M);
  a.kchunk = a.K / a.ksplit;
  if ((size_t)a.ksplit * M * a.n_blocks * a.rows_per_wg > md->part_floats)
    return fail(DPK_EINVAL, "partial buffer too small");
  a.x = x;
  a.ldx = ldx;
  a.rs = rs;
  a.gain = (const uint16_t*)gain;
  a.part = md->part;
  a.counters = md->counters;
  a.epi = epi;
  a.out = out;
  a.ldo = ldo;
  a.sq = md->sq;
  a.rs_out = md->rs;
  a.eps = c.rms_eps;
  a.rows_param = md->rows_dev;
  a.rope_cos = md->rope_cos;
  a.rope_sin = md->rope_sin;
  a.qout = md->qbuf;
  a.n_heads = c.n_heads;
  a.layer = layer;
  a.kv = md->kvd;
  a.cand_val = md->cand_val;
  a.cand_idx = md->cand_idx;
  if (epi == EPI_QKV) {
    const LayerW& L = md->layers[layer];
    a.qn = c.qk_norm ? (const uint16_t*)L.q_norm : nullptr;
    a.kn = c.qk_norm ? (const uint16_t*)L.k_norm : nullptr;
    if (!c.qk_norm) return fail(DPK_EINVAL, "fused QKV epilogue needs qk_norm");
  }
  {
    const double nrows = (epi == EPI_SWIGLU) ? 2.0 * a.N : (double)a.N;
    const double wb = nrows * a.K * wbytes_per_elem(md->fmt);
    const double io = (double)M * a.K * 4 + (double)M * a.N * 4;
    ProfScope ps(md, st, cls, wb + io, 2.0 * M * nrows * a.K);
    HIP_TRY(launch_skinny(a, st));
  }
  return DPK_OK;
}

// one_seq: the rows are positions of one sequence (not with qkv_raw); on the
// fp16-cache kernel their query heads then share each chunk's cache reads.
// out16: if non-null (fp16-cache kernel only), the output goes there as bf16
// hi / lo rows instead of to out.
dpk_status attn_decode(dpk_model* md, int M, int max_ctx, const float* q, float* out, int layer, hipStream_t st,
                       double kv_positions, const float* qkv_raw = nullptr, bool one_seq = false,
                       uint16_t* const* out16 = nullptr) {
  const dpk_config& c = md->cfg;
  AttnDecodeArgs a{};
  a.M = M;
  a.n_heads = c.n_heads;
  a.n_kv = c.n_kv_heads;
  a.d = c.head_dim;
  a.rows_param = md->rows_dev;
  a.q = q;
  a.kv = md->kvd;
  a.layer = layer;
  a.share = (one_seq && !qkv_raw && !md->kvd.is_f32) ? 16 / (c.n_heads / c.n_kv_heads) : 1;
  if (a.share > M) a.share = M;
  a.chunk = md->kvd.is_f32 ? attn_decode_chunk()
                           : attn_decode_mfma_chunk(max_ctx, (M + a.share - 1) / a.share * c.n_kv_heads, md->n_cu);
  a.max_chunks = (max_ctx + a.chunk - 1) / a.chunk;
  if (a.max_chunks > md->attn_chunks_cap) return fail(DPK_EINVAL, "attention chunk cap");
  a.part = md->attn_part;
  a.counters = md->attn_counters;
  a.out = out;
  a.scale = 1.0f / sqrtf((float)c.head_dim);
  a.merge = a.max_chunks > 1 || out16;  // a second launch merges the chunks
  if (out16) {
    if (md->kvd.is_f32) return fail(DPK_EINVAL, "internal: split attention output needs the fp16 cache");
    a.out_hi = out16[0];
    a.out_lo = out16[1];
  }
  if (qkv_raw) {
    const LayerW& L = md->layers[layer];
    a.qkv_raw = qkv_raw;
    a.ld_raw = md->Nqkv;
    a.qn = c.qk_norm ? (const uint16_t*)L.q_norm : nullptr;
    a.kn = c.qk_norm ? (const uint16_t*)L.k_norm : nullptr;
    a.rope_cos = md->rope_cos;
    a.rope_sin = md->rope_sin;
    a.eps = c.rms_eps;
  }
  {
    const double elt = md->kvd.is_f32 ? 4 : md->kvd.i8 ? 1 + 4.0 / c.head_dim : 2;
    const double kvb = kv_positions * 2.0 * c.n_kv_heads * c.head_dim * elt;
    const double io = 2.0 * M * c.n_heads * c.head_dim * 4;
    ProfScope ps(md, st, K_ATTN_DECODE, kvb + io, 4.0 * kv_positions * c.n_heads * c.head_dim);
    HIP_TRY(md->kvd.is_f32 ? launch_attn_decode(a, st) : launch_attn_decode_mfma(a, st));
  }
  return DPK_OK;
}

// One decode GEMV launch (whole K per workgroup, gemv.hip).
GemvArgs gemv_args(dpk_model* md, int M, const float* x, int ldx, const float* sq_in, int sq_nb, const void* gain,
                   const LinearW* segs, int nseg, int epi, bool swiglu, int tiles, float* out, int ldo, float* sq_out,
                   int32_t* argmax) {
  const dpk_config& c = md->cfg;
  GemvArgs a{};
  a.M = M;
  a.K = segs[0].cols;
  a.fmt = wfmt(md);
  a.tiles = tiles;
  a.swiglu = swiglu;
  a.epi = epi;
  int n = 0;
  for (int i = 0; i < 3; ++i) {
    const LinearW& sg = segs[i < nseg ? i : nseg - 1];
    a.w[i] = sg.wt;
    a.sb[i] = md->fmt == DPK_FMT_I8 ? (const void*)sg.sc : sg.sbt;  // int8: the bf16 row scales as given
    if (i < nseg) n += sg.rows;
    a.seg_end[i] = n;
    a.seg_rows[i] = sg.rows;
  }
  a.N = swiglu ? segs[0].rows : n;
  a.grid = md->n_cu;
  a.x = x;
  a.ldx = ldx;
  a.sq_in = sq_in;
  a.sq_nb = sq_nb;
  a.gain = (const uint16_t*)gain;
  a.eps = c.rms_eps;
  a.out = out;
  a.ldo = ldo;
  a.sq_out = sq_out;
  a.counters = md->counters;
  a.cand_val = md->cand_val;
  a.cand_idx = md->cand_idx;
  a.argmax_out = argmax ? argmax : md->argmax_sink;
  return a;
}

dpk_status gemv(dpk_model* md, int cls, int M, const float* x, int ldx, const float* sq_in, int sq_nb,
                const void* gain, const LinearW* segs, int nseg, int epi, bool swiglu, int tiles, float* out,
                int ldo, float* sq_out, int32_t* argmax, hipStream_t st) {
  const GemvArgs a = gemv_args(md, M, x, ldx, sq_in, sq_nb, gain, segs, nseg, epi, swiglu, tiles, out, ldo, sq_out,
                               argmax);
  const double nrows = swiglu ? 2.0 * a.N : (double)a.N;
  ProfScope ps(md, st, cls, nrows * a.K * wbytes_per_elem(md->fmt) + (double)M * a.K * 4 + (double)M * a.N * 4,
               2.0 * M * nrows * a.K);
  HIP_TRY(launch_gemv(a, st));
  return DPK_OK;
}

// One GEMV launch on ready-made bf16 hi / lo activations xin (xg_index
// layout, rows xrow0 .. xrow0 + M - 1; sq_in: per-row sums of squares whose
// norm scale the outputs take).  xout: where a RESID / SWIGLU epilogue also
// writes the next GEMV's activations (times xo_gain for RESID).
dpk_status gemv_xg(dpk_model* md, int cls, int M, uint16_t* const* xin, int xrow0, const float* sq_in, int sq_nb,
                   const LinearW* segs, int nseg, int epi, bool swiglu, int tiles, float* out, int ldo,
                   float* sq_out, int32_t* argmax, uint16_t* const* xout, const void* xo_gain, hipStream_t st) {
  GemvArgs a = gemv_args(md, M, nullptr, 0, sq_in, sq_nb, nullptr, segs, nseg, epi, swiglu, tiles, out, ldo, sq_out,
                         argmax);
  a.xb_hi = xin[0];
  a.xb_lo = xin[1];
  a.xrow0 = xrow0;
  // up to two row tiles per compute unit all at once (the 4-wave workgroups
  // fit two to a unit), else a persistent grid
  const int n_tiles = (swiglu ? 2 * a.N : a.N) / (16 * tiles);
  if (epi != EPI_HEAD && n_tiles > a.grid && n_tiles <= 2 * a.grid) a.grid = n_tiles;
  if (epi == EPI_HEAD && M > 8) a.grid = 2 * md->n_cu;  // measured: more rows want more workgroups in flight
  if (epi == EPI_HEAD && a.grid > MAX_HEAD_WG) return fail(DPK_EINVAL, "lm_head grid beyond the candidate buffer");
  if (xout) {
    a.xo_hi = xout[0];
    a.xo_lo = xout[1];
    a.xo_gain = (const uint16_t*)xo_gain;
  }
  const double nrows = swiglu ? 2.0 * a.N : (double)a.N;
  const double outb = (xout ? 4.0 : 0.0) * M * a.N + (epi == EPI_SWIGLU && xout ? 0.0 : 4.0 * M * a.N);
  ProfScope ps(md, st, cls, nrows * a.K * 2.0 + (double)M * a.K * 4 + outb, 2.0 * M * nrows * a.K);
  HIP_TRY(launch_gemv(a, st));
  return DPK_OK;
}

// Can M rows of this model run on the ready-made-activation GEMVs?
bool batch_fits(const dpk_model* md, int M) {
  const dpk_config& c = md->cfg;
  if (md->fmt != DPK_FMT_BF16 || !md->xb[0][0] || M < 1 || M > SKINNY_MAX) return false;
  for (int K : {c.hidden, c.n_heads * c.head_dim, c.intermediate})
    if (K % 1024) return false;
  // 32-row tiles for QKV and the head, 16-row segments
  if (md->Nqkv % 32 || c.vocab % 32 || (c.n_kv_heads * c.head_dim) % 16) return false;
  return true;
}

// M rows (parameters in md->rows_dev; one_seq: consecutive positions of one
// sequence, as in a verify pass, else distinct sequences with one new position
// each) on the ready-made-activation GEMVs.  Each layer: QKV GEMV -> [QK-norm,
// RoPE, KV write] -> attention (its chunk merge writing the O GEMV's bf16
// hi / lo activations) -> O GEMV + residual
// (writing norm-gained bf16 activations of the new h) -> gate/up GEMV + SwiGLU
// (writing the down GEMV's activations) -> down GEMV + residual (writing the
// next layer's QKV activations); the row norm scales are applied to the GEMV
// outputs.  Then the lm_head on rows [head_r0, head_r0 + head_n).
dpk_status forward_batch(dpk_model* md, int M, int max_ctx, const int32_t* ids_dev, int head_r0, int head_n,
                         float* logits, int32_t* argmax, hipStream_t st, double kv_positions, bool one_seq) {
  const dpk_config& c = md->cfg;
  const int H = c.hidden, Qd = c.n_heads * c.head_dim, I = c.intermediate;
  uint16_t* const* X0 = md->xb[0];
  uint16_t* const* X1 = md->xb[1];
  {
    ProfScope ps(md, st, K_EMBED, (double)M * H * 6, 0);
    HIP_TRY(launch_embed(M, H, W_BF16, md->embed.w, md->embed.sc, md->embed.bi, md->rows_dev, ids_dev, c.vocab,
                         md->h, nullptr, c.rms_eps, md->err_flag, st, md->sq));
  }
  {
    ProfScope ps(md, st, K_XPREP, (double)M * H * 8, 0);
    HIP_TRY(launch_xprep(M, H, md->h, H, nullptr, 0, (const uint16_t*)md->layers[0].in_norm, c.rms_eps, X0[0], X0[1],
                         st));
  }
  int sq_nb = 1;
  dpk_status s;
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& L = md->layers[l];
    LinearW qkv[3] = {L.q, L.k, L.v};
    // 32-row tiles for QKV and the head (each activation fragment serves two
    // weight tiles; measured faster there), 16-row tiles for O and down
    if ((s = gemv_xg(md, K_GEMV_QKV, M, X0, 0, md->sq, sq_nb, qkv, 3, EPI_STORE, false, 2, md->qkv, md->Nqkv,
                     nullptr, nullptr, nullptr, nullptr, st)))
      return s;
    if (one_seq) {
      {
        ProfScope ps(md, st, K_QK_ROPE_KV, (double)M * md->Nqkv * 6, 0);
        HIP_TRY(launch_qk_rope_kv(M, md->qkv, c.n_heads, c.n_kv_heads, c.head_dim, c.qk_norm, L.q_norm, L.k_norm, 0,
                                  c.rms_eps, md->rope_cos, md->rope_sin, md->rows_dev, md->qbuf, 0, md->kvd, l, st));
      }
      if ((s = attn_decode(md, M, max_ctx, md->qbuf, md->attn_o, l, st, kv_positions, nullptr, true, X1))) return s;
    } else if ((s = attn_decode(md, M, max_ctx, nullptr, md->attn_o, l, st, kv_positions, md->qkv, false, X1))) {
      return s;
    }
    if ((s = gemv_xg(md, K_GEMV_O, M, X1, 0, nullptr, 0, &L.o, 1, EPI_RESID, false, 1, md->h, H, md->sq, nullptr,
                     X0, L.post_norm, st)))
      return s;
    sq_nb = H / 16;
    LinearW gu[2] = {L.gate, L.up};
    if ((s = gemv_xg(md, K_GEMV_GATEUP, M, X0, 0, md->sq, sq_nb, gu, 2, EPI_SWIGLU, true, 2, md->act, I, nullptr,
                     nullptr, X1, nullptr, st)))
      return s;
    const void* next_gain = l + 1 < c.n_layers ? md->layers[l + 1].in_norm : md->final_norm;
    if ((s = gemv_xg(md, K_GEMV_DOWN, M, X1, 0, nullptr, 0, &L.down, 1, EPI_RESID, false, 1, md->h, H, md->sq,
                     nullptr, X0, next_gain, st)))
      return s;
  }
  if (head_n <= 0) return DPK_OK;
  float* dst = logits ? logits : md->sink;
  return gemv_xg(md, K_GEMV_HEAD, head_n, X0, head_r0, md->sq + (size_t)head_r0 * sq_nb, sq_nb, &md->head, 1,
                 EPI_HEAD, false, 2, dst, c.vocab, nullptr, argmax, nullptr, nullptr, st);
}

// Can a decode step of M rows run on the whole-K GEMV kernels?
bool decode_fits(const dpk_model* md, int M) {
  if (md->fmt != DPK_FMT_BF16 && md->fmt != DPK_FMT_Q4G64 && md->fmt != DPK_FMT_I8) return false;
  const dpk_config& c = md->cfg;
  const int fmt = wfmt(md);
  for (int K : {c.hidden, c.n_heads * c.head_dim, c.intermediate}) {
    if (K % 1024) return false;
    if (gemv_lds_bytes(M, K, 4, fmt) > 64 * 1024) return false;
  }
  return true;
}

// Decode step of M rows (distinct sequences, one new position each) whose
// parameters are in md->rows_dev: every layer is QKV GEMV -> attention (with
// QK-norm, RoPE and the KV write) -> O GEMV + residual -> gate/up GEMV +
// SwiGLU -> down GEMV + residual; then the lm_head with the greedy argmax.
constexpr int HEAD_I8_TILES = 4;  // the one-launch-per-kernel int8 lm_head's 16-row tiles per tile
dpk_status forward_decode(dpk_model* md, int M, int max_ctx, const int32_t* ids_dev, float* logits, int32_t* argmax,
                          hipStream_t st, double kv_positions) {
  const dpk_config& c = md->cfg;
  const int H = c.hidden, Qd = c.n_heads * c.head_dim;
  {
    ProfScope ps(md, st, K_EMBED, (double)M * H * 6, 0);
    HIP_TRY(launch_embed(M, H, wfmt(md), md->embed.w, embed_scales(md), md->embed.bi,
                         md->rows_dev, ids_dev, c.vocab, md->h, nullptr, c.rms_eps, md->err_flag, st, md->sq));
  }
  int sq_nb = 1;
  const int nb_resid = H / 16;
  dpk_status s;
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& L = md->layers[l];
    LinearW qkv[3] = {L.q, L.k, L.v};
    if ((s = gemv(md, K_GEMV_QKV, M, md->h, H, md->sq, sq_nb, L.in_norm, qkv, 3, EPI_STORE, false, 1, md->qkv,
                  md->Nqkv, nullptr, nullptr, st)))
      return s;
    if ((s = attn_decode(md, M, max_ctx, nullptr, md->attn_o, l, st, kv_positions, md->qkv))) return s;
    if ((s = gemv(md, K_GEMV_O, M, md->attn_o, Qd, nullptr, 0, nullptr, &L.o, 1, EPI_RESID, false, 1, md->h, H, md->sq,
                  nullptr, st)))
      return s;
    sq_nb = nb_resid;
    LinearW gu[2] = {L.gate, L.up};
    if ((s = gemv(md, K_GEMV_GATEUP, M, md->h, H, md->sq, sq_nb, L.post_norm, gu, 2, EPI_SWIGLU, true, 2, md->act,
                  c.intermediate, nullptr, nullptr, st)))
      return s;
    if ((s = gemv(md, K_GEMV_DOWN, M, md->act, c.intermediate, nullptr, 0, nullptr, &L.down, 1, EPI_RESID, false, 1,
                  md->h, H, md->sq, nullptr, st)))
      return s;
  }
  float* dst = logits ? logits : md->sink;
  // (int8: 64-row tiles; fewer tiles per workgroup measured faster: 0.6B head 78.8 -> 46.3 us)
  return gemv(md, K_GEMV_HEAD, M, md->h, H, md->sq, sq_nb, md->final_norm, &md->head, 1, EPI_HEAD, false,
              md->fmt == DPK_FMT_I8 ? HEAD_I8_TILES : 1, dst, c.vocab, nullptr, argmax, st);
}

// GEMV tiling of the persistent decode kernel for the loaded model: 0 when
// every GEMV row splits over eight waves at 256 columns per iteration (bf16,
// int8 per row, Q8, Q4_0), 1 at 128 columns (every row length a multiple of 1024;
// bf16 or MLX 4-bit), -1 when neither fits.
int mega_variant(const dpk_model* md) {
  const dpk_config& c = md->cfg;
  const int H = c.hidden, Qd = c.n_heads * c.head_dim, I = c.intermediate;
  if (md->fmt == DPK_FMT_BF16 && gemv_waves(H, 1, W_BF16) == 8 && gemv_waves(Qd, 1, W_BF16) == 8 &&
      gemv_waves(H, 2, W_BF16) == 8 && gemv_waves(I, 1, W_BF16) == 8)
    return 0;
  if ((md->fmt == DPK_FMT_BF16 || md->fmt == DPK_FMT_Q4G64) && H % 1024 == 0 && Qd % 1024 == 0 && I % 1024 == 0)
    return 1;
  // int8 codes with one scale per row: 256 columns per iteration on eight waves only
  if (md->fmt == DPK_FMT_I8 && gemv_waves(H, 1, W_I8) == 8 && gemv_waves(Qd, 1, W_I8) == 8 &&
      gemv_waves(H, 2, W_I8) == 8 && gemv_waves(I, 1, W_I8) == 8)
    return 0;
  // Q4_0: 512 (one-tile GEMVs: O, down) or 256 columns or fewer per wave and
  // iteration on eight waves; gate / up in 96-row and the lm_head in 64-row tiles
  if (md->fmt == DPK_FMT_Q40 && H % 2048 == 0 && Qd % 4096 == 0 && I % 4096 == 0 &&
      (2 * I) % (16 * mega_gu_tiles(W_Q40)) == 0 && c.vocab % (16 * mega_head_tiles(W_Q40, false)) == 0)
    return 0;
  // Q8: 256 columns or fewer per wave and iteration, whole 256-column chunks of
  // block scales per wave; the lm_head in 64-row tiles
  if (md->fmt == DPK_FMT_Q8 && H % 2048 == 0 && Qd % 2048 == 0 && I % 2048 == 0 &&
      (2 * I) % (16 * mega_gu_tiles(W_Q8)) == 0 && c.vocab % (16 * mega_head_tiles(W_Q8, false)) == 0)
    return 0;
  return -1;
}

// 16-row tiles per O-projection item when the persistent step runs the O
// projection inside the attention phase (bf16 weights, hidden size 2048 or
// more; the largest of 8, 4, 2, 1 that still gives every compute unit an
// item), 0 when it runs as a GEMV after attention.  Measured on the 1024-wide
// 0.6B shapes the fused phase saves ~1.9 us per layer but the O sums cost
// gate/up and down ~2 us, so narrow models keep the GEMV.
int mega_o_rt(const dpk_model* md, int M) {
  const dpk_config& c = md->cfg;
  // (attention keeps at most half the grid: the rest, at least n_kv
  // workgroups, runs the O projection)
  if (md->fmt != DPK_FMT_BF16 || !md->oacc || c.hidden < 2048 || c.n_kv_heads > 16 || c.hidden % 16 ||
      md->n_cu < 2 * c.n_kv_heads)
    return 0;
  const int G = c.n_heads / c.n_kv_heads, tiles = c.hidden / 16;
  for (int rt = 8; rt >= 1; rt /= 2) {
    if (tiles % rt || (rt > 1 && (tiles / rt) * c.n_kv_heads < md->n_cu)) continue;
    if (mega_o_lds_bytes(M, G, rt)) return rt;
  }
  return 0;
}

// LDS bytes of the persistent decode kernel for M rows, or 0 if the model or
// M does not fit it: bf16, MLX 4-bit, int8-per-row, Q8 or Q4_0 weights (with an
// int8 KV cache: bf16 with the fused O projection, int8, Q8 or Q4_0), head_dim 128, 1, 2 or 4 query
// heads per KV head (2 or 4 for the 128-column tiling), every GEMV on eight
// waves, LDS within the device's per-workgroup limit, one resident workgroup
// per CU.
size_t mega_lds_for(dpk_model* md, int M, int max_ctx) {
  const dpk_config& c = md->cfg;
  if ((c.flags & DPK_FLAG_DECODE_MULTI) || !md->mega_layers) return 0;
  if (c.head_dim != 128 || c.n_heads % c.n_kv_heads) return 0;
  const int G = c.n_heads / c.n_kv_heads;
  if (G != 1 && G != 2 && G != 4) return 0;
  // (the integer-code formats are bounded by the LDS check below alone: their
  // one-launch-per-kernel GEMVs are not the gemv_kernel decode_fits sizes)
  if (md->fmt != DPK_FMT_Q40 && md->fmt != DPK_FMT_Q8 && md->fmt != DPK_FMT_I8 && !decode_fits(md, M)) return 0;
  const int var = mega_variant(md);
  if (var < 0) return 0;
  const int fmt = wfmt(md);
  const int H = c.hidden, Qd = c.n_heads * c.head_dim, I = c.intermediate;
  if ((max_ctx + mega_attn_chunk() - 1) / mega_attn_chunk() > MEGA_ATTN_MAXCH) return 0;
  size_t lds = mega_attn_lds_bytes(G);
  if (const int ort = mega_o_rt(md, M)) {
    const size_t ob = mega_o_lds_bytes(M, G, ort);
    if (ob > lds) lds = ob;
  }
  for (size_t b : {gemv_lds_bytes_waves(M, H, var ? 1 : 2, fmt, 8), gemv_lds_bytes_waves(M, Qd, 1, fmt, 8),
                   gemv_lds_bytes_waves(M, H, mega_gu_tiles(fmt), fmt, 8), gemv_lds_bytes_waves(M, I, 1, fmt, 8),
                   gemv_lds_bytes_waves(M, H, mega_head_tiles(fmt, var == 1), fmt, 8)})
    lds = b > lds ? b : lds;
  // + the staged layer / head arguments and row parameters, + (bf16) the
  // GEMVs' prefetch slots
  lds = (lds + 15) / 16 * 16 + MEGA_ARGS_LDS + (fmt == W_BF16 ? MEGA_PF_LDS : 0);
  if (lds > (size_t)md->lds_max) return 0;
  // (an int8 KV cache: the 256-column variants with bf16 weights and the
  // fused O projection, or int8 weights; mega_occupancy is 0 for the others)
  if (mega_occupancy(G, fmt, var == 1, mega_o_rt(md, M) > 0, (c.flags & DPK_FLAG_KV_I8) != 0, lds) < 1) return 0;
  return lds;
}

// Device table of the per-layer GEMV arguments of the persistent kernel.
dpk_status mega_table(dpk_model* md, hipStream_t st) {
  const dpk_config& c = md->cfg;
  const int H = c.hidden, Qd = c.n_heads * c.head_dim, I = c.intermediate;
  std::vector<MegaLayer> t(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& L = md->layers[l];
    LinearW qkv[3] = {L.q, L.k, L.v};
    LinearW gu[2] = {L.gate, L.up};
    t[l].qkv = gemv_args(md, 1, md->h, H, md->sq, H / 16, L.in_norm, qkv, 3, EPI_STORE, false,
                         mega_variant(md) == 1 ? 1 : 2, md->qkv, md->Nqkv, nullptr, nullptr);
    t[l].o = gemv_args(md, 1, md->attn_o, Qd, nullptr, 0, nullptr, &L.o, 1, EPI_RESID, false, 1, md->h, H, md->sq,
                       nullptr);
    t[l].gu = gemv_args(md, 1, md->h, H, md->sq, H / 16, L.post_norm, gu, 2, EPI_SWIGLU, true, 2, md->act, I, nullptr,
                        nullptr);
    t[l].down = gemv_args(md, 1, md->act, I, nullptr, 0, nullptr, &L.down, 1, EPI_RESID, false, 1, md->h, H, md->sq,
                          nullptr);
    // the fixed-point O sums (zero when the O projection runs as a GEMV)
    // join h where gate/up stages it and where down adds to it
    if (md->fmt == DPK_FMT_BF16) {
      t[l].gu.xacc = md->oacc;
      t[l].down.racc = md->oacc;
    }
    t[l].qn = c.qk_norm ? (const uint16_t*)L.q_norm : nullptr;
    t[l].kn = c.qk_norm ? (const uint16_t*)L.k_norm : nullptr;
  }
  HIP_TRY(hipMemcpyAsync(md->mega_layers, t.data(), sizeof(MegaLayer) * t.size(), hipMemcpyHostToDevice, st));
  HIP_TRY(hipStreamSynchronize(st));  // t is a host temporary
  md->mega_table = true;
  return DPK_OK;
}

// Decode step of M rows (parameters in md->rows_dev) as one persistent launch.
// rows: the M rows' parameters (host), passed in the launch arguments.
dpk_status forward_mega(dpk_model* md, int M, int max_ctx, size_t lds, const RowParam* rows, const int32_t* ids_dev,
                        float* logits, int32_t* argmax, hipStream_t st, double kv_positions) {
  const dpk_config& c = md->cfg;
  dpk_status s;
  if (!md->mega_table && (s = mega_table(md, st))) return s;
  const int H = c.hidden;
  MegaArgs a{};
  a.M = M;
  a.n_layers = c.n_layers;
  a.H = H;
  a.vocab = c.vocab;
  a.layers = md->mega_layers;
  a.head = gemv_args(md, M, md->h, H, md->sq, H / 16, md->final_norm, &md->head, 1, EPI_HEAD, false, 1,
                     logits ? logits : md->sink, c.vocab, nullptr, argmax);
  a.fmt = wfmt(md);
  a.small = mega_variant(md) == 1;
  a.emb = md->embed.w;
  a.emb_sc = (const uint16_t*)embed_scales(md);
  a.emb_bi = md->embed.bi;
  if (M > 16) return fail(DPK_EINVAL, "internal: persistent step of more than 16 rows");
  for (int m = 0; m < M; ++m) a.rows[m] = rows[m];
  a.ids_dev = ids_dev;
  a.h = md->h;
  a.sq = md->sq;
  a.err = md->err_flag;
  a.n_heads = c.n_heads;
  a.n_kv = c.n_kv_heads;
  a.kv = md->kvd;
  a.qkv = md->qkv;
  a.ld_qkv = md->Nqkv;
  a.rope_cos = md->rope_cos;
  a.rope_sin = md->rope_sin;
  a.eps = c.rms_eps;
  a.scale = 1.0f / sqrtf((float)c.head_dim);
  a.max_chunks = (max_ctx + mega_attn_chunk() - 1) / mega_attn_chunk();
  a.part = md->attn_part;
  a.attn_counters = md->attn_counters;
  a.attn_out = md->attn_o;
  a.o_rt = mega_o_rt(md, M);
  a.oacc = a.o_rt ? md->oacc : nullptr;
  a.bar = md->mega_bar;
  a.trace = md->prof ? md->mega_trace : nullptr;
  a.lds_args = (int)(lds - MEGA_ARGS_LDS - (md->fmt == DPK_FMT_BF16 ? MEGA_PF_LDS : 0));
  // algorithmic work: every linear weight (lm_head included) once, the KV of
  // every attended position, the new positions' K/V
  const double Qd = (double)c.n_heads * c.head_dim;
  const double params = (double)c.n_layers * ((double)md->Nqkv * H + H * Qd + 3.0 * c.intermediate * H) +
                        (double)c.vocab * H;
  const double kv_elt = md->kvd.i8 ? 1 + 4.0 / c.head_dim : 2.0;  // (int8 cache: codes + one fp32 scale per vector)
  const double kvb = (kv_positions + M) * 2.0 * c.n_kv_heads * c.head_dim * kv_elt * c.n_layers;
  ProfScope ps(md, st, K_DECODE_STEP, params * wbytes_per_elem(md->fmt) + kvb,
               2.0 * M * params + 4.0 * kv_positions * Qd * c.n_layers);
  if (md->prof) md->prof_step_kv += kv_positions + M;
  if (md->n_cu > MAX_HEAD_WG) return fail(DPK_EINVAL, "more compute units than the candidate buffer holds");
  HIP_TRY(launch_decode_step(a, c.n_heads / c.n_kv_heads, md->n_cu, lds, st));
  return DPK_OK;
}

// Final norm + lm_head + greedy argmax for `rows` rows of x (weight-streaming
// path).  x' = x * rs * gain; logits go to the caller's buffer or a sink.
dpk_status head(dpk_model* md, int rows, const float* x, const float* rs, const void* gain, float* logits,
                int32_t* argmax, hipStream_t st) {
  const dpk_config& c = md->cfg;
  const int H = c.hidden;
  const LinearW& hw = md->head;
  SkinnyArgs h{};
  h.M = rows;
  h.K = H;
  h.fmt = wfmt(md);
  for (int i = 0; i < 3; ++i) {
    h.w[i] = int_code_fmt(md->fmt) ? hw.wt : hw.w;
    h.sc[i] = hw.sc;
    h.bi[i] = hw.bi;
    h.sf[i] = (const float*)hw.sbt;
    h.seg_end[i] = hw.rows;
    h.seg_rows[i] = hw.rows;
  }
  h.N = hw.rows;
  h.rows_per_wg = 64;
  h.n_blocks = (hw.rows + 63) / 64;
  h.ksplit = choose_ksplit(H, h.n_blocks, rows, 64, h.fmt);
  if (h.ksplit == 0) return fail(DPK_EINVAL, "no K split for the head");
  h.kchunk = H / h.ksplit;
  if ((size_t)h.ksplit * rows * h.n_blocks * 64 > md->part_floats) return fail(DPK_EINVAL, "partial buffer too small");
  h.x = x;
  h.ldx = H;
  h.rs = rs;
  h.gain = (const uint16_t*)gain;
  h.part = md->part;
  h.counters = md->counters;
  h.epi = EPI_HEAD;
  h.out = logits ? logits : md->sink;
  h.ldo = c.vocab;
  h.eps = c.rms_eps;
  h.cand_val = md->cand_val;
  h.cand_idx = md->cand_idx;
  h.argmax_out = argmax ? argmax : md->argmax_sink;
  {
    const double wb = (double)hw.rows * H * wbytes_per_elem(md->fmt);
    ProfScope ps(md, st, K_GEMV_HEAD, wb + (double)rows * H * 4 + (double)rows * hw.rows * 4, 2.0 * rows * hw.rows * H);
    HIP_TRY(launch_skinny(h, st));
  }
  return DPK_OK;
}

// Rows whose parameters are already in md->rows_dev.  M <= 16, bf16 / q4
// weights.  Writes logits/argmax for rows [head_r0, head_r0 + head_n).
dpk_status forward_skinny(dpk_model* md, int M, int max_ctx, const int32_t* ids_dev, int head_r0, int head_n,
                          float* logits, int32_t* argmax, hipStream_t st, double kv_positions, bool one_seq) {
  const dpk_config& c = md->cfg;
  const int H = c.hidden;
  {
    ProfScope ps(md, st, K_EMBED, (double)M * H * 6, 0);
    HIP_TRY(launch_embed(M, H, wfmt(md), md->embed.w, embed_scales(md), md->embed.bi,
                         md->rows_dev, ids_dev, c.vocab, md->h, md->rs, c.rms_eps, md->err_flag, st));
  }
  dpk_status s;
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& L = md->layers[l];
    LinearW qkv[3] = {L.q, L.k, L.v};
    if ((s = skinny(md, K_GEMV_QKV, M, md->h, H, md->rs, L.in_norm, qkv, 3, EPI_QKV, nullptr, 0, st, l))) return s;
    if ((s = attn_decode(md, M, max_ctx, md->qbuf, md->attn_o, l, st, kv_positions, nullptr, one_seq))) return s;
    if ((s = skinny(md, K_GEMV_O, M, md->attn_o, c.n_heads * c.head_dim, nullptr, nullptr, &L.o, 1, EPI_RESID, md->h,
                    H, st)))
      return s;
    LinearW gu[2] = {L.gate, L.up};
    if ((s = skinny(md, K_GEMV_GATEUP, M, md->h, H, md->rs, L.post_norm, gu, 2, EPI_SWIGLU, md->act, c.intermediate,
                    st)))
      return s;
    if ((s = skinny(md, K_GEMV_DOWN, M, md->act, c.intermediate, nullptr, nullptr, &L.down, 1, EPI_RESID, md->h, H,
                    st)))
      return s;
  }
  if (head_n > 0) return head(md, head_n, md->h + (size_t)head_r0 * H, md->rs + head_r0, md->final_norm, logits, argmax, st);
  return DPK_OK;
}

// Prefill block of M > 16 rows of one sequence at positions start..start+M-1
// (bf16 / q4 models): fp16 MFMA GEMMs over the prep copy of the weights,
// flash attention over the cache, then the head on the last row.
dpk_status forward_gemm(dpk_model* md, int M, int start, int seq, bool want_head, float* logits, int32_t* argmax,
                        hipStream_t st) {
  const dpk_config& c = md->cfg;
  const int H = c.hidden, I = c.intermediate, d = c.head_dim, Qd = c.n_heads * d;
  auto gemm_prof = [&](int cls, const GemmArgs& g) -> dpk_status {
    const double n = (g.epi == GEMM_SWIGLU_F16) ? 2.0 * g.N : g.N;
    const double outb = (g.epi == GEMM_SWIGLU_F16) ? (double)g.M * g.N * 2 : (double)g.M * g.N * 4;
    const double kb = g.Kb ? g.Kb : g.K;  // algorithmic K (the hi/lo split doubles the MFMA work)
    ProfScope ps(md, st, cls, ((double)g.M * g.K + n * kb) * 2 + outb, 2.0 * g.M * n * kb);
    GemmArgs gs = g;
    gs.splits = md->gemm_ws ? gemm_choose_splits(g.M, g.N, g.K, g.epi, md->n_cu) : 1;
    gs.ws = md->gemm_ws;
    gs.counters = md->gemm_counters;
    HIP_TRY(launch_gemm(gs, st));
    return DPK_OK;
  };
  dpk_status s2;
  {
    ProfScope ps(md, st, K_EMBED, (double)M * H * 6, 0);
    HIP_TRY(launch_embed(M, H, wfmt(md), md->embed.w, embed_scales(md), md->embed.bi,
                         md->rows_dev, nullptr, c.vocab, md->h, nullptr, c.rms_eps, md->err_flag, st));
  }
  const double norm_bytes = (double)M * H * 6;
  // the QKV epilogue takes QK-norm / RoPE / the cache write when the
  // projection runs on full 256 x 256 tiles (a narrow-tile grid splits a head
  // over two waves)
  const bool qkv_fused = d == 128 && !gemm_prefers_narrow(M, md->Nqkv, md->n_cu) && !md->kvd.i8;
  // int8 weights, one scale per row: the fp16 copies hold the codes and the
  // GEMMs scale their product columns (rs: the segments' bf16 row scales)
  const bool row_sc = md->fmt == DPK_FMT_I8;
  auto set_rs = [&](GemmArgs& g, const LinearW* a, const LinearW* b, const LinearW* c3) {
    g.rs_end[0] = g.rs_end[1] = 1 << 30;
    if (!row_sc) return;
    g.rs[0] = a->sc;
    g.rs[1] = b ? b->sc : nullptr;
    g.rs[2] = c3 ? c3->sc : nullptr;
    if (c3) {
      g.rs_end[0] = a->rows;
      g.rs_end[1] = a->rows + b->rows;
    }
  };
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& L = md->layers[l];
    {
      ProfScope ps(md, st, K_RMSNORM, norm_bytes, 0);
      // fp16 hi + lo: the QKV projection gets near-fp32 activations
      HIP_TRY(launch_rmsnorm_rows(M, H, md->h, H, L.in_norm, 0, c.rms_eps, md->y16, 2, 2 * H, st));
    }
    GemmArgs g{};
    g.M = M; g.N = md->Nqkv; g.K = 2 * H; g.Kb = H;
    g.A = md->y16; g.lda = 2 * H; g.B = L.qkv16; g.ldb = H;
    set_rs(g, &L.q, &L.k, &L.v);
    if (qkv_fused) {
      // QK-norm, RoPE, the q hi / lo split and the KV-cache write in the epilogue
      g.epi = GEMM_QKV_F16;
      g.n_heads = c.n_heads; g.n_kv = c.n_kv_heads; g.start = start; g.seq = seq; g.layer = l;
      g.qn = c.qk_norm ? (const uint16_t*)L.q_norm : nullptr;
      g.kn = c.qk_norm ? (const uint16_t*)L.k_norm : nullptr;
      g.eps = c.rms_eps; g.rope_cos = md->rope_cos; g.rope_sin = md->rope_sin;
      g.q16 = md->q16; g.kv = md->kvd;
      if ((s2 = gemm_prof(K_GEMM_QKV, g))) return s2;
    } else {
      g.epi = GEMM_STORE_F32; g.C = md->qkv; g.ldc = md->Nqkv;
      if ((s2 = gemm_prof(K_GEMM_QKV, g))) return s2;
      if (L.kvlo16) {  // + the K and V rows' rounding residuals (block formats over an int8 cache)
        GemmArgs g2{};
        g2.M = M; g2.N = 2 * c.n_kv_heads * d; g2.K = 2 * H; g2.Kb = H;
        g2.A = md->y16; g2.lda = 2 * H; g2.B = L.kvlo16; g2.ldb = H;
        g2.epi = GEMM_ADD_F32; g2.C = md->qkv + Qd; g2.ldc = md->Nqkv;
        if ((s2 = gemm_prof(K_GEMM_QKV, g2))) return s2;
      }
      ProfScope ps(md, st, K_QK_ROPE_KV, (double)M * md->Nqkv * 6, 0);
      HIP_TRY(launch_qk_rope_kv(M, md->qkv, c.n_heads, c.n_kv_heads, d, c.qk_norm, L.q_norm, L.k_norm, 0, c.rms_eps,
                                md->rope_cos, md->rope_sin, md->rows_dev, md->q16, 2, md->kvd, l, st));
    }
    AttnPrefillArgs at{};
    at.M = M; at.start = start; at.seq = seq;
    at.n_heads = c.n_heads; at.n_kv = c.n_kv_heads; at.d = d;
    at.q = md->q16; at.kv = md->kvd; at.layer = l; at.out = md->o16;
    at.scale = 1.0f / sqrtf((float)d);
    {
      const double keys = (double)M * start + (double)M * (M + 1) / 2;  // causal (query, key) pairs
      const double kvb = (double)(start + M) * 2 * c.n_kv_heads * d * 2;
      ProfScope ps(md, st, K_ATTN_PREFILL, kvb + 2.0 * M * Qd * 2, 4.0 * c.n_heads * d * keys);
      HIP_TRY(launch_attn_prefill(at, st));
    }
    g = GemmArgs{};
    g.M = M; g.N = H; g.K = 2 * Qd; g.Kb = Qd;
    g.A = md->o16; g.lda = 2 * Qd; g.B = L.o16; g.ldb = Qd;
    set_rs(g, &L.o, nullptr, nullptr);
    g.epi = GEMM_ADD_F32; g.C = md->h; g.ldc = H;
    if ((s2 = gemm_prof(K_GEMM_O, g))) return s2;
    {
      ProfScope ps(md, st, K_RMSNORM, norm_bytes, 0);
      HIP_TRY(launch_rmsnorm_rows(M, H, md->h, H, L.post_norm, 0, c.rms_eps, md->y16, 1, H, st));
    }
    g = GemmArgs{};
    g.M = M; g.N = I; g.K = H;
    g.A = md->y16; g.lda = H; g.B = L.gate16; g.B2 = L.up16; g.ldb = H;
    set_rs(g, &L.gate, &L.up, nullptr);
    g.epi = GEMM_SWIGLU_F16; g.C16 = md->act16; g.ldc16 = I;
    if ((s2 = gemm_prof(K_GEMM_GATEUP, g))) return s2;
    g = GemmArgs{};
    g.M = M; g.N = H; g.K = I;
    g.A = md->act16; g.lda = I; g.B = L.down16; g.ldb = I;
    set_rs(g, &L.down, nullptr, nullptr);
    g.epi = GEMM_ADD_F32; g.C = md->h; g.ldc = H;
    if ((s2 = gemm_prof(K_GEMM_DOWN, g))) return s2;
  }
  if (!want_head) return DPK_OK;
  // final RMSNorm of the last row (fp32), then the weight-streaming head
  HIP_TRY(launch_rmsnorm_rows(1, H, md->h + (size_t)(M - 1) * H, H, md->final_norm, 0, c.rms_eps, md->y32, 0, H, st));
  return head(md, 1, md->y32, nullptr, nullptr, logits, argmax, st);
}

// fp32 weights (any M <= max_rows): plain kernels.
dpk_status forward_f32(dpk_model* md, int M, int max_ctx, const int32_t* ids_dev, int head_r0, int head_n,
                       float* logits, int32_t* argmax, hipStream_t st, double kv_positions) {
  const dpk_config& c = md->cfg;
  const int H = c.hidden, d = c.head_dim, Qd = c.n_heads * d, KVd = c.n_kv_heads * d;
  const int Nqkv = Qd + 2 * KVd;
  HIP_TRY(launch_embed(M, H, W_F32, md->embed.w, nullptr, nullptr, md->rows_dev, ids_dev, c.vocab, md->h, nullptr,
                       c.rms_eps, md->err_flag, st));
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& L = md->layers[l];
    HIP_TRY(launch_rmsnorm_rows(M, H, md->h, H, L.in_norm, 1, c.rms_eps, md->y32, 0, H, st));
    HIP_TRY(launch_gemv_f32(M, Qd, H, (const float*)L.q.w, nullptr, md->y32, H, md->qkv, Nqkv, 0, st));
    HIP_TRY(launch_gemv_f32(M, KVd, H, (const float*)L.k.w, nullptr, md->y32, H, md->qkv + Qd, Nqkv, 0, st));
    HIP_TRY(launch_gemv_f32(M, KVd, H, (const float*)L.v.w, nullptr, md->y32, H, md->qkv + Qd + KVd, Nqkv, 0, st));
    HIP_TRY(launch_qk_rope_kv(M, md->qkv, c.n_heads, c.n_kv_heads, d, c.qk_norm, L.q_norm, L.k_norm, 1, c.rms_eps,
                              md->rope_cos, md->rope_sin, md->rows_dev, md->qbuf, 0, md->kvd, l, st));
    dpk_status s = attn_decode(md, M, max_ctx, md->qbuf, md->attn_o, l, st, kv_positions);
    if (s) return s;
    HIP_TRY(launch_gemv_f32(M, H, Qd, (const float*)L.o.w, nullptr, md->attn_o, Qd, md->h, H, 1, st));
    HIP_TRY(launch_rmsnorm_rows(M, H, md->h, H, L.post_norm, 1, c.rms_eps, md->y32, 0, H, st));
    HIP_TRY(launch_gemv_f32(M, c.intermediate, H, (const float*)L.gate.w, (const float*)L.up.w, md->y32, H, md->act,
                            c.intermediate, 2, st));
    HIP_TRY(launch_gemv_f32(M, H, c.intermediate, (const float*)L.down.w, nullptr, md->act, c.intermediate, md->h, H,
                            1, st));
  }
  if (head_n > 0) {
    HIP_TRY(launch_rmsnorm_rows(head_n, H, md->h + (size_t)head_r0 * H, H, md->final_norm, 1, c.rms_eps, md->y32, 0,
                                H, st));
    float* dst = logits ? logits : md->sink;
    HIP_TRY(launch_gemv_f32(head_n, c.vocab, H, (const float*)md->head.w, nullptr, md->y32, H, dst, c.vocab, 0, st));
    if (argmax) HIP_TRY(launch_argmax_rows(head_n, c.vocab, dst, c.vocab, argmax, st));
  }
  return DPK_OK;
}

// Rows already uploaded; pick the path by format and row count.
// kv_positions: cached positions the attention must read (per distinct
// sequence), for the profiler's byte count
// one_seq: the rows are consecutive positions of one sequence, else distinct
// sequences with one new position each.
dpk_status forward_rows(dpk_model* md, int M, int max_ctx, const int32_t* ids_dev, int head_r0, int head_n,
                        float* logits, int32_t* argmax, hipStream_t st, double kv_positions, bool one_seq) {
  if (md->fmt == DPK_FMT_F32)
    return forward_f32(md, M, max_ctx, ids_dev, head_r0, head_n, logits, argmax, st, kv_positions);
  if (batch_fits(md, M))
    return forward_batch(md, M, max_ctx, ids_dev, head_r0, head_n, logits, argmax, st, kv_positions, one_seq);
  return forward_skinny(md, M, max_ctx, ids_dev, head_r0, head_n, logits, argmax, st, kv_positions, one_seq);
}

int max_rows_for_path(const dpk_model* md) {
  return md->fmt == DPK_FMT_F32 ? md->cfg.max_rows : SKINNY_MAX;
}

}  // namespace

// ============================================================================ C ABI

extern "C" {

const char* dpk_last_error(void) { return g_err.c_str(); }

dpk_status dpk_create(const dpk_config* cfg, dpk_model** out) {
  if (!cfg || !out) return fail(DPK_EINVAL, "null argument");
  const dpk_config& c = *cfg;
  if (c.n_layers < 1 || c.hidden < 1 || c.n_heads < 1 || c.n_kv_heads < 1 || c.intermediate < 1 || c.vocab < 1)
    return fail(DPK_EINVAL, "sizes must be positive");
  if (c.head_dim != 64 && c.head_dim != 128) return fail(DPK_EINVAL, "head_dim must be 64 or 128");
  if (c.n_heads % c.n_kv_heads) return fail(DPK_EINVAL, "n_heads must be a multiple of n_kv_heads");
  if (c.n_heads / c.n_kv_heads > 8) return fail(DPK_EINVAL, "at most 8 query heads per KV head");
  if (c.hidden % 256 || c.intermediate % 256 || (c.n_heads * c.head_dim) % 256)
    return fail(DPK_EINVAL, "hidden, intermediate and n_heads*head_dim must be multiples of 256");
  if (c.weight_format < 0 || c.weight_format > 5) return fail(DPK_EINVAL, "unknown weight_format");
  if (c.weight_format != DPK_FMT_F32 && c.head_dim != 128) return fail(DPK_EINVAL, "non-f32 formats need head_dim 128");
  if (c.weight_format != DPK_FMT_F32 && !c.qk_norm) return fail(DPK_EINVAL, "non-f32 formats need qk_norm");
  if (c.weight_format != DPK_FMT_F32 && c.vocab % 64) return fail(DPK_EINVAL, "non-f32 formats need vocab % 64 == 0");
  if ((c.flags & DPK_FLAG_KV_I8) && c.weight_format == DPK_FMT_F32)
    return fail(DPK_EINVAL, "the int8 KV cache needs a non-f32 weight format");
  if (c.max_batch < 1 || c.max_seq < 1 || c.max_rows < SKINNY_MAX)
    return fail(DPK_EINVAL, "max_batch, max_seq >= 1 and max_rows >= 16 required");
  if (!(c.rms_eps >= 0.0f) || !(c.rope_theta > 0.0)) return fail(DPK_EINVAL, "bad eps / theta");
  dpk_model* md = new (std::nothrow) dpk_model();
  if (!md) return fail(DPK_ENOMEM, "out of host memory");
  md->cfg = c;
  md->fmt = c.weight_format;
  md->Nqkv = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  md->layers.resize(c.n_layers);
  md->seq_len.assign(c.max_batch, 0);
  *out = md;
  g_err.clear();
  return DPK_OK;
}

dpk_status dpk_workspace_size(const dpk_model* md, size_t* kvb, size_t* scb, size_t* prb) {
  if (!md || !kvb || !scb || !prb) return fail(DPK_EINVAL, "null argument");
  *kvb = kv_bytes(md->cfg);
  *scb = scratch_layout(md->cfg).total;
  *prb = prep_bytes(md->cfg);
  return DPK_OK;
}

dpk_status dpk_bind_workspace(dpk_model* md, void* kv, void* scratch, void* prep, void* stream) {
  if (!md || !kv || !scratch) return fail(DPK_EINVAL, "null argument");
  if (md->failed) return fail(DPK_ESTATE, "model failed");
  if (prep_bytes(md->cfg) && !prep) return fail(DPK_EINVAL, "prep buffer required for this format");
  if (((uintptr_t)kv | (uintptr_t)scratch | (uintptr_t)prep) % ALIGN) return fail(DPK_EINVAL, "buffers must be 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const dpk_config& c = md->cfg;
  const ScratchLayout L = scratch_layout(c);
  char* s = (char*)scratch;
  md->kv = kv;
  md->scratch = scratch;
  md->prep = prep;
  md->kvd.base = kv;
  md->kvd.is_f32 = md->fmt == DPK_FMT_F32;
  md->kvd.n_layers = c.n_layers;
  md->kvd.n_kv = c.n_kv_heads;
  md->kvd.max_seq = kv_seq(c);
  md->kvd.d = c.head_dim;
  md->kvd.i8 = (c.flags & DPK_FLAG_KV_I8) ? 1 : 0;
  md->kvd.scales = md->kvd.i8 ? (float*)((char*)kv + up(kv_code_bytes(c))) : nullptr;
  md->rope_cos = (float*)(s + L.rope_cos);
  md->rope_sin = (float*)(s + L.rope_sin);
  md->rows_dev = (RowParam*)(s + L.rows);
  md->h = (float*)(s + L.h);
  md->rs = (float*)(s + L.rs);
  md->qkv = (float*)(s + L.qkv);
  md->y32 = (float*)(s + L.y32);
  md->qbuf = (float*)(s + L.qbuf);
  md->attn_o = (float*)(s + L.attn_o);
  md->act = (float*)(s + L.act);
  md->part = (float*)(s + L.part);
  md->sink = (float*)(s + L.sink);
  md->sq = (float*)(s + L.sq);
  md->cand_val = (float*)(s + L.cand_val);
  md->cand_idx = (int*)(s + L.cand_idx);
  md->attn_part = (float*)(s + L.attn_part);
  md->y16 = (_Float16*)(s + L.y16);
  md->q16 = (_Float16*)(s + L.q16);
  md->o16 = (_Float16*)(s + L.o16);
  md->act16 = (_Float16*)(s + L.act16);
  md->counters = (unsigned*)(s + L.counters);
  md->attn_counters = (unsigned*)(s + L.attn_counters);
  md->err_flag = (int*)(s + L.err);
  md->argmax_sink = (int*)(s + L.argmax_sink);
  md->spec_ids = (int*)(s + L.spec_ids);
  md->gemm_ws = L.gemm_counters > L.gemm_ws ? (float*)(s + L.gemm_ws) : nullptr;
  md->gemm_counters = L.mega_layers > L.gemm_counters ? (unsigned*)(s + L.gemm_counters) : nullptr;
  md->mega_layers = L.mega_bar > L.mega_layers ? (MegaLayer*)(s + L.mega_layers) : nullptr;
  md->mega_bar = (unsigned*)(s + L.mega_bar);
  md->mega_trace = (unsigned long long*)(s + L.mega_trace);
  md->oacc = L.total > L.oacc ? (long long*)(s + L.oacc) : nullptr;
  md->xb_w = (int)L.xb_w;
  for (int i = 0; i < 4; ++i)
    md->xb[i / 2][i % 2] = L.total > L.xb ? (uint16_t*)(s + L.xb) + (size_t)i * SKINNY_MAX * L.xb_w : nullptr;
  md->mega_table = false;
  md->rows_f32 = L.rows_f32;
  md->attn_chunks_cap = L.attn_chunks_cap;
  md->part_floats = L.part_floats;
  for (int i = 0; i < dpk_model::NSTAGE; ++i) {
    if (!md->stage[i]) HIP_TRY(hipHostMalloc((void**)&md->stage[i], sizeof(RowParam) * c.max_rows, hipHostMallocDefault));
    if (!md->stage_ev[i]) HIP_TRY(hipEventCreateWithFlags(&md->stage_ev[i], hipEventDisableTiming));
  }
  if (!md->acc_host) HIP_TRY(hipHostMalloc((void**)&md->acc_host, sizeof(int32_t) * 32, hipHostMallocDefault));
  {
    int dev = 0, ncu = 0;
    HIP_TRY(hipGetDevice(&dev));
    HIP_TRY(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
    if (ncu > 0) md->n_cu = ncu;
    int lmax = 0;
    HIP_TRY(hipDeviceGetAttribute(&lmax, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
    if (lmax > 0) md->lds_max = lmax;
  }
  HIP_TRY(hipMemsetAsync(md->counters, 0, (1 + nblocks_max(c)) * 4, st));
  HIP_TRY(hipMemsetAsync(md->attn_counters, 0, attn_counter_bytes(md), st));
  HIP_TRY(hipMemsetAsync(md->err_flag, 0, 4, st));
  if (md->gemm_counters) HIP_TRY(hipMemsetAsync(md->gemm_counters, 0, GEMM_WS_TILES * 4, st));
  HIP_TRY(hipMemsetAsync(md->mega_bar, 0, MEGA_BAR_WORDS * 4, st));
  if (md->oacc) HIP_TRY(hipMemsetAsync(md->oacc, 0, (size_t)SKINNY_MAX * c.hidden * 8, st));
  HIP_TRY(launch_rope_table(md->rope_cos, md->rope_sin, c.max_seq, c.head_dim, c.rope_theta, st));
  md->bound = true;
  return DPK_OK;
}

dpk_status dpk_load_weights(dpk_model* md, const dpk_tensor* t, int32_t n, void* stream) {
  if (!md || (!t && n)) return fail(DPK_EINVAL, "null argument");
  if (md->failed) return fail(DPK_ESTATE, "model failed");
  if (!md->bound) return fail(DPK_ESTATE, "bind the workspace before loading weights");
  md->mega_table = false;
  const dpk_config& c = md->cfg;
  const int fmt = md->fmt;
  const int gdt = fmt == DPK_FMT_F32 ? DPK_DT_F32 : DPK_DT_BF16;
  struct Want {
    int dtype;
    int64_t rows, cols;
    const void** slot;
    bool seen;
  };
  std::map<std::string, Want> want;
  const int H = c.hidden, I = c.intermediate, d = c.head_dim, Qd = c.n_heads * d, KVd = c.n_kv_heads * d;
  std::vector<LinearW*> lin_slots;
  std::vector<std::string> lin_names;
  auto add_linear = [&](const std::string& name, LinearW* lw, int rows, int cols) {
    lw->rows = rows;
    lw->cols = cols;
    if (fmt == DPK_FMT_I8) {
      want[name + ".q"] = {DPK_DT_I8, rows, cols, &lw->w, false};
      want[name + ".scales"] = {DPK_DT_BF16, rows, 1, (const void**)&lw->sc, false};
    } else if (fmt == DPK_FMT_Q8) {
      want[name + ".q"] = {DPK_DT_I8, rows, cols, &lw->w, false};
      want[name + ".scales"] = {DPK_DT_F32, rows, cols / 32, (const void**)&lw->sf, false};
    } else if (fmt == DPK_FMT_Q40) {
      want[name + ".q"] = {DPK_DT_U8, rows, cols / 2, &lw->w, false};
      want[name + ".scales"] = {DPK_DT_F16, rows, cols / 32, (const void**)&lw->sf, false};
    } else if (fmt == DPK_FMT_Q4G64) {
      want[name + ".codes"] = {DPK_DT_U32, rows, cols / 8, &lw->w, false};
      want[name + ".scales"] = {DPK_DT_BF16, rows, cols / 64, (const void**)&lw->sc, false};
      want[name + ".biases"] = {DPK_DT_BF16, rows, cols / 64, (const void**)&lw->bi, false};
    } else {
      want[name] = {fmt == DPK_FMT_F32 ? DPK_DT_F32 : DPK_DT_BF16, rows, cols, &lw->w, false};
    }
  };
  auto add_gain = [&](const std::string& name, const void** slot, int len) { want[name] = {gdt, 1, len, slot, false}; };
  add_linear("embed_tokens", &md->embed, c.vocab, H);
  if (!c.tied_embedding) add_linear("lm_head", &md->head, c.vocab, H);
  add_gain("norm", &md->final_norm, H);
  for (int l = 0; l < c.n_layers; ++l) {
    LayerW& L = md->layers[l];
    const std::string p = "layers." + std::to_string(l) + ".";
    add_linear(p + "self_attn.q_proj", &L.q, Qd, H);
    add_linear(p + "self_attn.k_proj", &L.k, KVd, H);
    add_linear(p + "self_attn.v_proj", &L.v, KVd, H);
    add_linear(p + "self_attn.o_proj", &L.o, H, Qd);
    add_linear(p + "mlp.gate_proj", &L.gate, I, H);
    add_linear(p + "mlp.up_proj", &L.up, I, H);
    add_linear(p + "mlp.down_proj", &L.down, H, I);
    add_gain(p + "input_layernorm", &L.in_norm, H);
    add_gain(p + "post_attention_layernorm", &L.post_norm, H);
    if (c.qk_norm) {
      add_gain(p + "self_attn.q_norm", &L.q_norm, d);
      add_gain(p + "self_attn.k_norm", &L.k_norm, d);
    }
  }
  for (int i = 0; i < n; ++i) {
    if (!t[i].name) return fail(DPK_EINVAL, "tensor %d has no name", i);
    auto it = want.find(t[i].name);
    if (it == want.end()) return fail(DPK_EINVAL, "unexpected tensor '%s'", t[i].name);
    Want& w = it->second;
    if (w.seen) return fail(DPK_EINVAL, "tensor '%s' given twice", t[i].name);
    if (!t[i].data) return fail(DPK_EINVAL, "tensor '%s' has a null data pointer", t[i].name);
    if (t[i].dtype != w.dtype) return fail(DPK_EINVAL, "tensor '%s': dtype %d, expected %d", t[i].name, t[i].dtype, w.dtype);
    if (t[i].rows != w.rows || t[i].cols != w.cols)
      return fail(DPK_EINVAL, "tensor '%s': shape [%lld, %lld], expected [%lld, %lld]", t[i].name,
                  (long long)t[i].rows, (long long)t[i].cols, (long long)w.rows, (long long)w.cols);
    if ((uintptr_t)t[i].data % 16) return fail(DPK_EINVAL, "tensor '%s' must be 16-byte aligned", t[i].name);
    w.seen = true;
  }
  for (auto& kv : want)
    if (!kv.second.seen) return fail(DPK_EINVAL, "missing tensor '%s'", kv.first.c_str());
  for (int i = 0; i < n; ++i) *want[t[i].name].slot = t[i].data;
  if (c.tied_embedding) md->head = md->embed;
  // prefill operand copies
  hipStream_t st = (hipStream_t)stream;
  if (fmt != DPK_FMT_F32) {
    char* p = (char*)md->prep;
    auto conv = [&](const LinearW& w, _Float16* dst, bool lo = false) -> hipError_t {
      if (fmt == DPK_FMT_BF16) return launch_bf16_to_f16((const uint16_t*)w.w, dst, (size_t)w.rows * w.cols, st);
      // int8 per row: the codes (exact in fp16); the GEMMs apply the row scales
      if (fmt == DPK_FMT_I8) return launch_i8_to_f16((const int8_t*)w.w, nullptr, w.rows, w.cols, dst, st);
      if (fmt == DPK_FMT_Q8) return launch_q8_to_f16((const int8_t*)w.w, w.sf, w.rows, w.cols, dst, st, lo);
      if (fmt == DPK_FMT_Q40)
        return launch_q40_to_f16((const uint8_t*)w.w, (const uint16_t*)w.sf, w.rows, w.cols, dst, st, lo);
      return launch_q4_to_f16((const uint32_t*)w.w, w.sc, w.bi, w.rows, w.cols, dst, st, lo);
    };
    for (int l = 0; l < c.n_layers; ++l) {
      LayerW& L = md->layers[l];
      L.qkv16 = (_Float16*)p;
      HIP_TRY(conv(L.q, L.qkv16));
      HIP_TRY(conv(L.k, L.qkv16 + (size_t)Qd * H));
      HIP_TRY(conv(L.v, L.qkv16 + (size_t)(Qd + KVd) * H));
      p += up((size_t)md->Nqkv * H * 2);
      L.o16 = (_Float16*)p;
      HIP_TRY(conv(L.o, L.o16));
      p += up((size_t)H * Qd * 2);
      L.gate16 = (_Float16*)p;
      HIP_TRY(conv(L.gate, L.gate16));
      p += up((size_t)I * H * 2);
      L.up16 = (_Float16*)p;
      HIP_TRY(conv(L.up, L.up16));
      p += up((size_t)I * H * 2);
      L.down16 = (_Float16*)p;
      HIP_TRY(conv(L.down, L.down16));
      p += up((size_t)H * I * 2);
      if (kv_lo_copy(c)) {
        L.kvlo16 = (_Float16*)p;
        HIP_TRY(conv(L.k, L.kvlo16, true));
        HIP_TRY(conv(L.v, L.kvlo16 + (size_t)KVd * H, true));
        p += up((size_t)2 * KVd * H * 2);
      }
    }
    // fragment-order decode copies
    auto tile = [&](LinearW& w) -> hipError_t {
      w.wt = p;
      if (fmt == DPK_FMT_Q40) {  // codes + block scales (fp16)
        p += up((size_t)w.rows * w.cols / 2);
        const hipError_t e = launch_tile_q40((const uint8_t*)w.w, (uint32_t*)w.wt, w.rows, w.cols, st);
        if (e != hipSuccess) return e;
        w.sbt = p;
        p += up((size_t)w.rows * (w.cols / 32) * 2);
        return launch_tile_q40s((const uint16_t*)w.sf, (uint16_t*)w.sbt, w.rows, w.cols, st);
      }
      if (fmt == DPK_FMT_I8 || fmt == DPK_FMT_Q8) {  // codes (+ q8 block scales); i8 row scales are read as given
        p += up((size_t)w.rows * w.cols);
        const hipError_t e = launch_tile_i8((const int8_t*)w.w, (int8_t*)w.wt, w.rows, w.cols, st);
        if (e != hipSuccess || fmt == DPK_FMT_I8) return e;
        w.sbt = p;
        p += up((size_t)w.rows * (w.cols / 32) * 4);
        return launch_tile_q8s(w.sf, (float*)w.sbt, w.rows, w.cols, st);
      }
      if (fmt == DPK_FMT_BF16) {
        p += up((size_t)w.rows * w.cols * 2);
        return launch_tile_bf16((const uint16_t*)w.w, (uint16_t*)w.wt, w.rows, w.cols, st);
      }
      p += up((size_t)w.rows * w.cols / 2);
      w.sbt = p;
      p += up((size_t)w.rows * (w.cols / 64) * 4);
      return launch_tile_q4((const uint32_t*)w.w, w.sc, w.bi, (uint32_t*)w.wt, (uint32_t*)w.sbt, w.rows, w.cols, st);
    };
    for (int l = 0; l < c.n_layers; ++l) {
      LayerW& L = md->layers[l];
      for (LinearW* w : {&L.q, &L.k, &L.v, &L.o, &L.gate, &L.up, &L.down}) HIP_TRY(tile(*w));
    }
    HIP_TRY(tile(md->head));
    if ((size_t)(p - (char*)md->prep) > prep_bytes(c)) return fail(DPK_EINVAL, "internal: prep layout overflow");
  }
  md->loaded = true;
  return DPK_OK;
}

dpk_status dpk_prefill_at(dpk_model* md, int32_t seq, int32_t start, const int32_t* ids, int32_t n, float* logits,
                          int32_t* argmax, void* stream) {
  dpk_status s = check_ready(md);
  if (s) return s;
  const dpk_config& c = md->cfg;
  if (!ids) return fail(DPK_EINVAL, "null ids");
  if (n < 1) return fail(DPK_EINVAL, "n must be >= 1");
  if (seq < 0 || seq >= c.max_batch) return fail(DPK_ERANGE, "seq %d outside [0, %d)", seq, c.max_batch);
  if (start < 0 || start > md->seq_len[seq])
    return fail(DPK_ERANGE, "start %d beyond the cursor %d of slot %d", start, md->seq_len[seq], seq);
  if ((int64_t)start + n > c.max_seq)
    return fail(DPK_ERANGE, "start %d + %d tokens exceeds max_seq %d", start, n, c.max_seq);
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= c.vocab) return fail(DPK_ERANGE, "id %d at %d outside [0, %d)", ids[i], i, c.vocab);
  hipStream_t st = (hipStream_t)stream;
  const bool gemm_path = md->fmt != DPK_FMT_F32 && !(c.flags & DPK_FLAG_PREFILL_STREAM) && n > SKINNY_MAX;
  const int chunk = gemm_path ? c.max_rows : max_rows_for_path(md);
  std::vector<RowParam> rows(chunk);
  for (int r0 = 0; r0 < n; r0 += chunk) {
    const int M = (n - r0 < chunk) ? n - r0 : chunk;
    const int p0 = start + r0;  // position of the chunk's first row
    for (int i = 0; i < M; ++i) rows[i] = RowParam{ids[r0 + i], p0 + i, seq, 0};
    if ((s = upload_rows(md, rows.data(), M, st))) return s;
    const bool last = r0 + M == n;
    if (gemm_path && M > SKINNY_MAX)
      s = forward_gemm(md, M, p0, seq, last, logits, argmax, st);
    else
      s = forward_rows(md, M, p0 + M, nullptr, M - 1, last ? 1 : 0, logits, argmax, st, p0 + M, true);
    if (s) return s;
  }
  md->seq_len[seq] = start + n;
  return DPK_OK;
}

dpk_status dpk_prefill(dpk_model* md, int32_t seq, const int32_t* ids, int32_t n, float* logits, int32_t* argmax,
                       void* stream) {
  return dpk_prefill_at(md, seq, 0, ids, n, logits, argmax, stream);
}

dpk_status dpk_decode_step(dpk_model* md, int32_t batch, const int32_t* seqs, const int32_t* ids,
                           const int32_t* ids_dev, const int32_t* pos, float* logits, int32_t* argmax, void* stream) {
  dpk_status s = check_ready(md);
  if (s) return s;
  const dpk_config& c = md->cfg;
  if (!seqs || !pos || (!ids && !ids_dev) || !argmax) return fail(DPK_EINVAL, "null argument");
  if (batch < 1 || batch > SKINNY_MAX) return fail(DPK_EINVAL, "batch must be in [1, 16]");
  RowParam rows[SKINNY_MAX];
  int max_ctx = 0;
  for (int b = 0; b < batch; ++b) {
    if (seqs[b] < 0 || seqs[b] >= c.max_batch) return fail(DPK_ERANGE, "seq %d outside [0, %d)", seqs[b], c.max_batch);
    for (int b2 = 0; b2 < b; ++b2)
      if (seqs[b2] == seqs[b]) return fail(DPK_EINVAL, "slot %d appears twice in one step", seqs[b]);
    if (pos[b] < 0 || pos[b] >= c.max_seq) return fail(DPK_ERANGE, "pos %d outside [0, %d)", pos[b], c.max_seq);
    if (pos[b] > md->seq_len[seqs[b]])
      return fail(DPK_ERANGE, "pos %d beyond the cursor %d of slot %d", pos[b], md->seq_len[seqs[b]], seqs[b]);
    if (!ids_dev && (ids[b] < 0 || ids[b] >= c.vocab)) return fail(DPK_ERANGE, "id %d outside [0, %d)", ids[b], c.vocab);
    rows[b] = RowParam{ids_dev ? 0 : ids[b], pos[b], seqs[b], 0};
    if (pos[b] + 1 > max_ctx) max_ctx = pos[b] + 1;
  }
  hipStream_t st = (hipStream_t)stream;
  double kvpos = 0;
  for (int b = 0; b < batch; ++b) kvpos += pos[b] + 1;
  // the persistent step takes the rows in its launch arguments; the other
  // paths read them from device memory
  const size_t mega_lds = mega_lds_for(md, batch, max_ctx);
  if (!mega_lds && (s = upload_rows(md, rows, batch, st))) return s;
  if (mega_lds)
    s = forward_mega(md, batch, max_ctx, mega_lds, rows, ids_dev, logits, argmax, st, kvpos);
  else if (decode_fits(md, batch))
    s = forward_decode(md, batch, max_ctx, ids_dev, logits, argmax, st, kvpos);
  else
    s = forward_rows(md, batch, max_ctx, ids_dev, 0, batch, logits, argmax, st, kvpos, false);
  if (s) return s;
  for (int b = 0; b < batch; ++b) md->seq_len[seqs[b]] = pos[b] + 1;
  return DPK_OK;
}

dpk_status dpk_verify(dpk_model* md, int32_t seq, const int32_t* ids, int32_t kp1, int32_t pos, float* logits,
                      int32_t* argmax, int32_t* accepted, void* stream) {
  dpk_status s = check_ready(md);
  if (s) return s;
  const dpk_config& c = md->cfg;
  if (!ids || !argmax || !accepted) return fail(DPK_EINVAL, "null argument");
  if (kp1 < 1 || kp1 > SKINNY_MAX) return fail(DPK_EINVAL, "k_plus_1 must be in [1, 16]");
  if (seq < 0 || seq >= c.max_batch) return fail(DPK_ERANGE, "seq %d outside [0, %d)", seq, c.max_batch);
  if (pos < 0 || pos > md->seq_len[seq]) return fail(DPK_ERANGE, "pos %d beyond the cursor %d", pos, md->seq_len[seq]);
  if (pos + kp1 > c.max_seq) return fail(DPK_ERANGE, "pos + k_plus_1 = %d exceeds max_seq %d", pos + kp1, c.max_seq);
  RowParam rows[SKINNY_MAX];
  for (int i = 0; i < kp1; ++i) {
    if (ids[i] < 0 || ids[i] >= c.vocab) return fail(DPK_ERANGE, "id %d outside [0, %d)", ids[i], c.vocab);
    rows[i] = RowParam{ids[i], pos + i, seq, 0};
  }
  hipStream_t st = (hipStream_t)stream;
  if ((s = upload_rows(md, rows, kp1, st))) return s;
  if ((s = forward_rows(md, kp1, pos + kp1, nullptr, 0, kp1, logits, argmax, st, pos + kp1, true))) return s;
  HIP_TRY(hipMemcpyAsync(md->acc_host, argmax, sizeof(int32_t) * kp1, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
  int m = 0;
  while (m < kp1 - 1 && ids[m + 1] == md->acc_host[m]) ++m;
  *accepted = m;
  md->seq_len[seq] = pos + m + 1;
  return DPK_OK;
}

dpk_status dpk_seq_length(const dpk_model* md, int32_t seq, int32_t* length) {
  if (!md || !length) return fail(DPK_EINVAL, "null argument");
  if (seq < 0 || seq >= md->cfg.max_batch) return fail(DPK_ERANGE, "seq outside range");
  *length = md->seq_len[seq];
  return DPK_OK;
}

// Zero every cross-workgroup counter of the library.  After a persistent
// step whose barrier wait gave up, its workgroups ran the phases out of step:
// arrivals of different layers may have met on one attention-merge counter,
// and an arrival that lands between the last arriver's increment and its
// reset is lost, which would leave the counter off by one for every later
// step.
dpk_status reset_counters(dpk_model* md, hipStream_t st) {
  const dpk_config& c = md->cfg;
  HIP_TRY(hipMemsetAsync(md->counters, 0, (1 + nblocks_max(c)) * 4, st));
  HIP_TRY(hipMemsetAsync(md->attn_counters, 0, attn_counter_bytes(md), st));
  if (md->gemm_counters) HIP_TRY(hipMemsetAsync(md->gemm_counters, 0, GEMM_WS_TILES * 4, st));
  HIP_TRY(hipMemsetAsync(md->mega_bar, 0, MEGA_BAR_WORDS * 4, st));
  if (md->oacc) HIP_TRY(hipMemsetAsync(md->oacc, 0, (size_t)SKINNY_MAX * c.hidden * 8, st));
  return DPK_OK;
}

dpk_status dpk_check_device_errors(dpk_model* md, void* stream) {
  if (!md) return fail(DPK_EINVAL, "null model");
  if (!md->bound) return fail(DPK_ESTATE, "workspace not bound");
  hipStream_t st = (hipStream_t)stream;
  int flag = 0;
  HIP_TRY(hipMemcpyAsync(&flag, md->err_flag, 4, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
  if (flag) {
    HIP_TRY(hipMemsetAsync(md->err_flag, 0, 4, st));
    if (flag & 2) {
      dpk_status s = reset_counters(md, st);
      if (s) return s;
    }
    HIP_TRY(hipStreamSynchronize(st));
    if (flag & 2)
      return fail(DPK_EHIP,
                  "a persistent decode step's grid barrier wait gave up: the logits, argmax and KV entries written "
                  "by steps since the last check are invalid (the counters have been reset; decode again from the "
                  "last position known good)");
    return fail(DPK_ERANGE, "a device-side token id was outside [0, vocab) (replaced by 0)");
  }
  return DPK_OK;
}

dpk_status dpk_test_set_barrier_abort(dpk_model* md, void* stream) {
  dpk_status s = check_ready(md);
  if (s) return s;
  const unsigned one = 1u;
  HIP_TRY(hipMemcpyAsync(md->mega_bar + MEGA_BAR_ABORT, &one, 4, hipMemcpyHostToDevice, (hipStream_t)stream));
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
  return DPK_OK;
}

dpk_status dpk_profile_begin(dpk_model* md, int32_t max_launches) {
  if (!md) return fail(DPK_EINVAL, "null model");
  if (max_launches < 1) return fail(DPK_EINVAL, "max_launches must be >= 1");
  if (md->prof) return fail(DPK_ESTATE, "profiling already active");
  while ((int)md->prof_ev.size() < 2 * max_launches) {
    hipEvent_t e;
    // timing-only events: no system-scope fence (cache writeback) at record time
    HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
    md->prof_ev.push_back(e);
  }
  md->prof_max = max_launches;
  md->prof_rec.clear();
  md->prof_dropped = 0;
  md->prof_step_kv = 0;
  if (md->mega_trace) HIP_TRY(hipMemset(md->mega_trace, 0, MEGA_TRACE_WORDS * 8));
  md->prof = true;
  return DPK_OK;
}

dpk_status dpk_profile_end(dpk_model* md, dpk_kernel_stat* stats, int32_t max_stats, int32_t* n_stats) {
  if (!md || !n_stats || (!stats && max_stats)) return fail(DPK_EINVAL, "null argument");
  if (!md->prof) return fail(DPK_ESTATE, "profiling not active");
  md->prof = false;
  double ms[K_NCLASS] = {}, by[K_NCLASS] = {}, fl[K_NCLASS] = {};
  long cnt[K_NCLASS] = {};
  if (!md->prof_rec.empty()) HIP_TRY(hipDeviceSynchronize());
  for (size_t i = 0; i < md->prof_rec.size(); ++i) {
    float t = 0.f;
    HIP_TRY(hipEventElapsedTime(&t, md->prof_ev[2 * i], md->prof_ev[2 * i + 1]));
    const int c = md->prof_rec[i].cls;
    ms[c] += t;
    by[c] += md->prof_rec[i].bytes;
    fl[c] += md->prof_rec[i].flops;
    ++cnt[c];
  }
  // phases of the persistent decode kernel: wall-clock ticks of workgroup 0
  // from one barrier release to the next (a phase and the barrier after it)
  unsigned long long tr[MEGA_TRACE_WORDS] = {};
  if (md->mega_trace) HIP_TRY(hipMemcpy(tr, md->mega_trace, sizeof tr, hipMemcpyDeviceToHost));
  if (tr[MP_STEPS]) {
    int dev = 0, khz = 0;
    HIP_TRY(hipGetDevice(&dev));
    HIP_TRY(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev));
    const dpk_config& c = md->cfg;
    const double steps = (double)tr[MP_STEPS], L = c.n_layers, H = c.hidden, I = c.intermediate;
    const double Qd = (double)c.n_heads * c.head_dim, wb = wbytes_per_elem(md->fmt);
    struct P { int phase, cls; double per_step, wbytes; };
    const P ps[] = {{MP_EMBED, K_STEP_EMBED, 1, 0},
                    {MP_QKV, K_STEP_QKV, L, md->Nqkv * H * wb},
                    // the attention phase reads every cached position's K and V (fp16)
                    {MP_ATTN, K_STEP_ATTN, L, md->prof_step_kv / steps * 2.0 * c.n_kv_heads * c.head_dim * 2.0},
                    {MP_O, K_STEP_O, L, H * Qd * wb},
                    {MP_GATEUP, K_STEP_GATEUP, L, 2 * I * H * wb},
                    {MP_DOWN, K_STEP_DOWN, L, H * I * wb},
                    {MP_HEAD, K_STEP_HEAD, 1, (double)c.vocab * H * wb}};
    for (const P& p : ps) {
      ms[p.cls] += khz > 0 ? (double)tr[p.phase] / khz : 0.0;
      cnt[p.cls] += (long)(steps * p.per_step);
      by[p.cls] += steps * p.per_step * p.wbytes;
    }
  }
  int n = 0;
  for (int c = 0; c < K_NCLASS; ++c) {
    if (!cnt[c]) continue;
    if (n < max_stats) stats[n] = dpk_kernel_stat{kclass_name[c], cnt[c], ms[c], by[c], fl[c]};
    ++n;
  }
  *n_stats = n;
  if (md->prof_dropped) return fail(DPK_ERANGE, "%ld launches were not recorded (raise max_launches)", md->prof_dropped);
  return DPK_OK;
}

// ---------------------------------------------------------------- speculative loop

dpk_status dpk_spec_generate(dpk_model* target, dpk_model* draft, int32_t seq, int32_t pos, int32_t token,
                             int32_t n_new, const dpk_spec_config* sc, int32_t* out_ids, dpk_spec_stats* stats,
                             void* stream) {
  dpk_status s = check_ready(target);
  if (s) return s;
  if ((s = check_ready(draft))) return s;
  if (target == draft) return fail(DPK_EINVAL, "the draft must be a separate model handle");
  if (!sc || !out_ids) return fail(DPK_EINVAL, "null argument");
  const dpk_config &tc = target->cfg, &dc = draft->cfg;
  if (tc.vocab != dc.vocab) return fail(DPK_EINVAL, "draft vocab %d differs from target vocab %d", dc.vocab, tc.vocab);
  if (sc->k_min < 1 || sc->k_min > sc->k_init || sc->k_init > sc->k_max || sc->k_max > SKINNY_MAX - 1)
    return fail(DPK_EINVAL, "need 1 <= k_min <= k_init <= k_max <= %d", SKINNY_MAX - 1);
  if (n_new < 1) return fail(DPK_EINVAL, "n_new must be >= 1");
  if (seq < 0 || seq >= tc.max_batch || seq >= dc.max_batch) return fail(DPK_ERANGE, "seq %d outside both models", seq);
  if (pos < 0 || pos > target->seq_len[seq] || pos > draft->seq_len[seq])
    return fail(DPK_ERANGE, "pos %d beyond a cursor (target %d, draft %d)", pos, target->seq_len[seq],
                draft->seq_len[seq]);
  if ((int64_t)pos + n_new + sc->k_max > tc.max_seq || (int64_t)pos + n_new + sc->k_max > dc.max_seq)
    return fail(DPK_ERANGE, "pos + n_new + k_max exceeds max_seq");
  if (token < 0 || token >= tc.vocab) return fail(DPK_ERANGE, "token %d outside [0, %d)", token, tc.vocab);
  hipStream_t st = (hipStream_t)stream;
  dpk_spec_stats stt{};
  int k = sc->k_init, emitted = 0, cur = pos, t_last = token;
  int pending = -1;  // a committed token the draft cache lacks (at cur - 1), or -1
  int* dd = draft->spec_ids;  // draft tokens d_1..d_K (device)
  while (emitted < n_new) {
    const int K = k;
    // the draft catches up on the last draft token of a fully accepted round
    if (pending >= 0) {
      const int p = cur - 1;
      if ((s = dpk_decode_step(draft, 1, &seq, &pending, nullptr, &p, nullptr, dd + 32, stream))) return s;
      ++stt.draft_steps;
      pending = -1;
    }
    // K greedy draft steps chained on the device: d_{i+1} = argmax(draft(d_i at cur + i))
    for (int i = 0; i < K; ++i) {
      const int p = cur + i;
      if ((s = dpk_decode_step(draft, 1, &seq, i == 0 ? &t_last : nullptr, i == 0 ? nullptr : dd + i - 1, &p,
                               nullptr, dd + i, stream)))
        return s;
    }
    stt.draft_steps += K;
    HIP_TRY_M(draft, hipMemcpyAsync(draft->acc_host, dd, sizeof(int32_t) * K, hipMemcpyDeviceToHost, st));
    HIP_TRY_M(draft, hipStreamSynchronize(st));
    int32_t ids[SKINNY_MAX];
    ids[0] = t_last;
    for (int i = 0; i < K; ++i) ids[1 + i] = draft->acc_host[i];
    int32_t m = 0;
    if ((s = dpk_verify(target, seq, ids, K + 1, cur, nullptr, target->spec_ids, &m, stream))) return s;
    ++stt.rounds;
    stt.drafted += K;
    stt.accepted += m;
    const int bonus = target->acc_host[m];
    // emit d_1..d_m and the bonus, up to n_new
    int e = 0;
    for (; e < m && emitted < n_new; ++e) out_ids[emitted++] = ids[1 + e];
    if (emitted < n_new) {
      out_ids[emitted++] = bonus;
      e = m + 1;
    }
    // positions cur..cur+e-1 now hold committed tokens (t_last, d_1..d_{e-1});
    // the next pending token is the last emitted one
    const int next = cur + e;
    target->seq_len[seq] = next;
    // the draft holds t_last, d_1..d_{K-1} at cur..cur+K-1
    const int draft_valid = cur + (e < K ? e : K);
    draft->seq_len[seq] = draft_valid;
    if (e == K + 1) pending = ids[K];  // d_K at cur + K is missing from the draft
    t_last = out_ids[emitted - 1];
    cur = next;
    // adaptive draft length: longer after a fully accepted round, shorter
    // after one that accepted fewer than half
    if (m == K && k < sc->k_max) ++k;
    else if (2 * m < K && k > sc->k_min) --k;
  }
  if (pending >= 0) {
    // leave the draft consistent with the target's committed prefix
    const int p = cur - 1;
    if ((s = dpk_decode_step(draft, 1, &seq, &pending, nullptr, &p, nullptr, dd + 32, stream))) return s;
    ++stt.draft_steps;
  }
  if (stats) *stats = stt;
  return DPK_OK;
}

// ---------------------------------------------------------------- sampling

namespace {
dpk_status check_sampler(const dpk_sampler* sp) {
  if (!sp) return fail(DPK_EINVAL, "null sampler");
  if (!(sp->temperature >= 0.0f) || !(sp->temperature < INFINITY))
    return fail(DPK_EINVAL, "temperature must be finite and >= 0");
  if (sp->top_k < 0) return fail(DPK_EINVAL, "top_k must be >= 0");
  if (!(sp->top_p > 0.0f && sp->top_p <= 1.0f)) return fail(DPK_EINVAL, "top_p must be in (0, 1]");
  return DPK_OK;
}
}  // namespace

dpk_status dpk_sample(const float* logits, int32_t rows, int32_t vocab, int64_t ld, const dpk_sampler* sp,
                      const float* u, int32_t* out, void* stream) {
  if (!logits || !u || !out) return fail(DPK_EINVAL, "null argument");
  if (rows < 1 || vocab < 1 || ld < vocab) return fail(DPK_EINVAL, "rows, vocab >= 1 and ld >= vocab required");
  dpk_status s = check_sampler(sp);
  if (s) return s;
  const hipError_t e = launch_sample(logits, ld, rows, vocab, sp->temperature, sp->top_k, sp->top_p, u, out,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return fail(DPK_EHIP, "sampling launch failed: %s", hipGetErrorString(e));
  return DPK_OK;
}

dpk_status dpk_spec_accept_workspace_size(int32_t k, size_t* bytes) {
  if (!bytes) return fail(DPK_EINVAL, "null argument");
  if (k < 1 || k > DPK_SPEC_MAX_K) return fail(DPK_EINVAL, "k must be in [1, %d]", DPK_SPEC_MAX_K);
  *bytes = spec_dist_bytes(k);
  return DPK_OK;
}

dpk_status dpk_spec_accept(const float* target_logits, const float* draft_logits, int64_t ld, int32_t vocab,
                           int32_t k, const int32_t* drafts, const dpk_sampler* sp, const float* r, const float* u,
                           int32_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!target_logits || !draft_logits || !drafts || !r || !u || !out || !workspace)
    return fail(DPK_EINVAL, "null argument");
  if (k < 1 || k > DPK_SPEC_MAX_K) return fail(DPK_EINVAL, "k must be in [1, %d]", DPK_SPEC_MAX_K);
  if (vocab < 1 || ld < vocab) return fail(DPK_EINVAL, "vocab >= 1 and ld >= vocab required");
  if (workspace_bytes < spec_dist_bytes(k) || (uintptr_t)workspace % 16)
    return fail(DPK_EINVAL, "workspace: %zu bytes (16-byte aligned) needed, %zu given", spec_dist_bytes(k),
                workspace_bytes);
  dpk_status s = check_sampler(sp);
  if (s) return s;
  const hipError_t e = launch_spec_accept(target_logits, draft_logits, ld, vocab, k, sp->temperature, sp->top_k,
                                          sp->top_p, drafts, r, u, workspace, out, (hipStream_t)stream);
  if (e != hipSuccess) return fail(DPK_EHIP, "speculative acceptance launch failed: %s", hipGetErrorString(e));
  return DPK_OK;
}

dpk_status dpk_spec_accept_noalloc(const float* target_logits, const float* draft_logits, int64_t ld, int32_t vocab,
                                   int32_t k, const int32_t* drafts, const dpk_sampler* sp, const float* r,
                                   const float* u, int32_t* out, void* stream) {
  if (!target_logits || !draft_logits || !drafts || !r || !u || !out) return fail(DPK_EINVAL, "null argument");
  if (k < 1 || k > spec_noalloc_max_k())
    return fail(DPK_EINVAL, "k = %d outside [1, %d], the most drafts the built-in workspace holds", k,
                spec_noalloc_max_k());
  if (vocab < 1 || ld < vocab) return fail(DPK_EINVAL, "vocab >= 1 and ld >= vocab required");
  dpk_status s = check_sampler(sp);
  if (s) return s;
  void* ws = nullptr;
  hipError_t e = spec_noalloc_scratch(&ws);
  if (e != hipSuccess) return fail(DPK_EHIP, "built-in workspace lookup failed: %s", hipGetErrorString(e));
  e = launch_spec_accept(target_logits, draft_logits, ld, vocab, k, sp->temperature, sp->top_k, sp->top_p, drafts, r,
                         u, ws, out, (hipStream_t)stream);
  if (e != hipSuccess) return fail(DPK_EHIP, "speculative acceptance launch failed: %s", hipGetErrorString(e));
  return DPK_OK;
}

void dpk_destroy(dpk_model* md) {
  if (!md) return;
  for (hipEvent_t e : md->prof_ev) (void)hipEventDestroy(e);
  for (int i = 0; i < dpk_model::NSTAGE; ++i) {
    if (md->stage_ev[i]) {
      (void)hipEventSynchronize(md->stage_ev[i]);
      (void)hipEventDestroy(md->stage_ev[i]);
    }
    if (md->stage[i]) (void)hipHostFree(md->stage[i]);
  }
  if (md->acc_host) (void)hipHostFree(md->acc_host);
  delete md;
}

}  // extern "C"
