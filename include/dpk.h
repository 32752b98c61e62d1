/*
 * dpk: forward pass of a dense pre-norm decoder (Llama / Qwen3 style) on one
 * AMD Instinct MI355X (gfx950): prompt prefill, single-token KV-cache decode,
 * batched decode and greedy speculative verify.
 *
 * The operations follow the pages this library was built from:
 *  - the block (RMSNorm -> QKV -> RoPE -> grouped-query causal attention ->
 *    SwiGLU MLP, residuals) and the Qwen3 per-head QK-norm before RoPE:
 *    "LLMs on the ANE" (ANEForge docs), sections "What's inside" and
 *    "Correctness";
 *  - prefill returns the next-token logits of a whole prompt, decode feeds one
 *    token against a resident KV cache: same page, "API" and "Prefill and
 *    decode";
 *  - the per-token decode order and the on-GPU greedy argmax: Butter
 *    architecture notes, single-token decode and GPU sampling diagrams;
 *  - MLX 4-bit affine weights (w = scale * code + bias, group 64): oxinfer
 *    0.0.5 docs, "MLX checkpoints";
 *  - greedy verify (accept while draft == argmax, one bonus token, rollback by
 *    moving the cache cursor): Butter notes, speculative decoding loop.
 *
 * Conventions
 *  - All device pointers are HIP device addresses; "host" arrays are ordinary
 *    host memory read before the call returns.
 *  - The caller allocates and owns every device buffer (weights, KV cache,
 *    scratch, prefill weight copy, outputs) and keeps them alive until
 *    dpk_destroy.  The library owns only the handle, pinned staging for
 *    per-call row parameters and a few events.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  All
 *    device work is enqueued on it; calls return after enqueue, except
 *    dpk_verify (which waits to return the accepted count).  Calls on one
 *    model must be issued on one stream, or serialized by the caller.
 *  - Every entry point validates its arguments before enqueuing anything; on
 *    a validation error nothing is enqueued and the model state is unchanged.
 *    A HIP failure returns DPK_EHIP and marks the model failed: later calls
 *    return DPK_ESTATE.  dpk_last_error() describes the last failure on the
 *    calling thread.
 */
#ifndef DPK_H
#define DPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DPK_OK = 0,
  DPK_EINVAL = -1, /* null pointer, bad name / shape / dtype, n < 1 */
  DPK_ERANGE = -2, /* id outside [0, vocab), pos > cursor, pos + n > max_seq, seq >= max_batch */
  DPK_ESTATE = -3, /* weights or workspace not bound, or the model failed earlier */
  DPK_ENOMEM = -4, /* host allocation failed */
  DPK_EHIP = -5    /* a HIP runtime call failed */
} dpk_status;

/* Storage format of the linear layers (q, k, v, o, gate, up, down, head). */
typedef enum {
  DPK_FMT_F32 = 0,  /* fp32 weights, fp32 KV cache */
  DPK_FMT_BF16 = 1, /* bf16 weights, fp16 KV cache */
  DPK_FMT_Q4G64 = 2, /* MLX 4-bit affine, group 64 along the input dim; fp16 KV cache */
  DPK_FMT_I8 = 3,    /* int8 with one bf16 scale per output row (w = scale * q); fp16 KV cache.
                        Decoded by the weight-streaming GEMV (one launch per kernel), prefilled
                        through the fp16 GEMMs ("LLMs on the ANE", section "Quantized weights":
                        int8 weights) */
  DPK_FMT_Q8 = 4,    /* int8 in blocks of 32 weights along the input dim, one fp32 scale per
                        block (w = scale[n][k / 32] * q[n][k]); fp16 KV cache.  Decoded by the
                        weight-streaming GEMV, prefilled through the fp16 GEMMs (oxinfer docs,
                        "Build and run": the q8 quantization of streamed weights) */
  DPK_FMT_Q40 = 5    /* GGUF-style Q4_0: blocks of 32 four-bit codes c along the input dim with
                        one fp16 scale d, w = d * (c - 8); fp16 KV cache.  Decoded by the
                        weight-streaming GEMV, prefilled through the fp16 GEMMs (oxinfer docs,
                        "Build and run": the q4 quantization) */
} dpk_format;

/* Element types of dpk_tensor entries. */
typedef enum { DPK_DT_F32 = 0, DPK_DT_BF16 = 1, DPK_DT_U32 = 2, DPK_DT_I8 = 3, DPK_DT_U8 = 4, DPK_DT_F16 = 5 } dpk_dtype;

typedef struct {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, intermediate, vocab;
  float rms_eps;          /* RMSNorm epsilon (all norms) */
  double rope_theta;      /* RoPE base; inv_freq_i = theta^(-2i/head_dim), half-split pairs */
  int32_t qk_norm;        /* 1: per-head RMSNorm of q and k before RoPE (Qwen3) */
  int32_t tied_embedding; /* 1: the lm_head is the embedding table */
  int32_t weight_format;  /* dpk_format */
  int32_t max_batch;      /* KV-cache sequence slots */
  int32_t max_seq;        /* positions per slot */
  int32_t max_rows;       /* rows per internal forward chunk (>= 16); longer prompts are chunked */
  int32_t flags;          /* DPK_FLAG_* */
} dpk_config;

/* Prefill through the weight-streaming (decode) kernels in chunks of 16 rows
 * instead of the MFMA GEMM path (bf16 / q4 formats). */
#define DPK_FLAG_PREFILL_STREAM 1
/* Decode steps as one kernel launch per GEMV / attention instead of one
 * persistent launch for the whole step.  bf16 and 4-bit models whose shapes
 * the persistent kernel supports use it by default for a step of up to a few
 * rows.  That launch is cooperative (one workgroup on every compute unit,
 * grid-wide barriers inside); its barrier waits are bounded, so if other work
 * on the device keeps its workgroups from running together the step ends with
 * a device error (dpk_check_device_errors) instead of hanging.  Callers that
 * share the GPU with other kernels may prefer this flag. */
#define DPK_FLAG_DECODE_MULTI 2
/* KV cache as int8: each position's K and V head vectors are int8 codes with one
 * fp32 scale, s = max|x| / 127, q = round(x / s) clipped to +-127, read back as s * q
 * (Butter notes, architecture: an affine-quantized KV cache; here its offset is
 * zero).  Needs a non-fp32 weight format (head_dim 128).  The kv buffer then holds
 * the codes in the fp16 cache's element layout at one byte each, followed (at a
 * 256-byte boundary) by the scales [max_batch][n_layers][K|V][n_kv][S] fp32.
 * Decode steps run one launch per kernel (the persistent step keeps the fp16
 * cache), and the prefill's QKV projection hands QK-norm / RoPE and the cache
 * write to a separate kernel. */
#define DPK_FLAG_KV_I8 4

/*
 * One weight tensor.  Names (transformers-style):
 *   embed_tokens, lm_head (absent when tied), norm,
 *   layers.{i}.input_layernorm, layers.{i}.post_attention_layernorm,
 *   layers.{i}.self_attn.{q,k,v,o}_proj, layers.{i}.self_attn.{q,k}_norm (qk_norm only),
 *   layers.{i}.mlp.{gate,up,down}_proj.
 * Linear weights are [out, in] row-major.  Norm gains are 1-D ([hidden] or
 * [head_dim], rows = 1) and have the dtype of the format (F32 for DPK_FMT_F32,
 * BF16 otherwise).  In DPK_FMT_Q4G64 each linear tensor (including
 * embed_tokens / lm_head) is three entries: "<name>.codes" U32 [out, in/8]
 * (element 8w+j in bits 4j..4j+3 of word w), "<name>.scales" and
 * "<name>.biases" BF16 [out, in/64].  In DPK_FMT_I8 each linear tensor
 * (including embed_tokens / lm_head) is two entries: "<name>.q" I8 [out, in]
 * and "<name>.scales" BF16 [out, 1].  In DPK_FMT_Q8 each linear tensor
 * (including embed_tokens / lm_head) is "<name>.q" I8 [out, in] and
 * "<name>.scales" F32 [out, in/32] (the scale of codes 32j .. 32j+31 of a row).
 * In DPK_FMT_Q40 each linear tensor (including embed_tokens / lm_head) is
 * "<name>.q" U8 [out, in/2] (per block of 32 codes, 16 bytes: byte j holds code
 * j in its low nibble and code j + 16 in its high nibble) and "<name>.scales"
 * F16 [out, in/32].
 */
typedef struct {
  const char* name;
  const void* data; /* device address */
  int32_t dtype;    /* dpk_dtype */
  int64_t rows, cols;
} dpk_tensor;

typedef struct dpk_model dpk_model;

/* Validate the configuration and create a handle.  Supported shapes:
 * head_dim 64 or 128, n_heads a multiple of n_kv_heads with at most 8 query
 * heads per KV head, hidden and intermediate multiples of 256; bf16 / q4 /
 * i8 / q8 / q4_0 models need head_dim 128, per-head QK-norm and vocab % 64 == 0.  Does not touch the GPU. */
dpk_status dpk_create(const dpk_config* cfg, dpk_model** out);

/* Bytes of the three caller-provided device buffers:
 *   kv:      max_batch x n_layers x {K, V} x n_kv_heads x S x head_dim elements with
 *            S = max_seq rounded up to a multiple of 64 (fp32 for DPK_FMT_F32, fp16
 *            otherwise, int8 codes with DPK_FLAG_KV_I8 followed by the fp32 scales);
 *            K rows per position, V stored transposed (positions contiguous per
 *            channel);
 *   scratch: activations, partial sums, counters, RoPE tables (256-byte aligned);
 *   prep:    fp16 copy of the linear layers used as prefill MFMA operands (int8
 *            per row: the codes themselves), the fragment-order copies the decode
 *            GEMVs stream, and for block-scaled formats over an int8 cache the
 *            fp16 rounding residuals of the K and V projections (0 for
 *            DPK_FMT_F32). */
dpk_status dpk_workspace_size(const dpk_model* m, size_t* kv_bytes, size_t* scratch_bytes,
                              size_t* prep_bytes);

/* Bind the buffers (device addresses, 256-byte aligned, sizes as above).
 * Enqueues the RoPE table and counter initialisation on `stream`. */
dpk_status dpk_bind_workspace(dpk_model* m, void* kv, void* scratch, void* prep, void* stream);

/* Register the weights.  Every expected tensor must appear exactly once with
 * the expected dtype and shape; unknown names are an error.  Enqueues the
 * conversion of the linear layers into the prep buffer on `stream`.  Requires
 * dpk_bind_workspace first. */
dpk_status dpk_load_weights(dpk_model* m, const dpk_tensor* tensors, int32_t n, void* stream);

/* Prefill: overwrite sequence slot `seq` with the n prompt ids (host array) at
 * positions 0..n-1, set its cursor to n, and write the next-token logits
 * (fp32 [vocab], device) and, if argmax_dev is not NULL, the greedy id (int32
 * [1], device; lowest index on ties).  logits_dev may be NULL. */
dpk_status dpk_prefill(dpk_model* m, int32_t seq, const int32_t* ids, int32_t n, float* logits_dev,
                       int32_t* argmax_dev, void* stream);

/* Prefill onto an existing cache (multi-turn, or a prompt fed in pieces):
 * write the n ids (host array) at positions start..start+n-1 of slot `seq`,
 * attending causally within the block and to the cached positions
 * 0..start-1, set the cursor to start + n and return the last token's logits
 * / greedy id as dpk_prefill does.  Requires start <= cursor (an earlier
 * start drops the positions after it, as a rollback) and start + n <=
 * max_seq (DPK_ERANGE otherwise, nothing enqueued).  dpk_prefill is this call
 * with start = 0.  The block is the same computation as a verify pass of n
 * rows (Butter notes, speculative decoding loop: a batch of positions put
 * through attention over the cache together); oxinfer 0.0.5 docs, "Build and
 * run", chunked prefill. */
dpk_status dpk_prefill_at(dpk_model* m, int32_t seq, int32_t start, const int32_t* ids, int32_t n,
                          float* logits_dev, int32_t* argmax_dev, void* stream);

/* Decode one token for each of `batch` rows (batch <= 16).  Row b feeds token
 * ids[b] at position pos[b] of slot seqs[b] (host arrays; slots distinct).
 * Requires pos[b] <= cursor and pos[b] < max_seq; writes K/V at pos[b],
 * attends to positions 0..pos[b] and sets the cursor to pos[b] + 1 (an earlier
 * pos rolls the slot back).  If ids_dev is not NULL the tokens are read from
 * that device int32 [batch] array instead of `ids` (for example the previous
 * step's argmax output); out-of-range device ids are replaced by 0 and
 * reported by dpk_check_device_errors.  Outputs: logits fp32 [batch, vocab]
 * (nullable) and argmax int32 [batch] (device). */
dpk_status dpk_decode_step(dpk_model* m, int32_t batch, const int32_t* seqs, const int32_t* ids,
                           const int32_t* ids_dev, const int32_t* pos, float* logits_dev,
                           int32_t* argmax_dev, void* stream);

/* Greedy speculative verify of k_plus_1 <= 16 tokens [t, d_1..d_K] (host) at
 * positions pos..pos+K of slot `seq` (pos <= cursor): one forward pass that is
 * causal within the block and sees cached positions 0..pos-1.  Writes logits
 * fp32 [K+1, vocab] (nullable) and argmax int32 [K+1] (device), waits for the
 * stream, and returns in *accepted the number m of leading drafts with
 * d_{i+1} == argmax[i]; the cursor becomes pos + m + 1 and argmax[m] is the
 * bonus token. */
dpk_status dpk_verify(dpk_model* m, int32_t seq, const int32_t* ids, int32_t k_plus_1, int32_t pos,
                      float* logits_dev, int32_t* argmax_dev, int32_t* accepted, void* stream);

/* Current cursor (cached positions) of a slot. */
dpk_status dpk_seq_length(const dpk_model* m, int32_t seq, int32_t* length);

/* Synchronize `stream` and report device-side errors seen since the last
 * check, then clear them:
 *  - DPK_EHIP if a persistent decode step's bounded grid-barrier wait gave
 *    up (the device was shared with other work, or a test forced it): the
 *    logits, argmax and KV entries written by the steps since the last check
 *    are invalid.  The library's cross-workgroup counters are reset, so the
 *    caller may decode again from the last position known good (an earlier
 *    pos rolls the slot back);
 *  - else DPK_ERANGE for device-side token ids outside [0, vocab) (each
 *    replaced by 0);
 *  - else DPK_OK. */
dpk_status dpk_check_device_errors(dpk_model* m, void* stream);

/* Failure-path test support: set the persistent decode step's abort word, as
 * a barrier wait that gives up does.  The next persistent step then passes
 * every grid barrier without waiting (its outputs are invalid, every
 * workgroup still finishes) and dpk_check_device_errors reports DPK_EHIP.
 * Synchronizes `stream`. */
dpk_status dpk_test_set_barrier_abort(dpk_model* m, void* stream);

/* Per-kernel-class timing.  Between dpk_profile_begin and dpk_profile_end
 * every launch of the library records a HIP event pair on its stream (at most
 * max_launches launches; later ones are counted as dropped).  dpk_profile_end
 * waits for the last event and returns, per kernel class, the number of
 * launches, their summed duration in ms, and the summed algorithmic bytes and
 * FLOPs of those launches (computed from the shapes: weights + activations
 * read and written, causal attention pairs).  `name` points to a static
 * string. */
typedef struct {
  const char* name;
  int64_t launches;
  double total_ms;
  double bytes;
  double flops;
} dpk_kernel_stat;
dpk_status dpk_profile_begin(dpk_model* m, int32_t max_launches);
dpk_status dpk_profile_end(dpk_model* m, dpk_kernel_stat* stats, int32_t max_stats, int32_t* n_stats);

/* ------------------------------------------------------------ speculative loop
 * Greedy speculative decoding with a draft model (LLMs on the ANE, section
 * "Speculative decoding": a small model of the same family drafts, the large
 * one verifies K drafts in one pass; Butter notes, speculative decoding loop:
 * draft K, verify, accept the leading matches plus one bonus token, roll the
 * caches back by moving their cursors; oxinfer 0.0.5 docs, "Speculative
 * decoding": the number of drafts adapts, 2 to 6 by default).
 *
 * Both models hold slot `seq` with the same committed tokens cached at
 * positions 0..pos-1 (pos <= both cursors; positions past pos are dropped)
 * and share the vocabulary; `token` is the last committed token, not yet
 * cached, which goes at `pos`.  Each round the draft decodes K tokens
 * greedily (its steps chained on the device), the target verifies
 * [last, d_1..d_K] with dpk_verify, and the accepted drafts plus the bonus
 * token are emitted.  The emitted tokens are the target's greedy
 * continuation: out_ids[0..n_new) (host) receives the tokens that follow
 * `token`.  K starts at k_init, grows by one after a round that accepted
 * all K drafts and shrinks by one after a round that accepted fewer than
 * half, within [k_min, k_max].  On return the target's cursor is pos plus
 * the tokens consumed (the last emitted token is not cached, as `token` was
 * not), and the draft's cursor equals it.  Requires
 * 1 <= k_min <= k_init <= k_max <= 15 and pos + n_new + k_max <= max_seq of
 * both models.  Synchronizes `stream` once per round (the drafts and the
 * accepted count are read back). */
typedef struct {
  int32_t k_init, k_min, k_max;
} dpk_spec_config;
typedef struct {
  int32_t rounds;       /* verify passes of the target */
  int32_t drafted;      /* draft tokens proposed */
  int32_t accepted;     /* of which accepted */
  int32_t draft_steps;  /* draft decode steps run (drafts plus catch-up steps) */
} dpk_spec_stats;
dpk_status dpk_spec_generate(dpk_model* target, dpk_model* draft, int32_t seq, int32_t pos, int32_t token,
                             int32_t n_new, const dpk_spec_config* sc, int32_t* out_ids, dpk_spec_stats* stats,
                             void* stream);

/* ------------------------------------------------------------ sampling
 * Sampling as a final kernel on the logits (Butter architecture notes, GPU
 * sampling diagram: only the 4-byte token leaves the GPU).  Per logit row x:
 *  - z = x / temperature; temperature 0 is greedy (lowest index of the max);
 *  - top_k > 0: keep the tokens whose z is at least the k-th largest z (ties
 *    with it kept); 0 keeps all;
 *  - the kept tokens' weights are exp(z - max z);
 *  - top_p < 1: the cut is the weight at which the mass of the heaviest
 *    kept tokens first reaches top_p of their total; every token at or
 *    above the cut stays (ties kept); 1 keeps all;
 *  - the token is the smallest index (index order) whose cumulative kept
 *    weight exceeds u times the kept total, for the row's uniform u in
 *    [0, 1) (the caller supplies the random numbers).
 * Weights are summed in 64-bit fixed point (2^-40 resolution), so a call is
 * deterministic.  Logits must be finite. */
typedef struct {
  float temperature; /* >= 0 */
  int32_t top_k;     /* >= 0; 0 = no top-k */
  float top_p;       /* (0, 1]; 1 = no top-p */
} dpk_sampler;

/* One token per row: logits fp32 [rows, ld] (device, the first vocab
 * entries of each row used), u fp32 [rows] (device), out int32 [rows]
 * (device).  Enqueued on `stream`; no workspace.  DPK_EINVAL for bad sizes
 * or sampler fields (nothing enqueued). */
dpk_status dpk_sample(const float* logits_dev, int32_t rows, int32_t vocab, int64_t ld, const dpk_sampler* sp,
                      const float* u_dev, int32_t* out_dev, void* stream);

/* Speculative-sampling acceptance (oxinfer 0.0.5 docs, "Speculative
 * decoding": the standard speculative-sampling rule; Butter notes,
 * speculative decoding loop).  k drafts d_1..d_k (device int32 [k]) were
 * drawn from the draft model's rows draft_logits [k, ld] (row i-1 drew d_i);
 * target_logits [k+1, ld] are the target's rows for the same positions (one
 * verify pass).  Both are turned into distributions p (target) and q
 * (draft) by the sampler above.  Draft d_i is accepted while
 * r[i-1] < p_{i-1}(d_i) / q_{i-1}(d_i); at the first rejection the next token
 * is drawn with u[i-1] from max(0, p - q) renormalised (from p if that is
 * zero everywhere); if all k are accepted it is drawn from target row k
 * with u[k].  r fp32 [k], u fp32 [k+1] (device uniforms in [0, 1)).  out
 * int32 [2] (device): accepted count m, next token.  With temperature 0 the
 * rule is the greedy one (accept while d_i equals the argmax).  A draft id
 * outside [0, vocab) counts as rejected.  workspace:
 * device, 16-byte aligned, dpk_spec_accept_workspace_size(k) bytes, owned
 * by the caller; calls that share one workspace must not overlap. */
#define DPK_SPEC_MAX_K 16
dpk_status dpk_spec_accept_workspace_size(int32_t k, size_t* bytes);
dpk_status dpk_spec_accept(const float* target_logits_dev, const float* draft_logits_dev, int64_t ld, int32_t vocab,
                           int32_t k, const int32_t* drafts_dev, const dpk_sampler* sp, const float* r_dev,
                           const float* u_dev, int32_t* out_dev, void* workspace_dev, size_t workspace_bytes,
                           void* stream);

/* dpk_spec_accept without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The distribution records live in a
 * 4 KB array built into the library, one per GPU, held until the process
 * ends; k may be at most 16.  Every call on one GPU shares that array, so
 * calls that overlap on one GPU (concurrent streams or threads) race and
 * must be serialized by the caller.  Allocates nothing (no hipMalloc, no
 * allocating library call); arguments and results as dpk_spec_accept. */
dpk_status dpk_spec_accept_noalloc(const float* target_logits_dev, const float* draft_logits_dev, int64_t ld,
                                   int32_t vocab, int32_t k, const int32_t* drafts_dev, const dpk_sampler* sp,
                                   const float* r_dev, const float* u_dev, int32_t* out_dev, void* stream);

/* Message of the last failure on the calling thread (valid until the next
 * call on this thread); "" if none. */
const char* dpk_last_error(void);

void dpk_destroy(dpk_model* m);

#ifdef __cplusplus
}
#endif
#endif /* DPK_H */
