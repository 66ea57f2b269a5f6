/*
 * nc.h -- C ABI of the MI355X (gfx950) training-step library.
 *
 * The library computes one forward + backward pass of a small decoder-only
 * GPT on one GPU: token embedding, parameter-free RMSNorm, causal multi-head
 * attention with QK-norm and RoPE, a ReLU-squared MLP, an untied LM head and
 * the mean next-token softmax cross-entropy.  Sources, cited by page and
 * section (the nanochat pages):
 *   - "nanochat explainer" (cloudtoid LLM book), Modern architecture choices:
 *     RoPE, RMSNorm, ReLU-squared, QK-norm, untied embeddings;
 *   - same page, Architecture Choices -> RoPE Intuition and ReLU² Sparsity;
 *   - same page, The 'One Dial' Design -> How dimensions are derived:
 *     d_model = 64*depth, heads = d_model/128, head_dim = 128, FFN = 4*d_model;
 *   - same page, The Full Pipeline -> Pretraining: causal next-token
 *     prediction, cross-entropy loss; Tokenizer Training: V = 65,536.
 *
 * Conventions for every entry point:
 *   - Device pointers are plain addresses of GPU memory the CALLER owns
 *     (allocated e.g. by torch).  The library never allocates device memory;
 *     scratch space is a caller-provided workspace.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns without synchronising;
 *     results are valid once the stream has been synchronised.
 *   - Return value: NC_OK or an nc_status code; no exception crosses the ABI.
 *     Argument and configuration errors are detected on the host before any
 *     GPU work is enqueued, and nothing is enqueued in that case.
 *   - Data-dependent errors (a token or target id outside [0, vocab), a
 *     non-finite loss) set a device status word instead; nc_check() reports
 *     it.  An out-of-range id is clamped so that no access leaves its buffer.
 *   - Element types: NC_BF16 stores weights and activations as bfloat16 and
 *     accumulates in fp32; NC_FP32 (debug path) stores everything as fp32.
 *     Gradients, losses and logits are always fp32.
 *   - Matrices are row-major.  Weights are [out, in] (y = x W^T).
 */
#ifndef NC_H
#define NC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NC_OK = 0,
  NC_ERR_CONFIG = 1,      /* invalid or inconsistent configuration */
  NC_ERR_NULL = 2,        /* a required pointer is NULL */
  NC_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  NC_ERR_TOKEN_RANGE = 4, /* (device) an id was outside [0, vocab) */
  NC_ERR_NONFINITE = 5,   /* (device) the loss was NaN or infinite */
  NC_ERR_HIP = 6,         /* a HIP runtime call failed */
  NC_ERR_UNSUPPORTED = 7, /* valid request outside what the kernels handle */
  NC_ERR_ARG = 8          /* invalid size or flag argument */
} nc_status;

typedef enum { NC_BF16 = 0, NC_FP32 = 1 } nc_dtype;

/*
 * Model configuration.  A zero in d_model / n_heads / head_dim / d_ff is
 * derived from `depth` by the depth dial ("nanochat explainer", How
 * dimensions are derived); a nonzero value overrides it.  Zero rope_base
 * means 10000, zero norm_eps means 1e-6.  n_kv_heads (zero: n_heads) below
 * n_heads is grouped-query attention, 1 multi-query attention ("nanochat
 * explainer", Inference & KV Cache): query head h uses key/value head
 * h / (n_heads / n_kv_heads), and the KV cache holds n_kv_heads heads.
 * Constraints: depth >= 1; head_dim in {16, 32, 64, 128} (the bf16 path:
 * 64 or 128); d_model, d_ff multiples of 64; vocab >= 64 and a multiple of
 * 64; seq_len >= 1 (the bf16 path with head_dim 128: at most 32640, its
 * attention backward keeps dS per sequence and head); max_batch >= 1;
 * n_kv_heads divides n_heads.
 */
typedef struct {
  int32_t depth;
  int32_t d_model;
  int32_t n_heads;
  int32_t head_dim;
  int32_t d_ff;
  int32_t vocab;
  int32_t seq_len;
  int32_t max_batch;
  float rope_base;
  float norm_eps;
  int32_t dtype; /* nc_dtype */
  int32_t n_kv_heads;
} nc_config;

typedef struct nc_ctx nc_ctx;

/* One parameter tensor inside the flat parameter / gradient buffers. */
typedef struct {
  char name[48];   /* "E", "layers.<l>.W_qkv" (rows: n_heads query heads,
                      then n_kv_heads key heads, then n_kv_heads value
                      heads, head_dim rows each), "layers.<l>.W_o",
                      "layers.<l>.W_1", "layers.<l>.W_2", "W_lm" */
  uint64_t offset; /* in elements from the start of the flat buffer */
  int32_t rows;    /* out features (vocab for E and W_lm) */
  int32_t cols;    /* in features */
} nc_tensor_desc;

/* Human-readable text for a status code.  Never NULL. */
const char* nc_strerror(int status);

/*
 * Validate `cfg`, apply the depth dial and plan the parameter layout and the
 * workspace.  Host only: makes no HIP call, so it also works without a GPU.
 * On success *out is a new context bound to `stream`.
 * Errors: NC_ERR_NULL (cfg or out NULL), NC_ERR_CONFIG.
 */
int nc_init(const nc_config* cfg, void* stream, nc_ctx** out);

/* Free the host context (the caller's device buffers are untouched). */
void nc_destroy(nc_ctx* ctx);

/* Copy the resolved configuration (derived fields filled in). */
int nc_get_config(const nc_ctx* ctx, nc_config* out);

/* Rebind the context to another stream. */
int nc_set_stream(nc_ctx* ctx, void* stream);

/*
 * Flat parameter layout: E [V,d]; then per layer l: W_qkv [3*H*hd, d]
 * (all q rows, then k, then v; head h owns rows h*hd..h*hd+hd-1 of each),
 * W_o [d, H*hd], W_1 [d_ff, d], W_2 [d, d_ff]; then W_lm [V, d].  Tensors are
 * packed back to back with no padding.  The gradient buffer uses the same
 * layout in fp32.
 */
uint64_t nc_param_count(const nc_ctx* ctx);
/* Writes min(cap, n) descriptors; returns n (the number of tensors). */
int nc_param_layout(const nc_ctx* ctx, nc_tensor_desc* out, int cap);

/* Workspace bytes needed by nc_forward_backward / nc_forward_logits for
 * `batch` sequences (batch <= max_batch). 0 for an invalid batch. */
uint64_t nc_workspace_bytes(const nc_ctx* ctx, int batch);

/* Attach caller-owned device workspace (256-byte aligned). */
int nc_set_workspace(nc_ctx* ctx, void* dev_ptr, uint64_t bytes);

/*
 * One training step's forward and backward pass.
 *   params  : device, flat layout above, element type cfg.dtype.
 *   tokens  : device int32 [batch, seq_len]; targets: device int32 [batch, seq_len]
 *             (targets[b][t] is the id that follows tokens[b][t]; a negative
 *             target leaves the position out of the loss: the loss mask of
 *             supervised fine-tuning, "nanochat explainer", Supervised
 *             Fine-Tuning; a target >= vocab is a status error).
 *   loss    : device fp32 scalar; the mean cross-entropy over the positions
 *             whose target is >= 0 (all batch*seq_len in pretraining), in
 *             nats; 0 when no position counts.
 *   grads   : device fp32, flat layout, the gradient of that loss;
 *             accumulate = 0 overwrites it, accumulate = 1 adds to it.
 * Saved activations live in the workspace, which must hold
 * nc_workspace_bytes(ctx, batch) bytes.  Not re-entrant: one context per stream.
 * The backward runs its weight-gradient products on a second stream that
 * the context creates on first use (default priority, ordered against the
 * context's stream by events; the context's stream waits for it before the
 * call returns), so the results are ordered on the context's stream as
 * usual.  NC_ERR_HIP if that stream or its events cannot be created.
 */
int nc_forward_backward(nc_ctx* ctx, const void* params, const int32_t* tokens,
                        const int32_t* targets, int batch, float* loss,
                        float* grads, int accumulate);

/*
 * One step over n_micro * micro_batch sequences run as n_micro microbatches
 * of micro_batch (gradient accumulation; the workspace only holds one
 * microbatch: the smaller batch that "nanochat explained: Karpathy's pipeline
 * from raw text to a chat model", What you need to run it, asks of GPUs with
 * less memory, at an unchanged step).  tokens, targets: device int32
 * [n_micro * micro_batch, seq_len], microbatch m in rows m*micro_batch ..
 * loss and grads (overwritten) are those of the whole step: the mean over
 * every counted position of all microbatches, so the result equals one
 * nc_forward_backward over all the sequences.
 * Errors: NC_ERR_NULL, NC_ERR_ARG (n_micro < 1, micro_batch outside
 * [1, max_batch]), NC_ERR_WORKSPACE (workspace < nc_workspace_bytes(ctx,
 * micro_batch)).
 */
int nc_forward_backward_accum(nc_ctx* ctx, const void* params, const int32_t* tokens,
                              const int32_t* targets, int n_micro, int micro_batch,
                              float* loss, float* grads);

/*
 * Forward pass only ("nanochat explainer", The Full Pipeline -> Pretraining:
 * the next-token logits the cross-entropy is taken over; Modern architecture
 * choices: the untied LM head).  tokens: device int32 [batch, seq_len];
 * logits: device fp32 [batch, seq_len, vocab], overwritten (caller-owned).
 * Uses the context's workspace (nc_workspace_bytes(ctx, batch)).
 * Errors: NC_ERR_NULL, NC_ERR_ARG (batch outside [1, max_batch]),
 * NC_ERR_WORKSPACE; an id outside [0, vocab) sets the status word.
 */
int nc_forward_logits(nc_ctx* ctx, const void* params, const int32_t* tokens,
                      int batch, float* logits);

/* ------------------------------------------------------------------------
 * Inference with a KV cache ("nanochat explainer", Inference & KV Cache):
 * prefill runs prompts through the forward and stores every layer's keys
 * and values; decode runs one new token per sequence against them.
 *
 * Cache (caller-owned device memory, nc_kv_cache_bytes): per layer K, then
 * V, each [cache_batch][n_kv_heads][max_len][head_dim] in the element type;
 * keys are stored QK-normalised and rotated.  Slot b of the cache holds
 * sequence b; 1 <= max_len <= 65536.
 * ------------------------------------------------------------------------ */
uint64_t nc_kv_cache_bytes(const nc_ctx* ctx, int cache_batch, int max_len);
/* Workspace of nc_decode for `batch` sequences and a cache of max_len. */
uint64_t nc_decode_workspace_bytes(const nc_ctx* ctx, int batch, int max_len);
/*
 * Prefill: tokens int32 [batch, len] (1 <= len <= seq_len <= max_len) run
 * through the forward (the context's workspace, nc_workspace_bytes(ctx,
 * batch)); their keys and values go to cache slots slot0 .. slot0+batch-1,
 * positions 0 .. len-1; logits fp32 [batch, vocab] receives the logits of
 * each sequence's last position.
 * Errors: NC_ERR_NULL, NC_ERR_ARG, NC_ERR_WORKSPACE.
 */
int nc_prefill(nc_ctx* ctx, const void* params, const int32_t* tokens, int batch, int len,
               void* cache, int cache_batch, int max_len, int slot0, float* logits);
/*
 * Decode one token per sequence: tokens int32 [batch], pos int32 [batch]
 * (device; the position of each token, i.e. its sequence's length so far;
 * may differ per sequence).  The token's key and value are written to the
 * cache (cache_batch == batch) at pos[b], it attends to positions 0..pos[b],
 * and logits fp32 [batch, vocab] receives the next-token logits.  workspace:
 * device, 256-byte aligned, nc_decode_workspace_bytes(ctx, batch, max_len)
 * bytes; its first word is a status word that the caller zeroes before the
 * first call and reads (and clears) with nc_op_status: a position outside
 * [0, max_len) or an id outside [0, vocab) sets it.
 * Enqueued on the context's stream with no host synchronisation and no
 * allocation, so the call can be captured in a HIP graph.
 * Errors: NC_ERR_NULL, NC_ERR_ARG, NC_ERR_WORKSPACE.
 */
int nc_decode(nc_ctx* ctx, const void* params, const int32_t* tokens, const int32_t* pos,
              int batch, void* cache, int max_len, void* workspace, uint64_t ws_bytes,
              float* logits);

/*
 * nc_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same step, with the workspace replaced by a static device array of
 * NC_DECODE_SCRATCH_BYTES owned by the library (one per GPU, held until the
 * process ends; its address is looked up on the first call on each device).
 * Arguments as for nc_decode, except:
 *   status: device int32, required; cleared at the start of the call, then
 *           set to the status bits of this call (1: a position or id out of
 *           range), the same codes nc_op_status decodes.
 * The call allocates nothing and never synchronises.  Calls on one GPU share
 * its array: calls that overlap on one GPU (other streams, other threads, a
 * graph replayed while one runs) race and must not be issued.  Run it with
 * the device of the context's stream current.
 * Errors: NC_ERR_NULL, NC_ERR_ARG, NC_ERR_WORKSPACE (the step needs more than
 * NC_DECODE_SCRATCH_BYTES: nc_decode_workspace_bytes(ctx, batch, max_len)
 * gives its need), NC_ERR_HIP (the array's address could not be found).
 */
#define NC_DECODE_SCRATCH_BYTES (32u << 20)
int nc_decode_static(nc_ctx* ctx, const void* params, const int32_t* tokens, const int32_t* pos, int batch,
                     void* cache, int max_len, float* logits, int* status);

/*
 * Synchronise the context's stream, then read and clear the device status
 * word.  Returns NC_OK, NC_ERR_TOKEN_RANGE (an id outside the vocabulary of
 * "nanochat explainer", Tokenizer Training), NC_ERR_NONFINITE (the loss of
 * The Full Pipeline -> Pretraining came out NaN or infinite) or NC_ERR_HIP.
 * Errors: NC_ERR_NULL, NC_ERR_WORKSPACE (no workspace attached).
 */
int nc_check(nc_ctx* ctx);

/*
 * Precision of the residual stream's addends on the bf16 path ("nanochat
 * explainer", Modern architecture choices: each block's attention and MLP
 * outputs are added to the residual stream).  The stream x is fp32 on both
 * paths.  With on = 0 (the default) the attention and MLP output projections
 * store their result rounded to bf16 and the next RMSNorm adds it to x; with
 * on = 1 they add their fp32 accumulators into x in the product's epilogue,
 * as the fp32 path always does.  Affects nc_forward_backward,
 * nc_forward_backward_accum, nc_forward_logits and nc_prefill; no effect on
 * an fp32 context or on nc_decode (which adds in fp32).
 * Errors: NC_ERR_NULL, NC_ERR_ARG (on not 0 or 1).
 */
int nc_set_residual_fp32(nc_ctx* ctx, int on);

/*
 * Debugging aid (no passage of the pages: it checks this library's use of
 * the caller's workspace).  With on = 1, nc_forward_backward,
 * nc_forward_backward_accum and nc_forward_logits first fill the whole
 * workspace except its 256-byte status block with all-ones bytes (NaN in
 * fp32 and bf16), so any read of workspace memory not written earlier in the
 * same call would change the results; they must come out bitwise identical
 * to a run with on = 0.  Costs one fill pass per call.
 * Errors: NC_ERR_NULL, NC_ERR_ARG (on not 0 or 1).
 */
int nc_debug_poison_workspace(nc_ctx* ctx, int on);

/*
 * Tracing: per-kernel-class GPU time.  When enabled, every launch made by
 * nc_forward_backward / nc_forward_logits is bracketed by HIP events on the
 * context's stream and credited to its class ("gemm", "attn_fwd",
 * "attn_bwd", "rmsnorm_fwd", "rmsnorm_bwd", "qknorm_rope_fwd",
 * "qknorm_rope_bwd", "embed_fwd", "embed_bwd", "ce_rows", "other") with the
 * call's algorithmic FLOPs (GEMMs: 2MNK; attention: causal model FLOPs) or
 * HBM bytes (bandwidth-bound kernels: each input read once, each output
 * written once).  nc_profile_enable synchronises the stream and clears the
 * records.  nc_profile_read synchronises, writes min(cap, n) entries and
 * returns n (negative nc_status on error).
 */
typedef struct {
  char name[32];
  int64_t launches;
  double ms;
  double flops;
  double bytes;
} nc_prof_entry;
int nc_profile_enable(nc_ctx* ctx, int on);
int nc_profile_read(nc_ctx* ctx, nc_prof_entry* out, int cap);

/* ------------------------------------------------------------------------
 * Optimizer step ("nanochat explainer", The Full Pipeline -> Pretraining,
 * which outlines the optimizer; settings taken: two groups, Muon and AdamW;
 * warmup then cosine learning-rate decay; gradient-norm bound 1.0; weight
 * decay 0.1).  The pages give only this outline;
 * AdamW is the decoupled form of Loshchilov and Hutter, Muon follows its
 * published description (Jordan et al., 2024).  Groups: AdamW for E and
 * W_lm; Muon for every layer tensor (W_qkv as one [3*H*hd, d] matrix, W_o,
 * W_1, W_2).  With s the 0-based step and m the schedule multiplier
 *   m = (s + 1) / warmup_steps                         for s < warmup_steps,
 *   m = f + (1 - f) (1 + cos(pi p)) / 2, p = (s - warmup) / max(1, total - warmup),
 * every gradient is first multiplied by min(1, clip / (|g|_2 + 1e-6)), |g|_2
 * the norm over all gradients; then
 *   AdamW (t = s + 1): m1 = b1 m1 + (1-b1) g, m2 = b2 m2 + (1-b2) g^2,
 *     w -= lr_adamw m (m1/(1-b1^t) / (sqrt(m2/(1-b2^t)) + eps) + wd w);
 *   Muon: B = mu B + G, U = G + mu B, O = NS(U) (ns_steps quintic
 *     Newton-Schulz steps with (a, b, c) = (3.4445, -4.7750, 2.0315) on
 *     U/(|U|_F + 1e-7), run on the wide orientation),
 *     W -= lr_muon m (sqrt(max(1, rows/cols)) O + wd W).
 * The weights being updated are fp32 masters kept in the optimizer state;
 * after the step the model's parameters (element type cfg.dtype) are
 * rewritten from them.  On the bf16 path the Newton-Schulz operands are
 * bf16 with fp32 accumulation.
 * ------------------------------------------------------------------------ */
typedef struct {
  float lr_adamw;      /* peak learning rate of E and W_lm */
  float lr_muon;       /* peak learning rate of the layer matrices */
  float beta1, beta2;  /* AdamW moment decays, in [0, 1) */
  float eps;           /* AdamW denominator term, > 0 */
  float momentum;      /* Muon (Nesterov) momentum, in [0, 1) */
  float weight_decay;  /* decoupled, both groups, >= 0 */
  float clip;          /* global gradient-norm bound, > 0 */
  float final_frac;    /* learning rate at the end of the decay / peak, in [0, 1] */
  int32_t warmup_steps;  /* >= 1 */
  int32_t total_steps;   /* >= warmup_steps */
  int32_t ns_steps;      /* Newton-Schulz iterations, >= 0 (5) */
} nc_optim_config;

/*
 * Bytes of optimizer state (device, fp32, 256-byte aligned, owned by the
 * caller): the master weights in the flat layout, then the AdamW moments of
 * E and W_lm, then the Muon momentum of the layer tensors.  0 for a NULL ctx.
 */
uint64_t nc_optim_state_bytes(const nc_ctx* ctx);
/* Bytes of workspace nc_optim_step needs (norm partials, Newton-Schulz temporaries). */
uint64_t nc_optim_workspace_bytes(const nc_ctx* ctx);
/*
 * Start the optimizer: masters = params (element type cfg.dtype, flat
 * layout), every moment and momentum = 0.  Enqueued on the context's stream.
 * Errors: NC_ERR_NULL.
 */
int nc_optim_init(nc_ctx* ctx, const void* params, void* state);
/*
 * One optimizer step `step` (0-based) from the fp32 gradients `grads` (flat
 * layout): updates the state and rewrites params.  grad_norm (device fp32
 * scalar, may be NULL) receives |g|_2 before clipping.  grads, params,
 * state and workspace are device buffers with 16-byte aligned starts.
 * Enqueued on the context's stream; nothing is read back to the host.
 * Errors: NC_ERR_NULL, NC_ERR_ARG (a hyperparameter outside its range,
 * step < 0, or a misaligned buffer), NC_ERR_WORKSPACE (ws_bytes <
 * nc_optim_workspace_bytes).
 */
int nc_optim_step(nc_ctx* ctx, const nc_optim_config* cfg, int step, const float* grads, void* params,
                  void* state, void* workspace, uint64_t ws_bytes, float* grad_norm);

/* ------------------------------------------------------------------------
 * Operation entry points (stateless).  Each takes its own workspace; the
 * matching *_workspace_bytes() gives its size.  `dtype` is an nc_dtype and
 * sets the element type of the non-fp32 arguments marked "(dt)".
 * ------------------------------------------------------------------------ */

/*
 * Causal attention with QK-norm and RoPE, forward and backward
 * ("nanochat explainer", Modern architecture choices; RoPE Intuition):
 *   qh = R_t rho(q), kh = R_t rho(k)  (rho: RMSNorm over head_dim, eps),
 *   out = softmax_{j<=t}(qh kh^T / sqrt(hd)) v,
 * and, for the upstream gradient dout, the gradients dq, dk, dv w.r.t. the
 * pre-norm q, k and v.  RoPE pairs element i with i + hd/2 and rotates by
 * t * rope_base^(-2i/hd), t = position within the sequence.
 * Layout of q, k, v, dout, out, dq, dk, dv: (dt) [B, T, H, hd] contiguous.
 * hd must be 16, 32, 64 or 128.  Errors: NC_ERR_NULL, NC_ERR_ARG (sizes),
 * NC_ERR_UNSUPPORTED (hd not in {64, 128} on the bf16 path, or T > 32640
 * with hd 128 on the bf16 path), NC_ERR_WORKSPACE.
 */
uint64_t nc_attention_workspace_bytes(int B, int H, int T, int hd, int dtype);
int nc_attention_fwd_bwd(const void* q, const void* k, const void* v,
                         const void* dout, void* out, void* dq, void* dk,
                         void* dv, int B, int H, int T, int hd,
                         float rope_base, float eps, int dtype,
                         void* workspace, uint64_t ws_bytes, void* stream);

/*
 * Fused LM head + softmax cross-entropy, forward and backward ("nanochat
 * explainer", Pretraining: next-token cross-entropy), processed in chunks of
 * tokens so that the full [N, V] logits never exist:
 *   l = z W^T; loss = mean_n [logsumexp(l_n) - l_{n,y_n}] over the n with
 *   y_n >= 0 (a negative id is not counted; 0 if none is);
 *   G = (softmax(l) - onehot(y)) / count (0 on rows not counted);
 *   dz = G W;  dW = G^T z.
 * z: (dt) [N, d]; W: (dt) [V, d]; y: int32 [N]; loss: fp32 scalar;
 * dz: fp32 [N, d] (overwritten); dW: fp32 [V, d] (overwritten).
 * Errors: NC_ERR_NULL, NC_ERR_ARG, NC_ERR_WORKSPACE.  Ids outside [0, V)
 * set the device status word read by nc_op_status().
 */
uint64_t nc_lmhead_ce_workspace_bytes(int N, int d, int V, int dtype);
int nc_lmhead_ce_fwd_bwd(const void* z, const void* W, const int32_t* y,
                         int N, int d, int V, float* loss, float* dz,
                         float* dW, int dtype, void* workspace,
                         uint64_t ws_bytes, void* stream);

/*
 * Read and clear the device status word at the start of an operation
 * workspace (synchronises `stream`).  Same codes as nc_check().
 */
int nc_op_status(void* workspace, void* stream);

/*
 * Row RMSNorm ("nanochat explainer", Modern architecture choices: RMSNorm),
 * parameter-free: y = x / sqrt(mean(x^2) + eps), r = 1/sqrt(mean(x^2) + eps).
 * x: fp32 [N, d]; y: (dt) [N, d]; r: fp32 [N].  d must be a multiple of 4;
 * N = 0 is a no-op.
 */
int nc_rmsnorm_fwd(const float* x, void* y, float* r, int N, int d, float eps,
                   int dtype, void* stream);
/*
 * Backward: dx (+)= r * (dy - y * mean(dy * y)).  dy: fp32 [N, d];
 * y: (dt) [N, d]; r: fp32 [N]; dx: fp32 [N, d], overwritten when
 * accumulate = 0 and added to when 1; dx_lp: optional (dt) copy of the
 * resulting dx (may be NULL).
 */
int nc_rmsnorm_bwd(const float* dy, const void* y, const float* r, float* dx,
                   void* dx_lp, int N, int d, int accumulate, int dtype,
                   void* stream);

/*
 * Token embedding ("nanochat explainer", Modern architecture choices:
 * untied embeddings).  Forward: x[n] = E[tokens[n]]; E: (dt) [V, d];
 * x: fp32 [N, d].  Uses the first 256 bytes of `workspace` for the status
 * word (nc_op_status reads it).
 */
int nc_embedding_fwd(const void* E, const int32_t* tokens, float* x, int N,
                     int d, int V, int dtype, void* workspace, void* stream);
/*
 * Backward without floating-point atomics: dE[v] = sum over the positions n
 * with tokens[n] == v, in increasing n, of dx[n]; rows of ids that do not
 * occur are 0 (accumulate = 0) or unchanged (accumulate = 1).
 * dx: fp32 [N, d]; dE: fp32 [V, d].  Deterministic run to run.
 */
uint64_t nc_embedding_bwd_workspace_bytes(int N, int d, int V);
int nc_embedding_bwd(const float* dx, const int32_t* tokens, float* dE, int N,
                     int d, int V, int accumulate, void* workspace,
                     uint64_t ws_bytes, void* stream);

/*
 * Matrix product with fp32 accumulation, the building block of every linear
 * layer (y = x W^T), its input gradient (dx = dy W) and weight gradient
 * (dW = dy^T x):   C[i, j] (+)= sum_k A(i, k) * B(j, k),
 * for i < M, j < N, k < K.  a_kmajor = 1: A(i,k) = A[i*lda + k], else
 * A(i,k) = A[k*lda + i]; likewise b_kmajor for B(j,k) = B[j*ldb + k] or
 * B[k*ldb + j].  A, B: (dt); C: fp32 [M, N] with row stride ldc,
 * overwritten (beta = 0) or added to (beta = 1).  The contiguous dimension
 * of A and B must be a multiple of 8.
 */
uint64_t nc_gemm_workspace_bytes(int M, int N, int K, int dtype);
int nc_gemm(const void* A, int lda, int a_kmajor, const void* B, int ldb,
            int b_kmajor, float* C, int ldc, int M, int N, int K, int beta,
            int dtype, void* workspace, uint64_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NC_H */
