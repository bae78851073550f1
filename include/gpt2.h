/*
 * gpt2.h -- C ABI of the MI355X (gfx950) GPT-2 training-step library.
 *
 * One training step of a pre-LayerNorm, decoder-only GPT-2 on one GPU: embedding, n_layer
 * blocks of causal multi-head attention and a 4x GELU-tanh MLP, final LayerNorm, lm_head
 * tied to the token embedding, mean cross-entropy; the backward pass; global-norm gradient
 * clipping and AdamW. The model follows the code excerpts of "Karpathy's Zero to Hero,
 * Lecture 9: Reproduce GPT-2 (124M) -- notes, code and timestamps" (section "Code you'll
 * write": Block/MLP, causal self-attention, model skeleton and initialization, forward pass
 * with loss, the optimizer step) and the "Architecture" section of the reproduce-gpt2 README.
 *
 * Conventions shared by every call:
 *  - Return value: GPT2_OK (0) or a negative error code. On error nothing has been
 *    enqueued after the failing launch, and gpt2_last_error() returns a message. The
 *    library never aborts the process.
 *  - Memory: the caller owns all device memory. The library allocates no device memory: it
 *    carves every buffer (parameters, gradients, AdamW moments, saved activations, scratch)
 *    out of one caller-provided workspace of gpt2_workspace_bytes() bytes, and it never
 *    frees caller memory.
 *  - Streams: every kernel is enqueued on the handle's HIP stream (set at creation or with
 *    gpt2_set_stream). Only calls that return a value through a host pointer synchronize
 *    that stream.
 *  - A handle is not thread-safe; calls on one handle must be serialized by the caller.
 *  - Device pointers are plain addresses on the device the handle was created on.
 *  - Token ids must lie in [0, vocab_size); they are not checked on the device.
 */
#ifndef GPT2_STEP_H
#define GPT2_STEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes. */
#define GPT2_OK 0
#define GPT2_EINVAL (-1) /* bad argument: null pointer, bad shape, T > block_size, B > max_batch, workspace too small */
#define GPT2_ESTATE (-2) /* call out of order, e.g. backward without a forward that had targets */
#define GPT2_EHIP (-3)   /* a HIP runtime call or kernel launch failed; the message names it */

/* Arithmetic modes (what each stores; every accumulation is fp32 in all three):
 * GPT2_FP32        every tensor fp32, products on fp32 MFMA (a check mode).
 * GPT2_BF16        the autocast recipe of chapter 1:36:50-1:48:25 of the lecture notes:
 *                  product and attention operands bf16 (bf16 copies of the 2-D weights; LayerNorm
 *                  outputs, q|k|v, attention output, GELU input and output, logits and their
 *                  gradient, and every activation gradient that feeds a product); the residual
 *                  stream (embedding sum and every residual add) and its gradient fp32, with a
 *                  bf16 copy of that gradient as the products' operand; LayerNorm statistics,
 *                  softmax and loss math, master weights, gradients and AdamW moments fp32.
 * GPT2_BF16_RES16  GPT2_BF16 with the residual stream and its gradient also stored in bf16
 *                  (narrower than the autocast recipe; fewer bytes per LayerNorm and residual add).
 * fp32 -> bf16 conversions round to nearest even. */
#define GPT2_FP32 0
#define GPT2_BF16 1
#define GPT2_BF16_RES16 2

/* Model and capacity. The counting and layout calls need only positive sizes, n_embd a
 * multiple of n_head and padded_vocab_size >= vocab_size. Sizing the workspace and creating
 * a handle also need: head size n_embd/n_head of 64 or 32, n_embd <= 2048, n_embd and
 * mlp_hidden multiples of 8, padded_vocab_size a multiple of 8 and below 2^18 (50304 for
 * GPT-2: chapter 2:06:39-2:14:58 pads 50257 up to a multiple of 128). max_batch *
 * block_size bounds the tokens of one forward. */
typedef struct gpt2_config {
    int32_t n_layer;
    int32_t n_head;
    int32_t n_embd;
    int32_t mlp_hidden;
    int32_t block_size;
    int32_t vocab_size;        /* V: token ids lie in [0, V) */
    int32_t padded_vocab_size; /* Vp: rows of wte and width of the softmax */
    int32_t max_batch;
    int32_t dtype;             /* GPT2_FP32, GPT2_BF16 or GPT2_BF16_RES16 */
} gpt2_config;

typedef struct gpt2 gpt2_t;

/* ---------------------------------------------------------------- sizing (host only) */

/* Bytes of device workspace a handle for this config needs (0 if the config is invalid). */
size_t gpt2_workspace_bytes(const gpt2_config* cfg);

/* Number of parameters (wte counted once, with padded_vocab_size rows). Pass
 * padded_vocab_size = vocab_size = 50257 to get the 124,439,808 of the README's
 * "Architecture" table. Returns -1 for an invalid config (layout checks only). */
int64_t gpt2_num_params(const gpt2_config* cfg);

/* Number of parameter tensors (148 at n_layer 12) and the count that receive weight decay
 * (tensors with two dimensions: 50 at n_layer 12, chapter 2:25:57-2:34:49). */
int32_t gpt2_num_tensors(const gpt2_config* cfg);
int32_t gpt2_num_decay_tensors(const gpt2_config* cfg);

/* Describe tensor i (0 <= i < gpt2_num_tensors) of the canonical flat fp32 parameter
 * arena: Hugging Face style name (static string), element offset, shape (shape[1] = 0 for
 * 1-D tensors). Layout: every 2-D tensor first (wte [Vp,C], wpe [block_size,C], then per
 * layer attn.c_attn.weight [3C,C], attn.c_proj.weight [C,C], mlp.c_fc.weight [F,C],
 * mlp.c_proj.weight [C,F]), then every 1-D tensor (per layer ln_1.weight, ln_1.bias,
 * attn.c_attn.bias, attn.c_proj.bias, ln_2.weight, ln_2.bias, mlp.c_fc.bias,
 * mlp.c_proj.bias, then ln_f.weight, ln_f.bias). Linear weights are [out, in] row-major.
 * The weight-decayed tensors are therefore exactly the prefix [0, decay_end). The same
 * layout is used for gradients and AdamW moments. */
int gpt2_param_info(const gpt2_config* cfg, int32_t i, const char** name, int64_t* offset,
                    int64_t shape[2]);
int64_t gpt2_decay_end(const gpt2_config* cfg);

/* ---------------------------------------------------------------- lifetime */

/* Create a handle over the caller's workspace d_ws (device memory, >= gpt2_workspace_bytes,
 * 256-byte aligned) and initialize the parameters on the device from `seed`: N(0, 0.02)
 * for both embeddings and every Linear weight, std 0.02/sqrt(2*n_layer) for attn.c_proj
 * and mlp.c_proj weights, biases 0, LayerNorm gains 1 and biases 0 (chapter 1:13:27-1:22:16
 * and the _init_weights excerpt). Gradients and moments are zeroed. `stream` is a
 * hipStream_t (NULL = the null stream). The normal deviates come from a counter-based
 * generator (Philox-4x32-10 with Box-Muller), so they are reproducible but are not meant
 * to match any other generator. */
int gpt2_create(const gpt2_config* cfg, void* d_ws, size_t ws_bytes, uint64_t seed, void* stream,
                gpt2_t** out);

/* Release host-side state. The workspace stays the caller's. */
int gpt2_destroy(gpt2_t* h);

/* Change the stream later calls enqueue on. */
int gpt2_set_stream(gpt2_t* h, void* stream);

/* ---------------------------------------------------------------- parameter I/O */

/* Copy the whole canonical fp32 arena (gpt2_num_params floats) in or out. `on_device`
 * says whether src/dst is device memory (1) or host memory (0). Host copies synchronize the
 * stream. Setting parameters also refreshes the bf16 copies of the weights. */
int gpt2_set_params(gpt2_t* h, const float* src, int on_device);
int gpt2_get_params(gpt2_t* h, float* dst, int on_device);
int gpt2_get_grads(gpt2_t* h, float* dst, int on_device);
int gpt2_set_grads(gpt2_t* h, const float* src, int on_device);
/* AdamW first and second moments (either pointer may be NULL to skip it). */
int gpt2_get_moments(gpt2_t* h, float* m, float* v, int on_device);
int gpt2_set_moments(gpt2_t* h, const float* m, const float* v, int on_device);
/* Device addresses of the arenas inside the workspace (for zero-copy inspection). */
float* gpt2_params_device(gpt2_t* h);
float* gpt2_grads_device(gpt2_t* h);

/* ---------------------------------------------------------------- the step */

/* Forward pass over B sequences of T tokens (T <= block_size, B <= max_batch).
 *   d_idx      int32 [B, T] device, token ids (copied into the workspace; reusable at return)
 *   d_targets  int32 [B, T] device or NULL. With targets, the mean cross-entropy over all
 *              B*T positions and all padded_vocab_size columns is computed (F.cross_entropy
 *              on the flattened logits, "Code you'll write", forward with loss), and the
 *              activations needed by gpt2_backward are kept.
 *   d_logits   float [B, T, Vp] device or NULL: receives the logits (fp32).
 *   d_loss     float device scalar or NULL: receives the loss without synchronizing.
 *   h_loss     float host scalar or NULL: receives the loss (synchronizes the stream).
 * Without targets, d_logits is required and d_loss/h_loss must be NULL. */
int gpt2_forward(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, int32_t B, int32_t T,
                 float* d_logits, float* d_loss, float* h_loss);

/* Forward-only evaluation: the validation loss and completion scoring of the lecture notes
 * (chapter 3:22:33-3:28:16: the loss averaged over validation batches with no backward pass;
 * chapter 3:28:16-3:41:50: each candidate row is the shared context followed by one ending,
 * padded to a common length, and the row whose ending tokens have the lowest mean
 * cross-entropy is the prediction). Runs the forward over B sequences of T tokens and the
 * per-position cross-entropy of the targets (as gpt2_forward, without forming its gradient),
 * then reduces it per sequence over the positions the mask selects.
 *   d_idx, d_targets  int32 [B, T] device; the target of position t is the token that
 *              follows it, as in gpt2_forward (copied into the workspace; reusable at return)
 *   d_mask     uint8 [B, T] device or NULL: nonzero selects a position; NULL selects all
 *   d_row_sum  float [B] device or NULL: sum of the selected positions' losses per sequence
 *   d_row_mean float [B] device or NULL: that sum over the number of selected positions
 *              (0 for a sequence with none selected)
 *   d_loss     float device scalar or NULL: mean loss over every selected position of the
 *              batch (without a mask, exactly the loss gpt2_forward reports for these inputs)
 * Sums are formed in double in a fixed order (deterministic). Nothing synchronizes. The call
 * overwrites the saved activations: a following gpt2_backward fails with GPT2_ESTATE until
 * gpt2_forward runs again. Gradients and optimizer state are untouched. */
int gpt2_evaluate(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, const uint8_t* d_mask, int32_t B,
                  int32_t T, float* d_row_sum, float* d_row_mean, float* d_loss);

/* For callers that cannot allocate device memory or use a workspace-backed scratch between
 * calls (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): gpt2_evaluate with the same arguments, results and errors, whose own scratch
 * (the per-position losses, the mask copy and the per-sequence double sums) lives in a
 * fixed device array of the library instead of the handle's workspace. The array is
 * GPT2_NOALLOC_MAX_SEQ * 16 + GPT2_NOALLOC_MAX_ROWS * 5 bytes (1.3 MiB); each GPU the library
 * runs on holds one copy until the process ends. Calls with B > GPT2_NOALLOC_MAX_SEQ or
 * B*T > GPT2_NOALLOC_MAX_ROWS fail with GPT2_EINVAL before anything is enqueued. Every call
 * on a GPU shares that GPU's array (it keeps the last call's contents; every value a call
 * reads is written by that call first), so calls that overlap on one GPU -- from two handles
 * on different streams, or two threads -- race and must be serialized by the caller. The
 * handle's activations are used as by gpt2_evaluate. Nothing here allocates: no hipMalloc,
 * hipFree or allocating library routine. */
#define GPT2_NOALLOC_MAX_SEQ 4096
#define GPT2_NOALLOC_MAX_ROWS 262144
int gpt2_evaluate_noalloc(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, const uint8_t* d_mask,
                          int32_t B, int32_t T, float* d_row_sum, float* d_row_mean, float* d_loss);

/* ---------------------------------------------------------------- incremental decoding */

/* Sampling as the lecture notes do it (chapter 0:28:07-0:41:44 and the sampling code of
 * chapter 3:22:33-3:28:16): the logits of the last position go through the softmax, the
 * top_k most probable tokens are kept (50 there) and one of them is drawn in proportion to
 * its probability; the token is appended and the loop repeats. Here the keys and values of
 * the earlier positions stay in a cache, so each step runs the model on one new position per
 * sequence. The cache lives in the handle's activation buffers: gpt2_forward and
 * gpt2_evaluate overwrite it (a later step fails with GPT2_ESTATE until a reset), and
 * decoding overwrites the activations a gpt2_backward would need. */
#define GPT2_TOPK_MAX 64       /* largest top_k */
#define GPT2_DECODE_MAX_T 8192 /* largest block_size that decoding supports */

/* Start (or restart) B sequences with an empty cache (B <= max_batch). */
int gpt2_decode_reset(gpt2_t* h, int32_t B);

/* Append one token to each of the B sequences at position p = the number of steps since the
 * reset (p < block_size) and compute the logits of that position. A prompt is fed one step
 * per token; the outputs of all but its last step can be ignored.
 *   d_tokens    int32 [B] device: the tokens at position p (copied; reusable at return)
 *   d_logits    float [B, Vp] device or NULL: the logits (fp32 copy of the model's output)
 *   top_k       1..GPT2_TOPK_MAX, used when any of the three outputs below is requested
 *   d_uniform   float [B] device, each in [0, 1): the caller's random numbers (needed with d_next)
 *   d_next      int32 [B] device or NULL: the drawn token: over the top_k logits (all Vp
 *               columns compete, larger first, equal ones by lower token id), their softmax
 *               p_1..p_k (the top-k probabilities renormalized), the first i whose cumulative
 *               sum p_1 + .. + p_i exceeds d_uniform[b] (the last one if rounding leaves none)
 *   d_topk_idx  int32 [B, top_k] device or NULL: the top_k token ids in that order
 *   d_topk_prob float [B, top_k] device or NULL: their renormalized probabilities
 * d_next may be the next step's d_tokens. Nothing synchronizes. */
int gpt2_decode_step(gpt2_t* h, const int32_t* d_tokens, float* d_logits, int32_t top_k, const float* d_uniform,
                     int32_t* d_next, int32_t* d_topk_idx, float* d_topk_prob);

/* gpt2_decode_step at the position held in device memory, for a step captured once in a HIP
 * graph and replayed (the host's arguments of a replayed launch cannot change):
 *   d_pos  int32 [1] device: the position p of this step; the kernels read it when they run,
 *          and the step leaves min(p + 1, block_size) there for the next one.
 * The caller keeps p < block_size (a larger value is clamped to block_size - 1, so the step
 * overwrites the last cached position: no memory outside the cache is touched) and sets
 * *d_pos to the number of positions already cached (e.g. after feeding a prompt with
 * gpt2_decode_step). gpt2_decode_position does not count these steps. Other arguments,
 * outputs and errors as in gpt2_decode_step. */
int gpt2_decode_step_device(gpt2_t* h, const int32_t* d_tokens, int32_t* d_pos, float* d_logits, int32_t top_k,
                            const float* d_uniform, int32_t* d_next, int32_t* d_topk_idx, float* d_topk_prob);

/* Positions in the cache (-1 without a reset or after the cache was overwritten). */
int32_t gpt2_decode_position(const gpt2_t* h);

/* Backward pass of the last forward (which must have had targets):
 *   grads = (accumulate ? grads : 0) + grad_scale * d loss / d params
 * grad_scale is the 1/micro_steps factor of gradient accumulation (chapter 2:34:49-2:46:43:
 * the loss is divided by the number of micro-steps before backward). The gradients of the
 * two uses of wte (embedding and lm_head) add into one tensor. Deterministic: the same
 * inputs give bitwise identical gradients. */
int gpt2_backward(gpt2_t* h, float grad_scale, int32_t accumulate);

/* Clip and update (chapter 2:14:58-2:34:49 and the optimizer-step excerpt):
 *   norm = sqrt(sum of squares of every gradient)            (pre-clip; wte counted once)
 *   c    = min(1, max_grad_norm / (norm + 1e-6))              (clip_grad_norm_)
 *   for every element, with g = c * grad:
 *     p *= 1 - lr * weight_decay    (only the 2-D tensors: offsets < gpt2_decay_end)
 *     m  = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2
 *     p -= lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 * t is the 1-based AdamW step count. Gradients are left as they are. h_grad_norm (host,
 * nullable) receives the pre-clip norm and synchronizes; d_grad_norm (device, nullable)
 * receives it without synchronizing. */
int gpt2_adamw_step(gpt2_t* h, float lr, float beta1, float beta2, float eps, float weight_decay,
                    float max_grad_norm, int32_t t, float* d_grad_norm, float* h_grad_norm);

/* The learning-rate schedule of the optimizer-step excerpt (host arithmetic): linear warmup
 * max_lr*(it+1)/warmup_steps for it < warmup_steps, min_lr after max_steps, cosine decay
 * from max_lr to min_lr in between. */
double gpt2_cosine_lr(int64_t it, double max_lr, double min_lr, int64_t warmup_steps,
                      int64_t max_steps);

/* Graph-replayable optimizer step ("Karpathy's Zero to Hero, Lecture 9" notes, "Code you'll
 * write", training step: the learning rate set from the schedule each step, then AdamW). For a
 * training step captured once in a HIP graph (gpt2_set_stream to the capture stream) and
 * replayed: the scalars a host call would pass live in device memory and are read when the
 * kernels run, so every replay advances the schedule.
 * gpt2_schedule_step_device: with it = *d_step (0-based optimizer step, device int32):
 *   *d_lr = gpt2_cosine_lr(it, max_lr, min_lr, warmup_steps, max_steps) (the same double
 *   arithmetic, rounded to float), *d_t = it + 1, then *d_step = it + 1. Requires
 *   1 <= warmup_steps < max_steps (GPT2_EINVAL otherwise). Enqueued on the handle's stream.
 * gpt2_adamw_step_device: gpt2_adamw_step with lr = *d_lr and t = *d_t (device float and
 *   int32, read when the update runs; t >= 1), bias corrections 1 - beta^t in double as on
 *   the host path. d_grad_norm (device, nullable) receives the pre-clip norm. There is no
 *   host-norm output (that would synchronize). */
int gpt2_schedule_step_device(gpt2_t* h, int32_t* d_step, float* d_lr, int32_t* d_t, double max_lr,
                              double min_lr, int64_t warmup_steps, int64_t max_steps);
int gpt2_adamw_step_device(gpt2_t* h, const float* d_lr, const int32_t* d_t, float beta1, float beta2,
                           float eps, float weight_decay, float max_grad_norm, float* d_grad_norm);

/* ---------------------------------------------------------------- diagnostics */

/* Message of the last error on this thread ("" if none). */
const char* gpt2_last_error(void);

/* Per-kernel timing with HIP events on the handle's stream. gpt2_timing_begin(h, name)
 * records an event pair around every later launch of the kernel class `name` (NULL = all
 * classes); gpt2_timing_end(h) stops recording and synchronizes; gpt2_timing_get returns
 * the summed milliseconds and the number of launches of class `name`. Class names are
 * listed by gpt2_kernel_class(i) (NULL past the end). */
int gpt2_timing_begin(gpt2_t* h, const char* name);
int gpt2_timing_end(gpt2_t* h);
int gpt2_timing_get(gpt2_t* h, const char* name, double* total_ms, int64_t* launches);
const char* gpt2_kernel_class(int32_t i);

/* Copy a saved activation of the last forward for inspection: which = "x_in" (the residual
 * stream entering layer `layer`; layer = n_layer is ln_f's input), "h1", "qkv",
 * "att", "lse", "h2", "u", "a", "x_out", "hf" (layer ignored for the last two) or "dz"
 * (after a forward with targets: the cross-entropy gradient (softmax - onehot)/(B*T),
 * unscaled). Values are converted to fp32 into d_dst (device), which must hold
 * *count floats; pass d_dst = NULL to query *count. */
int gpt2_debug_tensor(gpt2_t* h, const char* which, int32_t layer, float* d_dst, int64_t* count);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_STEP_H */
