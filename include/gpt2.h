/*
 * gpt2.h - C ABI of the MI355X (gfx950) GPT-2 training-step library.
 *
 * One GPT-2 training micro-step -- forward, backward, AdamW -- over a
 * decoder-only transformer, every step in hand-written HIP kernels.  The model
 * and its step follow the "train_gpt2.cu" page (llm.c, mixed precision):
 * GPT2Config, ParameterTensors, gpt2_forward, gpt2_zero_grad, gpt2_backward and
 * gpt2_update.  Differences from that page are listed per function.
 *
 * Conventions for every entry point:
 *  - All pointers named d_* (and every pointer inside gpt2_buffers) are DEVICE
 *    pointers, allocated and owned by the caller, 256-byte aligned, valid on the
 *    device that is current when the call is made.  The library never allocates
 *    or frees device memory.
 *  - hip_stream is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it and returns; results are ready when the stream is.
 *  - Return value: GPT2_OK (0) or a negative GPT2_E_* code; no entry point
 *    exits the process.  gpt2_strerror names the code.
 *  - A context is not thread-safe: calls on one context must be serialised by
 *    the caller.
 *  - Layout: every matrix is row-major.  Weights are (out_features,
 *    in_features), as on the page.  Activations are [B*T, channels].
 */
#ifndef GPT2_MI355X_H
#define GPT2_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* train_gpt2.cu, GPT2Config.  padded_vocab_size >= vocab_size; the classifier
 * runs over padded_vocab_size columns, the loss over vocab_size of them. */
typedef struct {
    int max_seq_len;
    int vocab_size;
    int padded_vocab_size;
    int num_layers;
    int num_heads;
    int channels;
} gpt2_config;

/* Arithmetic mode (train_gpt2.cu, PrecisionMode; fp16 is not offered because
 * the page leaves it unsupported).
 *  GPT2_FP32: fp32 parameters, activations and products (full-precision fp32
 *             products, no reduced-precision inputs).
 *  GPT2_BF16: bf16 parameters, activations and matrix-core products with fp32
 *             accumulation; fp32 master weights, fp32 gradients, fp32 AdamW
 *             state, fp32 LayerNorm statistics, losses and residual gradient.
 *  GPT2_BF16_SR: GPT2_BF16 without the fp32 master weights (train_gpt2.cu,
 *             adamw_kernel3 without master_params): `master` is unused (0
 *             bytes), the caller writes the bf16 initial values into `params`,
 *             and each update rounds the new fp32 values to bf16
 *             stochastically (see gpt2_adamw_update). */
enum { GPT2_FP32 = 0, GPT2_BF16 = 1, GPT2_BF16_SR = 2 };

enum {
    GPT2_OK = 0,
    GPT2_E_ARG = -1,    /* NULL / out-of-range argument */
    GPT2_E_SHAPE = -2,  /* unsupported shape (see gpt2_init) */
    GPT2_E_STATE = -3,  /* call order violated (e.g. backward without a forward with targets) */
    GPT2_E_TOKEN = -4,  /* a token or target id outside [0, vocab_size) was seen on the device */
    GPT2_E_ALIGN = -5,  /* a pointer is not 256-byte aligned */
    GPT2_E_HIP = -6,    /* a HIP runtime call or kernel launch failed */
    GPT2_E_FILE = -7    /* a model file cannot be read or is not a valid model file */
};

typedef struct gpt2_ctx gpt2_ctx;

/* Byte sizes of the caller-owned device buffers for one (config, precision,
 * B, T).  master is 0 in GPT2_FP32 mode. */
typedef struct {
    size_t params, master, grads, adam_m, adam_v, acts, scratch;
} gpt2_sizes;

/* The device buffers, each at least the size gpt2_query_sizes reports.
 *  params : the 16 parameter tensors, flat, in gpt2_param_layout order;
 *           fp32 (GPT2_FP32) or bf16 (GPT2_BF16).
 *  master : GPT2_BF16 only: fp32 copy of params (the AdamW master weights);
 *           NULL in GPT2_FP32 mode.
 *  grads, adam_m, adam_v : fp32, flat, same layout.
 *  acts   : forward activations and backward scratch (opaque except for the
 *           tensors gpt2_act_tensor exposes).
 *  scratch: workspaces (opaque): the split-K partials of the products that
 *           split, the LayerNorm backwards' partial column sums and the
 *           embedding backward's sort. */
typedef struct {
    void *params, *master, *grads, *adam_m, *adam_v, *acts, *scratch;
} gpt2_buffers;

/* Fills *out with the buffer sizes.  Errors: GPT2_E_ARG, GPT2_E_SHAPE. */
int gpt2_query_sizes(const gpt2_config* cfg, int precision, int B, int T, gpt2_sizes* out);

/* Element offsets and counts of the 16 parameter tensors in the page's order
 * (train_gpt2.cu, ParameterTensors / fill_in_parameter_sizes): wte (Vp,C),
 * wpe (maxT,C), ln1w (L,C), ln1b (L,C), qkvw (L,3C,C), qkvb (L,3C),
 * attprojw (L,C,C), attprojb (L,C), ln2w (L,C), ln2b (L,C), fcw (L,4C,C),
 * fcb (L,4C), fcprojw (L,C,4C), fcprojb (L,C), lnfw (C), lnfb (C).
 * *total receives the parameter count.  Errors: GPT2_E_ARG. */
int gpt2_param_layout(const gpt2_config* cfg, size_t offset[16], size_t count[16], size_t* total);

/* Creates a context bound to the caller's buffers for fixed B and T (the page
 * fixes them at the first forward).  Enqueues on hip_stream: zeroing of
 * adam_m and adam_v (as gpt2_update does at its first call) and, in GPT2_BF16
 * mode, the round-to-nearest-even cast master -> params (the caller writes the
 * fp32 initial values into master).  In GPT2_FP32 mode the caller writes
 * params directly.
 * Shape limits: channels % num_heads == 0; head size C/NH a multiple of 16 and
 * at most 128; channels and padded_vocab_size multiples of 8;
 * 1 <= T <= max_seq_len; B >= 1; padded_vocab_size <= 53248.
 * Also creates the context's internal stream (default priority, not blocking
 * on the null stream) and its events, used by gpt2_backward.
 * Errors: GPT2_E_ARG, GPT2_E_SHAPE, GPT2_E_ALIGN, GPT2_E_HIP. */
int gpt2_init(gpt2_ctx** out, const gpt2_config* cfg, int precision, int B, int T,
              const gpt2_buffers* bufs, void* hip_stream);

/* train_gpt2.cu, gpt2_forward.  d_inputs [B*T] int32 token ids.  d_targets
 * [B*T] int32 or NULL.  With targets: per-position losses are written to
 * d_losses [B*T] fp32 (if not NULL), their mean to d_mean_loss [1] fp32 (if not
 * NULL), and the logits are overwritten in place by softmax - onehot (over the
 * first vocab_size columns; the padded columns are set to 0), which backward
 * consumes -- so logits are not readable after a forward with targets.
 * Without targets the logits stay readable (gpt2_act_tensor).  Ids outside
 * [0, vocab_size) are clamped for memory safety and raise a device flag that
 * gpt2_check_device_error reports (the page asserts on the host).
 * Errors: GPT2_E_ARG, GPT2_E_ALIGN, GPT2_E_HIP. */
int gpt2_forward(gpt2_ctx* ctx, const int32_t* d_inputs, const int32_t* d_targets,
                 float* d_losses, float* d_mean_loss, void* hip_stream);

/* train_gpt2.cu, gpt2_zero_grad, restricted to the parameter gradients (the
 * activation gradients are internal and overwritten by every backward).
 * Errors: GPT2_E_ARG, GPT2_E_HIP. */
int gpt2_zero_grad(gpt2_ctx* ctx, void* hip_stream);

/* train_gpt2.cu, gpt2_backward.  Parameter gradients are ADDED into grads, so
 * consecutive backwards accumulate (gradient accumulation).  dloss scales the
 * loss gradient: dloss <= 0 means 1/(B*T), the page's fixed choice; with
 * accumulation over n micro-steps pass 1/(n*B*T).  The residual-stream
 * gradient is kept in fp32 and re-initialised by every backward.  Every
 * kernel is enqueued on hip_stream; in bf16 mode all weight and bias
 * gradients of the pass run in one launch after the input-gradient chain.
 * Errors: GPT2_E_ARG, GPT2_E_STATE (the last forward had no targets),
 * GPT2_E_HIP. */
int gpt2_backward(gpt2_ctx* ctx, float dloss, void* hip_stream);

/* train_gpt2.cu, gpt2_update / adamw_kernel3: for every parameter
 * m = b1 m + (1-b1) g, v = b2 v + (1-b2) g^2, p -= lr (m/(1-b1^t)) /
 * (sqrt(v/(1-b2^t)) + eps) + lr wd p, with one weight decay for all
 * parameters.  t is the 1-based step.  GPT2_BF16: the fp32 master weights are
 * updated and params receives their round-to-nearest-even bf16 value.
 * GPT2_BF16_SR (the page's path without master weights): the update starts
 * from the bf16 parameter and is evaluated in fp32 operation by operation as
 * the page writes it (the moment updates as fused multiply-adds, bias
 * corrections 1 - powf(b, t) in fp32, no other contraction); the result x is
 * rounded to bf16 stochastically: with r the low 16 bits of a 32-bit noise
 * value, x's low 16 bits are set to all ones if they exceed r (then rounded
 * to nearest-even, i.e. up) and cleared otherwise, so x rounds up with
 * probability (low 16 bits) / 65536.  The noise of parameter i is the
 * page's Get2dNoiseUint applied twice at (i mod 512, i div 512) -- the
 * page's 512-thread launch -- seeded first with s and then with the first
 * value: SquirrelNoise5(p, SquirrelNoise5(p, s)), p = (i mod 512) +
 * 198491317 (i div 512) mod 2^32.  s is drawn per call from the context's
 * xorshift64* state (the page's random_u32; initial state 13371337, see
 * gpt2_set_rng_state).
 * Errors: GPT2_E_ARG (t < 1), GPT2_E_HIP. */
int gpt2_adamw_update(gpt2_ctx* ctx, float lr, float beta1, float beta2, float eps,
                      float weight_decay, int t, void* hip_stream);

/* Sets (state != 0) and reads back (*old, if not NULL) the 64-bit xorshift64*
 * state from which GPT2_BF16_SR updates draw their noise seeds (gpt2_init
 * sets 13371337, the page's rng_state).  Errors: GPT2_E_ARG (NULL ctx). */
int gpt2_set_rng_state(gpt2_ctx* ctx, uint64_t state, uint64_t* old);

/* Synchronises hip_stream and reports device-side conditions raised since the
 * last call (GPT2_E_TOKEN for an out-of-range id), then clears them. */
int gpt2_check_device_error(gpt2_ctx* ctx, void* hip_stream);

/* Device pointer and element count of an internal activation tensor, for
 * inspection.  Tensor ids: GPT2_T_LOGITS [B*T, Vp] (logits after a forward
 * without targets; softmax - onehot after one with targets), GPT2_T_LNF
 * [B*T, C], GPT2_T_RESIDUAL [B*T, C] (final residual stream),
 * GPT2_T_DRESIDUAL [B*T, C] fp32 (residual gradient after a backward, i.e.
 * the gradient of the loss w.r.t. the encoder output), GPT2_T_ENCODED
 * [B*T, C] (token + position encoding).  Element type is the activation
 * type (fp32 or bf16) except where stated.
 * Errors: GPT2_E_ARG. */
enum { GPT2_T_LOGITS = 0, GPT2_T_LNF = 1, GPT2_T_RESIDUAL = 2, GPT2_T_DRESIDUAL = 3, GPT2_T_ENCODED = 4 };
int gpt2_act_tensor(gpt2_ctx* ctx, int which, void** d_ptr, size_t* count);

/* Timing hook (diagnostics): with n > 0, every later gpt2_forward records
 * d_start_events[i] just before and d_end_events[i] just after its classifier
 * product on its hip_stream, i = number of earlier forwards since this call,
 * modulo n; hipEventElapsedTime of a pair then gives that product's duration
 * inside the step.  The arrays hold n hipEvent_t handles each, owned by the
 * caller and kept valid while the hook is set; n = 0 removes the hook.
 * Errors: GPT2_E_ARG. */
int gpt2_set_classifier_events(gpt2_ctx* ctx, void* const* d_start_events, void* const* d_end_events, int n);

/* Timing hooks (diagnostics), one per launch point of the step: with n > 0
 * every later launch at `point` is bracketed by d_start_events[i] and
 * d_end_events[i] recorded on the call's hip_stream, i = number of earlier
 * launches at that point since this call, modulo n.  Launch order within one
 * call is fixed: GPT2_TP_LAYER_FWD brackets, for layers 0 .. L-1, the qkv,
 * attention-projection, fc and fc-projection products (4 per layer);
 * GPT2_TP_LAYER_DX the input-gradient products of layers L-1 .. 0 in the
 * order fc-projection (with the GELU backward), fc, attention projection,
 * qkv; GPT2_TP_LN_FWD the 2L + 1 forward LayerNorms (ln1, ln2 per layer,
 * then the final one); GPT2_TP_LN_BWD the final one's backward, then ln2,
 * ln1 of layers L-1 .. 0, then one launch that reduces the parameter
 * gradients of all of them (one per 128 LayerNorms);
 * GPT2_TP_ATTN_FWD / GPT2_TP_ATTN_BWD one per layer; GPT2_TP_WEIGHT_GRAD
 * the one launch of every weight gradient (bf16 contexts; fp32 contexts
 * bracket each weight-gradient product, classifier first, then the layers in
 * the order of GPT2_TP_LAYER_DX); GPT2_TP_CLASSIFIER_DX the classifier's
 * input gradient (with its K-split reduction); GPT2_TP_CE the fused softmax
 * cross-entropy; GPT2_TP_ENCODER_BWD the token/position embedding backward;
 * GPT2_TP_ADAMW the optimizer update.  Arrays of n hipEvent_t handles each,
 * owned by the caller and kept valid while the hook is set; n = 0 removes
 * it.  gpt2_set_classifier_events(ctx, ...) is the GPT2_TP_CLASSIFIER_FWD
 * hook.  Errors: GPT2_E_ARG (NULL context, point out of range, n < 0, n > 0
 * with a NULL array). */
enum { GPT2_TP_CLASSIFIER_FWD = 0, GPT2_TP_WEIGHT_GRAD = 1, GPT2_TP_CLASSIFIER_DX = 2, GPT2_TP_LAYER_FWD = 3,
       GPT2_TP_LAYER_DX = 4, GPT2_TP_ATTN_FWD = 5, GPT2_TP_ATTN_BWD = 6, GPT2_TP_LN_FWD = 7, GPT2_TP_LN_BWD = 8,
       GPT2_TP_CE = 9, GPT2_TP_ENCODER_BWD = 10, GPT2_TP_ADAMW = 11, GPT2_TP_COUNT = 12 };
int gpt2_set_timing_events(gpt2_ctx* ctx, int point, void* const* d_start_events, void* const* d_end_events, int n);

/* train_gpt2.cu, sample_softmax with the generation loop's indexing: for
 * every batch row b, sets d_tokens[b*T + t] to the token drawn from the
 * softmax over the first vocab_size logits of position t-1 of the last
 * gpt2_forward, which must have been made without targets (GPT2_E_STATE
 * otherwise).  The draw inverts the CDF with the coin d_coins[b] in [0, 1):
 * the smallest i with coin * Z < p_0 + ... + p_i, where p_j = exp(z_j - max z)
 * and Z = sum of all p_j (fp64 sums in a fixed order, so the draw is
 * deterministic), or vocab_size - 1 if there is none.  d_tokens: device int32 [B,T] (typically the inputs of the
 * next forward); d_coins: device fp32 [B]; 1 <= t < T.  Asynchronous on
 * hip_stream.  Errors: GPT2_E_ARG, GPT2_E_STATE, GPT2_E_ALIGN, GPT2_E_HIP. */
int gpt2_sample(gpt2_ctx* ctx, const float* d_coins, int32_t* d_tokens, int t, void* hip_stream);

/* The page's generation loop: for t = t_begin .. t_end - 1, a forward without
 * targets over all of d_tokens [B,T] (the page recomputes every position for
 * each new token), then gpt2_sample(ctx, d_coins + (t - t_begin) * B,
 * d_tokens, t).  d_coins: device fp32 [(t_end - t_begin) * B].  Positions
 * t_begin .. t_end - 1 of every row are overwritten; 1 <= t_begin <= t_end <= T.
 * Errors: as gpt2_forward and gpt2_sample. */
int gpt2_generate(gpt2_ctx* ctx, int32_t* d_tokens, const float* d_coins, int t_begin, int t_end, void* hip_stream);

/* Model files (train_gpt2.cu, gpt2_build_from_checkpoint): a header of 256
 * little-endian int32 -- [0] magic 20240326, [1] version (3: fp32 parameters;
 * 5: bf16 parameters, LayerNorm ones included), [2] max_seq_len,
 * [3] vocab_size, [4] num_layers, [5] num_heads, [6] channels,
 * [7] padded_vocab_size, the rest unused -- followed by the P parameters of
 * that config in gpt2_param_layout order (4 or 2 bytes each).  Host-only
 * calls: no device memory or stream is touched.
 *
 * gpt2_checkpoint_header reads the header into *cfg and the precision of the
 * stored parameters (GPT2_FP32 for version 3, GPT2_BF16 for 5) into
 * *file_precision.  Errors: GPT2_E_ARG (NULL argument), GPT2_E_FILE (the file
 * cannot be opened or holds less than a header, bad magic or version, or a
 * config that gpt2_query_sizes would reject for B = T = 1). */
int gpt2_checkpoint_header(const char* path, gpt2_config* cfg, int* file_precision);

/* Reads the P parameters into h_params (caller-owned host memory of count
 * fp32 values): version 3 values as stored, version 5 values widened exactly
 * from bf16.  count must equal P of the header's config.  The result is what
 * gpt2_init expects, after a host-to-device copy, in `params` (GPT2_FP32) or
 * `master` (GPT2_BF16).  Bytes after the parameters are ignored.
 * Errors: as gpt2_checkpoint_header; GPT2_E_ARG also for count != P;
 * GPT2_E_FILE also for a file shorter than the header plus P values. */
int gpt2_checkpoint_read(const char* path, float* h_params, size_t count);

/* Frees the context: its host state and its internal stream and events (no
 * device memory is owned).  Work already enqueued is not waited for: the
 * caller synchronises hip_stream first. */
int gpt2_free(gpt2_ctx* ctx);

const char* gpt2_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif
