/*
 * gpt2.h -- C ABI of the GPT-2 training-step library for MI355X (gfx950).
 *
 * One training step is: token + position encoder, L pre-LayerNorm blocks
 * (causal multi-head attention, GELU-tanh MLP, residual adds), final
 * LayerNorm, a classifier tied to the token table with softmax
 * cross-entropy, the full backward pass, and AdamW.  The page
 * "State of the Union [May 3, 2024]" (karpathy/llm.c discussion #344)
 * describes this step: its opening bullet list names bf16 mixed precision
 * with an fp32 master copy of the parameters, a fused classifier that never
 * materialises normalised logits and evaluates the loss only at the label's
 * index, and flash attention; its kernel table (section "Runtime, DRAM
 * traffic, instructions") lists the kernels of the step; its "Fine print"
 * section pads the vocabulary 50257 -> 50304 (a multiple of 64) and requires
 * the padded logits to be masked to -inf.
 *
 * Conventions
 *   - Every function is extern "C"; no C++ type or exception crosses it (a
 *     C++ exception inside the library becomes GPT2_E_OOM for a failed host
 *     allocation, GPT2_E_INTERNAL otherwise).
 *   - Pointers named d_* are device pointers (HIP global memory of the
 *     current device); pointers named host_* are host memory.
 *   - Every int-returning function returns a status: GPT2_OK (0) or one of
 *     GPT2_E_*; gpt2_last_error() returns a thread-local text for the last
 *     failure on the calling thread (errors of host-only calls have no model
 *     to attach to, hence no model argument).
 *   - "stream" arguments are hipStream_t values passed as void*; NULL means
 *     the null stream.  Work is enqueued on that stream; only the calls that
 *     say so synchronise.  A device buffer handed to a call that returns
 *     without synchronising must stay valid and unchanged until the stream
 *     has executed the work that reads it.
 *
 * Parameter layout (one flat array, this order, weights stored [out, in]
 * row-major so that y = x W^T + b; QKV output columns ordered [q | k | v],
 * head h owning columns h*hd .. h*hd + hd - 1 inside each):
 *   wte[Vp,C] wpe[maxT,C] ln1w[L,C] ln1b[L,C] qkvw[L,3C,C] qkvb[L,3C]
 *   attprojw[L,C,C] attprojb[L,C] ln2w[L,C] ln2b[L,C] fcw[L,4C,C] fcb[L,4C]
 *   fcprojw[L,C,4C] fcprojb[L,C] lnfw[C] lnfb[C]
 * Rows V..Vp-1 of wte are padding: initialised to zero, their logits are
 * masked to -inf, so their gradient is exactly zero and AdamW keeps them 0.
 */
#ifndef GPT2_H
#define GPT2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  GPT2_OK = 0,
  GPT2_E_INVALID_ARG = 1, /* null pointer, bad config, unsupported shape */
  GPT2_E_STATE = 2,       /* calls out of order (e.g. backward before forward with targets) */
  GPT2_E_OOM = 3,         /* device or host allocation failed, or workspace too small */
  GPT2_E_HIP = 4,         /* a HIP runtime call failed; text in gpt2_last_error() */
  GPT2_E_INTERNAL = 5     /* an unexpected C++ exception inside the library */
};

enum {
  GPT2_FP32 = 0,     /* every tensor fp32 (parity mode) */
  GPT2_BF16 = 1,     /* bf16 weights copy, activations and activation gradients;
                        fp32 master weights, parameter gradients, AdamW moments,
                        LayerNorm statistics, softmax statistics, residual-stream
                        gradient and every accumulator */
  GPT2_BF16_FP8 = 2  /* GPT2_BF16, with the products of the QKV projection,
                        the MLP (fc, fc-proj) and the head (logits) forward and
                        backward in FP8 ("NanoGPT (124M) in 90 seconds",
                        section "How it works", item "Precision & Hardware"):
                        OCP E4M3 weights (quantised from the fp32 master after
                        every update) and activations, OCP E5M2 output
                        gradients, per-tensor scales from each tensor's
                        absolute maximum (inv = FMAX / amax, s = amax / FMAX in
                        fp32), round to nearest even, fp32 accumulation, the
                        sums multiplied by s_a s_b; bias gradients from the
                        unquantised gradient */
};

/* Architecture variants of the block ("NanoGPT (124M) in 90 seconds",
 * section "How it works", item "Architecture Changes": rotary embeddings,
 * QK-Norm and ReLU^2; the page gives no formulas, these are the plainest
 * readings).  0 is GPT-2 as published; the bits combine.  The parameter
 * layout is the same for every combination. */
enum {
  GPT2_ARCH_RELU2 = 1,   /* MLP activation relu(u)^2 instead of GELU-tanh              */
  GPT2_ARCH_QK_NORM = 2, /* q and k of every head divided by sqrt(mean(x^2) + 1e-6)
                            over the head dimension (no gain; scale 1/sqrt(hd) kept)   */
  GPT2_ARCH_ROPE = 4     /* rotary embedding of q and k (after QK-Norm): at position t
                            the pair (i, i + hd/2) rotated by t * 10000^(-2i/hd); the
                            position table wpe is then not used (zero gradient)        */
};

typedef struct gpt2_config {
  int32_t vocab_size;        /* V, e.g. 50257                                  */
  int32_t padded_vocab_size; /* Vp >= V, multiple of 64, e.g. 50304            */
  int32_t max_seq_len;       /* maxT, rows of wpe                              */
  int32_t num_layers;        /* L >= 0                                         */
  int32_t num_heads;         /* H, C % H == 0                                  */
  int32_t channels;          /* C, multiple of 64                              */
  int32_t batch_size;        /* B: activation buffers are sized for B x T      */
  int32_t seq_len;           /* T <= maxT; B*T a multiple of 64, <= 4194304;
                                 bf16 modes: B*T*Vp*2 < 4 GiB (B*T <= 42688 at
                                 Vp = 50304: the classifier products address the
                                 logits with 32-bit offsets)                    */
  int32_t dtype;             /* GPT2_FP32, GPT2_BF16 or GPT2_BF16_FP8           */
  int32_t arch_flags;        /* GPT2_ARCH_* bits, 0 for GPT-2                  */
} gpt2_config;

typedef struct gpt2_model gpt2_model; /* opaque */

/* ---- host-only queries (no HIP call; usable without a GPU) -------------- */

/* Checks every field; returns GPT2_OK or GPT2_E_INVALID_ARG with a reason in
 * gpt2_last_error().  Head dimension C/H must be 16, 32, 64 or 128. */
int gpt2_validate_config(const gpt2_config* cfg);

/* Number of parameters; padded != 0 counts the Vp-row token table (the
 * "Fine print" padding of "State of the Union [May 3, 2024]"), padded == 0
 * the V-row one.  Returns -1 for an invalid config. */
int64_t gpt2_num_parameters(const gpt2_config* cfg, int padded);

/* Number of parameter tensors (16). */
int gpt2_num_param_tensors(void);

/* Tensor i of the flat layout: *name (static string), *offset (elements from
 * the start of the flat array), shape[0..2] (unused trailing dims are 1; the
 * per-layer tensors are 3-D [L, out, in], and int64 so no product overflows)
 * and *ndim.  Returns GPT2_E_INVALID_ARG for i out of range or a bad config. */
int gpt2_param_info(const gpt2_config* cfg, int i, const char** name, int64_t* offset,
                    int64_t shape[3], int32_t* ndim);

/* Device bytes gpt2_create needs for all model state (parameters, master,
 * gradients, AdamW moments, activations, scratch).  0 for a bad config or a
 * failed host allocation (reason in gpt2_last_error()). */
size_t gpt2_workspace_bytes(const gpt2_config* cfg);

/* Status code -> static text. */
const char* gpt2_status_string(int status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* gpt2_last_error(void);

/* Test hook for the error paths: the next n host allocations the library
 * makes for its own bookkeeping (arena plan, timing events) fail as if the
 * host were out of memory; n = 0 turns it off.  Always GPT2_OK. */
int gpt2_test_fail_host_allocations(int n);

/* ---- model lifecycle and the training step ------------------------------ */

/* Creates a model on the current HIP device and initialises the parameters
 * from seed (GPT-2 scheme: N(0, 0.02); the two residual projections
 * N(0, 0.02/sqrt(2L)); biases 0; LayerNorm gains 1; padded wte rows 0),
 * drawn with the counter-based SplitMix64 + Box-Muller generator
 * (element e of tensor i uses stream outputs 2c and 2c+1, c = (i << 40) | e).
 * The page lists random initialisation in C among the pending pieces
 * ("State of the Union [May 3, 2024]", paragraph "Functional").
 * workspace: NULL -> the library allocates gpt2_workspace_bytes(cfg) bytes
 * and frees them in gpt2_destroy; otherwise a caller-owned device buffer of
 * at least that many bytes, 256-byte aligned, that outlives the model.
 * stream: the stream every later call of this model enqueues on.
 * Synchronises the stream before returning. */
int gpt2_create(const gpt2_config* cfg, uint64_t seed, void* stream, void* workspace,
                size_t workspace_bytes, gpt2_model** out);

/* Forward pass ("State of the Union [May 3, 2024]", kernel table: encoder,
 * per block layernorm -> QKV matmul -> attention -> projection + residual ->
 * layernorm -> fc + GELU -> projection + residual, final layernorm, logits,
 * fused classifier) over d_tokens [B, T] int32 (ids in [0, V)).  With
 * d_targets (int32 [B, T], ids in [0, V)) it also evaluates softmax
 * cross-entropy (the page's fused classifier: loss read at the label's index,
 * padded columns masked), writes the per-position losses, stores dlogits in
 * place of the logits (ready for gpt2_backward) and, if mean_loss != NULL,
 * writes the mean loss to *mean_loss (host) and synchronises the stream, after
 * which d_tokens and d_targets may be reused.  With mean_loss == NULL (or
 * d_targets == NULL) nothing waits: the ids are copied into the model's
 * arena and d_targets is read by the classifier kernel, both in stream
 * order, so both buffers must stay valid and unchanged until the stream has
 * passed this forward; gpt2_get_mean_loss reads the loss later.  With
 * d_targets == NULL it stops at the logits and does not touch *mean_loss.
 * Token ids outside [0, V) are undefined behaviour. */
int gpt2_forward(gpt2_model* m, const int32_t* d_tokens, const int32_t* d_targets,
                 float* mean_loss);

/* gpt2_forward, except that the gradients the next backward computes are
 * those of loss_scale x (the mean loss); *mean_loss still reports the
 * unscaled mean.  For gradient accumulation over k micro-batches (pending
 * work on "State of the Union [May 3, 2024]", paragraph "Functional") pass
 * loss_scale = 1/k to each: the accumulated gradient is then that of the
 * mean loss over all k micro-batches (the mean of their gradients).
 * loss_scale must be finite (GPT2_E_INVALID_ARG otherwise). */
int gpt2_forward_scaled(gpt2_model* m, const int32_t* d_tokens, const int32_t* d_targets,
                        float loss_scale, float* mean_loss);

/* Backward pass of the mean loss of the last forward-with-targets (the
 * backward kernels of the kernel table of "State of the Union [May 3, 2024]":
 * matmul dX/dW with the bias gradient, GELU backward, layernorm backward,
 * attention backward, encoder backward).  Parameter gradients (fp32) are
 * overwritten.  GPT2_E_STATE if the last forward had no targets.  Does not
 * synchronise. */
int gpt2_backward(gpt2_model* m);

/* Gradient accumulation ("State of the Union [May 3, 2024]", paragraph
 * "Functional"): the same backward, with every parameter gradient added to
 * the one held (from gpt2_backward and any accumulating backwards since the
 * last update) instead of overwriting it.  Summation order is fixed, so the
 * result is deterministic.  GPT2_E_STATE if the last forward had no targets
 * or no gradient is held. */
int gpt2_backward_accumulate(gpt2_model* m);

/* One AdamW update of every parameter (fp32 master; the adamw kernel of the
 * kernel table of "State of the Union [May 3, 2024]"), then refreshes the
 * bf16 copy used by the forward (the page's copy-and-cast, folded in):
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   theta -= lr (m/(1-b1^t) / (sqrt(v/(1-b2^t)) + eps) + wd theta).
 * Requires t >= 1 and a completed backward (GPT2_E_STATE otherwise).  Does not
 * synchronise. */
int gpt2_adamw_step(gpt2_model* m, float lr, float beta1, float beta2, float eps,
                    float weight_decay, int32_t t);

/* gpt2_adamw_step with global-norm gradient clipping (pending work on "State
 * of the Union [May 3, 2024]", paragraph "Functional").  n = the L2 norm of
 * all parameter gradients taken as one vector (fp32 partial sums per block,
 * added in a fixed order in fp64).  If max_grad_norm > 0 and
 * n > max_grad_norm, every gradient enters the update multiplied by
 * max_grad_norm / n (the stored gradients are left as they are);
 * max_grad_norm <= 0 disables clipping.  If grad_norm != NULL, n (before
 * clipping) is written there (host) and the stream is synchronised;
 * otherwise nothing waits on the host.  The norm and the factor are computed
 * on the device, so clipping needs no host round trip. */
int gpt2_adamw_step_clipped(gpt2_model* m, float lr, float beta1, float beta2, float eps,
                            float weight_decay, int32_t t, float max_grad_norm, float* grad_norm);

/* ---- the whole step as one HIP graph ------------------------------------ */
/* "NanoGPT (124M) in 90 seconds", section "How it works", item "Precision &
 * Hardware", names graph capture of the training step. */

/* Captures one training step -- forward with targets (loss scale 1, no
 * readback), backward, AdamW without clipping and the refresh of the bf16
 * weight copies, including the side-stream work of the encoder backward --
 * into a HIP graph held by the model (replacing any earlier one).  Nothing
 * runs during the capture.  The graph reads the token ids and targets from
 * d_tokens and d_targets at every replay: the caller refills those buffers
 * (in stream order) before each gpt2_graph_step, and they must outlive the
 * graph.  Needs a model stream other than the null stream and no timing site
 * enabled (GPT2_E_INVALID_ARG / GPT2_E_STATE otherwise). */
int gpt2_graph_capture(gpt2_model* m, const int32_t* d_tokens, const int32_t* d_targets);

/* Replays the captured step with these AdamW hyperparameters (written to the
 * device ahead of the replay, in stream order; same update as
 * gpt2_adamw_step).  The result is bit-identical to gpt2_forward +
 * gpt2_backward + gpt2_adamw_step on the same inputs.  If mean_loss != NULL
 * the step's mean loss is written there (host) and the stream synchronised.
 * GPT2_E_STATE without a captured graph or for t < 1. */
int gpt2_graph_step(gpt2_model* m, float lr, float beta1, float beta2, float eps,
                    float weight_decay, int32_t t, float* mean_loss);

/* Releases the model (and the workspace if the library allocated it, and any
 * captured graph).  Synchronises the model's stream first.  NULL is a no-op;
 * never fails. */
void gpt2_destroy(gpt2_model* m);

/* ---- state access (synchronous copies through host memory) -------------- */

/* Mean loss of the last forward with targets (one float). */
int gpt2_get_mean_loss(gpt2_model* m, float* host_out);

/* fp32 master parameters in the flat layout, num_parameters(cfg, 1) floats. */
int gpt2_get_params(gpt2_model* m, float* host_out);
/* Sets the fp32 master parameters (flat layout), refreshes the bf16 copy and
 * clears the AdamW moments. */
int gpt2_set_params(gpt2_model* m, const float* host_in);
/* fp32 parameter gradients of the last backward, flat layout. */
int gpt2_get_grads(gpt2_model* m, float* host_out);
/* AdamW first and second moments, flat layout (either pointer may be NULL). */
int gpt2_get_adam_state(gpt2_model* m, float* host_m, float* host_v);
/* Per-position losses [B*T] of the last forward with targets. */
int gpt2_get_token_losses(gpt2_model* m, float* host_out);
/* Logits [B*T, Vp] of the last forward WITHOUT targets, converted to fp32
 * (after a forward with targets the buffer holds dlogits instead; this call
 * returns whichever is there). */
int gpt2_get_logits(gpt2_model* m, float* host_out);

/* ---- timing hooks ------------------------------------------------------- */

/* Enables (1) or disables (0) HIP-event timing of one site of the step.
 * Every site times exactly one kernel per launch (the main kernel of the
 * operation there; split-K reductions and column sums are not included):
 * 0 QKV fwd, 1 attn-proj fwd, 2 fc fwd, 3 fc-proj fwd, 4 logits fwd,
 * 5 fc-proj dX, 6 fc-proj dW, 7 fc dX, 8 fc dW, 9 attn-proj dX,
 * 10 attn-proj dW, 11 QKV dX, 12 QKV dW, 13 classifier dX, 14 classifier dW,
 * 15 attention fwd, 16 attention bwd dK/dV, 17 attention bwd dQ,
 * 18 attention bwd rowsum(dO*O), 19 softmax-CE, 20 LayerNorm fwd,
 * 21 LayerNorm bwd, 22 encoder fwd, 23 AdamW, 24 transposed bf16 weight
 * copies (written after each AdamW step for the dX products), 25 gradient
 * norm (partial sums of squares; gpt2_adamw_step_clipped), 26 QK-Norm /
 * rotary transform of q and k, 27 its backward (GPT2_ARCH_QK_NORM or
 * GPT2_ARCH_ROPE), 28 fp8 quantisation (the codes of one operand;
 * GPT2_BF16_FP8).  Events are recorded on the model's stream immediately
 * around that kernel.  Sites are valid in [0, 29); others give
 * GPT2_E_INVALID_ARG. */
int gpt2_timing_enable(gpt2_model* m, int site, int enable);
/* Total elapsed milliseconds and launch count recorded for a site since it
 * was enabled (synchronises the stream), with the algorithmic FLOPs and HBM
 * bytes of one launch (the attention dK/dV site is credited with the dV, dP
 * and dK products, the dQ site with dQ; recomputed products are not
 * counted). */
int gpt2_timing_read(gpt2_model* m, int site, double* total_ms, int64_t* launches,
                     double* flops_per_launch, double* bytes_per_launch);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_H */
