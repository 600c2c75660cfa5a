/*
 * gpt2_ops.h -- op-level C ABI of the GPT-2 step library (gfx950).
 *
 * Each call launches exactly the kernels the training step uses for that
 * operation (same GEMM planner, operand layouts and epilogues: the linear
 * backward's dX reads the weight through the same transposed bf16 copy the
 * step keeps; gpt2_op_linear_plans / gpt2_step_gemm_plans report the kernel
 * configuration each launch gets), on caller-owned device buffers, so every
 * step of the path can be checked in isolation at its real shapes.  All
 * calls are asynchronous on
 * `stream` (a hipStream_t as void*, NULL = null stream) and return a gpt2
 * status (see gpt2.h); on failure nothing has been enqueued.
 *
 * dtype: GPT2_FP32 (0) -> every "T" buffer is float; GPT2_BF16 (1) -> every
 * "T" buffer is bfloat16 (uint16 storage).  Buffers marked f32 are always
 * float.  Row-major everywhere; "ld" arguments are row strides in elements.
 * Scratch: calls that need it take (workspace, workspace_bytes) and a
 * matching *_workspace_bytes() query; the workspace is caller-owned device
 * memory and is clobbered.
 */
#ifndef GPT2_OPS_H
#define GPT2_OPS_H

#include <stddef.h>
#include <stdint.h>

#include "gpt2.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Linear layer forward, y = x W^T + b (the block's QKV, attention-projection,
 * fc and fc-projection matmuls and the tied classifier; the kernel table of
 * "State of the Union [May 3, 2024]", section "Runtime, DRAM traffic,
 * instructions", attributes most of the step to these GEMMs and lists the
 * residual add and GELU as kernels of their own, fused here into the GEMM):
 *   x [M, K] T, W [N, K] T, b [N] T or NULL (no bias), y [M, N] T.
 *   residual [M, N] T or NULL:  y += residual   (the block's residual add)
 *   gelu_grad [M, N] T or NULL: with u = x W^T + b, y = GELU_tanh(u) and
 *                               gelu_grad = GELU_tanh'(u) (the fc layer; the
 *                               backward multiplies by the saved derivative)
 * residual and gelu_grad are exclusive and need b.  bf16: K % 8 == 0 and
 * 16-byte aligned x and W (reduction tails are zero-filled inside the
 * kernel). */
int gpt2_op_linear_forward(int dtype, int M, int N, int K, const void* x, const void* W,
                           const void* b, const void* residual, void* y, void* gelu_grad,
                           void* stream);

/* Linear layer backward for y = x W^T + b with upstream gradient dy [M, N]
 * (the kernel table's matmul backward and bias-gradient kernels, and the
 * GELU backward, which becomes the multiply below):
 *   dx [M, K] T      = dy W                  (skipped if dx == NULL)
 *       if gelu_grad [M, K] T != NULL:  dx = (dy W) * gelu_grad
 *   dW [N, K] f32    = dy^T x   (overwrite, or add if accumulate)
 *   db [N] f32       = sum over rows of dy (or NULL; fused into the dW pass)
 * dW == NULL skips the weight gradient.  bf16: M, N and K multiples of 8; dx
 * reads W through a transposed copy W^T [K, N] that this call writes at the
 * start of the workspace (the training step keeps the same copy of each
 * weight matrix, refreshed after every update).
 * workspace: at least gpt2_op_linear_backward_workspace_bytes() bytes of
 * device scratch (the transposed copy; fp32 partial sums of dW over row
 * blocks and, when N is long, of dx over N blocks, summed in a fixed order,
 * so results are deterministic); GPT2_E_OOM if it is smaller. */
size_t gpt2_op_linear_backward_workspace_bytes(int dtype, int M, int N, int K);
int gpt2_op_linear_backward(int dtype, int M, int N, int K, const void* dy, const void* x,
                            const void* W, const void* gelu_grad, void* dx, float* dW, float* db,
                            int accumulate, void* workspace, size_t workspace_bytes, void* stream);

/* ---- GEMM launch plans (host-only introspection, no HIP call) ------------
 * The configuration the library's GEMM kernel is launched with for one
 * product C[M, N] = sum over k of A(m, k) B(n, k): block tile, waves per
 * block, K-groups of waves, K-splits (fp32 partial sums reduced in a fixed
 * order) and whether the bias gradient is fused.  The fp32 parity kernel
 * reports a 64 x 64 tile, 4 waves, no split. */
enum {
  GPT2_EPI_STORE = 0,         /* C = sum                                      */
  GPT2_EPI_BIAS = 1,          /* C = sum + bias                               */
  GPT2_EPI_BIAS_RESIDUAL = 2, /* C = sum + bias + residual                    */
  GPT2_EPI_BIAS_RELU2 = 3,    /* C = relu(sum + bias)^2, U = 2 relu(sum + bias) */
  GPT2_EPI_WGRAD = 5,         /* fp32 weight gradient (+ fused bias gradient) */
  GPT2_EPI_BIAS_GELU = 6,     /* C = GELU(sum + bias), U = GELU'(sum + bias)  */
  GPT2_EPI_MUL = 7            /* C = sum * U                                  */
};

typedef struct gpt2_gemm_plan {
  char site[16];                /* timing-site name ("qkv", "fcproj_dx", ...), or
                                   "forward" / "dW" / "dX" for the op plans       */
  int32_t M, N, K;              /* product shape                                 */
  int32_t epilogue;             /* GPT2_EPI_*                                    */
  int32_t a_kmajor, b_kmajor;   /* operand layouts (1: k contiguous in memory)    */
  int32_t tile_m, tile_n;       /* block tile                                    */
  int32_t waves;                /* waves per block                               */
  int32_t k_groups;             /* groups of waves splitting each K step         */
  int32_t k_splits;             /* blocks splitting K (partial sums)             */
  int32_t bias_grad;            /* 1: bias gradient fused into the dW product     */
  int32_t fp8;                  /* 0 bf16 / fp32; 1 fp8 E4M3 x E4M3; 2 fp8 E5M2 x E4M3 */
} gpt2_gemm_plan;

/* Every GEMM one training step of cfg launches (forward with targets, then
 * backward; one entry per launch, in launch order): *count is set to their
 * number and the first min(count, max_plans) are written to out. */
int gpt2_step_gemm_plans(const gpt2_config* cfg, gpt2_gemm_plan* out, int max_plans, int* count);

/* The three GEMMs of gpt2_op_linear_forward and gpt2_op_linear_backward for
 * these shapes and options: out[0] the forward, out[1] dW, out[2] dX. */
int gpt2_op_linear_plans(int dtype, int M, int N, int K, int has_bias, int has_residual, int has_gelu,
                         int has_db, gpt2_gemm_plan out[3]);

/* ---- FP8 products ("NanoGPT (124M) in 90 seconds", section "How it works",
 * item "Precision & Hardware"; the training step's GPT2_BF16_FP8 mode) ------
 * Per-tensor scaling from the tensor's absolute maximum: inv = FMAX / amax
 * and s = amax / FMAX in fp32 (1 and 1 for amax = 0), FMAX = 448 (fmt 0, OCP
 * E4M3) or 57344 (fmt 1, OCP E5M2); code = fp8(fp32(x * inv)), round to
 * nearest even with subnormals. */

/* scale [4] f32 (device, 16-byte aligned) = {amax, inv, s, 0}; q [R, C] and
 * / or qt [C, R] (either may be NULL) receive the codes of x [R, C] (in_dtype
 * GPT2_FP32 or GPT2_BF16), row-major and transposed.  C % 8 == 0, R % 16 ==
 * 0 when qt.  workspace: gpt2_op_fp8_quantize_workspace_bytes() bytes. */
size_t gpt2_op_fp8_quantize_workspace_bytes(void);
int gpt2_op_fp8_quantize(int in_dtype, int fmt, int R, int C, const void* x, float* scale, uint8_t* q,
                         uint8_t* qt, void* workspace, size_t workspace_bytes, void* stream);

/* The step's fp8 linear layer on bf16 buffers (same arguments and epilogues
 * as gpt2_op_linear_forward / _backward in GPT2_BF16): x and W are quantised
 * to E4M3 and dy to E5M2 per tensor inside the call (into the workspace),
 * y = s_x s_w Q(x) Q(W)^T (+ epilogue), dx = s_dy s_w Q(dy) Q(W),
 * dW = s_dy s_x Q(dy)^T Q(x) (fp32 accumulation), db = the sum over rows of
 * the unquantised dy.  M, N, K multiples of 16 (N, K for the forward). */
size_t gpt2_op_linear_fp8_workspace_bytes(int M, int N, int K);
int gpt2_op_linear_fp8_forward(int M, int N, int K, const void* x, const void* W, const void* b,
                               const void* residual, void* y, void* gelu_grad, void* workspace,
                               size_t workspace_bytes, void* stream);
int gpt2_op_linear_fp8_backward(int M, int N, int K, const void* dy, const void* x, const void* W,
                                const void* gelu_grad, void* dx, float* dW, float* db, int accumulate,
                                void* workspace, size_t workspace_bytes, void* stream);

/* LayerNorm forward over rows of C (eps 1e-5, biased variance):
 *   x [N, C] T, w, b [C] T -> y [N, C] T, mean [N] f32, rstd [N] f32. C % 8 == 0. */
int gpt2_op_layernorm_forward(int dtype, int N, int C, const void* x, const void* w, const void* b,
                              void* y, float* mean, float* rstd, void* stream);

/* LayerNorm backward: dres [N, C] f32 += dx (or = dx if dres_overwrite);
 * dres_copy [N, C] T (optional) = the new dres; dw, db [C] f32 = (or += if
 * accumulate) sum over rows of dy * xhat and dy. */
size_t gpt2_op_layernorm_backward_workspace_bytes(int N, int C);
int gpt2_op_layernorm_backward(int dtype, int N, int C, const void* dy, const void* x, const void* w,
                               const float* mean, const float* rstd, float* dres, int dres_overwrite,
                               void* dres_copy, float* dw, float* db, int accumulate, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Causal attention forward (exact; flash-style, no T x T buffer in memory):
 * qkv [B, T, 3C] T with q | k | v column blocks, head h at h*hd in each;
 * out [B, T, C] T; lse [B, H, T] f32 = log-sum-exp of each scaled score row. */
int gpt2_op_attention_forward(int dtype, int B, int T, int H, int hd, const void* qkv, void* out,
                              float* lse, void* stream);

/* Causal attention backward: dout [B, T, C] T -> dqkv [B, T, 3C] T (overwritten). */
size_t gpt2_op_attention_backward_workspace_bytes(int B, int T, int H, int hd);
int gpt2_op_attention_backward(int dtype, int B, int T, int H, int hd, const void* qkv,
                               const void* out, const void* dout, const float* lse, void* dqkv,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free attention backward, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): gpt2_op_attention_backward with the same kernels
 * and results, but its scratch (rowsum(dO * O) and the base-2 log-sum-exp,
 * two floats per (b, h, t) row) lives in a library-owned device array of
 * GPT2_NOALLOC_SCRATCH_BYTES per GPU (held from the first call on a device
 * until the process ends) instead of a workspace argument.  Shapes whose
 * scratch exceeds that (B*H*T above about one million rows) are rejected with
 * GPT2_E_INVALID_ARG before anything is enqueued.  The call allocates nothing
 * (no hipMalloc, no allocating library routine).  Every call on one GPU uses
 * that GPU's single array: calls that overlap on one GPU (other streams or
 * threads) race on it and must be serialised by the caller.  Every scratch
 * element a call reads is written earlier in the same call, so nothing needs
 * clearing between calls. */
#define GPT2_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int gpt2_op_attention_backward_noalloc(int dtype, int B, int T, int H, int hd, const void* qkv,
                                       const void* out, const void* dout, const float* lse, void* dqkv,
                                       void* stream);

/* Fused softmax cross-entropy in place over logits [N, Vp] T (columns >= V
 * are padding, masked to -inf):  losses [N] f32 = logsumexp - logit at the
 * label; logits <- (softmax - onehot(label)) * dscale, 0 in padded columns.
 * labels [N] int32 in [0, V). */
int gpt2_op_softmax_xent(int dtype, int N, int V, int Vp, void* logits, const int32_t* labels,
                         float* losses, float dscale, void* stream);

/* The stand-alone tied classifier at one position batch (hidden [N, C] T,
 * wte [Vp, C] T, labels [N]):  logits = hidden wte^T -> fused softmax-CE with
 * dscale = 1/N written into logits -> d_hidden [N, C] T = dlogits wte,
 * d_wte [Vp, C] f32 = dlogits^T hidden (overwrite).  losses [N] f32. */
size_t gpt2_op_classifier_workspace_bytes(int dtype, int N, int C, int Vp);
int gpt2_op_classifier_fwd_bwd(int dtype, int N, int C, int V, int Vp, const void* hidden,
                               const void* wte, const int32_t* labels, float* losses, void* logits,
                               void* d_hidden, float* d_wte, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Encoder forward: out [B, T, C] T = wte[tokens] + wpe[0:T]. */
int gpt2_op_encoder_forward(int dtype, int B, int T, int C, int V, const int32_t* tokens,
                            const void* wte, const void* wpe, void* out, void* stream);

/* Encoder backward: dwte [V.., C] f32 += scatter of dx0 [B, T, C] f32 rows by
 * token (deterministic order); dwpe [T, C] f32 = (or += if accumulate_wpe)
 * sum over the batch.  B*T <= 4194304. */
size_t gpt2_op_encoder_backward_workspace_bytes(int B, int T, int C);
int gpt2_op_encoder_backward(int B, int T, int C, int V, const int32_t* tokens, const float* dx0,
                             float* dwte, float* dwpe, int accumulate_wpe, void* workspace,
                             size_t workspace_bytes, void* stream);

/* AdamW over n fp32 parameters (16-byte aligned buffers); param_bf16 (n,
 * bfloat16) receives the rounded copy if not NULL.  t >= 1. */
int gpt2_op_adamw(int64_t n, float* master, const float* grad, float* m, float* v, void* param_bf16,
                  float lr, float beta1, float beta2, float eps, float weight_decay, int32_t t,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_OPS_H */
