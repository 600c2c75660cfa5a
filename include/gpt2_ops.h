/*
 * gpt2_ops.h -- op-level C ABI of the GPT-2 step library (gfx950).
 *
 * Each call launches exactly the kernels the training step uses for that
 * operation, on caller-owned device buffers, so every step of the path can be
 * checked in isolation at its real shapes.  All calls are asynchronous on
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

#ifdef __cplusplus
extern "C" {
#endif

/* Linear layer forward, y = x W^T + b (the block's QKV, attention-projection,
 * fc and fc-projection matmuls and the tied classifier; the kernel table of
 * "State of the Union [May 3, 2024]", section "Runtime, DRAM traffic,
 * instructions", attributes most of the step to these GEMMs):
 *   x [M, K] T, W [N, K] T, b [N] T or NULL (no bias), y [M, N] T.
 *   residual [M, N] T or NULL:  y += residual   (the block's residual add)
 *   gelu_out [M, N] T or NULL:  y holds u = xW^T + b and gelu_out = GELU_tanh(u)
 * residual and gelu_out are exclusive.  bf16: K % 8 == 0 and 16-byte aligned
 * x and W (reduction tails are zero-filled inside the kernel). */
int gpt2_op_linear_forward(int dtype, int M, int N, int K, const void* x, const void* W,
                           const void* b, const void* residual, void* y, void* gelu_out,
                           void* stream);

/* Linear layer backward for y = x W^T + b with upstream gradient dy [M, N]:
 *   dx [M, K] T      = dy W                  (skipped if dx == NULL)
 *       if gelu_u [M, K] T != NULL:  dx = (dy W) * GELU_tanh'(gelu_u)
 *   dW [N, K] f32    = dy^T x   (overwrite, or add if accumulate)
 *   db [N] f32       = sum over rows of dy (or NULL; fused into the dW pass)
 * dW == NULL skips the weight gradient.  bf16: M, N and K multiples of 8.
 * workspace: at least gpt2_op_linear_backward_workspace_bytes() bytes of
 * device scratch (fp32 partial sums of dW over row blocks and, when N is
 * long, of dx over N blocks; summed in a fixed order, so results are
 * deterministic); GPT2_E_OOM if it is smaller. */
size_t gpt2_op_linear_backward_workspace_bytes(int dtype, int M, int N, int K);
int gpt2_op_linear_backward(int dtype, int M, int N, int K, const void* dy, const void* x,
                            const void* W, const void* gelu_u, void* dx, float* dW, float* db,
                            int accumulate, void* workspace, size_t workspace_bytes, void* stream);

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
 * sum over the batch.  B*T <= 32768, V <= 65536. */
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
