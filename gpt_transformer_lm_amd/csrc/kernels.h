// Launchers of the GPT-2 step kernels (internal C++ interface of the library).
// Every launcher enqueues on `stream` and returns a gpt2 status code.
#pragma once

#include "common.h"

namespace gpt2k {

enum DType { F32 = 0, BF16 = 1 };

// ------------------------------------------------------------------ timing marks
// When armed by the caller (per host thread), a launcher records
// kernel_marks()[i].begin / .end on its stream immediately before and after
// its i-th main kernel, so that one event pair brackets exactly one kernel.
// Null events are skipped.  Used only for timing.
struct KernelMark {
  hipEvent_t begin, end;
};
constexpr int kMaxMarks = 3;
KernelMark* kernel_marks();
inline void mark_begin(int i, hipStream_t s) {
  if (hipEvent_t e = kernel_marks()[i].begin) (void)hipEventRecord(e, s);
}
inline void mark_end(int i, hipStream_t s) {
  if (hipEvent_t e = kernel_marks()[i].end) (void)hipEventRecord(e, s);
}

// ------------------------------------------------------------------ GEMM
//
// C[M, N] = sum_k A(m, k) * B(n, k)
//   A(m, k) = A[m * lda + k]  (a_kmajor)   or  A[k * lda + m]  (!a_kmajor)
//   B(n, k) = B[n * ldb + k]  (b_kmajor)   or  B[k * ldb + n]  (!b_kmajor)
// Epilogues (element (m, n), v = the fp32 sum):
//   STORE        C = v
//   BIAS         C = v + bias[n]
//   BIAS_RES     C = v + bias[n] + R[m * ld_aux + n]
//   WGRAD        fp32 result into out32[m * N + n] (overwrite, or add if
//                accumulate), and if bias_grad32 != null also
//                bias_grad32[m] = sum_k A(m, k) (A must be !a_kmajor).
//                Split over K into partial sums that a second kernel reduces
//                in a fixed order (deterministic).
//   BIAS_GELU_D  C = gelu_tanh(v + bias[n]);  U[m * ldc + n] = gelu_tanh'(v + bias[n])
//   BIAS_RELU2_D C = relu(v + bias[n])^2;     U[m * ldc + n] = 2 relu(v + bias[n])
//   MUL          C = v * U[m * ld_aux + n]
//   (the step stores the activation's derivative in the forward, so the
//   backward epilogue of the fc-proj dX is one multiply)
enum Epi { EPI_STORE = 0, EPI_BIAS = 1, EPI_BIAS_RES = 2, EPI_BIAS_RELU2_D = 3, EPI_WGRAD = 5, EPI_BIAS_GELU_D = 6,
           EPI_MUL = 7 };

struct GemmDesc {
  int dtype;            // F32 or BF16 (type of A, B, C, bias, R, U)
  bool a_kmajor, b_kmajor;
  int M, N, K;
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  int epi;
  void* C; int64_t ldc;
  const void* bias;
  const void* aux_in; int64_t ld_aux;   // R (BIAS_RES) or U (MUL)
  void* aux_out;                        // U (BIAS_GELU_D)
  float* out32;                         // WGRAD result [M, N]
  float* bias_grad32;                   // WGRAD bias gradient [M] (optional)
  bool accumulate;                      // WGRAD: add into out32 / bias_grad32
  void* workspace; size_t workspace_bytes;
  // FP8 product (dtype BF16 for C, bias, R and U): 0 off; 1 A and B E4M3
  // (forward); 2 A E5M2, B E4M3 (backward, A the gradient).  A and B are then
  // byte arrays of fp8 codes, both k-major, K and the row strides multiples of
  // 16; scale_a / scale_b (device, one float each) multiply the sums.
  int fp8;
  const float* scale_a;
  const float* scale_b;
  // fp8 products with epilogue BIAS_GELU_D, BIAS_RELU2_D or MUL (unsplit, C
  // rows 16-byte aligned): also the maximum |C| (as stored) into the slots
  // amax (kAmaxWays x kAmaxStride floats, zero beforehand; amax_atomic_bf16),
  // for the quantisation of C that follows.  NULL: not taken.
  float* amax;
};

// Kernel configuration gemm() launches for a descriptor (host-only): block
// tile, waves per block, K-groups, K-splits and whether the bias gradient is
// fused (the fp32 parity kernel reports 64 x 64, 4 waves, no split).
struct GemmLaunchInfo {
  int tile_m, tile_n, waves, kgroups, splits;
  bool bias_grad;
};
GemmLaunchInfo gemm_launch_info(const GemmDesc& d);

// Device bytes of scratch a GEMM with this descriptor needs (WGRAD and split
// plain stores).
size_t gemm_workspace_bytes(int dtype, int epi, int M, int N, int K, bool a_kmajor, bool b_kmajor, int fp8 = 0);
int gemm(const GemmDesc& d, hipStream_t stream);

// ------------------------------------------------------------------ LayerNorm
// y = (x - mean) * rstd * w + b per row of C; mean, rstd fp32 [N].  With
// amax (bf16 only; kAmaxWays x kAmaxStride floats, zero beforehand) also the
// maximum |y| (as stored) into those slots (amax_atomic_bf16), for
// fp8_quantize.
int layernorm_forward(int dtype, int N, int C, const void* x, const void* w, const void* b,
                      void* y, float* mean, float* rstd, hipStream_t stream, float* amax = nullptr);
// dres[N, C] (fp32) += dx; dres_copy (dtype, optional) = new dres;
// dw, db (fp32 [C]) = (or +=, if accumulate) column sums.  If dres_overwrite,
// dres is written (= dx) instead of accumulated.  With amax (bf16 with
// dres_copy only) also the maximum |dres_copy| into those slots, as in the
// forward.
size_t layernorm_backward_workspace_bytes(int N, int C);
int layernorm_backward(int dtype, int N, int C, const void* dy, const void* x, const void* w,
                       const float* mean, const float* rstd, float* dres, bool dres_overwrite,
                       void* dres_copy, float* dw, float* db, bool accumulate, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, float* amax = nullptr);

// ------------------------------------------------------------------ attention
// qkv [B, T, 3C] -> out [B, T, C], lse [B, H, T] fp32.
int attention_forward(int dtype, int B, int T, int H, int hd, const void* qkv, void* out,
                      float* lse, hipStream_t stream);
size_t attention_backward_workspace_bytes(int B, int T, int H, int hd);
// Matrix-core kernels (attention_mfma.hip) for bf16 with head dim 64; the
// launchers above dispatch to them when attention_mfma_supported().
bool attention_mfma_supported(int dtype, int hd);
int attention_forward_mfma(int B, int T, int H, const void* qkv, void* out, float* lse, hipStream_t stream);
// lse2 = lse * log2(e) (base-2 log-sum-exp) and D = rowsum(dO * O), both
// [B, H, T] scratch, are computed by the dQ kernel and read by the dK / dV one.
int attention_backward_mfma(int B, int T, int H, const void* qkv, const void* out, const void* dout,
                            const float* lse, float* lse2, float* D, void* dqkv, hipStream_t stream,
                            float* amax = nullptr);
// amax (only where attention_mfma_supported; kAmaxWays x kAmaxStride floats,
// zero beforehand): also the maximum |dqkv| written, into those slots
// (amax_atomic_bf16), for the fp8 quantisation of dqkv.
int attention_backward(int dtype, int B, int T, int H, int hd, const void* qkv, const void* out,
                       const void* dout, const float* lse, void* dqkv, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, float* amax = nullptr);

// ------------------------------------------------------------------ FP8 quantisation
// Per-tensor scale of an fp8 operand: inv = FMAX / amax, s = amax / FMAX
// (fp32; 1 and 1 for amax = 0); FMAX 448 for fmt 0 (E4M3), 57344 for fmt 1
// (E5M2).
struct Fp8Scale {
  float amax, inv, s, unused;
};
size_t fp8_scale_workspace_bytes();
// Per-block maxima of |x| over the n contiguous values x (bf16 or fp32,
// 16-byte aligned) into workspace (fp8_scale_workspace_bytes()), for the
// quantisation of the same n values.
int fp8_amax(int dtype_in, int64_t n, const void* x, float* workspace, hipStream_t stream);
// The scale of x from those maxima (stored into *sc) and the codes of
// fp8(x * inv) for x [R, Cc] (row stride ldx, R * Cc the n of fp8_amax):
// row-major into qrow [R, Cc] and / or transposed into qt [Cc, R] (either may
// be NULL).  Cc % 8 == 0; R % 16 == 0 when qt.  With colsum
// (fp8_colsum_bytes(R, Cc), device) also the per-row-block column sums of
// x that colsum_reduce turns into a bias gradient.  amax_np > 0 (at most
// kAmaxWays): amax_part holds that many slots, kAmaxStride floats apart, left
// by a producer kernel (amax_atomic_bf16), instead of fp8_amax's maxima.
// layers > 1 (producer slots, no colsum): that many tensors of the same shape
// in one launch, tensor l at x + l R ldx with slots amax_part + l kAmaxWays
// kAmaxStride, scale sc[l] and codes qrow / qt + l R Cc.
int fp8_quantize(int dtype_in, int fmt, int R, int Cc, const void* x, int64_t ldx, const float* amax_part,
                 Fp8Scale* sc, uint8_t* qrow, uint8_t* qt, hipStream_t stream, float* colsum = nullptr,
                 int amax_np = 0, int layers = 1);
size_t fp8_colsum_bytes(int R, int N);
// db[n] (+)= sum of the column sums left by fp8_quantize for R rows, in a
// fixed order.
int colsum_reduce(int R, int N, const float* colsum, float* db, bool accumulate, hipStream_t stream);

// ------------------------------------------------------------------ QK-Norm / rotary
// In place on the q and k columns of qkv [BT, 3C] (hd = C / H): QK-Norm (RMS
// normalisation per head, eps 1e-6; rstd [BT, 2H] fp32 saved, q heads then k
// heads per token) and the rotary embedding with cos / sin table cs
// [maxT][hd/2] (position t = row mod T).  The backward works in place on
// dqkv, reading the transformed values from qkv.
int rope_table(int maxT, int hd, float2* cs, hipStream_t stream);
int qk_transform_forward(int dtype, int BT, int T, int H, int hd, void* qkv, float* rstd, const float2* cs,
                         bool norm, bool rope, hipStream_t stream);
int qk_transform_backward(int dtype, int BT, int T, int H, int hd, const void* qkv, void* dqkv, const float* rstd,
                          const float2* cs, bool norm, bool rope, hipStream_t stream);

// ------------------------------------------------------------------ classifier
// In place over logits [N, Vp] (row stride Vp): columns >= V are masked.
// losses[i] = logsumexp_{j<V} z_ij - z_i,y_i;  z_ij <- (softmax_ij - [j==y_i]) * dscale
// for j < V and 0 for j >= V.  With amax (kAmaxWays x kAmaxStride floats,
// zero beforehand; bf16 only, and only where softmax_xent_has_amax holds), the
// maximum |z_ij| written is max-ed into those slots (amax_atomic_bf16).
int softmax_xent(int dtype, int N, int V, int Vp, void* logits, const int32_t* labels,
                 float* losses, float dscale, hipStream_t stream, float* amax = nullptr);
bool softmax_xent_has_amax(int dtype, int V, int Vp);
// out[0] = sum_i x[i] * scale  (fixed order; single block).
int sum_scaled(int n, const float* x, float scale, float* out, hipStream_t stream);

// ------------------------------------------------------------------ encoder
// Token ids are clamped to [0, vocab_rows) for memory safety only (ids outside
// [0, V) are undefined behaviour of the step).  wpe == NULL: no position
// term (out = wte[tokens]); the backward skips dwpe when it is NULL.
int encoder_forward(int dtype, int B, int T, int C, int vocab_rows, const int32_t* tokens,
                    const void* wte, const void* wpe, void* out, hipStream_t stream);
size_t encoder_backward_workspace_bytes(int B, int T, int C);
// dwte[tok] += dx0 rows (fp32, deterministic order); dwpe[0:T] = (or +=) sum over b.
// B*T <= 4194304 (the key sort's buffer).
int encoder_backward(int B, int T, int C, int vocab_rows, const int32_t* tokens, const float* dx0,
                     float* dwte, float* dwpe, bool accumulate_wpe, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);
// The two parts of encoder_backward: the key sort depends only on the ids
// (sorted: encoder_sort_keys_bytes(B*T) bytes of 64-bit keys, the first B*T
// of them valid afterwards), the rest on dx0.
size_t encoder_sort_keys_bytes(int n);
int encoder_sort_keys(int n, int vocab_rows, const int32_t* tokens, uint64_t* sorted, hipStream_t stream);
size_t encoder_backward_sorted_workspace_bytes(int B, int T, int C);
int encoder_backward_sorted(int B, int T, int C, const uint64_t* sorted, const float* dx0, float* dwte,
                            float* dwpe, bool accumulate_wpe, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

// ------------------------------------------------------------------ optimizer
// AdamW hyperparameters with the bias corrections c1 = 1 / (1 - b1^t) and
// c2 = 1 / (1 - b2^t) (evaluated in double on the host).
struct AdamHP {
  float lr, b1, b2, eps, wd, c1, c2;
};
AdamHP adam_hparams(float lr, float beta1, float beta2, float eps, float wd, int t);
// *dst = v on the device, in stream order (a one-thread kernel: the values
// travel as kernel arguments, so no host buffer must outlive the call).
int set_adam_hparams(AdamHP* dst, const AdamHP& v, hipStream_t stream);
// AdamW over n fp32 parameters; writes the bf16 copy if param_bf16 != null.
// With gscale (device, one float) every gradient enters multiplied by *gscale.
// With hp_dev (device) the kernel reads its hyperparameters there instead of
// taking (lr, beta1, beta2, eps, wd, t).
int adamw(int64_t n, float* master, const float* grad, float* m, float* v, bf16* param_bf16,
          float lr, float beta1, float beta2, float eps, float wd, int t, hipStream_t stream,
          const float* gscale = nullptr, const AdamHP* hp_dev = nullptr);
// AdamW as above (hyperparameters from hp_dev) that also writes, for each
// listed matrix block (`batches` row-major [R][Cc] fp32 matrices starting at
// element `off`, in increasing order, R % 8 == 0, Cc % 4 == 0), the
// transposed bf16 copy dst_t[b][c][r]; the ranges between the matrices must
// start and end on multiples of 4 elements.  One launch.
constexpr int kAdamMaxMats = 6;
struct AdamMatrix {
  int64_t off;
  int batches, R, Cc;
  bf16* dst_t;   // transposed bf16 copy [batches][Cc][R], or NULL (none)
  int tiles;     // set by the launcher
  // or NULL: the maximum |updated fp32 value| of batch b max-ed into the slots
  // amax + b * kAmaxWays * kAmaxStride (amax_atomic_f32; zero beforehand),
  // for the fp8 quantisation of the matrices
  float* amax;
};
struct AdamSegs {
  int nflat, nmat, flat_blocks;
  int64_t flat_total;
  int64_t flat_off[kAdamMaxMats + 1], flat_len[kAdamMaxMats + 1];
  AdamMatrix mat[kAdamMaxMats];
};
int adamw_transposed(int64_t n, float* master, const float* grad, float* m, float* v, bf16* param_bf16,
                     const AdamMatrix* mats, int nmats, hipStream_t stream, const float* gscale,
                     const AdamHP* hp_dev);
// dst[i] = src[i], i < n (device int32 arrays).
int copy_i32(int64_t n, const int32_t* src, int32_t* dst, hipStream_t stream);
// Global L2 norm of n fp32 gradients (16-byte aligned) into workspace[0] and
// the clipping factor (max_norm / norm if norm > max_norm > 0, else 1) into
// workspace[1]; workspace holds grad_norm_workspace_bytes() (device).
size_t grad_norm_workspace_bytes();
int grad_norm(int64_t n, const float* grad, float max_norm, float* workspace, hipStream_t stream);
// dst = RNE bf16 of src.
int cast_f32_to_bf16(int64_t n, const float* src, bf16* dst, hipStream_t stream);
// dst[b][c][r] = src[b][r][c] for `batches` bf16 matrices [R, Cc]; R, Cc multiples of 8.
int transpose_bf16(int batches, int R, int Cc, const bf16* src, bf16* dst, hipStream_t stream);
// Seeded GPT-2-style normal init of one tensor (see gpt2.h).
int init_normal(int64_t n, float* dst, uint64_t seed, int tensor_index, double stddev,
                hipStream_t stream);
int fill_f32(int64_t n, float* dst, float value, hipStream_t stream);
int convert_to_f32(int dtype, int64_t n, const void* src, float* dst, hipStream_t stream);

}  // namespace gpt2k
