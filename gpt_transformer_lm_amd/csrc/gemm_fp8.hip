// FP8 products of the GPT-2 step ("NanoGPT (124M) in 90 seconds", section
// "How it works", item "Precision & Hardware": FP8 for the MLP's forward and
// backward products, the QKV projection and the head): the matrix-core
// kernel of gemm_kernel.h instantiated with fp8 operands -- E4M3 weights and
// activations, E5M2 gradients as the A operand of the backward products --
// on v_mfma_scale_f32_32x32x64_f8f6f4, both operands k-major, or both
// m-major for the weight gradients (the row-major codes of dY and X, read
// with transposing LDS reads), with the step's epilogues on the rescaled fp32
// sums.

#include "gemm_kernel.h"

namespace gpt2k {
namespace {

template <int EPI, int FMT_A>
int launch_f8(const MfmaArgs& a, const Plan& pl, hipStream_t s) {
  if constexpr (EPI == EPI_STORE || EPI == EPI_BIAS_RES)
    if (pl.bm == 384) return launch_tile<384, 192, EPI, true, true, false, 1, true, FMT_A>(a, pl.splits, s);
  if constexpr (!epi_has_aux(EPI))
    if (pl.bm == 256) return launch_tile<256, 256, EPI, true, true, false, 1, true, FMT_A>(a, pl.splits, s);
  return launch_tile<128, 128, EPI, true, true, false, 1, true, FMT_A>(a, pl.splits, s);
}

}  // namespace

int gemm_fp8_launch(int epi, int fmt_a, bool kmajor, const MfmaArgs& a, const Plan& pl, hipStream_t stream) {
  if (!kmajor) {      // weight gradient from the row-major codes of dY (E5M2) and X (E4M3)
    if (epi != EPI_WGRAD || fmt_a != 1)
      return gpt2_internal_fail(1, "gemm(fp8): m-major operands only for the weight gradient");
    if (pl.bm == 256) return launch_tile<256, 256, EPI_WGRAD, false, false, false, 1, true, 1>(a, pl.splits, stream);
    return launch_tile<128, 128, EPI_WGRAD, false, false, false, 1, true, 1>(a, pl.splits, stream);
  }
  if (fmt_a == 0) {   // forward: activations and weights E4M3
    switch (epi) {
      case EPI_STORE: return launch_f8<EPI_STORE, 0>(a, pl, stream);
      case EPI_BIAS: return launch_f8<EPI_BIAS, 0>(a, pl, stream);
      case EPI_BIAS_RES: return launch_f8<EPI_BIAS_RES, 0>(a, pl, stream);
      case EPI_BIAS_GELU_D: return launch_f8<EPI_BIAS_GELU_D, 0>(a, pl, stream);
      case EPI_BIAS_RELU2_D: return launch_f8<EPI_BIAS_RELU2_D, 0>(a, pl, stream);
    }
  } else {            // backward: the gradient (A) E5M2
    switch (epi) {
      case EPI_STORE: return launch_f8<EPI_STORE, 1>(a, pl, stream);
      case EPI_MUL: return launch_f8<EPI_MUL, 1>(a, pl, stream);
      case EPI_WGRAD: return launch_f8<EPI_WGRAD, 1>(a, pl, stream);
    }
  }
  return gpt2_internal_fail(1, "gemm(fp8): epilogue %d with A format %d not instantiated", epi, fmt_a);
}

}  // namespace gpt2k
