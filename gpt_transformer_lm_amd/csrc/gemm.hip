// GEMM dispatch of the GPT-2 step (bf16 matrix-core and fp32 parity
// kernels): launch plans, epilogue / layout instantiations, split-K
// reductions.  The kernels themselves are in gemm_kernel.h; the FP8 products
// are dispatched by gemm_fp8.hip.

#include "gemm_kernel.h"

namespace gpt2k {
namespace {

// Instantiated (layout, epilogue) pairs: forward X W^T (k-major both) with the
// store / bias / residual / GELU epilogues; dX = dY W (B n-major) with store and
// GELU'; dW = dY^T X (both m/n-major) with the split-K partial epilogue.
template <int EPI>
int dispatch_layout_bf16(const GemmDesc& d, const MfmaArgs& a, const Plan& pl, bool bias_grad, hipStream_t s) {
  if constexpr (EPI == EPI_WGRAD) {
    if (!d.a_kmajor && !d.b_kmajor) {
      if (bias_grad) return launch_mfma<EPI, false, false, true>(a, pl, s);
      return launch_mfma<EPI, false, false, false>(a, pl, s);
    }
    // split-K partials of a plain-store dX = dY W (W n-major, or its k-major transpose)
    if (d.a_kmajor && !d.b_kmajor && !bias_grad) return launch_mfma<EPI, true, false, false>(a, pl, s);
    if (d.a_kmajor && d.b_kmajor && !bias_grad) return launch_mfma<EPI, true, true, false>(a, pl, s);
  } else if constexpr (EPI == EPI_STORE || EPI == EPI_MUL) {
    if (d.a_kmajor && !d.b_kmajor) return launch_mfma<EPI, true, false, false>(a, pl, s);
    if (d.a_kmajor && d.b_kmajor) return launch_mfma<EPI, true, true, false>(a, pl, s);
  } else {
    if (d.a_kmajor && d.b_kmajor) return launch_mfma<EPI, true, true, false>(a, pl, s);
  }
  return gpt2_internal_fail(1, "gemm(bf16): layout (a_kmajor=%d, b_kmajor=%d) not instantiated for epilogue %d",
                            (int)d.a_kmajor, (int)d.b_kmajor, EPI);
}

template <int EPI>
int dispatch_layout_f32(const GemmDesc& d, const SimtArgs& a, int splits, hipStream_t s) {
  if (d.a_kmajor && d.b_kmajor) return launch_simt<EPI, true, true>(a, splits, s);
  if (d.a_kmajor && !d.b_kmajor) return launch_simt<EPI, true, false>(a, splits, s);
  if (!d.a_kmajor && !d.b_kmajor) return launch_simt<EPI, false, false>(a, splits, s);
  return launch_simt<EPI, false, true>(a, splits, s);
}

}  // namespace

GemmLaunchInfo gemm_launch_info(const GemmDesc& d) {
  GemmLaunchInfo r{};
  const bool wgrad = d.epi == EPI_WGRAD;
  r.bias_grad = wgrad && d.bias_grad32 != nullptr;
  if (d.dtype != BF16) {   // fp32 SIMT kernel: 64 x 64 tiles, 4 waves, no split
    r.tile_m = r.tile_n = 64;
    r.waves = 4;
    r.kgroups = r.splits = 1;
    return r;
  }
  const Plan pl = plan_gemm(d.dtype, d.fp8, d.epi, d.M, d.N, d.K, d.a_kmajor, d.b_kmajor);
  r.tile_m = pl.bm;
  r.tile_n = pl.bn;
  r.kgroups = pl.kgroups;
  r.splits = pl.splits;
  // a split plain store runs the partial-sum (WGRAD) instantiation
  const int epi = (!wgrad && pl.splits > 1) ? (int)EPI_WGRAD : d.epi;
  r.waves = gemm_waves(pl.bm, pl.bn, epi, pl.kgroups);
  return r;
}

size_t gemm_workspace_bytes(int dtype, int epi, int M, int N, int K, bool a_kmajor, bool b_kmajor, int fp8) {
  const int s = gemm_splits(dtype, epi, M, N, K, a_kmajor, b_kmajor, fp8);
  if (epi == EPI_WGRAD) return (size_t)s * ((size_t)M * N + (size_t)M) * sizeof(float) + 256;
  if (s > 1) return (size_t)s * M * N * sizeof(float) + 256;   // split plain store
  return 0;
}

int gemm(const GemmDesc& d, hipStream_t stream) {
  if (d.M < 0 || d.N < 0 || d.K < 0 || !d.A || !d.B)
    return gpt2_internal_fail(1, "gemm: bad arguments");
  if (d.M == 0 || d.N == 0) return 0;
  const bool wgrad = d.epi == EPI_WGRAD;
  if (wgrad && !d.out32) return gpt2_internal_fail(1, "gemm: WGRAD needs out32");
  if (!wgrad && !d.C) return gpt2_internal_fail(1, "gemm: missing C");
  if ((d.epi == EPI_BIAS || d.epi == EPI_BIAS_RES || d.epi == EPI_BIAS_GELU_D || d.epi == EPI_BIAS_RELU2_D) &&
      !d.bias)
    return gpt2_internal_fail(1, "gemm: missing bias");
  if ((d.epi == EPI_BIAS_RES || d.epi == EPI_MUL) && !d.aux_in)
    return gpt2_internal_fail(1, "gemm: missing aux input");
  if ((d.epi == EPI_BIAS_GELU_D || d.epi == EPI_BIAS_RELU2_D) && !d.aux_out)
    return gpt2_internal_fail(1, "gemm: missing U output");

  const int splits = gemm_splits(d.dtype, d.epi, d.M, d.N, d.K, d.a_kmajor, d.b_kmajor, d.fp8);
  // a plain store split over K runs the partial-tile kernel, then a reduction into C
  const bool split_store = !wgrad && splits > 1;
  float* partial = nullptr;
  float* partial_bias = nullptr;
  if (wgrad || split_store) {
    size_t need = gemm_workspace_bytes(d.dtype, d.epi, d.M, d.N, d.K, d.a_kmajor, d.b_kmajor, d.fp8);
    if (!d.workspace || d.workspace_bytes < need)
      return gpt2_internal_fail(3, "gemm: workspace too small (%zu < %zu)", d.workspace_bytes, need);
    partial = reinterpret_cast<float*>(d.workspace);
    partial_bias = partial + (size_t)splits * d.M * d.N;
  }
  EpiArgs e{d.epi, d.M, d.N, d.C, d.ldc, d.bias, d.aux_in, d.ld_aux, d.aux_out, partial, partial_bias, d.amax};

  if (d.K == 0) return gpt2_internal_fail(1, "gemm: K == 0 is not supported");

  int rc = 0;
  if (d.amax && !d.fp8) return gpt2_internal_fail(1, "gemm: the output maximum is taken only by fp8 products");
  if (d.fp8 && (d.dtype != BF16 || !d.scale_a || !d.scale_b || d.K % 16 || d.lda % 16 || d.ldb % 16 || d.fp8 > 2 ||
                (wgrad && d.bias_grad32) || (d.a_kmajor != d.b_kmajor) || (!d.a_kmajor && !wgrad) ||
                (!d.a_kmajor && (d.M % 16 || d.N % 16))))
    return gpt2_internal_fail(1, "gemm(fp8): needs bf16 outputs, K and row strides multiples of 16, both scales, no "
                                 "fused bias gradient, and both operands k-major (or, for a weight gradient, both "
                                 "m-major with M and N multiples of 16)");
  if (d.dtype == BF16) {
    // shape contract of the MFMA kernel: K a multiple of 8, 16-byte aligned rows,
    // contiguous axis of m-/n-major operands a multiple of 8.
    if (d.K % 8 != 0) return gpt2_internal_fail(1, "gemm(bf16): K=%d not a multiple of 8", d.K);
    if (d.lda % 8 || d.ldb % 8) return gpt2_internal_fail(1, "gemm(bf16): lda/ldb not multiples of 8");
    if ((!d.a_kmajor && d.M % 8) || (!d.b_kmajor && d.N % 8))
      return gpt2_internal_fail(1, "gemm(bf16): m/n-major operand extent not a multiple of 8");
    if (((uintptr_t)d.A | (uintptr_t)d.B) % 16)
      return gpt2_internal_fail(1, "gemm(bf16): A/B not 16-byte aligned");
    const Plan pl = plan_gemm(d.dtype, d.fp8, d.epi, d.M, d.N, d.K, d.a_kmajor, d.b_kmajor);
    const int64_t opb = d.fp8 ? 1 : 2;   // bytes per operand element
    auto al16 = [](const void* q) { return ((uintptr_t)q % 16) == 0; };
    bool vec = d.N % 8 == 0;
    if (!wgrad && !split_store) vec = vec && d.ldc % 8 == 0 && al16(d.C);
    if (d.bias && !wgrad) vec = vec && al16(d.bias);
    if (d.aux_in) vec = vec && al16(d.aux_in) && d.ld_aux % 8 == 0;
    if (d.aux_out) vec = vec && al16(d.aux_out);
    // readable byte extents of the operands (rows x stride); buffer offsets are 32-bit
    const int64_t a_ext = (d.a_kmajor ? (int64_t)d.M : (int64_t)d.K) * d.lda * opb;
    const int64_t b_ext = (d.b_kmajor ? (int64_t)d.N : (int64_t)d.K) * d.ldb * opb;
    if (a_ext >= (int64_t)kOutOfRange || b_ext >= (int64_t)kOutOfRange)
      return gpt2_internal_fail(1, "gemm(bf16): operand larger than 4 GiB (%lld, %lld bytes)", (long long)a_ext,
                                (long long)b_ext);
    const int64_t x_ext = d.aux_in ? (int64_t)d.M * d.ld_aux * 2 : 0;
    if (x_ext >= (int64_t)kOutOfRange)
      return gpt2_internal_fail(1, "gemm(bf16): epilogue input larger than 4 GiB (%lld bytes)", (long long)x_ext);
    if (d.amax && (!d.fp8 || split_store || !vec ||
                   (d.epi != EPI_BIAS_GELU_D && d.epi != EPI_BIAS_RELU2_D && d.epi != EPI_MUL)))
      return gpt2_internal_fail(1, "gemm: the output maximum is taken only by unsplit fp8 activation epilogues with "
                                   "16-byte aligned rows");
    MfmaArgs a{d.A, d.lda, d.B, d.ldb, (uint32_t)a_ext, (uint32_t)b_ext, (uint32_t)x_ext, d.M, d.N, d.K,
               pl.k_per_split, vec, e, d.scale_a, d.scale_b};
    const bool bias_grad = wgrad && d.bias_grad32 != nullptr;
    if (bias_grad && d.a_kmajor)
      return gpt2_internal_fail(1, "gemm: fused bias gradient needs an m-major A");
    if (d.fp8) rc = gemm_fp8_launch(split_store ? EPI_WGRAD : d.epi, d.fp8 - 1, d.a_kmajor, a, pl, stream);
    else switch (split_store ? EPI_WGRAD : d.epi) {
      case EPI_STORE: rc = dispatch_layout_bf16<EPI_STORE>(d, a, pl, false, stream); break;
      case EPI_BIAS: rc = dispatch_layout_bf16<EPI_BIAS>(d, a, pl, false, stream); break;
      case EPI_BIAS_RES: rc = dispatch_layout_bf16<EPI_BIAS_RES>(d, a, pl, false, stream); break;
      case EPI_BIAS_GELU_D: rc = dispatch_layout_bf16<EPI_BIAS_GELU_D>(d, a, pl, false, stream); break;
      case EPI_BIAS_RELU2_D: rc = dispatch_layout_bf16<EPI_BIAS_RELU2_D>(d, a, pl, false, stream); break;
      case EPI_MUL: rc = dispatch_layout_bf16<EPI_MUL>(d, a, pl, false, stream); break;
      case EPI_WGRAD: rc = dispatch_layout_bf16<EPI_WGRAD>(d, a, pl, bias_grad, stream); break;
      default: return gpt2_internal_fail(1, "gemm: unknown epilogue %d", d.epi);
    }
    if (rc) return rc;
    if (wgrad) {
      const int64_t MN = (int64_t)d.M * d.N;
      const unsigned main_blocks = (unsigned)ceil_div64(MN, 4 * 256);
      const unsigned bias_blocks = bias_grad ? (unsigned)ceil_div64(d.M, 4 * 256) : 0u;
      hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(main_blocks + bias_blocks), dim3(256), 0, stream, partial, splits,
                         MN, d.out32, d.accumulate, main_blocks, partial_bias, (int64_t)d.M, d.bias_grad32);
      GPT2_LAUNCH_CHECK();
    }
    if (split_store) {
      hipLaunchKernelGGL(splitk_store_bf16_kernel, dim3((unsigned)ceil_div64((int64_t)d.M * d.N, 4 * 256)),
                         dim3(256), 0, stream, partial, splits, d.M, d.N, reinterpret_cast<bf16*>(d.C), d.ldc);
      GPT2_LAUNCH_CHECK();
    }
    return 0;
  }

  SimtArgs a{reinterpret_cast<const float*>(d.A), d.lda, reinterpret_cast<const float*>(d.B), d.ldb,
             d.M, d.N, d.K, (int)ceil_div64(d.K, splits), e};
  switch (d.epi) {
    case EPI_STORE: rc = dispatch_layout_f32<EPI_STORE>(d, a, 1, stream); break;
    case EPI_BIAS: rc = dispatch_layout_f32<EPI_BIAS>(d, a, 1, stream); break;
    case EPI_BIAS_RES: rc = dispatch_layout_f32<EPI_BIAS_RES>(d, a, 1, stream); break;
    case EPI_BIAS_GELU_D: rc = dispatch_layout_f32<EPI_BIAS_GELU_D>(d, a, 1, stream); break;
    case EPI_BIAS_RELU2_D: rc = dispatch_layout_f32<EPI_BIAS_RELU2_D>(d, a, 1, stream); break;
    case EPI_MUL: rc = dispatch_layout_f32<EPI_MUL>(d, a, 1, stream); break;
    case EPI_WGRAD: rc = dispatch_layout_f32<EPI_WGRAD>(d, a, splits, stream); break;
    default: return gpt2_internal_fail(1, "gemm: unknown epilogue %d", d.epi);
  }
  if (rc) return rc;
  if (wgrad) {
    int64_t MN = (int64_t)d.M * d.N;
    const unsigned main_blocks = (unsigned)ceil_div64(MN, 4 * 256);
    hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(main_blocks), dim3(256), 0, stream, partial, splits, MN, d.out32,
                       d.accumulate, main_blocks, (const float*)nullptr, (int64_t)0, (float*)nullptr);
    GPT2_LAUNCH_CHECK();
    if (d.bias_grad32) {
      if (d.a_kmajor) return gpt2_internal_fail(1, "gemm: bias gradient needs an m-major A");
      hipLaunchKernelGGL(colsum_f32_kernel, dim3((unsigned)ceil_div64(d.M, 256)), dim3(256), 0, stream,
                         reinterpret_cast<const float*>(d.A), d.lda, d.M, d.K, d.bias_grad32,
                         d.accumulate);
      GPT2_LAUNCH_CHECK();
    }
  }
  return 0;
}

}  // namespace gpt2k

