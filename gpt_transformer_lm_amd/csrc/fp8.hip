// FP8 quantisation for the FP8 products of the step ("NanoGPT (124M) in 90
// seconds", section "How it works", item "Precision & Hardware").
//
// Per-tensor scaling: amax = max |x| over the tensor (per-block maxima, then
// one block takes the maximum of those -- exact, so independent of the
// order), inv = FMAX / amax and s = amax / FMAX in fp32 (1 and 1 when
// amax = 0), with FMAX = 448 (OCP E4M3: activations, weights) or 57344 (OCP
// E5M2: gradients).  Each element becomes fp8(fp32(x * inv)) by the hardware
// conversion (round to nearest even, subnormals kept); x * inv never exceeds
// FMAX by more than two fp32 roundings, which the conversion rounds back to
// FMAX.  The quantisation kernel writes the codes row-major and/or
// transposed (64 x 64 tiles through LDS), so every fp8 product reads both
// operands k-major.
//
// The bias gradient of an fp8 weight-gradient product is the column sum of
// the unquantised bf16 gradient: per-row-block partial sums (256 row blocks,
// eight columns per thread), then an in-order sum (deterministic).

#include "kernels.h"

namespace gpt2k {
namespace {

constexpr int kAmaxBlocks = 1024;
constexpr int kColsumRowBlocks = 256;

template <typename T>
__global__ __launch_bounds__(256) void absmax_partial_kernel(int64_t n, const T* __restrict__ x,
                                                             float* __restrict__ partial) {
  float m = 0.f;
  const int64_t n8 = n / 8, stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  // four independent 8-element loads in flight per thread
  for (; i + 3 * stride < n8; i += 4 * stride) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) Chunk8<T>::load(x + (i + u * stride) * 8, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[u][e]));
  }
  for (; i < n8; i += stride) {
    float v[8];
    Chunk8<T>::load(x + i * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  }
  if (blockIdx.x == 0)
    for (int64_t j = n8 * 8 + threadIdx.x; j < n; j += 256) m = fmaxf(m, fabsf(to_f32(x[j])));
  __shared__ float sh[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

__global__ __launch_bounds__(256) void fp8_scale_finalize_kernel(const float* __restrict__ partial, int np, float fmax,
                                                                 Fp8Scale* __restrict__ out) {
  float m = 0.f;
  for (int i = threadIdx.x; i < np; i += 256) m = fmaxf(m, partial[i]);
  __shared__ float sh[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float amax = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
    Fp8Scale r;
    r.amax = amax;
    r.inv = amax > 0.f ? fmax / amax : 1.0f;      // correctly rounded fp32 divisions
    r.s = amax > 0.f ? amax / fmax : 1.0f;
    r.unused = 0.f;
    *out = r;
  }
}

// Four values -> four fp8 codes (byte i = value i).
template <int FMT>
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  int w;
  if constexpr (FMT == 0) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

// x [R, Cc] (row stride ldx) -> qrow [R, Cc] and / or qt [Cc, R] codes.
// Grid (ceil(Cc / 64), ceil(R / 64)); Cc % 8 == 0, R % 16 == 0 when qt.
template <typename T, int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(int R, int Cc, const T* __restrict__ x, int64_t ldx,
                                                       const Fp8Scale* __restrict__ sc, uint8_t* __restrict__ qrow,
                                                       uint8_t* __restrict__ qt) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[64][64 + 16];
  const float inv = sc->inv;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int r = i >> 3, cc = (i & 7) * 8;
    const bool in = r0 + r < R && c0 + cc < Cc;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
    if (in) Chunk8<T>::load(x + (int64_t)(r0 + r) * ldx + c0 + cc, v);
    uint2 w;
    w.x = pack4<FMT>(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    w.y = pack4<FMT>(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    if (qrow && in) *reinterpret_cast<uint2*>(qrow + (int64_t)(r0 + r) * Cc + c0 + cc) = w;
    if (qt) *reinterpret_cast<uint2*>(&tile[r][cc]) = w;
  }
  if (qt) {
    __syncthreads();
    const int c = threadIdx.x >> 2, rr = (threadIdx.x & 3) * 16;
    if (c0 + c < Cc && r0 + rr < R) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = (uint32_t)tile[rr + 4 * q][c] | ((uint32_t)tile[rr + 4 * q + 1][c] << 8) |
               ((uint32_t)tile[rr + 4 * q + 2][c] << 16) | ((uint32_t)tile[rr + 4 * q + 3][c] << 24);
      *reinterpret_cast<uint4*>(qt + (int64_t)(c0 + c) * R + r0 + rr) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// part[b][n] = sum of dy[r][n] over rows r of row block b; each thread sums
// eight adjacent columns (one 16-byte load per row), N % 8 == 0.
__global__ __launch_bounds__(256) void colsum_partial_kernel(int R, int N, const bf16* __restrict__ dy,
                                                             float* __restrict__ part) {
  const int c8 = blockIdx.x * 256 + threadIdx.x;
  if (c8 * 8 >= N) return;
  const int rows = (R + gridDim.y - 1) / gridDim.y;
  const int r_beg = blockIdx.y * rows, r_end = min(R, r_beg + rows);
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.f;
  for (int r = r_beg; r < r_end; ++r) {
    float v[8];
    Chunk8<bf16>::load(dy + (int64_t)r * N + c8 * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += v[e];
  }
  Chunk8<float>::store(part + (int64_t)blockIdx.y * N + c8 * 8, s);
}

__global__ __launch_bounds__(256) void colsum_final_kernel(int N, int nb, const float* __restrict__ part,
                                                           float* __restrict__ db, bool acc) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = acc ? db[n] : 0.f;
  for (int b = 0; b < nb; ++b) s += part[(int64_t)b * N + n];
  db[n] = s;
}

}  // namespace

size_t fp8_scale_workspace_bytes() { return kAmaxBlocks * sizeof(float); }

int fp8_compute_scale(int dtype_in, int64_t n, const void* x, int fmt, Fp8Scale* out, float* workspace,
                      hipStream_t stream) {
  if (n < 0 || !x || !out || !workspace || (fmt != 0 && fmt != 1) || (uintptr_t)x % 16)
    return gpt2_internal_fail(1, "fp8_compute_scale: bad arguments");
  const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>(kAmaxBlocks, ceil_div64(n, 8 * 256)));
  if (dtype_in == BF16)
    hipLaunchKernelGGL(absmax_partial_kernel<bf16>, dim3(blocks), dim3(256), 0, stream, n, (const bf16*)x, workspace);
  else
    hipLaunchKernelGGL(absmax_partial_kernel<float>, dim3(blocks), dim3(256), 0, stream, n, (const float*)x,
                       workspace);
  GPT2_LAUNCH_CHECK();
  hipLaunchKernelGGL(fp8_scale_finalize_kernel, dim3(1), dim3(256), 0, stream, workspace, (int)blocks,
                     fmt == 0 ? 448.0f : 57344.0f, out);
  GPT2_LAUNCH_CHECK();
  return 0;
}

int fp8_quantize(int dtype_in, int fmt, int R, int Cc, const void* x, int64_t ldx, const Fp8Scale* sc, uint8_t* qrow,
                 uint8_t* qt, hipStream_t stream) {
  if (R < 0 || Cc < 0 || !x || !sc || (!qrow && !qt) || Cc % 8 || ldx % 8 || (qt && R % 16) || (uintptr_t)x % 16 ||
      (fmt != 0 && fmt != 1))
    return gpt2_internal_fail(1, "fp8_quantize: bad arguments (R=%d, C=%d)", R, Cc);
  if (R == 0 || Cc == 0) return 0;
  dim3 grid((unsigned)ceil_div64(Cc, 64), (unsigned)ceil_div64(R, 64));
  mark_begin(0, stream);
  if (dtype_in == BF16) {
    if (fmt == 0)
      hipLaunchKernelGGL((quantize_kernel<bf16, 0>), grid, dim3(256), 0, stream, R, Cc, (const bf16*)x, ldx, sc, qrow,
                         qt);
    else
      hipLaunchKernelGGL((quantize_kernel<bf16, 1>), grid, dim3(256), 0, stream, R, Cc, (const bf16*)x, ldx, sc, qrow,
                         qt);
  } else {
    if (fmt == 0)
      hipLaunchKernelGGL((quantize_kernel<float, 0>), grid, dim3(256), 0, stream, R, Cc, (const float*)x, ldx, sc,
                         qrow, qt);
    else
      hipLaunchKernelGGL((quantize_kernel<float, 1>), grid, dim3(256), 0, stream, R, Cc, (const float*)x, ldx, sc,
                         qrow, qt);
  }
  GPT2_LAUNCH_CHECK();
  mark_end(0, stream);
  return 0;
}

size_t bias_grad_workspace_bytes(int N) { return (size_t)kColsumRowBlocks * N * sizeof(float); }

int bias_grad_bf16(int R, int N, const bf16* dy, float* db, bool accumulate, float* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  if (R < 0 || N < 0 || N % 8 || !dy || (uintptr_t)dy % 16 || !db || !workspace ||
      workspace_bytes < bias_grad_workspace_bytes(N))
    return gpt2_internal_fail(1, "bias_grad_bf16: bad arguments");
  if (N == 0) return 0;
  hipLaunchKernelGGL(colsum_partial_kernel, dim3((unsigned)ceil_div64(N / 8, 256), kColsumRowBlocks), dim3(256), 0,
                     stream, R, N, dy, workspace);
  GPT2_LAUNCH_CHECK();
  const unsigned nx = (unsigned)ceil_div64(N, 256);
  hipLaunchKernelGGL(colsum_final_kernel, dim3(nx), dim3(256), 0, stream, N, kColsumRowBlocks, workspace, db,
                     accumulate);
  GPT2_LAUNCH_CHECK();
  return 0;
}

}  // namespace gpt2k
