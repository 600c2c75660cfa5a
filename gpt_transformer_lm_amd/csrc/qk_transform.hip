// QK-Norm and rotary position embedding of the attention's queries and keys
// (two of the architecture changes the page "NanoGPT (124M) in 90 seconds"
// names, section "How it works", item "Architecture Changes"), in place on
// the QKV activation so that the attention kernels read the transformed
// values unchanged.
//
// For every token p (position t = p mod T), head h and each of q (columns
// h*hd ..) and k (columns C + h*hd ..) of qkv [B*T, 3C]:
//   QK-Norm:  r = 1 / sqrt(mean(x^2) + eps),  x <- x r       (r saved, fp32)
//   rotary:   for i < hd/2, with (c, s) = (cos, sin)(t * 10000^(-2i/hd)):
//             (x_i, x_{i+hd/2}) <- (x_i c - x_{i+hd/2} s, x_i s + x_{i+hd/2} c)
// Backward, in place on dqkv (the gradient with respect to the values the
// attention read):  rotary: g <- R^T g (the inverse rotation); QK-Norm:
// g <- r (g - y mean(g y)), with y the normalised value before the rotation,
// recovered from the stored transformed value as R^T x.
//
// Layout of the work: hd/8 lanes per vector, 8 consecutive elements (one
// 16-byte bf16 chunk) per lane; the sum of squares and mean(g y) are
// reductions over those lanes, and each rotation partner (element i + hd/2)
// sits in the lane hd/16 further on.  Memory-bound: one read and one write of
// 2/3 of the QKV activation (plus the stored values in the backward).

#include "kernels.h"

namespace gpt2k {
namespace {

constexpr float kQkEps = 1e-6f;

// cos / sin table [maxT][hd/2] (float2), angles evaluated in double.
__global__ void rope_table_kernel(int maxT, int hd, float2* __restrict__ cs) {
  const int half = hd / 2;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= maxT * half) return;
  const int t = idx / half, i = idx % half;
  const double a = (double)t * pow(10000.0, -2.0 * i / hd);
  cs[idx] = make_float2((float)cos(a), (float)sin(a));
}

template <int LPV>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = LPV / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Applies the rotation (inverse = transpose when inv) to this lane's 8
// values x, exchanging with the partner lane; i0 is the pair index of x[0].
template <int LPV>
__device__ __forceinline__ void rotate8(float x[8], bool first_half, int i0, const float2* __restrict__ cs_row,
                                        bool inv) {
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = __shfl_xor(x[e], LPV / 2, 64);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float2 c = cs_row[i0 + e];
    const float s = inv ? -c.y : c.y;
    // first half holds a (partner b): a c - b s;  second half holds b (partner a): a s + b c
    x[e] = first_half ? x[e] * c.x - o[e] * s : o[e] * s + x[e] * c.x;
  }
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void qk_fwd_kernel(int BT, int T_, int H, T* __restrict__ qkv,
                                                     float* __restrict__ rstd, const float2* __restrict__ cs,
                                                     bool norm, bool rope) {
  constexpr int LPV = HD / 8;
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t v = gt / LPV;                  // vector index: (p, which, h)
  const int j = (int)(gt % LPV);
  const int64_t nvec = (int64_t)BT * 2 * H;
  // whole groups of LPV lanes are inside or outside together (LPV divides 64)
  if (v >= nvec) return;
  const int C = H * HD;
  const int64_t p = v / (2 * H);
  const int rem = (int)(v % (2 * H)), which = rem / H, h = rem % H;
  T* ptr = qkv + p * 3 * (int64_t)C + which * C + h * HD + j * 8;
  float x[8];
  Chunk8<T>::load(ptr, x);
  if (norm) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    ss = group_sum<LPV>(ss);
    const float r = 1.0f / sqrtf(ss * (1.0f / HD) + kQkEps);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= r;
    if (j == 0) rstd[v] = r;
  }
  if (rope) {
    const int t = (int)(p % T_);
    const bool first = j < LPV / 2;
    rotate8<LPV>(x, first, (first ? j : j - LPV / 2) * 8, cs + (int64_t)t * (HD / 2), false);
  }
  Chunk8<T>::store(ptr, x);
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void qk_bwd_kernel(int BT, int T_, int H, const T* __restrict__ qkv,
                                                     T* __restrict__ dqkv, const float* __restrict__ rstd,
                                                     const float2* __restrict__ cs, bool norm, bool rope) {
  constexpr int LPV = HD / 8;
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t v = gt / LPV;
  const int j = (int)(gt % LPV);
  const int64_t nvec = (int64_t)BT * 2 * H;
  if (v >= nvec) return;
  const int C = H * HD;
  const int64_t p = v / (2 * H);
  const int rem = (int)(v % (2 * H)), which = rem / H, h = rem % H;
  const int64_t off = p * 3 * (int64_t)C + which * C + h * HD + j * 8;
  float g[8], y[8];
  Chunk8<T>::load(dqkv + off, g);
  if (norm) Chunk8<T>::load(qkv + off, y);
  if (rope) {
    const int t = (int)(p % T_);
    const bool first = j < LPV / 2;
    const float2* row = cs + (int64_t)t * (HD / 2);
    const int i0 = (first ? j : j - LPV / 2) * 8;
    rotate8<LPV>(g, first, i0, row, true);
    if (norm) rotate8<LPV>(y, first, i0, row, true);
  }
  if (norm) {
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) d += g[e] * y[e];
    d = group_sum<LPV>(d) * (1.0f / HD);
    const float r = rstd[v];
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = r * (g[e] - y[e] * d);
  }
  Chunk8<T>::store(dqkv + off, g);
}

template <typename T, int HD>
int launch_fwd(int BT, int T_, int H, void* qkv, float* rstd, const float2* cs, bool norm, bool rope, hipStream_t s) {
  const int64_t lanes = (int64_t)BT * 2 * H * (HD / 8);
  mark_begin(0, s);
  hipLaunchKernelGGL((qk_fwd_kernel<T, HD>), dim3((unsigned)ceil_div64(lanes, 256)), dim3(256), 0, s, BT, T_, H,
                     static_cast<T*>(qkv), rstd, cs, norm, rope);
  GPT2_LAUNCH_CHECK();
  mark_end(0, s);
  return 0;
}

template <typename T, int HD>
int launch_bwd(int BT, int T_, int H, const void* qkv, void* dqkv, const float* rstd, const float2* cs, bool norm,
               bool rope, hipStream_t s) {
  const int64_t lanes = (int64_t)BT * 2 * H * (HD / 8);
  mark_begin(0, s);
  hipLaunchKernelGGL((qk_bwd_kernel<T, HD>), dim3((unsigned)ceil_div64(lanes, 256)), dim3(256), 0, s, BT, T_, H,
                     static_cast<const T*>(qkv), static_cast<T*>(dqkv), rstd, cs, norm, rope);
  GPT2_LAUNCH_CHECK();
  mark_end(0, s);
  return 0;
}

template <typename T>
int fwd_hd(int hd, int BT, int T_, int H, void* qkv, float* rstd, const float2* cs, bool norm, bool rope,
           hipStream_t s) {
  switch (hd) {
    case 16: return launch_fwd<T, 16>(BT, T_, H, qkv, rstd, cs, norm, rope, s);
    case 32: return launch_fwd<T, 32>(BT, T_, H, qkv, rstd, cs, norm, rope, s);
    case 64: return launch_fwd<T, 64>(BT, T_, H, qkv, rstd, cs, norm, rope, s);
    case 128: return launch_fwd<T, 128>(BT, T_, H, qkv, rstd, cs, norm, rope, s);
  }
  return gpt2_internal_fail(1, "qk transform: head dim %d unsupported", hd);
}

template <typename T>
int bwd_hd(int hd, int BT, int T_, int H, const void* qkv, void* dqkv, const float* rstd, const float2* cs, bool norm,
           bool rope, hipStream_t s) {
  switch (hd) {
    case 16: return launch_bwd<T, 16>(BT, T_, H, qkv, dqkv, rstd, cs, norm, rope, s);
    case 32: return launch_bwd<T, 32>(BT, T_, H, qkv, dqkv, rstd, cs, norm, rope, s);
    case 64: return launch_bwd<T, 64>(BT, T_, H, qkv, dqkv, rstd, cs, norm, rope, s);
    case 128: return launch_bwd<T, 128>(BT, T_, H, qkv, dqkv, rstd, cs, norm, rope, s);
  }
  return gpt2_internal_fail(1, "qk transform: head dim %d unsupported", hd);
}

}  // namespace

int rope_table(int maxT, int hd, float2* cs, hipStream_t stream) {
  if (maxT <= 0 || hd <= 0 || hd % 2 || !cs) return gpt2_internal_fail(1, "rope_table: bad arguments");
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)ceil_div64((int64_t)maxT * (hd / 2), 256)), dim3(256), 0,
                     stream, maxT, hd, cs);
  GPT2_LAUNCH_CHECK();
  return 0;
}

int qk_transform_forward(int dtype, int BT, int T_, int H, int hd, void* qkv, float* rstd, const float2* cs,
                         bool norm, bool rope, hipStream_t stream) {
  if (BT < 0 || T_ <= 0 || H <= 0 || !qkv || (norm && !rstd) || (rope && !cs))
    return gpt2_internal_fail(1, "qk_transform_forward: bad arguments");
  if (BT == 0 || (!norm && !rope)) return 0;
  return dtype == BF16 ? fwd_hd<bf16>(hd, BT, T_, H, qkv, rstd, cs, norm, rope, stream)
                       : fwd_hd<float>(hd, BT, T_, H, qkv, rstd, cs, norm, rope, stream);
}

int qk_transform_backward(int dtype, int BT, int T_, int H, int hd, const void* qkv, void* dqkv, const float* rstd,
                          const float2* cs, bool norm, bool rope, hipStream_t stream) {
  if (BT < 0 || T_ <= 0 || H <= 0 || !qkv || !dqkv || (norm && !rstd) || (rope && !cs))
    return gpt2_internal_fail(1, "qk_transform_backward: bad arguments");
  if (BT == 0 || (!norm && !rope)) return 0;
  return dtype == BF16 ? bwd_hd<bf16>(hd, BT, T_, H, qkv, dqkv, rstd, cs, norm, rope, stream)
                       : bwd_hd<float>(hd, BT, T_, H, qkv, dqkv, rstd, cs, norm, rope, stream);
}

}  // namespace gpt2k
