// Fused softmax cross-entropy over the logits of the tied classifier.
//
// "State of the Union [May 3, 2024]" (opening bullet list) describes the
// fused classifier: it never materialises the normalised logits and evaluates
// the loss only at the label's index; its "Fine print" section pads the
// vocabulary to 50304 with the padded logits masked to -inf.  Here each row
// (one position) is handled by one 1024-thread block that keeps the whole row
// in registers: one read of the logits gives the row maximum m and the sum
// s = sum_{j<V} exp(z_j - m) (online: per-thread (max, sum) pairs combined in
// one block reduction; padded columns j >= V are excluded, i.e. -inf);
// the loss is m + ln s - z_y; then the gradient of the mean loss,
// (exp(z_j - m) / s - [j == y]) * dscale for j < V and 0 for j >= V, is
// written over the logits.  HBM traffic: one read and one write of the row.

#include "kernels.h"

namespace gpt2k {
namespace {

constexpr int kCeThreads = 1024;
constexpr int kCeWaves = kCeThreads / 64;

// (max, sum of exp(x - max)) pairs of a wave / block, combined so that the
// sum is rescaled to the larger maximum.
__device__ __forceinline__ void combine(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  s = (mn == -INFINITY) ? 0.f : s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}

__device__ __forceinline__ void block_reduce_max_sum(float& m, float& s, float* shm, float* shs) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) combine(m, s, __shfl_xor(m, o, 64), __shfl_xor(s, o, 64));
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) { shm[w] = m; shs[w] = s; }
  __syncthreads();
  m = shm[0];
  s = shs[0];
#pragma unroll
  for (int i = 1; i < kCeWaves; ++i) combine(m, s, shm[i], shs[i]);
}

// NC: chunks of 8 columns per thread (covers Vp <= NC * 8 * 1024).  The row is
// kept in registers in its storage type (bf16: 4 registers per chunk) so that
// two blocks fit on a compute unit; the exponentials are recomputed for the
// write.
template <typename T, int NC>
__global__ __launch_bounds__(kCeThreads) void softmax_xent_kernel(int V, int Vp, T* __restrict__ logits,
                                                                  const int32_t* __restrict__ labels,
                                                                  float* __restrict__ losses, float dscale) {
  __shared__ float shm[kCeWaves], shs[kCeWaves];
  __shared__ float s_zy;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  T* z = logits + (size_t)row * Vp;
  int y = labels[row];
  y = y < 0 ? 0 : (y >= V ? V - 1 : y);   // memory safety only; valid labels are in [0, V)
  if (tid == 0) s_zy = to_f32(z[y]);
  const int nch = Vp / 8;
  typedef T T8 __attribute__((ext_vector_type(8)));
  T8 raw[NC];
  // per-thread maximum and sum of exp(z - max) over its columns j < V
  float mx = -INFINITY, sm = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = tid + kCeThreads * c;
    if (ch < nch) {
      raw[c] = *reinterpret_cast<const T8*>(z + ch * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ch * 8 + e < V) mx = fmaxf(mx, (float)raw[c][e]);
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = tid + kCeThreads * c;
    if (ch < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ch * 8 + e < V) sm += __expf((float)raw[c][e] - mx);
    }
  }
  block_reduce_max_sum(mx, sm, shm, shs);   // contains a barrier: s_zy is visible after it
  if (tid == 0) losses[row] = mx + logf(sm) - s_zy;
  const float inv = dscale / sm;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = tid + kCeThreads * c;
    if (ch < nch) {
      T8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = ch * 8 + e;
        const float g = (j < V) ? __expf((float)raw[c][e] - mx) * inv - (j == y ? dscale : 0.f) : 0.f;
        o[e] = (T)g;
      }
      *reinterpret_cast<T8*>(z + ch * 8) = o;
    }
  }
}

__global__ __launch_bounds__(1024) void sum_scaled_kernel(int n, const float* __restrict__ x, float scale,
                                                          float* __restrict__ out) {
  __shared__ float sh[16];
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += 1024) s += x[i];
  s = wave_sum(s);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sh[w] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = 0.f;
    for (int i = 0; i < 16; ++i) r += sh[i];
    out[0] = r * scale;
  }
}

template <typename T>
int launch_t(int N, int V, int Vp, void* logits, const int32_t* labels, float* losses, float dscale,
             hipStream_t s) {
  const int nch = Vp / 8;
  const int need = (nch + kCeThreads - 1) / kCeThreads;
  T* L = (T*)logits;
  mark_begin(0, s);
  if (need <= 1)
    hipLaunchKernelGGL((softmax_xent_kernel<T, 1>), dim3(N), dim3(kCeThreads), 0, s, V, Vp, L, labels, losses, dscale);
  else if (need <= 2)
    hipLaunchKernelGGL((softmax_xent_kernel<T, 2>), dim3(N), dim3(kCeThreads), 0, s, V, Vp, L, labels, losses, dscale);
  else if (need <= 4)
    hipLaunchKernelGGL((softmax_xent_kernel<T, 4>), dim3(N), dim3(kCeThreads), 0, s, V, Vp, L, labels, losses, dscale);
  else if (need <= 7)
    hipLaunchKernelGGL((softmax_xent_kernel<T, 7>), dim3(N), dim3(kCeThreads), 0, s, V, Vp, L, labels, losses, dscale);
  else if (need <= 8)
    hipLaunchKernelGGL((softmax_xent_kernel<T, 8>), dim3(N), dim3(kCeThreads), 0, s, V, Vp, L, labels, losses, dscale);
  else
    return gpt2_internal_fail(1, "softmax_xent: Vp=%d too large", Vp);
  GPT2_LAUNCH_CHECK();
  mark_end(0, s);
  return 0;
}

}  // namespace

int softmax_xent(int dtype, int N, int V, int Vp, void* logits, const int32_t* labels, float* losses,
                 float dscale, hipStream_t stream) {
  if (N < 0 || V <= 0 || Vp < V || Vp % 8 || !logits || !labels || !losses)
    return gpt2_internal_fail(1, "softmax_xent: bad arguments");
  if (N == 0) return 0;
  return dtype == BF16 ? launch_t<bf16>(N, V, Vp, logits, labels, losses, dscale, stream)
                       : launch_t<float>(N, V, Vp, logits, labels, losses, dscale, stream);
}

int sum_scaled(int n, const float* x, float scale, float* out, hipStream_t stream) {
  if (n < 0 || !x || !out) return gpt2_internal_fail(1, "sum_scaled: bad arguments");
  hipLaunchKernelGGL(sum_scaled_kernel, dim3(1), dim3(1024), 0, stream, n, x, scale, out);
  GPT2_LAUNCH_CHECK();
  return 0;
}

}  // namespace gpt2k
