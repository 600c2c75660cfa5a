// Causal multi-head attention, forward and backward, computed exactly without
// materialising the T x T score matrix in HBM (flash attention: the opening
// bullet list of "State of the Union [May 3, 2024]" names it; its kernel
// table lists the forward/backward kernels and the backward's helpers that
// form rowsum(dO * O) and finalise dQ).
//
// Layout: qkv [B, T, 3C] with q, k, v at column offsets 0, C, 2C and head h at
// h*hd inside each; out [B, T, C]; lse [B, H, T] fp32 (natural log of the
// softmax normaliser, including the row maximum).
//
// Per query row i:  s_ij = q_i . k_j / sqrt(hd) for j <= i,
//   m_i = max_j s_ij,  l_i = sum_j exp(s_ij - m_i),  out_i = sum_j exp(s_ij - m_i) v_j / l_i,
//   lse_i = m_i + ln l_i  (online: running max and rescaled running sums).
// Backward:  D_i = dO_i . O_i,  p_ij = exp(s_ij - lse_i),  dp_ij = dO_i . v_j,
//   ds_ij = p_ij (dp_ij - D_i),  dq_i = sum_j ds_ij k_j / sqrt(hd),
//   dk_j = sum_i ds_ij q_i / sqrt(hd),  dv_j = sum_i p_ij dO_i.
//
// This file holds the general path (any head dim 16/32/64/128, fp32 or bf16
// storage, fp32 arithmetic on the vector ALUs): one thread (or TPR threads
// splitting the head dim) per row, the other operand staged through LDS in
// 64-row tiles.  dQ and dK/dV are separate kernels so no atomics are needed.
// bf16 with head dim 64 (every GPT-2 size) runs on the matrix cores instead
// (attention_mfma.hip); the rowsum(dO * O) pass is shared.

#include "kernels.h"

namespace gpt2k {
namespace {

constexpr int kRows = 64;   // rows per block / per LDS tile

template <int TPR>
__device__ __forceinline__ float row_sum(float s) {
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) s += __shfl_xor(s, o, 64);
  return s;
}

template <typename T, int HD, int TPR>
__global__ __launch_bounds__(kRows * TPR) void attn_fwd_simt(int T_, int H, const T* __restrict__ qkv,
                                                             T* __restrict__ out, float* __restrict__ lse) {
  constexpr int EPT = HD / TPR;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int C = H * HD;
  const size_t C3 = 3 * (size_t)C;
  const int tid = threadIdx.x, qi = tid / TPR, part = tid % TPR;
  const int q0 = blockIdx.x * kRows;
  const int i = q0 + qi;
  const float scale = 1.0f / sqrtf((float)HD);
  __shared__ float Ks[kRows][HD];
  __shared__ float Vs[kRows][HD];
  const T* base = qkv + (size_t)b * T_ * C3 + h * HD;
  float q[EPT], o[EPT];
  float m = -INFINITY, l = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    q[e] = (i < T_) ? to_f32(base[(size_t)i * C3 + part * EPT + e]) * scale : 0.f;
    o[e] = 0.f;
  }
  const int kend = min(T_, q0 + kRows);
  for (int k0 = 0; k0 < kend; k0 += kRows) {
    __syncthreads();
    for (int idx = tid; idx < kRows * HD; idx += kRows * TPR) {
      int r = idx / HD, d = idx % HD;
      int j = k0 + r;
      Ks[r][d] = j < T_ ? to_f32(base[(size_t)j * C3 + C + d]) : 0.f;
      Vs[r][d] = j < T_ ? to_f32(base[(size_t)j * C3 + 2 * C + d]) : 0.f;
    }
    __syncthreads();
    if (i < T_) {
      const int jn = min(kRows, i - k0 + 1);
      for (int j = 0; j < jn; ++j) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) s += q[e] * Ks[j][part * EPT + e];
        s = row_sum<TPR>(s);
        const float mn = fmaxf(m, s);
        const float corr = __expf(m - mn);
        const float p = __expf(s - mn);
        l = l * corr + p;
#pragma unroll
        for (int e = 0; e < EPT; ++e) o[e] = o[e] * corr + p * Vs[j][part * EPT + e];
        m = mn;
      }
    }
  }
  if (i < T_) {
    const float inv = 1.0f / l;
    T* orow = out + ((size_t)b * T_ + i) * C + h * HD + part * EPT;
#pragma unroll
    for (int e = 0; e < EPT; ++e) orow[e] = from_f32<T>(o[e] * inv);
    if (part == 0) lse[(size_t)bh * T_ + i] = m + logf(l);
  }
}

// D[bh, i] = dO_i . O_i.  hd/8 lanes per row, each taking one 16-byte chunk
// of O and dO, combined with lane swizzles.
template <typename T>
// D_i = dO_i . O_i per (b, h, i), and the log-sum-exp in base 2
// (L2_i = lse_i * log2(e)) that the matrix-core backward kernels use.
__global__ __launch_bounds__(256) void attn_bwd_dot_kernel(int B, int T_, int H, int hd, const T* __restrict__ out,
                                                           const T* __restrict__ dout, const float* __restrict__ lse,
                                                           float* __restrict__ D, float* __restrict__ L2) {
  const int lpr = hd / 8;                       // lanes per row: 2, 4, 8 or 16
  const int64_t gl = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gl / lpr;                 // (b, h, i) in lse order
  const int part = (int)(gl % lpr);
  float s = 0.f;
  if (row < (int64_t)B * H * T_) {
    const int i = (int)(row % T_), bh = (int)(row / T_), b = bh / H, h = bh % H;
    const size_t off = ((size_t)b * T_ + i) * (size_t)(H * hd) + h * hd + part * 8;
    float o[8], d[8];
    Chunk8<T>::load(out + off, o);
    Chunk8<T>::load(dout + off, d);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += o[e] * d[e];
  }
  for (int m = 1; m < lpr; m <<= 1) s += __shfl_xor(s, m, 64);
  if (row < (int64_t)B * H * T_ && part == 0) {
    D[row] = s;
    L2[row] = lse[row] * 1.4426950408889634f;
  }
}

template <typename T, int HD, int TPR>
__global__ __launch_bounds__(kRows * TPR) void attn_bwd_dq_simt(int T_, int H, const T* __restrict__ qkv,
                                                                const T* __restrict__ dout,
                                                                const float* __restrict__ lse,
                                                                const float* __restrict__ Dv,
                                                                T* __restrict__ dqkv) {
  constexpr int EPT = HD / TPR;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int C = H * HD;
  const size_t C3 = 3 * (size_t)C;
  const int tid = threadIdx.x, qi = tid / TPR, part = tid % TPR;
  const int q0 = blockIdx.x * kRows;
  const int i = q0 + qi;
  const float scale = 1.0f / sqrtf((float)HD);
  __shared__ float Ks[kRows][HD];
  __shared__ float Vs[kRows][HD];
  const T* base = qkv + (size_t)b * T_ * C3 + h * HD;
  float q[EPT], dov[EPT], dq[EPT];
  float lse_i = 0.f, D_i = 0.f;
  if (i < T_) {
    lse_i = lse[(size_t)bh * T_ + i];
    D_i = Dv[(size_t)bh * T_ + i];
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    q[e] = (i < T_) ? to_f32(base[(size_t)i * C3 + part * EPT + e]) * scale : 0.f;
    dov[e] = (i < T_) ? to_f32(dout[((size_t)b * T_ + i) * C + h * HD + part * EPT + e]) : 0.f;
    dq[e] = 0.f;
  }
  const int kend = min(T_, q0 + kRows);
  for (int k0 = 0; k0 < kend; k0 += kRows) {
    __syncthreads();
    for (int idx = tid; idx < kRows * HD; idx += kRows * TPR) {
      int r = idx / HD, d = idx % HD;
      int j = k0 + r;
      Ks[r][d] = j < T_ ? to_f32(base[(size_t)j * C3 + C + d]) : 0.f;
      Vs[r][d] = j < T_ ? to_f32(base[(size_t)j * C3 + 2 * C + d]) : 0.f;
    }
    __syncthreads();
    if (i < T_) {
      const int jn = min(kRows, i - k0 + 1);
      for (int j = 0; j < jn; ++j) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          s += q[e] * Ks[j][part * EPT + e];
          dp += dov[e] * Vs[j][part * EPT + e];
        }
        s = row_sum<TPR>(s);
        dp = row_sum<TPR>(dp);
        const float p = __expf(s - lse_i);
        const float ds = p * (dp - D_i);
#pragma unroll
        for (int e = 0; e < EPT; ++e) dq[e] += ds * Ks[j][part * EPT + e];
      }
    }
  }
  if (i < T_) {
    T* dst = dqkv + ((size_t)b * T_ + i) * C3 + h * HD + part * EPT;
#pragma unroll
    for (int e = 0; e < EPT; ++e) dst[e] = from_f32<T>(dq[e] * scale);
  }
}

template <typename T, int HD, int TPR>
__global__ __launch_bounds__(kRows * TPR) void attn_bwd_dkdv_simt(int T_, int H, const T* __restrict__ qkv,
                                                                  const T* __restrict__ dout,
                                                                  const float* __restrict__ lse,
                                                                  const float* __restrict__ Dv,
                                                                  T* __restrict__ dqkv) {
  constexpr int EPT = HD / TPR;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int C = H * HD;
  const size_t C3 = 3 * (size_t)C;
  const int tid = threadIdx.x, kj = tid / TPR, part = tid % TPR;
  const int k0 = blockIdx.x * kRows;
  const int j = k0 + kj;
  const float scale = 1.0f / sqrtf((float)HD);
  __shared__ float Qs[kRows][HD];
  __shared__ float Os[kRows][HD];   // dO tile
  __shared__ float Ls[kRows], Ds[kRows];
  const T* base = qkv + (size_t)b * T_ * C3 + h * HD;
  float k[EPT], v[EPT], dk[EPT], dv[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    k[e] = (j < T_) ? to_f32(base[(size_t)j * C3 + C + part * EPT + e]) : 0.f;
    v[e] = (j < T_) ? to_f32(base[(size_t)j * C3 + 2 * C + part * EPT + e]) : 0.f;
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  for (int q0 = k0; q0 < T_; q0 += kRows) {
    __syncthreads();
    for (int idx = tid; idx < kRows * HD; idx += kRows * TPR) {
      int r = idx / HD, d = idx % HD;
      int i = q0 + r;
      Qs[r][d] = i < T_ ? to_f32(base[(size_t)i * C3 + d]) * scale : 0.f;
      Os[r][d] = i < T_ ? to_f32(dout[((size_t)b * T_ + i) * C + h * HD + d]) : 0.f;
    }
    for (int r = tid; r < kRows; r += kRows * TPR) {
      int i = q0 + r;
      Ls[r] = i < T_ ? lse[(size_t)bh * T_ + i] : 0.f;
      Ds[r] = i < T_ ? Dv[(size_t)bh * T_ + i] : 0.f;
    }
    __syncthreads();
    if (j < T_) {
      const int ib = max(0, j - q0);                 // first query row >= j in this tile
      const int ie = min(kRows, T_ - q0);
      for (int r = ib; r < ie; ++r) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          s += Qs[r][part * EPT + e] * k[e];
          dp += Os[r][part * EPT + e] * v[e];
        }
        s = row_sum<TPR>(s);
        dp = row_sum<TPR>(dp);
        const float p = __expf(s - Ls[r]);
        const float ds = p * (dp - Ds[r]);
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          dv[e] += p * Os[r][part * EPT + e];
          dk[e] += ds * Qs[r][part * EPT + e];   // Qs already carries 1/sqrt(hd)
        }
      }
    }
  }
  if (j < T_) {
    T* dst = dqkv + ((size_t)b * T_ + j) * C3 + h * HD + part * EPT;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      dst[C + e] = from_f32<T>(dk[e]);
      dst[2 * C + e] = from_f32<T>(dv[e]);
    }
  }
}

template <typename T, int HD, int TPR>
int fwd_launch(int B, int T_, int H, const void* qkv, void* out, float* lse, hipStream_t s) {
  dim3 grid((unsigned)ceil_div64(T_, kRows), (unsigned)(B * H));
  mark_begin(0, s);
  hipLaunchKernelGGL((attn_fwd_simt<T, HD, TPR>), grid, dim3(kRows * TPR), 0, s, T_, H, (const T*)qkv,
                     (T*)out, lse);
  GPT2_LAUNCH_CHECK();
  mark_end(0, s);
  return 0;
}

template <typename T, int HD, int TPR>
int bwd_launch(int B, int T_, int H, const void* qkv, const void* dout, const float* lse, float* D,
               void* dqkv, hipStream_t s) {
  dim3 grid((unsigned)ceil_div64(T_, kRows), (unsigned)(B * H));
  mark_begin(2, s);
  hipLaunchKernelGGL((attn_bwd_dq_simt<T, HD, TPR>), grid, dim3(kRows * TPR), 0, s, T_, H, (const T*)qkv,
                     (const T*)dout, lse, D, (T*)dqkv);
  GPT2_LAUNCH_CHECK();
  mark_end(2, s);
  mark_begin(1, s);
  hipLaunchKernelGGL((attn_bwd_dkdv_simt<T, HD, TPR>), grid, dim3(kRows * TPR), 0, s, T_, H,
                     (const T*)qkv, (const T*)dout, lse, D, (T*)dqkv);
  GPT2_LAUNCH_CHECK();
  mark_end(1, s);
  return 0;
}

template <typename T>
int fwd_dispatch(int B, int T_, int H, int hd, const void* qkv, void* out, float* lse, hipStream_t s) {
  switch (hd) {
    case 16: return fwd_launch<T, 16, 1>(B, T_, H, qkv, out, lse, s);
    case 32: return fwd_launch<T, 32, 1>(B, T_, H, qkv, out, lse, s);
    case 64: return fwd_launch<T, 64, 2>(B, T_, H, qkv, out, lse, s);
    case 128: return fwd_launch<T, 128, 4>(B, T_, H, qkv, out, lse, s);
  }
  return gpt2_internal_fail(1, "attention: head dim %d unsupported", hd);
}

template <typename T>
int bwd_dispatch(int B, int T_, int H, int hd, const void* qkv, const void* dout, const float* lse,
                 float* D, void* dqkv, hipStream_t s) {
  switch (hd) {
    case 16: return bwd_launch<T, 16, 1>(B, T_, H, qkv, dout, lse, D, dqkv, s);
    case 32: return bwd_launch<T, 32, 1>(B, T_, H, qkv, dout, lse, D, dqkv, s);
    case 64: return bwd_launch<T, 64, 2>(B, T_, H, qkv, dout, lse, D, dqkv, s);
    case 128: return bwd_launch<T, 128, 4>(B, T_, H, qkv, dout, lse, D, dqkv, s);
  }
  return gpt2_internal_fail(1, "attention: head dim %d unsupported", hd);
}

}  // namespace

int attention_forward(int dtype, int B, int T_, int H, int hd, const void* qkv, void* out, float* lse,
                      hipStream_t stream) {
  if (B < 0 || T_ < 0 || H <= 0 || !qkv || !out || !lse)
    return gpt2_internal_fail(1, "attention_forward: bad arguments");
  if (B == 0 || T_ == 0) return 0;
  if (attention_mfma_supported(dtype, hd)) return attention_forward_mfma(B, T_, H, qkv, out, lse, stream);
  return dtype == BF16 ? fwd_dispatch<bf16>(B, T_, H, hd, qkv, out, lse, stream)
                       : fwd_dispatch<float>(B, T_, H, hd, qkv, out, lse, stream);
}

size_t attention_backward_workspace_bytes(int B, int T_, int H, int hd) {
  (void)hd;
  return 2 * (((size_t)B * H * T_ + 63) / 64 * 64) * sizeof(float) + 256;
}

int attention_backward(int dtype, int B, int T_, int H, int hd, const void* qkv, const void* out,
                       const void* dout, const float* lse, void* dqkv, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, float* amax) {
  if (B < 0 || T_ < 0 || H <= 0 || !qkv || !out || !dout || !lse || !dqkv ||
      (amax && !attention_mfma_supported(dtype, hd)))
    return gpt2_internal_fail(1, "attention_backward: bad arguments");
  if (B == 0 || T_ == 0) return 0;
  if (!workspace || workspace_bytes < attention_backward_workspace_bytes(B, T_, H, hd))
    return gpt2_internal_fail(3, "attention_backward: workspace too small");
  // workspace: D [B*H*T], then L2 [B*H*T] at a 256-byte boundary
  float* D = (float*)workspace;
  float* L2 = D + ((size_t)B * H * T_ + 63) / 64 * 64;
  if (attention_mfma_supported(dtype, hd))
    return attention_backward_mfma(B, T_, H, qkv, out, dout, lse, L2, D, dqkv, stream, amax);
  const int64_t lanes = (int64_t)B * H * T_ * (hd / 8);
  mark_begin(0, stream);
  if (dtype == BF16) {
    hipLaunchKernelGGL(attn_bwd_dot_kernel<bf16>, dim3((unsigned)ceil_div64(lanes, 256)), dim3(256), 0, stream,
                       B, T_, H, hd, (const bf16*)out, (const bf16*)dout, lse, D, L2);
  } else {
    hipLaunchKernelGGL(attn_bwd_dot_kernel<float>, dim3((unsigned)ceil_div64(lanes, 256)), dim3(256), 0,
                       stream, B, T_, H, hd, (const float*)out, (const float*)dout, lse, D, L2);
  }
  GPT2_LAUNCH_CHECK();
  mark_end(0, stream);
  return dtype == BF16 ? bwd_dispatch<bf16>(B, T_, H, hd, qkv, dout, lse, D, dqkv, stream)
                       : bwd_dispatch<float>(B, T_, H, hd, qkv, dout, lse, D, dqkv, stream);
}

}  // namespace gpt2k
