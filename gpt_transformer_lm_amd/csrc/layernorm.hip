// LayerNorm forward and backward (the layernorm_forward / layernorm_backward
// rows of the kernel table in "State of the Union [May 3, 2024]", section
// "Runtime, DRAM traffic, instructions": 25 launches each per GPT-2 124M step,
// two per block plus the final one).
//
// One wavefront per row; each lane holds up to NCH 16-byte chunks of the row
// in registers, so a row is read once.  Statistics are fp32:
//   mean = sum(x) / C,  var = sum((x - mean)^2) / C (biased),  rstd = 1/sqrt(var + 1e-5).
// Backward, with xhat = (x - mean) * rstd and g = dy * w:
//   dx = rstd * (g - sum(g)/C - xhat * sum(g * xhat)/C)
// accumulated into the fp32 residual-stream gradient (the residual add of the
// block is the identity, so its gradient is this running sum), with a
// storage-type copy for the next GEMM.  dw = sum_rows dy * xhat and
// db = sum_rows dy are accumulated per wave in registers, combined per block
// in LDS into one partial row, and the partial rows are summed by a second
// kernel in a fixed order (deterministic).

#include "kernels.h"

namespace gpt2k {
namespace {

constexpr float kLnEps = 1e-5f;

// AM: also the maximum |y| over the block's rows into the amax slots (the fp8
// quantisation of y reads them instead of taking a pass of its own).  Waves
// past the last row compute on a copy of it and store nothing, so every wave
// reaches the block's barrier.
template <typename T, int NCH, bool AM>
__global__ __launch_bounds__(256) void ln_fwd_kernel(int N, int C, const T* __restrict__ x,
                                                     const T* __restrict__ w, const T* __restrict__ b,
                                                     T* __restrict__ y, float* __restrict__ mean,
                                                     float* __restrict__ rstd, float* __restrict__ amax) {
  const int row_ = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (!AM && row_ >= N) return;
  const bool live = row_ < N;
  const int row = live ? row_ : N - 1;
  const int nch = C / 8;
  const T* xr = x + (size_t)row * C;
  float v[NCH][8], wv[NCH][8], bv[NCH][8];
  // the gain and bias are loaded with the row, so the row needs one memory
  // round trip before its reductions instead of two
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    int ch = lane + 64 * c;
    if (ch < nch) {
      Chunk8<T>::load(xr + ch * 8, v[c]);
      Chunk8<T>::load(w + ch * 8, wv[c]);
      Chunk8<T>::load(b + ch * 8, bv[c]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    int ch = lane + 64 * c;
    if (ch < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[c][e];
    }
  }
  const float mu = wave_sum(s) / (float)C;
  float s2 = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    int ch = lane + 64 * c;
    if (ch < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float d = v[c][e] - mu;
        s2 += d * d;
      }
    }
  }
  const float var = wave_sum(s2) / (float)C;
  const float rs = 1.0f / sqrtf(var + kLnEps);
  T* yr = y + (size_t)row * C;
  float am = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    int ch = lane + 64 * c;
    if (ch < nch) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v[c][e] - mu) * rs * wv[c][e] + bv[c][e];
      if (live) Chunk8<T>::store(yr + ch * 8, o);
      if constexpr (AM) {
#pragma unroll
        for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(o[e]));
      }
    }
  }
  if (live && lane == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
  if constexpr (AM) {
    __shared__ float wm[4];
    am = wave_max(live ? am : 0.f);
    if (lane == 0) wm[threadIdx.x >> 6] = am;
    __syncthreads();
    if (threadIdx.x == 0)
      amax_atomic_bf16(amax, blockIdx.x, fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3])));
  }
}

// Rows of 32 * 8 * NCH elements exactly (C = 768: NCH = 3): one half-wave
// per row, so no lane idles (a whole wave would leave a third of its lanes
// idle in the second chunk), 8 rows per 256-thread block.  The reductions
// use xor distances below 32, so each half-wave reduces its own row.
template <typename T, int NCH, bool AM>
__global__ __launch_bounds__(256) void ln_fwd_half_kernel(int N, int C, const T* __restrict__ x,
                                                          const T* __restrict__ w, const T* __restrict__ b,
                                                          T* __restrict__ y, float* __restrict__ mean,
                                                          float* __restrict__ rstd, float* __restrict__ amax) {
  const int row_ = blockIdx.x * 8 + (threadIdx.x >> 5);
  const int l = threadIdx.x & 31;
  if (!AM && row_ >= N) return;             // whole half-waves leave together
  const bool live = row_ < N;               // (AM: every wave reaches the barrier)
  const int row = live ? row_ : N - 1;
  const T* xr = x + (size_t)row * C;
  float v[NCH][8], wv[NCH][8], bv[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = l + 32 * c;
    Chunk8<T>::load(xr + ch * 8, v[c]);
    Chunk8<T>::load(w + ch * 8, wv[c]);
    Chunk8<T>::load(b + ch * 8, bv[c]);
  }
  auto half_sum = [](float t) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
    return t;
  };
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) s += v[c][e];
  const float mu = half_sum(s) / (float)C;
  float s2 = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = v[c][e] - mu;
      s2 += d * d;
    }
  const float rs = 1.0f / sqrtf(half_sum(s2) / (float)C + kLnEps);
  T* yr = y + (size_t)row * C;
  float am = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (v[c][e] - mu) * rs * wv[c][e] + bv[c][e];
    if (live) Chunk8<T>::store(yr + (l + 32 * c) * 8, o);
    if constexpr (AM) {
#pragma unroll
      for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(o[e]));
    }
  }
  if (live && l == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
  if constexpr (AM) {
    __shared__ float wm[4];
    am = wave_max(live ? am : 0.f);   // the wave's two rows
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = am;
    __syncthreads();
    if (threadIdx.x == 0)
      amax_atomic_bf16(amax, blockIdx.x, fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3])));
  }
}

// WPB waves per block (1024 threads for C <= 1024, fewer for wider rows so
// that the row cache fits the registers); each block writes one partial row
// of dw and db.
// AM: also the maximum |dres_copy| over the block's rows into the amax slots.
template <typename T, int NCH, int WPB, bool AM>
__global__ __launch_bounds__(WPB * 64) void ln_bwd_kernel(int N, int C, const T* __restrict__ dy,
                                                     const T* __restrict__ x, const T* __restrict__ w,
                                                     const float* __restrict__ mean,
                                                     const float* __restrict__ rstd,
                                                     float* __restrict__ dres, bool dres_overwrite,
                                                     T* __restrict__ dres_copy,
                                                     float* __restrict__ part_dw,
                                                     float* __restrict__ part_db, float* __restrict__ amax) {
  const int wave_id = blockIdx.x * WPB + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * WPB;
  const int lane = threadIdx.x & 63;
  const int nch = C / 8;
  const float invC = 1.0f / (float)C;
  float wv[NCH][8], dwa[NCH][8], dba[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    int ch = lane + 64 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) { dwa[c][e] = 0.f; dba[c][e] = 0.f; wv[c][e] = 0.f; }
    if (ch < nch) Chunk8<T>::load(w + ch * 8, wv[c]);
  }
  float am = 0.f;   // AM: over this wave's rows
  for (int row = wave_id; row < N; row += nwaves) {
    const float mu = mean[row], rs = rstd[row];
    const T* dyr = dy + (size_t)row * C;
    const T* xr = x + (size_t)row * C;
    float dyv[NCH][8], xh[NCH][8];
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      int ch = lane + 64 * c;
      if (ch < nch) {
        float xv[8];
        Chunk8<T>::load(dyr + ch * 8, dyv[c]);
        Chunk8<T>::load(xr + ch * 8, xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xh[c][e] = (xv[e] - mu) * rs;
          float g = dyv[c][e] * wv[c][e];
          sg += g;
          sgx += g * xh[c][e];
          dwa[c][e] += dyv[c][e] * xh[c][e];
          dba[c][e] += dyv[c][e];
        }
      }
    }
    const float mg = wave_sum(sg) * invC;
    const float mgx = wave_sum(sgx) * invC;
    float* dr = dres + (size_t)row * C;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      int ch = lane + 64 * c;
      if (ch < nch) {
        float o[8];
        if (dres_overwrite) {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = 0.f;
        } else {
          Chunk8<float>::load(dr + ch * 8, o);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[e] += rs * (dyv[c][e] * wv[c][e] - mg - xh[c][e] * mgx);
        Chunk8<float>::store(dr + ch * 8, o);
        if (dres_copy) Chunk8<T>::store(dres_copy + (size_t)row * C + ch * 8, o);
        if constexpr (AM) {
#pragma unroll
          for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(o[e]));
        }
      }
    }
  }
  // reduce the block's waves in LDS, in wave order: one partial row per block (dw, then db)
  extern __shared__ float red[];   // [WPB][C]
  const int wi = threadIdx.x >> 6;
  __shared__ float wm[AM ? WPB : 1];
  if constexpr (AM) {
    am = wave_max(am);
    if (lane == 0) wm[wi] = am;
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    float(*acc)[8] = pass == 0 ? dwa : dba;
    float* dst = pass == 0 ? part_dw : part_db;
    if (pass == 1) __syncthreads();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      int ch = lane + 64 * c;
      if (ch < nch) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wi * C + ch * 8 + e] = acc[c][e];
      }
    }
    __syncthreads();
    if constexpr (AM) {
      if (pass == 0 && threadIdx.x == 0) {
        float mb = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < WPB; ++w2) mb = fmaxf(mb, wm[w2]);
        amax_atomic_bf16(amax, blockIdx.x, mb);
      }
    }
    for (int i = threadIdx.x; i < C; i += blockDim.x) {
      float t = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < WPB; ++w2) t += red[w2 * C + i];
      dst[(size_t)blockIdx.x * C + i] = t;
    }
  }
}

// dw[c] (+)= sum over the P partial rows of part_dw, db[c] likewise, in a
// fixed order.  The 2C output columns (dw then db) are split into blocks of 16;
// thread (g, c) of a block sums partial rows g, g + 16, ... of its column and
// the 16 row groups are combined in order.
__global__ __launch_bounds__(256) void column_reduce_kernel(const float* __restrict__ part_dw,
                                                            const float* __restrict__ part_db, int P, int C,
                                                            float* __restrict__ dw, float* __restrict__ db,
                                                            bool accumulate) {
  __shared__ float sh[16][17];
  const int cl = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int col = blockIdx.x * 16 + cl;
  const bool is_b = col >= C;
  const int c = is_b ? col - C : col;
  const float* part = is_b ? part_db : part_dw;
  float s = 0.f;
  if (col < 2 * C) {
    // the first 16 partial rows of this thread are loaded together, then
    // summed in the same order as the loop below would
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int p = g + 16 * j;
      v[j] = p < P ? part[(size_t)p * C + c] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) s += v[j];
    for (int p = g + 256; p < P; p += 16) s += part[(size_t)p * C + c];
  }
  sh[g][cl] = s;
  __syncthreads();
  if (g == 0 && col < 2 * C) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) t += sh[i][cl];
    float* out = is_b ? db : dw;
    out[c] = accumulate ? out[c] + t : t;
  }
}

int nch_for(int C) {
  int nch = C / 8;
  if (nch <= 64) return 1;
  if (nch <= 128) return 2;
  if (nch <= 256) return 4;
  if (nch <= 512) return 8;
  return -1;
}

// waves per backward block, and blocks: 4096 waves keep 4 on every SIMD of the
// 256 compute units; each block writes one partial row
int bwd_wpb(int C) {
  const int n = nch_for(C);
  return n <= 2 ? 16 : (n == 4 ? 8 : 4);
}
int bwd_blocks(int N, int C) {
  const int wpb = bwd_wpb(C);
  return (int)std::min<int64_t>(4096 / wpb, ((int64_t)N + wpb - 1) / wpb);
}

template <typename T, bool AM>
int fwd_t(int N, int C, const void* x, const void* w, const void* b, void* y, float* mean, float* rstd, float* amax,
          hipStream_t s) {
  dim3 grid((unsigned)ceil_div64(N, 4)), block(256);
  const T* X = (const T*)x;
  const T* W = (const T*)w;
  const T* Bb = (const T*)b;
  T* Y = (T*)y;
  mark_begin(0, s);
  if (C == 32 * 8 * 3) {
    hipLaunchKernelGGL((ln_fwd_half_kernel<T, 3, AM>), dim3((unsigned)ceil_div64(N, 8)), block, 0, s, N, C, X, W, Bb,
                       Y, mean, rstd, amax);
    GPT2_LAUNCH_CHECK();
    mark_end(0, s);
    return 0;
  }
  switch (nch_for(C)) {
    case 1: hipLaunchKernelGGL((ln_fwd_kernel<T, 1, AM>), grid, block, 0, s, N, C, X, W, Bb, Y, mean, rstd, amax); break;
    case 2: hipLaunchKernelGGL((ln_fwd_kernel<T, 2, AM>), grid, block, 0, s, N, C, X, W, Bb, Y, mean, rstd, amax); break;
    case 4: hipLaunchKernelGGL((ln_fwd_kernel<T, 4, AM>), grid, block, 0, s, N, C, X, W, Bb, Y, mean, rstd, amax); break;
    case 8: hipLaunchKernelGGL((ln_fwd_kernel<T, 8, AM>), grid, block, 0, s, N, C, X, W, Bb, Y, mean, rstd, amax); break;
    default: return gpt2_internal_fail(1, "layernorm: C=%d unsupported", C);
  }
  GPT2_LAUNCH_CHECK();
  mark_end(0, s);
  return 0;
}

template <typename T, bool AM>
int bwd_t(int N, int C, const void* dy, const void* x, const void* w, const float* mean,
          const float* rstd, float* dres, bool ovw, void* dres_copy, float* pdw, float* pdb, float* amax,
          hipStream_t s) {
  const int wpb = bwd_wpb(C);
  dim3 grid((unsigned)bwd_blocks(N, C)), block(wpb * 64);
  const size_t lds = (size_t)wpb * C * sizeof(float);
  const T* DY = (const T*)dy;
  const T* X = (const T*)x;
  const T* W = (const T*)w;
  T* DC = (T*)dres_copy;
  mark_begin(0, s);
  switch (nch_for(C)) {
    case 1: hipLaunchKernelGGL((ln_bwd_kernel<T, 1, 16, AM>), grid, block, lds, s, N, C, DY, X, W, mean, rstd, dres, ovw, DC, pdw, pdb, amax); break;
    case 2: hipLaunchKernelGGL((ln_bwd_kernel<T, 2, 16, AM>), grid, block, lds, s, N, C, DY, X, W, mean, rstd, dres, ovw, DC, pdw, pdb, amax); break;
    case 4: hipLaunchKernelGGL((ln_bwd_kernel<T, 4, 8, AM>), grid, block, lds, s, N, C, DY, X, W, mean, rstd, dres, ovw, DC, pdw, pdb, amax); break;
    case 8: hipLaunchKernelGGL((ln_bwd_kernel<T, 8, 4, AM>), grid, block, lds, s, N, C, DY, X, W, mean, rstd, dres, ovw, DC, pdw, pdb, amax); break;
    default: return gpt2_internal_fail(1, "layernorm: C=%d unsupported", C);
  }
  GPT2_LAUNCH_CHECK();
  mark_end(0, s);
  return 0;
}

}  // namespace

int layernorm_forward(int dtype, int N, int C, const void* x, const void* w, const void* b, void* y,
                      float* mean, float* rstd, hipStream_t stream, float* amax) {
  if (N < 0 || C <= 0 || C % 8 || !x || !w || !b || !y || !mean || !rstd || (amax && dtype != BF16))
    return gpt2_internal_fail(1, "layernorm_forward: bad arguments");
  if (N == 0) return 0;
  if (amax) return fwd_t<bf16, true>(N, C, x, w, b, y, mean, rstd, amax, stream);
  return dtype == BF16 ? fwd_t<bf16, false>(N, C, x, w, b, y, mean, rstd, nullptr, stream)
                       : fwd_t<float, false>(N, C, x, w, b, y, mean, rstd, nullptr, stream);
}

size_t layernorm_backward_workspace_bytes(int N, int C) {
  return 2 * (size_t)bwd_blocks(N, C) * C * sizeof(float) + 256;
}

int layernorm_backward(int dtype, int N, int C, const void* dy, const void* x, const void* w,
                       const float* mean, const float* rstd, float* dres, bool dres_overwrite,
                       void* dres_copy, float* dw, float* db, bool accumulate, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, float* amax) {
  if (N < 0 || C <= 0 || C % 8 || !dy || !x || !w || !mean || !rstd || !dres || !dw || !db ||
      (amax && (dtype != BF16 || !dres_copy)))
    return gpt2_internal_fail(1, "layernorm_backward: bad arguments");
  if (N == 0) return 0;
  size_t need = layernorm_backward_workspace_bytes(N, C);
  if (!workspace || workspace_bytes < need)
    return gpt2_internal_fail(3, "layernorm_backward: workspace too small");
  const int P = bwd_blocks(N, C);
  float* pdw = (float*)workspace;
  float* pdb = pdw + (size_t)P * C;
  int rc = amax ? bwd_t<bf16, true>(N, C, dy, x, w, mean, rstd, dres, dres_overwrite, dres_copy, pdw, pdb, amax, stream)
           : dtype == BF16
               ? bwd_t<bf16, false>(N, C, dy, x, w, mean, rstd, dres, dres_overwrite, dres_copy, pdw, pdb, nullptr, stream)
               : bwd_t<float, false>(N, C, dy, x, w, mean, rstd, dres, dres_overwrite, dres_copy, pdw, pdb, nullptr,
                                     stream);
  if (rc) return rc;
  hipLaunchKernelGGL(column_reduce_kernel, dim3((unsigned)ceil_div64(2 * (int64_t)C, 16)), dim3(256), 0, stream,
                     pdw, pdb, P, C, dw, db, accumulate);
  GPT2_LAUNCH_CHECK();
  return 0;
}

}  // namespace gpt2k
