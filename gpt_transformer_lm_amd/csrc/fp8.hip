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
// transposed (128 x 128 tiles through LDS), so every fp8 product reads both
// operands k-major.
//
// The bias gradient of an fp8 weight-gradient product is the column sum of
// the unquantised bf16 gradient, taken while the gradient is quantised: each
// 128 x 128 tile adds its 128 rows per column in a fixed order into a
// per-row-block partial, and a second kernel adds the row blocks in order
// (deterministic).

#include "kernels.h"

namespace gpt2k {
namespace {

constexpr int kAmaxBlocks = 1024;

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

__global__ __launch_bounds__(256) void fp8_scale_finalize_kernel(const float* __restrict__ partial, int np, int pstride,
                                                                 float fmax, Fp8Scale* __restrict__ out) {
  float m = 0.f;
  for (int i = threadIdx.x; i < np; i += 256) m = fmaxf(m, partial[(size_t)i * pstride]);
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

// Rows and columns of x per block of the quantisation (a multiple of 16:
// whole 128-byte lines of codes in both layouts).
constexpr int kQT = 128;

// x [R, Cc] (row stride ldx) -> qrow [R, Cc] and / or qt [Cc, R] codes.
// Grid (ceil(Cc / kQT), ceil(R / kQT)), 256 threads; Cc % 8 == 0, R % 16 == 0
// when qt.  Thread t takes columns 16 (t % 8) .. + 15 of rows t / 8 + 32 p
// (p < 4) of the tile: 16-byte code stores, whole lines per 8 threads.  The
// transposed codes go through LDS: thread t then gathers 4 columns x 16 rows
// (16 dword reads, a 4 x 4 byte transpose per dword quad) and stores 4
// 16-byte runs of qt.
// With CS, also colsum[blockIdx.y][c] = sum of x[r][c] over the tile's rows
// (each thread's 4 rows in order, then the 8 row groups of a wave by
// butterfly, then the 4 waves in order: fixed, so run to run identical), for
// the bias gradient.
// The scale comes from the np maxima amax_part[i * pstride] (the amax pass's
// per-block maxima, or a producer's slots): every block takes their maximum
// (exact, so all agree) and forms inv and s as above; block (0, 0) stores
// (amax, inv, s) for the products.  The tile's loads are issued first: they
// do not depend on the scale.  blockIdx.z selects one of several tensors of
// the same shape (x, slots, scale and codes advanced by their layer strides).
template <typename T, int FMT, bool CS>
__global__ __launch_bounds__(256) void quantize_kernel(int R, int Cc, const T* __restrict__ x, int64_t ldx,
                                                       const float* __restrict__ amax_part, int np, int pstride,
                                                       float fmax,
                                                       Fp8Scale* __restrict__ sc, uint8_t* __restrict__ qrow,
                                                       uint8_t* __restrict__ qt, float* __restrict__ colsum,
                                                       int64_t amax_lstride) {
  {
    const int64_t z = blockIdx.z;
    x += z * R * ldx;
    amax_part += z * amax_lstride;
    sc += z;
    if (qrow) qrow += z * R * Cc;
    if (qt) qt += z * R * Cc;
  }
  constexpr int kPitch = kQT / 4 + 2;   // dwords per LDS row: the two half-waves' rows 16 apart differ by 32 banks
  __shared__ uint32_t tile[kQT][kPitch];
  __shared__ float smax[4];
  __shared__ float csw[CS ? 4 : 1][CS ? kQT : 1];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r0 = blockIdx.y * kQT, c0 = blockIdx.x * kQT;
  const int cq = (tid & 7) * 16, rq = tid >> 3;
  const bool in0 = c0 + cq < Cc, in1 = c0 + cq + 8 < Cc;
  float v[4][16];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = r0 + rq + 32 * p;
#pragma unroll
    for (int e = 0; e < 16; ++e) v[p][e] = 0.f;
    if (r < R) {
      const T* src = x + (int64_t)r * ldx + c0 + cq;
      if (in0) Chunk8<T>::load(src, &v[p][0]);
      if (in1) Chunk8<T>::load(src + 8, &v[p][8]);
    }
  }
  float am = 0.f;
  for (int i = tid; i < np; i += 256) am = fmaxf(am, amax_part[(size_t)i * pstride]);
  am = wave_max(am);
  if (lane == 0) smax[wv] = am;
  __syncthreads();
  am = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
  const float inv = am > 0.f ? fmax / am : 1.0f;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    Fp8Scale r;
    r.amax = am;
    r.inv = inv;
    r.s = am > 0.f ? am / fmax : 1.0f;
    r.unused = 0.f;
    *sc = r;
  }
  float cs[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) cs[e] = 0.f;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int rl = rq + 32 * p, r = r0 + rl;
    if constexpr (CS) {
#pragma unroll
      for (int e = 0; e < 16; ++e) cs[e] += v[p][e];   // zeros outside the tensor
    }
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = pack4<FMT>(v[p][4 * k] * inv, v[p][4 * k + 1] * inv, v[p][4 * k + 2] * inv, v[p][4 * k + 3] * inv);
    if (qrow && r < R) {
      uint8_t* dst = qrow + (int64_t)r * Cc + c0 + cq;
      if (in1) *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      else if (in0) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    }
    if (qt) {
#pragma unroll
      for (int k = 0; k < 4; ++k) tile[rl][cq / 4 + k] = w[k];
    }
  }
  if constexpr (CS) {
    // lanes l, l ^ 8, l ^ 16, l ^ 32 hold the same columns
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      cs[e] += __shfl_xor(cs[e], 8, 64);
      cs[e] += __shfl_xor(cs[e], 16, 64);
      cs[e] += __shfl_xor(cs[e], 32, 64);
    }
    if (lane < 8) {
#pragma unroll
      for (int e = 0; e < 16; ++e) csw[wv][cq + e] = cs[e];
    }
  }
  if (CS || qt) __syncthreads();
  if constexpr (CS) {
    if (tid < kQT && c0 + tid < Cc)
      colsum[(int64_t)blockIdx.y * Cc + c0 + tid] = ((csw[0][tid] + csw[1][tid]) + csw[2][tid]) + csw[3][tid];
  }
  if (qt) {
    const int cg = (tid & 31) * 4, rg = (tid >> 5) * 16;
    if (r0 + rg < R) {
      uint32_t d[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) d[k] = tile[rg + k][cg / 4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c0 + cg + j < Cc) {
          uint32_t o[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)   // byte j of rows 4q .. 4q + 3
            o[q] = ((d[4 * q] >> (8 * j)) & 0xffu) | (((d[4 * q + 1] >> (8 * j)) & 0xffu) << 8) |
                   (((d[4 * q + 2] >> (8 * j)) & 0xffu) << 16) | (((d[4 * q + 3] >> (8 * j)) & 0xffu) << 24);
          *reinterpret_cast<uint4*>(qt + (int64_t)(c0 + cg + j) * R + r0 + rg) = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  }
}

// db[n] (+)= sum over the row blocks b of part[b][n], in a fixed order:
// sixteen groups of 64 threads take every sixteenth block, then the groups'
// sums are added in group order.
__global__ __launch_bounds__(1024) void colsum_reduce_kernel(int nb, int N, const float* __restrict__ part,
                                                             float* __restrict__ db, bool acc) {
  __shared__ float sh[16][64];
  const int c = threadIdx.x & 63, g = threadIdx.x >> 6, n = blockIdx.x * 64 + c;
  float t = 0.f;
  if (n < N)
#pragma unroll 4
    for (int b = g; b < nb; b += 16) t += part[(int64_t)b * N + n];
  sh[g][c] = t;
  __syncthreads();
  if (g == 0 && n < N) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += sh[k][c];
    db[n] = acc ? db[n] + s : s;
  }
}

}  // namespace

size_t fp8_scale_workspace_bytes() { return kAmaxBlocks * sizeof(float); }

int amax_blocks(int64_t n) {
  return (int)std::max<int64_t>(1, std::min<int64_t>(kAmaxBlocks, ceil_div64(n, 8 * 256)));
}

int fp8_amax(int dtype_in, int64_t n, const void* x, float* workspace, hipStream_t stream) {
  if (n < 0 || !x || !workspace || (uintptr_t)x % 16) return gpt2_internal_fail(1, "fp8_amax: bad arguments");
  const unsigned blocks = (unsigned)amax_blocks(n);
  if (dtype_in == BF16)
    hipLaunchKernelGGL(absmax_partial_kernel<bf16>, dim3(blocks), dim3(256), 0, stream, n, (const bf16*)x, workspace);
  else
    hipLaunchKernelGGL(absmax_partial_kernel<float>, dim3(blocks), dim3(256), 0, stream, n, (const float*)x,
                       workspace);
  GPT2_LAUNCH_CHECK();
  return 0;
}

template <typename T, int FMT>
void launch_quantize(dim3 grid, int R, int Cc, const void* x, int64_t ldx, const float* amax_part, int np,
                     int pstride, Fp8Scale* sc, uint8_t* qrow, uint8_t* qt, float* colsum, int64_t als,
                     hipStream_t stream) {
  const float fmax = FMT == 0 ? 448.0f : 57344.0f;
  if (colsum)
    hipLaunchKernelGGL((quantize_kernel<T, FMT, true>), grid, dim3(256), 0, stream, R, Cc, (const T*)x, ldx, amax_part,
                       np, pstride, fmax, sc, qrow, qt, colsum, als);
  else
    hipLaunchKernelGGL((quantize_kernel<T, FMT, false>), grid, dim3(256), 0, stream, R, Cc, (const T*)x, ldx,
                       amax_part, np, pstride, fmax, sc, qrow, qt, colsum, als);
}

int fp8_quantize(int dtype_in, int fmt, int R, int Cc, const void* x, int64_t ldx, const float* amax_part,
                 Fp8Scale* sc, uint8_t* qrow, uint8_t* qt, hipStream_t stream, float* colsum, int amax_np,
                 int layers) {
  if (R < 0 || Cc < 0 || !x || !amax_part || !sc || (!qrow && !qt) || Cc % 8 || ldx % 8 || (qt && R % 16) ||
      (uintptr_t)x % 16 || (fmt != 0 && fmt != 1))
    return gpt2_internal_fail(1, "fp8_quantize: bad arguments (R=%d, C=%d)", R, Cc);
  if (amax_np < 0 || amax_np > kAmaxWays) return gpt2_internal_fail(1, "fp8_quantize: amax_np=%d", amax_np);
  if (layers < 1 || layers > 65535 || (layers > 1 && (!amax_np || colsum || R == 0 || Cc == 0)))
    return gpt2_internal_fail(1, "fp8_quantize: %d layers need producer slots, no column sums, a non-empty shape",
                              layers);
  const int np = amax_np ? amax_np : amax_blocks((int64_t)R * Cc);
  const int ps = amax_np ? kAmaxStride : 1;
  if (R == 0 || Cc == 0) {   // no tile to store the scale: the one-block form
    hipLaunchKernelGGL(fp8_scale_finalize_kernel, dim3(1), dim3(256), 0, stream, amax_part, np, ps,
                       fmt == 0 ? 448.0f : 57344.0f, sc);
    GPT2_LAUNCH_CHECK();
    return 0;
  }
  dim3 grid((unsigned)ceil_div64(Cc, kQT), (unsigned)ceil_div64(R, kQT), (unsigned)layers);
  const int64_t als = (int64_t)kAmaxWays * kAmaxStride;   // slots of consecutive layers
  mark_begin(0, stream);
  if (dtype_in == BF16) {
    if (fmt == 0) launch_quantize<bf16, 0>(grid, R, Cc, x, ldx, amax_part, np, ps, sc, qrow, qt, colsum, als, stream);
    else launch_quantize<bf16, 1>(grid, R, Cc, x, ldx, amax_part, np, ps, sc, qrow, qt, colsum, als, stream);
  } else {
    if (fmt == 0) launch_quantize<float, 0>(grid, R, Cc, x, ldx, amax_part, np, ps, sc, qrow, qt, colsum, als, stream);
    else launch_quantize<float, 1>(grid, R, Cc, x, ldx, amax_part, np, ps, sc, qrow, qt, colsum, als, stream);
  }
  GPT2_LAUNCH_CHECK();
  mark_end(0, stream);
  return 0;
}

size_t fp8_colsum_bytes(int R, int N) { return (size_t)ceil_div64(R, kQT) * N * sizeof(float); }

int colsum_reduce(int R, int N, const float* part, float* db, bool accumulate, hipStream_t stream) {
  if (R < 0 || N < 0 || !part || !db) return gpt2_internal_fail(1, "colsum_reduce: bad arguments");
  if (N == 0) return 0;
  hipLaunchKernelGGL(colsum_reduce_kernel, dim3((unsigned)ceil_div64(N, 64)), dim3(1024), 0, stream,
                     (int)ceil_div64(R, kQT), N, part, db, accumulate);
  GPT2_LAUNCH_CHECK();
  return 0;
}

}  // namespace gpt2k
