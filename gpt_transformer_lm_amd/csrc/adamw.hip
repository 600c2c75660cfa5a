// Parameter update and parameter-state kernels.
//
// AdamW (the adamw_kernel3 row of the kernel table in "State of the Union
// [May 3, 2024]", section "Runtime, DRAM traffic, instructions"; the opening
// bullet list keeps the master copy of the parameters in fp32), one pass over
// the flat parameter array:
//   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
//   theta -= lr * ((m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps) + wd * theta)
// and, in the same pass, the bf16 copy that the forward reads (the page's
// separate copy_and_cast kernel is folded in).  16-byte vector accesses;
// 30 bytes of HBM traffic per parameter (read theta, g, m, v; write theta,
// m, v and the bf16 copy).
//
// Seeded initialisation: counter-based SplitMix64 (Steele, Lea & Flood 2014)
// and the Box-Muller transform, evaluated in double precision, one element
// per thread (the pages list random init in C as pending work, paragraph
// "Functional").

#include "kernels.h"

namespace gpt2k {
namespace {

// Hyperparameters come by value, or from device memory when hp_dev is set
// (a captured graph replays with the values its caller last wrote there).
__global__ void adamw_kernel(int64_t n, float* __restrict__ master, const float* __restrict__ grad,
                             float* __restrict__ mom1, float* __restrict__ mom2, bf16* __restrict__ pbf,
                             AdamHP hp_val, const AdamHP* __restrict__ hp_dev, const float* __restrict__ gscale) {
  const AdamHP hp = hp_dev ? *hp_dev : hp_val;
  const float lr = hp.lr, b1 = hp.b1, b2 = hp.b2, eps = hp.eps, wd = hp.wd, c1 = hp.c1, c2 = hp.c2;
  // the gradient enters scaled by *gscale (global-norm clipping) when given
  const float gs = gscale ? *gscale : 1.0f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      float4 th = *reinterpret_cast<const float4*>(master + i);
      float4 g = *reinterpret_cast<const float4*>(grad + i);
      float4 m = *reinterpret_cast<const float4*>(mom1 + i);
      float4 v = *reinterpret_cast<const float4*>(mom2 + i);
      float tv[4] = {th.x, th.y, th.z, th.w}, gv[4] = {g.x * gs, g.y * gs, g.z * gs, g.w * gs};
      float mv[4] = {m.x, m.y, m.z, m.w}, vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mv[e] = b1 * mv[e] + (1.0f - b1) * gv[e];
        vv[e] = b2 * vv[e] + (1.0f - b2) * gv[e] * gv[e];
        const float mh = mv[e] * c1, vh = vv[e] * c2;
        tv[e] -= lr * (mh / (sqrtf(vh) + eps) + wd * tv[e]);
      }
      *reinterpret_cast<float4*>(master + i) = make_float4(tv[0], tv[1], tv[2], tv[3]);
      *reinterpret_cast<float4*>(mom1 + i) = make_float4(mv[0], mv[1], mv[2], mv[3]);
      *reinterpret_cast<float4*>(mom2 + i) = make_float4(vv[0], vv[1], vv[2], vv[3]);
      if (pbf) {
        typedef bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        bf16x4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)tv[e];
        *reinterpret_cast<bf16x4_t*>(pbf + i) = o;
      }
    } else {
      for (int64_t j = i; j < n; ++j) {
        const float gj = grad[j] * gs;
        float mv = b1 * mom1[j] + (1.0f - b1) * gj;
        float vv = b2 * mom2[j] + (1.0f - b2) * gj * gj;
        float th = master[j];
        th -= lr * ((mv * c1) / (sqrtf(vv * c2) + eps) + wd * th);
        master[j] = th;
        mom1[j] = mv;
        mom2[j] = vv;
        if (pbf) pbf[j] = (bf16)th;
      }
    }
  }
}

// One AdamW element update (the formula above).
__device__ __forceinline__ void adam_elem(float& th, float g, float& m, float& v, float lr, float b1, float b2,
                                          float eps, float wd, float c1, float c2) {
  m = b1 * m + (1.0f - b1) * g;
  v = b2 * v + (1.0f - b2) * g * g;
  th -= lr * ((m * c1) / (sqrtf(v * c2) + eps) + wd * th);
}

// The same update over the whole parameter array in one launch, where the
// matrices whose bf16 copy the backward also reads transposed get that copy
// here too: blocks [0, flat_blocks) sweep the flat ranges (everything but
// those matrices) four elements per thread; each later block updates one
// 64 x 64 tile of one matrix, stages its bf16 values in LDS and writes them
// transposed as well (so the transposed copy costs 2 bytes per element
// instead of a separate read-and-write pass).
__global__ __launch_bounds__(256) void adamw_fused_kernel(AdamSegs sg, float* __restrict__ master,
                                                          const float* __restrict__ grad, float* __restrict__ mom1,
                                                          float* __restrict__ mom2, bf16* __restrict__ pbf,
                                                          AdamHP hp_val, const AdamHP* __restrict__ hp_dev,
                                                          const float* __restrict__ gscale) {
  const AdamHP hp = hp_dev ? *hp_dev : hp_val;
  const float lr = hp.lr, b1 = hp.b1, b2 = hp.b2, eps = hp.eps, wd = hp.wd, c1 = hp.c1, c2 = hp.c2;
  const float gs = gscale ? *gscale : 1.0f;
  typedef bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  if ((int)blockIdx.x < sg.flat_blocks) {
    // flat ranges: index space [0, flat_total) in range order; every range
    // starts and ends on a multiple of 4 elements
    const int64_t stride = (int64_t)sg.flat_blocks * 256 * 4;
    for (int64_t x = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; x < sg.flat_total; x += stride) {
      int r = 0;
      int64_t base = 0;
      while (r + 1 < sg.nflat && x >= base + sg.flat_len[r]) base += sg.flat_len[r++];
      const int64_t i = sg.flat_off[r] + (x - base);
      float4 th = *reinterpret_cast<const float4*>(master + i);
      const float4 g = *reinterpret_cast<const float4*>(grad + i);
      float4 m = *reinterpret_cast<const float4*>(mom1 + i);
      float4 v = *reinterpret_cast<const float4*>(mom2 + i);
      adam_elem(th.x, g.x * gs, m.x, v.x, lr, b1, b2, eps, wd, c1, c2);
      adam_elem(th.y, g.y * gs, m.y, v.y, lr, b1, b2, eps, wd, c1, c2);
      adam_elem(th.z, g.z * gs, m.z, v.z, lr, b1, b2, eps, wd, c1, c2);
      adam_elem(th.w, g.w * gs, m.w, v.w, lr, b1, b2, eps, wd, c1, c2);
      *reinterpret_cast<float4*>(master + i) = th;
      *reinterpret_cast<float4*>(mom1 + i) = m;
      *reinterpret_cast<float4*>(mom2 + i) = v;
      if (pbf) {
        bf16x4_t o;
        o[0] = (bf16)th.x; o[1] = (bf16)th.y; o[2] = (bf16)th.z; o[3] = (bf16)th.w;
        *reinterpret_cast<bf16x4_t*>(pbf + i) = o;
      }
    }
    return;
  }
  // one 64 x 64 tile of matrix k (batch bt): rows r0 .., columns c0 ..
  int t = (int)blockIdx.x - sg.flat_blocks, k = 0;
  while (k + 1 < sg.nmat && t >= sg.mat[k].tiles) t -= sg.mat[k++].tiles;
  const AdamMatrix mt = sg.mat[k];
  const int tr = (mt.R + 63) / 64, tc = (mt.Cc + 63) / 64;
  const int bt = t / (tr * tc), rem = t % (tr * tc);
  const int r0 = (rem / tc) * 64, c0 = (rem % tc) * 64;
  const int64_t mbase = mt.off + (int64_t)bt * mt.R * mt.Cc;
  __shared__ __attribute__((aligned(16))) bf16 tile[64][72];   // 144-byte rows
  const int tid = threadIdx.x, cq = (tid & 15) * 4;
  float am = 0.f;   // largest |updated value| of the tile (matrices quantised to fp8)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = (tid >> 4) + 16 * q;
    bf16x4_t o;
    if (r0 + r < mt.R && c0 + cq < mt.Cc) {
      const int64_t i = mbase + (int64_t)(r0 + r) * mt.Cc + c0 + cq;
      float4 th = *reinterpret_cast<const float4*>(master + i);
      const float4 g = *reinterpret_cast<const float4*>(grad + i);
      float4 m = *reinterpret_cast<const float4*>(mom1 + i);
      float4 v = *reinterpret_cast<const float4*>(mom2 + i);
      adam_elem(th.x, g.x * gs, m.x, v.x, lr, b1, b2, eps, wd, c1, c2);
      adam_elem(th.y, g.y * gs, m.y, v.y, lr, b1, b2, eps, wd, c1, c2);
      adam_elem(th.z, g.z * gs, m.z, v.z, lr, b1, b2, eps, wd, c1, c2);
      adam_elem(th.w, g.w * gs, m.w, v.w, lr, b1, b2, eps, wd, c1, c2);
      *reinterpret_cast<float4*>(master + i) = th;
      *reinterpret_cast<float4*>(mom1 + i) = m;
      *reinterpret_cast<float4*>(mom2 + i) = v;
      o[0] = (bf16)th.x; o[1] = (bf16)th.y; o[2] = (bf16)th.z; o[3] = (bf16)th.w;
      *reinterpret_cast<bf16x4_t*>(pbf + i) = o;
      am = fmaxf(am, fmaxf(fmaxf(fabsf(th.x), fabsf(th.y)), fmaxf(fabsf(th.z), fabsf(th.w))));
    } else {
      o[0] = o[1] = o[2] = o[3] = (bf16)0.f;
    }
    *reinterpret_cast<bf16x4_t*>(&tile[r][cq]) = o;
  }
  if (mt.amax) {   // (uniform)
    am = wave_max(am);
    if ((tid & 63) == 0) amax_atomic_f32(mt.amax + (size_t)bt * kAmaxWays * kAmaxStride, t * 4 + (tid >> 6), am);
  }
  if (!mt.dst_t) return;   // (uniform)
  __syncthreads();
  // transposed: row c0 + c of [batch][Cc][R] gets tile column c, 16 rows per thread
  {
    typedef bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    const int c = tid >> 2, rr = (tid & 3) * 16;
    bf16* dst = mt.dst_t + (int64_t)bt * mt.R * mt.Cc + (int64_t)(c0 + c) * mt.R + r0 + rr;
    if (c0 + c < mt.Cc) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (r0 + rr + 8 * h + 8 <= mt.R) {
          bf16x8_t o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = tile[rr + 8 * h + e][c];
          *reinterpret_cast<bf16x8_t*>(dst + 8 * h) = o;
        }
      }
    }
  }
}

// Global gradient norm for clipping: per-block partial sums of squares (a
// fixed grid, grid-stride float4 reads), then one block adds the partials in
// index order (deterministic), takes the square root and the clipping factor
// max_norm / norm when norm > max_norm > 0, else 1.
constexpr int kNormBlocks = 1024;

__global__ __launch_bounds__(256) void grad_sumsq_kernel(int64_t n, const float* __restrict__ g,
                                                         float* __restrict__ partial) {
  float s = 0.f;
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const float4 v = reinterpret_cast<const float4*>(g)[i];
    s += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  if (blockIdx.x == 0)
    for (int64_t j = n4 * 4 + threadIdx.x; j < n; j += 256) s += g[j] * g[j];
  __shared__ float sh[4];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

__global__ __launch_bounds__(256) void grad_norm_finalize_kernel(const float* __restrict__ partial, int np,
                                                                 float max_norm, float* __restrict__ out) {
  __shared__ double sh[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < np; i += 256) s += (double)partial[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float norm = (float)sqrt(sh[0]);
    out[0] = norm;
    out[1] = (max_norm > 0.f && norm > max_norm) ? max_norm / norm : 1.0f;
  }
}

__global__ void set_adam_hp_kernel(AdamHP* dst, AdamHP v) { *dst = v; }

__global__ void copy_i32_kernel(int64_t n, const int32_t* __restrict__ src, int32_t* __restrict__ dst) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

__global__ void cast_kernel(int64_t n, const float* __restrict__ src, bf16* __restrict__ dst) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = (bf16)src[i];
}

__global__ void fill_kernel(int64_t n, float* __restrict__ dst, float value) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = value;
}

__global__ void bf16_to_f32_kernel(int64_t n, const bf16* __restrict__ src, float* __restrict__ dst) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = (float)src[i];
}

__device__ __forceinline__ uint64_t splitmix64_out(uint64_t seed, uint64_t n) {
  uint64_t z = seed + (n + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void init_normal_kernel(int64_t n, float* __restrict__ dst, uint64_t seed, uint64_t tensor_index,
                                   double stddev) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const uint64_t c = (tensor_index << 40) | (uint64_t)e;
  const uint64_t r0 = splitmix64_out(seed, 2 * c);
  const uint64_t r1 = splitmix64_out(seed, 2 * c + 1);
  const double u1 = ((double)(r0 >> 11) + 1.0) * 0x1.0p-53;
  const double u2 = (double)(r1 >> 11) * 0x1.0p-53;
  const double z = sqrt(-2.0 * log(u1)) * cos(2.0 * 3.14159265358979323846 * u2);
  dst[e] = (float)(stddev * z);
}

// dst[b][c][r] = src[b][r][c] for a batch of bf16 matrices [R, Cc] (R and Cc
// multiples of 8): 64 x 64 tiles through LDS, 16-byte global loads and stores.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16* __restrict__ src, bf16* __restrict__ dst,
                                                             int R, int Cc) {
  typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
  __shared__ __attribute__((aligned(16))) bf16 tile[64][72];   // 144-byte rows
  const size_t mat = (size_t)R * Cc * blockIdx.z;
  const bf16* S = src + mat;
  bf16* D = dst + mat;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int r = i >> 3, cc = (i & 7) * 8;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)0.f;
    if (r0 + r < R && c0 + cc < Cc) v = *reinterpret_cast<const bf16x8*>(S + (size_t)(r0 + r) * Cc + c0 + cc);
    *reinterpret_cast<bf16x8*>(&tile[r][cc]) = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int c = i >> 3, rr = (i & 7) * 8;
    if (c0 + c < Cc && r0 + rr < R) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = tile[rr + e][c];
      *reinterpret_cast<bf16x8*>(D + (size_t)(c0 + c) * R + r0 + rr) = o;
    }
  }
}

unsigned blocks_for(int64_t n, int per_thread = 1) {
  return (unsigned)ceil_div64(ceil_div64(n, per_thread), 256);
}

}  // namespace

size_t grad_norm_workspace_bytes() { return (kNormBlocks + 2) * sizeof(float); }

int grad_norm(int64_t n, const float* grad, float max_norm, float* workspace, hipStream_t stream) {
  if (n < 0 || !grad || !workspace) return gpt2_internal_fail(1, "grad_norm: bad arguments");
  if ((uintptr_t)grad % 16) return gpt2_internal_fail(1, "grad_norm: gradient must be 16-byte aligned");
  mark_begin(0, stream);
  hipLaunchKernelGGL(grad_sumsq_kernel, dim3(kNormBlocks), dim3(256), 0, stream, n, grad, workspace + 2);
  GPT2_LAUNCH_CHECK();
  mark_end(0, stream);
  hipLaunchKernelGGL(grad_norm_finalize_kernel, dim3(1), dim3(256), 0, stream, workspace + 2, kNormBlocks,
                     max_norm, workspace);
  GPT2_LAUNCH_CHECK();
  return 0;
}

AdamHP adam_hparams(float lr, float beta1, float beta2, float eps, float wd, int t) {
  AdamHP h;
  h.lr = lr; h.b1 = beta1; h.b2 = beta2; h.eps = eps; h.wd = wd;
  h.c1 = (float)(1.0 / (1.0 - pow((double)beta1, (double)t)));
  h.c2 = (float)(1.0 / (1.0 - pow((double)beta2, (double)t)));
  return h;
}

int set_adam_hparams(AdamHP* dst, const AdamHP& v, hipStream_t stream) {
  if (!dst) return gpt2_internal_fail(1, "set_adam_hparams: NULL destination");
  hipLaunchKernelGGL(set_adam_hp_kernel, dim3(1), dim3(1), 0, stream, dst, v);
  GPT2_LAUNCH_CHECK();
  return 0;
}

int adamw(int64_t n, float* master, const float* grad, float* m, float* v, bf16* param_bf16, float lr,
          float beta1, float beta2, float eps, float wd, int t, hipStream_t stream, const float* gscale,
          const AdamHP* hp_dev) {
  if (n < 0 || !master || !grad || !m || !v || t < 1) return gpt2_internal_fail(1, "adamw: bad arguments");
  if (n == 0) return 0;
  if (((uintptr_t)master | (uintptr_t)grad | (uintptr_t)m | (uintptr_t)v) % 16 ||
      (param_bf16 && (uintptr_t)param_bf16 % 8))
    return gpt2_internal_fail(1, "adamw: buffers must be 16-byte aligned");
  const AdamHP hp = adam_hparams(lr, beta1, beta2, eps, wd, t);
  unsigned grid = (unsigned)std::min<int64_t>(ceil_div64(n, 4 * 256), 8192);
  mark_begin(0, stream);
  hipLaunchKernelGGL(adamw_kernel, dim3(grid), dim3(256), 0, stream, n, master, grad, m, v, param_bf16, hp, hp_dev,
                     gscale);
  GPT2_LAUNCH_CHECK();
  mark_end(0, stream);
  return 0;
}

int adamw_transposed(int64_t n, float* master, const float* grad, float* m, float* v, bf16* param_bf16,
                     const AdamMatrix* mats, int nmats, hipStream_t stream, const float* gscale,
                     const AdamHP* hp_dev) {
  if (n < 0 || !master || !grad || !m || !v || !param_bf16 || !hp_dev || nmats < 0 || nmats > kAdamMaxMats ||
      (nmats && !mats))
    return gpt2_internal_fail(1, "adamw_transposed: bad arguments");
  if (((uintptr_t)master | (uintptr_t)grad | (uintptr_t)m | (uintptr_t)v) % 16 || (uintptr_t)param_bf16 % 8)
    return gpt2_internal_fail(1, "adamw_transposed: buffers must be 16-byte aligned");
  AdamSegs sg{};
  sg.nmat = nmats;
  int64_t prev_end = 0;
  int total_tiles = 0;
  for (int k = 0; k < nmats; ++k) {
    AdamMatrix mt = mats[k];
    const int64_t len = (int64_t)mt.batches * mt.R * mt.Cc;
    if (mt.off < prev_end || mt.off + len > n || mt.R <= 0 || mt.Cc <= 0 || mt.R % 8 || mt.Cc % 4 || mt.off % 4 ||
        (!mt.dst_t && !mt.amax) || (uintptr_t)mt.dst_t % 16)
      return gpt2_internal_fail(1, "adamw_transposed: matrix %d not in order, unaligned or out of range", k);
    if (mt.off > prev_end) {
      if (sg.nflat == kAdamMaxMats + 1) return gpt2_internal_fail(1, "adamw_transposed: too many ranges");
      sg.flat_off[sg.nflat] = prev_end;
      sg.flat_len[sg.nflat++] = mt.off - prev_end;
    }
    mt.tiles = mt.batches * ((mt.R + 63) / 64) * ((mt.Cc + 63) / 64);
    total_tiles += mt.tiles;
    sg.mat[k] = mt;
    prev_end = mt.off + len;
  }
  if (n > prev_end) {
    if (sg.nflat == kAdamMaxMats + 1) return gpt2_internal_fail(1, "adamw_transposed: too many ranges");
    sg.flat_off[sg.nflat] = prev_end;
    sg.flat_len[sg.nflat++] = n - prev_end;
  }
  for (int r = 0; r < sg.nflat; ++r) {
    if (sg.flat_off[r] % 4 || sg.flat_len[r] % 4)
      return gpt2_internal_fail(1, "adamw_transposed: flat range %d not a multiple of 4 elements", r);
    sg.flat_total += sg.flat_len[r];
  }
  sg.flat_blocks = (int)std::min<int64_t>(ceil_div64(sg.flat_total, 4 * 256), 2048);
  const unsigned grid = (unsigned)(sg.flat_blocks + total_tiles);
  if (grid == 0) return 0;
  mark_begin(0, stream);
  hipLaunchKernelGGL(adamw_fused_kernel, dim3(grid), dim3(256), 0, stream, sg, master, grad, m, v, param_bf16,
                     AdamHP{}, hp_dev, gscale);
  GPT2_LAUNCH_CHECK();
  mark_end(0, stream);
  return 0;
}

int copy_i32(int64_t n, const int32_t* src, int32_t* dst, hipStream_t stream) {
  if (n <= 0) return 0;
  if (!src || !dst) return gpt2_internal_fail(1, "copy_i32: NULL buffer");
  hipLaunchKernelGGL(copy_i32_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, n, src, dst);
  GPT2_LAUNCH_CHECK();
  return 0;
}

int cast_f32_to_bf16(int64_t n, const float* src, bf16* dst, hipStream_t stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(cast_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, n, src, dst);
  GPT2_LAUNCH_CHECK();
  return 0;
}

int transpose_bf16(int batches, int R, int Cc, const bf16* src, bf16* dst, hipStream_t stream) {
  if (batches < 0 || R < 0 || Cc < 0 || (R % 8) || (Cc % 8) || !src || !dst)
    return gpt2_internal_fail(1, "transpose_bf16: bad arguments (R=%d, C=%d must be multiples of 8)", R, Cc);
  if (batches == 0 || R == 0 || Cc == 0) return 0;
  dim3 grid((unsigned)ceil_div64(Cc, 64), (unsigned)ceil_div64(R, 64), (unsigned)batches);
  mark_begin(0, stream);
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, stream, src, dst, R, Cc);
  GPT2_LAUNCH_CHECK();
  mark_end(0, stream);
  return 0;
}

int init_normal(int64_t n, float* dst, uint64_t seed, int tensor_index, double stddev, hipStream_t stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(init_normal_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, n, dst, seed,
                     (uint64_t)tensor_index, stddev);
  GPT2_LAUNCH_CHECK();
  return 0;
}

int fill_f32(int64_t n, float* dst, float value, hipStream_t stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, n, dst, value);
  GPT2_LAUNCH_CHECK();
  return 0;
}

int convert_to_f32(int dtype, int64_t n, const void* src, float* dst, hipStream_t stream) {
  if (n <= 0) return 0;
  if (dtype == BF16) {
    hipLaunchKernelGGL(bf16_to_f32_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, n, (const bf16*)src, dst);
    GPT2_LAUNCH_CHECK();
    return 0;
  }
  GPT2_HIP_CHECK(hipMemcpyAsync(dst, src, n * sizeof(float), hipMemcpyDeviceToDevice, stream));
  return 0;
}

}  // namespace gpt2k
