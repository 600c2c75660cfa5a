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
constexpr float kLog2eCe = 1.4426950408889634f;

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

// bf16 logits: the same result with far fewer vector instructions per
// element (the generic form is bound by them rather than by HBM).  Per
// element: the bf16 -> fp32 widening is a shift or mask, the exponential is
// exp2 of one fused multiply-add, and it is kept in fp16 (relative to the
// thread's own maximum, so in (0, 1]) in the registers that held the row, for
// the write: g_j = e_j * exp(m_t - m) * dscale / s with the bracket one
// per-thread constant.  The block reduction takes the maximum first, then
// each thread rescales its sum once (one exponential per thread instead of
// one per combining step).  Requires Vp <= NC * 8192 and (NC - 1) * 8192 <= V:
// chunks c < NC - 1 are then whole columns j < V for every thread, and only
// chunk NC - 1 checks the row end and the padding.  The label's -dscale is
// applied afterwards by the thread that holds the label, with a 2-byte store
// over its chunk.
// AM: also the maximum |dz| of the row (as stored) into the amax slots, for
// the fp8 quantisation of the dlogits.
template <int NC, bool AM>
__global__ __launch_bounds__(kCeThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void softmax_xent_bf16_kernel(int V, int Vp, bf16* __restrict__ logits,
                                                                       const int32_t* __restrict__ labels,
                                                                       float* __restrict__ losses, float dscale,
                                                                       float* __restrict__ amax) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __shared__ float shm[kCeWaves], shs[kCeWaves];
  __shared__ float s_zy;
  const int row = blockIdx.x, tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  bf16* z = logits + (size_t)row * Vp;
  int y = labels[row];
  y = y < 0 ? 0 : (y >= V ? V - 1 : y);   // memory safety only; valid labels are in [0, V)
  const int nch = Vp / 8, ych = y >> 3;
  constexpr int L = NC - 1;                // the one chunk that may be partial or absent
  const int chL = tid + kCeThreads * L;
  const bool hasL = chL < nch;
  // the row, two bf16 per word (element 2k in the low half of word k); buffer
  // loads and stores with the chunk offset in a scalar register keep one
  // address register per thread
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(z, (uint32_t)Vp * 2u);
  const int voff = tid * 16;
  uint32_t w[NC][4];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c < L || hasL) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, kCeThreads * 16 * c, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) w[c][k] = v[k];
    }
  }
  auto lo = [](uint32_t u) { return __uint_as_float(u << 16); };
  auto hi = [](uint32_t u) { return __uint_as_float(u & 0xffff0000u); };
  // label logit, from the registers of the thread that holds it
  bool owner = false;
  float zy = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (tid + kCeThreads * c == ych) {
      owner = true;
      uint32_t u = w[c][0];
#pragma unroll
      for (int k = 1; k < 4; ++k) u = ((y & 7) >> 1) == k ? w[c][k] : u;
      zy = (y & 1) ? hi(u) : lo(u);
      s_zy = zy;
    }
  }
  float mt = -INFINITY;
#pragma unroll
  for (int c = 0; c < L; ++c)
#pragma unroll
    for (int k = 0; k < 4; ++k) mt = fmaxf(mt, fmaxf(lo(w[c][k]), hi(w[c][k])));
  if (hasL) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (chL * 8 + 2 * k < V) mt = fmaxf(mt, lo(w[L][k]));
      if (chL * 8 + 2 * k + 1 < V) mt = fmaxf(mt, hi(w[L][k]));
    }
  }
  // the widened values of the maximum pass are not kept for the exponentials
  // (56 more live registers); re-deriving them is one shift or mask each
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(w[c][k]));
  const float ml2 = mt * kLog2eCe;
  float st = 0.f;
  // exponentials of one word's pair, summed and returned as two fp16 (RNE)
  auto exps = [&](uint32_t u, bool ok0, bool ok1) -> uint32_t {
    float e0 = __builtin_amdgcn_exp2f(fmaf(lo(u), kLog2eCe, -ml2));
    float e1 = __builtin_amdgcn_exp2f(fmaf(hi(u), kLog2eCe, -ml2));
    e0 = ok0 ? e0 : 0.f;
    e1 = ok1 ? e1 : 0.f;
    st += e0 + e1;
    const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)e0);
    const uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)e1);
    return h0 | (h1 << 16);
  };
  // (scheduling barriers between chunks keep the live range of the
  // temporaries to one chunk, so the kernel fits 64 registers: 2 blocks per CU)
#pragma unroll
  for (int c = 0; c < L; ++c) {
#pragma unroll
    for (int k = 0; k < 4; ++k) w[c][k] = exps(w[c][k], true, true);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (hasL) {
#pragma unroll
    for (int k = 0; k < 4; ++k) w[L][k] = exps(w[L][k], chL * 8 + 2 * k < V, chL * 8 + 2 * k + 1 < V);
  }
  // the packed exponentials are formed here, not sunk into the write pass
  // (which would keep 56 fp32 values live across the reduction)
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(w[c][k]));
  float mb = mt;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mb = fmaxf(mb, __shfl_xor(mb, o, 64));
  if (lane == 0) shm[wv] = mb;
  __syncthreads();                          // also makes s_zy visible
#pragma unroll
  for (int i = 0; i < kCeWaves; ++i) mb = fmaxf(mb, shm[i]);
  const float r = __builtin_amdgcn_exp2f((mt - mb) * kLog2eCe);   // 0 for a thread with no columns
  const float sw = wave_sum(st * r);
  if (lane == 0) shs[wv] = sw;
  __syncthreads();
  float sb = 0.f;
#pragma unroll
  for (int i = 0; i < kCeWaves; ++i) sb += shs[i];
  if (tid == 0) losses[row] = mb + logf(sb) - s_zy;
  const float scale = r * (dscale / sb);
  uint32_t m16 = 0;   // AM: largest bf16 magnitude written (bits), the label's old entry excluded
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c < L || hasL) {
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float g0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[c][k] & 0xffffu)) * scale;
        const float g1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[c][k] >> 16)) * scale;
        const uint32_t b0 = __builtin_bit_cast(uint16_t, (bf16)g0);
        const uint32_t b1 = __builtin_bit_cast(uint16_t, (bf16)g1);
        o[k] = b0 | (b1 << 16);
        if constexpr (AM) {
          const bool lab = tid + kCeThreads * c == ych && k == ((y & 7) >> 1);
          m16 = max(m16, (lab && !(y & 1)) ? 0u : (b0 & 0x7fffu));
          m16 = max(m16, (lab && (y & 1)) ? 0u : (b1 & 0x7fffu));
        }
      }
      __builtin_amdgcn_raw_buffer_store_b128(o, rs, voff, kCeThreads * 16 * c, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (owner) {
    const bf16 zl = (bf16)(__builtin_amdgcn_exp2f(fmaf(zy, kLog2eCe, -ml2)) * scale - dscale);
    z[y] = zl;
    if constexpr (AM) m16 = max(m16, (uint32_t)__builtin_bit_cast(uint16_t, zl) & 0x7fffu);
  }
  if constexpr (AM) {
    __shared__ float sam[kCeWaves];
    const float mw = wave_max(__uint_as_float(m16 << 16));
    if (lane == 0) sam[wv] = mw;
    __syncthreads();
    if (tid == 0) {
      float mb2 = 0.f;
#pragma unroll
      for (int i = 0; i < kCeWaves; ++i) mb2 = fmaxf(mb2, sam[i]);
      amax_atomic_bf16(amax, row, mb2);   // already a bf16 value: rounding leaves it
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

bool bf16_kernel_fits(int V, int Vp) {
  const int need = (Vp / 8 + kCeThreads - 1) / kCeThreads;
  return need <= 7 && 6 * 8 * kCeThreads <= V;   // the bf16 kernel's precondition for NC = 7
}

template <typename T>
int launch_t(int N, int V, int Vp, void* logits, const int32_t* labels, float* losses, float dscale, float* amax,
             hipStream_t s) {
  const int nch = Vp / 8;
  const int need = (nch + kCeThreads - 1) / kCeThreads;
  T* L = (T*)logits;
  mark_begin(0, s);
  if constexpr (sizeof(T) == 2) {
    if (bf16_kernel_fits(V, Vp)) {
      if (amax)
        hipLaunchKernelGGL((softmax_xent_bf16_kernel<7, true>), dim3(N), dim3(kCeThreads), 0, s, V, Vp, L, labels,
                           losses, dscale, amax);
      else
        hipLaunchKernelGGL((softmax_xent_bf16_kernel<7, false>), dim3(N), dim3(kCeThreads), 0, s, V, Vp, L, labels,
                           losses, dscale, amax);
      GPT2_LAUNCH_CHECK();
      mark_end(0, s);
      return 0;
    }
  }
  if (amax) return gpt2_internal_fail(1, "softmax_xent: the dlogits maximum needs the bf16 full-vocabulary kernel");
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
                 float dscale, hipStream_t stream, float* amax) {
  if (N < 0 || V <= 0 || Vp < V || Vp % 8 || !logits || !labels || !losses)
    return gpt2_internal_fail(1, "softmax_xent: bad arguments");
  if (N == 0) return 0;
  return dtype == BF16 ? launch_t<bf16>(N, V, Vp, logits, labels, losses, dscale, amax, stream)
                       : launch_t<float>(N, V, Vp, logits, labels, losses, dscale, amax, stream);
}

bool softmax_xent_has_amax(int dtype, int V, int Vp) { return dtype == BF16 && bf16_kernel_fits(V, Vp); }

int sum_scaled(int n, const float* x, float scale, float* out, hipStream_t stream) {
  if (n < 0 || !x || !out) return gpt2_internal_fail(1, "sum_scaled: bad arguments");
  hipLaunchKernelGGL(sum_scaled_kernel, dim3(1), dim3(1024), 0, stream, n, x, scale, out);
  GPT2_LAUNCH_CHECK();
  return 0;
}

}  // namespace gpt2k
