// Device and host helpers shared by the GPT-2 HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <algorithm>

typedef __bf16 bf16;

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// ---------------------------------------------------------------- 8-wide vectors
// One "chunk" is 8 consecutive elements: 16 bytes of bf16 or 32 bytes of fp32.

template <typename T> struct Chunk8;

template <> struct Chunk8<float> {
  __device__ __forceinline__ static void load(const float* p, float v[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store(float* p, const float v[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

template <> struct Chunk8<bf16> {
  __device__ __forceinline__ static void load(const bf16* p, float v[8]) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void store(bf16* p, const float v[8]) {
    typedef bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    bf16x8_t o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
    *reinterpret_cast<bf16x8_t*>(p) = o;
  }
};

// ---------------------------------------------------------------- reductions

// Producers of a tensor that is quantised to fp8 next leave their maxima in
// kAmaxWays slots, kAmaxStride floats apart (each slot on a 128-byte line of
// its own, so atomics on different slots do not queue on one line); the
// quantisation takes the maximum of the slots.
constexpr int kAmaxWays = 64;
constexpr int kAmaxStride = 32;

// slot i % kAmaxWays of `slots` = max(itself, m) for m >= 0 (not NaN): the
// bit patterns of non-negative floats order like the values, so an integer
// atomic maximum gives the same result in any order.  m is first rounded to
// bf16 (rounding is monotonic, so this is the maximum of the rounded values a
// bf16 tensor holds).
__device__ __forceinline__ void amax_atomic_bf16(float* slots, int i, float m) {
  const uint32_t b = __float_as_uint(m);
  const uint32_t r = ((b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u);   // round to nearest even
  atomicMax(reinterpret_cast<unsigned int*>(slots + (i % kAmaxWays) * kAmaxStride), r);
}
// The same for an fp32 tensor: m is max-ed in exactly.
__device__ __forceinline__ void amax_atomic_f32(float* slots, int i, float m) {
  atomicMax(reinterpret_cast<unsigned int*>(slots + (i % kAmaxWays) * kAmaxStride), __float_as_uint(m));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------- math

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// GELU, tanh form (0.5 u (1 + tanh z), z = k0 (u + k1 u^3)), and its
// derivative, from one exponential, in the logistic form: with z = k0 (u + k1 u^3) and s = 1 / (1 + e^{-2z}),
// 1 + tanh z = 2 s and 1 - tanh^2 z = 4 s (1 - s), so
//   GELU(u) = u s,   GELU'(u) = s (1 + 2 u (1 - s) dz/du),
// dz/du = k0 (1 + 3 k1 u^2).  Eleven VALU operations besides v_exp_f32 and
// v_rcp_f32 (the fc forward's epilogue evaluates this per output element).
// Saturates: e^{-2z} -> inf gives s = 0 (GELU and GELU' 0), -> 0 gives s = 1.
__device__ __forceinline__ void gelu_tanh_and_grad_f(float u, float& g, float& d) {
  const float k0 = 0.7978845608028654f, k1 = 0.044715f;
  const float u2 = u * u;
  const float zu = u * fmaf(k1, u2, 1.0f);                                   // z / k0
  const float e = __builtin_amdgcn_exp2f(zu * (-2.0f * k0 * 1.4426950408889634f));  // e^{-2z}
  const float sg = __builtin_amdgcn_rcpf(1.0f + e);
  const float w = u * fmaf(6.0f * k0 * k1, u2, 2.0f * k0);                  // 2 u dz/du
  g = u * sg;
  d = sg * fmaf(w, 1.0f - sg, 1.0f);
}

// ---------------------------------------------------------------- host side

// ---------------------------------------------------------------- gfx950 memory helpers

// LDS address space (direct-to-LDS loads and LDS-only reads take such pointers).
#define GPT2_LDS __attribute__((address_space(3)))

// Buffer resource over `bytes` bytes from `base`: loads at offsets at or beyond
// `bytes` return zeros (and direct-to-LDS loads write zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The same resource as four dwords (base address bits 0-31 and 32-47, the
// byte range, the format word) for the inline-assembly DMA below.
typedef int i32x4_rsrc __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_rsrc make_rsrc4(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(size_t)base;
  i32x4_rsrc r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// Direct-to-LDS load of 16 bytes per lane: lane i's bytes at `voffset` (range
// checked against the resource) land at lds + 16 i.  Issued as inline
// assembly so that the compiler neither waits for it nor holds later LDS
// reads behind it (for the builtin form it puts a full vmcnt(0) wait in front
// of the next LDS read, which drains every later pipeline stage too).  The
// caller owns the synchronisation: wait_vmcnt for its own lanes' data, then a
// barrier before other waves read it.  `lds` must be wave-uniform.
// M0 is listed as clobbered so that the scheduler orders the statement after
// any earlier set-up of M0 and before any later one (the compiler sets M0
// right before each of its own uses; it has no value to preserve across this).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_lds16(i32x4_rsrc rsrc, GPT2_LDS void* lds, uint32_t voffset) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :: "v"(voffset), "s"(m0), "s"(rsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate that waits until at most N vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations
// (lgkmcnt) but, unlike __syncthreads(), not for its outstanding global loads,
// so that loads of later pipeline stages stay in flight across it.  A wave
// must have waited (vmcnt) for any LDS data its DMA wrote and others read.
// (The s_barrier intrinsic and __syncthreads() get a full vmcnt(0) wait in
// front of them from the compiler; the inline form keeps only the LDS wait.
// Its memory clobber stops the compiler from moving memory accesses across it.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

#define GPT2_HIP_CHECK(expr)                                  \
  do {                                                        \
    hipError_t _e = (expr);                                   \
    if (_e != hipSuccess) return gpt2_internal_hip_fail(_e, #expr, __FILE__, __LINE__); \
  } while (0)

#define GPT2_LAUNCH_CHECK() GPT2_HIP_CHECK(hipGetLastError())

int gpt2_internal_hip_fail(hipError_t e, const char* expr, const char* file, int line);
int gpt2_internal_fail(int status, const char* fmt, ...);

static inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }
