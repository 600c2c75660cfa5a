// GEMMs of the GPT-2 step: the four linear layers of each block, the tied
// classifier, and their dX / dW backward passes.
//
// The kernel table of "State of the Union [May 3, 2024]" (section "Runtime,
// DRAM traffic, instructions") attributes most of a step to these GEMMs
// (vendor-library kernels there) plus separate bias-gradient, GELU and
// residual kernels.  Here one hand-written bf16 MFMA kernel covers every GEMM
// of the step, with those elementwise pieces fused into its epilogue and the
// bias gradient fused into the weight-gradient pass.
//
// bf16 kernel (gfx950):
//   * block tile 128 x 128, K step 64, 256 threads = 4 waves in a 2 x 2
//     grid, each wave 64 x 64 = 2 x 2 tiles of v_mfma_f32_32x32x16_bf16;
//   * LDS holds both operands as [row][k] bf16 rows of 64 (128 bytes) with
//     16-byte chunks XOR-swizzled by row, so the MFMA operand reads
//     (ds_read_b128, 32 rows per half-wave) are bank-conflict free;
//   * operands whose K axis is strided in memory (dY^T and X in dW = dY^T X,
//     W in dX = dY W) are loaded as 16-byte runs along their contiguous axis
//     and transposed in registers before the LDS store;
//   * double-buffered LDS: the global loads of step k+1 are in flight while
//     step k runs on the matrix cores, one barrier per step;
//   * dW splits K (the B*T positions) over grid.z into fp32 partial tiles that
//     a second kernel sums in a fixed order, so results are deterministic.
// fp32 kernel (parity mode): plain LDS-tiled FMA GEMM with the same epilogues.

#include "kernels.h"

namespace gpt2k {
namespace {

typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;          // K step of the MFMA kernel
constexpr int kThreads = 256;

struct EpiArgs {
  int epi;
  int M, N;
  void* C; int64_t ldc;
  const void* bias;
  const void* aux_in; int64_t ld_aux;
  void* aux_out;
  float* partial;        // [splits][M][N]
  float* partial_bias;   // [splits][M]
};

template <int EPI, typename T>
__device__ __forceinline__ void epilogue_store(const EpiArgs& e, int m, int n, float v, int z) {
  if constexpr (EPI == EPI_WGRAD) {
    e.partial[((size_t)z * e.M + m) * (size_t)e.N + n] = v;
  } else {
    if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_RES || EPI == EPI_BIAS_GELU)
      v += to_f32(reinterpret_cast<const T*>(e.bias)[n]);
    if constexpr (EPI == EPI_BIAS_RES)
      v += to_f32(reinterpret_cast<const T*>(e.aux_in)[(size_t)m * e.ld_aux + n]);
    if constexpr (EPI == EPI_BIAS_GELU) {
      reinterpret_cast<T*>(e.aux_out)[(size_t)m * e.ldc + n] = from_f32<T>(v);
      v = gelu_tanh_f(v);
    }
    if constexpr (EPI == EPI_GELU_BWD)
      v *= gelu_tanh_grad_f(to_f32(reinterpret_cast<const T*>(e.aux_in)[(size_t)m * e.ld_aux + n]));
    reinterpret_cast<T*>(e.C)[(size_t)m * e.ldc + n] = from_f32<T>(v);
  }
}

// ---------------------------------------------------------------- bf16 MFMA

// Physical 16-byte chunk of logical chunk c (0..7) in LDS row `row`.
__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row ^ (row >> 3)) & 7); }

struct MfmaArgs {
  const bf16* A; int64_t lda;
  const bf16* B; int64_t ldb;
  int M, N, K;
  int k_per_split;
  EpiArgs e;
};

// Register staging of one operand tile: R rows (the M or N axis) x 64 k.
template <int R, bool KMAJ>
struct Stager {
  static constexpr int NLD = R / 32;  // 16-byte global loads per thread
  uint4 r[NLD];

  // rows [row0, row0 + R) of the operand, k in [k0, k0 + 64); rows >= nrows and
  // k >= K read as 0 (K is a multiple of 8, so a 16-byte run never straddles K).
  __device__ __forceinline__ void load(const bf16* __restrict__ G, int64_t ld, int row0, int nrows,
                                       int k0, int K, int tid) {
    if constexpr (KMAJ) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        int row = tid / 8 + 32 * i, c = tid % 8;
        if (row0 + row < nrows && k0 + c * 8 < K)
          r[i] = *reinterpret_cast<const uint4*>(G + (size_t)(row0 + row) * ld + k0 + c * 8);
        else
          r[i] = make_uint4(0, 0, 0, 0);
      }
    } else {
      // unit u: 8 consecutive rows (contiguous in memory) x 4 consecutive k.
#pragma unroll
      for (int j = 0; j < R / 128; ++j) {
        int u = tid + kThreads * j;
        int mc = u % (R / 8), kg = u / (R / 8);
        bool ok = row0 + mc * 8 < nrows;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = k0 + kg * 4 + i;
          if (ok && k < K)
            r[j * 4 + i] = *reinterpret_cast<const uint4*>(G + (size_t)k * ld + row0 + mc * 8);
          else
            r[j * 4 + i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  __device__ __forceinline__ void store(bf16* S, int tid) const {
    if constexpr (KMAJ) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        int row = tid / 8 + 32 * i, c = tid % 8;
        *reinterpret_cast<uint4*>(S + row * kBK + swz(row, c) * 8) = r[i];
      }
    } else {
#pragma unroll
      for (int j = 0; j < R / 128; ++j) {
        int u = tid + kThreads * j;
        int mc = u % (R / 8), kg = u / (R / 8);
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[j * 4 + 0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[j * 4 + 1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[j * 4 + 2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[j * 4 + 3]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t lo, hi;
          if (e % 2 == 0) {  // low halves of dword e/2
            lo = (w0[e / 2] & 0xffffu) | (w1[e / 2] << 16);
            hi = (w2[e / 2] & 0xffffu) | (w3[e / 2] << 16);
          } else {           // high halves
            lo = (w0[e / 2] >> 16) | (w1[e / 2] & 0xffff0000u);
            hi = (w2[e / 2] >> 16) | (w3[e / 2] & 0xffff0000u);
          }
          int row = mc * 8 + e;
          *reinterpret_cast<uint2*>(S + row * kBK + swz(row, kg / 2) * 8 + (kg % 2) * 4) =
              make_uint2(lo, hi);
        }
      }
    }
  }

  // Adds the staged values of each of this thread's rows into acc (M-major only).
  __device__ __forceinline__ void accumulate_rows(float* acc) const {
#pragma unroll
    for (int j = 0; j < R / 128; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(&r[j * 4 + i]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[j * 8 + e] += (e % 2 == 0) ? __uint_as_float(w[e / 2] << 16)
                                         : __uint_as_float(w[e / 2] & 0xffff0000u);
      }
  }
};

template <int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI, bool BIAS_GRAD>
__global__ __launch_bounds__(kThreads) void gemm_bf16_mfma_kernel(MfmaArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
  constexpr int TILE = (BM + BN) * kBK;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int kbeg = blockIdx.z * p.k_per_split;
  const int KT = p.k_per_split / kBK;
  const bool do_bias = BIAS_GRAD && blockIdx.x == 0;

  Stager<BM, A_KMAJ> sa;
  Stager<BN, B_KMAJ> sb;
  float bsum[BIAS_GRAD ? 8 * (BM / 128) : 1];
  if constexpr (BIAS_GRAD) {
#pragma unroll
    for (int i = 0; i < 8 * (BM / 128); ++i) bsum[i] = 0.f;
  }

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  sa.load(p.A, p.lda, m0, p.M, kbeg, p.K, tid);
  sb.load(p.B, p.ldb, n0, p.N, kbeg, p.K, tid);
  sa.store(smem, tid);
  sb.store(smem + BM * kBK, tid);
  if constexpr (BIAS_GRAD) if (do_bias) sa.accumulate_rows(bsum);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const bf16* As = smem + (kt & 1) * TILE;
    const bf16* Bs = As + BM * kBK;
    const bool more = kt + 1 < KT;
    if (more) {
      sa.load(p.A, p.lda, m0, p.M, kbeg + (kt + 1) * kBK, p.K, tid);
      sb.load(p.B, p.ldb, n0, p.N, kbeg + (kt + 1) * kBK, p.K, tid);
    }
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 a[FM], b[FN];
      const int c = kk * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        int row = wm * WM + i * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const bf16x8*>(As + row * kBK + swz(row, c) * 8);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        int row = wn * WN + j * 32 + (lane & 31);
        b[j] = *reinterpret_cast<const bf16x8*>(Bs + row * kBK + swz(row, c) * 8);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      bf16* An = smem + ((kt + 1) & 1) * TILE;
      sa.store(An, tid);
      sb.store(An + BM * kBK, tid);
      if constexpr (BIAS_GRAD) if (do_bias) sa.accumulate_rows(bsum);
    }
    __syncthreads();
  }

  // Epilogue.  Accumulator element r of lane l in a 32 x 32 tile is at
  // row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32.
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WN + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WM + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
        if (row < p.M && col < p.N) epilogue_store<EPI, bf16>(p.e, row, col, acc[i][j][r], blockIdx.z);
      }
    }

  if constexpr (BIAS_GRAD) {
    if (do_bias) {
      // reduce bsum over the 16 k-groups that share each row chunk
      float* red = reinterpret_cast<float*>(smem);   // [16][BM]
#pragma unroll
      for (int j = 0; j < BM / 128; ++j) {
        int u = tid + kThreads * j;
        int mc = u % (BM / 8), kg = u / (BM / 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) red[kg * BM + mc * 8 + e] = bsum[j * 8 + e];
      }
      __syncthreads();
      for (int m = tid; m < BM; m += kThreads) {
        float s = 0.f;
#pragma unroll
        for (int kg = 0; kg < 16; ++kg) s += red[kg * BM + m];
        if (m0 + m < p.M) p.e.partial_bias[(size_t)blockIdx.z * p.M + m0 + m] = s;
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 SIMT

struct SimtArgs {
  const float* A; int64_t lda;
  const float* B; int64_t ldb;
  int M, N, K;
  int k_per_split;
  EpiArgs e;
};

template <bool A_KMAJ, bool B_KMAJ, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_simt_kernel(SimtArgs p) {
  constexpr int BM = 64, BN = 64, BKs = 16;
  __shared__ float As[BKs][BM + 4];
  __shared__ float Bs[BKs][BN + 4];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int kbeg = blockIdx.z * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += BKs) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int idx = tid + 256 * e;
      int m, k;
      if (A_KMAJ) { m = idx / BKs; k = idx % BKs; } else { m = idx % BM; k = idx / BM; }
      int gm = m0 + m, gk = k0 + k;
      float v = 0.f;
      if (gm < p.M && gk < kend)
        v = A_KMAJ ? p.A[(size_t)gm * p.lda + gk] : p.A[(size_t)gk * p.lda + gm];
      As[k][m] = v;
      int n;
      if (B_KMAJ) { n = idx / BKs; k = idx % BKs; } else { n = idx % BN; k = idx / BN; }
      int gn = n0 + n;
      gk = k0 + k;
      v = 0.f;
      if (gn < p.N && gk < kend)
        v = B_KMAJ ? p.B[(size_t)gn * p.ldb + gk] : p.B[(size_t)gk * p.ldb + gn];
      Bs[k][n] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BKs; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int m = m0 + ty + 16 * i, n = n0 + tx + 16 * j;
      if (m < p.M && n < p.N) epilogue_store<EPI, float>(p.e, m, n, acc[i][j], blockIdx.z);
    }
}

// fp32 bias gradient for the parity path: out[m] (+)= sum_k A[k * lda + m].
__global__ void colsum_f32_kernel(const float* A, int64_t lda, int M, int K, float* out, bool acc) {
  int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s += A[(size_t)k * lda + m];
  out[m] = acc ? out[m] + s : s;
}

// ---------------------------------------------------------------- split-K reduce

__global__ void wgrad_reduce_kernel(const float* __restrict__ partial, int splits, int64_t MN,
                                    float* __restrict__ out, bool accumulate) {
  int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= MN) return;
  if (i4 + 4 <= MN && (MN % 4) == 0) {
    float4 s = accumulate ? *reinterpret_cast<const float4*>(out + i4) : make_float4(0, 0, 0, 0);
    for (int z = 0; z < splits; ++z) {
      float4 v = *reinterpret_cast<const float4*>(partial + (size_t)z * MN + i4);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    *reinterpret_cast<float4*>(out + i4) = s;
  } else {
    for (int64_t i = i4; i < MN && i < i4 + 4; ++i) {
      float s = accumulate ? out[i] : 0.f;
      for (int z = 0; z < splits; ++z) s += partial[(size_t)z * MN + i];
      out[i] = s;
    }
  }
}

// ---------------------------------------------------------------- dispatch

// Number of K splits of a WGRAD GEMM: enough blocks to fill the chip twice.
int wgrad_splits(int dtype, int M, int N, int K) {
  if (dtype == F32) return 1;
  int tiles = (int)(ceil_div64(M, 128) * ceil_div64(N, 128));
  int kt = (int)ceil_div64(K, kBK);
  int want = (512 + tiles - 1) / tiles;
  int s = 1;
  for (int c = 1; c <= kt && c <= 64; ++c)
    if (kt % c == 0 && c <= want) s = c;
  return s;
}

template <int EPI, bool A_KMAJ, bool B_KMAJ, bool BIAS_GRAD>
int launch_mfma(const MfmaArgs& a, int splits, hipStream_t stream) {
  dim3 grid((unsigned)ceil_div64(a.N, 128), (unsigned)ceil_div64(a.M, 128), (unsigned)splits);
  hipLaunchKernelGGL((gemm_bf16_mfma_kernel<128, 128, A_KMAJ, B_KMAJ, EPI, BIAS_GRAD>), grid,
                     dim3(kThreads), 0, stream, a);
  GPT2_LAUNCH_CHECK();
  return 0;
}

template <int EPI, bool A_KMAJ, bool B_KMAJ>
int launch_simt(const SimtArgs& a, int splits, hipStream_t stream) {
  dim3 grid((unsigned)ceil_div64(a.N, 64), (unsigned)ceil_div64(a.M, 64), (unsigned)splits);
  hipLaunchKernelGGL((gemm_f32_simt_kernel<A_KMAJ, B_KMAJ, EPI>), grid, dim3(256), 0, stream, a);
  GPT2_LAUNCH_CHECK();
  return 0;
}

template <int EPI>
int dispatch_layout_bf16(const GemmDesc& d, const MfmaArgs& a, int splits, bool bias_grad,
                         hipStream_t s) {
  if (d.a_kmajor && d.b_kmajor) return launch_mfma<EPI, true, true, false>(a, splits, s);
  if (d.a_kmajor && !d.b_kmajor) return launch_mfma<EPI, true, false, false>(a, splits, s);
  if (!d.a_kmajor && !d.b_kmajor) {
    if (bias_grad) return launch_mfma<EPI, false, false, true>(a, splits, s);
    return launch_mfma<EPI, false, false, false>(a, splits, s);
  }
  return gpt2_internal_fail(1, "gemm: layout (A m-major, B k-major) is not instantiated");
}

template <int EPI>
int dispatch_layout_f32(const GemmDesc& d, const SimtArgs& a, int splits, hipStream_t s) {
  if (d.a_kmajor && d.b_kmajor) return launch_simt<EPI, true, true>(a, splits, s);
  if (d.a_kmajor && !d.b_kmajor) return launch_simt<EPI, true, false>(a, splits, s);
  if (!d.a_kmajor && !d.b_kmajor) return launch_simt<EPI, false, false>(a, splits, s);
  return launch_simt<EPI, false, true>(a, splits, s);
}

}  // namespace

size_t gemm_workspace_bytes(int dtype, int epi, int M, int N, int K) {
  if (epi != EPI_WGRAD) return 0;
  int s = wgrad_splits(dtype, M, N, K);
  return (size_t)s * ((size_t)M * N + (size_t)M) * sizeof(float) + 256;
}

int gemm(const GemmDesc& d, hipStream_t stream) {
  if (d.M < 0 || d.N < 0 || d.K < 0 || !d.A || !d.B)
    return gpt2_internal_fail(1, "gemm: bad arguments");
  if (d.M == 0 || d.N == 0) return 0;
  const bool wgrad = d.epi == EPI_WGRAD;
  if (wgrad && !d.out32) return gpt2_internal_fail(1, "gemm: WGRAD needs out32");
  if (!wgrad && !d.C) return gpt2_internal_fail(1, "gemm: missing C");
  if ((d.epi == EPI_BIAS || d.epi == EPI_BIAS_RES || d.epi == EPI_BIAS_GELU) && !d.bias)
    return gpt2_internal_fail(1, "gemm: missing bias");
  if ((d.epi == EPI_BIAS_RES || d.epi == EPI_GELU_BWD) && !d.aux_in)
    return gpt2_internal_fail(1, "gemm: missing aux input");
  if (d.epi == EPI_BIAS_GELU && !d.aux_out) return gpt2_internal_fail(1, "gemm: missing U output");

  const int splits = wgrad ? wgrad_splits(d.dtype, d.M, d.N, d.K) : 1;
  float* partial = nullptr;
  float* partial_bias = nullptr;
  if (wgrad) {
    size_t need = gemm_workspace_bytes(d.dtype, d.epi, d.M, d.N, d.K);
    if (!d.workspace || d.workspace_bytes < need)
      return gpt2_internal_fail(3, "gemm: WGRAD workspace too small (%zu < %zu)", d.workspace_bytes, need);
    partial = reinterpret_cast<float*>(d.workspace);
    partial_bias = partial + (size_t)splits * d.M * d.N;
  }
  EpiArgs e{d.epi, d.M, d.N, d.C, d.ldc, d.bias, d.aux_in, d.ld_aux, d.aux_out, partial, partial_bias};

  if (d.K == 0) return gpt2_internal_fail(1, "gemm: K == 0 is not supported");

  int rc = 0;
  if (d.dtype == BF16) {
    // shape contract of the MFMA kernel: K a multiple of 8, 16-byte aligned rows,
    // contiguous axis of m-/n-major operands a multiple of 8.
    if (d.K % 8 != 0) return gpt2_internal_fail(1, "gemm(bf16): K=%d not a multiple of 8", d.K);
    if (d.lda % 8 || d.ldb % 8) return gpt2_internal_fail(1, "gemm(bf16): lda/ldb not multiples of 8");
    if ((!d.a_kmajor && d.M % 8) || (!d.b_kmajor && d.N % 8))
      return gpt2_internal_fail(1, "gemm(bf16): m/n-major operand extent not a multiple of 8");
    if (((uintptr_t)d.A | (uintptr_t)d.B) % 16)
      return gpt2_internal_fail(1, "gemm(bf16): A/B not 16-byte aligned");
    const int kt_total = (int)ceil_div64(d.K, kBK);
    MfmaArgs a{reinterpret_cast<const bf16*>(d.A), d.lda, reinterpret_cast<const bf16*>(d.B), d.ldb,
               d.M, d.N, d.K, (kt_total / splits) * kBK, e};
    const bool bias_grad = wgrad && d.bias_grad32 != nullptr;
    if (bias_grad && d.a_kmajor)
      return gpt2_internal_fail(1, "gemm: fused bias gradient needs an m-major A");
    switch (d.epi) {
      case EPI_STORE: rc = dispatch_layout_bf16<EPI_STORE>(d, a, 1, false, stream); break;
      case EPI_BIAS: rc = dispatch_layout_bf16<EPI_BIAS>(d, a, 1, false, stream); break;
      case EPI_BIAS_RES: rc = dispatch_layout_bf16<EPI_BIAS_RES>(d, a, 1, false, stream); break;
      case EPI_BIAS_GELU: rc = dispatch_layout_bf16<EPI_BIAS_GELU>(d, a, 1, false, stream); break;
      case EPI_GELU_BWD: rc = dispatch_layout_bf16<EPI_GELU_BWD>(d, a, 1, false, stream); break;
      case EPI_WGRAD: rc = dispatch_layout_bf16<EPI_WGRAD>(d, a, splits, bias_grad, stream); break;
      default: return gpt2_internal_fail(1, "gemm: unknown epilogue %d", d.epi);
    }
    if (rc) return rc;
    if (wgrad) {
      int64_t MN = (int64_t)d.M * d.N;
      hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((unsigned)ceil_div64(MN, 4 * 256)), dim3(256), 0,
                         stream, partial, splits, MN, d.out32, d.accumulate);
      GPT2_LAUNCH_CHECK();
      if (bias_grad) {
        hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((unsigned)ceil_div64(d.M, 4 * 256)), dim3(256), 0,
                           stream, partial_bias, splits, (int64_t)d.M, d.bias_grad32, d.accumulate);
        GPT2_LAUNCH_CHECK();
      }
    }
    return 0;
  }

  SimtArgs a{reinterpret_cast<const float*>(d.A), d.lda, reinterpret_cast<const float*>(d.B), d.ldb,
             d.M, d.N, d.K, (int)ceil_div64(d.K, splits), e};
  switch (d.epi) {
    case EPI_STORE: rc = dispatch_layout_f32<EPI_STORE>(d, a, 1, stream); break;
    case EPI_BIAS: rc = dispatch_layout_f32<EPI_BIAS>(d, a, 1, stream); break;
    case EPI_BIAS_RES: rc = dispatch_layout_f32<EPI_BIAS_RES>(d, a, 1, stream); break;
    case EPI_BIAS_GELU: rc = dispatch_layout_f32<EPI_BIAS_GELU>(d, a, 1, stream); break;
    case EPI_GELU_BWD: rc = dispatch_layout_f32<EPI_GELU_BWD>(d, a, 1, stream); break;
    case EPI_WGRAD: rc = dispatch_layout_f32<EPI_WGRAD>(d, a, splits, stream); break;
    default: return gpt2_internal_fail(1, "gemm: unknown epilogue %d", d.epi);
  }
  if (rc) return rc;
  if (wgrad) {
    int64_t MN = (int64_t)d.M * d.N;
    hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((unsigned)ceil_div64(MN, 4 * 256)), dim3(256), 0,
                       stream, partial, splits, MN, d.out32, d.accumulate);
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
