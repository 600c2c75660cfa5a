// GEMM kernels of the GPT-2 step (shared by gemm.hip, the bf16 / fp32
// dispatch, and gemm_fp8.hip, the FP8 dispatch): the four linear layers of
// each block, the tied classifier, and their dX / dW backward passes.
//
// The kernel table of "State of the Union [May 3, 2024]" (section "Runtime,
// DRAM traffic, instructions") attributes most of a step to these GEMMs
// (vendor-library kernels there) plus separate bias-gradient, GELU and
// residual kernels.  Here one hand-written bf16 MFMA kernel covers every GEMM
// of the step, with those elementwise pieces fused into its epilogue and the
// bias gradient fused into the weight-gradient pass.
//
// bf16 kernel (gfx950):
//   * block tiles 256x256, 256x128, 192x192, 128x256 or 128x128 (picked per
//     shape), K step 64; each wave owns a patch of v_mfma_f32_32x32x16_bf16
//     accumulators: 4 waves in a 2 x 2 grid, except the 256-row tiles without
//     an epilogue input, which run 8 waves (2 x 4 for 256x256, 4 x 2 for
//     256x128) so every SIMD holds two waves of the block, and the 192x192
//     tile of a long reduction, which runs two K-groups of 2 x 2 waves;
//   * operand tiles go from global memory straight into LDS with
//     buffer_load ... lds (no register staging), in a ring of 2-4 stages that
//     fills the LDS, so several K steps are in flight while the matrix cores
//     work on the current one; one barrier per K step; in tiles that run one
//     block per compute unit the refill of the ring is interleaved with the
//     step's first matrix instructions;
//   * k-major operands are stored as 128-byte rows with XOR-swizzled 16-byte
//     chunks and read with ds_read_b128; m-major operands (dY^T and X in
//     dW = dY^T X, W in dX = dY W) are stored as they lie in memory and read
//     with the transposing ds_read_b64_tr_b16, so no operand is transposed in
//     registers;
//   * the epilogue (bias, residual, GELU and its derivative, bf16 rounding)
//     goes through a wave-private LDS patch so stores are 16-byte vectors;
//   * blocks are mapped to tiles XCD by XCD (consecutive blocks land on
//     different XCDs) and in groups of 8 tile rows so each XCD's L2 sees
//     reuse;
//   * dW splits K (the B*T positions) over grid.y into fp32 partial tiles that
//     a second kernel sums in a fixed order, so results are deterministic.
// fp32 kernel (parity mode): plain LDS-tiled FMA GEMM with the same epilogues.

#pragma once

#include <type_traits>

#include "kernels.h"

namespace gpt2k {

// Argument blocks of the matrix-core kernel and its launch plan (shared by
// the bf16 and fp8 dispatch units, so declared outside the unnamed namespace).
struct EpiArgs {
  int epi;
  int M, N;
  void* C; int64_t ldc;
  const void* bias;
  const void* aux_in; int64_t ld_aux;
  void* aux_out;
  float* partial;        // [splits][M][N]
  float* partial_bias;   // [splits][M]
  float* amax;           // fp8 activation epilogues: max |C| into the amax slots (amax_atomic_bf16), or NULL
};

struct MfmaArgs {
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  uint32_t a_bytes, b_bytes;   // readable extent of A and B from their base pointers
  uint32_t aux_bytes;          // readable extent of the epilogue input (R or U), or 0
  int M, N, K;
  int k_per_split;
  bool vec_epilogue;     // every 8-column run is 16-byte aligned and inside N
  EpiArgs e;
  const float* scale_a;   // fp8: per-tensor scales of A and B (device), else unused
  const float* scale_b;
  int splits;             // K splits (units = tiles x splits)
  int persistent;         // the grid holds one block per compute unit slot and each block loops over units
};

struct Plan {
  int bm, bn, splits, k_per_split;
  int kgroups = 1;   // 2: the 192x192 tile's two K-groups of waves (long K per tile)
};

// Launches the fp8 kernel for a planned product (gemm_fp8.hip): epi is the
// epilogue the kernel runs (EPI_WGRAD for split-K partials), fmt_a the format
// of A (0: E4M3, 1: E5M2), kmajor whether both operands are k-major (else
// both m-major: weight gradients from the row-major codes).
int gemm_fp8_launch(int epi, int fmt_a, bool kmajor, const MfmaArgs& a, const Plan& pl, hipStream_t stream);

namespace {

typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));   // 32 fp8 values
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;          // K step of the bf16 MFMA kernel (128 bytes of each operand row)
constexpr int kBK8 = 128;        // K step of the fp8 kernel (the same 128 bytes)
constexpr int kThreads = 256;   // fp32 kernel, split-K reductions

// Waves per block of the MFMA kernel and their arrangement over the block
// tile: the 256-row tiles run 8 waves (two per SIMD) so that one wave's LDS
// reads and waits overlap the other's matrix instructions; the others run 4.
// (Tiles whose epilogue reads an input tile keep 4 waves: 8 waves' epilogue
// staging would not fit the LDS beside their stage ring.)
constexpr bool epi_has_aux(int epi) { return epi == EPI_BIAS_RES || epi == EPI_MUL; }
// With KGS = 2 (the planner's choice for a 192x192 tile whose K per tile is
// long) the block runs 8 waves as two K-groups of 2 x 2: each group takes two
// of the four k16 slices of every K step for the same 96 x 96 patches, and the
// second group's sums are added to the first's through the LDS before the
// epilogue.  (For K = 768 .. 3072 per tile that exchange costs more than the
// second wave per SIMD gains: measured 5-25 % slower there.)
constexpr int gemm_waves(int BM, int BN, int epi, int kgs) {
  return (BM == 256 && BN >= 128 && !epi_has_aux(epi)) || BM == 384 || kgs == 2 ? 8 : 4;
}
constexpr int gemm_wave_rows(int BM, int BN, int epi, int kgs) {
  return gemm_waves(BM, BN, epi, kgs) == 8 && (BN == 128 || BM == 384) ? 4 : 2;
}


template <int EPI, typename T>
__device__ __forceinline__ void epilogue_store(const EpiArgs& e, int m, int n, float v, int z) {
  if constexpr (EPI == EPI_WGRAD) {
    e.partial[((size_t)z * e.M + m) * (size_t)e.N + n] = v;
  } else {
    if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_RES || EPI == EPI_BIAS_GELU_D || EPI == EPI_BIAS_RELU2_D)
      v += to_f32(reinterpret_cast<const T*>(e.bias)[n]);
    if constexpr (EPI == EPI_BIAS_RES)
      v += to_f32(reinterpret_cast<const T*>(e.aux_in)[(size_t)m * e.ld_aux + n]);
    if constexpr (EPI == EPI_BIAS_GELU_D) {
      float g, d;
      gelu_tanh_and_grad_f(v, g, d);
      reinterpret_cast<T*>(e.aux_out)[(size_t)m * e.ldc + n] = from_f32<T>(d);
      v = g;
    }
    if constexpr (EPI == EPI_BIAS_RELU2_D) {
      const float r = fmaxf(v, 0.0f);
      reinterpret_cast<T*>(e.aux_out)[(size_t)m * e.ldc + n] = from_f32<T>(2.0f * r);
      v = r * r;
    }
    if constexpr (EPI == EPI_MUL) v *= to_f32(reinterpret_cast<const T*>(e.aux_in)[(size_t)m * e.ld_aux + n]);
    reinterpret_cast<T*>(e.C)[(size_t)m * e.ldc + n] = from_f32<T>(v);
  }
}

// ---------------------------------------------------------------- bf16 MFMA

// Physical 16-byte chunk of logical chunk c (0..7) in LDS row `row`.
__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row ^ (row >> 3)) & 7); }


// Offset past every operand extent (the host requires extents below it).
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;

// Stores of the vectorised epilogue, after bias, residual and the GELU'
// multiply have been applied from LDS: WGRAD partials, or C (and GELU'(u)).
template <int EPI>
__device__ __forceinline__ void epilogue_vec8_final(const EpiArgs& e, int m, int n, float v[8], int z) {
  if constexpr (EPI == EPI_WGRAD) {
    float* dst = e.partial + ((size_t)z * e.M + m) * (size_t)e.N + n;
    Chunk8<float>::store(dst, v);
  } else {
    if constexpr (EPI == EPI_BIAS_GELU_D) {
      float d[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) gelu_tanh_and_grad_f(v[i], v[i], d[i]);
      Chunk8<bf16>::store(reinterpret_cast<bf16*>(e.aux_out) + (size_t)m * e.ldc + n, d);
    }
    if constexpr (EPI == EPI_BIAS_RELU2_D) {
      float d[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float r = fmaxf(v[i], 0.0f);
        d[i] = 2.0f * r;
        v[i] = r * r;
      }
      Chunk8<bf16>::store(reinterpret_cast<bf16*>(e.aux_out) + (size_t)m * e.ldc + n, d);
    }
    Chunk8<bf16>::store(reinterpret_cast<bf16*>(e.C) + (size_t)m * e.ldc + n, v);
  }
}

// Work units are (split, tile) pairs, v = split * tiles + tile.  The
// dispatcher hands workgroups, in linear order, to the 8 XCDs in turn; each
// XCD is given a contiguous range of units, split major, so the units resident
// on one XCD share A and B slabs of one K range in its L2; inside a split,
// tiles run in groups of 8 M-tiles that sweep the N-tiles together.
__device__ __forceinline__ void xcd_range(int total, int xcd, int& beg, int& end) {
  const int base = total >> 3, rem = total & 7;
  beg = xcd * base + min(xcd, rem);
  end = beg + base + (xcd < rem ? 1 : 0);
}
__device__ __forceinline__ void unit_coords(int v, int nbm, int nbn, int& tm, int& tn, int& z) {
  const int ntiles = nbm * nbn;
  z = v / ntiles;
  const int t = v - z * ntiles;
  constexpr int GM = 8;
  const int group = t / (GM * nbn);
  const int first_m = group * GM;
  const int gsize = min(nbm - first_m, GM);
  const int r = t - group * GM * nbn;
  tm = first_m + r % gsize;
  tn = r / gsize;
}
// Units of this workgroup: one (grid = units, linear id -> its XCD's range)
// or, for a persistent grid of G blocks (G a multiple of 8), units
// beg + j, beg + j + G/8, ... of its XCD's range, j = its index on the XCD.
__device__ __forceinline__ void block_units(int total, bool persistent, int& u, int& u_end, int& u_step) {
  const int lin = (int)(blockIdx.y * gridDim.x + blockIdx.x);
  int beg, end;
  xcd_range(total, lin & 7, beg, end);
  if (persistent) {
    u = beg + (lin >> 3);
    u_end = end;
    u_step = (int)(gridDim.x * gridDim.y) >> 3;
  } else {
    u = beg + (lin >> 3);
    u_end = u + 1;
    u_step = 1;
  }
}

// ---------------------------------------------------------------- bf16 MFMA, direct-to-LDS


// Operand tile in LDS, R rows of the operand's M (or N) axis x 64 k, filled by
// buffer_load ... lds (each wave instruction writes 1 KiB, 16 bytes per lane,
// contiguous in lane order; the layout is realised by choosing which global
// 16-byte run each lane fetches).
//  * k-major operand (k contiguous in memory): [row][64 k], 128-byte rows whose
//    16-byte chunks are XOR-swizzled by row; fragments are ds_read_b128.
//  * m-major operand (m contiguous in memory): [k][R m], R * ES-byte rows
//    whose 16-byte chunk index is XORed with mswz(k): bf16 4 (k & 3), so the
//    4 x 64 bytes that one transposing read takes from k rows 4j .. 4j + 3
//    cover all 64 banks; fragments are two ds_read_b64_tr_b16 (the transpose
//    read hands lane j of each 16-lane group element j%4 of the 8-byte runs
//    of lanes j/4 + 4e, so with the per-lane addresses below every lane ends
//    up with 8 consecutive k of one m).  fp8 (k & 7), so the 8 x 16 bytes one
//    16-lane group of a ds_read_b64_tr_b8 takes from k rows 8j .. 8j + 7 sit
//    in 8 distinct bank groups; fragments are four such reads (that read
//    hands lane j of each 16-lane group byte j%8 of the 8-byte runs of lanes
//    2e + j/8, e = 0..7: 8 consecutive k of one m when lanes 2e and 2e + 1
//    address the two halves of the same 16 columns of k row e).
template <int R, bool KMAJ, int WAVES, int ES = 2>
struct DmaTile {
  // ES: bytes per element (2: bf16, 1: fp8); a K step is always 128 bytes of
  // every k-major row (64 bf16 / 128 fp8 k), i.e. 64 (bf16) or 128 (fp8)
  // m-major k rows
  static_assert(ES == 2 || ES == 1, "bf16 or fp8 operand tiles");
  static constexpr int BYTES = R * 128;
  static constexpr int NINST = BYTES / 1024 / WAVES;      // 1 KiB instructions per wave
  // m-major: chunk swizzle of k row k, lanes per k row, k rows per DMA instruction
  __device__ __forceinline__ static int mswz(int k) { return ES == 2 ? ((k & 3) << 2) : (k & 7); }
  static constexpr int MLPR = R * ES / 16;
  static constexpr int MRPI = 1024 / (R * ES);

  // Per-lane part of the DMA source addresses (two registers per operand); the
  // rest of each instruction's address is wave-uniform.
  //  k-major: instruction q of wave w covers tile rows 8 (w NINST + q) + lane/8,
  //    physical chunk lane%8; the swizzle (row ^ row>>3) & 7 splits into
  //    lane/8 (per lane) xor (w NINST + q) & 7 (uniform).
  //  m-major: instruction q covers k rows qk + lane / MLPR with
  //    qk = (w NINST + q) * MRPI, physical chunk lane % MLPR; the swizzle
  //    mswz(qk + kr) = mswz(qk) ^ mswz(kr) (MRPI is a power of two above kr)
  //    splits the same way.
  struct Lane {
    uint32_t base;    // bytes: row part (k-major) / row-in-group + column part (m-major)
    uint32_t c16;     // 16 * (per-lane part of the logical chunk index)
    int sub;          // k-major: chunk index; m-major: k row within the instruction's group
  };
  __device__ __forceinline__ static Lane lane_part(int wave, int lane, int row0, int64_t ld) {
    Lane L;
    if constexpr (KMAJ) {
      const int c = (lane & 7) ^ (lane >> 3);
      L.base = (uint32_t)((int64_t)(row0 + wave * NINST * 8 + (lane >> 3)) * ld * ES);
      L.c16 = (uint32_t)(c * 16);
      L.sub = c;
    } else {
      const int kr = lane / MLPR, phys = lane % MLPR;
      const int c = phys ^ mswz(kr);
      L.base = (uint32_t)((int64_t)kr * ld * ES + (int64_t)row0 * ES);
      L.c16 = (uint32_t)(c * 16);
      L.sub = kr;
    }
    return L;
  }

  // Issues this wave's NINST DMA instructions for the K step starting at k0.
  // Rows beyond the operand's extent only feed discarded outputs (and the
  // buffer range turns reads past the allocation into zeros); k >= K must be
  // zero, which only the last, partial K step checks (k_tail).
  __device__ __forceinline__ static void issue(i32x4_rsrc rs, GPT2_LDS char* tile, int wave, const Lane& L,
                                               int k0, int K, int64_t ld, bool k_tail) {
#pragma unroll
    for (int q = 0; q < NINST; ++q) {
      const int iq = wave * NINST + q;
      uint32_t off;
      bool ok = true;
      if constexpr (KMAJ) {
        const uint32_t u16 = (uint32_t)((iq & 7) * 16);
        const uint32_t c16 = L.c16 ^ u16;
        off = L.base + (uint32_t)q * (uint32_t)(8 * ld * ES) + (uint32_t)(k0 * ES) + c16;
        if (k_tail) ok = k0 + (int)(c16 >> 4) * (16 / ES) < K;
      } else {
        const int qk = iq * MRPI;
        const uint32_t u16 = (uint32_t)(mswz(qk) * 16);
        off = L.base + (uint32_t)((int64_t)(k0 + qk) * ld * ES) + (L.c16 ^ u16);
        if (k_tail) ok = k0 + qk + L.sub < K;
      }
      dma_lds16(rs, (GPT2_LDS void*)(tile + iq * 1024), ok ? off : kOutOfRange);
    }
  }

  // Instruction q alone of a K step that lies wholly inside K (no tail check).
  __device__ __forceinline__ static void issue_q_full(i32x4_rsrc rs, GPT2_LDS char* tile, int wave, const Lane& L,
                                                      int k0, int64_t ld, int q) {
    const int iq = wave * NINST + q;
    uint32_t off;
    if constexpr (KMAJ) {
      off = L.base + (uint32_t)q * (uint32_t)(8 * ld * ES) + (uint32_t)(k0 * ES) + (L.c16 ^ (uint32_t)((iq & 7) * 16));
    } else {
      const int qk = iq * MRPI;
      off = L.base + (uint32_t)((int64_t)(k0 + qk) * ld * ES) + (L.c16 ^ (uint32_t)(mswz(qk) * 16));
    }
    dma_lds16(rs, (GPT2_LDS void*)(tile + iq * 1024), off);
  }

  // fp8 MFMA operand fragment (v_mfma_scale_f32_32x32x64_f8f6f4): rows
  // [rbase, rbase + 32), k64 step kk (0 or 1 of the K step); lane l receives
  // row rbase + l%32, k = 64 kk + 32 (l/32) + 0..31 (32 bytes: two swizzled
  // 16-byte chunks of a k-major row, or four transposing reads of an m-major
  // tile).
  __device__ __forceinline__ static i32x8 frag8(const GPT2_LDS char* tile, int rbase, int kk, int lane) {
    static_assert(ES == 1, "fp8 fragments");
    i32x8 out;
    if constexpr (KMAJ) {
      typedef int i32x4 __attribute__((ext_vector_type(4)));
      const int row = rbase + (lane & 31), c = kk * 4 + (lane >> 5) * 2;
      const i32x4 lo = *reinterpret_cast<const GPT2_LDS i32x4*>(tile + row * 128 + swz(row, c) * 16);
      const i32x4 hi = *reinterpret_cast<const GPT2_LDS i32x4*>(tile + row * 128 + swz(row, c + 1) * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) { out[e] = lo[e]; out[4 + e] = hi[e]; }
    } else {
      // lane l = 16 g + j provides the run of k row 8 t + j/2 (of its half of
      // the k64 step) at columns m .. m + 7 and receives 8 consecutive k of
      // column rbase + l%32, four times
      typedef int i32x2 __attribute__((ext_vector_type(2)));
      const int g = lane >> 4, j = lane & 15;
      const int m = rbase + 16 * (g & 1) + 8 * (j & 1);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kr = 64 * kk + 32 * (g >> 1) + 8 * t + (j >> 1);
        const int c = (m >> 4) ^ mswz(kr);
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            const_cast<GPT2_LDS i32x2*>(reinterpret_cast<const GPT2_LDS i32x2*>(tile + kr * R + c * 16 + (m & 15))));
        out[2 * t] = v[0];
        out[2 * t + 1] = v[1];
      }
    }
    return out;
  }

  // MFMA operand fragment: rows [rbase, rbase + 32) of the tile, k16 step kk;
  // lane l receives row rbase + l%32, k = 16 kk + 8 (l/32) + 0..7.
  __device__ __forceinline__ static bf16x8 frag(const GPT2_LDS char* tile, int rbase, int kk, int lane) {
    if constexpr (KMAJ) {
      const int row = rbase + (lane & 31), c = kk * 2 + (lane >> 5);
      return *reinterpret_cast<const GPT2_LDS bf16x8*>(tile + row * 128 + swz(row, c) * 16);
    } else {
      typedef bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      const int g = lane >> 4, i = lane & 15;
      const int m = rbase + 16 * (g & 1) + 4 * (i & 3);
      bf16x8 out;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int kr = kk * 16 + 8 * (g >> 1) + 4 * r + (i >> 2);
        const int c = (m >> 3) ^ ((kr & 3) << 2);
        const GPT2_LDS bf16x4_t* q =
            reinterpret_cast<const GPT2_LDS bf16x4_t*>(tile + kr * (2 * R) + c * 16 + (m & 7) * 2);
        const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<GPT2_LDS bf16x4_t*>(q));
#pragma unroll
        for (int e = 0; e < 4; ++e) out[4 * r + e] = v[e];
      }
      return out;
    }
  }
};

// Block-tile geometry and LDS budget.  The stage ring is as deep as 160 KiB
// allows; the epilogue's staging (and the bias-gradient reduction) goes into
// the last stage buffer when the epilogue input tile (HAS_AUX) leaves it free,
// else into an array of its own.
template <int BM, int BN, int EPI, int KGS>
struct DmaShape {
  static constexpr bool HAS_AUX = epi_has_aux(EPI);
  static constexpr int WAVES = gemm_waves(BM, BN, EPI, KGS), NT = 64 * WAVES;
  static constexpr int KG = KGS;                                             // K-groups
  static constexpr int WGM = gemm_wave_rows(BM, BN, EPI, KGS), WGN = WAVES / (WGM * KG);   // wave grid
  static constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  static constexpr int STAGE_BYTES = (BM + BN) * 128;
  static constexpr int EP_PITCH = 36;                     // fp32 pitch of a 32 x 32 epilogue block
  static constexpr int EP_BYTES = WAVES * 32 * EP_PITCH * 4;  // one block per wave
  static constexpr int RED_BYTES = 8 * BM * 4;
  static constexpr int AUX_BYTES = EP_BYTES > RED_BYTES ? EP_BYTES : RED_BYTES;
  static constexpr int SUB_BYTES = BM * 128;              // [BM][64] bf16 sub-tile of the epilogue input
  static constexpr int PER_STAGE = STAGE_BYTES / SUB_BYTES;
  // 384x192: the epilogue input tile (144 KiB) would not fit beside the ring;
  // each wave loads its share straight into registers after the main loop
  // (the fragment registers are free by then)
  static constexpr bool AUX_DIRECT = HAS_AUX && BM == 384;
  static constexpr int AUX_STAGES = HAS_AUX && !AUX_DIRECT ? (BN / 64 + PER_STAGE - 1) / PER_STAGE : 0;
  static constexpr int LDS_LIMIT = 160 * 1024 - 2 * BN * 4 - 1024;   // two bias buffers
  static constexpr bool fits(int n) {
    return AUX_STAGES <= n && n * STAGE_BYTES + (AUX_STAGES < n ? 0 : AUX_BYTES) <= LDS_LIMIT;
  }
  // 128x128 runs two blocks per compute unit (2 stages, 64 KiB each), so one
  // block's epilogue overlaps the other's main loop; larger tiles run one
  // block with as deep a ring as fits.
  static constexpr int OCC = (BM == 128 && BN == 128) ? 2 : 1;
  static constexpr int NS = OCC == 2 ? 2 : fits(4) ? 4 : fits(3) ? 3 : 2;
  static constexpr bool EPI_IN_STAGE = AUX_STAGES < NS && AUX_BYTES <= STAGE_BYTES;
  // The epilogue input tile can be loaded during the last K step (into the
  // stages that step does not read) when it leaves one stage free.
  static constexpr bool EARLY_AUX = HAS_AUX && !AUX_DIRECT && AUX_STAGES < NS;
};

// F8: both operands fp8 (OCP formats; B E4M3, A E4M3 or, with FMT_A = 1,
// E5M2), products on v_mfma_scale_f32_32x32x64_f8f6f4 with unit block
// scales, the sums multiplied by the two per-tensor scales before the
// epilogue.
template <int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI, bool BIAS_GRAD, int KGS, bool F8 = false, int FMT_A = 0>
__global__ __launch_bounds__(64 * gemm_waves(BM, BN, EPI, KGS))
__attribute__((amdgpu_waves_per_eu(gemm_waves(BM, BN, EPI, KGS) / 4,
                                   (BM == 128 && BN == 128) ? 2 : gemm_waves(BM, BN, EPI, KGS) / 4)))
void gemm_bf16_dma_kernel(MfmaArgs p) {
  constexpr bool HAS_BIAS = EPI == EPI_BIAS || EPI == EPI_BIAS_RES || EPI == EPI_BIAS_GELU_D || EPI == EPI_BIAS_RELU2_D;
  constexpr bool HAS_AUX = epi_has_aux(EPI);
  using S = DmaShape<BM, BN, EPI, KGS>;
  constexpr int ES = F8 ? 1 : 2;                          // bytes per operand element
  constexpr int KE = F8 ? kBK8 : kBK;                      // K elements per step
  static_assert(!F8 || (!BIAS_GRAD && KGS == 1), "fp8: one K-group, bias gradient taken by the quantisation");
  using TA = DmaTile<BM, A_KMAJ, S::WAVES, ES>;
  using TB = DmaTile<BN, B_KMAJ, S::WAVES, ES>;
  constexpr int NT = S::NT;
  constexpr int WM = S::WM, WN = S::WN, FM = S::FM, FN = S::FN, NS = S::NS;
  constexpr int A_BYTES = TA::BYTES;
  constexpr int NDMA = TA::NINST + TB::NINST;              // DMA instructions per wave per stage
  constexpr bool IL = S::OCC == 1;  // refill spread over the MFMAs (one block per CU)
  __shared__ __attribute__((aligned(1024))) char st0[S::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st1[S::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st2[NS > 2 ? S::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char st3[NS > 3 ? S::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(16))) char epi_own[S::EPI_IN_STAGE ? 16 : S::AUX_BYTES];
  __shared__ __attribute__((aligned(16))) float bias_s[2][HAS_BIAS ? BN : 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wid = wave % (S::WGM * S::WGN), kg = wave / (S::WGM * S::WGN);
  const int wm = wid / S::WGN, wn = wid % S::WGN;
  constexpr int KK = KE / (F8 ? 64 : 16) / S::KG;         // MFMA k slices per K step of this wave
  // the spread refill issues one DMA instruction after each of the step's
  // KK * FM * FN matrix instructions, so it needs that many slots
  static_assert(!IL || NDMA <= KK * FM * FN, "one DMA instruction per MFMA at most");
  static_assert(S::KG == 1 || !BIAS_GRAD, "K-groups take no fused bias gradient");
  // A tile's epilogue stages its output through the last ring slot and reads
  // no input tile, so the next tile's first NS - 1 K steps can be loaded into
  // the other slots while it runs: such kernels run persistent (one block per
  // compute-unit slot, looping over their XCD's units) when the grid says so.
  constexpr bool PERSIST = !HAS_AUX && S::KG == 1 && S::EPI_IN_STAGE;
  const int nbm = (p.M + BM - 1) / BM, nbn = (p.N + BN - 1) / BN;
  const bool persistent = PERSIST && p.persistent;
  int u, u_end, u_step;
  block_units(nbm * nbn * p.splits, persistent, u, u_end, u_step);
  const i32x4_rsrc ra = make_rsrc4(p.A, p.a_bytes), rb = make_rsrc4(p.B, p.b_bytes);

  auto stage_ptr = [&](int s) -> GPT2_LDS char* {
    return (GPT2_LDS char*)(s == 0 ? st0 : s == 1 ? st1 : s == 2 ? st2 : st3);
  };
  // K step kt of the unit whose lane parts and first k are given, into ring slot s
  auto issue_unit = [&](const typename TA::Lane& la_, const typename TB::Lane& lb_, int kbeg_, int kt, int s) {
    GPT2_LDS char* base = stage_ptr(s);
    const int k0 = kbeg_ + kt * KE;
    const bool tail = k0 + KE > p.K;
    TA::issue(ra, base, wave, la_, k0, p.K, p.lda, tail);
    TB::issue(rb, base + A_BYTES, wave, lb_, k0, p.K, p.ldb, tail);
  };
  const bool vec = p.vec_epilogue;
  // fp8: the sums of products of the quantised operands times s_a s_b
  float sc = 1.0f;
  if constexpr (F8) sc = p.scale_a[0] * p.scale_b[0];
  // fp8 activation epilogues: the largest |C| this thread stores (its fp8
  // quantisation comes next); the host asks for it only with the vector epilogue
  constexpr bool AMX = F8 && (EPI == EPI_BIAS_GELU_D || EPI == EPI_BIAS_RELU2_D || EPI == EPI_MUL);
  float cmax = 0.f;

  for (int it = 0; u < u_end; u += u_step, ++it) {
  const bool first = it == 0;
  const int bp = it & 1;                     // bias buffer of this unit
  int tm, tn, z;
  unit_coords(u, nbm, nbn, tm, tn, z);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = z * p.k_per_split;
  const int KT = (min(p.K, kbeg + p.k_per_split) - kbeg + KE - 1) / KE;
  const bool do_bias = BIAS_GRAD && tn == 0;
  const typename TA::Lane la = TA::lane_part(wave, lane, m0, p.lda);
  const typename TB::Lane lb = TB::lane_part(wave, lane, n0, p.ldb);
  auto issue = [&](int kt, int s) { issue_unit(la, lb, kbeg, kt, s); };

  // the block's bias columns, read by the epilogue from LDS (two buffers: the
  // previous unit's epilogue may still be reading the other)
  if constexpr (HAS_BIAS) {
    for (int c = tid; c < BN; c += NT)
      bias_s[bp][c] = n0 + c < p.N ? (float)reinterpret_cast<const bf16*>(p.e.bias)[n0 + c] : 0.f;
  }

  // The residual / pre-activation tile the epilogue reads (R or U, [BM][BN]
  // bf16) comes into stage buffers with the same DMA as the operands:
  // [BM][64]-column sub-tiles with 128-byte swizzled rows (one memory round
  // trip for the whole tile).  aux_stage(j) gives the stage of its j-th part.
  auto issue_aux = [&](auto aux_stage) {
    using TX = DmaTile<BM, true, S::WAVES>;
    const i32x4_rsrc rx = make_rsrc4(p.e.aux_in, p.aux_bytes);
    const typename TX::Lane lx = TX::lane_part(wave, lane, m0, p.e.ld_aux);
#pragma unroll
    for (int c = 0; c < BN / 64; ++c) {
      const int c0 = n0 + 64 * c;
      TX::issue(rx, aux_stage(c / S::PER_STAGE) + (c % S::PER_STAGE) * S::SUB_BYTES, wave, lx, c0, p.N,
                p.e.ld_aux, c0 + 64 > p.N);
    }
  };


  float bsum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bsum[e] = 0.f;
  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // the first unit loads its first NS - 1 K steps here; later units' were
  // issued during the previous unit's epilogue
  if (first) {
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < KT) issue(s, s);
  }

  for (int kt0 = 0; kt0 < KT; kt0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int kt = kt0 + s;
      if (kt < KT) {
        // stage s of this K step has landed (for this wave), then everyone's has
        // (a later unit's first step waits for everything: the previous
        // epilogue's stores are in flight too, and stores and loads need not
        // complete in order)
        if (kt + NS - 2 < KT && (first || kt > 0)) wait_vmcnt<(NS - 2) * NDMA>();
        else wait_vmcnt<0>();
        lds_barrier();
        // Refill of the ring slot read in the previous K step.  For the tiles
        // that run one block per compute unit (nothing else covers the gap)
        // the refill is spread over this step's first matrix instructions,
        // one DMA instruction after each, so its address work issues while
        // the matrix core runs; for the two-block 128x128 tile (and in a
        // partial last K step) it is issued here, ahead of the fragment
        // reads, which measured faster there: the other block covers the gap
        // and the DMA gets more time to land.
        const bool refill = kt + NS - 1 < KT;
        GPT2_LDS char* const nbase = stage_ptr((s + NS - 1) % NS);
        const int k0n = kbeg + (kt + NS - 1) * KE;
        const bool tail_n = k0n + KE > p.K;
        const bool spread = IL && refill && !tail_n;
        if (refill && !spread) issue(kt + NS - 1, (s + NS - 1) % NS);
        auto dma_one = [&](int d) {
          if (d < TA::NINST) TA::issue_q_full(ra, nbase, wave, la, k0n, p.lda, d);
          else TB::issue_q_full(rb, nbase + A_BYTES, wave, lb, k0n, p.ldb, d - TA::NINST);
        };
        if constexpr (S::EARLY_AUX) {
          // last K step: every stage but s is idle
          if (kt == KT - 1 && vec) issue_aux([&](int j) { return stage_ptr((s + 1 + j) % NS); });
        }
        const GPT2_LDS char* As = stage_ptr(s);
        const GPT2_LDS char* Bs = As + A_BYTES;
        if constexpr (BIAS_GRAD) {
          // column sums of the m-major dY tile: thread t sums k rows 8*(t/32) .. +7 of chunk t%32
          if (do_bias) {
            constexpr int CH = BM / 8;
            for (int w8 = tid; w8 < CH * 8; w8 += NT) {
              const int cc = w8 % CH, kg = w8 / CH;
#pragma unroll
              for (int r = 0; r < 8; ++r) {
                const int kr = kg * 8 + r;
                const int c = cc ^ ((kr & 3) << 2);
                const bf16x8 v = *reinterpret_cast<const GPT2_LDS bf16x8*>(As + kr * (2 * BM) + c * 16);
#pragma unroll
                for (int e = 0; e < 8; ++e) bsum[e] += (float)v[e];
              }
            }
          }
        }
        using Frag = std::conditional_t<F8, i32x8, bf16x8>;
        auto frag_a = [&](int i, int kk) -> Frag {
          if constexpr (F8) return TA::frag8(As, wm * WM + i * 32, kk, lane);
          else return TA::frag(As, wm * WM + i * 32, kk, lane);
        };
        auto frag_b = [&](int j, int kk) -> Frag {
          if constexpr (F8) return TB::frag8(Bs, wn * WN + j * 32, kk, lane);
          else return TB::frag(Bs, wn * WN + j * 32, kk, lane);
        };
        // The next k slice's fragments load while this one's products run (two
        // buffers), except where that would not fit the 256 registers of a
        // wave at two waves per SIMD: fp8 (fragments twice as large, and only
        // two slices per K step), the K-grouped 192x192 tile, the 256-row
        // weight-gradient tile with the fused bias gradient and the 384x192
        // tile (96 x 96 patches: 144 accumulator registers)
        constexpr int NB = (F8 || S::KG == 2 || (BIAS_GRAD && S::WAVES == 8) || BM == 384) ? 1 : 2;
        Frag a[NB][FM], b[NB][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) a[0][i] = frag_a(i, kg * KK);
#pragma unroll
        for (int j = 0; j < FN; ++j) b[0][j] = frag_b(j, kg * KK);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if (NB == 2 && kk + 1 < KK) {
#pragma unroll
            for (int i = 0; i < FM; ++i) a[(kk + 1) % NB][i] = frag_a(i, kg * KK + kk + 1);
#pragma unroll
            for (int j = 0; j < FN; ++j) b[(kk + 1) % NB][j] = frag_b(j, kg * KK + kk + 1);
          }
          if (NB == 1 && kk > 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i) a[0][i] = frag_a(i, kg * KK + kk);
#pragma unroll
            for (int j = 0; j < FN; ++j) b[0][j] = frag_b(j, kg * KK + kk);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              if constexpr (F8)   // B operand E4M3 (0), A operand FMT_A; unit (2^0) block scales
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[kk % NB][j], a[kk % NB][i], acc[i][j],
                                                                           0, FMT_A, 0, 127, 0, 127);
              else
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[kk % NB][j], a[kk % NB][i], acc[i][j], 0, 0, 0);
              if constexpr (IL) {
                const int t = (kk * FM + i) * FN + j;
                if (t < NDMA) {
                  if (spread) dma_one(t);
                  __builtin_amdgcn_sched_barrier(0);
                }
              }
            }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  constexpr int SUB_BYTES = S::SUB_BYTES;
  constexpr int PER_STAGE = S::PER_STAGE;
  static_assert(PER_STAGE >= 1 && S::AUX_STAGES <= NS, "aux tile must fit the stages");
  const int s_last = (KT - 1) % NS;          // stage of the last K step
  if constexpr (S::EARLY_AUX) {
    if (vec) wait_vmcnt<0>();                // the epilogue input issued in the last K step
  }
  // bias and epilogue input visible; every wave done with the stage buffers reused below
  if constexpr (HAS_BIAS || HAS_AUX || S::EPI_IN_STAGE) __syncthreads();
  // AUX_DIRECT: this wave's part of the epilogue input (the two 16-byte runs
  // per lane of each 32 x 32 block, as the epilogue below reads them), all in
  // flight at once; out-of-range runs read zeros through the buffer range
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 auxr[S::AUX_DIRECT ? FM : 1][S::AUX_DIRECT ? FN : 1][2];
  if constexpr (S::AUX_DIRECT) {
    if (vec) {
      const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.e.aux_in, p.aux_bytes);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int idx = lane + 64 * q, rl = idx >> 2, cc = idx & 3;
            const int grow = m0 + wm * WM + i * 32 + rl, gcol = n0 + wn * WN + j * 32 + cc * 8;
            const uint32_t off = grow < p.M && gcol < p.N ? (uint32_t)(((int64_t)grow * p.e.ld_aux + gcol) * 2)
                                                          : kOutOfRange;
            auxr[i][j][q] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
          }
    }
  }
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  if constexpr (S::KG == 2) {
    // The second K-group's sums go through the idle stage buffers, one 4 KiB
    // block per accumulator tile (16-byte runs in lane order, conflict-free),
    // and the first group adds them to its own.
    constexpr int PER = S::STAGE_BYTES / 4096;
    static_assert(S::WGM * S::WGN * FM * FN <= NS * PER, "K-group partial sums must fit the stages");
    auto blk = [&](int i, int j) -> GPT2_LDS f32x4* {
      const int bi = (wid * FM + i) * FN + j;
      return reinterpret_cast<GPT2_LDS f32x4*>(stage_ptr(bi / PER) + (bi % PER) * 4096) + lane;
    };
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = acc[i][j][4 * g + e];
            blk(i, j)[64 * g] = w;
          }
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 w = blk(i, j)[64 * g];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][4 * g + e] += w[e];
          }
          // one tile at a time: hoisting every read would need 144 more registers
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();   // the epilogue staging below reuses the stage buffers
  }
  // Persistent: every wave is past the barrier above, so the ring slots
  // 0 .. NS - 2 are free; the next unit's first K steps load into them while
  // this unit's epilogue runs in slot NS - 1.
  if constexpr (PERSIST) {
    if (persistent && u + u_step < u_end) {
      int tm2, tn2, z2;
      unit_coords(u + u_step, nbm, nbn, tm2, tn2, z2);
      const int kbeg2 = z2 * p.k_per_split;
      const int KT2 = (min(p.K, kbeg2 + p.k_per_split) - kbeg2 + KE - 1) / KE;
      const typename TA::Lane la2 = TA::lane_part(wave, lane, tm2 * BM, p.lda);
      const typename TB::Lane lb2 = TB::lane_part(wave, lane, tn2 * BN, p.ldb);
#pragma unroll
      for (int s = 0; s < NS - 1; ++s)
        if (s < KT2) issue_unit(la2, lb2, kbeg2, s, s);
    }
  }
  GPT2_LDS char* epi_lds =
      S::EPI_IN_STAGE ? stage_ptr(S::EARLY_AUX ? s_last : NS - 1) : (GPT2_LDS char*)epi_own;
  auto aux_stage = [&](int j) { return S::EARLY_AUX ? stage_ptr((s_last + 1 + j) % NS) : stage_ptr(j); };
  if constexpr (HAS_AUX && !S::EARLY_AUX && !S::AUX_DIRECT) {
    if (vec) {
      issue_aux([&](int j) { return stage_ptr(j); });
      wait_vmcnt<0>();
      __syncthreads();
    }
  }

  // Epilogue, one 32 x 32 accumulator block at a time through this wave's own
  // LDS block (LDS operations of one wave complete in order, so no barrier).
  // The products were taken as B x A, so element r of lane l sits at row l%32,
  // column 8(r/4) + 4(l/32) + r%4: four consecutive columns per 16-byte write.
  GPT2_LDS float* ep = reinterpret_cast<GPT2_LDS float*>(epi_lds) + wid * 32 * S::EP_PITCH;
  const int hi = lane >> 5;
  if (S::KG == 1 || kg == 0) {   // the second K-group is done
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = F8 ? acc[i][j][4 * g + e] * sc : acc[i][j][4 * g + e];
          *reinterpret_cast<GPT2_LDS f32x4*>(ep + (lane & 31) * S::EP_PITCH + 8 * g + 4 * hi) = w;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int idx = lane + 64 * q, rl = idx >> 2, cc = idx & 3;
          const int grow = m0 + wm * WM + i * 32 + rl, gcol = n0 + wn * WN + j * 32 + cc * 8;
          if (grow < p.M && gcol < p.N) {
            float v[8];
            {
              const GPT2_LDS f32x4* q = reinterpret_cast<const GPT2_LDS f32x4*>(ep + rl * S::EP_PITCH + cc * 8);
              const f32x4 lo = q[0], hi4 = q[1];
#pragma unroll
              for (int e = 0; e < 4; ++e) { v[e] = lo[e]; v[4 + e] = hi4[e]; }
            }
            if (vec) {
              const int tr = wm * WM + i * 32 + rl, tc = wn * WN + j * 32 + cc * 8;
              if constexpr (HAS_BIAS) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] += bias_s[bp][tc + e];
              }
              if constexpr (HAS_AUX) {
                u32x4 raw;
                if constexpr (S::AUX_DIRECT) {
                  raw = auxr[i][j][q];
                } else {
                  const int sb = tc >> 6, ch = (tc & 63) >> 3;
                  const GPT2_LDS char* t = aux_stage(sb / PER_STAGE) + (sb % PER_STAGE) * SUB_BYTES;
                  raw = *reinterpret_cast<const GPT2_LDS u32x4*>(t + tr * 128 + swz(tr, ch) * 16);
                }
                const uint32_t w[4] = {raw[0], raw[1], raw[2], raw[3]};
                float x[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  x[2 * e] = __uint_as_float(w[e] << 16);
                  x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
                }
                if constexpr (EPI == EPI_BIAS_RES) {
#pragma unroll
                  for (int e = 0; e < 8; ++e) v[e] += x[e];
                } else {
#pragma unroll
                  for (int e = 0; e < 8; ++e) v[e] *= x[e];
                }
              }
              epilogue_vec8_final<EPI>(p.e, grow, gcol, v, z);
              if constexpr (AMX) {
#pragma unroll
                for (int e = 0; e < 8; ++e) cmax = fmaxf(cmax, fabsf(v[e]));
              }
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (gcol + e < p.N) epilogue_store<EPI, bf16>(p.e, grow, gcol + e, v[e], z);
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
  }

  if constexpr (BIAS_GRAD) {
    if (do_bias) {   // uniform over the block
      __syncthreads();
      GPT2_LDS float* red = reinterpret_cast<GPT2_LDS float*>(epi_lds);   // [8 k-groups][BM]
      constexpr int CH = BM / 8;
      for (int w8 = tid; w8 < CH * 8; w8 += NT) {
        const int cc = w8 % CH, kg = w8 / CH;
#pragma unroll
        for (int e = 0; e < 8; ++e) red[kg * BM + cc * 8 + e] = bsum[e];
      }
      __syncthreads();
      for (int m = tid; m < BM; m += NT) {
        float t = 0.f;
#pragma unroll
        for (int kg = 0; kg < 8; ++kg) t += red[kg * BM + m];
        if (m0 + m < p.M) p.e.partial_bias[(size_t)z * p.M + m0 + m] = t;
      }
    }
  }
  }   // units
  if constexpr (AMX) {
    if (p.e.amax) {   // uniform
      cmax = wave_max(cmax);
      if (lane == 0) amax_atomic_bf16(p.e.amax, blockIdx.x * S::WAVES + wave, cmax);   // rounded as C was
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

// out[i] (+)= sum over the splits of partial[z][i] (i < MN), in split order.
// Blocks from `first_bias_block` on do the same for the bias-gradient
// partials (pb [splits][M] -> bias_out), so one launch covers both.
__global__ void wgrad_reduce_kernel(const float* __restrict__ partial, int splits, int64_t MN,
                                    float* __restrict__ out, bool accumulate, unsigned first_bias_block,
                                    const float* __restrict__ pb, int64_t M, float* __restrict__ bias_out) {
  unsigned blk = blockIdx.x;
  if (blk >= first_bias_block) {   // bias segment (uniform per block)
    blk -= first_bias_block;
    partial = pb;
    MN = M;
    out = bias_out;
  }
  int64_t i4 = ((int64_t)blk * blockDim.x + threadIdx.x) * 4;
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

// Split-K of a plain-store GEMM: C[m, n] (bf16, row stride ldc) = sum over
// the splits of the fp32 partial tiles, in split order.
__global__ void splitk_store_bf16_kernel(const float* __restrict__ partial, int splits, int M, int N,
                                         bf16* __restrict__ C, int64_t ldc) {
  const int64_t MN = (int64_t)M * N;
  const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= MN) return;
  if ((N % 4) == 0) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int z = 0; z < splits; ++z) {
      const float4 v = *reinterpret_cast<const float4*>(partial + (size_t)z * MN + i4);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const int64_t m = i4 / N, n = i4 % N;
    bf16* dst = C + m * ldc + n;
    dst[0] = (bf16)s.x; dst[1] = (bf16)s.y; dst[2] = (bf16)s.z; dst[3] = (bf16)s.w;
  } else {
    for (int64_t i = i4; i < MN && i < i4 + 4; ++i) {
      float s = 0.f;
      for (int z = 0; z < splits; ++z) s += partial[(size_t)z * MN + i];
      C[(i / N) * ldc + i % N] = (bf16)s;
    }
  }
}

// ---------------------------------------------------------------- dispatch

// Launch plan of a bf16 GEMM: block tile and the split of K.
//
// The time of a candidate (tile BM x BN, s splits of K) is estimated as
//   rounds * K-steps per split * t_step(tile)  +  fp32 partial traffic / HBM rate
// with rounds = ceil(tiles * s / 256 CUs) and t_step the measured time of one
// 64-deep K step of a tile on one CU (256x256: 2.75 us; 256x128 and 128x256:
// 1.83 us; 192x192: 1.70 us, its smaller per-tile epilogue bursts included;
// 128x128: 1.25 us; the larger tile reads less LDS per MFMA).  WGRAD always goes through fp32 partials (s M N floats written
// and read, M N written); a plain store is split only when K is long enough
// for the partials to pay off.  Other epilogues are never split and choose
// between the default tile and 192x192 (both operands k-major only), which
// tiles M = 24576, N = 768 into exactly two rounds.

Plan plan_bf16(int epi, int M, int N, int K, bool a_kmajor, bool b_kmajor) {
  const int kt = (int)ceil_div64(K, kBK);
  const bool wgrad = epi == EPI_WGRAD;
  const bool may_split = wgrad || (epi == EPI_STORE && K >= 8192);
  struct Cand { int bm, bn; double t_step; };
  const Cand cands[5] = {{256, 256, 2.75e-6}, {256, 128, 1.83e-6}, {128, 256, 1.83e-6}, {128, 128, 1.25e-6},
                         {192, 192, 1.70e-6}};
  const int def_bm = M >= 2048 ? 256 : 128, def_bn = N >= 2048 ? 256 : 128;
  Plan best{def_bm, def_bn, 1, 0};
  double best_t = 1e300;
  // Short-K products with a bias or GELU epilogue (QKV, fc forward): the
  // 8-wave 384x192 tile where N is a multiple of 192 (QKV N = 2304: 768
  // tiles, three whole rounds, against 3.4 rounds of 256x256; fc N = 3072:
  // 1024 tiles, four rounds, against 4.5; 1.25 -> 1.16 and 2.07 -> 1.99 ms
  // per step), else for a wide N the 8-wave 256x256 tile (measured 3-5%
  // faster than 128x128 at M = 24576, K = 768).
  if (!may_split && (epi == EPI_BIAS_GELU_D || epi == EPI_BIAS_RELU2_D || epi == EPI_BIAS) && a_kmajor && b_kmajor &&
      M >= 8192 && N % 192 == 0 && K <= 1024) {
    best = Plan{384, 192, 1, kt * kBK};
    return best;
  }
  if (!may_split && (epi == EPI_BIAS_GELU_D || epi == EPI_BIAS_RELU2_D || epi == EPI_BIAS) && a_kmajor && b_kmajor &&
      M >= 2048 &&
      N >= 2048 && K <= 1024) {
    best = Plan{256, 256, 1, kt * kBK};
    return best;
  }
  // Other short-K products with an epilogue that reads an input tile (the
  // GELU' multiply; a residual add whose N is not a multiple of 192): the
  // epilogue is a large share of each tile, and 128x128 tiles at two blocks
  // per compute unit overlap it with the other block's main loop (measured
  // 15-25% faster than the 4-wave one-block tiles at M = 24576, K = 768).  A
  // residual add with N a multiple of 192 takes the 384x192 tile below (its
  // residual loaded to registers after the main loop; attn-proj forward,
  // N = 768: 256 tiles, one round, 0.62 -> 0.54 ms per step).
  if (!may_split && epi != EPI_STORE && !(epi == EPI_BIAS_RES && N % 192 == 0 && M >= 8192) && a_kmajor && b_kmajor &&
      M >= 2048 && K <= 1024) {
    best = Plan{128, 128, 1, 0};
    best.k_per_split = kt * kBK;
    return best;
  }
  // Plain stores and (past the short-K rule above) residual adds with N a
  // multiple of 192 (the N = 768 products' dX, the fc-proj forward): 384x192
  // tiles of 8 waves (4 x 2 patches of 96 x 96), 64 x 4 = 256 tiles at
  // M = 24576, one round, and a third less operand traffic per product than
  // 192x192; the residual tile goes straight to registers after the main loop
  if (!may_split && (epi == EPI_STORE || epi == EPI_BIAS_RES) && a_kmajor && b_kmajor && N % 192 == 0 &&
      M >= 8192) {
    best = Plan{384, 192, 1, kt * kBK};
    return best;
  }
  for (const Cand& c : cands) {
    const bool c192 = c.bm == 192;
    if (c192 && !(a_kmajor && b_kmajor)) continue;                  // m-major DMA needs 64 | 1024 / (2 R)
    if (!may_split && !c192 && (c.bm != def_bm || c.bn != def_bn)) continue;
    if (c192 && (M < 2048 || N < 192)) continue;
    const long tiles = ceil_div64(M, c.bm) * ceil_div64(N, c.bn);
    const double mn4 = (double)M * N * 4.0;
    for (int sc = 1; sc <= (may_split ? 64 : 1) && sc <= kt; ++sc) {
      const int kps = (kt + sc - 1) / sc;
      const int real = (kt + kps - 1) / kps;
      const double rounds = (double)ceil_div64(tiles * real, 256);
      double t = rounds * kps * c.t_step;
      if (wgrad) t += mn4 * (2.0 * real + 1.0) / 5e12;
      else if (real > 1) t += (mn4 * 2.0 * real + (double)M * N * 2.0) / 5e12;
      if (t < best_t * (1.0 - 1e-9)) { best_t = t; best = Plan{c.bm, c.bn, real, 0}; }
    }
  }
  const int kps = (kt + best.splits - 1) / best.splits;
  best.k_per_split = kps * kBK;
  best.splits = (kt + kps - 1) / kps;
  // a long K per tile amortises the K-groups' exchange of partial sums
  // (measured: classifier dX, K = 50304, 1.77 -> 1.59 ms)
  if (best.bm == 192 && best.k_per_split >= 8192 && !epi_has_aux(epi)) best.kgroups = 2;
  return best;
}

// Launch plan of an fp8 product (both operands k-major, K steps of 128): the
// 8-wave 256x256 tile or the two-block 128x128 tile, and a split of K for
// the weight gradient and long plain stores, by the bf16 cost model (an fp8
// K step of 128 takes as many matrix-core cycles as a bf16 step of 64).
// Epilogues that read an input tile (residual add, GELU' multiply) take the
// two-block 128x128 tile, as in bf16, and the N = 768 products the 384x192
// tile, as in bf16 (the plain-store form spills 12 registers with the larger
// fp8 fragments and is still faster: FP8 step 27.84 -> 27.41 ms).
Plan plan_fp8(int epi, int M, int N, int K) {
  const int kt = (int)ceil_div64(K, kBK8);
  const bool wgrad = epi == EPI_WGRAD;
  const bool may_split = wgrad || (epi == EPI_STORE && K >= 8192);
  // as in bf16: the 8-wave 384x192 tile for N = 768 plain stores (dX) and
  // the long-K residual add (fc-proj forward)
  if (!may_split && (epi == EPI_STORE || (epi == EPI_BIAS_RES && K > 1024)) && N % 192 == 0 && M >= 8192)
    return Plan{384, 192, 1, kt * kBK8};
  if (!may_split && epi_has_aux(epi)) return Plan{128, 128, 1, kt * kBK8};
  struct Cand { int bm, bn; double t_step; };
  const Cand cands[2] = {{256, 256, 2.75e-6}, {128, 128, 1.25e-6}};
  Plan best{128, 128, 1, kt * kBK8};
  double best_t = 1e300;
  for (const Cand& c : cands) {
    if (!may_split && c.bm == 256 && (M < 2048 || N < 2048)) continue;
    const long tiles = ceil_div64(M, c.bm) * ceil_div64(N, c.bn);
    const double mn4 = (double)M * N * 4.0;
    for (int sc = 1; sc <= (may_split ? 64 : 1) && sc <= kt; ++sc) {
      const int kps = (kt + sc - 1) / sc;
      const int real = (kt + kps - 1) / kps;
      double t = (double)ceil_div64(tiles * real, 256) * kps * c.t_step;
      if (wgrad) t += mn4 * (2.0 * real + 1.0) / 5e12;
      else if (real > 1) t += (mn4 * 2.0 * real + (double)M * N * 2.0) / 5e12;
      if (t < best_t * (1.0 - 1e-9)) { best_t = t; best = Plan{c.bm, c.bn, real, 0}; }
    }
  }
  const int kps = (kt + best.splits - 1) / best.splits;
  best.k_per_split = kps * kBK8;
  best.splits = (kt + kps - 1) / kps;
  return best;
}

Plan plan_gemm(int dtype, int fp8, int epi, int M, int N, int K, bool a_kmajor, bool b_kmajor) {
  if (fp8) return plan_fp8(epi, M, N, K);
  return plan_bf16(epi, M, N, K, a_kmajor, b_kmajor);
}

int gemm_splits(int dtype, int epi, int M, int N, int K, bool a_kmajor, bool b_kmajor, int fp8 = 0) {
  if (dtype == F32) return 1;
  return plan_gemm(dtype, fp8, epi, M, N, K, a_kmajor, b_kmajor).splits;
}

// Compute units of the current device (the persistent grid's size).
inline int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess)
    return 0;
  return cus;
}

// One block per unit, or -- for the kernels that prefetch the next unit
// during the epilogue, when there are more units than block slots -- one
// block per slot (compute units x blocks per unit; a multiple of the 8 XCDs)
// looping over units.
template <int BM, int BN, int EPI, bool A_KMAJ, bool B_KMAJ, bool BIAS_GRAD, int KGS = 1, bool F8 = false,
          int FMT_A = 0>
int launch_tile(const MfmaArgs& a, int splits, hipStream_t stream) {
  using S = DmaShape<BM, BN, EPI, KGS>;
  const unsigned tiles = (unsigned)(ceil_div64(a.M, BM) * ceil_div64(a.N, BN));
  MfmaArgs b = a;
  b.splits = splits;
  b.persistent = 0;
  dim3 grid(tiles, (unsigned)splits);
  if constexpr (!epi_has_aux(EPI) && KGS == 1 && S::EPI_IN_STAGE) {
    const long slots = (long)device_cus() * S::OCC;
    if (slots > 0 && slots % 8 == 0 && (long)tiles * splits > slots) {
      b.persistent = 1;
      grid = dim3((unsigned)slots, 1);
    }
  }
  mark_begin(0, stream);
  hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, A_KMAJ, B_KMAJ, EPI, BIAS_GRAD, KGS, F8, FMT_A>), grid,
                     dim3(64 * gemm_waves(BM, BN, EPI, KGS)), 0, stream, b);
  GPT2_LAUNCH_CHECK();
  mark_end(0, stream);
  return 0;
}

template <int EPI, bool A_KMAJ, bool B_KMAJ, bool BIAS_GRAD>
int launch_mfma(const MfmaArgs& a, const Plan& pl, hipStream_t stream) {
  if (pl.bm == 256 && pl.bn == 256) return launch_tile<256, 256, EPI, A_KMAJ, B_KMAJ, BIAS_GRAD>(a, pl.splits, stream);
  if (pl.bm == 256 && pl.bn == 128) return launch_tile<256, 128, EPI, A_KMAJ, B_KMAJ, BIAS_GRAD>(a, pl.splits, stream);
  if (pl.bm == 128 && pl.bn == 256) return launch_tile<128, 256, EPI, A_KMAJ, B_KMAJ, BIAS_GRAD>(a, pl.splits, stream);
  if constexpr (A_KMAJ && B_KMAJ && !BIAS_GRAD &&
                (EPI == EPI_STORE || EPI == EPI_BIAS_RES || EPI == EPI_BIAS || EPI == EPI_BIAS_GELU_D ||
                 EPI == EPI_BIAS_RELU2_D))
    if (pl.bm == 384 && pl.bn == 192) return launch_tile<384, 192, EPI, A_KMAJ, B_KMAJ, BIAS_GRAD>(a, pl.splits, stream);
  if constexpr (A_KMAJ && B_KMAJ)
    if (pl.bm == 192 && pl.bn == 192) {
      if constexpr (!BIAS_GRAD && !epi_has_aux(EPI))
        if (pl.kgroups == 2) return launch_tile<192, 192, EPI, A_KMAJ, B_KMAJ, BIAS_GRAD, 2>(a, pl.splits, stream);
      return launch_tile<192, 192, EPI, A_KMAJ, B_KMAJ, BIAS_GRAD>(a, pl.splits, stream);
    }
  return launch_tile<128, 128, EPI, A_KMAJ, B_KMAJ, BIAS_GRAD>(a, pl.splits, stream);
}

template <int EPI, bool A_KMAJ, bool B_KMAJ>
int launch_simt(const SimtArgs& a, int splits, hipStream_t stream) {
  dim3 grid((unsigned)ceil_div64(a.N, 64), (unsigned)ceil_div64(a.M, 64), (unsigned)splits);
  mark_begin(0, stream);
  hipLaunchKernelGGL((gemm_f32_simt_kernel<A_KMAJ, B_KMAJ, EPI>), grid, dim3(256), 0, stream, a);
  GPT2_LAUNCH_CHECK();
  mark_end(0, stream);
  return 0;
}

}  // namespace
}  // namespace gpt2k
