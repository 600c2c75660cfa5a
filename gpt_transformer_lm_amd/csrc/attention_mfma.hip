// Causal flash attention on the bf16 matrix cores (gfx950), head dim 64.
//
// Same mathematics as the general path in attention.hip (exact causal
// softmax attention, lse saved in fp32, backward from lse and
// D_i = dO_i . O_i), organised around v_mfma_f32_32x32x16_bf16:
//
// Forward: a block owns 128 queries of one (batch, head), 32 per wave; K and
// V stream through LDS in 64-key stages.  Each wave computes S^T = K Q^T per
// 32-key slice (K from LDS, Q fragments held in registers), so its
// accumulator holds one query per lane and 16 keys per lane: the running max
// / sum of the online softmax are per-lane scalars, the probabilities P
// (bf16) are already in the register layout of the B operand of
// O^T = V^T P^T, and the rescaling of O^T is a per-lane scalar multiply.
// Both 32-key slices of a 64-key stage are scored before one softmax update:
// the two half-waves holding the same query exchange their maxima once per
// stage with v_permlane32_swap, and each keeps its own share of the row sum
// until the end.
//
// Backward (deterministic, no atomics), two kernels:
//   dK/dV: a block owns 128 keys (32 per wave) and streams 64-query stages of
//     Q, dO, lse and D through LDS; per 32-query slice: S = Q K^T,
//     dP = dO V^T (K, V fragments in registers, one key per lane),
//     P = exp(S/sqrt(d) - lse), dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS.
//   dQ: a block owns 128 queries and streams 64-key stages of K and V:
//     S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
// Work per causal tile is unbalanced, so blocks take the heaviest tiles first.
//
// Streaming: every stage is a set of 64 x 64 bf16 tiles copied global -> LDS
// with buffer_load ... lds (no register staging) into a ring of NS stages, so
// NS - 1 stages are in flight while one is computed.  Tiles keep the natural
// [row][64] layout with XOR-swizzled 16-byte chunks; the transposed operands
// (V^T, Q^T, dO^T, K^T) are read from the same tiles with ds_read_b64_tr_b16,
// with per-lane addresses that deliver the keys / queries in exactly the order
// in which the 32 x 32 accumulator holds them, so P and dS feed the next
// product without any shuffle.  Rows past the sequence end read as zeros
// (buffer range check).

#include "kernels.h"

namespace gpt2k {
namespace {

typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int HD = 64;
constexpr int ROWS = 128;            // queries (fwd, dQ) or keys (dK/dV) per block
constexpr int STAGE = 64;            // rows streamed per LDS stage
// Stages in each kernel's LDS ring: as deep as the LDS allows at the
// occupancy the kernel's registers permit (forward: 4 blocks of 2 x 16 KiB per
// compute unit; dQ: 3 blocks of 3 x 16 KiB; dK/dV: 2 blocks of 4 x 18 KiB).
constexpr int NS_FWD = 2, NS_DQ = 3, NS_DKDV = 4;
// Products whose LDS fragments the dK/dV kernel has in flight ahead of the
// matrix instruction that uses them (LDS latency is several products long;
// measured at 124M: 1 -> 1.75, 2 -> 1.65, 3 -> 1.63, 4 -> 1.64, 6 -> 1.66 ms
// per step).
constexpr int DKDV_PREFETCH = 3;
constexpr int TILE = STAGE * HD * 2; // bytes of one 64 x 64 bf16 tile
constexpr uint32_t kOut = 0xFFFFFFF0u;   // offset past every buffer range
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row ^ (row >> 3)) & 7); }

__device__ __forceinline__ floatx16 mfma(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine of a value held per half-wave: every lane gets op(own, value of
// lane l ^ 32).  gfx950's v_permlane32_swap exchanges the two halves in the
// VALU (no LDS round trip); its two outputs hold, in each lane, the lane's own
// value and its partner's (in one order or the other), so the symmetric
// combine needs no lane select.
__device__ __forceinline__ float half_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Rows row0 .. row0+63, columns col0 .. col0+63 of a row-major bf16 matrix
// (row stride ld elements, addressed from the resource's base) into a tile:
// tile row r occupies bytes 128 r .. 128 r + 127 and its logical 16-byte chunk
// c sits at physical chunk swz(r, c).  Each of the 4 waves issues 2 of the 8
// one-KiB instructions (instruction iq fills rows 8 iq .. 8 iq + 7; lane L
// writes physical chunk L % 8 of row 8 iq + L / 8).
__device__ __forceinline__ void tile_dma(i32x4_rsrc rs, GPT2_LDS char* tile, int wave, int lane,
                                         int row0, int ld, int col0) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int iq = wave * 2 + q;
    const int r = 8 * iq + (lane >> 3);
    const int c = (lane & 7) ^ ((r ^ (r >> 3)) & 7);
    const uint32_t off = (uint32_t)(((int64_t)(row0 + r) * ld + col0 + c * 8) * 2);
    dma_lds16(rs, (GPT2_LDS void*)(tile + iq * 1024), off);
  }
}

// 64 consecutive fp32 values starting at element row0 into the first 256 bytes
// of a 1-KiB LDS region (lanes 0..15 move 16 bytes each, the others zeros).
__device__ __forceinline__ void vec_dma(i32x4_rsrc rs, GPT2_LDS char* dst, int lane, int row0) {
  const uint32_t off = lane < 16 ? (uint32_t)((row0 + 4 * lane) * 4) : kOut;
  dma_lds16(rs, (GPT2_LDS void*)dst, off);
}

// A-operand fragment, natural orientation: tile row row0 + lane % 32, k16 step s
// (columns 16 s + 8 (lane / 32) .. +7).
__device__ __forceinline__ bf16x8 frag_nat(const GPT2_LDS char* t, int row0, int s, int lane) {
  const int row = row0 + (lane & 31), c = 2 * s + (lane >> 5);
  return *reinterpret_cast<const GPT2_LDS bf16x8*>(t + row * 128 + swz(row, c) * 16);
}

// A-operand fragment of the transposed tile: column d0 + lane % 32 as the
// fragment row, and tile rows {r0 + 4 hi + 0..3, r0 + 8 + 4 hi + 0..3}
// (hi = lane / 32) as its 8 k values -- the row order of registers 8u..8u+7
// of a 32 x 32 accumulator.  Two ds_read_b64_tr_b16: within each 16-lane group
// lane j receives component j % 4 of the 8-byte runs read by lanes j / 4 + 4 e,
// so lane i of group g reads row r0 + 4 (g / 2) + 8 r + i / 4 at columns
// d0 + 16 (g % 2) + 4 (i % 4) .. +3.
__device__ __forceinline__ bf16x8 frag_tr(const GPT2_LDS char* t, int d0, int r0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int d = d0 + 16 * (g & 1) + 4 * (i & 3);
  bf16x8 out;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = r0 + 4 * (g >> 1) + 8 * r + (i >> 2);
    const GPT2_LDS bf16x4* p =
        reinterpret_cast<const GPT2_LDS bf16x4*>(t + row * 128 + swz(row, d >> 3) * 16 + (d & 7) * 2);
    const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<GPT2_LDS bf16x4*>(p));
#pragma unroll
    for (int e = 0; e < 4; ++e) out[4 * r + e] = v[e];
  }
  return out;
}

// The same two reads with the per-lane byte offsets precomputed (frag_off /
// frag_tr_off below), for loops whose tile base is a compile-time LDS address:
// each read is then one instruction with an immediate offset.
__device__ __forceinline__ uint32_t frag_off(int row0, int s, int lane) {
  const int row = row0 + (lane & 31), c = 2 * s + (lane >> 5);
  return (uint32_t)(row * 128 + swz(row, c) * 16);
}
__device__ __forceinline__ uint32_t frag_tr_off(int d0, int r0, int r, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int d = d0 + 16 * (g & 1) + 4 * (i & 3);
  const int row = r0 + 4 * (g >> 1) + 8 * r + (i >> 2);
  return (uint32_t)(row * 128 + swz(row, d >> 3) * 16 + (d & 7) * 2);
}
// Keeps a precomputed offset in one register (the compiler would otherwise
// re-form it from its parts with an add before every read).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
// An empty asm that rewrites x: x's producers stay before this point, in
// this block, instead of sinking towards a later use.
__device__ __forceinline__ void pin(bf16x8& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ bf16x8 frag_at(const GPT2_LDS char* t, uint32_t off) {
  return *reinterpret_cast<const GPT2_LDS bf16x8*>(t + off);
}
__device__ __forceinline__ bf16x8 frag_tr_at(const GPT2_LDS char* t, uint32_t off0, uint32_t off1) {
  const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      const_cast<GPT2_LDS bf16x4*>(reinterpret_cast<const GPT2_LDS bf16x4*>(t + off0)));
  const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      const_cast<GPT2_LDS bf16x4*>(reinterpret_cast<const GPT2_LDS bf16x4*>(t + off1)));
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[e] = v0[e];
    out[4 + e] = v1[e];
  }
  return out;
}

// Row (lane % 32) of a global [row][64] matrix as four B-operand fragments.
__device__ __forceinline__ void frags_global(const bf16* G, size_t ld, int row, int nrows, int lane, bf16x8 f[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (row < nrows) {
      f[s] = *reinterpret_cast<const bf16x8*>(G + (size_t)row * ld + 16 * s + 8 * (lane >> 5));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[s][e] = (bf16)0.f;
    }
  }
}

// Index (0..31) inside a 32-slice of the row that accumulator register r holds.
// The block's (tile, batch·head) pair, with whole heads on one XCD: the
// dispatcher hands consecutive linear block ids to the 8 XCDs in turn, so
// linear id n runs on XCD n % 8; renumbering n -> (n % 8) q + n / 8 (q =
// blocks / 8, the tail of a grid that is not a multiple of 8 left as it is)
// gives each XCD a run of consecutive ids, taken head-major, and the tiles of
// one head re-read its K / V (or Q / dO) rows from that XCD's L2 instead of
// from memory.  Within a head, tile 0 comes first.
__device__ __forceinline__ void head_major_block(int& tile, int& bh) {
  const int X = (int)gridDim.x, n = (int)(blockIdx.x + gridDim.x * blockIdx.y);
  const int q = (int)(gridDim.x * gridDim.y) / 8;
  const int id = n < 8 * q ? (n % 8) * q + n / 8 : n;
  bh = id / X;
  tile = id % X;
}

__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Writes 64 values of row `row` held as two 32 x 32 accumulators (d on registers).
// Returns the largest |acc * mul| stored (for an fp8 quantisation that follows).
__device__ __forceinline__ float store_row64(bf16* dst, const floatx16 acc[2], float mul, int lane) {
  float m = 0.f;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = acc[dt][4 * g + e] * mul;
        v[e] = (bf16)x;
        m = fmaxf(m, fabsf(x));
      }
      *reinterpret_cast<bf16x4*>(dst + dt * 32 + 8 * g + 4 * (lane >> 5)) = v;
    }
  return m;
}

// ------------------------------------------------------------------ forward

__global__ __launch_bounds__(256, 3) void attn_fwd_mfma_kernel(int T, int H, const bf16* __restrict__ qkv,
                                                            bf16* __restrict__ out, float* __restrict__ lse,
                                                            float scale) {
  constexpr int NS = NS_FWD;
  __shared__ __attribute__((aligned(1024))) char ring[NS][2 * TILE];   // K tile, V tile
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), hi = lane >> 5;
  const int nqt = (T + ROWS - 1) / ROWS;
  int tile, bh;
  head_major_block(tile, bh);
  const int qt = nqt - 1 - tile;   // longer rows first
  const int b = bh / H, h = bh % H;
  const int C = H * HD;
  const int ld = 3 * C;
  const bf16* Bg = qkv + (size_t)b * T * ld;                 // row 0 of this sequence
  const bf16* Qg = Bg + h * HD;
  const int q0 = qt * ROWS, qw0 = q0 + wave * 32, myq = qw0 + (lane & 31);
  const float sl2 = scale * kLog2e;

  bf16x8 qf[4];
  frags_global(Qg, ld, myq, T, lane, qf);
  floatx16 oacc[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_i = -INFINITY, l_i = 0.f;

  const int kend = min(T, q0 + ROWS);
  const int nst = (kend + STAGE - 1) / STAGE;
  // Per-lane byte offsets of this wave's two DMA instructions per tile,
  // relative to the first row of a stage; each stage gets a buffer resource
  // based at its first key row (scalar arithmetic), so the range check still
  // zero-fills rows past the sequence end and the lane offsets stay fixed.
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int iq = wave * 2 + q;
    const int r = 8 * iq + (lane >> 3);
    const int c = (lane & 7) ^ ((r ^ (r >> 3)) & 7);
    koff[q] = (uint32_t)((r * ld + C + h * HD + c * 8) * 2);
    voff[q] = (uint32_t)((r * ld + 2 * C + h * HD + c * 8) * 2);
  }
  auto issue = [&](int st, int slot) {
    const int row0 = st * STAGE;
    const i32x4_rsrc rst = make_rsrc4(Bg + (size_t)row0 * ld, (uint32_t)((size_t)(T - row0) * ld * 2));
    GPT2_LDS char* base = (GPT2_LDS char*)ring[slot];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int iq = wave * 2 + q;
      dma_lds16(rst, (GPT2_LDS void*)(base + iq * 1024), koff[q]);
      dma_lds16(rst, (GPT2_LDS void*)(base + TILE + iq * 1024), voff[q]);
    }
  };
  // LDS offsets of the K fragments (slice u2, k16 step k) and of the two
  // halves of the transposed V fragments (d block dt, 16-key group j, half r)
  uint32_t koffs[2][4], voffs[2][4][2];
#pragma unroll
  for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
    for (int k = 0; k < 4; ++k) koffs[u2][k] = opaque(frag_off(32 * u2, k, lane));
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 2; ++r) voffs[dt][j][r] = opaque(frag_tr_off(32 * dt, 16 * j, r, lane));
  // the fragments loaded to registers above have landed: the compiler's own
  // waits for them would otherwise sit in the loop and drain the DMA ring
  wait_vmcnt<0>();
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nst) issue(s, s);
  // The stage loop is unrolled by the ring depth so that every LDS address is
  // a per-lane offset computed once plus an immediate.
  for (int st0 = 0; st0 < nst; st0 += NS) {
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      const int st = st0 + sl;
      if (st >= nst) break;
      // this wave's part of stage st has landed, then everyone's has; the ring
      // slot refilled next was last read in the previous iteration
      if (st + NS - 2 < nst) wait_vmcnt<(NS - 2) * 4>();
      else wait_vmcnt<0>();
      lds_barrier();
      if (st + NS - 1 < nst) issue(st + NS - 1, (sl + NS - 1) % NS);
      const GPT2_LDS char* Kc = (const GPT2_LDS char*)ring[sl];
      const GPT2_LDS char* Vc = Kc + TILE;
      const int k0 = st * STAGE;
      // Both 32-key slices' score products first, then one softmax update for
      // the 64 keys (one max exchange, at most one rescale), then both P V
      // products.  The second slice is skipped when it lies wholly above this
      // wave's diagonal; keys k0 .. k0 + 31 always include key k0 <= every
      // query of the wave, so the running maximum is finite from the first
      // stage on.
      if (k0 <= qw0 + 31 && k0 < T) {
        const bool two = k0 + 32 <= qw0 + 31 && k0 + 32 < T;
        floatx16 s[2];
#pragma unroll
        for (int u2 = 0; u2 < 2; ++u2) {
          if (u2 == 0 || two) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[u2][r] = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) s[u2] = mfma(frag_at(Kc, koffs[u2][k]), qf[k], s[u2]);
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int u2 = 0; u2 < 2; ++u2) {
          if (u2 == 0 || two) {
            const int kb = k0 + 32 * u2;
            // the causal / end-of-sequence mask only touches slices on the
            // diagonal (a wave-uniform test, so the common case runs unmasked)
            if ((kb + 31 > qw0) || (kb + 32 > T)) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = kb + acc_row(r, lane);
                if (key > myq || key >= T) s[u2][r] = -INFINITY;
              }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[u2][r]);
          }
        }
        mx = half_max(mx);
        // The exponent's reference m_i only moves when some lane's maximum
        // exceeds it by more than 2^8 (a wave-uniform vote): below that the
        // probabilities exp2(s - m_i) stay under 256 and the row sum and O
        // just carry the common factor, which the final division and the
        // log-sum-exp (taken against the same m_i) remove exactly.  On the
        // first stage m_i = -inf, so it always moves there.
        const float m_run = fmaxf(m_i, mx * sl2);   // sl2 > 0: scaled max = max of scaled
        if (__any(m_run > m_i + 8.0f)) {
          const float alpha = ex2(m_i - m_run);
          l_i *= alpha;
#pragma unroll
          for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
          m_i = m_run;
        }
#pragma unroll
        for (int u2 = 0; u2 < 2; ++u2) {
          if (u2 == 0 || two) {
            float rs_ = 0.f;
            bf16x8 pb[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float p = ex2(fmaf(s[u2][r], sl2, -m_i));
              rs_ += p;
              pb[r >> 3][r & 7] = (bf16)p;
            }
            // l_i is this half-wave's share of the row sum (both halves use
            // the same reference, so their shares add up at the end)
            l_i += rs_;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int dt = 0; dt < 2; ++dt)
                oacc[dt] = mfma(frag_tr_at(Vc, voffs[dt][2 * u2 + u][0], voffs[dt][2 * u2 + u][1]), pb[u],
                                oacc[dt]);
          }
        }
      }
    }
  }
  l_i = half_sum(l_i);
  if (myq < T) {
    store_row64(out + ((size_t)b * T + myq) * C + h * HD, oacc, 1.0f / l_i, lane);
    if (hi == 0) lse[(size_t)bh * T + myq] = (m_i + __log2f(l_i)) * kLn2;
  }
}

// ------------------------------------------------------------------ backward dK, dV

constexpr int KV_STAGE_BYTES = 2 * TILE + 2048;   // Q tile, dO tile, lse (1 KiB), D (1 KiB)

__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_mfma_kernel(int T, int H, const bf16* __restrict__ qkv,
                                                                 const bf16* __restrict__ dout,
                                                                 const float* __restrict__ lse2,
                                                                 const float* __restrict__ Dv,
                                                                 bf16* __restrict__ dqkv, float scale,
                                                                 float* __restrict__ amax) {
  constexpr int NS = NS_DKDV;
  __shared__ __attribute__((aligned(1024))) char ring[NS][KV_STAGE_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int ktile, bh;
  head_major_block(ktile, bh);   // lower key tiles see more queries: launched first
  const int b = bh / H, h = bh % H;
  const int C = H * HD;
  const int ld = 3 * C;
  const bf16* Bg = qkv + (size_t)b * T * ld;
  const bf16* Kg = Bg + C + h * HD;
  const bf16* Vg = Bg + 2 * C + h * HD;
  const bf16* Og = dout + (size_t)b * T * C;
  const int k0 = ktile * ROWS, kw0 = k0 + wave * 32, mykey = kw0 + (lane & 31);
  const float sl2 = scale * kLog2e;

  bf16x8 kf[4], vf[4];
  frags_global(Kg, ld, mykey, T, lane, kf);
  frags_global(Vg, ld, mykey, T, lane, vf);
  floatx16 dk[2], dv[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[dt][r] = 0.f; dv[dt][r] = 0.f; }

  const int qbeg = k0;                          // queries before the tile see none of its keys
  const int nst = T > qbeg ? (T - qbeg + STAGE - 1) / STAGE : 0;
  // DMA with fixed per-lane offsets and one set of buffer resources per stage
  // based at its first query row (scalar arithmetic; the range check still
  // zero-fills rows past the sequence end)
  uint32_t qoff[2], ooff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int iq = wave * 2 + q;
    const int r = 8 * iq + (lane >> 3);
    const int c = (lane & 7) ^ ((r ^ (r >> 3)) & 7);
    qoff[q] = (uint32_t)((r * ld + h * HD + c * 8) * 2);
    ooff[q] = (uint32_t)((r * C + h * HD + c * 8) * 2);
  }
  const uint32_t vecoff = lane < 16 ? (uint32_t)(16 * lane) : kOut;
  auto issue = [&](int st, int slot) {
    GPT2_LDS char* base = (GPT2_LDS char*)ring[slot];
    const int q0 = qbeg + st * STAGE;
    const i32x4_rsrc rq = make_rsrc4(Bg + (size_t)q0 * ld, (uint32_t)((size_t)(T - q0) * ld * 2));
    const i32x4_rsrc ro = make_rsrc4(Og + (size_t)q0 * C, (uint32_t)((size_t)(T - q0) * C * 2));
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int iq = wave * 2 + q;
      dma_lds16(rq, (GPT2_LDS void*)(base + iq * 1024), qoff[q]);
      dma_lds16(ro, (GPT2_LDS void*)(base + TILE + iq * 1024), ooff[q]);
    }
    if (wave == 0)
      dma_lds16(make_rsrc4(lse2 + (size_t)bh * T + q0, (uint32_t)((T - q0) * 4)), (GPT2_LDS void*)(base + 2 * TILE),
                vecoff);
    if (wave == 1)
      dma_lds16(make_rsrc4(Dv + (size_t)bh * T + q0, (uint32_t)((T - q0) * 4)),
                (GPT2_LDS void*)(base + 2 * TILE + 1024), vecoff);
  };
  // LDS offsets of the Q / dO fragments (32-query slice u2, k16 step k), of
  // the two halves of the transposed ones (d block dt, 16-query group j) and
  // of this lane's lse / D values
  uint32_t noffs[2][4], toffs[2][4][2];
#pragma unroll
  for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
    for (int k = 0; k < 4; ++k) noffs[u2][k] = frag_off(32 * u2, k, lane);
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 2; ++r) toffs[dt][j][r] = frag_tr_off(32 * dt, 16 * j, r, lane);
  const uint32_t ldoff = (uint32_t)(16 * (lane >> 5));
  // the fragments loaded to registers above have landed: the compiler's own
  // waits for them would otherwise sit in the loop and drain the DMA ring
  wait_vmcnt<0>();
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nst) issue(s, s);
  // unrolled by the ring depth: LDS addresses are fixed offsets + immediates
  for (int st0 = 0; st0 < nst; st0 += NS) {
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      const int st = st0 + sl;
      if (st >= nst) break;
      // at most 5 DMA instructions per wave and stage: waiting until (NS - 2) * 4
      // remain is sufficient for every wave
      if (st + NS - 2 < nst) wait_vmcnt<(NS - 2) * 4>();
      else wait_vmcnt<0>();
      lds_barrier();
      if (st + NS - 1 < nst) issue(st + NS - 1, (sl + NS - 1) % NS);
      const GPT2_LDS char* Qs = (const GPT2_LDS char*)ring[sl];
      const GPT2_LDS char* Os = Qs + TILE;
      const GPT2_LDS char* Ls = Qs + 2 * TILE;
      const GPT2_LDS char* Ds = Qs + 2 * TILE + 1024;
      const int q0 = qbeg + st * STAGE;
      // Issue order: slice 0's score products; slice 1's score products, each
      // followed by two rows of slice 0's vector work; slice 0's dV / dK
      // products, each followed by two rows of slice 1's vector work; slice
      // 1's dV / dK products.  Each product's fragments are read a few
      // products ahead, and scheduling barriers keep the order (in-order
      // issue would otherwise leave the matrix cores idle during the
      // exponentials and the vector units idle during the products).  Masked
      // entries (key after query, query past the end) get S = -inf, so P = 0
      // and dS = 0 exactly (zero-filled rows past the end have dP = D = 0); a
      // slice no query of which sees a key of the wave only adds zeros.
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      floatx16 s[2], dp[2];
      bf16x8 pb[2][2], db[2][2];
      float lv[16];
      auto mask = [&](int u2) {   // only on slices that cross the diagonal or the end
        const int qb = q0 + 32 * u2;
        if (qb < kw0 + 31 || qb + 32 > T) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = qb + acc_row(r, lane);
            if (mykey > q || q >= T) s[u2][r] = -__builtin_inff();
          }
        }
      };
      // s[r] is query q0 + 32 u2 + acc_row(r), key mykey; the lane's 16 query
      // rows are 32 u2 + 4 hi + 8 g + 0..3 (g = 0..3): four 16-byte reads each
      // of lse·log2e (into lv) and of -D (dP's initial accumulator, so the
      // products leave dP - D)
      auto load_l = [&](int u2) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *reinterpret_cast<const GPT2_LDS f32x4*>(Ls + ldoff + 4 * (32 * u2 + 8 * g));
#pragma unroll
          for (int e = 0; e < 4; ++e) lv[4 * g + e] = l4[e];
        }
      };
      auto load_nd = [&](int u2) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 d4 = *reinterpret_cast<const GPT2_LDS f32x4*>(Ds + ldoff + 4 * (32 * u2 + 8 * g));
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[u2][4 * g + e] = d4[e];
        }
      };
      // P and dS of rows r, r + 1 of slice u2
      auto softgrad2 = [&](int u2, int r) {
#pragma unroll
        for (int e = r; e < r + 2; ++e) {
          const float p = ex2(fmaf(s[u2][e], sl2, -lv[e]));
          pb[u2][e >> 3][e & 7] = (bf16)p;
          db[u2][e >> 3][e & 7] = (bf16)(p * dp[u2][e]);
        }
      };
      // score product i of slice u2: k16 step i / 2 of S (i even) or dP (odd)
      auto score_frag = [&](int u2, int i) { return frag_at((i & 1) ? Os : Qs, noffs[u2][i >> 1]); };
      auto score_mfma = [&](int u2, int i, const bf16x8& a) {
        if (i & 1) dp[u2] = mfma(a, vf[i >> 1], dp[u2]);
        else s[u2] = mfma(a, kf[i >> 1], s[u2]);
      };
      // update product i of slice u2: u = i / 4, dt = (i / 2) % 2, dV (i even) or dK (odd)
      auto upd_frag = [&](int u2, int i) {
        const int u = i >> 2, dt = (i >> 1) & 1;
        return frag_tr_at((i & 1) ? Qs : Os, toffs[dt][2 * u2 + u][0], toffs[dt][2 * u2 + u][1]);
      };
      auto upd_mfma = [&](int u2, int i, const bf16x8& a) {
        const int u = i >> 2, dt = (i >> 1) & 1;
        if (i & 1) dk[dt] = mfma(a, db[u2][u], dk[dt]);
        else dv[dt] = mfma(a, pb[u2][u], dv[dt]);
      };
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[u2][r] = 0.f;
        load_nd(u2);
      }
      // The stage's 32 products in issue order: op 0..7 slice 0's S / dP,
      // 8..15 slice 1's, 16..23 slice 0's dV / dK, 24..31 slice 1's; the
      // fragments of op o + PD are read right after op o is issued.
      constexpr int PD = DKDV_PREFETCH;
      auto frag_of = [&](int o) {
        return o < 16 ? score_frag(o >> 3, o & 7) : upd_frag((o >> 3) & 1, o & 7);
      };
      auto mfma_of = [&](int o, const bf16x8& a) {
        if (o < 16) score_mfma(o >> 3, o & 7, a);
        else upd_mfma((o >> 3) & 1, o & 7, a);
      };
      bf16x8 fq[PD];
#pragma unroll
      for (int o = 0; o < PD; ++o) fq[o] = frag_of(o);
      auto op = [&](int o) {
        const bf16x8 a = fq[o % PD];
        if (o + PD < 32) fq[o % PD] = frag_of(o + PD);
        mfma_of(o, a);
      };
      // slice 0's score products
#pragma unroll
      for (int o = 0; o < 8; ++o) {
        op(o);
        __builtin_amdgcn_sched_barrier(0);
      }
      mask(0);
      // slice 1's score products with slice 0's vector work
      load_l(0);
#pragma unroll
      for (int o = 8; o < 16; ++o) {
        op(o);
        softgrad2(0, 2 * (o - 8));
        __builtin_amdgcn_sched_barrier(0);
      }
      // slice 0's P and dS are produced above: they would otherwise sink past
      // the next branch to their use and the interleaving would be lost
      pin(pb[0][0]); pin(pb[0][1]); pin(db[0][0]); pin(db[0][1]);
      mask(1);
      // slice 0's dV / dK products with slice 1's vector work
      load_l(1);
#pragma unroll
      for (int o = 16; o < 24; ++o) {
        op(o);
        softgrad2(1, 2 * (o - 16));
        __builtin_amdgcn_sched_barrier(0);
      }
      // slice 1's dV / dK products
#pragma unroll
      for (int o = 24; o < 32; ++o) {
        op(o);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  float mx = 0.f;
  if (mykey < T) {
    bf16* dst = dqkv + ((size_t)b * T + mykey) * ld + h * HD;
    mx = store_row64(dst + C, dk, scale, lane);
    mx = fmaxf(mx, store_row64(dst + 2 * C, dv, 1.0f, lane));
  }
  if (amax) {   // (uniform) the fp8 quantisation of dqkv reads the maximum from these slots
    mx = wave_max(mx);
    if (lane == 0) amax_atomic_bf16(amax, (int)(blockIdx.y * gridDim.x + blockIdx.x) * 4 + wave, mx);
  }
}

// ------------------------------------------------------------------ backward dQ

// Also the per-query quantities both backward kernels use, D_i = dO_i . O_i
// and lse_i log2(e), from the rows the kernel holds anyway (so it runs before
// the dK / dV kernel, which reads them).  AM: also dQ's maximum into the
// amax slots (an instance of its own: at three blocks per compute unit the
// extra epilogue work would cost the plain kernel a register).
template <bool AM>
__global__ __launch_bounds__(256, 3) void attn_bwd_dq_mfma_kernel(int T, int H, const bf16* __restrict__ qkv,
                                                               const bf16* __restrict__ out,
                                                               const bf16* __restrict__ dout,
                                                               const float* __restrict__ lse,
                                                               float* __restrict__ lse2,
                                                               float* __restrict__ Dv,
                                                               bf16* __restrict__ dqkv, float scale,
                                                               float* __restrict__ amax) {
  constexpr int NS = NS_DQ;
  __shared__ __attribute__((aligned(1024))) char ring[NS][2 * TILE];   // K tile, V tile
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqt = (T + ROWS - 1) / ROWS;
  int tile, bh;
  head_major_block(tile, bh);
  const int qt = nqt - 1 - tile;   // longer rows first
  const int b = bh / H, h = bh % H;
  const int C = H * HD;
  const int ld = 3 * C;
  const bf16* Bg = qkv + (size_t)b * T * ld;
  const bf16* Qg = Bg + h * HD;
  const bf16* Og = dout + (size_t)b * T * C + h * HD;
  const int q0 = qt * ROWS, qw0 = q0 + wave * 32, myq = qw0 + (lane & 31);
  const float sl2 = scale * kLog2e;

  bf16x8 qf[4], of[4];
  frags_global(Qg, ld, myq, T, lane, qf);
  frags_global(Og, (size_t)C, myq, T, lane, of);
  float Dq, lq;
  {
    // each half-wave holds 32 of the row's 64 dO and O values
    bf16x8 o_[4];
    frags_global(out + (size_t)b * T * C + h * HD, (size_t)C, myq, T, lane, o_);
    float d = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf((float)of[s][e], (float)o_[s][e], d);
    Dq = half_sum(d);
    lq = myq < T ? lse[(size_t)bh * T + myq] * kLog2e : 0.f;
    if (myq < T && lane < 32) {
      Dv[(size_t)bh * T + myq] = -Dq;   // the dK / dV kernel starts dP's sums from -D
      lse2[(size_t)bh * T + myq] = lq;
    }
  }
  floatx16 dq[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

  const int kend = min(T, q0 + ROWS);
  const int nst = (kend + STAGE - 1) / STAGE;
  // DMA as in the forward kernel: fixed per-lane offsets, one buffer resource
  // per stage based at its first key row
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int iq = wave * 2 + q;
    const int r = 8 * iq + (lane >> 3);
    const int c = (lane & 7) ^ ((r ^ (r >> 3)) & 7);
    koff[q] = (uint32_t)((r * ld + C + h * HD + c * 8) * 2);
    voff[q] = (uint32_t)((r * ld + 2 * C + h * HD + c * 8) * 2);
  }
  auto issue = [&](int st, int slot) {
    const int row0 = st * STAGE;
    const i32x4_rsrc rst = make_rsrc4(Bg + (size_t)row0 * ld, (uint32_t)((size_t)(T - row0) * ld * 2));
    GPT2_LDS char* base = (GPT2_LDS char*)ring[slot];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int iq = wave * 2 + q;
      dma_lds16(rst, (GPT2_LDS void*)(base + iq * 1024), koff[q]);
      dma_lds16(rst, (GPT2_LDS void*)(base + TILE + iq * 1024), voff[q]);
    }
  };
  // LDS offsets of the K / V fragments (32-key slice u2, k16 step k) and of
  // the two halves of the transposed K fragments (d block dt, 16-key group j)
  uint32_t noffs[2][4], toffs[2][4][2];
#pragma unroll
  for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
    for (int k = 0; k < 4; ++k) noffs[u2][k] = opaque(frag_off(32 * u2, k, lane));
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 2; ++r) toffs[dt][j][r] = opaque(frag_tr_off(32 * dt, 16 * j, r, lane));
  // the fragments loaded to registers above have landed: the compiler's own
  // waits for them would otherwise sit in the loop and drain the DMA ring
  wait_vmcnt<0>();
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nst) issue(s, s);
  // unrolled by the ring depth: LDS addresses are fixed offsets + immediates
  for (int st0 = 0; st0 < nst; st0 += NS) {
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      const int st = st0 + sl;
      if (st >= nst) break;
      if (st + NS - 2 < nst) wait_vmcnt<(NS - 2) * 4>();
      else wait_vmcnt<0>();
      lds_barrier();
      if (st + NS - 1 < nst) issue(st + NS - 1, (sl + NS - 1) % NS);
      const GPT2_LDS char* Ks = (const GPT2_LDS char*)ring[sl];
      const GPT2_LDS char* Vs = Ks + TILE;
      const int k0 = st * STAGE;
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        const int kb = k0 + 32 * u2;
        if (kb <= qw0 + 31 && kb < T) {
          floatx16 s, dp;
#pragma unroll
          for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            s = mfma(frag_at(Ks, noffs[u2][k]), qf[k], s);
            dp = mfma(frag_at(Vs, noffs[u2][k]), of[k], dp);
          }
          // s[r]: key kb + acc_row(r), query myq; the mask only touches diagonal slices
          float p[16];
          if ((kb + 31 > qw0) || (kb + 32 > T)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kb + acc_row(r, lane);
              p[r] = (key > myq || key >= T) ? 0.f : ex2(fmaf(s[r], sl2, -lq));
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = ex2(fmaf(s[r], sl2, -lq));
          }
          bf16x8 db[2];
#pragma unroll
          for (int r = 0; r < 16; ++r) db[r >> 3][r & 7] = (bf16)(p[r] * (dp[r] - Dq));
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
              dq[dt] = mfma(frag_tr_at(Ks, toffs[dt][2 * u2 + u][0], toffs[dt][2 * u2 + u][1]), db[u], dq[dt]);
        }
      }
    }
  }
  float mx = 0.f;
  if (myq < T) mx = store_row64(dqkv + ((size_t)b * T + myq) * ld + h * HD, dq, scale, lane);
  if constexpr (AM) {   // as in the dK / dV kernel
    mx = wave_max(mx);
    if (lane == 0) amax_atomic_bf16(amax, (int)(blockIdx.y * gridDim.x + blockIdx.x) * 4 + wave, mx);
  }
}

}  // namespace

bool attention_mfma_supported(int dtype, int hd) { return dtype == BF16 && hd == HD; }

int attention_forward_mfma(int B, int T, int H, const void* qkv, void* out, float* lse, hipStream_t stream) {
  dim3 grid((unsigned)ceil_div64(T, ROWS), (unsigned)(B * H));
  mark_begin(0, stream);
  hipLaunchKernelGGL(attn_fwd_mfma_kernel, grid, dim3(256), 0, stream, T, H, (const bf16*)qkv, (bf16*)out, lse,
                     1.0f / sqrtf((float)HD));
  GPT2_LAUNCH_CHECK();
  mark_end(0, stream);
  return 0;
}

int attention_backward_mfma(int B, int T, int H, const void* qkv, const void* out, const void* dout,
                            const float* lse, float* lse2, float* D, void* dqkv, hipStream_t stream, float* amax) {
  dim3 grid((unsigned)ceil_div64(T, ROWS), (unsigned)(B * H));
  const float scale = 1.0f / sqrtf((float)HD);
  // dQ first: it also writes D and lse2 for the dK / dV kernel
  mark_begin(2, stream);
  if (amax)
    hipLaunchKernelGGL(attn_bwd_dq_mfma_kernel<true>, grid, dim3(256), 0, stream, T, H, (const bf16*)qkv,
                       (const bf16*)out, (const bf16*)dout, lse, lse2, D, (bf16*)dqkv, scale, amax);
  else
    hipLaunchKernelGGL(attn_bwd_dq_mfma_kernel<false>, grid, dim3(256), 0, stream, T, H, (const bf16*)qkv,
                       (const bf16*)out, (const bf16*)dout, lse, lse2, D, (bf16*)dqkv, scale, amax);
  GPT2_LAUNCH_CHECK();
  mark_end(2, stream);
  mark_begin(1, stream);
  hipLaunchKernelGGL(attn_bwd_dkdv_mfma_kernel, grid, dim3(256), 0, stream, T, H, (const bf16*)qkv,
                     (const bf16*)dout, lse2, D, (bf16*)dqkv, scale, amax);
  GPT2_LAUNCH_CHECK();
  mark_end(1, stream);
  return 0;
}

}  // namespace gpt2k
