// Causal flash attention on the bf16 matrix cores (gfx950), head dim 64.
//
// Same mathematics as the general path in attention.hip (exact causal
// softmax attention, lse saved in fp32, backward from lse and
// D_i = dO_i . O_i), organised around v_mfma_f32_32x32x16_bf16:
//
// Forward: a block owns 128 queries of one (batch, head), 32 per wave; K and
// V stream through LDS in 64-key stages (double buffered).  Each wave
// computes S^T = K Q^T per 32-key slice (K from LDS, Q fragments held in
// registers), so its accumulator holds one query per lane and 16 keys per
// lane: the running max / sum of the online softmax are per-lane scalars
// (the two half-waves holding the same query combine with one swizzle), the
// probabilities P (bf16) are already in the register layout of the B operand
// of O^T = V^T P^T, and the rescaling of O^T is a per-lane scalar multiply.
// V is stored transposed in LDS (rows of 64 keys, padded pitch) so that the
// V^T operand reads are two 8-byte loads per lane.
//
// Backward (deterministic, no atomics), two kernels:
//   dK/dV: a block owns 128 keys (32 per wave) and streams 64-query stages of
//     Q, dO (natural and transposed), lse and D through LDS; per 32-query
//     slice: S = Q K^T, dP = dO V^T (K, V fragments in registers, one key per
//     lane), P = exp(S/sqrt(d) - lse), dS = P (dP - D),
//     dV^T += dO^T P, dK^T += Q^T dS.
//   dQ: a block owns 128 queries and streams 64-key stages of K, V and K^T:
//     S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
// Work per causal tile is unbalanced, so blocks take the heaviest tiles first.

#include "kernels.h"

namespace gpt2k {
namespace {

typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int HD = 64;
constexpr int ROWS = 128;     // queries (fwd, dQ) or keys (dK/dV) per block
constexpr int STAGE = 64;     // rows streamed per LDS stage
constexpr int TP = 68;        // pitch (bf16) of transposed LDS tiles: 136 bytes
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row ^ (row >> 3)) & 7); }

__device__ __forceinline__ floatx16 mfma(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// 64 rows x 64 bf16 of a row-major global matrix (row stride ld) into a
// swizzled [row][64] LDS tile; rows >= nrows are zero.  256 threads, 2 chunks each.
struct NaturalTile {
  uint4 r[2];
  __device__ __forceinline__ void load(const bf16* G, size_t ld, int row0, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = tid / 8 + 32 * i, c = tid % 8;
      r[i] = (row0 + row < nrows) ? *reinterpret_cast<const uint4*>(G + (size_t)(row0 + row) * ld + c * 8)
                                  : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16* S, int tid) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = tid / 8 + 32 * i, c = tid % 8;
      *reinterpret_cast<uint4*>(S + row * HD + swz(row, c) * 8) = r[i];
    }
  }
};

// The same 64 x 64 block stored transposed: S[d * TP + row].  Each of the 256
// threads moves 2 rows x 8 columns (two 16-byte loads, eight 4-byte stores;
// consecutive lanes write consecutive words of a row).
struct TransposedTile {
  uint4 r[2];
  __device__ __forceinline__ void load(const bf16* G, size_t ld, int row0, int nrows, int tid) {
    const int dc = tid / 32, rp = tid % 32;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = row0 + rp * 2 + i;
      r[i] = (row < nrows) ? *reinterpret_cast<const uint4*>(G + (size_t)row * ld + dc * 8)
                           : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16* S, int tid) const {
    const int dc = tid / 32, rp = tid % 32;
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t v = (e % 2 == 0) ? ((w0[e / 2] & 0xffffu) | (w1[e / 2] << 16))
                                      : ((w0[e / 2] >> 16) | (w1[e / 2] & 0xffff0000u));
      *reinterpret_cast<uint32_t*>(S + (dc * 8 + e) * TP + rp * 2) = v;
    }
  }
};

// A-operand fragment of a natural [row][64] tile: row (lane % 32) of the
// 32-row slice at `row0`, k16 step s.
__device__ __forceinline__ bf16x8 frag_natural(const bf16* S, int row0, int s, int lane) {
  const int row = row0 + (lane & 31);
  return *reinterpret_cast<const bf16x8*>(S + row * HD + swz(row, 2 * s + (lane >> 5)) * 8);
}

// A-operand fragment of a transposed tile: row d = d0 + lane % 32, columns
// {c0 + 4*hi + 0..3, c0 + 8 + 4*hi + 0..3} (the key/query order that the
// 32x32 accumulator uses for its registers 8u..8u+7).
__device__ __forceinline__ bf16x8 frag_transposed(const bf16* S, int d0, int c0, int lane) {
  const bf16* p = S + (d0 + (lane & 31)) * TP + c0 + 4 * (lane >> 5);
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 8);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
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
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Writes 64 values of row `row` held as two 32 x 32 accumulators (d on registers).
__device__ __forceinline__ void store_row64(bf16* dst, const floatx16 acc[2], float mul, int lane) {
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (bf16)(acc[dt][4 * g + e] * mul);
      *reinterpret_cast<bf16x4*>(dst + dt * 32 + 8 * g + 4 * (lane >> 5)) = v;
    }
}

// ------------------------------------------------------------------ forward

__global__ __launch_bounds__(256, 2) void attn_fwd_mfma_kernel(int T, int H, const bf16* __restrict__ qkv,
                                                            bf16* __restrict__ out, float* __restrict__ lse,
                                                            float scale) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][STAGE * HD];
  __shared__ __attribute__((aligned(16))) bf16 Vt[2][HD * TP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5;
  const int nqt = (T + ROWS - 1) / ROWS;
  const int qt = nqt - 1 - (int)blockIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int C = H * HD;
  const size_t ld = 3 * (size_t)C;
  const bf16* Qg = qkv + (size_t)b * T * ld + h * HD;
  const bf16* Kg = Qg + C;
  const bf16* Vg = Qg + 2 * C;
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
  NaturalTile kt;
  TransposedTile vt;
  kt.load(Kg, ld, 0, T, tid);
  vt.load(Vg, ld, 0, T, tid);
  kt.store(Ks[0], tid);
  vt.store(Vt[0], tid);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int k0 = st * STAGE;
    const bool more = st + 1 < nst;
    if (more) {
      kt.load(Kg, ld, k0 + STAGE, T, tid);
      vt.load(Vg, ld, k0 + STAGE, T, tid);
    }
    const bf16* Kc = Ks[st & 1];
    const bf16* Vc = Vt[st & 1];
#pragma unroll
    for (int ks = 0; ks < STAGE; ks += 32) {
      const int kb = k0 + ks;
      if (kb <= qw0 + 31 && kb < T) {
        floatx16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) s = mfma(frag_natural(Kc, ks, k, lane), qf[k], s);
        const bool edge = (kb + 31 > qw0) || (kb + 32 > T);
        float t[16];
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          t[r] = s[r] * sl2;
          if (edge) {
            const int key = kb + acc_row(r, lane);
            if (key > myq || key >= T) t[r] = -INFINITY;
          }
          mx = fmaxf(mx, t[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_i, mx);
        const float alpha = ex2(m_i - m_new);
        float rs = 0.f;
        bf16x8 pb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = ex2(t[r] - m_new);
          rs += p;
          pb[r >> 3][r & 7] = (bf16)p;
        }
        rs += __shfl_xor(rs, 32, 64);
        l_i = l_i * alpha + rs;
        m_i = m_new;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) oacc[dt] = mfma(frag_transposed(Vc, dt * 32, ks + 16 * u, lane), pb[u], oacc[dt]);
      }
    }
    if (more) {
      kt.store(Ks[(st + 1) & 1], tid);
      vt.store(Vt[(st + 1) & 1], tid);
    }
    __syncthreads();
  }
  if (myq < T) {
    store_row64(out + ((size_t)b * T + myq) * C + h * HD, oacc, 1.0f / l_i, lane);
    if (hi == 0) lse[(size_t)bh * T + myq] = (m_i + __log2f(l_i)) * kLn2;
  }
}

// ------------------------------------------------------------------ backward dK, dV

__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_mfma_kernel(int T, int H, const bf16* __restrict__ qkv,
                                                                 const bf16* __restrict__ dout,
                                                                 const float* __restrict__ lse,
                                                                 const float* __restrict__ Dv,
                                                                 bf16* __restrict__ dqkv, float scale) {
  __shared__ __attribute__((aligned(16))) bf16 Qn[2][STAGE * HD];
  __shared__ __attribute__((aligned(16))) bf16 Qt[2][HD * TP];
  __shared__ __attribute__((aligned(16))) bf16 On[2][STAGE * HD];
  __shared__ __attribute__((aligned(16))) bf16 Ot[2][HD * TP];
  __shared__ float Ls[2][STAGE], Ds[2][STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nkt = (T + ROWS - 1) / ROWS;
  const int ktile = (int)blockIdx.x;           // lower key tiles see more queries: launch them first
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int C = H * HD;
  const size_t ld = 3 * (size_t)C;
  const bf16* Qg = qkv + (size_t)b * T * ld + h * HD;
  const bf16* Kg = Qg + C;
  const bf16* Vg = Qg + 2 * C;
  const bf16* Og = dout + (size_t)b * T * C + h * HD;
  const float* lseg = lse + (size_t)bh * T;
  const float* Dg = Dv + (size_t)bh * T;
  const int k0 = ktile * ROWS, kw0 = k0 + wave * 32, mykey = kw0 + (lane & 31);
  const float sl2 = scale * kLog2e;
  (void)nkt;

  bf16x8 kf[4], vf[4];
  frags_global(Kg, ld, mykey, T, lane, kf);
  frags_global(Vg, ld, mykey, T, lane, vf);
  floatx16 dk[2], dv[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[dt][r] = 0.f; dv[dt][r] = 0.f; }

  const int qbeg = k0;                          // queries before the tile see none of its keys
  const int nst = (T - qbeg + STAGE - 1) / STAGE;
  NaturalTile qn, on;
  TransposedTile qtt, ott;
  auto load_stage = [&](int q0) {
    qn.load(Qg, ld, q0, T, tid);
    on.load(Og, (size_t)C, q0, T, tid);
    qtt.load(Qg, ld, q0, T, tid);
    ott.load(Og, (size_t)C, q0, T, tid);
  };
  auto store_stage = [&](int buf, int q0) {
    qn.store(Qn[buf], tid);
    on.store(On[buf], tid);
    qtt.store(Qt[buf], tid);
    ott.store(Ot[buf], tid);
    if (tid < STAGE) {
      const int q = q0 + tid;
      Ls[buf][tid] = q < T ? lseg[q] * kLog2e : 0.f;
      Ds[buf][tid] = q < T ? Dg[q] : 0.f;
    }
  };
  if (nst > 0) {
    load_stage(qbeg);
    store_stage(0, qbeg);
  }
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int q0 = qbeg + st * STAGE;
    const bool more = st + 1 < nst;
    if (more) load_stage(q0 + STAGE);
    const int buf = st & 1;
#pragma unroll
    for (int qs = 0; qs < STAGE; qs += 32) {
      const int qb = q0 + qs;
      if (qb + 31 >= kw0 && qb < T && kw0 < T) {
        floatx16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          s = mfma(frag_natural(Qn[buf], qs, k, lane), kf[k], s);
          dp = mfma(frag_natural(On[buf], qs, k, lane), vf[k], dp);
        }
        // s[r]: query qb + acc_row(r), key mykey
        const bool edge = (qb < kw0 + 31) || (qb + 32 > T);
        bf16x8 pb[2], db[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qs + acc_row(r, lane);
          float p = ex2(s[r] * sl2 - Ls[buf][ql]);
          if (edge && (mykey > qb + acc_row(r, lane) || qb + acc_row(r, lane) >= T)) p = 0.f;
          const float ds = p * (dp[r] - Ds[buf][ql]);
          pb[r >> 3][r & 7] = (bf16)p;
          db[r >> 3][r & 7] = (bf16)ds;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) {
            dv[dt] = mfma(frag_transposed(Ot[buf], dt * 32, qs + 16 * u, lane), pb[u], dv[dt]);
            dk[dt] = mfma(frag_transposed(Qt[buf], dt * 32, qs + 16 * u, lane), db[u], dk[dt]);
          }
      }
    }
    if (more) store_stage(buf ^ 1, q0 + STAGE);
    __syncthreads();
  }
  if (mykey < T) {
    bf16* dst = dqkv + ((size_t)b * T + mykey) * ld + h * HD;
    store_row64(dst + C, dk, scale, lane);
    store_row64(dst + 2 * C, dv, 1.0f, lane);
  }
}

// ------------------------------------------------------------------ backward dQ

__global__ __launch_bounds__(256, 2) void attn_bwd_dq_mfma_kernel(int T, int H, const bf16* __restrict__ qkv,
                                                               const bf16* __restrict__ dout,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ Dv,
                                                               bf16* __restrict__ dqkv, float scale) {
  __shared__ __attribute__((aligned(16))) bf16 Kn[2][STAGE * HD];
  __shared__ __attribute__((aligned(16))) bf16 Vn[2][STAGE * HD];
  __shared__ __attribute__((aligned(16))) bf16 Kt[2][HD * TP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nqt = (T + ROWS - 1) / ROWS;
  const int qt = nqt - 1 - (int)blockIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int C = H * HD;
  const size_t ld = 3 * (size_t)C;
  const bf16* Qg = qkv + (size_t)b * T * ld + h * HD;
  const bf16* Kg = Qg + C;
  const bf16* Vg = Qg + 2 * C;
  const bf16* Og = dout + (size_t)b * T * C + h * HD;
  const int q0 = qt * ROWS, qw0 = q0 + wave * 32, myq = qw0 + (lane & 31);
  const float sl2 = scale * kLog2e;

  bf16x8 qf[4], of[4];
  frags_global(Qg, ld, myq, T, lane, qf);
  frags_global(Og, (size_t)C, myq, T, lane, of);
  const float lse2 = myq < T ? lse[(size_t)bh * T + myq] * kLog2e : 0.f;
  const float Dq = myq < T ? Dv[(size_t)bh * T + myq] : 0.f;
  floatx16 dq[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

  const int kend = min(T, q0 + ROWS);
  const int nst = (kend + STAGE - 1) / STAGE;
  NaturalTile kn, vn;
  TransposedTile ktt;
  kn.load(Kg, ld, 0, T, tid);
  vn.load(Vg, ld, 0, T, tid);
  ktt.load(Kg, ld, 0, T, tid);
  kn.store(Kn[0], tid);
  vn.store(Vn[0], tid);
  ktt.store(Kt[0], tid);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int k0 = st * STAGE;
    const bool more = st + 1 < nst;
    if (more) {
      kn.load(Kg, ld, k0 + STAGE, T, tid);
      vn.load(Vg, ld, k0 + STAGE, T, tid);
      ktt.load(Kg, ld, k0 + STAGE, T, tid);
    }
    const int buf = st & 1;
#pragma unroll
    for (int ks = 0; ks < STAGE; ks += 32) {
      const int kb = k0 + ks;
      if (kb <= qw0 + 31 && kb < T) {
        floatx16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          s = mfma(frag_natural(Kn[buf], ks, k, lane), qf[k], s);
          dp = mfma(frag_natural(Vn[buf], ks, k, lane), of[k], dp);
        }
        // s[r]: key kb + acc_row(r), query myq
        const bool edge = (kb + 31 > qw0) || (kb + 32 > T);
        bf16x8 db[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = ex2(s[r] * sl2 - lse2);
          const int key = kb + acc_row(r, lane);
          if (edge && (key > myq || key >= T)) p = 0.f;
          db[r >> 3][r & 7] = (bf16)(p * (dp[r] - Dq));
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) dq[dt] = mfma(frag_transposed(Kt[buf], dt * 32, ks + 16 * u, lane), db[u], dq[dt]);
      }
    }
    if (more) {
      kn.store(Kn[buf ^ 1], tid);
      vn.store(Vn[buf ^ 1], tid);
      ktt.store(Kt[buf ^ 1], tid);
    }
    __syncthreads();
  }
  if (myq < T) store_row64(dqkv + ((size_t)b * T + myq) * ld + h * HD, dq, scale, lane);
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

int attention_backward_mfma(int B, int T, int H, const void* qkv, const void* dout, const float* lse,
                            const float* D, void* dqkv, hipStream_t stream) {
  dim3 grid((unsigned)ceil_div64(T, ROWS), (unsigned)(B * H));
  const float scale = 1.0f / sqrtf((float)HD);
  mark_begin(1, stream);
  hipLaunchKernelGGL(attn_bwd_dkdv_mfma_kernel, grid, dim3(256), 0, stream, T, H, (const bf16*)qkv,
                     (const bf16*)dout, lse, D, (bf16*)dqkv, scale);
  GPT2_LAUNCH_CHECK();
  mark_end(1, stream);
  mark_begin(2, stream);
  hipLaunchKernelGGL(attn_bwd_dq_mfma_kernel, grid, dim3(256), 0, stream, T, H, (const bf16*)qkv,
                     (const bf16*)dout, lse, D, (bf16*)dqkv, scale);
  GPT2_LAUNCH_CHECK();
  mark_end(2, stream);
  return 0;
}

}  // namespace gpt2k
