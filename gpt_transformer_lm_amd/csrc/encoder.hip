// Token + position encoder, forward and backward (the encoder_forward /
// encoder_backward rows of the kernel table in "State of the Union
// [May 3, 2024]", section "Runtime, DRAM traffic, instructions").
//
// Forward:  x0[b, t, :] = wte[tok[b, t], :] + wpe[t, :]  (16-byte chunks).
// Backward: dwpe[t] = sum_b dx0[b, t];  dwte[k] += sum_{positions p, tok[p] = k} dx0[p].
// Token ids are heavily skewed (Zipf-like text statistics: the most frequent
// id can own >10% of all positions), so the scatter is done without atomics
// and in a fixed order:
//   1. sort the 64-bit keys (token << 32) | position: a bitonic network whose
//      layers up to 4096 keys run inside one workgroup's LDS and whose longer
//      compare distances are one launch per layer over the whole array (the
//      keys are distinct, so the sorted order is unique);
//   2. cut the sorted list into pieces of 64 entries; each piece sums its runs
//      of equal tokens; a run that lies wholly inside the piece is added to
//      its dwte row directly (only this piece touches that row); a run that
//      crosses a piece boundary leaves a partial row;
//   3. the piece where a boundary-crossing run starts adds its partial and the
//      continuation partials of the following pieces, in order.
// The result is deterministic (independent of scheduling).

#include "kernels.h"

namespace gpt2k {
namespace {

constexpr int kSortChunk = 4096;        // keys sorted per workgroup in LDS (32 KiB)
constexpr int kSortMax = 1 << 22;       // B*T limit of the sort (keys buffer of 32 MiB)
constexpr int kPiece = 64;

template <typename T>
__global__ void encoder_fwd_kernel(int BT, int T_, int C, const int32_t* __restrict__ tokens,
                                   const T* __restrict__ wte, const T* __restrict__ wpe, T* __restrict__ out,
                                   int Vrows) {
  const int nch = C / 8;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)BT * nch) return;
  int p = idx / nch, ch = idx % nch;
  int t = p % T_;
  int tok = tokens[p];
  tok = tok < 0 ? 0 : (tok >= Vrows ? Vrows - 1 : tok);   // memory safety only
  float a[8], b[8];
  Chunk8<T>::load(wte + (size_t)tok * C + ch * 8, a);
  if (wpe) {
    Chunk8<T>::load(wpe + (size_t)t * C + ch * 8, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] += b[e];
  }
  Chunk8<T>::store(out + (size_t)p * C + ch * 8, a);
}

// dwpe[t, c] (+)= sum_b dx0[b, t, c]
__global__ void encoder_bwd_wpe_kernel(int B, int T_, int C, const float* __restrict__ dx0,
                                       float* __restrict__ dwpe, bool accumulate) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T_ * C) return;
  float s = 0.f;
  for (int b = 0; b < B; ++b) s += dx0[(size_t)b * T_ * C + idx];
  dwpe[idx] = accumulate ? dwpe[idx] + s : s;
}

// Bitonic network over np (a power of two) keys, ascending: layer (k, j)
// compares elements i and i ^ j and orders each pair ascending when
// i & k == 0, descending otherwise.

// Layers k = 2 .. chunk of the network on one chunk of the array, built from
// the tokens (keys past n are all-ones, so they sort last).
__global__ __launch_bounds__(1024) void sort_chunks_kernel(int n, int chunk, const int32_t* __restrict__ tokens,
                                                           int Vrows, uint64_t* __restrict__ keys) {
  __shared__ uint64_t sk[kSortChunk];
  const int base = blockIdx.x * chunk;
  for (int i = threadIdx.x; i < chunk; i += 1024) {
    const int g = base + i;
    if (g < n) {
      int tok = tokens[g];
      tok = tok < 0 ? 0 : (tok >= Vrows ? Vrows - 1 : tok);   // memory safety only
      sk[i] = ((uint64_t)(uint32_t)tok << 32) | (uint32_t)g;
    } else {
      sk[i] = ~0ull;
    }
  }
  __syncthreads();
  for (int k = 2; k <= chunk; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < chunk; i += 1024) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t a = sk[i], b = sk[l];
          if ((a > b) == (((base + i) & k) == 0)) { sk[i] = b; sk[l] = a; }
        }
      }
      __syncthreads();
    }
  for (int i = threadIdx.x; i < chunk; i += 1024) keys[base + i] = sk[i];
}

// One layer (k, j) with j >= chunk over the whole array.
__global__ __launch_bounds__(256) void sort_layer_kernel(int np, int k, int j, uint64_t* __restrict__ keys) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= np) return;
  const int l = i ^ j;
  if (l > i) {
    const uint64_t a = keys[i], b = keys[l];
    if ((a > b) == ((i & k) == 0)) { keys[i] = b; keys[l] = a; }
  }
}

// Layers (k, chunk/2) .. (k, 1) of one chunk in LDS.
__global__ __launch_bounds__(1024) void sort_chunk_merge_kernel(int chunk, int k, uint64_t* __restrict__ keys) {
  __shared__ uint64_t sk[kSortChunk];
  const int base = blockIdx.x * chunk;
  for (int i = threadIdx.x; i < chunk; i += 1024) sk[i] = keys[base + i];
  __syncthreads();
  for (int j = chunk >> 1; j > 0; j >>= 1) {
    for (int i = threadIdx.x; i < chunk; i += 1024) {
      const int l = i ^ j;
      if (l > i) {
        const uint64_t a = sk[i], b = sk[l];
        if ((a > b) == (((base + i) & k) == 0)) { sk[i] = b; sk[l] = a; }
      }
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < chunk; i += 1024) keys[base + i] = sk[i];
}

__device__ __forceinline__ int key_tok(uint64_t k) { return (int)(k >> 32); }
__device__ __forceinline__ int key_pos(uint64_t k) { return (int)(uint32_t)k; }

int next_pow2(int n) {
  int np = 1;
  while (np < n) np <<= 1;
  return np;
}

// Step 2: one block per piece; threads stride over groups of VW channels
// (VW = 4: 16-byte loads and stores).
template <int VW>
struct ChanVec;
template <> struct ChanVec<1> {
  typedef float T;
  __device__ static T zero() { return 0.f; }
  __device__ static T add(T a, T b) { return a + b; }
};
template <> struct ChanVec<4> {
  typedef float4 T;
  __device__ static T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ static T add(T a, T b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
};

template <int VW>
__global__ __launch_bounds__(256) void encoder_bwd_pieces_kernel(int n, int C,
                                                                 const uint64_t* __restrict__ sorted,
                                                                 const float* __restrict__ dx0,
                                                                 float* __restrict__ dwte,
                                                                 float* __restrict__ pcont,
                                                                 float* __restrict__ pown) {
  using CV = ChanVec<VW>;
  typedef typename CV::T V;
  const int piece = blockIdx.x;
  const int start = piece * kPiece;
  const int end = min(n, start + kPiece);
  __shared__ int stok[kPiece], spos[kPiece];
  for (int e = threadIdx.x; e < end - start; e += blockDim.x) {
    const uint64_t k = sorted[start + e];
    stok[e] = key_tok(k);
    spos[e] = key_pos(k);
  }
  __syncthreads();
  const int prev_tok = start > 0 ? key_tok(sorted[start - 1]) : -1;
  const int next_tok = end < n ? key_tok(sorted[end]) : -1;
  const int len = end - start;
  for (int c = threadIdx.x * VW; c < C; c += blockDim.x * VW) {
    int rs = 0;   // run start (index within piece)
    V acc = CV::zero();
    // rows are read 8 at a time ahead of the (sequential, fixed-order) sums,
    // so eight loads per thread are in flight instead of one
    for (int e0 = 0; e0 < len; e0 += 8) {
      V v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = e0 + j < len ? *reinterpret_cast<const V*>(dx0 + (size_t)spos[e0 + j] * C + c) : CV::zero();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = e0 + j;
        if (e >= len) break;
        acc = CV::add(acc, v[j]);
        const bool last = (e == len - 1) || (stok[e + 1] != stok[e]);
        if (last) {
          const int tok = stok[e];
          const bool from_prev = (rs == 0) && (prev_tok == tok);
          const bool to_next = (e == len - 1) && (next_tok == tok);
          if (from_prev)
            *reinterpret_cast<V*>(pcont + (size_t)piece * C + c) = acc;
          else if (to_next)
            *reinterpret_cast<V*>(pown + (size_t)piece * C + c) = acc;
          else {
            V* d = reinterpret_cast<V*>(dwte + (size_t)tok * C + c);
            *d = CV::add(*d, acc);
          }
          acc = CV::zero();
          rs = e + 1;
        }
      }
    }
  }
}

// Step 3: one block per piece whose last run starts a boundary-crossing run:
// the owner partial plus the continuation partials of the following pieces,
// in piece order.
template <int VW>
__global__ __launch_bounds__(256) void encoder_bwd_spans_kernel(int n, int C, int npieces,
                                                                const uint64_t* __restrict__ sorted,
                                                                const float* __restrict__ pcont,
                                                                const float* __restrict__ pown,
                                                                float* __restrict__ dwte) {
  using CV = ChanVec<VW>;
  typedef typename CV::T V;
  const int piece = blockIdx.x;
  const int start = piece * kPiece;
  const int end = min(n, start + kPiece);
  if (end >= n) return;
  const int tok = key_tok(sorted[end - 1]);
  if (key_tok(sorted[end]) != tok) return;    // last run does not continue
  // (keys are sorted: the last run covers the whole piece exactly when the
  // first key has its token too; then, if the run began before the piece,
  // this piece holds a continuation, not the owner partial)
  if (start > 0 && key_tok(sorted[start]) == tok && key_tok(sorted[start - 1]) == tok) return;
  // the run continues through pieces piece + 1 .. qend - 1 (found in parallel:
  // the first later piece whose first key has another token)
  __shared__ int s_end;
  if (threadIdx.x == 0) s_end = npieces;
  __syncthreads();
  for (int q = piece + 1 + (int)threadIdx.x; q < npieces; q += blockDim.x)
    if (key_tok(sorted[(size_t)q * kPiece]) != tok) atomicMin(&s_end, q);
  __syncthreads();
  const int qend = s_end;
  for (int c = threadIdx.x * VW; c < C; c += blockDim.x * VW) {
    V acc = *reinterpret_cast<const V*>(pown + (size_t)piece * C + c);
#pragma unroll 4
    for (int q = piece + 1; q < qend; ++q) acc = CV::add(acc, *reinterpret_cast<const V*>(pcont + (size_t)q * C + c));
    V* d = reinterpret_cast<V*>(dwte + (size_t)tok * C + c);
    *d = CV::add(*d, acc);
  }
}

}  // namespace

int encoder_forward(int dtype, int B, int T_, int C, int vocab_rows, const int32_t* tokens, const void* wte,
                    const void* wpe, void* out, hipStream_t stream) {
  if (B < 0 || T_ < 0 || C <= 0 || C % 8 || vocab_rows <= 0 || !tokens || !wte || !out)
    return gpt2_internal_fail(1, "encoder_forward: bad arguments");
  const int BT = B * T_;
  if (BT == 0) return 0;
  int64_t total = (int64_t)BT * (C / 8);
  dim3 grid((unsigned)ceil_div64(total, 256));
  mark_begin(0, stream);
  if (dtype == BF16)
    hipLaunchKernelGGL(encoder_fwd_kernel<bf16>, grid, dim3(256), 0, stream, BT, T_, C, tokens,
                       (const bf16*)wte, (const bf16*)wpe, (bf16*)out, vocab_rows);
  else
    hipLaunchKernelGGL(encoder_fwd_kernel<float>, grid, dim3(256), 0, stream, BT, T_, C, tokens,
                       (const float*)wte, (const float*)wpe, (float*)out, vocab_rows);
  GPT2_LAUNCH_CHECK();
  mark_end(0, stream);
  return 0;
}

size_t encoder_backward_sorted_workspace_bytes(int B, int T_, int C) {
  const int np = (int)ceil_div64((int64_t)B * T_, kPiece);
  return 2 * (size_t)np * C * sizeof(float) + 256;
}

size_t encoder_sort_keys_bytes(int n) { return n > 0 ? (((size_t)next_pow2(n) * 8 + 255) / 256) * 256 : 0; }

size_t encoder_backward_workspace_bytes(int B, int T_, int C) {
  return encoder_sort_keys_bytes(B * T_) + encoder_backward_sorted_workspace_bytes(B, T_, C);
}

int encoder_sort_keys(int n, int vocab_rows, const int32_t* tokens, uint64_t* sorted, hipStream_t stream) {
  if (n < 0 || vocab_rows <= 0 || !tokens || !sorted) return gpt2_internal_fail(1, "encoder_sort_keys: bad arguments");
  if (n == 0) return 0;
  if (n > kSortMax) return gpt2_internal_fail(1, "encoder_backward: B*T=%d exceeds %d", n, kSortMax);
  const int np = next_pow2(n), chunk = np < kSortChunk ? np : kSortChunk;
  hipLaunchKernelGGL(sort_chunks_kernel, dim3((unsigned)(np / chunk)), dim3(1024), 0, stream, n, chunk, tokens,
                     vocab_rows, sorted);
  GPT2_LAUNCH_CHECK();
  for (int k = 2 * chunk; k <= np; k <<= 1) {
    for (int j = k >> 1; j >= chunk; j >>= 1) {
      hipLaunchKernelGGL(sort_layer_kernel, dim3((unsigned)ceil_div64(np, 256)), dim3(256), 0, stream, np, k, j, sorted);
      GPT2_LAUNCH_CHECK();
    }
    hipLaunchKernelGGL(sort_chunk_merge_kernel, dim3((unsigned)(np / chunk)), dim3(1024), 0, stream, chunk, k, sorted);
    GPT2_LAUNCH_CHECK();
  }
  return 0;
}

int encoder_backward_sorted(int B, int T_, int C, const uint64_t* sorted, const float* dx0, float* dwte,
                            float* dwpe, bool accumulate_wpe, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  if (B < 0 || T_ < 0 || C <= 0 || !sorted || !dx0 || !dwte)
    return gpt2_internal_fail(1, "encoder_backward: bad arguments");
  const int n = B * T_;
  if (n == 0) return 0;
  if (n > kSortMax) return gpt2_internal_fail(1, "encoder_backward: B*T=%d exceeds %d", n, kSortMax);
  if (!workspace || workspace_bytes < encoder_backward_sorted_workspace_bytes(B, T_, C))
    return gpt2_internal_fail(3, "encoder_backward: workspace too small");
  const int npieces = (int)ceil_div64(n, kPiece);
  float* pcont = (float*)workspace;
  float* pown = pcont + (size_t)npieces * C;
  if (dwpe) {
    hipLaunchKernelGGL(encoder_bwd_wpe_kernel, dim3((unsigned)ceil_div64((int64_t)T_ * C, 256)), dim3(256), 0,
                       stream, B, T_, C, dx0, dwpe, accumulate_wpe);
    GPT2_LAUNCH_CHECK();
  }
  // 16-byte channel groups where every row of dx0, dwte and the partials
  // starts 16-byte aligned
  const bool v4 = C % 4 == 0 && (((uintptr_t)dx0 | (uintptr_t)dwte | (uintptr_t)pcont) % 16) == 0;
  if (v4) {
    hipLaunchKernelGGL(encoder_bwd_pieces_kernel<4>, dim3(npieces), dim3(256), 0, stream, n, C, sorted, dx0, dwte,
                       pcont, pown);
    GPT2_LAUNCH_CHECK();
    hipLaunchKernelGGL(encoder_bwd_spans_kernel<4>, dim3(npieces), dim3(256), 0, stream, n, C, npieces, sorted, pcont,
                       pown, dwte);
  } else {
    hipLaunchKernelGGL(encoder_bwd_pieces_kernel<1>, dim3(npieces), dim3(256), 0, stream, n, C, sorted, dx0, dwte,
                       pcont, pown);
    GPT2_LAUNCH_CHECK();
    hipLaunchKernelGGL(encoder_bwd_spans_kernel<1>, dim3(npieces), dim3(256), 0, stream, n, C, npieces, sorted, pcont,
                       pown, dwte);
  }
  GPT2_LAUNCH_CHECK();
  return 0;
}

int encoder_backward(int B, int T_, int C, int vocab_rows, const int32_t* tokens, const float* dx0,
                     float* dwte, float* dwpe, bool accumulate_wpe, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  if (B < 0 || T_ < 0 || C <= 0 || vocab_rows <= 0 || !tokens || !dx0 || !dwte || !dwpe)
    return gpt2_internal_fail(1, "encoder_backward: bad arguments");
  const int n = B * T_;
  if (n == 0) return 0;
  if (!workspace || workspace_bytes < encoder_backward_workspace_bytes(B, T_, C))
    return gpt2_internal_fail(3, "encoder_backward: workspace too small");
  uint64_t* sorted = (uint64_t*)workspace;
  const size_t head = encoder_sort_keys_bytes(n);
  int rc = encoder_sort_keys(n, vocab_rows, tokens, sorted, stream);
  if (rc) return rc;
  return encoder_backward_sorted(B, T_, C, sorted, dx0, dwte, dwpe, accumulate_wpe, (char*)workspace + head,
                                 workspace_bytes - head, stream);
}

}  // namespace gpt2k
