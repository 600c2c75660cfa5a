// Host runtime of the GPT-2 step library: configuration checks, the one-arena
// memory plan, parameter table, seeded initialisation, orchestration of the
// forward / backward / AdamW kernels on one HIP stream, state access, timing
// hooks, and the C ABI of gpt2.h and gpt2_ops.h.
//
// The step follows the pre-LayerNorm GPT-2 block of the pages' kernel table
// ("State of the Union [May 3, 2024]", section "Runtime, DRAM traffic,
// instructions"): encoder -> L x [LN1 -> QKV -> attention -> projection +
// residual -> LN2 -> fc + GELU -> fc-projection + residual] -> LNf -> tied
// logits -> fused softmax cross-entropy, then the reverse pass and AdamW.
// Memory: one arena holds parameters (fp32 master, bf16 copy), gradients,
// AdamW moments, every saved activation and one scratch region shared by the
// backward kernels (they run in order on one stream).  The opening bullet list
// of that page notes the memory saved by not keeping per-layer backward
// gradient buffers; likewise here the activation gradients live in four
// buffers reused by every layer.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <exception>
#include <new>
#include <stdexcept>
#include <vector>

#include "../../include/gpt2.h"
#include "../../include/gpt2_ops.h"
#include "kernels.h"

using namespace gpt2k;

// ---------------------------------------------------------------- errors

static thread_local char g_last_error[1024] = "";

namespace gpt2k {
KernelMark* kernel_marks() {
  static thread_local KernelMark marks[kMaxMarks] = {};
  return marks;
}
}  // namespace gpt2k

int gpt2_internal_fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int gpt2_internal_hip_fail(hipError_t e, const char* expr, const char* file, int line) {
  snprintf(g_last_error, sizeof(g_last_error), "%s failed: %s (%s:%d)", expr, hipGetErrorString(e), file, line);
  return GPT2_E_HIP;
}

#define RC(x)                \
  do {                       \
    int _rc = (x);           \
    if (_rc) return _rc;     \
  } while (0)

// No C++ exception crosses the C ABI: every extern "C" body runs inside
// GPT2_ABI_BEGIN / GPT2_ABI_END_STATUS (status-returning calls: the
// exception becomes GPT2_E_OOM for a failed host allocation, GPT2_E_INTERNAL
// otherwise, with its text in gpt2_last_error()) or GPT2_ABI_END(value)
// (other return types: the same text, and `value` is returned).
#define GPT2_ABI_BEGIN try {
#define GPT2_ABI_END_STATUS                                                                 \
  }                                                                                        \
  catch (const std::bad_alloc&) {                                                          \
    return gpt2_internal_fail(GPT2_E_OOM, "host allocation failed");                       \
  }                                                                                        \
  catch (const std::length_error&) {                                                       \
    return gpt2_internal_fail(GPT2_E_OOM, "host allocation failed (size out of range)");   \
  }                                                                                        \
  catch (const std::exception& ex) {                                                       \
    return gpt2_internal_fail(GPT2_E_INTERNAL, "unexpected C++ exception: %s", ex.what()); \
  }                                                                                        \
  catch (...) {                                                                            \
    return gpt2_internal_fail(GPT2_E_INTERNAL, "unexpected C++ exception");                \
  }
#define GPT2_ABI_END(fail_value)                                                           \
  }                                                                                        \
  catch (const std::bad_alloc&) {                                                          \
    gpt2_internal_fail(GPT2_E_OOM, "host allocation failed");                              \
    return fail_value;                                                                     \
  }                                                                                        \
  catch (const std::length_error&) {                                                       \
    gpt2_internal_fail(GPT2_E_OOM, "host allocation failed (size out of range)");          \
    return fail_value;                                                                     \
  }                                                                                        \
  catch (const std::exception& ex) {                                                       \
    gpt2_internal_fail(GPT2_E_INTERNAL, "unexpected C++ exception: %s", ex.what());        \
    return fail_value;                                                                     \
  }                                                                                        \
  catch (...) {                                                                            \
    gpt2_internal_fail(GPT2_E_INTERNAL, "unexpected C++ exception");                       \
    return fail_value;                                                                     \
  }

namespace {

// Host allocations of the library's own bookkeeping (arena plan, timing
// events) go through grow(), which fails the next g_fail_allocs of them on
// request (gpt2_test_fail_host_allocations) so the error paths can be tested.
std::atomic<int> g_fail_allocs{0};

template <typename V>
void grow(V& v, size_t n) {
  int k = g_fail_allocs.load();
  while (k > 0 && !g_fail_allocs.compare_exchange_weak(k, k - 1)) {
  }
  if (k > 0) throw std::bad_alloc();
  v.resize(n);
}

}  // namespace

// ---------------------------------------------------------------- config

namespace {

// Weight matrices the dX GEMMs read transposed (token table, then per layer
// W_qkv, W_o, W_fc, W_p); bf16 mode keeps a transposed copy of each so that
// both operands of dX = dY W are k-major.
const int kTransposed[5] = {0, 4, 6, 10, 12};

const char* kParamNames[16] = {"wte",  "wpe",      "ln1w",     "ln1b", "qkvw", "qkvb",    "attprojw", "attprojb",
                               "ln2w", "ln2b",     "fcw",      "fcb",  "fcprojw", "fcprojb", "lnfw", "lnfb"};

struct ParamTable {
  int64_t off[16];
  int64_t shape[16][3];
  int ndim[16];
  int64_t total;
};

void param_table(const gpt2_config& c, bool padded, ParamTable* t) {
  const int64_t V = padded ? c.padded_vocab_size : c.vocab_size;
  const int64_t T = c.max_seq_len, L = c.num_layers, C = c.channels;
  const int64_t sh[16][3] = {{V, C, 1},     {T, C, 1},     {L, C, 1},     {L, C, 1},
                             {L, 3 * C, C}, {L, 3 * C, 1}, {L, C, C},     {L, C, 1},
                             {L, C, 1},     {L, C, 1},     {L, 4 * C, C}, {L, 4 * C, 1},
                             {L, C, 4 * C}, {L, C, 1},     {C, 1, 1},     {C, 1, 1}};
  const int nd[16] = {2, 2, 2, 2, 3, 2, 3, 2, 2, 2, 3, 2, 3, 2, 1, 1};
  int64_t o = 0;
  for (int i = 0; i < 16; ++i) {
    t->off[i] = o;
    t->ndim[i] = nd[i];
    for (int d = 0; d < 3; ++d) t->shape[i][d] = sh[i][d];
    o += sh[i][0] * sh[i][1] * sh[i][2];
  }
  t->total = o;
}

// Storage of parameters copies, activations and activation gradients: bf16
// in the two mixed-precision modes, fp32 in the parity mode.
bool is_bf16(const gpt2_config& c) { return c.dtype != GPT2_FP32; }

int validate(const gpt2_config* c) {
  if (!c) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "config is NULL");
  if (c->dtype != GPT2_FP32 && c->dtype != GPT2_BF16 && c->dtype != GPT2_BF16_FP8)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "dtype %d is not GPT2_FP32, GPT2_BF16 or GPT2_BF16_FP8", c->dtype);
  if (c->vocab_size <= 0 || c->vocab_size > 65536)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "vocab_size %d outside (0, 65536]", c->vocab_size);
  if (c->padded_vocab_size < c->vocab_size || c->padded_vocab_size % 64 || c->padded_vocab_size > 65536)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "padded_vocab_size %d must be >= vocab_size, <= 65536 and a multiple of 64",
                              c->padded_vocab_size);
  if (c->num_layers < 0 || c->num_layers > 1024)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "num_layers %d", c->num_layers);
  if (c->channels <= 0 || c->channels % 64 || c->channels > 4096)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "channels %d must be a positive multiple of 64, <= 4096", c->channels);
  if (c->num_heads <= 0 || c->channels % c->num_heads)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "num_heads %d must divide channels %d", c->num_heads, c->channels);
  const int hd = c->channels / c->num_heads;
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "head dim %d unsupported (16, 32, 64, 128)", hd);
  if (c->max_seq_len <= 0 || c->seq_len <= 0 || c->seq_len > c->max_seq_len)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "seq_len %d / max_seq_len %d", c->seq_len, c->max_seq_len);
  if (c->batch_size <= 0) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "batch_size %d", c->batch_size);
  const int64_t BT = (int64_t)c->batch_size * c->seq_len;
  if (BT % 64 || BT > (1 << 22))
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "batch_size*seq_len = %lld must be a multiple of 64 and <= 4194304",
                              (long long)BT);
  // the classifier products address the bf16 logits with 32-bit offsets
  if (c->dtype != GPT2_FP32 && BT * c->padded_vocab_size * 2 >= (int64_t)0xFFFFFFF0)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG,
                              "batch_size*seq_len*padded_vocab_size*2 = %lld bytes of logits reach 4 GiB",
                              (long long)(BT * c->padded_vocab_size * 2));
  if (c->arch_flags & ~(GPT2_ARCH_RELU2 | GPT2_ARCH_QK_NORM | GPT2_ARCH_ROPE))
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "arch_flags 0x%x has unknown bits", (unsigned)c->arch_flags);
  return GPT2_OK;
}

// ---------------------------------------------------------------- arena plan

struct Plan {
  size_t total = 0;
  size_t alloc(size_t bytes) {
    size_t o = total;
    total += (bytes + 255) / 256 * 256;
    return o;
  }
};

struct LayerOffsets {
  size_t ln1, ln1_mean, ln1_rstd, qkv, atty, lse, h, ln2, ln2_mean, ln2_rstd;
  size_t u;   // activation derivative at the fc pre-activation (GELU' or 2 relu), for the backward
  size_t g;   // activation of the fc pre-activation (GELU or relu^2)
  size_t qk_rstd;   // QK-Norm: 1 / rms of every q and k head vector [BT, 2H] fp32 (0 if unused)
  // fp8 mode: codes of the fp8 products' inputs, row-major (q) and transposed (qt)
  size_t ln1_q, ln2_q, g_q;
};

// fp8 mode: the weight tensors of the fp8 products (token table, W_qkv, W_fc,
// W_p) and the slots of their per-tensor scales.
const int kFp8Weights[4] = {0, 4, 10, 12};
enum Fp8Kind { Q_WEIGHT = 0, Q_ACT = 1, Q_GRAD = 2 };
// Scale slot: weights (token table; then W_qkv, W_fc, W_p of each layer),
// activations (ln1, ln2, g of each layer; lnf), gradients (dlogits; the
// fc-proj, fc and QKV output gradients of each layer).
int fp8_slot(int L, int kind, int which, int l) {
  if (kind == Q_WEIGHT) return which == 0 ? 0 : 1 + (which - 1) * L + l;
  if (kind == Q_ACT) return which == 3 ? 1 + 6 * L : 1 + 3 * L + 3 * l + which;
  return which == 3 ? 2 + 6 * L : 3 + 6 * L + 3 * l + which;
}
int fp8_slots(int L) { return 3 + 9 * L; }

struct Layout {
  ParamTable pt;
  int64_t P;
  size_t master, grad, adam_m, adam_v, params_bf16;
  size_t params_t[16];                   // bf16 transposed copies of the weight matrices (0 if none)
  std::vector<size_t> resid;             // L + 1 buffers [BT, C]
  std::vector<LayerOffsets> layer;
  size_t tokens, lnf, lnf_mean, lnf_rstd, logits, losses, mean_loss;
  size_t gnorm;                          // gradient norm, clipping factor, per-block partial sums
  size_t adam_hp;                        // AdamW hyperparameters read by the update kernel
  size_t dres, dres_t, d_ln, d_big, d_qkv, scratch;
  size_t sorted_keys;                    // encoder-backward key sort (computed during the forward)
  size_t rope_cs;                        // rotary embedding cos / sin table [maxT][hd/2] (0 if unused)
  // fp8 mode (0 otherwise): weight codes per parameter tensor (row-major and
  // transposed, all layers), lnf codes, the current output gradient's codes
  // (row-major only: the weight-gradient products read activation and
  // gradient codes m-major),
  // per-tensor scales, absmax partials, the maxima producer kernels leave
  // (kAmaxWays slots, kAmaxStride floats apart, per scale slot)
  size_t wq[16], wqt[16], lnf_q, dq, fp8_scales, fp8_amax, fp8_colsum, fp8_slot_max;
  size_t scratch_bytes;
  size_t total;
};

size_t scratch_need(const gpt2_config& c) {
  const int dt = is_bf16(c) ? GPT2_BF16 : GPT2_FP32;
  const int BT = c.batch_size * c.seq_len, C = c.channels, Vp = c.padded_vocab_size;
  size_t s = 0;
  auto upd = [&](size_t x) { s = std::max(s, x); };
  upd(gemm_workspace_bytes(dt, EPI_WGRAD, Vp, C, BT, false, false));
  upd(gemm_workspace_bytes(dt, EPI_WGRAD, C, 4 * C, BT, false, false));
  upd(gemm_workspace_bytes(dt, EPI_WGRAD, 4 * C, C, BT, false, false));
  upd(gemm_workspace_bytes(dt, EPI_WGRAD, C, C, BT, false, false));
  upd(gemm_workspace_bytes(dt, EPI_WGRAD, 3 * C, C, BT, false, false));
  // dX GEMMs (plain store; long-K ones are split)
  const bool wt = dt == GPT2_BF16;   // bf16 dX reads transposed (k-major) weights
  upd(gemm_workspace_bytes(dt, EPI_STORE, BT, C, Vp, true, wt));
  upd(gemm_workspace_bytes(dt, EPI_STORE, BT, C, 4 * C, true, wt));
  upd(gemm_workspace_bytes(dt, EPI_STORE, BT, C, 3 * C, true, wt));
  upd(gemm_workspace_bytes(dt, EPI_STORE, BT, C, C, true, wt));
  upd(layernorm_backward_workspace_bytes(BT, C));
  if (c.dtype == GPT2_BF16_FP8) {   // fp8 weight gradients (split-K partials) and dX, bias gradients
    const int fp8_n[4][2] = {{Vp, C}, {3 * C, C}, {4 * C, C}, {C, 4 * C}};
    for (auto& nk : fp8_n) {
      upd(gemm_workspace_bytes(GPT2_BF16, EPI_WGRAD, nk[0], nk[1], BT, true, true, 2));
      upd(gemm_workspace_bytes(GPT2_BF16, EPI_STORE, BT, nk[1], nk[0], true, true, 2));
    }
  }
  upd(attention_backward_workspace_bytes(c.batch_size, c.seq_len, c.num_heads, C / c.num_heads));
  upd(encoder_backward_workspace_bytes(c.batch_size, c.seq_len, C));
  return s;
}

void make_layout(const gpt2_config& c, Layout* lo) {
  param_table(c, true, &lo->pt);
  lo->P = lo->pt.total;
  const size_t es = is_bf16(c) ? 2 : 4;
  const size_t BT = (size_t)c.batch_size * c.seq_len, C = c.channels, L = c.num_layers;
  const size_t BHT = (size_t)c.batch_size * c.num_heads * c.seq_len;
  Plan p;
  lo->master = p.alloc(lo->P * 4);
  lo->grad = p.alloc(lo->P * 4);
  lo->adam_m = p.alloc(lo->P * 4);
  lo->adam_v = p.alloc(lo->P * 4);
  lo->params_bf16 = is_bf16(c) ? p.alloc(lo->P * 2) : 0;
  for (int i = 0; i < 16; ++i) lo->params_t[i] = 0;
  if (is_bf16(c))
    for (int i : kTransposed) {
      if (c.dtype == GPT2_BF16_FP8 && i != 6) continue;   // the fp8 weights keep fp8 transposed codes instead
      const int64_t* sh = lo->pt.shape[i];
      lo->params_t[i] = p.alloc((size_t)sh[0] * sh[1] * sh[2] * 2);
    }
  lo->tokens = p.alloc(BT * 4);
  grow(lo->resid, L + 1);
  for (size_t l = 0; l <= L; ++l) lo->resid[l] = p.alloc(BT * C * es);
  grow(lo->layer, L);
  for (size_t l = 0; l < L; ++l) {
    LayerOffsets& o = lo->layer[l];
    o.ln1 = p.alloc(BT * C * es);
    o.ln1_mean = p.alloc(BT * 4);
    o.ln1_rstd = p.alloc(BT * 4);
    o.qkv = p.alloc(BT * 3 * C * es);
    o.atty = p.alloc(BT * C * es);
    o.lse = p.alloc(BHT * 4);
    o.h = p.alloc(BT * C * es);
    o.ln2 = p.alloc(BT * C * es);
    o.ln2_mean = p.alloc(BT * 4);
    o.ln2_rstd = p.alloc(BT * 4);
    o.u = p.alloc(BT * 4 * C * es);
    o.g = p.alloc(BT * 4 * C * es);
    o.qk_rstd = (c.arch_flags & GPT2_ARCH_QK_NORM) ? p.alloc((size_t)BT * 2 * c.num_heads * 4) : 0;
    const bool f8 = c.dtype == GPT2_BF16_FP8;
    o.ln1_q = f8 ? p.alloc(BT * C) : 0;
    o.ln2_q = f8 ? p.alloc(BT * C) : 0;
    o.g_q = f8 ? p.alloc(BT * 4 * C) : 0;
  }
  lo->lnf = p.alloc(BT * C * es);
  lo->lnf_mean = p.alloc(BT * 4);
  lo->lnf_rstd = p.alloc(BT * 4);
  lo->logits = p.alloc(BT * (size_t)c.padded_vocab_size * es);
  lo->losses = p.alloc(BT * 4);
  lo->mean_loss = p.alloc(4);
  lo->gnorm = p.alloc(grad_norm_workspace_bytes());
  lo->adam_hp = p.alloc(sizeof(AdamHP));
  lo->dres = p.alloc(BT * C * 4);
  lo->dres_t = is_bf16(c) ? p.alloc(BT * C * es) : lo->dres;
  lo->d_ln = p.alloc(BT * C * es);
  lo->d_big = p.alloc(BT * 4 * C * es);
  lo->d_qkv = p.alloc(BT * 3 * C * es);
  lo->sorted_keys = p.alloc(encoder_sort_keys_bytes((int)BT));
  lo->rope_cs = (c.arch_flags & GPT2_ARCH_ROPE)
                    ? p.alloc((size_t)c.max_seq_len * (c.channels / c.num_heads / 2) * sizeof(float2))
                    : 0;
  for (int i = 0; i < 16; ++i) lo->wq[i] = lo->wqt[i] = 0;
  lo->lnf_q = lo->dq = lo->fp8_scales = lo->fp8_amax = lo->fp8_colsum = lo->fp8_slot_max = 0;
  if (c.dtype == GPT2_BF16_FP8) {
    for (int i : kFp8Weights) {
      const int64_t* sh = lo->pt.shape[i];
      lo->wq[i] = p.alloc((size_t)sh[0] * sh[1] * sh[2]);
      lo->wqt[i] = p.alloc((size_t)sh[0] * sh[1] * sh[2]);
    }
    lo->lnf_q = p.alloc(BT * C);
    const size_t big = BT * std::max<size_t>((size_t)c.padded_vocab_size, 4 * C);   // the largest output gradient
    lo->dq = p.alloc(big);
    lo->fp8_scales = p.alloc((size_t)fp8_slots((int)L) * sizeof(Fp8Scale));
    lo->fp8_amax = p.alloc(fp8_scale_workspace_bytes());
    lo->fp8_colsum = p.alloc(fp8_colsum_bytes((int)BT, 4 * C));
    lo->fp8_slot_max = p.alloc((size_t)fp8_slots((int)L) * kAmaxWays * kAmaxStride * sizeof(float));
  }
  lo->scratch_bytes = scratch_need(c);
  lo->scratch = p.alloc(lo->scratch_bytes);
  lo->total = p.total;
}

// ---------------------------------------------------------------- timing sites

// Each site times one kernel: the main kernel of the launcher called there.
enum Site {
  S_QKV = 0, S_ATTPROJ, S_FC, S_FCPROJ, S_LOGITS, S_FCPROJ_DX, S_FCPROJ_DW, S_FC_DX, S_FC_DW,
  S_ATTPROJ_DX, S_ATTPROJ_DW, S_QKV_DX, S_QKV_DW, S_CLS_DX, S_CLS_DW, S_ATTN_FWD, S_ATTN_DKDV, S_ATTN_DQ,
  S_ATTN_DOT, S_XENT, S_LN_FWD, S_LN_BWD, S_ENC_FWD, S_ADAMW, S_WT, S_GRAD_NORM, S_QK_FWD, S_QK_BWD, S_FP8_QUANT,
  S_COUNT
};

struct SiteTimer {
  bool on = false;
  std::vector<hipEvent_t> ev;   // pairs
  size_t used = 0;              // events used (2 per launch)
  int64_t launches = 0;
  double flops = 0, bytes = 0;  // per launch
};

}  // namespace

struct gpt2_model {
  gpt2_config cfg;
  Layout lo;
  hipStream_t stream;
  // Side stream for work that depends only on the token ids (the encoder
  // backward's key sort): forked after the ids are copied, joined before the
  // encoder backward and before the ids are overwritten by the next forward.
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  bool side_pending = false;
  char* base;
  bool owns;
  bool have_dlogits = false;
  bool have_grads = false;
  int device = 0;
  SiteTimer timers[S_COUNT];
  // Planning mode (gpt2_step_gemm_plans): no device memory and nothing is
  // enqueued; the forward and backward sequences only record each GEMM they
  // would launch, with its timing site.
  std::vector<std::pair<int, GemmDesc>>* plan_log = nullptr;
  bool dry() const { return plan_log != nullptr; }
  // A captured training step (gpt2_graph_capture) and its executable form.
  hipGraph_t graph = nullptr;
  hipGraphExec_t graph_exec = nullptr;

  template <typename P> P* at(size_t off) { return reinterpret_cast<P*>(base + off); }
  float* master() { return at<float>(lo.master); }
  float* grad() { return at<float>(lo.grad); }
  // parameter tensor i as read by the forward (bf16 copy or fp32 master)
  void* param(int i) {
    if (is_bf16(cfg)) return at<bf16>(lo.params_bf16) + lo.pt.off[i];
    return master() + lo.pt.off[i];
  }
  // layer slice of a per-layer parameter tensor (storage type)
  void* lparam(int i, int l) {
    int64_t per = lo.pt.shape[i][1] * lo.pt.shape[i][2];
    if (is_bf16(cfg)) return at<bf16>(lo.params_bf16) + lo.pt.off[i] + (int64_t)l * per;
    return master() + lo.pt.off[i] + (int64_t)l * per;
  }
  // transposed bf16 copy of weight matrix i (layer l): [in, out] row-major
  void* wt(int i, int l) {
    const int64_t* sh = lo.pt.shape[i];
    const int64_t per = (lo.pt.ndim[i] == 3 ? sh[1] * sh[2] : sh[0] * sh[1]);
    return lo.params_t[i] ? at<bf16>(lo.params_t[i]) + (int64_t)l * per : nullptr;
  }
  float* lgrad(int i, int l) {
    int64_t per = lo.pt.shape[i][1] * lo.pt.shape[i][2];
    return grad() + lo.pt.off[i] + (int64_t)l * per;
  }
  int dt() const { return is_bf16(cfg) ? GPT2_BF16 : GPT2_FP32; }
  bool fp8() const { return cfg.dtype == GPT2_BF16_FP8; }
  bool qk_norm() const { return (cfg.arch_flags & GPT2_ARCH_QK_NORM) != 0; }
  bool rope() const { return (cfg.arch_flags & GPT2_ARCH_ROPE) != 0; }
  bool relu2() const { return (cfg.arch_flags & GPT2_ARCH_RELU2) != 0; }
  const float2* rope_cs() { return rope() ? at<float2>(lo.rope_cs) : nullptr; }
  // fp8 mode: scale slot, and the weight codes of tensor i, layer l
  Fp8Scale* fscale(int slot) { return at<Fp8Scale>(lo.fp8_scales) + slot; }
  // the maxima a producer kernel leaves for the quantisation into `slot`
  // (null outside fp8 mode)
  float* slot_max(int slot) {
    return fp8() ? at<float>(lo.fp8_slot_max) + (size_t)slot * kAmaxWays * kAmaxStride : nullptr;
  }
  int64_t wq_per_layer(int i) const {
    const int64_t* sh = lo.pt.shape[i];
    return lo.pt.ndim[i] == 3 ? sh[1] * sh[2] : 0;
  }
  uint8_t* wq(int i, int l) { return at<uint8_t>(lo.wq[i]) + (int64_t)l * wq_per_layer(i); }
  uint8_t* wqt(int i, int l) { return at<uint8_t>(lo.wqt[i]) + (int64_t)l * wq_per_layer(i); }
  size_t es() const { return is_bf16(cfg) ? 2 : 4; }
  void* scratch() { return base + lo.scratch; }
};

namespace {

// Points kernel mark `stage` at the next event pair of `site` (if it is being
// timed and has events left).
bool timer_arm(gpt2_model* m, int site, int stage) {
  SiteTimer& t = m->timers[site];
  if (!t.on || t.used + 2 > t.ev.size()) return false;
  kernel_marks()[stage] = KernelMark{t.ev[t.used], t.ev[t.used + 1]};
  return true;
}

void timer_commit(gpt2_model* m, int site, double flops, double bytes) {
  SiteTimer& t = m->timers[site];
  t.used += 2;
  t.launches++;
  t.flops = flops;
  t.bytes = bytes;
}

void marks_clear() {
  for (int i = 0; i < kMaxMarks; ++i) kernel_marks()[i] = KernelMark{nullptr, nullptr};
}

// Calls `launch` with the launcher's main kernel timed under `site`;
// flops / bytes are the algorithmic work of one such kernel.
template <typename F>
int timed(gpt2_model* m, int site, double flops, double bytes, F&& launch) {
  if (m->dry()) return 0;
  const bool armed = timer_arm(m, site, 0);
  const int rc = launch();
  marks_clear();
  if (armed && rc == 0) timer_commit(m, site, flops, bytes);
  return rc;
}

// GEMM wrapper that records the timing site.
int run_gemm(gpt2_model* m, int site, const GemmDesc& d) {
  if (m->dry()) {
    m->plan_log->push_back({site, d});
    return 0;
  }
  const double es = (double)m->es();
  const double bytes = ((double)d.M * d.K + (double)d.N * d.K) * es +
                       (d.epi == EPI_WGRAD ? (double)d.M * d.N * 4.0 : (double)d.M * d.N * es);
  return timed(m, site, 2.0 * d.M * d.N * d.K, bytes, [&] { return gemm(d, m->stream); });
}

GemmDesc gdesc(int dtype) {
  GemmDesc d;
  memset(&d, 0, sizeof(d));
  d.dtype = dtype;
  return d;
}

// The three GEMM forms of a linear layer y = x W^T + b (W stored [N, K]),
// shared by the training step and the op-level ABI so that both launch the
// same kernels.
// Forward y[M,N] = x[M,K] W[N,K]^T (+ epilogue): both operands k-major.
GemmDesc linear_fwd_desc(int dtype, int M, int N, int K, const void* x, const void* W, int epi, void* y,
                         const void* bias, const void* aux_in, void* aux_out) {
  GemmDesc d = gdesc(dtype);
  d.a_kmajor = true; d.b_kmajor = true;
  d.M = M; d.N = N; d.K = K;
  d.A = x; d.lda = K; d.B = W; d.ldb = K;
  d.epi = epi; d.C = y; d.ldc = N; d.bias = bias; d.aux_in = aux_in; d.ld_aux = N; d.aux_out = aux_out;
  return d;
}

// dx[M,K] = dy[M,N] W[N,K] (+ a multiply by U[M,K], the saved GELU'(u)).  W
// is read through its transposed copy WT [K, N] (k-major) when there is one
// (bf16), else n-major.
GemmDesc linear_dx_desc(int dtype, int M, int N, int K, const void* dy, const void* W, const void* WT, void* dx,
                        int epi, const void* gelu_grad, void* ws, size_t ws_bytes) {
  GemmDesc d = gdesc(dtype);
  d.a_kmajor = true; d.b_kmajor = WT != nullptr;
  d.M = M; d.N = K; d.K = N;
  d.A = dy; d.lda = N;
  if (WT) { d.B = WT; d.ldb = N; } else { d.B = W; d.ldb = K; }
  d.epi = epi; d.C = dx; d.ldc = K; d.aux_in = gelu_grad; d.ld_aux = K;
  d.workspace = ws; d.workspace_bytes = ws_bytes;
  return d;
}

// dW[N,K] (+)= dy[M,N]^T x[M,K];  db[N] (+)= sum_rows dy (fused; NULL: none).
GemmDesc linear_dw_desc(int dtype, int M, int N, int K, const void* dy, const void* x, float* dW, float* db, bool acc,
                        void* ws, size_t ws_bytes) {
  GemmDesc d = gdesc(dtype);
  d.a_kmajor = false; d.b_kmajor = false;
  d.M = N; d.N = K; d.K = M;
  d.A = dy; d.lda = N; d.B = x; d.ldb = K;
  d.epi = EPI_WGRAD; d.out32 = dW; d.bias_grad32 = db; d.accumulate = acc;
  d.workspace = ws; d.workspace_bytes = ws_bytes;
  return d;
}

GemmDesc fwd_desc(gpt2_model* m, int M, int N, int K, const void* x, const void* W, int epi, void* C,
                  const void* bias, const void* aux_in, void* aux_out) {
  return linear_fwd_desc(m->dt(), M, N, K, x, W, epi, C, bias, aux_in, aux_out);
}

GemmDesc dx_desc(gpt2_model* m, int M, int N, int K, const void* dy, const void* W, const void* WT, void* dx,
                 int epi, const void* gelu_grad) {
  return linear_dx_desc(m->dt(), M, N, K, dy, W, WT, dx, epi, gelu_grad, m->scratch(), m->lo.scratch_bytes);
}

GemmDesc dw_desc(gpt2_model* m, int M, int N, int K, const void* dy, const void* x, float* dW, float* db,
                 bool acc) {
  return linear_dw_desc(m->dt(), M, N, K, dy, x, dW, db, acc, m->scratch(), m->lo.scratch_bytes);
}

// ---- fp8 mode (QKV, fc, fc-proj and head products)

// Per-tensor scale of x [R, Cc] (bf16 or fp32) into `slot`, then its codes
// row-major (q) and / or transposed (qt).  fmt 0: E4M3, 1: E5M2.
// colsum: also leave the column sums of x (for a bias gradient) in the
// arena's column-sum buffer.  produced: the kernel that wrote x also left its
// maximum in slot_max(slot) (zeroed at the start of the forward), so no pass
// of its own takes it.
// (layers > 1: that many consecutive tensors of the same shape, with
// consecutive slots, from the producers' maxima, in one launch.)
int fp8_quant(gpt2_model* m, int dtype_in, const void* x, int R, int Cc, int fmt, int slot, uint8_t* q, uint8_t* qt,
              bool colsum = false, bool produced = false, int layers = 1) {
  if (m->dry()) return 0;
  Fp8Scale* sc = m->fscale(slot);
  float* amax = produced ? m->slot_max(slot) : m->at<float>(m->lo.fp8_amax);
  if (!produced) RC(fp8_amax(dtype_in, (int64_t)R * Cc, x, amax, m->stream));
  const double n = (double)layers * R * Cc;
  const double in_b = n * (dtype_in == GPT2_BF16 ? 2 : 4);
  return timed(m, S_FP8_QUANT, 0.0, in_b + n * ((q ? 1 : 0) + (qt ? 1 : 0)), [&] {
    return fp8_quantize(dtype_in, fmt, R, Cc, x, Cc, amax, sc, q, qt, m->stream,
                        colsum ? m->at<float>(m->lo.fp8_colsum) : nullptr, produced ? kAmaxWays : 0, layers);
  });
}

// The forward product x W^T as an fp8 product of the codes xq (scale slot
// xs) and wq (slot ws); d is the bf16 descriptor (shape, epilogue, outputs).
GemmDesc fp8_fwd(gpt2_model* m, GemmDesc d, const uint8_t* xq, int xs, const uint8_t* wq, int ws) {
  d.A = xq; d.B = wq; d.fp8 = 1;
  d.scale_a = &m->fscale(xs)->s; d.scale_b = &m->fscale(ws)->s;
  return d;
}

// dX = dY W from the gradient codes dq [M, N] (slot ds) and the transposed
// weight codes wqt [K, N] (slot ws).
GemmDesc fp8_dx(gpt2_model* m, int M, int N, int K, const uint8_t* dq, int ds, const uint8_t* wqt, int ws, void* dx,
                int epi, const void* gelu_grad) {
  GemmDesc d = linear_dx_desc(GPT2_BF16, M, N, K, dq, nullptr, wqt, dx, epi, gelu_grad, m->scratch(),
                              m->lo.scratch_bytes);
  d.fp8 = 2;
  d.scale_a = &m->fscale(ds)->s; d.scale_b = &m->fscale(ws)->s;
  return d;
}

// dW [N, K] (+)= dY^T X from the row-major codes dq [M, N] (slot ds) and
// xq [M, K] (slot xs), read m-major (no transposed copies); the bias
// gradient is taken separately.
GemmDesc fp8_dw(gpt2_model* m, int M, int N, int K, const uint8_t* dq, int ds, const uint8_t* xq, int xs, float* dW,
                bool acc) {
  GemmDesc d = gdesc(GPT2_BF16);
  d.a_kmajor = d.b_kmajor = false;
  d.M = N; d.N = K; d.K = M;
  d.A = dq; d.lda = N; d.B = xq; d.ldb = K;
  d.epi = EPI_WGRAD; d.out32 = dW; d.accumulate = acc;
  d.workspace = m->scratch(); d.workspace_bytes = m->lo.scratch_bytes;
  d.fp8 = 2;
  d.scale_a = &m->fscale(ds)->s; d.scale_b = &m->fscale(xs)->s;
  return d;
}

// Bias gradient of an fp8 weight-gradient product: the column sums of the
// unquantised bf16 gradient that its quantisation left (fp8_quant(colsum)).
int fp8_bias_grad(gpt2_model* m, int M, int N, float* db, bool acc) {
  if (m->dry()) return 0;
  return colsum_reduce(M, N, m->at<float>(m->lo.fp8_colsum), db, acc, m->stream);
}

// loss_scale: the dlogits (and so every gradient of the next backward) are
// those of loss_scale x the mean loss.
int forward_impl(gpt2_model* m, const int32_t* tokens, const int32_t* targets, float loss_scale) {
  const gpt2_config& c = m->cfg;
  const int B = c.batch_size, T = c.seq_len, C = c.channels, H = c.num_heads, hd = C / H;
  const int BT = B * T, Vp = c.padded_vocab_size, V = c.vocab_size, L = c.num_layers;
  const int dt = m->dt();
  hipStream_t s = m->stream;
  Layout& lo = m->lo;
  m->have_dlogits = false;
  // keep a copy of the ids for the encoder backward (the caller may reuse its buffer)
  int32_t* tok = m->at<int32_t>(lo.tokens);
  if (m->side_pending) {   // the previous sort still reads the ids
    GPT2_HIP_CHECK(hipStreamWaitEvent(s, m->ev_join, 0));
    m->side_pending = false;
  }
  if (!m->dry()) RC(copy_i32(BT, tokens, tok, s));
  if (m->fp8() && !m->dry())   // maxima of this forward and the backward after it
    RC(fill_f32((int64_t)fp8_slots(L) * kAmaxWays * kAmaxStride, m->slot_max(0), 0.0f, s));
  if (targets && !m->dry()) {
    // the key sort of the encoder backward runs beside the forward
    GPT2_HIP_CHECK(hipEventRecord(m->ev_fork, s));
    GPT2_HIP_CHECK(hipStreamWaitEvent(m->side, m->ev_fork, 0));
    RC(encoder_sort_keys(BT, V, tok, m->at<uint64_t>(lo.sorted_keys), m->side));
    GPT2_HIP_CHECK(hipEventRecord(m->ev_join, m->side));
    m->side_pending = true;
  }
  const double es = (double)m->es();
  const double act = (double)BT * C * es;  // bytes of one [BT, C] activation
  const double ln_fwd_bytes = 2.0 * act + BT * 8.0 + 2.0 * C * es;
  const double causal_mm = 2.0 * hd * ((double)T * (T + 1) / 2.0) * B * H;  // one causal T x T x hd product
  // with rotary embeddings positions enter through q and k only: no position table
  RC(timed(m, S_ENC_FWD, 0.0, (m->rope() ? 2.0 : 3.0) * act, [&] {
    return encoder_forward(dt, B, T, C, V, tok, m->param(0), m->rope() ? nullptr : m->param(1),
                           m->at<char>(lo.resid[0]), s);
  }));
  const double qk_bytes = 2.0 * (2.0 * act) + (m->qk_norm() ? (double)BT * 2 * H * 4 : 0.0);
  for (int l = 0; l < c.num_layers; ++l) {
    LayerOffsets& o = lo.layer[l];
    void* x = m->at<char>(lo.resid[l]);
    RC(timed(m, S_LN_FWD, 0.0, ln_fwd_bytes, [&] {
      return layernorm_forward(dt, BT, C, x, m->lparam(2, l), m->lparam(3, l), m->at<char>(o.ln1),
                               m->at<float>(o.ln1_mean), m->at<float>(o.ln1_rstd), s,
                               m->slot_max(fp8_slot(L, Q_ACT, 0, l)));
    }));
    {
      GemmDesc d = fwd_desc(m, BT, 3 * C, C, m->at<char>(o.ln1), m->lparam(4, l), EPI_BIAS, m->at<char>(o.qkv),
                            m->lparam(5, l), nullptr, nullptr);
      if (m->fp8()) {
        RC(fp8_quant(m, GPT2_BF16, m->at<char>(o.ln1), BT, C, 0, fp8_slot(L, Q_ACT, 0, l), m->at<uint8_t>(o.ln1_q),
                     nullptr, false, true));
        d = fp8_fwd(m, d, m->at<uint8_t>(o.ln1_q), fp8_slot(L, Q_ACT, 0, l), m->wq(4, l), fp8_slot(L, Q_WEIGHT, 1, l));
      }
      RC(run_gemm(m, S_QKV, d));
    }
    if (m->qk_norm() || m->rope())     // q and k transformed in place before the attention reads them
      RC(timed(m, S_QK_FWD, 0.0, qk_bytes, [&] {
        return qk_transform_forward(dt, BT, T, H, hd, m->at<char>(o.qkv), m->at<float>(o.qk_rstd), m->rope_cs(),
                                    m->qk_norm(), m->rope(), s);
      }));
    RC(timed(m, S_ATTN_FWD, 2.0 * causal_mm, 4.0 * act + (double)B * H * T * 4, [&] {
      return attention_forward(dt, B, T, H, hd, m->at<char>(o.qkv), m->at<char>(o.atty), m->at<float>(o.lse), s);
    }));
    RC(run_gemm(m, S_ATTPROJ, fwd_desc(m, BT, C, C, m->at<char>(o.atty), m->lparam(6, l), EPI_BIAS_RES,
                                       m->at<char>(o.h), m->lparam(7, l), x, nullptr)));
    RC(timed(m, S_LN_FWD, 0.0, ln_fwd_bytes, [&] {
      return layernorm_forward(dt, BT, C, m->at<char>(o.h), m->lparam(8, l), m->lparam(9, l), m->at<char>(o.ln2),
                               m->at<float>(o.ln2_mean), m->at<float>(o.ln2_rstd), s,
                               m->slot_max(fp8_slot(L, Q_ACT, 1, l)));
    }));
    // g = GELU(u) for the fc-proj product, and GELU'(u) kept for the backward
    {
      GemmDesc d = fwd_desc(m, BT, 4 * C, C, m->at<char>(o.ln2), m->lparam(10, l),
                            m->relu2() ? EPI_BIAS_RELU2_D : EPI_BIAS_GELU_D, m->at<char>(o.g), m->lparam(11, l),
                            nullptr, m->at<char>(o.u));
      if (m->fp8()) {
        RC(fp8_quant(m, GPT2_BF16, m->at<char>(o.ln2), BT, C, 0, fp8_slot(L, Q_ACT, 1, l), m->at<uint8_t>(o.ln2_q),
                     nullptr, false, true));
        d = fp8_fwd(m, d, m->at<uint8_t>(o.ln2_q), fp8_slot(L, Q_ACT, 1, l), m->wq(10, l),
                    fp8_slot(L, Q_WEIGHT, 2, l));
        d.amax = m->slot_max(fp8_slot(L, Q_ACT, 2, l));   // g's maximum, for its quantisation below
      }
      RC(run_gemm(m, S_FC, d));
    }
    {
      GemmDesc d = fwd_desc(m, BT, C, 4 * C, m->at<char>(o.g), m->lparam(12, l), EPI_BIAS_RES,
                            m->at<char>(lo.resid[l + 1]), m->lparam(13, l), m->at<char>(o.h), nullptr);
      if (m->fp8()) {
        RC(fp8_quant(m, GPT2_BF16, m->at<char>(o.g), BT, 4 * C, 0, fp8_slot(L, Q_ACT, 2, l), m->at<uint8_t>(o.g_q),
                     nullptr, false, true));
        d = fp8_fwd(m, d, m->at<uint8_t>(o.g_q), fp8_slot(L, Q_ACT, 2, l), m->wq(12, l),
                    fp8_slot(L, Q_WEIGHT, 3, l));
      }
      RC(run_gemm(m, S_FCPROJ, d));
    }
  }
  RC(timed(m, S_LN_FWD, 0.0, ln_fwd_bytes, [&] {
    return layernorm_forward(dt, BT, C, m->at<char>(lo.resid[c.num_layers]), m->param(14), m->param(15),
                             m->at<char>(lo.lnf), m->at<float>(lo.lnf_mean), m->at<float>(lo.lnf_rstd), s,
                             m->slot_max(fp8_slot(L, Q_ACT, 3, 0)));
  }));
  {
    GemmDesc d = fwd_desc(m, BT, Vp, C, m->at<char>(lo.lnf), m->param(0), EPI_STORE, m->at<char>(lo.logits), nullptr,
                          nullptr, nullptr);
    if (m->fp8()) {
      RC(fp8_quant(m, GPT2_BF16, m->at<char>(lo.lnf), BT, C, 0, fp8_slot(L, Q_ACT, 3, 0), m->at<uint8_t>(lo.lnf_q),
                   nullptr, false, true));
      d = fp8_fwd(m, d, m->at<uint8_t>(lo.lnf_q), fp8_slot(L, Q_ACT, 3, 0), m->wq(0, 0), fp8_slot(L, Q_WEIGHT, 0, 0));
    }
    RC(run_gemm(m, S_LOGITS, d));
  }
  if (targets) {
    RC(timed(m, S_XENT, 0.0, 2.0 * BT * (double)Vp * es + BT * 8.0, [&] {
      return softmax_xent(dt, BT, V, Vp, m->at<char>(lo.logits), targets, m->at<float>(lo.losses), loss_scale / BT,
                          s, softmax_xent_has_amax(dt, V, Vp) ? m->slot_max(fp8_slot(L, Q_GRAD, 3, 0)) : nullptr);
    }));
    if (!m->dry()) RC(sum_scaled(BT, m->at<float>(lo.losses), 1.0f / BT, m->at<float>(lo.mean_loss), s));
    m->have_dlogits = true;
  }
  return 0;
}

// acc: parameter gradients are added to the ones held (gradient accumulation)
// instead of overwriting them.
int backward_impl(gpt2_model* m, bool acc) {
  const gpt2_config& c = m->cfg;
  const int B = c.batch_size, T = c.seq_len, C = c.channels, H = c.num_heads, hd = C / H;
  const int BT = B * T, Vp = c.padded_vocab_size, L = c.num_layers;
  const int dt = m->dt();
  hipStream_t s = m->stream;
  Layout& lo = m->lo;
  void* d_ln = m->at<char>(lo.d_ln);
  void* d_big = m->at<char>(lo.d_big);
  void* d_qkv = m->at<char>(lo.d_qkv);
  float* dres = m->at<float>(lo.dres);
  void* dres_t = m->at<char>(lo.dres_t);
  void* dres_copy = dt == GPT2_BF16 ? dres_t : nullptr;
  void* logits = m->at<char>(lo.logits);
  const size_t sb = lo.scratch_bytes;
  const double es = (double)m->es();
  const double act = (double)BT * C * es;
  const double causal_mm = 2.0 * hd * ((double)T * (T + 1) / 2.0) * B * H;
  // dy, x read; fp32 residual gradient written (overwrite) or read + written; its copy; stats
  auto ln_bwd_bytes = [&](bool ovw) {
    return 2.0 * act + (double)BT * C * (ovw ? 4.0 : 8.0) + (dres_copy ? act : 0.0) + BT * 8.0 + C * es;
  };

  uint8_t* dq = m->at<uint8_t>(lo.dq);
  // classifier: d_lnf = dz wte;  d_wte = dz^T lnf (overwrite; padded rows get exactly 0)
  if (m->fp8()) {
    const int gs = fp8_slot(L, Q_GRAD, 3, 0);
    RC(fp8_quant(m, GPT2_BF16, logits, BT, Vp, 1, gs, dq, nullptr, false, softmax_xent_has_amax(dt, c.vocab_size, Vp)));
    RC(run_gemm(m, S_CLS_DX, fp8_dx(m, BT, Vp, C, dq, gs, m->wqt(0, 0), fp8_slot(L, Q_WEIGHT, 0, 0), d_ln, EPI_STORE,
                                    nullptr)));
    RC(run_gemm(m, S_CLS_DW, fp8_dw(m, BT, Vp, C, dq, gs, m->at<uint8_t>(lo.lnf_q), fp8_slot(L, Q_ACT, 3, 0),
                                    m->lgrad(0, 0), acc)));
  } else {
    RC(run_gemm(m, S_CLS_DX, dx_desc(m, BT, Vp, C, logits, m->param(0), m->wt(0, 0), d_ln, EPI_STORE, nullptr)));
    RC(run_gemm(m, S_CLS_DW, dw_desc(m, BT, Vp, C, logits, m->at<char>(lo.lnf), m->lgrad(0, 0), nullptr, acc)));
  }
  RC(timed(m, S_LN_BWD, 0.0, ln_bwd_bytes(true), [&] {
    return layernorm_backward(dt, BT, C, d_ln, m->at<char>(lo.resid[L]), m->param(14), m->at<float>(lo.lnf_mean),
                              m->at<float>(lo.lnf_rstd), dres, true, dres_copy, m->lgrad(14, 0), m->lgrad(15, 0),
                              acc, m->scratch(), sb, s, m->slot_max(fp8_slot(L, Q_GRAD, 0, L - 1)));
  }));
  for (int l = L - 1; l >= 0; --l) {
    LayerOffsets& o = lo.layer[l];
    if (m->fp8()) {
      // x_{l+1} = h + g Wp^T + bp: dY = the residual gradient (bf16 copy)
      const int gp = fp8_slot(L, Q_GRAD, 0, l), gf = fp8_slot(L, Q_GRAD, 1, l);
      RC(fp8_quant(m, GPT2_BF16, dres_t, BT, C, 1, gp, dq, nullptr, true, true));
      RC(run_gemm(m, S_FCPROJ_DW, fp8_dw(m, BT, C, 4 * C, dq, gp, m->at<uint8_t>(o.g_q), fp8_slot(L, Q_ACT, 2, l),
                                         m->lgrad(12, l), acc)));
      RC(fp8_bias_grad(m, BT, C, m->lgrad(13, l), acc));
      // du = (dy W_p) * GELU'(u), the derivative saved by the forward
      GemmDesc ddx = fp8_dx(m, BT, C, 4 * C, dq, gp, m->wqt(12, l), fp8_slot(L, Q_WEIGHT, 3, l), d_big, EPI_MUL,
                            m->at<char>(o.u));
      ddx.amax = m->slot_max(gf);   // du's maximum, for its quantisation below
      RC(run_gemm(m, S_FCPROJ_DX, ddx));
      // u = ln2 Wfc^T + bfc   (d_big now holds du)
      RC(fp8_quant(m, GPT2_BF16, d_big, BT, 4 * C, 1, gf, dq, nullptr, true, true));
      RC(run_gemm(m, S_FC_DW, fp8_dw(m, BT, 4 * C, C, dq, gf, m->at<uint8_t>(o.ln2_q), fp8_slot(L, Q_ACT, 1, l),
                                     m->lgrad(10, l), acc)));
      RC(fp8_bias_grad(m, BT, 4 * C, m->lgrad(11, l), acc));
      RC(run_gemm(m, S_FC_DX, fp8_dx(m, BT, 4 * C, C, dq, gf, m->wqt(10, l), fp8_slot(L, Q_WEIGHT, 2, l), d_ln,
                                     EPI_STORE, nullptr)));
    } else {
      // x_{l+1} = h + g Wp^T + bp
      RC(run_gemm(m, S_FCPROJ_DW, dw_desc(m, BT, C, 4 * C, dres_t, m->at<char>(o.g), m->lgrad(12, l),
                                          m->lgrad(13, l), acc)));
      // du = (dy W_p) * GELU'(u), the derivative saved by the forward
      RC(run_gemm(m, S_FCPROJ_DX, dx_desc(m, BT, C, 4 * C, dres_t, m->lparam(12, l), m->wt(12, l), d_big, EPI_MUL,
                                          m->at<char>(o.u))));
      // u = ln2 Wfc^T + bfc   (d_big now holds du)
      RC(run_gemm(m, S_FC_DW, dw_desc(m, BT, 4 * C, C, d_big, m->at<char>(o.ln2), m->lgrad(10, l),
                                      m->lgrad(11, l), acc)));
      RC(run_gemm(m, S_FC_DX, dx_desc(m, BT, 4 * C, C, d_big, m->lparam(10, l), m->wt(10, l), d_ln, EPI_STORE,
                                      nullptr)));
    }
    RC(timed(m, S_LN_BWD, 0.0, ln_bwd_bytes(false), [&] {
      return layernorm_backward(dt, BT, C, d_ln, m->at<char>(o.h), m->lparam(8, l), m->at<float>(o.ln2_mean),
                                m->at<float>(o.ln2_rstd), dres, false, dres_copy, m->lgrad(8, l), m->lgrad(9, l),
                                acc, m->scratch(), sb, s);
    }));
    // fp8: the attention backward kernels also take dqkv's maximum for its
    // quantisation, unless the QK transform rewrites dq and dk after them
    const bool qkv_max = m->fp8() && attention_mfma_supported(dt, hd) && !m->qk_norm() && !m->rope();
    // h = x + atty Wo^T + bo
    RC(run_gemm(m, S_ATTPROJ_DW, dw_desc(m, BT, C, C, dres_t, m->at<char>(o.atty), m->lgrad(6, l),
                                         m->lgrad(7, l), acc)));
    RC(run_gemm(m, S_ATTPROJ_DX, dx_desc(m, BT, C, C, dres_t, m->lparam(6, l), m->wt(6, l), d_ln, EPI_STORE, nullptr)));
    if (!m->dry()) {
      // dK, dV (recomputing S and dP) and dQ; D = rowsum(dO * O) is a kernel of
      // its own except on the matrix-core path, where the dQ kernel forms it
      const bool mfma = attention_mfma_supported(dt, hd);
      const bool a0 = !mfma && timer_arm(m, S_ATTN_DOT, 0), a1 = timer_arm(m, S_ATTN_DKDV, 1),
                 a2 = timer_arm(m, S_ATTN_DQ, 2);
      const int rc = attention_backward(dt, B, T, H, hd, m->at<char>(o.qkv), m->at<char>(o.atty), d_ln,
                                        m->at<float>(o.lse), d_qkv, m->scratch(), sb, s,
                                        qkv_max ? m->slot_max(fp8_slot(L, Q_GRAD, 2, l)) : nullptr);
      marks_clear();
      RC(rc);
      const double lse_b = (double)B * H * T * 4;
      // algorithmic work: the method's backward is four causal products (dV,
      // dP, dQ, dK); the dK/dV kernel is credited with dV, dP and dK, the dQ
      // kernel with dQ (the recomputed S, and dP again in the dQ kernel, are
      // not counted)
      if (a0) timer_commit(m, S_ATTN_DOT, 0.0, 2.0 * act + lse_b);
      if (a1) timer_commit(m, S_ATTN_DKDV, 3.0 * causal_mm, 4.0 * act + 2.0 * lse_b + 2.0 * act);
      if (a2) timer_commit(m, S_ATTN_DQ, 1.0 * causal_mm, 4.0 * act + 2.0 * lse_b + act + (mfma ? act + lse_b : 0.0));
    }
    if (m->qk_norm() || m->rope())     // gradient back through the rotation and the normalisation
      RC(timed(m, S_QK_BWD, 0.0, (m->qk_norm() ? 3.0 : 2.0) * (2.0 * act) + (m->qk_norm() ? (double)BT * 2 * H * 4 : 0.0), [&] {
        return qk_transform_backward(dt, BT, T, H, hd, m->at<char>(o.qkv), d_qkv, m->at<float>(o.qk_rstd),
                                     m->rope_cs(), m->qk_norm(), m->rope(), s);
      }));
    // qkv = ln1 Wqkv^T + bqkv
    if (m->fp8()) {
      const int gq = fp8_slot(L, Q_GRAD, 2, l);
      RC(fp8_quant(m, GPT2_BF16, d_qkv, BT, 3 * C, 1, gq, dq, nullptr, true, qkv_max));
      RC(run_gemm(m, S_QKV_DW, fp8_dw(m, BT, 3 * C, C, dq, gq, m->at<uint8_t>(o.ln1_q), fp8_slot(L, Q_ACT, 0, l),
                                      m->lgrad(4, l), acc)));
      RC(fp8_bias_grad(m, BT, 3 * C, m->lgrad(5, l), acc));
      RC(run_gemm(m, S_QKV_DX, fp8_dx(m, BT, 3 * C, C, dq, gq, m->wqt(4, l), fp8_slot(L, Q_WEIGHT, 1, l), d_ln,
                                      EPI_STORE, nullptr)));
    } else {
      RC(run_gemm(m, S_QKV_DW, dw_desc(m, BT, 3 * C, C, d_qkv, m->at<char>(o.ln1), m->lgrad(4, l),
                                       m->lgrad(5, l), acc)));
      RC(run_gemm(m, S_QKV_DX, dx_desc(m, BT, 3 * C, C, d_qkv, m->lparam(4, l), m->wt(4, l), d_ln, EPI_STORE,
                                       nullptr)));
    }
    RC(timed(m, S_LN_BWD, 0.0, ln_bwd_bytes(false), [&] {
      return layernorm_backward(dt, BT, C, d_ln, m->at<char>(lo.resid[l]), m->lparam(2, l),
                                m->at<float>(o.ln1_mean), m->at<float>(o.ln1_rstd), dres, false, dres_copy,
                                m->lgrad(2, l), m->lgrad(3, l), acc, m->scratch(), sb, s,
                                l > 0 ? m->slot_max(fp8_slot(L, Q_GRAD, 0, l - 1)) : nullptr);
    }));
  }
  // encoder: wpe rows >= T get no gradient (zero already when accumulating),
  // and none at all with rotary embeddings (the table is not used)
  float* dwpe = m->lgrad(1, 0);
  if (m->dry()) return 0;
  if (!acc) {
    const int first_zero = m->rope() ? 0 : T;
    RC(fill_f32((int64_t)(c.max_seq_len - first_zero) * C, dwpe + (size_t)first_zero * C, 0.f, s));
  }
  if (m->rope()) dwpe = nullptr;
  if (m->side_pending) {
    GPT2_HIP_CHECK(hipStreamWaitEvent(s, m->ev_join, 0));
    m->side_pending = false;
  }
  RC(encoder_backward_sorted(B, T, C, m->at<uint64_t>(lo.sorted_keys), dres, m->lgrad(0, 0), dwpe, acc, m->scratch(),
                             sb, s));
  return 0;
}

int init_params(gpt2_model* m, uint64_t seed) {
  const gpt2_config& c = m->cfg;
  hipStream_t s = m->stream;
  const double resid_std = 0.02 / sqrt(2.0 * (c.num_layers > 0 ? c.num_layers : 1));
  for (int i = 0; i < 16; ++i) {
    const int64_t n = m->lo.pt.shape[i][0] * m->lo.pt.shape[i][1] * m->lo.pt.shape[i][2];
    float* dst = m->master() + m->lo.pt.off[i];
    auto is = [&](const char* x) { return strcmp(kParamNames[i], x) == 0; };
    if (is("ln1w") || is("ln2w") || is("lnfw")) {
      RC(fill_f32(n, dst, 1.0f, s));
    } else if (is("wte") || is("wpe") || is("qkvw") || is("fcw") || is("attprojw") || is("fcprojw")) {
      const double sd = (is("attprojw") || is("fcprojw")) ? resid_std : 0.02;
      RC(init_normal(n, dst, seed, i, sd, s));
      if (i == 0)
        RC(fill_f32((int64_t)(c.padded_vocab_size - c.vocab_size) * c.channels,
                    dst + (size_t)c.vocab_size * c.channels, 0.f, s));
    } else {
      RC(fill_f32(n, dst, 0.f, s));
    }
  }
  return 0;
}

// Transposed copies of the weight matrices from the bf16 working copy.
int refresh_transposed(gpt2_model* m) {
  if (!is_bf16(m->cfg)) return 0;
  for (int i : kTransposed) {
    if (!m->lo.params_t[i]) continue;   // (fp8 mode: only the attention projection keeps a bf16 copy)
    const int64_t* sh = m->lo.pt.shape[i];
    const bool layered = m->lo.pt.ndim[i] == 3;
    const int batches = layered ? (int)sh[0] : 1;
    const int R = (int)(layered ? sh[1] : sh[0]), Cc = (int)(layered ? sh[2] : sh[1]);
    RC(timed(m, S_WT, 0.0, 4.0 * batches * (double)R * Cc, [&] {
      return transpose_bf16(batches, R, Cc, static_cast<const bf16*>(m->param(i)), static_cast<bf16*>(m->wt(i, 0)),
                            m->stream);
    }));
  }
  return 0;
}

// fp8 mode: E4M3 codes (row-major and transposed) of the fp8 products'
// weights, quantised per matrix from the fp32 master.  produced: the AdamW
// update left each matrix's maximum in its scale slot.
int refresh_fp8_weights(gpt2_model* m, bool produced = false) {
  if (!m->fp8()) return 0;
  const int L = m->cfg.num_layers;
  for (int w = 0; w < 4; ++w) {
    const int i = kFp8Weights[w];
    const int64_t* sh = m->lo.pt.shape[i];
    const bool layered = m->lo.pt.ndim[i] == 3;
    const int R = (int)(layered ? sh[1] : sh[0]), Cc = (int)(layered ? sh[2] : sh[1]);
    if (produced && layered) {   // every layer's matrix in one launch (their slots are consecutive)
      RC(fp8_quant(m, GPT2_FP32, m->master() + m->lo.pt.off[i], R, Cc, 0, fp8_slot(L, Q_WEIGHT, w, 0), m->wq(i, 0),
                   m->wqt(i, 0), false, true, L));
      continue;
    }
    for (int l = 0; l < (layered ? L : 1); ++l) {
      const float* src = m->master() + m->lo.pt.off[i] + (int64_t)l * R * Cc;
      RC(fp8_quant(m, GPT2_FP32, src, R, Cc, 0, fp8_slot(L, Q_WEIGHT, w, l), m->wq(i, l), m->wqt(i, l), false,
                   produced));
    }
  }
  return 0;
}

int refresh_bf16(gpt2_model* m) {
  if (!is_bf16(m->cfg)) return 0;
  RC(cast_f32_to_bf16(m->lo.P, m->master(), m->at<bf16>(m->lo.params_bf16), m->stream));
  RC(refresh_fp8_weights(m));
  return refresh_transposed(m);
}

// The parameter update: optional gradient norm and clipping factor, AdamW
// with its hyperparameters read from the arena's block (written beforehand in
// stream order), the transposed bf16 weight copies.
int update_impl(gpt2_model* m, float max_grad_norm, bool need_norm) {
  float* gn = m->at<float>(m->lo.gnorm);
  if (need_norm) {
    // fp32 gradients read once
    RC(timed(m, S_GRAD_NORM, 0.0, 4.0 * (double)m->lo.P,
             [&] { return grad_norm(m->lo.P, m->grad(), max_grad_norm, gn, m->stream); }));
  }
  const float* gscale = max_grad_norm > 0.f ? gn + 1 : nullptr;
  if (!is_bf16(m->cfg)) {
    // fp32 master, m, v read and written, fp32 gradient read
    return timed(m, S_ADAMW, 0.0, (double)m->lo.P * 28.0, [&] {
      return adamw(m->lo.P, m->master(), m->grad(), m->at<float>(m->lo.adam_m), m->at<float>(m->lo.adam_v),
                   nullptr, 0.f, 0.f, 0.f, 0.f, 0.f, 1, m->stream, gscale, m->at<AdamHP>(m->lo.adam_hp));
    });
  }
  // bf16 modes: one launch that also writes the transposed bf16 weight
  // copies and, in fp8 mode, takes the fp8 weights' maxima; bytes: master, m,
  // v read and written, gradient read, bf16 copy written (30 per parameter)
  // and the transposed copies (2 per element)
  AdamMatrix mats[kAdamMaxMats];
  int nm = 0;
  double tbytes = 0.0;
  const int L = m->cfg.num_layers;
  if (m->fp8() && !m->dry())   // the weight slots (0 .. 3L) start from zero
    RC(fill_f32((int64_t)(1 + 3 * L) * kAmaxWays * kAmaxStride, m->slot_max(0), 0.0f, m->stream));
  for (int i : kTransposed) {   // (in parameter order; a superset of the fp8 weights)
    float* amax = nullptr;
    for (int w = 0; w < 4; ++w)
      if (m->fp8() && kFp8Weights[w] == i) amax = m->slot_max(fp8_slot(L, Q_WEIGHT, w, 0));
    // (fp8 mode: only the attention projection keeps a transposed bf16 copy)
    bf16* dst_t = m->lo.params_t[i] ? static_cast<bf16*>(m->wt(i, 0)) : nullptr;
    if (!dst_t && !amax) continue;
    const int64_t* sh = m->lo.pt.shape[i];
    const bool layered = m->lo.pt.ndim[i] == 3;
    const int R = (int)(layered ? sh[1] : sh[0]), Cc = (int)(layered ? sh[2] : sh[1]);
    mats[nm++] = AdamMatrix{(int64_t)m->lo.pt.off[i], layered ? (int)sh[0] : 1, R, Cc, dst_t, 0, amax};
    if (dst_t) tbytes += 2.0 * (layered ? (double)sh[0] : 1.0) * R * Cc;
  }
  RC(timed(m, S_ADAMW, 0.0, (double)m->lo.P * 30.0 + tbytes, [&] {
    return adamw_transposed(m->lo.P, m->master(), m->grad(), m->at<float>(m->lo.adam_m), m->at<float>(m->lo.adam_v),
                            m->at<bf16>(m->lo.params_bf16), mats, nm, m->stream, gscale,
                            m->at<AdamHP>(m->lo.adam_hp));
  }));
  return refresh_fp8_weights(m, true);
}

void graph_release(gpt2_model* m) {
  if (m->graph_exec) (void)hipGraphExecDestroy(m->graph_exec);
  if (m->graph) (void)hipGraphDestroy(m->graph);
  m->graph_exec = nullptr;
  m->graph = nullptr;
}

}  // namespace

// ================================================================ C ABI

static_assert(GPT2_EPI_STORE == EPI_STORE && GPT2_EPI_BIAS == EPI_BIAS && GPT2_EPI_BIAS_RESIDUAL == EPI_BIAS_RES &&
                  GPT2_EPI_BIAS_RELU2 == EPI_BIAS_RELU2_D && GPT2_EPI_WGRAD == EPI_WGRAD &&
                  GPT2_EPI_BIAS_GELU == EPI_BIAS_GELU_D && GPT2_EPI_MUL == EPI_MUL,
              "epilogue codes of gpt2_ops.h");

namespace {

const char* site_name(int site) {
  static const char* const names[S_COUNT] = {
      "qkv", "attproj", "fc", "fcproj", "logits", "fcproj_dx", "fcproj_dw", "fc_dx", "fc_dw", "attproj_dx",
      "attproj_dw", "qkv_dx", "qkv_dw", "cls_dx", "cls_dw", "attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq",
      "attn_bwd_dot", "softmax_xent", "ln_fwd", "ln_bwd", "encoder_fwd", "adamw", "weight_transpose", "grad_norm",
      "qk_fwd", "qk_bwd", "fp8_quant"};
  return site >= 0 && site < S_COUNT ? names[site] : "";
}

void fill_plan(const GemmDesc& d, const char* site, gpt2_gemm_plan* out) {
  memset(out, 0, sizeof(*out));
  snprintf(out->site, sizeof(out->site), "%s", site);
  const GemmLaunchInfo li = gemm_launch_info(d);
  out->M = d.M; out->N = d.N; out->K = d.K;
  out->epilogue = d.epi;
  out->a_kmajor = d.a_kmajor; out->b_kmajor = d.b_kmajor;
  out->tile_m = li.tile_m; out->tile_n = li.tile_n;
  out->waves = li.waves; out->k_groups = li.kgroups; out->k_splits = li.splits;
  out->bias_grad = li.bias_grad;
  out->fp8 = d.fp8;
}

bool any_timer_on(const gpt2_model* m) {
  for (const auto& t : m->timers)
    if (t.on) return true;
  return false;
}

// The op-level linear layer's GEMMs (forward; dW; dX) for these arguments.
// bf16 dX reads W through a transposed copy WT [K, N] that the op writes at
// the start of its workspace (the step keeps the same copy of each weight).
size_t op_wt_bytes(int dtype, int N, int K) {
  return dtype == GPT2_BF16 ? ((size_t)N * K * 2 + 255) / 256 * 256 : 0;
}

}  // namespace

extern "C" {

const char* gpt2_status_string(int st) {
  switch (st) {
    case GPT2_OK: return "ok";
    case GPT2_E_INVALID_ARG: return "invalid argument";
    case GPT2_E_STATE: return "invalid call order";
    case GPT2_E_OOM: return "out of memory / workspace too small";
    case GPT2_E_HIP: return "HIP runtime error";
    case GPT2_E_INTERNAL: return "internal error";
  }
  return "unknown status";
}

const char* gpt2_last_error(void) { return g_last_error; }

int gpt2_test_fail_host_allocations(int n) {
  g_fail_allocs.store(n > 0 ? n : 0);
  return GPT2_OK;
}

int gpt2_validate_config(const gpt2_config* cfg) {
  g_last_error[0] = 0;
  return validate(cfg);
}

int64_t gpt2_num_parameters(const gpt2_config* cfg, int padded) {
  if (validate(cfg)) return -1;
  ParamTable t;
  param_table(*cfg, padded != 0, &t);
  return t.total;
}

int gpt2_num_param_tensors(void) { return 16; }

int gpt2_param_info(const gpt2_config* cfg, int i, const char** name, int64_t* offset, int64_t shape[3],
                    int32_t* ndim) {
  RC(validate(cfg));
  if (i < 0 || i >= 16) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "tensor index %d out of range", i);
  ParamTable t;
  param_table(*cfg, true, &t);
  if (name) *name = kParamNames[i];
  if (offset) *offset = t.off[i];
  if (shape)
    for (int d = 0; d < 3; ++d) shape[d] = t.shape[i][d];
  if (ndim) *ndim = t.ndim[i];
  return GPT2_OK;
}

size_t gpt2_workspace_bytes(const gpt2_config* cfg) {
  GPT2_ABI_BEGIN
  if (validate(cfg)) return 0;
  Layout lo;
  make_layout(*cfg, &lo);
  return lo.total;
  GPT2_ABI_END(0)
}

int gpt2_step_gemm_plans(const gpt2_config* cfg, gpt2_gemm_plan* out, int max_plans, int* count) {
  GPT2_ABI_BEGIN
  RC(validate(cfg));
  if (!count || max_plans < 0 || (max_plans > 0 && !out))
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "step_gemm_plans: bad output arguments");
  gpt2_model m;
  m.cfg = *cfg;
  make_layout(*cfg, &m.lo);
  m.base = nullptr;
  m.stream = nullptr;
  std::vector<std::pair<int, GemmDesc>> log;
  m.plan_log = &log;
  // a forward with targets and a full backward, planning only
  static const int32_t kNoIds = 0;
  RC(forward_impl(&m, &kNoIds, &kNoIds, 1.0f));
  RC(backward_impl(&m, false));
  const int n = (int)log.size();
  for (int i = 0; i < n && i < max_plans; ++i) fill_plan(log[i].second, site_name(log[i].first), &out[i]);
  *count = n;
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

int gpt2_create(const gpt2_config* cfg, uint64_t seed, void* stream, void* workspace, size_t workspace_bytes,
                gpt2_model** out) {
  GPT2_ABI_BEGIN
  g_last_error[0] = 0;
  if (!out) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  RC(validate(cfg));
  gpt2_model* m = new (std::nothrow) gpt2_model();
  if (!m) return gpt2_internal_fail(GPT2_E_OOM, "host allocation failed");
  try {
    m->cfg = *cfg;
    make_layout(*cfg, &m->lo);
  } catch (...) {
    delete m;
    throw;
  }
  m->stream = (hipStream_t)stream;
  if (hipGetDevice(&m->device) != hipSuccess) {
    delete m;
    return gpt2_internal_fail(GPT2_E_HIP, "hipGetDevice failed");
  }
  if (workspace) {
    if (workspace_bytes < m->lo.total || (uintptr_t)workspace % 256) {
      size_t need = m->lo.total;
      delete m;
      return gpt2_internal_fail(GPT2_E_OOM, "workspace of %zu bytes (need %zu, 256-byte aligned)", workspace_bytes,
                                need);
    }
    m->base = (char*)workspace;
    m->owns = false;
  } else {
    void* p = nullptr;
    if (hipMalloc(&p, m->lo.total) != hipSuccess) {
      (void)hipGetLastError();
      size_t need = m->lo.total;
      delete m;
      return gpt2_internal_fail(GPT2_E_OOM, "hipMalloc(%zu) failed", need);
    }
    m->base = (char*)p;
    m->owns = true;
  }
  int rc = 0;
  if (hipStreamCreateWithFlags(&m->side, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&m->ev_fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&m->ev_join, hipEventDisableTiming) != hipSuccess)
    rc = gpt2_internal_fail(GPT2_E_HIP, "side stream / event creation failed");
  if (!rc) rc = init_params(m, seed);
  if (!rc && m->rope()) rc = rope_table(cfg->max_seq_len, cfg->channels / cfg->num_heads, m->at<float2>(m->lo.rope_cs),
                                        m->stream);
  if (!rc) rc = fill_f32(m->lo.P, m->at<float>(m->lo.adam_m), 0.f, m->stream);
  if (!rc) rc = fill_f32(m->lo.P, m->at<float>(m->lo.adam_v), 0.f, m->stream);
  if (!rc) rc = fill_f32(m->lo.P, m->grad(), 0.f, m->stream);
  if (!rc) rc = refresh_bf16(m);
  if (!rc && hipStreamSynchronize(m->stream) != hipSuccess) rc = gpt2_internal_fail(GPT2_E_HIP, "sync failed");
  if (rc) {
    if (m->side) (void)hipStreamDestroy(m->side);
    if (m->ev_fork) (void)hipEventDestroy(m->ev_fork);
    if (m->ev_join) (void)hipEventDestroy(m->ev_join);
    if (m->owns) (void)hipFree(m->base);
    delete m;
    return rc;
  }
  *out = m;
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

void gpt2_destroy(gpt2_model* m) {
  if (!m) return;
  try {
    (void)hipStreamSynchronize(m->stream);
    graph_release(m);
    if (m->side) {
      (void)hipStreamSynchronize(m->side);
      (void)hipStreamDestroy(m->side);
    }
    if (m->ev_fork) (void)hipEventDestroy(m->ev_fork);
    if (m->ev_join) (void)hipEventDestroy(m->ev_join);
    for (auto& t : m->timers)
      for (auto e : t.ev)
        if (e) (void)hipEventDestroy(e);
    if (m->owns) (void)hipFree(m->base);
    delete m;
  } catch (...) {
    // nothing may escape; the model is leaked rather than half destroyed
  }
}

int gpt2_forward(gpt2_model* m, const int32_t* d_tokens, const int32_t* d_targets, float* mean_loss) {
  return gpt2_forward_scaled(m, d_tokens, d_targets, 1.0f, mean_loss);
}

int gpt2_forward_scaled(gpt2_model* m, const int32_t* d_tokens, const int32_t* d_targets, float loss_scale,
                        float* mean_loss) {
  GPT2_ABI_BEGIN
  if (!m || !d_tokens) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "forward: NULL model or tokens");
  if (!isfinite(loss_scale))
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "forward: loss_scale must be finite");
  RC(forward_impl(m, d_tokens, d_targets, loss_scale));
  if (d_targets && mean_loss) {
    GPT2_HIP_CHECK(hipMemcpyAsync(mean_loss, m->at<float>(m->lo.mean_loss), sizeof(float), hipMemcpyDeviceToHost,
                                  m->stream));
    GPT2_HIP_CHECK(hipStreamSynchronize(m->stream));
  }
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

int gpt2_backward(gpt2_model* m) {
  GPT2_ABI_BEGIN
  if (!m) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "backward: NULL model");
  if (!m->have_dlogits) return gpt2_internal_fail(GPT2_E_STATE, "backward needs a forward with targets first");
  RC(backward_impl(m, false));
  m->have_dlogits = false;
  m->have_grads = true;
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

int gpt2_backward_accumulate(gpt2_model* m) {
  GPT2_ABI_BEGIN
  if (!m) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "backward: NULL model");
  if (!m->have_dlogits) return gpt2_internal_fail(GPT2_E_STATE, "backward needs a forward with targets first");
  if (!m->have_grads)
    return gpt2_internal_fail(GPT2_E_STATE, "backward_accumulate needs gradients from a backward since the last update");
  RC(backward_impl(m, true));
  m->have_dlogits = false;
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

int gpt2_adamw_step(gpt2_model* m, float lr, float beta1, float beta2, float eps, float weight_decay, int32_t t) {
  return gpt2_adamw_step_clipped(m, lr, beta1, beta2, eps, weight_decay, t, 0.0f, nullptr);
}

int gpt2_adamw_step_clipped(gpt2_model* m, float lr, float beta1, float beta2, float eps, float weight_decay,
                            int32_t t, float max_grad_norm, float* grad_norm_out) {
  GPT2_ABI_BEGIN
  if (!m) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "adamw: NULL model");
  if (t < 1) return gpt2_internal_fail(GPT2_E_STATE, "adamw: t must be >= 1");
  if (!m->have_grads) return gpt2_internal_fail(GPT2_E_STATE, "adamw needs a completed backward first");
  RC(set_adam_hparams(m->at<AdamHP>(m->lo.adam_hp), adam_hparams(lr, beta1, beta2, eps, weight_decay, t), m->stream));
  // the norm (and the clipping factor, read by the update on the device) only when asked for
  RC(update_impl(m, max_grad_norm, max_grad_norm > 0.f || grad_norm_out != nullptr));
  m->have_grads = false;
  if (grad_norm_out) {
    GPT2_HIP_CHECK(hipMemcpyAsync(grad_norm_out, m->at<float>(m->lo.gnorm), sizeof(float), hipMemcpyDeviceToHost,
                                  m->stream));
    GPT2_HIP_CHECK(hipStreamSynchronize(m->stream));
  }
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

int gpt2_graph_capture(gpt2_model* m, const int32_t* d_tokens, const int32_t* d_targets) {
  GPT2_ABI_BEGIN
  if (!m || !d_tokens || !d_targets)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "graph_capture: NULL model, tokens or targets");
  if (!m->stream)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "graph_capture: the model's stream is the null stream");
  if (any_timer_on(m)) return gpt2_internal_fail(GPT2_E_STATE, "graph_capture: disable timing sites first");
  graph_release(m);
  if (m->side_pending) {   // the last eager forward's key sort joins before the capture starts
    GPT2_HIP_CHECK(hipStreamWaitEvent(m->stream, m->ev_join, 0));
    m->side_pending = false;
  }
  GPT2_HIP_CHECK(hipStreamBeginCapture(m->stream, hipStreamCaptureModeThreadLocal));
  int rc = forward_impl(m, d_tokens, d_targets, 1.0f);
  if (!rc) rc = backward_impl(m, false);
  if (!rc) rc = update_impl(m, 0.0f, false);
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(m->stream, &g);
  m->side_pending = false;
  m->have_dlogits = m->have_grads = false;
  if (rc || e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    if (rc) return rc;
    return gpt2_internal_hip_fail(e, "hipStreamEndCapture", __FILE__, __LINE__);
  }
  m->graph = g;
  const hipError_t ei = hipGraphInstantiate(&m->graph_exec, g, nullptr, nullptr, 0);
  if (ei != hipSuccess) {
    graph_release(m);
    return gpt2_internal_hip_fail(ei, "hipGraphInstantiate", __FILE__, __LINE__);
  }
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

int gpt2_graph_step(gpt2_model* m, float lr, float beta1, float beta2, float eps, float weight_decay, int32_t t,
                    float* mean_loss) {
  GPT2_ABI_BEGIN
  if (!m) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "graph_step: NULL model");
  if (!m->graph_exec) return gpt2_internal_fail(GPT2_E_STATE, "graph_step: no captured step (gpt2_graph_capture)");
  if (t < 1) return gpt2_internal_fail(GPT2_E_STATE, "graph_step: t must be >= 1");
  if (m->side_pending) {
    GPT2_HIP_CHECK(hipStreamWaitEvent(m->stream, m->ev_join, 0));
    m->side_pending = false;
  }
  RC(set_adam_hparams(m->at<AdamHP>(m->lo.adam_hp), adam_hparams(lr, beta1, beta2, eps, weight_decay, t), m->stream));
  GPT2_HIP_CHECK(hipGraphLaunch(m->graph_exec, m->stream));
  m->have_dlogits = m->have_grads = false;
  if (mean_loss) {
    GPT2_HIP_CHECK(hipMemcpyAsync(mean_loss, m->at<float>(m->lo.mean_loss), sizeof(float), hipMemcpyDeviceToHost,
                                  m->stream));
    GPT2_HIP_CHECK(hipStreamSynchronize(m->stream));
  }
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

static int copy_out(gpt2_model* m, const void* src, void* dst, size_t bytes) {
  GPT2_HIP_CHECK(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, m->stream));
  GPT2_HIP_CHECK(hipStreamSynchronize(m->stream));
  return GPT2_OK;
}

int gpt2_get_mean_loss(gpt2_model* m, float* host_out) {
  GPT2_ABI_BEGIN
  if (!m || !host_out) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "get_mean_loss: NULL");
  return copy_out(m, m->at<float>(m->lo.mean_loss), host_out, sizeof(float));
  GPT2_ABI_END_STATUS
}

int gpt2_get_params(gpt2_model* m, float* host_out) {
  GPT2_ABI_BEGIN
  if (!m || !host_out) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "get_params: NULL");
  return copy_out(m, m->master(), host_out, m->lo.P * sizeof(float));
  GPT2_ABI_END_STATUS
}

int gpt2_set_params(gpt2_model* m, const float* host_in) {
  GPT2_ABI_BEGIN
  if (!m || !host_in) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "set_params: NULL");
  GPT2_HIP_CHECK(hipMemcpyAsync(m->master(), host_in, m->lo.P * sizeof(float), hipMemcpyHostToDevice, m->stream));
  RC(fill_f32(m->lo.P, m->at<float>(m->lo.adam_m), 0.f, m->stream));
  RC(fill_f32(m->lo.P, m->at<float>(m->lo.adam_v), 0.f, m->stream));
  RC(refresh_bf16(m));
  GPT2_HIP_CHECK(hipStreamSynchronize(m->stream));
  m->have_dlogits = m->have_grads = false;
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

int gpt2_get_grads(gpt2_model* m, float* host_out) {
  GPT2_ABI_BEGIN
  if (!m || !host_out) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "get_grads: NULL");
  return copy_out(m, m->grad(), host_out, m->lo.P * sizeof(float));
  GPT2_ABI_END_STATUS
}

int gpt2_get_adam_state(gpt2_model* m, float* host_m, float* host_v) {
  GPT2_ABI_BEGIN
  if (!m) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "get_adam_state: NULL");
  if (host_m) RC(copy_out(m, m->at<float>(m->lo.adam_m), host_m, m->lo.P * sizeof(float)));
  if (host_v) RC(copy_out(m, m->at<float>(m->lo.adam_v), host_v, m->lo.P * sizeof(float)));
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

int gpt2_get_token_losses(gpt2_model* m, float* host_out) {
  GPT2_ABI_BEGIN
  if (!m || !host_out) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "get_token_losses: NULL");
  return copy_out(m, m->at<float>(m->lo.losses), host_out,
                  (size_t)m->cfg.batch_size * m->cfg.seq_len * sizeof(float));
  GPT2_ABI_END_STATUS
}

int gpt2_get_logits(gpt2_model* m, float* host_out) {
  GPT2_ABI_BEGIN
  if (!m || !host_out) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "get_logits: NULL");
  const int64_t n = (int64_t)m->cfg.batch_size * m->cfg.seq_len * m->cfg.padded_vocab_size;
  if (m->cfg.dtype == GPT2_FP32) return copy_out(m, m->at<float>(m->lo.logits), host_out, n * sizeof(float));
  // convert through the scratch region chunk by chunk
  float* tmp = m->at<float>(m->lo.scratch);
  const int64_t chunk = (int64_t)(m->lo.scratch_bytes / sizeof(float)) / 4096 * 4096;
  if (chunk <= 0) return gpt2_internal_fail(GPT2_E_OOM, "get_logits: scratch too small");
  for (int64_t i = 0; i < n; i += chunk) {
    const int64_t k = std::min(chunk, n - i);
    RC(convert_to_f32(GPT2_BF16, k, m->at<bf16>(m->lo.logits) + i, tmp, m->stream));
    RC(copy_out(m, tmp, host_out + i, k * sizeof(float)));
  }
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

int gpt2_timing_enable(gpt2_model* m, int site, int enable) {
  GPT2_ABI_BEGIN
  if (!m || site < 0 || site >= S_COUNT) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "timing_enable: bad site");
  SiteTimer& t = m->timers[site];
  if (enable && t.ev.empty()) {
    grow(t.ev, 2 * 4096);
    for (auto& e : t.ev) GPT2_HIP_CHECK(hipEventCreate(&e));
  }
  t.on = enable != 0;
  t.used = 0;
  t.launches = 0;
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

int gpt2_timing_read(gpt2_model* m, int site, double* total_ms, int64_t* launches, double* flops_per_launch,
                     double* bytes_per_launch) {
  GPT2_ABI_BEGIN
  if (!m || site < 0 || site >= S_COUNT) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "timing_read: bad site");
  SiteTimer& t = m->timers[site];
  GPT2_HIP_CHECK(hipStreamSynchronize(m->stream));
  double tot = 0;
  for (size_t i = 0; i + 1 < t.used; i += 2) {
    float ms = 0;
    GPT2_HIP_CHECK(hipEventElapsedTime(&ms, t.ev[i], t.ev[i + 1]));
    tot += ms;
  }
  if (total_ms) *total_ms = tot;
  if (launches) *launches = t.launches;
  if (flops_per_launch) *flops_per_launch = t.flops;
  if (bytes_per_launch) *bytes_per_launch = t.bytes;
  t.used = 0;
  t.launches = 0;
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

// ================================================================ op-level ABI

int gpt2_op_linear_forward(int dtype, int M, int N, int K, const void* x, const void* W, const void* b,
                           const void* residual, void* y, void* gelu_grad, void* stream) {
  GPT2_ABI_BEGIN
  if (residual && gelu_grad) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "residual and gelu_grad are exclusive");
  if ((residual || gelu_grad) && !b)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "the residual and GELU epilogues need a bias");
  const int epi = gelu_grad ? EPI_BIAS_GELU_D : residual ? EPI_BIAS_RES : b ? EPI_BIAS : EPI_STORE;
  return gemm(linear_fwd_desc(dtype, M, N, K, x, W, epi, y, b, residual, gelu_grad), (hipStream_t)stream);
  GPT2_ABI_END_STATUS
}

size_t gpt2_op_linear_backward_workspace_bytes(int dtype, int M, int N, int K) {
  GPT2_ABI_BEGIN
  const bool wt = dtype == GPT2_BF16;
  return op_wt_bytes(dtype, N, K) + std::max(gemm_workspace_bytes(dtype, EPI_WGRAD, N, K, M, false, false),
                                             gemm_workspace_bytes(dtype, EPI_STORE, M, K, N, true, wt));
  GPT2_ABI_END(0)
}

int gpt2_op_linear_backward(int dtype, int M, int N, int K, const void* dy, const void* x, const void* W,
                            const void* gelu_grad, void* dx, float* dW, float* db, int accumulate, void* workspace,
                            size_t workspace_bytes, void* stream) {
  GPT2_ABI_BEGIN
  hipStream_t s = (hipStream_t)stream;
  if (db && !dW) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "db is computed in the dW pass; pass dW too");
  const size_t wtb = dx ? op_wt_bytes(dtype, N, K) : 0;
  const size_t need = gpt2_op_linear_backward_workspace_bytes(dtype, M, N, K);
  if ((dx || dW) && (!workspace || workspace_bytes < need))
    return gpt2_internal_fail(GPT2_E_OOM, "linear_backward: workspace of %zu bytes (need %zu)", workspace_bytes, need);
  char* ws = static_cast<char*>(workspace);
  if (dW)
    RC(gemm(linear_dw_desc(dtype, M, N, K, dy, x, dW, db, accumulate != 0, ws + wtb, workspace_bytes - wtb), s));
  if (dx) {
    void* WT = nullptr;
    if (wtb) {   // W [N, K] -> WT [K, N], the layout the step's dX products read
      if (!W) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "linear_backward: W is NULL");
      RC(transpose_bf16(1, N, K, static_cast<const bf16*>(W), reinterpret_cast<bf16*>(ws), s));
      WT = ws;
    }
    RC(gemm(linear_dx_desc(dtype, M, N, K, dy, W, WT, dx, gelu_grad ? EPI_MUL : EPI_STORE, gelu_grad, ws + wtb,
                           workspace_bytes - wtb),
            s));
  }
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

int gpt2_op_linear_plans(int dtype, int M, int N, int K, int has_bias, int has_residual, int has_gelu, int has_db,
                         gpt2_gemm_plan out[3]) {
  GPT2_ABI_BEGIN
  if (!out) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "linear_plans: out is NULL");
  // placeholders: planning reads shapes, epilogues and layouts, never memory
  void* const p = reinterpret_cast<void*>((uintptr_t)4096);
  const int epi = has_gelu ? EPI_BIAS_GELU_D : has_residual ? EPI_BIAS_RES : has_bias ? EPI_BIAS : EPI_STORE;
  fill_plan(linear_fwd_desc(dtype, M, N, K, p, p, epi, p, has_bias ? p : nullptr, has_residual ? p : nullptr,
                            has_gelu ? p : nullptr),
            "forward", &out[0]);
  fill_plan(linear_dw_desc(dtype, M, N, K, p, p, static_cast<float*>(p), has_db ? static_cast<float*>(p) : nullptr,
                           false, p, 0),
            "dW", &out[1]);
  fill_plan(linear_dx_desc(dtype, M, N, K, p, p, dtype == GPT2_BF16 ? p : nullptr, p, has_gelu ? EPI_MUL : EPI_STORE,
                           has_gelu ? p : nullptr, p, 0),
            "dX", &out[2]);
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

size_t gpt2_op_fp8_quantize_workspace_bytes(void) { return fp8_scale_workspace_bytes(); }

int gpt2_op_fp8_quantize(int in_dtype, int fmt, int R, int C, const void* x, float* scale, uint8_t* q, uint8_t* qt,
                         void* workspace, size_t workspace_bytes, void* stream) {
  GPT2_ABI_BEGIN
  if (!scale || !workspace || workspace_bytes < fp8_scale_workspace_bytes() || (uintptr_t)scale % 16)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "fp8_quantize: scale (16-byte aligned) and workspace needed");
  hipStream_t s = (hipStream_t)stream;
  Fp8Scale* sc = reinterpret_cast<Fp8Scale*>(scale);
  RC(fp8_amax(in_dtype, (int64_t)R * C, x, static_cast<float*>(workspace), s));
  return fp8_quantize(in_dtype, fmt, R, C, x, C, static_cast<const float*>(workspace), sc, q, qt, s);
  GPT2_ABI_END_STATUS
}

namespace {
// Workspace of the op-level fp8 linear layer: 4 scales, absmax partials, the
// codes of x, W (row-major and transposed) and dY (row-major: the weight
// gradient reads it and x's codes m-major), then the products' split-K /
// bias-gradient scratch.
struct OpFp8Ws {
  size_t scales, amax, xq, wq, wqt, dq, colsum, scratch, scratch_bytes, total;
};
OpFp8Ws op_fp8_ws(int M, int N, int K) {
  Plan p;
  OpFp8Ws w;
  w.scales = p.alloc(4 * sizeof(Fp8Scale));
  w.amax = p.alloc(fp8_scale_workspace_bytes());
  w.xq = p.alloc((size_t)M * K);
  w.wq = p.alloc((size_t)N * K);
  w.wqt = p.alloc((size_t)N * K);
  w.dq = p.alloc((size_t)M * N);
  w.colsum = p.alloc(fp8_colsum_bytes(M, N));
  w.scratch_bytes = std::max({gemm_workspace_bytes(GPT2_BF16, EPI_WGRAD, N, K, M, false, false, 2),
                              gemm_workspace_bytes(GPT2_BF16, EPI_STORE, M, K, N, true, true, 2),
                              gemm_workspace_bytes(GPT2_BF16, EPI_STORE, M, N, K, true, true, 1)});
  w.scratch = p.alloc(w.scratch_bytes);
  w.total = p.total;
  return w;
}
}  // namespace

size_t gpt2_op_linear_fp8_workspace_bytes(int M, int N, int K) {
  GPT2_ABI_BEGIN
  if (M < 0 || N < 0 || K < 0) return 0;
  return op_fp8_ws(M, N, K).total;
  GPT2_ABI_END(0)
}

int gpt2_op_linear_fp8_forward(int M, int N, int K, const void* x, const void* W, const void* b, const void* residual,
                               void* y, void* gelu_grad, void* workspace, size_t workspace_bytes, void* stream) {
  GPT2_ABI_BEGIN
  if (residual && gelu_grad) return gpt2_internal_fail(GPT2_E_INVALID_ARG, "residual and gelu_grad are exclusive");
  if ((residual || gelu_grad) && !b)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "the residual and GELU epilogues need a bias");
  if (!x || !W || !y || M <= 0 || N <= 0 || K <= 0 || K % 16 || N % 16)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "linear_fp8_forward: bad arguments (K, N multiples of 16)");
  const OpFp8Ws w = op_fp8_ws(M, N, K);
  if (!workspace || workspace_bytes < w.total)
    return gpt2_internal_fail(GPT2_E_OOM, "linear_fp8_forward: workspace of %zu bytes (need %zu)", workspace_bytes,
                              w.total);
  hipStream_t s = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  Fp8Scale* sc = reinterpret_cast<Fp8Scale*>(ws + w.scales);
  float* amax = reinterpret_cast<float*>(ws + w.amax);
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + w.xq);
  uint8_t* wq = reinterpret_cast<uint8_t*>(ws + w.wq);
  RC(fp8_amax(GPT2_BF16, (int64_t)M * K, x, amax, s));
  RC(fp8_quantize(GPT2_BF16, 0, M, K, x, K, amax, &sc[0], xq, nullptr, s));
  RC(fp8_amax(GPT2_BF16, (int64_t)N * K, W, amax, s));
  RC(fp8_quantize(GPT2_BF16, 0, N, K, W, K, amax, &sc[1], wq, nullptr, s));
  const int epi = gelu_grad ? EPI_BIAS_GELU_D : residual ? EPI_BIAS_RES : b ? EPI_BIAS : EPI_STORE;
  GemmDesc d = linear_fwd_desc(GPT2_BF16, M, N, K, xq, wq, epi, y, b, residual, gelu_grad);
  d.fp8 = 1;
  d.scale_a = &sc[0].s; d.scale_b = &sc[1].s;
  d.workspace = ws + w.scratch; d.workspace_bytes = w.scratch_bytes;
  return gemm(d, s);
  GPT2_ABI_END_STATUS
}

int gpt2_op_linear_fp8_backward(int M, int N, int K, const void* dy, const void* x, const void* W,
                                const void* gelu_grad, void* dx, float* dW, float* db, int accumulate, void* workspace,
                                size_t workspace_bytes, void* stream) {
  GPT2_ABI_BEGIN
  if (!dy || M <= 0 || N <= 0 || K <= 0 || K % 16 || N % 16 || M % 16 || (dW && !x) || (dx && !W) || (db && !dW))
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "linear_fp8_backward: bad arguments (M, N, K multiples of 16)");
  const OpFp8Ws w = op_fp8_ws(M, N, K);
  if (!workspace || workspace_bytes < w.total)
    return gpt2_internal_fail(GPT2_E_OOM, "linear_fp8_backward: workspace of %zu bytes (need %zu)", workspace_bytes,
                              w.total);
  hipStream_t s = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  Fp8Scale* sc = reinterpret_cast<Fp8Scale*>(ws + w.scales);
  float* amax = reinterpret_cast<float*>(ws + w.amax);
  uint8_t* dq = reinterpret_cast<uint8_t*>(ws + w.dq);
  RC(fp8_amax(GPT2_BF16, (int64_t)M * N, dy, amax, s));
  float* colsum = db ? reinterpret_cast<float*>(ws + w.colsum) : nullptr;
  RC(fp8_quantize(GPT2_BF16, 1, M, N, dy, N, amax, &sc[2], dq, nullptr, s, colsum));
  if (dW) {   // as the training step: both operands' row-major codes, read m-major
    uint8_t* xq = reinterpret_cast<uint8_t*>(ws + w.xq);
    RC(fp8_amax(GPT2_BF16, (int64_t)M * K, x, amax, s));
    RC(fp8_quantize(GPT2_BF16, 0, M, K, x, K, amax, &sc[0], xq, nullptr, s));
    GemmDesc d = gdesc(GPT2_BF16);
    d.a_kmajor = d.b_kmajor = false;
    d.M = N; d.N = K; d.K = M;
    d.A = dq; d.lda = N; d.B = xq; d.ldb = K;
    d.epi = EPI_WGRAD; d.out32 = dW; d.accumulate = accumulate != 0;
    d.workspace = ws + w.scratch; d.workspace_bytes = w.scratch_bytes;
    d.fp8 = 2; d.scale_a = &sc[2].s; d.scale_b = &sc[0].s;
    RC(gemm(d, s));
    if (db) RC(colsum_reduce(M, N, colsum, db, accumulate != 0, s));
  }
  if (dx) {
    uint8_t* wqt = reinterpret_cast<uint8_t*>(ws + w.wqt);
    RC(fp8_amax(GPT2_BF16, (int64_t)N * K, W, amax, s));
    RC(fp8_quantize(GPT2_BF16, 0, N, K, W, K, amax, &sc[1], nullptr, wqt, s));
    GemmDesc d = linear_dx_desc(GPT2_BF16, M, N, K, dq, nullptr, wqt, dx, gelu_grad ? EPI_MUL : EPI_STORE, gelu_grad,
                                ws + w.scratch, w.scratch_bytes);
    d.fp8 = 2; d.scale_a = &sc[2].s; d.scale_b = &sc[1].s;
    RC(gemm(d, s));
  }
  return GPT2_OK;
  GPT2_ABI_END_STATUS
}

int gpt2_op_layernorm_forward(int dtype, int N, int C, const void* x, const void* w, const void* b, void* y,
                              float* mean, float* rstd, void* stream) {
  GPT2_ABI_BEGIN
  return layernorm_forward(dtype, N, C, x, w, b, y, mean, rstd, (hipStream_t)stream);
  GPT2_ABI_END_STATUS
}

size_t gpt2_op_layernorm_backward_workspace_bytes(int N, int C) { return layernorm_backward_workspace_bytes(N, C); }

int gpt2_op_layernorm_backward(int dtype, int N, int C, const void* dy, const void* x, const void* w,
                               const float* mean, const float* rstd, float* dres, int dres_overwrite,
                               void* dres_copy, float* dw, float* db, int accumulate, void* workspace,
                               size_t workspace_bytes, void* stream) {
  GPT2_ABI_BEGIN
  return layernorm_backward(dtype, N, C, dy, x, w, mean, rstd, dres, dres_overwrite != 0, dres_copy, dw, db,
                            accumulate != 0, workspace, workspace_bytes, (hipStream_t)stream);
  GPT2_ABI_END_STATUS
}

int gpt2_op_attention_forward(int dtype, int B, int T, int H, int hd, const void* qkv, void* out, float* lse,
                              void* stream) {
  GPT2_ABI_BEGIN
  return attention_forward(dtype, B, T, H, hd, qkv, out, lse, (hipStream_t)stream);
  GPT2_ABI_END_STATUS
}

size_t gpt2_op_attention_backward_workspace_bytes(int B, int T, int H, int hd) {
  return attention_backward_workspace_bytes(B, T, H, hd);
}

int gpt2_op_attention_backward(int dtype, int B, int T, int H, int hd, const void* qkv, const void* out,
                               const void* dout, const float* lse, void* dqkv, void* workspace,
                               size_t workspace_bytes, void* stream) {
  GPT2_ABI_BEGIN
  return attention_backward(dtype, B, T, H, hd, qkv, out, dout, lse, dqkv, workspace, workspace_bytes,
                            (hipStream_t)stream);
  GPT2_ABI_END_STATUS
}

int gpt2_op_softmax_xent(int dtype, int N, int V, int Vp, void* logits, const int32_t* labels, float* losses,
                         float dscale, void* stream) {
  GPT2_ABI_BEGIN
  return softmax_xent(dtype, N, V, Vp, logits, labels, losses, dscale, (hipStream_t)stream);
  GPT2_ABI_END_STATUS
}

size_t gpt2_op_classifier_workspace_bytes(int dtype, int N, int C, int Vp) {
  return gpt2_op_linear_backward_workspace_bytes(dtype, N, Vp, C);
}

int gpt2_op_classifier_fwd_bwd(int dtype, int N, int C, int V, int Vp, const void* hidden, const void* wte,
                               const int32_t* labels, float* losses, void* logits, void* d_hidden, float* d_wte,
                               void* workspace, size_t workspace_bytes, void* stream) {
  GPT2_ABI_BEGIN
  if (N <= 0 || C <= 0 || V <= 0 || Vp < V || !hidden || !wte || !labels || !losses || !logits || !d_hidden || !d_wte)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "classifier: bad arguments");
  hipStream_t s = (hipStream_t)stream;
  RC(gpt2_op_linear_forward(dtype, N, Vp, C, hidden, wte, nullptr, nullptr, logits, nullptr, stream));
  RC(softmax_xent(dtype, N, V, Vp, logits, labels, losses, 1.0f / N, s));
  // d_hidden = dlogits wte, d_wte = dlogits^T hidden: a linear backward with W = wte [Vp, C]
  return gpt2_op_linear_backward(dtype, N, Vp, C, logits, hidden, wte, nullptr, d_hidden, d_wte, nullptr, 0,
                                 workspace, workspace_bytes, stream);
  GPT2_ABI_END_STATUS
}

int gpt2_op_encoder_forward(int dtype, int B, int T, int C, int V, const int32_t* tokens, const void* wte,
                            const void* wpe, void* out, void* stream) {
  GPT2_ABI_BEGIN
  return encoder_forward(dtype, B, T, C, V, tokens, wte, wpe, out, (hipStream_t)stream);
  GPT2_ABI_END_STATUS
}

size_t gpt2_op_encoder_backward_workspace_bytes(int B, int T, int C) {
  return encoder_backward_workspace_bytes(B, T, C);
}

int gpt2_op_encoder_backward(int B, int T, int C, int V, const int32_t* tokens, const float* dx0, float* dwte,
                             float* dwpe, int accumulate_wpe, void* workspace, size_t workspace_bytes, void* stream) {
  GPT2_ABI_BEGIN
  return encoder_backward(B, T, C, V, tokens, dx0, dwte, dwpe, accumulate_wpe != 0, workspace, workspace_bytes,
                          (hipStream_t)stream);
  GPT2_ABI_END_STATUS
}

int gpt2_op_adamw(int64_t n, float* master, const float* grad, float* m, float* v, void* param_bf16, float lr,
                  float beta1, float beta2, float eps, float weight_decay, int32_t t, void* stream) {
  GPT2_ABI_BEGIN
  return adamw(n, master, grad, m, v, (bf16*)param_bf16, lr, beta1, beta2, eps, weight_decay, t,
               (hipStream_t)stream);
  GPT2_ABI_END_STATUS
}

}  // extern "C"
