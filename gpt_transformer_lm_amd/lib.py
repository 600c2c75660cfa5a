"""ctypes binding of libgpt2_hip.so (the C ABI in include/gpt2.h and
include/gpt2_ops.h).  Argument marshalling only: every step of the training
step runs in the library's HIP kernels.  torch supplies device memory
(tensors' data pointers) and streams.

Loading fails loudly if the library has not been built; there is no fallback.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt2_hip.so")

GPT2_FP32 = 0
GPT2_BF16 = 1
GPT2_BF16_FP8 = 2

SITES = ["qkv", "attproj", "fc", "fcproj", "logits", "fcproj_dx", "fcproj_dw", "fc_dx", "fc_dw",
         "attproj_dx", "attproj_dw", "qkv_dx", "qkv_dw", "cls_dx", "cls_dw", "attn_fwd", "attn_bwd_dkdv",
         "attn_bwd_dq", "attn_bwd_dot", "softmax_xent", "ln_fwd", "ln_bwd", "encoder_fwd", "adamw",
         "weight_transpose", "grad_norm", "qk_fwd", "qk_bwd", "fp8_quant"]


GPT2_ARCH_RELU2 = 1
GPT2_ARCH_QK_NORM = 2
GPT2_ARCH_ROPE = 4

EPILOGUES = {0: "store", 1: "bias", 2: "bias+residual", 3: "bias+relu2", 5: "wgrad", 6: "bias+gelu", 7: "mul"}


class Gpt2Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "vocab_size", "padded_vocab_size", "max_seq_len", "num_layers", "num_heads", "channels",
        "batch_size", "seq_len", "dtype", "arch_flags")]


class GemmPlan(C.Structure):
    _fields_ = [("site", C.c_char * 16)] + [(n, C.c_int32) for n in (
        "M", "N", "K", "epilogue", "a_kmajor", "b_kmajor", "tile_m", "tile_n", "waves", "k_groups", "k_splits",
        "bias_grad", "fp8")]

    def as_dict(self):
        d = {n: getattr(self, n) for n, _ in self._fields_[1:]}
        d["site"] = self.site.decode()
        return d


class Gpt2Error(RuntimeError):
    pass


_lib = None


def load():
    """Loads the shared library (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise Gpt2Error(f"{LIB_PATH} is missing: build it first (python -m gpt_transformer_lm_amd.build)")
    # torch first: its wheel carries its own HIP runtime (same soname as the
    # system one the library is linked against).  Loaded after torch, the
    # library binds to torch's runtime, so device pointers and streams are
    # shared; loaded before, a second runtime would be mapped beside torch's
    # and the library's kernels would not see torch's device state.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float
    cfgp = C.POINTER(Gpt2Config)
    fp = C.POINTER(C.c_float)
    sig = {
        "gpt2_validate_config": (C.c_int, [cfgp]),
        "gpt2_num_parameters": (i64, [cfgp, C.c_int]),
        "gpt2_num_param_tensors": (C.c_int, []),
        "gpt2_param_info": (C.c_int, [cfgp, C.c_int, C.POINTER(C.c_char_p), C.POINTER(i64),
                                      C.POINTER(i64), C.POINTER(i32)]),
        "gpt2_workspace_bytes": (sz, [cfgp]),
        "gpt2_status_string": (C.c_char_p, [C.c_int]),
        "gpt2_last_error": (C.c_char_p, []),
        "gpt2_test_fail_host_allocations": (C.c_int, [C.c_int]),
        "gpt2_step_gemm_plans": (C.c_int, [cfgp, C.POINTER(GemmPlan), C.c_int, C.POINTER(C.c_int)]),
        "gpt2_op_linear_plans": (C.c_int, [C.c_int] * 8 + [C.POINTER(GemmPlan)]),
        "gpt2_graph_capture": (C.c_int, [vp, vp, vp]),
        "gpt2_graph_step": (C.c_int, [vp, f32, f32, f32, f32, f32, i32, fp]),
        "gpt2_create": (C.c_int, [cfgp, C.c_uint64, vp, vp, sz, C.POINTER(vp)]),
        "gpt2_forward": (C.c_int, [vp, vp, vp, fp]),
        "gpt2_forward_scaled": (C.c_int, [vp, vp, vp, f32, fp]),
        "gpt2_backward": (C.c_int, [vp]),
        "gpt2_backward_accumulate": (C.c_int, [vp]),
        "gpt2_adamw_step": (C.c_int, [vp, f32, f32, f32, f32, f32, i32]),
        "gpt2_adamw_step_clipped": (C.c_int, [vp, f32, f32, f32, f32, f32, i32, f32, fp]),
        "gpt2_destroy": (None, [vp]),
        "gpt2_get_mean_loss": (C.c_int, [vp, fp]),
        "gpt2_get_params": (C.c_int, [vp, vp]),
        "gpt2_set_params": (C.c_int, [vp, vp]),
        "gpt2_get_grads": (C.c_int, [vp, vp]),
        "gpt2_get_adam_state": (C.c_int, [vp, vp, vp]),
        "gpt2_get_token_losses": (C.c_int, [vp, vp]),
        "gpt2_get_logits": (C.c_int, [vp, vp]),
        "gpt2_timing_enable": (C.c_int, [vp, C.c_int, C.c_int]),
        "gpt2_timing_read": (C.c_int, [vp, C.c_int, C.POINTER(C.c_double), C.POINTER(i64),
                                       C.POINTER(C.c_double), C.POINTER(C.c_double)]),
        "gpt2_op_linear_forward": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, vp, vp, vp, vp, vp, vp, vp]),
        "gpt2_op_linear_backward_workspace_bytes": (sz, [C.c_int, C.c_int, C.c_int, C.c_int]),
        "gpt2_op_linear_backward": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, vp, vp, vp, vp, vp, vp, vp,
                                              C.c_int, vp, sz, vp]),
        "gpt2_op_fp8_quantize_workspace_bytes": (sz, []),
        "gpt2_op_fp8_quantize": (C.c_int, [C.c_int] * 4 + [vp] * 4 + [vp, sz, vp]),
        "gpt2_op_linear_fp8_workspace_bytes": (sz, [C.c_int] * 3),
        "gpt2_op_linear_fp8_forward": (C.c_int, [C.c_int] * 3 + [vp] * 7 + [sz, vp]),
        "gpt2_op_linear_fp8_backward": (C.c_int, [C.c_int] * 3 + [vp] * 7 + [C.c_int, vp, sz, vp]),
        "gpt2_op_layernorm_forward": (C.c_int, [C.c_int, C.c_int, C.c_int, vp, vp, vp, vp, vp, vp, vp]),
        "gpt2_op_layernorm_backward_workspace_bytes": (sz, [C.c_int, C.c_int]),
        "gpt2_op_layernorm_backward": (C.c_int, [C.c_int, C.c_int, C.c_int, vp, vp, vp, vp, vp, vp, C.c_int, vp,
                                                 vp, vp, C.c_int, vp, sz, vp]),
        "gpt2_op_attention_forward": (C.c_int, [C.c_int] * 5 + [vp, vp, vp, vp]),
        "gpt2_op_attention_backward_workspace_bytes": (sz, [C.c_int] * 4),
        "gpt2_op_attention_backward": (C.c_int, [C.c_int] * 5 + [vp, vp, vp, vp, vp, vp, sz, vp]),
        "gpt2_op_attention_backward_noalloc": (C.c_int, [C.c_int] * 5 + [vp, vp, vp, vp, vp, vp]),
        "gpt2_op_softmax_xent": (C.c_int, [C.c_int] * 4 + [vp, vp, vp, f32, vp]),
        "gpt2_op_classifier_workspace_bytes": (sz, [C.c_int] * 4),
        "gpt2_op_classifier_fwd_bwd": (C.c_int, [C.c_int] * 5 + [vp] * 7 + [vp, sz, vp]),
        "gpt2_op_encoder_forward": (C.c_int, [C.c_int] * 5 + [vp, vp, vp, vp, vp]),
        "gpt2_op_encoder_backward_workspace_bytes": (sz, [C.c_int] * 3),
        "gpt2_op_encoder_backward": (C.c_int, [C.c_int] * 4 + [vp, vp, vp, vp, C.c_int, vp, sz, vp]),
        "gpt2_op_adamw": (C.c_int, [i64, vp, vp, vp, vp, vp, f32, f32, f32, f32, f32, i32, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols():
    """Names every header declares (checked against the library's exports)."""
    return [
        "gpt2_validate_config", "gpt2_num_parameters", "gpt2_num_param_tensors", "gpt2_param_info",
        "gpt2_workspace_bytes", "gpt2_status_string", "gpt2_last_error", "gpt2_test_fail_host_allocations",
        "gpt2_graph_capture", "gpt2_graph_step", "gpt2_step_gemm_plans", "gpt2_op_linear_plans",
        "gpt2_create", "gpt2_forward",
        "gpt2_forward_scaled", "gpt2_backward", "gpt2_backward_accumulate", "gpt2_adamw_step",
        "gpt2_adamw_step_clipped", "gpt2_destroy", "gpt2_get_mean_loss", "gpt2_get_params", "gpt2_set_params",
        "gpt2_get_grads", "gpt2_get_adam_state", "gpt2_get_token_losses", "gpt2_get_logits",
        "gpt2_timing_enable", "gpt2_timing_read",
        "gpt2_op_linear_forward", "gpt2_op_linear_backward_workspace_bytes", "gpt2_op_linear_backward",
        "gpt2_op_fp8_quantize_workspace_bytes", "gpt2_op_fp8_quantize", "gpt2_op_linear_fp8_workspace_bytes",
        "gpt2_op_linear_fp8_forward", "gpt2_op_linear_fp8_backward",
        "gpt2_op_layernorm_forward", "gpt2_op_layernorm_backward_workspace_bytes",
        "gpt2_op_layernorm_backward", "gpt2_op_attention_forward",
        "gpt2_op_attention_backward_workspace_bytes", "gpt2_op_attention_backward",
        "gpt2_op_attention_backward_noalloc",
        "gpt2_op_softmax_xent", "gpt2_op_classifier_workspace_bytes", "gpt2_op_classifier_fwd_bwd",
        "gpt2_op_encoder_forward", "gpt2_op_encoder_backward_workspace_bytes",
        "gpt2_op_encoder_backward", "gpt2_op_adamw",
    ]


def check(rc: int, what: str = ""):
    if rc != 0:
        lib = load()
        msg = lib.gpt2_last_error().decode(errors="replace")
        raise Gpt2Error(f"{what}: {lib.gpt2_status_string(rc).decode()} ({rc}): {msg}")


def make_config(V, Vp, maxT, L, H, C_, B, T, dtype, arch_flags=0) -> Gpt2Config:
    return Gpt2Config(V, Vp, maxT, L, H, C_, B, T, dtype, arch_flags)


def step_gemm_plans(cfg: Gpt2Config):
    """Every GEMM launch of one training step of cfg (host-only query)."""
    lib = load()
    n = C.c_int()
    check(lib.gpt2_step_gemm_plans(C.byref(cfg), None, 0, C.byref(n)), "step_gemm_plans")
    out = (GemmPlan * max(n.value, 1))()
    check(lib.gpt2_step_gemm_plans(C.byref(cfg), out, n.value, C.byref(n)), "step_gemm_plans")
    return [out[i].as_dict() for i in range(n.value)]


def op_linear_plans(dtype, M, N, K, bias=False, residual=False, gelu=False, db=False):
    """The GEMM launches of gpt2_op_linear_forward / _backward: forward, dW, dX."""
    out = (GemmPlan * 3)()
    check(load().gpt2_op_linear_plans(dtype, M, N, K, int(bias), int(residual), int(gelu), int(db), out),
          "op_linear_plans")
    return [out[i].as_dict() for i in range(3)]


def param_layout(cfg: Gpt2Config):
    """[(name, offset, shape)] of the flat parameter array, from the library."""
    lib = load()
    out = []
    for i in range(lib.gpt2_num_param_tensors()):
        name = C.c_char_p()
        off = C.c_int64()
        shape = (C.c_int64 * 3)()
        nd = C.c_int32()
        check(lib.gpt2_param_info(C.byref(cfg), i, C.byref(name), C.byref(off), shape, C.byref(nd)), "param_info")
        out.append((name.value.decode(), off.value, tuple(shape[: nd.value])))
    return out


def flatten_params(cfg: Gpt2Config, params: dict) -> np.ndarray:
    """Packs name -> array into the library's flat float32 layout."""
    lib = load()
    flat = np.zeros(lib.gpt2_num_parameters(C.byref(cfg), 1), dtype=np.float32)
    for name, off, shape in param_layout(cfg):
        n = int(np.prod(shape))
        a = np.asarray(params[name], dtype=np.float32).reshape(-1)
        assert a.size == n, (name, a.size, n)
        flat[off:off + n] = a
    return flat


def unflatten(cfg: Gpt2Config, flat: np.ndarray) -> dict:
    return {name: flat[off:off + int(np.prod(shape))].reshape(shape).copy()
            for name, off, shape in param_layout(cfg)}


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


class Model:
    """One GPT-2 model instance on the current HIP device."""

    def __init__(self, cfg: Gpt2Config, seed: int = 0, stream=None, workspace=None):
        import torch
        self.lib = load()
        self.cfg = cfg
        check(self.lib.gpt2_validate_config(C.byref(cfg)), "validate_config")
        self.nparams = self.lib.gpt2_num_parameters(C.byref(cfg), 1)
        self.ws_bytes = self.lib.gpt2_workspace_bytes(C.byref(cfg))
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        if workspace is None:
            workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.workspace = workspace
        h = C.c_void_p()
        check(self.lib.gpt2_create(C.byref(cfg), C.c_uint64(seed), C.c_void_p(self.stream.cuda_stream),
                                   ptr(workspace), C.c_size_t(workspace.numel()), C.byref(h)), "create")
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            self.lib.gpt2_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward(self, tokens, targets=None, read_loss=True):
        """Mean loss with targets (read back, synchronising) unless read_loss is
        False; then nothing waits and get_mean_loss() reads it later."""
        loss = C.c_float(0.0)
        want = targets is not None and read_loss
        check(self.lib.gpt2_forward(self.h, ptr(tokens), ptr(targets), C.byref(loss) if want else None), "forward")
        return loss.value if want else None

    def graph_capture(self, tokens, targets):
        """Captures one training step reading ids from these device buffers."""
        check(self.lib.gpt2_graph_capture(self.h, ptr(tokens), ptr(targets)), "graph_capture")

    def graph_step(self, lr, beta1, beta2, eps, weight_decay, t, read_loss=True):
        loss = C.c_float(0.0)
        check(self.lib.gpt2_graph_step(self.h, lr, beta1, beta2, eps, weight_decay, t,
                                       C.byref(loss) if read_loss else None), "graph_step")
        return loss.value if read_loss else None

    def get_mean_loss(self):
        loss = C.c_float(0.0)
        check(self.lib.gpt2_get_mean_loss(self.h, C.byref(loss)), "get_mean_loss")
        return loss.value

    def forward_scaled(self, tokens, targets, loss_scale):
        loss = C.c_float(0.0)
        check(self.lib.gpt2_forward_scaled(self.h, ptr(tokens), ptr(targets), loss_scale, C.byref(loss)),
              "forward_scaled")
        return loss.value if targets is not None else None

    def backward(self):
        check(self.lib.gpt2_backward(self.h), "backward")

    def backward_accumulate(self):
        check(self.lib.gpt2_backward_accumulate(self.h), "backward_accumulate")

    def adamw_step(self, lr, beta1, beta2, eps, weight_decay, t):
        check(self.lib.gpt2_adamw_step(self.h, lr, beta1, beta2, eps, weight_decay, t), "adamw_step")

    def adamw_step_clipped(self, lr, beta1, beta2, eps, weight_decay, t, max_grad_norm, want_norm=True):
        norm = C.c_float(0.0)
        check(self.lib.gpt2_adamw_step_clipped(self.h, lr, beta1, beta2, eps, weight_decay, t, max_grad_norm,
                                               C.byref(norm) if want_norm else None), "adamw_step_clipped")
        return norm.value if want_norm else None

    def _host(self, fn, n):
        out = np.empty(n, dtype=np.float32)
        check(fn(self.h, out.ctypes.data_as(C.c_void_p)), fn.__name__)
        return out

    def get_params(self):
        return self._host(self.lib.gpt2_get_params, self.nparams)

    def set_params(self, flat):
        flat = np.ascontiguousarray(flat, dtype=np.float32)
        assert flat.size == self.nparams
        check(self.lib.gpt2_set_params(self.h, flat.ctypes.data_as(C.c_void_p)), "set_params")

    def get_grads(self):
        return self._host(self.lib.gpt2_get_grads, self.nparams)

    def get_adam_state(self):
        m = np.empty(self.nparams, dtype=np.float32)
        v = np.empty(self.nparams, dtype=np.float32)
        check(self.lib.gpt2_get_adam_state(self.h, m.ctypes.data_as(C.c_void_p), v.ctypes.data_as(C.c_void_p)),
              "get_adam_state")
        return m, v

    def get_token_losses(self):
        return self._host(self.lib.gpt2_get_token_losses, self.cfg.batch_size * self.cfg.seq_len)

    def get_logits(self):
        n = self.cfg.batch_size * self.cfg.seq_len * self.cfg.padded_vocab_size
        return self._host(self.lib.gpt2_get_logits, n).reshape(
            self.cfg.batch_size, self.cfg.seq_len, self.cfg.padded_vocab_size)

    def timing_enable(self, site: str, on: bool = True):
        check(self.lib.gpt2_timing_enable(self.h, SITES.index(site), int(on)), "timing_enable")

    def timing_read(self, site: str):
        ms, n = C.c_double(), C.c_int64()
        fl, by = C.c_double(), C.c_double()
        check(self.lib.gpt2_timing_read(self.h, SITES.index(site), C.byref(ms), C.byref(n), C.byref(fl),
                                        C.byref(by)), "timing_read")
        return dict(total_ms=ms.value, launches=n.value, flops_per_launch=fl.value, bytes_per_launch=by.value)


# ---------------------------------------------------------------- op-level calls

def _ws(nbytes):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device="cuda")


def linear_forward(dtype, x, W, b=None, residual=None, gelu_grad=None, y=None, stream=None):
    M, K = x.shape
    N = W.shape[0]
    check(load().gpt2_op_linear_forward(dtype, M, N, K, ptr(x), ptr(W), ptr(b), ptr(residual), ptr(y),
                                        ptr(gelu_grad), _stream_ptr(stream)), "linear_forward")


def linear_backward(dtype, dy, x, W, dx=None, dW=None, db=None, gelu_grad=None, accumulate=False, stream=None):
    lib = load()
    M, N = dy.shape
    K = x.shape[1]
    ws = _ws(lib.gpt2_op_linear_backward_workspace_bytes(dtype, M, N, K))
    check(lib.gpt2_op_linear_backward(dtype, M, N, K, ptr(dy), ptr(x), ptr(W), ptr(gelu_grad), ptr(dx), ptr(dW),
                                      ptr(db), int(accumulate), ptr(ws), ws.numel(), _stream_ptr(stream)),
          "linear_backward")
    return ws


def fp8_quantize(in_dtype, fmt, x, scale, q=None, qt=None, stream=None):
    lib = load()
    R, Cc = x.shape
    ws = _ws(lib.gpt2_op_fp8_quantize_workspace_bytes())
    check(lib.gpt2_op_fp8_quantize(in_dtype, fmt, R, Cc, ptr(x), ptr(scale), ptr(q), ptr(qt), ptr(ws), ws.numel(),
                                   _stream_ptr(stream)), "fp8_quantize")
    return ws


def linear_fp8_forward(x, W, b=None, residual=None, gelu_grad=None, y=None, stream=None):
    lib = load()
    M, K = x.shape
    N = W.shape[0]
    ws = _ws(lib.gpt2_op_linear_fp8_workspace_bytes(M, N, K))
    check(lib.gpt2_op_linear_fp8_forward(M, N, K, ptr(x), ptr(W), ptr(b), ptr(residual), ptr(y), ptr(gelu_grad),
                                         ptr(ws), ws.numel(), _stream_ptr(stream)), "linear_fp8_forward")
    return ws


def linear_fp8_backward(dy, x, W, dx=None, dW=None, db=None, gelu_grad=None, accumulate=False, stream=None):
    lib = load()
    M, N = dy.shape
    K = x.shape[1]
    ws = _ws(lib.gpt2_op_linear_fp8_workspace_bytes(M, N, K))
    check(lib.gpt2_op_linear_fp8_backward(M, N, K, ptr(dy), ptr(x), ptr(W), ptr(gelu_grad), ptr(dx), ptr(dW), ptr(db),
                                          int(accumulate), ptr(ws), ws.numel(), _stream_ptr(stream)),
          "linear_fp8_backward")
    return ws


def layernorm_forward(dtype, x, w, b, y, mean, rstd, stream=None):
    N, Cc = x.shape
    check(load().gpt2_op_layernorm_forward(dtype, N, Cc, ptr(x), ptr(w), ptr(b), ptr(y), ptr(mean), ptr(rstd),
                                           _stream_ptr(stream)), "layernorm_forward")


def layernorm_backward(dtype, dy, x, w, mean, rstd, dres, dres_overwrite, dres_copy, dw, db, accumulate=False,
                       stream=None):
    lib = load()
    N, Cc = dy.shape
    ws = _ws(lib.gpt2_op_layernorm_backward_workspace_bytes(N, Cc))
    check(lib.gpt2_op_layernorm_backward(dtype, N, Cc, ptr(dy), ptr(x), ptr(w), ptr(mean), ptr(rstd), ptr(dres),
                                         int(dres_overwrite), ptr(dres_copy), ptr(dw), ptr(db), int(accumulate),
                                         ptr(ws), ws.numel(), _stream_ptr(stream)), "layernorm_backward")
    return ws


def attention_forward(dtype, B, T, H, hd, qkv, out, lse, stream=None):
    check(load().gpt2_op_attention_forward(dtype, B, T, H, hd, ptr(qkv), ptr(out), ptr(lse), _stream_ptr(stream)),
          "attention_forward")


def attention_backward(dtype, B, T, H, hd, qkv, out, dout, lse, dqkv, stream=None):
    lib = load()
    ws = _ws(lib.gpt2_op_attention_backward_workspace_bytes(B, T, H, hd))
    check(lib.gpt2_op_attention_backward(dtype, B, T, H, hd, ptr(qkv), ptr(out), ptr(dout), ptr(lse), ptr(dqkv),
                                         ptr(ws), ws.numel(), _stream_ptr(stream)), "attention_backward")
    return ws


def attention_backward_noalloc(dtype, B, T, H, hd, qkv, out, dout, lse, dqkv, stream=None):
    check(load().gpt2_op_attention_backward_noalloc(dtype, B, T, H, hd, ptr(qkv), ptr(out), ptr(dout), ptr(lse),
                                                    ptr(dqkv), _stream_ptr(stream)), "attention_backward_noalloc")


def softmax_xent(dtype, logits, labels, losses, V, dscale, stream=None):
    N, Vp = logits.shape
    check(load().gpt2_op_softmax_xent(dtype, N, V, Vp, ptr(logits), ptr(labels), ptr(losses), dscale,
                                      _stream_ptr(stream)), "softmax_xent")


def classifier_fwd_bwd(dtype, hidden, wte, labels, V, losses, logits, d_hidden, d_wte, stream=None):
    lib = load()
    N, Cc = hidden.shape
    Vp = wte.shape[0]
    ws = _ws(lib.gpt2_op_classifier_workspace_bytes(dtype, N, Cc, Vp))
    check(lib.gpt2_op_classifier_fwd_bwd(dtype, N, Cc, V, Vp, ptr(hidden), ptr(wte), ptr(labels), ptr(losses),
                                         ptr(logits), ptr(d_hidden), ptr(d_wte), ptr(ws), ws.numel(),
                                         _stream_ptr(stream)), "classifier_fwd_bwd")
    return ws


def encoder_forward(dtype, tokens, wte, wpe, out, V, stream=None):
    B, T = tokens.shape
    Cc = wte.shape[1]
    check(load().gpt2_op_encoder_forward(dtype, B, T, Cc, V, ptr(tokens), ptr(wte), ptr(wpe), ptr(out),
                                         _stream_ptr(stream)), "encoder_forward")


def encoder_backward(tokens, dx0, dwte, dwpe, V, accumulate_wpe=False, stream=None):
    lib = load()
    B, T = tokens.shape
    Cc = dx0.shape[-1]
    ws = _ws(lib.gpt2_op_encoder_backward_workspace_bytes(B, T, Cc))
    check(lib.gpt2_op_encoder_backward(B, T, Cc, V, ptr(tokens), ptr(dx0), ptr(dwte), ptr(dwpe),
                                       int(accumulate_wpe), ptr(ws), ws.numel(), _stream_ptr(stream)),
          "encoder_backward")
    return ws


def adamw(master, grad, m, v, param_bf16, lr, beta1, beta2, eps, wd, t, stream=None):
    check(load().gpt2_op_adamw(master.numel(), ptr(master), ptr(grad), ptr(m), ptr(v), ptr(param_bf16), lr, beta1,
                               beta2, eps, wd, t, _stream_ptr(stream)), "adamw")
