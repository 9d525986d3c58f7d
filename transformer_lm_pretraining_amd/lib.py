"""ctypes binding of libgpt2mi (include/gpt2mi.h, include/gpt2mi_kernels.h).

Argument marshalling only: every step of the training path runs in the HIP
library.  PyTorch provides device memory (torch.empty on the ROCm device) and
the current stream.  There is no fallback: if the library is missing or the
device is not gfx950, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char, c_double, c_float, c_int32, c_int64, c_uint64, c_void_p

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt2mi.so")

GPT2_OK, GPT2_E_INVALID, GPT2_E_SHAPE, GPT2_E_STATE, GPT2_E_HIP, GPT2_E_DATA, GPT2_E_UNSUPPORTED = range(7)
IGNORE_TARGET = -100  # GPT2_IGNORE_TARGET: a position whose loss is not taken
MAX_LANES = 3         # GPT2_MAX_LANES: lanes per model (so at most four micro-steps in flight)
# kernel classes whose work is counted in FLOP (the others count bytes)
MFMA_CLASSES = ("gemm_nt", "gemm_nt_gelu", "gemm_nt_dgelu", "gemm_tn_acc", "gemm_tn_splitk", "attn_fwd", "attn_dkdv",
                "attn_dq")


class Gpt2Error(RuntimeError):
    def __init__(self, status, what, lib=None):
        msg = lib.gpt2_strerror(status).decode() if lib is not None else str(status)
        super().__init__(f"{what}: status {status} ({msg})")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("L", "H", "C", "V", "Vp", "Tmax", "B", "T")]


class Sizes(ctypes.Structure):
    _fields_ = [(n, c_int64) for n in ("n_params", "n_params_real", "n_decay", "n_shadow_t", "n_tensors",
                                       "acts_bytes", "scratch_bytes")]


class TensorInfo(ctypes.Structure):
    _fields_ = [("name", c_char * 48), ("offset", c_int64), ("rows", c_int64), ("cols", c_int64),
                ("decayed", c_int32), ("shadow_t_offset", c_int64)]


class Buffers(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("params", "grads", "m", "v", "shadow", "shadow_t", "acts", "scratch")]


class AdamwArgs(ctypes.Structure):
    _fields_ = [("lr", c_float), ("beta1", c_float), ("beta2", c_float), ("eps", c_float),
                ("weight_decay", c_float), ("max_norm", c_float), ("t", c_int32)]


_LIB = None

_SIGS = {
    "gpt2_sizes": (c_int32, [POINTER(Config), POINTER(Sizes)]),
    "gpt2_tensor_info": (c_int32, [POINTER(Config), c_int32, POINTER(TensorInfo)]),
    "gpt2_init": (c_int32, [POINTER(Config), c_uint64, c_void_p, POINTER(Buffers), c_void_p, POINTER(c_void_p)]),
    "gpt2_forward": (c_int32, [c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p]),
    "gpt2_backward": (c_int32, [c_void_p, c_void_p]),
    "gpt2_lane_init": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, POINTER(c_void_p)]),
    "gpt2_clip_adamw": (c_int32, [c_void_p, POINTER(AdamwArgs), c_void_p, c_void_p]),
    "gpt2_eval_loss": (c_int32, [c_void_p, c_void_p, c_void_p, POINTER(c_float), c_void_p]),
    "gpt2_sync_status": (c_int32, [c_void_p, c_void_p]),
    "gpt2_logits_ptr": (c_void_p, [c_void_p]),
    "gpt2_row_loss_ptr": (c_void_p, [c_void_p]),
    "gpt2_residual_ptr": (c_void_p, [c_void_p, c_int32]),
    "gpt2_last_hip_error": (c_int32, [c_void_p]),
    "gpt2_destroy": (None, [c_void_p]),
    "gpt2_strerror": (ctypes.c_char_p, [c_int32]),
    "gpt2_prof_enable": (c_int32, [c_void_p, c_int32]),
    "gpt2_prof_read": (c_int32, [c_void_p, c_void_p, c_int32, POINTER(c_double), POINTER(c_int64),
                                 POINTER(c_double)]),
    "gpt2_prof_class_name": (ctypes.c_char_p, [c_int32]),
    "gpt2k_xent": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_int32, c_float, c_int32, c_void_p,
                             c_void_p]),
    "gpt2k_layernorm_fwd": (c_int32, [c_void_p] * 6 + [c_int64, c_int32, c_void_p]),
    "gpt2k_layernorm_bwd": (c_int32, [c_void_p] * 6 + [c_int32, c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                                       c_int32, c_void_p]),
    "gpt2k_bias_gelu_fwd": (c_int32, [c_void_p] * 4 + [c_int64, c_int32, c_void_p]),
    "gpt2k_bias_gelu_bwd": (c_int32, [c_void_p] * 5 + [c_int64, c_int64, c_int32, c_void_p]),
    "gpt2k_bias_grad": (c_int32, [c_void_p] * 3 + [c_int64, c_int64, c_int32, c_void_p]),
    "gpt2k_gemm_nt": (c_int32, [c_void_p] * 5 + [c_int64] * 3 + [c_void_p]),
    "gpt2k_gemm_nt_gelu": (c_int32, [c_void_p] * 5 + [c_int64] * 3 + [c_void_p]),
    "gpt2k_gemm_nt_dgelu": (c_int32, [c_void_p] * 4 + [c_int64] * 3 + [c_void_p]),
    "gpt2k_gemm_tn_acc": (c_int32, [c_void_p] * 5 + [c_int64] * 4 + [c_void_p]),
    "gpt2k_attention_fwd": (c_int32, [c_void_p] * 3 + [c_int32] * 4 + [c_void_p]),
    "gpt2k_attention_bwd": (c_int32, [c_void_p] * 6 + [c_int32] * 4 + [c_void_p]),
    "gpt2k_clip_adamw": (c_int32, [c_void_p] * 5 + [c_int64, c_int64, POINTER(AdamwArgs), c_void_p, c_void_p,
                                                    c_int64, c_void_p]),
    "gpt2k_clip_adamw_noalloc": (c_int32, [c_void_p] * 5 + [c_int64, c_int64, POINTER(AdamwArgs), c_void_p,
                                            c_void_p]),
    "gpt2k_embedding_fwd": (c_int32, [c_void_p] * 4 + [c_int32] * 4 + [c_void_p, c_void_p]),
    "gpt2k_embedding_bwd": (c_int32, [c_void_p] * 4 + [c_int32] * 4 + [c_void_p, c_int64, c_void_p]),
    "gpt2k_scratch_bytes": (c_int32, [c_int32, c_int64, c_int64, c_int64, POINTER(c_int64)]),
}

EXPORTED = tuple(_SIGS)


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m transformer_lm_pretraining_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def check(status, what):
    if status != GPT2_OK:
        raise Gpt2Error(status, what, _LIB)


def make_config(L, H, C, V, Vp, Tmax, B, T) -> Config:
    return Config(L, H, C, V, Vp, Tmax, B, T)


def sizes(cfg: Config) -> Sizes:
    lib = load()
    s = Sizes()
    check(lib.gpt2_sizes(ctypes.byref(cfg), ctypes.byref(s)), "gpt2_sizes")
    return s


def tensor_table(cfg: Config):
    """[(name, offset, rows, cols, decayed, shadow_t_offset)] of the flat layout."""
    lib = load()
    n = sizes(cfg).n_tensors
    out = []
    for i in range(n):
        ti = TensorInfo()
        check(lib.gpt2_tensor_info(ctypes.byref(cfg), i, ctypes.byref(ti)), "gpt2_tensor_info")
        out.append((ti.name.decode(), ti.offset, ti.rows, ti.cols, bool(ti.decayed), ti.shadow_t_offset))
    return out


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class _Pass:
    """Forward / backward / evaluation and timing calls shared by a model and its lanes."""

    def __del__(self):
        if getattr(self, "h", None):
            self.lib.gpt2_destroy(self.h)
            self.h = None

    def forward(self, tok, tgt=None, dloss=None, loss_out=None):
        """tok, tgt: int32 device tensors [B, T].  Returns the device loss tensor (mean over B*T) or None."""
        if dloss is None:
            dloss = 1.0 / (self.cfg.B * self.cfg.T)
        out = loss_out if loss_out is not None else self.loss_dev
        self._keep = tok  # the backward reads the ids again
        check(self.lib.gpt2_forward(self.h, _ptr(tok), _ptr(tgt), float(dloss), _ptr(out) if tgt is not None else None,
                                    _stream()), "gpt2_forward")
        return out if tgt is not None else None

    def backward(self):
        check(self.lib.gpt2_backward(self.h, _stream()), "gpt2_backward")

    def eval_loss(self, tok, tgt) -> float:
        out = c_float()
        check(self.lib.gpt2_eval_loss(self.h, _ptr(tok), _ptr(tgt), ctypes.byref(out), _stream()), "gpt2_eval_loss")
        return out.value

    def sync_status(self) -> int:
        return self.lib.gpt2_sync_status(self.h, _stream())

    # -- views for tests and tools
    def _acts_view(self, ptr, nbytes):
        off = ptr - self.acts.data_ptr()
        return self.acts[off:off + nbytes]

    def logits(self):
        import torch
        BT = self.cfg.B * self.cfg.T
        v = self._acts_view(self.lib.gpt2_logits_ptr(self.h), BT * self.cfg.Vp * 2)
        return v.view(torch.bfloat16).view(BT, self.cfg.Vp)

    def row_losses(self):
        import torch
        BT = self.cfg.B * self.cfg.T
        return self._acts_view(self.lib.gpt2_row_loss_ptr(self.h), BT * 4).view(torch.float32)

    def residual(self, l):
        import torch
        BT = self.cfg.B * self.cfg.T
        v = self._acts_view(self.lib.gpt2_residual_ptr(self.h, l), BT * self.cfg.C * 2)
        return v.view(torch.bfloat16).view(BT, self.cfg.C)

    def tensor(self, flat, name):
        for n, off, rows, cols, _, _ in self.table:
            if n == name:
                t = flat[off:off + rows * cols]
                return t.view(rows, cols) if rows > 1 else t
        raise KeyError(name)

    def prof_enable(self, kclass):
        check(self.lib.gpt2_prof_enable(self.h, kclass), "gpt2_prof_enable")

    def prof_read(self, kclass=-1):
        """(total ms, launches, algorithmic work) over the recorded launches of kclass (-1: all)."""
        ms, n, work = c_double(), c_int64(), c_double()
        check(self.lib.gpt2_prof_read(self.h, _stream(), kclass, ctypes.byref(ms), ctypes.byref(n),
                                      ctypes.byref(work)), "gpt2_prof_read")
        return ms.value, n.value, work.value


class GPT2(_Pass):
    """A model instance: caller-owned device buffers (torch) + the library handle."""

    def __init__(self, cfg: Config, seed: int = 1337, init=None, device="cuda"):
        import torch
        self.lib = load()
        self.cfg = cfg
        self.sz = sizes(cfg)
        self.table = tensor_table(cfg)
        dev = torch.device(device)
        f32 = dict(dtype=torch.float32, device=dev)
        n = self.sz.n_params
        self.params = torch.empty(n, **f32)
        self.grads = torch.empty(n, **f32)
        self.m = torch.empty(n, **f32)
        self.v = torch.empty(n, **f32)
        self.shadow = torch.empty(self.sz.n_decay, dtype=torch.bfloat16, device=dev)
        self.shadow_t = torch.empty(self.sz.n_shadow_t, dtype=torch.bfloat16, device=dev)
        self.acts = torch.empty(self.sz.acts_bytes, dtype=torch.uint8, device=dev)
        self.scratch = torch.empty(self.sz.scratch_bytes, dtype=torch.uint8, device=dev)
        self.loss_dev = torch.zeros(1, **f32)
        self.norm_dev = torch.zeros(1, **f32)
        bufs = Buffers(*[t.data_ptr() for t in (self.params, self.grads, self.m, self.v, self.shadow, self.shadow_t,
                                                self.acts, self.scratch)])
        host = None
        if init is not None:
            host_arr = np.ascontiguousarray(init, dtype=np.float32)
            assert host_arr.size == n
            host = host_arr.ctypes.data_as(c_void_p)
        h = c_void_p()
        check(self.lib.gpt2_init(ctypes.byref(cfg), seed, host, ctypes.byref(bufs), _stream(), ctypes.byref(h)),
              "gpt2_init")
        self.h = h
        self._keep = None
        self.lanes = []

    def __del__(self):
        for ln in getattr(self, "lanes", []):  # lanes go before their model
            ln.close()
        super().__del__()

    def add_lane(self):
        """A lane of this model (gpt2_lane_init): its own gradient accumulator, activations and scratch."""
        ln = Lane(self)
        self.lanes.append(ln)
        return ln

    def clip_adamw(self, lr, t, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0, norm_out=None):
        """norm_out: optional fp32 device scalar for the pre-clip norm (default: the model's own).
        The gradient is the sum of the model's and its lanes' accumulators."""
        a = AdamwArgs(lr, beta1, beta2, eps, weight_decay, max_norm, t)
        out = norm_out if norm_out is not None else self.norm_dev
        check(self.lib.gpt2_clip_adamw(self.h, ctypes.byref(a), _ptr(out), _stream()), "gpt2_clip_adamw")
        return out


class Lane(_Pass):
    """A lane of a model: reads the model's parameters and shadows, owns grads, acts and scratch."""

    def __init__(self, model: GPT2):
        import torch
        self.lib = model.lib
        self.cfg = model.cfg
        self.sz = model.sz
        self.table = model.table
        dev = model.params.device
        self.grads = torch.empty(self.sz.n_params, dtype=torch.float32, device=dev)
        self.acts = torch.empty(self.sz.acts_bytes, dtype=torch.uint8, device=dev)
        self.scratch = torch.empty(self.sz.scratch_bytes, dtype=torch.uint8, device=dev)
        self.loss_dev = torch.zeros(1, dtype=torch.float32, device=dev)
        h = c_void_p()
        check(self.lib.gpt2_lane_init(model.h, _ptr(self.grads), _ptr(self.acts), _ptr(self.scratch), _stream(),
                                      ctypes.byref(h)), "gpt2_lane_init")
        self.h = h
        self._keep = None

    def close(self):
        if getattr(self, "h", None):
            self.lib.gpt2_destroy(self.h)
            self.h = None


def kernel_class_names():
    """{class id: kernel name} of the timing classes."""
    lib = load()
    out = {}
    for k in range(1, 64):
        n = lib.gpt2_prof_class_name(k)
        if n is None:
            break
        out[k] = n.decode()
    return out


# ---------------------------------------------------------------- kernel-level calls

def scratch_bytes(kind, a, b=0, c=0) -> int:
    out = c_int64()
    check(load().gpt2k_scratch_bytes(kind, a, b, c, ctypes.byref(out)), "gpt2k_scratch_bytes")
    return out.value


def _scratch(nbytes, device="cuda"):
    import torch
    return torch.empty(max(256, nbytes), dtype=torch.uint8, device=device)


def xent(logits, tgt, V, dloss, write_grad=True, flag=None):
    """In place on bf16 logits [R, Vp]; returns fp32 row losses [R]."""
    import torch
    R, Vp = logits.shape
    loss = torch.empty(R, dtype=torch.float32, device=logits.device)
    check(load().gpt2k_xent(_ptr(logits), _ptr(tgt), _ptr(loss), R, V, Vp, float(dloss), int(write_grad), _ptr(flag),
                            _stream()), "gpt2k_xent")
    return loss


def layernorm_fwd(x, w, b):
    import torch
    R, C = x.shape
    y = torch.empty_like(x)
    mean = torch.empty(R, dtype=torch.float32, device=x.device)
    rstd = torch.empty(R, dtype=torch.float32, device=x.device)
    check(load().gpt2k_layernorm_fwd(_ptr(x), _ptr(w), _ptr(b), _ptr(y), _ptr(mean), _ptr(rstd), R, C, _stream()),
          "gpt2k_layernorm_fwd")
    return y, mean, rstd


def layernorm_bwd(x, dy, w, mean, rstd, dres, accumulate, dw, db):
    R, C = x.shape
    n = scratch_bytes(1, R, C)
    s = _scratch(n, x.device)
    check(load().gpt2k_layernorm_bwd(_ptr(x), _ptr(dy), _ptr(w), _ptr(mean), _ptr(rstd), _ptr(dres), int(accumulate),
                                     _ptr(dw), _ptr(db), _ptr(s), s.numel(), R, C, _stream()), "gpt2k_layernorm_bwd")


def bias_gelu_fwd(u, b):
    import torch
    R, N = u.shape
    pre = torch.empty_like(u)
    g = torch.empty_like(u)
    check(load().gpt2k_bias_gelu_fwd(_ptr(u), _ptr(b), _ptr(pre), _ptr(g), R, N, _stream()), "gpt2k_bias_gelu_fwd")
    return pre, g


def bias_gelu_bwd(pre, dg, db, out=None):
    import torch
    R, N = pre.shape
    dpre = out if out is not None else torch.empty_like(pre)
    s = _scratch(scratch_bytes(2, R, N), pre.device)
    check(load().gpt2k_bias_gelu_bwd(_ptr(pre), _ptr(dg), _ptr(dpre), _ptr(db), _ptr(s), s.numel(), R, N, _stream()),
          "gpt2k_bias_gelu_bwd")
    return dpre


def bias_grad(dY, db):
    R, N = dY.shape
    s = _scratch(scratch_bytes(2, R, N), dY.device)
    check(load().gpt2k_bias_grad(_ptr(dY), _ptr(db), _ptr(s), s.numel(), R, N, _stream()), "gpt2k_bias_grad")


def gemm_nt(A, B, bias=None, res=None, out=None):
    import torch
    M, K = A.shape
    N = B.shape[0]
    o = out if out is not None else torch.empty(M, N, dtype=torch.bfloat16, device=A.device)
    check(load().gpt2k_gemm_nt(_ptr(A), _ptr(B), _ptr(bias), _ptr(res), _ptr(o), M, N, K, _stream()), "gpt2k_gemm_nt")
    return o


def gemm_nt_gelu(A, B, bias):
    """Returns (GELU'(pre), GELU(pre)) with pre = A . B^T + bias in bf16."""
    import torch
    M, K = A.shape
    N = B.shape[0]
    gprime = torch.empty(M, N, dtype=torch.bfloat16, device=A.device)
    g = torch.empty_like(gprime)
    check(load().gpt2k_gemm_nt_gelu(_ptr(A), _ptr(B), _ptr(bias), _ptr(gprime), _ptr(g), M, N, K, _stream()),
          "gpt2k_gemm_nt_gelu")
    return gprime, g


def gemm_nt_dgelu(A, B, gprime):
    import torch
    M, K = A.shape
    N = B.shape[0]
    out = torch.empty(M, N, dtype=torch.bfloat16, device=A.device)
    check(load().gpt2k_gemm_nt_dgelu(_ptr(A), _ptr(B), _ptr(gprime), _ptr(out), M, N, K, _stream()),
          "gpt2k_gemm_nt_dgelu")
    return out


def gemm_tn_acc(dY, X, dW, db=None):
    M, N = dY.shape
    K = X.shape[1]
    s = _scratch(scratch_bytes(3, M, N, K), dY.device)
    check(load().gpt2k_gemm_tn_acc(_ptr(dY), _ptr(X), _ptr(dW), _ptr(db), _ptr(s), s.numel(), M, N, K, _stream()),
          "gpt2k_gemm_tn_acc")


def attention_fwd(qkv, B, T, H, C):
    import torch
    out = torch.empty(B * T, C, dtype=torch.bfloat16, device=qkv.device)
    lse = torch.empty(B, H, T, dtype=torch.float32, device=qkv.device)
    check(load().gpt2k_attention_fwd(_ptr(qkv), _ptr(out), _ptr(lse), B, T, H, C, _stream()), "gpt2k_attention_fwd")
    return out, lse


def attention_bwd(qkv, out, dout, lse, B, T, H, C):
    import torch
    dqkv = torch.empty_like(qkv)
    dvec = torch.empty(B, H, T, dtype=torch.float32, device=qkv.device)
    check(load().gpt2k_attention_bwd(_ptr(qkv), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dqkv), _ptr(dvec), B, T, H, C,
                                     _stream()), "gpt2k_attention_bwd")
    return dqkv


def clip_adamw(p, g, m, v, shadow, n_decay, lr, t, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
               max_norm=1.0):
    import torch
    n = p.numel()
    a = AdamwArgs(lr, beta1, beta2, eps, weight_decay, max_norm, t)
    s = _scratch(scratch_bytes(4, n), p.device)
    norm = torch.zeros(1, dtype=torch.float32, device=p.device)
    check(load().gpt2k_clip_adamw(_ptr(p), _ptr(g), _ptr(m), _ptr(v), _ptr(shadow), n, n_decay, ctypes.byref(a),
                                  _ptr(norm), _ptr(s), s.numel(), _stream()), "gpt2k_clip_adamw")
    return norm


def clip_adamw_noalloc(p, g, m, v, shadow, n_decay, lr, t, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
                       max_norm=1.0, norm=None):
    """gpt2k_clip_adamw_noalloc: the library's own static scratch; norm (fp32 device
    scalar) must be given by a caller that allocates nothing here."""
    import torch
    a = AdamwArgs(lr, beta1, beta2, eps, weight_decay, max_norm, t)
    if norm is None:
        norm = torch.zeros(1, dtype=torch.float32, device=p.device)
    check(load().gpt2k_clip_adamw_noalloc(_ptr(p), _ptr(g), _ptr(m), _ptr(v), _ptr(shadow), p.numel(), n_decay,
                                          ctypes.byref(a), _ptr(norm), _stream()), "gpt2k_clip_adamw_noalloc")
    return norm


def embedding_fwd(tok, wte, wpe, V, flag=None):
    import torch
    B, T = tok.shape
    C = wte.shape[1]
    x = torch.empty(B * T, C, dtype=torch.bfloat16, device=tok.device)
    check(load().gpt2k_embedding_fwd(_ptr(tok), _ptr(wte), _ptr(wpe), _ptr(x), B, T, C, V, _ptr(flag), _stream()),
          "gpt2k_embedding_fwd")
    return x


def embedding_bwd(tok, dx, dwte, dwpe, V):
    B, T = tok.shape
    C = dx.shape[1]
    s = _scratch(scratch_bytes(5, B * T, V, C), dx.device)
    check(load().gpt2k_embedding_bwd(_ptr(tok), _ptr(dx), _ptr(dwte), _ptr(dwpe), B, T, C, V, _ptr(s), s.numel(),
                                     _stream()), "gpt2k_embedding_bwd")
