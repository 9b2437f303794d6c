"""ctypes binding of libgpt2_mi355x.so (include/gpt2.h): argument marshalling only.

Every computation runs in the library's HIP kernels. torch supplies device memory and the
stream: by default a model and every per-kernel call use torch's current HIP stream, so the
library's work is ordered with the caller's torch work. There is no fallback: if the
library is missing or was built for another device, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgpt2_mi355x.so")

GPT2_OK = 0
ERRORS = {-1: "GPT2_ERR_ARG", -2: "GPT2_ERR_SHAPE", -3: "GPT2_ERR_TOKEN", -4: "GPT2_ERR_STATE",
          -5: "GPT2_ERR_OOM", -6: "GPT2_ERR_HIP", -7: "GPT2_ERR_IO"}

_vp = ctypes.c_void_p
_int = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

# name -> (restype, argtypes): mirrors include/gpt2.h
SIGNATURES = {
    "gpt2_build": (_int, [ctypes.POINTER(_vp), _int, _int, _int, _int, _int]),
    "gpt2_build_ex": (_int, [ctypes.POINTER(_vp), _int, _int, _int, _int, _int, _int, _int,
                             _int, _vp]),
    "gpt2_free": (None, [_vp]),
    "gpt2_set_stream": (_int, [_vp, _vp]),
    "gpt2_synchronize": (_int, [_vp]),
    "gpt2_num_params": (_sz, [_vp]),
    "gpt2_get_config": (_int, [_vp, ctypes.POINTER(_int)]),
    "gpt2_checkpoint_info": (_int, [ctypes.c_char_p, ctypes.POINTER(_int), ctypes.POINTER(_int),
                                    ctypes.POINTER(_int), ctypes.POINTER(_int),
                                    ctypes.POINTER(_int), ctypes.POINTER(_sz)]),
    "gpt2_checkpoint_read": (_int, [ctypes.c_char_p, _vp, _sz]),
    "gpt2_checkpoint_write": (_int, [ctypes.c_char_p, _int, _int, _int, _int, _int, _vp]),
    "gpt2_build_from_checkpoint": (_int, [ctypes.POINTER(_vp), ctypes.c_char_p, _int, _int, _int,
                                          _vp]),
    "gpt2_save_checkpoint": (_int, [_vp, ctypes.c_char_p]),
    "gpt2_dataloader_init": (_int, [ctypes.POINTER(_vp), ctypes.c_char_p, _int, _int]),
    "gpt2_dataloader_num_batches": (_int, [_vp]),
    "gpt2_dataloader_reset": (_int, [_vp]),
    "gpt2_dataloader_next_batch": (_int, [_vp, _vp, _vp, _int, _vp]),
    "gpt2_dataloader_free": (None, [_vp]),
    "gpt2_random_u32": (ctypes.c_uint32, [ctypes.POINTER(ctypes.c_uint64)]),
    "gpt2_random_f32": (_f, [ctypes.POINTER(ctypes.c_uint64)]),
    "gpt2_sample": (_int, [_vp, _int, _int, _f, ctypes.POINTER(ctypes.c_int32)]),
    "gpt2_k_sample_mult": (_int, [_vp, _vp, _int, _f, _vp]),
    "gpt2_param_layout": (_int, [_vp, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "gpt2_set_params": (_int, [_vp, _vp, _int]),
    "gpt2_get_params": (_int, [_vp, _vp, _int]),
    "gpt2_get_grads": (_int, [_vp, _vp, _int]),
    "gpt2_set_grads": (_int, [_vp, _vp, _int]),
    "gpt2_get_adam_state": (_int, [_vp, _vp, _vp, _int]),
    "gpt2_forward": (_int, [_vp, _vp, _vp, _int, _int, ctypes.POINTER(_f)]),
    "gpt2_get_losses": (_int, [_vp, _vp, _int]),
    "gpt2_get_logits": (_int, [_vp, _vp, _int]),
    "gpt2_zero_grad": (_int, [_vp]),
    "gpt2_backward": (_int, [_vp]),
    "gpt2_adamw_step": (_int, [_vp, _f, _f, _f, _f, _f, _int]),
    "gpt2_profile_enable": (_int, [_int]),
    "gpt2_profile_summary": (_int, [ctypes.c_char_p, _sz]),
    "gpt2_profile_only": (_int, [ctypes.c_char_p]),
    "gpt2_last_error": (ctypes.c_char_p, [_vp]),
    "gpt2_last_global_error": (ctypes.c_char_p, []),
    "gpt2_version": (ctypes.c_char_p, []),
    "gpt2_k_encoder_forward": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp, _vp]),
    "gpt2_k_encoder_backward": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp]),
    "gpt2_k_layernorm_forward": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _vp]),
    "gpt2_k_layernorm_backward": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int,
                                         _vp]),
    "gpt2_k_matmul_forward": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int,
                                     _vp]),
    "gpt2_k_matmul_backward": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int,
                                      _vp]),
    "gpt2_k_matmul_backward_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int,
                                              _int, _int, _vp]),
    "gpt2_k_attention_forward": (_int, [_vp, _vp, _vp, _int, _int, _int, _int, _vp]),
    "gpt2_k_attention_backward": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp]),
    "gpt2_k_crossentropy_forward": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _vp, _vp]),
    "gpt2_k_crossentropy_backward": (_int, [_vp, _vp, _vp, _f, _int, _int, _int, _vp]),
    "gpt2_k_mean": (_int, [_vp, _vp, _int, _vp]),
    "gpt2_k_adamw": (_int, [_vp, _vp, _vp, _vp, _sz, _f, _f, _f, _f, _f, _int, _vp]),
    "gpt2_k_gemm_bf16": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int,
                                _int, _int, _int, _int, _vp]),
    "gpt2_k_gemm_f16": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int,
                               _int, _int, _int, _int, _vp]),
    "gpt2_k_attention_forward_f16": (_int, [_vp, _vp, _vp, _int, _int, _int, _int, _vp]),
    "gpt2_k_attention_backward_f16": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int,
                                             _vp]),
    "gpt2_set_loss_scale": (_int, [_vp, _f, _int]),
    "gpt2_set_loss_grad_in_forward": (_int, [_vp, _int]),
    "gpt2_k_crossentropy_fused": (_int, [_vp, _vp, _vp, _vp, _vp, _f, _int, _int, _int, _vp, _vp]),
    "gpt2_get_loss_scale": (_int, [_vp, ctypes.POINTER(_f), ctypes.POINTER(_int)]),
    "gpt2_k_encoder_forward_bf16": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp,
                                           _vp]),
    "gpt2_k_layernorm_forward_bf16": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _vp]),
    "gpt2_k_layernorm_backward_bf16": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int,
                                              _int, _vp]),
    "gpt2_k_attention_forward_bf16": (_int, [_vp, _vp, _vp, _int, _int, _int, _int, _vp]),
    "gpt2_k_attention_backward_bf16": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int,
                                              _vp]),
    "gpt2_k_crossentropy_forward_bf16": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _vp,
                                                _vp]),
    "gpt2_k_crossentropy_backward_bf16": (_int, [_vp, _vp, _vp, _f, _int, _int, _int, _vp]),
    "gpt2_k_adamw_bf16": (_int, [_vp, _vp, _vp, _vp, _vp, _sz, _f, _f, _f, _f, _f, _int, _vp]),
    "gpt2_k_cast_bf16": (_int, [_vp, _vp, _sz, _vp]),
}

DTYPES = {"fp32": 0, "bf16": 1, "fp16": 2}

_lib = None


class GPT2Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m decoder_only_transformer_05_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(rc: int, model=None):
    if rc != GPT2_OK:
        msg = (lib().gpt2_last_error(model) if model else lib().gpt2_last_global_error())
        raise GPT2Error(rc, (msg or b"").decode(errors="replace"))


def _torch():
    import torch
    return torch


def current_stream() -> int:
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def _ptr(t, kind: str = "f32") -> int | None:
    """Device pointer of a contiguous torch tensor of the expected dtype, or None."""
    if t is None:
        return None
    torch = _torch()
    want = {"f32": torch.float32, "i32": torch.int32, "bf16": torch.bfloat16,
            "f16": torch.float16}[kind]
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if t.dtype != want:
        raise ValueError(f"expected a {want} tensor, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _iptr(t) -> int | None:
    return _ptr(t, "i32")


def _hptr(t) -> int | None:
    return _ptr(t, "bf16")


def _f16ptr(t) -> int | None:
    return _ptr(t, "f16")


def _host_or_device(buf):
    """(pointer, is_device) for a torch tensor or a contiguous numpy float32 array."""
    if isinstance(buf, np.ndarray):
        if buf.dtype != np.float32 or not buf.flags.c_contiguous:
            raise ValueError("expected a contiguous float32 array")
        return buf.ctypes.data, 0
    torch = _torch()
    if buf.dtype != torch.float32 or not buf.is_contiguous():
        raise ValueError("expected a contiguous float32 tensor")
    return buf.data_ptr(), 1 if buf.is_cuda else 0


def _path(p) -> bytes:
    return os.fsencode(p)


def checkpoint_info(path) -> dict:
    """Configuration and parameter count of a checkpoint file (no GPU needed)."""
    v = [_int() for _ in range(5)]
    n = _sz()
    _check(lib().gpt2_checkpoint_info(_path(path), *[ctypes.byref(x) for x in v],
                                      ctypes.byref(n)))
    return {"maxT": v[0].value, "V": v[1].value, "L": v[2].value, "H": v[3].value,
            "C": v[4].value, "num_params": n.value}


def checkpoint_read(path) -> np.ndarray:
    n = checkpoint_info(path)["num_params"]
    out = np.empty(n, np.float32)
    _check(lib().gpt2_checkpoint_read(_path(path), out.ctypes.data, n))
    return out


def checkpoint_write(path, params, L, C, H, V, maxT):
    p = np.ascontiguousarray(params, dtype=np.float32)
    _check(lib().gpt2_checkpoint_write(_path(path), maxT, V, L, H, C, p.ctypes.data))


class Rng:
    """The pages' xorshift* generator (random_u32 / random_f32) on a host 64-bit state."""

    def __init__(self, seed: int):
        self.state = ctypes.c_uint64(seed)

    def u32(self) -> int:
        return int(lib().gpt2_random_u32(ctypes.byref(self.state)))

    def f32(self) -> float:
        return float(lib().gpt2_random_f32(ctypes.byref(self.state)))


class DataLoader:
    """Batches of (inputs, targets) from a file of int32 tokens (include/gpt2.h)."""

    def __init__(self, path, B: int, T: int):
        h = _vp()
        _check(lib().gpt2_dataloader_init(ctypes.byref(h), _path(path), B, T))
        self.h, self.B, self.T = h, B, T
        self.num_batches = int(lib().gpt2_dataloader_num_batches(h))

    def reset(self):
        _check(lib().gpt2_dataloader_reset(self.h))

    def next_batch(self, inputs=None, targets=None):
        """Fills int32 (B,T) host arrays or device tensors (new host arrays if None)."""
        if inputs is None:
            inputs = np.empty((self.B, self.T), np.int32)
            targets = np.empty((self.B, self.T), np.int32)
        if isinstance(inputs, np.ndarray):
            for a in (inputs, targets):
                if a.dtype != np.int32 or not a.flags.c_contiguous or a.size != self.B * self.T:
                    raise ValueError("expected contiguous int32 arrays of B*T tokens")
            _check(lib().gpt2_dataloader_next_batch(self.h, inputs.ctypes.data,
                                                    targets.ctypes.data, 0, None))
        else:
            for a in (inputs, targets):
                if a.numel() != self.B * self.T:
                    raise ValueError("expected tensors of B*T tokens")
            _check(lib().gpt2_dataloader_next_batch(self.h, _iptr(inputs), _iptr(targets), 1,
                                                    current_stream()))
        return inputs, targets

    def close(self):
        if getattr(self, "h", None):
            lib().gpt2_dataloader_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class GPT2:
    """One model on the current device (see include/gpt2.h for the semantics)."""

    def __init__(self, L: int, C: int, H: int, V: int, maxT: int, B: int = 0, T: int = 0,
                 stream: int | None = None, dtype: str = "fp32", _handle=None):
        if _handle is None:
            h = _vp()
            st = current_stream() if stream is None else stream
            _check(lib().gpt2_build_ex(ctypes.byref(h), L, C, H, V, maxT, DTYPES[dtype], B, T,
                                       st))
        else:
            h = _handle
        self.h = h
        self.dtype = dtype
        self.L, self.C, self.H, self.V, self.maxT = L, C, H, V, maxT
        self.num_params = int(lib().gpt2_num_params(h))

    @classmethod
    def from_checkpoint(cls, path, B: int = 0, T: int = 0, stream: int | None = None,
                        dtype: str = "fp32"):
        h = _vp()
        st = current_stream() if stream is None else stream
        _check(lib().gpt2_build_from_checkpoint(ctypes.byref(h), _path(path), DTYPES[dtype], B, T,
                                                st))
        cfg = (_int * 5)()
        _check(lib().gpt2_get_config(h, cfg))
        L, C, H, V, maxT = list(cfg)
        return cls(L, C, H, V, maxT, dtype=dtype, _handle=h)

    def save_checkpoint(self, path):
        self._c(lib().gpt2_save_checkpoint(self.h, _path(path)))

    def set_loss_grad_in_forward(self, on: bool):
        self._c(lib().gpt2_set_loss_grad_in_forward(self.h, 1 if on else 0))

    def set_loss_scale(self, scale: float, growth_interval: int = 2000):
        self._c(lib().gpt2_set_loss_scale(self.h, scale, growth_interval))

    def get_loss_scale(self):
        """(scale, last step skipped) -- fp16 models; others report (1.0, False)."""
        sc, sk = _f(), _int()
        self._c(lib().gpt2_get_loss_scale(self.h, ctypes.byref(sc), ctypes.byref(sk)))
        return float(sc.value), bool(sk.value)

    def sample(self, b: int, t: int, coin: float) -> int:
        tok = ctypes.c_int32()
        self._c(lib().gpt2_sample(self.h, b, t, coin, ctypes.byref(tok)))
        return int(tok.value)

    def close(self):
        if getattr(self, "h", None):
            lib().gpt2_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _c(self, rc):
        _check(rc, self.h)

    def layout(self):
        off, ln = (_sz * 16)(), (_sz * 16)()
        self._c(lib().gpt2_param_layout(self.h, off, ln))
        return list(off), list(ln)

    def set_stream(self, stream: int | None):
        self._c(lib().gpt2_set_stream(self.h, stream))

    def synchronize(self):
        self._c(lib().gpt2_synchronize(self.h))

    def set_params(self, buf):
        p, dev = _host_or_device(buf)
        self._c(lib().gpt2_set_params(self.h, p, dev))

    def get_params(self, out=None):
        out = np.empty(self.num_params, np.float32) if out is None else out
        p, dev = _host_or_device(out)
        self._c(lib().gpt2_get_params(self.h, p, dev))
        return out

    def get_grads(self, out=None):
        out = np.empty(self.num_params, np.float32) if out is None else out
        p, dev = _host_or_device(out)
        self._c(lib().gpt2_get_grads(self.h, p, dev))
        return out

    def set_grads(self, buf):
        p, dev = _host_or_device(buf)
        self._c(lib().gpt2_set_grads(self.h, p, dev))

    def get_adam_state(self):
        m = np.empty(self.num_params, np.float32)
        v = np.empty(self.num_params, np.float32)
        self._c(lib().gpt2_get_adam_state(self.h, m.ctypes.data, v.ctypes.data, 0))
        return m, v

    def forward(self, tokens, targets=None, B: int | None = None, T: int | None = None,
                want_loss: bool = True):
        """tokens/targets: int32 device tensors (B,T). Returns the mean loss (or None)."""
        torch = _torch()
        for t in (tokens, targets):
            if t is not None and t.dtype != torch.int32:
                raise ValueError("tokens and targets must be int32")
        B = tokens.shape[0] if B is None else B
        T = tokens.shape[1] if T is None else T
        loss = _f(0.0)
        self._c(lib().gpt2_forward(self.h, _iptr(tokens), _iptr(targets), B, T,
                                   ctypes.byref(loss) if want_loss else None))
        return float(loss.value) if want_loss else None

    def zero_grad(self):
        self._c(lib().gpt2_zero_grad(self.h))

    def backward(self):
        self._c(lib().gpt2_backward(self.h))

    def adamw_step(self, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, t=1):
        self._c(lib().gpt2_adamw_step(self.h, lr, beta1, beta2, eps, weight_decay, t))

    def get_logits(self, out):
        p, dev = _host_or_device(out)
        self._c(lib().gpt2_get_logits(self.h, p, dev))
        return out

    def get_losses(self, out):
        p, dev = _host_or_device(out)
        self._c(lib().gpt2_get_losses(self.h, p, dev))
        return out


def profile_enable(on: bool = True, shapes: bool = False):
    _check(lib().gpt2_profile_enable((2 if shapes else 1) if on else 0))


def profile_only(name: str | None):
    """Record only launches named `name` (None: all)."""
    _check(lib().gpt2_profile_only(None if not name else name.encode()))


def profile_summary() -> dict:
    """{kernel name: {"launches", "ms", "flop", "bytes"}} of the launches recorded so far."""
    buf = ctypes.create_string_buffer(1 << 20)
    _check(lib().gpt2_profile_summary(buf, len(buf)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, ms, flop, nbytes = line.split("\t")
        out[name] = {"launches": int(n), "ms": float(ms), "flop": float(flop),
                     "bytes": float(nbytes)}
    return out


# ---- per-kernel entry points (device tensors; torch's current stream) --------------------
def k_encoder_forward(out, tok, wte, wpe, B, T, C, V, err_flag=None):
    _check(lib().gpt2_k_encoder_forward(_ptr(out), _iptr(tok), _ptr(wte), _ptr(wpe), B, T, C, V,
                                        _iptr(err_flag), current_stream()))


def k_encoder_backward(dwte, dwpe, dout, tok, B, T, C, V):
    _check(lib().gpt2_k_encoder_backward(_ptr(dwte), _ptr(dwpe), _ptr(dout), _iptr(tok), B, T, C,
                                         V, current_stream()))


def k_layernorm_forward(out, mean, rstd, x, w, b, N, C):
    _check(lib().gpt2_k_layernorm_forward(_ptr(out), _ptr(mean), _ptr(rstd), _ptr(x), _ptr(w),
                                          _ptr(b), N, C, current_stream()))


def k_layernorm_backward(dx, dw, db, dout, x, w, mean, rstd, N, C):
    _check(lib().gpt2_k_layernorm_backward(_ptr(dx), _ptr(dw), _ptr(db), _ptr(dout), _ptr(x),
                                           _ptr(w), _ptr(mean), _ptr(rstd), N, C,
                                           current_stream()))


def k_matmul_forward(out, inp, W, bias, N, C, OC, ld_out=None, epilogue=0, out2=None,
                     resid=None):
    _check(lib().gpt2_k_matmul_forward(_ptr(out), _ptr(out2), _ptr(resid), _ptr(inp), _ptr(W),
                                       _ptr(bias), N, C, OC, OC if ld_out is None else ld_out,
                                       epilogue, current_stream()))


def k_matmul_backward(dinp, dW, dbias, dout, inp, W, N, C, OC, gelu_pre=None, ld_dout=None):
    _check(lib().gpt2_k_matmul_backward(_ptr(dinp), _ptr(dW), _ptr(dbias), _ptr(dout), _ptr(inp),
                                        _ptr(W), _ptr(gelu_pre), N, C, OC,
                                        OC if ld_dout is None else ld_dout, current_stream()))


def k_matmul_backward_noalloc(dinp, dW, dbias, dout, inp, W, N, C, OC, gelu_pre=None,
                              ld_dout=None):
    _check(lib().gpt2_k_matmul_backward_noalloc(
        _ptr(dinp), _ptr(dW), _ptr(dbias), _ptr(dout), _ptr(inp), _ptr(W), _ptr(gelu_pre), N, C,
        OC, OC if ld_dout is None else ld_dout, current_stream()))


def k_attention_forward(out, lse, qkv, B, T, C, NH):
    _check(lib().gpt2_k_attention_forward(_ptr(out), _ptr(lse), _ptr(qkv), B, T, C, NH,
                                          current_stream()))


def k_attention_backward(dqkv, dout, qkv, out, lse, B, T, C, NH):
    _check(lib().gpt2_k_attention_backward(_ptr(dqkv), _ptr(dout), _ptr(qkv), _ptr(out),
                                           _ptr(lse), B, T, C, NH, current_stream()))


def k_crossentropy_forward(losses, lse, logits, targets, N, V, ld, err_flag=None):
    _check(lib().gpt2_k_crossentropy_forward(_ptr(losses), _ptr(lse), _ptr(logits),
                                             _iptr(targets), N, V, ld, _iptr(err_flag),
                                             current_stream()))


def k_crossentropy_backward(logits, lse, targets, dloss, N, V, ld):
    _check(lib().gpt2_k_crossentropy_backward(_ptr(logits), _ptr(lse), _iptr(targets), dloss, N, V,
                                              ld, current_stream()))


def k_crossentropy_fused(losses, lse, dlogits, logits, targets, dloss, N, V, ld, err_flag=None):
    _check(lib().gpt2_k_crossentropy_fused(_ptr(losses), _ptr(lse), _ptr(dlogits), _ptr(logits),
                                           _iptr(targets), dloss, N, V, ld, _iptr(err_flag),
                                           current_stream()))


def k_sample_mult(token, logits, V, coin):
    _check(lib().gpt2_k_sample_mult(_iptr(token), _ptr(logits), V, coin, current_stream()))


def k_mean(out, x, n):
    _check(lib().gpt2_k_mean(_ptr(out), _ptr(x), n, current_stream()))


def k_adamw(p, g, m, v, n, lr, beta1, beta2, eps, wd, t):
    _check(lib().gpt2_k_adamw(_ptr(p), _ptr(g), _ptr(m), _ptr(v), n, lr, beta1, beta2, eps, wd,
                              t, current_stream()))


# ---- bf16 forms (bf16 tensors are torch.bfloat16) ------------------------------------------
def k_gemm_bf16(C, A, B, M, N, K, lda, ldb, ldc, a_trans=False, b_trans=False, epilogue=0,
                bias=None, C2=None, R=None, colsum=None):
    """C (bf16, or fp32 for epilogue 3) = op(A) . op(B) with the fused epilogue."""
    c_ptr = _ptr(C) if epilogue == 3 else _hptr(C)
    _check(lib().gpt2_k_gemm_bf16(c_ptr, _hptr(C2), _hptr(R), _hptr(A), _hptr(B), _ptr(bias),
                                  _ptr(colsum), M, N, K, lda, ldb, ldc, int(a_trans),
                                  int(b_trans), epilogue, current_stream()))


def k_gemm_f16(C, A, B, M, N, K, lda, ldb, ldc, a_trans=False, b_trans=False, epilogue=0,
               bias=None, C2=None, R=None, colsum=None):
    """C (fp16, or fp32 for epilogue 3) = op(A) . op(B) with the fused epilogue."""
    c_ptr = _ptr(C) if epilogue == 3 else _f16ptr(C)
    _check(lib().gpt2_k_gemm_f16(c_ptr, _f16ptr(C2), _f16ptr(R), _f16ptr(A), _f16ptr(B),
                                 _ptr(bias), _ptr(colsum), M, N, K, lda, ldb, ldc, int(a_trans),
                                 int(b_trans), epilogue, current_stream()))


def k_attention_forward_f16(out, lse, qkv, B, T, C, NH):
    _check(lib().gpt2_k_attention_forward_f16(_f16ptr(out), _ptr(lse), _f16ptr(qkv), B, T, C, NH,
                                              current_stream()))


def k_attention_backward_f16(dqkv, dout, qkv, out, lse, B, T, C, NH):
    _check(lib().gpt2_k_attention_backward_f16(_f16ptr(dqkv), _f16ptr(dout), _f16ptr(qkv),
                                               _f16ptr(out), _ptr(lse), B, T, C, NH,
                                               current_stream()))


def k_encoder_forward_bf16(out, tok, wte, wpe, B, T, C, V, err_flag=None):
    _check(lib().gpt2_k_encoder_forward_bf16(_hptr(out), _iptr(tok), _ptr(wte), _ptr(wpe), B, T,
                                             C, V, _iptr(err_flag), current_stream()))


def k_layernorm_forward_bf16(out, mean, rstd, x, w, b, N, C):
    _check(lib().gpt2_k_layernorm_forward_bf16(_hptr(out), _ptr(mean), _ptr(rstd), _hptr(x),
                                               _ptr(w), _ptr(b), N, C, current_stream()))


def k_layernorm_backward_bf16(dx, dx_copy, dw, db, dout, x, w, mean, rstd, N, C):
    _check(lib().gpt2_k_layernorm_backward_bf16(_ptr(dx), _hptr(dx_copy), _ptr(dw), _ptr(db),
                                                _hptr(dout), _hptr(x), _ptr(w), _ptr(mean),
                                                _ptr(rstd), N, C, current_stream()))


def k_attention_forward_bf16(out, lse, qkv, B, T, C, NH):
    _check(lib().gpt2_k_attention_forward_bf16(_hptr(out), _ptr(lse), _hptr(qkv), B, T, C, NH,
                                               current_stream()))


def k_attention_backward_bf16(dqkv, dout, qkv, out, lse, B, T, C, NH):
    _check(lib().gpt2_k_attention_backward_bf16(_hptr(dqkv), _hptr(dout), _hptr(qkv),
                                                _hptr(out), _ptr(lse), B, T, C, NH,
                                                current_stream()))


def k_crossentropy_forward_bf16(losses, lse, logits, targets, N, V, ld, err_flag=None):
    _check(lib().gpt2_k_crossentropy_forward_bf16(_ptr(losses), _ptr(lse), _hptr(logits),
                                                  _iptr(targets), N, V, ld, _iptr(err_flag),
                                                  current_stream()))


def k_crossentropy_backward_bf16(logits, lse, targets, dloss, N, V, ld):
    _check(lib().gpt2_k_crossentropy_backward_bf16(_hptr(logits), _ptr(lse), _iptr(targets),
                                                   dloss, N, V, ld, current_stream()))


def k_adamw_bf16(p, p_bf16, g, m, v, n, lr, beta1, beta2, eps, wd, t):
    _check(lib().gpt2_k_adamw_bf16(_ptr(p), _hptr(p_bf16), _ptr(g), _ptr(m), _ptr(v), n, lr,
                                   beta1, beta2, eps, wd, t, current_stream()))


def k_cast_bf16(dst, src, n):
    _check(lib().gpt2_k_cast_bf16(_hptr(dst), _ptr(src), n, current_stream()))
