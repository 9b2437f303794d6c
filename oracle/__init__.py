"""fp64 CPU oracle of one GPT-2 training step -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this package. It wraps ``liboracle_gpt2.so`` (built from ``gpt2_oracle.cpp`` by
``build()``) with numpy-facing helpers. Nothing here is shared with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gpt2_oracle.cpp")
LIB_PATH = os.path.join(_HERE, "liboracle_gpt2.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (-O3 with AVX2 vectors, strict IEEE: no fast-math, no FMA
    contraction, so vectorising independent outputs changes no result)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", "-O3", "-mavx2", "-std=c++17", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)
_i64 = ctypes.c_int64
_int = ctypes.c_int

_SIGS = {
    "oracle_encoder_forward": (None, [_D, _I, _D, _D, _int, _int, _int]),
    "oracle_encoder_backward": (None, [_D, _D, _D, _I, _int, _int, _int]),
    "oracle_layernorm_forward": (None, [_D, _D, _D, _D, _D, _D, _i64, _int]),
    "oracle_layernorm_backward": (None, [_D, _D, _D, _D, _D, _D, _D, _D, _i64, _int]),
    "oracle_matmul_forward": (None, [_D, _D, _D, _D, _i64, _int, _int]),
    "oracle_matmul_backward": (None, [_D, _D, _D, _D, _D, _D, _i64, _int, _int]),
    "oracle_attention_forward": (None, [_D, _D, _D, _int, _int, _int, _int]),
    "oracle_attention_backward": (None, [_D, _D, _D, _D, _int, _int, _int, _int]),
    "oracle_softmax_jacobian_backward": (None, [_D, _D, _D, _int]),
    "oracle_softmax_closed_backward": (None, [_D, _D, _D, _int]),
    "oracle_gelu_forward": (None, [_D, _D, _i64]),
    "oracle_gelu_backward": (None, [_D, _D, _D, _i64]),
    "oracle_softmax_forward": (None, [_D, _D, _i64, _int]),
    "oracle_crossentropy_forward": (_int, [_D, _D, _I, _i64, _int]),
    "oracle_crossentropy_softmax_backward": (None, [_D, _D, _I, _D, _i64, _int]),
    "oracle_adamw": (None, [_i64, _D, _D, _D, _D, ctypes.c_double, ctypes.c_double,
                            ctypes.c_double, ctypes.c_double, ctypes.c_double, _int]),
    "oracle_num_params": (_i64, [_int, _int, _int, _int]),
    "oracle_sample_mult": (_int, [_D, _int, ctypes.c_double]),
    "oracle_gpt2_step": (_int, [_int, _int, _int, _int, _int, _D, _I, _I, _int, _int, _D, _D,
                                _D, _D]),
    "oracle_gpt2_step_mag": (_int, [_int, _int, _int, _int, _int, _D, _I, _I, _int, _int, _D,
                                    _D, _D, _D, _D, _D]),
}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _d(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_D)


def _i(a):
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(_I)


def f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


# ---- op-level helpers (inputs converted to fp64; outputs fresh arrays) -----------------
def encoder_forward(tok, wte, wpe):
    tok = i32(tok)
    B, T = tok.shape
    C = wte.shape[1]
    out = np.zeros((B, T, C))
    lib().oracle_encoder_forward(_d(out), _i(tok), _d(f64(wte)), _d(f64(wpe)), B, T, C)
    return out


def encoder_backward(dout, tok, V, maxT):
    tok = i32(tok)
    B, T = tok.shape
    C = dout.shape[-1]
    dwte, dwpe = np.zeros((V, C)), np.zeros((maxT, C))
    lib().oracle_encoder_backward(_d(dwte), _d(dwpe), _d(f64(dout)), _i(tok), B, T, C)
    return dwte, dwpe


def layernorm_forward(x, w, b):
    x = f64(x)
    C = x.shape[-1]
    N = x.size // C
    out = np.zeros_like(x)
    mean, rstd = np.zeros(N), np.zeros(N)
    lib().oracle_layernorm_forward(_d(out), _d(mean), _d(rstd), _d(x), _d(f64(w)), _d(f64(b)),
                                   N, C)
    return out, mean, rstd


def layernorm_backward(dout, x, w, mean, rstd):
    x = f64(x)
    C = x.shape[-1]
    N = x.size // C
    dx, dw, db = np.zeros_like(x), np.zeros(C), np.zeros(C)
    lib().oracle_layernorm_backward(_d(dx), _d(dw), _d(db), _d(f64(dout)), _d(x), _d(f64(w)),
                                    _d(f64(mean)), _d(f64(rstd)), N, C)
    return dx, dw, db


def matmul_forward(inp, W, b=None):
    inp = f64(inp)
    OC, C = W.shape
    N = inp.size // C
    out = np.zeros((N, OC))
    lib().oracle_matmul_forward(_d(out), _d(inp), _d(f64(W)), _d(None if b is None else f64(b)),
                                N, C, OC)
    return out


def matmul_backward(dout, inp, W, with_bias=True):
    inp = f64(inp)
    OC, C = W.shape
    N = inp.size // C
    dinp, dW = np.zeros((N, C)), np.zeros((OC, C))
    db = np.zeros(OC) if with_bias else None
    lib().oracle_matmul_backward(_d(dinp), _d(dW), _d(db), _d(f64(dout)), _d(inp), _d(f64(W)),
                                 N, C, OC)
    return dinp, dW, db


def attention_forward(qkv, NH):
    qkv = f64(qkv)
    B, T, C3 = qkv.shape
    C = C3 // 3
    out, att = np.zeros((B, T, C)), np.zeros((B, NH, T, T))
    lib().oracle_attention_forward(_d(out), _d(att), _d(qkv), B, T, C, NH)
    return out, att


def attention_backward(dout, qkv, att, NH):
    qkv = f64(qkv)
    B, T, C3 = qkv.shape
    C = C3 // 3
    dqkv = np.zeros_like(qkv)
    lib().oracle_attention_backward(_d(dqkv), _d(f64(dout)), _d(qkv), _d(f64(att)), B, T, C, NH)
    return dqkv


def softmax_jacobian_backward(att, datt):
    att, datt = f64(att), f64(datt)
    T = att.shape[-1]
    dpre = np.zeros_like(att)
    lib().oracle_softmax_jacobian_backward(_d(dpre), _d(att), _d(datt), T)
    return dpre


def softmax_closed_backward(att, datt):
    att, datt = f64(att), f64(datt)
    T = att.shape[-1]
    dpre = np.zeros_like(att)
    lib().oracle_softmax_closed_backward(_d(dpre), _d(att), _d(datt), T)
    return dpre


def gelu_forward(x):
    x = f64(x)
    out = np.zeros_like(x)
    lib().oracle_gelu_forward(_d(out), _d(x), x.size)
    return out


def gelu_backward(x, dout):
    x = f64(x)
    dx = np.zeros_like(x)
    lib().oracle_gelu_backward(_d(dx), _d(x), _d(f64(dout)), x.size)
    return dx


def softmax_forward(logits):
    z = f64(logits)
    V = z.shape[-1]
    out = np.zeros_like(z)
    lib().oracle_softmax_forward(_d(out), _d(z), z.size // V, V)
    return out


def crossentropy_forward(logits, targets):
    z = f64(logits)
    V = z.shape[-1]
    N = z.size // V
    losses = np.zeros(N)
    rc = lib().oracle_crossentropy_forward(_d(losses), _d(z), _i(i32(targets).reshape(-1)), N, V)
    if rc:
        raise ValueError("target outside [0, V)")
    return losses


def crossentropy_softmax_backward(logits, targets, dlosses):
    z = f64(logits)
    V = z.shape[-1]
    N = z.size // V
    dz = np.zeros((N, V))
    lib().oracle_crossentropy_softmax_backward(_d(dz), _d(z), _i(i32(targets).reshape(-1)),
                                               _d(f64(dlosses).reshape(-1)), N, V)
    return dz


def sample_mult(probs, coin) -> int:
    """Index drawn from ``probs`` (summing to 1) with ``coin`` in [0, 1)."""
    p = f64(probs).ravel()
    return int(lib().oracle_sample_mult(_d(p), p.size, float(coin)))


def adamw(p, g, m, v, lr, b1, b2, eps, wd, t):
    """Returns updated (p, m, v) as fresh fp64 arrays."""
    p, m, v = f64(p).copy(), f64(m).copy(), f64(v).copy()
    lib().oracle_adamw(p.size, _d(p), _d(f64(g)), _d(m), _d(v), lr, b1, b2, eps, wd, t)
    return p, m, v


def num_params(L, C, V, maxT) -> int:
    return int(lib().oracle_num_params(L, C, V, maxT))


def gpt2_step(shape, params, tokens, targets=None, want_logits=False, want_grads=True,
              want_losses=False, want_mags=False):
    """Forward (+ backward) of the whole model. ``shape`` has L, C, H, V, maxT.

    Returns a dict with ``loss`` (float; -1 without targets) and, on request, ``logits``
    (B,T,V), ``losses`` (B,T) and ``grads`` (flat, fp64). ``want_mags`` adds the magnitude
    envelopes used by the parity gates: ``grad_mag`` (flat, with grads) and, with logits,
    ``logit_mag`` (B,T,V) -- each entry's final sum taken over absolute values.
    """
    tokens = i32(tokens)
    B, T = tokens.shape
    tg = None if targets is None else i32(targets)
    P = num_params(shape.L, shape.C, shape.V, shape.maxT)
    params = f64(params)
    assert params.size == P
    loss = np.zeros(1)
    logits = np.zeros((B, T, shape.V)) if want_logits else None
    losses = np.zeros((B, T)) if (want_losses and tg is not None) else None
    grads = np.zeros(P) if (want_grads and tg is not None) else None
    gmag = np.zeros(P) if (want_mags and grads is not None) else None
    lmag = np.zeros((B, T, shape.V)) if (want_mags and want_logits) else None
    rc = lib().oracle_gpt2_step_mag(shape.L, shape.C, shape.H, shape.V, shape.maxT, _d(params),
                                    _i(tokens), _i(tg), B, T, _d(loss), _d(losses), _d(logits),
                                    _d(grads), _d(gmag), _d(lmag))
    if rc:
        raise ValueError("oracle_gpt2_step rejected its arguments")
    out = {"loss": float(loss[0])}
    if logits is not None:
        out["logits"] = logits
    if losses is not None:
        out["losses"] = losses
    if grads is not None:
        out["grads"] = grads
    if gmag is not None:
        out["grad_mag"] = gmag
    if lmag is not None:
        out["logit_mag"] = lmag
    return out
