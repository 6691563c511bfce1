"""Python access to the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline import this package.  It loads ``liboracle.so`` (plain C, float64,
OpenMP over output rows) and never touches the GPU path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

F32 = 0
BF16 = 1


def build() -> str:
    """Compile oracle.c with gcc (IEEE float64, no fast-math, no FMA contraction)."""
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                           os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm"])
    os.replace(tmp, _SO)
    return _SO


class _Model(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_double),
        ("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
        ("attn_norm", ctypes.c_void_p), ("mlp_norm", ctypes.c_void_p),
        ("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
        ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i32, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
        L.oracle_bf16_value.restype = f64
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_round_bf16.restype = ctypes.c_uint16
        L.oracle_round_bf16.argtypes = [f64]
        L.oracle_matvec.restype = None
        L.oracle_matvec.argtypes = [vp, i32, i32, i32, vp, vp]
        L.oracle_rmsnorm.restype = None
        L.oracle_rmsnorm.argtypes = [vp, vp, i32, f64, vp]
        L.oracle_rope.restype = None
        L.oracle_rope.argtypes = [vp, i32, i32, f64]
        L.oracle_silu.restype = f64
        L.oracle_silu.argtypes = [f64]
        L.oracle_attention.restype = None
        L.oracle_attention.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
        L.oracle_argmax_f32.restype = i32
        L.oracle_argmax_f32.argtypes = [vp, i32]
        L.oracle_step.restype = i32
        L.oracle_step.argtypes = [ctypes.POINTER(_Model), i32, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_prefill.restype = i32
        L.oracle_prefill.argtypes = [ctypes.POINTER(_Model), i32, i32, vp, i32, vp, vp, vp, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---- building blocks ------------------------------------------------------------

def bf16_value(bits: int) -> float:
    return lib().oracle_bf16_value(bits)


def round_bf16(x: float) -> int:
    return int(lib().oracle_round_bf16(float(x)))


def matvec(w: np.ndarray, x: np.ndarray, dtype: int) -> np.ndarray:
    rows, cols = w.shape
    w = np.ascontiguousarray(w)
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(rows, dtype=np.float64)
    lib().oracle_matvec(_ptr(w), dtype, rows, cols, _ptr(x), _ptr(y))
    return y


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float32)
    y = np.empty_like(x)
    lib().oracle_rmsnorm(_ptr(x), _ptr(g), x.size, eps, _ptr(y))
    return y


def rope(v: np.ndarray, pos: int, theta: float) -> np.ndarray:
    v = np.array(v, dtype=np.float64, copy=True)
    lib().oracle_rope(_ptr(v), v.size, pos, theta)
    return v


def silu(z: float) -> float:
    return lib().oracle_silu(float(z))


def attention(q: np.ndarray, kc: np.ndarray, vc: np.ndarray, n: int, dtype: int):
    """q [Hq][D] float64; kc, vc [Hkv][cap][D] cache dtype.  Returns (out [Hq][D], probs [Hq][n])."""
    hq, d = q.shape
    hkv, cap, d2 = kc.shape
    assert d2 == d and vc.shape == kc.shape
    q = np.ascontiguousarray(q, dtype=np.float64)
    kc = np.ascontiguousarray(kc)
    vc = np.ascontiguousarray(vc)
    out = np.empty((hq, d), dtype=np.float64)
    probs = np.empty((hq, max(n, 1)), dtype=np.float64)
    lib().oracle_attention(_ptr(q), _ptr(kc), _ptr(vc), dtype, hq, hkv, d, cap, n, _ptr(out), _ptr(probs))
    return out, probs[:, :n]


def argmax_f32(logits: np.ndarray) -> int:
    x = np.ascontiguousarray(logits, dtype=np.float64)
    return int(lib().oracle_argmax_f32(_ptr(x), x.size))


# ---- whole decode step ------------------------------------------------------------

class Model:
    """Holds a model's weights (numpy arrays in the layouts ``synth.make_weights``
    returns) and the C struct that points at them."""

    def __init__(self, cfg, weights: Dict[str, object]):
        self.cfg = cfg
        self.dtype = F32 if cfg.dtype == "f32" else BF16
        self._keep = []
        L = cfg.n_layers

        def arr(a):
            a = np.ascontiguousarray(a)
            self._keep.append(a)
            return a.ctypes.data

        def table(key):
            t = (ctypes.c_void_p * L)(*[arr(weights["layers"][l][key]) for l in range(L)])
            self._keep.append(t)
            return ctypes.cast(t, ctypes.c_void_p)

        m = _Model()
        m.n_layers, m.hidden, m.n_q_heads = L, cfg.hidden, cfg.n_q_heads
        m.n_kv_heads, m.head_dim, m.ffn, m.vocab = cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.vocab
        m.dtype = self.dtype
        m.rope_theta, m.rms_eps = cfg.rope_theta, cfg.rms_eps
        m.embed = arr(weights["embed"])
        m.final_norm = arr(np.asarray(weights["final_norm"], dtype=np.float32))
        m.attn_norm = table("attn_norm")
        m.mlp_norm = table("mlp_norm")
        m.w_qkv, m.w_o = table("w_qkv"), table("w_o")
        m.w_gate, m.w_up, m.w_down = table("w_gate"), table("w_up"), table("w_down")
        self._m = m

    def cache_dtype(self):
        return np.float32 if self.dtype == F32 else np.uint16

    def new_cache(self, batch: int, cap: int):
        shape = (self.cfg.n_layers, batch, self.cfg.n_kv_heads, cap, self.cfg.head_dim)
        return np.zeros(shape, self.cache_dtype()), np.zeros(shape, self.cache_dtype())

    def step(self, tokens, kcache, vcache, seq_len):
        """One decode step in place on (kcache, vcache, seq_len).
        Returns (logits float64 [B][V], next tokens int32 [B])."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        b = tokens.size
        cap = kcache.shape[3]
        assert kcache.flags["C_CONTIGUOUS"] and vcache.flags["C_CONTIGUOUS"]
        assert seq_len.dtype == np.int32 and seq_len.flags["C_CONTIGUOUS"]
        logits = np.empty((b, self.cfg.vocab), dtype=np.float64)
        out = np.empty(b, dtype=np.int32)
        rc = lib().oracle_step(ctypes.byref(self._m), b, cap, _ptr(tokens), _ptr(kcache), _ptr(vcache),
                               _ptr(seq_len), _ptr(logits), _ptr(out))
        if rc != 0:
            raise RuntimeError(f"oracle_step failed ({rc})")
        return logits, out

    def prefill(self, prompt, kcache, vcache, seq_len):
        """Teacher-forced prefill of prompt [B][T]; returns the last logits and the next tokens."""
        prompt = np.ascontiguousarray(prompt, dtype=np.int32)
        b, t = prompt.shape
        cap = kcache.shape[3]
        logits = np.empty((b, self.cfg.vocab), dtype=np.float64)
        out = np.empty(b, dtype=np.int32)
        rc = lib().oracle_prefill(ctypes.byref(self._m), b, cap, _ptr(prompt), t, _ptr(kcache),
                                  _ptr(vcache), _ptr(seq_len), _ptr(logits), _ptr(out))
        if rc != 0:
            raise RuntimeError(f"oracle_prefill failed ({rc})")
        return logits, out
