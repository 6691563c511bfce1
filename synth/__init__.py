"""Seeded synthetic inputs: model shapes, weights, prompts, context lengths, KV.

This package only draws numbers (counter-based splitmix64 + Box-Muller, in
``synth.c``); it holds none of the decode step's arithmetic, and both the CPU
oracle and the GPU path take their inputs from it.

Seeds follow one fixed recipe: weights seed 0, prompt tokens seed 1, context
lengths seed 2, synthetic KV seed 3.  Each tensor draws from its own stream of
its seed (stream ids below), so changing one tensor's shape never shifts
another's values.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

SEED_WEIGHTS = 0
SEED_TOKENS = 1
SEED_LENGTHS = 2
SEED_KV = 3


def build() -> str:
    """Compile synth.c into libsynth.so (gcc, OpenMP)."""
    src = os.path.join(_HERE, "synth.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", src, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, i64, i32, f64 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        lib.synth_splitmix64.restype = u64
        lib.synth_splitmix64.argtypes = [u64, u64]
        lib.synth_normal_f32.restype = None
        lib.synth_normal_f32.argtypes = [u64, u64, i64, f64, f64, ctypes.c_void_p]
        lib.synth_normal_bf16.restype = None
        lib.synth_normal_bf16.argtypes = [u64, u64, i64, f64, f64, ctypes.c_void_p]
        lib.synth_uniform_i32.restype = None
        lib.synth_uniform_i32.argtypes = [u64, u64, i64, i32, i32, ctypes.c_void_p]
        _lib = lib
    return _lib


def splitmix64(seed: int, k: int) -> int:
    return int(_load().synth_splitmix64(seed, k))


def normal(seed: int, stream: int, shape, scale: float = 1.0, mean: float = 0.0,
           dtype: str = "f32") -> np.ndarray:
    """N(mean, scale^2) draws; dtype "f32" -> float32, "bf16" -> uint16 bf16 bits."""
    n = int(np.prod(shape))
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        _load().synth_normal_f32(seed, stream, n, mean, scale, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        _load().synth_normal_bf16(seed, stream, n, mean, scale, out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def uniform_int(seed: int, stream: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform in [lo, hi)."""
    if hi <= lo:
        raise ValueError("empty range")
    out = np.empty(n, dtype=np.int32)
    _load().synth_uniform_i32(seed, stream, n, lo, hi, out.ctypes.data)
    return out


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    """Shape of a Llama-style decoder (pre-norm, GQA, SwiGLU, tied LM head)."""

    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    dtype: str  # "f32" or "bf16": weights and KV cache
    rope_theta: float = 500000.0
    rms_eps: float = 1e-5

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def n_matrix_params(self) -> int:
        h, f = self.hidden, self.ffn
        per_layer = self.qkv_rows * h + h * self.n_q_heads * self.head_dim + 3 * f * h
        return self.n_layers * per_layer + self.vocab * h

    def n_norm_params(self) -> int:
        return (2 * self.n_layers + 1) * self.hidden

    def n_params(self) -> int:
        return self.n_matrix_params() + self.n_norm_params()

    def weight_bytes(self) -> int:
        """Bytes of all weights as laid out here: matrices in the model dtype,
        RMSNorm gains in float32."""
        return self.n_matrix_params() * self.elt_bytes + self.n_norm_params() * 4


# The decoder shapes the measurements are quoted on.
TINY = ModelConfig("tiny", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                   ffn=1024, vocab=1024, dtype="f32")
LLAMA_1B = ModelConfig("llama-3.2-1b-shape", n_layers=16, hidden=2048, n_q_heads=32,
                       n_kv_heads=8, head_dim=64, ffn=8192, vocab=128256, dtype="bf16")
# A small bf16 decoder whose LM-head tile count is ragged (vocab 1000 is not a
# multiple of the rows per tile) for parity tests that cover partial tiles.
MINI = ModelConfig("mini-ragged", n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2,
                   head_dim=64, ffn=1024, vocab=1000, dtype="bf16")

# Stream ids within SEED_WEIGHTS.
_S_EMBED = 1
_S_FINAL_NORM = 2


def _layer_stream(layer: int, what: str) -> int:
    idx = {"w_qkv": 0, "w_o": 1, "w_gate": 2, "w_up": 3, "w_down": 4,
           "attn_norm": 5, "mlp_norm": 6}[what]
    return 16 + 8 * layer + idx


def make_weights(cfg: ModelConfig, weight_std: float = 0.02, gain_std: float = 0.0,
                 seed: int = SEED_WEIGHTS) -> Dict[str, object]:
    """Random-init weights, all matrices N(0, weight_std^2), row-major [out][in].

    Norm gains are 1 + N(0, gain_std^2) in float32 (gain_std = 0 gives the
    plain all-ones init).  Matrices are float32 for dtype "f32" and bf16 bits
    (uint16) for dtype "bf16".
    """
    h, d = cfg.hidden, cfg.head_dim
    w: Dict[str, object] = {}
    w["embed"] = normal(seed, _S_EMBED, (cfg.vocab, h), weight_std, dtype=cfg.dtype)
    w["final_norm"] = _gain(seed, _S_FINAL_NORM, h, gain_std)
    layers: List[Dict[str, np.ndarray]] = []
    shapes = {
        "w_qkv": (cfg.qkv_rows, h),
        "w_o": (h, cfg.n_q_heads * d),
        "w_gate": (cfg.ffn, h),
        "w_up": (cfg.ffn, h),
        "w_down": (h, cfg.ffn),
    }
    for l in range(cfg.n_layers):
        lw = {k: normal(seed, _layer_stream(l, k), s, weight_std, dtype=cfg.dtype)
              for k, s in shapes.items()}
        lw["attn_norm"] = _gain(seed, _layer_stream(l, "attn_norm"), h, gain_std)
        lw["mlp_norm"] = _gain(seed, _layer_stream(l, "mlp_norm"), h, gain_std)
        layers.append(lw)
    w["layers"] = layers
    return w


def _gain(seed: int, stream: int, n: int, gain_std: float) -> np.ndarray:
    if gain_std == 0.0:
        return np.ones(n, dtype=np.float32)
    return normal(seed, stream, (n,), gain_std, mean=1.0, dtype="f32")


def prompt_tokens(cfg: ModelConfig, batch: int, length: int, seed: int = SEED_TOKENS) -> np.ndarray:
    """[batch][length] token ids uniform in [0, vocab)."""
    return uniform_int(seed, 0, batch * length, 0, cfg.vocab).reshape(batch, length)


def context_lengths(batch: int, lo: int = 256, hi: int = 1024, seed: int = SEED_LENGTHS) -> np.ndarray:
    """Per-sequence cached lengths uniform in [lo, hi] (inclusive)."""
    return uniform_int(seed, 0, batch, lo, hi + 1)


def synthetic_kv(cfg: ModelConfig, batch: int, cap: int, lengths, kv_std: Optional[float] = None,
                 seed: int = SEED_KV):
    """Random KV cache contents, layout [L][B][Hkv][cap][D] for K and for V.

    Positions below lengths[b] hold N(0, kv_std^2) values (default
    0.02 * sqrt(hidden), the scale of a random-init K/V projection of a
    unit-RMS input); positions at or above it hold zeros.
    """
    if kv_std is None:
        kv_std = 0.02 * float(np.sqrt(cfg.hidden))
    shape = (batch, cfg.n_kv_heads, cap, cfg.head_dim)
    ks, vs = [], []
    pos = np.arange(cap)[None, None, :, None]
    mask = pos < np.asarray(lengths).reshape(batch, 1, 1, 1)
    for l in range(cfg.n_layers):
        for kind, dst in ((0, ks), (1, vs)):
            a = normal(seed, 2 * l + kind, shape, kv_std, dtype=cfg.dtype)
            a = np.where(mask, a, np.zeros((), dtype=a.dtype))
            dst.append(a)
    return np.stack(ks), np.stack(vs)
