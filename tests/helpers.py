"""Shared test plumbing: host descriptors, KV state, DAG/log checks."""
from __future__ import annotations

import re
import os
from typing import Dict, List

import numpy as np

import persistent_megakernel_latency_amd as wpk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols() -> List[str]:
    """Function names include/wpk.h declares."""
    src = open(os.path.join(ROOT, "include", "wpk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wpk_[a-z_]+)\s*\(", src)))


def host_desc(cfg, weights: Dict[str, object]) -> wpk.ModelDesc:
    """A descriptor pointing at numpy arrays (for the host executors)."""
    keep = []

    def ptr(a):
        a = np.ascontiguousarray(a)
        keep.append(a)
        return a.ctypes.data

    ptrs = {"embed": ptr(weights["embed"]), "final_norm": ptr(np.asarray(weights["final_norm"], np.float32))}
    for key in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down"):
        ptrs[key] = [ptr(lw[key]) for lw in weights["layers"]]
    return wpk.ModelDesc(cfg, ptrs, keep)


def dummy_desc(cfg) -> wpk.ModelDesc:
    """Non-null but never dereferenced pointers, for building a DAG only."""
    fake = 0x1000
    ptrs = {"embed": fake, "final_norm": fake}
    for key in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down"):
        ptrs[key] = [fake] * cfg.n_layers
    return wpk.ModelDesc(cfg, ptrs)


class HostState:
    """KV cache, seq_len and token buffers in host memory, shaped for a plan."""

    def __init__(self, kc: np.ndarray, vc: np.ndarray, seq_len: np.ndarray, tokens: np.ndarray, vocab: int):
        self.kc = np.ascontiguousarray(kc).copy()
        self.vc = np.ascontiguousarray(vc).copy()
        self.seq_len = np.ascontiguousarray(seq_len, dtype=np.int32).copy()
        self.tokens = np.ascontiguousarray(tokens, dtype=np.int32).copy()
        self.logits = np.zeros((len(self.tokens), vocab), np.float32)
        self.kv = wpk.wpk_kv(self.kc.ctypes.data, self.vc.ctypes.data, self.seq_len.ctypes.data)

    def serial(self, plan, seed: int, poison: bool = False) -> int:
        return wpk.wpk_serial_step(plan, self.tokens.ctypes.data, self.kv, self.logits.ctypes.data, seed, poison)

    def emulate(self, plan, threads: int, seed: int) -> int:
        return wpk.wpk_emulate_step(plan, self.tokens.ctypes.data, self.kv, self.logits.ctypes.data, threads, seed)


def dag_edges(wait: List[int], signal: List[int]):
    """Producer lists per group: edge u -> v iff signal[u] == wait[v]."""
    prod: Dict[int, List[int]] = {}
    for u, s in enumerate(signal):
        if s >= 0:
            prod.setdefault(s, []).append(u)
    return prod


LOG_DTYPE = np.dtype([("exec_count", "<i4"), ("wait_delta", "<i4"), ("worker", "<i4"), ("claim", "<i4"),
                      ("t_start", "<i8"), ("t_end", "<i8")])


def log_array(log) -> np.ndarray:
    """The wpk_log_rec records as a numpy structured array (no copy)."""
    return np.frombuffer(log, dtype=LOG_DTYPE)


def check_log(log, wait, signal, canonical_only: bool = False) -> None:
    """Canonical log: every tile ran once with its counter exactly complete;
    and the raw order is a linear extension of the DAG (every producer ended
    before its consumer started)."""
    a = log_array(log)
    wait = np.asarray(wait, np.int64)
    signal = np.asarray(signal, np.int64)
    n = len(wait)
    a = a[:n]
    ex, de = a["exec_count"], a["wait_delta"]
    assert np.all(ex == 1), f"tiles not run exactly once: {np.nonzero(ex != 1)[0][:10]}"
    assert np.all(de == 0), f"counters not exactly complete at start: {np.nonzero(de != 0)[0][:10]}"
    if canonical_only:
        return
    start, end = a["t_start"], a["t_end"]
    n_groups = int(max(wait.max(), signal.max())) + 1
    last_end = np.full(n_groups, np.iinfo(np.int64).min, np.int64)
    prod = signal >= 0
    np.maximum.at(last_end, signal[prod], end[prod])
    cons = np.nonzero(wait >= 0)[0]
    bad = cons[last_end[wait[cons]] > start[cons]]
    assert bad.size == 0, f"tiles started before a producer ended: {bad[:10]}"
