"""GPU-side test plumbing: device state for a plan and comparison rules."""
from __future__ import annotations

import sys

import numpy as np
import torch

import persistent_megakernel_latency_amd as wpk


def announce(msg: str) -> None:
    """Names the case on stderr before a GPU step, flushed, so a failing run
    still says what it was doing."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    return t.to("cuda")


def from_dev(t: torch.Tensor, like: np.ndarray) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if like.dtype == np.uint16 else a


class GpuPlan:
    """A plan plus the caller-owned device buffers one step reads and writes."""

    def __init__(self, cfg, weights, batch, cap, kc, vc, seq_len, tokens, baseline=False, opts=None, desc=None,
                 static=False):
        self.cfg = cfg
        if desc is None:
            desc, self.tensors = wpk.model_from_weights(cfg, weights, "cuda")
        self.desc = desc
        self.kc_like = kc
        self.kc = to_dev(kc)
        self.vc = to_dev(vc)
        self.seq_len = torch.from_numpy(np.asarray(seq_len, np.int32).copy()).cuda()
        self.tokens = torch.from_numpy(np.asarray(tokens, np.int32).copy()).cuda()
        self.logits = torch.zeros((batch, cfg.vocab), dtype=torch.float32, device="cuda")
        self.kv = wpk.wpk_kv(self.kc.data_ptr(), self.vc.data_ptr(), self.seq_len.data_ptr())
        if baseline:
            self.plan = wpk.wpk_build_graph_baseline(self.desc.desc, batch, cap)
        elif static:
            self.plan = wpk.wpk_build_static(self.desc.desc, batch, cap)
        else:
            self.plan = wpk.wpk_build_ex(self.desc.desc, batch, cap, opts)
        assert self.plan, wpk.wpk_last_error(None)
        self.info = wpk.wpk_get_info(self.plan)

    def step(self, check: bool = True) -> int:
        rc = wpk.wpk_step(self.plan, self.tokens.data_ptr(), self.kv, self.logits.data_ptr(), 0)
        if check:
            wpk.check(rc, self.plan, "wpk_step")
        rc2 = wpk.wpk_sync(self.plan)
        if check:
            wpk.check(rc2, self.plan, "wpk_sync")
        return rc if rc != 0 else rc2

    def set_tokens(self, tok) -> None:
        self.tokens.copy_(torch.from_numpy(np.asarray(tok, np.int32)))

    def state(self):
        return (from_dev(self.kc, self.kc_like), from_dev(self.vc, self.kc_like), self.seq_len.cpu().numpy(),
                self.tokens.cpu().numpy(), self.logits.cpu().numpy())

    def log(self):
        rc, log = wpk.wpk_get_log(self.plan, self.info.n_tiles)
        wpk.check(rc, self.plan, "wpk_get_log")
        return log

    def dag(self):
        return wpk.wpk_get_dag(self.plan, self.info.n_tiles)

    def close(self):
        if self.plan:
            wpk.wpk_destroy(self.plan)
            self.plan = None


def top2_margin_f32(logits64: np.ndarray) -> float:
    v = np.sort(logits64.astype(np.float32))
    return float(v[-1] - v[-2])


def tokens_agree(gpu_tok: int, oracle_tok: int, oracle_logits: np.ndarray, max_err: float):
    """Greedy tokens must be identical unless the oracle's own top-2 margin is
    within 4x the measured logit error (a near tie, reported, not hidden)."""
    if gpu_tok == oracle_tok:
        return True, None
    margin = top2_margin_f32(oracle_logits)
    near_tie = margin <= 4.0 * max_err and oracle_logits[gpu_tok] >= oracle_logits.max() - 4.0 * max_err
    return near_tie, f"token {gpu_tok} vs {oracle_tok}, margin {margin:.3g}, max err {max_err:.3g}"
