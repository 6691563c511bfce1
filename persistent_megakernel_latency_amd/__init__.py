"""Python binding of libwpk.so, the gfx950 decode-step megakernel.

Argument marshalling only: every function below calls the C entry point of the
same name (declared in include/wpk.h); every step of the decode path runs in
the library's kernels.  PyTorch is used by callers for device memory and
streams; the binding takes raw pointers (``tensor.data_ptr()``).

If libwpk.so has not been built, importing works but the first call raises:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwpk.so")

WPK_OK = 0
WPK_E_ARG = -1
WPK_E_NOMEM = -2
WPK_E_HIP = -3
WPK_E_OCCUPANCY = -4
WPK_E_TIMEOUT = -5
WPK_E_CTX_FULL = -6
WPK_E_TOKEN = -7
WPK_E_STATE = -8
WPK_E_NO_GPU = -9
WPK_E_IDLE = -10
WPK_E_RANGE = -11

WPK_F32 = 0
WPK_BF16 = 1

WPK_STATIC_SCRATCH_BYTES = 32 << 20

WPK_OPT_LOG = 1
WPK_OPT_WATCHDOG_US = 2
WPK_OPT_PERTURB_SEED = 3
WPK_OPT_DEBUG_DROP_TILE = 4
WPK_OPT_RESET = 5
WPK_OPT_PREFETCH = 6
WPK_OPT_WORKERS = 7
WPK_OPT_LAUNCH = 8
WPK_OPT_FIXED_REDUCER = 9
WPK_OPT_PERSIST_IDLE_US = 10

TILE_TYPES = ["qkv", "attn", "combine", "oproj", "gateup", "down", "lm", "argmax", "norm", "norm2", "normf",
              "attnc"]

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class wpk_model_desc(ctypes.Structure):
    _fields_ = [
        ("n_layers", _i32), ("hidden", _i32), ("n_q_heads", _i32), ("n_kv_heads", _i32),
        ("head_dim", _i32), ("ffn", _i32), ("vocab", _i32), ("tied_embeddings", _i32),
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("dtype", _i32),
        ("embed", _vp), ("final_norm", _vp),
        ("attn_norm", _vp), ("w_qkv", _vp), ("w_o", _vp), ("mlp_norm", _vp),
        ("w_gate", _vp), ("w_up", _vp), ("w_down", _vp),
    ]


class wpk_kv(ctypes.Structure):
    _fields_ = [("k", _vp), ("v", _vp), ("seq_len", _vp)]


class wpk_build_opts(ctypes.Structure):
    _fields_ = [("tile_bytes", _i32), ("workers_per_cu", _i32), ("queue_shards", _i32), ("attn_chunk", _i32),
                ("forward", _i32), ("barrier_edges", _i32), ("split_workers", _i32)]


class wpk_log_rec(ctypes.Structure):
    _fields_ = [("exec_count", _i32), ("wait_delta", _i32), ("worker", _i32), ("claim", _i32),
                ("t_start", ctypes.c_int64), ("t_end", ctypes.c_int64)]


class wpk_plan_info(ctypes.Structure):
    _fields_ = [("n_tiles", _i32), ("n_groups", _i32), ("n_queue_shards", _i32), ("workers", _i32),
                ("max_workers", _i32), ("rows_per_tile_h", _i32), ("rows_per_tile_f", _i32),
                ("attn_chunk", _i32), ("workspace_bytes", ctypes.c_int64), ("weight_bytes", ctypes.c_int64)]


WPK_SIM_TYPES = 12


class wpk_sim_params(ctypes.Structure):
    _fields_ = [("hbm_GBps", ctypes.c_double), ("load_latency_us", ctypes.c_double), ("hop_us", ctypes.c_double),
                ("launch_gap_us", ctypes.c_double), ("workers", _i32), ("prefetch", _i32), ("conventional", _i32),
                ("slots", _i32), ("stage_us", ctypes.c_double * WPK_SIM_TYPES),
                ("compute_us", ctypes.c_double * WPK_SIM_TYPES), ("epilogue_us", ctypes.c_double * WPK_SIM_TYPES),
                ("reduce_us", ctypes.c_double * WPK_SIM_TYPES)]


class wpk_sim_result(ctypes.Structure):
    _fields_ = [("step_us", ctypes.c_double), ("hbm_bytes", ctypes.c_double), ("achieved_GBps", ctypes.c_double),
                ("worker_busy_frac", ctypes.c_double)]


WPK_PREFILL_MEGAKERNEL = 0
WPK_PREFILL_SPLIT = 1
WPK_PREFILL_GRAPH = 2

PREFILL_TILE_TYPES = ["embed", "norm1", "qkv", "attn", "oproj", "norm2", "gateup", "down", "normf", "lm", "argmax"]


class wpk_prefill_opts(ctypes.Structure):
    _fields_ = [("mode", _i32), ("split_workers", _i32), ("workers_per_cu", _i32)]


class wpk_prefill_info(ctypes.Structure):
    _fields_ = [("n_tiles", _i32), ("n_groups", _i32), ("n_queues", _i32), ("workers", _i32), ("max_workers", _i32),
                ("split_workers", _i32), ("n_phases", _i32), ("rows_per_sequence", _i32),
                ("workspace_bytes", ctypes.c_int64), ("flops", ctypes.c_double)]


class wpk_prefill_sim_params(ctypes.Structure):
    _fields_ = [("tile_us", ctypes.c_double * 11), ("attn_step_us", ctypes.c_double), ("hop_us", ctypes.c_double),
                ("launch_gap_us", ctypes.c_double), ("workers", _i32), ("split_workers", _i32),
                ("conventional", _i32), ("pad", _i32)]


# Every symbol include/wpk.h declares, with its ctypes signature.
_SIGNATURES = {
    "wpk_build": (_vp, [ctypes.POINTER(wpk_model_desc), _i32, _i32]),
    "wpk_build_ex": (_vp, [ctypes.POINTER(wpk_model_desc), _i32, _i32, ctypes.POINTER(wpk_build_opts)]),
    "wpk_step": (_i32, [_vp, _vp, ctypes.POINTER(wpk_kv), _vp, _vp]),
    "wpk_sync": (_i32, [_vp]),
    "wpk_destroy": (None, [_vp]),
    "wpk_last_error": (ctypes.c_char_p, [_vp]),
    "wpk_set_option": (_i32, [_vp, _i32, ctypes.c_int64]),
    "wpk_get_log": (_i32, [_vp, _vp, ctypes.c_size_t]),
    "wpk_get_info": (_i32, [_vp, ctypes.POINTER(wpk_plan_info)]),
    "wpk_get_dag": (_i32, [_vp, _vp, _vp, _vp, _vp]),
    "wpk_build_graph_baseline": (_vp, [ctypes.POINTER(wpk_model_desc), _i32, _i32]),
    "wpk_build_static": (_vp, [ctypes.POINTER(wpk_model_desc), _i32, _i32]),
    "wpk_simulate": (_i32, [_vp, ctypes.POINTER(wpk_sim_params), _vp, ctypes.POINTER(wpk_sim_result)]),
    "wpk_persist_begin": (_i32, [_vp, _vp, ctypes.POINTER(wpk_kv), _vp, _vp]),
    "wpk_persist_ring": (_i32, [_vp, _i32]),
    "wpk_persist_wait": (_i32, [_vp, _i32, ctypes.c_int64]),
    "wpk_persist_end": (_i32, [_vp]),
    "wpk_persist_times": (_i32, [_vp, _vp, _i32]),
    "wpk_build_host": (_vp, [ctypes.POINTER(wpk_model_desc), _i32, _i32, ctypes.POINTER(wpk_build_opts)]),
    "wpk_serial_step": (_i32, [_vp, _vp, ctypes.POINTER(wpk_kv), _vp, ctypes.c_uint64, _i32]),
    "wpk_emulate_step": (_i32, [_vp, _vp, ctypes.POINTER(wpk_kv), _vp, _i32, ctypes.c_uint64]),
    "wpk_debug_drop_edge": (_i32, [_vp, _i32]),
    "wpk_debug_read_act": (_i32, [_vp, _vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]),
    "wpk_build_prefill": (_vp, [ctypes.POINTER(wpk_model_desc), _i32, _i32, _i32, ctypes.POINTER(wpk_prefill_opts)]),
    "wpk_build_prefill_host": (_vp, [ctypes.POINTER(wpk_model_desc), _i32, _i32, _i32,
                                     ctypes.POINTER(wpk_prefill_opts)]),
    "wpk_prefill": (_i32, [_vp, _vp, ctypes.POINTER(wpk_kv), _vp, _vp, _vp]),
    "wpk_prefill_sync": (_i32, [_vp]),
    "wpk_prefill_destroy": (None, [_vp]),
    "wpk_prefill_last_error": (ctypes.c_char_p, [_vp]),
    "wpk_prefill_set_option": (_i32, [_vp, _i32, ctypes.c_int64]),
    "wpk_prefill_get_log": (_i32, [_vp, _vp, ctypes.c_size_t]),
    "wpk_prefill_get_info": (_i32, [_vp, ctypes.POINTER(wpk_prefill_info)]),
    "wpk_prefill_get_dag": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp]),
    "wpk_prefill_simulate": (_i32, [_vp, ctypes.POINTER(wpk_prefill_sim_params), ctypes.POINTER(wpk_sim_result)]),
    "wpk_prefill_get_key_steps": (_i32, [_vp, _vp]),
}

_lib = None


def lib():
    """The loaded libwpk.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m persistent_megakernel_latency_amd.build` "
                               "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def symbols() -> List[str]:
    return list(_SIGNATURES)


# ---- the C entry points, same names --------------------------------------------------

def wpk_build(desc: wpk_model_desc, batch: int, ctx_len: int):
    return lib().wpk_build(ctypes.byref(desc), batch, ctx_len)


def wpk_build_ex(desc: wpk_model_desc, batch: int, ctx_len: int, opts: Optional[wpk_build_opts] = None):
    return lib().wpk_build_ex(ctypes.byref(desc), batch, ctx_len, ctypes.byref(opts) if opts else None)


def wpk_step(plan, tokens_ptr: int, kv: wpk_kv, logits_ptr: int, stream_ptr: int = 0) -> int:
    return lib().wpk_step(plan, tokens_ptr, ctypes.byref(kv), logits_ptr, stream_ptr or None)


def wpk_sync(plan) -> int:
    return lib().wpk_sync(plan)


def wpk_destroy(plan) -> None:
    lib().wpk_destroy(plan)


def wpk_last_error(plan=None) -> str:
    r = lib().wpk_last_error(plan)
    return r.decode() if r else ""


def wpk_set_option(plan, key: int, value: int) -> int:
    return lib().wpk_set_option(plan, key, value)


def wpk_get_log(plan, n_tiles: int):
    buf = (wpk_log_rec * n_tiles)()
    rc = lib().wpk_get_log(plan, ctypes.cast(buf, _vp), ctypes.sizeof(buf))
    return rc, buf


def wpk_get_info(plan) -> wpk_plan_info:
    info = wpk_plan_info()
    rc = lib().wpk_get_info(plan, ctypes.byref(info))
    if rc != WPK_OK:
        raise RuntimeError(f"wpk_get_info failed: {rc}")
    return info


def wpk_get_dag(plan, n_tiles: int):
    arrs = [(_i32 * n_tiles)() for _ in range(4)]
    rc = lib().wpk_get_dag(plan, *[ctypes.cast(a, _vp) for a in arrs])
    if rc != WPK_OK:
        raise RuntimeError(f"wpk_get_dag failed: {rc}")
    return [list(a) for a in arrs]


def wpk_build_graph_baseline(desc: wpk_model_desc, batch: int, ctx_len: int):
    return lib().wpk_build_graph_baseline(ctypes.byref(desc), batch, ctx_len)


def wpk_build_static(desc: wpk_model_desc, batch: int, ctx_len: int):
    return lib().wpk_build_static(ctypes.byref(desc), batch, ctx_len)


def wpk_simulate(plan, params: wpk_sim_params, positions=None):
    """(rc, wpk_sim_result) of the simulated step; positions: int32 per sequence or None."""
    import numpy as np
    res = wpk_sim_result()
    ptr = None
    if positions is not None:
        positions = np.ascontiguousarray(positions, dtype=np.int32)
        ptr = positions.ctypes.data
    rc = lib().wpk_simulate(plan, ctypes.byref(params), ptr, ctypes.byref(res))
    return rc, res


def wpk_persist_begin(plan, tokens_ptr: int, kv: wpk_kv, logits_ptr: int, stream_ptr: int = 0) -> int:
    return lib().wpk_persist_begin(plan, tokens_ptr, ctypes.byref(kv), logits_ptr, stream_ptr or None)


def wpk_persist_ring(plan, n_steps: int) -> int:
    return lib().wpk_persist_ring(plan, n_steps)


def wpk_persist_wait(plan, steps: int, timeout_us: int = -1) -> int:
    return lib().wpk_persist_wait(plan, steps, timeout_us)


def wpk_persist_end(plan) -> int:
    return lib().wpk_persist_end(plan)


def wpk_persist_times(plan, n_steps: int):
    """(rc, int64 array [n_steps][2]) of s_memrealtime stamps: grant seen, last worker out."""
    import numpy as np
    out = np.zeros((n_steps, 2), np.int64)
    rc = lib().wpk_persist_times(plan, out.ctypes.data, n_steps)
    return rc, out


def wpk_build_host(desc: wpk_model_desc, batch: int, ctx_len: int, opts: Optional[wpk_build_opts] = None):
    return lib().wpk_build_host(ctypes.byref(desc), batch, ctx_len, ctypes.byref(opts) if opts else None)


def wpk_serial_step(plan, tokens_ptr: int, kv: wpk_kv, logits_ptr: int, order_seed: int, poison: bool) -> int:
    return lib().wpk_serial_step(plan, tokens_ptr, ctypes.byref(kv), logits_ptr, order_seed, int(poison))


def wpk_emulate_step(plan, tokens_ptr: int, kv: wpk_kv, logits_ptr: int, n_threads: int, seed: int) -> int:
    return lib().wpk_emulate_step(plan, tokens_ptr, ctypes.byref(kv), logits_ptr, n_threads, seed)


def wpk_debug_drop_edge(plan, tile: int) -> int:
    return lib().wpk_debug_drop_edge(plan, tile)


def wpk_debug_read_act(plan):
    """The plan's activation arena as float32 (host executors' layout)."""
    import numpy as np
    n = ctypes.c_size_t(0)
    check(lib().wpk_debug_read_act(plan, None, 0, ctypes.byref(n)), plan, "wpk_debug_read_act")
    out = np.empty(n.value // 4, np.float32)
    check(lib().wpk_debug_read_act(plan, out.ctypes.data, n.value, ctypes.byref(n)), plan, "wpk_debug_read_act")
    return out


# ---- prompt prefill ---------------------------------------------------------------------

def wpk_build_prefill(desc: wpk_model_desc, batch: int, ctx_len: int, prompt_len: int,
                      opts: Optional[wpk_prefill_opts] = None):
    return lib().wpk_build_prefill(ctypes.byref(desc), batch, ctx_len, prompt_len,
                                   ctypes.byref(opts) if opts else None)


def wpk_build_prefill_host(desc: wpk_model_desc, batch: int, ctx_len: int, prompt_len: int,
                           opts: Optional[wpk_prefill_opts] = None):
    return lib().wpk_build_prefill_host(ctypes.byref(desc), batch, ctx_len, prompt_len,
                                        ctypes.byref(opts) if opts else None)


def wpk_prefill(plan, prompt_ptr: int, kv: wpk_kv, logits_ptr: int, tokens_out_ptr: int, stream_ptr: int = 0) -> int:
    return lib().wpk_prefill(plan, prompt_ptr, ctypes.byref(kv), logits_ptr, tokens_out_ptr, stream_ptr or None)


def wpk_prefill_sync(plan) -> int:
    return lib().wpk_prefill_sync(plan)


def wpk_prefill_destroy(plan) -> None:
    lib().wpk_prefill_destroy(plan)


def wpk_prefill_last_error(plan=None) -> str:
    r = lib().wpk_prefill_last_error(plan)
    return r.decode() if r else ""


def wpk_prefill_set_option(plan, key: int, value: int) -> int:
    return lib().wpk_prefill_set_option(plan, key, value)


def wpk_prefill_get_log(plan, n_tiles: int):
    buf = (wpk_log_rec * n_tiles)()
    rc = lib().wpk_prefill_get_log(plan, ctypes.cast(buf, _vp), ctypes.sizeof(buf))
    return rc, buf


def wpk_prefill_get_info(plan) -> wpk_prefill_info:
    info = wpk_prefill_info()
    rc = lib().wpk_prefill_get_info(plan, ctypes.byref(info))
    if rc != WPK_OK:
        raise RuntimeError(f"wpk_prefill_get_info failed: {rc}")
    return info


def wpk_prefill_get_dag(plan, n_tiles: int):
    """[type, layer, wait, signal, queue] lists, one entry per tile id."""
    arrs = [(_i32 * n_tiles)() for _ in range(5)]
    rc = lib().wpk_prefill_get_dag(plan, *[ctypes.cast(a, _vp) for a in arrs])
    if rc != WPK_OK:
        raise RuntimeError(f"wpk_prefill_get_dag failed: {rc}")
    return [list(a) for a in arrs]


def wpk_prefill_simulate(plan, params: wpk_prefill_sim_params):
    """(rc, wpk_sim_result) of the simulated prefill design."""
    res = wpk_sim_result()
    rc = lib().wpk_prefill_simulate(plan, ctypes.byref(params), ctypes.byref(res))
    return rc, res


def wpk_prefill_get_key_steps(plan, n_tiles: int):
    arr = (_i32 * n_tiles)()
    rc = lib().wpk_prefill_get_key_steps(plan, ctypes.cast(arr, _vp))
    if rc != WPK_OK:
        raise RuntimeError(f"wpk_prefill_get_key_steps failed: {rc}")
    return list(arr)


def check_prefill(rc: int, plan=None, what: str = "wpk_prefill call") -> None:
    if rc != WPK_OK:
        raise RuntimeError(f"{what} failed ({rc}): {wpk_prefill_last_error(plan)}")


def prefill_source_hash() -> str:
    """Hash of the sources that decide what the prefill kernels do."""
    import hashlib
    h = hashlib.sha256()
    for f in ("prefill.hip", "prefill_plan.h", "prefill_builder.cpp", "prefill_builder.h", "prefill_capi.cpp",
              "worker.h", "plan.h"):
        with open(os.path.join(_HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---- descriptor marshalling ------------------------------------------------------------

class ModelDesc:
    """A wpk_model_desc plus the pointer tables it refers to.

    ``ptrs`` maps "embed", "final_norm" to addresses and "attn_norm", "w_qkv",
    "w_o", "mlp_norm", "w_gate", "w_up", "w_down" to per-layer address lists.
    The caller keeps the memory those addresses point to alive."""

    def __init__(self, cfg, ptrs: Dict[str, object], keep: Sequence[object] = ()):
        self._keep = list(keep)
        d = wpk_model_desc()
        d.n_layers, d.hidden, d.n_q_heads = cfg.n_layers, cfg.hidden, cfg.n_q_heads
        d.n_kv_heads, d.head_dim, d.ffn, d.vocab = cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.vocab
        d.tied_embeddings = 1
        d.rope_theta, d.rms_eps = cfg.rope_theta, cfg.rms_eps
        d.dtype = WPK_F32 if cfg.dtype == "f32" else WPK_BF16
        d.embed = ptrs["embed"]
        d.final_norm = ptrs["final_norm"]
        for key in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down"):
            table = (_vp * cfg.n_layers)(*ptrs[key])
            self._keep.append(table)
            setattr(d, key, ctypes.cast(table, _vp))
        self.desc = d


def _tensor_of(a, device):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def model_from_weights(cfg, weights: Dict[str, object], device="cuda"):
    """Copies synth-layout weights (numpy) to `device` tensors and returns
    (ModelDesc, tensors); the tensors must outlive any plan built from it."""
    tensors: Dict[str, object] = {"embed": _tensor_of(weights["embed"], device),
                                  "final_norm": _tensor_of(weights["final_norm"], device), "layers": []}
    for lw in weights["layers"]:
        tensors["layers"].append({k: _tensor_of(v, device) for k, v in lw.items()})
    ptrs: Dict[str, object] = {"embed": tensors["embed"].data_ptr(), "final_norm": tensors["final_norm"].data_ptr()}
    for key in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down"):
        ptrs[key] = [lt[key].data_ptr() for lt in tensors["layers"]]
    keep = [tensors["embed"], tensors["final_norm"]] + [t for lt in tensors["layers"] for t in lt.values()]
    return ModelDesc(cfg, ptrs, keep), tensors


def source_hash() -> str:
    """Hash of the sources that decide what the megakernel does at run time
    (kernel, tile geometry, DAG builder, launch path); recorded profiles are
    only reported while it matches."""
    import hashlib
    h = hashlib.sha256()
    for f in ("megakernel.hip", "worker.h", "wide_layout.h", "persist.hip", "plan.h", "builder.cpp", "builder.h",
              "capi.cpp", "runtime.h"):
        with open(os.path.join(_HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def check(rc: int, plan=None, what: str = "wpk call") -> None:
    if rc != WPK_OK:
        raise RuntimeError(f"{what} failed ({rc}): {wpk_last_error(plan)}")
