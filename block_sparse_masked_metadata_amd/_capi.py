"""ctypes binding of libbsm.so: one Python function per C entry point, same names.

Argument marshalling only: host arrays are passed as numpy buffers, device
buffers as integer addresses, streams as integer hipStream_t handles.  Every
non-zero status raises BsmError with the library's error text.  The library is
opened at the first call into it (so the package imports, and builds itself,
from a tree where libbsm.so does not exist yet); that call raises ImportError
when the library has not been built.  There is no other implementation to fall
back to.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("BSM_LIB") or os.path.join(_HERE, "libbsm.so")  # BSM_LIB: alternate build

# PyTorch-ROCm ships its own HIP runtime (same SONAME as the system one).  Load
# torch first so that libbsm binds to the runtime already in the process; two
# HIP runtimes in one process crash.
try:
    import torch  # noqa: F401
except ImportError:  # the C ABI itself does not need torch
    pass


BSM_OK, BSM_E_INVALID, BSM_E_UNSUPPORTED, BSM_E_NOMEM, BSM_E_HIP = 0, -1, -2, -3, -4
BSM_WINDOW_INF = 0x7FFFFFFF
BSM_ORDER_CONTIGUOUS, BSM_ORDER_PTRR, BSM_ORDER_EXPLICIT = 0, 1, 2
BSM_TILE_EMPTY, BSM_TILE_PARTIAL, BSM_TILE_FULL = 0, 1, 2
BSM_FWD_KEEP_STATE = 1
BSM_FWD_STEP_ONLY = 2
BSM_CALL_FULL, BSM_CALL_CAUSAL, BSM_CALL_REVERSE, BSM_CALL_PAST_WINDOW = 0, 1, 2, 3

ORDERS = {"contiguous": BSM_ORDER_CONTIGUOUS, "ptrr": BSM_ORDER_PTRR,
          "explicit": BSM_ORDER_EXPLICIT}

EXPORTS = [
    "bsm_last_error", "bsm_version", "bsm_plan_build", "bsm_plan_free", "bsm_plan_get_info",
    "bsm_plan_permutation", "bsm_plan_block_cost", "bsm_plan_step_map", "bsm_plan_pairs",
    "bsm_plan_key_intervals", "bsm_plan_fetch_set", "bsm_plan_chunk_order", "bsm_fwd_fetched",
    "bsm_dplan_bytes", "bsm_dplan_upload", "bsm_dplan_free", "bsm_dplan_get_info",
    "bsm_fwd_step", "bsm_fwd_step_chain", "bsm_fwd_single", "bsm_fwd_merge_bf16", "bsm_fwd_merge_fp32",
    "bsm_bwd_prep", "bsm_bwd_step", "bsm_plan_dense_calls", "bsm_dplan_calls_bytes",
    "bsm_dplan_calls_upload", "bsm_state_unpack", "bsm_bwd_step_ws", "bsm_bwd_step_streams",
    "bsm_bwd_step_noalloc", "bsm_bwd_fetched", "bsm_fetched_accumulate", "bsm_vision_group_order",
]


class BsmError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libbsm error {code}: {msg}")
        self.code = code


class bsm_plan_desc(C.Structure):
    _fields_ = [("n", C.c_int64), ("sample", C.c_void_p), ("seg", C.c_void_p),
                ("noise", C.c_void_p), ("pos", C.c_void_p), ("window", C.c_int32),
                ("ranks", C.c_int32), ("block", C.c_int32), ("order", C.c_int32),
                ("explicit_block_perm", C.c_void_p), ("threads", C.c_int32)]


class bsm_plan_info(C.Structure):
    _fields_ = [("n", C.c_int64), ("ranks", C.c_int32), ("block", C.c_int32),
                ("order", C.c_int32), ("window", C.c_int32), ("shard_tokens", C.c_int64),
                ("tiles_per_shard", C.c_int32), ("tiles_total", C.c_int32),
                ("busiest_rank", C.c_int32), ("reserved", C.c_int32),
                ("total_pairs", C.c_int64), ("candidate_pairs", C.c_int64),
                ("full_tiles", C.c_int64), ("partial_tiles", C.c_int64),
                ("build_seconds", C.c_double), ("interval_keys", C.c_int64)]


class bsm_dplan_info(C.Structure):
    _fields_ = [("rank", C.c_int32), ("ranks", C.c_int32), ("shard_tokens", C.c_int64),
                ("tiles_per_shard", C.c_int32), ("window", C.c_int32),
                ("fwd_items", C.c_int64 * 64), ("bwd_items", C.c_int64 * 64),
                ("step_pairs", C.c_int64 * 64), ("single_items", C.c_int64),
                ("fetch_tiles", C.c_int64), ("fetch_rows", C.c_int64), ("dense_calls", C.c_int32),
                ("bwd_workspace_slots", C.c_int32), ("fwd_chain0_items", C.c_int64 * 64)]


class bsm_call(C.Structure):
    _fields_ = [("q0", C.c_int32), ("q_len", C.c_int32), ("k0", C.c_int32), ("k_len", C.c_int32),
                ("kind", C.c_int32)]


class bsm_chunk_info(C.Structure):
    _fields_ = [("chunks_per_rank", C.c_int32), ("strategy", C.c_int32), ("cost", C.c_double),
                ("step_max_sum", C.c_double), ("range_term", C.c_double)]


class bsm_heads(C.Structure):
    _fields_ = [("hq", C.c_int32), ("hkv", C.c_int32), ("d", C.c_int32), ("scale", C.c_float)]


_P = C.c_void_p
_sig = {
    "bsm_last_error": (C.c_char_p, []),
    "bsm_version": (C.c_int32, []),
    "bsm_plan_build": (C.c_int, [C.POINTER(bsm_plan_desc), C.POINTER(_P)]),
    "bsm_plan_free": (None, [_P]),
    "bsm_plan_get_info": (C.c_int, [_P, C.POINTER(bsm_plan_info)]),
    "bsm_plan_permutation": (C.c_int, [_P, _P]),
    "bsm_plan_block_cost": (C.c_int, [_P, _P, _P]),
    "bsm_plan_step_map": (C.c_int, [_P, C.c_int32, C.c_int32, _P, C.POINTER(C.c_int64)]),
    "bsm_plan_pairs": (C.c_int, [_P, _P]),
    "bsm_plan_key_intervals": (C.c_int, [_P, _P, _P]),
    "bsm_plan_fetch_set": (C.c_int, [_P, C.c_int32, _P, C.POINTER(C.c_int64)]),
    "bsm_plan_chunk_order": (C.c_int, [_P, C.c_int32, C.c_int32, C.c_double, C.c_int32, _P,
                                       C.POINTER(bsm_chunk_info)]),
    "bsm_fwd_fetched": (C.c_int, [_P, C.POINTER(bsm_heads), _P, _P, _P, _P, _P, _P, _P, _P,
                                  C.c_int32, _P]),
    "bsm_dplan_bytes": (C.c_int, [_P, C.c_int32, C.POINTER(C.c_int64)]),
    "bsm_dplan_upload": (C.c_int, [_P, C.c_int32, _P, C.c_int64, _P, C.POINTER(_P)]),
    "bsm_dplan_free": (None, [_P]),
    "bsm_state_unpack": (C.c_int, [C.POINTER(bsm_heads), C.c_int64, _P, _P, _P]),
    "bsm_dplan_calls_bytes": (C.c_int, [_P, C.c_int32, C.POINTER(C.c_int64)]),
    "bsm_dplan_calls_upload": (C.c_int, [_P, C.c_int32, _P, C.c_int64, _P, C.POINTER(_P)]),
    "bsm_plan_dense_calls": (C.c_int, [_P, C.c_int32, C.c_int32, _P, C.c_int64, C.POINTER(C.c_int64)]),
    "bsm_dplan_get_info": (C.c_int, [_P, C.POINTER(bsm_dplan_info)]),
    "bsm_fwd_step": (C.c_int, [_P, C.c_int32, C.POINTER(bsm_heads), _P, _P, _P, _P, _P, _P,
                               _P, _P, C.c_int32, _P]),
    "bsm_fwd_step_chain": (C.c_int, [_P, C.c_int32, C.c_int32, C.POINTER(bsm_heads), _P, _P, _P, _P, _P,
                                     _P, _P, _P, C.c_int32, _P]),
    "bsm_fwd_single": (C.c_int, [_P, C.POINTER(bsm_heads), _P, _P, _P, _P, _P, _P, _P, _P,
                                 C.c_int32, _P]),
    "bsm_fwd_merge_bf16": (C.c_int, [C.POINTER(bsm_heads), C.c_int64, _P, _P, _P, _P, _P]),
    "bsm_fwd_merge_fp32": (C.c_int, [C.POINTER(bsm_heads), C.c_int64, _P, _P, _P, _P, _P, _P, _P]),
    "bsm_bwd_prep": (C.c_int, [C.POINTER(bsm_heads), C.c_int64, _P, _P, _P, _P]),
    "bsm_bwd_step": (C.c_int, [_P, C.c_int32, C.POINTER(bsm_heads), _P, _P, _P, _P, _P, _P,
                               _P, _P, _P, _P]),
    "bsm_bwd_step_ws": (C.c_int, [_P, C.c_int32, C.POINTER(bsm_heads), _P, _P, _P, _P, _P, _P,
                                  _P, _P, _P, _P, C.c_int64, _P]),
    "bsm_bwd_step_streams": (C.c_int, [_P, C.c_int32, C.POINTER(bsm_heads), _P, _P, _P, _P, _P, _P,
                                       _P, _P, _P, _P, C.c_int64, _P, _P]),
    "bsm_bwd_step_noalloc": (C.c_int, [_P, C.c_int32, C.POINTER(bsm_heads), _P, _P, _P, _P, _P, _P,
                                       _P, _P, _P, _P]),
    "bsm_bwd_fetched": (C.c_int, [_P, C.POINTER(bsm_heads), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "bsm_fetched_accumulate": (C.c_int, [_P, C.POINTER(bsm_heads), _P, _P, _P, _P, _P]),
    "bsm_vision_group_order": (C.c_int, [C.c_int64, _P, _P, _P]),
}


def _open():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libbsm.so is not built ({LIB_PATH}); run "
                          "`python -m block_sparse_masked_metadata_amd.build`")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in _sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


class _Library:
    """libbsm.so, opened (and its signatures declared) on first attribute access."""
    handle = None

    def __getattr__(self, name):
        if _Library.handle is None:
            _Library.handle = _open()
        return getattr(_Library.handle, name)


_lib = _Library()


def load():
    """Open libbsm.so now (ImportError if it is not built); returns the ctypes handle."""
    _lib.bsm_version
    return _Library.handle


def bsm_last_error() -> str:
    return _lib.bsm_last_error().decode()


def bsm_version() -> int:
    return int(_lib.bsm_version())


def _check(rc):
    if rc != BSM_OK:
        raise BsmError(rc, bsm_last_error())


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def bsm_plan_build(sample, seg, noise, pos, window, ranks, block=128, order=BSM_ORDER_PTRR,
                   explicit_block_perm=None, threads=0):
    """Returns an opaque plan handle (int); free with bsm_plan_free."""
    arrs = [_i32(x) for x in (sample, seg, noise, pos)]
    n = len(arrs[0])
    if any(len(a) != n for a in arrs):
        raise ValueError("tracks must have equal length")
    ebp = None if explicit_block_perm is None else _i32(explicit_block_perm)
    desc = bsm_plan_desc(n, *(a.ctypes.data for a in arrs), int(min(window, BSM_WINDOW_INF)),
                         int(ranks), int(block), int(order),
                         None if ebp is None else ebp.ctypes.data, int(threads))
    out = _P()
    _check(_lib.bsm_plan_build(C.byref(desc), C.byref(out)))
    return out.value


def bsm_plan_free(plan):
    _lib.bsm_plan_free(plan)


def bsm_plan_get_info(plan) -> dict:
    info = bsm_plan_info()
    _check(_lib.bsm_plan_get_info(plan, C.byref(info)))
    return {k: getattr(info, k) for k, _ in bsm_plan_info._fields_}


def bsm_plan_permutation(plan):
    n = bsm_plan_get_info(plan)["n"]
    out = np.empty(n, np.int32)
    _check(_lib.bsm_plan_permutation(plan, out.ctypes.data))
    return out


def bsm_plan_block_cost(plan):
    t = bsm_plan_get_info(plan)["tiles_total"]
    cost = np.empty(t, np.int64)
    owner = np.empty(t, np.int32)
    _check(_lib.bsm_plan_block_cost(plan, cost.ctypes.data, owner.ctypes.data))
    return cost, owner


def bsm_plan_step_map(plan, r, s):
    t = bsm_plan_get_info(plan)["tiles_per_shard"]
    mp = np.empty((t, t), np.uint8)
    pairs = C.c_int64()
    _check(_lib.bsm_plan_step_map(plan, int(r), int(s), mp.ctypes.data, C.byref(pairs)))
    return mp, pairs.value


def bsm_plan_pairs(plan):
    rk = bsm_plan_get_info(plan)["ranks"]
    out = np.empty((rk, rk), np.int64)
    _check(_lib.bsm_plan_pairs(plan, out.ctypes.data))
    return out


def bsm_plan_key_intervals(plan):
    n = bsm_plan_get_info(plan)["n"]
    lo = np.empty(n, np.int32)
    hi = np.empty(n, np.int32)
    _check(_lib.bsm_plan_key_intervals(plan, lo.ctypes.data, hi.ctypes.data))
    return lo, hi


def bsm_plan_fetch_set(plan, r):
    info = bsm_plan_get_info(plan)
    need = np.empty(info["ranks"] * info["tiles_per_shard"], np.uint8)
    tiles = C.c_int64()
    _check(_lib.bsm_plan_fetch_set(plan, int(r), need.ctypes.data, C.byref(tiles)))
    return need.reshape(info["ranks"], info["tiles_per_shard"]), tiles.value


def bsm_plan_chunk_order(plan, min_chunks=1, max_chunks=64, tau=0.0, swaps=4):
    nt = bsm_plan_get_info(plan)["tiles_total"]
    perm = np.empty(nt, np.int32)
    info = bsm_chunk_info()
    _check(_lib.bsm_plan_chunk_order(plan, int(min_chunks), int(max_chunks), float(tau), int(swaps),
                                     perm.ctypes.data, C.byref(info)))
    return perm, {"chunks_per_rank": info.chunks_per_rank, "strategy": info.strategy,
                  "cost": info.cost, "step_max_sum": info.step_max_sum, "range_term": info.range_term}


def bsm_fwd_fetched(dplan, heads, q, k_fetch, v_fetch, o_acc, m, l, o, lse, flags, stream):
    _check(_lib.bsm_fwd_fetched(dplan, C.byref(heads), q, k_fetch, v_fetch, o_acc, m, l, o, lse,
                                int(flags), stream))


def bsm_dplan_bytes(plan, r) -> int:
    b = C.c_int64()
    _check(_lib.bsm_dplan_bytes(plan, int(r), C.byref(b)))
    return b.value


def bsm_dplan_upload(plan, r, dev_ptr, nbytes, stream):
    out = _P()
    _check(_lib.bsm_dplan_upload(plan, int(r), dev_ptr, int(nbytes), stream, C.byref(out)))
    return out.value


def bsm_dplan_calls_bytes(plan, r) -> int:
    b = C.c_int64()
    _check(_lib.bsm_dplan_calls_bytes(plan, int(r), C.byref(b)))
    return b.value


def bsm_dplan_calls_upload(plan, r, dev_ptr, nbytes, stream):
    out = _P()
    _check(_lib.bsm_dplan_calls_upload(plan, int(r), dev_ptr, int(nbytes), stream, C.byref(out)))
    return out.value


def bsm_plan_dense_calls(plan, r, s):
    """int32 array [count, 5]: q0, q_len, k0, k_len, kind per call."""
    cnt = C.c_int64()
    _check(_lib.bsm_plan_dense_calls(plan, int(r), int(s), None, 0, C.byref(cnt)))
    buf = (bsm_call * max(1, cnt.value))()
    _check(_lib.bsm_plan_dense_calls(plan, int(r), int(s), buf, cnt.value, C.byref(cnt)))
    return np.ctypeslib.as_array(C.cast(buf, C.POINTER(C.c_int32)), (max(1, cnt.value) * 5,)).reshape(
        -1, 5)[:cnt.value].copy()


def bsm_state_unpack(heads, rows, o_acc, out, stream):
    _check(_lib.bsm_state_unpack(C.byref(heads), int(rows), o_acc, out, stream))


def bsm_dplan_free(dplan):
    _lib.bsm_dplan_free(dplan)


def bsm_dplan_get_info(dplan) -> dict:
    info = bsm_dplan_info()
    _check(_lib.bsm_dplan_get_info(dplan, C.byref(info)))
    rk = info.ranks
    return {"rank": info.rank, "ranks": rk, "shard_tokens": info.shard_tokens,
            "tiles_per_shard": info.tiles_per_shard, "window": info.window,
            "fwd_items": list(info.fwd_items[:rk]), "bwd_items": list(info.bwd_items[:rk]),
            "step_pairs": list(info.step_pairs[:rk]), "single_items": info.single_items,
            "fetch_tiles": info.fetch_tiles, "fetch_rows": info.fetch_rows,
            "dense_calls": bool(info.dense_calls), "bwd_workspace_slots": info.bwd_workspace_slots,
            "fwd_chain0_items": list(info.fwd_chain0_items[:rk])}


def _heads(hq, hkv, d, scale):
    return bsm_heads(int(hq), int(hkv), int(d), float(scale))


def bsm_fwd_step(dplan, s, heads, q, k, v, o_acc, m, l, o, lse, flags, stream):
    _check(_lib.bsm_fwd_step(dplan, int(s), C.byref(heads), q, k, v, o_acc, m, l, o, lse,
                             int(flags), stream))


def bsm_fwd_step_chain(dplan, s, chain, heads, q, k, v, o_acc, m, l, o, lse, flags, stream):
    _check(_lib.bsm_fwd_step_chain(dplan, int(s), int(chain), C.byref(heads), q, k, v, o_acc, m, l, o, lse,
                                   int(flags), stream))


def bsm_fwd_single(dplan, heads, q, k_all, v_all, o_acc, m, l, o, lse, flags, stream):
    _check(_lib.bsm_fwd_single(dplan, C.byref(heads), q, k_all, v_all, o_acc, m, l, o, lse,
                               int(flags), stream))


def bsm_fwd_merge_bf16(heads, rows, o_run, lse_run, o_s, lse_s, stream):
    _check(_lib.bsm_fwd_merge_bf16(C.byref(heads), int(rows), o_run, lse_run, o_s, lse_s, stream))


def bsm_fwd_merge_fp32(heads, rows, o_run, lse_run, acc_s, m_s, l_s, o_bf16, stream):
    _check(_lib.bsm_fwd_merge_fp32(C.byref(heads), int(rows), o_run, lse_run, acc_s, m_s, l_s, o_bf16, stream))


def bsm_bwd_prep(heads, rows, o, dout, delta, stream):
    _check(_lib.bsm_bwd_prep(C.byref(heads), int(rows), o, dout, delta, stream))


def bsm_bwd_step(dplan, s, heads, q, k, v, dout, lse, delta, dq_acc, dk, dv, stream):
    _check(_lib.bsm_bwd_step(dplan, int(s), C.byref(heads), q, k, v, dout, lse, delta,
                             dq_acc, dk, dv, stream))


def bsm_bwd_step_ws(dplan, s, heads, q, k, v, dout, lse, delta, dq_acc, dk, dv, workspace,
                    workspace_bytes, stream):
    _check(_lib.bsm_bwd_step_ws(dplan, int(s), C.byref(heads), q, k, v, dout, lse, delta,
                                dq_acc, dk, dv, workspace, int(workspace_bytes), stream))


def bsm_bwd_step_streams(dplan, s, heads, q, k, v, dout, lse, delta, dq_acc, dk, dv, workspace,
                         workspace_bytes, dq_stream, kv_stream):
    _check(_lib.bsm_bwd_step_streams(dplan, int(s), C.byref(heads), q, k, v, dout, lse, delta,
                                     dq_acc, dk, dv, workspace, int(workspace_bytes), dq_stream,
                                     kv_stream))


def bsm_bwd_step_noalloc(dplan, s, heads, q, k, v, dout, lse, delta, dq_acc, dk, dv, stream):
    _check(_lib.bsm_bwd_step_noalloc(dplan, int(s), C.byref(heads), q, k, v, dout, lse, delta,
                                     dq_acc, dk, dv, stream))


def bsm_bwd_fetched(dplan, heads, q, k_fetch, v_fetch, dout, lse, delta, dq, dk_fetch, dv_fetch, stream):
    _check(_lib.bsm_bwd_fetched(dplan, C.byref(heads), q, k_fetch, v_fetch, dout, lse, delta, dq,
                                dk_fetch, dv_fetch, stream))


def bsm_fetched_accumulate(dplan, heads, dk_fetch, dv_fetch, dk_all, dv_all, stream):
    _check(_lib.bsm_fetched_accumulate(dplan, C.byref(heads), dk_fetch, dv_fetch, dk_all, dv_all, stream))


def bsm_vision_group_order(sample, seg):
    """new_to_orig (int32[n]) of the vision-group token order."""
    sm, sg = _i32(sample), _i32(seg)
    if len(sm) != len(sg):
        raise ValueError("tracks must have equal length")
    out = np.empty(len(sm), np.int32)
    _check(_lib.bsm_vision_group_order(len(sm), sm.ctypes.data, sg.ctypes.data, out.ctypes.data))
    return out
