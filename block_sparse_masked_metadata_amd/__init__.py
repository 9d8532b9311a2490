"""Exact block-sparse masked attention for packed multimodal sequences on MI355X.

One ring rank's share on one gfx950 GPU: a host planner (metadata tracks ->
exact tile classes + PTRR order), HIP kernels that carry the fp32 online-softmax
state across ring steps, and backward kernels against the final LSE.  The
compute lives in libbsm.so (C ABI, include/bsm.h); `_capi` binds it 1:1 and
`ring` adds torch-facing step loops.  The first call into the library raises
ImportError if libbsm.so has not been built (there is no fallback).
"""
from . import _capi
from ._capi import BsmError, LIB_PATH
from .ring import (Plan, DevicePlan, vision_group_order, heads, new_state, state_rows, fwd_step, fwd_chains, fwd_ring, fwd_ring_merged, fwd_single,
                   fetch_rows, gather_fetched, fwd_fetched, bwd_fetched, fetched_accumulate,
                   bwd_prep, bwd_step, bwd_ring, bwd_workspace, kv_side_streams)

__all__ = ["_capi", "BsmError", "LIB_PATH", "Plan", "DevicePlan", "vision_group_order", "heads", "new_state", "state_rows",
           "fwd_step", "fwd_chains", "fwd_ring", "fwd_ring_merged", "fwd_single", "fetch_rows", "gather_fetched",
           "fwd_fetched", "bwd_fetched", "fetched_accumulate", "bwd_prep", "bwd_step", "bwd_ring", "bwd_workspace",
           "kv_side_streams"]
