"""The decode as torch operators that declare what they write.

AMD-Ecosystem/flashinfer PR #397 ("Stop declaring the paged KV cache mutated on read-only
attention ops", sections "Summary", "What changed" and "Architecture / design notes") is about
this declaration: an attention op that only reads the paged cache but registers it as mutated
makes the functionalization pass of torch.compile copy the cache back into its base tensor (for
views such as one half of a [2, pages, ...] tensor or one layer of a multi-layer pool) and makes
captured graphs copy it on every replay. Its fix registers the read-only ops under new names
(so that stale compile caches of the old schema are not replayed) with only the real outputs
declared as written, and keeps the cache declared written only where an op really writes it
(the append).

Here:

* ``skvd::decode_v1`` returns fresh ``(o, lse)`` and declares nothing mutated;
* ``skvd::decode_out_v1`` writes caller-provided ``out`` and ``lse`` and declares exactly those
  two as mutated;
* ``skvd::prefill_v1`` and ``skvd::prefill_out_v1`` are the same pair for the multi-token route
  (a query block of T tokens per sequence, causal over its own last T positions): the page
  treats its paged prefill op the way it treats the decode ops, declaring only the real outputs;
* ``skvd::append_v1`` writes new tokens into the cache and declares the pools (and, for an int8
  cache, the scale pools) mutated, because it writes them.

The plan (shape, schedule, workspace) is a host object that is not a tensor argument: ops name
it by the integer id ``register_plan`` returns, and its workspace is owned by the plan, allocated
once outside any capture, so it is neither declared nor copied by a graph. Each op's fake
implementation gives output shapes without running anything. Every step of the computation runs
in libskvd.so's HIP kernels; these functions only marshal arguments (there is no CPU path).
"""
from __future__ import annotations

import itertools
import threading
from typing import Optional

import torch
from torch import Tensor

from ._binding import Plan

_PLANS: dict[int, Plan] = {}
_PLANS_LOCK = threading.Lock()
_NEXT_ID = itertools.count(1)


def register_plan(plan: Plan) -> int:
    """Make a plan available to the operators; returns the id to pass as ``plan_id``. The
    workspace is allocated here (outside any capture)."""
    plan.ensure_workspace()
    with _PLANS_LOCK:
        pid = next(_NEXT_ID)
        _PLANS[pid] = plan
    return pid


def unregister_plan(plan_id: int) -> None:
    with _PLANS_LOCK:
        _PLANS.pop(int(plan_id), None)


def _plan(plan_id: int) -> Plan:
    try:
        return _PLANS[int(plan_id)]
    except KeyError:
        raise KeyError(f"no plan registered under id {plan_id}") from None


# ---------------------------------------------------------------------------- decode
@torch.library.custom_op("skvd::decode_v1", mutates_args=(), device_types="cuda")
def decode_v1(q: Tensor, k_pages: Tensor, v_pages: Tensor, page_table: Tensor, kv_len: Tensor,
              k_scales: Optional[Tensor], v_scales: Optional[Tensor], sm_scale: float,
              q_per_seq: int, plan_id: int) -> tuple[Tensor, Tensor]:
    """Decode; returns (o [B*T, Hq, D] f16 dense, lse [B*T, Hq] f32). Reads every input."""
    return _plan(plan_id).run(q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales,
                              v_scales, q_per_seq=q_per_seq)


@decode_v1.register_fake
def _decode_v1_fake(q, k_pages, v_pages, page_table, kv_len, k_scales, v_scales, sm_scale,
                    q_per_seq, plan_id):
    o = q.new_empty(q.shape, dtype=torch.float16)
    lse = q.new_empty(q.shape[:2], dtype=torch.float32)
    return o, lse


@torch.library.custom_op("skvd::decode_out_v1", mutates_args=("out", "lse"),
                         device_types="cuda")
def decode_out_v1(q: Tensor, k_pages: Tensor, v_pages: Tensor, page_table: Tensor,
                  kv_len: Tensor, k_scales: Optional[Tensor], v_scales: Optional[Tensor],
                  sm_scale: float, q_per_seq: int, plan_id: int, out: Tensor, lse: Tensor) -> None:
    """Decode into caller-provided out (contiguous f16 [B*T, Hq, D]) and lse (contiguous f32
    [B*T, Hq]); declares exactly those two as written."""
    _plan(plan_id).run(q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales, v_scales,
                       out=out, lse=lse, q_per_seq=q_per_seq)


@decode_out_v1.register_fake
def _decode_out_v1_fake(q, k_pages, v_pages, page_table, kv_len, k_scales, v_scales, sm_scale,
                        q_per_seq, plan_id, out, lse):
    return None


# ---------------------------------------------------------------------------- multi-token
@torch.library.custom_op("skvd::prefill_v1", mutates_args=(), device_types="cuda")
def prefill_v1(q: Tensor, k_pages: Tensor, v_pages: Tensor, page_table: Tensor, kv_len: Tensor,
               k_scales: Optional[Tensor], v_scales: Optional[Tensor], sm_scale: float,
               q_per_seq: int, plan_id: int) -> tuple[Tensor, Tensor]:
    """Multi-token route; returns (o [B*T, Hq, D] f16 dense, lse [B*T, Hq] f32). Reads every
    input."""
    return _plan(plan_id).prefill(q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales,
                                  v_scales, q_per_seq=q_per_seq)


@prefill_v1.register_fake
def _prefill_v1_fake(q, k_pages, v_pages, page_table, kv_len, k_scales, v_scales, sm_scale,
                     q_per_seq, plan_id):
    o = q.new_empty(q.shape, dtype=torch.float16)
    lse = q.new_empty(q.shape[:2], dtype=torch.float32)
    return o, lse


@torch.library.custom_op("skvd::prefill_out_v1", mutates_args=("out", "lse"),
                         device_types="cuda")
def prefill_out_v1(q: Tensor, k_pages: Tensor, v_pages: Tensor, page_table: Tensor,
                   kv_len: Tensor, k_scales: Optional[Tensor], v_scales: Optional[Tensor],
                   sm_scale: float, q_per_seq: int, plan_id: int, out: Tensor,
                   lse: Tensor) -> None:
    """Multi-token route into caller-provided out (contiguous f16 [B*T, Hq, D]) and lse
    (contiguous f32 [B*T, Hq]); declares exactly those two as written."""
    _plan(plan_id).prefill(q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales,
                           v_scales, out=out, lse=lse, q_per_seq=q_per_seq)


@prefill_out_v1.register_fake
def _prefill_out_v1_fake(q, k_pages, v_pages, page_table, kv_len, k_scales, v_scales, sm_scale,
                         q_per_seq, plan_id, out, lse):
    return None


# ---------------------------------------------------------------------------- append
@torch.library.custom_op("skvd::append_v1", mutates_args=("k_pages", "v_pages", "k_scales",
                                                           "v_scales"), device_types="cuda")
def append_v1(k_new: Tensor, v_new: Tensor, batch_idx: Tensor, positions: Tensor,
              k_pages: Tensor, v_pages: Tensor, page_table: Tensor,
              k_scales: Optional[Tensor], v_scales: Optional[Tensor], plan_id: int) -> None:
    """Write new K/V rows into the cache (int8 quantized on write); declares the pools and
    scale pools written (an fp8 cache's one-element scales are only read, but share the
    argument)."""
    _plan(plan_id).append(k_new, v_new, batch_idx, positions, k_pages, v_pages, page_table,
                          k_scales, v_scales)


@append_v1.register_fake
def _append_v1_fake(k_new, v_new, batch_idx, positions, k_pages, v_pages, page_table, k_scales,
                    v_scales, plan_id):
    return None


def decode(plan_id: int, q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales=None,
           v_scales=None, q_per_seq=1, out=None, lse=None):
    """Convenience dispatch: ``decode_out_v1`` when out and lse are given, else ``decode_v1``."""
    if out is not None and lse is not None:
        torch.ops.skvd.decode_out_v1(q, k_pages, v_pages, page_table, kv_len, k_scales, v_scales,
                                     float(sm_scale), int(q_per_seq), int(plan_id), out, lse)
        return out, lse
    if out is not None or lse is not None:
        raise ValueError("pass both out and lse, or neither")
    return torch.ops.skvd.decode_v1(q, k_pages, v_pages, page_table, kv_len, k_scales, v_scales,
                                    float(sm_scale), int(q_per_seq), int(plan_id))


def prefill(plan_id: int, q, k_pages, v_pages, page_table, kv_len, sm_scale, k_scales=None,
            v_scales=None, q_per_seq=1, out=None, lse=None):
    """Convenience dispatch: ``prefill_out_v1`` when out and lse are given, else ``prefill_v1``."""
    if out is not None and lse is not None:
        torch.ops.skvd.prefill_out_v1(q, k_pages, v_pages, page_table, kv_len, k_scales,
                                      v_scales, float(sm_scale), int(q_per_seq), int(plan_id),
                                      out, lse)
        return out, lse
    if out is not None or lse is not None:
        raise ValueError("pass both out and lse, or neither")
    return torch.ops.skvd.prefill_v1(q, k_pages, v_pages, page_table, kv_len, k_scales,
                                     v_scales, float(sm_scale), int(q_per_seq), int(plan_id))
