"""Plain CPU oracle for rank-major MoE expert-parallel dispatch and combine.

TEST INFRASTRUCTURE ONLY.  This module is the checker, not the product: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run it.  It shares no code with the HIP path and
imports nothing from the product package.

It follows the FlashInfer ``flashinfer.moe_ep`` API pages:

* ``flashinfer.moe_ep.MoEEpCommunication`` -- the class description (one
  in-flight dispatch/combine pair), ``dispatch()`` (what travels, the
  ``runtime_max_tokens_per_rank`` bound) and ``combine()`` (sum over ranks of
  already-weighted expert outputs).
* ``flashinfer.moe_ep.NVLinkOneSidedAlltoAll`` -- the class description
  (rank-major placement at row ``source_rank * tokens_per_rank + token``,
  ``invalid_expert_id`` for rows beyond a source's count and for rows not
  routed here), ``active_rank_mask()`` and the mask notes of ``dispatch()``
  and ``combine()``, the all-or-none weights rule of ``dispatch()``.
* ``flashinfer.moe_ep.CakeAlltoAll`` -- the same beyond-count rule and mask
  notes.

Where the pages are silent the oracle takes these readings:

* expert ``e`` (``0 <= e < num_experts``) lives on rank ``e // (num_experts /
  ep_size)`` (contiguous blocks); ids outside that range route nowhere;
* ``runtime_max_tokens_per_rank`` must lie in ``[max_s n_s, capacity]``;
  receive rows are laid out at stride ``tokens_per_rank`` of the step;
* every ``top_k`` slot of an invalid row holds ``invalid_expert_id`` and its
  weights are 0.0; its hidden and scale bytes are unspecified (the oracle
  fills them with ``UNSPECIFIED_BYTE`` and comparisons skip them);
* a routed row carries the token's ``topk_ids`` and ``topk_weights``
  verbatim, once per destination rank, however many of its experts live there;
* the rank mask applies to destinations only: a masked-off rank's own tokens
  are still dispatched to the active ranks and still combined;
* combine adds, in float32, the rows of the ranks the token reached in
  ascending rank order starting from +0.0, then rounds once to the output
  type (bfloat16 or float16 with round-to-nearest-even, or float32 as is); a
  token that reached no rank gets zeros.  The output type is the input's:
  float32, bfloat16 or float16.

Every loop here is the definition written out, one token or one row at a
time, so that it can be checked against the pages by eye.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .numerics import bf16_bits_to_f32, f32_to_bf16_bits_rne

MAX_RANKS = 64            # the rank mask is a uint64 (NVLinkOneSidedAlltoAll, active_rank_mask())
ALL_RANKS = (1 << 64) - 1  # "no mask passed"
UNSPECIFIED_BYTE = 0xA5   # filler for hidden/scale bytes of invalid rows (never compared)


class OracleError(Exception):
    """A call that breaks the pages' contract.  ``kind`` names the broken rule:
    "state", "capacity", "mask" or "invalid_arg"."""

    def __init__(self, kind: str, msg: str):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


@dataclass
class Params:
    """The group's static sizes (the pages' MoEEpCommParams and backend config)."""

    ep_size: int
    num_experts: int
    top_k: int
    max_tokens_per_rank: int
    hidden_size: int          # elements of a combine row
    hidden_row_bytes: int     # bytes of a dispatched hidden row (opaque payload)
    scale_row_bytes: int = 0  # bytes of a dispatched scale row, 0 = no scales
    invalid_expert_id: int = -1
    enable_rank_mask: bool = False
    eplb_stats_bytes: int = 0   # bytes of one rank's expert-load statistics row

    def check(self) -> None:
        if not (1 <= self.ep_size <= MAX_RANKS):
            raise OracleError("invalid_arg", "ep_size must be in [1, 64]")
        if self.num_experts < self.ep_size or self.num_experts % self.ep_size:
            raise OracleError("invalid_arg", "num_experts must be a positive multiple of ep_size")
        if self.top_k < 1 or self.max_tokens_per_rank < 0 or self.hidden_size < 1:
            raise OracleError("invalid_arg", "bad top_k / capacity / hidden_size")
        if self.hidden_row_bytes < 1 or self.scale_row_bytes < 0:
            raise OracleError("invalid_arg", "bad row sizes")


@dataclass
class RankResult:
    """What one destination rank sees after dispatch (its receive region)."""

    hidden: np.ndarray                    # uint8 [ep*tpr, hidden_row_bytes]
    hidden_scale: Optional[np.ndarray]    # uint8 [ep*tpr, scale_row_bytes] or None
    topk_ids: np.ndarray                  # int32 [ep*tpr, top_k]
    topk_weights: Optional[np.ndarray]    # float32 [ep*tpr, top_k] or None
    tokens_per_rank: int
    valid: np.ndarray                     # bool [ep*tpr]: rows that hold a routed token
    eplb_global_stats: Optional[np.ndarray] = None   # uint8 [ep, eplb_stats_bytes] or None


@dataclass
class DispatchRecord:
    """What combine needs to remember about the dispatch it follows."""

    tokens_per_rank: int
    local_num_tokens: List[int]
    dest_masks: List[List[int]]          # dest_masks[s][t], t < tokens_per_rank
    active_rank_mask: int


def active_rank_mask(active_ranks: Sequence[int]) -> int:
    """The uint64 bitmask with bit r set for every listed rank
    (NVLinkOneSidedAlltoAll, active_rank_mask())."""
    m = 0
    for r in active_ranks:
        r = int(r)
        if not (0 <= r < MAX_RANKS):
            raise OracleError("mask", f"rank {r} outside [0, 64)")
        m |= 1 << r
    return m


def expert_owner(params: Params, expert_id: int) -> Optional[int]:
    """Rank that owns a global expert id under contiguous ownership, or None
    when the id is outside [0, num_experts)."""
    if 0 <= expert_id < params.num_experts:
        return expert_id // (params.num_experts // params.ep_size)
    return None


def destination_mask(params: Params, ids_row: Sequence[int], active: int) -> int:
    """Ranks a token is sent to: the owners of its selected experts
    (MoEEpCommunication, dispatch()), less the masked-off ranks
    (NVLinkOneSidedAlltoAll / CakeAlltoAll, dispatch() mask note)."""
    m = 0
    for e in ids_row:
        d = expert_owner(params, int(e))
        if d is not None:
            m |= 1 << d
    return m & active & ((1 << params.ep_size) - 1)


def step_tokens_per_rank(params: Params, local_num_tokens: Sequence[int],
                         runtime_max_tokens_per_rank: Optional[int]) -> int:
    """tokens_per_rank of a step: the runtime bound, or the capacity when None
    (MoEEpCommunication, dispatch(), runtime_max_tokens_per_rank)."""
    cap = params.max_tokens_per_rank
    largest = max(local_num_tokens) if len(local_num_tokens) else 0
    if largest > cap:
        raise OracleError("capacity", f"a rank has {largest} tokens > capacity {cap}")
    tpr = cap if runtime_max_tokens_per_rank is None else int(runtime_max_tokens_per_rank)
    if tpr > cap:
        raise OracleError("capacity", f"runtime_max_tokens_per_rank {tpr} > capacity {cap}")
    if tpr < largest:
        raise OracleError("capacity", f"runtime_max_tokens_per_rank {tpr} < largest local count {largest}")
    return tpr


def _check_mask(params: Params, mask: Optional[int]) -> int:
    if mask is None:
        return ALL_RANKS
    mask = int(mask)
    if not params.enable_rank_mask:
        raise OracleError("mask", "active_rank_mask needs enable_rank_mask")
    if mask >> params.ep_size:
        raise OracleError("mask", "mask has bits at or above ep_size")
    return mask


class OracleMoEEp:
    """One EP group of ``ep_size`` ranks held in one process, with the pages'
    call protocol: dispatch, then exactly one combine, then the next dispatch
    (MoEEpCommunication, class description)."""

    def __init__(self, params: Params):
        params.check()
        self.params = params
        self.record: Optional[DispatchRecord] = None
        self.destroyed = False

    # -- dispatch -------------------------------------------------------------
    def dispatch(self, hidden_states: Sequence[np.ndarray], topk_ids: Sequence[np.ndarray],
                 topk_weights: Optional[Sequence[Optional[np.ndarray]]] = None, *,
                 hidden_states_scale: Optional[Sequence[Optional[np.ndarray]]] = None,
                 runtime_max_tokens_per_rank: Optional[int] = None,
                 active_rank_mask: Optional[int] = None,
                 eplb_local_stats: Optional[Sequence[Optional[np.ndarray]]] = None) -> List[RankResult]:
        """Per-rank inputs in, per-rank receive regions out.

        ``hidden_states[s]`` is a uint8 ``[n_s, hidden_row_bytes]`` array (rows
        are opaque bytes, quantized or not), ``topk_ids[s]`` an int
        ``[n_s, top_k]`` array, ``topk_weights[s]`` a float32 ``[n_s, top_k]``
        array and ``hidden_states_scale[s]`` a uint8 ``[n_s, scale_row_bytes]``
        array.  ``eplb_local_stats[s]`` (optional, uint8 ``[eplb_stats_bytes]``)
        is rank s's expert-load statistics row; dispatch all-gathers these
        (MoEEpCommunication, dispatch(), eplb_local_stats): every rank's
        result holds all of them, row s from rank s.
        """
        p = self.params
        ep, K = p.ep_size, p.top_k
        if self.destroyed or self.record is not None:
            raise OracleError("state", "dispatch needs an idle instance")
        if len(hidden_states) != ep or len(topk_ids) != ep:
            raise OracleError("invalid_arg", "one input per rank expected")
        n = [int(np.asarray(topk_ids[s]).reshape(-1, K).shape[0]) for s in range(ep)]
        for s in range(ep):
            if np.asarray(hidden_states[s]).shape[0] != n[s]:
                raise OracleError("invalid_arg", f"rank {s}: hidden rows != topk_ids rows")
        tpr = step_tokens_per_rank(p, n, runtime_max_tokens_per_rank)
        active = _check_mask(p, active_rank_mask)

        # Weights: every rank or none (NVLinkOneSidedAlltoAll, dispatch()).
        has_w = topk_weights is not None and any(w is not None for w in topk_weights)
        if has_w and any(w is None for w in topk_weights):
            raise OracleError("invalid_arg", "topk_weights passed by some ranks only")
        has_s = hidden_states_scale is not None and any(x is not None for x in hidden_states_scale)
        if has_s and any(x is None for x in hidden_states_scale):
            raise OracleError("invalid_arg", "hidden_states_scale passed by some ranks only")
        if has_s and p.scale_row_bytes == 0:
            raise OracleError("invalid_arg", "scales passed but scale_row_bytes is 0")
        has_e = eplb_local_stats is not None and any(x is not None for x in eplb_local_stats)
        if has_e and any(x is None for x in eplb_local_stats):
            raise OracleError("invalid_arg", "eplb_local_stats passed by some ranks only")
        if has_e and p.eplb_stats_bytes == 0:
            raise OracleError("invalid_arg", "eplb_local_stats passed but eplb_stats_bytes is 0")
        gathered = None
        if has_e:
            # All-gather: row s of every rank's copy is rank s's statistics.
            gathered = np.empty((ep, p.eplb_stats_bytes), np.uint8)
            for s in range(ep):
                gathered[s] = np.asarray(eplb_local_stats[s], np.uint8).reshape(p.eplb_stats_bytes)

        # Destination ranks of every token; padding rows (t >= n_s) go nowhere.
        dest_masks = []
        for s in range(ep):
            ids_s = np.asarray(topk_ids[s]).reshape(-1, K)
            row_masks = []
            for t in range(tpr):
                row_masks.append(destination_mask(p, ids_s[t], active) if t < n[s] else 0)
            dest_masks.append(row_masks)

        # Rank-major placement: destination d, row s * tpr + t holds token (s, t)
        # when d is one of its destinations; every other row is invalid
        # (NVLinkOneSidedAlltoAll class description; CakeAlltoAll class description).
        rows = ep * tpr
        results = []
        for d in range(ep):
            out_hidden = np.full((rows, p.hidden_row_bytes), UNSPECIFIED_BYTE, np.uint8)
            out_scale = np.full((rows, p.scale_row_bytes), UNSPECIFIED_BYTE, np.uint8) if has_s else None
            out_ids = np.empty((rows, K), np.int32)
            out_w = np.empty((rows, K), np.float32) if has_w else None
            valid = np.zeros(rows, bool)
            for s in range(ep):
                hid_s = np.asarray(hidden_states[s], np.uint8).reshape(n[s], p.hidden_row_bytes)
                ids_s = np.asarray(topk_ids[s]).reshape(n[s], K)
                if has_s:
                    scl_s = np.asarray(hidden_states_scale[s], np.uint8).reshape(n[s], p.scale_row_bytes)
                if has_w:
                    w_s = np.asarray(topk_weights[s], np.float32).reshape(n[s], K)
                for t in range(tpr):
                    r = s * tpr + t
                    if (dest_masks[s][t] >> d) & 1:
                        valid[r] = True
                        out_hidden[r] = hid_s[t]
                        out_ids[r] = ids_s[t]
                        if has_s:
                            out_scale[r] = scl_s[t]
                        if has_w:
                            out_w[r] = w_s[t]
                    else:
                        out_ids[r] = p.invalid_expert_id
                        if has_w:
                            out_w[r] = 0.0
            results.append(RankResult(out_hidden, out_scale, out_ids, out_w, tpr, valid,
                                      None if gathered is None else gathered.copy()))

        self.record = DispatchRecord(tpr, n, dest_masks, active)
        return results

    # -- combine --------------------------------------------------------------
    def combine(self, expert_output: Sequence[np.ndarray], dtype: str, *,
                active_rank_mask: Optional[int] = None) -> List[np.ndarray]:
        """Sum each token's already-weighted rows over the ranks it reached
        (MoEEpCommunication, combine()).

        ``expert_output[d]`` is rank d's ``[ep*tpr, hidden]`` or
        ``[ep, tpr, hidden]`` array: float32 for ``dtype="f32"``, bfloat16 bit
        patterns (uint16) for ``dtype="bf16"``, NumPy float16 for
        ``dtype="f16"`` (the pages' combine input buffer takes any dtype,
        MoEEpCommunication, get_combine_input_buffer()).  Returns per source
        rank s an ``[n_s, hidden]`` array of the same representation.
        """
        p = self.params
        rec = self.record
        if self.destroyed or rec is None:
            raise OracleError("state", "combine needs a preceding dispatch")
        mask = _check_mask(p, active_rank_mask)
        if mask != rec.active_rank_mask:
            raise OracleError("mask", "combine mask differs from the dispatch mask")
        if dtype not in ("f32", "bf16", "f16"):
            raise OracleError("invalid_arg", f"dtype {dtype}")
        ep, tpr, hid = p.ep_size, rec.tokens_per_rank, p.hidden_size
        outputs = []
        rows_of = [None if expert_output[d] is None else np.asarray(expert_output[d]).reshape(ep * tpr, hid)
                   for d in range(ep)]
        for s in range(ep):
            out = np.empty((rec.local_num_tokens[s], hid),
                           {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}[dtype])
            for t in range(rec.local_num_tokens[s]):
                r = s * tpr + t
                acc = np.zeros(hid, np.float32)
                for d in range(ep):                      # ascending rank order
                    if (rec.dest_masks[s][t] >> d) & 1:
                        row = rows_of[d][r]
                        # widening to float32 is exact for all three types
                        term = bf16_bits_to_f32(row) if dtype == "bf16" else row.astype(np.float32)
                        acc = (acc + term).astype(np.float32)
                if dtype == "f32":
                    out[t] = acc
                elif dtype == "bf16":
                    out[t] = f32_to_bf16_bits_rne(acc)
                else:
                    with np.errstate(over="ignore"):       # overflow rounds to infinity
                        out[t] = acc.astype(np.float16)   # NumPy rounds to nearest even
            outputs.append(out)
        self.record = None
        return outputs

    def destroy(self) -> None:
        """Idempotent (MoEEpCommunication, destroy())."""
        self.destroyed = True
        self.record = None


def expert_standin(params: Params, results: Sequence[RankResult],
                   token_values: Sequence[np.ndarray], dtype: str) -> List[np.ndarray]:
    """A stand-in for the expert computation between dispatch and combine.

    Not part of the method: it makes combine inputs with a known sum.  On rank
    d, a routed row r = s*tpr + t becomes ``token_values[s][t] * W`` rounded to
    ``dtype``, where W is the sum of the row's weights whose experts live on d
    (the expert output is "already weighted and reduced over this rank's local
    experts", MoEEpCommunication, combine()).  Rows that hold no token are NaN,
    so a combine that reads one shows it.
    """
    ep = params.ep_size
    outs = []
    for d in range(ep):
        res = results[d]
        tpr = res.tokens_per_rank
        out = np.full((ep * tpr, params.hidden_size), np.nan, np.float32)
        for r in range(ep * tpr):
            if not res.valid[r]:
                continue
            s, t = divmod(r, tpr)
            w_local = np.float32(0.0)
            for j in range(params.top_k):
                if expert_owner(params, int(res.topk_ids[r, j])) == d:
                    w_local = np.float32(w_local + res.topk_weights[r, j])
            out[r] = (np.asarray(token_values[s][t], np.float32) * w_local).astype(np.float32)
        if dtype == "f32":
            outs.append(out)
        elif dtype == "bf16":
            outs.append(f32_to_bf16_bits_rne(out))
        else:
            with np.errstate(over="ignore"):
                outs.append(out.astype(np.float16))
    return outs
