"""Pins of the CPU oracle to facts other than its own code.

* hand-worked examples under tests/golden/ (values from the pages'
  definitions, worked by hand);
* brute force over every id row of tiny groups, checked against a
  table-driven description of ownership (rank d owns the d-th block of
  experts), built without the oracle's division;
* special cases of combine whose result is known in closed form (rank
  indicators 2^d sum to the destination mask, ones sum to the fan-out);
* the invariant that combining the expert stand-in reproduces each token's
  value times the weights of its active experts, within the recursive
  summation bound;
* the contract's error rules;
* bfloat16 rounding against torch's CPU conversion (a library routine).
"""

from __future__ import annotations

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import OracleError, OracleMoEEp, Params
from synth import workloads as wl
from tests.golden_cases import all_cases

GOLDEN = all_cases()


def params_from_dict(p: dict) -> Params:
    return Params(**p)


# --------------------------------------------------------------------------
# Hand-worked examples
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", GOLDEN, ids=[c.name for c in GOLDEN])
def test_golden_dispatch_and_combine(case):
    p = params_from_dict(case.params)
    o = OracleMoEEp(p)
    res = o.dispatch(case.hidden, case.topk_ids, case.topk_weights, hidden_states_scale=case.scale,
                     runtime_max_tokens_per_rank=case.runtime_max_tokens_per_rank,
                     active_rank_mask=case.active_rank_mask, eplb_local_stats=case.eplb_local_stats)
    e = case.expect
    for d in range(p.ep_size):
        assert res[d].tokens_per_rank == e["tokens_per_rank"]
        np.testing.assert_array_equal(res[d].valid, np.array(e["valid"][d]))
        np.testing.assert_array_equal(res[d].topk_ids, np.array(e["topk_ids"][d], np.int32))
        np.testing.assert_array_equal(res[d].topk_weights, np.array(e["topk_weights"][d], np.float32))
        for r, row in e["hidden_valid_rows"][d].items():
            np.testing.assert_array_equal(res[d].hidden[int(r)], np.array(row, np.uint8))
        if "scale_valid_rows" in e:
            for r, row in e["scale_valid_rows"][d].items():
                np.testing.assert_array_equal(res[d].hidden_scale[int(r)], np.array(row, np.uint8))
        if "eplb_global_stats" in e:
            np.testing.assert_array_equal(res[d].eplb_global_stats, np.array(e["eplb_global_stats"], np.uint8))
        else:
            assert res[d].eplb_global_stats is None
    out = o.combine(case.expert_output, case.combine_dtype, active_rank_mask=case.combine_mask)
    for s in range(p.ep_size):
        if case.combine_dtype == "f32":
            np.testing.assert_array_equal(out[s], case.expect_combine[s])
        else:
            np.testing.assert_array_equal(out[s].view(np.uint16), case.expect_combine[s])


# --------------------------------------------------------------------------
# Brute force over id rows of tiny groups
# --------------------------------------------------------------------------
def owner_table(ep: int, E: int) -> np.ndarray:
    """Rank of each expert when rank d holds the d-th of ep equal blocks."""
    return np.repeat(np.arange(ep), E // ep)


def expected_destinations(ids_row, table, E, active, ep):
    owners = {int(table[e]) for e in ids_row if 0 <= e < E}
    return {d for d in owners if (active >> d) & 1 and d < ep}


def check_layout(p: Params, res, n, tpr, ids, w, hidden, active):
    """Every routed (token, rank) pair appears once at row s*tpr+t of that
    rank with the token's bytes; every other row is invalid."""
    table = owner_table(p.ep_size, p.num_experts)
    valid_total = 0
    pairs = 0
    for d in range(p.ep_size):
        assert res[d].topk_ids.shape == (p.ep_size * tpr, p.top_k)
        for s in range(p.ep_size):
            for t in range(tpr):
                r = s * tpr + t
                dests = expected_destinations(ids[s][t], table, p.num_experts, active, p.ep_size) \
                    if t < n[s] else set()
                routed = d in dests
                assert bool(res[d].valid[r]) == routed
                if routed:
                    np.testing.assert_array_equal(res[d].topk_ids[r], ids[s][t])
                    np.testing.assert_array_equal(res[d].topk_weights[r], w[s][t])
                    np.testing.assert_array_equal(res[d].hidden[r], hidden[s][t])
                else:
                    assert (res[d].topk_ids[r] == p.invalid_expert_id).all()
                    assert (res[d].topk_weights[r] == 0.0).all()
        valid_total += int(res[d].valid.sum())
    for s in range(p.ep_size):
        for t in range(n[s]):
            pairs += len(expected_destinations(ids[s][t], table, p.num_experts, active, p.ep_size))
    assert valid_total == pairs


@pytest.mark.parametrize("ep", [1, 2, 3])
@pytest.mark.parametrize("epr", [1, 2])
@pytest.mark.parametrize("K", [1, 2])
def test_bruteforce_every_id_row(ep, epr, K):
    E = ep * epr
    cap = 3
    n = [2, 0, 1][:ep]
    rng = np.random.default_rng(7 + ep * 100 + epr * 10 + K)
    id_values = list(range(-1, E + 1))            # includes one id below and one above the range
    masks = list(range(1 << ep))
    positions = [(s, t) for s in range(ep) for t in range(n[s])]
    for row in itertools.product(id_values, repeat=K):
        for (s0, t0) in positions:
            for tpr in sorted({max(n), cap}):
                for mask in masks:
                    p = Params(ep, E, K, cap, 2, 3, invalid_expert_id=E + 5, enable_rank_mask=True)
                    ids = [rng.integers(-1, E + 1, size=(n[s], K)).astype(np.int32) for s in range(ep)]
                    ids[s0][t0] = np.array(row, np.int32)
                    w = [rng.random((n[s], K)).astype(np.float32) for s in range(ep)]
                    hidden = [rng.integers(0, 256, size=(n[s], 3)).astype(np.uint8) for s in range(ep)]
                    o = OracleMoEEp(p)
                    res = o.dispatch(hidden, ids, w, runtime_max_tokens_per_rank=tpr,
                                     active_rank_mask=mask)
                    check_layout(p, res, n, tpr, ids, w, hidden, mask)


def test_workload_layout_tiny_and_ragged_small():
    for w, nt in ((wl.BY_NAME["tiny"], None), (wl.BY_NAME["ragged"], [5, 0, 9, 3, 0, 0, 7, 2])):
        inp = wl.make_inputs(w, local_num_tokens=nt)
        p = Params(w.ep_size, w.num_experts, w.top_k, w.max_tokens_per_rank, w.hidden_size,
                   w.hidden_row_bytes, w.scale_row_bytes, enable_rank_mask=inp.active_rank_mask is not None)
        o = OracleMoEEp(p)
        rtpr = max(inp.local_num_tokens) if w.runtime_max == "max" else None
        res = o.dispatch(inp.hidden, inp.topk_ids, inp.topk_weights, runtime_max_tokens_per_rank=rtpr,
                         active_rank_mask=inp.active_rank_mask)
        tpr = res[0].tokens_per_rank
        active = oracle.ALL_RANKS if inp.active_rank_mask is None else inp.active_rank_mask
        check_layout(p, res, inp.local_num_tokens, tpr, inp.topk_ids, inp.topk_weights, inp.hidden, active)
        # masked-off destinations hold no valid row at all
        for d in w.masked_ranks:
            assert not res[d].valid.any()


# --------------------------------------------------------------------------
# Combine special cases and invariants
# --------------------------------------------------------------------------
def _dispatch_tiny(mask=None, nt=None, seed=None):
    w = wl.BY_NAME["tiny"]
    inp = wl.make_inputs(w, seed=seed, local_num_tokens=nt)
    p = Params(w.ep_size, w.num_experts, w.top_k, w.max_tokens_per_rank, w.hidden_size,
               w.hidden_row_bytes, 0, enable_rank_mask=True)
    o = OracleMoEEp(p)
    res = o.dispatch(inp.hidden, inp.topk_ids, inp.topk_weights, active_rank_mask=mask)
    return p, o, res, inp


def independent_masks(p, inp, active):
    table = owner_table(p.ep_size, p.num_experts)
    out = []
    for s in range(p.ep_size):
        row = []
        for t in range(inp.local_num_tokens[s]):
            dests = expected_destinations(inp.topk_ids[s][t], table, p.num_experts, active, p.ep_size)
            row.append(sum(1 << d for d in dests))
        out.append(row)
    return out


def _to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    return {"f32": lambda x: x, "bf16": oracle.f32_to_bf16_bits_rne,
            "f16": lambda x: x.astype(np.float16)}[dtype](a)


def _from_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    return oracle.bf16_bits_to_f32(a) if dtype == "bf16" else a.astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("mask", [None, 0b1011, 0b0001])
def test_combine_rank_indicators_sum_to_destination_mask(dtype, mask):
    p, o, res, inp = _dispatch_tiny(mask)
    tpr = res[0].tokens_per_rank
    eo = []
    for d in range(p.ep_size):
        a = np.full((p.ep_size * tpr, p.hidden_size), np.nan, np.float32)
        a[res[d].valid] = float(2 ** d)
        eo.append(_to_dtype(a, dtype))
    out = o.combine(eo, dtype, active_rank_mask=mask)
    expect = independent_masks(p, inp, oracle.ALL_RANKS if mask is None else mask)
    for s in range(p.ep_size):
        got = _from_dtype(out[s], dtype)
        for t in range(inp.local_num_tokens[s]):
            assert (got[t] == float(expect[s][t])).all()


def test_f16_combine_rounds_ties_to_even_and_overflows():
    """Two-rank sums that are exact in float32 and fall halfway between two
    binary16 values, worked from the format (11 significant bits, largest
    finite 65504, smallest subnormal 2^-24): 1 + 2^-11 -> 1 (even),
    1 + 3*2^-11 -> 1 + 2^-9 (even), 65504 + 16 = 65520 -> infinity (the
    tie goes to the even neighbour 2^16, past the largest finite value),
    -1 - 2^-11 -> -1; and 2^-24 + 2^-24 = 2^-23 exactly among the
    subnormals (binary16 values are all multiples of 2^-24, so no sum of
    them falls between two subnormals)."""
    p = Params(2, 2, 2, 1, 5, 4)
    o = OracleMoEEp(p)
    o.dispatch([np.zeros((1, 4), np.uint8), np.zeros((0, 4), np.uint8)],
               [np.array([[0, 1]], np.int32), np.zeros((0, 2), np.int32)])
    a = np.array([[1.0, 1.0 + 2.0 ** -10, 65504.0, -1.0, 2.0 ** -24], [np.nan] * 5], np.float16)
    b = np.array([[2.0 ** -11, 2.0 ** -11, 16.0, -(2.0 ** -11), 2.0 ** -24], [np.nan] * 5], np.float16)
    out = o.combine([a, b], "f16")[0][0]
    bits = out.view(np.uint16)
    assert bits[0] == 0x3C00                        # 1.0
    assert bits[1] == 0x3C02                        # 1 + 2^-9
    assert bits[2] == 0x7C00                        # +infinity
    assert bits[3] == 0xBC00                        # -1.0
    assert bits[4] == 0x0002                        # 2^-23


def test_f16_rounding_matches_torch_random_sums():
    """Sums of two random binary16 values rounded to binary16: the oracle's
    (NumPy) against torch's CPU conversion of the same float32 sums."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 4096)).astype(np.float16)
    p = Params(2, 2, 2, 1, 4096, 4)
    o = OracleMoEEp(p)
    o.dispatch([np.zeros((1, 4), np.uint8), np.zeros((0, 4), np.uint8)],
               [np.array([[0, 1]], np.int32), np.zeros((0, 2), np.int32)])
    eo = [np.stack([x[0], x[0]]), np.stack([x[1], x[1]])]
    out = o.combine(eo, "f16")[0][0]
    s32 = torch.from_numpy(x[0].astype(np.float32)) + torch.from_numpy(x[1].astype(np.float32))
    np.testing.assert_array_equal(out.view(np.uint16), s32.to(torch.float16).numpy().view(np.uint16))


def test_combine_ones_sum_to_fanout():
    p, o, res, inp = _dispatch_tiny()
    tpr = res[0].tokens_per_rank
    eo = [np.where(res[d].valid[:, None], 1.0, np.nan).astype(np.float32)
          * np.ones((1, p.hidden_size), np.float32) for d in range(p.ep_size)]
    out = o.combine(eo, "f32")
    expect = independent_masks(p, inp, oracle.ALL_RANKS)
    for s in range(p.ep_size):
        for t in range(inp.local_num_tokens[s]):
            assert (out[s][t] == bin(expect[s][t]).count("1")).all()


def test_combine_ascending_rank_order():
    """2^24 + 1 - 2^24 in float32 is 0 in ascending rank order (1 is lost
    to rounding) and 1 in most other orders."""
    p = Params(3, 3, 3, 1, 1, 4)
    o = OracleMoEEp(p)
    o.dispatch([np.zeros((1, 4), np.uint8)] + [np.zeros((0, 4), np.uint8)] * 2, [np.array([[0, 1, 2]], np.int32)] + [np.zeros((0, 3), np.int32)] * 2,
               [np.array([[0.3, 0.3, 0.4]], np.float32)] + [np.zeros((0, 3), np.float32)] * 2)
    eo = [np.array([[2.0 ** 24], [np.nan], [np.nan]], np.float32),
          np.array([[1.0], [np.nan], [np.nan]], np.float32),
          np.array([[-(2.0 ** 24)], [np.nan], [np.nan]], np.float32)]
    out = o.combine(eo, "f32")
    assert out[0][0, 0] == 0.0


@pytest.mark.parametrize("mask", [None, 0b0111, 0b1000])
def test_combine_standin_reproduces_weighted_values(mask):
    """With expert rows = value x (weights of the rank's local experts), the
    combine output is value x (weights of the active experts)."""
    p, o, res, inp = _dispatch_tiny(mask)
    eo = oracle.expert_standin(p, res, inp.values, "f32")
    out = o.combine(eo, "f32", active_rank_mask=mask)
    active = oracle.ALL_RANKS if mask is None else mask
    table = owner_table(p.ep_size, p.num_experts)
    u = 2.0 ** -24
    for s in range(p.ep_size):
        assert not np.isnan(out[s]).any()
        for t in range(inp.local_num_tokens[s]):
            ids = inp.topk_ids[s][t]
            ws = [float(inp.topk_weights[s][t][j]) for j in range(p.top_k)
                  if (active >> int(table[ids[j]])) & 1]
            v = inp.values[s][t].astype(np.float64)
            expect = v * sum(ws)
            fan = len({int(table[e]) for e in ids if (active >> int(table[e])) & 1})
            bound = (fan + 2 * p.top_k + 2) * u * np.abs(v) * sum(abs(x) for x in ws) + 1e-30
            assert (np.abs(out[s][t] - expect) <= bound).all()
            if mask is None:
                assert abs(sum(ws) - 1.0) < 1e-6   # softmax weights of all K experts


def test_masked_rank_contributes_nothing():
    mask = 0b1101
    p, o, res, inp = _dispatch_tiny(mask)
    eo = oracle.expert_standin(p, res, inp.values, "f32")
    out1 = o.combine(eo, "f32", active_rank_mask=mask)
    o2 = OracleMoEEp(p)
    res2 = o2.dispatch(inp.hidden, inp.topk_ids, inp.topk_weights, active_rank_mask=mask)
    eo2 = [a.copy() for a in oracle.expert_standin(p, res2, inp.values, "f32")]
    eo2[1][:] = 1e30                                # rank 1 is masked off
    out2 = o2.combine(eo2, "f32", active_rank_mask=mask)
    for s in range(p.ep_size):
        np.testing.assert_array_equal(out1[s], out2[s])


def test_token_without_destination_combines_to_zero():
    p = Params(2, 4, 2, 2, 3, 4, enable_rank_mask=True)
    o = OracleMoEEp(p)
    ids = [np.array([[2, 3], [0, 9]], np.int32), np.array([[-1, 5]], np.int32)]
    o.dispatch([np.zeros((2, 4), np.uint8), np.zeros((1, 4), np.uint8)], ids,
               [np.ones((2, 2), np.float32), np.ones((1, 2), np.float32)], active_rank_mask=0b01)
    eo = [np.full((4, 3), np.nan, np.float32), np.full((4, 3), 7.0, np.float32)]
    eo[0][1] = 5.0                                   # token (0, 1) reached rank 0 only
    out = o.combine(eo, "f32", active_rank_mask=0b01)
    np.testing.assert_array_equal(out[0][0], np.zeros(3, np.float32))
    np.testing.assert_array_equal(out[0][1], np.full(3, 5.0, np.float32))
    np.testing.assert_array_equal(out[1][0], np.zeros(3, np.float32))
    assert not np.signbit(out[0][0]).any()


# --------------------------------------------------------------------------
# Contract rules
# --------------------------------------------------------------------------
def _small():
    p = Params(2, 4, 2, 4, 2, 4, enable_rank_mask=False)
    hid = [np.zeros((2, 4), np.uint8), np.zeros((1, 4), np.uint8)]
    ids = [np.array([[0, 2], [1, 3]], np.int32), np.array([[2, 3]], np.int32)]
    w = [np.ones((2, 2), np.float32), np.ones((1, 2), np.float32)]
    return p, hid, ids, w


def test_error_rules():
    p, hid, ids, w = _small()
    o = OracleMoEEp(p)
    with pytest.raises(OracleError) as e:
        o.combine([np.zeros((8, 2), np.float32)] * 2, "f32")
    assert e.value.kind == "state"
    for bad in (5, 1):
        with pytest.raises(OracleError) as e:
            o.dispatch(hid, ids, w, runtime_max_tokens_per_rank=bad)
        assert e.value.kind == "capacity"
    with pytest.raises(OracleError) as e:
        o.dispatch(hid, ids, w, active_rank_mask=1)
    assert e.value.kind == "mask"
    with pytest.raises(OracleError) as e:
        o.dispatch(hid, ids, [w[0], None])
    assert e.value.kind == "invalid_arg"
    res = o.dispatch(hid, ids, w, runtime_max_tokens_per_rank=2)
    assert res[0].tokens_per_rank == 2
    with pytest.raises(OracleError) as e:
        o.dispatch(hid, ids, w)
    assert e.value.kind == "state"
    o.combine([np.zeros((4, 2), np.float32)] * 2, "f32")
    # The pair is done: a second combine has nothing to combine, and the
    # next dispatch starts a new pair (one pair in flight at a time).
    with pytest.raises(OracleError) as e:
        o.combine([np.zeros((4, 2), np.float32)] * 2, "f32")
    assert e.value.kind == "state"
    res = o.dispatch(hid, ids, w)
    assert res[0].tokens_per_rank == 4
    o.combine([np.zeros((8, 2), np.float32)] * 2, "f32")
    o.destroy()
    o.destroy()
    with pytest.raises(OracleError) as e:
        o.dispatch(hid, ids, w)
    assert e.value.kind == "state"


def test_mask_rules():
    p, hid, ids, w = _small()
    p.enable_rank_mask = True
    o = OracleMoEEp(p)
    with pytest.raises(OracleError) as e:
        o.dispatch(hid, ids, w, active_rank_mask=0b100)
    assert e.value.kind == "mask"
    o.dispatch(hid, ids, w, active_rank_mask=0b01)
    with pytest.raises(OracleError) as e:
        o.combine([np.zeros((8, 2), np.float32)] * 2, "f32", active_rank_mask=0b11)
    assert e.value.kind == "mask"
    with pytest.raises(OracleError):
        o.combine([np.zeros((8, 2), np.float32)] * 2, "f32")
    o.combine([np.zeros((8, 2), np.float32)] * 2, "f32", active_rank_mask=0b01)


def test_active_rank_mask_helper():
    assert oracle.active_rank_mask([0, 2, 5]) == 0b100101
    assert oracle.active_rank_mask([]) == 0
    assert oracle.active_rank_mask([63]) == 1 << 63
    with pytest.raises(OracleError):
        oracle.active_rank_mask([64])


def test_eplb_rules():
    p, hid, ids, w = _small()
    stats = [np.arange(6, dtype=np.uint8), np.arange(6, 12, dtype=np.uint8)]
    with pytest.raises(OracleError) as e:
        OracleMoEEp(p).dispatch(hid, ids, w, eplb_local_stats=stats)      # no statistics configured
    assert e.value.kind == "invalid_arg"
    p.eplb_stats_bytes = 6
    with pytest.raises(OracleError) as e:
        OracleMoEEp(p).dispatch(hid, ids, w, eplb_local_stats=[stats[0], None])
    assert e.value.kind == "invalid_arg"
    res = OracleMoEEp(p).dispatch(hid, ids, w, eplb_local_stats=stats)
    for d in range(2):
        np.testing.assert_array_equal(res[d].eplb_global_stats, np.stack(stats))
    res = OracleMoEEp(p).dispatch(hid, ids, w)
    assert res[0].eplb_global_stats is None


def test_weights_absent_everywhere_is_allowed():
    p, hid, ids, _ = _small()
    o = OracleMoEEp(p)
    res = o.dispatch(hid, ids, None)
    assert res[0].topk_weights is None


def _params(**kw):
    base = dict(ep_size=2, num_experts=4, top_k=2, max_tokens_per_rank=4, hidden_size=2,
                hidden_row_bytes=4)
    base.update(kw)
    return Params(**base)


@pytest.mark.parametrize("kw", [
    # The active-rank mask is one uint64, one bit per rank
    # (NVLinkOneSidedAlltoAll, active_rank_mask()): 1..64 ranks.
    dict(ep_size=0, num_experts=4), dict(ep_size=65, num_experts=65), dict(ep_size=-1),
    # Contiguous ownership of equal blocks (the reading of "ranks that own
    # its selected experts", MoEEpCommunication, dispatch()) needs a positive
    # multiple of ep_size.
    dict(num_experts=3), dict(num_experts=6, ep_size=4), dict(num_experts=1, ep_size=2),
    dict(num_experts=0),
    # A token selects at least one expert (topk_ids is [local_num_tokens,
    # top_k], MoEEpCommunication, dispatch()); capacity, combine row size and
    # dispatched row size are sizes.
    dict(top_k=0), dict(top_k=-3), dict(max_tokens_per_rank=-1), dict(hidden_size=0),
    dict(hidden_row_bytes=0), dict(scale_row_bytes=-4),
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_params_rules_reject(kw):
    with pytest.raises(OracleError) as e:
        OracleMoEEp(_params(**kw))
    assert e.value.kind == "invalid_arg"


@pytest.mark.parametrize("kw", [
    dict(ep_size=1, num_experts=1), dict(ep_size=64, num_experts=64), dict(ep_size=64, num_experts=128),
    dict(num_experts=2), dict(top_k=1), dict(top_k=9), dict(max_tokens_per_rank=0),
    dict(scale_row_bytes=0), dict(scale_row_bytes=8), dict(hidden_size=1, hidden_row_bytes=1),
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_params_rules_accept(kw):
    OracleMoEEp(_params(**kw))


def test_ep_64_routes_to_rank_63():
    """At the largest group the top mask bit is a real rank: expert E-1 lives
    on rank 63 (NVLinkOneSidedAlltoAll, active_rank_mask(): a uint64 mask)."""
    p = _params(ep_size=64, num_experts=128, max_tokens_per_rank=1)
    o = OracleMoEEp(p)
    hid = [np.full((1, 4), s, np.uint8) for s in range(64)]
    ids = [np.array([[127, 0]], np.int32) for _ in range(64)]
    res = o.dispatch(hid, ids, None)
    for d in range(64):
        want = d in (0, 63)
        assert bool(res[d].valid.all()) == want
        assert bool(res[d].valid.any()) == want


def test_scales_all_or_none():
    """hidden_states_scale travels row-aligned with hidden_states
    (MoEEpCommunication, dispatch()), under the same every-rank-or-none rule
    as the weights (NVLinkOneSidedAlltoAll, dispatch()).  Ranks with no
    tokens still pass an empty [0, scale_row_bytes] array."""
    p, hid, ids, w = _small()
    p.scale_row_bytes = 3
    scl = [np.arange(6, dtype=np.uint8).reshape(2, 3), np.arange(10, 13, dtype=np.uint8).reshape(1, 3)]
    for partial in ([scl[0], None], [None, scl[1]]):
        with pytest.raises(OracleError) as e:
            OracleMoEEp(p).dispatch(hid, ids, w, hidden_states_scale=partial)
        assert e.value.kind == "invalid_arg"
    res = OracleMoEEp(p).dispatch(hid, ids, w, hidden_states_scale=scl)
    # token (0, 0) has experts 0 and 2: ranks 0 and 1; token (1, 0) experts 2, 3: rank 1
    np.testing.assert_array_equal(res[0].hidden_scale[0], scl[0][0])
    np.testing.assert_array_equal(res[1].hidden_scale[4], scl[1][0])
    res = OracleMoEEp(p).dispatch(hid, ids, w, hidden_states_scale=[None, None])
    assert res[0].hidden_scale is None


def test_scales_need_scale_row_bytes():
    """Scale rows are sized at creation (the pages' params); a step that
    passes scales to a group created without them is refused."""
    p, hid, ids, w = _small()
    assert p.scale_row_bytes == 0
    scl = [np.zeros((2, 0), np.uint8), np.zeros((1, 0), np.uint8)]
    with pytest.raises(OracleError) as e:
        OracleMoEEp(p).dispatch(hid, ids, w, hidden_states_scale=scl)
    assert e.value.kind == "invalid_arg"
    scl = [np.zeros((2, 4), np.uint8), np.zeros((1, 4), np.uint8)]
    with pytest.raises(OracleError) as e:
        OracleMoEEp(p).dispatch(hid, ids, w, hidden_states_scale=scl)
    assert e.value.kind == "invalid_arg"


@pytest.mark.parametrize("dtype", ["f64", "bytes", "fp8", "F32", "", "bfloat16"])
def test_combine_rejects_unknown_dtype(dtype):
    """The combine element types are float32, bfloat16 and float16; any
    other name is refused before anything is summed, and the dispatch stays
    pending (MoEEpCommunication, combine(): one combine per dispatch)."""
    p, hid, ids, w = _small()
    o = OracleMoEEp(p)
    o.dispatch(hid, ids, w)
    with pytest.raises(OracleError) as e:
        o.combine([np.zeros((8, 2), np.float32)] * 2, dtype)
    assert e.value.kind == "invalid_arg"
    o.combine([np.zeros((8, 2), np.float32)] * 2, "f32")


# --------------------------------------------------------------------------
# bfloat16 rounding against torch's CPU conversion
# --------------------------------------------------------------------------
def _torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_random_bits():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    ours = oracle.f32_to_bf16_bits_rne(x)
    ref = _torch_bf16_bits(x)
    nan = np.isnan(x)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert np.isnan(oracle.bf16_bits_to_f32(ours[nan])).all()


def test_bf16_rne_edge_cases():
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    specials = np.concatenate([
        hi | 0x8000,            # every exact tie
        hi | 0x7FFF, hi | 0x8001, hi,
    ]).astype(np.uint32)
    x = specials.view(np.float32)
    ours = oracle.f32_to_bf16_bits_rne(x)
    ref = _torch_bf16_bits(x)
    nan = np.isnan(x)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert np.isnan(oracle.bf16_bits_to_f32(ours[nan])).all()
    # named values
    f = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895313892515355e38, 1e-45], np.float32)
    np.testing.assert_array_equal(oracle.f32_to_bf16_bits_rne(f), _torch_bf16_bits(f))


def test_bf16_widen_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    np.testing.assert_array_equal(ours[~both_nan], ref[~both_nan])


# --------------------------------------------------------------------------
# Routing statistics against the closed form of the input recipe
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["dsv3", "large"])
def test_fanout_matches_closed_form(name):
    """Uniform distinct top-k: a rank holding epr of E experts is reached with
    probability 1 - C(E-epr, K)/C(E, K)."""
    w = wl.BY_NAME[name]
    inp = wl.make_inputs(w)
    p = Params(w.ep_size, w.num_experts, w.top_k, w.max_tokens_per_rank, w.hidden_size,
               w.hidden_row_bytes)
    fan = [bin(oracle.destination_mask(p, inp.topk_ids[s][t], oracle.ALL_RANKS)).count("1")
           for s in range(w.ep_size) for t in range(inp.local_num_tokens[s])]
    epr = w.num_experts // w.ep_size
    q = 1 - math.comb(w.num_experts - epr, w.top_k) / math.comb(w.num_experts, w.top_k)
    mean = w.ep_size * q
    sd = math.sqrt(np.var(fan) / len(fan))
    assert abs(np.mean(fan) - mean) < 5 * sd + 1e-9
    for s in range(w.ep_size):
        ids = inp.topk_ids[s]
        assert all(len(set(r)) == w.top_k for r in ids.tolist())
