"""moe_ep_dispatch_noalloc against moe_ep_dispatch, through the C ABI.

The noalloc entry point is the same dispatch with its routing records in the
library's fixed device array instead of the workspace.  Each case runs the
existing entry point and the new one on the same seeded inputs, two rounds
in a row (the second with fewer tokens), and requires identical receive
regions and combine outputs, both also equal to the CPU oracle's.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from combine_token_dest_amd import _lib
from synth import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu


def _snapshot(res):
    """Host copies of what each destination received (ids, weights, and the
    hidden / scale rows of routed rows only: other rows are unspecified)."""
    out = []
    for r in res:
        ids = r.topk_ids.cpu().numpy()
        valid = ids[:, 0] != -1 if ids.size else np.zeros(0, bool)
        hid = r.hidden.view(torch.uint8).cpu().numpy().reshape(ids.shape[0], -1)[valid]
        w = None if r.topk_weights is None else r.topk_weights.cpu().numpy().view(np.uint32)
        sc = None if r.hidden_scale is None else \
            r.hidden_scale.view(torch.uint8).cpu().numpy().reshape(ids.shape[0], -1)[valid]
        out.append((r.tokens_per_rank, ids, w, hid, sc))
    return out


def _same(a, b, tag):
    assert len(a) == len(b)
    for d, (x, y) in enumerate(zip(a, b)):
        assert x[0] == y[0], f"{tag} rank {d}: tokens_per_rank"
        for i, what in ((1, "topk_ids"), (2, "topk_weights bits"), (3, "hidden bytes"), (4, "scale bytes")):
            if x[i] is None or y[i] is None:
                assert x[i] is None and y[i] is None, f"{tag} rank {d}: {what} presence"
            else:
                np.testing.assert_array_equal(x[i], y[i], err_msg=f"{tag} rank {d}: {what}")


def _round(c: parity.Case, moe, noalloc: bool, eo_host, device_counts=None):
    hid, ids, w, sc = parity.upload(c)
    kw = {}
    if device_counts is not None:
        kw["local_num_tokens_device"] = torch.tensor(device_counts, dtype=torch.int32, device="cuda")
    res = moe.dispatch(hid, ids, w, hidden_states_scale=sc, runtime_max_tokens_per_rank=c.rtpr,
                       active_rank_mask=c.mask, noalloc=noalloc, **kw)
    torch.cuda.synchronize()
    snap = _snapshot(res)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[c.combine_dtype]
    bufs = []
    for d in range(c.ep):
        buf = moe.get_combine_input_buffer(d, tdt)
        buf.copy_(parity.host_to_torch(eo_host[d], c.combine_dtype).view(buf.shape))
        bufs.append(buf)
    out = moe.combine(bufs, active_rank_mask=c.mask)
    torch.cuda.synchronize()
    return res, snap, [o.clone() for o in out]


def _oracle(c: parity.Case):
    om = parity.oracle.OracleMoEEp(parity.oracle_params(c))
    ores = om.dispatch(c.hidden, c.ids, c.weights, hidden_states_scale=c.scale,
                       runtime_max_tokens_per_rank=c.rtpr, active_rank_mask=c.mask)
    eo = parity.combine_inputs_host(c, ores)
    return ores, eo, om.combine(eo, c.combine_dtype, active_rank_mask=c.mask)


def _case(name, nt=None, seed=None):
    w = wl.BY_NAME[name]
    return parity.case_from_workload(w, local_num_tokens=nt, seed=seed)


# (workload, first step's token counts, second (smaller) step's token counts)
STEPS = [
    ("dsv3", None, [100, 0, 37, 128, 5, 64, 1, 90]),        # destination-major dispatch
    ("ragged", None, [7, 0, 19, 3, 0, 0, 11, 1]),            # source-row dispatch, mask, runtime bound
    ("fp8", None, [3] * 16),                                 # scale rows
    ("tiny", None, [16, 2, 0, 9]),
]


@pytest.mark.parametrize("name,nt1,nt2", STEPS, ids=[s[0] for s in STEPS])
def test_noalloc_matches_dispatch_two_rounds(name, nt1, nt2):
    print(f"[noalloc] {name}", flush=True)
    regular = noalloc = None
    try:
        for step, nt in enumerate((nt1, nt2)):
            c = _case(name, nt, seed=None if step == 0 else 7 + step)
            if regular is None:
                regular = parity.make_gpu(c)
                noalloc = parity.make_gpu(c)
            ores, eo, oout = _oracle(c)
            gres_a, snap_a, out_a = _round(c, regular, False, eo)
            gres_b, snap_b, out_b = _round(c, noalloc, True, eo)
            tag = f"{name} step {step}"
            _same(snap_a, snap_b, tag)
            parity.compare_dispatch(c, gres_b, ores, tag + " noalloc")
            parity.compare_combine(c, out_b, oout, tag + " noalloc")
            for s in range(c.ep):
                assert torch.equal(out_a[s].view(torch.uint8), out_b[s].view(torch.uint8)), f"{tag} rank {s}"
    finally:
        for m in (regular, noalloc):
            if m is not None:
                m.destroy()


def test_noalloc_device_counts_and_handles_in_turn():
    """Device-resident counts (the counts live in the fixed array too), and
    two handles taking turns with the array: each combine follows its own
    dispatch before the other handle's next noalloc dispatch."""
    c = _case("dsv3")
    ores, eo, oout = _oracle(c)
    a = parity.make_gpu(c)
    b = parity.make_gpu(c)
    try:
        counts = c.n
        _, snap_ref, out_ref = _round(c, a, False, eo, device_counts=counts)
        for moe in (a, b, a):
            _, snap, out = _round(c, moe, True, eo, device_counts=counts)
            _same(snap_ref, snap, "device counts")
            parity.compare_combine(c, out, oout, "device counts noalloc")
        small = [64, 0, 1, 128, 7, 0, 33, 2]
        c2 = _case("dsv3", small, seed=11)
        # the second, smaller step keeps full-size buffers (device counts)
        o2 = parity.oracle.OracleMoEEp(parity.oracle_params(c2))
        ores2 = o2.dispatch(c2.hidden, c2.ids, c2.weights)
        eo2 = parity.combine_inputs_host(c2, ores2)
        oout2 = o2.combine(eo2, c2.combine_dtype)
        full = _case("dsv3", seed=11)
        for s in range(c2.ep):                     # pad each rank's inputs to tpr rows
            n = small[s]
            full.hidden[s][:n] = c2.hidden[s]
            full.ids[s][:n] = c2.ids[s]
            full.weights[s][:n] = c2.weights[s]
        _, snap_r, out_r = _round(full, a, False, eo2, device_counts=small)
        _, snap_n, out_n = _round(full, b, True, eo2, device_counts=small)
        _same(snap_r, snap_n, "device counts, smaller step")
        for s in range(c2.ep):
            got = out_n[s][:small[s]]
            assert torch.equal(got.view(torch.uint8), out_r[s][:small[s]].view(torch.uint8)), f"rank {s}"
            np.testing.assert_array_equal(parity.torch_to_host(got, "bf16"), oout2[s], err_msg=f"rank {s}")
    finally:
        a.destroy()
        b.destroy()


def test_noalloc_at_the_largest_step():
    """64 ranks x 1024 tokens: exactly MOE_EP_NOALLOC_MAX_ROWS receive rows."""
    ep, tpr, K = 64, 1024, 2
    rng = np.random.default_rng(3)
    n = [int(x) for x in rng.integers(0, tpr + 1, ep)]
    n[5] = 0
    n[9] = tpr
    E = 128
    hidden = [rng.integers(0, 256, (k, 16), dtype=np.uint8) for k in n]
    ids = [np.stack([rng.choice(E, K, replace=False) for _ in range(k)]).astype(np.int32) if k
           else np.zeros((0, K), np.int32) for k in n]
    weights = [rng.random((k, K), dtype=np.float32) for k in n]
    c = parity.Case(ep, E, K, tpr, 8, 16, 0, hidden, ids, weights, None, None, None, None, "bf16",
                    name="ep64x1024")
    assert ep * tpr == _lib.MOE_EP_NOALLOC_MAX_ROWS
    eo = [wl.random_rows(rng, ep * tpr, 8, "bf16") for _ in range(ep)]
    a = parity.make_gpu(c)
    b = parity.make_gpu(c)
    try:
        _, snap_a, out_a = _round(c, a, False, eo)
        _, snap_b, out_b = _round(c, b, True, eo)
        _same(snap_a, snap_b, "64 x 1024")
        for s in range(ep):
            assert torch.equal(out_a[s].view(torch.uint8), out_b[s].view(torch.uint8)), f"rank {s}"
        # one row more than the area holds is refused on the host
        big = parity.Case(ep, E, K, tpr + 1, 8, 16, 0, hidden, ids, weights, None, None, None, None, "bf16")
        m = parity.make_gpu(big)
        try:
            hid, idt, wt, _ = parity.upload(big)
            with pytest.raises(_lib.MoeEpError) as e:
                m.dispatch(hid, idt, wt, noalloc=True)
            assert e.value.status == _lib.MOE_EP_ERR_CAPACITY
        finally:
            m.destroy()
    finally:
        a.destroy()
        b.destroy()


@pytest.mark.parametrize("name", ["dsv3", "ragged"])
def test_noalloc_round_replays_from_a_graph(name):
    """The callers the entry point is for capture it: a noalloc dispatch and
    its combine captured in one HIP graph, replayed on new inputs written in
    place (eager work and synchronisations between the replays), every
    replay equal to the oracle's round."""
    w = wl.BY_NAME[name]
    print(f"[noalloc] graph {name}", flush=True)
    c0 = _case(name)
    moe = parity.make_gpu(c0)
    try:
        hid, ids, wts, sc = parity.upload(c0)
        tdt = torch.float32 if c0.combine_dtype == "f32" else torch.bfloat16
        tpr = c0.rtpr if c0.rtpr is not None else w.max_tokens_per_rank
        rows = w.ep_size * tpr
        eo = [torch.zeros((rows, w.hidden_size), dtype=tdt, device="cuda") for _ in range(w.ep_size)]
        outs = [torch.empty((n, w.hidden_size), dtype=tdt, device="cuda") for n in c0.n]
        kw = dict(hidden_states_scale=sc, runtime_max_tokens_per_rank=c0.rtpr, active_rank_mask=c0.mask)
        moe.dispatch(hid, ids, wts, noalloc=True, **kw)
        moe.combine(eo, output=outs, active_rank_mask=c0.mask)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            res = moe.dispatch(hid, ids, wts, noalloc=True, **kw)
            moe.combine(eo, output=outs, active_rank_mask=c0.mask)
        torch.cuda.synchronize()
        for i, seed in enumerate([21, 22, 23]):
            # same token counts as the captured step (host counts are baked in)
            c = parity.case_from_workload(w, local_num_tokens=c0.n, seed=seed)
            ores, eo_host, oout = _oracle(c)
            for s in range(w.ep_size):
                if c.n[s]:
                    hid[s].copy_(torch.from_numpy(c.hidden[s]))
                    ids[s].copy_(torch.from_numpy(c.ids[s]))
                    wts[s].copy_(torch.from_numpy(c.weights[s]))
                    if sc is not None:
                        sc[s].copy_(torch.from_numpy(c.scale[s]))
            for d in range(w.ep_size):
                eo[d].copy_(parity.host_to_torch(eo_host[d], c.combine_dtype))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            parity.compare_dispatch(c, res, ores, f"{name} noalloc replay {i}")
            parity.compare_combine(c, outs, oout, f"{name} noalloc replay {i}")
    finally:
        moe.destroy()
