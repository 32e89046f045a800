"""HIP-graph capture and replay of dispatch + combine at static shapes
(runtime_max_tokens_per_rank=None keeps shapes static: flashinfer.moe_ep.
MoEEpCommunication, dispatch()).  Both calls enqueue kernels only: no host
synchronisation, no allocation and no memset, so a captured round replays
on new inputs written in place.  Every replay is checked against the CPU
oracle, with eager work and synchronisations between replays.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from synth import workloads as wl
from tests import parity
from tests.parity import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from combine_token_dest_amd import _lib
    _lib.load()
    assert _lib.moe_ep_is_platform_supported(), "not a gfx950 device"


@pytest.mark.parametrize("name", ["tiny", "dsv3", "fp8"])
def test_graph_replays_match_oracle(name):
    w = wl.BY_NAME[name]
    log(f"[graph] capture {name}")
    c0 = parity.case_from_workload(w)
    c0.eplb = [np.full(64, s, np.uint8) for s in range(w.ep_size)]
    c0.eplb_bytes = 64
    moe = parity.make_gpu(c0)
    hid, ids, wts, sc = parity.upload(c0)
    stats = parity.upload_eplb(c0)
    tdt = torch.float32 if c0.combine_dtype == "f32" else torch.bfloat16
    rows = w.ep_size * w.max_tokens_per_rank
    eo = [torch.zeros((rows, w.hidden_size), dtype=tdt, device="cuda") for _ in range(w.ep_size)]
    outs = [torch.empty((n, w.hidden_size), dtype=tdt, device="cuda") for n in c0.n]

    # Warm-up round outside capture, then capture one full round.
    moe.dispatch(hid, ids, wts, hidden_states_scale=sc, eplb_local_stats=stats)
    moe.combine(eo, output=outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = moe.dispatch(hid, ids, wts, hidden_states_scale=sc, eplb_local_stats=stats)
        moe.combine(eo, output=outs)
    torch.cuda.synchronize()

    for i, seed in enumerate([11, 12, 13]):
        log(f"[graph] {name} replay {i} seed {seed}")
        c = parity.case_from_workload(w, seed=seed)
        c.eplb = [np.random.default_rng(seed + s).integers(0, 256, 64).astype(np.uint8) for s in range(w.ep_size)]
        c.eplb_bytes = 64
        om = oracle.OracleMoEEp(parity.oracle_params(c))
        ores = om.dispatch(c.hidden, c.ids, c.weights, hidden_states_scale=c.scale, eplb_local_stats=c.eplb)
        eo_host = parity.combine_inputs_host(c, ores)
        oout = om.combine(eo_host, c.combine_dtype)
        # eager work between replays: new inputs and expert outputs in place
        for s in range(w.ep_size):
            hid[s].copy_(torch.from_numpy(c.hidden[s]))
            ids[s].copy_(torch.from_numpy(c.ids[s]))
            wts[s].copy_(torch.from_numpy(c.weights[s]))
            if sc is not None:
                sc[s].copy_(torch.from_numpy(c.scale[s]))
            stats[s].copy_(torch.from_numpy(c.eplb[s]))
        for d in range(w.ep_size):
            eo[d].copy_(parity.host_to_torch(eo_host[d], c.combine_dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        parity.compare_dispatch(c, res, ores, f"{name} replay {i}")
        parity.compare_combine(c, outs, oout, f"{name} replay {i}")
    moe.destroy()


@pytest.mark.parametrize("order", ["source", "destination"])
def test_graph_replays_ragged_steps_with_device_counts(order):
    """One captured round replays steps whose token counts differ: the counts
    live in device memory and the kernels read them when they run."""
    w = wl.BY_NAME["ragged"]
    cap = w.max_tokens_per_rank
    log(f"[graph] capture ragged with device-resident counts, {order} order")
    full = parity.case_from_workload(w, local_num_tokens=[cap] * w.ep_size, seed=500)
    full.rtpr = None
    moe = parity.make_gpu(full, order=order)
    hid, ids, wts, _ = parity.upload(full)
    counts = torch.full((w.ep_size,), cap, dtype=torch.int32, device="cuda")
    rows = w.ep_size * cap
    eo = [torch.zeros((rows, w.hidden_size), dtype=torch.bfloat16, device="cuda") for _ in range(w.ep_size)]
    outs = [torch.zeros((cap, w.hidden_size), dtype=torch.bfloat16, device="cuda") for _ in range(w.ep_size)]
    mask = full.mask
    moe.dispatch(hid, ids, wts, active_rank_mask=mask, local_num_tokens_device=counts)
    moe.combine(eo, output=outs, active_rank_mask=mask)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = moe.dispatch(hid, ids, wts, active_rank_mask=mask, local_num_tokens_device=counts)
        moe.combine(eo, output=outs, active_rank_mask=mask)
    torch.cuda.synchronize()

    steps = [[5, 0, 300, 512, 0, 1, 17, 64], [0] * 8, [512] * 8, [3, 0, 2, 9, 0, 0, 4, 1]]
    for i, nt in enumerate(steps):
        log(f"[graph] ragged replay {i} n={nt}")
        c = parity.case_from_workload(w, local_num_tokens=nt, seed=600 + i)
        c.rtpr = cap
        om = oracle.OracleMoEEp(parity.oracle_params(c))
        ores = om.dispatch(c.hidden, c.ids, c.weights, runtime_max_tokens_per_rank=cap, active_rank_mask=mask)
        eo_host = parity.combine_inputs_host(c, ores)
        oout = om.combine(eo_host, "bf16", active_rank_mask=mask)
        for s in range(w.ep_size):
            n = nt[s]
            if n:
                hid[s][:n].copy_(torch.from_numpy(c.hidden[s]))
                ids[s][:n].copy_(torch.from_numpy(c.ids[s]))
                wts[s][:n].copy_(torch.from_numpy(c.weights[s]))
        counts.copy_(torch.tensor(nt, dtype=torch.int32))
        for d in range(w.ep_size):
            eo[d].copy_(parity.host_to_torch(eo_host[d], "bf16"))
        for o in outs:
            o.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        parity.compare_dispatch(c, res, ores, f"ragged replay {i}")
        parity.compare_combine(c, [outs[s][:nt[s]] for s in range(w.ep_size)], oout, f"ragged replay {i}")
        for s in range(w.ep_size):      # rows past the count are left alone
            assert (outs[s][nt[s]:].float() == 7.0).all()
    moe.destroy()


@pytest.mark.parametrize("order", ["source", "destination"])
@pytest.mark.parametrize("name", ["tiny", "fp8"])
def test_device_counts_are_clamped_to_the_buffers(name, order):
    """Counts outside [0, tokens_per_rank] are clamped by the kernels (4
    ranks, and 16 ranks with scale rows: both sizes of the kernels'
    argument blocks)."""
    w = wl.BY_NAME[name]
    cap = w.max_tokens_per_rank
    log(f"[graph] device counts clamped, {name}, {order} order")
    full = parity.case_from_workload(w)
    moe = parity.make_gpu(full, order=order)
    hid, ids, wts, scl = parity.upload(full)
    dev = ([-3, cap + 100, 5, cap] * w.ep_size)[:w.ep_size]
    counts = torch.tensor(dev, dtype=torch.int32, device="cuda")
    res = moe.dispatch(hid, ids, wts, hidden_states_scale=scl, local_num_tokens_device=counts)
    cdt = torch.float32 if w.combine_dtype == "f32" else torch.bfloat16
    outs = moe.combine([moe.get_combine_input_buffer(d, cdt) for d in range(w.ep_size)])
    torch.cuda.synchronize()
    nt = [min(max(x, 0), cap) for x in dev]
    c = parity.case_from_workload(w)
    c.hidden = [h[:n] for h, n in zip(c.hidden, nt)]
    c.ids = [x[:n] for x, n in zip(c.ids, nt)]
    c.weights = [x[:n] for x, n in zip(c.weights, nt)]
    if c.scale is not None:
        c.scale = [x[:n] for x, n in zip(c.scale, nt)]
    om = oracle.OracleMoEEp(parity.oracle_params(c))
    ores = om.dispatch(c.hidden, c.ids, c.weights, hidden_states_scale=c.scale, runtime_max_tokens_per_rank=cap)
    parity.compare_dispatch(c, res, ores, "clamped")
    assert [tuple(o.shape) for o in outs] == [(cap, w.hidden_size)] * w.ep_size
    moe.destroy()
