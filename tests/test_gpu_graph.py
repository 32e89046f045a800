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
