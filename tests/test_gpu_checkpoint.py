"""checkpoint_prepare / checkpoint_restore on a library-mapped workspace
(flashinfer.moe_ep.NVLinkOneSidedAlltoAll and CakeAlltoAll,
checkpoint_prepare() and checkpoint_restore()): the physical memory is
released and re-backed while the workspace keeps its addresses, so a graph
captured before the checkpoint replays correctly after the restore.  Both
calls repeat as no-ops, and the round's entry points refuse to run while
the memory is released.
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


def _load_round(c, hid, ids, wts, eo):
    om = oracle.OracleMoEEp(parity.oracle_params(c))
    ores = om.dispatch(c.hidden, c.ids, c.weights)
    eo_host = parity.combine_inputs_host(c, ores)
    oout = om.combine(eo_host, c.combine_dtype)
    for s in range(c.ep):
        hid[s].copy_(torch.from_numpy(c.hidden[s]))
        ids[s].copy_(torch.from_numpy(c.ids[s]))
        wts[s].copy_(torch.from_numpy(c.weights[s]))
    for d in range(c.ep):
        eo[d].copy_(parity.host_to_torch(eo_host[d], c.combine_dtype))
    torch.cuda.synchronize()
    return ores, oout


def test_eager_round_on_library_mapped_workspace():
    log("[checkpoint] eager round, vmm workspace")
    c = parity.case_from_workload(wl.BY_NAME["dsv3"])
    moe = parity.make_gpu(c, checkpointable=True)
    parity.run_step(c, moe=moe)
    moe.destroy()


def test_checkpoint_release_restore_and_graph_replay():
    from combine_token_dest_amd import MoeEpError, _lib
    w = wl.BY_NAME["dsv3"]
    log("[checkpoint] capture dsv3 on a vmm workspace")
    c0 = parity.case_from_workload(w)
    moe = parity.make_gpu(c0, checkpointable=True)
    hid, ids, wts, _ = parity.upload(c0)
    rows = w.ep_size * w.max_tokens_per_rank
    eo = [torch.zeros((rows, w.hidden_size), dtype=torch.bfloat16, device="cuda") for _ in range(w.ep_size)]
    outs = [torch.empty((n, w.hidden_size), dtype=torch.bfloat16, device="cuda") for n in c0.n]
    moe.dispatch(hid, ids, wts)
    moe.combine(eo, output=outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = moe.dispatch(hid, ids, wts)
        moe.combine(eo, output=outs)
    torch.cuda.synchronize()

    c = parity.case_from_workload(w, seed=31)
    ores, oout = _load_round(c, hid, ids, wts, eo)
    g.replay()
    torch.cuda.synchronize()
    parity.compare_dispatch(c, res, ores, "before checkpoint")
    parity.compare_combine(c, outs, oout, "before checkpoint")

    ws_bytes = moe.workspace.numel()
    free0 = torch.cuda.mem_get_info()[0]
    log("[checkpoint] prepare")
    moe.checkpoint_prepare()
    moe.checkpoint_prepare()                      # a repeat does nothing
    free1 = torch.cuda.mem_get_info()[0]
    log(f"[checkpoint] freed {free1 - free0} of {ws_bytes} workspace bytes")
    assert free1 - free0 >= 0.9 * ws_bytes
    with pytest.raises(MoeEpError) as e:          # refused on the host, nothing enqueued
        moe.dispatch(hid, ids, wts)
    assert e.value.status == _lib.MOE_EP_ERR_STATE

    log("[checkpoint] restore")
    moe.checkpoint_restore()
    moe.checkpoint_restore()                      # nothing to restore
    free2 = torch.cuda.mem_get_info()[0]
    assert free1 - free2 >= 0.9 * ws_bytes

    for i, seed in enumerate([32, 33]):
        log(f"[checkpoint] replay after restore {i}")
        c = parity.case_from_workload(w, seed=seed)
        ores, oout = _load_round(c, hid, ids, wts, eo)
        g.replay()
        torch.cuda.synchronize()
        parity.compare_dispatch(c, res, ores, f"after restore {i}")
        parity.compare_combine(c, outs, oout, f"after restore {i}")
    # eager rounds keep working on the restored workspace
    parity.run_step(parity.case_from_workload(w, seed=34), moe=moe)
    del g
    moe.destroy()


def test_checkpoint_only_between_rounds():
    from combine_token_dest_amd import MoeEpError, _lib
    log("[checkpoint] refused mid-round")
    c = parity.case_from_workload(wl.BY_NAME["tiny"])
    moe = parity.make_gpu(c, checkpointable=True)
    hid, ids, wts, _ = parity.upload(c)
    moe.dispatch(hid, ids, wts)
    with pytest.raises(MoeEpError) as e:
        moe.checkpoint_prepare()
    assert e.value.status == _lib.MOE_EP_ERR_STATE
    moe.combine([moe.get_combine_input_buffer(d, torch.float32) for d in range(c.ep)])
    torch.cuda.synchronize()
    moe.checkpoint_prepare()
    moe.checkpoint_restore()
    parity.run_step(c, moe=moe)
    moe.destroy()


def test_caller_owned_workspace_cannot_checkpoint():
    from combine_token_dest_amd import MoeEpError, _lib
    c = parity.case_from_workload(wl.BY_NAME["tiny"])
    moe = parity.make_gpu(c)
    with pytest.raises(MoeEpError) as e:
        moe.checkpoint_prepare()
    assert e.value.status == _lib.MOE_EP_ERR_UNSUPPORTED
    moe.destroy()
