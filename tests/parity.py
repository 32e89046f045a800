"""Shared helpers of the GPU parity tests: run one dispatch/combine step on
both the HIP path (through the C ABI via combine_token_dest_amd.MoEEp) and
the CPU oracle on identical seeded inputs, and compare.

Bars (from the method's definition): receive-region ids, weights, and the
bytes of every routed hidden/scale row are bit-exact; combine outputs are
within 1e-5 relative (float32), 2e-2 absolute (bfloat16) or 1e-2 absolute
(float16) of the oracle's, and bit-identical, because both add in float32
in ascending rank order and round once.
"""

from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

import oracle
from synth import workloads as wl

# Combine tolerances.  Both sides add in the same order, so the tests also
# require identical bits; these bound what a different order could change:
# float32 relative 1e-5; bfloat16 absolute 2e-2 and float16 absolute 1e-2,
# above half an ulp for the |sums| < 8 (bfloat16) and < 32 (float16) the
# tests produce.
F32_RTOL = 1e-5
BF16_ATOL = 2e-2
F16_ATOL = 1e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class Case:
    """One step: params plus per-rank host inputs (all numpy)."""

    ep: int
    E: int
    K: int
    cap: int
    hidden_size: int
    H: int                                  # hidden row bytes
    S: int                                  # scale row bytes
    hidden: List[np.ndarray]
    ids: List[np.ndarray]
    weights: Optional[List[np.ndarray]]
    scale: Optional[List[np.ndarray]]
    values: Optional[List[np.ndarray]]      # float32 [n_s, hidden_size] for the stand-in
    rtpr: Optional[int]
    mask: Optional[int]
    combine_dtype: str
    invalid_id: int = -1
    enable_rank_mask: bool = False
    name: str = ""
    eplb: Optional[List[np.ndarray]] = None     # uint8 [eplb_bytes] per rank
    eplb_bytes: int = 0

    @property
    def n(self):
        return [a.shape[0] for a in self.ids]


def case_from_workload(w: wl.Workload, local_num_tokens=None, seed=None) -> Case:
    inp = wl.make_inputs(w, seed=seed, local_num_tokens=local_num_tokens)
    rtpr = max(inp.local_num_tokens) if w.runtime_max == "max" else None
    return Case(w.ep_size, w.num_experts, w.top_k, w.max_tokens_per_rank, w.hidden_size,
                w.hidden_row_bytes, w.scale_row_bytes, inp.hidden, inp.topk_ids, inp.topk_weights,
                inp.scale, inp.values, rtpr, inp.active_rank_mask, w.combine_dtype,
                enable_rank_mask=inp.active_rank_mask is not None, name=w.name)


def oracle_params(c: Case) -> oracle.Params:
    return oracle.Params(c.ep, c.E, c.K, c.cap, c.hidden_size, c.H, c.S, c.invalid_id, c.enable_rank_mask,
                         c.eplb_bytes)


def make_gpu(c: Case, device="cuda", checkpointable=False, order="auto"):
    from combine_token_dest_amd import MoEEp
    return MoEEp(c.ep, c.E, c.K, c.cap, c.hidden_size, hidden_row_bytes=c.H, scale_row_bytes=c.S,
                 combine_max_elem_bytes=4 if c.combine_dtype == "f32" else 2,
                 invalid_expert_id=c.invalid_id, enable_rank_mask=c.enable_rank_mask,
                 eplb_stats_bytes=c.eplb_bytes, checkpointable=checkpointable, dispatch_order=order,
                 device=device)


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload(c: Case, device="cuda"):
    hid = [to_dev(h, device) for h in c.hidden]
    ids = [to_dev(i.astype(np.int32), device) for i in c.ids]
    w = None if c.weights is None else [to_dev(x, device) for x in c.weights]
    sc = None if c.scale is None else [to_dev(x, device) for x in c.scale]
    return hid, ids, w, sc


def upload_eplb(c: Case, device="cuda"):
    return None if c.eplb is None else [to_dev(x, device) for x in c.eplb]


def combine_inputs_host(c: Case, ores) -> List[np.ndarray]:
    """Combine inputs from the oracle's own dispatch result (never the GPU's)."""
    p = oracle_params(c)
    if c.values is not None and c.weights is not None:
        return oracle.expert_standin(p, ores, c.values, c.combine_dtype)
    rng = np.random.default_rng(99)
    out = []
    for d in range(c.ep):
        a = wl.random_rows(rng, c.ep * ores[d].tokens_per_rank, c.hidden_size, c.combine_dtype)
        if c.combine_dtype == "bf16":
            a[~ores[d].valid] = 0x7FC0                 # a bfloat16 NaN
        else:
            a[~ores[d].valid] = np.nan
        out.append(a)
    return out


def host_to_torch(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "f32":
        return to_dev(a.astype(np.float32), device)
    if dtype == "f16":
        return to_dev(a.astype(np.float16), device)
    return to_dev(a.view(np.int16), device).view(torch.bfloat16)


def torch_to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype in ("f32", "f16"):
        return t.cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def compare_dispatch(c: Case, gres, ores, tag=""):
    """Bit-exact comparison of every receive region."""
    for d in range(c.ep):
        g, o = gres[d], ores[d]
        assert g.tokens_per_rank == o.tokens_per_rank, f"{tag} rank {d}: tokens_per_rank"
        gi = g.topk_ids.cpu().numpy()
        np.testing.assert_array_equal(gi, o.topk_ids, err_msg=f"{tag} rank {d}: topk_ids")
        if o.topk_weights is None:
            assert g.topk_weights is None
        else:
            gw = g.topk_weights.cpu().numpy()
            np.testing.assert_array_equal(gw.view(np.uint32), o.topk_weights.view(np.uint32),
                                          err_msg=f"{tag} rank {d}: topk_weights bits")
        v = o.valid
        gh = g.hidden.view(torch.uint8).cpu().numpy().reshape(len(v), c.H)
        np.testing.assert_array_equal(gh[v], o.hidden[v], err_msg=f"{tag} rank {d}: hidden bytes")
        if o.hidden_scale is None:
            assert g.hidden_scale is None
        else:
            gs = g.hidden_scale.view(torch.uint8).cpu().numpy().reshape(len(v), c.S)
            np.testing.assert_array_equal(gs[v], o.hidden_scale[v], err_msg=f"{tag} rank {d}: scale bytes")
        if o.eplb_global_stats is None:
            assert g.eplb_global_stats is None
        else:
            ge = g.eplb_global_stats.view(torch.uint8).cpu().numpy().reshape(c.ep, c.eplb_bytes)
            np.testing.assert_array_equal(ge, o.eplb_global_stats, err_msg=f"{tag} rank {d}: eplb stats")


def compare_combine(c: Case, gout, oout, tag=""):
    for s in range(c.ep):
        g = torch_to_host(gout[s], c.combine_dtype)
        o = oout[s]
        assert g.shape == o.shape, f"{tag} rank {s}: shape {g.shape} vs {o.shape}"
        if c.combine_dtype == "f32":
            gf, of = g, o
            assert not np.isnan(gf).any(), f"{tag} rank {s}: NaN in output"
            np.testing.assert_allclose(gf, of, rtol=F32_RTOL, atol=0, err_msg=f"{tag} rank {s}")
            np.testing.assert_array_equal(gf.view(np.uint32), of.view(np.uint32),
                                          err_msg=f"{tag} rank {s}: float32 bits")
        elif c.combine_dtype == "f16":
            gf, of = g.astype(np.float32), o.astype(np.float32)
            assert not np.isnan(gf).any(), f"{tag} rank {s}: NaN in output"
            np.testing.assert_allclose(gf, of, rtol=0, atol=F16_ATOL, err_msg=f"{tag} rank {s}")
            np.testing.assert_array_equal(g.view(np.uint16), o.view(np.uint16),
                                          err_msg=f"{tag} rank {s}: float16 bits")
        else:
            gf, of = oracle.bf16_bits_to_f32(g), oracle.bf16_bits_to_f32(o)
            assert not np.isnan(gf).any(), f"{tag} rank {s}: NaN in output"
            np.testing.assert_allclose(gf, of, rtol=0, atol=BF16_ATOL, err_msg=f"{tag} rank {s}")
            np.testing.assert_array_equal(g, o, err_msg=f"{tag} rank {s}: bfloat16 bits")


def run_step(c: Case, *, zero_copy=True, device="cuda", check=True, moe=None, order="auto"):
    """One dispatch + combine on the GPU and in the oracle; compare both."""
    p = oracle_params(c)
    om = oracle.OracleMoEEp(p)
    ores = om.dispatch(c.hidden, c.ids, c.weights, hidden_states_scale=c.scale,
                       runtime_max_tokens_per_rank=c.rtpr, active_rank_mask=c.mask, eplb_local_stats=c.eplb)
    eo_host = combine_inputs_host(c, ores)
    oout = om.combine(eo_host, c.combine_dtype, active_rank_mask=c.mask)

    own = moe is None
    if own:
        moe = make_gpu(c, device, order=order)
    hid, ids, w, sc = upload(c, device)
    mask_arg = None if c.mask is None else c.mask
    gres = moe.dispatch(hid, ids, w, hidden_states_scale=sc, runtime_max_tokens_per_rank=c.rtpr,
                        active_rank_mask=mask_arg, eplb_local_stats=upload_eplb(c, device))
    torch.cuda.synchronize()
    if check:
        compare_dispatch(c, gres, ores, c.name)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[c.combine_dtype]
    eo_dev = []
    for d in range(c.ep):
        if zero_copy:
            buf = moe.get_combine_input_buffer(d, tdt)
            buf.copy_(host_to_torch(eo_host[d], c.combine_dtype, device).view(buf.shape))
            eo_dev.append(buf)
        else:
            eo_dev.append(host_to_torch(eo_host[d], c.combine_dtype, device))
    gout = moe.combine(eo_dev, active_rank_mask=mask_arg)
    torch.cuda.synchronize()
    if check:
        compare_combine(c, gout, oout, c.name)
    if own:
        moe.destroy()
    return gres, ores, gout, oout
