"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every test prints the case it runs before touching the GPU.
"""

from __future__ import annotations

import dataclasses
import zlib

import numpy as np
import pytest
import torch

import oracle
from synth import workloads as wl
from tests import parity
from tests.golden_cases import all_cases
from tests.parity import Case, log

pytestmark = pytest.mark.gpu

GOLDEN = all_cases()


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from combine_token_dest_amd import _lib
    _lib.load()      # raises when the library is missing: no fallback
    assert _lib.moe_ep_is_platform_supported(), "not a gfx950 device"


# --------------------------------------------------------------------------
# The five workloads at full size
# --------------------------------------------------------------------------
ORDERS = ["source", "destination"]


@pytest.mark.parametrize("order", ORDERS)
@pytest.mark.parametrize("name", [w.name for w in wl.WORKLOADS])
def test_workload_full_size(name, order):
    w = wl.BY_NAME[name]
    log(f"[parity] workload {name} seed {w.seed} order {order}")
    c = parity.case_from_workload(w)
    parity.run_step(c, zero_copy=True, order=order)


@pytest.mark.parametrize("tpr", [1, 3, 32, 64, 256])
def test_dsv3_shape_at_decode_capacities(tpr):
    """The DeepSeek-V3 shape (8 ranks, 14 KiB rows) at other capacities: the
    destination-major grid from a fraction of one XCD block up to four
    resident generations, and the source-row grid from 8 rows up, both
    orders and AUTO.  At 32 tokens per rank a ragged step also runs under a
    runtime bound of 5."""
    w = dataclasses.replace(wl.BY_NAME["dsv3"], max_tokens_per_rank=tpr)
    c = parity.case_from_workload(w, seed=9000 + tpr)
    for order in ORDERS + ["auto"]:
        log(f"[parity] dsv3 shape tpr {tpr} order {order}")
        parity.run_step(c, zero_copy=order != "source", order=order)
    if tpr == 32:
        c = parity.case_from_workload(w, local_num_tokens=[5, 0, 1, 2, 0, 5, 3, 0], seed=9100)
        c.rtpr = 5
        for order in ORDERS:
            log(f"[parity] dsv3 shape tpr 32, runtime bound 5, ragged, order {order}")
            parity.run_step(c, zero_copy=True, order=order)


@pytest.mark.parametrize("order", ORDERS)
def test_f16_combine_dsv3_shape(order):
    """The DeepSeek-V3-shaped round with float16 expert outputs: combine
    widens, adds in float32 and rounds once to float16."""
    w = wl.BY_NAME["dsv3"]
    c = parity.case_from_workload(w)
    c.combine_dtype = "f16"
    log(f"[parity] dsv3 float16 combine order {order}")
    parity.run_step(c, zero_copy=order == "destination", order=order)


@pytest.mark.parametrize("name,expect", [("tiny", "destination"), ("dsv3", "destination"),
                                         ("fp8", "source"), ("ragged", "source")])
def test_auto_order_choice(name, expect):
    """AUTO takes the destination-major kernel only for groups of at most 16
    ranks with ep^2 * tokens_per_rank <= 16384 whose source rows alone do
    not fill the chip, and stays bit-exact."""
    w = wl.BY_NAME[name]
    log(f"[parity] workload {name} auto order")
    c = parity.case_from_workload(w)
    moe = parity.make_gpu(c)
    parity.run_step(c, moe=moe)
    assert moe.last_dispatch_order == expect
    moe.destroy()


@pytest.mark.parametrize("fill,expect", [(512, "destination"), (410, "destination"), (307, "source")])
def test_auto_order_at_prefill_capacity(fill, expect):
    """Past the ep^2 * tokens_per_rank bound (8 ranks x 512 tokens of 14 KiB
    rows), AUTO takes the destination-major order only when at least 80% of
    the rows are real tokens (host counts); either way the step is bit-exact,
    with combine under its residency cap (rows of 14 chunks)."""
    w = dataclasses.replace(wl.BY_NAME["dsv3"], max_tokens_per_rank=512)
    c = parity.case_from_workload(w, local_num_tokens=[fill] * 8, seed=9512 + fill)
    log(f"[parity] dsv3 shape tpr 512, {fill} tokens per rank, auto order")
    moe = parity.make_gpu(c)
    parity.run_step(c, moe=moe)
    assert moe.last_dispatch_order == expect
    moe.destroy()


def test_dsv3_with_expert_load_statistics():
    """The DeepSeek-V3-shaped round with int32 [256] per-rank statistics gathered."""
    w = wl.BY_NAME["dsv3"]
    log("[parity] dsv3 + eplb statistics")
    c = parity.case_from_workload(w)
    rng = np.random.default_rng(77)
    c.eplb = [rng.integers(0, 1000, size=w.num_experts).astype(np.int32).view(np.uint8) for _ in range(w.ep_size)]
    c.eplb_bytes = w.num_experts * 4
    parity.run_step(c, zero_copy=True)


@pytest.mark.parametrize("name", ["dsv3", "ragged"])
def test_workload_separate_combine_input(name):
    w = wl.BY_NAME[name]
    log(f"[parity] workload {name} separate expert_output tensors")
    c = parity.case_from_workload(w)
    parity.run_step(c, zero_copy=False)


@pytest.mark.parametrize("order", ORDERS)
def test_ragged_steps_on_one_handle(order):
    """Steps with different local counts and tokens_per_rank reuse one handle."""
    w = wl.BY_NAME["ragged"]
    c0 = parity.case_from_workload(w)
    moe = parity.make_gpu(c0, order=order)
    for i, nt in enumerate([[5, 0, 300, 512, 0, 1, 17, 64], [0] * 8, [1, 0, 0, 0, 0, 0, 0, 0],
                            [512] * 8, [3, 0, 2, 9, 0, 0, 4, 1]]):
        log(f"[parity] ragged step {i} n={nt} order {order}")
        c = parity.case_from_workload(w, local_num_tokens=nt, seed=2000 + i)
        parity.run_step(c, moe=moe)
    moe.destroy()


# --------------------------------------------------------------------------
# Hand-worked examples through the GPU
# --------------------------------------------------------------------------
@pytest.mark.parametrize("order", ORDERS)
@pytest.mark.parametrize("case", GOLDEN, ids=[g.name for g in GOLDEN])
def test_golden_on_gpu(case, order):
    log(f"[parity] golden {case.name} order {order}")
    p = case.params
    c = Case(p["ep_size"], p["num_experts"], p["top_k"], p["max_tokens_per_rank"], p["hidden_size"],
             p["hidden_row_bytes"], p["scale_row_bytes"], case.hidden, case.topk_ids, case.topk_weights,
             case.scale, None, case.runtime_max_tokens_per_rank, case.active_rank_mask, case.combine_dtype,
             invalid_id=p["invalid_expert_id"], enable_rank_mask=bool(p["enable_rank_mask"]), name=case.name,
             eplb=case.eplb_local_stats, eplb_bytes=p.get("eplb_stats_bytes", 0))
    moe = parity.make_gpu(c, order=order)
    hid, ids, w, sc = parity.upload(c)
    res = moe.dispatch(hid, ids, w, hidden_states_scale=sc, runtime_max_tokens_per_rank=c.rtpr,
                       active_rank_mask=c.mask, eplb_local_stats=parity.upload_eplb(c))
    e = case.expect
    for d in range(c.ep):
        assert res[d].tokens_per_rank == e["tokens_per_rank"]
        np.testing.assert_array_equal(res[d].topk_ids.cpu().numpy(), np.array(e["topk_ids"][d], np.int32))
        np.testing.assert_array_equal(res[d].topk_weights.cpu().numpy(),
                                      np.array(e["topk_weights"][d], np.float32))
        gh = res[d].hidden.view(torch.uint8).cpu().numpy().reshape(-1, c.H)
        for r, row in e["hidden_valid_rows"][d].items():
            np.testing.assert_array_equal(gh[int(r)], np.array(row, np.uint8))
        if "scale_valid_rows" in e:
            gs = res[d].hidden_scale.view(torch.uint8).cpu().numpy().reshape(-1, c.S)
            for r, row in e["scale_valid_rows"][d].items():
                np.testing.assert_array_equal(gs[int(r)], np.array(row, np.uint8))
        if "eplb_global_stats" in e:
            np.testing.assert_array_equal(res[d].eplb_global_stats.cpu().numpy(),
                                          np.array(e["eplb_global_stats"], np.uint8))
    eo = [parity.host_to_torch(case.expert_output[d], c.combine_dtype) for d in range(c.ep)]
    out = moe.combine(eo, active_rank_mask=case.combine_mask)
    for s in range(c.ep):
        g = parity.torch_to_host(out[s], c.combine_dtype)
        if c.combine_dtype == "f32":
            np.testing.assert_array_equal(g, case.expect_combine[s])
        else:
            np.testing.assert_array_equal(g, case.expect_combine[s])
    moe.destroy()


# --------------------------------------------------------------------------
# Edge cases: shapes, vector widths, masks, ids, empty ranks
# --------------------------------------------------------------------------
def random_case(seed, ep, E, K, cap, n, hidden_size, H, S=0, rtpr=None, mask=None, dtype="bf16",
                weights=True, invalid=-1, id_lo=None, id_hi=None, name="", eplb=0):
    rng = np.random.default_rng(seed)
    lo = 0 if id_lo is None else id_lo
    hi = E if id_hi is None else id_hi
    ids = [rng.integers(lo, hi, size=(n[s], K)).astype(np.int32) for s in range(ep)]
    hidden = [rng.integers(0, 256, size=(n[s], H)).astype(np.uint8) for s in range(ep)]
    w = [rng.standard_normal((n[s], K)).astype(np.float32) for s in range(ep)] if weights else None
    sc = [rng.integers(0, 256, size=(n[s], S)).astype(np.uint8) for s in range(ep)] if S else None
    st = [rng.integers(0, 256, size=eplb).astype(np.uint8) for _ in range(ep)] if eplb else None
    return Case(ep, E, K, cap, hidden_size, H, S, hidden, ids, w, sc, None, rtpr, mask, dtype,
                invalid_id=invalid, enable_rank_mask=mask is not None, name=name, eplb=st, eplb_bytes=eplb)


EDGE = [
    # name, kwargs
    ("ep1", dict(ep=1, E=4, K=2, cap=7, n=[7], hidden_size=64, H=128)),
    ("ep3_oddK", dict(ep=3, E=9, K=3, cap=33, n=[33, 0, 20], hidden_size=100, H=200)),
    ("ep5_rtpr", dict(ep=5, E=10, K=4, cap=64, n=[3, 40, 0, 17, 1], hidden_size=130, H=260, rtpr=50)),
    ("vec8_hidden", dict(ep=4, E=8, K=2, cap=9, n=[9, 9, 9, 9], hidden_size=4, H=24)),
    ("vec4_hidden", dict(ep=4, E=8, K=2, cap=9, n=[9, 2, 9, 0], hidden_size=6, H=12)),
    ("vec2_hidden", dict(ep=4, E=8, K=2, cap=9, n=[1, 2, 3, 4], hidden_size=3, H=6)),
    ("vec1_hidden", dict(ep=4, E=8, K=2, cap=9, n=[9, 8, 7, 6], hidden_size=7, H=7)),
    ("f32_odd_hidden", dict(ep=4, E=8, K=2, cap=12, n=[12, 5, 0, 11], hidden_size=37, H=148, dtype="f32")),
    ("f32_hidden2", dict(ep=2, E=2, K=1, cap=5, n=[5, 4], hidden_size=2, H=8, dtype="f32")),
    ("bf16_hidden1", dict(ep=3, E=3, K=2, cap=5, n=[5, 4, 3], hidden_size=1, H=2)),
    ("f16_vec8", dict(ep=4, E=8, K=3, cap=12, n=[12, 5, 0, 11], hidden_size=512, H=1024, dtype="f16")),
    ("f16_odd_hidden", dict(ep=5, E=10, K=2, cap=9, n=[9, 1, 4, 0, 7], hidden_size=37, H=74, dtype="f16")),
    ("f16_hidden1_mask", dict(ep=4, E=8, K=2, cap=6, n=[6, 6, 2, 0], hidden_size=1, H=2, dtype="f16",
                              mask=0b1011)),
    ("scales_odd", dict(ep=4, E=16, K=4, cap=16, n=[16, 3, 0, 9], hidden_size=256, H=256, S=13)),
    ("scales_vec4", dict(ep=4, E=16, K=4, cap=16, n=[16, 3, 0, 9], hidden_size=256, H=256, S=36)),
    ("ids_out_of_range", dict(ep=4, E=8, K=4, cap=10, n=[10, 10, 10, 10], hidden_size=64, H=128,
                              id_lo=-3, id_hi=12)),
    ("invalid_is_E", dict(ep=4, E=8, K=2, cap=10, n=[10, 0, 10, 3], hidden_size=64, H=128, invalid=8)),
    # every token reaches no rank: combine writes zeros without loading a row
    ("no_token_reaches_a_rank", dict(ep=4, E=8, K=3, cap=10, n=[10, 3, 0, 7], hidden_size=64, H=128,
                                     id_lo=-5, id_hi=0, dtype="f32")),
    ("mask_some", dict(ep=8, E=64, K=6, cap=40, n=[40, 39, 0, 1, 2, 40, 13, 7], hidden_size=512, H=1024,
                       mask=0b10110101)),
    ("mask_none_active", dict(ep=4, E=8, K=2, cap=8, n=[8, 8, 8, 8], hidden_size=32, H=64, mask=0)),
    ("no_weights", dict(ep=4, E=8, K=3, cap=8, n=[8, 1, 0, 5], hidden_size=32, H=64, weights=False)),
    ("big_row_multi_pass", dict(ep=2, E=4, K=2, cap=6, n=[6, 5], hidden_size=40000, H=80000)),
    ("k16", dict(ep=8, E=256, K=16, cap=32, n=[32] * 8, hidden_size=128, H=256)),
    ("k65_crosses_a_wave", dict(ep=4, E=256, K=65, cap=5, n=[5, 3, 0, 2], hidden_size=64, H=128)),
    ("k130_crosses_a_workgroup", dict(ep=2, E=512, K=130, cap=3, n=[3, 1], hidden_size=32, H=64)),
    ("wide_ep64", dict(ep=64, E=128, K=8, cap=4, n=[4] * 64, hidden_size=64, H=128,
                       mask=((1 << 64) - 1) & ~(1 << 5))),
    ("ep64_bit63_only", dict(ep=64, E=64, K=4, cap=3, n=[3] * 64, hidden_size=16, H=32, mask=1 << 63)),
    ("all_empty_cap", dict(ep=4, E=8, K=2, cap=6, n=[0, 0, 0, 0], hidden_size=16, H=32)),
    ("all_empty_rtpr0", dict(ep=4, E=8, K=2, cap=6, n=[0, 0, 0, 0], hidden_size=16, H=32, rtpr=0)),
    ("cap0", dict(ep=2, E=2, K=1, cap=0, n=[0, 0], hidden_size=16, H=32)),
    ("eplb_int32_experts", dict(ep=8, E=64, K=4, cap=20, n=[20, 0, 3, 20, 7, 0, 1, 19], hidden_size=256, H=512,
                                eplb=64 * 4)),
    ("eplb_odd_bytes", dict(ep=5, E=10, K=2, cap=6, n=[6, 2, 0, 5, 1], hidden_size=32, H=64, eplb=13)),
    ("eplb_all_empty_rtpr0", dict(ep=4, E=8, K=2, cap=6, n=[0, 0, 0, 0], hidden_size=16, H=32, rtpr=0, eplb=40)),
    ("eplb_mask", dict(ep=8, E=64, K=6, cap=40, n=[40, 39, 0, 1, 2, 40, 13, 7], hidden_size=512, H=1024,
                       mask=0b10110101, eplb=256)),
    # the kernels' argument blocks hold 8 ranks up to ep = 8 and 64 above:
    # the last rank's rows, records and statistics on each side of the switch
    ("ep8_last_rank_block", dict(ep=8, E=32, K=5, cap=24, n=[3, 0, 24, 9, 1, 0, 17, 24], hidden_size=256,
                                 H=512, S=36, eplb=40, mask=0b11011111)),
    ("ep9_first_large_block", dict(ep=9, E=36, K=5, cap=24, n=[3, 0, 24, 9, 1, 0, 17, 24, 11], hidden_size=256,
                                   H=512, S=36, eplb=40, mask=0b110111111)),
    ("ep9_f16_rtpr", dict(ep=9, E=18, K=3, cap=20, n=[20, 4, 0, 7, 20, 1, 0, 3, 19], hidden_size=100, H=200,
                          rtpr=20, dtype="f16")),
]


@pytest.mark.parametrize("name,kw", EDGE, ids=[e[0] for e in EDGE])
def test_edge_case(name, kw):
    c = random_case(zlib.crc32(name.encode()) % 10000, name=name, **kw)
    for order in ORDERS:
        log(f"[parity] edge {name} order {order}")
        parity.run_step(c, zero_copy=True, order=order)
    log(f"[parity] edge {name} separate combine input")
    parity.run_step(c, zero_copy=False)


def random_small_config(seed):
    """A random small step: any ep up to 16, top_k up to 10, ragged counts
    (some ranks empty), odd row sizes, optional scales, weights, mask,
    runtime bound and statistics."""
    rng = np.random.default_rng(seed)
    ep = int(rng.integers(1, 17))
    K = int(rng.integers(1, 11))
    E = ep * int(rng.integers(1, 9))
    cap = int(rng.integers(0, 41))
    n = [int(rng.integers(0, cap + 1)) if rng.random() < 0.8 else 0 for _ in range(ep)]
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    hidden_size = int(rng.choice([1, 3, 8, 50, 128, 515, 2048]))
    H = int(rng.choice([2, 6, 12, 24, 100, 256, 1030, 4104]))
    S = int(rng.choice([0, 0, 4, 13, 56]))
    rtpr = None if rng.random() < 0.5 else int(rng.integers(max(n + [0]), cap + 1))
    mask = None
    if ep > 1 and rng.random() < 0.4:
        mask = int(rng.integers(0, 1 << ep))
    invalid = -1 if rng.random() < 0.7 else E
    eplb = int(rng.choice([0, 0, 7, 64]))
    return dict(ep=ep, E=E, K=K, cap=cap, n=n, hidden_size=hidden_size, H=H, S=S, rtpr=rtpr, mask=mask,
                dtype=dtype, weights=rng.random() < 0.85, invalid=invalid, id_lo=-1, id_hi=E + 1, eplb=eplb)


def test_random_small_configs():
    """120 seeded random steps, both dispatch orders, against the oracle."""
    for seed in range(120):
        kw = random_small_config(seed)
        c = random_case(7000 + seed, name=f"random{seed}", **kw)
        for order in ORDERS:
            log(f"[parity] random config {seed} order {order}: ep={kw['ep']} K={kw['K']} "
                f"n={kw['n']} H={kw['H']} S={kw['S']} {kw['dtype']}")
            parity.run_step(c, zero_copy=order == "source", order=order)


def random_larger_config(seed):
    """A random step with model-sized rows: up to 16 ranks and 64 tokens per
    rank, rows of 1-14 KiB (odd element counts too), fp8-style scale rows."""
    rng = np.random.default_rng(seed)
    ep = int(rng.integers(1, 17))
    K = int(rng.integers(1, 11))
    E = ep * int(rng.integers(1, 9))
    cap = int(rng.integers(0, 65))
    n = [int(rng.integers(0, cap + 1)) if rng.random() < 0.85 else 0 for _ in range(ep)]
    hidden_size = int(rng.choice([1024, 2048, 4096, 7168, 7169]))
    H = int(rng.choice([hidden_size * 2, hidden_size, 14336, 8192, 7168 + 16]))
    S = int(rng.choice([0, 0, 224, 56]))
    rtpr = None if rng.random() < 0.5 else int(rng.integers(max(n + [0]), cap + 1))
    mask = int(rng.integers(0, 1 << ep)) if ep > 1 and rng.random() < 0.3 else None
    return dict(ep=ep, E=E, K=K, cap=cap, n=n, hidden_size=hidden_size, H=H, S=S, rtpr=rtpr, mask=mask,
                dtype="f32" if rng.random() < 0.2 else "bf16", weights=rng.random() < 0.9,
                invalid=-1, id_lo=-1, id_hi=E + 1, eplb=int(rng.choice([0, 0, 64])))


def test_random_larger_configs():
    """60 seeded random steps with model-sized rows, both dispatch orders."""
    for seed in range(60):
        kw = random_larger_config(seed)
        c = random_case(8000 + seed, name=f"larger{seed}", **kw)
        for order in ORDERS:
            log(f"[parity] random larger config {seed} order {order}: ep={kw['ep']} K={kw['K']} "
                f"n={kw['n']} H={kw['H']} S={kw['S']} hidden={kw['hidden_size']} {kw['dtype']}")
            parity.run_step(c, zero_copy=order == "destination", order=order)


def test_misaligned_rows_use_narrow_vectors():
    """Row pointers offset by 1, 2, 4 and 8 bytes from 16-byte alignment."""
    for off in (1, 2, 4, 8):
        log(f"[parity] misaligned hidden pointers offset {off}")
        c = random_case(off, ep=3, E=6, K=2, cap=8, n=[8, 3, 5], hidden_size=256, H=512, name=f"mis{off}")
        p = parity.oracle_params(c)
        om = oracle.OracleMoEEp(p)
        ores = om.dispatch(c.hidden, c.ids, c.weights)
        moe = parity.make_gpu(c)
        hid = []
        for h in c.hidden:
            big = torch.zeros(h.size + 64, dtype=torch.uint8, device="cuda")
            view = big[off:off + h.size].view(h.shape)
            view.copy_(torch.from_numpy(h).cuda())
            hid.append(view)
        ids = [parity.to_dev(i) for i in c.ids]
        w = [parity.to_dev(x) for x in c.weights]
        gres = moe.dispatch(hid, ids, w)
        parity.compare_dispatch(c, gres, ores, f"mis{off}")
        eo_host = parity.combine_inputs_host(c, ores)
        oout = om.combine(eo_host, "bf16")
        # misaligned expert_output and output by one element (2 bytes)
        eo = []
        for d in range(c.ep):
            big = torch.zeros(eo_host[d].size + 16, dtype=torch.bfloat16, device="cuda")
            v = big[1:1 + eo_host[d].size].view(eo_host[d].shape)
            v.copy_(parity.host_to_torch(eo_host[d], "bf16"))
            eo.append(v)
        outs = []
        for s in range(c.ep):
            big = torch.zeros(c.n[s] * c.hidden_size + 16, dtype=torch.bfloat16, device="cuda")
            outs.append(big[3:3 + c.n[s] * c.hidden_size].view(c.n[s], c.hidden_size))
        gout = moe.combine(eo, output=outs)
        torch.cuda.synchronize()
        parity.compare_combine(c, gout, oout, f"mis{off}")
        moe.destroy()


def test_int64_topk_ids_are_accepted():
    """The wrapper converts int64 expert ids to the library's int32."""
    log("[parity] int64 topk_ids")
    c = random_case(21, ep=4, E=16, K=4, cap=9, n=[9, 0, 4, 7], hidden_size=64, H=128)
    p = parity.oracle_params(c)
    om = oracle.OracleMoEEp(p)
    ores = om.dispatch(c.hidden, c.ids, c.weights)
    moe = parity.make_gpu(c)
    hid, ids, w, _ = parity.upload(c)
    gres = moe.dispatch(hid, [i.to(torch.int64) for i in ids], w)
    torch.cuda.synchronize()
    parity.compare_dispatch(c, gres, ores, "int64 ids")
    moe.combine([moe.get_combine_input_buffer(d, torch.bfloat16) for d in range(c.ep)])
    moe.destroy()


def test_expert_output_3d_form():
    """[ep, tpr, hidden] is accepted as the same memory as [ep*tpr, hidden]."""
    log("[parity] expert_output as [ep, tpr, hidden]")
    c = random_case(5, ep=4, E=8, K=2, cap=10, n=[10, 4, 0, 7], hidden_size=96, H=192)
    p = parity.oracle_params(c)
    om = oracle.OracleMoEEp(p)
    ores = om.dispatch(c.hidden, c.ids, c.weights)
    eo_host = parity.combine_inputs_host(c, ores)
    oout = om.combine(eo_host, "bf16")
    moe = parity.make_gpu(c)
    hid, ids, w, _ = parity.upload(c)
    moe.dispatch(hid, ids, w)
    tpr = 10
    eo = [parity.host_to_torch(eo_host[d], "bf16").view(c.ep, tpr, c.hidden_size) for d in range(c.ep)]
    gout = moe.combine(eo)
    torch.cuda.synchronize()
    parity.compare_combine(c, gout, oout, "3d")
    moe.destroy()


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_combine_of_buffers_only_takes_the_buffer_dtype(dtype):
    """combine([None] * ep) with no output tensors reads every rank's combine
    input buffer in the dtype the caller asked that buffer for."""
    log(f"[parity] combine of the workspace buffers only, {dtype}")
    c = random_case(6, ep=4, E=8, K=2, cap=9, n=[9, 3, 0, 8], hidden_size=40, H=80, dtype=dtype)
    p = parity.oracle_params(c)
    om = oracle.OracleMoEEp(p)
    ores = om.dispatch(c.hidden, c.ids, c.weights)
    eo_host = parity.combine_inputs_host(c, ores)
    oout = om.combine(eo_host, dtype)
    moe = parity.make_gpu(c)
    hid, ids, w, _ = parity.upload(c)
    moe.dispatch(hid, ids, w)
    tdt = torch.float32 if dtype == "f32" else torch.float16
    for d in range(c.ep):
        buf = moe.get_combine_input_buffer(d, tdt)
        buf.copy_(parity.host_to_torch(eo_host[d], dtype).view(buf.shape))
    gout = moe.combine([None] * c.ep)
    torch.cuda.synchronize()
    assert all(o.dtype == tdt for o in gout)
    parity.compare_combine(c, gout, oout, "buffers only")
    moe.destroy()


# --------------------------------------------------------------------------
# Writes stay where the method puts them; reads skip what it never needs
# --------------------------------------------------------------------------
@pytest.mark.parametrize("order", ORDERS)
def test_writes_stay_in_bounds(order):
    """Workspace bytes the step has no business touching keep a canary, and
    output guard bands stay intact."""
    log(f"[parity] canary / guard bands order {order}")
    c = random_case(11, ep=4, E=8, K=2, cap=16, n=[9, 0, 12, 5], hidden_size=64, H=128, S=20, rtpr=12)
    p = parity.oracle_params(c)
    om = oracle.OracleMoEEp(p)
    ores = om.dispatch(c.hidden, c.ids, c.weights, hidden_states_scale=c.scale, runtime_max_tokens_per_rank=12)
    moe = parity.make_gpu(c, order=order)
    moe.workspace.fill_(0x5A)
    hid, ids, w, sc = parity.upload(c)
    gres = moe.dispatch(hid, ids, w, hidden_states_scale=sc, runtime_max_tokens_per_rank=12)
    torch.cuda.synchronize()
    parity.compare_dispatch(c, gres, ores, "canary")
    tpr = 12
    rows = c.ep * tpr
    for d in range(c.ep):
        # hidden / scale bytes of invalid rows are not written
        gh = gres[d].hidden.view(torch.uint8).cpu().numpy().reshape(rows, c.H)
        assert (gh[~ores[d].valid] == 0x5A).all()
        gs = gres[d].hidden_scale.view(torch.uint8).cpu().numpy().reshape(rows, c.S)
        assert (gs[~ores[d].valid] == 0x5A).all()
        # rows past ep*tpr of the capacity-sized regions are not written
        ws = moe.workspace
        base = gres[d].hidden.data_ptr() - ws.data_ptr()
        tail = ws[base + rows * c.H: base + c.ep * c.cap * c.H].cpu().numpy()
        assert (tail == 0x5A).all()
        ib = gres[d].topk_ids.data_ptr() - ws.data_ptr()
        tail = ws[ib + rows * c.K * 4: ib + c.ep * c.cap * c.K * 4].cpu().numpy()
        assert (tail == 0x5A).all()
        # dispatch leaves the combine input buffer alone
        cb = moe.get_combine_input_buffer(d, torch.bfloat16)
        assert (cb.view(torch.uint8).cpu().numpy() == 0x5A).all()
    eo_host = parity.combine_inputs_host(c, ores)
    oout = om.combine(eo_host, "bf16")
    eo = [parity.host_to_torch(eo_host[d], "bf16") for d in range(c.ep)]
    guard = 64
    outs, bigs = [], []
    for s in range(c.ep):
        big = torch.full((c.n[s] * c.hidden_size + 2 * guard,), 7.0, dtype=torch.bfloat16, device="cuda")
        bigs.append(big)
        outs.append(big[guard:guard + c.n[s] * c.hidden_size].view(c.n[s], c.hidden_size))
    gout = moe.combine(eo, output=outs)
    torch.cuda.synchronize()
    parity.compare_combine(c, gout, oout, "canary")
    for s in range(c.ep):
        b = bigs[s].float().cpu().numpy()
        assert (b[:guard] == 7.0).all() and (b[len(b) - guard:] == 7.0).all()
    moe.destroy()


def test_masked_rank_buffers_never_read():
    """NaN in every row of a masked-off rank and in every unrouted row."""
    log("[parity] NaN poison on masked ranks")
    w = wl.BY_NAME["ragged"]
    c = parity.case_from_workload(w, local_num_tokens=[50, 0, 31, 7, 0, 0, 64, 9])
    p = parity.oracle_params(c)
    om = oracle.OracleMoEEp(p)
    ores = om.dispatch(c.hidden, c.ids, c.weights, runtime_max_tokens_per_rank=c.rtpr, active_rank_mask=c.mask)
    eo_host = [a.copy() for a in parity.combine_inputs_host(c, ores)]
    for d in w.masked_ranks:
        eo_host[d][:] = 0x7FC0
    oout = om.combine(eo_host, "bf16", active_rank_mask=c.mask)
    moe = parity.make_gpu(c)
    hid, ids, wt, _ = parity.upload(c)
    moe.dispatch(hid, ids, wt, runtime_max_tokens_per_rank=c.rtpr, active_rank_mask=c.mask)
    eo = [parity.host_to_torch(eo_host[d], "bf16") for d in range(c.ep)]
    gout = moe.combine(eo, active_rank_mask=c.mask)
    torch.cuda.synchronize()
    parity.compare_combine(c, gout, oout, "poison")
    moe.destroy()


@pytest.mark.parametrize("layout", ["forward", "reverse", "uneven", "misaligned", "misaligned_uneven", "masked", "mixed"])
def test_combine_input_layouts(layout):
    """Combine inputs placed in one buffer in different layouts.  The kernel
    computes row addresses from a base and a stride when the read ranks'
    inputs lie at a constant stride (forward, reverse, masked: the masked
    ranks are never read, so their inputs do not count) and reads the
    per-rank table otherwise (uneven; mixed: some ranks pass their combine
    input buffer).  The misaligned layouts (2-byte alignment only, so one
    element per lane) take each path once."""
    log(f"[parity] combine input layout {layout}")
    if layout == "masked":
        w = wl.BY_NAME["ragged"]
        c = parity.case_from_workload(w, local_num_tokens=[50, 0, 31, 7, 0, 0, 64, 9])
    else:
        w = dataclasses.replace(wl.BY_NAME["dsv3"], max_tokens_per_rank=16)
        c = parity.case_from_workload(w)
    p = parity.oracle_params(c)
    om = oracle.OracleMoEEp(p)
    ores = om.dispatch(c.hidden, c.ids, c.weights, runtime_max_tokens_per_rank=c.rtpr, active_rank_mask=c.mask)
    eo_host = parity.combine_inputs_host(c, ores)
    oout = om.combine(eo_host, c.combine_dtype, active_rank_mask=c.mask)
    moe = parity.make_gpu(c)
    hid, ids, wt, _ = parity.upload(c)
    moe.dispatch(hid, ids, wt, runtime_max_tokens_per_rank=c.rtpr, active_rank_mask=c.mask)
    n = eo_host[0].size                        # elements per rank
    ep = c.ep
    gap = 4096                                 # elements between consecutive inputs
    if layout in ("forward", "masked", "mixed"):
        offs = [d * (n + gap) for d in range(ep)]
    elif layout == "reverse":
        offs = [(ep - 1 - d) * (n + gap) for d in range(ep)]
    elif layout == "uneven":
        offs, o = [], 0
        for d in range(ep):
            offs.append(o)
            o += n + gap + 64 * d * d
    elif layout == "misaligned":               # odd element offsets at a constant stride
        offs = [d * (n + gap) + 1 for d in range(ep)]
    else:                                      # misaligned_uneven
        offs = [d * (n + gap) + 1 + (d % 3) for d in range(ep)]
    big = torch.full((max(offs) + n + 8,), float("nan"), dtype=torch.bfloat16, device="cuda")
    eo = []
    for d in range(ep):
        v = big[offs[d]:offs[d] + n].view(eo_host[d].shape)
        v.copy_(parity.host_to_torch(eo_host[d], c.combine_dtype).view(eo_host[d].shape))
        eo.append(v)
    if layout == "mixed":
        for d in (2, 5):
            buf = moe.get_combine_input_buffer(d, torch.bfloat16)
            buf.copy_(eo[d].view(buf.shape))
            eo[d] = None
    gout = moe.combine(eo, active_rank_mask=c.mask)
    torch.cuda.synchronize()
    parity.compare_combine(c, gout, oout, f"layout {layout}")
    moe.destroy()


@pytest.mark.parametrize("layout", ["forward", "reverse", "uneven", "misaligned", "empty_ranks", "one_rank"])
def test_combine_output_layouts(layout):
    """Outputs placed in one buffer in different layouts, the inputs in the
    combine input buffers.  Outputs at a constant stride (forward, reverse,
    misaligned; with empty ranks, whose outputs are NULL and do not count;
    a single rank with tokens) take the compact launch, the uneven layout
    the per-rank output table.  Every output row matches the oracle and no
    byte between the outputs is written."""
    log(f"[parity] combine output layout {layout}")
    w = dataclasses.replace(wl.BY_NAME["dsv3"], max_tokens_per_rank=16)
    nt = {"empty_ranks": [16, 0, 3, 16, 0, 0, 9, 1], "one_rank": [0, 0, 0, 0, 0, 11, 0, 0]}.get(layout)
    c = parity.case_from_workload(w, local_num_tokens=nt, seed=7300)
    p = parity.oracle_params(c)
    om = oracle.OracleMoEEp(p)
    ores = om.dispatch(c.hidden, c.ids, c.weights)
    eo_host = parity.combine_inputs_host(c, ores)
    oout = om.combine(eo_host, c.combine_dtype)
    moe = parity.make_gpu(c)
    hid, ids, wt, _ = parity.upload(c)
    moe.dispatch(hid, ids, wt)
    for d in range(c.ep):
        buf = moe.get_combine_input_buffer(d, torch.bfloat16)
        buf.copy_(parity.host_to_torch(eo_host[d], c.combine_dtype).view(buf.shape))
    hs, ep, n = c.hidden_size, c.ep, c.n
    stride = c.cap * hs + 512                  # elements between consecutive outputs
    if layout == "reverse":
        offs = [(ep - 1 - s) * stride for s in range(ep)]
    elif layout == "uneven":
        offs = [s * stride + 64 * s * s for s in range(ep)]
    elif layout == "misaligned":
        offs = [s * stride + 1 for s in range(ep)]
    else:
        offs = [s * stride for s in range(ep)]
    canary = -1024.0
    big = torch.full((max(offs) + stride + 8,), canary, dtype=torch.bfloat16, device="cuda")
    outs = [big[offs[s]:offs[s] + n[s] * hs].view(n[s], hs) for s in range(ep)]
    gout = moe.combine([None] * ep, output=outs)
    torch.cuda.synchronize()
    parity.compare_combine(c, gout, oout, f"output layout {layout}")
    written = torch.zeros(big.numel(), dtype=torch.bool, device="cuda")
    for s in range(ep):
        written[offs[s]:offs[s] + n[s] * hs] = True
    assert bool((big[~written] == canary).all()), "combine wrote outside its output rows"
    moe.destroy()


@pytest.mark.parametrize("ep,cap,nt", [(3, 5, [5, 0, 3]), (5, 7, [7, 1, 0, 6, 2])])
@pytest.mark.parametrize("order", ORDERS)
def test_device_counts_with_a_partial_slot_group(ep, cap, nt, order):
    """Device-resident counts with ep * tpr not a multiple of 8 (15 and 35
    slots): combine's grid holds whole groups of 8 slots, and the slots past
    the last one must store nothing.  Both combine input paths: the
    library's buffers (constant stride) and per-rank tensors at uneven
    offsets (the per-rank table)."""
    name = f"devn_ep{ep}_cap{cap}"
    full = random_case(zlib.crc32(name.encode()) % 10000, ep=ep, E=2 * ep, K=2, cap=cap, n=[cap] * ep,
                       hidden_size=96, H=192, name=name)
    for zero_copy in (True, False):
        log(f"[parity] {name} device counts {nt}, order {order}, zero_copy {zero_copy}")
        moe = parity.make_gpu(full, order=order)
        hid, ids, wts, _ = parity.upload(full)
        counts = torch.tensor(nt, dtype=torch.int32, device="cuda")
        res = moe.dispatch(hid, ids, wts, local_num_tokens_device=counts)
        c = dataclasses.replace(full, hidden=[h[:n] for h, n in zip(full.hidden, nt)],
                                ids=[x[:n] for x, n in zip(full.ids, nt)],
                                weights=[x[:n] for x, n in zip(full.weights, nt)])
        om = oracle.OracleMoEEp(parity.oracle_params(c))
        ores = om.dispatch(c.hidden, c.ids, c.weights, runtime_max_tokens_per_rank=cap)
        eo_host = parity.combine_inputs_host(c, ores)
        oout = om.combine(eo_host, "bf16")
        torch.cuda.synchronize()
        parity.compare_dispatch(c, res, ores, name)
        if zero_copy:
            eo = []
            for d in range(ep):
                buf = moe.get_combine_input_buffer(d, torch.bfloat16)
                buf.copy_(parity.host_to_torch(eo_host[d], "bf16").view(buf.shape))
                eo.append(buf)
        else:
            n_el = eo_host[0].size
            big = torch.full((ep * (n_el + 64) + 64 * ep * ep,), float("nan"), dtype=torch.bfloat16, device="cuda")
            eo, off = [], 0
            for d in range(ep):
                v = big[off:off + n_el].view(eo_host[d].shape)
                v.copy_(parity.host_to_torch(eo_host[d], "bf16").view(eo_host[d].shape))
                eo.append(v)
                off += n_el + 64 + 64 * d
        outs = [torch.full((cap, full.hidden_size), 7.0, dtype=torch.bfloat16, device="cuda") for _ in range(ep)]
        moe.combine(eo, output=outs)
        torch.cuda.synchronize()
        parity.compare_combine(c, [outs[s][:nt[s]] for s in range(ep)], oout, name)
        for s in range(ep):      # rows past the count are left alone
            assert (outs[s][nt[s]:].float() == 7.0).all()
        moe.destroy()


# --------------------------------------------------------------------------
# Call protocol on the GPU path
# --------------------------------------------------------------------------
def test_call_protocol_errors_leave_state_unchanged():
    from combine_token_dest_amd import MoeEpError, _lib
    log("[parity] call protocol")
    c = random_case(3, ep=4, E=8, K=2, cap=8, n=[8, 2, 0, 5], hidden_size=32, H=64, mask=0b1011)
    moe = parity.make_gpu(c)
    hid, ids, w, _ = parity.upload(c)
    with pytest.raises(MoeEpError) as e:
        moe.combine([None] * c.ep, active_rank_mask=0b1011)
    assert e.value.status == _lib.MOE_EP_ERR_STATE
    with pytest.raises(MoeEpError) as e:
        moe.get_combine_input_buffer(0, torch.bfloat16)
    assert e.value.status == _lib.MOE_EP_ERR_STATE
    moe.dispatch(hid, ids, w, active_rank_mask=0b1011)
    with pytest.raises(MoeEpError) as e:
        moe.dispatch(hid, ids, w, active_rank_mask=0b1011)
    assert e.value.status == _lib.MOE_EP_ERR_STATE
    with pytest.raises(MoeEpError) as e:
        moe.combine([None] * c.ep, active_rank_mask=0b1111)
    assert e.value.status == _lib.MOE_EP_ERR_MASK
    with pytest.raises(MoeEpError) as e:
        moe.combine([None] * c.ep)
    assert e.value.status == _lib.MOE_EP_ERR_MASK
    outs = moe.combine([moe.get_combine_input_buffer(d, torch.bfloat16) for d in range(c.ep)],
                       active_rank_mask=0b1011)
    torch.cuda.synchronize()
    assert [tuple(o.shape) for o in outs] == [(8, 32), (2, 32), (0, 32), (5, 32)]
    moe.destroy()
    moe.destroy()


def test_wrapper_rejects_host_and_strided_tensors():
    """MoEEp refuses a CPU tensor or a non-contiguous one, naming the
    argument and rank, before anything reaches the library."""
    log("[parity] wrapper argument checks")
    c = random_case(5, ep=4, E=8, K=2, cap=8, n=[8, 2, 0, 5], hidden_size=32, H=64)
    moe = parity.make_gpu(c)
    hid, ids, w, _ = parity.upload(c)
    bad = list(hid)
    bad[1] = hid[1].cpu()
    with pytest.raises(ValueError, match=r"hidden_states\[1\] is on cpu"):
        moe.dispatch(bad, ids, w)
    strided = list(w)
    strided[3] = torch.empty((c.n[3], 2 * c.K), dtype=torch.float32, device="cuda")[:, ::2]
    with pytest.raises(ValueError, match=r"topk_weights\[3\] must be contiguous"):
        moe.dispatch(hid, ids, strided)
    moe.dispatch(hid, ids, w)                  # nothing was enqueued: the handle is still idle
    outs = moe.combine([moe.get_combine_input_buffer(d, torch.bfloat16) for d in range(c.ep)])
    torch.cuda.synchronize()
    assert [tuple(o.shape) for o in outs] == [(8, 32), (2, 32), (0, 32), (5, 32)]
    moe.destroy()


def test_two_instances_interleaved():
    log("[parity] two instances")
    c1 = parity.case_from_workload(wl.BY_NAME["tiny"])
    c2 = random_case(8, ep=3, E=6, K=2, cap=5, n=[5, 1, 4], hidden_size=48, H=96, name="second")
    m1, m2 = parity.make_gpu(c1), parity.make_gpu(c2)
    parity.run_step(c1, moe=m1)
    parity.run_step(c2, moe=m2)
    parity.run_step(c1, moe=m1)
    m1.destroy()
    m2.destroy()
