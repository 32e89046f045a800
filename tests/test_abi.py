"""The C ABI on the CPU: the library loads, exports exactly what
include/moe_ep.h declares with matching struct layouts, and its host-side
validation returns the documented status codes before any device work.

Nothing here launches a kernel: every dispatch below fails validation, and
create only records a (fake, never dereferenced) workspace address.
"""

from __future__ import annotations

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from combine_token_dest_amd import _lib
from synth import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ep.h")
FAKE_WS = 1 << 40            # a 256-byte aligned address that is never dereferenced


def header_functions():
    text = open(HEADER).read()
    return re.findall(r"MOE_EP_API\s+[\w\s\*]+?\b(moe_ep_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import combine_token_dest_amd.build as b
        b.build()
    return _lib.load()


def test_exports_match_header(lib):
    declared = header_functions()
    assert sorted(declared) == sorted(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared)


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c99"), ("g++", "-std=c++11")])
def test_header_stands_alone(compiler, std):
    """include/moe_ep.h compiles on its own as C and as C++, warning-free."""
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "use.c" if compiler == "gcc" else "use.cpp")
        open(src, "w").write('#include "moe_ep.h"\nint main(void) { moe_ep_params p; (void)p; return 0; }\n')
        subprocess.run([compiler, std, "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), src], check=True)


def test_struct_layouts_match_header(lib):
    """ctypes mirrors of the header structs have C's sizes and offsets."""
    structs = {
        "moe_ep_params": _lib.moe_ep_params,
        "moe_ep_dispatch_args": _lib.moe_ep_dispatch_args,
        "moe_ep_dispatch_result": _lib.moe_ep_dispatch_result,
        "moe_ep_combine_args": _lib.moe_ep_combine_args,
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "moe_ep.h"', "int main(void) {"]
    for name, cls in structs.items():
        lines.append(f'printf("{name} sizeof %zu\\n", sizeof({name}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{name} {f} %zu\\n", offsetof({name}, {f}));')
    lines.append("return 0; }")
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "layout.c")
        exe = os.path.join(tmp, "layout")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    for line in out.splitlines():
        name, field, value = line.split()
        cls = structs[name]
        got = ctypes.sizeof(cls) if field == "sizeof" else getattr(cls, field).offset
        assert got == int(value), f"{name}.{field}: ctypes {got} vs C {value}"


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: loading a library that is not there raises."""
    with pytest.raises(OSError, match="missing"):
        _lib.load(str(tmp_path / "libmoe_ep.so"))


def test_constants_match_header():
    """Every MOE_EP_* constant of the binding has the header's value, and
    the header defines no constant the binding lacks."""
    text = open(HEADER).read()
    names = sorted(set(re.findall(r"\b(MOE_EP_(?:OK|ERR_\w+|F32|BF16|F16|ORDER_\w+|MAX_RANKS|ALL_RANKS|NOALLOC_MAX_ROWS))\b",
                                  text)))
    lines = ["#include <stdio.h>", '#include "moe_ep.h"', "int main(void) {"]
    lines += [f'printf("{n} %llu\\n", (unsigned long long)(long long)({n}));' for n in names
              if n != "MOE_EP_ALL_RANKS"]
    lines += ['printf("MOE_EP_ALL_RANKS %llu\\n", (unsigned long long)MOE_EP_ALL_RANKS);', "return 0; }"]
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "consts.c")
        exe = os.path.join(tmp, "consts")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    seen = 0
    for line in out.splitlines():
        name, value = line.split()
        assert hasattr(_lib, name), f"the binding lacks {name}"
        assert getattr(_lib, name) % (1 << 64) == int(value), f"{name}: binding {getattr(_lib, name)} vs C {value}"
        seen += 1
    assert seen == len(names) and seen >= 16


def params(**kw):
    base = dict(ep_size=4, num_experts=8, top_k=2, max_tokens_per_rank=16, hidden_size=128,
                combine_max_elem_bytes=4, hidden_row_bytes=512, scale_row_bytes=0,
                invalid_expert_id=-1, enable_rank_mask=0)
    base.update(kw)
    return _lib.moe_ep_params(**base)


def status_of(fn, *args):
    try:
        fn(*args)
    except _lib.MoeEpError as e:
        return e.status
    return _lib.MOE_EP_OK


@pytest.mark.parametrize("w", wl.WORKLOADS, ids=[w.name for w in wl.WORKLOADS])
def test_workspace_bytes_cover_the_regions(lib, w):
    p = params(ep_size=w.ep_size, num_experts=w.num_experts, top_k=w.top_k,
               max_tokens_per_rank=w.max_tokens_per_rank, hidden_size=w.hidden_size,
               combine_max_elem_bytes=w.combine_elem_bytes, hidden_row_bytes=w.hidden_row_bytes,
               scale_row_bytes=w.scale_row_bytes)
    n = _lib.moe_ep_workspace_bytes(p)
    rows = w.ep_size * w.max_tokens_per_rank
    per_rank = rows * (w.hidden_row_bytes + w.scale_row_bytes + 8 * w.top_k
                       + w.hidden_size * w.combine_elem_bytes)
    assert n >= w.ep_size * per_rank + rows * (8 + 16)
    assert n <= w.ep_size * (per_rank + 6 * 4096) + rows * (8 + 16) + 3 * 4096
    if w.name == "large":
        assert n > 2 ** 32           # 64-bit offsets are exercised


@pytest.mark.parametrize("bad", [
    dict(ep_size=0), dict(ep_size=65), dict(num_experts=6, ep_size=4), dict(num_experts=2, ep_size=4),
    dict(top_k=0), dict(max_tokens_per_rank=-1), dict(hidden_size=0), dict(combine_max_elem_bytes=3),
    dict(hidden_row_bytes=0), dict(scale_row_bytes=-4), dict(dispatch_order=3), dict(dispatch_order=-1),
])
def test_bad_params_rejected(lib, bad):
    assert status_of(_lib.moe_ep_workspace_bytes, params(**bad)) == _lib.MOE_EP_ERR_INVALID_ARG
    assert status_of(_lib.moe_ep_create, params(**bad), FAKE_WS, 1 << 30) == _lib.MOE_EP_ERR_INVALID_ARG


def test_create_checks_workspace(lib):
    p = params()
    n = _lib.moe_ep_workspace_bytes(p)
    assert status_of(_lib.moe_ep_create, p, 0, n) == _lib.MOE_EP_ERR_INVALID_ARG
    assert status_of(_lib.moe_ep_create, p, FAKE_WS + 16, n) == _lib.MOE_EP_ERR_ALIGN
    assert status_of(_lib.moe_ep_create, p, FAKE_WS, n - 1) == _lib.MOE_EP_ERR_INVALID_ARG
    h = _lib.moe_ep_create(p, FAKE_WS, n)
    assert h
    _lib.moe_ep_destroy(h)
    _lib.moe_ep_destroy(None)


def dispatch_args(n, *, ids=True, hidden=True, weights=None, rtpr=-1, mask=_lib.MOE_EP_ALL_RANKS):
    a = _lib.moe_ep_dispatch_args()
    for s, ns in enumerate(n):
        a.local_num_tokens[s] = ns
        if ns:
            a.hidden[s] = FAKE_WS + 4096 * (s + 1) if hidden else None
            a.topk_ids[s] = FAKE_WS + 4096 * (s + 100) if ids else None
    if weights is not None:
        a.weights_present = weights
        for s, ns in enumerate(n):
            if (weights >> s) & 1 and ns:
                a.topk_weights[s] = FAKE_WS + 4096 * (s + 200)
    a.runtime_max_tokens_per_rank = rtpr
    a.active_rank_mask = mask
    return a


@pytest.mark.parametrize("entry", ["moe_ep_dispatch", "moe_ep_dispatch_noalloc"])
def test_dispatch_validation(lib, entry):
    """Both dispatch entry points validate alike, before any device work."""
    p = params()
    h = _lib.moe_ep_create(p, FAKE_WS, _lib.moe_ep_workspace_bytes(p))
    D = getattr(_lib, entry)
    cases = [
        (dispatch_args([17, 0, 0, 0]), _lib.MOE_EP_ERR_CAPACITY),            # n > capacity
        (dispatch_args([5, 0, 3, 0], rtpr=4), _lib.MOE_EP_ERR_CAPACITY),     # rtpr < largest n
        (dispatch_args([5, 0, 3, 0], rtpr=17), _lib.MOE_EP_ERR_CAPACITY),    # rtpr > capacity
        (dispatch_args([5, 0, 3, 0], mask=0b0011), _lib.MOE_EP_ERR_MASK),    # mask needs enable
        (dispatch_args([5, 0, 3, 0], weights=0b0111), _lib.MOE_EP_ERR_INVALID_ARG),  # some ranks only
        (dispatch_args([5, 0, 3, 0], hidden=False), _lib.MOE_EP_ERR_INVALID_ARG),
        (dispatch_args([5, 0, 3, 0], ids=False), _lib.MOE_EP_ERR_INVALID_ARG),
        (dispatch_args([-1, 0, 3, 0]), _lib.MOE_EP_ERR_INVALID_ARG),
    ]
    for a, want in cases:
        assert status_of(D, h, a, 4, 0) == want, _lib.moe_ep_last_error()
    a = dispatch_args([5, 0, 3, 0])
    a.topk_ids[0] = FAKE_WS + 2                                               # misaligned int32
    assert status_of(D, h, a, 4, 0) == _lib.MOE_EP_ERR_ALIGN
    a = dispatch_args([5, 0, 3, 0])
    a.scales_present = 0b1111                                                 # no scale rows configured
    assert status_of(D, h, a, 4, 0) == _lib.MOE_EP_ERR_INVALID_ARG
    # nothing was dispatched, so combine and the combine buffer are still out of order
    ca = _lib.moe_ep_combine_args()
    ca.active_rank_mask = _lib.MOE_EP_ALL_RANKS
    assert status_of(_lib.moe_ep_combine, h, ca, 0) == _lib.MOE_EP_ERR_STATE
    assert status_of(_lib.moe_ep_get_combine_input_buffer, h, 0, _lib.MOE_EP_F32) == _lib.MOE_EP_ERR_STATE
    _lib.moe_ep_destroy(h)


def test_noalloc_dispatch_rejects_steps_past_the_fixed_area(lib):
    """moe_ep_dispatch_noalloc keeps its records in a fixed area of
    MOE_EP_NOALLOC_MAX_ROWS receive rows: a larger step is refused on the
    host with ERR_CAPACITY (no device work, the handle stays idle)."""
    p = params(ep_size=64, num_experts=64, top_k=1, max_tokens_per_rank=1025, hidden_size=4,
               hidden_row_bytes=16)
    h = _lib.moe_ep_create(p, FAKE_WS, _lib.moe_ep_workspace_bytes(p))
    a = _lib.moe_ep_dispatch_args()
    a.runtime_max_tokens_per_rank = -1              # capacity: 64 x 1025 rows
    a.active_rank_mask = _lib.MOE_EP_ALL_RANKS
    assert status_of(_lib.moe_ep_dispatch_noalloc, h, a, 64, 0) == _lib.MOE_EP_ERR_CAPACITY
    assert "fixed record area" in _lib.moe_ep_last_error()
    a.runtime_max_tokens_per_rank = 1025
    assert status_of(_lib.moe_ep_dispatch_noalloc, h, a, 64, 0) == _lib.MOE_EP_ERR_CAPACITY
    ca = _lib.moe_ep_combine_args()
    ca.active_rank_mask = _lib.MOE_EP_ALL_RANKS
    assert status_of(_lib.moe_ep_combine, h, ca, 0) == _lib.MOE_EP_ERR_STATE
    _lib.moe_ep_destroy(h)
    assert 64 * 1024 == _lib.MOE_EP_NOALLOC_MAX_ROWS


def test_eplb_validation(lib):
    p = params()
    h = _lib.moe_ep_create(p, FAKE_WS, _lib.moe_ep_workspace_bytes(p))
    a = dispatch_args([5, 0, 3, 0])
    a.eplb_present = 0b1111                                                   # no statistics configured
    for s in range(4):
        a.eplb_local_stats[s] = FAKE_WS + 64 * s
    assert status_of(_lib.moe_ep_dispatch, h, a, 4, 0) == _lib.MOE_EP_ERR_INVALID_ARG
    _lib.moe_ep_destroy(h)
    p = params(eplb_stats_bytes=1024)
    h = _lib.moe_ep_create(p, FAKE_WS, _lib.moe_ep_workspace_bytes(p))
    a.eplb_present = 0b0111                                                   # some ranks only
    assert status_of(_lib.moe_ep_dispatch, h, a, 4, 0) == _lib.MOE_EP_ERR_INVALID_ARG
    a.eplb_present = 0b1111
    a.eplb_local_stats[2] = None                                              # NULL row
    assert status_of(_lib.moe_ep_dispatch, h, a, 4, 0) == _lib.MOE_EP_ERR_INVALID_ARG
    _lib.moe_ep_destroy(h)
    assert status_of(_lib.moe_ep_workspace_bytes, params(eplb_stats_bytes=-1)) == _lib.MOE_EP_ERR_INVALID_ARG
    assert _lib.moe_ep_workspace_bytes(params(eplb_stats_bytes=1024)) >= \
        _lib.moe_ep_workspace_bytes(params()) + 4 * 4 * 1024


def test_checkpoint_needs_a_library_mapped_workspace(lib):
    p = params()
    h = _lib.moe_ep_create(p, FAKE_WS, _lib.moe_ep_workspace_bytes(p))
    assert status_of(_lib.moe_ep_checkpoint_prepare, h) == _lib.MOE_EP_ERR_UNSUPPORTED
    assert status_of(_lib.moe_ep_checkpoint_restore, h) == _lib.MOE_EP_ERR_UNSUPPORTED
    ptr, n = _lib.moe_ep_workspace(h)
    assert ptr == FAKE_WS and n == _lib.moe_ep_workspace_bytes(p)
    _lib.moe_ep_destroy(h)
    assert status_of(_lib.moe_ep_checkpoint_prepare, None) == _lib.MOE_EP_ERR_INVALID_ARG
    assert status_of(_lib.moe_ep_create_vmm, params(ep_size=0)) == _lib.MOE_EP_ERR_INVALID_ARG


def test_mask_validation(lib):
    p = params(enable_rank_mask=1)
    h = _lib.moe_ep_create(p, FAKE_WS, _lib.moe_ep_workspace_bytes(p))
    a = dispatch_args([5, 0, 3, 0], mask=0b10000)                             # bit >= ep_size
    assert status_of(_lib.moe_ep_dispatch, h, a, 4, 0) == _lib.MOE_EP_ERR_MASK
    _lib.moe_ep_destroy(h)


def test_active_rank_mask(lib):
    assert _lib.moe_ep_active_rank_mask([0, 2, 5]) == 0b100101
    assert _lib.moe_ep_active_rank_mask([]) == 0
    assert _lib.moe_ep_active_rank_mask([63, 0]) == (1 << 63) | 1
    assert status_of(_lib.moe_ep_active_rank_mask, [64]) == _lib.MOE_EP_ERR_MASK
    assert status_of(_lib.moe_ep_active_rank_mask, [-1]) == _lib.MOE_EP_ERR_MASK


def test_status_strings(lib):
    for code, name in [(0, "MOE_EP_OK"), (-1, "MOE_EP_ERR_INVALID_ARG"), (-2, "MOE_EP_ERR_STATE"),
                       (-3, "MOE_EP_ERR_CAPACITY"), (-4, "MOE_EP_ERR_MASK"), (-5, "MOE_EP_ERR_ALIGN"),
                       (-6, "MOE_EP_ERR_HIP"), (-7, "MOE_EP_ERR_UNSUPPORTED")]:
        assert _lib.moe_ep_status_string(code) == name


def test_platform_query_does_not_crash(lib):
    assert _lib.moe_ep_is_platform_supported() in (True, False)


def test_destination_order_grid_limit(lib):
    """An explicit destination-major request whose grid would pass 2^31 - 1
    workgroups fails before anything is enqueued (64 ranks x 2^19 tokens of
    16-byte rows: 2^31 items), and leaves the handle idle."""
    p = params(ep_size=64, num_experts=64, top_k=1, max_tokens_per_rank=1 << 19, hidden_size=8,
               combine_max_elem_bytes=2, hidden_row_bytes=16, dispatch_order=_lib.MOE_EP_ORDER_DESTINATION)
    h = _lib.moe_ep_create(p, FAKE_WS, _lib.moe_ep_workspace_bytes(p))
    a = dispatch_args([0] * 64, rtpr=1 << 19)
    assert status_of(_lib.moe_ep_dispatch, h, a, 64, 0) == _lib.MOE_EP_ERR_INVALID_ARG
    assert "grid" in _lib.moe_ep_last_error()
    ca = _lib.moe_ep_combine_args()
    ca.active_rank_mask = _lib.MOE_EP_ALL_RANKS
    assert status_of(_lib.moe_ep_combine, h, ca, 0) == _lib.MOE_EP_ERR_STATE
    _lib.moe_ep_destroy(h)


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="valid steps would launch kernels on the fake workspace")
def test_validation_agrees_with_the_oracle(lib):
    """The library's host validation and the oracle's rules, written
    separately from the same passages, accept and refuse the same steps:
    random small groups with counts past the capacity, runtime bounds on
    either side, masks with and without enable_rank_mask and with bits past
    ep_size, and weights / scales passed by all, none or some ranks.  A step
    both accept gets as far as the kernel launch, which fails on a host with
    no GPU (MOE_EP_ERR_HIP) before anything runs; one with no receive rows
    launches nothing and succeeds."""
    import numpy as np
    from hypothesis import given, settings, strategies as st, HealthCheck
    import oracle

    kinds = {"capacity": _lib.MOE_EP_ERR_CAPACITY, "mask": _lib.MOE_EP_ERR_MASK,
             "invalid_arg": _lib.MOE_EP_ERR_INVALID_ARG}

    @st.composite
    def steps(draw):
        ep = draw(st.integers(1, 6))
        epr = draw(st.integers(1, 3))
        K = draw(st.integers(1, 4))
        cap = draw(st.integers(0, 5))
        n = [draw(st.integers(0, cap + 1)) for _ in range(ep)]
        rtpr = draw(st.one_of(st.none(), st.integers(0, cap + 1)))
        enable = draw(st.booleans())
        mask = draw(st.one_of(st.none(), st.integers(0, (1 << (ep + 1)) - 1)))
        S = draw(st.sampled_from([0, 8]))
        wsel = draw(st.sampled_from(["all", "none", "some"]))
        ssel = draw(st.sampled_from(["all", "none", "some"]))
        return ep, epr, K, cap, n, rtpr, enable, mask, S, wsel, ssel

    def present(sel, ep, s):
        return sel == "all" or (sel == "some" and s != ep - 1)

    @settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.too_slow])
    @given(steps())
    def check(step):
        ep, epr, K, cap, n, rtpr, enable, mask, S, wsel, ssel = step
        if wsel == "some" and ep == 1:
            wsel = "none"
        if ssel == "some" and ep == 1:
            ssel = "none"
        H = 8
        # the oracle
        P = oracle.Params(ep, ep * epr, K, cap, 2, H, S, -1, enable)
        hid = [np.zeros((k, H), np.uint8) for k in n]
        ids = [np.zeros((k, K), np.int32) for k in n]
        wts = [np.zeros((k, K), np.float32) if present(wsel, ep, s) else None for s, k in enumerate(n)]
        scl = [np.zeros((k, S), np.uint8) if present(ssel, ep, s) else None for s, k in enumerate(n)]
        try:
            oracle.OracleMoEEp(P).dispatch(hid, ids, wts if wsel != "none" else None,
                                           hidden_states_scale=scl if ssel != "none" else None,
                                           runtime_max_tokens_per_rank=rtpr, active_rank_mask=mask)
            # a step of no receive rows launches nothing and succeeds
            want = _lib.MOE_EP_OK if (cap if rtpr is None else rtpr) == 0 else _lib.MOE_EP_ERR_HIP
        except oracle.OracleError as e:
            want = kinds[e.kind]
        # the library
        p = params(ep_size=ep, num_experts=ep * epr, top_k=K, max_tokens_per_rank=cap, hidden_size=2,
                   hidden_row_bytes=H, scale_row_bytes=S, enable_rank_mask=1 if enable else 0)
        h = _lib.moe_ep_create(p, FAKE_WS, _lib.moe_ep_workspace_bytes(p))
        try:
            a = _lib.moe_ep_dispatch_args()
            for s, k in enumerate(n):
                a.local_num_tokens[s] = k
                if k:
                    a.hidden[s] = FAKE_WS + 4096 * (s + 1)
                    a.topk_ids[s] = FAKE_WS + 4096 * (s + 100)
                if present(wsel, ep, s) and wsel != "none":
                    a.weights_present |= 1 << s
                    if k:
                        a.topk_weights[s] = FAKE_WS + 4096 * (s + 200)
                if present(ssel, ep, s) and ssel != "none":
                    a.scales_present |= 1 << s
                    if k:
                        a.hidden_scale[s] = FAKE_WS + 4096 * (s + 300)
            a.runtime_max_tokens_per_rank = -1 if rtpr is None else rtpr
            a.active_rank_mask = _lib.MOE_EP_ALL_RANKS if mask is None else mask
            got = status_of(_lib.moe_ep_dispatch, h, a, ep, 0)
        finally:
            _lib.moe_ep_destroy(h)
        assert got == want, (step, _lib.moe_ep_last_error())

    check()
