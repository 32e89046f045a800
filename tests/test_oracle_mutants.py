"""The oracle's pins catch plausible mistakes.

Each mutant below plants one mistake in a copy of oracle/ (a wrong owner
rule, a transposed placement, a dropped zero fill, a reversed summation
order, a wrong rounding, ...) and runs tests/test_oracle_pins.py against
that copy in a subprocess; every mutant must make the pins fail, and the
unmodified copy must pass.  CPU only; nothing here touches the GPU path.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, file under oracle/, text to replace, replacement)
MUTANTS = [
    ("owner by modulo", "moe_ep.py",
     "return expert_id // (params.num_experts // params.ep_size)", "return expert_id % params.ep_size"),
    ("placement transposed", "moe_ep.py",
     "                    r = s * tpr + t\n                    if (dest_masks",
     "                    r = t * ep + s\n                    if (dest_masks"),
    ("invalid weights not zeroed", "moe_ep.py",
     "                        if has_w:\n                            out_w[r] = 0.0",
     "                        if has_w:\n                            out_w[r] = 1.0"),
    ("combine in descending rank order", "moe_ep.py",
     "for d in range(ep):                      # ascending rank order", "for d in reversed(range(ep)):"),
    ("rank mask ignored in routing", "moe_ep.py",
     "return m & active & ((1 << params.ep_size) - 1)", "return m & ((1 << params.ep_size) - 1)"),
    ("ids not copied verbatim", "moe_ep.py", "out_ids[r] = ids_s[t]", "out_ids[r] = np.abs(ids_s[t])"),
    ("padding rows routed", "moe_ep.py",
     "destination_mask(p, ids_s[t], active) if t < n[s] else 0",
     "destination_mask(p, ids_s[min(t, n[s] - 1)], active) if n[s] else 0"),
    ("sum starts at -0.0", "moe_ep.py", "acc = np.zeros(hid, np.float32)", "acc = np.full(hid, -0.0, np.float32)"),
    ("sum kept in float64", "moe_ep.py",
     "acc = (acc + term).astype(np.float32)", "acc = acc.astype(np.float64) + term"),
    ("combine mask not checked", "moe_ep.py",
     "        if mask != rec.active_rank_mask:\n", "        if False:\n"),
    ("None bound means the largest count", "moe_ep.py",
     "tpr = cap if runtime_max_tokens_per_rank is None else int(runtime_max_tokens_per_rank)",
     "tpr = largest if runtime_max_tokens_per_rank is None else int(runtime_max_tokens_per_rank)"),
    ("statistics rows reversed", "moe_ep.py",
     "gathered[s] = np.asarray(eplb_local_stats[s], np.uint8)",
     "gathered[s] = np.asarray(eplb_local_stats[ep - 1 - s], np.uint8)"),
    ("weights all-or-none not checked", "moe_ep.py",
     "        if has_w and any(w is None for w in topk_weights):\n", "        if False:\n"),
    ("scale rows not copied", "moe_ep.py", "                            out_scale[r] = scl_s[t]",
     "                            out_scale[r] = 0"),
    ("hidden row off by one", "moe_ep.py", "out_hidden[r] = hid_s[t]", "out_hidden[r] = hid_s[max(t - 1, 0)]"),
    ("invalid id fixed at -1", "moe_ep.py",
     "out_ids[r] = p.invalid_expert_id", "out_ids[r] = -1"),
    ("combine reads the transposed row", "moe_ep.py",
     "                r = s * tpr + t\n                acc = np.zeros",
     "                r = t * ep + s\n                acc = np.zeros"),
    ("combine skips the last rank", "moe_ep.py",
     "for d in range(ep):                      # ascending rank order", "for d in range(ep - 1):"),
    ("f32 combine rounded through bf16", "moe_ep.py",
     "if dtype == \"f32\":\n                    out[t] = acc\n",
     "if dtype == \"f32\":\n                    out[t] = bf16_bits_to_f32(f32_to_bf16_bits_rne(acc))\n"),
    ("f16 combine truncated", "moe_ep.py",
     "out[t] = acc.astype(np.float16)",
     "out[t] = (acc.view(np.uint32) & np.uint32(0xFFFFE000)).view(np.float32).astype(np.float16)"),
    ("f16 combine rounded through bf16", "moe_ep.py",
     "out[t] = acc.astype(np.float16)",
     "out[t] = bf16_bits_to_f32(f32_to_bf16_bits_rne(acc)).astype(np.float16)"),
    ("negative ids routed to rank 0", "moe_ep.py",
     "    if 0 <= expert_id < params.num_experts:\n",
     "    if expert_id < params.num_experts:\n        expert_id = max(expert_id, 0)\n"),
    ("call state kept after combine", "moe_ep.py",
     "            outputs.append(out)\n        self.record = None\n",
     "            outputs.append(out)\n"),
    ("statistics gathered to rank 0 only", "moe_ep.py",
     "None if gathered is None else gathered.copy()",
     "None if gathered is None else (gathered.copy() if d == 0 else np.zeros_like(gathered))"),
    ("weights of routed rows zeroed", "moe_ep.py",
     "                            out_w[r] = w_s[t]", "                            out_w[r] = 0.0"),
    ("65 ranks accepted", "moe_ep.py",
     "if not (1 <= self.ep_size <= MAX_RANKS):", "if not (1 <= self.ep_size <= MAX_RANKS + 1):"),
    ("0 ranks accepted", "moe_ep.py",
     "if not (1 <= self.ep_size <= MAX_RANKS):", "if not (0 <= self.ep_size <= MAX_RANKS):"),
    ("expert count not a multiple of ep_size accepted", "moe_ep.py",
     "if self.num_experts < self.ep_size or self.num_experts % self.ep_size:",
     "if self.num_experts < self.ep_size:"),
    ("top_k 0 accepted", "moe_ep.py", "if self.top_k < 1 or", "if self.top_k < 0 or"),
    ("negative capacity accepted", "moe_ep.py",
     "self.max_tokens_per_rank < 0 or", "self.max_tokens_per_rank < -1 or"),
    ("scales all-or-none not checked", "moe_ep.py",
     "        if has_s and any(x is None for x in hidden_states_scale):\n", "        if False:\n"),
    ("scales accepted without scale_row_bytes", "moe_ep.py",
     "        if has_s and p.scale_row_bytes == 0:\n", "        if False:\n"),
    ("unknown combine dtype accepted", "moe_ep.py",
     "if dtype not in (\"f32\", \"bf16\", \"f16\"):", "if dtype not in (\"f32\", \"bf16\", \"f16\", \"f64\"):"),
    ("bf16 widened by an 8-bit shift", "numerics.py",
     "<< np.uint32(16)).view(np.float32)", "<< np.uint32(8)).view(np.float32)"),
    ("bf16 ties rounded away from zero", "numerics.py",
     "rounded = (u + (np.uint32(0x7FFF) + lsb))", "rounded = (u + np.uint32(0x8000))"),
    ("bf16 by truncation", "numerics.py",
     "def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:\n",
     "def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:\n"
     "    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)\n\n\n"
     "def _unused_rne(x: np.ndarray) -> np.ndarray:\n"),
]


def _run_pins(mutant):
    """Pins against a copy of oracle/ with `mutant` applied (None: no change);
    returns True when they pass."""
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        for part in ("oracle", "tests", "synth"):
            shutil.copytree(os.path.join(ROOT, part), os.path.join(tmp, part),
                            ignore=shutil.ignore_patterns("__pycache__"))
        shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp)
        if mutant is not None:
            _, fname, old, new = mutant
            path = os.path.join(tmp, "oracle", fname)
            src = open(path).read()
            assert src.count(old) >= 1, f"mutant text not found: {old!r}"
            open(path, "w").write(src.replace(old, new, 1))
        env = dict(os.environ, PYTHONPATH=tmp, PYTHONDONTWRITEBYTECODE="1")
        p = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q",
                            "-p", "no:cacheprovider", "-m", "not gpu"],
                           cwd=tmp, env=env, capture_output=True, text=True, timeout=900)
        return p.returncode == 0
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_every_planted_mistake_fails_a_pin():
    jobs = [None] + MUTANTS
    workers = max(1, min(8, (os.cpu_count() or 2) // 2))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        passed = list(pool.map(_run_pins, jobs))
    assert passed[0], "the unmodified oracle copy must pass its pins"
    survivors = [m[0] for m, ok in zip(MUTANTS, passed[1:]) if ok]
    assert not survivors, f"mistakes the pins do not catch: {survivors}"
