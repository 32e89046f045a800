"""Loader for the hand-worked examples under tests/golden/.

Each JSON file holds a tiny dispatch/combine step worked out by hand from the
pages (its "source" field gives the passages and the readings used) together
with the expected receive regions and combine outputs.  No expected value in
them came from any implementation.
"""

from __future__ import annotations

import glob
import json
import os
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@dataclass
class GoldenCase:
    name: str
    params: dict
    hidden: List[np.ndarray]
    topk_ids: List[np.ndarray]
    topk_weights: Optional[List[np.ndarray]]
    scale: Optional[List[np.ndarray]]
    runtime_max_tokens_per_rank: Optional[int]
    active_rank_mask: Optional[int]
    expect: dict
    combine_dtype: str
    combine_mask: Optional[int]
    expert_output: List[np.ndarray]       # float32, or uint16 bf16 bits
    expect_combine: List[np.ndarray]
    eplb_local_stats: Optional[List[np.ndarray]] = None


def _f32(x):
    return np.array(x, dtype=np.float64).astype(np.float32) if len(x) else np.zeros((0,), np.float32)


def load(path: str) -> GoldenCase:
    with open(path) as f:
        g = json.load(f)
    p = g["params"]
    K, H, S, hid = p["top_k"], p["hidden_row_bytes"], p["scale_row_bytes"], p["hidden_size"]
    dd = g["dispatch"]
    ep = p["ep_size"]
    hidden = [np.array(dd["hidden"][s], np.uint8).reshape(-1, H) for s in range(ep)]
    ids = [np.array(dd["topk_ids"][s], np.int32).reshape(-1, K) for s in range(ep)]
    w = None if dd["topk_weights"] is None else [
        np.array(dd["topk_weights"][s], np.float32).reshape(-1, K) for s in range(ep)]
    sc = None if dd["scale"] is None else [
        np.array(dd["scale"][s], np.uint8).reshape(-1, S) for s in range(ep)]
    cb = g["combine"]
    dtype = cb["dtype"]
    if dtype == "f32":
        eo = [np.array([[float(v) for v in row] for row in cb["expert_output"][d]], np.float32)
              for d in range(ep)]
        ec = [np.array(g["expect_combine"][s], np.float32).reshape(-1, hid) for s in range(ep)]
    else:
        eo = [np.array(cb["expert_output_bits"][d], np.uint16) for d in range(ep)]
        ec = [np.array(g["expect_combine_bits"][s], np.uint16).reshape(-1, hid) for s in range(ep)]
    es = dd.get("eplb_local_stats")
    es = None if es is None else [np.array(x, np.uint8) for x in es]
    return GoldenCase(os.path.splitext(os.path.basename(path))[0], p, hidden, ids, w, sc,
                      dd["runtime_max_tokens_per_rank"], dd["active_rank_mask"], g["expect_dispatch"],
                      dtype, cb["active_rank_mask"], eo, ec, es)


def all_cases() -> List[GoldenCase]:
    return [load(p) for p in sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.json")))]
