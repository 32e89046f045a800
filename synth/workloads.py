"""Seeded synthetic inputs for MoE expert-parallel dispatch/combine.

This module only draws numbers: it holds no step of dispatch or combine, so
both the HIP path's tests and the CPU oracle can consume its output.  Every
input is generated on the CPU with ``numpy.random.default_rng(seed)`` and
handed to both sides as identical bytes.

Workloads (the five shapes the path is measured and checked on):

=====  ========  ====  ====  ======  =====  ===  ============================
index  name      ep    cap   hidden  E      K    notes
=====  ========  ====  ====  ======  =====  ===  ============================
0      tiny      4     16    128     8      2    fp32 rows, uniform routing
1      dsv3      8     128   7168    256    8    bf16 rows (DeepSeek-V3 decode)
2      fp8       16    256   7168    256    8    e4m3 bytes + fp32 block scales
3      ragged    8     512   4096    128    8    ragged n_s, Zipf(1.2), mask 0xB7
4      large     32    256   4096    128    8    bf16 rows, ~2 GiB receive regions
=====  ========  ====  ====  ======  =====  ===  ============================

Recipe, per rank s in ascending order, from one generator seeded with
``1000 + index``:

* ``topk_ids``: Gumbel-top-k over ``log p_e`` (uniform p, or ``p_e ∝
  (e+1)^-1.2`` for the Zipf workload): the K largest perturbed keys, in
  descending key order.  This draws K distinct experts without replacement
  with probability proportional to p.
* ``topk_weights``: float32 softmax along K of standard-normal logits.
* hidden rows: standard-normal float32 values, stored as float32 (tiny),
  bfloat16 with round-to-nearest-even, or e4m3 bytes quantized per 1x128
  block with ``scale = absmax / 448`` (float32 scale rows of 56 entries).
* ``values``: the float32 value each stored row represents (the bf16 value,
  or the dequantized fp8 value ``f32(q) * scale``).  Only the expert stand-in
  between dispatch and combine uses it.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

FP8_BLOCK = 128
FP8_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    ep_size: int
    max_tokens_per_rank: int
    hidden_size: int
    num_experts: int
    top_k: int
    row_format: str                 # "f32", "bf16" or "fp8"
    routing: str = "uniform"        # "uniform" or "zipf"
    zipf_s: float = 1.2
    ragged: bool = False            # n_s ~ U[0, cap] with some ranks forced empty
    empty_ranks: tuple = ()
    masked_ranks: tuple = ()        # ranks left out of active_rank_mask
    runtime_max: str = "none"       # "none" (capacity) or "max" (largest n_s)
    index: int = -1

    @property
    def hidden_row_bytes(self) -> int:
        return self.hidden_size * {"f32": 4, "bf16": 2, "fp8": 1}[self.row_format]

    @property
    def scale_row_bytes(self) -> int:
        return (self.hidden_size // FP8_BLOCK) * 4 if self.row_format == "fp8" else 0

    @property
    def combine_dtype(self) -> str:
        return "f32" if self.row_format == "f32" else "bf16"

    @property
    def combine_elem_bytes(self) -> int:
        return 4 if self.combine_dtype == "f32" else 2

    @property
    def seed(self) -> int:
        return 1000 + self.index


WORKLOADS: List[Workload] = [
    Workload("tiny", 4, 16, 128, 8, 2, "f32", index=0),
    Workload("dsv3", 8, 128, 7168, 256, 8, "bf16", index=1),
    Workload("fp8", 16, 256, 7168, 256, 8, "fp8", index=2),
    Workload("ragged", 8, 512, 4096, 128, 8, "bf16", routing="zipf", ragged=True,
             empty_ranks=(1, 5), masked_ranks=(3, 6), runtime_max="max", index=3),
    Workload("large", 32, 256, 4096, 128, 8, "bf16", index=4),
]
BY_NAME = {w.name: w for w in WORKLOADS}


@dataclass
class Inputs:
    """Per-rank inputs of one dispatch step, as host arrays."""

    workload: Workload
    local_num_tokens: List[int]
    hidden: List[np.ndarray]                  # uint8 [n_s, hidden_row_bytes]
    scale: Optional[List[np.ndarray]]         # uint8 [n_s, scale_row_bytes] or None
    topk_ids: List[np.ndarray]                # int32 [n_s, K]
    topk_weights: List[np.ndarray]            # float32 [n_s, K]
    values: List[np.ndarray]                  # float32 [n_s, hidden]
    runtime_max_tokens_per_rank: Optional[int]
    active_rank_mask: Optional[int]           # None = no mask passed
    extra: dict = field(default_factory=dict)


def expert_logp(w: Workload) -> np.ndarray:
    if w.routing == "uniform":
        return np.zeros(w.num_experts)
    return -w.zipf_s * np.log(np.arange(1, w.num_experts + 1, dtype=np.float64))


def gumbel_topk(rng: np.random.Generator, logp: np.ndarray, n: int, k: int) -> np.ndarray:
    keys = logp[None, :] + rng.gumbel(size=(n, logp.shape[0]))
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def softmax_weights(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    logits = rng.standard_normal((n, k))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def encode_rows(x: np.ndarray, fmt: str):
    """Store float32 rows in the workload's row format.  Returns
    (row bytes uint8 [n, B], scale bytes uint8 [n, S] or None, values float32)."""
    n, h = x.shape
    if fmt == "f32":
        return x.view(np.uint8).reshape(n, h * 4).copy(), None, x.copy()
    if fmt == "bf16":
        b = torch.from_numpy(x).to(torch.bfloat16)
        vals = b.to(torch.float32).numpy()
        return b.view(torch.int16).numpy().view(np.uint8).reshape(n, h * 2).copy(), None, vals
    if fmt == "fp8":
        blocks = torch.from_numpy(x).reshape(n, h // FP8_BLOCK, FP8_BLOCK)
        absmax = blocks.abs().amax(dim=2)
        scale = (absmax / FP8_MAX).to(torch.float32)
        scale = torch.where(scale > 0, scale, torch.ones_like(scale))
        q = (blocks / scale[:, :, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
        vals = (q.to(torch.float32) * scale[:, :, None]).reshape(n, h)
        qbytes = q.view(torch.uint8).reshape(n, h).numpy().copy() if n else np.zeros((0, h), np.uint8)
        sbytes = scale.contiguous().numpy().view(np.uint8).reshape(n, (h // FP8_BLOCK) * 4).copy()
        return qbytes, sbytes, vals.numpy().copy()
    raise ValueError(fmt)


def make_inputs(w: Workload, seed: Optional[int] = None, *,
                local_num_tokens: Optional[List[int]] = None) -> Inputs:
    """Draw one step's inputs for workload ``w`` (see the module docstring)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    ep, cap, K = w.ep_size, w.max_tokens_per_rank, w.top_k
    if local_num_tokens is not None:
        n = [int(v) for v in local_num_tokens]
    elif w.ragged:
        n = [int(v) for v in rng.integers(0, cap + 1, size=ep)]
        for r in w.empty_ranks:
            n[r] = 0
    else:
        n = [cap] * ep
    logp = expert_logp(w)
    hidden, scale, ids, weights, values = [], [], [], [], []
    for s in range(ep):
        ids.append(gumbel_topk(rng, logp, n[s], K))
        weights.append(softmax_weights(rng, n[s], K))
        x = rng.standard_normal((n[s], w.hidden_size), dtype=np.float32)
        hb, sb, v = encode_rows(x, w.row_format)
        hidden.append(hb)
        scale.append(sb)
        values.append(v)
    mask = None
    if w.masked_ranks:
        mask = ((1 << ep) - 1) & ~sum(1 << r for r in w.masked_ranks)
    rtpr = max(n) if w.runtime_max == "max" else None
    return Inputs(w, n, hidden, scale if w.row_format == "fp8" else None, ids, weights, values,
                  rtpr, mask)


def random_rows(rng: np.random.Generator, rows: int, hidden: int, dtype: str) -> np.ndarray:
    """Standard-normal rows in a combine dtype: float32, bfloat16 bit
    patterns (uint16) or NumPy float16, rounded to nearest even by torch."""
    x = rng.standard_normal((rows, hidden), dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return torch.from_numpy(x).to(torch.float16).numpy().copy()
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
