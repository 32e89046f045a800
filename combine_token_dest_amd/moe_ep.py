"""MoEEp: the flashinfer.moe_ep API shape over the gfx950 library, one
process holding all ep_size ranks of a group.

Per-rank arguments of the pages' API become lists indexed by rank.  torch is
used for device memory (the workspace, output tensors) and for the current
stream only; every step of dispatch and combine runs in libmoe_ep.so.

Sources: flashinfer.moe_ep.MoEEpCommunication (class description,
is_platform_supported(), dispatch(), combine(), get_combine_input_buffer(),
destroy()); flashinfer.moe_ep.NVLinkOneSidedAlltoAll (active_rank_mask(), the
mask notes of dispatch() and combine()).
"""

from __future__ import annotations

from dataclasses import dataclass
from types import SimpleNamespace
from typing import List, Optional, Sequence

import torch

from . import _lib
from ._lib import MOE_EP_ALL_RANKS, MOE_EP_BF16, MOE_EP_F16, MOE_EP_F32

_COMBINE_DTYPES = {torch.float32: MOE_EP_F32, torch.bfloat16: MOE_EP_BF16, torch.float16: MOE_EP_F16}


@dataclass
class DispatchResult:
    """What one destination rank received (views into the workspace, valid
    until the next dispatch)."""

    hidden: torch.Tensor                    # [ep*tpr, hidden_row_bytes / itemsize] of the hidden dtype
    hidden_scale: Optional[torch.Tensor]    # [ep*tpr, scale_row_bytes / itemsize] or None
    topk_ids: torch.Tensor                  # int32 [ep*tpr, top_k]
    topk_weights: Optional[torch.Tensor]    # float32 [ep*tpr, top_k] or None
    tokens_per_rank: int
    eplb_global_stats: Optional[torch.Tensor] = None   # [ep, stats elements]: every rank's stats


def _mask_value(mask) -> int:
    if mask is None:
        return MOE_EP_ALL_RANKS
    if isinstance(mask, torch.Tensor):
        if mask.device.type != "cpu" or mask.numel() != 1:
            raise ValueError("active_rank_mask must be a one-element CPU tensor")
        return int(mask.item()) & MOE_EP_ALL_RANKS
    return int(mask) & MOE_EP_ALL_RANKS


class _DeviceBytes:
    """A device byte range exposed through __cuda_array_interface__, so torch
    can view memory the library mapped itself (no copy, no ownership)."""

    def __init__(self, ptr: int, nbytes: int):
        self.__cuda_array_interface__ = {"shape": (nbytes,), "typestr": "|u1", "data": (ptr, False),
                                         "strides": None, "version": 3}


def _dev_ptr(t: torch.Tensor, dev_index: int, what: str, rank: Optional[int] = None) -> int:
    """Address of a contiguous tensor on GPU ``dev_index``; the argument's
    name (``what``, with ``[rank]``) is only formatted for an error."""
    # get_device() is -1 for CPU tensors, so it is the whole device check
    if t.get_device() != dev_index:
        name = what if rank is None else f"{what}[{rank}]"
        raise ValueError(f"{name} is on {t.device}, expected cuda:{dev_index}")
    if not t.is_contiguous():
        name = what if rank is None else f"{what}[{rank}]"
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


# Copy order of the dispatch kernel (both give identical results): "source"
# walks the source rows once and writes each to all its destinations;
# "destination" writes each destination's rows as one sweep and re-reads the
# source rows from L2; "auto" lets the library choose from the shape.
_ORDERS = {"auto": _lib.MOE_EP_ORDER_AUTO, "source": _lib.MOE_EP_ORDER_SOURCE_ROW,
           "destination": _lib.MOE_EP_ORDER_DESTINATION}
_ORDER_NAMES = {v: k for k, v in _ORDERS.items()}


class MoEEp:
    """One EP group of ``ep_size`` logical ranks on one GPU."""

    def __init__(self, ep_size: int, num_experts: int, top_k: int, max_tokens_per_rank: int,
                 hidden_size: int, *, hidden_row_bytes: Optional[int] = None, scale_row_bytes: int = 0,
                 combine_max_elem_bytes: int = 2, invalid_expert_id: int = -1,
                 enable_rank_mask: bool = False, eplb_stats_bytes: int = 0, checkpointable: bool = False,
                 dispatch_order: str = "auto", device=None):
        dev = torch.device("cuda") if device is None else torch.device(device)
        if dev.type != "cuda":
            raise ValueError(f"MoEEp needs a GPU device, got {dev}")
        self.device = dev if dev.index is not None else torch.device("cuda", torch.cuda.current_device())
        self.params = _lib.moe_ep_params(
            ep_size=ep_size, num_experts=num_experts, top_k=top_k,
            max_tokens_per_rank=max_tokens_per_rank, hidden_size=hidden_size,
            combine_max_elem_bytes=combine_max_elem_bytes,
            hidden_row_bytes=hidden_row_bytes if hidden_row_bytes is not None else hidden_size * 2,
            scale_row_bytes=scale_row_bytes, invalid_expert_id=invalid_expert_id,
            enable_rank_mask=1 if enable_rank_mask else 0, eplb_stats_bytes=eplb_stats_bytes,
            dispatch_order=_ORDERS[dispatch_order] if isinstance(dispatch_order, str) else int(dispatch_order))
        # the sizes as plain ints (a ctypes field read costs more than an attribute)
        self._p = SimpleNamespace(**{f: getattr(self.params, f) for f, _ in _lib.moe_ep_params._fields_})
        self._dev_index = self.device.index
        self.checkpointable = checkpointable
        if checkpointable:
            # The library maps the workspace itself (HIP virtual memory), so
            # its physical memory can be released and re-backed at the same
            # addresses around a process checkpoint.
            with torch.cuda.device(self.device):
                self._handle = _lib.moe_ep_create_vmm(self.params)
            ptr, nbytes = _lib.moe_ep_workspace(self._handle)
            self.workspace = torch.as_tensor(_DeviceBytes(ptr, nbytes), device=self.device)
        else:
            nbytes = _lib.moe_ep_workspace_bytes(self.params)
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self._handle = _lib.moe_ep_create(self.params, self.workspace.data_ptr(), nbytes)
        self._ws_base = self.workspace.data_ptr()
        self._views = {}
        self.last_dispatch_order = None
        self._tpr = None
        self._n = None
        self._hidden_dtype = None
        self._scale_dtype = None
        self._buffer_dtype = None      # dtype of the last get_combine_input_buffer() of this round

    # -- pages' API --------------------------------------------------------
    @classmethod
    def is_platform_supported(cls) -> bool:
        """Whether the current device is a gfx950 GPU; no collective work."""
        return _lib.moe_ep_is_platform_supported()

    @staticmethod
    def active_rank_mask(active_ranks: Sequence[int]) -> torch.Tensor:
        """CPU uint64 bitmask of the active ranks."""
        return torch.tensor(_lib.moe_ep_active_rank_mask(list(active_ranks)), dtype=torch.uint64)

    @property
    def ep_size(self) -> int:
        return self.params.ep_size

    def _view(self, ptr: int, rows: int, row_bytes: int, dtype: torch.dtype) -> torch.Tensor:
        # Views of the workspace, kept per (address, shape, dtype): the
        # layout is fixed for the handle, and building torch views cost most
        # of a decode-size round's host time.
        key = (ptr, rows, row_bytes, dtype)
        v = self._views.get(key)
        if v is None:
            off = ptr - self._ws_base
            v = self.workspace[off:off + rows * row_bytes].view(dtype).view(rows, row_bytes // dtype.itemsize)
            if len(self._views) > 4096:
                self._views.clear()
            self._views[key] = v
        return v

    def dispatch(self, hidden_states: Sequence[torch.Tensor], topk_ids: Sequence[torch.Tensor],
                 topk_weights: Optional[Sequence[Optional[torch.Tensor]]] = None, *,
                 hidden_states_scale: Optional[Sequence[Optional[torch.Tensor]]] = None,
                 runtime_max_tokens_per_rank: Optional[int] = None,
                 eplb_local_stats=None, active_rank_mask=None,
                 local_num_tokens_device: Optional[torch.Tensor] = None,
                 noalloc: bool = False) -> List[DispatchResult]:
        """Send every token to the ranks owning its experts; see
        include/moe_ep.h, moe_ep_dispatch.

        ``local_num_tokens_device`` (optional int32 ``[ep_size]`` on the GPU)
        makes the kernels read the token counts when they run, so a captured
        graph can replay steps with other counts.  Every per-rank buffer must
        then hold ``tokens_per_rank`` rows (the runtime bound, else the
        capacity), and so do the combine outputs.

        ``noalloc=True`` calls moe_ep_dispatch_noalloc: the same dispatch,
        with the records combine reads kept in the library's fixed device
        array (steps of at most MOE_EP_NOALLOC_MAX_ROWS receive rows)."""
        if self._handle is None:
            raise RuntimeError("MoEEp has been destroyed")
        p = self._p
        di = self._dev_index
        ep = p.ep_size
        if len(hidden_states) != ep or len(topk_ids) != ep:
            raise ValueError(f"expected {ep} per-rank hidden_states and topk_ids")
        a = _lib.moe_ep_dispatch_args()
        # the struct's array fields, fetched once (each field access builds a new proxy)
        a_n, a_hidden, a_ids, a_w, a_scale = (a.local_num_tokens, a.hidden, a.topk_ids, a.topk_weights,
                                             a.hidden_scale)
        wp = sp = 0
        n = []
        keep = []              # int32 copies of int64 ids, alive until the call returns
        for s in range(ep):
            h, ids = hidden_states[s], topk_ids[s]
            if ids.dtype == torch.int64:
                # The library takes int32 ids; expert ids must fit in int32.
                ids = ids.to(torch.int32)
                keep.append(ids)
            if ids.dtype != torch.int32:
                raise TypeError("topk_ids must be int32 (or int64, converted)")
            if ids.dim() != 2 or ids.shape[1] != p.top_k:
                raise ValueError(f"rank {s}: topk_ids must be [n, {p.top_k}]")
            ns = ids.shape[0]
            if h.shape[0] != ns or h.numel() * h.element_size() != ns * p.hidden_row_bytes:
                raise ValueError(f"rank {s}: hidden_states must be {ns} rows of {p.hidden_row_bytes} bytes")
            n.append(ns)
            a_n[s] = ns
            a_hidden[s] = _dev_ptr(h, di, "hidden_states", s) if ns else None
            a_ids[s] = _dev_ptr(ids, di, "topk_ids", s) if ns else None
            if topk_weights is not None and topk_weights[s] is not None:
                w = topk_weights[s]
                if w.dtype != torch.float32 or tuple(w.shape) != (ns, p.top_k):
                    raise ValueError(f"rank {s}: topk_weights must be float32 [{ns}, {p.top_k}]")
                wp |= 1 << s
                a_w[s] = _dev_ptr(w, di, "topk_weights", s) if ns else None
            if hidden_states_scale is not None and hidden_states_scale[s] is not None:
                sc = hidden_states_scale[s]
                if sc.shape[0] != ns or sc.numel() * sc.element_size() != ns * p.scale_row_bytes:
                    raise ValueError(f"rank {s}: hidden_states_scale must be {ns} rows of "
                                     f"{p.scale_row_bytes} bytes")
                sp |= 1 << s
                a_scale[s] = _dev_ptr(sc, di, "hidden_states_scale", s) if ns else None
        ep_present = 0
        if eplb_local_stats is not None:
            if len(eplb_local_stats) != ep:
                raise ValueError(f"expected {ep} per-rank eplb_local_stats")
            for s in range(ep):
                st = eplb_local_stats[s]
                if st is None:
                    continue
                if st.numel() * st.element_size() != p.eplb_stats_bytes:
                    raise ValueError(f"rank {s}: eplb_local_stats must hold {p.eplb_stats_bytes} bytes")
                ep_present |= 1 << s
                a.eplb_local_stats[s] = _dev_ptr(st, di, "eplb_local_stats", s)
        a.eplb_present = ep_present
        a.weights_present = wp
        a.scales_present = sp
        if local_num_tokens_device is not None:
            t = local_num_tokens_device
            if t.dtype != torch.int32 or t.numel() != ep:
                raise ValueError(f"local_num_tokens_device must be int32 [{ep}]")
            bound = p.max_tokens_per_rank if runtime_max_tokens_per_rank is None else int(runtime_max_tokens_per_rank)
            if min(n) < bound:
                raise ValueError(f"with device token counts every rank's buffers must hold {bound} rows")
            a.local_num_tokens_device = _dev_ptr(t, di, "local_num_tokens_device")
            n = [bound] * ep
        a.runtime_max_tokens_per_rank = -1 if runtime_max_tokens_per_rank is None \
            else int(runtime_max_tokens_per_rank)
        a.active_rank_mask = _mask_value(active_rank_mask)
        stream = torch.cuda.current_stream(self.device).cuda_stream
        entry = _lib.moe_ep_dispatch_noalloc if noalloc else _lib.moe_ep_dispatch
        res = entry(self._handle, a, ep, stream)
        self._tpr = res[0].tokens_per_rank if ep else 0
        self._buffer_dtype = None
        # the copy order the library chose for this step ("source" / "destination")
        self.last_dispatch_order = _ORDER_NAMES.get(res[0].dispatch_order if ep else 0)
        self._n = n
        hdt = hidden_states[0].dtype
        sdt = None
        if sp:
            sdt = next(x for x in hidden_states_scale if x is not None).dtype
        edt = None
        if ep_present:
            edt = next(x for x in eplb_local_stats if x is not None).dtype
        out = []
        for d in range(ep):
            r = res[d]
            rows = r.num_rows
            out.append(DispatchResult(
                hidden=self._view(r.hidden, rows, p.hidden_row_bytes, hdt),
                hidden_scale=self._view(r.hidden_scale, rows, p.scale_row_bytes, sdt) if r.hidden_scale else None,
                topk_ids=self._view(r.topk_ids, rows, p.top_k * 4, torch.int32),
                topk_weights=self._view(r.topk_weights, rows, p.top_k * 4, torch.float32)
                if r.topk_weights else None,
                tokens_per_rank=r.tokens_per_rank,
                eplb_global_stats=self._view(r.eplb_global_stats, ep, p.eplb_stats_bytes, edt)
                if r.eplb_global_stats else None))
        return out

    def get_combine_input_buffer(self, rank: int, dtype: torch.dtype) -> torch.Tensor:
        """Rank ``rank``'s ``[ep*tpr, hidden]`` buffer in the workspace; valid
        between dispatch and combine.  Passing it to combine saves a copy."""
        if dtype not in _COMBINE_DTYPES:
            raise TypeError(f"combine dtype must be float32, bfloat16 or float16, got {dtype}")
        ptr = _lib.moe_ep_get_combine_input_buffer(self._handle, rank, _COMBINE_DTYPES[dtype])
        self._buffer_dtype = dtype
        return self._view(ptr, self._p.ep_size * self._tpr, self._p.hidden_size * dtype.itemsize, dtype)

    def combine(self, expert_output: Sequence[Optional[torch.Tensor]], *,
                output: Optional[Sequence[Optional[torch.Tensor]]] = None,
                active_rank_mask=None) -> List[torch.Tensor]:
        """Sum every token's rows over the ranks it reached; see
        include/moe_ep.h, moe_ep_combine.  ``expert_output[d]`` may be
        ``[ep*tpr, hidden]`` or ``[ep, tpr, hidden]``; None means rank d's
        combine input buffer.  When every entry is None the element type is
        the output's, else the one last requested from
        get_combine_input_buffer() this round, else bfloat16.  Outputs not
        passed are returned as slices [s, :n_s] of one new
        [ep, max n_s, hidden] tensor."""
        if self._handle is None:
            raise RuntimeError("MoEEp has been destroyed")
        p = self._p
        di = self._dev_index
        ep = p.ep_size
        if len(expert_output) != ep:
            raise ValueError(f"expected {ep} per-rank expert_output tensors")
        dtype = next((t.dtype for t in expert_output if t is not None), None)
        if dtype is None:       # every rank's input is its combine input buffer
            if output is not None and output[0] is not None:
                dtype = output[0].dtype
            else:
                dtype = self._buffer_dtype if self._buffer_dtype is not None else torch.bfloat16
        if dtype not in _COMBINE_DTYPES:
            raise TypeError(f"combine dtype must be float32, bfloat16 or float16, got {dtype}")
        if self._tpr is None:
            raise _lib.MoeEpError(_lib.MOE_EP_ERR_STATE, "combine", "no dispatch to combine")
        rows = ep * self._tpr
        a = _lib.moe_ep_combine_args()
        a_eo, a_out = a.expert_output, a.output
        for d in range(ep):
            t = expert_output[d]
            if t is None:
                a_eo[d] = None
                continue
            if t.dtype != dtype or t.numel() != rows * p.hidden_size:
                raise ValueError(f"rank {d}: expert_output must be {dtype} [{rows}, {p.hidden_size}]")
            a_eo[d] = _dev_ptr(t, di, "expert_output", d)
        outs = []
        # Outputs the caller leaves to us are slices [s, :n_s] of one
        # allocation: at a constant stride, so the library can take its
        # compact launch (all-scalar kernel arguments, cheaper to enqueue).
        fresh = None
        if output is None or any(o is None for o in output):
            fresh = torch.empty((ep, max(self._n), p.hidden_size), dtype=dtype, device=self.device)
        for s in range(ep):
            ns = self._n[s]
            o = output[s] if output is not None else None
            if o is None:
                o = fresh[s, :ns]
            elif o.dtype != dtype or tuple(o.shape) != (ns, p.hidden_size):
                raise ValueError(f"rank {s}: output must be {dtype} [{ns}, {p.hidden_size}]")
            a_out[s] = _dev_ptr(o, di, "output", s) if ns else None
            outs.append(o)
        a.dtype = _COMBINE_DTYPES[dtype]
        a.active_rank_mask = _mask_value(active_rank_mask)
        stream = torch.cuda.current_stream(self.device).cuda_stream
        _lib.moe_ep_combine(self._handle, a, stream)
        return outs

    def checkpoint_prepare(self) -> None:
        """Release the workspace's physical memory before a process
        checkpoint; its addresses stay reserved, so graphs captured on it
        replay after checkpoint_restore().  Only between rounds; a repeat
        call does nothing.  Workspace views must not be touched until the
        restore (NVLinkOneSidedAlltoAll, checkpoint_prepare())."""
        _lib.moe_ep_checkpoint_prepare(self._handle)

    def checkpoint_restore(self) -> None:
        """Back the workspace with new memory; does nothing when it is
        mapped (NVLinkOneSidedAlltoAll, checkpoint_restore())."""
        _lib.moe_ep_checkpoint_restore(self._handle)

    def destroy(self) -> None:
        """Release the handle; repeated calls do nothing."""
        if self._handle is not None:
            _lib.moe_ep_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
