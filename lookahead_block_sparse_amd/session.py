"""Device state of a batch of requests running the LSA decode loop on one GPU.

An LSASession owns the buffers the three library calls work on and issues the
calls in the order the loop needs them.  It moves data (uploads, the device to
host copy of each new selection) and keeps the host-side residency state; all
arithmetic of the path happens inside liblsa.so.

Layouts:
  * W_q                [n_idx][d_idx][d_model]
  * keys               request r at element n_idx*d_idx*blk_off[r], [n_idx][B_r][d_idx]
  * cold pool          per request B_r blocks (library block format), pinned host
                       memory, or device memory when cold_on_device=True
  * hot pool           sum of the per-request capacities, slots of request r are
                       slot_base[r] .. slot_base[r] + capacity[r] - 1
  * window ring        [R][win_cap/64] blocks
  * block table        request r's (block id, slot) pairs at pair slot_base[r]
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import (
    BLOCK_TOKENS,
    DecodeArgs,
    DeviceGatherArgs,
    GatherArgs,
    LIB,
    RefreshArgs,
    _check,
    _dtype_code,
    lsa_block_bytes,
    lsa_index_refresh,
    lsa_index_refresh_workspace,
    lsa_pack_blocks,
    lsa_query_latent,
    lsa_sparse_decode,
    lsa_sparse_decode_workspace,
)
import ctypes


def _raw_tensor(arr: np.ndarray, device) -> torch.Tensor:
    """Upload the raw bytes of a uint16 (bf16 bits) or float32 array."""
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16))
    elif arr.dtype == np.float32:
        t = torch.from_numpy(arr)
    else:
        raise TypeError(f"unexpected dtype {arr.dtype}")
    return t.to(device)


class LSASession:
    def __init__(self, *, dtype: str, n_idx: int, d_model: int, d_idx: int, n_heads: int, head_dim: int,
                 win_cap: int, n_blocks: Sequence[int], w_q: np.ndarray, keys: Sequence[np.ndarray],
                 capacity: Optional[Sequence[int]] = None, cold_on_device: bool = False,
                 with_masks: bool = False, device: str = "cuda", stream: Optional[torch.cuda.Stream] = None,
                 max_groups: int = 0, n_layers: int = 1, w_down: Optional[np.ndarray] = None,
                 device_plan: bool = False, cold_host_mirror: bool = False, select_level: float = 0.5):
        self.dtype = dtype
        self.select_level = float(select_level)  # keep a block when sigmoid(logit) > this
        self.n_idx, self.d_model, self.d_idx = n_idx, d_model, d_idx
        # low-rank query projection: w_down = A [n_idx][rank][d_model], w_q = B [n_idx][d_idx][rank];
        # every refresh first forms the latents c_i = A_i h, and the Query Encoder reads them
        self.rank = int(w_down.shape[1]) if w_down is not None else 0
        self.q_in = self.rank if self.rank else d_model
        self.n_heads, self.head_dim, self.win_cap = n_heads, head_dim, win_cap
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.max_groups = max_groups
        # attention layers whose block loads one selection drives: each has its own cold pool, hot
        # pool and window ring at a fixed stride from layer 0's; slots and the table are shared
        self.n_layers = int(n_layers)
        if not 1 <= self.n_layers <= 256:
            raise ValueError("n_layers must be in 1..256")
        self.n_req = len(n_blocks)
        self.n_blocks = np.asarray(n_blocks, dtype=np.int64)
        self.blk_off = np.concatenate([[0], np.cumsum(self.n_blocks)]).astype(np.int64)
        self.block_bytes = lsa_block_bytes(dtype, head_dim)
        if self.block_bytes == 0:
            raise ValueError("unsupported dtype/head_dim")
        self.elt = 2 if dtype == "bf16" else 4
        self.cold_on_device = cold_on_device
        # with the cold pool in HBM, an optional copy in pinned host memory: use_cold("host") then
        # makes the gathers cross the host link, with the same blocks and the same residency state
        self.cold_host_mirror = bool(cold_host_mirror and cold_on_device)
        self.cold_src = "device" if cold_on_device else "host"

        with torch.cuda.stream(self.stream):
            self.w_q = _raw_tensor(w_q, self.device)
            self.w_down = _raw_tensor(w_down, self.device) if w_down is not None else None
            self.keys = _raw_tensor(np.concatenate([np.ascontiguousarray(k).reshape(-1) for k in keys]), self.device)
            total_blocks = int(self.blk_off[-1])
            self.sel_ids = torch.zeros(total_blocks, dtype=torch.int32, device=self.device)
            self.sel_count = torch.zeros(self.n_req, dtype=torch.int32, device=self.device)
            self.word_off = np.concatenate([[0], np.cumsum((self.n_blocks + 63) // 64)]).astype(np.int64)
            self.masks = (torch.zeros(int(self.word_off[-1]) * (n_idx + 1), dtype=torch.int64, device=self.device)
                          if with_masks or device_plan else None)
            ws = lsa_index_refresh_workspace(dtype=dtype, d_model=self.q_in, d_idx=d_idx, n_idx=n_idx,
                                             blk_off=self.blk_off)
            self.latent = (torch.empty((self.n_req, n_idx, self.rank), dtype=torch.int16 if dtype == "bf16"
                                       else torch.float32, device=self.device) if self.rank else None)
            self.refresh_ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=self.device)
            self.sel_ids_h = torch.empty(total_blocks, dtype=torch.int32, pin_memory=True)
            self.sel_count_h = torch.empty(self.n_req, dtype=torch.int32, pin_memory=True)
            self._sel_ids_np = self.sel_ids_h.numpy()
            self._sel_count_np = self.sel_count_h.numpy()

            # hot pool and residency state
            cap = np.asarray(capacity if capacity is not None else self.n_blocks, dtype=np.int64)
            self.capacity = cap
            self.slot_base = np.concatenate([[0], np.cumsum(cap)]).astype(np.int64)
            self.n_slots = int(self.slot_base[-1])
            self.hot_layer_bytes = max(1, self.n_slots) * self.block_bytes
            self.hot = torch.empty(self.n_layers * self.hot_layer_bytes, dtype=torch.uint8, device=self.device)
            self.table = torch.zeros(max(1, self.n_slots) * 2, dtype=torch.int32, device=self.device)
            self.slot_of_block = [np.full(int(b), -1, dtype=np.int32) for b in self.n_blocks]
            self.free_slots = [np.arange(self.slot_base[r + 1] - 1, self.slot_base[r] - 1, -1, dtype=np.int32)
                               for r in range(self.n_req)]
            self.n_free = [np.array([int(c)], dtype=np.int32) for c in cap]
            self.stage = [torch.empty(max(4, 4 * int(c)), dtype=torch.int32, pin_memory=True) for c in cap]
            self.n_sel = np.zeros(self.n_req, dtype=np.int32)
            self.sel_host: List[np.ndarray] = [np.zeros(0, dtype=np.int32) for _ in range(self.n_req)]
            self.sel_version = np.zeros(self.n_req, dtype=np.int64)

            # cold pools and rings
            self.cold: List[Optional[torch.Tensor]] = [None] * self.n_req
            self.cold_host: List[Optional[torch.Tensor]] = [None] * self.n_req  # the pinned mirror
            n_chunks = win_cap // BLOCK_TOKENS
            self.ring_layer_bytes = self.n_req * n_chunks * self.block_bytes
            self.ring = torch.zeros(self.n_layers * self.ring_layer_bytes, dtype=torch.uint8, device=self.device)
            ws = lsa_sparse_decode_workspace(dtype=dtype, n_heads=n_heads, head_dim=head_dim, win_cap=win_cap,
                                             n_req=self.n_req, max_groups=max_groups)
            self.decode_ws = torch.empty(ws, dtype=torch.uint8, device=self.device)
        self._gargs: List[Optional[tuple]] = [None] * self.n_req
        self._pargs = {}  # device-plan argument structs per run of requests
        self._rargs = {}  # refresh argument structs per (run of requests, table_out)
        self._stage_ev: List[Optional[torch.cuda.Event]] = [None] * self.n_req
        # residency planned on the device (lsa_gather_plan_device): the state lives in HBM and a
        # refresh never waits for the host
        self.device_plan = bool(device_plan)
        if self.device_plan:
            with torch.cuda.stream(self.stream):
                dev = self.device
                self.resident_dev = torch.zeros(int(self.word_off[-1]), dtype=torch.int64, device=dev)
                self.slot_of_block_dev = torch.empty(int(self.blk_off[-1]), dtype=torch.int32, device=dev)
                self.free_dev = torch.empty(max(1, self.n_slots), dtype=torch.int32, device=dev)
                self.n_free_dev = torch.empty(self.n_req, dtype=torch.int32, device=dev)
                self.table_count = torch.zeros(self.n_req, dtype=torch.int32, device=dev)
                self.copied_dev = torch.zeros(self.n_req, dtype=torch.int32, device=dev)
                self.plan_status = torch.zeros(self.n_req, dtype=torch.int32, device=dev)
                self.plan_status_any = torch.zeros(self.n_req, dtype=torch.int32, device=dev)
            a = self._plan_args(0, self.n_req)[0]
            ws = ctypes.c_size_t(0)
            _check(LIB.lsa_gather_plan_device_workspace(ctypes.byref(a), ctypes.byref(ws)))
            self.plan_ws = torch.empty(int(ws.value), dtype=torch.uint8, device=self.device)
            self._pargs = {}
            a = self._plan_args(0, self.n_req)[0]
            _check(LIB.lsa_residency_reset(ctypes.byref(a), ctypes.c_void_p(self.stream.cuda_stream)))

    # ---------------------------------------------------------------------------------------
    def load_prefill(self, r: int, k_tok: np.ndarray, v_tok: np.ndarray, layer: int = 0) -> None:
        """Pack request r's prefill K/V ([N_r][D] raw) of one layer into its cold pool and window
        ring."""
        n = int(self.n_blocks[r]) * BLOCK_TOKENS
        assert k_tok.shape[0] == n and v_tok.shape[0] == n
        assert 0 <= layer < self.n_layers
        k_tok = np.ascontiguousarray(k_tok)
        v_tok = np.ascontiguousarray(v_tok)
        lb = int(self.n_blocks[r]) * self.block_bytes  # bytes of one layer's cold pool
        if self.cold[r] is None:
            self._pargs.clear()  # they hold the cold pools' addresses
            self.cold[r] = (torch.empty(self.n_layers * lb, dtype=torch.uint8, device=self.device)
                            if self.cold_on_device else
                            torch.empty(self.n_layers * lb, dtype=torch.uint8, pin_memory=True))
            if self.cold_host_mirror:
                self.cold_host[r] = torch.empty(self.n_layers * lb, dtype=torch.uint8, pin_memory=True)
            self._gargs[r] = None
        if self.cold_on_device:
            cold_h = (self.cold_host[r][layer * lb:(layer + 1) * lb] if self.cold_host_mirror
                      else torch.empty(lb, dtype=torch.uint8))
            lsa_pack_blocks(self.dtype, self.head_dim, k_tok, v_tok, 0, n, cold_h, int(self.n_blocks[r]))
            with torch.cuda.stream(self.stream):
                self.cold[r][layer * lb:(layer + 1) * lb].copy_(cold_h)
            self.stream.synchronize()
        else:
            lsa_pack_blocks(self.dtype, self.head_dim, k_tok, v_tok, 0, n, self.cold[r][layer * lb:(layer + 1) * lb],
                            int(self.n_blocks[r]))
        n_chunks = self.win_cap // BLOCK_TOKENS
        ring_h = np.zeros(n_chunks * self.block_bytes, dtype=np.uint8)
        w = min(self.win_cap, n)
        lsa_pack_blocks(self.dtype, self.head_dim, k_tok[n - w:], v_tok[n - w:], n - w, w, ring_h, n_chunks)
        lo = layer * self.ring_layer_bytes + r * n_chunks * self.block_bytes
        with torch.cuda.stream(self.stream):
            self.ring[lo:lo + len(ring_h)].copy_(torch.from_numpy(ring_h).to(self.device))

    def _cold_ptr(self, r: int) -> int:
        """Address of request r's cold pool in use (HBM or pinned host memory)."""
        if self.cold_src == "host" and self.cold_on_device:
            return self.cold_host[r].data_ptr()
        return self.cold[r].data_ptr()

    def use_cold(self, where: str) -> None:
        """Gather from the HBM cold pool ("device") or from its pinned host mirror ("host"); the
        blocks are the same, so the residency state carries over.  Order with the stream: call it
        between refreshes."""
        if where not in ("device", "host"):
            raise ValueError("where is 'device' or 'host'")
        if where == "host" and self.cold_on_device and not self.cold_host_mirror:
            raise ValueError("the session keeps no pinned host copy of its cold pool (cold_host_mirror)")
        if where == "device" and not self.cold_on_device:
            raise ValueError("the cold pool of this session is in pinned host memory")
        if where != self.cold_src:
            self.cold_src = where
            self._pargs.clear()
            self._gargs = [None] * self.n_req

    def layer_views(self, layer: int):
        """(hot pool, window ring) of one layer."""
        h, g = self.hot_layer_bytes, self.ring_layer_bytes
        return self.hot[layer * h:(layer + 1) * h], self.ring[layer * g:(layer + 1) * g]

    # ---------------------------------------------------------------------------------------
    def refresh(self, reqs: Sequence[int], hidden: np.ndarray, bias: np.ndarray, ev_begin=None,
                ev_end=None, ev_latent=(None, None)) -> Dict[int, np.ndarray]:
        """Index refresh for requests `reqs` (hidden [len][d_model] raw or a device tensor, bias
        [len][n_idx] float32 array or device tensor).

        Enqueues lsa_index_refresh per contiguous run of requests, copies the selections back
        (one synchronisation) and returns {r: ascending ids}.  ev_begin / ev_end (torch events)
        time the refresh kernel only (its dispatch, when the requests form one run)."""
        reqs = list(reqs)
        with torch.cuda.stream(self.stream):
            if isinstance(hidden, torch.Tensor):
                hid = hidden.reshape(len(reqs), self.d_model)
            else:
                hid = _raw_tensor(np.ascontiguousarray(hidden).reshape(len(reqs), self.d_model), self.device)
            if isinstance(bias, torch.Tensor):
                bias_d = bias.reshape(len(reqs), self.n_idx)
            else:
                bias_d = torch.from_numpy(np.ascontiguousarray(bias, dtype=np.float32).reshape(
                    len(reqs), self.n_idx)).to(self.device)
            runs = []
            i = 0
            while i < len(reqs):
                j = i
                while j + 1 < len(reqs) and reqs[j + 1] == reqs[j] + 1:
                    j += 1
                runs.append((i, j + 1))
                i = j + 1
            if len(runs) == 1:
                # the library times its own dispatch
                self._refresh_run(reqs[0], reqs[-1] + 1, hid, bias_d, ev_begin, ev_end, ev_latent=ev_latent)
            else:
                if ev_begin is not None:
                    ev_begin.record(self.stream)
                for i, j in runs:
                    r0, r1 = reqs[i], reqs[j - 1] + 1
                    self._refresh_run(r0, r1, hid[i:j], bias_d[i:j])
                if ev_end is not None:
                    ev_end.record(self.stream)
            for i, j in runs:  # one copy per contiguous run of requests
                b0, b1 = int(self.blk_off[reqs[i]]), int(self.blk_off[reqs[j - 1] + 1])
                self.sel_ids_h[b0:b1].copy_(self.sel_ids[b0:b1], non_blocking=True)
            self.sel_count_h.copy_(self.sel_count, non_blocking=True)
        self.stream.synchronize()
        out = {}
        ids_h, count_h = self._sel_ids_np, self._sel_count_np
        for r in reqs:
            b0 = int(self.blk_off[r])
            c = int(count_h[r])
            if c < 0:
                raise RuntimeError(f"index refresh of request {r} reported an incomplete compaction")
            out[r] = ids_h[b0:b0 + c].copy()
        return out

    def _refresh_run(self, r0: int, r1: int, hid: torch.Tensor, bias_d: torch.Tensor, ev_begin=None,
                     ev_end=None, table_out: bool = False, ev_latent=(None, None),
                     stream: Optional[torch.cuda.Stream] = None, bits_only: bool = False) -> None:
        st = self.stream if stream is None else stream
        stride = self.d_model
        if self.rank:
            # the latents of these requests, then the Query Encoder reads them in place of h
            lat = self.latent[r0:r1]
            lsa_query_latent(dtype=self.dtype, d_model=self.d_model, rank=self.rank, n_idx=self.n_idx,
                             n_req=r1 - r0, hidden=hid, w_down=self.w_down, latent=lat, ev_begin=ev_latent[0],
                             ev_end=ev_latent[1], stream=st)
            hid = lat
            stride = self.n_idx * self.rank
        key = (r0, r1, bool(table_out), bool(bits_only))
        cached = self._rargs.get(key)
        if cached is None:
            # the first call of a run of requests goes through the checked wrapper; the argument
            # struct it builds is kept, and later calls only swap the hidden states, the biases and
            # the events (the library validates every call)
            off = self.blk_off[r0:r1 + 1] - self.blk_off[r0]
            key_elem0 = int(self.n_idx * self.d_idx * self.blk_off[r0])
            masks = None
            if self.masks is not None:
                masks = self.masks[int(self.word_off[r0]) * (self.n_idx + 1):]
            lsa_index_refresh(dtype=self.dtype, d_model=self.q_in, d_idx=self.d_idx, n_idx=self.n_idx, hidden=hid,
                              hidden_req_stride=stride, hidden_idx_stride=self.rank,
                              w_q=self.w_q, keys=self.keys[key_elem0:], blk_off=off, bias=bias_d,
                              sel_ids=None if bits_only else self.sel_ids[int(self.blk_off[r0]):],
                              sel_count=self.sel_count[r0:r1],
                              workspace=self.refresh_ws, masks=masks, ev_begin=ev_begin, ev_end=ev_end,
                              table_out=(self.table[2 * int(self.slot_base[r0]):] if table_out else None),
                              table_slot_base=(self.slot_base[r0:r1] if table_out else None),
                              stream=st, select_level=self.select_level)
            self._rargs[key] = self._refresh_struct(r0, r1, stride, table_out, masks, bits_only)
            return
        a, _keep, need_hid, need_bias = cached
        if not (hid.is_cuda and bias_d.is_cuda and hid.is_contiguous() and bias_d.is_contiguous()
                and hid.numel() * hid.element_size() >= need_hid and bias_d.numel() * 4 >= need_bias):
            raise ValueError("refresh: hidden states and biases must be contiguous device tensors of the run's size")
        a.hidden, a.bias = hid.data_ptr(), bias_d.data_ptr()
        a.ev_begin = ev_begin.cuda_event if ev_begin is not None else None
        a.ev_end = ev_end.cuda_event if ev_end is not None else None
        _check(LIB.lsa_index_refresh(ctypes.byref(a), ctypes.c_void_p(st.cuda_stream)))

    def _refresh_struct(self, r0: int, r1: int, stride: int, table_out: bool, masks, bits_only: bool = False):
        """The refresh argument struct of a run of requests (every field but the hidden states, the
        biases and the events), with the arrays it points into."""
        off = np.ascontiguousarray(self.blk_off[r0:r1 + 1] - self.blk_off[r0], dtype=np.int64)
        a = RefreshArgs()
        a.n_req, a.d_model, a.d_idx, a.n_idx = r1 - r0, self.q_in, self.d_idx, self.n_idx
        a.dtype = _dtype_code(self.dtype)
        a.select_level = float(self.select_level)
        a.hidden_req_stride, a.hidden_idx_stride = int(stride), int(self.rank)
        a.w_q = self.w_q.data_ptr()
        a.keys = self.keys.data_ptr() + int(self.n_idx * self.d_idx * self.blk_off[r0]) * self.keys.element_size()
        a.blk_off = off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        a.sel_ids = None if bits_only else self.sel_ids.data_ptr() + int(self.blk_off[r0]) * 4
        a.sel_count = self.sel_count.data_ptr() + r0 * 4
        a.masks = masks.data_ptr() if masks is not None else None
        a.workspace = self.refresh_ws.data_ptr()
        a.workspace_bytes = self.refresh_ws.numel() * self.refresh_ws.element_size()
        tsb = None
        if table_out:
            tsb = np.ascontiguousarray(self.slot_base[r0:r1], dtype=np.int32)
            a.table_out = self.table.data_ptr() + 4 * 2 * int(self.slot_base[r0])
            a.table_slot_base = tsb.ctypes.data
        e = 2 if self.dtype == "bf16" else 4
        need_hid = ((r1 - r0 - 1) * stride + (self.n_idx - 1) * self.rank + self.q_in) * e
        need_bias = (r1 - r0) * self.n_idx * 4
        return a, (off, tsb), need_hid, need_bias

    def union_ids(self, r: int) -> np.ndarray:
        """Request r's selected block ids, ascending, read from the union plane of its last refresh
        (a device-planned refresh writes the bit planes and no ids)."""
        u = np.unpackbits(np.ascontiguousarray(self.masks_of(r)[self.n_idx]).view(np.uint8), bitorder="little")
        return np.flatnonzero(u[:int(self.n_blocks[r])]).astype(np.int32)

    def masks_of(self, r: int) -> np.ndarray:
        """Request r's bit planes [n_idx+1][words] (after a refresh with masks enabled)."""
        w = int(self.word_off[r + 1] - self.word_off[r])
        base = int(self.word_off[r]) * (self.n_idx + 1)
        m = self.masks[base:base + w * (self.n_idx + 1)].cpu().numpy().view(np.uint64)
        return m.reshape(self.n_idx + 1, w)

    # ---------------------------------------------------------------------------------------
    def _plan_args(self, r0: int, r1: int):
        """lsa_device_gather_args for requests r0 .. r1-1 (built once per run of requests)."""
        key = (r0, r1)
        if key not in self._pargs:
            a = DeviceGatherArgs()
            a.n_req, a.n_idx, a.block_bytes, a.n_layers = r1 - r0, self.n_idx, self.block_bytes, self.n_layers
            blk = np.ascontiguousarray(self.blk_off[r0:r1 + 1] - self.blk_off[r0], dtype=np.int64)
            slo = np.ascontiguousarray(self.slot_base[r0:r1 + 1] - self.slot_base[r0], dtype=np.int32)
            w0, s0, b0 = int(self.word_off[r0]), int(self.slot_base[r0]), int(self.blk_off[r0])
            a.blk_off, a.slot_off = blk.ctypes.data, slo.ctypes.data
            a.masks = self.masks.data_ptr() + 8 * w0 * (self.n_idx + 1)
            a.sel_count = self.sel_count.data_ptr() + 4 * r0
            a.resident = self.resident_dev.data_ptr() + 8 * w0
            a.slot_of_block = self.slot_of_block_dev.data_ptr() + 4 * b0
            a.free_slots = self.free_dev.data_ptr() + 4 * s0
            a.n_free = self.n_free_dev.data_ptr() + 4 * r0
            cold = (ctypes.c_void_p * (r1 - r0))(*[self._cold_ptr(r) if self.cold[r] is not None else None
                                                   for r in range(r0, r1)])
            a.cold = ctypes.cast(cold, ctypes.c_void_p)
            if self.n_layers > 1 and r1 - r0 > 1 and len(set(self.n_blocks[r0:r1].tolist())) > 1:
                raise ValueError("device planning over several layers needs equal block counts in a run")
            a.cold_layer_bytes = int(self.n_blocks[r0]) * self.block_bytes
            a.hot, a.hot_layer_bytes = self.hot.data_ptr(), self.hot_layer_bytes
            a.table = self.table.data_ptr() + 8 * s0
            a.table_count = self.table_count.data_ptr() + 4 * r0
            a.copied = self.copied_dev.data_ptr() + 4 * r0
            a.status = self.plan_status.data_ptr() + 4 * r0
            a.status_any = self.plan_status_any.data_ptr() + 4 * r0
            ws = getattr(self, "plan_ws", None)
            a.workspace = ws.data_ptr() if ws is not None else None
            a.workspace_bytes = ws.numel() if ws is not None else 0
            self._pargs[key] = (a, blk, slo, cold)
        return self._pargs[key]

    def refresh_device(self, reqs: Sequence[int], hidden: torch.Tensor, bias: torch.Tensor, ev_begin=None,
                       ev_end=None, ev_plan=(None, None), ev_latent=(None, None),
                       copied_out: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Index refresh of `reqs` followed by the gather planned and run on the device
        (lsa_gather_plan_device): nothing is copied back and nothing waits for the host.  The
        refresh writes the bit planes only (the plan ranks the selected blocks from the union plane
        and writes the counts to `sel_count`; `union_ids` reads a selection back).  The decode then
        reads the tables' counts on the device (DecodeLoop(..., device_counts=True)).
        The plan writes the number of blocks it copied for request r to entry r of `copied_out`
        (an int32 device tensor of n_req entries) when given, else to `copied_dev`.  Everything is
        enqueued on `stream` (default: the session's stream)."""
        if not self.device_plan:
            raise RuntimeError("the session was built without device_plan")
        if copied_out is not None and not (copied_out.is_cuda and copied_out.dtype == torch.int32 and
                                           copied_out.is_contiguous() and copied_out.numel() >= self.n_req):
            raise ValueError(f"copied_out must be a contiguous int32 device tensor of {self.n_req} entries")
        copied_base = (copied_out if copied_out is not None else self.copied_dev).data_ptr()
        st = self.stream if stream is None else stream
        reqs = list(reqs)
        hid = hidden.reshape(len(reqs), self.d_model)
        bias_d = bias.reshape(len(reqs), self.n_idx)
        i = 0
        while i < len(reqs):
            j = i
            while j + 1 < len(reqs) and reqs[j + 1] == reqs[j] + 1:
                j += 1
            r0, r1 = reqs[i], reqs[j] + 1
            one_run = i == 0 and j == len(reqs) - 1
            # the plan ranks the selected blocks from the union plane: the refresh writes bit planes only
            self._refresh_run(r0, r1, hid[i:j + 1], bias_d[i:j + 1], ev_begin if one_run else None,
                              ev_end if one_run else None, ev_latent=ev_latent if one_run else (None, None),
                              stream=st, bits_only=True)
            a = self._plan_args(r0, r1)[0]
            a.copied = copied_base + 4 * r0
            a.ev_begin = ev_plan[0].cuda_event if (ev_plan[0] is not None and one_run) else None
            a.ev_end = ev_plan[1].cuda_event if (ev_plan[1] is not None and one_run) else None
            _check(LIB.lsa_gather_plan_device(ctypes.byref(a), ctypes.c_void_p(st.cuda_stream)))
            i = j + 1
        self.sel_version[reqs] += 1

    def check_plan_status(self) -> None:
        """Raise if any device-planned refresh since the last check gave up or did not fit its
        request's slots (then that request kept its previous table); clears the record.  Reads
        one small device array, so it waits for the stream."""
        if not self.device_plan:
            return
        with torch.cuda.stream(self.stream):
            st = self.plan_status_any.cpu().numpy()
            self.plan_status_any.zero_()
        bad = np.flatnonzero(st)
        if len(bad):
            what = {1: "did not fit its slots", 2: "gave up (incomplete compaction)", 3: "gave up and did not fit"}
            raise RuntimeError("device-planned refresh failed: " +
                               "; ".join(f"request {r} {what.get(int(st[r]), int(st[r]))}" for r in bad))

    def gather(self, r: int, ids: np.ndarray):
        """Make request r's hot pool hold exactly `ids` (returns (copied, kept))."""
        return self.gather_many({r: ids})[r]

    def _gather_args(self, r: int):
        if self.cold[r] is None:
            raise RuntimeError(f"request {r} has no cold pool: call load_prefill first")
        if self._gargs[r] is None:
            # every field but the selection is fixed for the session: built once per request
            a = GatherArgs()
            a.n_blocks, a.n_slots_total, a.block_bytes = int(self.n_blocks[r]), self.n_slots, self.block_bytes
            a.cold, a.hot = self._cold_ptr(r), self.hot.data_ptr()
            a.stage_ints = self.stage[r].numel()
            a.slot_of_block = self.slot_of_block[r].ctypes.data
            a.free_slots = self.free_slots[r].ctypes.data
            a.n_free = self.n_free[r].ctypes.data
            a.capacity, a.n_layers = int(self.capacity[r]), self.n_layers
            a.cold_layer_bytes = int(self.n_blocks[r]) * self.block_bytes
            a.hot_layer_bytes = self.hot_layer_bytes
            a.stage = self.stage[r].data_ptr()
            a.table_dev = self.table.data_ptr() + 4 * 2 * int(self.slot_base[r])
            counts = np.zeros(2, dtype=np.int32)
            a.n_copied, a.n_kept = counts.ctypes.data, counts.ctypes.data + 4
            self._gargs[r] = (a, counts)
        return self._gargs[r]

    def gather_many(self, sel: Dict[int, np.ndarray], ev_copy=(None, None)):
        """Gathers of several requests after one refresh, planned together and copied by one kernel
        launch (lsa_gather_blocks_batch) on the session's stream, so they follow every decode step
        enqueued before them (slots of leaving blocks are overwritten) and precede every later one.
        Returns {r: (copied, kept)}.  ev_copy (a pair of torch.cuda.Event) takes the copy kernel's
        dispatch stamps."""
        st = self.stream
        reqs = list(sel)
        ids = {r: np.ascontiguousarray(sel[r], dtype=np.int32) for r in reqs}
        arr = (GatherArgs * len(reqs))()
        counts = []
        for k, r in enumerate(reqs):
            a, c = self._gather_args(r)
            if self._stage_ev[r] is not None:
                self._stage_ev[r].synchronize()  # the previous copy kernel may still read stage[r]
            a.new_ids, a.n_new = ids[r].ctypes.data, len(ids[r])
            arr[k] = a
            counts.append(c)
        arr[0].ev_begin = ev_copy[0].cuda_event if ev_copy[0] is not None else None
        arr[0].ev_end = ev_copy[1].cuda_event if ev_copy[1] is not None else None
        _check(LIB.lsa_gather_blocks_batch(arr, len(reqs), st.cuda_stream))
        ev = torch.cuda.Event()
        ev.record(st)
        out = {}
        for k, r in enumerate(reqs):
            self._stage_ev[r] = ev
            self.n_sel[r] = len(ids[r])
            self.sel_host[r] = ids[r]
            self.sel_version[r] += 1
            out[r] = (int(counts[k][0]), int(counts[k][1]))
        return out

    def make_resident(self) -> None:
        """Load every block of every request into the hot pool (capacity must equal the block
        count), block b of request r at slot slot_base[r] + b: the fully resident pool that
        ResidentLoop reads through the table the refresh writes."""
        if not np.array_equal(self.capacity, self.n_blocks):
            raise ValueError("a resident pool needs capacity == n_blocks for every request")
        res = self.gather_many({r: np.arange(int(self.n_blocks[r]), dtype=np.int32) for r in range(self.n_req)})
        self.stream.synchronize()
        for r in range(self.n_req):
            want = np.arange(int(self.slot_base[r]), int(self.slot_base[r + 1]), dtype=np.int32)
            if not np.array_equal(self.slot_of_block[r], want):
                raise RuntimeError(f"request {r}: blocks were not placed in block order (gathered before?)")
        return res

    # ---------------------------------------------------------------------------------------
    def decode(self, q: torch.Tensor, seq_len: Sequence[int], window: Sequence[int], out: torch.Tensor,
               k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
               max_groups: Optional[int] = None, ev_attn_begin=None, ev_attn_end=None, layer: int = 0) -> None:
        """One decode step of one layer for all requests of the session."""
        pool, ring = self.layer_views(layer)
        lsa_sparse_decode(dtype=self.dtype, n_heads=self.n_heads, head_dim=self.head_dim, win_cap=self.win_cap,
                          q=q, ring=ring, out=out, workspace=self.decode_ws,
                          tbl_off=self.slot_base[:-1], n_sel=self.n_sel,
                          seq_len=seq_len, window=window,
                          pool=pool, n_slots_total=self.n_slots, table=self.table, k_new=k_new, v_new=v_new,
                          max_groups=self.max_groups if max_groups is None else max_groups,
                          ev_attn_begin=ev_attn_begin, ev_attn_end=ev_attn_end, stream=self.stream)


class DecodeLoop:
    """Per-step decode calls with the argument struct built once.

    For a fixed session, window and stream, step(t) only rewrites the per-request lengths (prefill +
    t + 1), the table counts and the q / k_new / v_new addresses, then calls lsa_sparse_decode (which
    itself leaves out the table's blocks that lie inside the window).  Events (torch.cuda.Event) may be passed per call to time the attention kernel.
    """

    def __init__(self, sess: LSASession, prefill: Sequence[int], window: Sequence[int], out: torch.Tensor,
                 layer: int = 0, device_counts: bool = False):
        self.sess = sess
        self.device_counts = bool(device_counts)
        self.prefill = np.asarray(prefill, dtype=np.int64)
        self.window = np.ascontiguousarray(window, dtype=np.int32)
        self.seq_len = np.zeros(sess.n_req, dtype=np.int32)
        self.n_sel = np.zeros(sess.n_req, dtype=np.int32)
        self.tbl_off = np.ascontiguousarray(sess.slot_base[:-1], dtype=np.int32)
        a = DecodeArgs()
        a.n_req, a.n_heads, a.head_dim = sess.n_req, sess.n_heads, sess.head_dim
        a.dtype = 1 if sess.dtype == "bf16" else 0
        a.win_cap = sess.win_cap
        a.scale = float(1.0 / np.sqrt(sess.head_dim))
        pool, ring = sess.layer_views(layer)
        a.ring, a.pool, a.table = ring.data_ptr(), pool.data_ptr(), sess.table.data_ptr()
        a.n_slots_total, a.reserved0 = sess.n_slots, 0
        a.tbl_off, a.n_sel = self.tbl_off.ctypes.data, self.n_sel.ctypes.data
        a.seq_len, a.window = self.seq_len.ctypes.data, self.window.ctypes.data
        a.out = out.data_ptr()
        a.workspace, a.workspace_bytes = sess.decode_ws.data_ptr(), sess.decode_ws.numel()
        a.max_groups, a.reserved1 = sess.max_groups, 0
        if self.device_counts:
            # the tables the device planner writes: counts on the device, capacities on the host
            if not sess.device_plan:
                raise ValueError("device_counts needs a session with device_plan")
            self.n_sel[:] = np.asarray(sess.capacity, dtype=np.int32)
            a.n_sel_dev = sess.table_count.data_ptr()
        self.args = a
        self.ref = ctypes.byref(a)
        self.stream = ctypes.c_void_p(sess.stream.cuda_stream)
        self._subs = {}  # (requests, workspace) -> argument struct of a call over those rows

    def _subset(self, reqs: tuple, ws: torch.Tensor):
        key = (reqs, ws.data_ptr())
        sub = self._subs.get(key)
        if sub is None:
            idx = np.asarray(reqs, dtype=np.int64)
            a = DecodeArgs()
            ctypes.memmove(ctypes.byref(a), ctypes.byref(self.args), ctypes.sizeof(DecodeArgs))
            arrays = {"rows": np.ascontiguousarray(idx, dtype=np.int32),
                      "tbl_off": np.ascontiguousarray(self.tbl_off[idx]),
                      "n_sel": np.ascontiguousarray(self.n_sel[idx]),
                      "window": np.ascontiguousarray(self.window[idx]),
                      "seq_len": np.zeros(len(idx), dtype=np.int32)}
            a.n_req = len(idx)
            a.req_rows, a.tbl_off = arrays["rows"].ctypes.data, arrays["tbl_off"].ctypes.data
            a.n_sel, a.window = arrays["n_sel"].ctypes.data, arrays["window"].ctypes.data
            a.seq_len = arrays["seq_len"].ctypes.data
            a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
            sub = self._subs[key] = (a, ctypes.byref(a), idx, arrays)
        return sub

    def step_rows(self, t: int, reqs: Sequence[int], q: torch.Tensor, k_new: Optional[torch.Tensor],
                  v_new: Optional[torch.Tensor], stream: torch.cuda.Stream, workspace: torch.Tensor,
                  ev_begin=None, ev_end=None) -> None:
        """Step t for the requests `reqs` only (rows of q, k_new, v_new and out), on `stream`, with
        its split-K partials in `workspace` (at least the session's decode workspace in size)."""
        if workspace.numel() < self.sess.decode_ws.numel():
            raise ValueError("step_rows: workspace smaller than the session's decode workspace")
        a, ref, idx, arrays = self._subset(tuple(int(r) for r in reqs), workspace)
        np.add(self.prefill[idx], t + 1, out=arrays["seq_len"], casting="unsafe")
        if not self.device_counts:
            arrays["n_sel"][:] = self.sess.n_sel[idx]
        a.q = q.data_ptr()
        a.k_new = k_new.data_ptr() if k_new is not None else None
        a.v_new = v_new.data_ptr() if v_new is not None else None
        a.ev_attn_begin = ev_begin.cuda_event if ev_begin is not None else None
        a.ev_attn_end = ev_end.cuda_event if ev_end is not None else None
        _check(LIB.lsa_sparse_decode(ref, ctypes.c_void_p(stream.cuda_stream)))

    def step(self, t: int, q: torch.Tensor, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
             ev_begin=None, ev_end=None) -> None:
        np.add(self.prefill, t + 1, out=self.seq_len, casting="unsafe")
        if not self.device_counts:  # the table counts of the host-planned selections
            self.n_sel[:] = self.sess.n_sel
        a = self.args
        a.q = q.data_ptr()
        a.k_new = k_new.data_ptr() if k_new is not None else None
        a.v_new = v_new.data_ptr() if v_new is not None else None
        a.ev_attn_begin = ev_begin.cuda_event if ev_begin is not None else None
        a.ev_attn_end = ev_end.cuda_event if ev_end is not None else None
        _check(LIB.lsa_sparse_decode(self.ref, self.stream))


class StaggeredLoop:
    """Decode steps of a device-planned session whose requests refresh at different steps.  At a
    step where some requests refresh, their refresh, residency plan, block copy and their own
    attention run on a second stream while the other requests' attention runs on the session's
    stream; the session's stream then waits for the second one, so the next step sees every new
    table.  No request attends over a selection before its copy has landed (both are on the second
    stream, in that order), and the second stream starts only when the previous step's work on the
    session's stream is done (that work still reads the refreshing requests' old slots).  Steps
    without a refresh are one call, as in DecodeLoop."""

    def __init__(self, sess: LSASession, prefill: Sequence[int], window: Sequence[int], out: torch.Tensor,
                 side_stream: Optional[torch.cuda.Stream] = None):
        if not sess.device_plan:
            raise ValueError("StaggeredLoop needs a session with device_plan")
        self.sess = sess
        self.loop = DecodeLoop(sess, prefill, window, out, device_counts=True)
        self.side = side_stream if side_stream is not None else torch.cuda.Stream(device=sess.device)
        self.ws_side = torch.empty_like(sess.decode_ws)
        self.fork, self.join = torch.cuda.Event(), torch.cuda.Event()

    def step(self, t: int, q: torch.Tensor, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
             refresh: Sequence[int] = (), hidden: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
             ev_begin=None, ev_end=None, ev_refresh=(None, None), ev_plan=(None, None),
             copied_out: Optional[torch.Tensor] = None) -> None:
        """Step t; `refresh` lists the requests that refresh first (hidden states and biases of
        those requests, in that order).  ev_begin/ev_end time the attention of the requests that
        do not refresh (or of all of them at a step without a refresh)."""
        sess = self.sess
        S = sorted(int(r) for r in refresh)
        if not S:
            self.loop.step(t, q, k_new, v_new, ev_begin, ev_end)
            return
        if S != [int(r) for r in refresh]:
            raise ValueError("StaggeredLoop.step: list the refreshing requests in ascending order")
        if hidden is None or bias is None:
            raise ValueError("StaggeredLoop.step: refreshing requests need their hidden states and biases")
        others = [r for r in range(sess.n_req) if r not in set(S)]
        # the inputs are read on the second stream: keep the allocator from reusing them meanwhile
        for x in (q, k_new, v_new, hidden, bias, copied_out):
            if x is not None:
                x.record_stream(self.side)
        self.fork.record(sess.stream)
        self.side.wait_event(self.fork)
        sess.refresh_device(S, hidden, bias, ev_begin=ev_refresh[0], ev_end=ev_refresh[1], ev_plan=ev_plan,
                            copied_out=copied_out, stream=self.side)
        self.loop.step_rows(t, S, q, k_new, v_new, self.side, self.ws_side)
        if others:
            self.loop.step_rows(t, others, q, k_new, v_new, sess.stream, sess.decode_ws, ev_begin, ev_end)
        self.join.record(self.side)
        sess.stream.wait_event(self.join)


class ResidentLoop:
    """Reactive comparator: at every step the index is refreshed with that step's hidden state and the
    decode attends over the window and the blocks just selected, read straight from a hot pool that
    holds every block (LSASession.make_resident).  The refresh writes the decode's block table and
    the decode reads the per-request counts on the device, so a step makes no host round trip and
    moves no block.  Events (torch.cuda.Event pairs) may be passed per call to time the refresh and
    the attention kernel."""

    def __init__(self, sess: LSASession, prefill: Sequence[int], window: Sequence[int], out: torch.Tensor,
                 layer: int = 0):
        if not np.array_equal(sess.capacity, sess.n_blocks):
            raise ValueError("ResidentLoop needs a session with capacity == n_blocks, made resident")
        self.sess = sess
        self.loop = DecodeLoop(sess, prefill, window, out, layer=layer)
        a = self.loop.args
        # capacities on the host, counts from the refresh on the device
        self.cap = np.ascontiguousarray(sess.n_blocks, dtype=np.int32)
        a.n_sel = self.cap.ctypes.data
        a.n_sel_dev = sess.sel_count.data_ptr()

    def step(self, t: int, hidden: torch.Tensor, bias: torch.Tensor, q: torch.Tensor, k_new: Optional[torch.Tensor],
             v_new: Optional[torch.Tensor], ev_refresh=(None, None), ev_attn=(None, None)) -> None:
        sess = self.sess
        sess._refresh_run(0, sess.n_req, hidden.reshape(sess.n_req, sess.d_model),
                          bias.reshape(sess.n_req, sess.n_idx), ev_refresh[0], ev_refresh[1], table_out=True)
        lp = self.loop
        np.add(lp.prefill, t + 1, out=lp.seq_len, casting="unsafe")
        a = lp.args
        a.q = q.data_ptr()
        a.k_new = k_new.data_ptr() if k_new is not None else None
        a.v_new = v_new.data_ptr() if v_new is not None else None
        a.ev_attn_begin = ev_attn[0].cuda_event if ev_attn[0] is not None else None
        a.ev_attn_end = ev_attn[1].cuda_event if ev_attn[1] is not None else None
        _check(LIB.lsa_sparse_decode(lp.ref, lp.stream))
