"""Python binding of liblsa.so, the MI355X (gfx950) Lookahead Sparse Attention decode path.

Argument marshalling only: every step of the path runs in the library's HIP
kernels and host planner.  The functions carry the C names:

    lsa_index_refresh_workspace / lsa_index_refresh
    lsa_gather_blocks
    lsa_sparse_decode_workspace / lsa_sparse_decode
    lsa_pack_blocks, lsa_block_bytes

Device buffers are torch tensors on a ROCm device (raw bit patterns are fine:
bf16 data may live in int16/uint16 tensors); host-side planner state is NumPy.
Importing fails with an error if the built library is missing; build it with
``python lookahead_block_sparse_amd/_build.py``.
"""

from __future__ import annotations

import ctypes
from ctypes import POINTER, Structure, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p
from pathlib import Path
from typing import Optional, Sequence

import numpy as np

_LIB_PATH = Path(__file__).resolve().parent / "liblsa.so"

LSA_OK = 0
LSA_ERR_INVALID = -1
LSA_ERR_UNSUPPORTED = -2
LSA_ERR_CAPACITY = -3
LSA_ERR_WORKSPACE = -4
LSA_ERR_HIP = -5
LSA_F32 = 0
LSA_BF16 = 1
BLOCK_TOKENS = 64
MAX_REFRESH_REQ = 64
MAX_DECODE_REQ = 64
ABI_VERSION = 14

_STATUS_NAMES = {
    LSA_ERR_INVALID: "LSA_ERR_INVALID",
    LSA_ERR_UNSUPPORTED: "LSA_ERR_UNSUPPORTED",
    LSA_ERR_CAPACITY: "LSA_ERR_CAPACITY",
    LSA_ERR_WORKSPACE: "LSA_ERR_WORKSPACE",
    LSA_ERR_HIP: "LSA_ERR_HIP",
}

EXPORTED_SYMBOLS = (
    "lsa_last_error",
    "lsa_abi_version",
    "lsa_struct_size",
    "lsa_block_bytes",
    "lsa_pack_blocks",
    "lsa_index_refresh_workspace",
    "lsa_index_refresh",
    "lsa_query_latent",
    "lsa_gather_blocks",
    "lsa_gather_blocks_batch",
    "lsa_gather_plan_device_workspace",
    "lsa_gather_plan_device",
    "lsa_residency_reset",
    "lsa_sparse_decode_workspace",
    "lsa_sparse_decode",
    "lsa_sparse_decode_noalloc",
    "lsa_label_denoise_workspace",
    "lsa_label_denoise",
)


class LSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class RefreshArgs(Structure):
    _fields_ = [
        ("n_req", c_int32), ("d_model", c_int32), ("d_idx", c_int32), ("n_idx", c_int32),
        ("dtype", c_int32), ("select_level", c_float),
        ("hidden", c_void_p), ("hidden_req_stride", c_int64), ("hidden_idx_stride", c_int64),
        ("w_q", c_void_p), ("keys", c_void_p), ("blk_off", POINTER(c_int64)), ("bias", c_void_p),
        ("sel_ids", c_void_p), ("sel_count", c_void_p), ("masks", c_void_p),
        ("workspace", c_void_p), ("workspace_bytes", c_size_t),
        ("ev_begin", c_void_p), ("ev_end", c_void_p),
        ("table_out", c_void_p), ("table_slot_base", c_void_p), ("logits", c_void_p),
    ]


class LatentArgs(Structure):
    _fields_ = [
        ("n_req", c_int32), ("d_model", c_int32), ("rank", c_int32), ("n_idx", c_int32),
        ("dtype", c_int32), ("reserved0", c_int32),
        ("hidden", c_void_p), ("hidden_req_stride", c_int64), ("hidden_idx_stride", c_int64),
        ("w_down", c_void_p), ("latent", c_void_p),
        ("ev_begin", c_void_p), ("ev_end", c_void_p),
    ]


class DenoiseArgs(Structure):
    _fields_ = [
        ("n_layers", c_int32), ("n_windows", c_int32), ("min_votes", c_int32), ("reserved0", c_int32),
        ("top_p", ctypes.c_double), ("logits", c_void_p), ("logit_stride", c_int64),
        ("n_blk", c_void_p), ("n_blk_dev", c_void_p), ("layer_sets", c_void_p), ("labels", c_void_p),
        ("n_pos", c_void_p), ("n_naive", c_void_p), ("workspace", c_void_p), ("workspace_bytes", c_size_t),
        ("ev_begin", c_void_p), ("ev_end", c_void_p),
    ]


class DeviceGatherArgs(Structure):
    _fields_ = [
        ("n_req", c_int32), ("n_idx", c_int32), ("block_bytes", c_int32), ("n_layers", c_int32),
        ("blk_off", c_void_p), ("slot_off", c_void_p), ("masks", c_void_p), ("sel_count", c_void_p),
        ("resident", c_void_p), ("slot_of_block", c_void_p), ("free_slots", c_void_p), ("n_free", c_void_p),
        ("cold", c_void_p), ("cold_layer_bytes", c_int64), ("hot", c_void_p), ("hot_layer_bytes", c_int64),
        ("table", c_void_p), ("table_count", c_void_p), ("copied", c_void_p), ("status", c_void_p),
        ("status_any", c_void_p),
        ("workspace", c_void_p), ("workspace_bytes", c_size_t), ("ev_begin", c_void_p), ("ev_end", c_void_p),
    ]


class GatherArgs(Structure):
    _fields_ = [
        ("n_blocks", c_int64), ("n_slots_total", c_int32), ("block_bytes", c_int32),
        ("cold", c_void_p), ("hot", c_void_p), ("new_ids", c_void_p), ("n_new", c_int32),
        ("stage_ints", c_int32), ("slot_of_block", c_void_p), ("free_slots", c_void_p),
        ("n_free", c_void_p), ("capacity", c_int32), ("n_layers", c_int32), ("stage", c_void_p),
        ("table_dev", c_void_p), ("n_copied", c_void_p), ("n_kept", c_void_p),
        ("cold_layer_bytes", c_int64), ("hot_layer_bytes", c_int64),
        ("ev_begin", c_void_p), ("ev_end", c_void_p),
    ]


class DecodeArgs(Structure):
    _fields_ = [
        ("n_req", c_int32), ("n_heads", c_int32), ("head_dim", c_int32), ("dtype", c_int32),
        ("win_cap", c_int32), ("scale", c_float),
        ("q", c_void_p), ("k_new", c_void_p), ("v_new", c_void_p), ("ring", c_void_p), ("pool", c_void_p),
        ("n_slots_total", c_int32), ("reserved0", c_int32),
        ("table", c_void_p), ("tbl_off", c_void_p), ("n_sel", c_void_p), ("seq_len", c_void_p),
        ("window", c_void_p), ("out", c_void_p), ("workspace", c_void_p), ("workspace_bytes", c_size_t),
        ("max_groups", c_int32), ("reserved1", c_int32),
        ("ev_attn_begin", c_void_p), ("ev_attn_end", c_void_p),
        ("n_sel_dev", c_void_p), ("req_rows", c_void_p),
    ]


def _load():
    # liblsa.so needs libamdhip64.so.7.  PyTorch ships its own copy under that soname; importing
    # torch first makes the library bind to the runtime torch already uses, so device memory,
    # streams and events are shared by one HIP runtime in the process.
    import torch  # noqa: F401

    if not _LIB_PATH.exists():
        raise ImportError(
            f"{_LIB_PATH} is missing: the LSA path has no fallback; build it with "
            "`python lookahead_block_sparse_amd/_build.py`")
    lib = ctypes.CDLL(str(_LIB_PATH))
    lib.lsa_last_error.restype = c_char_p
    lib.lsa_abi_version.restype = c_int32
    lib.lsa_struct_size.restype = c_size_t
    lib.lsa_struct_size.argtypes = [c_int32]
    lib.lsa_block_bytes.restype = c_size_t
    lib.lsa_block_bytes.argtypes = [c_int32, c_int32]
    lib.lsa_pack_blocks.restype = c_int32
    lib.lsa_pack_blocks.argtypes = [c_int32, c_int32, c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int32]
    lib.lsa_index_refresh_workspace.restype = c_int32
    lib.lsa_index_refresh_workspace.argtypes = [POINTER(RefreshArgs), POINTER(c_size_t)]
    lib.lsa_index_refresh.restype = c_int32
    lib.lsa_index_refresh.argtypes = [POINTER(RefreshArgs), c_void_p]
    lib.lsa_query_latent.restype = c_int32
    lib.lsa_query_latent.argtypes = [POINTER(LatentArgs), c_void_p]
    lib.lsa_label_denoise_workspace.restype = c_int32
    lib.lsa_label_denoise_workspace.argtypes = [POINTER(DenoiseArgs), POINTER(c_size_t)]
    lib.lsa_label_denoise.restype = c_int32
    lib.lsa_label_denoise.argtypes = [POINTER(DenoiseArgs), c_void_p]
    for fn in ("lsa_gather_plan_device", "lsa_residency_reset"):
        getattr(lib, fn).restype = c_int32
        getattr(lib, fn).argtypes = [POINTER(DeviceGatherArgs), c_void_p]
    lib.lsa_gather_plan_device_workspace.restype = c_int32
    lib.lsa_gather_plan_device_workspace.argtypes = [POINTER(DeviceGatherArgs), POINTER(c_size_t)]
    lib.lsa_gather_blocks.restype = c_int32
    lib.lsa_gather_blocks.argtypes = [POINTER(GatherArgs), c_void_p]
    lib.lsa_gather_blocks_batch.restype = c_int32
    lib.lsa_gather_blocks_batch.argtypes = [POINTER(GatherArgs), c_int32, c_void_p]
    lib.lsa_sparse_decode_workspace.restype = c_int32
    lib.lsa_sparse_decode_workspace.argtypes = [POINTER(DecodeArgs), POINTER(c_size_t)]
    for fn in ("lsa_sparse_decode", "lsa_sparse_decode_noalloc"):
        getattr(lib, fn).restype = c_int32
        getattr(lib, fn).argtypes = [POINTER(DecodeArgs), c_void_p]
    if lib.lsa_abi_version() != ABI_VERSION:
        raise ImportError(f"liblsa.so ABI {lib.lsa_abi_version()} != binding ABI {ABI_VERSION}")
    for i, st in enumerate((RefreshArgs, GatherArgs, DecodeArgs, LatentArgs, DenoiseArgs, DeviceGatherArgs)):
        if lib.lsa_struct_size(i) != ctypes.sizeof(st):
            raise ImportError(f"{st.__name__}: binding layout {ctypes.sizeof(st)} B != library {lib.lsa_struct_size(i)} B")
    return lib


LIB = _load()


def _check(status: int) -> None:
    if status != LSA_OK:
        raise LSAError(status, LIB.lsa_last_error().decode(errors="replace"))


def _ptr(x) -> Optional[int]:
    """Address of a torch tensor, NumPy array, int address or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _nbytes(x) -> int:
    return x.numel() * x.element_size()


def _dev(x, name: str, min_bytes: int = 0) -> Optional[int]:
    """Address of a buffer the kernels read or write in device memory: a contiguous CUDA tensor of at
    least min_bytes (or a raw int address, taken as is).  A host buffer here would fault the GPU, so
    it is refused before anything is enqueued."""
    if x is None or isinstance(x, int):
        return x
    if isinstance(x, np.ndarray) or not getattr(x, "is_cuda", False):
        raise TypeError(f"{name} must be a CUDA tensor (device memory), got {type(x).__name__}"
                        + ("" if isinstance(x, np.ndarray) else f" on {getattr(x, 'device', '?')}"))
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if _nbytes(x) < min_bytes:
        raise ValueError(f"{name} holds {_nbytes(x)} bytes, the call needs {min_bytes}")
    return x.data_ptr()


def _pinned_or_dev(x, name: str, min_bytes: int = 0, pinned_only: bool = False) -> Optional[int]:
    """Address of a buffer the kernels may read over the host link: pinned host memory (or, unless
    pinned_only, device memory), contiguous, of at least min_bytes."""
    if x is None or isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        raise TypeError(f"{name} must be a pinned or CUDA torch tensor, got a NumPy array")
    if x.is_cuda:
        if pinned_only:
            raise TypeError(f"{name} must be pinned host memory")
    elif not x.is_pinned():
        raise TypeError(f"{name} is host memory that is not pinned")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if _nbytes(x) < min_bytes:
        raise ValueError(f"{name} holds {_nbytes(x)} bytes, the call needs {min_bytes}")
    return x.data_ptr()


def _elt(dtype) -> int:
    return 2 if _dtype_code(dtype) == LSA_BF16 else 4


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(dtype) -> int:
    """'bf16' / 'f32' names, or an integer code passed through for the library to validate."""
    if isinstance(dtype, (int, np.integer)):
        return int(dtype)
    if dtype == "bf16":
        return LSA_BF16
    if dtype == "f32":
        return LSA_F32
    raise ValueError(f"dtype {dtype!r}")


def _i32(a) -> np.ndarray:
    out = np.ascontiguousarray(a, dtype=np.int32)
    return out


# ------------------------------------------------------------------------------------------
def lsa_block_bytes(dtype, head_dim: int) -> int:
    return int(LIB.lsa_block_bytes(_dtype_code(dtype), int(head_dim)))


def lsa_pack_blocks(dtype, head_dim: int, k_tok, v_tok, pos0: int, n_tokens: int, dst, n_dst_blocks: int,
                    n_threads: int = 0) -> None:
    _check(LIB.lsa_pack_blocks(_dtype_code(dtype), int(head_dim), _ptr(k_tok), _ptr(v_tok), int(pos0),
                               int(n_tokens), _ptr(dst), int(n_dst_blocks), int(n_threads)))


def _refresh_args(*, dtype, d_model, d_idx, n_idx, hidden, hidden_req_stride, hidden_idx_stride, w_q, keys,
                  blk_off, bias, sel_ids, sel_count, masks, workspace, workspace_bytes):
    blk = np.ascontiguousarray(blk_off, dtype=np.int64)
    a = RefreshArgs()
    a.n_req = len(blk) - 1
    a.d_model, a.d_idx, a.n_idx, a.dtype = int(d_model), int(d_idx), int(n_idx), _dtype_code(dtype)
    a.select_level = 0.0
    a.hidden = _ptr(hidden)
    a.hidden_req_stride = int(hidden_req_stride)
    a.hidden_idx_stride = int(hidden_idx_stride)
    a.w_q, a.keys, a.bias = _ptr(w_q), _ptr(keys), _ptr(bias)
    a.blk_off = blk.ctypes.data_as(POINTER(c_int64))
    a.sel_ids, a.sel_count, a.masks = _ptr(sel_ids), _ptr(sel_count), _ptr(masks)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = int(workspace_bytes)
    return a, blk


def lsa_index_refresh_workspace(*, dtype, d_model, d_idx, n_idx, blk_off) -> int:
    a, keep = _refresh_args(dtype=dtype, d_model=d_model, d_idx=d_idx, n_idx=n_idx, hidden=None,
                            hidden_req_stride=d_model, hidden_idx_stride=0, w_q=None, keys=None, blk_off=blk_off,
                            bias=None, sel_ids=None, sel_count=None, masks=None, workspace=None, workspace_bytes=0)
    out = c_size_t(0)
    _check(LIB.lsa_index_refresh_workspace(ctypes.byref(a), ctypes.byref(out)))
    return int(out.value)


def lsa_index_refresh(*, dtype, d_model, d_idx, n_idx, hidden, w_q, keys, blk_off, bias, sel_ids, sel_count,
                      workspace, hidden_req_stride=None, hidden_idx_stride=0, masks=None, ev_begin=None,
                      ev_end=None, table_out=None, table_slot_base=None, stream=None, select_level=0.5,
                      logits=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    blk = np.asarray(blk_off, dtype=np.int64)
    n_req, n_blk, e = len(blk) - 1, int(blk[-1]), _elt(dtype)
    rs = d_model if hidden_req_stride is None else hidden_req_stride
    n_words = int(((blk[1:] - blk[:-1] + 63) // 64).sum())
    _dev(hidden, "hidden", ((n_req - 1) * rs + (n_idx - 1) * hidden_idx_stride + d_model) * e)
    _dev(w_q, "w_q", n_idx * d_model * d_idx * e)
    _dev(keys, "keys", n_idx * n_blk * d_idx * e)
    _dev(bias, "bias", n_req * n_idx * 4)
    _dev(sel_ids, "sel_ids", n_blk * 4)
    _dev(sel_count, "sel_count", n_req * 4)
    _dev(masks, "masks", (n_idx + 1) * n_words * 8)
    _dev(workspace, "workspace")
    _dev(table_out, "table_out", n_blk * 8)
    _dev(logits, "logits", n_idx * n_blk * 4)
    a, keep = _refresh_args(dtype=dtype, d_model=d_model, d_idx=d_idx, n_idx=n_idx, hidden=hidden,
                            hidden_req_stride=d_model if hidden_req_stride is None else hidden_req_stride,
                            hidden_idx_stride=hidden_idx_stride, w_q=w_q, keys=keys, blk_off=blk_off, bias=bias,
                            sel_ids=sel_ids, sel_count=sel_count, masks=masks, workspace=workspace,
                            workspace_bytes=ws_bytes)
    a.ev_begin = ev_begin.cuda_event if ev_begin is not None else None
    a.ev_end = ev_end.cuda_event if ev_end is not None else None
    tsb = _i32(table_slot_base) if table_slot_base is not None else None
    a.table_out, a.table_slot_base = _ptr(table_out), _ptr(tsb)
    a.logits = _ptr(logits)
    a.select_level = float(select_level)
    _check(LIB.lsa_index_refresh(ctypes.byref(a), _stream(stream)))


def _latent_args(*, dtype, d_model, rank, n_idx, n_req, hidden, w_down, latent, hidden_req_stride=None,
                 hidden_idx_stride=0, ev_begin=None, ev_end=None):
    a = LatentArgs()
    a.n_req = int(n_req)
    a.d_model, a.rank, a.n_idx, a.dtype, a.reserved0 = int(d_model), int(rank), int(n_idx), _dtype_code(dtype), 0
    a.hidden = _ptr(hidden)
    a.hidden_req_stride = int(d_model if hidden_req_stride is None else hidden_req_stride)
    a.hidden_idx_stride = int(hidden_idx_stride)
    a.w_down, a.latent = _ptr(w_down), _ptr(latent)
    a.ev_begin = ev_begin.cuda_event if ev_begin is not None else None
    a.ev_end = ev_end.cuda_event if ev_end is not None else None
    return a


def lsa_query_latent(*, dtype, d_model, rank, n_idx, hidden, w_down, latent, n_req=None, hidden_req_stride=None,
                     hidden_idx_stride=0, ev_begin=None, ev_end=None, stream=None) -> None:
    """latent [n_req][n_idx][rank] = A_i h of every request and indexer (A = w_down [n_idx][rank][d_model])."""
    nr, e = (n_req if n_req is not None else hidden.shape[0]), _elt(dtype)
    rs = d_model if hidden_req_stride is None else hidden_req_stride
    _dev(hidden, "hidden", ((nr - 1) * rs + (n_idx - 1) * hidden_idx_stride + d_model) * e)
    _dev(w_down, "w_down", n_idx * rank * d_model * e)
    _dev(latent, "latent", nr * n_idx * rank * e)
    a = _latent_args(dtype=dtype, d_model=d_model, rank=rank, n_idx=n_idx,
                     n_req=n_req if n_req is not None else hidden.shape[0], hidden=hidden, w_down=w_down,
                     latent=latent, hidden_req_stride=hidden_req_stride, hidden_idx_stride=hidden_idx_stride,
                     ev_begin=ev_begin, ev_end=ev_end)
    _check(LIB.lsa_query_latent(ctypes.byref(a), _stream(stream)))


def _denoise_args(*, n_layers, n_blk, top_p, min_votes, logits=None, logit_stride=0, n_blk_dev=None,
                  layer_sets=None, labels=None, n_pos=None, n_naive=None, workspace=None, ev_begin=None,
                  ev_end=None):
    nb = _i32(n_blk)
    a = DenoiseArgs()
    a.n_layers, a.n_windows, a.min_votes, a.reserved0 = int(n_layers), len(nb), int(min_votes), 0
    a.top_p = float(top_p)
    a.logits, a.logit_stride = _ptr(logits), int(logit_stride)
    a.n_blk, a.n_blk_dev = nb.ctypes.data, _ptr(n_blk_dev)
    a.layer_sets, a.labels, a.n_pos, a.n_naive = _ptr(layer_sets), _ptr(labels), _ptr(n_pos), _ptr(n_naive)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    a.ev_begin = ev_begin.cuda_event if ev_begin is not None else None
    a.ev_end = ev_end.cuda_event if ev_end is not None else None
    return a, nb


def lsa_label_denoise_workspace(*, n_layers, n_blk, top_p=0.6, min_votes=3, with_layer_sets=False) -> int:
    a, keep = _denoise_args(n_layers=n_layers, n_blk=n_blk, top_p=top_p, min_votes=min_votes,
                            logit_stride=int(np.max(n_blk)), layer_sets=1 if with_layer_sets else None)
    out = c_size_t(0)
    _check(LIB.lsa_label_denoise_workspace(ctypes.byref(a), ctypes.byref(out)))
    return int(out.value)


def lsa_label_denoise(*, logits, n_blk, n_blk_dev, labels, n_pos, top_p=0.6, min_votes=3, n_naive=None,
                      layer_sets=None, workspace=None, ev_begin=None, ev_end=None, stream=None) -> None:
    """Label denoising of logits [n_layers][n_windows][stride] (fp32 device tensor): per-layer top-p
    sets, then the min_votes vote; labels [n_windows][W] int64 bit words, n_pos / n_naive [n_windows]."""
    n_win = len(np.atleast_1d(n_blk))
    for name, x, need in (("logits", logits, 0), ("n_blk_dev", n_blk_dev, n_win * 4), ("labels", labels, 0),
                          ("n_pos", n_pos, n_win * 4), ("n_naive", n_naive, n_win * 4),
                          ("layer_sets", layer_sets, 0), ("workspace", workspace, 0)):
        _dev(x, name, need)
    a, keep = _denoise_args(n_layers=logits.shape[0], n_blk=n_blk, top_p=top_p, min_votes=min_votes,
                            logits=logits, logit_stride=logits.shape[2], n_blk_dev=n_blk_dev,
                            layer_sets=layer_sets, labels=labels, n_pos=n_pos, n_naive=n_naive,
                            workspace=workspace, ev_begin=ev_begin, ev_end=ev_end)
    _check(LIB.lsa_label_denoise(ctypes.byref(a), _stream(stream)))


def lsa_gather_blocks(*, n_blocks, n_slots_total, block_bytes, cold, hot, new_ids, slot_of_block, free_slots,
                      n_free, capacity, stage, table_dev, stream=None, ev_begin=None, ev_end=None):
    """Returns (n_copied, n_kept).  slot_of_block, free_slots, n_free: int32 NumPy arrays updated in place.
    ev_begin / ev_end (torch.cuda.Event, optional) take the copy kernel's dispatch stamps."""
    ids = _i32(new_ids)
    for name, arr in (("slot_of_block", slot_of_block), ("free_slots", free_slots), ("n_free", n_free)):
        if not (isinstance(arr, np.ndarray) and arr.dtype == np.int32 and arr.flags.c_contiguous):
            raise TypeError(f"{name} must be a C-contiguous int32 NumPy array (updated in place)")
    _pinned_or_dev(cold, "cold", int(n_blocks) * int(block_bytes))
    _dev(hot, "hot", int(n_slots_total) * int(block_bytes))
    _pinned_or_dev(stage, "stage", 4 * 4 * len(ids), pinned_only=True)
    _dev(table_dev, "table_dev", 8 * int(capacity))
    n_copied = np.zeros(1, dtype=np.int32)
    n_kept = np.zeros(1, dtype=np.int32)
    a = GatherArgs()
    a.n_blocks, a.n_slots_total, a.block_bytes = int(n_blocks), int(n_slots_total), int(block_bytes)
    a.cold, a.hot = _ptr(cold), _ptr(hot)
    a.new_ids, a.n_new = _ptr(ids), len(ids)
    a.stage_ints = int(stage.numel()) if stage is not None else 0
    a.slot_of_block, a.free_slots, a.n_free = _ptr(slot_of_block), _ptr(free_slots), _ptr(n_free)
    a.capacity, a.n_layers = int(capacity), 0
    a.stage, a.table_dev = _ptr(stage), _ptr(table_dev)
    a.n_copied, a.n_kept = _ptr(n_copied), _ptr(n_kept)
    a.ev_begin = ev_begin.cuda_event if ev_begin is not None else None
    a.ev_end = ev_end.cuda_event if ev_end is not None else None
    _check(LIB.lsa_gather_blocks(ctypes.byref(a), _stream(stream)))
    return int(n_copied[0]), int(n_kept[0])


def _decode_args(*, dtype, n_heads, head_dim, win_cap, scale, q, k_new, v_new, ring, pool, n_slots_total, table,
                 tbl_off, n_sel, seq_len, window, out, workspace, max_groups, ev_begin, ev_end, n_sel_dev=None):
    host = [_i32(tbl_off), _i32(n_sel), _i32(seq_len), _i32(window)]
    a = DecodeArgs()
    a.n_req = len(host[2])
    a.n_heads, a.head_dim, a.dtype, a.win_cap = int(n_heads), int(head_dim), _dtype_code(dtype), int(win_cap)
    a.scale = float(scale if scale is not None else 1.0 / np.sqrt(head_dim))
    a.q, a.k_new, a.v_new, a.ring, a.pool = _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(ring), _ptr(pool)
    a.n_slots_total, a.reserved0 = int(n_slots_total), 0
    a.table = _ptr(table)
    a.tbl_off, a.n_sel, a.seq_len, a.window = (_ptr(h) for h in host)
    a.out = _ptr(out)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    a.max_groups, a.reserved1 = int(max_groups), 0
    a.ev_attn_begin = ev_begin.cuda_event if ev_begin is not None else None
    a.ev_attn_end = ev_end.cuda_event if ev_end is not None else None
    a.n_sel_dev = _ptr(n_sel_dev)
    return a, host


def lsa_sparse_decode_workspace(*, dtype, n_heads, head_dim, win_cap, n_req, max_groups=0) -> int:
    a, keep = _decode_args(dtype=dtype, n_heads=n_heads, head_dim=head_dim, win_cap=win_cap, scale=None, q=None,
                           k_new=None, v_new=None, ring=None, pool=None, n_slots_total=0, table=None,
                           tbl_off=[0] * n_req, n_sel=[0] * n_req, seq_len=[1] * n_req, window=[1] * n_req,
                           out=None, workspace=None, max_groups=max_groups, ev_begin=None, ev_end=None)
    out = c_size_t(0)
    _check(LIB.lsa_sparse_decode_workspace(ctypes.byref(a), ctypes.byref(out)))
    return int(out.value)


def lsa_sparse_decode(*, dtype, n_heads, head_dim, win_cap, q, ring, out, workspace, tbl_off, n_sel, seq_len,
                      window, pool=None, n_slots_total=0, table=None, k_new=None, v_new=None, scale=None,
                      max_groups=0, ev_attn_begin=None, ev_attn_end=None, n_sel_dev=None, stream=None) -> None:
    R, e = len(np.atleast_1d(seq_len)), _elt(dtype)
    bb = lsa_block_bytes(dtype, head_dim)
    _dev(q, "q", R * n_heads * head_dim * e)
    _dev(k_new, "k_new", R * head_dim * e)
    _dev(v_new, "v_new", R * head_dim * e)
    _dev(ring, "ring", R * (int(win_cap) // BLOCK_TOKENS) * bb)
    _dev(pool, "pool", int(n_slots_total) * bb)
    _dev(table, "table")
    _dev(out, "out", R * n_heads * head_dim * 4)
    _dev(workspace, "workspace")
    _dev(n_sel_dev, "n_sel_dev", R * 4)
    a, keep = _decode_args(dtype=dtype, n_heads=n_heads, head_dim=head_dim, win_cap=win_cap, scale=scale, q=q,
                           k_new=k_new, v_new=v_new, ring=ring, pool=pool, n_slots_total=n_slots_total,
                           table=table, tbl_off=tbl_off, n_sel=n_sel, seq_len=seq_len, window=window, out=out,
                           workspace=workspace, max_groups=max_groups, ev_begin=ev_attn_begin, ev_end=ev_attn_end,
                           n_sel_dev=n_sel_dev)
    _check(LIB.lsa_sparse_decode(ctypes.byref(a), _stream(stream)))


__all__ = [n for n in dir() if n.startswith("lsa_") or n.startswith("LSA_")] + [
    "LSAError", "LIB", "BLOCK_TOKENS", "EXPORTED_SYMBOLS", "RefreshArgs", "GatherArgs", "DecodeArgs", "LatentArgs", "DenoiseArgs",
    "DeviceGatherArgs"]
