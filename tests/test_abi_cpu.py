"""The C-ABI library on the CPU: it loads, exports every function include/lsa.h declares,
matches the binding's struct layouts, validates arguments before any HIP call, and packs the
block format correctly.  No compute kernel is launched here."""

import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

import lookahead_block_sparse_amd as L

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "lsa.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(lsa_\w+)\s*\(", text, flags=re.M)))


def test_header_functions_are_exported():
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L.LIB, n), f"{n} declared in lsa.h but not exported"
    assert sorted(L.EXPORTED_SYMBOLS) == names


def test_abi_version_and_struct_sizes():
    assert L.LIB.lsa_abi_version() == L.ABI_VERSION
    for i, st in enumerate((L.RefreshArgs, L.GatherArgs, L.DecodeArgs, L.LatentArgs, L.DenoiseArgs,
                            L.DeviceGatherArgs)):
        assert L.LIB.lsa_struct_size(i) == ctypes.sizeof(st)
    assert L.LIB.lsa_struct_size(7) == 0


def test_block_bytes():
    assert L.lsa_block_bytes("bf16", 128) == 2 * 64 * 128 * 2
    assert L.lsa_block_bytes("bf16", 64) == 2 * 64 * 64 * 2
    assert L.lsa_block_bytes("f32", 64) == 2 * 64 * 64 * 4
    assert L.LIB.lsa_block_bytes(1, 96) == 0
    assert L.LIB.lsa_block_bytes(7, 128) == 0


FAKE = 1 << 40  # a non-null address that validation rejects before anything dereferences it


def _refresh_kwargs(**over):
    kw = dict(dtype="bf16", d_model=4096, d_idx=256, n_idx=3, blk_off=[0, 2048])
    kw.update(over)
    return kw


@pytest.mark.parametrize("over,status", [
    (dict(d_idx=192), L.LSA_ERR_UNSUPPORTED),
    (dict(n_idx=5), L.LSA_ERR_UNSUPPORTED),
    (dict(d_model=4000), L.LSA_ERR_UNSUPPORTED),
    (dict(dtype=7), L.LSA_ERR_UNSUPPORTED),
    (dict(blk_off=[0, 0]), L.LSA_ERR_INVALID),
    (dict(blk_off=[1, 10]), L.LSA_ERR_INVALID),
    (dict(blk_off=list(range(0, 66))), L.LSA_ERR_INVALID),
])
def test_refresh_workspace_validation(over, status):
    with pytest.raises(L.LSAError) as e:
        L.lsa_index_refresh_workspace(**_refresh_kwargs(**over))
    assert e.value.status == status
    assert L.LIB.lsa_last_error().decode()


def test_refresh_table_out_validation_before_any_hip_call():
    """The resident block table needs a slot base per request that keeps every slot in int32."""
    a, keep = L._refresh_args(dtype="bf16", d_model=4096, d_idx=256, n_idx=3, hidden=FAKE, hidden_req_stride=4096,
                              hidden_idx_stride=0, w_q=FAKE, keys=FAKE, blk_off=[0, 2048, 4096], bias=FAKE,
                              sel_ids=FAKE, sel_count=FAKE, masks=None, workspace=FAKE, workspace_bytes=16)
    a.table_out = FAKE
    assert L.LIB.lsa_index_refresh(ctypes.byref(a), None) == L.LSA_ERR_INVALID
    assert "table_slot_base" in L.LIB.lsa_last_error().decode()
    base = np.array([0, 2**31 - 2048], dtype=np.int32)   # second request's last slot past int32
    a.table_slot_base = base.ctypes.data
    assert L.LIB.lsa_index_refresh(ctypes.byref(a), None) == L.LSA_ERR_INVALID
    base[1] = 2**31 - 2049                               # fits: only the small workspace is left
    assert L.LIB.lsa_index_refresh(ctypes.byref(a), None) == L.LSA_ERR_WORKSPACE
    a.table_out = FAKE + 4                               # pairs must be 8-byte aligned
    assert L.LIB.lsa_index_refresh(ctypes.byref(a), None) == L.LSA_ERR_INVALID


@pytest.mark.parametrize("over,status", [
    (dict(rank=1000), L.LSA_ERR_UNSUPPORTED),
    (dict(rank=0), L.LSA_ERR_UNSUPPORTED),
    (dict(d_model=4000), L.LSA_ERR_UNSUPPORTED),
    (dict(n_idx=5), L.LSA_ERR_UNSUPPORTED),
    (dict(dtype=7), L.LSA_ERR_UNSUPPORTED),
    (dict(n_req=0), L.LSA_ERR_INVALID),
    (dict(n_req=65), L.LSA_ERR_INVALID),
    (dict(hidden=None), L.LSA_ERR_INVALID),
    (dict(latent=FAKE + 8), L.LSA_ERR_INVALID),
    (dict(hidden_req_stride=100), L.LSA_ERR_INVALID),
    (dict(hidden_idx_stride=-4096), L.LSA_ERR_INVALID),
])
def test_latent_validation_before_any_hip_call(over, status):
    kw = dict(dtype="bf16", d_model=4096, rank=2048, n_idx=3, n_req=4, hidden=FAKE, w_down=FAKE, latent=FAKE,
              hidden_req_stride=4096, hidden_idx_stride=0)
    kw.update(over)
    a = L._latent_args(**kw)
    assert L.LIB.lsa_query_latent(ctypes.byref(a), None) == status
    assert L.LIB.lsa_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(n_layers=0), L.LSA_ERR_INVALID),
    (dict(n_layers=65), L.LSA_ERR_INVALID),
    (dict(min_votes=0), L.LSA_ERR_INVALID),
    (dict(min_votes=22), L.LSA_ERR_INVALID),
    (dict(top_p=0.0), L.LSA_ERR_INVALID),
    (dict(top_p=1.5), L.LSA_ERR_INVALID),
    (dict(n_blk=[100, 0]), L.LSA_ERR_UNSUPPORTED),
    (dict(n_blk=[100, 16385]), L.LSA_ERR_UNSUPPORTED),
    (dict(logit_stride=99), L.LSA_ERR_INVALID),
    (dict(logits=None), L.LSA_ERR_INVALID),
    (dict(labels=FAKE + 4), L.LSA_ERR_INVALID),
    (dict(workspace=None), L.LSA_ERR_WORKSPACE),
])
def test_denoise_validation_before_any_hip_call(over, status):
    kw = dict(n_layers=21, n_blk=[100, 64], top_p=0.6, min_votes=3, logits=FAKE, logit_stride=100,
              n_blk_dev=FAKE, labels=FAKE, n_pos=FAKE)
    kw.update(over)
    a, keep = L._denoise_args(**kw)
    assert L.LIB.lsa_label_denoise(ctypes.byref(a), None) == status
    assert L.LIB.lsa_last_error().decode()


def test_denoise_workspace_size():
    # layer sets (21 layers x windows x ceil(max blocks / 64) words, 256-byte aligned) + one int flag per row
    def al(x):
        return (x + 255) // 256 * 256
    assert L.lsa_label_denoise_workspace(n_layers=21, n_blk=[16384, 100, 5000]) == al(21 * 3 * 256 * 8) + 21 * 3 * 4
    assert L.lsa_label_denoise_workspace(n_layers=21, n_blk=[65, 64]) == al(21 * 2 * 2 * 8) + 21 * 2 * 4
    assert L.lsa_label_denoise_workspace(n_layers=21, n_blk=[65, 64], with_layer_sets=True) == 21 * 2 * 4


def test_refresh_workspace_size():
    n = L.lsa_index_refresh_workspace(**_refresh_kwargs(blk_off=[0, 16384, 32768, 49152, 65536]))
    assert n >= 4 * 3 * 256 * 4 + 1024 * 8 + 16


def test_refresh_rejects_small_workspace_before_any_hip_call():
    a, keep = L._refresh_args(dtype="bf16", d_model=4096, d_idx=256, n_idx=3, hidden=FAKE, hidden_req_stride=4096,
                              hidden_idx_stride=0, w_q=FAKE, keys=FAKE, blk_off=[0, 2048], bias=FAKE, sel_ids=FAKE,
                              sel_count=FAKE, masks=None, workspace=FAKE, workspace_bytes=16)
    st = L.LIB.lsa_index_refresh(ctypes.byref(a), None)
    assert st == L.LSA_ERR_WORKSPACE
    a.workspace = None
    a.workspace_bytes = 1 << 30
    assert L.LIB.lsa_index_refresh(ctypes.byref(a), None) == L.LSA_ERR_WORKSPACE
    a.workspace = FAKE
    a.hidden = None
    assert L.LIB.lsa_index_refresh(ctypes.byref(a), None) == L.LSA_ERR_INVALID


def _gather_args(n_blocks=100, capacity=8, new_ids=(1, 5, 9), slot_of_block=None, n_free=None, stage_ints=64):
    sob = np.full(n_blocks, -1, dtype=np.int32) if slot_of_block is None else slot_of_block
    free = np.arange(capacity, dtype=np.int32)
    nf = np.array([capacity if n_free is None else n_free], dtype=np.int32)
    ids = np.asarray(new_ids, dtype=np.int32)
    outs = np.zeros(2, dtype=np.int32)
    a = L.GatherArgs()
    a.n_blocks, a.n_slots_total, a.block_bytes = n_blocks, capacity, 32768
    a.cold, a.hot = FAKE, FAKE
    a.new_ids, a.n_new = ids.ctypes.data, len(ids)
    a.stage_ints = stage_ints
    a.slot_of_block, a.free_slots, a.n_free = sob.ctypes.data, free.ctypes.data, nf.ctypes.data
    a.capacity, a.n_layers = capacity, 0
    a.stage, a.table_dev = FAKE, FAKE
    a.n_copied, a.n_kept = outs.ctypes.data, outs[1:].ctypes.data
    return a, (sob, free, nf, ids, outs)


def test_gather_capacity_error_leaves_state_untouched():
    a, keep = _gather_args(capacity=2, new_ids=(1, 5, 9))
    sob, free, nf = keep[0].copy(), keep[1].copy(), keep[2].copy()
    assert L.LIB.lsa_gather_blocks(ctypes.byref(a), None) == L.LSA_ERR_CAPACITY
    assert np.array_equal(sob, keep[0]) and np.array_equal(free, keep[1]) and np.array_equal(nf, keep[2])
    assert "exceed" in L.LIB.lsa_last_error().decode()


@pytest.mark.parametrize("case", ["unsorted", "dup", "range", "stage", "state", "badslot"])
def test_gather_validation(case):
    kw = {}
    if case == "unsorted":
        kw = dict(new_ids=(5, 1))
    elif case == "dup":
        kw = dict(new_ids=(5, 5))
    elif case == "range":
        kw = dict(new_ids=(1, 100))
    elif case == "stage":
        kw = dict(stage_ints=4)
    elif case == "state":
        kw = dict(n_free=3)  # 0 resident + 3 free != capacity 8
    elif case == "badslot":
        sob = np.full(100, -1, dtype=np.int32)
        sob[3] = 50
        kw = dict(slot_of_block=sob, n_free=7)
    a, keep = _gather_args(**kw)
    before = [x.copy() for x in keep[:3]]
    assert L.LIB.lsa_gather_blocks(ctypes.byref(a), None) == L.LSA_ERR_INVALID
    for b, x in zip(before, keep[:3]):
        assert np.array_equal(b, x)


@pytest.mark.parametrize("n", [0, 65])
def test_gather_batch_rejects_request_count(n):
    a, keep = _gather_args()
    arr = (L.GatherArgs * 1)(a)
    assert L.LIB.lsa_gather_blocks_batch(arr, n, None) == L.LSA_ERR_INVALID


def test_gather_batch_rejects_shared_state():
    a, keep = _gather_args()
    b, keep_b = _gather_args(new_ids=(2, 3))
    b.slot_of_block = a.slot_of_block
    arr = (L.GatherArgs * 2)(a, b)
    before = [x.copy() for x in keep[:3]]
    assert L.LIB.lsa_gather_blocks_batch(arr, 2, None) == L.LSA_ERR_INVALID
    assert "share" in L.LIB.lsa_last_error().decode()
    for x, y in zip(before, keep[:3]):
        assert np.array_equal(x, y)


def test_gather_batch_stops_at_first_invalid_request():
    a, keep = _gather_args(capacity=2, new_ids=(1, 5, 9))  # overflow
    b, keep_b = _gather_args(new_ids=(2, 3))
    b.stage = FAKE + (1 << 20)  # its own staging buffer
    arr = (L.GatherArgs * 2)(a, b)
    before = [x.copy() for x in keep[:3] + keep_b[:3]]
    assert L.LIB.lsa_gather_blocks_batch(arr, 2, None) == L.LSA_ERR_CAPACITY
    for x, y in zip(before, keep[:3] + keep_b[:3]):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=96), L.LSA_ERR_UNSUPPORTED),
    (dict(n_heads=17), L.LSA_ERR_UNSUPPORTED),
    (dict(win_cap=100), L.LSA_ERR_INVALID),
    (dict(window=[9000]), L.LSA_ERR_INVALID),
    (dict(seq_len=[0]), L.LSA_ERR_INVALID),
    (dict(k_only=True), L.LSA_ERR_INVALID),
    (dict(n_req=65), L.LSA_ERR_INVALID),
])
def test_decode_validation_before_any_hip_call(over, status):
    n_req = over.pop("n_req", 1)
    k_only = over.pop("k_only", False)
    kw = dict(dtype="bf16", n_heads=16, head_dim=128, win_cap=8192, scale=None, q=FAKE, k_new=FAKE if k_only else None,
              v_new=None, ring=FAKE, pool=None, n_slots_total=0, table=None, tbl_off=[0] * n_req, n_sel=[0] * n_req,
              seq_len=[100] * n_req, window=[64] * n_req, out=FAKE, workspace=None, max_groups=0, ev_begin=None,
              ev_end=None)
    kw.update(over)
    a, keep = L._decode_args(**kw)
    a.workspace, a.workspace_bytes = FAKE, 1 << 30
    assert L.LIB.lsa_sparse_decode(ctypes.byref(a), None) == status


@pytest.mark.parametrize("rows", [[0, 0], [2, -1], [1, 3, 1]])
def test_decode_rejects_bad_request_rows_before_any_hip_call(rows):
    """req_rows maps each call request to its row of the device arrays: rows must be distinct and
    non-negative (two requests on one row would write the same ring and output rows)."""
    n = len(rows)
    a, keep = L._decode_args(dtype="bf16", n_heads=16, head_dim=128, win_cap=8192, scale=None, q=FAKE, k_new=None,
                             v_new=None, ring=FAKE, pool=None, n_slots_total=0, table=None, tbl_off=[0] * n,
                             n_sel=[0] * n, seq_len=[100] * n, window=[64] * n, out=FAKE, workspace=None,
                             max_groups=0, ev_begin=None, ev_end=None)
    r = np.ascontiguousarray(rows, dtype=np.int32)
    a.req_rows = r.ctypes.data
    a.workspace, a.workspace_bytes = FAKE, 1 << 30
    assert L.LIB.lsa_sparse_decode(ctypes.byref(a), None) == L.LSA_ERR_INVALID
    assert "req_rows" in L.LIB.lsa_last_error().decode()
    assert L.LIB.lsa_sparse_decode_noalloc(ctypes.byref(a), None) == L.LSA_ERR_INVALID


# ---- block format packing (pure host) ------------------------------------------------------
def _bf16_offsets(D):
    """Element offsets of key (t, d) and value (t, d) inside a bf16 block, [64][D] each, written from
    the format's definition: 16-byte pieces in matrix-core fragment order."""
    t = np.arange(64)[:, None]
    d = np.arange(D)[None, :]
    KS = D // 32
    j = 2 * (t // 32) + (t // 4) % 2
    u = 4 * ((t // 8) % 4) + t % 4
    koff = (((j * KS + d // 32) * 4 + (d // 8) % 4) * 16 + u) * 8 + d % 8
    voff = 64 * D + ((((d // 16) * 2 + t // 32) * 4 + (t // 8) % 4) * 16 + d % 16) * 8 + t % 8
    return koff, voff


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_block_format_is_a_fragment_order_permutation(D):
    """Every element of the block has exactly one (t, d) source, and each 1 KiB run of the key half
    is one matrix-core operand: 16 tokens (one per lane u) x 32 dimensions, 8 consecutive
    dimensions per 16-byte piece."""
    koff, voff = _bf16_offsets(D)
    allo = np.concatenate([koff.ravel(), voff.ravel()])
    assert np.array_equal(np.sort(allo), np.arange(2 * 64 * D))
    run = koff // 512                       # 1 KiB = 512 bf16 elements
    for r in range(64 * D // 512):
        t, d = np.nonzero(run == r)
        assert len(set(t.tolist())) == 16 and len(set(d.tolist())) == 32
        assert np.all((koff[t, d] % 8) == d % 8)


def _ref_pack(k, v, pos0, n_dst):
    """Blocks written out with NumPy as (K [64][D], V [64][D]) per destination block, token p ->
    block (p//64)%n_dst, row p%64."""
    D = k.shape[1]
    out = {}
    for i in range(k.shape[0]):
        p = pos0 + i
        b = (p // 64) % n_dst
        K, V = out.setdefault(b, (np.zeros((64, D), k.dtype), np.zeros((64, D), k.dtype)))
        K[p % 64] = k[i]
        V[p % 64] = v[i]
    return out


@pytest.mark.parametrize("dtype,D,pos0,n,n_dst", [
    ("bf16", 128, 0, 640, 10), ("bf16", 64, 0, 128, 2), ("f32", 64, 0, 256, 4),
    ("bf16", 128, 4096 - 256, 256, 4),   # a window ring: last 256 tokens into 4 blocks
    ("bf16", 128, 130, 256, 4),          # unaligned start wraps into the first block
    ("f32", 128, 7, 200, 5),
])
def test_pack_blocks_matches_numpy(dtype, D, pos0, n, n_dst):
    rng = np.random.default_rng(0)
    st = np.uint16 if dtype == "bf16" else np.float32
    k = (rng.integers(0, 60000, (n, D)) if dtype == "bf16" else rng.standard_normal((n, D))).astype(st)
    v = (rng.integers(0, 60000, (n, D)) if dtype == "bf16" else rng.standard_normal((n, D))).astype(st)
    bb = L.lsa_block_bytes(dtype, D)
    dst = np.zeros(n_dst * bb, dtype=np.uint8)
    L.lsa_pack_blocks(dtype, D, k, v, pos0, n, dst, n_dst, n_threads=3)
    want = _ref_pack(k, v, pos0, n_dst)
    blocks = dst.view(st).reshape(n_dst, 2 * 64 * D)
    for b, (K, V) in want.items():
        if dtype == "bf16":
            koff, voff = _bf16_offsets(D)
            got_k, got_v = blocks[b][koff], blocks[b][voff]
        else:
            got_k = blocks[b, :64 * D].reshape(64, D)
            got_v = blocks[b, 64 * D:].reshape(D, 64).T   # f32: K row-major, then V transposed
        rows = sorted({(pos0 + i) % 64 for i in range(n) if ((pos0 + i) // 64) % n_dst == b})
        assert np.array_equal(got_k[rows], K[rows])
        assert np.array_equal(got_v[rows], V[rows])
        untouched = sorted(set(range(64)) - set(rows))
        assert not got_k[untouched].any() and not got_v[untouched].any()


def test_pack_blocks_rejects_overflow():
    k = np.zeros((200, 64), dtype=np.float32)
    with pytest.raises(L.LSAError) as e:
        L.lsa_pack_blocks("f32", 64, k, k, 0, 200, np.zeros(3 * 32768, np.uint8), 3)
    assert e.value.status == L.LSA_ERR_INVALID


def _dev_gather_args(**over):
    blk = np.array(over.pop("blk_off", [0, 100, 164]), dtype=np.int64)
    slo = np.array(over.pop("slot_off", [0, 50, 80]), dtype=np.int32)
    cold = (ctypes.c_void_p * (len(blk) - 1))(*([FAKE] * (len(blk) - 1)))
    a = L.DeviceGatherArgs()
    a.n_req, a.n_idx, a.block_bytes, a.n_layers = len(blk) - 1, 3, 32768, 1
    a.blk_off, a.slot_off = blk.ctypes.data, slo.ctypes.data
    for f in ("masks", "sel_count", "resident", "slot_of_block", "free_slots", "n_free", "hot", "table",
              "table_count", "copied", "status", "workspace"):
        setattr(a, f, FAKE)
    a.cold = ctypes.cast(cold, ctypes.c_void_p)
    a.workspace_bytes = 1 << 30
    for k, v in over.items():
        setattr(a, k, v)
    return a, (blk, slo, cold)


def test_device_gather_workspace_size():
    a, keep = _dev_gather_args()
    n = ctypes.c_size_t(0)
    assert L.LIB.lsa_gather_plan_device_workspace(ctypes.byref(a), ctypes.byref(n)) == L.LSA_OK
    assert n.value >= 80 * 8 + 65 * 4


@pytest.mark.parametrize("over,status", [
    (dict(n_req=0), L.LSA_ERR_INVALID),
    (dict(n_idx=5), L.LSA_ERR_UNSUPPORTED),
    (dict(block_bytes=1000), L.LSA_ERR_UNSUPPORTED),
    (dict(n_layers=0), L.LSA_ERR_INVALID),
    (dict(blk_off=[0, 0, 64]), L.LSA_ERR_INVALID),
    (dict(slot_off=[1, 50, 80]), L.LSA_ERR_INVALID),
    (dict(resident=None), L.LSA_ERR_INVALID),
    (dict(masks=None), L.LSA_ERR_INVALID),
    (dict(workspace_bytes=16), L.LSA_ERR_WORKSPACE),
    (dict(hot=FAKE + 8), L.LSA_ERR_INVALID),
])
def test_device_gather_validation_before_any_hip_call(over, status):
    a, keep = _dev_gather_args(**over)
    assert L.LIB.lsa_gather_plan_device(ctypes.byref(a), None) == status
    assert L.LIB.lsa_last_error().decode()


# ---- the Python wrappers refuse host buffers where the kernels need device memory ----------------
def _host(n, dtype=None):
    import torch
    return torch.zeros(n, dtype=dtype or torch.uint8)


@pytest.mark.parametrize("name", ["q", "ring", "out", "workspace", "pool", "table", "k_new", "v_new", "n_sel_dev"])
def test_decode_wrapper_refuses_host_buffers(name):
    kw = dict(dtype="bf16", n_heads=16, head_dim=128, win_cap=128, q=FAKE, ring=FAKE, out=FAKE, workspace=FAKE,
              tbl_off=[0], n_sel=[0], seq_len=[10], window=[10])
    kw[name] = _host(1 << 20)
    with pytest.raises(TypeError, match=name):
        L.lsa_sparse_decode(**kw)
    kw[name] = np.zeros(1 << 20, dtype=np.uint8)
    with pytest.raises(TypeError, match=name):
        L.lsa_sparse_decode(**kw)


@pytest.mark.parametrize("name", ["hidden", "w_q", "keys", "bias", "sel_ids", "sel_count", "masks", "workspace",
                                  "table_out"])
def test_refresh_wrapper_refuses_host_buffers(name):
    kw = dict(dtype="bf16", d_model=512, d_idx=128, n_idx=3, hidden=FAKE, w_q=FAKE, keys=FAKE, blk_off=[0, 64],
              bias=FAKE, sel_ids=FAKE, sel_count=FAKE, workspace=None)
    kw[name] = _host(1 << 20)
    with pytest.raises(TypeError, match=name):
        L.lsa_index_refresh(**kw)


@pytest.mark.parametrize("name", ["hidden", "w_down", "latent"])
def test_latent_wrapper_refuses_host_buffers(name):
    kw = dict(dtype="bf16", d_model=512, rank=256, n_idx=3, n_req=1, hidden=FAKE, w_down=FAKE, latent=FAKE)
    kw[name] = _host(1 << 22)
    with pytest.raises(TypeError, match=name):
        L.lsa_query_latent(**kw)


def test_gather_wrapper_wants_pinned_stage_and_cold():
    sob = np.full(64, -1, dtype=np.int32)
    free = np.arange(8, dtype=np.int32)
    nf = np.array([8], dtype=np.int32)
    kw = dict(n_blocks=64, n_slots_total=8, block_bytes=32768, cold=FAKE, hot=FAKE, new_ids=[1, 2],
              slot_of_block=sob, free_slots=free, n_free=nf, capacity=8, stage=FAKE, table_dev=FAKE)
    for name in ("stage", "cold"):
        bad = dict(kw, **{name: _host(64 * 32768)})  # host memory that is not pinned
        with pytest.raises(TypeError, match=name):
            L.lsa_gather_blocks(**bad)
    with pytest.raises(TypeError, match="hot"):
        L.lsa_gather_blocks(**dict(kw, hot=_host(8 * 32768)))
    # nothing changed in the caller's state
    assert (sob == -1).all() and nf[0] == 8


def test_denoise_wrapper_refuses_host_buffers():
    import torch
    kw = dict(logits=torch.zeros((21, 2, 64)), n_blk=[64, 64], n_blk_dev=FAKE, labels=FAKE, n_pos=FAKE,
              workspace=FAKE)
    with pytest.raises(TypeError, match="logits"):
        L.lsa_label_denoise(**kw)


@pytest.mark.parametrize("level,ok", [(0.0, True), (0.5, True), (0.05, True), (0.95, True), (1.0, False),
                                      (-0.2, False), (1.5, False), (float("nan"), False)])
def test_refresh_select_level_validation(level, ok):
    """select_level: 0 (the pages' 0.5) or strictly between 0 and 1; anything else is refused before
    any HIP call."""
    a, keep = L._refresh_args(dtype="bf16", d_model=4096, d_idx=256, n_idx=3, hidden=None, hidden_req_stride=4096,
                              hidden_idx_stride=0, w_q=None, keys=None, blk_off=[0, 2048], bias=None,
                              sel_ids=None, sel_count=None, masks=None, workspace=None, workspace_bytes=0)
    a.select_level = level
    n = ctypes.c_size_t(0)
    st = L.LIB.lsa_index_refresh_workspace(ctypes.byref(a), ctypes.byref(n))
    assert (st == L.LSA_OK) == ok, (level, st)
    if not ok:
        assert st == L.LSA_ERR_INVALID and b"select_level" in L.LIB.lsa_last_error()


def test_refresh_without_ids_needs_masks_and_no_table():
    """sel_ids NULL asks for the bit planes only: the masks must be given and table_out (built from
    the ids) must not; both are refused before any HIP call."""
    a, keep = L._refresh_args(dtype="bf16", d_model=4096, d_idx=256, n_idx=3, hidden=FAKE, hidden_req_stride=4096,
                              hidden_idx_stride=0, w_q=FAKE, keys=FAKE, blk_off=[0, 2048], bias=FAKE, sel_ids=None,
                              sel_count=FAKE, masks=None, workspace=FAKE, workspace_bytes=1 << 30)
    assert L.LIB.lsa_index_refresh(ctypes.byref(a), None) == L.LSA_ERR_INVALID
    assert "masks" in L.LIB.lsa_last_error().decode()
    a.masks = FAKE
    a.table_out = FAKE
    a.table_slot_base = FAKE
    assert L.LIB.lsa_index_refresh(ctypes.byref(a), None) == L.LSA_ERR_INVALID
