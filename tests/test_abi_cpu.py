"""C-ABI checks that need no GPU: the library loads, exports what include/btk.h
declares, and rejects bad arguments on the host before any HIP call.  Every
call here is invalid on purpose, so none of them reaches the HIP runtime."""
import ctypes

import pytest

import block_top_sparse_btk_amd as btk

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: each call below fails validation first


def _problem(**kw):
    base = dict(batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                num_pages=100, max_blocks_per_seq=20, dtype=btk.BTK_BF16, sm_scale=0.0)
    base.update(kw)
    return btk.btk_problem_t(*[base[f] for f, _ in btk.btk_problem_t._fields_])


def test_library_exports_every_declared_symbol():
    lib = btk._lib()
    names = btk.header_symbols()
    assert {"btk_centroid_update", "btk_select", "btk_sparse_attend", "btk_dense_attend",
            "btk_workspace_bytes"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    assert lib.btk_abi_version() == 1


def test_status_strings():
    lib = btk._lib()
    for s in range(6):
        assert lib.btk_status_string(s)
    assert lib.btk_status_string(99) == b"unknown status"


@pytest.mark.parametrize("kw,ok", [
    ({}, True),
    (dict(dtype=btk.BTK_F32, head_dim=64), True),
    (dict(head_dim=96), False),
    (dict(page_size=32), False),
    (dict(num_q_heads=7), False),
    (dict(num_q_heads=34, num_kv_heads=2), False),  # group of 17
    (dict(max_blocks_per_seq=8193), False),
    (dict(dtype=7), False),
    (dict(batch=0), False),
    (dict(num_pages=0), False),
    (dict(sm_scale=float("nan")), False),
])
def test_workspace_bytes_validates_problem(kw, ok):
    n = btk.btk_workspace_bytes(_problem(**kw), 16)
    assert (n > 0) == ok


def test_workspace_bytes_grows_with_problem_and_rejects_bad_top_k():
    small = btk.btk_workspace_bytes(_problem(), 16)
    big = btk.btk_workspace_bytes(_problem(batch=64, max_blocks_per_seq=2048), 16)
    assert big > small > 0
    assert btk.btk_workspace_bytes(_problem(), 0) == 0
    assert btk.btk_workspace_bytes(_problem(), 8193) == 0
    # the region for the scores scratch alone: B*Hkv*max_blocks floats
    assert big >= 64 * 2 * 2048 * 4


def test_null_problem_and_null_pointers():
    lib = btk._lib()
    assert lib.btk_centroid_update(None, FAKE, FAKE, FAKE, None, FAKE, None) == btk.BTK_ERR_NULL
    p = ctypes.byref(_problem())
    assert lib.btk_centroid_update(p, None, FAKE, FAKE, None, FAKE, None) == btk.BTK_ERR_NULL
    assert lib.btk_centroid_update(p, FAKE, FAKE, FAKE, None, None, None) == btk.BTK_ERR_NULL
    assert lib.btk_select(p, None, FAKE, FAKE, FAKE, 4, FAKE, None, FAKE, 1 << 30,
                          None) == btk.BTK_ERR_NULL
    assert lib.btk_select(p, FAKE, FAKE, FAKE, FAKE, 4, None, None, FAKE, 1 << 30,
                          None) == btk.BTK_ERR_NULL
    assert lib.btk_sparse_attend(p, FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, FAKE, None, FAKE,
                                 1 << 30, None) == btk.BTK_ERR_NULL
    assert lib.btk_dense_attend(p, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 30,
                                None) == btk.BTK_ERR_NULL


def test_unsupported_and_shape_errors_come_first():
    lib = btk._lib()
    bad = ctypes.byref(_problem(head_dim=96))
    assert lib.btk_select(bad, FAKE, FAKE, FAKE, FAKE, 4, FAKE, None, FAKE, 1 << 30,
                          None) == btk.BTK_ERR_UNSUPPORTED
    bad = ctypes.byref(_problem(num_q_heads=9))
    assert lib.btk_dense_attend(bad, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30,
                                None) == btk.BTK_ERR_SHAPE
    p = ctypes.byref(_problem())
    assert lib.btk_select(p, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, FAKE, 1 << 30,
                          None) == btk.BTK_ERR_SHAPE
    assert lib.btk_sparse_attend(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -3, FAKE, None, FAKE,
                                 1 << 30, None) == btk.BTK_ERR_SHAPE


def test_workspace_too_small_is_rejected_before_launch():
    lib = btk._lib()
    prob = _problem()
    need = btk.btk_workspace_bytes(prob, 8)
    p = ctypes.byref(prob)
    assert lib.btk_select(p, FAKE, FAKE, FAKE, FAKE, 8, FAKE, None, FAKE, need - 1,
                          None) == btk.BTK_ERR_WORKSPACE
    assert lib.btk_select(p, FAKE, FAKE, FAKE, FAKE, 8, FAKE, None, None, need,
                          None) == btk.BTK_ERR_WORKSPACE
    assert lib.btk_sparse_attend(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, None, FAKE,
                                 need - 1, None) == btk.BTK_ERR_WORKSPACE
    dense_need = btk.btk_workspace_bytes(prob, 1)
    assert lib.btk_dense_attend(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                dense_need - 1, None) == btk.BTK_ERR_WORKSPACE


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 2, 64)
    with pytest.raises(ValueError):
        btk.btk_dense_attend(q, torch.zeros(4, 1, 16, 64), torch.zeros(4, 1, 64, 16),
                             torch.zeros(1, 4, dtype=torch.int32), torch.ones(1, dtype=torch.int32),
                             torch.zeros(10, dtype=torch.uint8))


def test_local_attend_and_decode_step_validate_before_launch():
    lib = btk._lib()
    prob = _problem()
    p = ctypes.byref(prob)
    need = btk.btk_workspace_bytes(prob, 8)
    # local window: nulls, window range, workspace
    assert lib.btk_local_attend(p, FAKE, None, FAKE, FAKE, FAKE, 8, FAKE, None, FAKE, need,
                                None) == btk.BTK_ERR_NULL
    assert lib.btk_local_attend(p, FAKE, FAKE, FAKE, FAKE, FAKE, 8, None, None, FAKE, need,
                                None) == btk.BTK_ERR_NULL
    for w in (0, -1, 8193):
        assert lib.btk_local_attend(p, FAKE, FAKE, FAKE, FAKE, FAKE, w, FAKE, None, FAKE, 1 << 30,
                                    None) == btk.BTK_ERR_SHAPE
    assert lib.btk_local_attend(p, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, None, FAKE, need - 1,
                                None) == btk.BTK_ERR_WORKSPACE
    assert lib.btk_local_attend(None, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, None, FAKE, need,
                                None) == btk.BTK_ERR_NULL
    # single-launch step: nulls (first_pos and lse may be NULL), top_k, workspace, batch limit
    args = lambda **o: [o.get(n, FAKE) for n in ("q", "k", "v", "bt", "sl")] + \
        [o.get("fp", None), o.get("cent", FAKE), o.get("k_", 8), o.get("idx", FAKE),
         o.get("out", FAKE), None, o.get("ws", FAKE), o.get("wsn", need), None]  # noqa: E731
    assert lib.btk_decode_step(p, *args(cent=None)) == btk.BTK_ERR_NULL
    assert lib.btk_decode_step(p, *args(idx=None)) == btk.BTK_ERR_NULL
    assert lib.btk_decode_step(p, *args(v=None)) == btk.BTK_ERR_NULL
    assert lib.btk_decode_step(p, *args(k_=0)) == btk.BTK_ERR_SHAPE
    assert lib.btk_decode_step(p, *args(wsn=need - 1)) == btk.BTK_ERR_WORKSPACE
    assert lib.btk_decode_step(p, *args(ws=None)) == btk.BTK_ERR_WORKSPACE
    big = _problem(batch=65537, max_blocks_per_seq=64)
    assert lib.btk_decode_step(ctypes.byref(big), *args(wsn=1 << 40)) == btk.BTK_ERR_UNSUPPORTED
    bad = ctypes.byref(_problem(head_dim=96))
    assert lib.btk_decode_step(bad, *args()) == btk.BTK_ERR_UNSUPPORTED
    # the step with the fused KV append: the new key and value are required
    app = lambda **o: [o.get(n, FAKE) for n in ("q", "kn", "vn", "k", "v", "bt", "sl", "cent")] + \
        [o.get("k_", 8), o.get("idx", FAKE), o.get("out", FAKE), None, o.get("ws", FAKE),
         o.get("wsn", need), None]  # noqa: E731
    assert lib.btk_decode_step_append(p, *app(kn=None)) == btk.BTK_ERR_NULL
    assert lib.btk_decode_step_append(p, *app(vn=None)) == btk.BTK_ERR_NULL
    assert lib.btk_decode_step_append(p, *app(k=None)) == btk.BTK_ERR_NULL
    assert lib.btk_decode_step_append(p, *app(k_=0)) == btk.BTK_ERR_SHAPE
    assert lib.btk_decode_step_append(p, *app(wsn=need - 1)) == btk.BTK_ERR_WORKSPACE
    assert lib.btk_decode_step_append(ctypes.byref(big), *app(wsn=1 << 40)) == \
        btk.BTK_ERR_UNSUPPORTED
    # the step's 32-bit row counters: batch * Hkv * (max_blocks + 520) must stay below 2^32
    rows_over = _problem(batch=1024, num_q_heads=4096, num_kv_heads=4096, max_blocks_per_seq=512)
    assert lib.btk_decode_step(ctypes.byref(rows_over), *args(wsn=1 << 40)) == \
        btk.BTK_ERR_UNSUPPORTED
    rows_fit = _problem(batch=1024, num_q_heads=2048, num_kv_heads=2048, max_blocks_per_seq=512)
    need_fit = btk.btk_workspace_bytes(rows_fit, 8)
    assert lib.btk_decode_step(ctypes.byref(rows_fit), *args(wsn=need_fit - 1)) == \
        btk.BTK_ERR_WORKSPACE


def test_token_baseline_validates_before_launch():
    lib = btk._lib()
    prob = _problem()
    p = ctypes.byref(prob)
    need = btk.btk_token_workspace_bytes(prob, 64)
    # holds every valid token's score
    assert need >= 4 * prob.batch * prob.num_kv_heads * prob.max_blocks_per_seq * 16
    assert btk.btk_token_workspace_bytes(prob, 0) == 0
    assert btk.btk_token_workspace_bytes(prob, 131073) == 0
    ok = lambda **o: [o.get(n, FAKE) for n in ("q", "k", "v", "bt", "sl")] + \
        [o.get("t", 64), None, o.get("out", FAKE), None, o.get("ws", FAKE), o.get("wsn", need),
         None]  # noqa: E731
    assert lib.btk_token_topk_attend(p, *ok(k=None)) == btk.BTK_ERR_NULL
    assert lib.btk_token_topk_attend(p, *ok(out=None)) == btk.BTK_ERR_NULL
    assert lib.btk_token_topk_attend(p, *ok(t=0)) == btk.BTK_ERR_SHAPE
    assert lib.btk_token_topk_attend(p, *ok(t=131073)) == btk.BTK_ERR_SHAPE
    assert lib.btk_token_topk_attend(p, *ok(wsn=need - 1)) == btk.BTK_ERR_WORKSPACE
    assert lib.btk_token_topk_attend(p, *ok(ws=None)) == btk.BTK_ERR_WORKSPACE
    assert lib.btk_token_topk_attend(None, *ok()) == btk.BTK_ERR_NULL


def test_select_shared_validates_groups_before_launch():
    lib = btk._lib()
    prob = _problem()  # batch 4, max_blocks 20
    p = ctypes.byref(prob)
    need = btk.btk_workspace_bytes(prob, 4)
    I32 = ctypes.c_int32

    def call(starts, blocks, ws=FAKE, wsn=need, k=4):
        gs = (I32 * len(starts))(*starts)
        pb = (I32 * max(1, len(blocks)))(*blocks) if blocks else None
        return lib.btk_select_shared(p, FAKE, FAKE, FAKE, FAKE, len(blocks),
                                     ctypes.cast(gs, ctypes.c_void_p),
                                     ctypes.cast(pb, ctypes.c_void_p) if pb is not None else None,
                                     k, FAKE, None, ws, wsn, None)
    assert call([0, 3], [5], ws=None) == btk.BTK_ERR_WORKSPACE
    assert call([0, 3], [5], wsn=need - 1) == btk.BTK_ERR_WORKSPACE
    assert call([0, 3], [5], k=0) == btk.BTK_ERR_SHAPE
    assert call([0, 3], []) == btk.BTK_ERR_NULL            # no prefix array
    assert call([0, 3, 2], [5, 5]) == btk.BTK_ERR_SHAPE     # not increasing
    assert call([0, 5], [5]) == btk.BTK_ERR_SHAPE           # past the batch
    assert call([-1, 2], [5]) == btk.BTK_ERR_SHAPE
    assert call([0, 2], [21]) == btk.BTK_ERR_SHAPE          # longer than max_blocks
    assert call([0, 2], [-1]) == btk.BTK_ERR_SHAPE
    big = _problem(batch=40, max_blocks_per_seq=8)
    gs = (I32 * 2)(0, 33)
    pb = (I32 * 1)(4)
    assert lib.btk_select_shared(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, 1,
                                 ctypes.cast(gs, ctypes.c_void_p), ctypes.cast(pb, ctypes.c_void_p),
                                 4, FAKE, None, FAKE, 1 << 40, None) == btk.BTK_ERR_UNSUPPORTED


def test_decode_step_noalloc_validates_before_any_hip_call():
    """The allocation-free step: the same argument checks as btk_decode_step, and a
    problem whose scratch exceeds the library's per-GPU array is refused."""
    lib = btk._lib()
    prob = _problem()
    p = ctypes.byref(prob)
    args = lambda **o: [o.get(n, FAKE) for n in ("q", "k", "v", "bt", "sl")] + \
        [o.get("fp", None), o.get("cent", FAKE), o.get("k_", 8), o.get("idx", FAKE),
         o.get("out", FAKE), None, None]  # noqa: E731
    assert lib.btk_decode_step_noalloc(None, *args()) == btk.BTK_ERR_NULL
    for name in ("q", "k", "v", "bt", "sl", "cent", "idx", "out"):
        assert lib.btk_decode_step_noalloc(p, *args(**{name: None})) == btk.BTK_ERR_NULL, name
    assert lib.btk_decode_step_noalloc(p, *args(k_=0)) == btk.BTK_ERR_SHAPE
    assert lib.btk_decode_step_noalloc(p, *args(k_=8193)) == btk.BTK_ERR_SHAPE
    bad = ctypes.byref(_problem(head_dim=96))
    assert lib.btk_decode_step_noalloc(bad, *args()) == btk.BTK_ERR_UNSUPPORTED
    big = _problem(batch=65537, max_blocks_per_seq=64)
    assert lib.btk_decode_step_noalloc(ctypes.byref(big), *args()) == btk.BTK_ERR_UNSUPPORTED
    # more than 16384 units, or scores beyond the 64 MiB array
    units = _problem(batch=1024, num_q_heads=32, num_kv_heads=32, max_blocks_per_seq=16)
    assert lib.btk_decode_step_noalloc(ctypes.byref(units), *args()) == btk.BTK_ERR_WORKSPACE
    scores = _problem(batch=1024, num_q_heads=16, num_kv_heads=8, max_blocks_per_seq=4096)
    assert lib.btk_decode_step_noalloc(ctypes.byref(scores), *args()) == btk.BTK_ERR_WORKSPACE


def test_probe_row_read_validates_on_host():
    lib = btk._lib()
    sink = FAKE
    assert lib.btk_probe_row_read(None, 4096, None, 8, sink, None) == btk.BTK_ERR_NULL
    assert lib.btk_probe_row_read(FAKE, 4096, None, -1, sink, None) == btk.BTK_ERR_SHAPE
    assert lib.btk_probe_row_read(FAKE, 4096, None, 9, sink, None) == btk.BTK_ERR_SHAPE
    assert lib.btk_probe_row_read(FAKE, 4096, None, 0, sink, None) == btk.BTK_OK


def test_check_workspace_names_the_error_bits():
    import torch
    ws = torch.zeros(256, dtype=torch.uint8)
    btk.check_workspace(ws)  # no bits: no error
    ws[:4].view(torch.int32)[0] = 8 | 2
    with pytest.raises(btk.BtkDeviceError) as e:
        btk.check_workspace(ws, "step")
    assert e.value.bits == 10
    assert "wait gave up" in str(e.value) and "page id" in str(e.value)


def test_sketch_calls_validate_on_host():
    lib = btk._lib()
    p = _problem()
    pp = ctypes.byref(p)
    sk = lib.btk_sketch_bytes(pp)
    # B * Hkv * max_blocks rows: 8-byte headers (256-aligned) then head_dim code bytes
    rows = p.batch * p.num_kv_heads * p.max_blocks_per_seq
    assert sk == ((8 * rows + 255) // 256) * 256 + rows * p.head_dim
    assert lib.btk_sketch_bytes(ctypes.byref(_problem(head_dim=96))) == 0
    need = btk.btk_workspace_bytes(p, 8)
    args = lambda **o: [o.get("cent", FAKE), FAKE, FAKE, None, o.get("sk", FAKE), o.get("skn", sk),
                        o.get("ws", FAKE), o.get("wsn", need), None]  # noqa: E731
    assert lib.btk_sketch_update(pp, *args(sk=None)) == btk.BTK_ERR_NULL
    assert lib.btk_sketch_update(pp, *args(cent=None)) == btk.BTK_ERR_NULL
    assert lib.btk_sketch_update(pp, *args(skn=sk - 1)) == btk.BTK_ERR_WORKSPACE
    assert lib.btk_sketch_update(pp, *args(ws=None)) == btk.BTK_ERR_WORKSPACE
    sel = lambda **o: [FAKE, FAKE, o.get("sk", FAKE), o.get("skn", sk), FAKE, FAKE, o.get("k_", 8),
                       FAKE, FAKE, o.get("wsn", need), None]  # noqa: E731
    assert lib.btk_select_sketch(pp, *sel(sk=None)) == btk.BTK_ERR_NULL
    assert lib.btk_select_sketch(pp, *sel(k_=0)) == btk.BTK_ERR_SHAPE
    assert lib.btk_select_sketch(pp, *sel(skn=sk - 1)) == btk.BTK_ERR_WORKSPACE
    assert lib.btk_select_sketch(pp, *sel(wsn=need - 1)) == btk.BTK_ERR_WORKSPACE
    # the step through the sketch: the step's checks, then the sketch's
    need_k = btk.btk_workspace_bytes(p, 64)
    st = lambda **o: [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, o.get("sk", FAKE),
                      o.get("skn", sk), o.get("k_", 64), o.get("idx", FAKE), FAKE, None, None,
                      o.get("ws", FAKE), o.get("wsn", need_k), None]  # noqa: E731
    assert lib.btk_decode_step_sketch(None, *st()) == btk.BTK_ERR_NULL
    assert lib.btk_decode_step_sketch(pp, *st(sk=None)) == btk.BTK_ERR_NULL
    assert lib.btk_decode_step_sketch(pp, *st(idx=None)) == btk.BTK_ERR_NULL
    assert lib.btk_decode_step_sketch(pp, *st(k_=0)) == btk.BTK_ERR_SHAPE
    assert lib.btk_decode_step_sketch(pp, *st(skn=sk - 1)) == btk.BTK_ERR_WORKSPACE
    assert lib.btk_decode_step_sketch(pp, *st(wsn=need_k - 1)) == btk.BTK_ERR_WORKSPACE
    assert lib.btk_decode_step_sketch(pp, *st(ws=None)) == btk.BTK_ERR_WORKSPACE
    # rows beyond the 32-bit counters (batch * Hkv * (max_blocks + 512) >= 2^32)
    big = _problem(batch=65536, num_q_heads=8, num_kv_heads=8, max_blocks_per_seq=8192)
    assert lib.btk_decode_step_sketch(ctypes.byref(big), *st()) == btk.BTK_ERR_UNSUPPORTED
