"""C ABI of libdflash on the CPU: the library loads, exports every entry point
``include/dflash.h`` declares, and rejects bad arguments on the host (no GPU
call is made on any path exercised here)."""
import ctypes
import os
import re

import pytest

from block_diffusion_drafter_gemm_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dflash_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libdflash.so is not built (run __graft_entry__.build())")
    return L.load()


def test_header_declares_the_hot_calls():
    syms = declared_symbols()
    for s in ("dflash_inject_context", "dflash_draft_block", "dflash_lmhead_argmax", "dflash_accept_len"):
        assert s in syms
    assert set(syms) == set(L.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for s in declared_symbols():
        assert hasattr(lib, s), s
    out = os.popen(f"nm -D --defined-only {L.LIB_PATH}").read()
    for s in declared_symbols():
        assert re.search(rf"\bT {s}\b", out), s


def test_status_strings(lib):
    assert L.status_str(0) == "ok"
    assert "workspace" in L.status_str(-5)
    assert L.status_str(12345) == "unknown status"


FAKE = 0x10000  # never dereferenced: validation fails or the call stops before any launch


def good_config(**kw):
    c = dict(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512, vocab=1024, n_layers=2,
             n_feat_layers=3, block_size=4, mask_token_id=1023, dtype="bf16", rope_theta=1e6, rms_eps=1e-6)
    c.update(kw)
    return L.make_config(**c)


def fake_weights(n_layers=2):
    arr = (ctypes.c_void_p * n_layers)(*([FAKE] * n_layers))
    pp = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    return L.DflashWeights(FAKE, FAKE, FAKE, FAKE, pp, pp, pp, pp, pp, pp), arr


def create(cfg):
    w, keep = fake_weights(cfg.n_layers)
    h = ctypes.c_void_p()
    st = L.load().dflash_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h))
    return st, h.value


@pytest.mark.parametrize("bad,code", [
    (dict(head_dim=96), -2), (dict(n_q_heads=5), -2), (dict(hidden=100), -2), (dict(hidden=16384 + 64), -2),
    (dict(ffn=100), -2),
    (dict(vocab=1000 + 3), -2), (dict(block_size=1), -2), (dict(block_size=65), -2), (dict(n_layers=0), -2),
    (dict(n_layers=65), -2), (dict(mask_token_id=1024), -4), (dict(dtype="bf16", rope_theta=0.0), -4),
    (dict(n_q_heads=32, n_kv_heads=1, block_size=16), -2), (dict(window=-1), -4), (dict(ctx_norm=2), -4),
    (dict(ctx_norm=1), -1),   # the RMSNorm gain is missing
])
def test_create_rejects_bad_config(lib, bad, code):
    st, h = create(good_config(**bad))
    assert st == code and not h


def test_create_rejects_bad_dtype(lib):
    cfg = good_config()
    cfg.dtype = 7
    assert create(cfg)[0] == -3


def test_create_rejects_null(lib):
    h = ctypes.c_void_p()
    assert lib.dflash_create(None, None, ctypes.byref(h)) == -1
    cfg = good_config()
    w, keep = fake_weights()
    w.embed = None
    assert lib.dflash_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)) == -1


def test_target_handle_without_fusion_weights(lib):
    # a target decoder has no fusion projection: creation accepts it, inject refuses
    cfg = good_config()
    w, keep = fake_weights()
    w.w_fc = None
    h = ctypes.c_void_p()
    assert lib.dflash_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)) == 0 and h.value
    try:
        kv = L.DflashKV(FAKE, FAKE, FAKE, FAKE, 1, 8, 8, 64)
        n1 = L.dflash_workspace_size(h.value, 1, 64, 16)
        assert lib.dflash_inject_context(h.value, FAKE, FAKE, FAKE, 4, ctypes.byref(kv), FAKE, n1, None) == -1
    finally:
        assert lib.dflash_destroy(h.value) == 0


def test_target_verify_host_validation(lib):
    st, h = create(good_config())
    assert st == 0 and h
    try:
        n1 = L.dflash_workspace_size(h, 1, 64, 16)
        kv = L.DflashKV(FAKE, FAKE, FAKE, FAKE, 1, 8, 8, 64)
        taps = (ctypes.c_int32 * 2)(0, 1)
        bad_taps = (ctypes.c_int32 * 2)(0, 2)        # layer 2 of a 2-layer decoder
        tv = lib.dflash_target_verify
        assert tv(h, None, ctypes.byref(kv), taps, 2, FAKE, FAKE, FAKE, n1, None) == -1
        assert tv(h, FAKE, ctypes.byref(kv), taps, 2, None, FAKE, FAKE, n1, None) == -1
        assert tv(h, FAKE, ctypes.byref(kv), None, 2, FAKE, FAKE, FAKE, n1, None) == -1
        assert tv(h, FAKE, ctypes.byref(kv), taps, -1, FAKE, FAKE, FAKE, n1, None) == -2
        assert tv(h, FAKE, ctypes.byref(kv), taps, 65, FAKE, FAKE, FAKE, n1, None) == -2
        assert tv(h, FAKE, ctypes.byref(kv), bad_taps, 2, FAKE, FAKE, FAKE, n1, None) == -4
        assert tv(h, FAKE, ctypes.byref(kv), taps, 2, FAKE, FAKE, FAKE, 1024, None) == -5
        bad = L.DflashKV(FAKE, FAKE, FAKE, FAKE, 0, 8, 8, 64)
        assert tv(h, FAKE, ctypes.byref(bad), taps, 2, FAKE, FAKE, FAKE, n1, None) == -2
    finally:
        assert lib.dflash_destroy(h) == 0


def test_launch_shapes_are_checked_before_anything_is_enqueued(lib):
    """A call whose GEMM grid would not fit (fp32 handle: the few-rows kernel puts
    row groups x weight slices in grid.y, at most 65535) returns
    DFLASH_ERR_SHAPE before its first launch.  On this host any launch would
    fail with DFLASH_ERR_HIP, so the shape error also shows nothing was
    enqueued first (draft: the embedding kernel; inject: the fusion GEMM, whose
    row groups alone still fit)."""
    cfg = good_config(dtype="f32", block_size=16)
    st, h = create(cfg)
    assert st == 0 and h
    huge = 1 << 62          # workspace size large enough for any of these calls
    try:
        rows = 64 * 65535 + 1
        kv = L.DflashKV(FAKE, FAKE, FAKE, FAKE, (rows + 15) // 16, 8, 8, 64)
        assert lib.dflash_draft_block(h, FAKE, ctypes.byref(kv), FAKE, FAKE, huge, None) == -2
        assert lib.dflash_target_verify(h, FAKE, ctypes.byref(kv), None, 0, None, FAKE, FAKE, huge, None) == -2
        kv1 = L.DflashKV(FAKE, FAKE, FAKE, FAKE, 1, 8, 8, 64)
        n_new = 64 * 40000      # 40000 row groups: the fusion fits, 2 layers of K/V do not
        assert lib.dflash_inject_context(h, FAKE, FAKE, FAKE, n_new, ctypes.byref(kv1), FAKE, huge, None) == -2
    finally:
        assert lib.dflash_destroy(h) == 0


def test_stage_events_host_validation(lib):
    """The measurement hook stores event handles only (no HIP call): NULL turns
    it off; the count must be 2 * stages * layers; entries must not be NULL."""
    st, h = create(good_config())
    assert st == 0 and h
    try:
        n = 2 * len(L.STAGES) * 2
        ev = (ctypes.c_void_p * n)(*([FAKE] * n))
        se = lib.dflash_set_stage_events
        assert se(None, ev, n) == -1
        assert se(h, ev, n - 2) == -2
        assert se(h, ev, n) == 0
        assert se(h, None, 0) == 0
        ev[3] = None
        assert se(h, ev, n) == -1
    finally:
        assert lib.dflash_destroy(h) == 0


def test_check_inputs_host_validation(lib):
    st, h = create(good_config())
    assert st == 0 and h
    try:
        kv = L.DflashKV(FAKE, FAKE, FAKE, FAKE, 1, 8, 8, 64)
        f = lib.dflash_check_inputs
        assert f(None, ctypes.byref(kv), None, None, 0, None, None, 0, FAKE, None) == -1
        assert f(h, None, None, None, 0, None, None, 0, FAKE, None) == -1
        assert f(h, ctypes.byref(kv), None, None, 0, None, None, 0, None, None) == -1
        assert f(h, ctypes.byref(kv), None, None, -1, None, None, 0, FAKE, None) == -2
        assert f(h, ctypes.byref(kv), None, None, 0, None, None, -1, FAKE, None) == -2
        assert f(h, ctypes.byref(kv), None, None, 3, None, None, 0, FAKE, None) == -1
        assert f(h, ctypes.byref(kv), None, None, 0, FAKE, None, 2, FAKE, None) == -1
        bad = L.DflashKV(FAKE, FAKE, FAKE, FAKE, 0, 8, 8, 64)
        assert f(h, ctypes.byref(bad), None, None, 0, None, None, 0, FAKE, None) == -2
    finally:
        assert lib.dflash_destroy(h) == 0


def test_kv_cache_must_be_16_byte_aligned(lib):
    """Cache rows are read and written in 16-byte pieces: a K or V base that is
    not 16-byte aligned is refused (DFLASH_ERR_RANGE) before anything runs."""
    st, h = create(good_config())
    assert st == 0 and h
    try:
        n1 = L.dflash_workspace_size(h, 1, 64, 16)
        for k, v in ((FAKE + 8, FAKE), (FAKE, FAKE + 2)):
            kv = L.DflashKV(k, v, FAKE, FAKE, 1, 8, 8, 64)
            assert lib.dflash_inject_context(h, FAKE, FAKE, FAKE, 4, ctypes.byref(kv), FAKE, n1, None) == -4
            assert lib.dflash_draft_block(h, FAKE, ctypes.byref(kv), FAKE, FAKE, n1, None) == -4
            assert lib.dflash_check_inputs(h, ctypes.byref(kv), None, None, 0, None, None, 0, FAKE, None) == -4
    finally:
        assert lib.dflash_destroy(h) == 0


def test_workspace_size_and_host_validation(lib):
    st, h = create(good_config())
    assert st == 0 and h
    try:
        n1 = L.dflash_workspace_size(h, 1, 64, 16)
        n2 = L.dflash_workspace_size(h, 8, 4096, 256)
        assert 0 < n1 < n2
        with pytest.raises(L.DflashError) as e:
            L.dflash_workspace_size(h, 0, 64, 16)
        assert e.value.status == -2
        kv = L.DflashKV(FAKE, FAKE, FAKE, FAKE, 1, 8, 8, 64)
        # null anchor / workspace: rejected before any launch
        assert lib.dflash_draft_block(h, None, ctypes.byref(kv), FAKE, FAKE, n1, None) == -1
        assert lib.dflash_draft_block(h, FAKE, None, FAKE, FAKE, n1, None) == -1
        # workspace too small
        assert lib.dflash_draft_block(h, FAKE, ctypes.byref(kv), FAKE, FAKE, 1024, None) == -5
        assert lib.dflash_lmhead_argmax(h, FAKE, 3, FAKE, None, None, FAKE, 1024, None) == -5
        assert lib.dflash_inject_context(h, FAKE, FAKE, FAKE, 16, ctypes.byref(kv), FAKE, 1024, None) == -5
        # empty work is a no-op
        assert lib.dflash_lmhead_argmax(h, None, 0, None, None, None, None, 0, None) == 0
        assert lib.dflash_inject_context(h, None, None, None, 0, ctypes.byref(kv), None, 0, None) == 0
        # bad cache descriptors
        bad = L.DflashKV(FAKE, FAKE, FAKE, FAKE, 0, 8, 8, 64)
        assert lib.dflash_draft_block(h, FAKE, ctypes.byref(bad), FAKE, FAKE, n1, None) == -2
        nul = L.DflashKV(FAKE, None, FAKE, FAKE, 1, 8, 8, 64)
        assert lib.dflash_draft_block(h, FAKE, ctypes.byref(nul), FAKE, FAKE, n1, None) == -1
        assert lib.dflash_lmhead_argmax(h, FAKE, -1, FAKE, None, None, FAKE, n1, None) == -2
        assert lib.dflash_workspace_init(h, FAKE, 16, None) == -5
    finally:
        assert lib.dflash_destroy(h) == 0
    assert lib.dflash_destroy(None) == -1


def test_accept_len_host_validation(lib):
    assert lib.dflash_accept_len(FAKE, FAKE, 4, 1, FAKE, FAKE, None) == -2
    assert lib.dflash_accept_len(FAKE, FAKE, 4, 65, FAKE, FAKE, None) == -2
    assert lib.dflash_accept_len(None, FAKE, 4, 16, FAKE, FAKE, None) == -1
    assert lib.dflash_accept_len(FAKE, FAKE, -1, 16, FAKE, FAKE, None) == -2
    assert lib.dflash_accept_len(None, None, 0, 16, None, None, None) == 0


def test_accept_len_ragged_host_validation(lib):
    f = lib.dflash_accept_len_ragged
    assert f(FAKE, FAKE, 4, 1, FAKE, FAKE, FAKE, None) == -2
    assert f(FAKE, FAKE, 4, 65, None, FAKE, FAKE, None) == -2
    assert f(None, FAKE, 4, 16, FAKE, FAKE, FAKE, None) == -1
    assert f(FAKE, FAKE, 4, 16, FAKE, None, FAKE, None) == -1
    assert f(FAKE, FAKE, -1, 16, FAKE, FAKE, FAKE, None) == -2
    assert f(None, None, 0, 16, None, None, None, None) == 0


def test_sample_host_validation(lib):
    import ctypes
    n = ctypes.c_size_t(0)
    assert lib.dflash_sample_workspace_size(3, 4097, ctypes.byref(n)) == 0 and n.value == 3 * 5 * 16
    assert lib.dflash_sample_workspace_size(-1, 10, ctypes.byref(n)) == -2
    assert lib.dflash_sample_workspace_size(1, 0, ctypes.byref(n)) == -2
    assert lib.dflash_sample_workspace_size(1, 10, None) == -1
    f = lib.dflash_sample
    for T in (0.0, -1.0, float("nan"), float("inf"), 1e-45):
        assert f(FAKE, 4, 10, T, 1, 0, 0, FAKE, None, FAKE, 1 << 20, None) == -4, T
    assert f(FAKE, 4, 10, 1.0, 1, 0, 0xFFFFFFFE, FAKE, None, FAKE, 1 << 20, None) == -4
    assert f(FAKE, 4, 10, 1.0, 1, 0, 0xFFFFFFFF, FAKE, None, FAKE, 1 << 20, None) == -4
    assert f(FAKE, -1, 10, 1.0, 1, 0, 0, FAKE, None, FAKE, 1 << 20, None) == -2
    assert f(FAKE, 4, 0, 1.0, 1, 0, 0, FAKE, None, FAKE, 1 << 20, None) == -2
    assert f(None, 0, 10, 1.0, 1, 0, 0, None, None, None, 0, None) == 0
    assert f(None, 4, 10, 1.0, 1, 0, 0, FAKE, None, FAKE, 1 << 20, None) == -1
    assert f(FAKE, 4, 10, 1.0, 1, 0, 0, None, None, FAKE, 1 << 20, None) == -1
    assert f(FAKE, 4, 10, 1.0, 1, 0, 0, FAKE, None, FAKE, 4 * 16 - 1, None) == -5


def test_accept_sample_host_validation(lib):
    f = lib.dflash_accept_sample
    args = lambda **k: [k.get("dz", FAKE), FAKE, FAKE, FAKE, FAKE, FAKE, k.get("batch", 4), k.get("B", 16), None,
                        k.get("V", 100), k.get("T", 1.0), 9, 0, FAKE, k.get("bonus", FAKE), FAKE,
                        k.get("ws", 1 << 20), None]
    assert f(*args(B=1)) == -2
    assert f(*args(B=65)) == -2
    assert f(*args(batch=-1)) == -2
    assert f(*args(V=0)) == -2
    assert f(*args(T=0.0)) == -4
    assert f(*args(T=float("nan"))) == -4
    assert f(*args(dz=None)) == -1
    assert f(*args(bonus=None)) == -1
    assert f(*args(ws=4 * 16 - 1)) == -5
    assert f(*args(batch=0, dz=None)) == 0


def test_stream_read_validation(lib):
    # host-side checks only: nothing is launched on these paths
    assert lib.dflash_stream_read(None, 16, FAKE, None) == -1
    assert lib.dflash_stream_read(FAKE, 16, None, None) == -1
    assert lib.dflash_stream_read(FAKE, 24, FAKE, None) == -2      # not a multiple of 16
    assert lib.dflash_stream_read(FAKE + 8, 16, FAKE, None) == -2  # misaligned
    assert lib.dflash_stream_read(FAKE, 0, FAKE, None) == 0        # empty: no-op
