"""Target verify (``dflash_target_verify``) in bf16 at the Qwen3-8B layer shape
(hidden 4096, 32 query heads, 8 KV heads of 128, FFN 12288) against the
oracle's causal block pass under the same rounding contract
(``oracle.target.verify_block``).

Three launch paths of the verify:
* 1 sequence x 16 rows: the streaming GEMMs, whose QKV epilogue writes the
  block's K/V into the paged cache itself;
* 2 sequences x 16 rows: the few-rows QKV GEMM, the O projection in 16-row
  slices and the cache append kernel;
* 8 sequences x 32 rows (256 rows, one sequence a prompt prefill at context 0):
  the LDS-tiled GEMMs and the cache append kernel.
Each runs with one and with two decoder layers, and with per-sequence block
sizes B_s < B (rows below B_s against the oracle's pass over the first B_s
tokens).  The cache outside the written rows must be untouched.

Bars (derived on the CPU by ``tests/test_bf16_floor.py::test_bf16_verify_floor_at_qwen3_8b_layer``,
which evaluates the same pass with fp32 accumulation, as the GPU does):
* the first layer's block K/V rows in the cache: elementwise
  |g - o| <= 2e-2 * max(1, |o|) (floor 6e-3);
* the first layer's residual tap and, with one layer, the final hidden states:
  elementwise |g - o| <= 5e-2 * max(1, |o|, RMS of the oracle row) (floor
  1.2e-2) and per-row relative error <= 2e-2 (floor 3.4e-3).  The taps are the
  raw residual stream (row RMS ~2.4 here), and a rounding flip in a row's
  normalised input moves every K/V element of that row, so within one causal
  layer the flips cascade further than in the drafter's pass;
* everything after the first layer (its K/V rows, taps and the final hidden
  states of the two-layer cases): per-row relative error <= 5e-2, the
  multi-layer bar (``tests/test_bf16_floor.py``).
"""
import dataclasses

import numpy as np
import pytest

import dflash_synth as S
from oracle import target as T
from oracle.numerics import from_storage

from gpu_cases import assert_close, assert_rows_close, gather_ctx, log


def assert_row_scaled(got, want, tol, what):
    """|got - want| <= tol * max(1, |want|, RMS of want's row), elementwise."""
    rms = np.sqrt((want ** 2).mean(axis=-1, keepdims=True))
    err = np.abs(got - want) / np.maximum(np.maximum(1.0, np.abs(want)), rms)
    log(f"  {what}: max row-scaled error {err.max():.3e} (tol {tol:g})")
    assert err.max() <= tol, f"{what}: max row-scaled error {err.max():.3e} > {tol:g}"

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BASE = S.get_config("qwen3_8b")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_gemm_amd import _lib
    _lib.load()


def target_cfg(layers, B, batch, ctx_min, ctx_max):
    # a vocabulary of 2048 ids keeps the (unused) heads small; the layers keep the
    # full Qwen3-8B shape
    return dataclasses.replace(BASE, name=f"verify_l{layers}_b{batch}x{B}", cid=120 + layers, vocab=2048,
                               n_layers=layers, n_feat_layers=1, block_size=B, batch=batch, ctx_min=ctx_min,
                               ctx_max=ctx_max)


_W = {}


def weights(layers):
    """Storage weights and their float64 copies (converted once for the oracle)."""
    if layers not in _W:
        _W.clear()
        cfg = target_cfg(layers, 16, 1, 0, 0)
        log(f"generating {layers}-layer target weights")
        w = S.drafter_weights(cfg, seed=3, random_gain=True)
        w64 = {k: ([from_storage(x) for x in v] if isinstance(v, list) else from_storage(v)) for k, v in w.items()}
        _W[layers] = (w, w64)
    return _W[layers]


CASES = [  # (layers, B, lens, block sizes or None)
    (1, 16, [300], None), (2, 16, [1043], None), (1, 16, [77], [9]), (2, 16, [300], [1]),
    (1, 16, [130, 5], None), (2, 16, [64, 401], [16, 6]),
    (1, 32, [0, 17, 250, 33, 96, 5, 160, 64], None), (2, 32, [200, 0, 31, 512, 9, 70, 128, 1], None),
    (1, 32, [40, 3, 90, 0, 120, 15, 66, 240], [32, 1, 7, 32, 20, 2, 31, 16]),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("layers,B,lens,blens", CASES)
def test_target_verify_bf16_qwen3_8b_layers(layers, B, lens, blens):
    lens = np.array(lens, dtype=np.int32)
    cfg = target_cfg(layers, B, len(lens), int(lens.min()), int(lens.max()))
    w, w64 = weights(layers)
    run_verify(cfg, w, w64, lens, blens)


def test_target_verify_bf16_qkv_16_column_tiles():
    """1 sequence x 16 rows at hidden 512 with 16 query and 4 KV heads of 128:
    192 QKV tiles of 16 columns, which the streaming QKV keeps (the Qwen3-8B
    layer's 384 run as 768 8-column tiles), with the epilogue that writes the
    block K/V into the cache; one layer against the oracle, same bars."""
    cfg = dataclasses.replace(BASE, name="verify_q16", cid=130, hidden=512, n_q_heads=16, n_kv_heads=4, ffn=1024,
                              vocab=1024, n_layers=1, n_feat_layers=1, block_size=16, batch=1, ctx_min=200,
                              ctx_max=200)
    w = S.drafter_weights(cfg, seed=5, random_gain=True)
    w64 = {k: ([from_storage(x) for x in v] if isinstance(v, list) else from_storage(v)) for k, v in w.items()}
    run_verify(cfg, w, w64, np.array([200], dtype=np.int32), None)


def run_verify(cfg, w, w64, lens, blens):
    from block_diffusion_drafter_gemm_amd import runtime as R
    layers, B, batch = cfg.n_layers, cfg.block_size, len(lens)
    log(f"[{cfg.name}] bf16 target verify, contexts {lens.tolist()}, block sizes {blens}")
    lay = S.paged_layout(cfg, lens, headroom=B, seed=4)
    Kp, Vp = S.ctx_kv_cache(cfg, lay, seed=4)
    rng = np.random.default_rng(int(lens.sum()) + B)
    ids = rng.integers(0, cfg.vocab, size=(batch, B)).astype(np.int32)
    taps = list(range(layers))
    dr = R.Drafter(cfg, w, max_batch=batch, max_ctx=int(lens.max()), max_new=1)
    kv = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages, k=Kp, v=Vp)
    if blens is not None:
        kv.set_block_len(np.array(blens))
    hid, tp = dr.target_verify(torch.from_numpy(ids).cuda(), kv, taps)
    torch.cuda.synchronize()
    hid_h = from_storage(R.to_host_storage(hid)).reshape(batch, B, cfg.hidden)
    tp_h = from_storage(R.to_host_storage(tp)).reshape(batch, B, layers * cfg.hidden)
    Kg, Vg = R.to_host_storage(kv.k), R.to_host_storage(kv.v)
    written = np.zeros(Kg.shape[:3], dtype=bool)
    H = cfg.hidden
    for s in range(batch):
        p = int(lens[s])
        n = B if blens is None else min(max(int(blens[s]), 1), B)
        Kc, Vc = gather_ctx(cfg, Kp, Vp, lay.block_table, s, p)
        Z, To, Kb, Vb = T.verify_block(w64, cfg, ids[s, :n], Kc, Vc, tap_layers=taps)
        what = f"seq {s} (ctx {p}, {n} rows)"
        pos = np.arange(p, p + B)
        pages, slots = lay.block_table[s, pos // cfg.page_size], pos % cfg.page_size
        written[:, pages, slots] = True
        Kg_s = from_storage(Kg[:, pages[:n], slots[:n]])
        Vg_s = from_storage(Vg[:, pages[:n], slots[:n]])
        # the first layer's outputs
        assert_close(Kg_s[0], Kb[0], 2e-2, f"{what} cache K layer 0")
        assert_close(Vg_s[0], Vb[0], 2e-2, f"{what} cache V layer 0")
        assert_row_scaled(tp_h[s, :n, :H], To[:, :H], 5e-2, f"{what} tap after layer 0")
        assert_rows_close(tp_h[s, :n, :H], To[:, :H], 2e-2, f"{what} tap after layer 0")
        if layers == 1:
            assert_row_scaled(hid_h[s, :n], Z, 5e-2, f"{what} hidden")
            assert_rows_close(hid_h[s, :n], Z, 2e-2, f"{what} hidden")
        else:
            for l in range(1, layers):
                assert_rows_close(Kg_s[l].reshape(n, -1), Kb[l].reshape(n, -1), 5e-2, f"{what} cache K layer {l}")
                assert_rows_close(Vg_s[l].reshape(n, -1), Vb[l].reshape(n, -1), 5e-2, f"{what} cache V layer {l}")
            assert_rows_close(tp_h[s, :n, H:], To[:, H:], 5e-2, f"{what} taps after layers 1..")
            assert_rows_close(hid_h[s, :n], Z, 5e-2, f"{what} hidden")
    # the context rows and every other slot are unchanged
    assert np.array_equal(Kg[~written], Kp[~written]) and np.array_equal(Vg[~written], Vp[~written])
    dr.close()
