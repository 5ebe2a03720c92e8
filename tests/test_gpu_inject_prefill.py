"""Prefill-scale context injection on the GPU: the 256 x 256-tile GEMM kernels
that serve ``dflash_inject_context`` over a whole prompt, against the oracle.

The target's hidden states are extracted during its prefill, then fused and
injected into every drafter layer's K/V ("기술 요약: DFlash", §2.2); long inputs
are a workload of the field notes (§4.3).  At these sizes the launches select:
* Qwen3-8B shape, 2048 positions: the fusion projection on the 128 x 128-tile
  kernel (128 tiles of 256 x 256 are below the big-tile threshold), the K/V
  projections of all 5 layers on the 256 x 256-tile kernel (320 tiles);
* Qwen3-Coder-30B-A3B shape (hidden 2048, 8 layers), 8192 positions: both the
  fusion projection (256 tiles) and the K/V projections on the 256 x 256-tile
  kernel; with the optional RMSNorm after the fusion the projection goes through
  its fp32-output form and the norm kernel;
* exact fp32 ties through the 256 x 256-tile epilogues (one-hot fusion weights,
  identity V projection, hidden 2048, 8192 positions), compared bit for bit with
  torch's CPU round-to-nearest-even.
Injected K/V are compared elementwise with ``oracle.drafter.inject`` within
2e-2 * max(1, |oracle|) on a seeded sample of rows that includes the first and
last rows (a ragged last tile); the oracle is row-independent, so the sample is
the full computation for those rows.
"""
import dataclasses

import numpy as np
import pytest

import dflash_synth as S
from oracle import drafter as D
from oracle.numerics import from_storage

from gpu_cases import assert_close, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BIG_MIN_TILES = 160   # the host's rule: 256 x 256 tiles for M > 128 and at least this many tiles


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_gemm_amd import _lib
    _lib.load()


def big_tiles(M, N, z):
    return ((M + 255) // 256) * ((N // 128 + 1) // 2) * z


def sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(8, n - 8), size=k, replace=False)
    return np.unique(np.concatenate([np.arange(8), mid, np.arange(n - 8, n)]))


def run_prefill(cfg, n_new, seed, fusion_big):
    from block_diffusion_drafter_gemm_amd import runtime as R
    kvd = cfg.n_kv_heads * cfg.head_dim
    assert (big_tiles(n_new, cfg.hidden, 1) >= BIG_MIN_TILES) == fusion_big
    assert big_tiles(n_new, 2 * kvd, cfg.n_layers) >= BIG_MIN_TILES
    log(f"[{cfg.name}] prefill inject of {n_new} positions (ctx_norm={cfg.ctx_norm})")
    w = S.drafter_weights(cfg, seed=seed, random_gain=True)
    lens = np.array([n_new], dtype=np.int32)
    lay = S.paged_layout(cfg, lens, headroom=0, seed=seed)
    feats = S.features(cfg, n_new, seed=seed)
    # positions in a seeded order, so rows scatter over the pages
    pos = np.random.default_rng(seed).permutation(n_new).astype(np.int32)
    seq = np.zeros(n_new, dtype=np.int32)
    dr = R.Drafter(cfg, w, max_batch=1, max_ctx=n_new, max_new=n_new)
    kv = R.PagedKV(cfg, lay.block_table, np.array([0]), lay.n_pages, max_ctx=n_new)
    dr.inject_context(R.to_device(feats), torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), kv)
    torch.cuda.synchronize()
    Kg, Vg = R.to_host_storage(kv.k), R.to_host_storage(kv.v)
    dr.close()
    rows = sample_rows(n_new, 112, seed)
    K_o, V_o = D.inject(w, cfg, feats[rows], pos[rows])
    pages = lay.block_table[0, pos[rows] // cfg.page_size]
    sl = pos[rows] % cfg.page_size
    assert_close(from_storage(Kg[:, pages, sl]), K_o, 2e-2, f"{cfg.name} injected K ({len(rows)} rows)")
    assert_close(from_storage(Vg[:, pages, sl]), V_o, 2e-2, f"{cfg.name} injected V ({len(rows)} rows)")
    # every written slot of the pool is covered (n_new fills whole pages) and nonzero somewhere
    assert np.count_nonzero(Kg.reshape(cfg.n_layers, -1, kvd).any(axis=2)) == cfg.n_layers * n_new


@pytest.mark.timeout(900)
def test_prefill_inject_qwen3_8b_2048_positions():
    cfg = dataclasses.replace(S.get_config("qwen3_8b"), vocab=2048)
    run_prefill(cfg, 2048, seed=21, fusion_big=False)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ctx_norm", [0, 1])
def test_prefill_inject_qwen3_coder_30b_8192_positions(ctx_norm):
    cfg = dataclasses.replace(S.get_config("qwen3_coder_30b"), vocab=2048, ctx_norm=ctx_norm)
    run_prefill(cfg, 8192, seed=22 + ctx_norm, fusion_big=True)


@pytest.mark.timeout(900)
def test_bf16_ties_through_big_tile_inject():
    from block_diffusion_drafter_gemm_amd import runtime as R
    from tie_cases import tie_case
    n_new = 8192
    cfg = S.get_config("tiny", dtype="bf16", hidden=2048, n_q_heads=16, n_kv_heads=16, head_dim=128, ffn=256,
                       n_layers=1, n_feat_layers=2)
    assert big_tiles(n_new, cfg.hidden, 1) >= BIG_MIN_TILES
    assert big_tiles(n_new, 2 * cfg.hidden, 1) >= BIG_MIN_TILES
    log(f"bf16 ties through the 256 x 256-tile inject, {n_new} positions")
    w, feats, expect, n_ties = tie_case(cfg, n_new, seed=31)
    lens = np.array([n_new], dtype=np.int32)
    lay = S.paged_layout(cfg, lens, headroom=0, seed=31)
    pos = np.arange(n_new, dtype=np.int32)
    dr = R.Drafter(cfg, w, max_batch=1, max_ctx=n_new, max_new=n_new)
    kv = R.PagedKV(cfg, lay.block_table, np.array([0]), lay.n_pages, max_ctx=n_new)
    dr.inject_context(R.to_device(feats), torch.zeros(n_new, dtype=torch.int32, device="cuda"),
                      torch.from_numpy(pos).cuda(), kv)
    torch.cuda.synchronize()
    Vg = R.to_host_storage(kv.v)
    dr.close()
    pages = lay.block_table[0, pos // cfg.page_size]
    got = Vg[0, pages, pos % cfg.page_size].reshape(n_new, cfg.hidden)
    bad = int((got != expect).sum())
    log(f"  {bad} of {expect.size} elements differ from round-to-nearest-even ({n_ties} exact ties)")
    assert bad == 0
    rows = sample_rows(n_new, 24, 31)
    _, V_o = D.inject(w, cfg, feats[rows], pos[rows])
    assert np.array_equal(from_storage(got[rows]), V_o[0].reshape(len(rows), cfg.hidden))
