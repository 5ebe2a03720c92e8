"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: Qwen3-8B shape (batch 1, context 2048, B=16), LLaMA-3.1-8B
shape (batch 1, context 4096, B=10), Qwen3-8B shape at batch 32 with ragged
contexts 512..8192, and the Qwen3-Coder-30B-A3B shape (8 layers, batch 4,
context 16384).  The oracle recomputes sampled sequences one by one.

Each workload runs in three variants:
* bf16 storage, all layers.  Bar: per-row relative error of the hidden states
  and of the logit vectors <= 5e-2.  The bar is derived on the CPU by
  ``tests/test_bf16_floor.py``: evaluating the same bf16 rounding contract with
  fp32 instead of float64 accumulation already moves the Qwen3-8B-shape hidden
  states by ~2.3% per row after 5 layers (rounding flips cascade through the
  layers); 5e-2 is that floor with a factor ~2 margin.
* fp32 storage of the same shapes, all layers: hidden states elementwise
  within 1e-4 * max(1, |oracle|); the full logit vectors elementwise within
  1e-4 against the oracle's LM head on the GPU's hidden states (identical
  inputs), and per row within 1e-4 against the oracle's own logits (end to
  end, the 4096-term products of hidden states that each sit within 1e-4 land
  up to ~1.1e-4 off elementwise).  Same kernels and indexing as bf16, tight bar.
* bf16 storage, one layer: elementwise <= 2e-2 * max(1, |oracle|).
Token ids must match except on oracle near-ties (2e-2 bf16 / 1e-4 fp32 of
max(1, |logit|)).  Accept lengths and bonus tokens are compared bit for bit on
identical inputs for every sampled sequence: the GPU's accept kernel on the
oracle's own drafts (with the synthetic targets drawn for them) against the
oracle's accept length, whatever the tie excuses.
"""
import dataclasses

import numpy as np
import pytest

import dflash_synth as S
from oracle import drafter as D
from oracle.numerics import from_storage

from gpu_cases import assert_close, assert_rows_close, check_ids, log, oracle_draft, tol_of

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]

_STATE = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    for st in _STATE.values():
        st["dr"].close()
    _STATE.clear()


def variant_cfg(name, dtype, layers):
    cfg = S.get_config(name)
    over = {}
    if dtype != cfg.dtype:
        over["dtype"] = dtype
    if layers is not None:
        over["n_layers"] = layers
    return dataclasses.replace(cfg, **over) if over else cfg


def state(name, dtype, layers):
    """Weights, drafter and synthetic paged cache of a variant (one resident at a time)."""
    from block_diffusion_drafter_gemm_amd import runtime as R
    key = (name, dtype, layers)
    if key in _STATE:
        return _STATE[key]
    for other in list(_STATE):
        _STATE.pop(other)["dr"].close()
    torch.cuda.empty_cache()
    cfg = variant_cfg(name, dtype, layers)
    log(f"[{key}] generating weights")
    w = S.drafter_weights(cfg, seed=0)
    lens = S.ctx_lens(cfg, seed=0)
    lay = S.paged_layout(cfg, lens, headroom=cfg.block_size, seed=0)
    log(f"[{key}] generating context cache ({lay.n_pages} pages)")
    Kp, Vp = S.ctx_kv_cache(cfg, lay, seed=0)
    dr = R.Drafter(cfg, w, max_batch=cfg.batch, max_ctx=int(lens.max()), max_new=256)
    kv = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages, k=Kp, v=Vp)
    _STATE[key] = dict(cfg=cfg, w=w, lens=lens, lay=lay, Kp=Kp, Vp=Vp, dr=dr, kv=kv, R=R)
    return _STATE[key]


SAMPLED = {"qwen3_8b": None, "llama31_8b": None, "qwen3_8b_b32": "minmax", "qwen3_coder_30b": [2]}
VARIANTS = [("qwen3_8b", "bf16", None), ("qwen3_8b", "f32", None), ("qwen3_8b", "bf16", 1),
            ("llama31_8b", "bf16", None), ("llama31_8b", "f32", None),
            ("qwen3_8b_b32", "bf16", None), ("qwen3_8b_b32", "f32", None),
            ("qwen3_coder_30b", "bf16", None), ("qwen3_coder_30b", "f32", None), ("qwen3_coder_30b", "bf16", 1)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,dtype,layers", VARIANTS)
def test_full_draft_step(name, dtype, layers):
    st = state(name, dtype, layers)
    cfg, w, lens, lay, dr, kv = st["cfg"], st["w"], st["lens"], st["lay"], st["dr"], st["kv"]
    b, B = cfg.batch, cfg.block_size
    anchors = S.anchor_ids(cfg, seed=0)
    log(f"[{name} {dtype} layers={cfg.n_layers}] GPU draft step")
    k0 = kv.k[:, :4].clone()
    hid = dr.draft_block(torch.from_numpy(anchors).cuda(), kv)
    ids, mx, lg = dr.lmhead_argmax(hid, want_logits=cfg.dtype == "f32")
    torch.cuda.synchronize()
    d_gpu = ids.cpu().numpy().reshape(b, B - 1)
    y_gpu = S.target_ids_for(cfg, d_gpu, seed=0)
    tau, bonus = dr.accept_len(ids.view(b, B - 1), torch.from_numpy(y_gpu).cuda(), B)
    torch.cuda.synchronize()
    assert torch.equal(kv.k[:, :4], k0)
    tau, bonus = tau.cpu().numpy(), bonus.cpu().numpy()
    hid_h = from_storage(st["R"].to_host_storage(hid)).reshape(b, B - 1, cfg.hidden)
    lg_h = lg.cpu().numpy().reshape(b, B - 1, cfg.vocab) if lg is not None else None
    pick = SAMPLED[name]
    seqs = (list(range(b)) if pick is None else
            [int(np.argmin(lens)), int(np.argmax(lens))] if pick == "minmax" else pick)
    tol = tol_of(cfg)
    d_oracle = d_gpu.copy()
    for s in seqs:
        log(f"  oracle for sequence {s} (context {lens[s]})")
        Z = oracle_draft(cfg, w, anchors[s], st["Kp"], st["Vp"], lay.block_table, s, int(lens[s]))
        ids_o, best_o, logits_o = D.lm_argmax(w["lm_head"], Z)
        if cfg.dtype == "f32":
            assert_close(hid_h[s], Z, 1e-4, f"seq {s} hidden")
            # the LM head on identical inputs (the GPU's hidden states): elementwise
            assert_close(lg_h[s], D.lm_logits(w["lm_head"], hid_h[s]), 1e-4,
                         f"seq {s} logits of the GPU hidden states ({cfg.vocab} per row)")
            # end to end: per row (a 4096-term product of hidden states that
            # are each within 1e-4 lands ~1.1e-4 off elementwise)
            assert_rows_close(lg_h[s], logits_o, 1e-4, f"seq {s} logits")
            assert_close(mx.cpu().numpy().reshape(b, B - 1)[s], best_o, 1e-4, f"seq {s} max logit")
        elif cfg.n_layers == 1:
            assert_close(hid_h[s], Z, 2e-2, f"seq {s} hidden")
            assert_close(mx.cpu().numpy().reshape(b, B - 1)[s], best_o, 2e-2, f"seq {s} max logit")
        else:
            assert_rows_close(hid_h[s], Z, 5e-2, f"seq {s} hidden")
            logits_g = D.lm_logits(w["lm_head"], hid_h[s])   # oracle LM head on the GPU's hidden states
            assert_rows_close(logits_g, logits_o, 5e-2, f"seq {s} logits")
        check_ids(d_gpu[s], ids_o, logits_o, tol, f"seq {s} ids")
        # accept length on identical inputs: the GPU's own drafts ...
        assert (tau[s], bonus[s]) == D.accept_len(d_gpu[s], y_gpu[s])
        d_oracle[s] = ids_o
    # ... and the oracle's drafts with the targets drawn for them, through the
    # GPU accept kernel: bit for bit, excused ids or not
    y_oracle = S.target_ids_for(cfg, d_oracle, seed=0)
    tau_o, bonus_o = dr.accept_len(torch.from_numpy(d_oracle).cuda(), torch.from_numpy(y_oracle).cuda(), B)
    tau_o, bonus_o = tau_o.cpu().numpy(), bonus_o.cpu().numpy()
    for s in seqs:
        want = D.accept_len(d_oracle[s], y_oracle[s])
        log(f"  seq {s}: tau {tau_o[s]} bonus {bonus_o[s]} on the oracle's drafts (oracle {want})")
        assert (tau_o[s], bonus_o[s]) == want
    assert np.all((tau >= 1) & (tau <= B))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,dtype,n_new", [("qwen3_8b", "bf16", 16), ("qwen3_8b", "bf16", 200),
                                              ("qwen3_8b", "f32", 16), ("qwen3_coder_30b", "bf16", 16),
                                              ("llama31_8b", "bf16", 10)])
def test_full_inject(name, dtype, n_new):
    from block_diffusion_drafter_gemm_amd import runtime as R
    st = state(name, dtype, None)
    cfg, w, dr = st["cfg"], st["w"], st["dr"]
    lens = np.full(cfg.batch, 0, dtype=np.int32)
    lay = S.paged_layout(cfg, np.array([n_new] * cfg.batch), headroom=0, seed=1)
    kv = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages)
    pos = np.arange(n_new, dtype=np.int32)
    seq = np.full(n_new, cfg.batch - 1, dtype=np.int32)
    feats = S.features(cfg, n_new, seed=5)
    log(f"[{name} {dtype}] GPU inject n_new={n_new}")
    dr.inject_context(R.to_device(feats), torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), kv)
    torch.cuda.synchronize()
    K_o, V_o = D.inject(w, cfg, feats, pos)
    pages = lay.block_table[seq, pos // 16]
    Kg = from_storage(R.to_host_storage(kv.k)[:, pages, pos % 16])
    Vg = from_storage(R.to_host_storage(kv.v)[:, pages, pos % 16])
    assert_close(Kg, K_o, tol_of(cfg), "K")
    assert_close(Vg, V_o, tol_of(cfg), "V")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("rows", [15, 31])
def test_full_lmhead_identical_input(rows):
    """Full vocabulary on fixed hidden states: 15 rows (one streaming pass) and
    31 rows (two 16-row streaming slices sharing the weight tiles)."""
    st = state("qwen3_8b", "bf16", None)
    cfg, w, dr = st["cfg"], st["w"], st["dr"]
    z = S.normal_matrix(cfg, 88, (rows, cfg.hidden), 1.0, seed=0)
    log(f"[qwen3_8b] GPU LM head on fixed hidden states, {rows} rows")
    h = dr if rows <= 15 else st["R"].Drafter(cfg, dr.w, max_batch=3, max_ctx=16, max_new=1)
    ids, mx, lg = h.lmhead_argmax(st["R"].to_device(z), want_logits=True)
    torch.cuda.synchronize()
    if h is not dr:
        h.close()
    ids_o, best_o, logits_o = D.lm_argmax(w["lm_head"], z)
    assert_close(lg.cpu().numpy(), logits_o, 1e-4, "full-vocab logits")
    # identical inputs: ids may differ only within the fp32 logit bar
    check_ids(ids.cpu().numpy(), ids_o, logits_o, 1e-4, "full-vocab ids")
