"""Where the bf16 tolerance of the multi-layer GPU parity tests comes from (CPU).

The drafter's rounding contract fixes where values are rounded to bf16, not the
order in which a GEMM accumulates.  Two correct evaluations of the contract --
the oracle (float64 accumulation) and one that accumulates in fp32, as the GPU
does -- already differ: a product that lands near a bf16 rounding boundary
rounds one way in one and the other way in the other, and every such flip
shifts later rounding decisions, layer after layer.  This test measures that
floor at the Qwen3-8B shape (hidden 4096, FFN 12288, 32/8 heads, context 2048,
B = 16) with the seeded inputs of the benchmark and asserts:

* one layer: elementwise within 1e-2 * max(1, |oracle|), half the one-layer bar
  2e-2 the GPU tests use;
* five layers: a per-row relative error of the hidden states above 1.5e-2
  (measured 2.17e-2 here, 8.4e-2 elementwise: a 2e-2 bar would leave an
  fp32-exact implementation of the contract no margin) and within 2.5e-2, half
  the multi-layer bar 5e-2 the GPU tests use; the logit rows (a 16384-id slice
  of the vocabulary through the shared LM head) likewise.

The target's causal verify pass (``oracle.target.verify_block``) over a block of
random tokens at the same layer shape cascades further inside one layer: its
residual-stream taps have a row RMS of ~2.4, and a flip in a row's normalised
input moves every K/V element of the row.  ``test_bf16_verify_floor_at_qwen3_8b_layer``
measures one layer at contexts 17, 77 and 300 and asserts that the floor stays
within half the bars ``tests/test_gpu_target_bf16.py`` uses: the layer's own
cache K/V rows elementwise (2e-2 * max(1, |oracle|)), the taps and final hidden
states elementwise against max(1, |oracle|, RMS of the oracle row) (5e-2) and
per row (2e-2).
"""
import dataclasses

import numpy as np
import pytest

import dflash_synth as S
from oracle import drafter as D
from oracle.numerics import from_storage, round_bf16

F32 = np.float32


def _st(x):
    """bf16 storage rounding of fp32 values (exact in fp32 afterwards)."""
    return round_bf16(np.asarray(x, dtype=np.float64)).astype(F32)


def _rms(x, g, eps):
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=F32)
    return x / np.sqrt(ms + F32(eps)) * g


def _rope(x, pos, theta):
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang).astype(F32)[:, None, :], np.sin(ang).astype(F32)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def draft_block_fp32_acc(w, cfg, anchor, Kc, Vc, n_layers):
    """The oracle's drafter pass with every product accumulated in fp32 (numpy
    float32 BLAS and reductions) and the same bf16 rounding points."""
    B, nq, nkv, d, Fw = cfg.block_size, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn
    p = Kc.shape[1]
    pos = np.arange(p, p + B)
    X = from_storage(w["embed_rows"]).astype(F32)
    for l in range(n_layers):
        W = lambda k: from_storage(w[k][l]).astype(F32)
        Y = _st(_rms(X, W("attn_norm"), cfg.rms_eps))
        qkv = Y @ W("w_qkv").T
        q = _st(_rope(qkv[:, :nq * d].reshape(B, nq, d), pos, cfg.rope_theta))
        k = _st(_rope(qkv[:, nq * d:(nq + nkv) * d].reshape(B, nkv, d), pos, cfg.rope_theta))
        v = _st(qkv[:, (nq + nkv) * d:].reshape(B, nkv, d))
        K = np.concatenate([Kc[l].astype(F32), k])
        V = np.concatenate([Vc[l].astype(F32), v])
        O = np.empty((B, nq, d), dtype=F32)
        for h in range(nq):
            g = h // (nq // nkv)
            sc = (q[:, h] @ K[:, g].T) / F32(np.sqrt(d))
            e = np.exp(sc - sc.max(axis=1, keepdims=True))
            O[:, h] = (e / e.sum(axis=1, keepdims=True, dtype=F32)) @ V[:, g]
        X = X + _st(O).reshape(B, nq * d) @ W("w_o").T
        Y = _st(_rms(X, W("mlp_norm"), cfg.rms_eps))
        gu = Y @ W("w_gate_up").T
        hm = _st(gu[:, :Fw] / (F32(1) + np.exp(-gu[:, :Fw])) * gu[:, Fw:])
        X = X + hm @ W("w_down").T
    return _st(_rms(X[1:], from_storage(w["final_norm"]).astype(F32), cfg.rms_eps)).astype(np.float64)


def _row_rel(a, b):
    return float((np.linalg.norm(a - b, axis=1) / np.linalg.norm(b, axis=1)).max())


@pytest.fixture(scope="module")
def qwen3_inputs():
    cfg = S.get_config("qwen3_8b")
    w = S.drafter_weights(cfg, seed=0, include_heads=False)
    anchor = int(S.anchor_ids(cfg, seed=0)[0])
    # only the anchor and mask rows of the shared embedding are read
    ids = [anchor, cfg.mask_token_id]
    rows = [S.normal_matrix(cfg, S.TAG_EMBED, (cfg.vocab, cfg.hidden), 0.02, seed=0, row_range=(i, i + 1))[0]
            for i in ids]
    w["embed"] = {anchor: rows[0], cfg.mask_token_id: rows[1]}
    w["embed_rows"] = np.stack([rows[0]] + [rows[1]] * (cfg.block_size - 1))
    lens = S.ctx_lens(cfg, seed=0)
    lay = S.paged_layout(cfg, lens, headroom=cfg.block_size, seed=0)
    Kp, Vp = S.ctx_kv_cache(cfg, lay, seed=0)
    t = np.arange(int(lens[0]))
    Kc = from_storage(Kp[:, lay.block_table[0, t // 16], t % 16])
    Vc = from_storage(Vp[:, lay.block_table[0, t // 16], t % 16])
    lm = S.normal_matrix(cfg, S.TAG_LM_HEAD, (cfg.vocab, cfg.hidden), 0.02, seed=0, row_range=(0, 16384))
    return cfg, w, anchor, Kc, Vc, lm


class _Embed:
    """The two embedding rows the pass reads, indexed like the full table."""

    def __init__(self, rows):
        self.rows = rows

    def __getitem__(self, ids):
        return np.stack([self.rows[int(i)] for i in np.atleast_1d(ids)])


def _oracle(cfg, w, anchor, Kc, Vc, layers):
    c = dataclasses.replace(cfg, n_layers=layers)
    ww = dict(w)
    ww["embed"] = _Embed(w["embed"])
    return D.draft_block(ww, c, anchor, Kc[:layers], Vc[:layers])


@pytest.mark.timeout(900)
def test_bf16_contract_floor_at_qwen3_8b_shape(qwen3_inputs):
    cfg, w, anchor, Kc, Vc, lm = qwen3_inputs
    # one layer: elementwise
    z1 = _oracle(cfg, w, anchor, Kc, Vc, 1)
    g1 = draft_block_fp32_acc(w, cfg, anchor, Kc, Vc, 1)
    el1 = float((np.abs(g1 - z1) / np.maximum(1.0, np.abs(z1))).max())
    # five layers: per row
    z5 = _oracle(cfg, w, anchor, Kc, Vc, 5)
    g5 = draft_block_fp32_acc(w, cfg, anchor, Kc, Vc, 5)
    rows5 = _row_rel(g5, z5)
    el5 = float((np.abs(g5 - z5) / np.maximum(1.0, np.abs(z5))).max())
    W = from_storage(lm)
    lg5 = _row_rel(g5 @ W.T, z5 @ W.T)
    print(f"fp32-accumulation floor: 1 layer elementwise {el1:.3e}; 5 layers per row {rows5:.3e} "
          f"(elementwise {el5:.3e}), logits per row {lg5:.3e}")
    assert el1 <= 1e-2
    assert 1.5e-2 < rows5 <= 2.5e-2
    assert lg5 <= 2.5e-2


def verify_block_fp32_acc(w, cfg, ids, Kc, Vc):
    """The oracle's causal verify pass (one layer per ``cfg.n_layers``) with every
    product accumulated in fp32 and the same bf16 rounding points; returns the
    final hidden states, the tap after every layer and the block K/V."""
    n, p = len(ids), Kc.shape[1]
    pos = np.arange(p, p + n)
    nq, nkv, d, Fw = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn
    X = np.stack([from_storage(w["embed"][i]) for i in ids]).astype(F32)
    taps, Kb, Vb = [], [], []
    allow = np.arange(p + n)[None, :] <= (p + np.arange(n))[:, None]
    for l in range(cfg.n_layers):
        W = lambda k: from_storage(w[k][l]).astype(F32)
        Y = _st(_rms(X, W("attn_norm"), cfg.rms_eps))
        qkv = Y @ W("w_qkv").T
        q = _st(_rope(qkv[:, :nq * d].reshape(n, nq, d), pos, cfg.rope_theta))
        k = _st(_rope(qkv[:, nq * d:(nq + nkv) * d].reshape(n, nkv, d), pos, cfg.rope_theta))
        v = _st(qkv[:, (nq + nkv) * d:].reshape(n, nkv, d))
        K = np.concatenate([Kc[l].astype(F32), k])
        V = np.concatenate([Vc[l].astype(F32), v])
        O = np.empty((n, nq, d), dtype=F32)
        for h in range(nq):
            g = h // (nq // nkv)
            sc = np.where(allow, (q[:, h] @ K[:, g].T) / F32(np.sqrt(d)), F32(-np.inf))
            e = np.exp(sc - sc.max(axis=1, keepdims=True))
            O[:, h] = (e / e.sum(axis=1, keepdims=True, dtype=F32)) @ V[:, g]
        X = X + _st(O).reshape(n, nq * d) @ W("w_o").T
        Y = _st(_rms(X, W("mlp_norm"), cfg.rms_eps))
        gu = Y @ W("w_gate_up").T
        hm = _st(gu[:, :Fw] / (F32(1) + np.exp(-gu[:, :Fw])) * gu[:, Fw:])
        X = X + hm @ W("w_down").T
        taps.append(_st(X).astype(np.float64))
        Kb.append(k.astype(np.float64))
        Vb.append(v.astype(np.float64))
    Z = _st(_rms(X, from_storage(w["final_norm"]).astype(F32), cfg.rms_eps)).astype(np.float64)
    return Z, taps, np.stack(Kb), np.stack(Vb)


def scaled_by_row(got, want):
    """max |got - want| / max(1, |want|, RMS of want's row)."""
    rms = np.sqrt((want ** 2).mean(axis=-1, keepdims=True))
    return float((np.abs(got - want) / np.maximum(np.maximum(1.0, np.abs(want)), rms)).max())


@pytest.mark.timeout(900)
def test_bf16_verify_floor_at_qwen3_8b_layer():
    from oracle import target as T
    base = S.get_config("qwen3_8b")
    worst = dict(kv=0.0, el=0.0, rows=0.0)
    for ctx in (17, 77, 300):
        cfg = dataclasses.replace(base, name="verify_floor", cid=121, vocab=2048, n_layers=1, n_feat_layers=1,
                                  block_size=16, batch=1, ctx_min=ctx, ctx_max=ctx)
        w = S.drafter_weights(cfg, seed=3, random_gain=True)
        lens = np.array([ctx], dtype=np.int32)
        lay = S.paged_layout(cfg, lens, headroom=16, seed=4)
        Kp, Vp = S.ctx_kv_cache(cfg, lay, seed=4)
        t = np.arange(ctx)
        Kc = from_storage(Kp[:, lay.block_table[0, t // 16], t % 16])
        Vc = from_storage(Vp[:, lay.block_table[0, t // 16], t % 16])
        ids = np.random.default_rng(ctx + 16).integers(0, cfg.vocab, 16)
        Z, To, Kb, Vb = T.verify_block(w, cfg, ids, Kc, Vc, tap_layers=[0])
        Z32, taps32, Kb32, Vb32 = verify_block_fp32_acc(w, cfg, ids, Kc, Vc)
        kv = max(float((np.abs(a - b) / np.maximum(1.0, np.abs(b))).max()) for a, b in ((Kb32, Kb), (Vb32, Vb)))
        el = max(scaled_by_row(taps32[0], To), scaled_by_row(Z32, Z))
        rows = max(_row_rel(taps32[0], To), _row_rel(Z32, Z))
        print(f"verify floor, context {ctx}: cache K/V {kv:.3e}; taps and hidden {el:.3e} (row-scaled), "
              f"{rows:.3e} per row")
        worst = {k: max(worst[k], v) for k, v in dict(kv=kv, el=el, rows=rows).items()}
    assert worst["kv"] <= 1e-2
    assert worst["el"] <= 2.5e-2
    assert worst["rows"] <= 1e-2
