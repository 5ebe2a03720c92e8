"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-derived
golden values, closed forms, invariants, library routines (torch CPU in
float64) or brute-force scalar loops on tiny shapes.  No GPU is needed.
"""
import dataclasses
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import dflash_synth as S
from oracle import drafter as D
from oracle import target as T
from oracle.numerics import bf16_bits, from_storage, round_bf16, round_f32, round_storage

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_cfg(dtype="f64", **kw):
    base = dict(hidden=8, n_q_heads=2, n_kv_heads=1, head_dim=4, ffn=6, vocab=12, n_layers=2,
                n_feat_layers=2, block_size=3, batch=1, ctx_min=2, ctx_max=2, rope_theta=100.0,
                target_layers=0, feat_layer_ids=(), prompt_len=0, new_tokens=0)
    base.update(kw)
    return dataclasses.replace(S.get_config("tiny"), name="small", cid=77, dtype=dtype, **base)


def small_setup(cfg, seed=0, p=None):
    """Weights (random gains), context from inject of seeded features, anchor."""
    w = S.drafter_weights(cfg, seed=seed, random_gain=True)
    p = cfg.ctx_min if p is None else p
    feats = S.features(cfg, p, seed=seed)
    K, V = D.inject(w, cfg, feats, np.arange(p))
    anchor = int(S.anchor_ids(cfg, seed=seed, batch=1)[0])
    return w, feats, K, V, anchor


# ----------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------
def test_bf16_golden_table():
    n = 0
    with open(os.path.join(GOLDEN, "bf16_rne.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            x_hex, bits_hex = line.split()
            x = float.fromhex(x_hex)
            assert int(bf16_bits(np.array([x]))[0]) == int(bits_hex, 16), line
            n += 1
    assert n >= 10


def test_bf16_matches_torch_on_fp32_values():
    """For fp32-representable inputs, direct float64 -> bf16 rounding equals
    torch's fp32 -> bf16 conversion (round to nearest even)."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(20000) * 1e-30).astype(np.float32),
        # exact ties: bf16 values plus half a bf16 ulp
        (S.f32_from_bf16_bits(rng.integers(0x3000, 0x5000, 5000).astype(np.uint16)).view(np.uint32)
         + np.uint32(0x8000)).view(np.float32),
    ])
    ours = bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # the synthetic generator's fp32 -> bf16 conversion agrees as well
    assert np.array_equal(S.bf16_bits_from_f32(x), ref)


def test_bf16_round_is_idempotent_and_monotone():
    rng = np.random.default_rng(1)
    x = np.sort(rng.standard_normal(100000) * 10)
    r = round_bf16(x)
    assert np.array_equal(round_bf16(r), r)
    assert np.all(np.diff(r) >= 0)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8 + 1e-300)


def test_round_f32_matches_numpy_cast():
    x = np.random.default_rng(2).standard_normal(1000)
    assert np.array_equal(round_f32(x), x.astype(np.float32).astype(np.float64))


# ----------------------------------------------------------------------------
# P2: primitives against torch CPU (float64)
# ----------------------------------------------------------------------------
def test_rms_norm_matches_torch():
    rng = np.random.default_rng(3)
    x, g = rng.standard_normal((7, 64)), rng.standard_normal(64)
    ref = F.rms_norm(torch.from_numpy(x), (64,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(D.rms_norm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-14)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(D.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-300)


@pytest.mark.parametrize("nq,nkv,M,T_", [(8, 2, 5, 11), (4, 4, 3, 7), (6, 1, 16, 40)])
def test_attention_matches_torch_sdpa_gqa(nq, nkv, M, T_):
    rng = np.random.default_rng(nq * 100 + nkv)
    d = 16
    q, k, v = rng.standard_normal((M, nq, d)), rng.standard_normal((T_, nkv, d)), rng.standard_normal((T_, nkv, d))
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2))[None], torch.from_numpy(k.transpose(1, 0, 2))[None],
        torch.from_numpy(v.transpose(1, 0, 2))[None], enable_gqa=True)[0].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(D.attention(q, k, v), ref, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# P3: RoPE
# ----------------------------------------------------------------------------
def test_rope_closed_form_values():
    """Unit vectors rotate by pos * theta^(-2i/d) in the (i, i + d/2) plane."""
    d, theta = 4, 100.0
    x = np.zeros((1, 1, d))
    x[0, 0, 1] = 1.0                          # i = 1: inverse frequency 100^(-2/4) = 0.1
    out = D.rope(x, np.array([5]), theta)[0, 0]
    np.testing.assert_allclose(out, [0.0, math.cos(0.5), 0.0, math.sin(0.5)], atol=1e-15)
    x = np.zeros((1, 1, d))
    x[0, 0, 2] = 1.0                          # the partner of i = 0 (frequency 1)
    out = D.rope(x, np.array([3]), theta)[0, 0]
    np.testing.assert_allclose(out, [-math.sin(3.0), 0.0, math.cos(3.0), 0.0], atol=1e-15)


def test_rope_identity_at_zero_norm_and_relative_position():
    rng = np.random.default_rng(4)
    d, theta = 128, 1e6
    x = rng.standard_normal((5, 3, d))
    assert np.array_equal(D.rope(x, np.zeros(5), theta), x)
    y = D.rope(x, np.arange(5) * 997, theta)
    h = d // 2
    np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:] ** 2, x[..., :h] ** 2 + x[..., h:] ** 2, rtol=1e-12)
    q, k = rng.standard_normal((1, 1, d)), rng.standard_normal((1, 1, d))
    dots = [float(np.sum(D.rope(q, np.array([m + s]), theta) * D.rope(k, np.array([n + s]), theta)))
            for (m, n) in [(40, 7)] for s in (0, 13, 5000)]
    np.testing.assert_allclose(dots, dots[0], rtol=1e-10)


# ----------------------------------------------------------------------------
# P4: attention special cases
# ----------------------------------------------------------------------------
def test_attention_special_cases():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 4, 8))
    k1, v1 = rng.standard_normal((1, 2, 8)), rng.standard_normal((1, 2, 8))
    out = D.attention(q, k1, v1)                 # one key: output is that value
    for h in range(4):
        np.testing.assert_array_equal(out[:, h], np.broadcast_to(v1[0, h // 2], (4, 8)))
    kz, v = np.zeros((9, 2, 8)), rng.standard_normal((9, 2, 8))
    out = D.attention(q, kz, v)                  # equal scores: mean of the values
    for h in range(4):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(v[:, h // 2].mean(0), (4, 8)), rtol=1e-13)
    k, v = rng.standard_normal((9, 4, 8)), rng.standard_normal((9, 4, 8))
    out = D.attention(q, k, v)                   # nkv == nq: each head alone
    for h in range(4):
        np.testing.assert_allclose(out[:, h:h + 1], D.attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1]),
                                   rtol=1e-14)


def test_draft_with_empty_context_is_a_block_encoder():
    cfg = small_cfg()
    w = S.drafter_weights(cfg, random_gain=True)
    empty = np.zeros((cfg.n_layers, 0, cfg.n_kv_heads, cfg.head_dim))
    Z = D.draft_block(w, cfg, 3, empty, empty)
    assert Z.shape == (cfg.block_size - 1, cfg.hidden) and np.all(np.isfinite(Z))


# ----------------------------------------------------------------------------
# P1: brute-force scalar loops on tiny shapes
# ----------------------------------------------------------------------------
def _bf_round(x, dt):
    if dt == "f64":
        return x
    t = torch.tensor([x], dtype=torch.float32)
    if dt == "bf16":
        t = t.to(torch.bfloat16)
    return float(t.to(torch.float64)[0])


def _bf_rms(x, g, eps):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [x[i] * r * g[i] for i in range(len(x))]


def _bf_matvec(W, x):
    return [sum(W[n][k] * x[k] for k in range(len(x))) for n in range(len(W))]


def _bf_rope(v, pos, theta):
    d = len(v)
    h = d // 2
    out = list(v)
    for i in range(h):
        a = pos * theta ** (-2.0 * i / d)
        out[i] = v[i] * math.cos(a) - v[i + h] * math.sin(a)
        out[i + h] = v[i + h] * math.cos(a) + v[i] * math.sin(a)
    return out


def _bf_inject(w, cfg, feats, positions):
    L = lambda a: from_storage(a).tolist()
    dt, nq, nkv, d = cfg.dtype, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    Wfc = L(w["w_fc"])
    K = [[None] * len(positions) for _ in range(cfg.n_layers)]
    V = [[None] * len(positions) for _ in range(cfg.n_layers)]
    for t, f in enumerate(L(feats)):
        c = [_bf_round(v, dt) for v in _bf_matvec(Wfc, f)]
        for l in range(cfg.n_layers):
            Wqkv = L(w["w_qkv"][l])
            kk = _bf_matvec(Wqkv[nq * d:(nq + nkv) * d], c)
            vv = _bf_matvec(Wqkv[(nq + nkv) * d:], c)
            K[l][t] = [[_bf_round(x, dt) for x in _bf_rope(kk[g * d:(g + 1) * d], positions[t], cfg.rope_theta)]
                       for g in range(nkv)]
            V[l][t] = [[_bf_round(x, dt) for x in vv[g * d:(g + 1) * d]] for g in range(nkv)]
    return K, V


def _bf_draft(w, cfg, anchor, Kc, Vc):
    L = lambda a: from_storage(a).tolist()
    dt, B, H = cfg.dtype, cfg.block_size, cfg.hidden
    nq, nkv, d, Fw = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn
    p = len(Kc[0])
    res = (lambda v: v) if dt == "f64" else (lambda v: _bf_round(v, "f32"))
    E = L(w["embed"])
    ids = [anchor] + [cfg.vocab - 1] * (B - 1)
    X = [[res(v) for v in E[t]] for t in ids]
    for l in range(cfg.n_layers):
        Wqkv, Wo, Wgu, Wd = L(w["w_qkv"][l]), L(w["w_o"][l]), L(w["w_gate_up"][l]), L(w["w_down"][l])
        ga, gm = L(w["attn_norm"][l]), L(w["mlp_norm"][l])
        q, k, v = [], [], []
        for r in range(B):
            y = [_bf_round(t, dt) for t in _bf_rms(X[r], ga, cfg.rms_eps)]
            o = _bf_matvec(Wqkv, y)
            q.append([[_bf_round(t, dt) for t in _bf_rope(o[h * d:(h + 1) * d], p + r, cfg.rope_theta)]
                      for h in range(nq)])
            k.append([[_bf_round(t, dt) for t in _bf_rope(o[(nq + g) * d:(nq + g + 1) * d], p + r, cfg.rope_theta)]
                      for g in range(nkv)])
            v.append([[_bf_round(t, dt) for t in o[(nq + nkv + g) * d:(nq + nkv + g + 1) * d]] for g in range(nkv)])
        keys = [Kc[l][t] for t in range(p)] + k
        vals = [Vc[l][t] for t in range(p)] + v
        for r in range(B):
            att = []
            for h in range(nq):
                g = h * nkv // nq
                s = [sum(q[r][h][j] * keys[t][g][j] for j in range(d)) / math.sqrt(d) for t in range(len(keys))]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                att += [_bf_round(sum(e[t] / z * vals[t][g][j] for t in range(len(keys))), dt) for j in range(d)]
            delta = _bf_matvec(Wo, att)
            X[r] = [res(X[r][i] + delta[i]) for i in range(H)]
        for r in range(B):
            y = [_bf_round(t, dt) for t in _bf_rms(X[r], gm, cfg.rms_eps)]
            gu = _bf_matvec(Wgu, y)
            hm = [_bf_round(gu[i] / (1.0 + math.exp(-gu[i])) * gu[Fw + i], dt) for i in range(Fw)]
            delta = _bf_matvec(Wd, hm)
            X[r] = [res(X[r][i] + delta[i]) for i in range(H)]
    gf = L(w["final_norm"])
    return [[_bf_round(t, dt) for t in _bf_rms(X[r], gf, cfg.rms_eps)] for r in range(1, B)]


@pytest.mark.parametrize("dtype,nq,nkv", [("f64", 2, 1), ("f64", 2, 2), ("f64", 4, 2), ("bf16", 2, 1), ("f32", 4, 2)])
def test_inject_and_draft_match_brute_force(dtype, nq, nkv):
    cfg = small_cfg(dtype, n_q_heads=nq, n_kv_heads=nkv)
    w, feats, K, V, anchor = small_setup(cfg, seed=nq + nkv)
    p = cfg.ctx_min
    Kb, Vb = _bf_inject(w, cfg, feats, list(range(p)))
    tol = dict(rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(K, np.array(Kb), **tol)
    np.testing.assert_allclose(V, np.array(Vb), **tol)
    Z = D.draft_block(w, cfg, anchor, K, V)
    Zb = np.array(_bf_draft(w, cfg, anchor, Kb, Vb))
    np.testing.assert_allclose(Z, Zb, **tol)
    # LM head: logits and argmax from explicit sums
    Wlm = from_storage(w["lm_head"]).tolist()
    logits_b = np.array([[sum(Wlm[n][j] * z[j] for j in range(cfg.hidden)) for n in range(cfg.vocab)] for z in Zb])
    ids, best, logits = D.lm_argmax(w["lm_head"], Z)
    np.testing.assert_allclose(logits, logits_b, **tol)
    for r in range(len(ids)):
        assert logits_b[r, ids[r]] == pytest.approx(logits_b[r].max(), abs=1e-12)


def test_rounding_points_leave_storage_values():
    """bf16 outputs of inject and draft are exactly bf16-representable."""
    cfg = small_cfg("bf16")
    w, feats, K, V, anchor = small_setup(cfg)
    Z = D.draft_block(w, cfg, anchor, K, V)
    for a in (K, V, Z):
        assert np.array_equal(round_bf16(a), a)


# ----------------------------------------------------------------------------
# P5: non-causality / exchangeability
# ----------------------------------------------------------------------------
def test_mask_rows_identical_without_rope():
    cfg = small_cfg("f64", block_size=5)
    w, feats, K, V, anchor = small_setup(cfg)
    Z = D.draft_block(w, cfg, anchor, K, V, use_rope=False)
    for r in range(1, Z.shape[0]):
        np.testing.assert_allclose(Z[r], Z[0], rtol=1e-12, atol=1e-13)
    Zr = D.draft_block(w, cfg, anchor, K, V)         # positions make the rows differ
    assert np.max(np.abs(Zr[1] - Zr[0])) > 1e-6


def test_context_permutation_invariance_and_causality():
    cfg = small_cfg("f64", ctx_min=6, ctx_max=6, block_size=4)
    w, feats, K, V, anchor = small_setup(cfg)
    Z = D.draft_block(w, cfg, anchor, K, V)
    perm = np.random.default_rng(6).permutation(K.shape[1])
    np.testing.assert_allclose(D.draft_block(w, cfg, anchor, K[:, perm], V[:, perm]), Z, rtol=1e-12, atol=1e-13)
    Zc = D.draft_block(w, cfg, anchor, K, V, causal=True)
    assert np.max(np.abs(Zc - Z)) > 1e-6            # the block is not causal
    # the anchor row sees the masks: its hidden state changes with the mask token
    w2 = dict(w)
    w2["embed"] = w["embed"].copy()
    w2["embed"][cfg.vocab - 1] = w["embed"][0]
    assert np.max(np.abs(D.draft_block(w2, cfg, anchor, K, V) - Z)) > 1e-6


def test_sliding_window_reads_only_the_last_positions():
    """With a sliding window of W positions the drafter's output does not
    depend on older context K/V, depends on every position inside the window,
    and equals the full-context pass when W covers the context (or W = 0)."""
    cfg = small_cfg("f64", ctx_min=12, ctx_max=12, block_size=4)
    w, feats, K, V, anchor = small_setup(cfg)
    p, W = K.shape[1], 5
    full = D.draft_block(w, cfg, anchor, K, V)
    for wide in (0, p, p + 3):
        np.testing.assert_array_equal(D.draft_block(w, dataclasses.replace(cfg, window=wide), anchor, K, V), full)
    cw = dataclasses.replace(cfg, window=W)
    Zw = D.draft_block(w, cw, anchor, K, V)
    assert np.max(np.abs(Zw - full)) > 1e-6
    rng = np.random.default_rng(11)
    K2, V2 = K.copy(), V.copy()
    K2[:, :p - W] = rng.normal(size=K2[:, :p - W].shape)
    V2[:, :p - W] = rng.normal(size=V2[:, :p - W].shape)
    np.testing.assert_array_equal(D.draft_block(w, cw, anchor, K2, V2), Zw)
    for t in (p - W, p - 1):                          # the window's edges
        K3 = K.copy()
        K3[:, t] = rng.normal(size=K3[:, t].shape)
        assert np.max(np.abs(D.draft_block(w, cw, anchor, K3, V) - Zw)) > 1e-9


# ----------------------------------------------------------------------------
# P6: context injection
# ----------------------------------------------------------------------------
def test_inject_row_independence_and_zero_features():
    cfg = small_cfg("bf16", ctx_min=9, ctx_max=9)
    w = S.drafter_weights(cfg, random_gain=True)
    f = S.features(cfg, 9)
    K, V = D.inject(w, cfg, f, np.arange(9))
    K2, V2 = D.inject(w, cfg, f[3:7], np.arange(3, 7))
    assert np.array_equal(K[:, 3:7], K2) and np.array_equal(V[:, 3:7], V2)
    Kz, Vz = D.inject(w, cfg, np.zeros_like(f), np.arange(9))
    assert not Kz.any() and not Vz.any()
    # V does not depend on the position; K only through its rotation (norm kept per pair)
    K3, V3 = D.inject(w, cfg, f[:1], np.array([0]))
    K4, V4 = D.inject(w, cfg, f[:1], np.array([123]))
    assert np.array_equal(V3, V4)
    h = cfg.head_dim // 2
    n3 = K3[..., :h] ** 2 + K3[..., h:] ** 2
    n4 = K4[..., :h] ** 2 + K4[..., h:] ** 2
    np.testing.assert_allclose(n3, n4, rtol=2e-2)


def test_draft_depends_on_features_not_cache_writes():
    cfg = small_cfg("f64", ctx_min=5, ctx_max=5)
    w, feats, K, V, anchor = small_setup(cfg)
    K0, V0 = K.copy(), V.copy()
    Z = D.draft_block(w, cfg, anchor, K, V)
    assert np.array_equal(K, K0) and np.array_equal(V, V0)
    K2, V2 = D.inject(w, cfg, S.features(cfg, 5, seed=9), np.arange(5))
    assert np.max(np.abs(D.draft_block(w, cfg, anchor, K2, V2) - Z)) > 1e-6


# ----------------------------------------------------------------------------
# P7: LM head argmax
# ----------------------------------------------------------------------------
def test_lm_argmax_ties_take_lowest_id():
    rng = np.random.default_rng(7)
    W = rng.standard_normal((50, 16))
    Z = rng.standard_normal((3, 16))
    logits = Z @ W.T
    top = np.argmax(logits, axis=1)
    W2 = np.concatenate([W, W[top]], axis=0)          # exact duplicates at higher ids
    ids, best, _ = D.lm_argmax(W2, Z)
    assert np.array_equal(ids, top)
    W3 = W2.copy()
    W3[[30, 7]] = 10.0 * Z[0]                          # a dominant exact tie at ids 7 and 30
    ids3, _, _ = D.lm_argmax(W3, Z[:1])
    assert ids3[0] == 7


# ----------------------------------------------------------------------------
# P8: accept length
# ----------------------------------------------------------------------------
def test_accept_len_golden_cases():
    with open(os.path.join(GOLDEN, "accept_len.txt")) as f:
        rows = [l for l in (x.split("#")[0].strip() for x in f) if l]
    assert len(rows) >= 5
    for r in rows:
        d, y, res = (list(map(int, part.split())) for part in r.split("|"))
        assert D.accept_len(d, y) == (res[0], res[1]), r


@pytest.mark.parametrize("B", [2, 4, 10, 16])
def test_accept_len_exhaustive_match_patterns(B):
    """All 2^(B-1) match patterns against tau = 1 + index of the first miss."""
    rng = np.random.default_rng(B)
    base = rng.integers(0, 1000, B - 1)
    for pat in range(1 << (B - 1)):
        match = [(pat >> i) & 1 for i in range(B - 1)]
        y = [int(base[i]) if match[i] else int(base[i]) + 1 for i in range(B - 1)] + [555]
        first_miss = next((i for i, m in enumerate(match) if not m), B - 1)
        assert D.accept_len(base, y) == (first_miss + 1, y[first_miss])


@pytest.mark.parametrize("B,expected", [(10, 3.239), (16, 3.322)])
def test_accept_len_mean_closed_form(B, expected):
    """With i.i.d. per-position agreement rate a, E[tau] = (1 - a^B) / (1 - a)."""
    a = 0.7
    assert (1 - a ** B) / (1 - a) == pytest.approx(expected, abs=1e-3)
    cfg = dataclasses.replace(S.get_config("llama31_8b"), block_size=B, vocab=1000)
    d = S.draft_ids_random(cfg, 40000, seed=1)
    y = S.target_ids_for(cfg, d, seed=1)
    taus, _ = D.accept_len_batch(d, y)
    assert taus.mean() == pytest.approx(expected, abs=0.05)


def test_synthetic_target_rule():
    cfg = dataclasses.replace(S.get_config("llama31_8b"), vocab=5)
    d = S.draft_ids_random(cfg, 20000, seed=3)
    y = S.target_ids_for(cfg, d, seed=3)
    agree = (y[:, :-1] == d)
    assert abs(agree.mean() - 0.7) < 0.01           # only the Bernoulli draws match
    assert y.min() >= 0 and y.max() < cfg.vocab


# ----------------------------------------------------------------------------
# P9: losslessness of greedy speculative decoding (tiny configuration)
# ----------------------------------------------------------------------------
def _torch_target_logits(w, cfg, tokens):
    """Independent float64 torch forward of the tiny causal target."""
    t = lambda a: torch.from_numpy(from_storage(a))
    n = len(tokens)
    nq, nkv, d, Fw = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn
    x = t(w["embed"])[torch.tensor(tokens)]
    pos = torch.arange(n, dtype=torch.float64)
    inv = cfg.rope_theta ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    ang = pos[:, None] * inv[None]
    cos, sin = torch.cos(ang)[:, None], torch.sin(ang)[:, None]
    rot = lambda u: torch.cat([u[..., :d // 2] * cos - u[..., d // 2:] * sin,
                               u[..., d // 2:] * cos + u[..., :d // 2] * sin], -1)
    for l in range(cfg.target_layers):
        y = F.rms_norm(x, (cfg.hidden,), t(w["attn_norm"][l]), cfg.rms_eps)
        qkv = y @ t(w["w_qkv"][l]).T
        q = rot(qkv[:, :nq * d].reshape(n, nq, d))
        k = rot(qkv[:, nq * d:(nq + nkv) * d].reshape(n, nkv, d))
        v = qkv[:, (nq + nkv) * d:].reshape(n, nkv, d)
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                           v.transpose(0, 1)[None], is_causal=True, enable_gqa=True)
        x = x + o[0].transpose(0, 1).reshape(n, nq * d) @ t(w["w_o"][l]).T
        y = F.rms_norm(x, (cfg.hidden,), t(w["mlp_norm"][l]), cfg.rms_eps)
        gu = y @ t(w["w_gate_up"][l]).T
        x = x + (F.silu(gu[:, :Fw]) * gu[:, Fw:]) @ t(w["w_down"][l]).T
    return (F.rms_norm(x, (cfg.hidden,), t(w["final_norm"]), cfg.rms_eps) @ t(w["lm_head"]).T).numpy()


def test_tiny_target_matches_torch_decoder():
    cfg = S.get_config("tiny")
    w = S.target_weights(cfg, seed=0, layer_std=0.1)
    toks = S.prompt_ids(cfg)[:24]
    logits, taps = T.TinyTarget(w, cfg).run(toks, 0)
    np.testing.assert_allclose(logits, _torch_target_logits(w, cfg, toks), rtol=1e-9, atol=1e-11)
    assert taps.shape == (24, cfg.feat_dim)


class _PerfectDrafter:
    """Returns the target's own greedy continuation (tau = B every cycle)."""

    def __init__(self, cfg, greedy_ext, P):
        self.cfg, self.g, self.P, self.n = cfg, greedy_ext, P, 0

    def inject(self, feats, pos):
        self.n += len(pos)

    def draft(self, anchor):
        p = self.n
        return np.array([self.g[p + j - self.P] for j in range(1, self.cfg.block_size)])


class _WrongDrafter(_PerfectDrafter):
    def draft(self, anchor):
        return (super().draft(anchor) + 1) % self.cfg.vocab


class _ZeroDrafter(D.OracleDrafter):
    def __init__(self, cfg):
        w = S.drafter_weights(cfg)
        zero = lambda a: np.zeros_like(a)
        super().__init__({k: ([zero(x) for x in v] if isinstance(v, list) else
                              (v if k in ("embed", "lm_head") else zero(v))) for k, v in w.items()}, cfg)


@pytest.mark.parametrize("seed,layer_std", [(0, 0.02), (1, 0.02), (0, 0.1), (1, 0.1), (2, 0.05)])
def test_lossless_with_oracle_drafter(seed, layer_std):
    cfg = S.get_config("tiny")
    tgt = T.TinyTarget(S.target_weights(cfg, seed, layer_std=layer_std), cfg)
    prompt = S.prompt_ids(cfg, seed)
    g = T.greedy_decode(tgt, prompt, cfg.new_tokens)
    s, taus = T.spec_decode(tgt, D.OracleDrafter(S.drafter_weights(cfg, seed), cfg), prompt,
                            cfg.new_tokens, cfg.dtype)
    assert np.array_equal(g, s)
    assert all(1 <= t <= cfg.block_size for t in taus)


def test_lossless_with_extreme_drafters():
    cfg = S.get_config("tiny")
    tgt = T.TinyTarget(S.target_weights(cfg, 3, layer_std=0.1), cfg)
    prompt = S.prompt_ids(cfg, 3)
    n, B = cfg.new_tokens, cfg.block_size
    g_ext = T.greedy_decode(tgt, prompt, n + B)
    g = g_ext[:n]
    s, taus = T.spec_decode(tgt, _PerfectDrafter(cfg, g_ext, len(prompt)), prompt, n, cfg.dtype)
    assert np.array_equal(s, g) and all(t == B for t in taus) and len(taus) == math.ceil((n - 1) / B)
    s, taus = T.spec_decode(tgt, _WrongDrafter(cfg, g_ext, len(prompt)), prompt, n, cfg.dtype)
    assert np.array_equal(s, g) and all(t == 1 for t in taus) and len(taus) == n - 1
    s, taus = T.spec_decode(tgt, _ZeroDrafter(cfg), prompt, n, cfg.dtype)
    assert np.array_equal(s, g)


# ----------------------------------------------------------------------------
# the target's causal block verify under the storage rounding contract
# ----------------------------------------------------------------------------
def _bf_verify(w, cfg, ids, Kc, Vc, tap_layers):
    """Scalar-loop causal pass: row r sees the p context keys and block keys 0..r."""
    L = lambda a: from_storage(a).tolist()
    dt, H = cfg.dtype, cfg.hidden
    nq, nkv, d, Fw = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn
    n, p = len(ids), len(Kc[0])
    res = (lambda v: v) if dt == "f64" else (lambda v: _bf_round(v, "f32"))
    E = L(w["embed"])
    X = [[res(v) for v in E[t]] for t in ids]
    taps = {}
    kb_all, vb_all = [], []
    for l in range(cfg.n_layers):
        Wqkv, Wo, Wgu, Wd = L(w["w_qkv"][l]), L(w["w_o"][l]), L(w["w_gate_up"][l]), L(w["w_down"][l])
        ga, gm = L(w["attn_norm"][l]), L(w["mlp_norm"][l])
        q, k, v = [], [], []
        for r in range(n):
            y = [_bf_round(t, dt) for t in _bf_rms(X[r], ga, cfg.rms_eps)]
            o = _bf_matvec(Wqkv, y)
            q.append([[_bf_round(t, dt) for t in _bf_rope(o[h * d:(h + 1) * d], p + r, cfg.rope_theta)]
                      for h in range(nq)])
            k.append([[_bf_round(t, dt) for t in _bf_rope(o[(nq + g) * d:(nq + g + 1) * d], p + r, cfg.rope_theta)]
                      for g in range(nkv)])
            v.append([[_bf_round(t, dt) for t in o[(nq + nkv + g) * d:(nq + nkv + g + 1) * d]] for g in range(nkv)])
        kb_all.append(k)
        vb_all.append(v)
        for r in range(n):
            keys = [Kc[l][t] for t in range(p)] + k[:r + 1]
            vals = [Vc[l][t] for t in range(p)] + v[:r + 1]
            att = []
            for h in range(nq):
                g = h * nkv // nq
                sc = [sum(q[r][h][j] * keys[t][g][j] for j in range(d)) / math.sqrt(d) for t in range(len(keys))]
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                z = sum(e)
                att += [_bf_round(sum(e[t] / z * vals[t][g][j] for t in range(len(keys))), dt) for j in range(d)]
            delta = _bf_matvec(Wo, att)
            X[r] = [res(X[r][i] + delta[i]) for i in range(H)]
        for r in range(n):
            y = [_bf_round(t, dt) for t in _bf_rms(X[r], gm, cfg.rms_eps)]
            gu = _bf_matvec(Wgu, y)
            hm = [_bf_round(gu[i] / (1.0 + math.exp(-gu[i])) * gu[Fw + i], dt) for i in range(Fw)]
            delta = _bf_matvec(Wd, hm)
            X[r] = [res(X[r][i] + delta[i]) for i in range(H)]
        taps[l] = [[_bf_round(t, dt) for t in X[r]] for r in range(n)]
    gf = L(w["final_norm"])
    Z = [[_bf_round(t, dt) for t in _bf_rms(X[r], gf, cfg.rms_eps)] for r in range(n)]
    T_ = [sum((taps[l][r] for l in tap_layers), []) for r in range(n)]
    return Z, T_, kb_all, vb_all


@pytest.mark.parametrize("dtype,nq,nkv", [("bf16", 2, 1), ("f32", 4, 2), ("f64", 2, 2)])
def test_verify_block_matches_brute_force(dtype, nq, nkv):
    cfg = small_cfg(dtype, n_q_heads=nq, n_kv_heads=nkv, block_size=4)
    w, feats, K, V, anchor = small_setup(cfg, seed=5 + nq)
    ids = [anchor, 3, 7, 3]
    Z, T_, Kb, Vb = T.verify_block(w, cfg, ids, K, V, tap_layers=(1, 0))
    Zb, Tb, Kbb, Vbb = _bf_verify(w, cfg, ids, K.tolist(), V.tolist(), (1, 0))
    tol = dict(rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Z, np.array(Zb), **tol)
    np.testing.assert_allclose(T_, np.array(Tb), **tol)
    np.testing.assert_allclose(Kb, np.array(Kbb), **tol)
    np.testing.assert_allclose(Vb, np.array(Vbb), **tol)
    if dtype == "bf16":
        for a in (Z, T_, Kb, Vb):
            assert np.array_equal(round_bf16(a), a)


def test_verify_block_equals_tiny_target_in_float64():
    """Without storage rounding the block pass is the tiny target's own
    row-by-row decoding: logits, taps and the appended cache rows agree."""
    cfg = S.get_config("tiny")
    w = S.target_weights(cfg, seed=2, layer_std=0.1)
    c64 = dataclasses.replace(cfg, dtype="f64", n_layers=cfg.target_layers)
    prompt = S.prompt_ids(cfg, 2)
    tgt = T.TinyTarget(w, cfg)
    tgt.run(prompt[:40], 0)
    Kc, Vc = np.stack(tgt.K), np.stack(tgt.V)
    block = [int(t) for t in prompt[40:40 + 6]]
    lo, to = tgt.run(block, 40)
    Z, T_, Kb, Vb = T.verify_block(w, c64, block, Kc, Vc, tap_layers=cfg.feat_layer_ids)
    np.testing.assert_allclose(Z @ from_storage(w["lm_head"]).T, lo, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(T_, to, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Kb, np.stack(tgt.K)[:, 40:], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Vb, np.stack(tgt.V)[:, 40:], rtol=1e-10, atol=1e-12)


def test_verify_block_reproduces_incremental_decoding():
    """bf16 storage: one pass over n rows equals n one-row passes, each appending
    its rounded K/V to the cache (causality and the position of every row)."""
    cfg = small_cfg("bf16", n_q_heads=4, n_kv_heads=2, block_size=5)
    w, feats, K, V, anchor = small_setup(cfg, seed=9)
    ids = [anchor, 4, 4, 11, 0]
    Z, T_, Kb, Vb = T.verify_block(w, cfg, ids, K, V, tap_layers=(0, 1))
    Kc, Vc = K, V
    for r, t in enumerate(ids):
        z1, t1, k1, v1 = T.verify_block(w, cfg, [t], Kc, Vc, tap_layers=(0, 1))
        np.testing.assert_allclose(z1[0], Z[r], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(t1[0], T_[r], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(k1[:, 0], Kb[:, r], rtol=1e-12, atol=1e-12)
        Kc, Vc = np.concatenate([Kc, k1], axis=1), np.concatenate([Vc, v1], axis=1)
    # a later token never changes an earlier row
    ids2 = ids[:2] + [7, 7, 7]
    Z2, T2, _, _ = T.verify_block(w, cfg, ids2, K, V, tap_layers=(0, 1))
    np.testing.assert_array_equal(Z2[:2], Z[:2])
    assert not np.allclose(Z2[2:], Z[2:])


# ----------------------------------------------------------------------------
# P10: shape plausibility
# ----------------------------------------------------------------------------
def test_drafter_size_matches_pages():
    """A 5-layer drafter at the Qwen3-8B shape holds 0.5B-1B parameters ([FN] §3.1)."""
    cfg = S.get_config("qwen3_8b")
    layers = cfg.layer_params() - cfg.feat_dim * cfg.hidden - cfg.hidden
    assert 0.5e9 <= layers <= 1.0e9
    assert layers == pytest.approx(964.7e6, rel=1e-3)


def test_inject_rounds_exact_ties_to_even():
    """The oracle's storage rounding of the fused context c (read back through
    identity V projections) on exact fp32 ties between bf16 neighbours, against
    torch's CPU conversion: round to nearest, ties to even."""
    from tie_cases import tie_case
    cfg = S.get_config("tiny", dtype="bf16", n_feat_layers=3)
    w, feats, expect, n_ties = tie_case(cfg, 12, seed=7)
    assert n_ties > 1000
    _, V = D.inject(w, cfg, feats, np.arange(12))
    got = bf16_bits(V.reshape(cfg.n_layers, 12, cfg.hidden))
    for l in range(cfg.n_layers):
        assert np.array_equal(got[l], expect)


def test_ctx_norm_rows_have_unit_rms_and_scale_invariance():
    """The optional RMSNorm after the fusion projection: with gain 1 every row of
    c has root mean square 1 (to eps and fp32 rounding), scaling the features
    changes nothing, and a gain scales each column; off, c is the plain product."""
    import dataclasses as dc
    cfg = dc.replace(S.get_config("tiny"), ctx_norm=1, rms_eps=0.0)
    w = S.drafter_weights(cfg, seed=1)
    f = S.features(cfg, 7, seed=2)
    c = D.fuse_context(w, cfg, f)
    assert np.allclose(np.sqrt((c ** 2).mean(axis=1)), 1.0, atol=1e-6)
    f64 = from_storage(f)
    assert np.allclose(D.fuse_context(w, cfg, f64 * 7.0), c, atol=1e-6)
    g = np.linspace(0.5, 2.0, cfg.hidden).astype(np.float32)
    w2 = dict(w, ctx_norm=g)
    assert np.allclose(D.fuse_context(w2, cfg, f), c * g, atol=1e-5)
    off = D.fuse_context(w, dc.replace(cfg, ctx_norm=0), f)
    assert np.allclose(off, f64 @ from_storage(w["w_fc"]).T, atol=1e-6)
