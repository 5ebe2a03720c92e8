"""Inputs whose fused context values are exact fp32 ties between bf16 neighbours
(not collected by pytest).

The fusion weights are one-hot pairs, c[i] = f[i] + f[H + i], so every element
of c is the exact fp32 sum of two bf16 values, chosen to fall halfway between
two bf16 numbers (or just off halfway).  Each layer's V projection is the
identity, so the injected V rows hold c as the storage rounded it.  Expected
values come from torch's CPU fp32 -> bf16 conversion (round to nearest, ties to
even), an implementation independent of both the oracle and the HIP path.
"""
from __future__ import annotations

import numpy as np
import torch

import dflash_synth as S

ONE_BF16 = np.uint16(0x3F80)


def bf16_bits_of(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of the exactly representable values ``x``."""
    b = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    assert torch.equal(b.to(torch.float32), torch.from_numpy(np.asarray(x, dtype=np.float32))), "not bf16-exact"
    return b.view(torch.int16).numpy().view(np.uint16)


def tie_case(cfg, n: int, seed: int):
    """Weights (one-hot fusion, identity V), features [n, L*H] (bf16 bits) and the
    expected bf16 bits of c [n, H]."""
    H, L = cfg.hidden, cfg.n_feat_layers
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    assert cfg.dtype == "bf16" and L >= 2 and nkv * d == H
    rng = np.random.default_rng(seed)
    e = rng.integers(-6, 7, size=(n, H))
    k = rng.integers(0, 128, size=(n, H))
    sgn = rng.choice([-1.0, 1.0], size=(n, H))
    s = rng.choice([-1.0, 1.0], size=(n, H))
    # b sits exactly half a bf16 step from a (ties), or a 1/128 of a half step
    # beside it (near ties that must round toward the nearer neighbour)
    near = rng.choice([0.0, 1.0, -1.0], size=(n, H), p=[0.6, 0.2, 0.2])
    a = sgn * (1.0 + k / 128.0) * np.exp2(e)
    b = sgn * s * np.exp2(e - 8.0) * (1.0 + near / 128.0)
    c32 = (a.astype(np.float32) + b.astype(np.float32)).astype(np.float32)   # exact in fp32
    assert np.array_equal(c32.astype(np.float64), a + b)
    feats = np.zeros((n, L * H), dtype=np.uint16)
    feats[:, :H] = bf16_bits_of(a)
    feats[:, H:2 * H] = bf16_bits_of(b)
    expect = torch.from_numpy(c32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w = S.drafter_weights(cfg, seed=seed)
    wfc = np.zeros((H, L * H), dtype=np.uint16)
    wfc[np.arange(H), np.arange(H)] = ONE_BF16
    wfc[np.arange(H), H + np.arange(H)] = ONE_BF16
    w["w_fc"] = wfc
    for l in range(cfg.n_layers):
        q = np.array(w["w_qkv"][l], copy=True)
        v0 = (nq + nkv) * d
        q[v0:v0 + H] = 0
        q[v0 + np.arange(H), np.arange(H)] = ONE_BF16
        w["w_qkv"][l] = q
    n_ties = int((near == 0).sum())
    return w, feats, expect, n_ties
