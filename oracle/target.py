"""Tiny target model, plain greedy decoding and greedy speculative decoding with
a block drafter.  TEST INFRASTRUCTURE ONLY (page abbreviations: see the package
docstring).

The target is a causal pre-norm decoder (RMSNorm, RoPE, multi-head attention,
SwiGLU MLP, final norm) in float64 without storage rounding: it exists only on
the CPU.  Every row is computed on its own with the same code, whether it comes
from a prefill, a block verify or a one-token decode step, so a verify
reproduces incremental decoding bit for bit and losslessness is an exact
equality.

Speculative cycle ([FN] §1, §2; [PKR] ``spec_generate`` example):
1. the last accepted token is the anchor, at position p;
2. the drafter fills the B-1 following positions in one pass;
3. the target verifies the block [anchor, d_1..d_{B-1}] in one pass and yields
   y_1..y_B, its greedy token for positions p+1..p+B;
4. drafts are kept up to the first mismatch and the target's token is taken
   there, so output equals the target's own greedy decoding ([FN] §1).
The target's hidden states at the tapped layers for the committed positions are
the drafter's new context features ([SUM] §2.2).

``verify_block`` is the same causal pass over a whole block at once, with the
storage rounding of the drafter's layers (bf16 or fp32): the reference for the
GPU target verify at the large model shapes.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .drafter import accept_len, attention, rms_norm, rope, silu
from .numerics import from_storage, round_f32, round_storage


class TinyTarget:
    """Causal decoder with a growing KV cache; one row at a time."""

    def __init__(self, w: dict, cfg):
        self.cfg = cfg
        self.E = from_storage(w["embed"])
        self.W_lm = from_storage(w["lm_head"])
        self.g_final = from_storage(w["final_norm"])
        self.layers = []
        for l in range(cfg.target_layers):
            self.layers.append(dict(
                g_attn=from_storage(w["attn_norm"][l]), w_qkv=from_storage(w["w_qkv"][l]),
                w_o=from_storage(w["w_o"][l]), g_mlp=from_storage(w["mlp_norm"][l]),
                w_gu=from_storage(w["w_gate_up"][l]), w_d=from_storage(w["w_down"][l])))
        self.reset()

    def reset(self) -> None:
        c = self.cfg
        self.K = [np.zeros((0, c.n_kv_heads, c.head_dim)) for _ in self.layers]
        self.V = [np.zeros((0, c.n_kv_heads, c.head_dim)) for _ in self.layers]

    @property
    def length(self) -> int:
        return self.K[0].shape[0] if self.K else 0

    def truncate(self, n: int) -> None:
        self.K = [k[:n] for k in self.K]
        self.V = [v[:n] for v in self.V]

    def step(self, token: int, pos: int) -> Tuple[np.ndarray, np.ndarray]:
        """Append one token at position ``pos`` (== current length).

        Returns (logits [V], taps [L*H]); taps are the residual stream after
        the configured 0-indexed layers, before the final norm, concatenated
        in layer order.
        """
        c = self.cfg
        assert pos == self.length
        nq, nkv, d, F = c.n_q_heads, c.n_kv_heads, c.head_dim, c.ffn
        x = self.E[token].copy()
        taps = []
        for l, Lw in enumerate(self.layers):
            y = rms_norm(x, Lw["g_attn"], c.rms_eps)
            qkv = Lw["w_qkv"] @ y
            q = rope(qkv[:nq * d].reshape(1, nq, d), np.array([pos]), c.rope_theta)[0]
            k = rope(qkv[nq * d:(nq + nkv) * d].reshape(1, nkv, d), np.array([pos]), c.rope_theta)[0]
            v = qkv[(nq + nkv) * d:].reshape(nkv, d)
            self.K[l] = np.concatenate([self.K[l], k[None]], axis=0)
            self.V[l] = np.concatenate([self.V[l], v[None]], axis=0)
            o = np.empty((nq, d))
            group = nq // nkv
            for h in range(nq):
                g = h // group
                s = self.K[l][:, g, :] @ q[h] / np.sqrt(d)    # causal: keys 0..pos
                s = s - s.max()
                p = np.exp(s)
                o[h] = (p / p.sum()) @ self.V[l][:, g, :]
            x = x + Lw["w_o"] @ o.reshape(-1)
            y = rms_norm(x, Lw["g_mlp"], c.rms_eps)
            gu = Lw["w_gu"] @ y
            x = x + Lw["w_d"] @ (silu(gu[:F]) * gu[F:])
            if l in c.feat_layer_ids:
                taps.append(x.copy())
        logits = self.W_lm @ rms_norm(x, self.g_final, c.rms_eps)
        return logits, np.concatenate(taps)

    def run(self, tokens: Sequence[int], start: int) -> Tuple[np.ndarray, np.ndarray]:
        """Process ``tokens`` at positions start.. one row at a time."""
        logits, taps = [], []
        for i, t in enumerate(tokens):
            lg, tp = self.step(int(t), start + i)
            logits.append(lg)
            taps.append(tp)
        return np.stack(logits), np.stack(taps)


def verify_block(w: dict, cfg, ids: Sequence[int], K_ctx: np.ndarray, V_ctx: np.ndarray,
                 tap_layers: Sequence[int] = ()) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """The target's causal pass over one drafted block, under the storage
    rounding contract of the drafter's layers.

    The target checks the whole block [anchor, d_1 .. d_{B-1}] in one forward
    pass ([FN] §1 and the §2 cycle, step 4), and its hidden states at a few
    uniformly spaced layers are the drafter's context features ([SUM] §2.2;
    [INS]).  ``w`` holds a decoder of the drafter's layer structure (keys as
    ``dflash_synth.drafter_weights``; ``cfg.n_layers`` layers), ``ids`` the
    block's tokens at positions p .. p+len(ids)-1 with p = ``K_ctx.shape[1]``,
    and ``K_ctx, V_ctx [n_layers, p, nkv, d]`` the target's cached keys and
    values of positions 0 .. p-1.

    Row j attends to the p context keys and to block keys 0 .. j (causal).
    Rounding points as in ``drafter.draft_block`` (storage type ``cfg.dtype``;
    "f64" rounds nothing and keeps a float64 residual): RMSNorm outputs, q/k/v
    after RoPE, the attention output, the SwiGLU product, the taps and the
    final hidden states are rounded; the residual stream is fp32.

    Returns ``Z [n, H]`` (final-norm hidden states of every row), ``taps [n,
    len(tap_layers) * H]`` (the residual stream after each listed 0-indexed
    layer, before the final norm, in list order) and the block's own keys and
    values ``Kb, Vb [n_layers, n, nkv, d]`` as they join the cache.
    """
    dt = cfg.dtype
    H = cfg.hidden
    nq, nkv, d, F = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn
    ids = np.asarray(ids, dtype=np.int64)
    n = len(ids)
    p = K_ctx.shape[1]
    pos = np.arange(p, p + n)
    res = (lambda a: a) if dt == "f64" else round_f32      # fp32 residual stream
    X = res(from_storage(w["embed"][ids]))
    taps = {}
    Kb = np.empty((cfg.n_layers, n, nkv, d))
    Vb = np.empty((cfg.n_layers, n, nkv, d))
    for l in range(cfg.n_layers):
        Y = round_storage(rms_norm(X, from_storage(w["attn_norm"][l]), cfg.rms_eps), dt)
        qkv = Y @ from_storage(w["w_qkv"][l]).T
        q = rope(qkv[:, :nq * d].reshape(n, nq, d), pos, cfg.rope_theta)
        k = rope(qkv[:, nq * d:(nq + nkv) * d].reshape(n, nkv, d), pos, cfg.rope_theta)
        v = qkv[:, (nq + nkv) * d:].reshape(n, nkv, d)
        q, Kb[l], Vb[l] = round_storage(q, dt), round_storage(k, dt), round_storage(v, dt)
        Kall = np.concatenate([K_ctx[l], Kb[l]], axis=0)
        Vall = np.concatenate([V_ctx[l], Vb[l]], axis=0)
        O = round_storage(attention(q, Kall, Vall, causal_from=p), dt)   # row j sees keys 0 .. p+j
        X = res(X + O.reshape(n, nq * d) @ from_storage(w["w_o"][l]).T)
        Y = round_storage(rms_norm(X, from_storage(w["mlp_norm"][l]), cfg.rms_eps), dt)
        gu = Y @ from_storage(w["w_gate_up"][l]).T
        hmid = round_storage(silu(gu[:, :F]) * gu[:, F:], dt)
        X = res(X + hmid @ from_storage(w["w_down"][l]).T)
        taps[l] = round_storage(X, dt)
    Z = round_storage(rms_norm(X, from_storage(w["final_norm"]), cfg.rms_eps), dt)
    T = np.concatenate([taps[l] for l in tap_layers], axis=1) if len(tap_layers) else np.zeros((n, 0))
    return Z, T, Kb, Vb


def greedy_decode(target: TinyTarget, prompt: Sequence[int], n_new: int) -> np.ndarray:
    """Plain greedy decoding: ``n_new`` tokens, the first one from the prefill."""
    target.reset()
    logits, _ = target.run(prompt, 0)
    out = [int(np.argmax(logits[-1]))]
    while len(out) < n_new:
        lg, _ = target.step(out[-1], len(prompt) + len(out) - 1)
        out.append(int(np.argmax(lg)))
    return np.array(out, dtype=np.int32)


def spec_decode(target: TinyTarget, drafter, prompt: Sequence[int], n_new: int,
                feat_dtype: str) -> Tuple[np.ndarray, List[int]]:
    """Greedy speculative decoding with a block drafter.

    ``drafter`` provides ``inject(feats [n, L*H], pos [n])`` and
    ``draft(anchor) -> ids [B-1]`` for one sequence whose context length
    advances by the injected positions.  Target taps are handed over in the
    drafter's storage type ``feat_dtype`` ("f32" or "bf16").  Returns the
    ``n_new`` new tokens and the acceptance length of every cycle.
    """
    B = target.cfg.block_size
    target.reset()
    P = len(prompt)
    logits, taps = target.run(prompt, 0)
    drafter.inject(round_storage(taps, feat_dtype), np.arange(P))
    out = [int(np.argmax(logits[-1]))]
    taus: List[int] = []
    p = P                                            # position of the anchor
    while len(out) < n_new:
        anchor = out[-1]
        d = [int(t) for t in drafter.draft(anchor)]
        assert len(d) == B - 1
        logits, taps = target.run([anchor] + d, p)   # verify block, positions p..p+B-1
        y = [int(np.argmax(row)) for row in logits]  # y_1..y_B
        tau, bonus = accept_len(d, y)
        taus.append(tau)
        out.extend(d[:tau - 1])
        out.append(bonus)
        target.truncate(p + tau)                     # keep anchor + accepted drafts
        drafter.inject(round_storage(taps[:tau], feat_dtype), np.arange(p, p + tau))
        p += tau
    return np.array(out[:n_new], dtype=np.int32), taus
