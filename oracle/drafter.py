"""Oracle of the DFlash drafter: context injection, one-pass block draft, shared
LM head argmax and greedy accept length.  TEST INFRASTRUCTURE ONLY (see the
package docstring for the page abbreviations [FN], [INS], [SUM], [PKR]).

Rounding points (storage type ``dt`` = bf16, or fp32 in the tiny
configuration): the fused context feature c, the RMSNorm outputs, q/k/v after
RoPE, the attention output, the SwiGLU product and the final hidden state are
rounded to ``dt``; the residual stream is fp32; everything else is float64.

Readings of points the pages leave open (each listed in the design notes):
* the block is the anchor followed by B-1 mask tokens; B counts the anchor,
  and mask row j predicts the token at position p+j (no shift);
* the mask token is the last vocabulary row of the shared embedding;
* absolute positions continue the target's: context 0..p-1, block p..p+B-1;
  RoPE pairs dimension i with i + d/2, inverse frequency theta^(-2i/d);
* the lightweight projection is one bias-free linear map of the concatenated
  features; each layer's own K and V projections are applied to it directly;
* query head h reads KV head floor(h / (nq/nkv));
* the drafter has its own final RMSNorm; argmax ties go to the lowest id.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .numerics import from_storage, round_f32, round_storage


# ----------------------------------------------------------------------------
# primitives
# ----------------------------------------------------------------------------
def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary position embedding of ``x [n, heads, d]`` at positions ``pos [n]``.

    Dimension i is rotated together with i + d/2 by the angle pos * theta^(-2i/d).
    """
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              causal_from: Optional[int] = None) -> np.ndarray:
    """Softmax attention of queries ``q [M, nq, d]`` over keys/values ``[T, nkv, d]``.

    No mask: every query sees every key (the in-block attention is non-causal,
    [FN] §6).  Query head h uses KV head floor(h / (nq/nkv)).  ``causal_from``
    (tests only) lets query row i see keys [0, causal_from + i] instead.
    """
    M, nq, d = q.shape
    T, nkv, _ = k.shape
    group = nq // nkv
    out = np.empty((M, nq, d), dtype=np.float64)
    for h in range(nq):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(d)
        if causal_from is not None:
            allowed = np.arange(T)[None, :] <= (causal_from + np.arange(M))[:, None]
            s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


def _w(a) -> np.ndarray:
    return from_storage(a)


# ----------------------------------------------------------------------------
# A1 + A2: feature fusion and KV injection
# ----------------------------------------------------------------------------
def fuse_context(w: dict, cfg, feats: np.ndarray) -> np.ndarray:
    """Context feature c = W_fc f of the concatenated target-layer features.

    The hidden states of several uniformly spaced target layers are
    concatenated and fused by a lightweight projection ([INS]; [SUM] §2.2).
    Returns c ``[n, H]`` rounded to the storage type.  With ``cfg.ctx_norm``
    the projection is followed by an RMSNorm with gain ``w["ctx_norm"]``
    (an option; the pages name only the projection), rounded once after it.
    """
    f = _w(feats)
    c = f @ _w(w["w_fc"]).T
    if getattr(cfg, "ctx_norm", 0):
        c = rms_norm(c, _w(w["ctx_norm"]), cfg.rms_eps)
    return round_storage(c, cfg.dtype)


def inject(w: dict, cfg, feats: np.ndarray, pos: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """KV injection: every drafter layer's K and V projections applied to c.

    The fused context feature enters the Key/Value projections of every drafter
    layer and is kept in the drafter's KV cache ([FN] §2 KV injection;
    [SUM] §2.2).  K gets RoPE at the context position.  Returns K, V
    ``[n_layers, n, nkv, d]`` rounded to the storage type.
    """
    c = fuse_context(w, cfg, feats)
    n = c.shape[0]
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    K = np.empty((cfg.n_layers, n, nkv, d))
    V = np.empty((cfg.n_layers, n, nkv, d))
    for l in range(cfg.n_layers):
        wqkv = _w(w["w_qkv"][l])
        wk = wqkv[nq * d:(nq + nkv) * d]
        wv = wqkv[(nq + nkv) * d:]
        k = (c @ wk.T).reshape(n, nkv, d)
        K[l] = round_storage(rope(k, pos, cfg.rope_theta), cfg.dtype)
        V[l] = round_storage((c @ wv.T).reshape(n, nkv, d), cfg.dtype)
    return K, V


# ----------------------------------------------------------------------------
# A3 .. A8: one drafter pass over the block
# ----------------------------------------------------------------------------
def draft_block(w: dict, cfg, anchor: int, K_ctx: np.ndarray, V_ctx: np.ndarray,
                use_rope: bool = True, causal: bool = False,
                positions: Optional[np.ndarray] = None) -> np.ndarray:
    """One forward pass of the drafter over [anchor, mask x (B-1)].

    The last accepted token is the anchor, the B-1 following slots are masked,
    and one pass predicts all of them in parallel ([FN] §2 cycle; [FN] §7 and
    [SUM] §2.2: a single step, not multi-step denoising).  Attention covers the
    injected context K/V (positions 0..p-1) and the block's own K/V, without a
    mask ([FN] §6).  Each layer: pre-norm attention, then a pre-norm SwiGLU MLP,
    both with residual connections.

    ``K_ctx, V_ctx`` are ``[n_layers, p, nkv, d]``.  Returns the final-norm
    hidden states of the mask rows, ``Z [B-1, H]``, rounded to the storage type.
    ``use_rope``, ``causal`` and ``positions`` exist for the oracle's own
    invariance tests.
    """
    dt = cfg.dtype
    B, H = cfg.block_size, cfg.hidden
    nq, nkv, d, F = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn
    p = K_ctx.shape[1]
    W = getattr(cfg, "window", 0)
    if W and p > W:
        # sliding-window context: only the last W positions are attended; the
        # block keeps its absolute positions p .. p+B-1 ([PKR] usage notes:
        # long-context inference with a sliding-window KV cache)
        K_ctx, V_ctx = K_ctx[:, p - W:], V_ctx[:, p - W:]
    pc = K_ctx.shape[1]
    ids = np.array([anchor] + [cfg.mask_token_id] * (B - 1), dtype=np.int64)
    pos = np.arange(p, p + B) if positions is None else np.asarray(positions)
    res = (lambda a: a) if dt == "f64" else round_f32   # fp32 residual stream
    X = res(_w(w["embed"][ids]))
    for l in range(cfg.n_layers):
        Y = round_storage(rms_norm(X, _w(w["attn_norm"][l]), cfg.rms_eps), dt)
        qkv = Y @ _w(w["w_qkv"][l]).T
        q = qkv[:, :nq * d].reshape(B, nq, d)
        k = qkv[:, nq * d:(nq + nkv) * d].reshape(B, nkv, d)
        v = qkv[:, (nq + nkv) * d:].reshape(B, nkv, d)
        if use_rope:
            q = rope(q, pos, cfg.rope_theta)
            k = rope(k, pos, cfg.rope_theta)
        q, k, v = round_storage(q, dt), round_storage(k, dt), round_storage(v, dt)
        Kall = np.concatenate([K_ctx[l], k], axis=0)
        Vall = np.concatenate([V_ctx[l], v], axis=0)
        O = round_storage(attention(q, Kall, Vall, causal_from=pc if causal else None), dt)
        X = res(X + O.reshape(B, nq * d) @ _w(w["w_o"][l]).T)
        Y = round_storage(rms_norm(X, _w(w["mlp_norm"][l]), cfg.rms_eps), dt)
        gu = Y @ _w(w["w_gate_up"][l]).T
        hmid = round_storage(silu(gu[:, :F]) * gu[:, F:], dt)
        X = res(X + hmid @ _w(w["w_down"][l]).T)
    return round_storage(rms_norm(X[1:], _w(w["final_norm"]), cfg.rms_eps), dt)


# ----------------------------------------------------------------------------
# A9: shared LM head and argmax
# ----------------------------------------------------------------------------
def lm_logits(lm_head: np.ndarray, Z: np.ndarray, chunk: int = 16384) -> np.ndarray:
    """Logits Z W_lm^T in float64 with the target's shared, frozen LM head
    ([FN] §3.1; [SUM] §2.3)."""
    Z = _w(Z)
    V = lm_head.shape[0]
    out = np.empty((Z.shape[0], V))
    for a in range(0, V, chunk):
        out[:, a:a + chunk] = Z @ _w(lm_head[a:a + chunk]).T
    return out


def lm_argmax(lm_head: np.ndarray, Z: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Greedy ids (lowest id on exact ties), their logits, and all logits."""
    logits = lm_logits(lm_head, Z)
    ids = np.argmax(logits, axis=1)          # first maximum = lowest id
    return ids.astype(np.int32), logits[np.arange(len(ids)), ids], logits


# ----------------------------------------------------------------------------
# A10: greedy verify
# ----------------------------------------------------------------------------
def accept_len(draft: Sequence[int], target: Sequence[int]) -> Tuple[int, int]:
    """Acceptance length and bonus token of one block under greedy verify.

    Drafts are kept up to the first position where the target disagrees, and
    the target's own token is taken there ([FN] §1, §2 box (b)).  ``draft`` is
    d_1..d_{B-1}; ``target`` is y_1..y_B, the target's greedy token for each of
    the same positions plus one more.  Returns tau = (matched prefix) + 1, in
    [1, B], and the bonus y_tau.
    """
    bm1 = len(draft)
    assert len(target) == bm1 + 1
    k = 0
    while k < bm1 and int(draft[k]) == int(target[k]):
        k += 1
    return k + 1, int(target[k])


def accept_len_batch(draft: np.ndarray, target: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    res = [accept_len(d, y) for d, y in zip(draft, target)]
    return (np.array([r[0] for r in res], dtype=np.int32),
            np.array([r[1] for r in res], dtype=np.int32))


# ----------------------------------------------------------------------------
# stateful drafter used by the speculative loop
# ----------------------------------------------------------------------------
class OracleDrafter:
    """Drafter with a dense per-sequence context cache (one sequence)."""

    def __init__(self, w: dict, cfg):
        self.w, self.cfg = w, cfg
        shape = (cfg.n_layers, 0, cfg.n_kv_heads, cfg.head_dim)
        self.K = np.zeros(shape)
        self.V = np.zeros(shape)

    @property
    def ctx_len(self) -> int:
        return self.K.shape[1]

    def inject(self, feats: np.ndarray, pos: np.ndarray) -> None:
        assert np.array_equal(pos, np.arange(self.ctx_len, self.ctx_len + len(pos)))
        K, V = inject(self.w, self.cfg, feats, pos)
        self.K = np.concatenate([self.K, K], axis=1)
        self.V = np.concatenate([self.V, V], axis=1)

    def draft(self, anchor: int) -> np.ndarray:
        Z = draft_block(self.w, self.cfg, anchor, self.K, self.V)
        ids, _, _ = lm_argmax(self.w["lm_head"], Z)
        return ids

    def draft_logits(self, anchor: int) -> np.ndarray:
        return lm_logits(self.w["lm_head"], draft_block(self.w, self.cfg, anchor, self.K, self.V))
