"""Oracle of lossless verification at temperature > 0.  TEST INFRASTRUCTURE ONLY
(page abbreviations: see the package docstring).

[FN] §1 recalls standard speculative decoding: drafts that pass verification
are kept, and from the first position where they fail the token is drawn again
from the target's distribution, so the output has the distribution of the
target decoding on its own.  The pages give no more detail, so the rule taken
is the published speculative-sampling rule (Leviathan, Kalman and Matias 2023,
the paper [FN] §1 names):

* p_i and q_i are the target's and the drafter's distributions for position
  p+i at temperature T: softmax(z / T) of their logits z;
* draft d_i (drawn from q_i) is accepted when u_i < p_i(d_i) / q_i(d_i), u_i
  uniform on (0, 1), scanning i = 1, 2, ... in order;
* at the first rejection the token is drawn from the residual distribution
  max(0, p_i - q_i) / sum(max(0, p_i - q_i)); when every draft is accepted the
  extra token is drawn from p_B.

The drafter's q_i at position p+i does not depend on the drafts before it (one
pass fills the whole block, [FN] §2, §7); the rule stays exact because it only
needs d_i to be drawn from the q_i it is tested against.

Random numbers: every draw comes from one counter-based generator, Philox4x32-10
(Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC 2011), keyed by a 64-bit seed, with the counter (column / 4, row, offset,
tag) and word column mod 4.  A 32-bit word w gives u = (floor(w / 2^9) + 1/2) *
2^-23, exactly representable in float32 and float64, in (0, 1).  Categorical
draws use the Gumbel-max rule: argmax_v (log weight_v - log(-log u_v)), lowest
id on ties.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .numerics import round_storage

M0, M1 = 0xD2511F53, 0xCD9E8D57          # Philox4x32 multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85          # Weyl key increments
MASK32 = 0xFFFFFFFF

# tags the accept rule draws with (the caller's sampling uses other tags)
TAG_ACCEPT = 0xFFFFFFFE
TAG_RESIDUAL = 0xFFFFFFFF
# tags of the speculative loop below: drafts, the target's rows, the prefill's token
TAG_DRAFT, TAG_TARGET, TAG_PREFILL = 0, 1, 2


def philox4x32_10(ctr: np.ndarray, key: Tuple[int, int]) -> np.ndarray:
    """Philox4x32 with 10 rounds on counters ctr [..., 4] (uint32 values).

    One round: (hi0, lo0) = M0 * c0, (hi1, lo1) = M1 * c2 as 64-bit products;
    the new counter is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0).  The key
    (k0, k1) grows by (W0, W1) mod 2^32 between rounds.
    """
    c = np.asarray(ctr, dtype=np.uint64) & np.uint64(MASK32)
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = int(key[0]) & MASK32, int(key[1]) & MASK32
    m32 = np.uint64(MASK32)
    for rnd in range(10):
        if rnd:
            k0, k1 = (k0 + W0) & MASK32, (k1 + W1) & MASK32
        p0 = np.uint64(M0) * c0
        p1 = np.uint64(M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & m32
        hi1, lo1 = p1 >> np.uint64(32), p1 & m32
        c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def seed_key(seed: int) -> Tuple[int, int]:
    return seed & MASK32, (seed >> 32) & MASK32


def uniforms(seed: int, tag: int, offset: int, row: int, cols: np.ndarray) -> np.ndarray:
    """u in (0, 1) for the given columns of one row (float64, exact)."""
    cols = np.asarray(cols, dtype=np.int64)
    ctr = np.stack([cols >> 2, np.full_like(cols, row), np.full_like(cols, offset), np.full_like(cols, tag)],
                   axis=-1)
    words = philox4x32_10(ctr, seed_key(seed))
    w = words[np.arange(len(cols)), cols & 3].astype(np.int64)
    return ((w >> 9).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel(u: np.ndarray) -> np.ndarray:
    return -np.log(-np.log(u))


def log_softmax(z: np.ndarray, T: float) -> np.ndarray:
    """log softmax(z / T) along the last axis (float64)."""
    x = np.asarray(z, dtype=np.float64) / T
    m = x.max(axis=-1, keepdims=True)
    return x - (m + np.log(np.exp(x - m).sum(axis=-1, keepdims=True)))


def logsumexp(z: np.ndarray, T: float) -> np.ndarray:
    x = np.asarray(z, dtype=np.float64) / T
    m = x.max(axis=-1)
    return m + np.log(np.exp(x - m[..., None]).sum(axis=-1))


def sample_row(z: np.ndarray, T: float, seed: int, tag: int, offset: int, row: int) -> int:
    """One draw from softmax(z / T) by the Gumbel-max rule."""
    key = np.asarray(z, dtype=np.float64) / T + gumbel(uniforms(seed, tag, offset, row, np.arange(len(z))))
    return int(np.argmax(key))


def sample_rows(Z: np.ndarray, T: float, seed: int, tag: int, offset: int) -> Tuple[np.ndarray, np.ndarray]:
    """Row r of Z [rows, V] is drawn with counter row r.  Returns (ids, lse of Z / T)."""
    ids = np.array([sample_row(Z[r], T, seed, tag, offset, r) for r in range(len(Z))], dtype=np.int32)
    return ids, logsumexp(Z, T)


def residual_sample(zt: np.ndarray, zd: np.ndarray, T: float, seed: int, offset: int, s: int) -> int:
    """One draw from max(0, p - q), normalised (p = softmax(zt / T), q = softmax(zd / T))."""
    r = np.maximum(0.0, np.exp(log_softmax(zt, T)) - np.exp(log_softmax(zd, T)))
    with np.errstate(divide="ignore"):
        key = np.log(r) + gumbel(uniforms(seed, TAG_RESIDUAL, offset, s, np.arange(len(zt))))
    return int(np.argmax(key))


def accept_sample(draft_logits: np.ndarray, draft_ids, target_logits: np.ndarray, target_last_id: int,
                  T: float, seed: int, offset: int, s: int) -> Tuple[int, int]:
    """Acceptance length and the next token of one block at temperature T.

    draft_logits [B-1, V]: the drafter's logits for positions p+1..p+B-1;
    draft_ids: d_1..d_{B-1}, drawn from them; target_logits [B, V]: the
    target's logits for positions p+1..p+B (verify rows 0..B-1);
    target_last_id: the token drawn from the target's last row, taken when
    every draft is accepted; s: the sequence's counter row.
    Returns (tau in [1, B], the token at position p + tau).
    """
    bm1 = len(draft_ids)
    assert draft_logits.shape[0] == bm1 and target_logits.shape[0] == bm1 + 1
    u = uniforms(seed, TAG_ACCEPT, offset, s, np.arange(bm1))
    for i in range(bm1):
        d = int(draft_ids[i])
        p = np.exp(log_softmax(target_logits[i], T)[d])
        q = np.exp(log_softmax(draft_logits[i], T)[d])
        if not u[i] < p / q:
            return i + 1, residual_sample(target_logits[i], draft_logits[i], T, seed, offset, s)
    return bm1 + 1, int(target_last_id)


def spec_sample(target, drafter, prompt: Sequence[int], n_new: int, T: float, seed: int,
                feat_dtype: str) -> Tuple[np.ndarray, List[int]]:
    """Speculative sampling with a block drafter at temperature T ([FN] §1, §2).

    As the greedy loop (``target.spec_decode``), with draws in place of
    argmaxes: the prefill's token is drawn from its last row (tag TAG_PREFILL,
    offset 0, row 0); in cycle c (offset c) the drafts are drawn from the
    drafter's rows (tag TAG_DRAFT, row i), the target's rows are drawn (tag
    TAG_TARGET, row i; the last one is the token taken when every draft is
    kept), and ``accept_sample`` (sequence row 0) decides.  ``drafter``
    provides ``inject(feats, pos)`` and ``draft_logits(anchor) -> [B-1, V]``.
    """
    B = target.cfg.block_size
    target.reset()
    P = len(prompt)
    logits, taps = target.run(prompt, 0)
    drafter.inject(round_storage(taps, feat_dtype), np.arange(P))
    out = [sample_row(logits[-1], T, seed, TAG_PREFILL, 0, 0)]
    taus: List[int] = []
    p, c = P, 0
    while len(out) < n_new:
        anchor = out[-1]
        zd = drafter.draft_logits(anchor)
        d, _ = sample_rows(zd, T, seed, TAG_DRAFT, c)
        zt, taps = target.run([anchor] + [int(t) for t in d], p)
        y, _ = sample_rows(zt, T, seed, TAG_TARGET, c)
        tau, bonus = accept_sample(zd, d, zt, int(y[B - 1]), T, seed, c, 0)
        taus.append(tau)
        out.extend(int(t) for t in d[:tau - 1])
        out.append(bonus)
        target.truncate(p + tau)
        drafter.inject(round_storage(taps[:tau], feat_dtype), np.arange(p, p + tau))
        p += tau
        c += 1
    return np.array(out[:n_new], dtype=np.int32), taus
