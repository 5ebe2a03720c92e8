"""Pins of the temperature > 0 oracle (``oracle/sampling.py``) to facts outside
it: the generator's published known-answer vectors, the distribution a
Gumbel-max draw must have, the output distribution of speculative sampling
(the target's own, position by position), its greedy limit at T -> 0, and the
cases whose outcome is forced (identical draft and target, residual support).
"""
from pathlib import Path

import numpy as np
import pytest

from oracle import drafter as D
from oracle import sampling as P

GOLDEN = Path(__file__).parent / "golden"


def test_philox_known_answers():
    rows = 0
    for line in (GOLDEN / "philox4x32_10_kat.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        ctr, key, out = (part.split() for part in line.split("|"))
        got = P.philox4x32_10(np.array([int(x, 16) for x in ctr]), tuple(int(x, 16) for x in key))
        assert [int(x) for x in got] == [int(x, 16) for x in out], line
        rows += 1
    assert rows == 3


def test_uniforms_open_interval_and_float32_exact():
    u = P.uniforms(0x1234_5678_9ABC_DEF0, 7, 3, 11, np.arange(4096))
    assert np.all(u > 0) and np.all(u < 1)
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)
    # counters differ in every field: column, row, offset, tag and seed
    base = P.uniforms(5, 0, 0, 0, np.arange(64))
    for other in (P.uniforms(5, 1, 0, 0, np.arange(64)), P.uniforms(5, 0, 1, 0, np.arange(64)),
                  P.uniforms(5, 0, 0, 1, np.arange(64)), P.uniforms(6, 0, 0, 0, np.arange(64)),
                  P.uniforms(5 + (1 << 32), 0, 0, 0, np.arange(64))):
        assert not np.any(other == base)
    assert len(np.unique(base)) == 64


def freq_ok(samples, probs, what):
    """Empirical frequencies within 4.5 standard errors of the probabilities."""
    n = len(samples)
    counts = np.bincount(samples, minlength=len(probs)) / n
    se = np.sqrt(np.maximum(probs * (1 - probs), 1e-12) / n)
    z = np.abs(counts - probs) / se
    assert z.max() < 4.5, f"{what}: freq {counts} vs {probs} (z {z.max():.2f})"


def test_gumbel_max_draws_follow_the_softmax():
    z = np.array([1.0, -0.5, 0.3, 2.0, 0.0])
    T = 0.7
    ids = np.array([P.sample_row(z, T, 99, 0, 0, r) for r in range(12000)])
    freq_ok(ids, np.exp(P.log_softmax(z, T)), "Gumbel-max")


def test_speculative_sampling_outputs_the_target_distribution():
    """Each emitted position has the target's distribution, whatever the drafter's
    (B = 3, V = 4; the target's rows do not depend on the prefix here)."""
    rng = np.random.default_rng(0)
    T = 1.0
    zt = rng.normal(size=(3, 4)) * 1.5
    zd = rng.normal(size=(2, 4)) * 1.5
    first, second, third = [], [], []
    for t in range(12000):
        d = [P.sample_row(zd[i], T, 1000 + t, 0, 0, i) for i in range(2)]
        last = P.sample_row(zt[2], T, 1000 + t, 1, 0, 2)
        tau, bonus = P.accept_sample(zd, d, zt, last, T, 1000 + t, 0, 0)
        out = d[:tau - 1] + [bonus]
        first.append(out[0])
        if tau >= 2:
            second.append(out[1])
        if tau == 3:
            third.append(out[2])
    p = np.exp(P.log_softmax(zt, T))
    freq_ok(np.array(first), p[0], "position 1")
    freq_ok(np.array(second), p[1], "position 2 | d_1 accepted")
    freq_ok(np.array(third), p[2], "position 3 | all accepted")
    # and the drafts are neither always kept nor always dropped
    assert 0.1 < len(second) / len(first) < 0.95


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_zero_temperature_limit_is_greedy_verify(seed):
    """At T -> 0, p and q are one-hot at the argmax: a draft is kept exactly when
    it equals the target's greedy token, and the residual is the target's token."""
    rng = np.random.default_rng(seed)
    B, V, T = 6, 40, 1e-3
    for trial in range(30):
        zt = rng.normal(size=(B, V))
        y = rng.integers(0, V, size=B)
        zt[np.arange(B), y] = zt.max(axis=1) + 0.5            # top-2 gaps >> T: one-hot softmax
        d = np.where(rng.random(B - 1) < 0.6, y[:B - 1], rng.integers(0, V, size=B - 1))
        zd = rng.normal(size=(B - 1, V))
        zd[np.arange(B - 1), d] = zd.max(axis=1) + 0.5
        tau, bonus = P.accept_sample(zd, d, zt, int(y[-1]), T, seed, trial, 0)
        assert (tau, bonus) == D.accept_len(d, y), (trial, d, y)


def test_identical_draft_and_target_accept_everything():
    rng = np.random.default_rng(3)
    B, V = 8, 50
    for t in range(20):
        z = rng.normal(size=(B, V)) * 3
        d = [P.sample_row(z[i], 0.8, t, 0, 0, i) for i in range(B - 1)]
        tau, bonus = P.accept_sample(z[:B - 1], d, z, 17, 0.8, t, 0, 0)
        assert (tau, bonus) == (B, 17)


def test_residual_draw_is_where_the_target_exceeds_the_draft():
    rng = np.random.default_rng(4)
    V, T = 30, 1.3
    hits = 0
    for t in range(200):
        zt, zd = rng.normal(size=(2, V)), rng.normal(size=(1, V)) * 2
        d = [P.sample_row(zd[0], T, t, 0, 0, 0)]
        tau, bonus = P.accept_sample(zd, d, zt, 0, T, t, 0, 0)
        if tau == 1:
            p, q = np.exp(P.log_softmax(zt[0], T)), np.exp(P.log_softmax(zd[0], T))
            assert p[bonus] > q[bonus]
            hits += 1
    assert hits > 20


@pytest.mark.parametrize("seed", [0, 1])
def test_speculative_sampling_loop_at_zero_temperature_is_greedy_decoding(seed):
    """The whole speculative-sampling loop (draws, accept rule, commit and
    inject) at T -> 0 reproduces the target's greedy decoding token for token."""
    import dflash_synth as S
    from oracle import target as T
    cfg = S.get_config("tiny")
    tw = S.target_weights(cfg, seed, layer_std=0.05)
    prompt = S.prompt_ids(cfg, seed)
    greedy = T.greedy_decode(T.TinyTarget(tw, cfg), prompt, cfg.new_tokens)
    out, taus = P.spec_sample(T.TinyTarget(tw, cfg), D.OracleDrafter(S.drafter_weights(cfg, seed), cfg), prompt,
                              cfg.new_tokens, 1e-6, 1234 + seed, cfg.dtype)
    assert np.array_equal(out, greedy)
    assert all(1 <= t <= cfg.block_size for t in taus)
