"""Verification at temperature > 0 on the GPU (``dflash_sample``,
``dflash_accept_sample``) against ``oracle/sampling.py`` on the same seeded
logits and the same Philox streams.

Token ids and accept lengths must match exactly, except where the oracle's own
decision is a near-tie at fp32 resolution (a Gumbel-max key within 1e-4 of the
best, or an acceptance ratio within 1e-4 of its uniform); log-sum-exp values
within 1e-5 (scaled by max(1, |lse|)).
"""
import numpy as np
import pytest

from gpu_cases import assert_close, log
from oracle import sampling as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_gemm_amd import _lib
    _lib.load()


def runtime():
    from block_diffusion_drafter_gemm_amd import runtime as R
    return R


def gumbel_keys(z, T, seed, tag, offset, row):
    return np.asarray(z, np.float64) / T + P.gumbel(P.uniforms(seed, tag, offset, row, np.arange(len(z))))


def check_draw(got, want, keys, what):
    if got == want:
        return 0
    assert 0 <= got < len(keys), (what, got)
    assert keys[got] >= keys[want] - TOL * max(1.0, abs(keys[want])), \
        f"{what}: gpu {got} (key {keys[got]:.6f}) vs oracle {want} (key {keys[want]:.6f})"
    return 1


@pytest.mark.parametrize("rows,vocab,T", [(7, 1, 1.0), (5, 5, 0.6), (9, 4097, 1.0), (3, 12345, 0.35),
                                          (40, 151936, 1.0), (300, 60001, 0.9), (9, 4097, 0.05)])
def test_sample_matches_oracle(rows, vocab, T):
    log(f"sample rows={rows} vocab={vocab} T={T}")
    rng = np.random.default_rng(vocab + rows)
    Z = (rng.normal(size=(rows, vocab)) * 2.0).astype(np.float32)
    seed, offset, tag = 0x5EED_0000_0001 + vocab, 3, 0
    ids, lse = runtime().Drafter.sample(torch.from_numpy(Z).cuda(), T, seed, offset, tag)
    ids, lse = ids.cpu().numpy(), lse.cpu().numpy()
    ids_o, lse_o = P.sample_rows(Z, T, seed, tag, offset)
    assert_close(lse, lse_o, 1e-5, "lse")
    ex = sum(check_draw(int(ids[r]), int(ids_o[r]), gumbel_keys(Z[r], T, seed, tag, offset, r), f"row {r}")
             for r in range(rows))
    log(f"  {rows - ex}/{rows} draws identical, {ex} tie-excused")
    # a different offset or tag changes the draws (vocabularies with room to differ)
    if vocab > 1000:
        ids2, _ = runtime().Drafter.sample(torch.from_numpy(Z).cuda(), T, seed, offset + 1, tag)
        assert not np.array_equal(ids2.cpu().numpy(), ids)


def make_block_logits(rng, batch, B, V, agree):
    """Drafter and target logits that agree to a degree, and drafts that are
    mostly the drafter's likely tokens."""
    zt = (rng.normal(size=(batch * B, V)) * 2.5).astype(np.float32)
    zd = (zt.reshape(batch, B, V)[:, :B - 1].reshape(-1, V) * agree
          + rng.normal(size=(batch * (B - 1), V)) * 2.5 * (1 - agree)).astype(np.float32)
    top = np.argsort(-zd, axis=1)[:, :4]
    d = top[np.arange(len(top)), rng.integers(0, 4, size=len(top))].astype(np.int32)
    return zd, zt, d.reshape(batch, B - 1)


@pytest.mark.parametrize("batch,B,V,T,agree", [(40, 4, 3000, 1.0, 0.9), (24, 16, 5000, 0.7, 0.97),
                                               (16, 16, 40000, 1.0, 0.99), (8, 2, 300, 1.5, 0.5),
                                               (20, 8, 2001, 0.2, 0.995)])
def test_accept_sample_matches_oracle(batch, B, V, T, agree):
    log(f"accept_sample batch={batch} B={B} V={V} T={T}")
    R = runtime()
    rng = np.random.default_rng(B * 1000 + V)
    zd, zt, d = make_block_logits(rng, batch, B, V, agree)
    seed, offset = 77 + V, 5
    dz, tz = torch.from_numpy(zd).cuda(), torch.from_numpy(zt).cuda()
    _, dlse = R.Drafter.sample(dz, T, seed, offset, 0)
    tids, tlse = R.Drafter.sample(tz, T, seed, offset, 1)
    tau, bonus = R.Drafter.accept_sample(dz, dlse, torch.from_numpy(d).cuda(), tz, tlse, tids, B, T, seed, offset)
    tau, bonus = tau.cpu().numpy(), bonus.cpu().numpy()
    tids_o, _ = P.sample_rows(zt, T, seed, 1, offset)
    zd3, zt3 = zd.reshape(batch, B - 1, V), zt.reshape(batch, B, V)
    excused = 0
    for s in range(batch):
        t_o, b_o = P.accept_sample(zd3[s], d[s], zt3[s], tids_o[s * B + B - 1], T, seed, offset, s)
        u = P.uniforms(seed, P.TAG_ACCEPT, offset, s, np.arange(B - 1))
        if tau[s] != t_o:                       # only at an acceptance near-tie
            i = min(tau[s], t_o) - 1
            ratio = np.exp(P.log_softmax(zt3[s, i], T)[d[s, i]] - P.log_softmax(zd3[s, i], T)[d[s, i]])
            assert abs(u[i] - ratio) <= TOL * max(1.0, ratio), (s, tau[s], t_o, u[i], ratio)
            excused += 1
            continue
        if t_o == B:
            excused += check_draw(int(bonus[s]), int(b_o), gumbel_keys(zt3[s, B - 1], T, seed, 1, offset,
                                                                       s * B + B - 1), f"seq {s} bonus")
        else:
            k = t_o - 1
            r = np.maximum(0.0, np.exp(P.log_softmax(zt3[s, k], T)) - np.exp(P.log_softmax(zd3[s, k], T)))
            with np.errstate(divide="ignore"):
                keys = np.log(r) + P.gumbel(P.uniforms(seed, P.TAG_RESIDUAL, offset, s, np.arange(V)))
            excused += check_draw(int(bonus[s]), int(b_o), keys, f"seq {s} residual")
    log(f"  taus {np.bincount(tau, minlength=B + 1)[1:]}, {excused} tie-excused")
    assert excused <= max(1, batch // 10)
    assert len(set(tau.tolist())) > 1 or B == 2


def test_accept_sample_block_len_and_zero_batch():
    R = runtime()
    rng = np.random.default_rng(11)
    batch, B, V, T = 12, 8, 700, 1.0
    zd, zt, d = make_block_logits(rng, batch, B, V, 0.95)
    seed, offset = 1234, 0
    dz, tz = torch.from_numpy(zd).cuda(), torch.from_numpy(zt).cuda()
    _, dlse = R.Drafter.sample(dz, T, seed, offset, 0)
    tids, tlse = R.Drafter.sample(tz, T, seed, offset, 1)
    bl = np.array([8, 1, 2, 5, 8, 3, 4, 7, 6, 2, 9, 0], dtype=np.int32)
    tau, bonus = R.Drafter.accept_sample(dz, dlse, torch.from_numpy(d).cuda(), tz, tlse, tids, B, T, seed, offset,
                                         block_len=torch.from_numpy(bl).cuda())
    tau, bonus = tau.cpu().numpy(), bonus.cpu().numpy()
    tids_o, _ = P.sample_rows(zt, T, seed, 1, offset)
    for s in range(batch):
        bs = min(max(int(bl[s]), 1), B)
        t_o, b_o = P.accept_sample(zd.reshape(batch, B - 1, V)[s, :bs - 1], d[s, :bs - 1],
                                   zt.reshape(batch, B, V)[s, :bs], tids_o[s * B + bs - 1], T, seed, offset, s)
        assert 1 <= tau[s] <= bs
        assert (tau[s], bonus[s]) == (t_o, b_o), (s, bs)
    z = torch.zeros(0, dtype=torch.int32, device="cuda")
    t0, b0 = R.Drafter.accept_sample(dz[:0], dlse[:0], z.view(0, B - 1), tz[:0], tlse[:0], z, B, T, seed, offset)
    assert t0.numel() == 0 and b0.numel() == 0


def test_accept_sample_rejects_ids_outside_the_vocabulary():
    """A draft id outside [0, V) is rejected at its position; the next token is
    then the residual draw there (compared with the oracle's residual draw)."""
    R = runtime()
    rng = np.random.default_rng(21)
    batch, B, V, T = 6, 5, 900, 1.0
    zd, zt, d = make_block_logits(rng, batch, B, V, 0.9)
    d[:, 0] = np.array([-1, V, V + 5, -7, 2 ** 30, -(2 ** 31)], dtype=np.int32)
    seed, offset = 99, 4
    dz, tz = torch.from_numpy(zd).cuda(), torch.from_numpy(zt).cuda()
    _, dlse = R.Drafter.sample(dz, T, seed, offset, 0)
    tids, tlse = R.Drafter.sample(tz, T, seed, offset, 1)
    tau, bonus = R.Drafter.accept_sample(dz, dlse, torch.from_numpy(d).cuda(), tz, tlse, tids, B, T, seed, offset)
    tau, bonus = tau.cpu().numpy(), bonus.cpu().numpy()
    assert np.all(tau == 1)
    zd3, zt3 = zd.reshape(batch, B - 1, V), zt.reshape(batch, B, V)
    for s in range(batch):
        assert bonus[s] == P.residual_sample(zt3[s, 0], zd3[s, 0], T, seed, offset, s), s
