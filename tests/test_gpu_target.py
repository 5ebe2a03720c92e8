"""Target verify on the GPU (``dflash_target_verify``): the causal target pass
that checks a drafted block and taps the target's hidden states, against the
oracle's tiny target; then greedy speculative decoding with drafter and target
both on the GPU, which must reproduce the GPU target's own greedy decoding token
for token (and the oracle's, up to logit near-ties).

The tiny configuration is fp32 (4-layer target, taps after layers 1, 2, 3,
2-layer drafter, B = 4, a 64-token prompt, 32 new tokens).
"""
import dataclasses

import numpy as np
import pytest
import torch

import dflash_synth as S
from gpu_cases import MINI, assert_close, check_ids, log
from oracle import drafter as D
from oracle import sampling as P
from oracle import target as T

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_gemm_amd import _lib
    _lib.load()


def runtime():
    from block_diffusion_drafter_gemm_amd import runtime as R
    return R


def target_cfg(cfg, B):
    return dataclasses.replace(cfg, n_layers=cfg.target_layers, block_size=B)


class GpuTarget:
    """The tiny target behind the C ABI: one handle per block size (prefill,
    verify, one-token decode) over shared weights and one paged cache."""

    def __init__(self, cfg, w, capacity, blocks):
        R = runtime()
        self.R, self.cfg = R, cfg
        self.taps = list(cfg.feat_layer_ids)
        self.h = {B: R.Drafter(target_cfg(cfg, B), w, max_batch=1, max_ctx=capacity, max_new=1) for B in blocks}
        big = target_cfg(cfg, max(blocks))
        lay = S.paged_layout(big, np.array([capacity]), headroom=max(blocks), seed=5)
        self.kv = R.PagedKV(big, lay.block_table, np.array([0]), lay.n_pages, max_ctx=capacity)
        self.ctx = 0

    def run(self, tokens, pos):
        """Causal pass over ``tokens`` at positions pos.. (pos == committed
        length); returns logits [n, V] (fp32), taps [n, L*H] (storage type)."""
        assert pos == self.ctx
        d = self.h[len(tokens)]
        ids = torch.tensor([list(tokens)], dtype=torch.int32, device="cuda")
        hid, taps = d.target_verify(ids, self.kv, self.taps)
        _, _, lg = d.lmhead_argmax(hid, want_max=False, want_logits=True)
        return lg.cpu().numpy(), self.R.to_host_storage(taps)

    def run_logits(self, tokens, pos):
        """As run, with the logits left on the device (logits-only LM head)."""
        assert pos == self.ctx
        d = self.h[len(tokens)]
        ids = torch.tensor([list(tokens)], dtype=torch.int32, device="cuda")
        hid, taps = d.target_verify(ids, self.kv, self.taps)
        return d.lmhead_logits(hid), self.R.to_host_storage(taps)

    def commit(self, n):
        self.ctx += n
        self.kv.set_ctx_len(np.array([self.ctx]), max_ctx=self.kv.max_ctx)

    def close(self):
        for d in self.h.values():
            d.close()


def test_target_verify_matches_oracle_target():
    """Prefill (64 rows, the many-rows kernels) and a 4-row verify block (the
    streaming kernels): logits and taps against the oracle's float64 target."""
    cfg = MINI["tiny"]
    log("target verify vs oracle target")
    tw = S.target_weights(cfg, 0, layer_std=0.05)
    tgt = T.TinyTarget(tw, cfg)
    prompt = S.prompt_ids(cfg, 0)
    P, B = len(prompt), cfg.block_size
    g = GpuTarget(cfg, tw, P + 2 * B, (P, B))
    lg, taps = g.run(prompt, 0)
    lo, to = tgt.run(prompt, 0)
    assert_close(lg, lo, 1e-4, "prefill logits")
    assert_close(taps, to, 1e-4, "prefill taps")
    g.commit(P)
    block = [int(np.argmax(lo[-1]))] + [int(t) for t in S.prompt_ids(cfg, 1)[:B - 1]]
    lg, taps = g.run(block, P)
    lo, to = tgt.run(block, P)
    assert_close(lg, lo, 1e-4, "verify logits")
    assert_close(taps, to, 1e-4, "verify taps")
    check_ids(lg.argmax(axis=1), lo.argmax(axis=1), lo, 1e-4, "verify ids")
    g.close()


def test_target_verify_is_causal_and_appends_the_cache():
    """Row j of a verify block does not depend on the block tokens after it, and
    the block's K/V land in the cache at positions ctx .. ctx + B - 1."""
    cfg = MINI["tiny"]
    tw = S.target_weights(cfg, 3, layer_std=0.05)
    B = cfg.block_size
    g = GpuTarget(cfg, tw, 16 + 2 * B, (16, B))
    prompt = S.prompt_ids(cfg, 3)[:16]
    g.run(prompt, 0)
    g.commit(16)
    a = [5, 6, 7, 8]
    b = [5, 6, 900, 901]                                 # differs after row 1
    la, _ = g.run(a, 16)
    k_a = g.kv.k.clone()
    lb, _ = g.run(b, 16)
    assert np.array_equal(la[:2], lb[:2]), "rows 0..1 saw later block tokens"
    assert not np.array_equal(la[2:], lb[2:])
    # positions 16, 17 hold the same K in both runs; 18, 19 differ
    tab = g.kv.block_table.cpu().numpy()[0]
    kh_a, kh_b = k_a.cpu().numpy(), g.kv.k.cpu().numpy()
    for pos, same in [(16, True), (17, True), (18, False), (19, False)]:
        pg, sl = tab[pos // 16], pos % 16
        assert np.array_equal(kh_a[:, pg, sl], kh_b[:, pg, sl]) == same, pos
    g.close()


class GpuDrafter:
    """The GPU drafter for the speculative loop (inject, draft)."""

    def __init__(self, cfg, w, max_positions):
        R = runtime()
        self.R, self.cfg = R, cfg
        self.d = R.Drafter(cfg, w, max_batch=1, max_ctx=max_positions, max_new=max_positions)
        lay = S.paged_layout(cfg, np.array([max_positions]), headroom=0, seed=9)
        self.kv = R.PagedKV(cfg, lay.block_table, np.array([0]), lay.n_pages, max_ctx=max_positions)
        self.ctx = 0

    def inject(self, feats, pos):
        f = self.R.to_device(np.ascontiguousarray(feats))
        seq = torch.zeros(len(pos), dtype=torch.int32, device="cuda")
        p = torch.from_numpy(np.asarray(pos, dtype=np.int32)).cuda()
        self.d.inject_context(f, seq, p, self.kv)
        self.ctx += len(pos)
        self.kv.set_ctx_len(np.array([self.ctx]), max_ctx=self.kv.max_ctx)

    def draft(self, anchor):
        hid = self.d.draft_block(torch.tensor([anchor], dtype=torch.int32, device="cuda"), self.kv)
        ids, _, _ = self.d.lmhead_argmax(hid, want_max=False)
        return ids.cpu().numpy()

    def draft_logits(self, anchor):
        hid = self.d.draft_block(torch.tensor([anchor], dtype=torch.int32, device="cuda"), self.kv)
        return self.d.lmhead_logits(hid)


def gpu_greedy(cfg, tw, prompt, n_new):
    """Plain greedy decoding with the GPU target: one new token per pass (a
    2-row block whose second row is a placeholder the causal mask hides)."""
    P = len(prompt)
    g = GpuTarget(cfg, tw, P + n_new + 2, (P, 2))
    lg, _ = g.run(prompt, 0)
    g.commit(P)
    out = [int(np.argmax(lg[-1]))]
    while len(out) < n_new:
        lg, _ = g.run([out[-1], 0], P + len(out) - 1)
        g.commit(1)
        out.append(int(np.argmax(lg[0])))
    g.close()
    return np.array(out, dtype=np.int32)


def gpu_spec(cfg, tw, dw, prompt, n_new, script=None):
    """Greedy speculative decoding, drafter and target both on the GPU: the
    target verifies each drafted block in one causal pass and its taps of the
    accepted positions are injected into the drafter's cache.  ``script``
    (optional) replaces the drafter: script(n_out) -> the B - 1 drafts."""
    B, P = cfg.block_size, len(prompt)
    cap = P + n_new + 2 * B
    g = GpuTarget(cfg, tw, cap, (P, B))
    dr = GpuDrafter(cfg, dw, cap)
    lg, taps = g.run(prompt, 0)
    g.commit(P)
    dr.inject(taps, np.arange(P))
    out = [int(np.argmax(lg[-1]))]
    taus = []
    p = P
    while len(out) < n_new:
        anchor = out[-1]
        d = [int(t) for t in (dr.draft(anchor) if script is None else script(len(out)))]
        lg, taps = g.run([anchor] + d, p)
        y = torch.from_numpy(lg.argmax(axis=1).astype(np.int32)).cuda().view(1, B)
        tau, bonus = dr.d.accept_len(torch.tensor([d], dtype=torch.int32, device="cuda"), y, B)
        tau, bonus = int(tau.cpu()[0]), int(bonus.cpu()[0])
        taus.append(tau)
        out.extend(d[:tau - 1])
        out.append(bonus)
        g.commit(tau)
        dr.inject(taps[:tau], np.arange(p, p + tau))
        p += tau
    g.close()
    dr.d.close()
    return np.array(out[:n_new], dtype=np.int32), taus


@pytest.mark.parametrize("seed,layer_std", [(0, 0.02), (1, 0.1), (2, 0.05)])
def test_lossless_speculative_decoding_on_gpu(seed, layer_std):
    cfg = MINI["tiny"]
    log(f"GPU target + GPU drafter, seed={seed} layer_std={layer_std}")
    tw = S.target_weights(cfg, seed, layer_std=layer_std)
    prompt = S.prompt_ids(cfg, seed)
    greedy = gpu_greedy(cfg, tw, prompt, cfg.new_tokens)
    spec, taus = gpu_spec(cfg, tw, S.drafter_weights(cfg, seed), prompt, cfg.new_tokens)
    log(f"  taus {taus}")
    assert np.array_equal(spec, greedy)
    # and the GPU target decodes what the oracle target decodes
    o = T.greedy_decode(T.TinyTarget(tw, cfg), prompt, cfg.new_tokens)
    assert np.array_equal(greedy, o)


@pytest.mark.parametrize("kind", ["perfect", "first_right"])
def test_speculative_commits_accepted_drafts_on_gpu(kind):
    """Drafts scripted from the GPU target's own greedy output: all right
    (tau = B every cycle) or only the first right (tau = 2), so blocks of
    accepted drafts are committed, their cache rows kept and their taps
    injected; the output must still equal greedy decoding."""
    cfg = MINI["tiny"]
    B = cfg.block_size
    tw = S.target_weights(cfg, 4, layer_std=0.1)
    prompt = S.prompt_ids(cfg, 4)
    n = cfg.new_tokens
    greedy = gpu_greedy(cfg, tw, prompt, n + B)

    def script(n_out):
        d = [int(t) for t in greedy[n_out:n_out + B - 1]]
        if kind == "first_right":
            d = d[:1] + [(t + 1) % cfg.vocab for t in d[1:]]
        return d

    spec, taus = gpu_spec(cfg, tw, S.drafter_weights(cfg, 4), prompt, n, script=script)
    log(f"  {kind}: taus {taus}")
    assert np.array_equal(spec, greedy[:n])
    assert all(t == (B if kind == "perfect" else 2) for t in taus)


def gpu_spec_sample(cfg, tw, dw, prompt, n_new, temp, seed):
    """Speculative sampling at temperature ``temp``, everything on the GPU: the
    loop and counter conventions of the oracle's ``spec_sample``."""
    R = runtime()
    B, Pl = cfg.block_size, len(prompt)
    cap = Pl + n_new + 2 * B
    g = GpuTarget(cfg, tw, cap, (Pl, B))
    dr = GpuDrafter(cfg, dw, cap)
    lg, taps = g.run_logits(prompt, 0)
    g.commit(Pl)
    dr.inject(taps, np.arange(Pl))
    first, _ = R.Drafter.sample(lg[-1:].contiguous(), temp, seed, 0, P.TAG_PREFILL)
    out = [int(first.cpu()[0])]
    taus = []
    p, c = Pl, 0
    while len(out) < n_new:
        anchor = out[-1]
        zd = dr.draft_logits(anchor)
        d, dlse = R.Drafter.sample(zd, temp, seed, c, P.TAG_DRAFT)
        dh = [int(t) for t in d.cpu().numpy()]
        zt, taps = g.run_logits([anchor] + dh, p)
        y, tlse = R.Drafter.sample(zt, temp, seed, c, P.TAG_TARGET)
        tau, bonus = R.Drafter.accept_sample(zd, dlse, d.view(1, B - 1), zt, tlse, y.view(1, B), B, temp, seed, c)
        tau, bonus = int(tau.cpu()[0]), int(bonus.cpu()[0])
        taus.append(tau)
        out.extend(dh[:tau - 1])
        out.append(bonus)
        g.commit(tau)
        dr.inject(taps[:tau], np.arange(p, p + tau))
        p += tau
        c += 1
    g.close()
    dr.d.close()
    return np.array(out[:n_new], dtype=np.int32), taus


@pytest.mark.parametrize("seed,temp", [(0, 1.0), (1, 0.7), (2, 1.3)])
def test_speculative_sampling_on_gpu_matches_oracle(seed, temp):
    """Temperature > 0: drafter, target, draws and the accept / resample rule on
    the GPU reproduce the oracle's speculative sampling token for token (same
    Philox streams; fp32 tiny configuration)."""
    cfg = MINI["tiny"]
    log(f"speculative sampling seed={seed} T={temp}")
    tw = S.target_weights(cfg, seed, layer_std=0.05)
    dw = S.drafter_weights(cfg, seed)
    prompt = S.prompt_ids(cfg, seed)
    got, taus = gpu_spec_sample(cfg, tw, dw, prompt, cfg.new_tokens, temp, seed + 100)
    want, taus_o = P.spec_sample(T.TinyTarget(tw, cfg), D.OracleDrafter(dw, cfg), prompt, cfg.new_tokens, temp,
                                 seed + 100, cfg.dtype)
    log(f"  taus gpu {taus} oracle {taus_o}")
    assert np.array_equal(got, want)
    assert taus == taus_o


def test_target_verify_with_a_smaller_block_size():
    """A verify block of B_s < B rows (dflash_kv::block_len): rows 0..B_s-1
    equal the oracle target's pass over those B_s tokens."""
    cfg = MINI["tiny"]
    tw = S.target_weights(cfg, 6, layer_std=0.05)
    tgt = T.TinyTarget(tw, cfg)
    prompt = S.prompt_ids(cfg, 6)
    P_, B = len(prompt), cfg.block_size
    g = GpuTarget(cfg, tw, P_ + 2 * B, (P_, B))
    g.run(prompt, 0)
    tgt.run(prompt, 0)
    g.commit(P_)
    block = [int(t) for t in S.prompt_ids(cfg, 7)[:B]]
    for bs in (3, 2, 1):
        g.kv.set_block_len(np.array([bs]))
        lg, taps = g.run(block, P_)
        tgt.truncate(P_)
        lo, to = tgt.run(block[:bs], P_)
        assert_close(lg[:bs], lo, 1e-4, f"verify logits, B_s = {bs}")
        assert_close(taps[:bs], to, 1e-4, f"verify taps, B_s = {bs}")
    g.kv.set_block_len(None)
    g.close()
