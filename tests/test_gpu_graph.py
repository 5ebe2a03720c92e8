"""The drafter step captured in a HIP graph (as the benchmark times it) and
replayed: every replay, with eager work and synchronisation between replays,
must give exactly the eager results.  Greedy step (draft block + LM head argmax
+ accept length) and the temperature > 0 step (logits-only LM head + draws +
sampled accept).  The library issues no memset and allocates nothing inside
these calls; their workspace counters return to zero by themselves."""
import numpy as np
import pytest

import dflash_synth as S
from gpu_cases import MINI, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_gemm_amd import _lib
    _lib.load()


def setup(name):
    from block_diffusion_drafter_gemm_amd import runtime as R
    cfg = MINI[name]
    w = S.drafter_weights(cfg, seed=12, random_gain=True)
    lens = S.ctx_lens(cfg, seed=12)
    b, B = len(lens), cfg.block_size
    lay = S.paged_layout(cfg, lens, headroom=B, seed=12)
    Kp, Vp = S.ctx_kv_cache(cfg, lay, seed=12)
    dr = R.Drafter(cfg, w, max_batch=b, max_ctx=int(lens.max()), max_new=B)
    kv = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages, k=Kp, v=Vp)
    anchors = torch.from_numpy(S.anchor_ids(cfg, seed=12, batch=b)).cuda()
    d = S.draft_ids_random(cfg, b, seed=12)
    y = torch.from_numpy(S.target_ids_for(cfg, d, seed=12)).cuda()
    return R, cfg, dr, kv, anchors, y, b, B


def capture_and_replay(step, outputs, replays=4, n_fill=None):
    """Eager run, then capture; each replay is compared with the eager outputs,
    with eager work and a synchronisation between replays.  The first n_fill
    outputs (all by default) are overwritten before each replay."""
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    junk = torch.randn(1 << 20, device="cuda")
    for i in range(replays):
        for o in outputs[:n_fill]:
            o.fill_(-7)                          # a replay that did nothing would leave this
        g.replay()
        torch.cuda.synchronize()
        for o, wnt in zip(outputs, want):
            assert torch.equal(o, wnt), f"replay {i} differs from the eager run"
        junk.mul_(1.0001).add_(0.5)              # eager work between replays
        torch.cuda.synchronize()
    return want


@pytest.mark.parametrize("name", ["mini_bf16", "mini_b8", "tiny", "mini_ffn_b1"])
def test_greedy_step_graph_replays_match_eager(name):
    R, cfg, dr, kv, anchors, y, b, B = setup(name)
    log(f"graph greedy step {name}")
    hid = torch.empty((b * (B - 1), cfg.hidden), dtype=R.storage_dtype(cfg), device="cuda")
    ids = torch.empty(b * (B - 1), dtype=torch.int32, device="cuda")
    mx = torch.empty(b * (B - 1), dtype=torch.float32, device="cuda")
    tau = torch.empty(b, dtype=torch.int32, device="cuda")
    bonus = torch.empty(b, dtype=torch.int32, device="cuda")
    L = R.L
    # steady-state inject of B positions per sequence just past its context
    # (ctx_len is not advanced, so the draft reads the same context each time)
    feats = R.to_device(S.features(cfg, b * B, seed=13))
    seq = torch.arange(b, dtype=torch.int32, device="cuda").repeat_interleave(B)
    pos = (kv.ctx_len.repeat_interleave(B) + torch.arange(B, dtype=torch.int32, device="cuda").repeat(b)).int()

    def step():
        L.dflash_inject_context(dr.handle, feats, seq, pos, b * B, kv.struct(), dr.ws)
        L.dflash_draft_block(dr.handle, anchors, kv.struct(), hid, dr.ws)
        L.dflash_lmhead_argmax(dr.handle, hid, b * (B - 1), ids, mx, None, dr.ws)
        L.dflash_accept_len(ids.view(b, B - 1), y, b, B, tau, bonus)

    capture_and_replay(step, [ids, mx, tau, bonus, kv.k, kv.v], n_fill=4)
    dr.close()


@pytest.mark.parametrize("name", ["mini_bf16", "mini_f32"])
def test_sampled_step_graph_replays_match_eager(name):
    R, cfg, dr, kv, anchors, y, b, B = setup(name)
    log(f"graph sampled step {name}")
    rows = b * (B - 1)
    hid = torch.empty((rows, cfg.hidden), dtype=R.storage_dtype(cfg), device="cuda")
    dz = torch.empty((rows, cfg.vocab), dtype=torch.float32, device="cuda")
    d = torch.empty(rows, dtype=torch.int32, device="cuda")
    dlse = torch.empty(rows, dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(3)
    tz = torch.randn((b * B, cfg.vocab), generator=gen, device="cuda")
    tids, tlse = R.Drafter.sample(tz, 0.8, 5, 0, 1)
    tau = torch.empty(b, dtype=torch.int32, device="cuda")
    bonus = torch.empty(b, dtype=torch.int32, device="cuda")
    L = R.L
    sws = torch.empty(L.dflash_sample_workspace_size(max(rows, b), cfg.vocab), dtype=torch.uint8, device="cuda")

    def step():
        L.dflash_draft_block(dr.handle, anchors, kv.struct(), hid, dr.ws)
        L.dflash_lmhead_argmax(dr.handle, hid, rows, None, None, dz, dr.ws)
        L.dflash_sample(dz, rows, cfg.vocab, 0.8, 5, 0, 0, d, dlse, sws)
        L.dflash_accept_sample(dz, dlse, d, tz, tlse, tids, b, B, None, cfg.vocab, 0.8, 5, 0, tau, bonus, sws)

    capture_and_replay(step, [d, dlse, tau, bonus])
    dr.close()
