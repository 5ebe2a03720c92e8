"""Memory safety of the hot calls on the GPU: a workspace poisoned with NaN bit
patterns (only its counter area cleared by dflash_workspace_init) gives
bitwise the same results as a zero-filled one, and canary regions around every
output are left untouched."""
import numpy as np
import pytest

import dflash_synth as S
from gpu_cases import MINI, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GUARD = 64          # canary rows / elements on each side of an output


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_gemm_amd import _lib
    _lib.load()


def guarded(shape, dtype, fill):
    """A tensor with GUARD canary rows before and after; returns (buffer, view)."""
    rows = shape[0]
    buf = torch.full((rows + 2 * GUARD,) + tuple(shape[1:]), fill, dtype=dtype, device="cuda")
    return buf, buf[GUARD:GUARD + rows]


def canaries_intact(buf, fill):
    head, tail = buf[:GUARD], buf[-GUARD:]
    ref = torch.full_like(head, fill)
    return torch.equal(head, ref) and torch.equal(tail, ref)


@pytest.mark.parametrize("name", ["mini_bf16", "mini_b8", "tiny", "mini_port"])
def test_poisoned_workspace_and_canaries(name):
    from block_diffusion_drafter_gemm_amd import runtime as R
    L = R.L
    cfg = MINI[name]
    log(f"memory safety {name}")
    w = S.drafter_weights(cfg, seed=14, random_gain=True)
    lens = S.ctx_lens(cfg, seed=14)
    b, B, H = len(lens), cfg.block_size, cfg.hidden
    lay = S.paged_layout(cfg, lens, headroom=B, seed=14)
    Kp, Vp = S.ctx_kv_cache(cfg, lay, seed=14)
    dr = R.Drafter(cfg, w, max_batch=b, max_ctx=int(lens.max()), max_new=b * B)
    anchors = torch.from_numpy(S.anchor_ids(cfg, seed=14, batch=b)).cuda()
    feats = R.to_device(S.features(cfg, b * B, seed=15))
    seq = torch.arange(b, dtype=torch.int32, device="cuda").repeat_interleave(B)
    pos = (torch.from_numpy(lens).cuda().repeat_interleave(B) +
           torch.arange(B, dtype=torch.int32, device="cuda").repeat(b)).int()
    rows = b * (B - 1)
    dt = R.storage_dtype(cfg)
    hfill = -3.5                                           # exact in bf16 and fp32

    poison = torch.full_like(dr.ws, 0xFF)                 # NaN in fp32 and in bf16
    L.dflash_workspace_init(dr.handle, poison)
    results = []
    for ws in (dr.ws, poison):
        kv = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages, k=Kp, v=Vp)
        hbuf, hid = guarded((rows, H), dt, hfill)
        ibuf, ids = guarded((rows,), torch.int32, -12345)
        mbuf, mx = guarded((rows,), torch.float32, hfill)
        L.dflash_inject_context(dr.handle, feats, seq, pos, b * B, kv.struct(), ws)
        L.dflash_draft_block(dr.handle, anchors, kv.struct(), hid, ws)
        L.dflash_lmhead_argmax(dr.handle, hid, rows, ids, mx, None, ws)
        torch.cuda.synchronize()
        assert canaries_intact(ibuf, -12345) and canaries_intact(hbuf, hfill) and canaries_intact(mbuf, hfill)
        assert not torch.isnan(hid.float()).any() and not torch.isnan(mx).any()
        results.append((kv.k.clone(), kv.v.clone(), hid.clone(), ids.clone(), mx.clone()))
    for a, c in zip(results[0], results[1]):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           c.view(torch.uint8) if c.dtype == torch.bfloat16 else c), "poisoned workspace changed a result"
    dr.close()


def test_sampling_with_poisoned_workspace():
    from block_diffusion_drafter_gemm_amd import runtime as R
    L = R.L
    gen = torch.Generator(device="cuda").manual_seed(5)
    rows, V = 37, 5003
    z = torch.randn((rows, V), generator=gen, device="cuda")
    n = L.dflash_sample_workspace_size(rows, V)
    outs = []
    for fill in (0, 0xFF):
        ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda")
        ibuf, ids = guarded((rows,), torch.int32, -9)
        lbuf, lse = guarded((rows,), torch.float32, -9.0)
        L.dflash_sample(z, rows, V, 0.9, 77, 3, 0, ids, lse, ws)
        torch.cuda.synchronize()
        assert canaries_intact(ibuf, -9) and canaries_intact(lbuf, -9.0)
        outs.append((ids.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
