"""dflash_lmhead_argmax_noalloc -- the LM head and vocabulary argmax with the
library's own scratch memory, for callers that cannot allocate -- against
dflash_lmhead_argmax with a caller workspace: two calls in a row on one
device, the second with fewer rows, on each LM-head path (LDS-tiled, streaming,
two 16-row slices, 256 x 256 tiles, fp32 few-rows).  Same kernels, same
order: ids and max logits must be bit-identical.  Rows past the scratch size
are refused on the host.
"""
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


def scratch_rows_limit(vocab):
    align = lambda x: (x + 255) // 256 * 256
    ng = vocab // 16
    r = 1
    while 262144 + 2 * align((r + 1) * ng * 4) <= 8 << 20:
        r += 1
    return r


@pytest.mark.parametrize("name,rows", [("mini_bf16", (70, 15)), ("mini_bf16", (31, 1)), ("mini_f32", (40, 7)),
                                       ("mini_big", (300, 150))])
def test_noalloc_lmhead_matches_workspace_entry_point(name, rows):
    from block_diffusion_drafter_gemm_amd import _lib as L
    from block_diffusion_drafter_gemm_amd import runtime as R
    cfg = MINI[name]
    log(f"lmhead_argmax_noalloc {name} rows {rows}")
    w = S.drafter_weights(cfg, seed=12)
    dr = R.Drafter(cfg, w, max_batch=(max(rows) + cfg.block_size - 2) // (cfg.block_size - 1), max_ctx=16,
                   max_new=1)
    for n in rows:
        z = R.to_device(S.normal_matrix(cfg, 79, (n, cfg.hidden), 1.0, seed=n))
        ids_w, mx_w, _ = dr.lmhead_argmax(z, want_max=True)
        ids_s = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        mx_s = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        L.dflash_lmhead_argmax_noalloc(dr.handle, z, n, ids_s, mx_s)
        torch.cuda.synchronize()
        assert torch.equal(ids_s, ids_w), n
        assert torch.equal(mx_s, mx_w), n
        assert int(ids_s.min()) >= 0 and int(ids_s.max()) < cfg.vocab
    # past the scratch size: refused before any launch
    big = scratch_rows_limit(cfg.vocab) + 1
    st = L.load().dflash_lmhead_argmax_noalloc(dr.handle, 0x1000, big, 0x1000, None, None)
    assert st == -5, st
    dr.close()
