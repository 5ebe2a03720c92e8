"""GPU parity of every libdflash entry point against the CPU oracle, on small
shapes with ragged tails (several tiles, partial column groups, contexts that
are not page multiples, padded query tiles, fp32 and bf16 storage).

Token ids and accept lengths must match exactly (ids may differ only on an
oracle near-tie); hidden states, cache entries and logits must be within
1e-4 (fp32) or 2e-2 (bf16) of the oracle, scaled by max(1, |oracle|).
"""
import dataclasses

import numpy as np
import pytest

import dflash_synth as S
from oracle import drafter as D
from oracle.numerics import bf16_bits, from_storage, round_storage

from gpu_cases import MINI, assert_close, check_ids, gather_ctx, log, oracle_draft, tol_of

torch = pytest.importorskip("torch")
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


def storage_of(cfg, x):
    """float64 values already representable in the storage type -> storage array."""
    return bf16_bits(x) if cfg.dtype == "bf16" else np.asarray(x, dtype=np.float32)


# ----------------------------------------------------------------------------
# A10 accept length
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("B", [2, 4, 10, 16, 64])
def test_accept_len(B):
    log(f"accept_len B={B}")
    cfg = S.get_config("llama31_8b", block_size=B)
    n = 3000
    d = S.draft_ids_random(cfg, n, seed=B)
    y = S.target_ids_for(cfg, d, seed=B)
    y[0, :-1] = d[0]                       # all drafts accepted
    y[1, 0] = (d[1, 0] + 1) % cfg.vocab    # first draft rejected
    tau_o, bonus_o = D.accept_len_batch(d, y)
    dt, yt = torch.from_numpy(d).cuda(), torch.from_numpy(y).cuda()
    tau, bonus = runtime().Drafter.accept_len(dt, yt, B)
    torch.cuda.synchronize()
    assert np.array_equal(tau.cpu().numpy(), tau_o)
    assert np.array_equal(bonus.cpu().numpy(), bonus_o)
    assert tau_o[0] == B and tau_o[1] == 1


# ----------------------------------------------------------------------------
# A9 LM head + argmax
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name,rows", [(n, r) for n in ["tiny", "mini_bf16", "mini_f32", "mini_b10"]
                                       for r in [1, 15, 33, 70]] + [("mini_b8", r) for r in [65, 130, 300]]
                         + [("mini_bf16", 17), ("mini_f32", 31), ("tiny", 32), ("mini_b10", 24)]
                         + [("mini_wide", r) for r in [20, 47]] + [("mini_big", r) for r in [150, 300]])
def test_lmhead_argmax(name, rows):
    cfg = MINI[name]
    log(f"lmhead_argmax {name} rows={rows}")
    R = runtime()
    w = S.drafter_weights(cfg, seed=1)
    # duplicate a vocabulary row at a higher id: exact ties must go to the lower id
    w["lm_head"][cfg.vocab - 3] = w["lm_head"][5]
    dr = R.Drafter(cfg, w, max_batch=(rows + cfg.block_size - 2) // (cfg.block_size - 1), max_ctx=16, max_new=1)
    z = S.normal_matrix(cfg, 77, (rows, cfg.hidden), 1.0, seed=rows)
    # rows 0, 17 and 31 (the first, second and third 16-row groups when there are
    # that many rows) point at vocabulary row 5, so ids 5 and vocab-3 tie
    # exactly at the top
    tie_rows = [r for r in (0, 17, 31) if r < rows]
    for r in tie_rows:
        z[r] = storage_of(cfg, round_storage(from_storage(w["lm_head"][5]) * (50.0 + r), cfg.dtype))
    z_dev = R.to_device(z)
    ids, mx, lg = dr.lmhead_argmax(z_dev, want_max=True, want_logits=True)
    torch.cuda.synchronize()
    ids_o, best_o, logits_o = D.lm_argmax(w["lm_head"], z)
    assert_close(lg.cpu().numpy(), logits_o, 1e-4, f"{name} logits")
    assert_close(mx.cpu().numpy(), best_o, 1e-4, f"{name} max logit")
    # identical inputs: ids may differ only within the fp32 logit bar
    check_ids(ids.cpu().numpy(), ids_o, logits_o, 1e-4, f"{name} ids")
    # rows whose best is the duplicated row: the GPU must return the lower id 5
    g = ids.cpu().numpy()
    for r in tie_rows:
        assert g[r] == 5 and ids_o[r] == 5, r
    assert not np.any(g == cfg.vocab - 3)
    dr.close()


@pytest.mark.parametrize("rows", [150, 300])
def test_lmhead_argmax_ties_inside_one_block(rows):
    """Exact ties inside one 128-column block of the 256 x 256-tile LM head:
    five copies of one vocabulary row at ids in different lanes and column
    tiles of block 3 (ids 384 + {70, 5, 100, 38, 6}); rows in both 128-row
    halves of both row blocks point at it, so the winner is decided by the
    per-row reduction inside the block, and it must be the lowest id, 389."""
    cfg = MINI["mini_big"]
    log(f"lmhead_argmax in-block ties mini_big rows={rows}")
    R = runtime()
    w = S.drafter_weights(cfg, seed=5)
    base = 3 * 128
    src = base + 70
    for c in (5, 100, 38, 6):
        w["lm_head"][base + c] = w["lm_head"][src]
    z = S.normal_matrix(cfg, 79, (rows, cfg.hidden), 1.0, seed=rows)
    tie_rows = [r for r in (0, 5, 37, 127, 128, 131, 200, 255, 256, 290, 299) if r < rows]
    for r in tie_rows:
        z[r] = storage_of(cfg, round_storage(from_storage(w["lm_head"][src]) * (40.0 + r % 7), cfg.dtype))
    dr = R.Drafter(cfg, w, max_batch=(rows + cfg.block_size - 2) // (cfg.block_size - 1), max_ctx=16, max_new=1)
    ids, mx, lg = dr.lmhead_argmax(R.to_device(z), want_max=True, want_logits=True)
    torch.cuda.synchronize()
    ids_o, best_o, logits_o = D.lm_argmax(w["lm_head"], z)
    g = ids.cpu().numpy()
    for r in tie_rows:
        assert ids_o[r] == base + 5, (r, ids_o[r])
        assert g[r] == base + 5, (r, g[r])
    assert_close(mx.cpu().numpy(), best_o, 1e-4, "max logit")
    check_ids(g, ids_o, logits_o, 1e-4, "ids")
    dr.close()


@pytest.mark.parametrize("name,rows", [("mini_b8", 130), ("mini_big", 300)])
def test_lmhead_logits_into_an_unaligned_buffer(name, rows):
    """fp32 logits of the LDS-tiled (130 rows) and 256 x 256-tile (300 rows)
    LM head written into a buffer that starts 4 bytes past a 16-byte boundary:
    the epilogue then stores one element at a time instead of 16-byte pieces,
    with the same values and ids as into an aligned buffer."""
    cfg = MINI[name]
    log(f"lmhead logits into an unaligned buffer {name} rows={rows}")
    R = runtime()
    from block_diffusion_drafter_gemm_amd import _lib as Lb
    w = S.drafter_weights(cfg, seed=4)
    dr = R.Drafter(cfg, w, max_batch=(rows + cfg.block_size - 2) // (cfg.block_size - 1), max_ctx=16, max_new=1)
    z = R.to_device(S.normal_matrix(cfg, 80, (rows, cfg.hidden), 1.0, seed=rows))
    ids_a, mx_a, lg_a = dr.lmhead_argmax(z, want_max=True, want_logits=True)
    buf = torch.full((rows * cfg.vocab + 4,), float("nan"), dtype=torch.float32, device="cuda")
    lg_u = buf[1:1 + rows * cfg.vocab]
    assert lg_u.data_ptr() % 16 == 4
    ids_u = torch.empty(rows, dtype=torch.int32, device="cuda")
    mx_u = torch.empty(rows, dtype=torch.float32, device="cuda")
    Lb.dflash_lmhead_argmax(dr.handle, z, rows, ids_u, mx_u, lg_u, dr.ws)
    torch.cuda.synchronize()
    assert torch.equal(lg_u.view(rows, cfg.vocab), lg_a)
    assert torch.equal(ids_u, ids_a) and torch.equal(mx_u, mx_a)
    assert torch.isnan(buf[0]) and torch.isnan(buf[1 + rows * cfg.vocab:]).all()   # nothing written outside
    dr.close()


@pytest.mark.parametrize("name,rows", [("mini_bf16", 15), ("mini_bf16", 31), ("mini_b8", 130), ("mini_f32", 40),
                                       ("mini_big", 300)])
def test_lmhead_argmax_nan_logits(name, rows):
    """NaN logits never win, and a row whose logits are all NaN returns id 0 with
    max logit -inf (an id inside the vocabulary) on every LM-head path: the
    streaming kernel (15 rows), two 16-row slices (31), the LDS-tiled (130) and
    256 x 256-tile (300) kernels, and the fp32 few-rows kernel (40)."""
    cfg = MINI[name]
    log(f"lmhead_argmax NaN logits {name} rows={rows}")
    R = runtime()
    w = S.drafter_weights(cfg, seed=3)
    nan = np.uint16(0x7FC0) if cfg.dtype == "bf16" else np.float32(np.nan)   # a quiet NaN
    w["lm_head"][7] = nan                                     # column 7 of every row is NaN
    z = S.normal_matrix(cfg, 78, (rows, cfg.hidden), 1.0, seed=rows)
    z[rows // 2] = nan                                        # every logit of this row is NaN
    dr = R.Drafter(cfg, w, max_batch=(rows + cfg.block_size - 2) // (cfg.block_size - 1), max_ctx=16, max_new=1)
    ids, mx, _ = dr.lmhead_argmax(R.to_device(z), want_max=True)
    torch.cuda.synchronize()
    g, m = ids.cpu().numpy(), mx.cpu().numpy()
    with np.errstate(invalid="ignore"):
        logits_o = D.lm_logits(w["lm_head"], z)
    for r in range(rows):
        if r == rows // 2:
            assert g[r] == 0 and m[r] == -np.inf, (r, g[r], m[r])
            continue
        o = int(np.nanargmax(logits_o[r]))
        assert g[r] != 7 and 0 <= g[r] < cfg.vocab
        lo = logits_o[r, o]
        assert logits_o[r, g[r]] >= lo - 1e-4 * max(1.0, abs(lo)), (r, g[r], o)
    dr.close()


# ----------------------------------------------------------------------------
# A1 + A2 inject
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name,n_new", [(n, k) for n in ["tiny", "mini_bf16", "mini_d64", "mini_f32"]
                                        for k in [1, 16, 90]] + [("mini_bf16", 200), ("mini_d64", 300), ("mini_port", 5), ("mini_port", 16)])
def test_inject_context(name, n_new):
    run_inject_case(MINI[name], n_new)


@pytest.mark.parametrize("name,n_new", [("mini_bf16", 5), ("mini_bf16", 300), ("mini_f32", 16), ("mini_f32", 90),
                                        ("mini_port", 40), ("mini_port", 3), ("mini_port", 16)])
def test_inject_context_with_ctx_norm(name, n_new):
    """The optional RMSNorm after the fusion projection (random gain), on the
    streaming (<= 16 rows, K-portions for mini_port's K = 17 x 256), few-rows and
    LDS-tiled paths."""
    run_inject_case(dataclasses.replace(MINI[name], ctx_norm=1), n_new, random_gain=True)


def run_inject_case(cfg, n_new, random_gain=False):
    name = cfg.name
    log(f"inject {name} n_new={n_new} ctx_norm={cfg.ctx_norm}")
    R = runtime()
    w = S.drafter_weights(cfg, seed=2, random_gain=random_gain)
    batch = 3
    lens = np.array([n_new, n_new + 7, 3], dtype=np.int32)
    lay = S.paged_layout(cfg, lens, headroom=cfg.block_size, seed=2)
    rng = np.random.default_rng(n_new)
    # n_new distinct (seq, pos) slots, scattered over the sequences
    slots = [(s, p) for s in range(batch) for p in range(int(lens[s]) + cfg.block_size)]
    pick = rng.choice(len(slots), size=n_new, replace=False)
    seq = np.array([slots[i][0] for i in pick], dtype=np.int32)
    pos = np.array([slots[i][1] for i in pick], dtype=np.int32)
    feats = S.features(cfg, n_new, seed=3)
    dr = R.Drafter(cfg, w, max_batch=batch, max_ctx=int(lens.max()), max_new=n_new)
    kv = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages)
    dr.inject_context(R.to_device(feats), torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), kv)
    torch.cuda.synchronize()
    K_o, V_o = D.inject(w, cfg, feats, pos)
    Kg, Vg = R.to_host_storage(kv.k), R.to_host_storage(kv.v)
    pages = lay.block_table[seq, pos // cfg.page_size]
    sl = pos % cfg.page_size
    tol = tol_of(cfg)
    assert_close(from_storage(Kg[:, pages, sl]), K_o, tol, f"{name} injected K")
    assert_close(from_storage(Vg[:, pages, sl]), V_o, tol, f"{name} injected V")
    # nothing else was written
    mask = np.ones(Kg.shape[:3], dtype=bool)
    mask[:, pages, sl] = False
    assert not from_storage(Kg[mask]).any() and not from_storage(Vg[mask]).any()
    dr.close()


@pytest.mark.parametrize("n_new", [16, 40, 100])
def test_bf16_ties_through_inject(n_new):
    """fp32 -> bf16 rounding in the GPU epilogues on exact ties and near ties:
    c = feats . W_fc^T from one-hot fusion weights, read back through identity V
    projections.  16 rows take the streaming GEMM, 40 the few-rows GEMM, 100 the
    LDS-tiled GEMM; all must equal torch's CPU conversion (ties to even) bit for
    bit, as the oracle does."""
    from tie_cases import tie_case
    cfg = S.get_config("tiny", dtype="bf16", n_feat_layers=3)
    log(f"bf16 ties through inject, n_new={n_new}")
    R = runtime()
    w, feats, expect, _ = tie_case(cfg, n_new, seed=11)
    lens = np.array([n_new], dtype=np.int32)
    lay = S.paged_layout(cfg, lens, headroom=cfg.block_size, seed=11)
    pos = np.arange(n_new, dtype=np.int32)
    seq = np.zeros(n_new, dtype=np.int32)
    dr = R.Drafter(cfg, w, max_batch=1, max_ctx=n_new, max_new=n_new)
    kv = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages)
    dr.inject_context(R.to_device(feats), torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), kv)
    torch.cuda.synchronize()
    Vg = R.to_host_storage(kv.v)
    pages = lay.block_table[seq, pos // cfg.page_size]
    got = Vg[:, pages, pos % cfg.page_size].reshape(cfg.n_layers, n_new, cfg.hidden)
    _, V_o = D.inject(w, cfg, feats, pos)
    for l in range(cfg.n_layers):
        bad = int((got[l] != expect).sum())
        log(f"  layer {l}: {bad} of {expect.size} elements differ from round-to-nearest-even")
        assert bad == 0
        assert np.array_equal(from_storage(got[l]), V_o[l].reshape(n_new, cfg.hidden))
    dr.close()


# ----------------------------------------------------------------------------
# A3..A8 draft block (+ A9 on its output)
# ----------------------------------------------------------------------------
def run_draft_case(cfg, seed=0, lens=None, check_seqs=None):
    R = runtime()
    w = S.drafter_weights(cfg, seed=seed, random_gain=True)
    lens = S.ctx_lens(cfg, seed=seed) if lens is None else np.asarray(lens, dtype=np.int32)
    batch = len(lens)
    lay = S.paged_layout(cfg, lens, headroom=cfg.block_size, seed=seed)
    Kp, Vp = S.ctx_kv_cache(cfg, lay, seed=seed)
    anchors = S.anchor_ids(cfg, seed=seed, batch=batch)
    dr = R.Drafter(cfg, w, max_batch=batch, max_ctx=int(lens.max()), max_new=1)
    kv = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages, k=Kp, v=Vp)
    k0, v0 = kv.k.clone(), kv.v.clone()
    hid = dr.draft_block(torch.from_numpy(anchors).cuda(), kv)
    ids, mx, _ = dr.lmhead_argmax(hid)
    hid2 = dr.draft_block(torch.from_numpy(anchors).cuda(), kv)     # determinism
    torch.cuda.synchronize()
    assert torch.equal(hid, hid2), "draft_block is not deterministic"
    assert torch.equal(kv.k, k0) and torch.equal(kv.v, v0), "draft_block wrote the context cache"
    hid_h = from_storage(R.to_host_storage(hid)).reshape(batch, cfg.block_size - 1, cfg.hidden)
    ids_h = ids.cpu().numpy().reshape(batch, cfg.block_size - 1)
    tol = tol_of(cfg)
    seqs = range(batch) if check_seqs is None else check_seqs
    for s in seqs:
        Z = oracle_draft(cfg, w, anchors[s], Kp, Vp, lay.block_table, s, int(lens[s]))
        assert_close(hid_h[s], Z, tol, f"{cfg.name} seq {s} (ctx {lens[s]}) hidden")
        ids_o, best_o, logits_o = D.lm_argmax(w["lm_head"], Z)
        check_ids(ids_h[s], ids_o, logits_o, tol, f"{cfg.name} seq {s} draft ids")
        mx_h = mx.cpu().numpy().reshape(batch, cfg.block_size - 1)
        assert_close(mx_h[s], best_o, tol, f"{cfg.name} seq {s} max logit")
    dr.close()
    return hid_h, ids_h


@pytest.mark.parametrize("name", ["tiny", "mini_bf16", "mini_b10", "mini_d64", "mini_f32", "mini_b8", "mini_port",
                                  "mini_wide", "mini_g8", "mini_big", "mini_split", "mini_long"])
def test_draft_block(name):
    log(f"draft_block {name}")
    run_draft_case(MINI[name], seed=0)


def test_draft_block_gate_up_256x192_tiles():
    """20 sequences x B 16 = 320 block rows of the mini_big shape (FFN 20544):
    gate/up takes the 256 x 192-tile kernel with two row blocks, the second
    ragged (64 of 256 rows), and 214 column tiles; checked against the oracle
    on the first, a middle and the last sequence (rows 0, 150, 319)."""
    cfg = dataclasses.replace(MINI["mini_big"], name="mini_big20", batch=20)
    log("draft_block mini_big x 20 sequences (256 x 192 gate/up tiles)")
    run_draft_case(cfg, seed=3, check_seqs=[0, 9, 19])


@pytest.mark.parametrize("ctx,window,blen", [(17, 0, 0), (1500, 0, 0), (3000, 0, 0), (1500, 100, 0), (3000, 0, 5),
                                              (0, 0, 0)])
def test_draft_block_single_sequence(ctx, window, blen):
    """One sequence (the batch-1 attention path: page-table entries requested
    with the context length, four-wave merge of the chunk partials) at contexts
    of 1, 24 and 48 chunks, with a sliding window and with a block size B_s < B,
    against the oracle."""
    cfg = dataclasses.replace(MINI["mini_bf16"], name="mini_one", batch=1, window=window)
    log(f"draft_block one sequence ctx={ctx} window={window} B_s={blen or cfg.block_size}")
    R = runtime()
    w = S.drafter_weights(cfg, seed=7, random_gain=True)
    lens = np.array([ctx], dtype=np.int32)
    lay = S.paged_layout(cfg, lens, headroom=cfg.block_size, seed=7)
    Kp, Vp = S.ctx_kv_cache(cfg, lay, seed=7)
    anchors = S.anchor_ids(cfg, seed=7, batch=1)
    dr = R.Drafter(cfg, w, max_batch=1, max_ctx=ctx, max_new=1)
    kv = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages, k=Kp, v=Vp)
    bs = blen or cfg.block_size
    if blen:
        kv.set_block_len(np.array([blen]))
    hid = dr.draft_block(torch.from_numpy(anchors).cuda(), kv)
    torch.cuda.synchronize()
    hid_h = from_storage(R.to_host_storage(hid)).reshape(cfg.block_size - 1, cfg.hidden)
    Z = oracle_draft(dataclasses.replace(cfg, block_size=bs), w, anchors[0], Kp, Vp, lay.block_table, 0, ctx)
    assert_close(hid_h[:bs - 1], Z, tol_of(cfg), f"one sequence ctx {ctx} hidden")
    dr.close()


@pytest.mark.parametrize("nq,nkv", [(8, 2), (16, 4)])
def test_draft_block_qkv_tile_widths(nq, nkv):
    """Batch 1 x B 16 on the streaming GEMMs with 12 and 24 heads of 128 in the
    QKV projection: 96 16-column tiles run as 192 8-column tiles (4 RoPE pairs,
    two k-chunks per weight load), 192 16-column tiles stay 16 wide (8-column
    tiles would not lower the busiest workgroup's share on 256 compute units);
    hidden states against the oracle."""
    cfg = dataclasses.replace(MINI["mini_bf16"], name=f"mini_q{nq}", batch=1, n_q_heads=nq, n_kv_heads=nkv)
    log(f"draft_block batch 1, {nq} q heads, {nkv} kv heads")
    run_draft_case(cfg, seed=8)


@pytest.mark.parametrize("ffn,B", [(4608, 16), (8320, 10)])
def test_draft_block_split_down_projection(ffn, B):
    """Batch 1 with an FFN past the 4096 resident columns: the down projection
    runs as 32-column tiles in pairs of workgroups, each pair half over half
    of K (2304 of 4608: 36 k-steps, the last four waves idle; 4160 of 8320:
    65 k-steps), the second half to finish adding both partials to the
    residual; B = 10 leaves rows 10-15 of each tile unused.  Hidden states and
    draft ids against the oracle, and two calls bit-identical (the arrival
    counters are back at zero after each call)."""
    cfg = dataclasses.replace(MINI["mini_bf16"], name=f"mini_ffn{ffn}", batch=1, ffn=ffn, block_size=B)
    log(f"draft_block batch 1, FFN {ffn}, B {B} (split down projection)")
    run_draft_case(cfg, seed=9)


@pytest.mark.parametrize("name,window", [("mini_bf16", 100), ("mini_d64", 50), ("mini_f32", 40)])
def test_draft_block_sliding_window(name, window):
    """Sliding-window context (ragged contexts above and below the window;
    streaming and many-rows paths) against the oracle's windowed pass."""
    log(f"draft_block {name} window={window}")
    run_draft_case(dataclasses.replace(MINI[name], window=window), seed=4)


@pytest.mark.parametrize("name,blens", [("mini_bf16", [16, 5, 9]), ("mini_d64", [4, 2]), ("mini_f32", [3, 8]),
                                        ("mini_b8", [16, 1, 7, 12, 2, 16, 9, 4])])
def test_draft_block_per_sequence_block_sizes(name, blens):
    """Dynamic block size: sequence s drafts B_s - 1 tokens; its rows 1..B_s-1
    must equal the oracle's pass with block size B_s (block rows >= B_s are
    left out of attention), on the streaming and many-rows paths."""
    cfg = MINI[name]
    log(f"draft_block {name} block sizes {blens}")
    R = runtime()
    w = S.drafter_weights(cfg, seed=6, random_gain=True)
    lens = S.ctx_lens(cfg, seed=6)
    batch = len(lens)
    assert batch == len(blens)
    lay = S.paged_layout(cfg, lens, headroom=cfg.block_size, seed=6)
    Kp, Vp = S.ctx_kv_cache(cfg, lay, seed=6)
    anchors = S.anchor_ids(cfg, seed=6, batch=batch)
    dr = R.Drafter(cfg, w, max_batch=batch, max_ctx=int(lens.max()), max_new=1)
    kv = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages, k=Kp, v=Vp)
    kv.set_block_len(np.array(blens))
    hid = dr.draft_block(torch.from_numpy(anchors).cuda(), kv)
    torch.cuda.synchronize()
    hid_h = from_storage(R.to_host_storage(hid)).reshape(batch, cfg.block_size - 1, cfg.hidden)
    for s, bs in enumerate(blens):
        if bs < 2:                                               # nothing drafted
            continue
        Z = oracle_draft(dataclasses.replace(cfg, block_size=bs), w, anchors[s], Kp, Vp, lay.block_table, s,
                         int(lens[s]))
        assert_close(hid_h[s, :bs - 1], Z, tol_of(cfg), f"{name} seq {s} (B_s {bs}) hidden")
    dr.close()


@pytest.mark.parametrize("B", [2, 10, 16, 64])
def test_accept_len_per_sequence_block_sizes(B):
    R = runtime()
    rng = np.random.default_rng(B)
    batch = 300
    d = rng.integers(0, 50, size=(batch, B - 1)).astype(np.int32)
    y = np.where(rng.random((batch, B)) < 0.8, np.pad(d, ((0, 0), (0, 1))), rng.integers(0, 50, (batch, B)))
    y = y.astype(np.int32)
    bl = rng.integers(0, B + 3, size=batch).astype(np.int32)         # includes values clamped to 1..B
    tau, bonus = R.Drafter.accept_len_ragged(torch.from_numpy(d).cuda(), torch.from_numpy(y).cuda(), B,
                                             torch.from_numpy(bl).cuda())
    tau, bonus = tau.cpu().numpy(), bonus.cpu().numpy()
    for s in range(batch):
        bs = min(max(int(bl[s]), 1), B)
        t_o, b_o = D.accept_len(d[s, :bs - 1], y[s, :bs])
        assert (tau[s], bonus[s]) == (t_o, b_o), (s, bs)
    t0, b0 = R.Drafter.accept_len_ragged(torch.from_numpy(d).cuda(), torch.from_numpy(y).cuda(), B, None)
    t1, b1 = R.Drafter.accept_len(torch.from_numpy(d).cuda(), torch.from_numpy(y).cuda(), B)
    assert torch.equal(t0, t1) and torch.equal(b0, b1)


def test_check_inputs_flags_each_bad_index():
    """dflash_check_inputs on valid indices reports 0, and each kind of bad
    device index sets its own bit (the bad values go to the check kernel only)."""
    cfg = MINI["mini_bf16"]
    R = runtime()
    w = S.drafter_weights(cfg, seed=8)
    lens = np.array([5, 300, 17], dtype=np.int32)
    B, ps = cfg.block_size, cfg.page_size
    lay = S.paged_layout(cfg, lens, headroom=B, seed=8)
    dr = R.Drafter(cfg, w, max_batch=3, max_ctx=int(lens.max()), max_new=4)
    anchors = torch.from_numpy(S.anchor_ids(cfg, seed=8, batch=3)).cuda()
    ids = torch.randint(0, cfg.vocab, (40,), dtype=torch.int32, device="cuda")
    seq = torch.tensor([0, 1, 2, 1], dtype=torch.int32, device="cuda")
    pos = torch.tensor([0, 299, 20, 310], dtype=torch.int32, device="cuda")

    def run(table=None, ctx=None, anc=anchors, tok=ids, sq=seq, ps_=pos):
        kv = R.PagedKV(cfg, lay.block_table if table is None else table, lens if ctx is None else ctx, lay.n_pages,
                       max_ctx=int(lens.max()))
        return dr.check_inputs(kv, anchor_ids=anc, ids=tok, seq=sq, pos=ps_)

    assert run() == 0
    assert run(anc=None, tok=None, sq=None, ps_=None) == 0
    assert run(ctx=np.array([5, 301, 17], dtype=np.int32)) & 1           # above max_ctx
    assert run(ctx=np.array([-1, 300, 17], dtype=np.int32)) == 1
    t = lay.block_table.copy(); t[1, 3] = lay.n_pages                    # a context page of seq 1
    assert run(table=t) == 2
    t = lay.block_table.copy(); t[2, (17 + B - 1) // ps] = -1            # a page only the block covers
    assert run(table=t) == 4
    bad_anc = anchors.clone(); bad_anc[2] = cfg.vocab
    assert run(anc=bad_anc) == 8
    bad_ids = ids.clone(); bad_ids[39] = -5
    assert run(tok=bad_ids) == 8
    assert run(sq=torch.tensor([0, 3, 2, 1], dtype=torch.int32, device="cuda")) == 16
    big = lay.block_table.shape[1] * ps
    assert run(ps_=torch.tensor([0, big, 20, 1], dtype=torch.int32, device="cuda")) == 16
    t = lay.block_table.copy(); t[1, 310 // ps] = lay.n_pages + 7        # the page an inject slot lands in
    assert run(table=t) & 16
    dr.close()


def test_draft_block_empty_and_short_context():
    cfg = MINI["mini_bf16"]
    log("draft_block ctx 0/1/16")
    run_draft_case(cfg, seed=5, lens=[0, 1, 16])


def test_draft_independent_of_anchor_for_cache():
    """Context K/V written by inject depend on the features only."""
    cfg = MINI["mini_bf16"]
    R = runtime()
    log("inject/draft cache independence")
    w = S.drafter_weights(cfg, seed=4)
    lens = np.array([40], dtype=np.int32)
    lay = S.paged_layout(cfg, lens, headroom=cfg.block_size, seed=4)
    feats = R.to_device(S.features(cfg, 40, seed=4))
    seq = torch.zeros(40, dtype=torch.int32, device="cuda")
    pos = torch.arange(40, dtype=torch.int32, device="cuda")
    dr = R.Drafter(cfg, w, max_batch=1, max_ctx=40, max_new=40)
    kv = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages)
    dr.inject_context(feats, seq, pos, kv)
    k0 = kv.k.clone()
    for a in (3, 77, cfg.vocab - 1):
        dr.draft_block(torch.tensor([a], dtype=torch.int32, device="cuda"), kv)
    kv2 = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages)
    dr.inject_context(feats, seq, pos, kv2)
    torch.cuda.synchronize()
    assert torch.equal(kv.k, k0) and torch.equal(kv2.k, k0) and torch.equal(kv2.v, kv.v)
    dr.close()


# ----------------------------------------------------------------------------
# end to end: greedy speculative decoding with the GPU drafter is lossless
# ----------------------------------------------------------------------------
class GpuDrafter:
    """Speculative-loop adapter: the GPU drafter behind the C ABI."""

    def __init__(self, cfg, w, max_positions):
        R = runtime()
        self.R, self.cfg = R, cfg
        self.d = R.Drafter(cfg, w, max_batch=1, max_ctx=max_positions, max_new=max_positions)
        lay = S.paged_layout(cfg, np.array([max_positions]), headroom=0, seed=9)
        self.kv = R.PagedKV(cfg, lay.block_table, np.array([0]), lay.n_pages)
        self.ctx = 0

    def inject(self, feats, pos):
        R = self.R
        f = R.to_device(storage_of(self.cfg, feats))
        seq = torch.zeros(len(pos), dtype=torch.int32, device="cuda")
        p = torch.from_numpy(np.asarray(pos, dtype=np.int32)).cuda()
        self.d.inject_context(f, seq, p, self.kv)
        self.ctx += len(pos)
        self.kv.set_ctx_len(np.array([self.ctx]))

    def draft(self, anchor):
        hid = self.d.draft_block(torch.tensor([anchor], dtype=torch.int32, device="cuda"), self.kv)
        ids, _, _ = self.d.lmhead_argmax(hid, want_max=False)
        return ids.cpu().numpy()


class ShadowDrafter:
    """The GPU drafter, checked at every cycle against the oracle drafter fed the
    same injected features: the drafts must agree (ids may differ only on an
    oracle near-tie within the fp32 bar)."""

    def __init__(self, gpu: GpuDrafter, oracle: D.OracleDrafter):
        self.gpu, self.oracle = gpu, oracle
        self.excused, self.cycles = 0, 0

    def inject(self, feats, pos):
        self.gpu.inject(feats, pos)
        self.oracle.inject(feats, pos)

    def draft(self, anchor):
        g = self.gpu.draft(anchor)
        o = self.oracle
        Z = D.draft_block(o.w, o.cfg, anchor, o.K, o.V)
        ids_o, _, logits_o = D.lm_argmax(o.w["lm_head"], Z)
        self.excused += check_ids(g, ids_o, logits_o, 1e-4, f"cycle {self.cycles} drafts")
        self.cycles += 1
        return g


@pytest.mark.parametrize("seed,layer_std", [(0, 0.02), (1, 0.1), (2, 0.05)])
def test_lossless_speculative_decoding_with_gpu_drafter(seed, layer_std):
    from oracle import target as T
    cfg = MINI["tiny"]
    log(f"lossless e2e seed={seed} layer_std={layer_std}")
    tgt = T.TinyTarget(S.target_weights(cfg, seed, layer_std=layer_std), cfg)
    prompt = S.prompt_ids(cfg, seed)
    g = T.greedy_decode(tgt, prompt, cfg.new_tokens)
    gd = GpuDrafter(cfg, S.drafter_weights(cfg, seed), cfg.prompt_len + cfg.new_tokens + 2 * cfg.block_size)
    shadow = ShadowDrafter(gd, D.OracleDrafter(S.drafter_weights(cfg, seed), cfg))
    s, taus = T.spec_decode(tgt, shadow, prompt, cfg.new_tokens, cfg.dtype)
    assert np.array_equal(g, s)
    # the oracle drafter alone takes the same cycles unless a near-tie was excused
    s2, taus2 = T.spec_decode(tgt, D.OracleDrafter(S.drafter_weights(cfg, seed), cfg), prompt, cfg.new_tokens,
                              cfg.dtype)
    assert np.array_equal(s2, g)
    log(f"  taus gpu {taus} oracle {taus2}; {shadow.excused} draft ids tie-excused over {shadow.cycles} cycles")
    if shadow.excused == 0:
        assert taus == taus2
    gd.d.close()


# ----------------------------------------------------------------------------
# streaming-read helper (measures the read ceiling the draft step is reported against)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("n16", [1, 1000, 8192 * 3 + 77])
def test_stream_read_folds_every_word(n16):
    log(f"stream_read n16={n16}")
    from block_diffusion_drafter_gemm_amd import _lib
    rng = np.random.default_rng(n16)
    words = rng.integers(0, 2 ** 31 - 1, size=4 * n16, dtype=np.int64).astype(np.int32)
    x = torch.from_numpy(words).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    _lib.dflash_stream_read(x, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy()[0]) == int(np.bitwise_xor.reduce(words))
