"""Shared setup of the GPU parity tests (not collected by pytest).

Inputs come from ``dflash_synth`` only; expected values come from ``oracle``
only.  The HIP path is reached through the C ABI (``runtime.Drafter``).
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np

import dflash_synth as S
from oracle import drafter as D
from oracle.numerics import from_storage


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def mini(name: str, cid: int, **kw) -> S.Config:
    base = S.get_config("tiny")
    f = dict(target_layers=0, feat_layer_ids=(), prompt_len=0, new_tokens=0)
    f.update(kw)
    return dataclasses.replace(base, name=name, cid=cid, **f)


# small shapes with ragged tails (vocab not a multiple of 128, contexts not a
# multiple of the page size, padded query tiles)
MINI = {
    "mini_bf16": mini("mini_bf16", 101, dtype="bf16", hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                      ffn=1088, vocab=4112, n_layers=2, n_feat_layers=3, block_size=16, batch=3,
                      ctx_min=5, ctx_max=300, rope_theta=1e6),
    "mini_b10": mini("mini_b10", 102, dtype="bf16", hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                     ffn=1024, vocab=2064, n_layers=2, n_feat_layers=2, block_size=10, batch=2,
                     ctx_min=1, ctx_max=700, rope_theta=5e5),
    "mini_d64": mini("mini_d64", 103, dtype="bf16", hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
                     ffn=512, vocab=1024, n_layers=2, n_feat_layers=3, block_size=4, batch=2,
                     ctx_min=40, ctx_max=90, rope_theta=1e6),
    "mini_f32": mini("mini_f32", 104, dtype="f32", hidden=256, n_q_heads=8, n_kv_heads=2, head_dim=128,
                     ffn=256, vocab=528, n_layers=2, n_feat_layers=2, block_size=8, batch=2,
                     ctx_min=17, ctx_max=150, rope_theta=1e6),
    # batch 8 x B 16 = 128 block rows: the many-rows (LDS-tiled) GEMM path
    "mini_b8": mini("mini_b8", 105, dtype="bf16", hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                    ffn=1088, vocab=4096, n_layers=2, n_feat_layers=3, block_size=16, batch=8,
                    ctx_min=3, ctx_max=400, rope_theta=1e6),
    # FFN and feature widths above one 4096-wide LDS portion (ragged last portion)
    "mini_port": mini("mini_port", 106, dtype="bf16", hidden=256, n_q_heads=2, n_kv_heads=1, head_dim=128,
                      ffn=4352, vocab=1040, n_layers=2, n_feat_layers=17, block_size=8, batch=2,
                      ctx_min=30, ctx_max=200, rope_theta=1e6),
    # 48 block rows with wide outputs (FFN 4096, vocabulary 66 x 128): gate/up and
    # the LM head take the many-rows (LDS-tiled) GEMM below 65 rows
    "mini_wide": mini("mini_wide", 107, dtype="bf16", hidden=256, n_q_heads=2, n_kv_heads=2, head_dim=128,
                      ffn=4096, vocab=8448, n_layers=2, n_feat_layers=2, block_size=16, batch=3,
                      ctx_min=20, ctx_max=180, rope_theta=1e6),
    # 8 query heads per KV head x B 16 = 128 block queries per KV head (8 query tiles)
    "mini_g8": mini("mini_g8", 108, dtype="bf16", hidden=512, n_q_heads=8, n_kv_heads=1, head_dim=128,
                    ffn=512, vocab=1040, n_layers=2, n_feat_layers=2, block_size=16, batch=2,
                    ctx_min=10, ctx_max=260, rope_theta=1e6),
    # 160 block rows, FFN and vocabulary of 321 128-column blocks each: gate/up and
    # the LM head take the 256 x 256-tile GEMM, whose last tile has a second
    # column block past the end, with a ragged row block
    "mini_big": mini("mini_big", 109, dtype="bf16", hidden=256, n_q_heads=2, n_kv_heads=2, head_dim=128,
                     ffn=20544, vocab=41088, n_layers=2, n_feat_layers=2, block_size=16, batch=10,
                     ctx_min=5, ctx_max=150, rope_theta=1e6),
    # 144 block rows (ragged second 128-row block), FFN 4096: the down projection
    # has 4 tiles and splits K over 4 workgroups per tile (fp32 partials + reduction)
    "mini_split": mini("mini_split", 110, dtype="bf16", hidden=256, n_q_heads=2, n_kv_heads=2, head_dim=128,
                       ffn=4096, vocab=8448, n_layers=2, n_feat_layers=2, block_size=16, batch=9,
                       ctx_min=3, ctx_max=120, rope_theta=1e6),
    # 8 ragged sequences of up to 16384 positions: attention items of 256
    # keys (4 K/V sub-blocks per item, the last item of a sequence partly
    # empty), one layer
    "mini_long": mini("mini_long", 111, dtype="bf16", hidden=256, n_q_heads=8, n_kv_heads=2, head_dim=128,
                      ffn=512, vocab=1040, n_layers=1, n_feat_layers=2, block_size=16, batch=8,
                      ctx_min=2000, ctx_max=16384, rope_theta=1e6),
    # one sequence with an FFN past the 4096 resident columns: the down projection
    # on split pairs (two workgroups per 32-column tile, half of K each)
    "mini_ffn_b1": mini("mini_ffn_b1", 112, dtype="bf16", hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                        ffn=4608, vocab=2064, n_layers=2, n_feat_layers=2, block_size=16, batch=1,
                        ctx_min=150, ctx_max=150, rope_theta=1e6),
    "tiny": S.get_config("tiny"),
}


def tol_of(cfg) -> float:
    return 1e-4 if cfg.dtype == "f32" else 2e-2


def assert_close(got, want, tol: float, what: str) -> None:
    """|got - want| <= tol * max(1, |want|) elementwise."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got - want) / np.maximum(1.0, np.abs(want))
    worst = float(err.max()) if err.size else 0.0
    log(f"  {what}: max scaled error {worst:.3e} (tol {tol:g})")
    assert worst <= tol, f"{what}: max scaled error {worst:.3e} > {tol:g}"


def assert_rows_close(got, want, tol: float, what: str) -> float:
    """Per-row normwise relative error ||got - want|| / ||want|| <= tol."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(want)[-1])
    want = np.asarray(want, dtype=np.float64).reshape(got.shape)
    num = np.linalg.norm(got - want, axis=1)
    den = np.maximum(np.linalg.norm(want, axis=1), 1e-30)
    rel = num / den
    el = np.abs(got - want) / np.maximum(1.0, np.abs(want))
    log(f"  {what}: row-norm relative error max {rel.max():.3e} mean {rel.mean():.3e} "
        f"(tol {tol:g}); elementwise max {el.max():.3e}")
    assert rel.max() <= tol, f"{what}: row-norm relative error {rel.max():.3e} > {tol:g}"
    return float(rel.max())


def check_ids(ids_gpu, ids_oracle, logits_oracle, tol: float, what: str) -> int:
    """Token ids must match, except where the GPU's choice is an oracle near-tie:
    oracle_logit[g] >= oracle_logit[o] - tol * max(1, |oracle_logit[o]|)."""
    ids_gpu = np.asarray(ids_gpu).reshape(-1)
    ids_oracle = np.asarray(ids_oracle).reshape(-1)
    excused = 0
    for r, (g, o) in enumerate(zip(ids_gpu, ids_oracle)):
        if g == o:
            continue
        lo = logits_oracle[r, o]
        assert 0 <= g < logits_oracle.shape[1], (what, r, g)
        assert logits_oracle[r, g] >= lo - tol * max(1.0, abs(lo)), \
            f"{what}: row {r} gpu id {g} (logit {logits_oracle[r, g]:.6f}) vs oracle id {o} (logit {lo:.6f})"
        excused += 1
    log(f"  {what}: {len(ids_gpu) - excused}/{len(ids_gpu)} ids identical, {excused} tie-excused")
    return excused


def layout_for(cfg, lens, headroom, seed=0):
    return S.paged_layout(cfg, lens, headroom, seed=seed)


def gather_ctx(cfg, Kp: np.ndarray, Vp: np.ndarray, table: np.ndarray, s: int, ctx: int):
    """Dense float64 context K/V [n_layers, ctx, nkv, d] of sequence s from the paged arrays."""
    t = np.arange(ctx)
    pages = table[s, t // cfg.page_size]
    slots = t % cfg.page_size
    return from_storage(Kp[:, pages, slots]), from_storage(Vp[:, pages, slots])


def oracle_draft(cfg, w, anchor, Kp, Vp, table, s, ctx):
    Kc, Vc = gather_ctx(cfg, Kp, Vp, table, s, ctx)
    return D.draft_block(w, cfg, int(anchor), Kc, Vc)
