"""Seeded synthetic inputs for the DFlash drafter step.

This module only holds workload shapes and seeded random draws.  It performs
none of the drafter's arithmetic: both the CPU oracle and the HIP path consume
the arrays it returns, so the two sides see identical bytes.

Shapes follow the models the DFlash pages evaluate (Qwen3-8B, LLaMA-3.1-8B,
Qwen3-Coder-30B-A3B; "기술 요약: DFlash" summary, section 4), the block sizes
the field notes give (B=16 for Qwen3, B=10 for LLaMA-3.1-8B; DFlash field
notes, section 2), single-stream and concurrency-32 serving (field notes,
section 4.4) and long inputs (field notes, section 4.3).

Storage conventions
-------------------
* bf16 tensors are returned as ``numpy.uint16`` arrays holding the raw bf16
  bit patterns (round-to-nearest-even from an fp32 draw).
* fp32 tensors (the tiny end-to-end configuration) are ``numpy.float32``.
* Every large tensor is drawn in row chunks, each from its own generator keyed
  by ``(config id, tensor tag, seed, chunk index)``.  Chunks can therefore be
  drawn in parallel and any row can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Config", "CONFIGS", "get_config", "bf16_bits_from_f32", "f32_from_bf16_bits",
    "normal_matrix", "drafter_weights", "target_weights", "features", "prompt_ids",
    "anchor_ids", "ctx_lens", "PagedLayout", "paged_layout", "ctx_kv_cache",
    "target_ids_for", "draft_ids_random", "kv_sigma",
]


# ----------------------------------------------------------------------------
# Workload configurations
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cid: int                    # seed namespace of the configuration
    dtype: str                  # "f32" or "bf16": storage type of weights/features
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_layers: int               # drafter layers
    n_feat_layers: int          # target layers whose hidden states are fused
    block_size: int             # B: anchor + (B-1) masks
    batch: int
    ctx_min: int                # context length range (inclusive); min == max: fixed
    ctx_max: int
    rope_theta: float
    rms_eps: float = 1e-6
    page_size: int = 16
    match_rate: float = 0.7     # synthetic target agreement per position
    window: int = 0             # > 0: sliding-window context (last `window` positions)
    ctx_norm: int = 0           # 1: RMSNorm after the fusion projection (gain "ctx_norm")
    # tiny end-to-end target (only the "tiny" configuration)
    target_layers: int = 0
    feat_layer_ids: Tuple[int, ...] = ()
    prompt_len: int = 0
    new_tokens: int = 0

    @property
    def mask_token_id(self) -> int:
        return self.vocab - 1

    @property
    def feat_dim(self) -> int:
        return self.n_feat_layers * self.hidden

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def rows(self) -> int:
        return self.batch * self.block_size

    def layer_params(self) -> int:
        h, d = self.hidden, self.head_dim
        qkv = self.qkv_rows * h
        o = h * self.n_q_heads * d
        mlp = 3 * self.ffn * h
        return self.n_layers * (qkv + o + mlp + 2 * h) + self.feat_dim * h + h


CONFIGS: Dict[str, Config] = {
    # Tiny fp32 end-to-end check: 4-layer target, 2-layer drafter of the same
    # shape, features from target layers {1,2,3}, B=4, 64-token prompt, 32 new.
    "tiny": Config("tiny", 1, "f32", hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
                   ffn=512, vocab=1024, n_layers=2, n_feat_layers=3, block_size=4,
                   batch=1, ctx_min=64, ctx_max=64, rope_theta=1e6,
                   target_layers=4, feat_layer_ids=(1, 2, 3), prompt_len=64, new_tokens=32),
    # Qwen3-8B-shaped drafter, batch 1, context 2048, B=16.
    "qwen3_8b": Config("qwen3_8b", 2, "bf16", hidden=4096, n_q_heads=32, n_kv_heads=8,
                       head_dim=128, ffn=12288, vocab=151936, n_layers=5, n_feat_layers=5,
                       block_size=16, batch=1, ctx_min=2048, ctx_max=2048, rope_theta=1e6),
    # LLaMA-3.1-8B-shaped drafter, batch 1, context 4096, B=10.
    "llama31_8b": Config("llama31_8b", 3, "bf16", hidden=4096, n_q_heads=32, n_kv_heads=8,
                         head_dim=128, ffn=14336, vocab=128256, n_layers=5, n_feat_layers=5,
                         block_size=10, batch=1, ctx_min=4096, ctx_max=4096, rope_theta=5e5),
    # Batched serving: Qwen3-8B drafter, 32 sequences, ragged context 512..8192.
    "qwen3_8b_b32": Config("qwen3_8b_b32", 4, "bf16", hidden=4096, n_q_heads=32, n_kv_heads=8,
                           head_dim=128, ffn=12288, vocab=151936, n_layers=5, n_feat_layers=5,
                           block_size=16, batch=32, ctx_min=512, ctx_max=8192, rope_theta=1e6),
    # Qwen3-Coder-30B-A3B-shaped 8-layer dense drafter, batch 4, context 16384.
    "qwen3_coder_30b": Config("qwen3_coder_30b", 5, "bf16", hidden=2048, n_q_heads=32,
                              n_kv_heads=4, head_dim=128, ffn=6144, vocab=151936, n_layers=8,
                              n_feat_layers=5, block_size=16, batch=4, ctx_min=16384,
                              ctx_max=16384, rope_theta=1e6),
}

CONFIG_ORDER = ["tiny", "qwen3_8b", "llama31_8b", "qwen3_8b_b32", "qwen3_coder_30b"]


def get_config(name: str, **overrides) -> Config:
    """Return a named configuration, optionally with fields replaced (small test shapes)."""
    cfg = CONFIGS[name]
    return dataclasses.replace(cfg, **overrides) if overrides else cfg


# ----------------------------------------------------------------------------
# bf16 storage (bit patterns)
# ----------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> the fp32 value it encodes (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Chunked, seeded normal draws
# ----------------------------------------------------------------------------
_CHUNK_ELEMS = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))

# tensor tags (the seed namespace inside a configuration)
TAG_EMBED, TAG_LM_HEAD, TAG_W_FC, TAG_FEATS, TAG_CACHE_K, TAG_CACHE_V = 1, 2, 3, 4, 5, 6
TAG_ANCHOR, TAG_CTX, TAG_PAGES, TAG_TARGET, TAG_PROMPT, TAG_DRAFT, TAG_GAIN = 7, 8, 9, 10, 11, 12, 13
TAG_LAYER = 100          # + 16 * layer + slot
TAG_TARGET_LAYER = 1000  # + 16 * layer + slot (tiny target)
TAG_TARGET_MISC = 2000


def _rng(cfg: Config, tag: int, seed: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg.cid, tag, seed, chunk])


def normal_matrix(cfg: Config, tag: int, shape: Tuple[int, ...], std: float, seed: int = 0,
                  dtype: Optional[str] = None, row_range: Optional[Tuple[int, int]] = None) -> np.ndarray:
    """N(0, std^2) matrix drawn in fp32 row chunks, returned in the storage dtype.

    ``row_range`` regenerates only rows [r0, r1) (same values as the full draw).
    """
    dtype = dtype or cfg.dtype
    rows = int(shape[0])
    cols = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    chunk_rows = max(1, _CHUNK_ELEMS // max(cols, 1))
    r0, r1 = row_range if row_range is not None else (0, rows)
    out = np.empty((r1 - r0, cols), dtype=np.uint16 if dtype == "bf16" else np.float32)
    c_first, c_last = r0 // chunk_rows, (r1 - 1) // chunk_rows if r1 > r0 else -1

    def work(c: int) -> None:
        cr0 = c * chunk_rows
        cr1 = min(rows, cr0 + chunk_rows)
        blk = _rng(cfg, tag, seed, c).standard_normal((cr1 - cr0, cols), dtype=np.float32)
        blk *= np.float32(std)
        a, b = max(cr0, r0), min(cr1, r1)
        sub = blk[a - cr0:b - cr0]
        out[a - r0:b - r0] = bf16_bits_from_f32(sub) if dtype == "bf16" else sub

    chunks = list(range(c_first, c_last + 1))
    if len(chunks) > 1:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, chunks))
    else:
        for c in chunks:
            work(c)
    return out.reshape((r1 - r0,) + tuple(shape[1:]))


def _gain(cfg: Config, tag: int, n: int, seed: int, random_gain: bool) -> np.ndarray:
    """RMSNorm gain: 1.0 by default; N(1, 0.1^2) when ``random_gain`` (tests only)."""
    if random_gain:
        g = 1.0 + 0.1 * _rng(cfg, TAG_GAIN, seed, tag).standard_normal(n).astype(np.float32)
    else:
        g = np.ones(n, dtype=np.float32)
    return bf16_bits_from_f32(g) if cfg.dtype == "bf16" else g


# ----------------------------------------------------------------------------
# Weights
# ----------------------------------------------------------------------------
def drafter_weights(cfg: Config, seed: int = 0, random_gain: bool = False,
                    include_heads: bool = True) -> dict:
    """Drafter weights in the storage dtype, row-major ``[out, in]``.

    Keys: ``embed [V,H]``, ``lm_head [V,H]`` (shared with the target),
    ``w_fc [H, L*H]``, ``final_norm [H]`` and per layer (lists)
    ``attn_norm [H]``, ``w_qkv [(nq+2nkv)*d, H]`` (q rows, then k, then v),
    ``w_o [H, nq*d]``, ``mlp_norm [H]``, ``w_gate_up [2F, H]`` (gate rows first),
    ``w_down [H, F]``.  Matrices are N(0, 0.02^2); gains are 1.
    """
    H, std = cfg.hidden, 0.02
    w = {}
    if include_heads:
        w["embed"] = normal_matrix(cfg, TAG_EMBED, (cfg.vocab, H), std, seed)
        w["lm_head"] = normal_matrix(cfg, TAG_LM_HEAD, (cfg.vocab, H), std, seed)
    w["w_fc"] = normal_matrix(cfg, TAG_W_FC, (H, cfg.feat_dim), std, seed)
    w["final_norm"] = _gain(cfg, 3, H, seed, random_gain)
    if cfg.ctx_norm:
        w["ctx_norm"] = _gain(cfg, 4, H, seed, random_gain)
    for key in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down"):
        w[key] = []
    for l in range(cfg.n_layers):
        base = TAG_LAYER + 16 * l
        w["attn_norm"].append(_gain(cfg, base + 0, H, seed, random_gain))
        w["w_qkv"].append(normal_matrix(cfg, base + 1, (cfg.qkv_rows, H), std, seed))
        w["w_o"].append(normal_matrix(cfg, base + 2, (H, cfg.n_q_heads * cfg.head_dim), std, seed))
        w["mlp_norm"].append(_gain(cfg, base + 3, H, seed, random_gain))
        w["w_gate_up"].append(normal_matrix(cfg, base + 4, (2 * cfg.ffn, H), std, seed))
        w["w_down"].append(normal_matrix(cfg, base + 5, (H, cfg.ffn), std, seed))
    return w


def target_weights(cfg: Config, seed: int = 0, layer_std: float = 0.02) -> dict:
    """Tiny target decoder weights (same layout as the drafter's layers).

    ``embed`` and ``lm_head`` are the same draws as the drafter's (shared heads),
    N(0, 0.02^2).  ``layer_std`` scales the decoder-layer matrices; values above
    0.02 give a target whose greedy output depends on more than the last token.
    """
    H, std = cfg.hidden, 0.02
    w = {"embed": normal_matrix(cfg, TAG_EMBED, (cfg.vocab, H), std, seed),
         "lm_head": normal_matrix(cfg, TAG_LM_HEAD, (cfg.vocab, H), std, seed),
         "final_norm": _gain(cfg, TAG_TARGET_MISC, H, seed, False)}
    for key in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down"):
        w[key] = []
    for l in range(cfg.target_layers):
        base = TAG_TARGET_LAYER + 16 * l
        ls = layer_std
        w["attn_norm"].append(_gain(cfg, base + 0, H, seed, False))
        w["w_qkv"].append(normal_matrix(cfg, base + 1, (cfg.qkv_rows, H), ls, seed))
        w["w_o"].append(normal_matrix(cfg, base + 2, (H, cfg.n_q_heads * cfg.head_dim), ls, seed))
        w["mlp_norm"].append(_gain(cfg, base + 3, H, seed, False))
        w["w_gate_up"].append(normal_matrix(cfg, base + 4, (2 * cfg.ffn, H), ls, seed))
        w["w_down"].append(normal_matrix(cfg, base + 5, (H, cfg.ffn), ls, seed))
    return w


# ----------------------------------------------------------------------------
# Activations, ids, lengths, page tables
# ----------------------------------------------------------------------------
def features(cfg: Config, n: int, seed: int = 0, stream: int = 0) -> np.ndarray:
    """Concatenated target-layer features ``[n, L*H]`` ~ N(0, 1), storage dtype.

    Rows are drawn in fixed chunks, so the first rows do not depend on ``n``.
    """
    return normal_matrix(cfg, TAG_FEATS + 100 * stream, (n, cfg.feat_dim), 1.0, seed)


def prompt_ids(cfg: Config, seed: int = 0) -> np.ndarray:
    return _rng(cfg, TAG_PROMPT, seed).integers(0, cfg.vocab, cfg.prompt_len, dtype=np.int64).astype(np.int32)


def anchor_ids(cfg: Config, seed: int = 0, batch: Optional[int] = None) -> np.ndarray:
    b = cfg.batch if batch is None else batch
    return _rng(cfg, TAG_ANCHOR, seed).integers(0, cfg.vocab, b, dtype=np.int64).astype(np.int32)


def draft_ids_random(cfg: Config, batch: int, seed: int = 0) -> np.ndarray:
    """Uniform draft ids ``[batch, B-1]`` (stand-in drafts for verify tests)."""
    return _rng(cfg, TAG_DRAFT, seed).integers(
        0, cfg.vocab, (batch, cfg.block_size - 1), dtype=np.int64).astype(np.int32)


def ctx_lens(cfg: Config, seed: int = 0, batch: Optional[int] = None) -> np.ndarray:
    b = cfg.batch if batch is None else batch
    if cfg.ctx_min == cfg.ctx_max:
        return np.full(b, cfg.ctx_min, dtype=np.int32)
    return _rng(cfg, TAG_CTX, seed).integers(cfg.ctx_min, cfg.ctx_max + 1, b, dtype=np.int64).astype(np.int32)


@dataclasses.dataclass
class PagedLayout:
    """Page table of a paged context cache (page size ``page_size`` positions)."""
    block_table: np.ndarray  # [batch, max_pages] int32 physical page ids (-1: unused)
    max_pages: int
    n_pages: int


def paged_layout(cfg: Config, lens: np.ndarray, headroom: int, seed: int = 0,
                 permute: bool = True) -> PagedLayout:
    """Assign physical pages for ``lens[s] + headroom`` positions of every sequence.

    The pool is a seeded random permutation of the physical pages, so a
    sequence's logical pages are scattered through memory.
    """
    ps = cfg.page_size
    need = [(int(n) + headroom + ps - 1) // ps for n in lens]
    max_pages = max(need) if need else 1
    n_pages = int(sum(need))
    perm = (_rng(cfg, TAG_PAGES, seed).permutation(n_pages) if permute
            else np.arange(n_pages)).astype(np.int32)
    table = np.full((len(lens), max_pages), -1, dtype=np.int32)
    off = 0
    for s, k in enumerate(need):
        table[s, :k] = perm[off:off + k]
        off += k
    return PagedLayout(table, max_pages, n_pages)


def kv_sigma(cfg: Config) -> float:
    """Std of injected context K/V for N(0,1) features and N(0,0.02^2) weights.

    c = W_fc f has variance L*H*0.02^2; k = W_k c then has variance
    H*0.02^2 times that.  Synthetic caches use this scale.
    """
    return float(np.sqrt(cfg.hidden * 0.02 ** 2 * cfg.feat_dim * 0.02 ** 2))


def ctx_kv_cache(cfg: Config, layout: PagedLayout, seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Synthetic paged context K and V ``[n_layers, n_pages, page, nkv, d]``.

    Entries are N(0, kv_sigma^2), drawn per (layer, page) in the storage dtype.
    Unused slots hold draws too; readers only touch valid positions.
    """
    shape = (cfg.n_layers * layout.n_pages, cfg.page_size * cfg.n_kv_heads * cfg.head_dim)
    full = (cfg.n_layers, layout.n_pages, cfg.page_size, cfg.n_kv_heads, cfg.head_dim)
    sig = kv_sigma(cfg)
    k = normal_matrix(cfg, TAG_CACHE_K, shape, sig, seed).reshape(full)
    v = normal_matrix(cfg, TAG_CACHE_V, shape, sig, seed).reshape(full)
    return k, v


def target_ids_for(cfg: Config, draft: np.ndarray, seed: int = 0) -> np.ndarray:
    """Synthetic target ids ``[batch, B]`` agreeing with ``draft`` at rate ``match_rate``.

    Per position i < B-1: with probability match_rate y_i = d_i, otherwise
    y_i = (d_i + 1 + u_i) mod V with u_i uniform in [0, V-1), which never equals
    d_i.  y_{B-1} (the last target row) is uniform in [0, V).  The random draws
    do not depend on ``draft``, so equal drafts give equal targets.
    """
    draft = np.asarray(draft, dtype=np.int64)
    b, bm1 = draft.shape
    rng = _rng(cfg, TAG_TARGET, seed)
    match = rng.random((b, bm1)) < cfg.match_rate
    u = rng.integers(0, cfg.vocab - 1, (b, bm1), dtype=np.int64)
    last = rng.integers(0, cfg.vocab, (b, 1), dtype=np.int64)
    y = np.where(match, draft, (draft + 1 + u) % cfg.vocab)
    return np.concatenate([y, last], axis=1).astype(np.int32)
