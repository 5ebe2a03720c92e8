"""Device-resident drafter state around the C ABI: weights, paged context cache
and workspace as torch tensors (torch only supplies memory and streams).

``Drafter`` takes any configuration object exposing the drafter shape fields
(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, n_layers, n_feat_layers,
block_size, mask_token_id, dtype, rope_theta, rms_eps) and host weight arrays
(bf16 as uint16 bit patterns, or float32).
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _lib as L

_LAYER_KEYS = ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Host array -> device tensor with the same bytes (bf16 bits travel as int16);
    a torch tensor already on the device is kept as it is."""
    if isinstance(a, torch.Tensor):
        return a.to(device)
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


def to_host_storage(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array (int16-held bf16 back to uint16 bit patterns)."""
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def storage_dtype(cfg) -> torch.dtype:
    return torch.int16 if cfg.dtype == "bf16" else torch.float32


class PagedKV:
    """Paged context cache [n_layers][n_pages][16][nkv][d] plus page table and lengths."""

    def __init__(self, cfg, block_table: np.ndarray, ctx_len: np.ndarray, n_pages: int,
                 k: Optional[np.ndarray] = None, v: Optional[np.ndarray] = None, device="cuda",
                 max_ctx: Optional[int] = None):
        self.cfg = cfg
        shape = (cfg.n_layers, n_pages, cfg.page_size, cfg.n_kv_heads, cfg.head_dim)
        dt = storage_dtype(cfg)
        self.k = to_device(k, device) if k is not None else torch.zeros(shape, dtype=dt, device=device)
        self.v = to_device(v, device) if v is not None else torch.zeros(shape, dtype=dt, device=device)
        assert tuple(self.k.shape) == shape and tuple(self.v.shape) == shape
        self.block_table = torch.from_numpy(np.ascontiguousarray(block_table, dtype=np.int32)).to(device)
        self.ctx_len = torch.from_numpy(np.ascontiguousarray(ctx_len, dtype=np.int32)).to(device)
        self.batch, self.max_pages = int(block_table.shape[0]), int(block_table.shape[1])
        self.n_pages = int(n_pages)
        self.max_ctx = int(max_ctx if max_ctx is not None else int(np.max(ctx_len)))
        self.block_len = None   # optional device [batch] int32: per-sequence block sizes

    def set_block_len(self, block_len: Optional[np.ndarray]) -> None:
        self.block_len = None if block_len is None else torch.from_numpy(
            np.ascontiguousarray(block_len, dtype=np.int32)).to(self.ctx_len.device)

    def set_ctx_len(self, ctx_len: np.ndarray, max_ctx: Optional[int] = None) -> None:
        self.ctx_len.copy_(torch.from_numpy(np.ascontiguousarray(ctx_len, dtype=np.int32)))
        self.max_ctx = int(max_ctx if max_ctx is not None else int(np.max(ctx_len)))

    def struct(self) -> L.DflashKV:
        return L.make_kv(self.k, self.v, self.block_table, self.ctx_len, self.batch, self.max_pages,
                         self.n_pages, self.max_ctx, self.block_len)


class Drafter:
    """One drafter handle with its device weights and a workspace."""

    def __init__(self, cfg, weights: dict, max_batch: int, max_ctx: int, max_new: int, device="cuda"):
        L.load()
        self.cfg = cfg
        self.device = device
        self.w = {k: ([to_device(x, device) for x in v] if isinstance(v, list) else to_device(v, device))
                  for k, v in weights.items()}
        c = L.make_config(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.vocab,
                          cfg.n_layers, cfg.n_feat_layers, cfg.block_size, cfg.mask_token_id, cfg.dtype,
                          cfg.rope_theta, cfg.rms_eps, cfg.page_size, getattr(cfg, "window", 0),
                          getattr(cfg, "ctx_norm", 0))
        ws, self._keep = L.make_weights(self.w["embed"], self.w["lm_head"], self.w.get("w_fc"), self.w["final_norm"],
                                        *[self.w[k] for k in _LAYER_KEYS], ctx_norm=self.w.get("ctx_norm"))
        self.handle = L.dflash_create(c, ws)
        self.ws_bytes = L.dflash_workspace_size(self.handle, max_batch, max_ctx, max_new)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=device)

    def close(self) -> None:
        if getattr(self, "handle", None):
            L.dflash_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- the four hot calls ------------------------------------------------
    def inject_context(self, feats: torch.Tensor, seq: torch.Tensor, pos: torch.Tensor, kv: PagedKV) -> None:
        L.dflash_inject_context(self.handle, feats, seq, pos, int(feats.shape[0]), kv.struct(), self.ws)

    def draft_block(self, anchor_ids: torch.Tensor, kv: PagedKV, hidden_out: Optional[torch.Tensor] = None):
        B = self.cfg.block_size
        if hidden_out is None:
            hidden_out = torch.empty((kv.batch * (B - 1), self.cfg.hidden), dtype=storage_dtype(self.cfg),
                                     device=self.device)
        L.dflash_draft_block(self.handle, anchor_ids, kv.struct(), hidden_out, self.ws)
        return hidden_out

    def target_verify(self, ids: torch.Tensor, kv: PagedKV, tap_layers=(), hidden_out=None, taps_out=None):
        """Causal pass of a target handle over ids [batch, B]; returns
        (hidden [batch*B, H], taps [batch*B, len(tap_layers)*H] or None)."""
        R = kv.batch * self.cfg.block_size
        if hidden_out is None:
            hidden_out = torch.empty((R, self.cfg.hidden), dtype=storage_dtype(self.cfg), device=self.device)
        if taps_out is None and len(tap_layers):
            taps_out = torch.empty((R, len(tap_layers) * self.cfg.hidden), dtype=storage_dtype(self.cfg),
                                   device=self.device)
        L.dflash_target_verify(self.handle, ids, kv.struct(), list(tap_layers), taps_out, hidden_out, self.ws)
        return hidden_out, taps_out

    def lmhead_argmax(self, hidden: torch.Tensor, want_max: bool = True, want_logits: bool = False):
        rows = int(hidden.shape[0])
        ids = torch.empty(rows, dtype=torch.int32, device=self.device)
        mx = torch.empty(rows, dtype=torch.float32, device=self.device) if want_max else None
        lg = torch.empty((rows, self.cfg.vocab), dtype=torch.float32, device=self.device) if want_logits else None
        L.dflash_lmhead_argmax(self.handle, hidden, rows, ids, mx, lg, self.ws)
        return ids, mx, lg

    def check_inputs(self, kv: "PagedKV", anchor_ids=None, ids=None, seq=None, pos=None) -> int:
        """Range check of the device-resident indices; returns the DFLASH_BAD_* bits."""
        err = torch.zeros(1, dtype=torch.int32, device=self.device)
        L.dflash_check_inputs(self.handle, kv.struct(), anchor_ids, ids, seq, pos, err)
        return int(err.cpu()[0])

    def lmhead_logits(self, hidden: torch.Tensor) -> torch.Tensor:
        """fp32 logits [rows, vocab] only (the input of temperature sampling)."""
        rows = int(hidden.shape[0])
        lg = torch.empty((rows, self.cfg.vocab), dtype=torch.float32, device=self.device)
        L.dflash_lmhead_argmax(self.handle, hidden, rows, None, None, lg, self.ws)
        return lg

    @staticmethod
    def sample(logits: torch.Tensor, temperature: float, seed: int, offset: int, tag: int, ws=None):
        """One draw per row from softmax(logits / T); returns (ids, lse)."""
        rows, vocab = int(logits.shape[0]), int(logits.shape[1])
        ids = torch.empty(rows, dtype=torch.int32, device=logits.device)
        lse = torch.empty(rows, dtype=torch.float32, device=logits.device)
        if ws is None:
            ws = torch.empty(max(1, L.dflash_sample_workspace_size(rows, vocab)), dtype=torch.uint8,
                             device=logits.device)
        L.dflash_sample(logits, rows, vocab, temperature, seed, offset, tag, ids, lse, ws)
        return ids, lse

    @staticmethod
    def accept_sample(draft_logits, draft_lse, draft_ids, target_logits, target_lse, target_ids, block_size: int,
                      temperature: float, seed: int, offset: int, block_len=None, ws=None):
        """Speculative-sampling accept / resample; returns (tau, bonus)."""
        b = int(draft_ids.shape[0])
        vocab = int(target_logits.shape[-1])
        tau = torch.empty(b, dtype=torch.int32, device=draft_ids.device)
        bonus = torch.empty(b, dtype=torch.int32, device=draft_ids.device)
        if ws is None:
            ws = torch.empty(max(1, L.dflash_sample_workspace_size(b, vocab)), dtype=torch.uint8,
                             device=draft_ids.device)
        L.dflash_accept_sample(draft_logits, draft_lse, draft_ids, target_logits, target_lse, target_ids, b,
                               block_size, block_len, vocab, temperature, seed, offset, tau, bonus, ws)
        return tau, bonus

    @staticmethod
    def accept_len_ragged(draft_ids: torch.Tensor, target_ids: torch.Tensor, block_size: int,
                          block_len: Optional[torch.Tensor]):
        b = int(draft_ids.shape[0])
        tau = torch.empty(b, dtype=torch.int32, device=draft_ids.device)
        bonus = torch.empty(b, dtype=torch.int32, device=draft_ids.device)
        L.dflash_accept_len_ragged(draft_ids, target_ids, b, block_size, block_len, tau, bonus)
        return tau, bonus

    @staticmethod
    def accept_len(draft_ids: torch.Tensor, target_ids: torch.Tensor, block_size: int):
        b = int(draft_ids.shape[0])
        tau = torch.empty(b, dtype=torch.int32, device=draft_ids.device)
        bonus = torch.empty(b, dtype=torch.int32, device=draft_ids.device)
        L.dflash_accept_len(draft_ids, target_ids, b, block_size, tau, bonus)
        return tau, bonus
