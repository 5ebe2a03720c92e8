"""ctypes binding of libdflash (argument marshalling only).

Every compute step runs in the HIP library; this module converts torch
tensors to device pointers and the current HIP stream, mirrors the C structs of
``include/dflash.h`` and turns status codes into exceptions.  It never computes
any part of the drafter step itself and has no fallback: if the library is not
built, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libdflash.so")

DFLASH_F32, DFLASH_BF16 = 0, 1

EXPORTS = ("dflash_create", "dflash_destroy", "dflash_workspace_size", "dflash_workspace_init",
           "dflash_inject_context", "dflash_draft_block", "dflash_target_verify", "dflash_lmhead_argmax",
           "dflash_lmhead_argmax_noalloc",
           "dflash_accept_len", "dflash_accept_len_ragged", "dflash_sample_workspace_size", "dflash_sample",
           "dflash_accept_sample", "dflash_check_inputs", "dflash_set_stage_events", "dflash_stream_read",
           "dflash_status_str")

# measurement hook stages (include/dflash.h)
STAGES = ("qkv", "attention", "o", "gate_up", "down")


class DflashError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


class DflashConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("n_feat_layers", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("mask_token_id", ctypes.c_int32), ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("window", ctypes.c_int32),
                ("ctx_norm", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class DflashWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("w_fc", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("attn_norm", _PP), ("w_qkv", _PP), ("w_o", _PP),
                ("mlp_norm", _PP), ("w_gate_up", _PP), ("w_down", _PP), ("ctx_norm", ctypes.c_void_p)]


class DflashKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("ctx_len", ctypes.c_void_p), ("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("n_pages", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("block_len", ctypes.c_void_p)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libdflash.so (built in-tree).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_diffusion_drafter_gemm_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.dflash_create.argtypes = [ctypes.POINTER(DflashConfig), ctypes.POINTER(DflashWeights), ctypes.POINTER(vp)]
    lib.dflash_destroy.argtypes = [vp]
    lib.dflash_workspace_size.argtypes = [vp, i32, i32, i32, ctypes.POINTER(sz)]
    lib.dflash_workspace_init.argtypes = [vp, vp, sz, vp]
    lib.dflash_inject_context.argtypes = [vp, vp, vp, vp, i32, ctypes.POINTER(DflashKV), vp, sz, vp]
    lib.dflash_draft_block.argtypes = [vp, vp, ctypes.POINTER(DflashKV), vp, vp, sz, vp]
    lib.dflash_target_verify.argtypes = [vp, vp, ctypes.POINTER(DflashKV), vp, i32, vp, vp, vp, sz, vp]
    lib.dflash_lmhead_argmax.argtypes = [vp, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.dflash_lmhead_argmax_noalloc.argtypes = [vp, vp, i32, vp, vp, vp]
    lib.dflash_accept_len.argtypes = [vp, vp, i32, i32, vp, vp, vp]
    lib.dflash_accept_len_ragged.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp]
    u32, u64, f32 = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float
    lib.dflash_sample_workspace_size.argtypes = [i32, i32, ctypes.POINTER(sz)]
    lib.dflash_sample.argtypes = [vp, i32, i32, f32, u64, u32, u32, vp, vp, vp, sz, vp]
    lib.dflash_accept_sample.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, i32, f32, u64, u32, vp, vp, vp, sz,
                                         vp]
    lib.dflash_check_inputs.argtypes = [vp, ctypes.POINTER(DflashKV), vp, vp, i32, vp, vp, i32, vp, vp]
    lib.dflash_set_stage_events.argtypes = [vp, ctypes.POINTER(vp), i32]
    lib.dflash_stream_read.argtypes = [vp, sz, vp, vp]
    lib.dflash_status_str.argtypes = [ctypes.c_int]
    lib.dflash_status_str.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name != "dflash_status_str":
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().dflash_status_str(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise DflashError(status, what)


def ptr(t) -> Optional[int]:
    """Device pointer of a torch tensor (None -> NULL)."""
    if t is None:
        return None
    return t.data_ptr()


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------
def dflash_create(cfg: DflashConfig, weights: DflashWeights) -> int:
    h = ctypes.c_void_p()
    _check(load().dflash_create(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(h)), "dflash_create")
    return h.value


def dflash_destroy(h: int) -> None:
    _check(load().dflash_destroy(h), "dflash_destroy")


def dflash_workspace_size(h: int, max_batch: int, max_ctx: int, max_new: int) -> int:
    n = ctypes.c_size_t()
    _check(load().dflash_workspace_size(h, max_batch, max_ctx, max_new, ctypes.byref(n)), "dflash_workspace_size")
    return n.value


def dflash_workspace_init(h: int, ws, stream: Optional[int] = None) -> None:
    _check(load().dflash_workspace_init(h, ptr(ws), ws.numel() * ws.element_size(),
                                        current_stream() if stream is None else stream), "dflash_workspace_init")


def dflash_inject_context(h: int, feats, seq, pos, n_new: int, kv: DflashKV, ws, stream: Optional[int] = None) -> None:
    _check(load().dflash_inject_context(h, ptr(feats), ptr(seq), ptr(pos), n_new, ctypes.byref(kv), ptr(ws),
                                        ws.numel() * ws.element_size(),
                                        current_stream() if stream is None else stream), "dflash_inject_context")


def dflash_draft_block(h: int, anchor_ids, kv: DflashKV, hidden_out, ws, stream: Optional[int] = None) -> None:
    _check(load().dflash_draft_block(h, ptr(anchor_ids), ctypes.byref(kv), ptr(hidden_out), ptr(ws),
                                     ws.numel() * ws.element_size(),
                                     current_stream() if stream is None else stream), "dflash_draft_block")


def dflash_target_verify(h: int, ids, kv: DflashKV, tap_layers: Sequence[int], taps_out, hidden_out, ws,
                         stream: Optional[int] = None) -> None:
    taps = (ctypes.c_int32 * max(1, len(tap_layers)))(*tap_layers)
    _check(load().dflash_target_verify(h, ptr(ids), ctypes.byref(kv), ctypes.cast(taps, ctypes.c_void_p),
                                       len(tap_layers), ptr(taps_out), ptr(hidden_out), ptr(ws),
                                       ws.numel() * ws.element_size(),
                                       current_stream() if stream is None else stream), "dflash_target_verify")


def dflash_lmhead_argmax(h: int, hidden, rows: int, ids_out, max_logit_out, logits_out, ws,
                         stream: Optional[int] = None) -> None:
    _check(load().dflash_lmhead_argmax(h, ptr(hidden), rows, ptr(ids_out), ptr(max_logit_out), ptr(logits_out),
                                       ptr(ws), ws.numel() * ws.element_size(),
                                       current_stream() if stream is None else stream), "dflash_lmhead_argmax")


def dflash_lmhead_argmax_noalloc(h: int, hidden, rows: int, ids_out, max_logit_out,
                                 stream: Optional[int] = None) -> None:
    _check(load().dflash_lmhead_argmax_noalloc(h, ptr(hidden), rows, ptr(ids_out), ptr(max_logit_out),
                                               current_stream() if stream is None else stream),
           "dflash_lmhead_argmax_noalloc")


def dflash_accept_len(draft_ids, target_ids, batch: int, block_size: int, accept_len_out, bonus_out,
                      stream: Optional[int] = None) -> None:
    _check(load().dflash_accept_len(ptr(draft_ids), ptr(target_ids), batch, block_size, ptr(accept_len_out),
                                    ptr(bonus_out), current_stream() if stream is None else stream),
           "dflash_accept_len")


def dflash_accept_len_ragged(draft_ids, target_ids, batch: int, block_size: int, block_len, accept_len_out,
                             bonus_out, stream: Optional[int] = None) -> None:
    _check(load().dflash_accept_len_ragged(ptr(draft_ids), ptr(target_ids), batch, block_size, ptr(block_len),
                                           ptr(accept_len_out), ptr(bonus_out),
                                           current_stream() if stream is None else stream),
           "dflash_accept_len_ragged")


def dflash_check_inputs(h: int, kv, anchor_ids, ids, seq, pos, err_out, stream: Optional[int] = None) -> None:
    _check(load().dflash_check_inputs(h, ctypes.byref(kv), ptr(anchor_ids), ptr(ids),
                                      0 if ids is None else ids.numel(), ptr(seq), ptr(pos),
                                      0 if seq is None else seq.numel(), ptr(err_out),
                                      current_stream() if stream is None else stream), "dflash_check_inputs")


def dflash_sample_workspace_size(rows: int, vocab: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().dflash_sample_workspace_size(rows, vocab, ctypes.byref(n)), "dflash_sample_workspace_size")
    return n.value


def dflash_sample(logits, rows: int, vocab: int, temperature: float, seed: int, offset: int, tag: int, ids_out,
                  lse_out, ws, stream: Optional[int] = None) -> None:
    _check(load().dflash_sample(ptr(logits), rows, vocab, temperature, seed, offset, tag, ptr(ids_out),
                                ptr(lse_out), ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                current_stream() if stream is None else stream), "dflash_sample")


def dflash_accept_sample(draft_logits, draft_lse, draft_ids, target_logits, target_lse, target_ids, batch: int,
                         block_size: int, block_len, vocab: int, temperature: float, seed: int, offset: int,
                         accept_len_out, bonus_out, ws, stream: Optional[int] = None) -> None:
    _check(load().dflash_accept_sample(ptr(draft_logits), ptr(draft_lse), ptr(draft_ids), ptr(target_logits),
                                       ptr(target_lse), ptr(target_ids), batch, block_size, ptr(block_len), vocab,
                                       temperature, seed, offset, ptr(accept_len_out), ptr(bonus_out), ptr(ws),
                                       0 if ws is None else ws.numel() * ws.element_size(),
                                       current_stream() if stream is None else stream), "dflash_accept_sample")


# ----------------------------------------------------------------------------
# struct helpers
# ----------------------------------------------------------------------------
def make_config(hidden: int, n_q_heads: int, n_kv_heads: int, head_dim: int, ffn: int, vocab: int, n_layers: int,
                n_feat_layers: int, block_size: int, mask_token_id: int, dtype: str, rope_theta: float,
                rms_eps: float, page_size: int = 16, window: int = 0, ctx_norm: int = 0) -> DflashConfig:
    return DflashConfig(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, n_layers, n_feat_layers, block_size,
                        mask_token_id, page_size, DFLASH_BF16 if dtype == "bf16" else DFLASH_F32,
                        float(rope_theta), float(rms_eps), int(window), int(ctx_norm))


def make_weights(embed, lm_head, w_fc, final_norm, attn_norm: Sequence, w_qkv: Sequence, w_o: Sequence,
                 mlp_norm: Sequence, w_gate_up: Sequence, w_down: Sequence, ctx_norm=None):
    """Returns (DflashWeights, keepalive) - keep the second object alive while the struct is used."""
    arrays = []

    def arr(ts):
        a = (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
        arrays.append(a)
        return ctypes.cast(a, _PP)

    w = DflashWeights(embed.data_ptr(), lm_head.data_ptr(), None if w_fc is None else w_fc.data_ptr(),
                      final_norm.data_ptr(),
                      arr(attn_norm), arr(w_qkv), arr(w_o), arr(mlp_norm), arr(w_gate_up), arr(w_down),
                      ptr(ctx_norm))
    return w, arrays


def make_kv(k, v, block_table, ctx_len, batch: int, max_pages: int, n_pages: int, max_ctx: int,
            block_len=None) -> DflashKV:
    return DflashKV(k.data_ptr(), v.data_ptr(), block_table.data_ptr(), ctx_len.data_ptr(), batch, max_pages,
                    n_pages, max_ctx, ptr(block_len))


def dflash_set_stage_events(h: int, events: Optional[Sequence[int]]) -> None:
    """Turn the per-stage event hook on (a list of 2 * len(STAGES) * n_layers
    raw hipEvent_t handles) or off (None)."""
    if events is None:
        _check(load().dflash_set_stage_events(h, None, 0), "dflash_set_stage_events")
        return
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(load().dflash_set_stage_events(h, arr, len(events)), "dflash_set_stage_events")


def dflash_stream_read(src, sink, stream: Optional[int] = None) -> None:
    """Streaming read of the whole of ``src`` (device tensor), XOR-folded into
    ``sink`` (one int32 on the device, zeroed by the caller)."""
    _check(load().dflash_stream_read(ptr(src), src.numel() * src.element_size(), ptr(sink),
                                     current_stream() if stream is None else stream), "dflash_stream_read")
