#!/usr/bin/env python3
"""Benchmark of the DFlash drafter step on one MI355X.

One step = dflash_draft_block + dflash_lmhead_argmax + dflash_accept_len over
one batch of synthetic input (the Qwen3-8B-shaped drafter at batch 1, context
2048, B = 16 by default), with weights, context cache and ids resident in HBM
before the timed region.  Prints one JSON line: drafted tokens/s as ``value``,
the step latency, the HBM fraction of the step, per-stage kernel times (HIP
events recorded by the library around each stage of every layer, on the launch
stream, during the eager timed steps), the roofline of the stage with the
largest share of the step, and the CPU oracle timed on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E
MFMA_PEAK_FLOPS = 2.5e15  # MI355X dense bf16 matrix-core peak
METRIC = "draft-block latency (µs) + drafted tokens/s, Qwen3-8B-shape B=16; % HBM peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="qwen3_8b")
    ap.add_argument("--block-size", type=int, default=0,
                    help="> 0: replace the configuration's block size B (drafting cost against B)")
    ap.add_argument("--no-graph", action="store_true", help="report eager launches only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--inject", action="store_true", help="also time steady-state inject (B positions)")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="> 0: draws drafts at this temperature (logits-only LM head + dflash_sample) and "
                         "verifies with dflash_accept_sample against synthetic target logits")
    ap.add_argument("--e2e", type=int, default=0, metavar="LAYERS",
                    help="also time the target side of the cycle with a LAYERS-layer target of the drafter's "
                         "layer shape (random weights, shared embedding and LM head): block verify, one-token "
                         "decode, and the speculative cycle")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy (reference for HBM byte counters)")
    return ap.parse_args()


def step_bytes(cfg, lens):
    """Algorithmic HBM bytes of one draft step: every weight matrix once, the
    valid context K/V once, the embedding rows read; activations excluded."""
    e = 2 if cfg.dtype == "bf16" else 4
    H, F, nq, nkv, d = cfg.hidden, cfg.ffn, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    layer = (cfg.qkv_rows * H + H * nq * d + 2 * F * H + H * F + 2 * H) * e
    lm = cfg.vocab * H * e
    kv = cfg.n_layers * int(sum(lens)) * nkv * d * 2 * e
    emb = 2 * H * e + H * e
    return cfg.n_layers * layer, lm, kv, emb


def step_flops(cfg, lens):
    H, F, nq, nkv, d, B = cfg.hidden, cfg.ffn, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block_size
    R = cfg.batch * B
    gemm = 2 * R * (cfg.qkv_rows * H + H * nq * d + 2 * F * H + H * F) * cfg.n_layers
    lm = 2 * cfg.batch * (B - 1) * cfg.vocab * H
    attn = sum(4 * B * nq * d * (int(p) + B) for p in lens) * cfg.n_layers
    return gemm, lm, attn


# counter summaries of the batch-1 Qwen3-8B-shape step: HBM bytes per launch of
# each kernel, valid while the kernel sources hash to the recorded value
PROFILE = os.path.join(ROOT, "profiles", "draft_step_qwen3_8b_b1.md")
KERNEL_SOURCES = ["block_diffusion_drafter_gemm_amd/csrc/gemm_stream.hip",
                  "block_diffusion_drafter_gemm_amd/csrc/attention.hip",
                  "block_diffusion_drafter_gemm_amd/csrc/dflash_device.h",
                  "block_diffusion_drafter_gemm_amd/csrc/dflash_internal.h"]


def read_stream_gbs(torch, nbytes=1 << 30, reps=10):
    """Read bandwidth of the library's plain streaming-read kernel over 1 GiB on
    this GPU, the practical ceiling of an HBM-bound step."""
    from block_diffusion_drafter_gemm_amd import _lib as L
    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        L.dflash_stream_read(x, sink)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        L.dflash_stream_read(x, sink)
    b.record()
    torch.cuda.synchronize()
    gbs = nbytes * reps / (a.elapsed_time(b) / 1e3) / 1e9
    del x
    return gbs


def recorded_traffic(stage: str):
    """HBM bytes (read + written) per launch of a stage's kernel from the
    committed counter summary, or None when the kernel sources changed since the
    counters were taken."""
    import hashlib
    import re
    try:
        text = open(PROFILE).read()
        h = hashlib.sha256()
        for src in KERNEL_SOURCES:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        sha = re.search(r"kernel_source_sha256_16: (\w+)", text).group(1)
        if sha != h.hexdigest()[:16]:
            return None
        return int(re.search(rf"traffic_bytes_per_launch\[{stage}\]: (\d+)", text).group(1))
    except (OSError, AttributeError):
        return None


class FenceFreeEvents:
    """HIP timing events created with hipEventDisableSystemFence: recording one
    adds no system-scope cache writeback and invalidate to the stream (torch's
    events do), so a pair brackets a stage the way the kernel trace times it.
    Made through the HIP runtime that torch and the library share in this
    process."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                parts = line.split()
                if len(parts) >= 6 and os.path.basename(parts[-1]).startswith("libamdhip64.so"):
                    path = parts[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime library is not loaded")
        rt = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        rt.hipEventRecord.argtypes = [vp, vp]
        rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        rt.hipEventDestroy.argtypes = [vp]
        self.ctypes, self.rt, self.ev = ctypes, rt, []
        for _ in range(n):
            e = vp()
            self._check(rt.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE), "create")
            self.ev.append(e.value)

    @staticmethod
    def _check(err, what):
        if err != 0:
            raise RuntimeError(f"hipEvent {what} failed: error {err}")

    def record(self, i: int, stream: int) -> None:
        self._check(self.rt.hipEventRecord(self.ev[i], stream), "record")

    def ms(self, i: int, j: int) -> float:
        f = self.ctypes.c_float()
        self._check(self.rt.hipEventElapsedTime(self.ctypes.byref(f), self.ev[i], self.ev[j]), "elapsed")
        return f.value

    def close(self) -> None:
        for e in self.ev:
            self.rt.hipEventDestroy(e)
        self.ev = []


def stage_costs(cfg, lens):
    """Algorithmic bytes and flops of one launch of each stage (one layer; the
    LM head over all mask rows): weights once, valid context K/V once."""
    e = 2 if cfg.dtype == "bf16" else 4
    H, F, nq, nkv, d, B = cfg.hidden, cfg.ffn, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block_size
    R = cfg.batch * B
    ctx = int(sum(lens))
    return {
        "qkv": (cfg.qkv_rows * H * e + H * e, 2 * R * cfg.qkv_rows * H),
        "attention": (ctx * nkv * d * 2 * e, sum(4 * B * nq * d * (int(p) + B) for p in lens)),
        "o": (H * nq * d * e, 2 * R * H * nq * d),
        "gate_up": (2 * F * H * e + H * e, 2 * R * 2 * F * H),
        "down": (H * F * e, 2 * R * H * F),
        "lm_head": (cfg.vocab * H * e, 2 * cfg.batch * (B - 1) * cfg.vocab * H),
    }


def roofline_of(name, nbytes, flops, us):
    """Roofline entry of one launch: MFMA-bound above the ridge (peak flops /
    peak bandwidth, ~312 flop per byte), HBM-bound below it."""
    if flops > nbytes * MFMA_PEAK_FLOPS / (HBM_PEAK_GBS * 1e9):
        a = flops / (us / 1e6)
        return {"kernel": name, "bound": "mfma", "achieved": round(a / 1e12, 1), "peak": MFMA_PEAK_FLOPS / 1e12,
                "unit": "TFLOP/s", "frac": round(a / MFMA_PEAK_FLOPS, 4), "flops_per_launch": int(flops),
                "bytes_per_launch": int(nbytes), "avg_launch_us": round(us, 2)}
    a = nbytes / (us / 1e6) / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4), "bytes_per_launch": int(nbytes), "flops_per_launch": int(flops),
            "avg_launch_us": round(us, 2)}


def host_threads():
    """Threads the CPU oracle may use: this process's cores, capped by
    OMP_NUM_THREADS when the environment sets it (the share of a shared host)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(1, n)


def cpu_baseline(cfg, w, Kp, Vp, lay, lens, anchors, y, min_seconds=10.0, max_steps=20):
    """The float64 oracle on the host cores: full draft steps of sequence 0 (draft
    block, LM-head argmax, accept length), repeated until at least min_seconds of
    work (at most max_steps steps)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import drafter as D
    from oracle.numerics import from_storage
    cores = host_threads()
    t = np.arange(int(lens[0]))
    pages, slots = lay.block_table[0, t // cfg.page_size], t % cfg.page_size
    Kc, Vc = from_storage(Kp[:, pages, slots]), from_storage(Vp[:, pages, slots])
    with threadpool_limits(limits=cores):
        used = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
        t0 = time.perf_counter()
        steps = 0
        while steps < max_steps and (steps == 0 or time.perf_counter() - t0 < min_seconds):
            Z = D.draft_block(w, cfg, int(anchors[0]), Kc, Vc)
            ids, _, _ = D.lm_argmax(w["lm_head"], Z)
            D.accept_len(ids, y[0])
            steps += 1
        dt = time.perf_counter() - t0
    # one more step on a single host thread
    with threadpool_limits(limits=1):
        t1 = time.perf_counter()
        Z = D.draft_block(w, cfg, int(anchors[0]), Kc, Vc)
        D.lm_argmax(w["lm_head"], Z)
        d1 = time.perf_counter() - t1
    single = {"value": round((cfg.block_size - 1) / d1, 3), "seconds": round(d1, 2)}
    return {"value": round(steps * (cfg.block_size - 1) / dt, 3), "unit": "drafted tokens/s",
            "cores": int(used), "host_cpu_count": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "kind": "oracle", "seconds": round(dt, 2), "single_thread": single,
            "sample": f"{steps} draft steps of sequence 0 ({cfg.block_size - 1} drafted tokens each, context "
                      f"{int(lens[0])}) in float64 numpy"}


def e2e_cycle(args, cfg, R, dr, lens, b, B, draft_step_ms, inject_ms):
    """Target side of the speculative cycle on this GPU: a target decoder of the
    drafter's layer shape with ``args.e2e`` layers (weights N(0, 0.02^2) drawn on
    the device; embedding and LM head shared with the drafter), its paged cache
    filled to the same context lengths, feature taps at 5 uniformly spaced
    layers.  Times one block verify (B rows + LM head argmax over B rows), one
    plain decode step (a 2-row block, the second row hidden by the causal mask)
    and the cycle (draft step + verify + inject of B positions); the speedup
    over plain decoding follows for a mean acceptance length tau as
    tau * decode / cycle."""
    import dataclasses
    import numpy as np
    import torch

    import dflash_synth as S
    nL = args.e2e
    gen = torch.Generator(device="cuda").manual_seed(1234)

    def normal(shape):
        return (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * 0.02).to(
            torch.bfloat16).view(torch.int16)

    H, F, d = cfg.hidden, cfg.ffn, cfg.head_dim
    qkv = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * d
    ones = torch.ones(H, dtype=torch.bfloat16, device="cuda").view(torch.int16)
    tw = {"embed": dr.w["embed"], "lm_head": dr.w["lm_head"], "final_norm": ones,
          "attn_norm": [ones] * nL, "mlp_norm": [ones] * nL,
          "w_qkv": [normal((qkv, H)) for _ in range(nL)], "w_o": [normal((H, cfg.n_q_heads * d)) for _ in range(nL)],
          "w_gate_up": [normal((2 * F, H)) for _ in range(nL)], "w_down": [normal((H, F)) for _ in range(nL)]}
    taps = [int(round(i * (nL - 1) / 4)) for i in range(5)]
    max_ctx = int(lens.max())
    tv = {Bt: R.Drafter(dataclasses.replace(cfg, n_layers=nL, block_size=Bt), tw, max_batch=b, max_ctx=max_ctx,
                        max_new=1) for Bt in (B, 2)}
    tcfg = dataclasses.replace(cfg, n_layers=nL, block_size=B)
    lay = S.paged_layout(tcfg, lens, headroom=B, seed=3)
    shape = (nL, lay.n_pages, cfg.page_size, cfg.n_kv_heads, d)
    sig = S.kv_sigma(cfg)
    kc = (torch.randn(shape, generator=gen, device="cuda") * sig).to(torch.bfloat16).view(torch.int16)
    vc = (torch.randn(shape, generator=gen, device="cuda") * sig).to(torch.bfloat16).view(torch.int16)
    tkv = R.PagedKV(tcfg, lay.block_table, lens, lay.n_pages)
    tkv.k, tkv.v = kc, vc
    out = {}
    temp, L, V = args.temperature, R.L, cfg.vocab
    if temp > 0:
        # at temperature > 0 the verify also writes the target's logits, draws
        # its rows and runs the accept / resample rule against drafter logits
        # (a synthetic stand-in, drawn once); a decode step draws its token
        dz = torch.randn((b * (B - 1), V), generator=gen, device="cuda")
        sws = torch.empty(L.dflash_sample_workspace_size(b * B, V), dtype=torch.uint8, device="cuda")
        dids, dlse = R.Drafter.sample(dz, temp, 7, 0, 0, ws=sws)
        tau = torch.empty(b, dtype=torch.int32, device="cuda")
        bonus = torch.empty(b, dtype=torch.int32, device="cuda")
    for Bt, name in ((B, "verify"), (2, "decode")):
        h = tv[Bt]
        ids = torch.randint(0, cfg.vocab, (b, Bt), generator=gen, device="cuda", dtype=torch.int32)
        hid = torch.empty((b * Bt, H), dtype=torch.int16, device="cuda")
        tp = torch.empty((b * Bt, len(taps) * H), dtype=torch.int16, device="cuda")
        if temp > 0:
            lg = torch.empty((b * Bt, V), dtype=torch.float32, device="cuda")
            tids = torch.empty(b * Bt, dtype=torch.int32, device="cuda")
            tlse = torch.empty(b * Bt, dtype=torch.float32, device="cuda")

        def once():
            h.target_verify(ids, tkv, taps, hidden_out=hid, taps_out=tp)
            if temp <= 0:
                h.lmhead_argmax(hid, want_max=False)
                return
            L.dflash_lmhead_argmax(h.handle, hid, b * Bt, None, None, lg, h.ws)
            L.dflash_sample(lg, b * Bt, V, temp, 7, 0, 1, tids, tlse, sws)
            if Bt == B:
                L.dflash_accept_sample(dz, dlse, dids, lg, tlse, tids, b, B, None, V, temp, 7, 0, tau, bonus, sws)
        for _ in range(3):
            once()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            once()
        e1.record()
        torch.cuda.synchronize()
        out[f"target_{name}_ms"] = round(e0.elapsed_time(e1) / args.steps, 4)
    for h in tv.values():
        h.close()
    weight_bytes = nL * (qkv * H + H * cfg.n_q_heads * d + 3 * F * H) * 2 + cfg.vocab * H * 2
    cycle = draft_step_ms + out["target_verify_ms"] + (inject_ms or 0.0)
    a = 0.7   # the synthetic per-position agreement of the verify targets
    tau_syn = (1 - a ** B) / (1 - a)
    out.update({
        "target": f"{nL} layers of the drafter's shape, hidden {H}, vocab {cfg.vocab}, taps {taps}",
        "temperature": temp,
        "target_weight_bytes": int(weight_bytes),
        "target_verify_hbm_gbs": round(weight_bytes / (out["target_verify_ms"] / 1e3) / 1e9, 1),
        "cycle_ms": round(cycle, 4), "inject_in_cycle": inject_ms is not None,
        "speedup_at_tau": {f"{tau_syn:.2f} (70% agreement, B={B})": round(tau_syn * out["target_decode_ms"] / cycle, 2),
                           "6.49 (the pages' mean at B=16, context only)":
                               round(6.49 * out["target_decode_ms"] / cycle, 2)},
    })
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the drafter step is measured per GPU",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import dflash_synth as S
    from block_diffusion_drafter_gemm_amd import _lib as L
    from block_diffusion_drafter_gemm_amd import runtime as R

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 3}), flush=True)
        return
    cfg = S.get_config(args.config, **({"block_size": args.block_size} if args.block_size > 0 else {}))
    b, B = cfg.batch, cfg.block_size
    w = S.drafter_weights(cfg, seed=0)
    lens = S.ctx_lens(cfg, seed=0)
    lay = S.paged_layout(cfg, lens, headroom=B, seed=0)
    Kp, Vp = S.ctx_kv_cache(cfg, lay, seed=0)
    anchors = S.anchor_ids(cfg, seed=0)
    dr = R.Drafter(cfg, w, max_batch=b, max_ctx=int(lens.max()), max_new=B)
    kv = R.PagedKV(cfg, lay.block_table, lens, lay.n_pages, k=Kp, v=Vp)
    kvs = kv.struct()
    st = torch.cuda.current_stream().cuda_stream
    anc = torch.from_numpy(anchors).cuda()
    hid = torch.empty((b * (B - 1), cfg.hidden), dtype=R.storage_dtype(cfg), device="cuda")
    ids = torch.empty(b * (B - 1), dtype=torch.int32, device="cuda")
    tau = torch.empty(b, dtype=torch.int32, device="cuda")
    bonus = torch.empty(b, dtype=torch.int32, device="cuda")
    lib, ws, wsb, h = L.load(), dr.ws, dr.ws_bytes, dr.handle
    rows = b * (B - 1)

    def draft():
        assert lib.dflash_draft_block(h, anc.data_ptr(), kvs, hid.data_ptr(), ws.data_ptr(), wsb, st) == 0

    def lmhead():
        assert lib.dflash_lmhead_argmax(h, hid.data_ptr(), rows, ids.data_ptr(), None, None, ws.data_ptr(), wsb,
                                        st) == 0

    def accept():
        assert lib.dflash_accept_len(ids.data_ptr(), y_dev.data_ptr(), b, B, tau.data_ptr(), bonus.data_ptr(),
                                     st) == 0

    temp = args.temperature
    if temp > 0:
        # drafts drawn from softmax(logits / T); the verifier's logits are a
        # synthetic stand-in (the drafter's logits plus noise), their draws and
        # lse taken once outside the timed region
        dz = torch.empty((rows, cfg.vocab), dtype=torch.float32, device="cuda")
        dlse = torch.empty(rows, dtype=torch.float32, device="cuda")
        sws = torch.empty(L.dflash_sample_workspace_size(max(rows, b * B), cfg.vocab), dtype=torch.uint8,
                          device="cuda")
        seed = 2024

        def lmhead():
            assert lib.dflash_lmhead_argmax(h, hid.data_ptr(), rows, None, None, dz.data_ptr(), ws.data_ptr(), wsb,
                                            st) == 0
            assert lib.dflash_sample(dz.data_ptr(), rows, cfg.vocab, temp, seed, 0, 0, ids.data_ptr(),
                                     dlse.data_ptr(), sws.data_ptr(), sws.numel(), st) == 0

        def accept():
            assert lib.dflash_accept_sample(dz.data_ptr(), dlse.data_ptr(), ids.data_ptr(), tz.data_ptr(),
                                            tlse.data_ptr(), tids.data_ptr(), b, B, None, cfg.vocab, temp, seed, 0,
                                            tau.data_ptr(), bonus.data_ptr(), sws.data_ptr(), sws.numel(), st) == 0

    # synthetic target ids (70% agreement) from the first step's drafts
    draft()
    lmhead()
    torch.cuda.synchronize()
    d0 = ids.cpu().numpy().reshape(b, B - 1)
    y = S.target_ids_for(cfg, d0, seed=0)
    y_dev = torch.from_numpy(y).cuda()
    if temp > 0:
        tz = torch.empty((b, B, cfg.vocab), dtype=torch.float32, device="cuda")
        tz[:, :B - 1] = dz.view(b, B - 1, -1)
        tz[:, B - 1] = dz.view(b, B - 1, -1)[:, -1]
        tz = (tz + 0.5 * torch.randn(tz.shape, generator=torch.Generator("cuda").manual_seed(0), device="cuda"))
        tz = tz.view(b * B, -1).contiguous()
        tids, tlse = R.Drafter.sample(tz, temp, seed, 0, 1)
        torch.cuda.synchronize()

    def step():
        draft()
        lmhead()
        accept()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # eager timed region: events on the launch stream bracket the draft pass and
    # the LM head, and the library records a pair around each stage of every
    # layer (dflash_set_stage_events) on the same stream.  Event i of step k is
    # E.ev[2 + k * per + i]: 0, 1, 2 around the draft pass and the LM head, then
    # the stage pairs; E.ev[0], E.ev[1] bracket all K steps.
    K = args.steps
    n_ev = 2 * len(L.STAGES) * cfg.n_layers
    per = 3 + n_ev
    E = FenceFreeEvents(2 + K * per)
    ev = lambda k, i: 2 + k * per + i
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    # hold the stream with a spin kernel while the host enqueues the K steps, so
    # the GPU runs them back to back: launched one by one, an eager step takes
    # longer to enqueue than to run, and the gaps would count as stage time
    torch.cuda._sleep(int(K * 3e-3 * 2.1e9))
    E.record(0, stream)
    for i in range(K):
        L.dflash_set_stage_events(h, E.ev[ev(i, 3):ev(i, per)])
        E.record(ev(i, 0), stream)
        draft()
        E.record(ev(i, 1), stream)
        lmhead()
        E.record(ev(i, 2), stream)
        accept()
    E.record(1, stream)
    torch.cuda.synchronize()
    L.dflash_set_stage_events(h, None)
    eager_ms = E.ms(0, 1) / K
    draft_ms = np.array([E.ms(ev(i, 0), ev(i, 1)) for i in range(K)])
    lm_ms = np.array([E.ms(ev(i, 1), ev(i, 2)) for i in range(K)])
    # stage_us[name]: every launch's duration in microseconds (K steps x layers)
    stage_us = {name: np.array([E.ms(ev(i, 3 + 2 * (l * len(L.STAGES) + j)), ev(i, 4 + 2 * (l * len(L.STAGES) + j)))
                                * 1e3 for i in range(K) for l in range(cfg.n_layers)])
                for j, name in enumerate(L.STAGES)}
    stage_us["lm_head"] = lm_ms * 1e3
    E.close()
    assert np.array_equal(ids.cpu().numpy().reshape(b, B - 1), d0), "drafts changed between steps"

    graph_ms = None
    graph_step_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            step()
        torch.cuda.current_stream().wait_stream(s2)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            st_cap = torch.cuda.current_stream().cuda_stream
            st_saved, st = st, st_cap
            step()
            st = st_saved
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        ids.zero_()
        # event i brackets replay i - 1 and i (fence-free events, as above)
        GE = FenceFreeEvents(K + 1)
        GE.record(0, stream)
        for i in range(K):
            g.replay()
            GE.record(i + 1, stream)
        torch.cuda.synchronize()
        graph_ms = GE.ms(0, K) / K
        graph_step_ms = np.array([GE.ms(i, i + 1) for i in range(K)])
        GE.close()
        assert np.array_equal(ids.cpu().numpy().reshape(b, B - 1), d0), "graph replay drafts differ from eager"

    ms = graph_ms if graph_ms is not None else eager_ms
    per_step = graph_step_ms if graph_step_ms is not None else draft_ms + lm_ms
    pct = {"median_ms": round(float(np.median(per_step)), 4), "p10_ms": round(float(np.percentile(per_step, 10)), 4),
           "p90_ms": round(float(np.percentile(per_step, 90)), 4)}
    stream_gbs = read_stream_gbs(torch)
    layers_b, lm_b, kv_b, emb_b = step_bytes(cfg, lens)
    total_b = layers_b + lm_b + kv_b + emb_b
    gemm_f, lm_f, attn_f = step_flops(cfg, lens)
    # per-stage figures; the roofline entry is the stage with the largest share
    # of the step (its launches per step x average launch time)
    costs = stage_costs(cfg, lens)
    if temp > 0:   # logits written and read back by the draw
        nb, nf = costs["lm_head"]
        costs["lm_head"] = (nb + 2 * b * (B - 1) * cfg.vocab * 4, nf)
    stage_step_us = {k: (1 if k == "lm_head" else cfg.n_layers) * float(np.mean(v)) for k, v in stage_us.items()}
    stages = {}
    for k, v in stage_us.items():
        stages[k] = roofline_of(k, *costs[k], float(np.mean(v)))
        stages[k].pop("kernel")
        stages[k]["us_per_step"] = round(stage_step_us[k], 2)
        stages[k]["share_of_step"] = round(stage_step_us[k] / (float(np.mean(draft_ms + lm_ms)) * 1e3), 4)
    dom = max(stage_step_us, key=stage_step_us.get)
    names = {"qkv": "attention RMSNorm + QKV projection + RoPE (one layer)",
             "attention": "block attention over context + block (one layer)",
             "o": "O projection + residual (one layer)",
             "gate_up": "MLP RMSNorm + gate/up projection + SwiGLU (one layer)",
             "down": "down projection + residual (one layer)",
             "lm_head": ("lmhead_argmax (vocabulary GEMM with argmax epilogue + argmax reduce)" if temp <= 0
                         else "lmhead logits (vocabulary GEMM, fp32 store) + dflash_sample")}
    roof = roofline_of(names[dom], *costs[dom], float(np.mean(stage_us[dom])))
    default_shape = args.config == "qwen3_8b" and temp <= 0 and args.block_size in (0, 16)
    roof["traffic"] = recorded_traffic(dom) if default_shape else None
    roof["launches_per_step"] = 1 if dom == "lm_head" else cfg.n_layers
    roof["share_of_step"] = stages[dom]["share_of_step"]
    out = {
        "metric": METRIC,
        "value": round(b * (B - 1) / (ms / 1e3), 1),
        "unit": "drafted tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "latency_us": round(ms * 1e3, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,0.02) weights, N(0,sigma) context K/V, uniform anchor ids)",
        "config": {"workload": f"{cfg.name} drafter step: batch {b}, context {int(lens.max())}, B={B}, "
                               f"{cfg.n_layers} layers, hidden {cfg.hidden}, vocab {cfg.vocab}",
                   "batch": b, "block_size": B, "ctx_len": int(lens.max()), "temperature": temp,
                   "launch": "hipgraph" if graph_ms is not None else "eager"},
        "step": {"eager_ms": round(eager_ms, 4), "graph_ms": None if graph_ms is None else round(graph_ms, 4),
                 "draft_block_ms": round(float(np.mean(draft_ms)), 4),
                 "lmhead_ms": round(float(np.mean(lm_ms)), 4),
                 "algorithmic_bytes": int(total_b), "algorithmic_flops": int(gemm_f + lm_f + attn_f),
                 **pct,
                 "hbm_gbs": round(total_b / (ms / 1e3) / 1e9, 1),
                 "hbm_frac": round(total_b / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                 "read_stream_gbs": round(stream_gbs, 1),
                 "hbm_frac_of_read_stream": round(total_b / (ms / 1e3) / 1e9 / stream_gbs, 4),
                 "mfma_frac_step": round((gemm_f + lm_f) / (ms / 1e3) / MFMA_PEAK_FLOPS, 4)},
        "roofline": roof,
        "stages": stages,
    }
    if args.inject:
        fe = R.to_device(S.features(cfg, B * b, seed=1))
        sq = torch.arange(b, dtype=torch.int32, device="cuda").repeat_interleave(B)
        ps = (torch.from_numpy(lens).cuda().repeat_interleave(B) +
              torch.arange(B, dtype=torch.int32, device="cuda").repeat(b)).to(torch.int32)
        for _ in range(3):
            dr.inject_context(fe, sq, ps, kv)
        i0, i1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        i0.record()
        for _ in range(K):
            dr.inject_context(fe, sq, ps, kv)
        i1.record()
        torch.cuda.synchronize()
        out["inject_steady_ms"] = round(i0.elapsed_time(i1) / K, 4)
        out["cycle_ms"] = round(ms + out["inject_steady_ms"], 4)
        # prefill injection: every context position of the first sequence at once
        T = int(lens[0])
        fp = R.to_device(S.features(cfg, T, seed=2))
        sp = torch.zeros(T, dtype=torch.int32, device="cuda")
        pp = torch.arange(T, dtype=torch.int32, device="cuda")
        drp = R.Drafter(cfg, w, max_batch=b, max_ctx=int(lens.max()), max_new=T)
        drp.inject_context(fp, sp, pp, kv)
        torch.cuda.synchronize()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record()
        for _ in range(3):
            drp.inject_context(fp, sp, pp, kv)
        p1.record()
        torch.cuda.synchronize()
        out["inject_prefill_ms"] = round(p0.elapsed_time(p1) / 3, 4)
        out["inject_prefill_positions"] = T
        # fusion projection (L*H -> H) and every layer's K and V projection per position
        inj_f = 2.0 * T * cfg.hidden * (cfg.feat_dim + cfg.n_layers * 2 * cfg.n_kv_heads * cfg.head_dim)
        out["inject_prefill_tflops"] = round(inj_f / (out["inject_prefill_ms"] / 1e3) / 1e12, 1)
        out["inject_prefill_mfma_frac"] = round(inj_f / (out["inject_prefill_ms"] / 1e3) / MFMA_PEAK_FLOPS, 4)
        drp.close()
    if args.e2e > 0:
        out["e2e"] = e2e_cycle(args, cfg, R, dr, lens, b, B, ms, out.get("inject_steady_ms"))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, w, Kp, Vp, lay, lens, anchors, y)
    dr.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
