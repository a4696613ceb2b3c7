"""Benchmark of the fused decode layer step (dl_layer_step) on one MI355X.

One step = one pass of the whole hot path (indexer + top-k, sparse attention, W_UV/W_O, router, expert FFN)
over one batch of seeded synthetic inputs resident in HBM.  The default workload is batch 8 at 128K context
(hidden 6144, 64 heads over a 576-wide FP8 latent, top-2,048, 256 experts top-8 + 1 shared, FP8 weights).

To keep the 256 MB last-level cache from serving repeats, the timed steps rotate over --instances distinct
layer instances (separate weights, caches and inputs; ~10.5 GB each).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_attention_moe_amd as dl  # noqa: E402
import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC_BASE = "decode layer-steps/s + achieved HBM GB/s (% of peak)"


def metric_label(spec) -> str:
    """The metric named for the workload actually run (the headline one is batch 8 @ 128K ctx)."""
    lens = [int(l) for l in spec.seq_lens]

    def ctx(n):
        return f"{n >> 20}M" if n % (1 << 20) == 0 else f"{n >> 10}K" if n % 1024 == 0 else str(n)
    c = f"{ctx(lens[0])} ctx" if len(set(lens)) == 1 else f"ragged {ctx(min(lens))}-{ctx(max(lens))} ctx"
    extra = (f", {spec.R} rows/seq" if getattr(spec, "R", 1) > 1 else "") + \
            (f", pools of {spec.pool}" if getattr(spec, "pool", 1) > 1 else "")
    return f"{METRIC_BASE}, batch {spec.B} @ {c}{extra}"
EXPERT_BYTES_GATE_UP = lambda s: 2 * s.I * s.D + 2 * (s.I // 128) * (s.D // 128) * 4  # per touched expert
EXPERT_BYTES_DOWN = lambda s: s.D * s.I + (s.D // 128) * (s.I // 128) * 4


def algorithmic_bytes(spec, lens, n_touched: int) -> dict:
    """Bytes the method must read per step (weights and caches once; activations are negligible)."""
    pool = getattr(spec, "pool", 1)  # > 1: one indexer key per pool of `pool` positions
    keys = sum((int(l) + pool - 1) // pool for l in lens) * spec.DI
    nb = (spec.Dc + 127) // 128
    R = getattr(spec, "R", 1)  # query rows per sequence: each row keeps its own positions (up to its own)
    kv = sum(min(max(0, int(l) - (R - 1 - r)), spec.topk) for l in lens for r in range(R)) * (spec.Dc + 4 * nb)
    hd = spec.head_dim or spec.Dv
    wuv = spec.H * hd * spec.Dv + spec.H * (hd // 128) * (spec.Dv // 128) * 4 if spec.head_dim else 0
    wo = spec.D * spec.wo_in + (spec.D // 128) * (spec.wo_in // 128) * 4
    wr = spec.E * spec.D * 4
    gu = n_touched * EXPERT_BYTES_GATE_UP(spec)
    dn = n_touched * EXPERT_BYTES_DOWN(spec)
    return dict(indexer_keys=keys, selected_kv=kv, w_uv=wuv, w_o=wo, w_r=wr, expert_gate_up=gu, expert_down=dn,
                total=keys + kv + wuv + wo + wr + gu + dn)


# HBM traffic of the gate/up kernel as read by rocprofv3 PMC counters (FETCH_SIZE + WRITE_SIZE per dispatch,
# scaled by what the same counters read for a plain copy of known size).  Reported only while the kernel's
# source is the one the counters were taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_b8-128k.md")
KERNEL_SOURCES = ("sparse_attention_moe_amd/csrc/k_gemv.hip", "sparse_attention_moe_amd/csrc/dl_common.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    vals = dict(re.findall(r"^- (\w+): (\S+)\s*$", text, re.M))
    if vals.get("kernel_source_sha256") != kernel_source_hash() or vals.get("workload") != workload:
        return None
    return int(vals["traffic_bytes_per_launch"])


def copy_calibration(mib: int, reps: int = 3):
    """A plain device copy of known size, for scaling the PMC byte counters (not timed, not reported)."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: {reps} x {mib << 20} bytes", file=sys.stderr, flush=True)


def read_ceiling(reps: int, mib: int = 1536) -> dict:
    """HBM read rate of a plain streaming read (dl_probe_read: the expert stream's access pattern without the
    arithmetic) over random bytes, like FP8 weights, and over a constant fill: context for `roofline`, whose
    peak stays the published 8 TB/s.  Each buffer is far larger than the 256 MB last-level cache."""
    out = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(12345)
    for kind in ("random", "constant"):
        buf = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
        if kind == "random":
            buf.random_(0, 256, generator=g)
        else:
            buf.fill_(0x3C)
        n = dl.probe_read(buf)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            dl.probe_read(buf)
        e1.record()
        torch.cuda.synchronize()
        out[f"{kind}_gbs"] = round(n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        del buf
    out["bytes_per_read"] = n
    return out


def null_phases(reps: int, kernels: int = 11, blocks: int = 256) -> dict:
    """Fixed cost of the step's dependent launches: `kernels` back-to-back launches of an empty kernel
    (dl_probe_null; the step launches 11 kernels up to 16 tokens), one workgroup per compute unit."""
    dl.probe_null(kernels, blocks)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dl.probe_null(kernels, blocks)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    return {"kernels": kernels, "workgroups": blocks, "us_per_chain": round(us, 2),
            "us_per_kernel": round(us / kernels, 3)}


class Unfused:
    """The step as its four separate entry points (dl_indexer_topk, dl_sparse_attn_decode with W_UV, W_O and the
    residual, dl_moe_route, dl_moe_ffn) on the same tiled weights and preallocated workspaces."""

    def __init__(self, spec, t, step):
        dev = t["x"].device
        B = spec.B
        self.spec, self.t = spec, t
        self.pg = dl.pages(t["seq_lens"], t["page_table"], spec.page_size, step.key_layout)
        self.sel = torch.empty(B, spec.topk, dtype=torch.int32, device=dev)
        self.h = torch.empty(B, spec.D, dtype=torch.float32, device=dev)
        self.ex = torch.empty(B, spec.ke, dtype=torch.int32, device=dev)
        self.g = torch.empty(B, spec.ke, dtype=torch.float32, device=dev)
        self.y = torch.empty_like(step.y)
        # a matrix the workload does not have (the tiny workload's W_UV) is passed as NULL
        self.m = {k: (step.mat(k) if step.mat(k).w else None) for k in ("w_uv", "w_o", "w_gate", "w_up", "w_down")}
        self.keep = step  # the tiled weights live in the step object
        import ctypes as C
        L = dl.load()
        self.ws_i = dl.workspace(L.dl_indexer_topk_workspace(C.byref(self.pg)), dev)
        ref = lambda m: C.byref(m) if m is not None else None
        self.ws_a = dl.workspace(L.dl_sparse_attn_workspace(B, spec.H, spec.Dv, spec.topk, ref(self.m["w_uv"]),
                                                            ref(self.m["w_o"])), dev)
        self.ws_r = dl.workspace(L.dl_moe_route_workspace(B, spec.D, spec.E), dev)
        self.ws_f = dl.workspace(L.dl_moe_ffn_workspace(B, spec.D, spec.I, spec.ke, spec.E, spec.n_shared), dev)

    def __call__(self):
        sp, t = self.spec, self.t
        dl.indexer_topk(self.pg, t["q_idx"], self.keep.keys, sp.topk, self.sel, ws=self.ws_i)
        dl.sparse_attn_decode(self.pg, t["q"], t["kv"], t.get("kv_scale"), sp.H, sp.Dc, sp.Dv, sp.scale, self.sel,
                              sp.topk, self.h, w_uv=self.m["w_uv"], w_o=self.m["w_o"], residual=t["x"], ws=self.ws_a)
        dl.moe_route(self.h, t["w_r"], t["r_bias"], sp.ke, self.ex, self.g, ws=self.ws_r)
        dl.moe_ffn(self.h, self.ex, self.g, self.m["w_gate"], self.m["w_up"], self.m["w_down"], sp.E, sp.n_shared,
                   self.y, residual=self.h, ws=self.ws_f)
        return self.y


def timed(fn_list, steps: int) -> float:
    """Mean milliseconds per call over `steps` calls (rotating over fn_list), two events around them all."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        fn_list[i % len(fn_list)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_step_ms(fn_list, steps: int) -> list:
    """Milliseconds of each of `steps` calls, one event between consecutive calls."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        fn_list[i % len(fn_list)]()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def touched(spec, experts: np.ndarray) -> int:
    return len(set(int(e) for e in experts.ravel())) + spec.n_shared


def cpu_baseline(spec, t, seconds: float):
    """The oracle, as it stands, on a bounded sample of one step: its rows (each row of a step is independent),
    cycled until about `seconds` of CPU work, then scaled to a whole step.  A first, untimed pass over the rows
    makes the host copies of the caches and of the experts the rows touch."""
    import oracle
    cores = oracle.threads()
    orc = oracle.LayerOracle(spec, t)
    rows = spec.B * getattr(spec, "R", 1)
    for b in range(rows):
        orc.row(b)
    n = 0
    t0 = time.perf_counter()
    while True:
        orc.row(n % rows)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= seconds or n >= 64 * rows:
            break
    per_step = dt / n * rows
    return {"value": 1.0 / per_step, "unit": "layer-steps/s", "cores": cores, "host_cpus": os.cpu_count(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "kind": "oracle",
            "sample": f"{n} row evaluations cycling over the {rows} rows of one {spec.name} step (indexer over the "
                      f"full context, attention, projections, router, FFN), {dt:.1f} s, scaled to a whole step"}


def share_step(args, spec, mode: str, n: int = 8):
    """One GPU's share of an n-GPU layer step (DP attention): the indexer and attention (+ W_UV, W_O, residual) for
    its B/n sequences, the router for all B tokens (each GPU routes every token after the all-gather of h), and
    - mode "tp8": the FFN for all B tokens on intermediate rows [0, I/n) of every expert (tensor-parallel experts);
    - mode "ep8": the FFN for the picks of the E/n routed experts the GPU holds, plus the shared expert
      (expert-parallel).  The GPU taken is the one whose experts the instance's routing touches most: the layer
      step waits for the slowest GPU.
    The all-gather of h and the reduce-scatter (or all-to-all) of y need a second GPU and are not run."""
    dev = "cuda"
    Bl = spec.B // n
    per = spec.E // n
    insts = []
    t0 = time.perf_counter()
    for i in range(args.instances):
        t = synth.make_layer(spec, seed=args.seed, device=dev, instance=i)
        h = (t["x"].float() + 0.1 * torch.randn(spec.B, spec.D, device=dev)).contiguous()  # all-gathered h
        ex = torch.empty(spec.B, spec.ke, dtype=torch.int32, device=dev)
        g = torch.empty(spec.B, spec.ke, dtype=torch.float32, device=dev)
        gpu, loads = 0, None
        if mode == "ep8":
            dl.moe_route(h, t["w_r"], t["r_bias"], spec.ke, ex, g)  # untimed: which GPU carries the most experts
            picks = ex.cpu().numpy().ravel()
            loads = [len(set(int(e) for e in picks if k * per <= e < (k + 1) * per)) for k in range(n)]
            gpu = int(np.argmax(loads))
            w = synth.ep_slice(t, spec, gpu, n)
        else:
            w = synth.tp_slice(t, spec, 0, n)
        for k in ("w_gate", "w_up", "w_down"):
            t[k] = None
        m = {k: dl.pack_weights(w[k], w[k + "_scale"]) for k in ("w_gate", "w_up", "w_down")}
        mats = {k: dl.mat(m[k], w[k + "_scale"], dl.DL_LAYOUT_TILES) for k in m}
        keep = (m, w)
        pg = dl.pages(t["seq_lens"][:Bl].contiguous(), t["page_table"][:Bl].contiguous(), spec.page_size)
        sel = torch.empty(Bl, spec.topk, dtype=torch.int32, device=dev)
        hl = torch.empty(Bl, spec.D, dtype=torch.float32, device=dev)
        y = torch.empty(spec.B, spec.D, dtype=torch.float32, device=dev)
        wuv = dl.mat(dl.pack_weights(t["w_uv"], t["w_uv_scale"]), t["w_uv_scale"], dl.DL_LAYOUT_TILES)
        wo = dl.mat(dl.pack_weights(t["w_o"], t["w_o_scale"]), t["w_o_scale"], dl.DL_LAYOUT_TILES)
        insts.append(dict(t=t, mats=mats, keep=keep, pg=pg, sel=sel, hl=hl, h=h, ex=ex, g=g, y=y, wuv=wuv, wo=wo,
                          gpu=gpu, loads=loads,
                          q_idx=t["q_idx"][:Bl].contiguous(), q=t["q"][:Bl].contiguous(), x=t["x"][:Bl].contiguous()))
    torch.cuda.synchronize()
    print(f"[bench] generated {args.instances} x {spec.name} shares in {time.perf_counter() - t0:.1f} s",
          file=sys.stderr, flush=True)
    ws = {}

    def step(it):
        t = it["t"]
        dl.indexer_topk(it["pg"], it["q_idx"], t["k_pool"], spec.topk, it["sel"], ws=ws.get("i"))
        dl.sparse_attn_decode(it["pg"], it["q"], t["kv"], t["kv_scale"], spec.H, spec.Dc, spec.Dv, spec.scale,
                              it["sel"], spec.topk, it["hl"], w_uv=it["wuv"], w_o=it["wo"], residual=it["x"],
                              ws=ws.get("a"))
        dl.moe_route(it["h"], t["w_r"], t["r_bias"], spec.ke, it["ex"], it["g"], ws=ws.get("r"))
        mt = it["mats"]
        if mode == "ep8":
            dl.moe_ffn_ep(it["h"], it["ex"], it["g"], it["gpu"] * per, mt["w_gate"], mt["w_up"], mt["w_down"], per,
                          spec.n_shared, it["y"], residual=it["h"], ws=ws.get("f"))
        else:
            dl.moe_ffn(it["h"], it["ex"], it["g"], mt["w_gate"], mt["w_up"], mt["w_down"], spec.E, spec.n_shared,
                       it["y"], residual=it["h"], ws=ws.get("f"))

    L = dl.load()
    it0 = insts[0]
    ws["i"] = dl.workspace(L.dl_indexer_topk_workspace(dl.C.byref(it0["pg"])), dev)
    ws["a"] = dl.workspace(L.dl_sparse_attn_workspace(Bl, spec.H, spec.Dv, spec.topk, dl.C.byref(it0["wuv"]),
                                                      dl.C.byref(it0["wo"])), dev)
    ws["r"] = dl.workspace(L.dl_moe_route_workspace(spec.B, spec.D, spec.E), dev)
    if mode == "ep8":
        ws["f"] = dl.workspace(L.dl_moe_ffn_workspace(spec.B, spec.D, spec.I, spec.ke, per, spec.n_shared), dev)
    else:
        ws["f"] = dl.workspace(L.dl_moe_ffn_workspace(spec.B, spec.D, spec.I // n, spec.ke, spec.E, spec.n_shared),
                               dev)
    for i in range(args.warmup):
        step(insts[i % len(insts)])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(insts[i % len(insts)])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    share = synth.spec_replace(spec, B=Bl, seq_lens=spec.seq_lens[:Bl])
    b = algorithmic_bytes(share, share.seq_lens, 0)
    if mode == "ep8":  # the GPU's touched routed experts + the shared expert, whole
        touched_n = sum(max(it["loads"]) + spec.n_shared for it in insts) / len(insts)
        gu = touched_n * EXPERT_BYTES_GATE_UP(spec)
        dn = touched_n * EXPERT_BYTES_DOWN(spec)
    else:  # 1/n of every touched expert
        touched_n = sum(touched(spec, it["ex"].cpu().numpy()) for it in insts) / len(insts)
        gu = touched_n * EXPERT_BYTES_GATE_UP(spec) / n
        dn = touched_n * EXPERT_BYTES_DOWN(spec) / n
    total = b["total"] + gu + dn
    rec = {"metric": f"one GPU's share of an 8-GPU decode layer step (exchanges not run), layer-steps/s, "
                     f"{metric_label(spec).split(', ', 2)[-1]}",
           "value": round(1000.0 / ms, 2), "unit": "layer-steps/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "fp8-weights/int8-indexer/fp32-accum", "data": "synthetic",
           "config": {"workload": f"{spec.name}-{mode[:2]}{n}-share", "sequences": Bl, "tokens_routed": spec.B,
                      "context": int(max(spec.seq_lens))},
           "share_hbm": {"algorithmic_bytes": int(total), "achieved_gbs": round(total / (ms * 1e-3) / 1e9, 1),
                         "frac": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "touched_experts": round(touched_n, 2)}}
    if mode == "ep8":
        rec["config"]["experts_per_gpu"] = per
        rec["expert_loads"] = [it["loads"] for it in insts]  # distinct routed experts each GPU would apply
    else:
        rec["config"]["inter_slice"] = spec.I // n
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=12,
                    help="untimed steps first (3 per rotated instance: the expert kernels' pool shares settle in 2-3 calls)")
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--instances", type=int, default=4)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU time of the oracle baseline sample")
    ap.add_argument("--no-read-ceiling", action="store_true", help="skip the streaming-read probe")
    ap.add_argument("--share", choices=["tp8", "ep8"], default=None,
                    help="time one GPU's share of an 8-GPU layer instead (DP attention on one sequence, router for "
                         "every token, and the FFN as a tensor-parallel slice of inter/8 rows of every expert (tp8) "
                         "or as the E/8 experts the GPU holds (ep8)); the exchanges are not run")
    ap.add_argument("--rows-per-seq", type=int, default=1,
                    help="query rows per sequence (multi-row decode, e.g. MTP verification); 1 = ordinary decode")
    ap.add_argument("--pool", type=int, default=1,
                    help="pool-granular selection: score one key per pool of this many positions and keep top_k/pool "
                         "pools; 1 = per-position selection")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the run, copy this many MiB device-to-device (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    spec = synth.config(args.config)
    if args.share:
        return share_step(args, spec, args.share)
    if args.rows_per_seq != 1:
        spec = synth.spec_replace(spec, R=args.rows_per_seq, name=f"{spec.name}-rows{args.rows_per_seq}")
    if args.pool != 1:
        spec = synth.spec_replace(spec, pool=args.pool, name=f"{spec.name}-pool{args.pool}")
    dev = "cuda"
    insts, steps_obj = [], []
    t0 = time.perf_counter()
    for i in range(args.instances):
        t = synth.make_layer(spec, seed=args.seed, device=dev, instance=i)
        insts.append(t)
        # debug outputs allocated but switched off: the timed steps write only y, as in production
        steps_obj.append(dl.LayerStep(spec, t, debug=True))
        steps_obj[-1].debug_outputs(False)
    torch.cuda.synchronize()
    print(f"[bench] generated {args.instances} x {spec.name} in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
          flush=True)
    n = len(steps_obj)
    for i in range(args.warmup):
        steps_obj[i % n]()
    torch.cuda.synchronize()
    # timed region 1: the whole step, nothing else recorded
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        steps_obj[i % n]()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # timed region 2: same steps with phase events on the library's stream (per-kernel durations)
    dl.profile_enable(True)
    torch.cuda.synchronize()
    for i in range(args.steps):
        steps_obj[i % n]()
    torch.cuda.synchronize()
    ph, nst = dl.profile_read()
    dl.profile_enable(False)
    ph = {k: v / nst for k, v in ph.items()}
    # timed region 3: one event between consecutive steps, for the spread of single steps
    each = per_step_ms(steps_obj, args.steps)
    # timed region 4: the same steps as four separate entry points
    unfused_ms = None
    if spec.R == 1 and spec.pool == 1:  # the separate entry points are the ordinary decode path
        unf = [Unfused(spec, t, so) for t, so in zip(insts, steps_obj)]
        for u in unf:
            u()
        unfused_ms = round(timed(unf, args.steps), 4)
        del unf
    nulls = null_phases(args.steps)
    # the current-token append (the step before S1; not part of the timed step): its own launches, bf16 inputs
    app_rec = None
    if spec.Dc >= 256:
        B_app = max(8, spec.B)
        app = synth.make_append(seed=args.seed, B=B_app, Dc=spec.Dc, DI=spec.DI, page_size=spec.page_size,
                                bf16=True, device=dev)
        apg = dl.pages(app["seq_lens"], app["page_table"], spec.page_size)
        call = lambda: dl.kv_append(apg, app["latent"], app["key"], float(app["key_scale"]), app["kv_pool"],
                                    app["kv_scale"], app["k_pool"])
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        app_us = e0.elapsed_time(e1) / args.steps * 1000.0
        nb = (spec.Dc + 127) // 128
        app_bytes = B_app * (2 * spec.Dc + 2 * spec.DI + spec.Dc + 4 * nb + spec.DI)
        app_rec = {"us_per_call": round(app_us, 2), "rows": B_app, "bytes_per_call": app_bytes,
                   "bound": "latency", "achieved_gbs": round(app_bytes / (app_us * 1e-6) / 1e9, 2)}
    # algorithmic bytes of the steps actually run (touched experts per instance, from one untimed step each with
    # the debug outputs on)
    for so in steps_obj:
        so.debug_outputs(True)
        so()
    torch.cuda.synchronize()
    per_inst = []
    for s in steps_obj:
        ex = s.dbg["experts"].cpu().numpy()
        per_inst.append((touched(spec, ex), algorithmic_bytes(spec, spec.seq_lens, touched(spec, ex))))
    avg_touch = sum(p[0] for p in per_inst) / n
    avg_bytes = {k: sum(p[1][k] for p in per_inst) / n for k in per_inst[0][1]}
    steps_per_s = 1000.0 / ms
    step_gbs = avg_bytes["total"] / (ms * 1e-3) / 1e9
    # the dominant kernel: the fused expert FFN (gate/up, SwiGLU split and down in one launch, phase 5) where the
    # step ran it, else the gate/up GEMV
    fused = dl.profile_ffn_fused() == 1
    dom_bytes = avg_bytes["expert_gate_up"] + (avg_bytes["expert_down"] if fused else 0)
    dom_name = ("k_ffn_fp8 (expert FFN: gate/up, SwiGLU split, down)" if fused else
                "k_gemv_fp8<2,SWIGLU> (expert gate/up)" if spec.fp8 else "k_gemv_f32<SWIGLU> (expert gate/up)")
    gu_gbs = dom_bytes / (ph["expert_gate_up"] * 1e-3) / 1e9
    rec = {
        "metric": metric_label(spec), "value": round(steps_per_s, 2), "unit": "layer-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8-weights/int8-indexer/fp32-accum",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.B, "context": int(max(spec.seq_lens)), "hidden": spec.D,
                   "heads": spec.H, "latent": spec.Dc, "top_k": spec.topk, "experts": f"{spec.E}+{spec.n_shared}",
                   "expert_top_k": spec.ke, "inter": spec.I, "rows_per_seq": spec.R, "pool": spec.pool,
                   "instances_rotated": n},
        "tokens_per_s_per_layer": round(steps_per_s * spec.B * spec.R, 1),
        "ms_per_step_median": round(float(np.median(each)), 4), "ms_per_step_min": round(float(np.min(each)), 4),
        "unfused_ms_per_step": unfused_ms, "null_phases": nulls,
        "step_hbm": {"algorithmic_bytes": int(avg_bytes["total"]), "achieved_gbs": round(step_gbs, 1),
                     "peak_gbs": HBM_PEAK_GBS, "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                     "touched_experts": round(avg_touch, 2)},
        "phase_ms": {k: round(v, 4) for k, v in ph.items()},
        "roofline": {"kernel": dom_name, "bound": "hbm",
                     "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(spec.name),
                     "bytes_per_launch": int(dom_bytes),
                     "ms_per_launch": round(ph["expert_gate_up"], 4)},
    }
    if app_rec:
        rec["kv_append"] = app_rec
    if not args.no_read_ceiling:
        rec["read_ceiling"] = read_ceiling(args.steps)
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(spec, insts[0], args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    if args.copy_mib:
        copy_calibration(args.copy_mib)


if __name__ == "__main__":
    main()
