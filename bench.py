#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X (gfx950).

A step is one whole layer forward -- router, dispatch, gate/up + SwiGLU grouped
GEMM, down grouped GEMM, combine -- over one batch of seeded synthetic input
already resident in HBM.  Default workload: the prefill-sized dots3-note
layer (T=16384 tokens, hidden 5120, 256 routed + 1 shared experts, top-8,
moe_intermediate 1536, bf16).  Prints ONE JSON line on stdout.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Extra objects in the line:
  roofline     the gate/up GEMM (the dominant kernel), timed live with HIP
               events recorded on the stream it runs on, against the dense
               bf16 MFMA peak; traffic from the committed rocprofv3 counter
               summary when its kernel source hash still matches.
  decode_T256  the same layer at T=256 tokens (weight streaming): time,
               algorithmic HBM GB/s and its fraction of 8 TB/s; also as
               one cooperative launch (moe_layer_forward_fused).
  grouped_routing  the router (logits GEMM + selection) with group-limited
               routing (8 groups, 4 chosen) next to the plain router.
  block        the decoder block around the layer (RMSNorm, layer, residual
               add in the combine) and the RMSNorm kernel alone against HBM.
  device_copy  a 2 GiB device-to-device torch copy (reads + writes over
               its time), as context for the HBM figures.
  row_major_weights  the same layer with the expert weights row-major
               (the timed line uses them packed into 16-row x 256-byte tiles
               once at load time, moe_pack_expert_weights; --weights rows
               times row-major weights instead).
  cpu_baseline the fp64 CPU oracle on the first tokens of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
METRIC = "MoE layer fwd tokens/s & TFLOP/s (T=16384); HBM GB/s at T=256; % roofline"
GEMM_SRCS = [os.path.join(ROOT, "sparse_moe_expert_amd", "csrc", f)
             for f in ("gemm.hip", "gemm_big.hip", "gemm_decode.hip", "gemm_decode_device.h",
                       "gemm_sched.h", "moe_device.h", "moe_internal.h")]
EXPERT_KEYS = ("w_gate_up", "w_down", "w_sh_gate_up", "w_sh_down")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def gemm_source_hash() -> str:
    """Hash of the GEMM kernel sources: counter figures taken on other sources
    no longer describe the kernel that runs."""
    h = hashlib.sha256()
    for f in GEMM_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def gate_up_flops(cfg) -> float:
    """Matmul flops of the gate/up GEMM: every routed (token, slot) row and
    every shared row multiplies [H] by the packed [2I, H] weight."""
    rows = cfg.T * cfg.k + cfg.T * cfg.S
    return 2.0 * rows * cfg.H * 2 * cfg.I


def weight_bytes_per_expert(cfg) -> float:
    esz = {"bf16": 2, "f32": 4, "fp8": 1}[cfg.expert]
    b = 3.0 * cfg.H * cfg.I * esz
    if cfg.expert == "fp8":
        b += 4.0 * (2 * cfg.I // 128 * cfg.H // 128 + cfg.H // 128 * cfg.I // 128)
    return b


def layer_bytes(cfg, counts) -> float:
    """Algorithmic HBM bytes of one layer forward: the weights of every expert
    that receives a token, the shared experts, the router weight and bias, x in
    and out; intermediates (h, y) excluded -- the method does not need them."""
    asz = {"bf16": 2, "f32": 4}[cfg.act]
    touched = int((counts > 0).sum())
    return (touched * weight_bytes_per_expert(cfg) + cfg.S * weight_bytes_per_expert(cfg)
            + cfg.E * cfg.H * asz + 4.0 * cfg.E + 2.0 * cfg.T * cfg.H * asz
            + 8.0 * cfg.T * cfg.k)


def gate_up_bytes(cfg, counts) -> float:
    """Algorithmic HBM bytes of one gate/up GEMM launch: the packed gate/up
    weights (and block scales) of every touched routed expert and of the
    shared experts, each token row of x read once, h written once."""
    esz = {"bf16": 2, "f32": 4, "fp8": 1}[cfg.expert]
    w = 2.0 * cfg.I * cfg.H * esz
    if cfg.expert == "fp8":
        w += 4.0 * (2 * cfg.I // 128) * (cfg.H // 128)
    touched = int((counts > 0).sum())
    rows = cfg.T * cfg.k + cfg.T * cfg.S
    x_b = cfg.T * cfg.H * (1 if cfg.expert == "fp8" else esz)
    h_b = rows * cfg.I * (1 if cfg.expert == "fp8" else 2)
    return (touched + cfg.S) * w + x_b + h_b


def gate_up_roofline(cfg, ms, counts, dtype):
    """The dominant kernel against the roof that bounds it: MFMA peak of its
    dtype when its intensity is above the ridge point, else HBM."""
    flops = gate_up_flops(cfg)
    byts = gate_up_bytes(cfg, counts)
    peak_f = PEAK_TFLOPS[dtype]
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    traffic = load_traffic(cfg.name)
    base = {"kernel": "grouped_gemm gate/up + SwiGLU", "kernel_ms": round(ms, 4),
            "flops_per_launch": flops, "bytes_per_launch": byts,
            "intensity_flop_per_byte": round(flops / byts, 1), "traffic": traffic}
    if flops / byts >= ridge:
        a = flops / (ms / 1e3) / 1e12
        return dict(base, bound="mfma", achieved=round(a, 1), peak=peak_f, unit="TFLOP/s",
                    frac=round(a / peak_f, 4))
    a = byts / (ms / 1e3) / 1e9
    return dict(base, bound="hbm", achieved=round(a, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                frac=round(a / PEAK_HBM_GBS, 4))


def load_traffic(workload: str):
    """Per-launch HBM bytes of the gate/up GEMM from the committed counter
    summary, or None if missing or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"gate_up_gemm_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    return d.get("bytes_per_launch")


def time_layer(lay, steps, warmup, timed_events=True):
    """K plain layer forwards timed by the host clock between two device
    synchronisations (the step time), then K more with HIP events recorded at
    the stage boundaries on the layer's stream (the stage times; the events
    themselves add ~25-50 us to a step, so they stay out of the first pass).
    Returns (step ms, instrumented step ms, event step ms, stage ms, counts,
    p10/p50/p90 of the per-step event times)."""
    import torch
    import sparse_moe_expert_amd as moe
    out = lay.empty_out()
    counts = torch.empty(lay.cfg.E, dtype=torch.int32, device="cuda")
    for _ in range(warmup):
        lay.forward(out=out, counts=counts)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        lay.forward(out=out, counts=counts)
    torch.cuda.synchronize()
    plain = (time.perf_counter() - t0) * 1e3 / steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    for row in ev:          # torch creates the HIP event on its first record
        for e in row:
            e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe.moe_layer_forward_timed(lay.ccfg, lay.weights, lay.t["x"], out, ev[i],
                                    opt_counts=counts, workspace=lay.workspace)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ["route", "dispatch", "quant_x", "gate_up_gemm", "down_gemm", "combine"]
    stage = {n: sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)) / steps
             for j, n in enumerate(names)}
    per_step = sorted(ev[i][0].elapsed_time(ev[i][6]) for i in range(steps))
    step_ev = sum(per_step) / steps

    def pct(q):
        return per_step[min(steps - 1, int(round(q * (steps - 1))))]

    spread = {"p10": round(pct(0.1), 4), "p50": round(pct(0.5), 4), "p90": round(pct(0.9), 4)}
    return plain, wall * 1e3 / steps, step_ev, stage, counts.cpu().numpy(), spread


def time_calls(fn, iters, warmup):
    """Mean ms per call of `fn`, timed with events on torch's current stream
    (the stream the library launches on)."""
    import torch
    for _ in range(warmup):
        fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def device_copy(gib=2.0, iters=5):
    """A plain device-to-device copy of `gib` GiB with torch's copy kernel:
    bytes read + written over its event time.  Context for the HBM figures:
    a copy mixes reads and writes half and half, so it is no ceiling for the
    read-dominated layer (which streams faster than it)."""
    import torch
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    ms = time_calls(lambda: b.copy_(a), iters, 2)
    del a, b
    return {"bytes_per_copy": 2 * n, "ms": round(ms, 4), "GBps": round(2 * n / (ms / 1e3) / 1e9, 1)}


def grouped_routing(lay, cfg, n_group=8, topk_group=4, iters=20):
    """Router time with and without the group limit on the same inputs."""
    import torch
    import sparse_moe_expert_amd as moe
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    cg = moe.make_config(cfg.T, cfg.H, cfg.E, cfg.S, cfg.k, cfg.I, cfg.Is, act=cfg.act,
                         expert=cfg.expert, n_group=n_group, topk_group=topk_group)
    ws = torch.empty(moe.moe_workspace_size(cg), dtype=torch.uint8, device="cuda")
    x = lay.t["x"]
    plain = time_calls(lambda: moe.moe_route(lay.ccfg, x, lay.weights, idx, tw, None,
                                             lay.workspace), iters, 3)
    grouped = time_calls(lambda: moe.moe_route(cg, x, lay.weights, idx, tw, None, ws), iters, 3)
    torch.cuda.synchronize()
    groups = (idx.cpu().numpy() // (cfg.E // n_group))
    return {"n_group": n_group, "topk_group": topk_group, "route_ms": round(grouped, 4),
            "plain_route_ms": round(plain, 4),
            "max_groups_per_token": int(max(len(set(r.tolist())) for r in groups))}


def block_forward(lay, cfg, steps):
    """The decoder block (RMSNorm -> layer -> residual) and the RMSNorm kernel
    alone: its algorithmic bytes (read h and gamma, write the normalised rows)
    over its time."""
    import numpy as np
    import torch
    import sparse_moe_expert_amd as moe
    from sparse_moe_expert_amd.device import to_device
    g = 1.0 + 0.1 * np.random.default_rng(5).standard_normal(cfg.H)
    gamma = to_device(g.astype(np.float32), "f32").to(lay.act_dtype)
    out = lay.empty_out()
    xn = lay.empty_out()
    h = lay.t["x"]
    eps = cfg.rms_norm_eps
    blk = time_calls(lambda: moe.moe_block_forward(lay.ccfg, lay.weights, h, gamma, eps, out,
                                                   None, None, lay.workspace), steps, 3)
    # the layer alone, timed the same way
    lyr = time_calls(lambda: moe.moe_layer_forward(lay.ccfg, lay.weights, h, out, None, None,
                                                   lay.workspace), steps, 3)
    norm = time_calls(lambda: moe.moe_rmsnorm(lay.ccfg, h, gamma, eps, xn), 50, 5)
    asz = h.element_size()
    nbytes = 2.0 * cfg.T * cfg.H * asz + cfg.H * asz
    gbs = nbytes / (norm / 1e3) / 1e9
    return {"ms_per_step": round(blk, 4), "tokens_per_s": round(cfg.T / (blk / 1e3), 1),
            "layer_ms_same_timing": round(lyr, 4),
            "overhead_vs_layer_ms": round(blk - lyr, 4),
            "rmsnorm": {"kernel_ms": round(norm, 4), "bytes_per_launch": nbytes,
                        "achieved_GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}}


def cpu_baseline(cfg, inp, n_tokens):
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    tokens = np.arange(min(n_tokens, cfg.T))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.layer_forward(cfg, inp, tokens=tokens)
        dt = time.perf_counter() - t0
    return {"value": round(tokens.size / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"first {tokens.size} tokens of {cfg.name} (full routing over all "
                      f"{cfg.E} experts, their SwiGLU experts and the shared expert), fp64 numpy, "
                      "one thread"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload id (default 2: T=16384)")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-decode", action="store_true", help="skip the T=256 line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the grouped-routing, block and row-major-weights lines")
    ap.add_argument("--cpu-tokens", type=int, default=1280)
    ap.add_argument("--weights", choices=("tiled", "rows"), default="tiled",
                    help="expert weight storage of the timed layer (default: packed tiles)")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="also run one plain device-to-device copy of this many GiB "
                         "(calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU only (asked for --gpus {args.gpus}); "
              "the layer would shard by experts across GPUs, which is not built here.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from moe_inputs import config, generate
    from sparse_moe_expert_amd.device import DeviceLayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = config(args.config)
    log(f"bench: generating {cfg.name} inputs")
    t0 = time.perf_counter()
    inp = generate(cfg)
    log(f"bench: generated in {time.perf_counter() - t0:.1f}s; uploading")
    lay_rows = DeviceLayer(cfg, inp)
    tiled = args.weights == "tiled"
    if tiled:
        # load-time preparation, outside the timed region: the expert weights
        # packed once into the tiled storage
        from sparse_moe_expert_amd.device import pack_expert_weights
        packed = {key: pack_expert_weights(lay_rows.t[key], cfg.expert) for key in EXPERT_KEYS}
        lay = _view(lay_rows, cfg, expert_t=packed, tiled=True)
    else:
        lay = lay_rows
    torch.cuda.synchronize()

    log(f"bench: {args.warmup} warmup + {args.steps} timed steps")
    ms, ms_inst, ms_ev, stage, counts, spread = time_layer(lay, args.steps, args.warmup)
    flops = cfg.flops()
    dtype = cfg.expert if cfg.expert != "f32" else "f32"
    res = {
        "metric": METRIC,
        "value": round(cfg.T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "S": cfg.S,
                   "k": cfg.k, "I": cfg.I, "precision": dtype, "seed": 0,
                   "expert_weights": "tiled16x256B" if tiled else "row_major"},
        "tflops": round(flops / (ms / 1e3) / 1e12, 2),
        "frac_of_peak_mfma_whole_step": round(flops / (ms / 1e3) / 1e12 / PEAK_TFLOPS[dtype], 4),
        "ms_per_step_instrumented": round(ms_inst, 4),
        "ms_per_step_events": round(ms_ev, 4),
        "ms_per_step_events_p10_p50_p90": spread,
        "stages_ms": {k: round(v, 4) for k, v in stage.items()},
        "rows_per_expert": {"max": int(counts.max()), "mean": float(counts.mean()),
                            "empty": int((counts == 0).sum())},
    }

    res["roofline"] = gate_up_roofline(cfg, stage["gate_up_gemm"], counts, dtype)

    if not args.no_decode and args.config == 2:
        # T = 256 tokens (the decode-sized workload's x, router weight and bias)
        # through the same resident expert weights: the two workloads share
        # every shape and weight distribution.
        cfg1 = config(1)
        inp1 = generate(cfg1, weights=False)
        lay1 = _view(lay, cfg1, inp1)
        log(f"bench: decode T={cfg1.T}: {args.decode_steps} steps")
        ms1, ms1_inst, _, stage1, counts1, spread1 = time_layer(lay1, args.decode_steps, 5)
        b1 = layer_bytes(cfg1, counts1)
        gbs = b1 / (ms1 / 1e3) / 1e9
        # the same layer as one cooperative launch
        import sparse_moe_expert_amd as moe
        out1 = lay1.empty_out()
        msf = time_calls(lambda: moe.moe_layer_forward_fused(
            lay1.ccfg, lay1.weights, lay1.t["x"], out1, None, None, lay1.workspace),
            args.decode_steps, 5)
        gbf = b1 / (msf / 1e3) / 1e9
        res["decode_T256"] = {
            "workload": cfg1.name, "ms_per_step": round(ms1, 4),
            "ms_per_step_instrumented": round(ms1_inst, 4),
            "ms_per_step_events_p10_p50_p90": spread1,
            "fused_single_launch": {"ms_per_step": round(msf, 4), "hbm_GBps": round(gbf, 1),
                                    "frac_of_hbm_peak": round(gbf / PEAK_HBM_GBS, 4)},
            "tokens_per_s": round(cfg1.T / (ms1 / 1e3), 1),
            "algorithmic_bytes": b1, "hbm_GBps": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "tflops": round(cfg1.flops() / (ms1 / 1e3) / 1e12, 2),
            "stages_ms": {k: round(v, 4) for k, v in stage1.items()},
            "experts_touched": int((counts1 > 0).sum()),
        }
        if tiled and not args.no_extras:
            ms1r = time_layer(_view(lay_rows, cfg1, inp1), args.decode_steps, 5)[0]
            g1r = b1 / (ms1r / 1e3) / 1e9
            res["decode_T256"]["row_major_weights"] = {
                "ms_per_step": round(ms1r, 4), "hbm_GBps": round(g1r, 1),
                "frac_of_hbm_peak": round(g1r / PEAK_HBM_GBS, 4)}

    if tiled and not args.no_extras:
        msr = time_layer(lay_rows, args.steps, args.warmup)[0]
        res["row_major_weights"] = {"ms_per_step": round(msr, 4),
                                    "tokens_per_s": round(cfg.T / (msr / 1e3), 1)}

    if not args.no_extras and args.config == 2:
        log("bench: grouped routing and block forward")
        res["grouped_routing"] = grouped_routing(lay, cfg)
        res["block"] = block_forward(lay, cfg, min(args.steps, 10))
        res["device_copy"] = device_copy()

    if args.calib_copy_gib > 0:
        n = int(args.calib_copy_gib * (1 << 30))
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        res["calib_copy_bytes"] = n

    if not args.no_cpu_baseline:
        log(f"bench: CPU oracle on {args.cpu_tokens} tokens")
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_tokens)
    else:
        res["cpu_baseline"] = None

    print(json.dumps(res), flush=True)


def _view(lay, cfg1, inp1=None, expert_t=None, tiled=None):
    """A DeviceLayer view of `lay` (same shapes) with another token batch and
    router (inp1) and/or other expert weight tensors (expert_t, stored as
    `tiled` says; default: as in `lay`).  Everything else is shared."""
    import torch

    from sparse_moe_expert_amd import _lib
    from sparse_moe_expert_amd.device import to_device

    class View:
        pass

    v = View()
    v.cfg = cfg1
    v.tiled = lay.tiled if tiled is None else tiled
    v.ccfg = _lib.make_config(cfg1.T, cfg1.H, cfg1.E, cfg1.S, cfg1.k, cfg1.I, cfg1.Is,
                              act=cfg1.act, expert=cfg1.expert,
                              norm_topk_prob=cfg1.norm_topk_prob,
                              routed_scaling_factor=cfg1.routed_scaling_factor,
                              n_group=cfg1.n_group, topk_group=cfg1.topk_group, tiled=v.tiled)
    t = dict(lay.t)
    if inp1 is not None:
        t["x"] = to_device(inp1["x"], cfg1.act)
        t["w_router"] = to_device(inp1["w_router"], cfg1.act)
        t["bias"] = to_device(inp1["bias"], "f32")
    if expert_t is not None:
        t.update(expert_t)
    v.t = t
    v.weights = _lib.make_weights(
        w_router=t["w_router"], router_bias=t["bias"], w_gate_up=t["w_gate_up"],
        w_down=t["w_down"], s_gate_up=t.get("s_gate_up"), s_down=t.get("s_down"),
        w_sh_gate_up=t["w_sh_gate_up"], w_sh_down=t["w_sh_down"],
        s_sh_gate_up=t.get("s_sh_gate_up"), s_sh_down=t.get("s_sh_down"))
    v.ws_bytes = _lib.moe_workspace_size(v.ccfg)
    v.workspace = torch.empty(v.ws_bytes, dtype=torch.uint8, device="cuda")
    v.act_dtype = lay.act_dtype
    v.empty_out = lambda: torch.empty((cfg1.T, cfg1.H), dtype=lay.act_dtype, device="cuda")

    def forward(out=None, counts=None, ties=None, stream=None):
        out = v.empty_out() if out is None else out
        _lib.moe_layer_forward(v.ccfg, v.weights, t["x"], out, counts, ties, v.workspace, stream)
        return out

    v.forward = forward
    return v


if __name__ == "__main__":
    main()
