#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X (gfx950).

A step is one whole layer forward -- router, dispatch, gate/up + SwiGLU grouped
GEMM, down grouped GEMM, combine -- over one batch of seeded synthetic input
already resident in HBM.  Default workload: the prefill-sized dots3-note
layer (T=16384 tokens, hidden 5120, 256 routed + 1 shared experts, top-8,
moe_intermediate 1536, bf16).  Prints ONE JSON line on stdout.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Extra objects in the line:
  roofline        the gate/up GEMM (the dominant kernel), timed live with HIP
                  events recorded on the stream it runs on, against the dense
                  bf16 MFMA peak; traffic from the committed rocprofv3 counter
                  summary when its kernel source hash still matches.
  decode_T256     the decode-sized workload on its own seeded weights:
                  time, algorithmic HBM GB/s and its fraction of 8 TB/s and of
                  the measured read ceiling; also as one cooperative launch.
  skewed_T8192    the Zipf-skewed dots.llm1-shaped workload (128 + 2 experts,
                  top-6, I 1408): time, TFLOP/s against the bf16 peak, bytes,
                  rows per expert, near-tie counts.
  fp8_T4096       the FP8 workload: time, fraction of 8 TB/s (it is below the
                  fp8 ridge) and of the fp8 MFMA peak, its gate/up roofline.
  ceilings        measured on the device: a streaming read of 4 GiB through
                  the library's read kernel, and the library's own prefill
                  GEMMs on one dense expert (E = 1, T = 16384).
  grouped_routing the router with group-limited routing (8 groups, 4 chosen)
                  next to the plain router.
  block           the decoder block around the layer (RMSNorm, layer,
                  residual add in the combine) and the RMSNorm kernel alone.
  device_copy     a 2 GiB device-to-device torch copy, as context.
  row_major_weights  the layer with row-major expert weights (the timed line
                  uses them packed into 16-row x 64-byte tiles once at load
                  time, moe_pack_expert_weights).
  cpu_baseline    the fp64 CPU oracle on a sample of the same workload, with
                  its BLAS threads set to the cores this process may use.
"""
from __future__ import annotations

import argparse
import gc
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
             for f in ("gemm.hip", "gemm_prefill.hip", "gemm_big.hip", "gemm_fp8.hip", "gemm_decode.hip",
                       "gemm_decode_device.h", "gemm_sched.h", "moe_device.h", "moe_internal.h")]
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


# ---------------------------------------------------------------- work models

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


# ---------------------------------------------------------------- timing

def time_layer(lay, steps, warmup):
    """K plain layer forwards timed by the host clock between two device
    synchronisations (the step time), then K more with HIP events recorded at
    the stage boundaries on the layer's stream (the stage times; the events
    themselves add ~25-50 us to a step, so they stay out of the first pass).
    Returns a dict: step ms, instrumented step ms, event step ms, stage ms,
    counts, near-tie counts, p10/p50/p90 of the per-step event times."""
    import torch
    import sparse_moe_expert_amd as moe
    out = lay.empty_out()
    counts = torch.empty(lay.cfg.E, dtype=torch.int32, device="cuda")
    ties = torch.zeros(2, dtype=torch.int32, device="cuda")
    lay.forward(out=out, counts=counts, ties=ties)
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

    def pct(q):
        return per_step[min(steps - 1, int(round(q * (steps - 1))))]

    return {"ms": plain, "ms_inst": wall * 1e3 / steps, "ms_ev": sum(per_step) / steps,
            "stage": stage, "counts": counts.cpu().numpy(), "ties": ties.cpu().tolist(),
            "spread": {"p10": round(pct(0.1), 4), "p50": round(pct(0.5), 4),
                       "p90": round(pct(0.9), 4)}}


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


def load_layer(cfg, tiled=True, keep_rows=False, keep_inputs=False, down_f16=True):
    """Generate the seeded inputs of `cfg`, upload them and (tiled) pack the
    expert weights once; with bf16 experts and down_f16, also make the fp16
    copies of the down weights (moe_convert_bf16_to_f16) once.  Returns
    (layer, row-major layer or None, host inputs or None)."""
    import torch
    import sparse_moe_expert_amd as moe
    from moe_inputs import generate
    from sparse_moe_expert_amd.device import DeviceLayer, pack_expert_weights
    t0 = time.perf_counter()
    inp = generate(cfg)
    log(f"bench: {cfg.name}: generated in {time.perf_counter() - t0:.1f}s; uploading")
    f16 = down_f16 and cfg.expert == "bf16"
    if tiled and not keep_rows:
        lay, rows = DeviceLayer(cfg, inp, tiled=True, down_f16=f16), None
    else:
        rows = DeviceLayer(cfg, inp)
        lay = rows
        if tiled:
            packed = {key: pack_expert_weights(rows.t[key], cfg.expert) for key in EXPERT_KEYS}
            if f16:
                for key in ("w_down", "w_sh_down"):
                    if packed[key].numel():
                        packed[key + "_f16"] = torch.empty(packed[key].shape, dtype=torch.float16,
                                                           device="cuda")
                        moe.moe_convert_bf16_to_f16(packed[key], packed[key + "_f16"],
                                                    packed[key].numel())
            lay = _view(rows, cfg, expert_t=packed, tiled=True)
    torch.cuda.synchronize()
    return lay, (rows if keep_rows else None), (inp if keep_inputs else None)


def stage_dict(r):
    return {k: round(v, 4) for k, v in r["stage"].items()}


def rows_stats(counts):
    return {"max": int(counts.max()), "mean": round(float(counts.mean()), 2),
            "empty": int((counts == 0).sum())}


# ---------------------------------------------------------------- sub-lines

def decode_line(cfg, steps, extras, fused=True):
    """T=256 tokens on the decode-sized workload's own seeded weights: the
    weight-streaming regime, measured against 8 TB/s."""
    import sparse_moe_expert_amd as moe
    lay, rows, _ = load_layer(cfg, keep_rows=extras)
    log(f"bench: {cfg.name}: {steps} steps")
    r = time_layer(lay, steps, 5)
    b = layer_bytes(cfg, r["counts"])
    gbs = b / (r["ms"] / 1e3) / 1e9
    if fused:
        out1 = lay.empty_out()
        msf = time_calls(lambda: moe.moe_layer_forward_fused(
            lay.ccfg, lay.weights, lay.t["x"], out1, None, None, lay.workspace), steps, 5)
        gbf = b / (msf / 1e3) / 1e9
    res = {
        "workload": cfg.name, "ms_per_step": round(r["ms"], 4),
        "ms_per_step_instrumented": round(r["ms_inst"], 4),
        "ms_per_step_events_p10_p50_p90": r["spread"],
        "tokens_per_s": round(cfg.T / (r["ms"] / 1e3), 1),
        "algorithmic_bytes": b, "hbm_GBps": round(gbs, 1),
        "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "tflops": round(cfg.flops() / (r["ms"] / 1e3) / 1e12, 2),
        "stages_ms": stage_dict(r), "experts_touched": int((r["counts"] > 0).sum()),
        "near_tie_tokens": {"selection": r["ties"][0], "slot_order": r["ties"][1]},
    }
    if fused:
        res["fused_single_launch"] = {"ms_per_step": round(msf, 4), "hbm_GBps": round(gbf, 1),
                                      "frac_of_hbm_peak": round(gbf / PEAK_HBM_GBS, 4)}
    if rows is not None:
        msr = time_layer(rows, steps, 5)["ms"]
        g1r = b / (msr / 1e3) / 1e9
        res["row_major_weights"] = {"ms_per_step": round(msr, 4), "hbm_GBps": round(g1r, 1),
                                    "frac_of_hbm_peak": round(g1r / PEAK_HBM_GBS, 4)}
    return res, lay


def workload_line(cfg, steps, warmup):
    """Another configuration of the layer: time, tokens/s, TFLOP/s, its
    algorithmic bytes, the fraction of both roofs, the governing one, its
    gate/up roofline and the near-tie counts of its routing."""
    lay, _, _ = load_layer(cfg)
    log(f"bench: {cfg.name}: {warmup} warmup + {steps} steps")
    r = time_layer(lay, steps, warmup)
    dtype = cfg.expert
    flops = cfg.flops()
    b = layer_bytes(cfg, r["counts"])
    tf = flops / (r["ms"] / 1e3) / 1e12
    gbs = b / (r["ms"] / 1e3) / 1e9
    ridge = PEAK_TFLOPS[dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    res = {
        "workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "S": cfg.S, "k": cfg.k,
        "I": cfg.I, "precision": dtype, "ms_per_step": round(r["ms"], 4),
        "ms_per_step_events_p10_p50_p90": r["spread"],
        "tokens_per_s": round(cfg.T / (r["ms"] / 1e3), 1), "tflops": round(tf, 2),
        "flops_per_step": flops, "algorithmic_bytes": b, "algorithmic_GBps": round(gbs, 1),
        "frac_of_mfma_peak": round(tf / PEAK_TFLOPS[dtype], 4),
        "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "bound": "mfma" if flops / b >= ridge else "hbm",
        "stages_ms": stage_dict(r), "rows_per_expert": rows_stats(r["counts"]),
        "near_tie_tokens": {"selection": r["ties"][0], "slot_order": r["ties"][1]},
        "gate_up_roofline": gate_up_roofline(cfg, r["stage"]["gate_up_gemm"], r["counts"], dtype),
    }
    res["frac_of_governing_roof"] = res["frac_of_mfma_peak" if res["bound"] == "mfma"
                                        else "frac_of_hbm_peak"]
    return res, lay


def ceilings(cfg2, steps):
    """Measured ceilings: a streaming read of 4 GiB with the library's read
    kernel, and the library's prefill GEMMs on one dense expert (E = 1, k = 1,
    no shared expert, T = 16384): the same kernels without gather or ragged
    experts."""
    import torch
    import sparse_moe_expert_amd as moe
    n = 4 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    res = {}
    for blocks in (2048, 8192):
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
        ms = time_calls(lambda: moe.moe_stream_read(buf, n, sink, blocks), 10, 2)
        res[f"stream_read_{blocks}_blocks"] = {"bytes": n, "ms": round(ms, 4),
                                               "GBps": round(n / (ms / 1e3) / 1e9, 1)}
    del buf
    best = max(v["GBps"] for v in res.values())
    res["stream_read_GBps"] = best
    cfg1 = cfg2.with_(name="dense_expert_T16384", E=1, k=1, S=0)
    lay, _, _ = load_layer(cfg1)
    r = time_layer(lay, steps, 3)
    gu = gate_up_flops(cfg1)
    dn = 2.0 * cfg1.T * cfg1.I * cfg1.H
    res["dense_expert_gemm"] = {
        "T": cfg1.T, "H": cfg1.H, "I": cfg1.I,
        "gate_up_ms": round(r["stage"]["gate_up_gemm"], 4),
        "gate_up_tflops": round(gu / (r["stage"]["gate_up_gemm"] / 1e3) / 1e12, 1),
        "down_ms": round(r["stage"]["down_gemm"], 4),
        "down_tflops": round(dn / (r["stage"]["down_gemm"] / 1e3) / 1e12, 1)}
    return res, lay


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


def device_copy(gib=2.0, iters=5):
    """A plain device-to-device copy of `gib` GiB with torch's copy kernel:
    bytes read + written over its event time.  Context for the HBM figures:
    a copy mixes reads and writes half and half."""
    import torch
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    ms = time_calls(lambda: b.copy_(a), iters, 2)
    del a, b
    return {"bytes_per_copy": 2 * n, "ms": round(ms, 4), "GBps": round(2 * n / (ms / 1e3) / 1e9, 1)}


def cpu_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(cfg, inp, n_tokens):
    """The fp64 CPU oracle as it stands, on the first `n_tokens` tokens of the
    same workload, with the BLAS thread pool set to the cores this process may
    use.  Its time includes widening every touched expert's weights to fp64,
    which the oracle does per call."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    cores = cpu_cores()
    tokens = np.arange(min(n_tokens, cfg.T))
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        oracle.layer_forward(cfg, inp, tokens=tokens)
        dt = time.perf_counter() - t0
    return {"value": round(tokens.size / dt, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"first {tokens.size} tokens of {cfg.name} (routing over all {cfg.E} "
                      f"experts, their SwiGLU experts and the shared expert), fp64 numpy, "
                      f"BLAS threads {cores}"}


def _teardown(objs):
    """Release device memory and let the runtime go idle before the
    interpreter exits: drop every device tensor, synchronise, empty torch's
    cache.  A profiler that unloads while tensors and streams are still alive
    at interpreter exit is what this avoids."""
    import torch
    objs.clear()
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload id (default 2: T=16384)")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-decode", action="store_true", help="skip the T=256 line")
    ap.add_argument("--no-workloads", action="store_true", help="skip the T=8192 and fp8 lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the single-launch (cooperative) layer in the T=256 line")
    ap.add_argument("--cpu-tokens", type=int, default=2048)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip ceilings, grouped routing, block, copy and row-major lines")
    ap.add_argument("--weights", choices=("tiled", "rows"), default="tiled",
                    help="expert weight storage of the timed layer (default: packed tiles)")
    ap.add_argument("--no-down-f16", action="store_true",
                    help="no fp16 copies of the bf16 down weights (the large-tile down GEMM "
                         "then converts its bf16 weight fragments in registers)")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="also run one plain device-to-device copy of this many GiB "
                         "(calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU only (asked for --gpus {args.gpus}); "
              "the layer would shard by experts across GPUs, which is not built here.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from moe_inputs import config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    held = []
    cfg = config(args.config)
    tiled = args.weights == "tiled"
    extras = not args.no_extras and args.config == 2
    down_f16 = not args.no_down_f16 and cfg.expert == "bf16"
    lay, lay_rows, inp = load_layer(cfg, tiled=tiled, keep_rows=tiled and extras,
                                    keep_inputs=not args.no_cpu_baseline, down_f16=down_f16)
    held += [lay, lay_rows]

    log(f"bench: {args.warmup} warmup + {args.steps} timed steps")
    r = time_layer(lay, args.steps, args.warmup)
    ms, counts = r["ms"], r["counts"]
    flops = cfg.flops()
    dtype = cfg.expert
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
                   "expert_weights": "tiled16x64B" if tiled else "row_major",
                   "down_weights_fp16_copy": down_f16},
        "tflops": round(flops / (ms / 1e3) / 1e12, 2),
        "frac_of_peak_mfma_whole_step": round(flops / (ms / 1e3) / 1e12 / PEAK_TFLOPS[dtype], 4),
        "ms_per_step_instrumented": round(r["ms_inst"], 4),
        "ms_per_step_events": round(r["ms_ev"], 4),
        "ms_per_step_events_p10_p50_p90": r["spread"],
        "stages_ms": stage_dict(r),
        "rows_per_expert": rows_stats(counts),
        "near_tie_tokens": {"selection": r["ties"][0], "slot_order": r["ties"][1]},
    }
    res["roofline"] = gate_up_roofline(cfg, r["stage"]["gate_up_gemm"], counts, dtype)
    if lay_rows is not None:
        msr = time_layer(lay_rows, args.steps, args.warmup)["ms"]
        res["row_major_weights"] = {"ms_per_step": round(msr, 4),
                                    "tokens_per_s": round(cfg.T / (msr / 1e3), 1),
                                    "down_weights_fp16_copy": False}
    if extras and down_f16:
        lay_nc = _view(lay, cfg, expert_t={"w_down_f16": None, "w_sh_down_f16": None})
        rn = time_layer(lay_nc, args.steps, args.warmup)
        res["without_down_f16_copy"] = {"ms_per_step": round(rn["ms"], 4),
                                        "tokens_per_s": round(cfg.T / (rn["ms"] / 1e3), 1),
                                        "stages_ms": stage_dict(rn)}
        del lay_nc
    if extras:
        log("bench: grouped routing and block forward")
        res["grouped_routing"] = grouped_routing(lay, cfg)
        res["block"] = block_forward(lay, cfg, min(args.steps, 10))
    if args.config == 2:
        # the other workloads load their own weights; the T=16384 layer's
        # weights stay only if the CPU baseline still needs its host inputs
        held.clear()
        del lay, lay_rows
        gc.collect()
        torch.cuda.empty_cache()
        if not args.no_decode:
            res["decode_T256"], l1 = decode_line(config(1), args.decode_steps, extras,
                                                 fused=not args.no_fused)
            del l1
            gc.collect()
            torch.cuda.empty_cache()
        if not args.no_workloads:
            for cid, key in ((3, "skewed_T8192"), (4, "fp8_T4096")):
                res[key], lw = workload_line(config(cid), args.steps, args.warmup)
                del lw
                gc.collect()
                torch.cuda.empty_cache()
        if extras:
            log("bench: measured ceilings and device copy")
            res["ceilings"], lc = ceilings(cfg, min(args.steps, 10))
            del lc
            gc.collect()
            torch.cuda.empty_cache()
            res["device_copy"] = device_copy()
            res["ceilings"]["decode_T256_frac_of_read_ceiling"] = (
                round(res["decode_T256"]["hbm_GBps"] / res["ceilings"]["stream_read_GBps"], 4)
                if "decode_T256" in res else None)

    if args.calib_copy_gib > 0:
        n = int(args.calib_copy_gib * (1 << 30))
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        res["calib_copy_bytes"] = n
        del a, b

    if not args.no_cpu_baseline:
        log(f"bench: CPU oracle on {args.cpu_tokens} tokens")
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_tokens)
    else:
        res["cpu_baseline"] = None

    _teardown(held)
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
        s_sh_gate_up=t.get("s_sh_gate_up"), s_sh_down=t.get("s_sh_down"),
        w_down_f16=t.get("w_down_f16"), w_sh_down_f16=t.get("w_sh_down_f16"))
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
