"""Decode-step throughput of the LLA latent-cache kernels on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload capacity]

Default workload ("capacity"): a 24-layer looped model with H=16 heads of width 128, T=4 loops,
per-head latent ranks r_k = r_v = 24 (21.3x compression), B=768 sequences at 4096 cached tokens,
bf16 latents: 116 GB of latent cache resident in HBM, filled from a seeded device generator (the
paper's capacity test also fabricates the decode cache; Section 7).

One step = one decode token for every sequence: for each loop t and layer l, one
lla_attend_decode read of that layer's latents (with the token's own loop-t K/V), then one
lla_encode per layer folding the token's T per-loop K/V into slot N. Sequence lengths stay at N,
so every step reads exactly N latents per (sequence, head). Inputs are resident before timing.

Prints one JSON line. value = tokens/s = B / step time. roofline: the decode kernel's average
launch time from HIP events on its stream, latent bytes per launch / that time, against 8 TB/s.
cpu_baseline: the CPU oracle (explicit reconstruction, float64) timed on a bounded sample of the
same step on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "LLA decode-attn tokens/s + latent HBM GB/s (% of peak), bf16, 4k ctx, 1 GPU"
# the sources the per-head decode kernel is compiled from (the measured traffic is valid for them)
DECODE_SRC = [os.path.join(ROOT, "decode_attention_lla_amd", "csrc", f)
              for f in ("decode.hip", "lla_device.h", "lla_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partial_capacity_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="capacity",
                    choices=["capacity", "ouro_layer", "deep_loop", "lla2d"])
    ap.add_argument("--layers", type=int, default=None, help="override the layer count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 4 GiB device copy (scale reference for HBM counters)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the LLA-2D decode and chunked-prefill figures")
    ap.add_argument("--only-prefill", action="store_true",
                    help="measure only the LLA-2D chunked prefill (for profiling)")
    ap.add_argument("--only-eviction", action="store_true",
                    help="measure only the gather-indexed (token-eviction) decode read")
    ap.add_argument("--only-low-bit", action="store_true",
                    help="measure only the capacity step with low-bit (E4M3 + scale) latent rows")
    ap.add_argument("--only-rope", action="store_true",
                    help="measure only the decode read with the decoupled rotary branch")
    ap.add_argument("--only-long-context", action="store_true",
                    help="measure only the 262k-token absorbed read against reconstruct-then-attend")
    ap.add_argument("--only-lla2d", action="store_true",
                    help="measure only the LLA-2D decode step (the MFMA read and its encode)")
    ap.add_argument("--only-small", action="store_true",
                    help="measure only the one-layer Ouro-shaped and deep-recurrence decode steps")
    return ap.parse_args()


def source_sha(paths):
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def load_traffic():
    """Per-launch HBM bytes of the decode kernel from committed counter runs, if still valid."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("decode_src_sha256_16") != source_sha(DECODE_SRC):
        return None  # the kernel changed since the counters were taken
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the LLA latent-cache path runs on a single MI355X "
              "here (the library has no multi-GPU path); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_attention_lla_amd import lla, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lla.library()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    if args.only_prefill:
        print(json.dumps({"lla2d_prefill": lla2d_prefill(args)}), flush=True)
        return
    if args.only_eviction:
        print(json.dumps({"eviction_decode": eviction_decode(args)}), flush=True)
        return
    if args.only_low_bit:
        print(json.dumps({"low_bit_capacity": low_bit_capacity(args, None),
                          "low_bit_deep_loop": low_bit_deep_loop(args),
                          "low_bit_lla2d": low_bit_lla2d(args)}), flush=True)
        return
    if args.only_rope:
        print(json.dumps({"rope_decode": rope_decode(args)}), flush=True)
        return
    if args.only_lla2d:
        print(json.dumps({"lla2d_decode": lla2d_decode(args)}), flush=True)
        return
    if args.only_long_context:
        print(json.dumps({"long_context_262k": long_context(args)}), flush=True)
        return
    if args.only_small:
        print(json.dumps({"ouro_layer": per_head_layer(args, "ouro_layer"),
                          "deep_loop": per_head_layer(args, "deep_loop")}), flush=True)
        return
    s = synth.CASES[args.workload]
    D = args.layers or s.D
    B, H, d, T, rk, rv, N = s.B, s.H, s.d, s.T, s.r_k, s.r_v, s.N
    n_max = N + 1
    bf = torch.bfloat16
    two_d = s.variant == "2d"
    desc = lla.make_desc(lla.LLA_2D if two_d else lla.LLA_PER_HEAD, lla.LLA_BF16, H, d, T, rk, rv, n_max)
    print(f"# workload {s.name}: D={D} H={H} d={d} T={T} r=({rk},{rv}) B={B} N={N}", file=sys.stderr, flush=True)

    # ---- resident inputs --------------------------------------------------------------------
    t0 = time.time()
    zk, zv, Wk, Wv, Ek, Ev = [], [], [], [], [], []
    zsk = (B, n_max, rk) if two_d else (B, H, n_max, rk)
    zsv = (B, n_max, rv) if two_d else (B, H, n_max, rv)
    for l in range(D):
        zk.append(synth.device_normal_(torch.empty(zsk, dtype=bf, device="cuda"),
                                       synth.seed(s.case, synth.SEED_ZK, l)))
        zv.append(synth.device_normal_(torch.empty(zsv, dtype=bf, device="cuda"),
                                       synth.seed(s.case, synth.SEED_ZV, l)))
        if two_d:
            wk = synth.orthonormal_W_2d(T, H, d, rk, synth.seed(s.case, synth.SEED_WK, l), "bf16")
            wv = synth.orthonormal_W_2d(T, H, d, rv, synth.seed(s.case, synth.SEED_WV, l), "bf16")
            ek, ev = synth.pinv_E_from_W_2d(wk, "bf16"), synth.pinv_E_from_W_2d(wv, "bf16")
        else:
            wk = synth.orthonormal_W(T, H, d, rk, synth.seed(s.case, synth.SEED_WK, l), "bf16")
            wv = synth.orthonormal_W(T, H, d, rv, synth.seed(s.case, synth.SEED_WV, l), "bf16")
            ek, ev = synth.pinv_E_from_W(wk, "bf16"), synth.pinv_E_from_W(wv, "bf16")
        Wk.append(torch.from_numpy(wk).to(bf).cuda())
        Wv.append(torch.from_numpy(wv).to(bf).cuda())
        Ek.append(torch.from_numpy(ek).to(bf).cuda())
        Ev.append(torch.from_numpy(ev).to(bf).cuda())
    q = synth.device_normal_(torch.empty(T, D, B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_Q))
    kself = synth.device_normal_(torch.empty(T, D, B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF))
    vself = synth.device_normal_(torch.empty(T, D, B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF) + 1)
    xk = synth.device_normal_(torch.empty(D, B, 1, T, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_XK))
    xv = synth.device_normal_(torch.empty(D, B, 1, T, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_XV))
    out = torch.empty(T, D, B, H, d, dtype=bf, device="cuda")
    lens = torch.full((B,), N, dtype=torch.int32, device="cuda")
    ws = lla.workspace(desc, B, 1)
    torch.cuda.synchronize()
    resident = sum(t.numel() * t.element_size() for t in zk + zv)
    print(f"# resident latents {resident / 1e9:.2f} GB, filled in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    ev = {}

    def step(record=None):
        for t in range(T):
            for l in range(D):
                if record is not None:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                lla.lla_attend_decode(desc, B, t, q[t, l], zk[l], zv[l], lens, Wk[l], Wv[l], None, None,
                                      kself[t, l], vself[t, l], out[t, l], None, ws, stream)
                if record is not None:
                    e1 = torch.cuda.Event(enable_timing=True)
                    e1.record(stream)
                    record.append((e0, e1))
        for l in range(D):
            lla.lla_encode(desc, B, 1, xk[l], xv[l], Ek[l], Ev[l], None, None, lens, zk[l], zv[l], stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region -------------------------------------------------------------------------
    pairs = []
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(pairs)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    launch_ms = np.array([a.elapsed_time(b) for a, b in pairs])
    avg_launch_ms = float(np.mean(launch_ms))
    print(f"# {args.steps} steps: {ms_step:.3f} ms/step; decode launch avg {avg_launch_ms * 1e3:.1f} us "
          f"(min {launch_ms.min() * 1e3:.1f}, max {launch_ms.max() * 1e3:.1f})", file=sys.stderr, flush=True)

    if args.copy_probe:
        a = torch.empty(2 ** 31, dtype=bf, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    copy_gbs = device_copy_ceiling(stream)

    tokens_per_s = B / (ms_step / 1e3)
    H_lat = 1 if two_d else H
    latent_bytes = B * H_lat * N * (rk + rv) * 2  # per read: every cached latent pair, once
    # everything else a read must move: q, the self K/V and out (B*H*d each), W^K_t and W^V_t, the
    # lengths, and the split partials written and read back when the plan splits the tokens
    other_bytes = 4 * B * H * d * 2 + H * d * (rk + rv) * 2 + B * 4 + 2 * lla.lla_workspace_bytes(desc, B, 1)
    achieved = latent_bytes / (avg_launch_ms / 1e3) / 1e9
    traffic = load_traffic() if args.workload == "capacity" and D == s.D else None

    # ---- CPU oracle baseline --------------------------------------------------------------------
    cpu = None
    if two_d:
        # MFMA work per read: scores and latent-V products for every (sequence, head, token)
        flops = 2.0 * B * H * N * (rk + rv)
        res_extra = {"mfma_tflops": round(flops / (avg_launch_ms / 1e3) / 1e12, 2),
                     "mfma_util_bf16_dense": round(flops / (avg_launch_ms / 1e3) / 2.5e15, 4)}
    else:
        res_extra = {}
    if not args.no_cpu_baseline and not two_d:
        cpu = cpu_baseline(args, s, D, zk, zv, Wk, Wv, Ek, Ev, q, kself, vself, xk, xv, lens)

    extras = None
    if not args.no_extras and args.workload == "capacity":
        del zk, zv, q, kself, vself, xk, xv, out
        torch.cuda.empty_cache()
        extras = {"ouro_layer": per_head_layer(args, "ouro_layer"),
                  "deep_loop": per_head_layer(args, "deep_loop"),
                  "lla2d_decode": lla2d_decode(args), "lla2d_prefill": lla2d_prefill(args),
                  "eviction_decode": eviction_decode(args),
                  "low_bit_capacity": low_bit_capacity(args, tokens_per_s),
                  "low_bit_deep_loop": low_bit_deep_loop(args),
                  "low_bit_lla2d": low_bit_lla2d(args),
                  "long_context_262k": long_context(args),
                  "rope_decode": rope_decode(args)}

    res = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{s.name}: {D} layers, H={H}, d_head={d}, T={T}, r_k={rk}, r_v={rv}, "
                        f"B={B}, N={N} cached tokens, bf16 latents",
            "layers": D, "batch": B, "context": N, "heads": H, "d_head": d, "loops": T,
            "r_k": rk, "r_v": rv, "variant": s.variant,
            "compression": round(2 * T * d * (H if two_d else 1) / (rk + rv), 2),
            "resident_latent_bytes": resident,
            "reads_per_step": D * T, "encodes_per_step": D,
        },
        "latent_GBps": round(achieved, 1),
        "latent_frac_of_peak": round(achieved / HBM_PEAK_GBS, 4),
        "total_GBps": round((latent_bytes + other_bytes) / (avg_launch_ms / 1e3) / 1e9, 1),
        "total_bytes_per_read": latent_bytes + other_bytes,
        "device_copy_GBps": round(copy_gbs, 1),
        "device_copy_frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": (f"decode2d qproj + partial<{rk},{rv}> (MFMA) + combine per read" if two_d else
                       f"decode_partial_kernel<BF16,{rk},{rv}> (one launch per read)"),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": latent_bytes,
            "avg_launch_us": round(avg_launch_ms * 1e3, 2),
        },
        "cpu_baseline": cpu,
    }
    res.update(res_extra)
    if cpu is not None:
        res["gpu_over_cpu"] = round(tokens_per_s / cpu["value"], 1)
    if extras is not None:
        res["extras"] = extras
    print(json.dumps(res), flush=True)


def _timed(fn, steps, warmup):
    """HIP-event time of fn() per call on the current stream (ms), after warm-up calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def per_head_layer(args, name):
    """Decode step of a one-layer per-head workload at full size: T loop reads (each with the
    token's own loop-t K/V, its own W^K_t/W^V_t), then the encode of the new token into slot N.
    ouro_layer: H=16, d=128, T=4, r=32/32, B=32, N=4096 (one Ouro-1.4B-shaped layer, 16x);
    deep_loop: H=40, d=96, T=32, r=96/96, B=64, N=4096 (square 96x96 factors, 32x).
    read_us is the time of a step's T back-to-back reads divided by T (HIP events on the launch
    stream before the first read and after the last, so no event sits between two reads)."""
    import torch
    from decode_attention_lla_amd import lla, synth
    s = synth.CASES[name]
    B, H, d, T, rk, rv, N = s.B, s.H, s.d, s.T, s.r_k, s.r_v, s.N
    n_max = N + 1
    bf = torch.bfloat16
    desc = lla.make_desc(lla.LLA_PER_HEAD, lla.LLA_BF16, H, d, T, rk, rv, n_max)
    zk = synth.device_normal_(torch.empty(B, H, n_max, rk, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZK))
    zv = synth.device_normal_(torch.empty(B, H, n_max, rv, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZV))
    wk = synth.orthonormal_W(T, H, d, rk, synth.seed(s.case, synth.SEED_WK), "bf16")
    wv = synth.orthonormal_W(T, H, d, rv, synth.seed(s.case, synth.SEED_WV), "bf16")
    Wk, Wv = torch.from_numpy(wk).to(bf).cuda(), torch.from_numpy(wv).to(bf).cuda()
    Ek = torch.from_numpy(synth.pinv_E_from_W(wk, "bf16")).to(bf).cuda()
    Ev = torch.from_numpy(synth.pinv_E_from_W(wv, "bf16")).to(bf).cuda()
    q = synth.device_normal_(torch.empty(T, B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_Q))
    ks = synth.device_normal_(torch.empty(T, B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF))
    vs = synth.device_normal_(torch.empty(T, B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF) + 1)
    x = synth.device_normal_(torch.empty(2, B, 1, T, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_XK))
    out = torch.empty(T, B, H, d, dtype=bf, device="cuda")
    lens = torch.full((B,), N, dtype=torch.int32, device="cuda")
    ws = lla.workspace(desc, B, 1)
    stream = torch.cuda.current_stream()
    pairs = []

    def step(record=False):
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        for t in range(T):
            lla.lla_attend_decode(desc, B, t, q[t], zk, zv, lens, Wk, Wv, None, None, ks[t], vs[t],
                                  out[t], None, ws, stream)
        if record:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record(stream)
            pairs.append((e0, e1))
        lla.lla_encode(desc, B, 1, x[0], x[1], Ek, Ev, None, None, lens, zk, zv, stream)

    steps = 20 if T <= 4 else 5
    ms_step = _timed(step, steps, 2)
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    ms_read = float(np.mean([a.elapsed_time(b) for a, b in pairs])) / T
    latent = B * H * N * (rk + rv) * 2
    # A layer's loop reads re-stream the same latents back to back; when they are about the size of
    # the 256 MB last-level cache, part of a read comes from it. The same read after a 1 GiB
    # read-only sweep of another buffer shows the cold figure.
    # Both are one read timed alone (events around it), after the same read or after the sweep.
    single = None
    if latent <= 2 ** 30:
        sweep = torch.zeros(2 ** 28, dtype=torch.float32, device="cuda")

        def read0():
            lla.lla_attend_decode(desc, B, 0, q[0], zk, zv, lens, Wk, Wv, None, None, ks[0], vs[0], out[0],
                                  None, ws, stream)

        def one(before):
            ts = []
            for _ in range(20):
                before()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                read0()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            return float(np.median(ts)) * 1e3

        single = (one(read0), one(lambda: sweep.sum()))
        del sweep
    res = {"workload": f"{name}: 1 layer, H={H}, d_head={d}, T={T}, r_k={rk}, r_v={rv}, B={B}, "
                       f"N={N}, bf16",
           "tokens_per_s": round(B / (ms_step / 1e3), 1), "ms_per_step": round(ms_step, 4),
           "read_us": round(ms_read * 1e3, 2),
           "latent_GBps": round(latent / (ms_read / 1e3) / 1e9, 1),
           "latent_frac_of_peak": round(latent / (ms_read / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
           "latent_bytes_per_read": latent}
    if single is not None:
        res["single_read_us_after_same_read"] = round(single[0], 2)
        res["single_read_us_after_cache_sweep"] = round(single[1], 2)
        res["latent_frac_of_peak_after_cache_sweep"] = round(latent / (single[1] / 1e6) / 1e9 / HBM_PEAK_GBS, 4)
    del zk, zv, x, q, ks, vs, out, ws
    torch.cuda.empty_cache()
    return res


def lla2d_decode(args):
    """LLA-2D decode step (H=16, d=128, T=4, r=256/256, B=128, N=8192): 4 loop reads + encode."""
    import torch
    from decode_attention_lla_amd import lla, synth
    s = synth.CASES["lla2d"]
    B, H, d, T, r, N = s.B, s.H, s.d, s.T, s.r_k, s.N
    n_max = N + 1
    bf = torch.bfloat16
    desc = lla.make_desc(lla.LLA_2D, lla.LLA_BF16, H, d, T, r, r, n_max)
    zk = synth.device_normal_(torch.empty(B, n_max, r, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZK))
    zv = synth.device_normal_(torch.empty(B, n_max, r, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZV))
    wk = synth.orthonormal_W_2d(T, H, d, r, synth.seed(s.case, synth.SEED_WK), "bf16")
    wv = synth.orthonormal_W_2d(T, H, d, r, synth.seed(s.case, synth.SEED_WV), "bf16")
    Wk, Wv = torch.from_numpy(wk).to(bf).cuda(), torch.from_numpy(wv).to(bf).cuda()
    Ek = torch.from_numpy(synth.pinv_E_from_W_2d(wk, "bf16")).to(bf).cuda()
    Ev = torch.from_numpy(synth.pinv_E_from_W_2d(wv, "bf16")).to(bf).cuda()
    q = synth.device_normal_(torch.empty(T, B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_Q))
    ks = synth.device_normal_(torch.empty(T, B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF))
    vs = synth.device_normal_(torch.empty(T, B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF) + 1)
    x = synth.device_normal_(torch.empty(2, B, 1, T, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_XK))
    out = torch.empty(T, B, H, d, dtype=bf, device="cuda")
    lens = torch.full((B,), N, dtype=torch.int32, device="cuda")
    ws = lla.workspace(desc, B, 1)

    def read(t):
        lla.lla_attend_decode(desc, B, t, q[t], zk, zv, lens, Wk, Wv, None, None, ks[t], vs[t], out[t], None, ws)

    def step():
        for t in range(T):
            read(t)
        lla.lla_encode(desc, B, 1, x[0], x[1], Ek, Ev, None, None, lens, zk, zv)

    ms_read = _timed(lambda: read(0), 20, 3)
    ms_step = _timed(step, 10, 2)
    latent = B * N * 2 * r * 2
    flops = 2.0 * B * H * N * 2 * r
    return {"workload": f"lla2d: H={H}, d_head={d}, T={T}, r_k=r_v={r}, B={B}, N={N}, bf16",
            "tokens_per_s": round(B / (ms_step / 1e3), 1), "ms_per_step": round(ms_step, 4),
            "read_us": round(ms_read * 1e3, 2),
            "latent_GBps": round(latent / (ms_read / 1e3) / 1e9, 1),
            "latent_frac_of_peak": round(latent / (ms_read / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_TFLOPs": round(flops / (ms_read / 1e3) / 1e12, 2),
            "mfma_util_bf16_dense": round(flops / (ms_read / 1e3) / 2.5e15, 4)}


def eviction_decode(args):
    """Token eviction composed with LLA at the capacity shape (one layer: B=768, H=16, d=128, T=4,
    r=24/24, 4096 cached tokens): each read attends a 1024-slot StreamingLLM list (4 sinks + the
    1020 most recent tokens) through lla_attend_decode_gather, beside the contiguous read of a
    1024-token cache of the same shape and a read of 1024 random slots (H2O-like scattered rows)."""
    import torch
    from decode_attention_lla_amd import lla, synth
    s = synth.CASES["capacity"]
    B, H, d, T, r, N = s.B, s.H, s.d, s.T, s.r_k, s.N
    keep = 1024
    n_max = N + 1
    bf = torch.bfloat16
    desc = lla.make_desc(lla.LLA_PER_HEAD, lla.LLA_BF16, H, d, T, r, r, n_max)
    zk = synth.device_normal_(torch.empty(B, H, n_max, r, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZK))
    zv = synth.device_normal_(torch.empty(B, H, n_max, r, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZV))
    Wk = torch.from_numpy(synth.orthonormal_W(T, H, d, r, synth.seed(s.case, synth.SEED_WK), "bf16")).to(bf).cuda()
    Wv = torch.from_numpy(synth.orthonormal_W(T, H, d, r, synth.seed(s.case, synth.SEED_WV), "bf16")).to(bf).cuda()
    q = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_Q))
    ks = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF))
    vs = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF) + 1)
    out = torch.empty(B, H, d, dtype=bf, device="cuda")
    sink, window = 4, keep - 4
    row = torch.cat([torch.arange(sink), torch.arange(N - window, N)]).to(torch.int32)
    slots = row.repeat(B, 1).contiguous().cuda()
    ws = lla.gather_workspace(desc, B, keep)
    lens = torch.full((B,), keep, dtype=torch.int32, device="cuda")
    desc_c = lla.make_desc(lla.LLA_PER_HEAD, lla.LLA_BF16, H, d, T, r, r, keep)
    zk_c, zv_c = zk[:, :, :keep].contiguous(), zv[:, :, :keep].contiguous()
    ws_c = lla.workspace(desc_c, B, 1)

    def gathered():
        lla.lla_attend_decode_gather(desc, B, 0, q, zk, zv, slots, None, Wk, Wv, None, None, ks, vs,
                                     out, None, ws)

    def contiguous():
        lla.lla_attend_decode(desc_c, B, 0, q, zk_c, zv_c, lens, Wk, Wv, None, None, ks, vs, out,
                              None, ws_c)

    rnd = torch.from_numpy(synth.random_slots(B, keep, N, synth.seed(s.case, synth.SEED_SLOTS))).cuda()

    # the same subsets listed in slot order (the read's result does not depend on the order)
    rnd_sorted = torch.sort(rnd, dim=1).values.contiguous()

    def gathered_random(lst):
        lla.lla_attend_decode_gather(desc, B, 0, q, zk, zv, lst, None, Wk, Wv, None, None, ks, vs,
                                     out, None, ws)

    ms_g = _timed(gathered, 20, 3)
    ms_r = _timed(lambda: gathered_random(rnd), 20, 3)
    ms_rs = _timed(lambda: gathered_random(rnd_sorted), 20, 3)
    ms_c = _timed(contiguous, 20, 3)
    kept_bytes = B * H * keep * 2 * r * 2
    return {"workload": f"capacity layer read through a {keep}-slot sink {sink} + window {window} "
                        f"list of a {N}-token cache: H={H}, d_head={d}, r_k=r_v={r}, B={B}, bf16",
            "read_us": round(ms_g * 1e3, 2),
            "kept_latent_GBps": round(kept_bytes / (ms_g / 1e3) / 1e9, 1),
            "kept_latent_frac_of_peak": round(kept_bytes / (ms_g / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "contiguous_read_of_the_same_count_us": round(ms_c * 1e3, 2),
            "random_1024_of_4096_read_us": round(ms_r * 1e3, 2),
            "random_1024_of_4096_sorted_by_slot_read_us": round(ms_rs * 1e3, 2),
            "cache_bytes_per_sequence_and_layer": {"cached": H * n_max * 2 * r * 2,
                                                   "read": H * keep * 2 * r * 2}}


def low_bit_capacity(args, bf16_tokens_per_s):
    """The capacity step (24 layers, H=16, d=128, T=4, r=24/24, B=768, 4096 cached tokens) with
    low-bit latent rows (24 codes + a float32 scale, 32 bytes per row instead of 48): 96 decode
    reads, then per layer an encode of the new token into a bf16 staging row and its quantisation
    into slot N. E4M3 codes (LLA_BF16_Q8) at the top level, int8 codes (LLA_BF16_I8) under "int8";
    each form's caches are built and freed in turn."""
    import torch
    from decode_attention_lla_amd import lla, synth
    s = synth.CASES["capacity"]
    D, B, H, d, T, r, N = s.D, s.B, s.H, s.d, s.T, s.r_k, s.N
    n_max = N + 1
    bf = torch.bfloat16

    def run(dtype):
        desc = lla.make_desc(lla.LLA_PER_HEAD, dtype, H, d, T, r, r, n_max)
        desc_stage = lla.make_desc(lla.LLA_PER_HEAD, lla.LLA_BF16, H, d, T, r, r, 1)
        rb = lla.lla_latent_row_bytes(dtype, r)
        zero = torch.zeros(B, dtype=torch.int32, device="cuda")
        stage = torch.empty(B, H, n_max, r, dtype=bf, device="cuda")
        stage_v = torch.empty_like(stage)
        ck, cv, Wk, Wv, Ek, Ev = [], [], [], [], [], []
        for l in range(D):
            synth.device_normal_(stage, synth.seed(s.case, synth.SEED_ZK, l))
            synth.device_normal_(stage_v, synth.seed(s.case, synth.SEED_ZV, l))
            ck.append(torch.empty(B, H, n_max, rb, dtype=torch.uint8, device="cuda"))
            cv.append(torch.empty(B, H, n_max, rb, dtype=torch.uint8, device="cuda"))
            lla.lla_quantize_latents(desc, B, n_max, stage, stage_v, zero, ck[l], cv[l])
            wk = synth.orthonormal_W(T, H, d, r, synth.seed(s.case, synth.SEED_WK, l), "bf16")
            wv = synth.orthonormal_W(T, H, d, r, synth.seed(s.case, synth.SEED_WV, l), "bf16")
            Wk.append(torch.from_numpy(wk).to(bf).cuda())
            Wv.append(torch.from_numpy(wv).to(bf).cuda())
            Ek.append(torch.from_numpy(synth.pinv_E_from_W(wk, "bf16")).to(bf).cuda())
            Ev.append(torch.from_numpy(synth.pinv_E_from_W(wv, "bf16")).to(bf).cuda())
        del stage, stage_v
        torch.cuda.empty_cache()
        q = synth.device_normal_(torch.empty(T, D, B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_Q))
        kself = synth.device_normal_(torch.empty(T, D, B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF))
        vself = synth.device_normal_(torch.empty(T, D, B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF) + 1)
        xk = synth.device_normal_(torch.empty(D, B, 1, T, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_XK))
        xv = synth.device_normal_(torch.empty(D, B, 1, T, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_XV))
        sk = torch.empty(B, H, 1, r, dtype=bf, device="cuda")
        sv = torch.empty_like(sk)
        out = torch.empty(B, H, d, dtype=bf, device="cuda")
        lens = torch.full((B,), N, dtype=torch.int32, device="cuda")
        ws = lla.workspace(desc, B, 1)
        stream = torch.cuda.current_stream()

        def read(t, l):
            lla.lla_attend_decode(desc, B, t, q[t, l], ck[l], cv[l], lens, Wk[l], Wv[l], None, None,
                                  kself[t, l], vself[t, l], out, None, ws, stream)

        def step():
            for t in range(T):
                for l in range(D):
                    read(t, l)
            for l in range(D):
                lla.lla_encode(desc_stage, B, 1, xk[l], xv[l], Ek[l], Ev[l], None, None, zero, sk, sv, stream)
                lla.lla_quantize_latents(desc, B, 1, sk, sv, lens, ck[l], cv[l], stream)

        ms_step = _timed(step, max(3, args.steps // 4), 1)
        ms_read = _timed(lambda: read(0, 0), 20, 3)
        row_bytes = B * H * N * 2 * rb
        res = {"tokens_per_s": round(B / (ms_step / 1e3), 1), "ms_per_step": round(ms_step, 4),
               "read_us": round(ms_read * 1e3, 2),
               "row_GBps": round(row_bytes / (ms_read / 1e3) / 1e9, 1),
               "row_frac_of_peak": round(row_bytes / (ms_read / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
               "resident_latent_bytes": sum(t.numel() for t in ck + cv)}
        if bf16_tokens_per_s:
            res["speedup_vs_bf16_latents"] = round(B / (ms_step / 1e3) / bf16_tokens_per_s, 3)
        del ck, cv
        torch.cuda.empty_cache()
        return res, rb

    res, rb = run(lla.LLA_BF16_Q8)
    res = {"workload": f"capacity with low-bit latents: {D} layers, H={H}, d_head={d}, T={T}, "
                       f"r_k=r_v={r}, B={B}, N={N}; {rb}-byte rows (E4M3 codes + float32 scale; "
                       f"int8: int8 codes + float32 scale)", **res}
    res["int8"] = run(lla.LLA_BF16_I8)[0]
    return res


def low_bit_deep_loop(args):
    """One decode read of the deep-recurrence layer (H=40, d=96, r=96/96, B=64, 4096 cached tokens)
    with low-bit rows (96 codes + a float32 scale in 112 bytes, read 4 lanes x 28 bytes per row)
    beside the same read on bf16 latents (192-byte rows). E4M3 codes at the top level, int8 codes
    under "int8"."""
    import torch
    from decode_attention_lla_amd import lla, synth
    s = synth.CASES["deep_loop"]
    B, H, d, T, r, N = s.B, s.H, s.d, s.T, s.r_k, s.N
    n_max = N + 1
    bf = torch.bfloat16
    zk = synth.device_normal_(torch.empty(B, H, n_max, r, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZK))
    zv = synth.device_normal_(torch.empty(B, H, n_max, r, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZV))
    Wk = torch.from_numpy(synth.orthonormal_W(T, H, d, r, synth.seed(s.case, synth.SEED_WK), "bf16")).to(bf).cuda()
    Wv = torch.from_numpy(synth.orthonormal_W(T, H, d, r, synth.seed(s.case, synth.SEED_WV), "bf16")).to(bf).cuda()
    q = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_Q))
    ks = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF))
    vs = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF) + 1)
    out = torch.empty(B, H, d, dtype=bf, device="cuda")
    lens = torch.full((B,), N, dtype=torch.int32, device="cuda")
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")

    def timed_read(desc, ck, cv):
        ws = lla.workspace(desc, B, 1)
        return _timed(lambda: lla.lla_attend_decode(desc, B, 0, q, ck, cv, lens, Wk, Wv, None, None,
                                                    ks, vs, out, None, ws), 20, 3)

    ms_bf16 = timed_read(lla.make_desc(lla.LLA_PER_HEAD, lla.LLA_BF16, H, d, T, r, r, n_max), zk, zv)
    rb = lla.lla_latent_row_bytes(lla.LLA_BF16_Q8, r)
    ck = torch.empty(B, H, n_max, rb, dtype=torch.uint8, device="cuda")
    cv = torch.empty_like(ck)
    res = {"workload": f"deep_loop read with low-bit latents: H={H}, d_head={d}, r_k=r_v={r}, B={B}, "
                       f"N={N}; {rb}-byte rows (codes + float32 scale) vs {2 * r}-byte bf16 rows",
           "bf16_read_us": round(ms_bf16 * 1e3, 2)}
    for key, dtype in (("e4m3", lla.LLA_BF16_Q8), ("int8", lla.LLA_BF16_I8)):
        desc = lla.make_desc(lla.LLA_PER_HEAD, dtype, H, d, T, r, r, n_max)
        lla.lla_quantize_latents(desc, B, n_max, zk, zv, zero, ck, cv)
        ms = timed_read(desc, ck, cv)
        row_bytes = B * H * N * 2 * rb
        sub = {"read_us": round(ms * 1e3, 2),
               "row_GBps": round(row_bytes / (ms / 1e3) / 1e9, 1),
               "row_frac_of_peak": round(row_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
               "speedup_vs_bf16_read": round(ms_bf16 / ms, 3)}
        if key == "e4m3":
            res.update(sub)
        else:
            res["int8"] = sub
    del zk, zv, ck, cv
    torch.cuda.empty_cache()
    return res


def low_bit_lla2d(args):
    """One LLA-2D decode read (H=16, d=128, r=256/256, B=128, 8192 cached tokens) on the MFMA path
    with low-bit rows (256 codes + a float32 scale in 272 bytes; codes converted to bf16 on the way
    to the MFMA) beside the same read on bf16 latents (512-byte rows). E4M3 codes at the top level,
    int8 codes under "int8"."""
    import torch
    from decode_attention_lla_amd import lla, synth
    s = synth.CASES["lla2d"]
    B, H, d, T, r, N = s.B, s.H, s.d, s.T, s.r_k, s.N
    n_max = N + 1
    bf = torch.bfloat16
    zk = synth.device_normal_(torch.empty(B, n_max, r, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZK))
    zv = synth.device_normal_(torch.empty(B, n_max, r, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZV))
    Wk = torch.from_numpy(synth.orthonormal_W_2d(T, H, d, r, synth.seed(s.case, synth.SEED_WK), "bf16")).to(bf).cuda()
    Wv = torch.from_numpy(synth.orthonormal_W_2d(T, H, d, r, synth.seed(s.case, synth.SEED_WV), "bf16")).to(bf).cuda()
    q = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_Q))
    ks = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF))
    vs = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF) + 1)
    out = torch.empty(B, H, d, dtype=bf, device="cuda")
    lens = torch.full((B,), N, dtype=torch.int32, device="cuda")
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")

    def timed_read(desc, ck, cv):
        ws = lla.workspace(desc, B, 1)
        return _timed(lambda: lla.lla_attend_decode(desc, B, 0, q, ck, cv, lens, Wk, Wv, None, None,
                                                    ks, vs, out, None, ws), 20, 3)

    ms_bf16 = timed_read(lla.make_desc(lla.LLA_2D, lla.LLA_BF16, H, d, T, r, r, n_max), zk, zv)
    rb = lla.lla_latent_row_bytes(lla.LLA_BF16_Q8, r)
    ck = torch.empty(B, n_max, rb, dtype=torch.uint8, device="cuda")
    cv = torch.empty_like(ck)
    res = {"workload": f"LLA-2D read with low-bit latents on MFMA: H={H}, d_head={d}, r_k=r_v={r}, B={B}, "
                       f"N={N}; {rb}-byte rows (codes + float32 scale) vs {2 * r}-byte bf16 rows",
           "bf16_read_us": round(ms_bf16 * 1e3, 2)}
    for key, dtype in (("e4m3", lla.LLA_BF16_Q8), ("int8", lla.LLA_BF16_I8)):
        desc = lla.make_desc(lla.LLA_2D, dtype, H, d, T, r, r, n_max)
        lla.lla_quantize_latents(desc, B, n_max, zk, zv, zero, ck, cv)
        ms = timed_read(desc, ck, cv)
        row_bytes = B * N * 2 * rb
        sub = {"read_us": round(ms * 1e3, 2),
               "row_GBps": round(row_bytes / (ms / 1e3) / 1e9, 1),
               "row_frac_of_peak": round(row_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
               "speedup_vs_bf16_read": round(ms_bf16 / ms, 3)}
        if key == "e4m3":
            res.update(sub)
        else:
            res["int8"] = sub
    del zk, zv, ck, cv
    torch.cuda.empty_cache()
    return res


def rope_decode(args):
    """The decoupled rotary branch (d_rope=64, one rotary key per token shared by heads and loops)
    on two decode reads, each beside the same read without the branch: the capacity layer (per
    head, B=768, H=16, d=128, r=24/24, 4096 cached tokens; the streaming read dots each token's
    rotary key in the token's lane group) and the LLA-2D layer (B=128, H=16, d=128, r=256/256,
    8192 cached tokens; the rotary keys are extra MFMA k-steps of the read)."""
    import torch
    from decode_attention_lla_amd import lla, synth
    d_rope = 64
    bf = torch.bfloat16
    res = {}
    for key in ("capacity", "lla2d"):
        s = synth.CASES[key]
        B, H, d, T, r, N = s.B, s.H, s.d, s.T, s.r_k, s.N
        n_max = N + 1
        two_d = s.variant == "2d"
        desc = lla.make_desc(lla.LLA_2D if two_d else lla.LLA_PER_HEAD, lla.LLA_BF16, H, d, T, r, r,
                             n_max)
        zshape = (B, n_max, r) if two_d else (B, H, n_max, r)
        zk = synth.device_normal_(torch.empty(zshape, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZK))
        zv = synth.device_normal_(torch.empty(zshape, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZV))
        mk_w = synth.orthonormal_W_2d if two_d else synth.orthonormal_W
        Wk = torch.from_numpy(mk_w(T, H, d, r, synth.seed(s.case, synth.SEED_WK), "bf16")).to(bf).cuda()
        Wv = torch.from_numpy(mk_w(T, H, d, r, synth.seed(s.case, synth.SEED_WV), "bf16")).to(bf).cuda()
        q = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_Q))
        ks = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF))
        vs = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_SELF) + 1)
        kr = synth.device_normal_(torch.empty(B, n_max, d_rope, dtype=bf, device="cuda"), 9980)
        qr = synth.device_normal_(torch.empty(B, H, d_rope, dtype=bf, device="cuda"), 9981)
        krs = synth.device_normal_(torch.empty(B, d_rope, dtype=bf, device="cuda"), 9982)
        out = torch.empty(B, H, d, dtype=bf, device="cuda")
        lens = torch.full((B,), N, dtype=torch.int32, device="cuda")
        ws = lla.workspace(desc, B)
        ws_r = lla.rope_workspace(desc, B)

        def plain():
            lla.lla_attend_decode(desc, B, 0, q, zk, zv, lens, Wk, Wv, None, None, ks, vs, out, None, ws)

        def with_rope():
            lla.lla_attend_decode_rope(desc, B, 0, q, qr, zk, zv, kr, d_rope, 0.0, lens, Wk, Wv,
                                       None, None, ks, vs, krs, out, None, ws_r)

        ms_p = _timed(plain, 20, 3)
        ms_r = _timed(with_rope, 20, 3)
        latent = B * (1 if two_d else H) * N * 2 * r * 2
        # the rotary keys, once per sequence (both reads form the rotary scores inside the read;
        # the heads of a sequence share its keys through L2)
        extra = B * N * d_rope * 2
        name = "lla2d" if two_d else "capacity"
        res[name] = {
            "workload": f"{'LLA-2D' if two_d else 'capacity'} layer read with a {d_rope}-wide rotary "
                        f"branch: H={H}, d_head={d}, r_k=r_v={r}, B={B}, N={N}, bf16",
            "read_us": round(ms_r * 1e3, 2), "read_without_rotary_us": round(ms_p * 1e3, 2),
            "algorithmic_GBps": round((latent + extra) / (ms_r / 1e3) / 1e9, 1),
            "algorithmic_frac_of_peak": round((latent + extra) / (ms_r / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "rotary_bytes_over_latent_bytes": round(extra / latent, 4)}
        del zk, zv, kr, ws, ws_r
        torch.cuda.empty_cache()
    return res


def long_context(args):
    """The paper's only speed ratio (Section 7): at 262k cached tokens and the 4x geometry (H=16,
    d=128, T=4, r_k/r_v = 96/160), one decode read in absorbed form (lla_attend_decode) against
    reconstruct-then-attend (lla_attend_decode_reconstruct: rebuild K_t and V_t of every token in
    bf16, then attend). B=1."""
    import torch
    from decode_attention_lla_amd import lla, synth
    B, H, d, T, rk, rv, N = 1, 16, 128, 4, 96, 160, 262144
    n_max = N + 1
    bf = torch.bfloat16
    desc = lla.make_desc(lla.LLA_PER_HEAD, lla.LLA_BF16, H, d, T, rk, rv, n_max)
    sd = 9800
    zk = synth.device_normal_(torch.empty(B, H, n_max, rk, dtype=bf, device="cuda"), sd + 1)
    zv = synth.device_normal_(torch.empty(B, H, n_max, rv, dtype=bf, device="cuda"), sd + 2)
    Wk = synth.device_normal_(torch.empty(T, H, d, rk, dtype=bf, device="cuda"), sd + 3, 1 / rk ** 0.5)
    Wv = synth.device_normal_(torch.empty(T, H, d, rv, dtype=bf, device="cuda"), sd + 4, 1 / rv ** 0.5)
    q = synth.device_normal_(torch.empty(B, H, d, dtype=bf, device="cuda"), sd + 5)
    out = torch.empty_like(q)
    lens = torch.full((B,), N, dtype=torch.int32, device="cuda")
    ws_a = lla.workspace(desc, B)
    ws_r = lla.reconstruct_workspace(desc, B)

    def absorbed():
        lla.lla_attend_decode(desc, B, 1, q, zk, zv, lens, Wk, Wv, None, None, None, None, out,
                              None, ws_a)

    def rebuilt():
        lla.lla_attend_decode_reconstruct(desc, B, 1, q, zk, zv, lens, Wk, Wv, None, None, None,
                                          None, out, None, ws_r)

    ms_a = _timed(absorbed, 20, 3)
    ms_r = _timed(rebuilt, 10, 2)
    latent = B * H * N * (rk + rv) * 2
    kv = B * H * N * 2 * d * 2
    return {"workload": f"one decode read at {N} cached tokens: B={B}, H={H}, d_head={d}, T={T}, "
                        f"r_k={rk}, r_v={rv} (4x), bf16",
            "absorbed_us": round(ms_a * 1e3, 2),
            "absorbed_latent_GBps": round(latent / (ms_a / 1e3) / 1e9, 1),
            "absorbed_frac_of_peak": round(latent / (ms_a / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "reconstruct_then_attend_us": round(ms_r * 1e3, 2),
            "reconstruct_hbm_bytes_algorithmic": latent + 2 * kv,
            "absorbed_speedup": round(ms_r / ms_a, 3),
            "paper_absorbed_speedup_H200": 2.3}


def lla2d_prefill(args):
    """LLA-2D chunked prefill (B=128, C=512, N_ctx=8192, r=256/256): encode the chunk, then one
    causal prefill read per loop (T=4)."""
    import torch
    from decode_attention_lla_amd import lla, synth
    s = synth.CASES["lla2d"]
    B, H, d, T, r, N, C = s.B, s.H, s.d, s.T, s.r_k, s.N, s.C
    n_max = N + C
    bf = torch.bfloat16
    desc = lla.make_desc(lla.LLA_2D, lla.LLA_BF16, H, d, T, r, r, n_max)
    zk = synth.device_normal_(torch.empty(B, n_max, r, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZK))
    zv = synth.device_normal_(torch.empty(B, n_max, r, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_ZV))
    wk = synth.orthonormal_W_2d(T, H, d, r, synth.seed(s.case, synth.SEED_WK), "bf16")
    wv = synth.orthonormal_W_2d(T, H, d, r, synth.seed(s.case, synth.SEED_WV), "bf16")
    Wk, Wv = torch.from_numpy(wk).to(bf).cuda(), torch.from_numpy(wv).to(bf).cuda()
    Ek = torch.from_numpy(synth.pinv_E_from_W_2d(wk, "bf16")).to(bf).cuda()
    Ev = torch.from_numpy(synth.pinv_E_from_W_2d(wv, "bf16")).to(bf).cuda()
    xk = synth.device_normal_(torch.empty(B, C, T, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_XK))
    xv = synth.device_normal_(torch.empty(B, C, T, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_XV))
    q = synth.device_normal_(torch.empty(T, B, C, H, d, dtype=bf, device="cuda"), synth.seed(s.case, synth.SEED_Q))
    out = torch.empty(B, C, H, d, dtype=bf, device="cuda")
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    ws = lla.workspace(desc, B, C)

    def encode():
        lla.lla_encode(desc, B, C, xk, xv, Ek, Ev, None, None, ctx, zk, zv)

    def attend(t):
        lla.lla_attend_prefill(desc, B, C, t, q[t], zk, zv, ctx, Wk, Wv, None, None, out, ws)

    def step():
        encode()
        for t in range(T):
            attend(t)

    ms_enc = _timed(encode, 3, 1)
    ms_att = _timed(lambda: attend(0), 3, 1)
    ms_step = _timed(step, 2, 1)
    # the same loop read with a 64-wide decoupled rotary branch (lla_attend_prefill_rope)
    d_rope = 64
    kr = synth.device_normal_(torch.empty(B, n_max, d_rope, dtype=bf, device="cuda"), 9997)
    qr = synth.device_normal_(torch.empty(B, C, H, d_rope, dtype=bf, device="cuda"), 10001)
    ms_rope = _timed(lambda: lla.lla_attend_prefill_rope(desc, B, C, 0, q[0], qr, zk, zv, kr, d_rope,
                                                         0.0, ctx, Wk, Wv, None, None, out, ws), 3, 1)
    keys = sum(N + j + 1 for j in range(C))                  # per (sequence, head)
    att_flops = 2.0 * B * H * keys * 2 * r                   # scores + latent-V products
    proj_flops = 2.0 * B * C * H * d * 2 * r                 # q~ and output projections
    enc_flops = 2.0 * B * C * 2 * r * T * H * d              # both axes
    # what the kernel issues: q~ and the latent sums enter their products as bf16 hi + lo pairs, so
    # the score products and the output projection run twice
    issued_flops = att_flops + proj_flops + 2.0 * B * H * keys * r + 2.0 * B * C * H * d * r
    return {"workload": f"lla2d prefill: C={C} per sequence, B={B}, N_ctx={N}, H={H}, d_head={d}, "
                        f"T={T}, r_k=r_v={r}, bf16",
            "tokens_per_s": round(B * C / (ms_step / 1e3), 1), "ms_per_chunk": round(ms_step, 3),
            "encode_ms": round(ms_enc, 3), "attend_ms_per_loop": round(ms_att, 3),
            "attend_with_64_wide_rotary_branch_ms_per_loop": round(ms_rope, 3),
            "attend_TFLOPs": round((att_flops + proj_flops) / (ms_att / 1e3) / 1e12, 1),
            "attend_mfma_util_bf16_dense": round((att_flops + proj_flops) / (ms_att / 1e3) / 2.5e15, 4),
            "attend_issued_TFLOPs_q_hi_lo": round(issued_flops / (ms_att / 1e3) / 1e12, 1),
            "attend_issued_frac_bf16_dense": round(issued_flops / (ms_att / 1e3) / 2.5e15, 4),
            "encode_TFLOPs": round(enc_flops / (ms_enc / 1e3) / 1e12, 1),
            "encode_mfma_util_bf16_dense": round(enc_flops / (ms_enc / 1e3) / 2.5e15, 4)}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def device_copy_ceiling(stream, gib=4, reps=5):
    """Measured device-to-device copy rate (bytes read + bytes written per second, GB/s) of a
    `gib` GiB buffer: the ceiling a plain copy reaches on this part, beside the datasheet peak."""
    import torch
    a = torch.empty(gib * 2 ** 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    b.copy_(a)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * gib * 2 ** 30 / (ms / 1e3) / 1e9


def cpu_baseline(args, s, D, zk, zv, Wk, Wv, Ek, Ev, q, kself, vself, xk, xv, lens):
    """The CPU oracle on one sequence's decode step (all layers and loops, then the encodes),
    stopped after about --cpu-seconds and extrapolated to the full step; tokens/s = 1 / step time
    (each step emits one token for this sequence)."""
    from oracle import lla_oracle as O
    affinity = len(os.sched_getaffinity(0))
    limiter = None
    try:  # BLAS threads = the CPUs this process may run on
        import threadpoolctl
        limiter = threadpoolctl.threadpool_limits(limits=affinity, user_api="blas")
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        cores = 1

    T, N = s.T, s.N
    b = 0
    sl = slice(b, b + 1)
    host = lambda t: t[sl].float().cpu().numpy()  # noqa: E731
    lens_h = np.array([N], np.int32)
    reads = 0
    t_read = 0.0
    enc_time = 0.0
    budget = args.cpu_seconds
    cache = {}
    for t in range(T):
        for l in range(D):
            if l not in cache:
                cache[l] = (host(zk[l]), host(zv[l]), Wk[l].float().cpu().numpy(), Wv[l].float().cpu().numpy())
            zkh, zvh, wk, wv = cache[l]
            qh = q[t, l][sl].float().cpu().numpy()
            ks = kself[t, l][sl].float().cpu().numpy()
            vs = vself[t, l][sl].float().cpu().numpy()
            c0 = time.perf_counter()
            O.attend_decode(qh, zkh, zvh, wk, wv, t, lens_h, None, None, ks, vs)
            t_read += time.perf_counter() - c0
            reads += 1
            if t_read > budget:
                break
        if t_read > budget:
            break
    # one layer's encode for this sequence, timed and scaled by the layer count
    zkh, zvh, _, _ = cache[0]
    xkh = xk[0][sl].float().cpu().numpy()
    xvh = xv[0][sl].float().cpu().numpy()
    c0 = time.perf_counter()
    O.encode_into_cache(zkh, zvh, xkh, xvh, Ek[0].float().cpu().numpy(), Ev[0].float().cpu().numpy(), lens_h)
    enc_time = time.perf_counter() - c0
    step_s = t_read / reads * (T * D) + enc_time * D
    if limiter is not None:
        limiter.restore_original_limits()
    return {
        "value": round(1.0 / step_s, 4),
        "unit": "tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"sequence 0 of {s.B}: {reads} of {T * D} loop reads (explicit reconstruction, "
                  f"float64, {t_read:.1f} s) plus one layer's encode, extrapolated to the full "
                  f"step of one sequence ({step_s:.1f} s per token)",
        "host_cpus": os.cpu_count(),
        "affinity_cpus": affinity,
        "cpu_model": _cpu_model(),
    }


if __name__ == "__main__":
    main()
