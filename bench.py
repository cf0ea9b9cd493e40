#!/usr/bin/env python3
"""Benchmark of the Deja Vu sparse decode step on one MI355X.

One step = one decode layer of the OPT-175B-shaped workload (d = 12288, 4d = 49152
neurons, 96 heads of 128, 2048 cached tokens, batch 1) through dv_decode_layer:
the next layer's low-rank predictor and top-k (look-ahead), the sparse MLP over
the selected 4915 neurons, the head-sparse attention over the selected 19 heads,
and the residual combine.  Steps walk a ring of layer replicas (distinct weights,
caches and inputs; the working set is many times the 256 MB Infinity Cache), and
each step's look-ahead sets feed the next step, as in a real layer stack.

Printed: one JSON line with whole-step throughput as effective HBM GB/s over the
bytes the step must read, microseconds per layer, the sparse MLP+MHA part alone
(given the sets), the roofline of the dominant launch (HIP events on the launch
stream), and the CPU oracle timed on host cores over a bounded sample.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/layer + effective HBM GB/s (selected bytes) for sparse MLP+MHA, OPT-175B shape"
PEAK_GBPS = 8000.0          # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "c4_b1_decode_layer_traffic.json")


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "contextual_sparsity_mlp_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(src_hash):
    """HBM traffic per launch from the committed counter summary, if it was taken on
    the current kernel sources; otherwise None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("source_hash") != src_hash:
        return None
    return t


def blas_threads() -> int:
    try:
        import threadpoolctl
        n = [i.get("num_threads", 0) for i in threadpoolctl.threadpool_info()
             if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--replicas", type=int, default=6)
    ap.add_argument("--cpu-layers", type=int, default=4,
                    help="decode layers the CPU oracle times (0 = skip)")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="run one plain 1 GiB device copy first (counter calibration)")
    ap.add_argument("--lookahead-only", action="store_true",
                    help="skip the per-launch event pass and the sparse-only pass")
    ap.add_argument("--wdt", choices=("bf16", "fp8"), default="bf16",
                    help="selected weights (W1, W2, W^Q, W^O): bf16, or weight-only fp8 E4M3 "
                         "with per-row scales (predictor factors and KV stay bf16)")
    ap.add_argument("--act", choices=("relu", "gelu"), default="relu",
                    help="sigma of the MLP (OPT uses ReLU; GeLU is the page's other choice)")
    ap.add_argument("--kv-append", action="store_true",
                    help="the full decode step: every head's k and v of the current token are "
                         "computed (W^K, W^V read in full), stored at row n_ctx of the cache "
                         "and attended with it")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {max(args.gpus, world)}): the decode "
              "step is built and measured for one MI355X; sharding across GPUs is not part of "
              "this build.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from contextual_sparsity_mlp_amd import accounting as acc
    from contextual_sparsity_mlp_amd import dv, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dv.lib()   # raises if the HIP library is missing
    dev = "cuda"
    cfg = synth.CONFIGS["c4"]
    B, R = args.batch, max(2, args.replicas)
    k_m, k_a = cfg.k_m, cfg.k_a
    cap_m, cap_a = min(cfg.F, B * k_m), min(cfg.h, B * k_a)

    if args.copy_calibrate:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE calibrate the counters
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy: 1073741824 bytes read, 1073741824 bytes written")

    log(f"generating {R} replicas of the c4 layer (batch {B}) on the GPU")
    layers, ys = [], []
    for l in range(R):
        Lt = synth.make_layer(cfg, dev, layer=l, batch=B, with_kv=not args.kv_append)
        if args.kv_append:
            # a cache with a free row n_ctx; every step of the loop appends there
            Lt.K, Lt.V = synth.make_kv_cache(cfg, cfg.n_ctx + 1, dev, layer=l, batch=B)
            Lt.extra["Wk"], Lt.extra["Wv"] = synth.make_kv_weights(cfg, dev, layer=l)
        if args.wdt == "fp8":
            # weight-only fp8 input preparation: E4M3 codes with one fp32 scale per row
            for k in ("W1t", "W2t", "Wq", "Wo") + (("Wk", "Wv") if args.kv_append else ()):
                if k in Lt.extra:
                    codes, sc = synth.quantize_rows_e4m3(Lt.extra[k])
                    Lt.extra[k] = codes
                    Lt.extra[k + "_scale"] = sc
                    continue
                codes, sc = synth.quantize_rows_e4m3(getattr(Lt, k))
                setattr(Lt, k, codes)
                Lt.extra[k + "_scale"] = sc
        layers.append(Lt)
        ys.append(synth.make_y(cfg, dev, layer=l, batch=B))
    torch.cuda.synchronize()
    def row_scales(L):
        if args.wdt != "fp8":
            return None
        return tuple(L.extra[k + "_scale"] for k in ("W1t", "W2t", "Wq", "Wo"))

    def kv_args(L):
        if not args.kv_append:
            return {}
        return dict(Wk=L.extra["Wk"], Wv=L.extra["Wv"], n_ctx=cfg.n_ctx,
                    kv_scales=((L.extra["Wk_scale"], L.extra["Wv_scale"]) if args.wdt == "fp8"
                               else None))

    dvl = [dv.Layer(L.W1t, L.W2t, L.Wq, L.Wo, L.K, L.V, L.A_M, L.B_M, L.A_A, L.B_A,
                    k_m=k_m, k_a=k_a, scale=cfg.scale,
                    act=dv.DV_ACT_GELU if args.act == "gelu" else dv.DV_ACT_RELU,
                    row_scales=row_scales(L), **kv_args(L)) for L in layers]

    i32 = lambda n: torch.zeros(n, dtype=torch.int32, device=dev)  # noqa: E731
    sets = [dict(m=i32(cap_m), cm=i32(1), a=i32(cap_a), ca=i32(1)) for _ in range(2)]
    ws = dv.workspace(dv.OP_DECODE_LAYER, batch=B, d=cfg.d, F=cfg.F, h=cfg.h, dh=cfg.dh,
                      n_ctx=cfg.n_ctx, r=cfg.r, max_count_m=cap_m, max_count_a=cap_a)
    y_out = torch.empty_like(ys[0])

    # Layer 0's sets from its own predictor (nothing runs ahead of it).
    s_m = torch.empty((B, cfg.F), dtype=torch.float32, device=dev)
    s_a = torch.empty((B, cfg.h), dtype=torch.float32, device=dev)
    wsp = dv.workspace(dv.OP_PREDICT, batch=B, d=cfg.d, r=cfg.r, N=cfg.F)
    wst = dv.workspace(dv.OP_SELECT_TOPK, batch=B, N=cfg.F)
    L0 = layers[0]
    dv.predict(ys[0], L0.A_M, L0.B_M, s_m, wsp)
    dv.select_topk(s_m, k_m, 1, sets[0]["m"], sets[0]["cm"], wst)
    dv.predict(ys[0], L0.A_A, L0.B_A, s_a, wsp)
    dv.select_topk(s_a, k_a, 1, sets[0]["a"], sets[0]["ca"], wst)

    def step(t, lookahead=True):
        l = t % R
        if lookahead:
            si, so = sets[t % 2], sets[(t + 1) % 2]
            dv.decode_layer(dvl[l], dvl[(l + 1) % R], ys[l], y_out, si["m"], si["cm"], cap_m,
                            si["a"], si["ca"], cap_a, so["m"], so["cm"], so["a"], so["ca"], ws)
        else:
            # the sparse MLP + MHA and the combine only, on a fixed valid set
            si = sets[0]
            dv.decode_layer(dvl[l], None, ys[l], y_out, si["m"], si["cm"], cap_m, si["a"],
                            si["ca"], cap_a, None, None, None, None, ws)

    def timed(n, lookahead=True):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for t in range(n):
            step(t, lookahead)
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / n
        return wall, e0.elapsed_time(e1) / n

    log(f"warmup {args.warmup} steps")
    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    u_m = int(sets[0]["cm"].cpu()[0])
    u_a = int(sets[0]["ca"].cpu()[0])
    shape = dict(batch=B, d=cfg.d, F=cfg.F, h=cfg.h, dh=cfg.dh, n_ctx=cfg.n_ctx, r=cfg.r,
                 u_m=u_m, u_a=u_a,
                 **(dict(w_bytes=1, p_bytes=2, row_scale_bytes=4) if args.wdt == "fp8" else {}),
                 kv_append=args.kv_append)
    full_bytes = acc.step_bytes(**shape)
    log(f"timing {args.steps} steps (|S_M|={u_m}, |S_A|={u_a})")
    ms_step, ev_step = timed(args.steps)
    if args.lookahead_only:
        print(json.dumps({"us_per_layer": round(ms_step * 1e3, 2), "steps": args.steps}), flush=True)
        return

    # Per-launch durations with HIP events recorded around each launch on its stream.
    dv.timing_enable(True)
    for t in range(args.steps):
        step(t)
    torch.cuda.synchronize()
    ph_ms, ph_n = dv.timing_read(8)
    dv.timing_enable(False)
    # three launches, or five when the attention runs alone before the predictor's
    # matrix-core row sums and their score histograms (a batch of tokens)
    n_la = sum(1 for n in ph_n if n > 0)
    ph_bytes = acc.phase_bytes(**shape, lookahead_launches=n_la)
    phases = []
    kvn = "; W^K, W^V of every head" if args.kv_append else ""
    names = ([f"row dots (W1, W^Q, A rows{kvn})", "attention", "predictor B rows",
              "score histograms", "row sum W2 + W^O rows, combine, top-k"] if n_la == 5 else
             [f"row dots (W1, W^Q, A rows{kvn})", "attention + predictor B rows",
              "row sum W2 + W^O rows, combine, top-k"])
    for i, (ms, n) in enumerate(zip(ph_ms, ph_n)):
        avg_us = ms * 1e3 / max(n, 1)
        b = ph_bytes[i] if i < len(ph_bytes) else 0
        phases.append(dict(launch=i, name=names[i] if i < len(names) else f"launch{i}",
                           avg_us=round(avg_us, 2), bytes=b,
                           GBps=round(b / (avg_us * 1e-6) / 1e9, 1) if b else None))
    dom = max(phases, key=lambda p: p["avg_us"])

    # The sparse MLP + MHA alone, given the sets (no predictor, no top-k).
    log("timing the sparse MLP+MHA part alone")
    ms_sparse, ev_sparse = timed(args.steps, lookahead=False)
    sel_bytes = acc.step_bytes(**shape, with_predictor=False).selected
    dv.timing_enable(True)
    for t in range(args.steps):
        step(t, lookahead=False)
    torch.cuda.synchronize()
    sp_ms, sp_n = dv.timing_read(8)
    dv.timing_enable(False)
    # two launches when the attention shares the row sum's launch, three otherwise
    n_sp = sum(1 for n in sp_n if n > 0)
    sp_bytes = acc.phase_bytes(**shape, with_predictor=False, sparse_launches=n_sp)
    sp_names = ([f"row dots (W1, W^Q rows{kvn})", "attention", "row sum W2 + W^O rows"]
                if n_sp == 3 else
                [f"row dots (W1, W^Q rows{kvn})", "attention + row sum W2 then W^O rows"])
    sparse_phases = [dict(launch=i, name=sp_names[i], avg_us=round(ms * 1e3 / max(n, 1), 2),
                          bytes=sp_bytes[i],
                          GBps=round(sp_bytes[i] / (ms * 1e-3 / max(n, 1)) / 1e9, 1))
                     for i, (ms, n) in enumerate(zip(sp_ms, sp_n)) if i < len(sp_bytes)]

    src = source_hash()
    traffic = load_traffic(src)
    roofline = dict(bound="hbm", kernel=f"phase_kernel launch {dom['launch']}: {dom['name']}",
                    achieved=dom["GBps"], peak=PEAK_GBPS, unit="GB/s",
                    frac=round(dom["GBps"] / PEAK_GBPS, 4),
                    traffic=(traffic["per_launch"].get(str(dom["launch"])) if traffic else None),
                    avg_launch_us=dom["avg_us"], algorithmic_bytes=dom["bytes"])

    cpu = None
    if args.cpu_layers > 0:
        cpu = cpu_baseline(args.cpu_layers, layers, ys, sets, cfg, B, u_m, u_a, full_bytes.total,
                           args.act, args.wdt == "fp8", args.kv_append)

    out = {
        "metric": METRIC,
        "value": round(full_bytes.total / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "weights_dtype": ("fp8 e4m3 rows with fp32 row scales (predictor bf16)"
                          if args.wdt == "fp8" else "bf16"),
        "data": "synthetic",
        "config": {"workload": f"opt-175b-shaped decode layer, batch {B}, look-ahead predictor"
                               + (", GeLU MLP" if args.act == "gelu" else "")
                               + (", fp8 weights" if args.wdt == "fp8" else "")
                               + (", KV append" if args.kv_append else ""),
                   "wdt": args.wdt,
                   "act": args.act,
                   "kv_append": args.kv_append,
                   "d": cfg.d, "F": cfg.F, "h": cfg.h, "dh": cfg.dh, "n_ctx": cfg.n_ctx,
                   "r": cfg.r, "batch": B, "k_m": k_m, "k_a": k_a, "U_M": u_m, "U_A": u_a,
                   "replicas": R},
        "us_per_layer": round(ms_step * 1e3, 2),
        "gpu_event_us_per_layer": round(ev_step * 1e3, 2),
        "bytes_per_step": full_bytes.total,
        "bytes_selected": full_bytes.selected,
        "bytes_predictor": full_bytes.predictor,
        "sparse_mlp_mha": {"us_per_layer": round(ms_sparse * 1e3, 2),
                           "gpu_event_us": round(ev_sparse * 1e3, 2),
                           "bytes": sel_bytes,
                           "GBps": round(sel_bytes / (ms_sparse * 1e-3) / 1e9, 1),
                           "frac_of_peak": round(sel_bytes / (ms_sparse * 1e-3) / 1e9 / PEAK_GBPS,
                                                 4),
                           "phases": sparse_phases},
        "frac_of_peak": round(full_bytes.total / (ms_step * 1e-3) / 1e9 / PEAK_GBPS, 4),
        "phases": phases,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "source_hash": src,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(n_layers, layers, ys, sets, cfg, B, u_m, u_a, step_bytes_total, act="relu",
                 fp8=False, kv_append=False):
    """The CPU oracle (float64 NumPy, as it stands) on host copies of replica 0."""
    import numpy as np
    import torch

    from oracle import dv_oracle as O

    def host(t):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    log(f"cpu baseline: {n_layers} oracle decode layers on host copies")
    L, L1 = layers[0], layers[1 % len(layers)]
    layer_h = dict(W1t=host(L.W1t), W2t=host(L.W2t), Wq=host(L.Wq), Wo=host(L.Wo), K=host(L.K),
                   V=host(L.V), act=act)
    if kv_append:
        layer_h["Wk"], layer_h["Wv"] = host(L.extra["Wk"]), host(L.extra["Wv"])
    if fp8:
        for k in ("W1t", "W2t", "Wq", "Wo"):
            layer_h[k] = O.Fp8Rows(layer_h[k], host(L.extra[k + "_scale"]))
        if kv_append:
            for k in ("Wk", "Wv"):
                layer_h[k] = O.Fp8Rows(layer_h[k], host(L.extra[k + "_scale"]))
    nxt_h = dict(A_M=host(L1.A_M), B_M=host(L1.B_M), A_A=host(L1.A_A), B_A=host(L1.B_A),
                 k_m=cfg.k_m, k_a=cfg.k_a, union=True)
    # replica 0's own sets, as the oracle would predict them from y_0
    yh = host(ys[0])
    S_M = O.predict_and_select(yh, host(L.A_M), host(L.B_M), cfg.k_m, True)
    S_A = O.predict_and_select(yh, host(L.A_A), host(L.B_A), cfg.k_a, True)
    times = []
    for _ in range(n_layers):
        t0 = time.perf_counter()
        if kv_append:
            O.decode_layer_append(yh, layer_h, S_M, S_A, nxt_h, cfg.n_ctx, cfg.scale)
        else:
            O.decode_layer(yh, layer_h, S_M, S_A, nxt_h, cfg.scale)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": round(step_bytes_total / t / 1e9, 3), "unit": "GB/s",
            "us_per_layer": round(t * 1e6, 1), "cores": blas_threads(), "kind": "oracle",
            "sample": f"{n_layers} full decode layers of the same workload (replica 0, batch {B}, "
                      f"look-ahead predictor + top-k + sparse MLP + sparse MHA"
                      f"{' + KV append' if kv_append else ''}), float64 NumPy, "
                      f"median of {n_layers}; same byte count as the GPU line"}


if __name__ == "__main__":
    main()
