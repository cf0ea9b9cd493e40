#!/usr/bin/env python3
"""Benchmark of the Deja Vu sparse decode step on one MI355X.

The measured step is the sparse MLP + head-sparse MHA of one OPT-175B-shaped decode
layer (d = 12288, 4d = 49152 neurons, 96 heads of 128, 2048 cached tokens, batch 1)
given its index sets (4915 neurons, 19 heads): the row dots of the selected W1 and
W^Q rows, the attention of the selected heads over their caches, and one row sum over
the selected W2 and W^O rows combined with the residual, through dv_decode_layer.
`value` is the effective HBM bandwidth over the bytes the step must read and write
(selected weight rows, the selected heads' KV, y in and out), `us_per_layer` its
time.  Steps walk a ring of layer replicas (distinct weights, caches and inputs; the
working set is many times the 256 MB Infinity Cache).

Also reported: the whole look-ahead layer (the same step plus the next layer's
low-rank predictor and top-k, its sets feeding the next step as in a layer stack),
per-launch durations from HIP events on the launch stream, the roofline of the
step's dominant launch, and the CPU oracle timed on the host cores (all of them and
one) over a bounded sample, and (`variants`) the same step with fp8 rows, with GeLU
and with the KV append.  `--sweep` prints one line per workload instead
(OPT-6.7B, OPT-30B at batch 4, OPT-175B at batch 1-16, the 24-layer stack's layer
at batch 32).
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "c4_b1_sparse_step_traffic.json")


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
    """HBM traffic per launch of the sparse step from the committed counter summary,
    if it was taken on the current kernel sources; otherwise None."""
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


# Kernel symbols behind each launch of the sparse step at batch 1 (bf16 rows), by the
# number of launches the library issued.
def sparse_kernels(n_launches, args):
    """Kernel symbols behind each launch of the sparse step at batch 1, by the number
    of launches the library issued (None where they are not pinned down here)."""
    if args.wdt == "fp8":
        rd = "rowdot_kv_kernel<385, 1>" if args.kv_append else "rowdot_kernel<129, 1>"
        return {2: [rd, "phase_kernel_bt<166, 1>"],
                3: [rd, "phase_kernel<2, 1>", "phase_kernel<132, 1>"]}.get(n_launches)
    rd = "rowdot_kv_kernel<257, 1>" if args.kv_append else "rowdot_kernel<1, 1>"
    return {1: ["stream_kernel<1>"], 2: [rd, "phase_kernel<38, 1>"],
            3: [rd, "phase_kernel<2, 1>", "phase_kernel<4, 1>"]}.get(n_launches)


class Workload:
    """Replicas of one decode-layer workload resident on the GPU, with index sets."""

    def __init__(self, cfg, B, replicas, args, dev="cuda"):
        import torch

        from contextual_sparsity_mlp_amd import dv, synth
        self.cfg, self.B, self.R, self.args = cfg, B, max(2, replicas), args
        self.dv = dv
        k_m, k_a = cfg.k_m, cfg.k_a
        self.cap_m, self.cap_a = min(cfg.F, B * k_m), min(cfg.h, B * k_a)
        log(f"{cfg.name}: generating {self.R} replicas (batch {B}) on the GPU")
        self.layers, self.ys = [], []
        for l in range(self.R):
            Lt = synth.make_layer(cfg, dev, layer=l, batch=B, with_kv=not args.kv_append)
            if args.kv_append:
                # a cache with a free row n_ctx; every step of the loop appends there
                Lt.K, Lt.V = synth.make_kv_cache(cfg, cfg.n_ctx + 1, dev, layer=l, batch=B)
                Lt.extra["Wk"], Lt.extra["Wv"] = synth.make_kv_weights(cfg, dev, layer=l)
            if args.wdt == "fp8":
                # weight-only fp8 input preparation: E4M3 codes with one fp32 scale per row
                for k in ("W1t", "W2t", "Wq", "Wo") + (("Wk", "Wv") if args.kv_append else ()):
                    src = Lt.extra[k] if k in Lt.extra else getattr(Lt, k)
                    codes, sc = synth.quantize_rows_e4m3(src)
                    if k in Lt.extra:
                        Lt.extra[k] = codes
                    else:
                        setattr(Lt, k, codes)
                    Lt.extra[k + "_scale"] = sc
            self.layers.append(Lt)
            self.ys.append(synth.make_y(cfg, dev, layer=l, batch=B))
        torch.cuda.synchronize()

        def row_scales(L):
            if args.wdt != "fp8":
                return None
            return tuple(L.extra[k + "_scale"] for k in ("W1t", "W2t", "Wq", "Wo"))

        def kv_args(L):
            if not args.kv_append:
                return {}
            return dict(Wk=L.extra["Wk"], Wv=L.extra["Wv"], n_ctx=cfg.n_ctx,
                        kv_scales=((L.extra["Wk_scale"], L.extra["Wv_scale"])
                                   if args.wdt == "fp8" else None))

        self.dvl = [dv.Layer(L.W1t, L.W2t, L.Wq, L.Wo, L.K, L.V, L.A_M, L.B_M, L.A_A, L.B_A,
                             k_m=k_m, k_a=k_a, scale=cfg.scale,
                             act=dv.DV_ACT_GELU if args.act == "gelu" else dv.DV_ACT_RELU,
                             row_scales=row_scales(L), **kv_args(L)) for L in self.layers]
        i32 = lambda n: torch.zeros(n, dtype=torch.int32, device=dev)  # noqa: E731
        self.sets = [dict(m=i32(self.cap_m), cm=i32(1), a=i32(self.cap_a), ca=i32(1))
                     for _ in range(2)]
        self.ws = dv.workspace(dv.OP_DECODE_LAYER, batch=B, d=cfg.d, F=cfg.F, h=cfg.h,
                               dh=cfg.dh, n_ctx=cfg.n_ctx, r=cfg.r, max_count_m=self.cap_m,
                               max_count_a=self.cap_a)
        self.y_out = torch.empty_like(self.ys[0])
        # Layer 0's sets from its own predictor (nothing runs ahead of it).
        s_m = torch.empty((B, cfg.F), dtype=torch.float32, device=dev)
        s_a = torch.empty((B, cfg.h), dtype=torch.float32, device=dev)
        wsp = dv.workspace(dv.OP_PREDICT, batch=B, d=cfg.d, r=cfg.r, N=cfg.F)
        wst = dv.workspace(dv.OP_SELECT_TOPK, batch=B, N=cfg.F)
        L0 = self.layers[0]
        dv.predict(self.ys[0], L0.A_M, L0.B_M, s_m, wsp)
        dv.select_topk(s_m, k_m, 1, self.sets[0]["m"], self.sets[0]["cm"], wst)
        dv.predict(self.ys[0], L0.A_A, L0.B_A, s_a, wsp)
        dv.select_topk(s_a, k_a, 1, self.sets[0]["a"], self.sets[0]["ca"], wst)

    def step(self, t, lookahead):
        dv, l = self.dv, t % self.R
        if lookahead:
            si, so = self.sets[t % 2], self.sets[(t + 1) % 2]
            dv.decode_layer(self.dvl[l], self.dvl[(l + 1) % self.R], self.ys[l], self.y_out,
                            si["m"], si["cm"], self.cap_m, si["a"], si["ca"], self.cap_a,
                            so["m"], so["cm"], so["a"], so["ca"], self.ws)
        else:
            # the sparse MLP + MHA and the combine only, on a fixed valid set
            si = self.sets[0]
            dv.decode_layer(self.dvl[l], None, self.ys[l], self.y_out, si["m"], si["cm"],
                            self.cap_m, si["a"], si["ca"], self.cap_a, None, None, None, None,
                            self.ws)

    def timed(self, n, lookahead):
        """Wall-clock and event time per step over n back-to-back steps."""
        import torch
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for t in range(n):
            self.step(t, lookahead)
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / n
        return wall, e0.elapsed_time(e1) / n

    def launches(self, n, lookahead):
        """Per-launch average durations (HIP events around each launch on its stream)."""
        import torch
        dv = self.dv
        dv.timing_enable(True)
        for t in range(n):
            self.step(t, lookahead)
        torch.cuda.synchronize()
        ms, cnt = dv.timing_read(8)
        dv.timing_enable(False)
        return [(m * 1e3 / max(c, 1)) for m, c in zip(ms, cnt) if c > 0]

    def shape(self):
        cfg, a = self.cfg, self.args
        u_m = int(self.sets[0]["cm"].cpu()[0])
        u_a = int(self.sets[0]["ca"].cpu()[0])
        return dict(batch=self.B, d=cfg.d, F=cfg.F, h=cfg.h, dh=cfg.dh, n_ctx=cfg.n_ctx, r=cfg.r,
                    u_m=u_m, u_a=u_a,
                    **(dict(w_bytes=1, p_bytes=2, row_scale_bytes=4) if a.wdt == "fp8" else {}),
                    kv_append=a.kv_append)


def gbps(nbytes, us):
    return round(nbytes / (us * 1e-6) / 1e9, 1)


def measure(W, steps, warmup):
    """Sparse step and look-ahead layer of one workload: timings, bytes, launches."""
    from contextual_sparsity_mlp_amd import accounting as acc
    for t in range(warmup):
        W.step(t, True)
    shape = W.shape()
    log(f"{W.cfg.name} batch {W.B}: |S_M|={shape['u_m']} |S_A|={shape['u_a']}, timing {steps} steps")
    kvn = "; W^K, W^V of every head" if W.args.kv_append else ""

    # the metric's step: the sparse MLP + MHA and the combine, given the sets
    for t in range(warmup):
        W.step(t, False)
    ms, ev = W.timed(steps, False)
    sel = acc.step_bytes(**shape, with_predictor=False).selected
    ph = W.launches(steps, False)
    ph_b = acc.phase_bytes(**shape, with_predictor=False, sparse_launches=len(ph))
    names = {1: ["sparse step: row dots, attention, row sums (one launch)"],
             2: [f"row dots (W1, W^Q rows{kvn})", "attention + row sum W2 then W^O rows"],
             3: [f"row dots (W1, W^Q rows{kvn})", "attention", "row sum W2 + W^O rows"]}
    sparse = {"us_per_layer": round(ms * 1e3, 2), "gpu_event_us": round(ev * 1e3, 2),
              "bytes": sel, "GBps": gbps(sel, ms * 1e3),
              "frac_of_peak": round(sel / (ms * 1e-3) / 1e9 / PEAK_GBPS, 4),
              "launches": [dict(launch=i, name=names.get(len(ph), [f"launch {i}"] * 8)[i],
                                kernel=(sparse_kernels(len(ph), W.args) or [None] * 8)[i]
                                if W.B == 1 else None,
                                avg_us=round(u, 2), bytes=b, GBps=gbps(b, u))
                           for i, (u, b) in enumerate(zip(ph, ph_b))]}

    # the look-ahead layer: the same plus the next layer's predictor and top-k
    ms2, ev2 = W.timed(steps, True)
    full = acc.step_bytes(**shape)
    ph2 = W.launches(steps, True)
    ph2_b = acc.phase_bytes(**shape, lookahead_launches=len(ph2))
    names2 = ([f"row dots (W1, W^Q, A rows{kvn})", "attention", "predictor B rows",
               "score histograms", "row sum W2 + W^O rows, combine, top-k"] if len(ph2) == 5 else
              [f"row dots (W1, W^Q, A rows{kvn})", "attention + predictor B rows",
               "row sum W2 + W^O rows, combine, top-k"])
    look = {"us_per_layer": round(ms2 * 1e3, 2), "gpu_event_us": round(ev2 * 1e3, 2),
            "bytes": full.total, "bytes_selected": full.selected,
            "bytes_predictor": full.predictor, "GBps": gbps(full.total, ms2 * 1e3),
            "frac_of_peak": round(full.total / (ms2 * 1e-3) / 1e9 / PEAK_GBPS, 4),
            "launches": [dict(launch=i, name=names2[i] if i < len(names2) else f"launch {i}",
                              avg_us=round(u, 2), bytes=b, GBps=gbps(b, u))
                         for i, (u, b) in enumerate(zip(ph2, ph2_b))]}
    return shape, sparse, look


def config_of(W, shape, workload):
    cfg, a = W.cfg, W.args
    return {"workload": workload, "wdt": a.wdt, "act": a.act, "kv_append": a.kv_append,
            "d": cfg.d, "F": cfg.F, "h": cfg.h, "dh": cfg.dh, "n_ctx": cfg.n_ctx, "r": cfg.r,
            "batch": W.B, "k_m": cfg.k_m, "k_a": cfg.k_a, "U_M": shape["u_m"],
            "U_A": shape["u_a"], "replicas": W.R}


def sweep(args):
    """One JSON line per workload: OPT-6.7B, OPT-30B (batch 4), OPT-175B at batch
    1, 2, 4, 8, 16, and one layer of the 24-layer OPT-175B stack at batch 32."""
    import torch

    from contextual_sparsity_mlp_amd import synth
    C = synth.CONFIGS
    cases = [("c2", 1, 6), ("c3", 4, 4)] + [("c4", b, 3) for b in synth.C4_BATCHES] + \
            [("c5", 32, 2)]
    if args.only:
        keep = set(args.only.split(","))
        cases = [c for c in cases if f"{c[0]}b{c[1]}" in keep or c[0] in keep]
    for name, B, R in cases:
        cfg = C[name]
        W = Workload(cfg, B, R, args)
        shape, sparse, look = measure(W, args.steps, args.warmup)
        wl = (f"{cfg.name}-shaped decode layer, batch {B}" if name != "c5" else
              f"one layer of the 24-layer {cfg.name} stack, batch {B}")
        print(json.dumps({"metric": METRIC, "workload": wl,
                          "config": config_of(W, shape, wl),
                          "sparse_mlp_mha": sparse, "lookahead_layer": look}), flush=True)
        del W
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--replicas", type=int, default=6)
    ap.add_argument("--cpu-layers", type=int, default=3,
                    help="sparse steps the CPU oracle times on all host cores (0 = skip); "
                         "it also times one on a single core")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="run one plain 1 GiB device copy first (counter calibration)")
    ap.add_argument("--sparse-only", action="store_true",
                    help="time only the sparse step's launches (a short run for profiling)")
    ap.add_argument("--sweep", action="store_true",
                    help="one line per workload (OPT-6.7B, OPT-30B, OPT-175B batch 1-16, "
                         "the stack's layer at batch 32) instead of the headline line")
    ap.add_argument("--only", default="",
                    help="with --sweep: comma-separated cases to keep (c2, c3, c4b8, c5, ...)")
    ap.add_argument("--wdt", choices=("bf16", "fp8"), default="bf16",
                    help="selected weights (W1, W2, W^Q, W^O): bf16, or weight-only fp8 E4M3 "
                         "with per-row scales (predictor factors and KV stay bf16)")
    ap.add_argument("--act", choices=("relu", "gelu"), default="relu",
                    help="sigma of the MLP (OPT uses ReLU; GeLU is the page's other choice)")
    ap.add_argument("--kv-append", action="store_true",
                    help="the full decode step: every head's k and v of the current token are "
                         "computed (W^K, W^V read in full), stored at row n_ctx of the cache "
                         "and attended with it")
    ap.add_argument("--variants", type=int, default=1,
                    help="with the headline line: also time the same step with fp8 rows, with "
                         "GeLU and with the KV append (2 replicas, 100 steps each; 0 = skip)")
    ap.add_argument("--step-path", choices=("auto", "two", "one"), default="auto",
                    help="launch plan of the one-token bf16 step: the library's default, the "
                         "two-launch plan, or the one-launch queue")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {max(args.gpus, world)}): the decode "
              "step is built and measured for one MI355X; sharding across GPUs is not part of "
              "this build.", file=sys.stderr)
        sys.exit(2)

    import torch

    from contextual_sparsity_mlp_amd import dv, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dv.lib()   # raises if the HIP library is missing
    dv.set_step_path({"auto": dv.PATH_AUTO, "two": dv.PATH_TWO_LAUNCH,
                      "one": dv.PATH_ONE_LAUNCH}[args.step_path])

    if args.copy_calibrate:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE calibrate the counters
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy: 1073741824 bytes read, 1073741824 bytes written")

    if args.sweep:
        sweep(args)
        return

    cfg = synth.CONFIGS["c4"]
    W = Workload(cfg, args.batch, args.replicas, args)
    if args.sparse_only:
        for t in range(args.warmup):
            W.step(t, False)
        ms, _ = W.timed(args.steps, False)
        print(json.dumps({"sparse_us_per_layer": round(ms * 1e3, 2), "steps": args.steps}),
              flush=True)
        return
    shape, sparse, look = measure(W, args.steps, args.warmup)

    src = source_hash()
    traffic = load_traffic(src)
    dom = max(sparse["launches"], key=lambda p: p["avg_us"])
    key = f"{len(sparse['launches'])}:{dom['launch']}"
    roofline = dict(bound="hbm", kernel=f"{dom['kernel']} (launch {dom['launch']}: {dom['name']})",
                    achieved=dom["GBps"], peak=PEAK_GBPS, unit="GB/s",
                    frac=round(dom["GBps"] / PEAK_GBPS, 4),
                    # (the counters were taken on the bf16 batch-1 step without the
                    # KV append; GeLU runs the same launches over the same bytes)
                    traffic=(traffic["per_launch"].get(key) if traffic and W.B == 1 and
                             args.wdt == "bf16" and not args.kv_append else None),
                    avg_launch_us=dom["avg_us"], algorithmic_bytes=dom["bytes"])

    cpu = None
    if args.cpu_layers > 0:
        cpu = cpu_baseline(args.cpu_layers, W, shape, sparse["bytes"])

    wl = (f"opt-175b-shaped sparse MLP+MHA layer step, batch {W.B}, given its index sets"
          + (", GeLU MLP" if args.act == "gelu" else "")
          + (", fp8 weights" if args.wdt == "fp8" else "")
          + (", KV append" if args.kv_append else ""))
    out = {
        "metric": METRIC,
        "value": sparse["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sparse["us_per_layer"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if args.wdt == "fp8" else "bf16",
        "data": "synthetic",
        "config": config_of(W, shape, wl),
        "us_per_layer": sparse["us_per_layer"],
        "frac_of_peak": sparse["frac_of_peak"],
        "sparse_mlp_mha": sparse,
        "lookahead_layer": look,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "variants": None,
        "source_hash": src,
    }
    # the same step with fp8 rows, with GeLU, and with the KV append (each measured like
    # the headline step over 2 replicas; not part of `value`)
    if args.variants and args.wdt == "bf16" and args.act == "relu" and not args.kv_append:
        del W
        torch.cuda.empty_cache()
        out["variants"] = {}
        for key, change in (("fp8", dict(wdt="fp8")), ("gelu", dict(act="gelu")),
                            ("kv_append", dict(kv_append=True))):
            va = argparse.Namespace(**{**vars(args), **change})
            V = Workload(cfg, args.batch, 2, va)
            _, vs, vl = measure(V, 100, 10)
            out["variants"][key] = {"us_per_layer": vs["us_per_layer"], "bytes": vs["bytes"],
                                    "GBps": vs["GBps"], "frac_of_peak": vs["frac_of_peak"],
                                    "launches": vs["launches"],
                                    "lookahead_us_per_layer": vl["us_per_layer"]}
            del V
            torch.cuda.empty_cache()

    print(json.dumps(out), flush=True)


def cpu_baseline(n_layers, W, shape, sel_bytes):
    """The CPU oracle (float64 NumPy, as it stands) on host copies of replica 0: the
    same sparse step on the same sets, timed on all host cores and on one."""
    import numpy as np
    import threadpoolctl
    import torch

    from oracle import dv_oracle as O

    def host(t):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    log(f"cpu baseline: {n_layers} oracle sparse steps on all cores, 1 on one core")
    L, args = W.layers[0], W.args
    layer_h = dict(W1t=host(L.W1t), W2t=host(L.W2t), Wq=host(L.Wq), Wo=host(L.Wo), K=host(L.K),
                   V=host(L.V), act=args.act)
    if args.kv_append:
        layer_h["Wk"], layer_h["Wv"] = host(L.extra["Wk"]), host(L.extra["Wv"])
    if args.wdt == "fp8":
        for k in ("W1t", "W2t", "Wq", "Wo") + (("Wk", "Wv") if args.kv_append else ()):
            layer_h[k] = O.Fp8Rows(layer_h[k], host(L.extra[k + "_scale"]))
    yh = host(W.ys[0])
    si = W.sets[0]
    S_M = si["m"].cpu().numpy()[: int(si["cm"].cpu()[0])]
    S_A = si["a"].cpu().numpy()[: int(si["ca"].cpu()[0])]

    def run():
        t0 = time.perf_counter()
        if args.kv_append:
            O.decode_layer_append(yh, layer_h, S_M, S_A, None, W.cfg.n_ctx, W.cfg.scale)
        else:
            O.decode_layer(yh, layer_h, S_M, S_A, None, W.cfg.scale)
        return time.perf_counter() - t0

    t_all = float(np.median([run() for _ in range(n_layers)]))
    cores = blas_threads()
    with threadpoolctl.threadpool_limits(1):
        t_one = run()
    return {"value": round(sel_bytes / t_all / 1e9, 3), "unit": "GB/s",
            "us_per_layer": round(t_all * 1e6, 1), "cores": cores, "kind": "oracle",
            "sample": f"{n_layers} sparse MLP+MHA steps of the same workload (replica 0, batch "
                      f"{W.B}, the GPU's index sets), float64 NumPy, median; same byte count "
                      f"as the GPU line",
            "single_core": {"value": round(sel_bytes / t_one / 1e9, 3), "unit": "GB/s",
                            "us_per_layer": round(t_one * 1e6, 1), "cores": 1,
                            "sample": "1 sparse step, BLAS limited to one thread"}}


if __name__ == "__main__":
    main()
