#!/usr/bin/env python3
"""Benchmark: one MoE layer forward (route -> shuffle -> expert FFN -> combine)
on one MI355X, seeded synthetic inputs resident in HBM.

The headline is the DeepSeek-V3-shaped prefill layer (T=8192 tokens, H=7168,
256 routed experts with grouped sigmoid gating top-8 + 1 shared expert,
I=2048, P=8 placement groups), the largest layer shape of the workload set.
Prints one JSON line: tokens/s over the timed steps, the roofline position of
the dominant kernel (the grouped GEMM1 + SwiGLU launch, timed with HIP events
recorded around it on the layer's stream in every timed step; no other events
are recorded in the timed steps) against its binding roof (HBM bytes or MFMA
flops, whichever takes longer at peak), the CPU oracle timed on a bounded
sample of the same workload, and the other layer shapes of the workload set
as extra keys ("other_layers": each layer's tokens/s, its stages against
their rooflines and the dispatch call).  The per-stage breakdown
("stages_ms") comes from a further untimed pass with events around every
stage.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
WORKLOAD = "dsv3_prefill"
OTHER_LAYERS = ("tiny", "dsv2lite", "qwen3", "dsv3_decode", "prism")
CPU_SAMPLE = {"dsv3_prefill": 8, "dsv3_decode": 8}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--fuse-gather", type=int, default=int(os.environ.get("MOE_BENCH_FUSE_GATHER", "1")))
    ap.add_argument("--blocked-weights", type=int, default=1,
                    help="1: expert weights packed once (untimed) into the tile-blocked layout the "
                         "grouped GEMMs read as contiguous blocks (moe_pack_weights); 0: row-major")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the sections after the layer (SRS/SAG, one device's share, "
                         "co-scheduling, the other layer shapes), e.g. for a per-kernel profile "
                         "of the layer alone")
    ap.add_argument("--no-other-layers", action="store_true",
                    help="skip the other layer shapes of the workload set")
    ap.add_argument("--other-steps", type=int, default=30,
                    help="timed steps of each other layer shape (after 10 warm-ups)")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="tokens in the oracle's timed sample (0: the workload's default, "
                         "capped at the layer's T)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB "
                         "(reference point for HBM byte counters)")
    return ap.parse_args(argv)


def algorithmic(cfg, A, n_touched=None):
    """Algorithmic work per launch of each stage (bytes or flops).
    n_touched: routed experts with at least one row (default: all E)."""
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    b = 2 if cfg.dtype == "bf16" else 4
    Ish = cfg.n_shared * cfg.I_shared
    ne = E if n_touched is None else n_touched
    return {
        # flops of the grouped GEMM1 (+SwiGLU): routed rows and shared experts
        "ffn_up_flops": 2.0 * A * H * 2 * I + 2.0 * T * H * 2 * Ish,
        "ffn_down_flops": 2.0 * A * I * H + 2.0 * T * Ish * H,
        # bytes of GEMM1: the touched experts' W1/W3 and the shared W1/W3
        # once, x once, the SwiGLU output written once (routed and shared)
        "ffn_up_bytes": (ne * 2.0 * I * H + 2.0 * Ish * H + T * H + A * I + T * Ish) * b,
        # bytes of GEMM2: W2 (touched and shared), the SwiGLU output once,
        # y_sorted and y_sh written once
        "ffn_down_bytes": (ne * 1.0 * H * I + 1.0 * H * Ish + A * I + T * Ish + A * H
                           + (T * H if Ish else 0)) * b,
        # bytes: read x once, write A rows (+ 8T + 12A index metadata)
        "dispatch_bytes": T * H * b + A * H * b + 8.0 * T + 12.0 * A,
        # bytes: read A rows + weights/indices, write T rows (+ shared rows)
        "combine_bytes": A * H * b + 8.0 * A + T * H * b + (T * H * b if Ish else 0),
    }


def binding_roofline(flops, nbytes, ms):
    """A kernel against its binding roof: whichever of HBM bytes at 8 TB/s
    and dense bf16 MFMA flops at 2.5 PFLOP/s takes longer bounds it."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    r = {"hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "mfma_frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
         "flops_per_launch": flops, "bytes_per_launch": nbytes, "avg_launch_ms": round(ms, 4),
         "roof_ms": round(max(t_hbm, t_mfma) * 1e3, 4)}
    if t_hbm >= t_mfma:
        r.update(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                 frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        r.update(bound="mfma", achieved=round(tf, 2), peak=BF16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                 frac=round(tf / BF16_MFMA_PEAK_TFLOPS, 4))
    return r


def describe(cfg):
    """The layer named by what it is, with its sizes."""
    names = {"tiny": "tiny fp32 MoE layer", "dsv2lite": "DeepSeek-V2-Lite-shaped MoE layer",
             "qwen3": "Qwen3-30B-A3B-shaped MoE layer (prefill)",
             "dsv3_decode": "DeepSeek-V3-shaped MoE layer (decode batch)",
             "dsv3_prefill": "DeepSeek-V3-shaped MoE layer (prefill)",
             "prism": "MoE-Prism sub-expert layer (Qwen3-shaped parents split 4 ways)"}
    if cfg.gate == "softmax":
        gate = "softmax%s" % (" renormalised" if cfg.renorm else "")
    else:
        gate = "sigmoid + expert bias, %d routing groups keep %d by top-%d sum, x%g" % (
            cfg.n_rgroups, cfg.topk_rgroups, cfg.rgroup_topn, cfg.route_scale)
    k = "ragged top-k in %s per %d-token request" % (list(cfg.k_choices), cfg.req_tokens) \
        if cfg.ragged else "top-%d" % cfg.k
    sh = " + %d shared (I=%d)" % (cfg.n_shared, cfg.I_shared) if cfg.n_shared else ""
    return "%s: T=%d H=%d E=%d %s %s%s, I=%d, P=%d, V=%d, %s" % (
        names.get(cfg.name, cfg.name), cfg.T, cfg.H, cfg.E, k, gate, sh, cfg.I, cfg.P, cfg.V, cfg.dtype)


class Layer:
    """One layer's device state: slot-ordered weights (optionally packed into
    the tile-blocked layout), the token->group table from a 65536-token
    profiling draw routed by the library, inputs, outputs and workspace."""

    def __init__(self, cfg, args, fuse_gather, blocked_weights):
        import numpy as np
        import torch
        from token_routing_shuffle_amd import moe, offline
        from token_routing_shuffle_amd import workload as wl
        dev = "cuda"
        self.cfg = cfg
        self.tables = tables = wl.make_tables(cfg)
        self.w = w = wl.make_weights(cfg, dev)
        self.x = wl.make_x(cfg, dev)
        d = offline.device_layer(cfg, tables, w, np.zeros(cfg.V, np.int32), dev)
        prof_x = wl.make_prof_x(cfg, dev)
        self.prof = offline.profile_routing(cfg, d, prof_x, tables.prof_tok)
        del prof_x
        epg = cfg.E // cfg.P
        d["lut"] = offline.lut_of_grouping(cfg, *self.prof, np.arange(cfg.E, dtype=np.int32) // epg)
        self.blocked = blocked = int(blocked_weights and cfg.dtype == "bf16")
        self.c = c = moe.make_cfg(cfg, fuse_gather=fuse_gather, weights_blocked=blocked)
        self.fuse_gather = fuse_gather
        if blocked:
            # one-time layout step, like the slot permutation: not part of the layer step
            for which, k13, k2 in ((moe.MOE_FFN_ROUTED, "W13", "W2"), (moe.MOE_FFN_SHARED, "Wsh13", "Wsh2")):
                if d.get(k13) is None:
                    continue
                b13, b2 = torch.empty_like(d[k13]), torch.empty_like(d[k2])
                moe.moe_pack_weights(c, which, d[k13], d[k2], b13, b2)
                d[k13], d[k2] = b13, b2
            torch.cuda.synchronize()
        self.d = d
        self.ws = moe.workspace(c)
        T, E, P = cfg.T, cfg.E, cfg.P
        self.tok = torch.as_tensor(tables.tok, device=dev)
        self.k_tok = None if tables.k_tok is None else torch.as_tensor(tables.k_tok, device=dev)
        self.out = torch.empty((T, cfg.H), dtype=torch.bfloat16 if cfg.dtype == "bf16" else torch.float32,
                               device=dev)
        self.row_ptr = torch.empty(T + 1, dtype=torch.int32, device=dev)
        self.pair = torch.empty(P * P, dtype=torch.int32, device=dev)
        self.ecount = torch.empty(E, dtype=torch.int32, device=dev)
        self.topk_slot = torch.empty(T * cfg.k, dtype=torch.int32, device=dev)
        self.W = moe.weights_struct(d)
        self.X = moe.inputs_struct(self.x, self.tok, self.k_tok)

    def run(self, steps, warmup, n_bd):
        """W warm-ups, K timed steps (events around GEMM1 only), then a
        breakdown pass with events around every stage."""
        import numpy as np
        import torch
        from token_routing_shuffle_amd import moe
        stream = torch.cuda.current_stream()
        up = moe.STAGES.index("ffn_up")

        def make_events(stages):
            evs = [torch.cuda.Event(enable_timing=True) if i // 2 in stages else None
                   for i in range(2 * moe.MOE_NSTAGES)]
            for e in evs:
                if e is not None:
                    e.record(stream)
            return evs

        base_ex = dict(row_ptr=self.row_ptr, pair_count=self.pair, expert_count=self.ecount,
                       topk_slot=self.topk_slot)
        for _ in range(warmup):
            moe.moe_forward(self.c, self.W, self.X, self.out, moe.exports_struct(base_ex), self.ws)
        torch.cuda.synchronize()
        ev_sets = [make_events({up}) for _ in range(steps)]
        exs = [moe.exports_struct(base_ex, events=ev_sets[i]) for i in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            moe.moe_forward(self.c, self.W, self.X, self.out, exs[i], self.ws)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_per_step = (t1 - t0) * 1e3 / steps
        up_ms = float(np.mean([ev_sets[i][2 * up].elapsed_time(ev_sets[i][2 * up + 1])
                               for i in range(steps)]))
        bd_sets = [make_events(set(range(moe.MOE_NSTAGES))) for _ in range(n_bd)]
        bd_exs = [moe.exports_struct(base_ex, events=bd_sets[i]) for i in range(n_bd)]
        torch.cuda.synchronize()
        for i in range(n_bd):
            moe.moe_forward(self.c, self.W, self.X, self.out, bd_exs[i], self.ws)
        torch.cuda.synchronize()
        stage_ms = {}
        for si, name in enumerate(moe.STAGES):
            v = [bd_sets[i][2 * si].elapsed_time(bd_sets[i][2 * si + 1]) for i in range(n_bd)]
            stage_ms[name] = float(np.mean(v))
        cfg = self.cfg
        A = int(self.row_ptr[cfg.T].item())
        counts = self.ecount.cpu().numpy()
        pc = self.pair.cpu().numpy().reshape(cfg.P, cfg.P)
        return dict(ms_per_step=ms_per_step, up_ms=up_ms, stage_ms=stage_ms, A=A, counts=counts,
                    n_touched=int((counts > 0).sum()),
                    lar=float(np.trace(pc)) / max(A, 1),
                    load=float(counts.max() / max(counts.mean(), 1e-9)), n_bd=n_bd)


def other_layer(name, args):
    """One more layer shape of the workload set, built and timed like the
    headline layer with fewer steps; its stages against their rooflines and
    the dispatch stage as a call of its own."""
    import torch
    from token_routing_shuffle_amd import moe
    from token_routing_shuffle_amd import workload as wl
    cfg = wl.CONFIGS[name]
    L = Layer(cfg, args, args.fuse_gather, args.blocked_weights)
    r = L.run(args.other_steps, 10, min(args.other_steps, 20))
    alg = algorithmic(cfg, r["A"], r["n_touched"])
    res = {"workload": describe(cfg), "value": round(cfg.T * 1e3 / r["ms_per_step"], 1), "unit": "tokens/s",
           "ms_per_step": round(r["ms_per_step"], 4), "steps": args.other_steps, "assignments": r["A"],
           "lar": round(r["lar"], 4), "max_over_mean_expert_load": round(r["load"], 3),
           "stages_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()}}
    if cfg.dtype == "bf16":
        res["ffn_up_roofline"] = binding_roofline(alg["ffn_up_flops"], alg["ffn_up_bytes"], r["up_ms"])
        res["stage_roofline"] = stage_rooflines(cfg, r["A"], alg, r["stage_ms"], r["up_ms"])
    res["dispatch"] = time_dispatch(cfg, L.c, L.d, L.x, L.tok, L.row_ptr, L.topk_slot, L.ws, r["A"], args,
                                    torch, moe, "cuda")
    del L
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(collectives are not implemented); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch
    from token_routing_shuffle_amd import moe
    from token_routing_shuffle_amd import workload as wl

    dev = "cuda"
    cfg = wl.CONFIGS[args.workload]
    L = Layer(cfg, args, args.fuse_gather, args.blocked_weights)
    T = cfg.T
    r = L.run(args.steps, args.warmup, min(args.steps, 50))
    ms_per_step, up_ms, stage_ms, A = r["ms_per_step"], r["up_ms"], r["stage_ms"], r["A"]

    if args.copy_calib_mb > 0:
        copy_calibration(args.copy_calib_mb, torch, dev)
    alg = algorithmic(cfg, A, r["n_touched"])
    traffic, traffic_note = measured_traffic(args.workload)
    roofline = binding_roofline(alg["ffn_up_flops"], alg["ffn_up_bytes"], up_ms)
    kname = "k_grouped_gemm<true,%d,%d,%s>" % (((256, 256) if moe_wide(cfg) else (128, 384))
                                               + ("true" if moe_stream_once(cfg) else "false",))
    roofline.update({"traffic": traffic, "traffic_unit": "bytes per launch", "traffic_source": traffic_note,
                     "kernel": kname + " (GEMM1 + SwiGLU, routed + shared)",
                     "touched_experts": r["n_touched"]})
    stage_roofline = stage_rooflines(cfg, A, alg, stage_ms, up_ms) if cfg.dtype == "bf16" else None
    down = binding_roofline(alg["ffn_down_flops"], alg["ffn_down_bytes"], stage_ms["ffn_down"]) \
        if cfg.dtype == "bf16" else None

    srs_sag = share = cosched = dispatch = None
    if not args.no_extras:
        dispatch = time_dispatch(cfg, L.c, L.d, L.x, L.tok, L.row_ptr, L.topk_slot, L.ws, A, args, torch, moe, dev)
        srs_sag = time_srs_sag(cfg, L.c, L.tables, args, torch, np, moe, wl, dev)
        share = group_share(cfg, L.c, L.d, L.x, L.tok, L.row_ptr, L.topk_slot, L.ws, args, torch, np, moe, dev)
        cosched = coschedule(cfg, L.c, L.tables, L.prof, L.tok, L.row_ptr, L.topk_slot, L.d["lut"], torch, np,
                             moe, dev)

    cpu = None
    if not args.no_cpu_baseline:
        n = args.cpu_sample or CPU_SAMPLE.get(args.workload, 4096)
        cpu = cpu_baseline(cfg, L.tables, L.w, L.x, np, torch, min(n, T))
    del L
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    others = None
    if not args.no_extras and not args.no_other_layers:
        others = {}
        for name in OTHER_LAYERS:
            if name != args.workload:
                others[name] = other_layer(name, args)

    res = {
        "metric": "MoE-layer tokens/s on 1 MI355X",
        "value": round(T * 1e3 / ms_per_step, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; Zipf token IDs, N(0,1) activations, N(0,1/fan_in) weights)",
        "config": {"workload": describe(cfg), "name": cfg.name,
                   "tokens": T, "assignments": A, "fuse_gather": args.fuse_gather,
                   "weights_blocked": int(args.blocked_weights and cfg.dtype == "bf16"),
                   "lar": round(r["lar"], 4),
                   "max_over_mean_expert_load": round(r["load"], 3)},
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stages_source": "separate pass of %d steps with HIP events around every stage "
                         "(each event pair adds GPU time; ffn_up in the timed steps: %.4f ms)"
                         % (r["n_bd"], up_ms),
        "stage_roofline": stage_roofline,
        "ffn_down_roofline": down,
        "roofline": roofline,
        "dispatch": dispatch,
        "srs_sag": srs_sag,
        "group_share": share,
        "coschedule": cosched,
        "other_layers": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def moe_wide(cfg):
    """256-wide GEMM1 tiles (2I and the shared 2*ns*Is multiples of 256)."""
    Ish = cfg.n_shared * cfg.I_shared
    return (2 * cfg.I) % 256 == 0 and (Ish == 0 or (2 * Ish) % 256 == 0)


def moe_stream_once(cfg):
    """The library's rule for streaming weight tiles read once per call: the
    routed experts' weights exceed 8x the 256 MB Infinity Cache."""
    return 3.0 * cfg.E * cfg.I * cfg.H * 2 > 8.0 * (256 << 20)


MALL_BYTES = 256 << 20


def stage_rooflines(cfg, A, alg, stage_ms, up_timed_ms):
    """Every stage of the layer step against its roofline: algorithmic bytes
    (HBM, 8 TB/s) or flops (dense bf16 MFMA, 2.5 PFLOP/s) over the stage's
    event-timed duration from the breakdown pass (GEMM1: the timed steps).
    The route stage is given both ways (its gate GEMM is a contraction, its
    bytes are the x read).  "mall_resident" marks stages whose bytes fit in
    the 256 MB Infinity Cache, where the HBM fraction can exceed what HBM
    alone would allow.  Each event pair adds a few microseconds to short
    stages."""
    T, H, E = cfg.T, cfg.H, cfg.E
    b = 2 if cfg.dtype == "bf16" else 4

    def hbm(nbytes, ms):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                "bytes": float(nbytes), "ms": round(ms, 4), "mall_resident": nbytes <= MALL_BYTES}

    def mfma(flops, ms):
        tf = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved_tflops": round(tf, 2),
                "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "flops": float(flops), "ms": round(ms, 4)}

    route_bytes = T * H * b + E * H * b + 8.0 * A + 4.0 * (T + 1) + 4.0 * T
    r = hbm(route_bytes, stage_ms["route"])
    r["mfma_frac"] = mfma(2.0 * T * H * E, stage_ms["route"])["frac"]
    return {
        "route": r,
        "shuffle_metadata": hbm(8.0 * T + 12.0 * A, stage_ms["shuffle"]),
        "ffn_up": mfma(alg["ffn_up_flops"], up_timed_ms),
        "ffn_down": mfma(alg["ffn_down_flops"], stage_ms["ffn_down"]),
        "combine": hbm(alg["combine_bytes"], stage_ms["combine"]),
    }


def time_dispatch(cfg, c, d, x, tok, row_ptr, topk_slot, ws, A, args, torch, moe, dev):
    """The dispatch stage as a call of its own (moe_shuffle: LUT lookup,
    counting sort and the gather of x into expert-contiguous rows) on the
    layer's routing, timed with one event pair around many calls; the same
    call without the gather gives the metadata part, the difference the
    gather kernel.  HBM roofline of the whole stage (x read once, A rows
    written, index metadata) and of the gather alone (T + A rows)."""
    T, H, E, P = cfg.T, cfg.H, cfg.E, cfg.P
    b = 2 if cfg.dtype == "bf16" else 4
    A_max = T * cfg.k
    i32 = dict(dtype=torch.int32, device=dev)
    o = [torch.empty(k, **i32) for k in (E, E + 1, P, P + 1, P * P, T, P + 1, A_max, A_max)]
    xs = torch.empty((A_max, H), dtype=x.dtype, device=dev)
    reps = max(10, min(args.steps, 100))

    def timed(dst):
        def call():
            moe.moe_shuffle(c, row_ptr, topk_slot, tok, d["lut"], x, *o, dst, ws)
        for _ in range(5):
            call()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            call()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    full_ms = timed(xs)
    meta_ms = timed(None)
    gather_ms = max(full_ms - meta_ms, 1e-6)
    nbytes = T * H * b + A * H * b + 8.0 * T + 12.0 * A
    gbytes = T * H * b + A * H * b
    gbs, ggbs = nbytes / (full_ms * 1e-3) / 1e9, gbytes / (gather_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes,
            "avg_launch_ms": round(full_ms, 4), "metadata_ms": round(meta_ms, 4),
            "gather": {"achieved": round(ggbs, 1), "frac": round(ggbs / HBM_PEAK_GBS, 4),
                       "bytes_per_launch": gbytes, "ms": round(gather_ms, 4)},
            "reps": reps, "mall_resident": nbytes <= MALL_BYTES,
            "note": "moe_shuffle with and without x_sorted, back to back; the layer step fuses "
                    "the gather into GEMM1's row loads"}


def time_srs_sag(cfg, c, tables, args, torch, np, moe, wl, dev):
    """The one-GPU shuffled reduce-scatter (P tensor-parallel partials of the
    layer input, reduced into predicted-group order) and shuffled all-gather
    (layer output back to token order) on the same workload, timed apart from
    the layer with HIP events; HBM roofline of each."""
    T, H, P = cfg.T, cfg.H, cfg.P
    b = 2 if cfg.dtype == "bf16" else 4
    x_part = wl.make_partials(cfg, P, dev)
    # tokens by (predicted group, token) for a v mod P table (any permutation
    # moves the same bytes)
    g = (tables.tok % P).astype(np.int64)
    perm = torch.as_tensor(np.lexsort((np.arange(T), g)).astype(np.int32), device=dev)
    y = torch.empty((T, H), dtype=x_part.dtype, device=dev)
    out = torch.empty_like(y)
    res = {}
    for name, fn, nbytes in (
            ("srs", lambda: moe.moe_srs(c, P, x_part, perm, y), P * T * H * b + T * H * b + 4 * T),
            ("sag", lambda: moe.moe_sag(c, y, perm, out), 2 * T * H * b + 4 * T)):
        for _ in range(args.warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(args.steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / args.steps
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes,
                     "avg_launch_ms": round(ms, 4)}
    res["partials"] = P
    return res


def group_share(cfg, c, d, x, tok, row_ptr, topk_slot, ws, args, torch, np, moe, dev):
    """One device's share under expert parallelism with P = EP devices: the
    routed expert FFN (GEMM1 + SwiGLU + GEMM2) over one placement group's
    slot range [g*E/P, (g+1)*E/P) with that group's real rows of this layer,
    timed with HIP events for every group (the slowest bounds an EP layer),
    next to the same call over all E slots."""
    T, H, E, P, I = cfg.T, cfg.H, cfg.E, cfg.P, cfg.I
    A_max = T * cfg.k
    i32 = dict(dtype=torch.int32, device=dev)
    o = {n: torch.empty(k, **i32) for n, k in (
        ("expert_count", E), ("expert_off", E + 1), ("group_count", P), ("group_off", P + 1),
        ("pair_count", P * P), ("tok_perm", T), ("tok_off", P + 1), ("s2a", A_max), ("a2s", A_max))}
    xs = torch.empty((A_max, H), dtype=x.dtype, device=dev)
    moe.moe_shuffle(c, row_ptr, topk_slot, tok, d["lut"], x, o["expert_count"], o["expert_off"],
                    o["group_count"], o["group_off"], o["pair_count"], o["tok_perm"], o["tok_off"],
                    o["s2a"], o["a2s"], xs, ws)
    y = torch.empty_like(xs)
    off = o["expert_off"]
    counts = o["expert_count"].cpu().numpy()
    epg = E // P
    reps = max(5, min(args.steps, 50))

    def timed(e0, e1):
        for _ in range(3):
            moe.moe_expert_ffn(c, moe.MOE_FFN_ROUTED, xs, None, None, None, off, d["W13"], d["W2"],
                               e0, e1, y, ws)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            moe.moe_expert_ffn(c, moe.MOE_FFN_ROUTED, xs, None, None, None, off, d["W13"], d["W2"],
                               e0, e1, y, ws)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    groups = []
    for g in range(P):
        rows = int(counts[g * epg:(g + 1) * epg].sum())
        ms = timed(g * epg, (g + 1) * epg)
        fl = 6.0 * rows * H * I
        groups.append({"group": g, "rows": rows, "ms": round(ms, 4),
                       "tflops": round(fl / (ms * 1e-3) / 1e12, 1)})
    all_ms = timed(0, E)
    rows_all = int(counts.sum())
    slow = max(groups, key=lambda r: r["ms"])
    return {"experts_per_group": epg, "reps": reps, "groups": groups,
            "slowest_group_ms": slow["ms"], "slowest_group_rows": slow["rows"],
            "all_slots_ms": round(all_ms, 4), "all_slots_rows": rows_all,
            "all_slots_tflops": round(6.0 * rows_all * H * I / (all_ms * 1e-3) / 1e12, 1),
            "note": "routed experts only; 6*rows*H*I flops per call"}


def coschedule(cfg, c, tables, prof, tok, row_ptr, topk_slot, lut0, torch, np, moe, dev):
    """Offline co-scheduling on the profiling draw's routing (65536 tokens,
    routed by the library): alternating optimisation of the expert grouping
    from the layer's random placement, then the local activation rate (LAR)
    of the timed layer's own tokens (held out from the profile) under both
    placements, and inter-request placement of 128-token requests on P
    data-parallel ranks against round robin."""
    T, E, P, V = cfg.T, cfg.E, cfg.P, cfg.V
    epg = E // P
    rp, sl, ptok = prof
    group0 = np.arange(E, dtype=np.int32) // epg           # slots as they are placed now
    lut = torch.empty(V, dtype=torch.int32, device=dev)
    cvp = torch.empty(V * P, dtype=torch.int32, device=dev)
    cpe = torch.empty(P * E, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    group, _, trace = moe.moe_optimize_placement(c, ptok.numel(), rp, sl, ptok, group0, lut, cvp, cpe,
                                                 max_iters=20)
    t_opt = time.perf_counter() - t0
    # held-out LAR from the timed layer's routing (slots of the random placement)
    A = int(row_ptr[T].item())
    rph = row_ptr.cpu().numpy()
    slh = topk_slot.cpu().numpy()[:A]
    t_of_a = np.repeat(np.arange(T), np.diff(rph))
    v = tables.tok[t_of_a]
    l0, l1 = lut0.cpu().numpy(), lut.cpu().numpy()
    lar0 = float((l0[v] == slh // epg).mean()) if A else 0.0
    lar1 = float((l1[v] == group[slh]).mean()) if A else 0.0
    # requests of 128 tokens to P ranks by the optimised table
    R = T // 128
    res_req = None
    if R >= P and R % P == 0:
        req_ptr = torch.arange(0, R * 128 + 1, 128, dtype=torch.int32, device=dev)
        hist = torch.empty(R * P, dtype=torch.int32, device=dev)
        moe.moe_request_group_hist(c, R, req_ptr, tok, lut, hist)
        Hh = hist.cpu().numpy().reshape(R, P).astype(np.int64)
        rank, best = moe.moe_balanced_assign(Hh)
        rr = int(sum(Hh[r, r % P] for r in range(R)))
        res_req = {"requests": R, "tokens_per_request": 128,
                   "dp_local_rate_round_robin": round(rr / (R * 128), 4),
                   "dp_local_rate_assigned": round(best / (R * 128), 4)}
    return {"profile_tokens": int(ptok.numel()), "objective_trace": [int(x) for x in trace],
            "optimiser_s": round(t_opt, 4), "lar_random_placement": round(lar0, 4),
            "lar_optimised_placement": round(lar1, 4), "requests": res_req}


def copy_calibration(mb, torch, dev):
    """One plain streaming kernel of known size for scaling HBM byte
    counters: bitwise_not over mb MiB of int32 (reads mb MiB, writes mb MiB).
    The source is written first and then pushed out of the 256 MB Infinity
    Cache by a 1 GiB fill, so the kernel's reads come from HBM."""
    n = (mb << 20) // 4
    src = torch.empty(n, dtype=torch.int32, device=dev).fill_(1)
    evict = torch.empty(1 << 28, dtype=torch.int32, device=dev).fill_(2)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst, evict


def _gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("ffn.hip", "common.h", "internal.h"):
        with open(os.path.join(ROOT, "token_routing_shuffle_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the GEMM1 kernel, from the committed summary of
    the rocprofv3 FETCH_SIZE / WRITE_SIZE passes (already scaled by the copy
    calibration).  None when there is no summary for this workload or when
    the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "ffn_up_gemm_%s_pmc.md" % workload)
    if not os.path.exists(path):
        return None, "no counter summary for this workload"
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- `"):
                k, _, v = line[3:].partition("`:")
                kv[k.strip()] = v.strip()
    try:
        if kv.get("source_sha256") != _gemm_source_hash():
            return None, "kernel changed since the counters were taken"
        return float(kv["traffic_bytes_per_launch"]), os.path.relpath(path, ROOT)
    except (KeyError, ValueError):
        return None, "counter summary unreadable"


class _HostExperts:
    """Host copies of single experts of a device weight stack [E, ...],
    fetched once each on first use (bf16 as uint16 bit patterns): the
    oracle's expert loop indexes the stack by original expert id, and a
    bounded token sample touches only a few of the 22.6 GB of experts of the
    largest layer."""

    def __init__(self, t, host):
        self.t, self.host, self.cache = t, host, {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = self.host(self.t[e])
        return self.cache[e]

    def prefetch(self, ids):
        for e in ids:
            self[e]


def cpu_info():
    """Logical CPUs this process may run on, and the CPU model."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def cpu_baseline(cfg, tables, w, x, np, torch, n_sample):
    """The oracle (unchanged) on a bounded sample of the same layer: gate
    logits, routing, dispatch metadata and the dense per-token MoE for the
    first n_sample tokens, repeated in whole passes until at least 10 s of
    CPU work; tokens/s = passes * n_sample / wall time.  The expert weights
    the sample routes to are copied to the host before the timing."""
    from oracle import moe_oracle as mo

    def h(t):
        if t is None:
            return None
        t = t.detach()
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    hw = {k: h(v) for k, v in w.items() if k not in ("W13", "W2")}
    W13, W2 = _HostExperts(w["W13"], h), _HostExperts(w["W2"], h)
    xs = h(x[:n_sample])
    tok = tables.tok[:n_sample]
    k_tok = None if tables.k_tok is None else tables.k_tok[:n_sample]

    def route():
        l64 = mo.logits(xs, hw["Wg"], tok, tables.pref, cfg.aff_bias if tables.pref is not None else 0.0)
        return mo.route(l64, cfg, k_tok, tables.ebias)

    sel0, _ = route()
    used = np.unique(sel0[sel0 >= 0])
    W13.prefetch(used)
    W2.prefetch(used)

    def one_pass():
        sel, wt = route()
        kt = k_tok if k_tok is not None else np.full(n_sample, cfg.k)
        rp = mo.row_ptr_of(kt)
        slot = tables.perm[sel[sel >= 0]]
        lut = np.arange(cfg.V, dtype=np.int32) % cfg.P
        mo.shuffle(rp, slot, tok, lut, cfg.E, cfg.P)
        mo.moe_output(xs, sel, wt, W13, W2, cfg.I, hw.get("Wsh13"), hw.get("Wsh2"),
                      cfg.n_shared, cfg.I_shared)

    passes = 0
    t0 = time.perf_counter()
    while True:
        one_pass()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or passes >= 30:
            break
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([1] + [i.get("num_threads", 1) for i in threadpool_info()])
    except Exception:
        pass
    nproc, model = cpu_info()
    return {"value": round(passes * n_sample / dt, 3), "unit": "tokens/s", "cores": threads,
            "nproc": nproc, "cpu_model": model, "kind": "oracle", "wall_s": round(dt, 2),
            "sample": "%d passes over the first %d of %d tokens of the same layer (fp64 numpy "
                      "oracle: logits, routing, dispatch metadata with a v mod P lookup table, "
                      "dense per-token MoE incl. shared experts; %d routed experts touched); "
                      "cores = the BLAS threads numpy's matrix products use (the rest of the "
                      "oracle is single-threaded numpy)" % (passes, n_sample, cfg.T, len(used))}


if __name__ == "__main__":
    main()
