"""Throughput bench of the LatentMoE layer on one MI355X.

One step = route (router top-k/softmax + permutation) + forward (down-proj,
shared experts, grouped expert FC1/FC2, combine + RMSNorm, up-proj) over one
batch of synthetic tokens, all through the C ABI.  Inputs are resident in HBM
before the timed region.  Several copies of every input (weights included)
are cycled through, so the expert weights are streamed from HBM rather than
re-read from the 256 MB last-level cache.

Prints one JSON line: tokens/s, the roofline of the dominant kernel (its
duration from HIP events recorded on the layer's stream around that kernel in
every timed step) and the CPU oracle's throughput on this host.

    python bench.py [--steps K] [--warmup W] [--workload decode|prefill|...]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (the w4a8 expert GEMMs issue at the fp8 rate)
LLC_BYTES = 256 << 20          # MI355X Infinity Cache
METRIC = "LatentMoE layer tokens/s at 1 GPU; grouped-GEMM TFLOP/s as % MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--copies", type=int, default=0, help="input copies cycled (0 = enough to beat the LLC)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle budget (0 = skip)")
    ap.add_argument("--no-stage-events", action="store_true")
    ap.add_argument("--api", choices=["layer", "route-forward"], default="layer",
                    help="where the logits are given: latent_moe_layer (one call, its plan reused) or "
                         "latent_moe_route + latent_moe_forward")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph",
                    help="graph: each copy's route+forward captured once in a HIP graph and replayed")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 5 plain device copies of BYTES bytes (the reference kernel that scales the "
                         "PMC FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    return ap.parse_args()


class Hip:
    """The few HIP runtime calls the bench needs for its own events."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.lib.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b):
        self.lib.hipEventSynchronize(ctypes.c_void_p(b))
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "latentmoe_expert_layer_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, src_hash):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it
    was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, inp_host, budget_s):
    """The oracle (as it stands) on this host's cores: routing and permutation
    of the whole batch, then the layer on consecutive token chunks (the whole
    batch at a time when it has <= 256 tokens) until the budget is used."""
    import oracle
    cores = oracle.num_threads()
    t0 = time.perf_counter()
    if cfg.rows_mode:
        ids, w = inp_host["ids"], inp_host["weights"]
    elif cfg.router_gemm:
        logits, _ = oracle.router_logits(inp_host["x"], inp_host["w_in"], inp_host["w_r"])
        ids, w = oracle.route(logits, cfg.k)
    else:
        ids, w = oracle.route(inp_host["logits"], cfg.k)
    oracle.permute(ids, cfg.E)
    chunk = min(cfg.T, 256)
    done = 0
    while True:
        toks = [(done + i) % cfg.T for i in range(chunk)]
        oracle.layer(inp_host, ids, w, eval_tokens=toks, act_quant=not cfg.w4a16)
        done += chunk
        el = time.perf_counter() - t0
        if el >= budget_s or done >= 10000 * cfg.T:
            break
    return {"value": done / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{'router gate + ' if cfg.router_gemm else ''}route + permute of the whole {cfg.name} "
                      f"batch ({cfg.T} tokens), then the layer on "
                      f"{done} tokens in chunks of {chunk}, {el:.1f} s in total"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer is built and "
              "measured on a single MI355X", file=sys.stderr)
        return 2
    import torch

    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}))
        return 0

    import latentmoe_expert_layer_amd as lm
    import workloads as W

    cfg = W.CONFIGS[args.workload]
    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream

    # ---------------- inputs: several resident copies, distinct seeds
    wbytes = (3 * cfg.E * cfg.I * cfg.l) * (0.53 if cfg.mxfp4 else 2)
    copies = args.copies or max(2, min(8, -(-2 * LLC_BYTES // max(int(wbytes), 1))))
    wfmt = (lm.LMOE_WFMT_MXFP4_W4A16 if cfg.w4a16 else lm.LMOE_WFMT_MXFP4) if cfg.mxfp4 else lm.LMOE_WFMT_BF16
    P = lambda t: None if t is None else t.data_ptr()
    sets = []
    for c in range(copies):
        inp = W.make_inputs(W.LayerConfig(**{**cfg.__dict__, "seed": c}), device="cuda")
        T, E, k = cfg.T, cfg.E, cfg.k
        R = T * k
        rws = torch.empty(lm.route_workspace_size(T, E, k), dtype=torch.uint8, device="cuda")
        fws = torch.empty(max(256, lm.forward_workspace_size(T, E, k, cfg.d, cfg.l, cfg.I, cfg.S, cfg.Is, wfmt,
                                                            cfg.rows_mode)), dtype=torch.uint8, device="cuda")
        out = dict(topk_ids=torch.empty(T, k, dtype=torch.int32, device="cuda"),
                   topk_w=torch.empty(T, k, dtype=torch.float32, device="cuda"),
                   sorted_row=torch.empty(R, dtype=torch.int32, device="cuda"),
                   row_pos=torch.empty(R, dtype=torch.int32, device="cuda"),
                   offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                   y=torch.empty(T, cfg.l if cfg.rows_mode else cfg.d, dtype=torch.bfloat16, device="cuda"))
        logits = None
        if cfg.router_gemm:   # latent_moe_layer: the logits are computed from the latent
            logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
            ra = lm.RouteArgs(T=T, E=E, k=k, topk_ids=P(out["topk_ids"]), topk_w=P(out["topk_w"]),
                              sorted_row=P(out["sorted_row"]), row_pos=P(out["row_pos"]),
                              offsets=P(out["offsets"]), workspace=P(rws), workspace_bytes=rws.numel())
        elif cfg.rows_mode:
            ra = lm.RouteArgs(T=T, E=E, k=k, ids_in=P(inp["ids"]), weights_in=P(inp["weights"]),
                              sorted_row=P(out["sorted_row"]), row_pos=P(out["row_pos"]),
                              offsets=P(out["offsets"]), workspace=P(rws), workspace_bytes=rws.numel())
        else:
            ra = lm.RouteArgs(T=T, E=E, k=k, logits=P(inp["logits"]), topk_ids=P(out["topk_ids"]),
                              topk_w=P(out["topk_w"]), sorted_row=P(out["sorted_row"]),
                              row_pos=P(out["row_pos"]), offsets=P(out["offsets"]), workspace=P(rws),
                              workspace_bytes=rws.numel())
        mx = cfg.mxfp4
        fa = lm.ForwardArgs(d=cfg.d, l=cfg.l, I=cfg.I, S=cfg.S, Is=cfg.Is, wfmt=wfmt, norm_eps=cfg.eps,
                            x=P(inp["x"]), w_in=P(inp.get("w_in")), w1=P(inp["w1q" if mx else "w1"]),
                            w3=P(inp["w3q" if mx else "w3"]), w2=P(inp["w2q" if mx else "w2"]),
                            s1=P(inp.get("s1")), s3=P(inp.get("s3")), s2=P(inp.get("s2")),
                            norm_w=P(inp.get("norm_w")), w_out=P(inp.get("w_out")),
                            ws1=P(inp.get("ws1")), ws3=P(inp.get("ws3")), ws2=P(inp.get("ws2")),
                            y=P(out["y"]), workspace=P(fws), workspace_bytes=fws.numel())
        sets.append(dict(inp=inp, rws=rws, fws=fws, out=out, ra=ra, fa=fa, logits=logits, plan=None))
    torch.cuda.synchronize()

    n_ev = lm.N_STAGE_EVENTS
    use_events = not args.no_stage_events

    one_call = cfg.router_gemm or (args.api == "layer" and not cfg.rows_mode)

    def run_call(s, strm, events=None):
        """One layer call on copy s: latent_moe_layer (its plan reused across
        calls; with the router gate or the given logits) or latent_moe_route +
        latent_moe_forward."""
        if one_call:
            if s["plan"] is not None:
                lm.latent_moe_plan_set_stage_events(s["plan"], events)
            gate = P(s["inp"]["w_r"]) if cfg.router_gemm else None
            s["plan"] = lm.latent_moe_layer(s["ra"], gate, P(s["logits"]), s["fa"], strm, s["plan"])
            return
        plan = lm.latent_moe_route(s["ra"], strm)
        if events is not None:
            lm.latent_moe_plan_set_stage_events(plan, events)
        lm.latent_moe_forward(plan, s["fa"], strm)
        lm.latent_moe_free(plan)

    def step(i, events=None):
        run_call(sets[i % copies], stream, events)

    # every copy runs once before the warm-up (untimed), so each one's routing
    # outputs, which the algorithmic byte count below reads, exist however
    # few steps are asked for
    for c in range(copies):
        step(c)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    mode = args.mode
    graphs = []
    if mode == "graph":
        try:
            cap = torch.cuda.Stream()
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    run_call(sets[c], torch.cuda.current_stream().cuda_stream)
                graphs.append(g)
            for i in range(args.warmup):
                graphs[i % copies].replay()
            torch.cuda.synchronize()
        except Exception as exc:  # capture unsupported here: time eager launches instead
            print(f"graph capture failed ({exc}); timing eager launches", file=sys.stderr)
            mode, graphs = "eager", []
            torch.cuda.synchronize()

    def timed(run_steps, with_events):
        """K steps between two events on the layer's stream; eager steps may
        carry one set of stage events each (read after the region)."""
        ev_sets = [[hip.event() for _ in range(n_ev)] for _ in range(args.steps)] if with_events else None
        t0, t1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(t0, stream)
        run_steps(ev_sets)
        hip.record(t1, stream)
        torch.cuda.synchronize()
        return hip.elapsed_ms(t0, t1), ev_sets

    def eager_steps(ev_sets):
        for i in range(args.steps):
            step(i, ev_sets[i] if ev_sets is not None else None)

    def graph_steps(_):
        for i in range(args.steps):
            graphs[i % copies].replay()

    wall0 = time.perf_counter()
    if mode == "graph":
        total_ms, _ = timed(graph_steps, False)
    else:
        total_ms, _ = timed(eager_steps, False)
    wall = time.perf_counter() - wall0
    ms_per_step = total_ms / args.steps
    tokens_per_s = cfg.T * args.steps / (total_ms / 1e3)

    # kernel durations: a second timed region of eager steps, each carrying the
    # library's stage events (events inside a replayed graph cannot be timed)
    stages, eager_ms = {}, None
    if use_events:
        eager_total, ev_sets = timed(eager_steps, True)
        eager_ms = eager_total / args.steps
        for j, name in enumerate(lm.STAGES):
            vals = [hip.elapsed_ms(ev[j], ev[j + 1]) for ev in ev_sets]
            stages[name] = 1e3 * sum(vals) / len(vals)
        fwd = [hip.elapsed_ms(ev[0], ev[n_ev - 1]) for ev in ev_sets]
        stages["forward_total"] = 1e3 * sum(fwd) / len(fwd)

    # ---------------- algorithmic work (per launch, averaged over the copies)
    T, E, k, d, l, I, S, Is = cfg.T, cfg.E, cfg.k, cfg.d, cfg.l, cfg.I, cfg.S, cfg.Is
    R = T * k
    touched = sum(int(((s["out"]["offsets"][1:] - s["out"]["offsets"][:-1]) > 0).sum()) for s in sets) / copies
    wb = 0.5 + 1 / 32 if cfg.mxfp4 else 2        # bytes per expert weight element (MXFP4: code + scale share)
    fc1_bytes = touched * 2 * I * l * wb + T * l * 2 + R * I * 2
    fc2_bytes = touched * l * I * wb + R * I * 2 + R * l * 2
    fc1_flop = 2.0 * R * l * 2 * I
    fc2_flop = 2.0 * R * I * l
    dense_flop = 0.0 if cfg.rows_mode else 2.0 * T * d * (l + 2 * S * Is) + 2.0 * T * (l + S * Is) * d
    layer_flop = fc1_flop + fc2_flop + dense_flop
    dense_bytes = 0 if cfg.rows_mode else 2 * (T * d + (l + 2 * S * Is) * d + T * l + T * S * Is + d * (l + S * Is) + T * d)
    route_bytes = T * E * 4 + R * (4 + 4 + 4 + 4 + 4)
    if cfg.router_gemm:   # the gate GEMM: z and the gate in, fp32 logits out
        layer_flop += 2.0 * T * l * E
        route_bytes += T * l * 2 + E * l * 2 + T * E * 4
    combine_bytes = R * l * 2 + T * l * 2 + R * 8
    layer_bytes = fc1_bytes + fc2_bytes + dense_bytes + route_bytes + combine_bytes

    # the library runs the w4a16 expert MLP at latent = intermediate = 256 as
    # one launch (its duration is the FC1 stage; H never reaches HBM)
    fused_mlp = cfg.mxfp4 and cfg.w4a16 and l == 256 and I == 256
    roofline = None
    if use_events:
        dom = "fc1" if fused_mlp else max(("fc1", "fc2"), key=lambda n: stages[n])
        dom_bytes = fc1_bytes if dom == "fc1" else fc2_bytes
        dom_flop = fc1_flop if dom == "fc1" else fc2_flop
        if fused_mlp:
            dom_bytes = fc1_bytes + fc2_bytes - 2 * R * I * 2
            dom_flop = fc1_flop + fc2_flop
        dur_s = stages[dom] / 1e6
        ai = dom_flop / dom_bytes
        fp8 = cfg.mxfp4 and not cfg.w4a16   # w4a8 issues at the fp8 rate; w4a16 multiplies in bf16
        mfma_peak = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS
        bound = "hbm" if ai < mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
        # which kernel ran the grouped GEMMs (the library's own choice: MXFP4
        # w4a8 -> block-scaled kernel; MXFP4 w4a16 -> its weight-streaming
        # kernel; <= 32 rows per expert on average -> weight-streaming kernel;
        # otherwise the LDS-tiled kernel)
        if fused_mlp:
            kern, src = "skinny_w4a16_mlp_kernel", "skinny.hip"
        elif cfg.mxfp4 and cfg.w4a16:
            kern, src = "skinny_w4a16_kernel", "skinny.hip"
        elif cfg.mxfp4:
            kern, src = "mx_grouped_kernel", "mx.hip"
        elif R <= 32 * E:   # LDS-staged weight loads when the GEMM's K is a multiple of 128
            kern = "skinny_lds_kernel" if (l if dom == "fc1" else I) % 128 == 0 else "skinny_grouped_kernel"
            src = "skinny.hip"
        else:
            kern, src = "tiled_gemm_kernel", "gemm.hip"
        # the kernel's source with the headers every kernel includes
        traffic = measured_traffic(f"{dom}", cfg.name, source_hash(src, "common.h", "kernels.h"))
        if bound == "hbm":
            achieved = dom_bytes / dur_s / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                        "kernel": f"{kern} ({'fc1+fc2' if fused_mlp else dom})",
                        "algorithmic_bytes_per_launch": int(dom_bytes),
                        "avg_launch_us": round(stages[dom], 2)}
        else:
            achieved = dom_flop / dur_s / 1e12
            roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": mfma_peak,
                        "unit": "TFLOP/s", "frac": round(achieved / mfma_peak, 4), "traffic": traffic,
                        "kernel": f"{kern} ({dom})", "algorithmic_flop_per_launch": dom_flop,
                        "avg_launch_us": round(stages[dom], 2)}

    extra = {
        "mode": mode,
        "api": "latent_moe_layer" if one_call else "latent_moe_route + latent_moe_forward",
        "eager_ms_per_step_with_stage_events": None if eager_ms is None else round(eager_ms, 5),
        "copies_cycled": copies,
        "wall_s": round(wall, 3),
        "stage_us": {n: round(v, 2) for n, v in stages.items()},
        "layer_tflops": round(layer_flop / (ms_per_step / 1e3) / 1e12, 2),
        "layer_hbm_gbs": round(layer_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "layer_hbm_frac": round(layer_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_algorithmic_bytes": int(layer_bytes),
        "touched_experts": touched,
    }
    if cfg.router_gemm:
        extra["stage_note"] = ("shared_gate_up also covers the router gate GEMM, the top-k and the permutation "
                               "(latent_moe_layer runs them between the down-projection and FC1)")
    elif one_call:
        extra["stage_note"] = ("down_proj also covers the top-k (in the same launch at T <= 512) and "
                               "shared_gate_up the permutation (latent_moe_layer with the logits given)")
    if use_events:
        for n, fl, by in (("fc1", fc1_flop, fc1_bytes), ("fc2", fc2_flop, fc2_bytes)):
            us = stages[n]
            if fused_mlp:   # one launch: report it under fc1 with both GEMMs' work
                if n == "fc2":
                    continue
                fl, by = fc1_flop + fc2_flop, fc1_bytes + fc2_bytes - 2 * R * I * 2
            extra[f"{n}_tflops"] = round(fl / us / 1e6, 2)
            extra[f"{n}_mfma_frac"] = round(fl / us / 1e6 / (FP8_PEAK_TFLOPS if cfg.mxfp4 and not cfg.w4a16
                                                              else BF16_PEAK_TFLOPS), 4)
            extra[f"{n}_hbm_frac"] = round(by / us / 1e3 / HBM_PEAK_GBS, 4)

    cpu = None
    if args.cpu_seconds > 0:
        from tests.parity import to_host
        cpu = cpu_baseline(cfg, to_host(sets[0]["inp"]), args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16 (experts: MXFP4 weights upcast to bf16, bf16 activations)" if cfg.w4a16 else
                  "bf16 (experts: MXFP4 weights x MXFP8 activations)") if cfg.mxfp4 else "bf16",
        "data": ("synthetic (seeded N(0,1) activations, N(0,0.02) bf16 weights, router gate "
                 "N(0, 1/sqrt(latent*d*0.02^2)) on the latent)" if cfg.router_gemm else
                 "synthetic (seeded N(0,1) activations, N(0,0.02) bf16 weights, gap-separated N(0,1) logits)"),
        "config": {"workload": (f"{cfg.name}: {T} received rows, {E} local experts, latent {l}, SwiGLU I={I}, "
                                f"Zipf({cfg.zipf_s}) expert load, combine weights given") if cfg.rows_mode else
                               (f"{cfg.name}: T={T} tokens, d={d} -> latent {l}, E={E} top-{k} + {S} shared, "
                                f"SwiGLU I={I}, shared I={Is}, RMSNorm on"
                                + (", logits computed by the router gate on the latent (latent_moe_layer)"
                                   if cfg.router_gemm else "")
                                + ((", MXFP4 experts (w4a16)" if cfg.w4a16 else ", MXFP4 experts (w4a8)")
                                   if cfg.mxfp4 else "")),
                   "T": T, "d": d, "latent": l, "E": E, "k": k, "shared": S, "I": I, "Is": Is},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
