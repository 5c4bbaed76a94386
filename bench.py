"""Throughput bench of the LatentMoE layer on one MI355X.

One step = the whole layer over one batch of synthetic tokens through the C
ABI: routing of the given logits (top-k/softmax + permutation) and the forward
(down-proj, shared experts, grouped expert FC1/FC2, combine + RMSNorm,
up-proj).  Inputs are resident in HBM before the timed region.  Several copies
of every input (weights included) are cycled through, so the expert weights
are streamed from HBM rather than re-read from the 256 MB last-level cache.

The headline workload is the prefill-shaped batch (8192 tokens, hidden 7168,
latent 2048, 896 experts top-16 + 2 shared, SwiGLU 512, bf16): the largest
bf16 configuration that fits one GPU.  The decode batch, the MXFP4 prefill
batch and one expert-parallel rank's share are measured in the same run and
reported under ``extra.workloads``.

Prints one JSON line: tokens/s, the per-step distribution, the roofline of the
dominant kernel (its duration from HIP events that the library records at that
kernel's own start and end, in every step of an eager timed pass), the
measured shader clock, and the CPU oracle's throughput on this host.

    python bench.py [--steps K] [--warmup W] [--workload prefill|decode|...]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (the w4a8 expert GEMMs issue at the fp8 rate)
LLC_BYTES = 256 << 20          # MI355X Infinity Cache
METRIC = "LatentMoE layer tokens/s at 1 GPU; grouped-GEMM TFLOP/s as % MFMA peak"
DEFAULT_EXTRA = "prefill@tiled,prefill_bf16_16k,decode,decode_os,decode_w4a16,decode_w4a16_os,prefill_mxfp4,prefill_w4a16,ep_share"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--extra-workloads", default=DEFAULT_EXTRA,
                    help="comma-separated workloads also measured and reported under extra.workloads ('' = none); "
                         "name@rows / name@tiled overrides --wlayout for one of them")
    ap.add_argument("--wlayout", choices=["tiled", "rows"], default="rows",
                    help="bf16 expert weights: tile-packed once at load time (latent_moe_pack_weights, outside the "
                         "timed region) or row-major; shapes the packed layout does not serve stay row-major")
    ap.add_argument("--copies", type=int, default=0, help="input copies cycled (0 = enough to beat the LLC)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle budget (0 = skip)")
    ap.add_argument("--no-stage-events", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip the shader-clock sampling phase")
    ap.add_argument("--api", choices=["layer", "route-forward"], default="layer",
                    help="where the logits are given: latent_moe_layer (one call, its plan reused) or "
                         "latent_moe_route + latent_moe_forward")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph",
                    help="graph: each copy's layer call captured once in a HIP graph and replayed")
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

    def destroy(self, e):
        self.lib.hipEventDestroy(ctypes.c_void_p(e))

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


def pct(vals, q):
    s = sorted(vals)
    if not s:
        return None
    i = min(len(s) - 1, max(0, int(round(q * (len(s) - 1)))))
    return s[i]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class ClockSampler:
    """Samples the GPU's shader (gfx) clock in MHz from a background thread
    while a phase of steps runs: the mean over the XCDs of amdsmi's GPU
    metrics (``current_gfxclks``), else amdsmi's clock info.
    The metrics refresh every 0.1-0.3 s, so the phase lasts >= 1 s and the
    first 0.3 s of samples are dropped."""

    SETTLE_S = 0.3

    def __init__(self):
        self.samples, self.source, self._stop = [], None, threading.Event()
        self._read = self._setup()

    def _setup(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if handles:
                h = handles[0]

                def read_metrics():
                    m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                    v = m.get("current_gfxclks")
                    if isinstance(v, (list, tuple)):
                        vals = [float(x) for x in v if isinstance(x, (int, float)) and x > 0]
                        if vals:
                            return sum(vals) / len(vals)
                    v = m.get("current_gfxclk")
                    if isinstance(v, (int, float)) and v > 0:
                        return float(v)
                    raise RuntimeError("no gfx clock in the metrics")
                try:
                    read_metrics()
                    self.source = "amdsmi gpu metrics: mean of current_gfxclks over the XCDs"
                    return read_metrics
                except Exception:
                    pass

                def read_info():
                    return float(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"])
                read_info()
                self.source = "amdsmi_get_clock_info(GFX)"
                return read_info
        except Exception:
            pass
        return None

    def _loop(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            try:
                v = self._read()
                if time.perf_counter() - t0 >= self.SETTLE_S:
                    self.samples.append(v)
            except Exception:
                pass
            time.sleep(0.01)

    def run_during(self, fn):
        self.samples = []
        self._stop.clear()
        if self._read is None:
            fn()
            return
        th = threading.Thread(target=self._loop, daemon=True)
        th.start()
        try:
            fn()
        finally:
            self._stop.set()
            th.join()

    def close(self):
        """End the amdsmi session (opened in _setup), so nothing of it
        outlives the run."""
        if self._read is not None:
            try:
                import amdsmi
                amdsmi.amdsmi_shut_down()
            except Exception:
                pass
            self._read = None

    def summary(self):
        if not self.samples:
            return None
        return {"median_mhz": round(statistics.median(self.samples), 1), "min_mhz": round(min(self.samples), 1),
                "max_mhz": round(max(self.samples), 1), "samples": len(self.samples), "source": self.source,
                "spec_peak_mhz": 2400}


def grouped_kernel(cfg, dom, fused_mlp, packed=False):
    """Which kernel runs the grouped GEMM ``dom`` (the library's own choice:
    MXFP4 w4a8 -> block-scaled kernel (its direct-to-LDS ring form when K is
    a multiple of 512); MXFP4 w4a16 -> its weight-streaming
    kernels at <= 32 rows per expert on average, else the direct-to-LDS ring
    with the weights upcast in registers (K a multiple of 512) or the
    register-staged grouped kernel in its MXFP4 form; bf16 at <= 32 rows per expert on average
    -> weight-streaming kernel; otherwise, tile-packed weights -> the
    register-staged grouped kernel in its packed form, row-major weights -> the
    64-wide direct-to-LDS ring when K is a multiple of 64 and at least 192,
    else the general tiled kernel)."""
    R = cfg.T * cfg.k
    K = cfg.l if dom == "fc1" else cfg.I
    if fused_mlp:
        return "skinny_w4a16_mlp_kernel", "skinny.hip"
    if cfg.mxfp4 and cfg.w4a16:
        if R <= 32 * cfg.E:
            return "skinny_w4a16_kernel", "skinny.hip"
        if K % 512 == 0:
            return "w4ring_grouped_kernel", "gemm.hip"
        return "grouped_tiled_kernel (MXFP4 w4a16)", "gemm.hip"
    if cfg.mxfp4:
        if K % 512 == 0:
            return "mx_ring_kernel", "mx.hip"
        return "mx_grouped_kernel", "mx.hip"
    if R <= 32 * cfg.E:
        return ("skinny_lds_kernel" if K % 128 == 0 else "skinny_grouped_kernel"), "skinny.hip"
    if packed:
        return "grouped_tiled_kernel (tile-packed)", "gemm.hip"
    if K % 64 == 0 and K >= 192:
        return "ring64_grouped_kernel", "gemm.hip"
    return "tiled_gemm_kernel", "gemm.hip"


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
    chunk = min(cfg.T, 256 if cfg.T <= 4096 else 64)
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


def cpu_single_thread(names, budget_s):
    """Single-thread oracle tokens/s on the small configurations."""
    import oracle
    import workloads as W
    out = {}
    prev = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        for n in names:
            cfg = W.CONFIGS[n]
            inp = W.make_inputs(cfg)
            ids, w = oracle.route(inp["logits"], cfg.k)
            oracle.permute(ids, cfg.E)
            t0, done = time.perf_counter(), 0
            chunk = min(cfg.T, 32)
            while True:
                toks = [(done + i) % cfg.T for i in range(chunk)]
                oracle.layer(inp, ids, w, eval_tokens=toks)
                done += chunk
                el = time.perf_counter() - t0
                if el >= budget_s:
                    break
            out[n] = {"tokens_per_s": round(done / el, 1), "tokens": done, "seconds": round(el, 2)}
    finally:
        oracle.set_num_threads(prev)
    return out


def packed_layout_serves(cfg):
    """The tile-packed layout serves bf16 experts with l and I multiples of
    128, at least 256."""
    return (not cfg.mxfp4) and cfg.l % 128 == 0 and cfg.I % 128 == 0 and cfg.l >= 256 and cfg.I >= 256


def measure(cfg, args, hip, lm, W, torch, stream, clock=None, wlayout="tiled"):
    """Builds the resident input copies of ``cfg``, times K steps (graph
    replays, one event per step boundary), then an eager pass with the
    library's stage events; returns the figures of this workload."""
    packed = wlayout == "tiled" and packed_layout_serves(cfg)
    wbytes = (3 * cfg.E * cfg.I * cfg.l) * (0.53 if cfg.mxfp4 else 2)
    copies = args.copies or max(2, min(8, -(-2 * LLC_BYTES // max(int(wbytes), 1))))
    wfmt = (lm.LMOE_WFMT_MXFP4_W4A16 if cfg.w4a16 else lm.LMOE_WFMT_MXFP4) if cfg.mxfp4 else lm.LMOE_WFMT_BF16
    P = lambda t: None if t is None else t.data_ptr()
    sets = []
    for c in range(copies):
        inp = W.make_inputs(W.LayerConfig(**{**cfg.__dict__, "seed": c}), device="cuda")
        if packed:   # load-time layout change of the expert weights (same values)
            for n in ("w1", "w3", "w2"):
                inp[n] = lm.pack_weights(inp[n])
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
                            y=P(out["y"]), workspace=P(fws), workspace_bytes=fws.numel(),
                            wlayout=lm.LMOE_WLAYOUT_TILED if packed else lm.LMOE_WLAYOUT_ROWS)
        sets.append(dict(inp=inp, rws=rws, fws=fws, out=out, ra=ra, fa=fa, logits=logits, plan=None))
    torch.cuda.synchronize()

    n_ev = lm.N_STAGE_EVENTS
    use_events = not args.no_stage_events and not cfg.os   # the output-stationary call keeps no plan
    one_call = cfg.router_gemm or (args.api == "layer" and not cfg.rows_mode)

    def run_call(s, strm, events=None):
        """One layer call on copy s: latent_moe_layer (its plan reused across
        calls; with the router gate or the given logits), latent_moe_layer_os,
        or latent_moe_route + latent_moe_forward."""
        if cfg.os:
            lm.latent_moe_layer_os(s["ra"], s["fa"], strm)
            return
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

    def one_step(i, events=None):
        if mode == "graph":
            graphs[i % copies].replay()
        else:
            step(i, events)

    # ---- timed region: K steps, an event at every step boundary on the layer's stream
    K = args.steps
    bounds = [hip.event() for _ in range(K + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    hip.record(bounds[0], stream)
    for i in range(K):
        one_step(i)
        hip.record(bounds[i + 1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = hip.elapsed_ms(bounds[0], bounds[K])
    per_step = [hip.elapsed_ms(bounds[i], bounds[i + 1]) for i in range(K)]
    for e in bounds:
        hip.destroy(e)
    ms_per_step = total_ms / K
    tokens_per_s = cfg.T * K / (total_ms / 1e3)

    # ---- shader clock while the same steps run (a separate phase of >= 1.2 s)
    clk = None
    if clock is not None:
        n_clk = max(K, int(1.2 / max(ms_per_step / 1e3, 1e-6)))

        def clk_phase():
            for i in range(n_clk):
                one_step(i)
                if i % 64 == 63:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
        clock.run_during(clk_phase)
        clk = clock.summary()

    # ---- kernel durations: eager steps, each carrying the library's stage
    # events (events inside a replayed graph cannot be timed)
    stages, eager_ms = {}, None
    if use_events:
        ev_sets = [[hip.event() for _ in range(n_ev)] for _ in range(K)]
        t0, t1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(t0, stream)
        for i in range(K):
            step(i, ev_sets[i])
        hip.record(t1, stream)
        torch.cuda.synchronize()
        eager_ms = hip.elapsed_ms(t0, t1) / K
        for j, name in enumerate(lm.STAGES):
            vals = [hip.elapsed_ms(ev[j], ev[j + 1]) for ev in ev_sets]
            stages[name] = 1e3 * sum(vals) / len(vals)
        fwd = [hip.elapsed_ms(ev[0], ev[n_ev - 1]) for ev in ev_sets]
        stages["forward_total"] = 1e3 * sum(fwd) / len(fwd)
        # the plans keep the events: switch them off before they are destroyed
        for s in sets:
            if s["plan"] is not None:
                lm.latent_moe_plan_set_stage_events(s["plan"], None)
        for ev in ev_sets:
            for e in ev:
                hip.destroy(e)
        hip.destroy(t0)
        hip.destroy(t1)

    # ---- algorithmic work (per launch, averaged over the copies)
    T, E, k, d, l, I, S, Is = cfg.T, cfg.E, cfg.k, cfg.d, cfg.l, cfg.I, cfg.S, cfg.Is
    R = T * k
    if cfg.os:   # no offsets: count the experts the router picked
        touched = sum(int(torch.unique(s["out"]["topk_ids"]).numel()) for s in sets) / copies
    else:
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
    if cfg.rows_mode:
        route_bytes = R * (4 + 4 + 4 + 4)
    if cfg.router_gemm:   # the gate GEMM: z and the gate in, fp32 logits out
        layer_flop += 2.0 * T * l * E
        route_bytes += T * l * 2 + E * l * 2 + T * E * 4
    combine_bytes = R * l * 2 + T * l * 2 + R * 8
    if cfg.rows_mode:
        combine_bytes = 2 * R * l * 2 + R * 8
    layer_bytes = fc1_bytes + fc2_bytes + dense_bytes + route_bytes + combine_bytes

    # the library runs the w4a16 expert MLP at latent = intermediate = 256 as
    # one launch (its duration is the FC1 stage; H never reaches HBM)
    fused_mlp = cfg.mxfp4 and cfg.w4a16 and l == 256 and I == 256 and cfg.T * cfg.k <= 32 * cfg.E
    fp8 = cfg.mxfp4 and not cfg.w4a16   # w4a8 issues at the fp8 rate; w4a16 multiplies in bf16
    mfma_peak = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS
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
        bound = "hbm" if ai < mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
        kern, src = grouped_kernel(cfg, dom, fused_mlp, packed)
        # the kernel's source with the headers every kernel includes
        traffic = measured_traffic(f"{dom}", cfg.name, source_hash(src, "common.h", "kernels.h"))
        if bound == "hbm":
            achieved = dom_bytes / dur_s / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                        "kernel": f"{kern} ({'fc1+fc2' if fused_mlp else dom})",
                        "algorithmic_bytes_per_launch": int(dom_bytes),
                        "avg_launch_us": round(stages[dom], 2),
                        "mfma_tflops": round(dom_flop / dur_s / 1e12, 1),
                        "mfma_frac": round(dom_flop / dur_s / 1e12 / mfma_peak, 4),
                        "arithmetic_intensity_flop_per_byte": round(ai, 1)}
        else:
            achieved = dom_flop / dur_s / 1e12
            roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": mfma_peak,
                        "unit": "TFLOP/s", "frac": round(achieved / mfma_peak, 4), "traffic": traffic,
                        "kernel": f"{kern} ({dom})", "algorithmic_flop_per_launch": dom_flop,
                        "avg_launch_us": round(stages[dom], 2),
                        "hbm_gbs": round(dom_bytes / dur_s / 1e9, 1)}

    res = {
        "ms_per_step": ms_per_step, "tokens_per_s": tokens_per_s, "mode": mode,
        "expert_weight_layout": ("tile-packed at load time (latent_moe_pack_weights)" if packed else
                                 "MXFP4 codes + scales" if cfg.mxfp4 else "row-major [E, N, K]"),
        "step_ms": {"median": round(statistics.median(per_step), 5), "p10": round(pct(per_step, 0.1), 5),
                    "p90": round(pct(per_step, 0.9), 5), "min": round(min(per_step), 5),
                    "max": round(max(per_step), 5)},
        "api": ("latent_moe_layer_os" if cfg.os else
                "latent_moe_layer" if one_call else "latent_moe_route + latent_moe_forward"),
        "eager_ms_per_step_with_stage_events": None if eager_ms is None else round(eager_ms, 5),
        "copies_cycled": copies, "wall_s": round(wall, 3),
        "stage_us": {n: round(v, 2) for n, v in stages.items()},
        "layer_tflops": round(layer_flop / (ms_per_step / 1e3) / 1e12, 2),
        "layer_mfma_frac": round(layer_flop / (ms_per_step / 1e3) / 1e12 / mfma_peak, 4),
        "layer_hbm_gbs": round(layer_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "layer_hbm_frac": round(layer_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_algorithmic_bytes": int(layer_bytes), "layer_algorithmic_flop": layer_flop,
        "touched_experts": touched, "roofline": roofline, "shader_clock": clk,
    }
    if cfg.os:
        res["stage_note"] = "output-stationary call: no permutation; kernel times from the rocprofv3 trace"
    elif cfg.router_gemm:
        res["stage_note"] = ("shared_gate_up also covers the router gate GEMM, the top-k and the permutation "
                             "(latent_moe_layer runs them between the down-projection and FC1)")
    elif one_call:
        res["stage_note"] = ("down_proj also covers the top-k (in the same launch at T <= 512) and "
                             "shared_gate_up the permutation (latent_moe_layer with the logits given)")
    if use_events:
        for n, fl, by in (("fc1", fc1_flop, fc1_bytes), ("fc2", fc2_flop, fc2_bytes)):
            us = stages[n]
            if fused_mlp:   # one launch: report it under fc1 with both GEMMs' work
                if n == "fc2":
                    continue
                fl, by = fc1_flop + fc2_flop, fc1_bytes + fc2_bytes - 2 * R * I * 2
            res[f"{n}_tflops"] = round(fl / us / 1e6, 2)
            res[f"{n}_mfma_frac"] = round(fl / us / 1e6 / mfma_peak, 4)
            res[f"{n}_hbm_frac"] = round(by / us / 1e3 / HBM_PEAK_GBS, 4)
        if not cfg.rows_mode:
            for n, fl in (("down_proj", 2.0 * T * d * l), ("up_proj", 2.0 * T * (l + S * Is) * d)):
                if stages.get(n, 0) > 0:
                    res[f"{n}_tflops"] = round(fl / stages[n] / 1e6, 2)
                    res[f"{n}_mfma_frac"] = round(fl / stages[n] / 1e6 / BF16_PEAK_TFLOPS, 4)
    res["_sets"] = sets
    return res


def describe(cfg):
    T, E, k, d, l, I, S, Is = cfg.T, cfg.E, cfg.k, cfg.d, cfg.l, cfg.I, cfg.S, cfg.Is
    if cfg.rows_mode:
        return (f"{cfg.name}: {T} received rows, {E} local experts, latent {l}, SwiGLU I={I}, "
                f"Zipf({cfg.zipf_s}) expert load, combine weights given")
    return (f"{cfg.name}: T={T} tokens, d={d} -> latent {l}, E={E} top-{k} + {S} shared, "
            f"SwiGLU I={I}, shared I={Is}, RMSNorm on"
            + (", logits computed by the router gate on the latent (latent_moe_layer)" if cfg.router_gemm else "")
            + ((", MXFP4 experts (w4a16)" if cfg.w4a16 else ", MXFP4 experts (w4a8)") if cfg.mxfp4 else "")
            + (", output-stationary experts (latent_moe_layer_os)" if cfg.os else ""))


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
    clock = None if args.no_clock else ClockSampler()

    main_res = measure(cfg, args, hip, lm, W, torch, stream, clock, args.wlayout)
    print(f"# {cfg.name}: {main_res['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)

    cpu = None
    if args.cpu_seconds > 0:
        from tests.parity import to_host
        cpu = cpu_baseline(cfg, to_host(main_res["_sets"][0]["inp"]), args.cpu_seconds)
    main_res.pop("_sets")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    others = {}
    for key in [n for n in args.extra_workloads.split(",") if n and n != cfg.name]:
        name, _, lay = key.partition("@")
        ocfg = W.CONFIGS[name]
        r = measure(ocfg, args, hip, lm, W, torch, stream, clock, lay or args.wlayout)
        r.pop("_sets")
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        r["config"] = describe(ocfg)
        r["ms_per_step"] = round(r["ms_per_step"], 5)
        r["tokens_per_s"] = round(r["tokens_per_s"], 1)
        others[key] = r
        print(f"# {key}: {r['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)

    single = None
    if args.cpu_seconds > 0:
        single = cpu_single_thread(["tiny", "decode"], min(3.0, args.cpu_seconds / 4))

    roofline = main_res.pop("roofline")
    extra = {k: v for k, v in main_res.items() if k not in ("ms_per_step", "tokens_per_s")}
    extra["host_cpu"] = {"model": cpu_model(), "logical_cpus": os.cpu_count(),
                         "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}
    extra["cpu_oracle_single_thread"] = single
    extra["workloads"] = others
    T = cfg.T
    line = {
        "metric": METRIC, "value": round(main_res["tokens_per_s"], 1),
        "unit": "tokens/s" if not cfg.rows_mode else "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16 (experts: MXFP4 weights upcast to bf16, bf16 activations)" if cfg.w4a16 else
                  "bf16 (experts: MXFP4 weights x MXFP8 activations)") if cfg.mxfp4 else "bf16",
        "data": ("synthetic (seeded N(0,1) activations, N(0,0.02) bf16 weights, router gate "
                 "N(0, 1/sqrt(latent*d*0.02^2)) on the latent)" if cfg.router_gemm else
                 "synthetic (seeded N(0,1) activations, N(0,0.02) bf16 weights, gap-separated N(0,1) logits)"),
        "config": {"workload": describe(cfg), "T": T, "d": cfg.d, "latent": cfg.l, "E": cfg.E, "k": cfg.k,
                   "shared": cfg.S, "I": cfg.I, "Is": cfg.Is,
                   "expert_weight_layout": main_res.get("expert_weight_layout")},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)
    # leave nothing behind: the amdsmi session, then the device memory
    if clock is not None:
        clock.close()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    rc = main()
    sys.stdout.flush()
    sys.exit(rc)
