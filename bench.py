"""Benchmark of the OCR-decoder decode step on one MI355X.

Workload: the 12-layer decoder (hidden 1280, 10 heads x 128, layer 0 dense
SwiGLU 3584 in Q4_0, layers 1-11 MoE with 64 routed + 2 shared Q4_0 experts of
896, top-6; attention and router Q8_0; fp16 embedding and LM head over 129280
tokens), every row with a 1100-position prefix and a 128-slot ring that starts
at generation index 100, so the ring wraps during a 64-step run.  All weights,
caches and first tokens are seeded synthetic data (``synth``).  The ring
starts at generation index t0 = 128 - warmup - steps // 2 (at least 0), so the
timed steps straddle the wrap at t = 128 whatever --steps and --warmup are.

A step is one ocrdec_decode_step call for all rows: embedding, 12 layers, final
norm, LM head with fused argmax; the token feeds the next step on the device.

Prints ONE JSON line: rows*steps/s of the timed steps, the roofline of the
dominant kernel (the LM-head GEMV with fused argmax, timed with HIP events on
its own stream), and the CPU oracle timed on this host on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
SEED = 1003
ROOT = os.path.dirname(os.path.abspath(__file__))
# Counter-measured HBM traffic per launch of each kernel kind of the decode
# step (rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs, calibrated on a copy
# of known size), at 1 and 24 rows.  It applies only while the kernel sources
# hash to the value recorded with it.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_traffic.md")
CSRC = os.path.join(ROOT, "quantized_decode_step_amd", "csrc")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(rows: int):
    """({kind: bytes per launch}, note) from the counter summary if it was
    taken at this row count and matches the current kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter summary"
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and line.strip().startswith(("source-hash", "traffic-r")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source-hash") != kernel_source_hash():
        return None, "kernel sources changed since the counters were taken"
    key = "traffic-r%d" % rows
    if key not in vals:
        return None, "counters taken at 1 and 24 rows only"
    return json.loads(vals[key]), "rocprofv3 FETCH_SIZE x2.0 + WRITE_SIZE x1.0 per launch (calibrated on a 512 MiB copy)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rows", type=int, default=1)
    ap.add_argument("--sweep", default="6,12,24", help="extra row counts timed after the main run ('' for none)")
    ap.add_argument("--no-graph", action="store_true", help="launch kernels directly instead of replaying a graph")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the CPU oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-cpu-sweep", action="store_true", help="time the oracle at one row only")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-shaped MoE layer line")
    ap.add_argument("--no-qhead", action="store_true", help="skip the Q4_0 LM-head and embedding variant")
    ap.add_argument("--lm-iters", type=int, default=50)
    ap.add_argument("--mode", choices=["full", "lm", "prefill", "prompt"], default="full",
                    help="lm: only the LM-head argmax loop and a device copy of known size (for counter runs); "
                         "prefill: only the prefill-shaped MoE layer (2048 tokens); "
                         "prompt: only the prompt pass of the 12-layer model (1100 positions)")
    ap.add_argument("--no-prompt", action="store_true", help="skip the prompt-pass line")
    ap.add_argument("--no-int8kv", action="store_true", help="skip the INT8 KV cache runs")
    ap.add_argument("--no-round", action="store_true", help="skip the round-scheduler line")
    ap.add_argument("--prompt-iters", type=int, default=5)
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-call HBM GB/s of one layer's entry points")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event timing inside the step")
    ap.add_argument("--no-layers", action="store_true", help="skip the single dense and MoE layer lines")
    ap.add_argument("--no-sink", action="store_true", help="skip the sink-augmented block lines")
    ap.add_argument("--prefill-iters", type=int, default=20)
    ap.add_argument("--copy-mb", type=int, default=512, help="size of the calibration copy in --mode lm")
    return ap.parse_args()


def algorithmic_bytes(dm, d, rows: int, distinct_experts_per_layer: float, avg_keys: float,
                      kv_bytes_per_value: float = 2.0) -> float:
    """Bytes the method must move per step: every weight matrix once, the
    routed experts actually used, the KV window of every row and layer, and
    the embedding rows."""
    def nb(m):  # packed bytes minus padding are the block bytes
        return {0: 2.0, 1: 34 / 32, 2: 18 / 32, 3: 36 / 32}[m.fmt] * m.n * m.k
    tot = 0.0
    H, F = d.hidden, d.expert_ff
    per_expert = {2: 18 / 32, 1: 34 / 32, 0: 2.0, 3: 36 / 32}[d.fmt_expert] * 3 * F * H
    n_moe = 0
    for lay in dm.src_layers:
        tot += nb(lay.wqkv) + nb(lay.wo) + 2 * 2 * H  # + the two norm gains
        if lay.is_moe:
            n_moe += 1
            tot += nb(lay.router) + nb(lay.sh_gate_up) + nb(lay.sh_down)
        else:
            tot += nb(lay.dense_gate_up) + nb(lay.dense_down)
    tot += n_moe * distinct_experts_per_layer * per_expert
    tot += nb(dm.src_lm) + 2 * H + rows * 2 * H
    tot += d.n_layers * rows * 2 * d.n_heads * d.head_dim * kv_bytes_per_value * avg_keys
    return tot


def kernel_bytes(dm, d, R: int, distinct: float, avg_keys: float, kv_bytes_per_value: float = 2.0) -> dict:
    """Algorithmic bytes of one launch of each kernel kind of the decode step
    (the weight blocks it must stream, the KV window, the rows it reads)."""
    def nb(m):
        return {0: 2.0, 1: 34 / 32, 2: 18 / 32, 3: 36 / 32}[m.fmt] * m.n * m.k
    lay = next(l for l in dm.src_layers if l.is_moe)
    dense = next((l for l in dm.src_layers if not l.is_moe), None)
    H, E = d.hidden, d.n_experts
    glu_e, down_e = nb(lay.exp_gate_up) / E, nb(lay.exp_down) / E
    glu_s, down_s = nb(lay.sh_gate_up) / d.n_shared, nb(lay.sh_down) / d.n_shared
    kv = R * 2 * d.n_heads * d.head_dim * kv_bytes_per_value * avg_keys
    out = {"qkv": nb(lay.wqkv) + R * H * 2, "attn": kv, "attn_merge_o": nb(lay.wo), "o_proj": nb(lay.wo),
           "route": nb(lay.router), "expert_glu": distinct * glu_e + d.n_shared * glu_s,
           "expert_down": distinct * down_e + d.n_shared * down_s, "lm_head": nb(dm.src_lm) + R * H * 2}
    if dense is not None:
        out["dense_glu"] = nb(dense.dense_gate_up)
        out["dense_down"] = nb(dense.dense_down)
    return out


def profile_step(q, torch, stream, step_fn, reps: int = 10, capacity: int = 512):
    """Per-kernel time inside the decode step: a HIP event before every kernel
    the library enqueues (ocrdec_profile_set) and one after the last, direct
    launches on the bench stream behind a short spin kernel (so that the whole
    step is queued before the GPU reaches it and host enqueue time does not
    show); the time between consecutive events is a kernel plus the gap
    before it.  Returns ({kind: [us per launch, ...]} averaged over `reps`
    steps, total us per step), or (None, None)."""
    import ctypes
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
    for e in evs:  # creates the runtime events (torch creates them on first record)
        e.record(stream)
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * capacity)(*[e.cuda_event for e in evs])
    kinds = (ctypes.c_int32 * capacity)()
    acc, names, tot = None, None, 0.0
    try:
        for _ in range(reps):
            prof = q.Profile(ctypes.cast(handles, ctypes.POINTER(ctypes.c_void_p)), kinds, capacity, 0)
            with torch.cuda.stream(stream):
                torch.cuda._sleep(2_000_000)
                q.ocrdec_profile_set(prof)
                try:
                    step_fn(stream)
                    q.ocrdec_profile_mark(stream)
                finally:
                    q.ocrdec_profile_set(None)
            torch.cuda.synchronize()
            n = prof.count
            t = np.array([evs[i].elapsed_time(evs[i + 1]) * 1000.0 for i in range(n - 1)])
            if acc is None:
                acc, names = t, [q.KERNEL_NAMES[kinds[i]] for i in range(n - 1)]
            else:
                acc += t
            tot += evs[0].elapsed_time(evs[n - 1]) * 1000.0
        acc /= reps
        out = {}
        for i, k in enumerate(names):
            out.setdefault(k, []).append(float(acc[i]))
        return out, tot / reps
    except Exception as ex:  # reported, not fatal: the rest of the line stands
        print("profile_step: %s" % ex, file=sys.stderr)
        return None, None
    finally:
        torch.cuda.synchronize()


def kernel_table(prof: dict, byts: dict, ms_step: float):
    """Rows of {kernel, launches, avg_us, us_per_step, share, bytes_per_launch, GBps, frac} sorted by time."""
    rows = []
    for k, v in prof.items():
        tot = float(np.sum(v))
        r = {"kernel": k, "launches_per_step": len(v), "avg_us": round(tot / len(v), 2), "us_per_step": round(tot, 1),
             "share_of_step": round(tot / (ms_step * 1000.0), 3)}
        if k in byts:
            gbs = byts[k] / (tot / len(v) * 1e-6) / 1e9
            r.update({"bytes_per_launch": round(byts[k]), "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)})
        rows.append(r)
    rows.sort(key=lambda r: -r["us_per_step"])
    return rows


def first_gen_index(steps: int, warmup: int, ring: int = 128) -> int:
    """Generation index of the first warm-up step: the timed steps then run
    over t = t0 + warmup .. t0 + warmup + steps - 1, which holds t = ring (the
    first step that overwrites a ring slot) in its middle."""
    return max(0, ring - warmup - steps // 2)


def main():
    args = parse()
    T0 = first_gen_index(args.steps, args.warmup)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU: the decode step here is single-GPU (no collectives); "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import quantized_decode_step_amd as q

    assert torch.cuda.is_available(), "no GPU visible"
    dev = torch.device("cuda:0")
    d = synth.dims_full()
    stream = torch.cuda.Stream()
    if args.mode == "prefill":
        print(json.dumps(prefill_moe(args, q, torch, dev, stream)), flush=True)
        return
    if args.mode == "lm":
        lm = synth.random_qmat(d.fmt_lm, synth.stream_id(SEED, "lm_head"), d.vocab, d.hidden, d.w_std)

        class _M:
            lm_head = q.DeviceQMat(lm)
        lm_only(args, _M, d, q, torch, dev, stream)
        return
    t_build = time.time()
    model = synth.make_model(d, SEED)
    dm = q.DeviceModel(model)
    dm.src_layers = model.layers
    dm.src_lm = model.lm_head
    t_build = time.time() - t_build
    if args.mode == "prompt":
        print(json.dumps(prompt_pass(args, q, torch, dev, stream, dm, d)), flush=True)
        return

    def run_rows(R: int, steps: int, warmup: int, want_sample: bool, int8_kv: bool = False):
        if int8_kv:
            st = synth.make_state_int8(d, SEED, [d.prefix_cap] * R, [T0] * R)
        else:
            st = synth.make_state(d, SEED, [d.prefix_cap] * R, [T0] * R)
        ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
        dm.bind_caches(ds.k_cache, ds.v_cache, ds.k_scale, ds.v_scale)
        wsb = q.ocrdec_step_workspace_bytes(dm.desc, ds.desc)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        tok = torch.from_numpy(synth.first_tokens(d, SEED, R)).to(dev)
        n_moe = d.n_layers - d.n_dense
        cap_idx = torch.zeros((n_moe, R, d.top_k), dtype=torch.int32, device=dev)
        cap = q.StepCapture(cap_idx.data_ptr(), None, None)
        distinct = []
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                q.ocrdec_decode_step(dm.desc, ds.desc, tok, None, tok, None, cap, ws, wsb, stream=stream)
                stream.synchronize()
                ci = cap_idx.cpu().numpy()
                distinct.append(np.mean([len(np.unique(ci[l])) for l in range(n_moe)]))
            graph = None
            if not args.no_graph:
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=stream):
                    q.ocrdec_decode_step(dm.desc, ds.desc, tok, None, tok, None, None, ws, wsb,
                                         stream=torch.cuda.current_stream())
                # the capture enqueued nothing: the state is where warmup left it
            stream.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(steps):
                if graph is not None:
                    graph.replay()
                else:
                    q.ocrdec_decode_step(dm.desc, ds.desc, tok, None, tok, None, None, ws, wsb, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        gi = ds.gen_index.cpu().numpy()
        assert np.all(gi == T0 + warmup + steps), "generation index did not advance once per step"
        toks = tok.cpu().numpy()
        assert np.all((toks >= 0) & (toks < d.vocab))
        out = {"rows": R, "ms_per_step": ms, "rows_steps_per_s": R * 1000.0 / ms,
               "distinct_experts_per_moe_layer": float(np.mean(distinct)) if distinct else None}
        # keys each row attends, averaged over the timed steps (prefix + ring so far, incl. the new token)
        ts = np.arange(T0 + warmup, T0 + warmup + steps)
        avg_keys = float(np.mean(d.prefix_cap + np.minimum(ts + 1, d.ring_cap)))
        byt = algorithmic_bytes(dm, d, R, out["distinct_experts_per_moe_layer"] or d.top_k, avg_keys,
                                kv_bytes_per_value=(1.0 + 2.0 / d.head_dim) if int8_kv else 2.0)
        out["algorithmic_MB_per_step"] = byt / 1e6
        out["step_GBps"] = byt / (ms * 1e-3) / 1e9
        del graph
        if want_sample and not args.no_profile:
            prof, prof_us = profile_step(q, torch, stream, lambda s: q.ocrdec_decode_step(dm.desc, ds.desc, tok, None,
                                                                                           tok, None, None, ws, wsb,
                                                                                           stream=s))
            if prof is not None:
                out["profiled_us_per_step"] = round(prof_us, 1)
                # each event and the direct launch add a roughly fixed time per
                # kernel: (profiled step - graph step) / launches, subtracted
                n_launch = sum(len(v) for v in prof.values())
                ovh = max(0.0, (prof_us - ms * 1000.0) / n_launch)
                out["event_overhead_us_per_launch"] = round(ovh, 2)
                prof = {k: [max(t - ovh, 0.5 * t) for t in v] for k, v in prof.items()}
                byk = kernel_bytes(dm, d, R, out["distinct_experts_per_moe_layer"] or d.top_k, avg_keys,
                                   kv_bytes_per_value=(1.0 + 2.0 / d.head_dim) if int8_kv else 2.0)
                out["kernels"] = kernel_table(prof, byk, ms)
        return out

    main_run = run_rows(args.rows, args.steps, args.warmup, True)
    sweep = []
    for r in [int(x) for x in args.sweep.split(",") if x.strip()]:
        if r != args.rows:
            sweep.append(run_rows(r, args.steps, args.warmup, True))

    # ---- the same step over an INT8 KV cache (codes + one fp16 scale per row, head and slot)
    int8_kv = None
    if not args.no_int8kv:
        runs8 = [run_rows(r, args.steps, args.warmup, False, int8_kv=True) for r in (1, 24)]
        int8_kv = {"cache": "int8 codes + fp16 scale per (row, head, slot)",
                   "runs": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()} for s in runs8]}

    # ---- roofline of the dominant kernel: the LM-head GEMV with fused argmax
    R = args.rows
    x = torch.from_numpy(synth.normal_f16(synth.stream_id(SEED, "lm_x"), (R, d.hidden)).view(np.int16)).to(dev)
    tok_out = torch.zeros(R, dtype=torch.int32, device=dev)
    lm_ws_b = q.ocrdec_lm_argmax_workspace_bytes(dm.lm_head.desc, R)
    lm_ws = torch.zeros(lm_ws_b, dtype=torch.uint8, device=dev)
    with torch.cuda.stream(stream):
        for _ in range(3):
            q.ocrdec_lm_argmax(dm.lm_head.desc, R, x, tok_out, None, lm_ws, lm_ws_b, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.lm_iters):
            q.ocrdec_lm_argmax(dm.lm_head.desc, R, x, tok_out, None, lm_ws, lm_ws_b, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
    lm_us = e0.elapsed_time(e1) * 1000.0 / args.lm_iters
    traffic_all, traffic_note = recorded_traffic(R)
    traffic = traffic_all.get("lm_head") if traffic_all else None
    lm_bytes = d.vocab * d.hidden * 2.0 + R * d.hidden * 2.0
    lm_gbs = lm_bytes / (lm_us * 1e-6) / 1e9

    # ---- the same step with the LM head and the embedding table in Q4_0 (quantised from the same draws)
    qhead = None
    if not args.no_qhead:
        lmq = synth.random_qmat(synth.Q4_0, synth.stream_id(SEED, "lm_head"), d.vocab, d.hidden, d.w_std)
        emq = synth.random_qmat(synth.Q4_0, synth.stream_id(SEED, "embed"), d.vocab, d.hidden, d.w_std)
        dlm, dem = q.DeviceQMat(lmq), q.DeviceQMat(emq)
        saved = (dm.desc.lm_head, dm.desc.embed, dm.desc.embed_q, dm.src_lm)
        dm.desc.lm_head, dm.desc.embed, dm.desc.embed_q, dm.src_lm = dlm.desc, None, dem.desc, lmq
        qrun = run_rows(args.rows, args.steps, args.warmup, False)
        ws_q = torch.zeros(q.ocrdec_lm_argmax_workspace_bytes(dlm.desc, args.rows), dtype=torch.uint8, device=dev)
        xq = torch.from_numpy(synth.normal_f16(synth.stream_id(SEED, "lm_x"), (args.rows, d.hidden)).view(np.int16)).to(dev)
        tq = torch.zeros(args.rows, dtype=torch.int32, device=dev)
        with torch.cuda.stream(stream):
            for _ in range(3):
                q.ocrdec_lm_argmax(dlm.desc, args.rows, xq, tq, None, ws_q, ws_q.numel(), stream=stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.lm_iters):
                q.ocrdec_lm_argmax(dlm.desc, args.rows, xq, tq, None, ws_q, ws_q.numel(), stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
        lmq_us = e0.elapsed_time(e1) * 1000.0 / args.lm_iters
        lmq_bytes = d.vocab * d.hidden * 18 / 32 + args.rows * d.hidden * 2.0
        dm.desc.lm_head, dm.desc.embed, dm.desc.embed_q, dm.src_lm = saved
        qhead = {"lm_head": "Q4_0", "embed": "Q4_0", "rows": args.rows,
                 "ms_per_step": round(qrun["ms_per_step"], 4),
                 "rows_steps_per_s": round(qrun["rows_steps_per_s"], 2),
                 "algorithmic_MB_per_step": round(qrun["algorithmic_MB_per_step"], 1),
                 "step_GBps": round(qrun["step_GBps"], 1),
                 "lm_head_us": round(lmq_us, 2), "lm_head_GBps": round(lmq_bytes / (lmq_us * 1e-6) / 1e9, 1),
                 "lm_head_frac": round(lmq_bytes / (lmq_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    # ---- HBM GB/s of one decoder layer's entry points at one row
    kernels = None if args.no_kernels else per_call_bandwidth(q, torch, dev, stream, dm, d)

    # ---- single decoder layers (dense fp16; Q8_0 MoE) and the sink-augmented block
    layers1 = None if args.no_layers else single_layers(q, torch, dev, stream)
    sink = None if args.no_sink else sink_blocks(q, torch, dev, stream)

    # ---- the prefill-shaped MoE layer (2048 tokens, MFMA path), reported beside the decode metric
    prefill = None if args.no_prefill else prefill_moe(args, q, torch, dev, stream)

    # ---- the prompt pass of the same 12-layer model (1100 positions), beside the decode metric
    prompt = None if args.no_prompt else prompt_pass(args, q, torch, dev, stream, dm, d)

    # ---- a queue of requests through the round scheduler
    round_line = None if args.no_round else round_queue(args, q, torch, dev, stream, dm, d)

    # ---- CPU oracle baseline on a bounded sample (1 row of the same workload)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(model, d, args.cpu_seconds, T0)
        # the same on one host thread: one whole step
        try:
            one = cpu_baseline(model, d, 0.0, T0, threads=1)
            cpu["single_thread"] = {k_: one[k_] for k_ in ("value", "cores", "sample")}
        except ImportError:
            pass
        # the oracle at every swept row count: one whole step of R rows each
        if not args.no_cpu_sweep:
            for s_ in sweep:
                s_["cpu_baseline"] = cpu_baseline(model, d, 0.0, T0, rows=s_["rows"])

    line = {
        "metric": "decode rows\u00b7steps/s (12-layer MoE step) + achieved HBM GB/s vs peak",
        "value": round(main_run["rows_steps_per_s"], 2),
        "unit": "rows\u00b7steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_run["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded weights ~N(0,0.02) quantised Q4_0/Q8_0, caches ~N(0,1))",
        "config": {
            "workload": "12-layer mixed-Q4_0 MoE OCR decoder decode step: %d row(s), prefix 1100 + 128-slot ring, "
                        "timed steps t=%d..%d (the ring wraps at t=128), vocab 129280, tokens fed back on device"
                        % (args.rows, T0 + args.warmup, T0 + args.warmup + args.steps - 1),
            "rows": args.rows, "layers": d.n_layers, "hidden": d.hidden, "experts": "64 routed top-6 + 2 shared",
            "graph": not args.no_graph,
        },
        "step_hbm": {"algorithmic_MB_per_step": round(main_run["algorithmic_MB_per_step"], 1),
                     "achieved_GBps": round(main_run["step_GBps"], 1),
                     "frac": round(main_run["step_GBps"] / HBM_PEAK_GBS, 4),
                     "distinct_experts_per_moe_layer": main_run["distinct_experts_per_moe_layer"]},
        "rows_sweep": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()} for s in sweep],
        "roofline": dominant_roofline(main_run.get("kernels"), traffic_all, traffic_note),
        "lm_head": {"kernel": ("lm_argmax_kernel<F16, ring 10> (LM head %dx%d + fused argmax, %d row(s); "
                               "one CU-balanced workgroup per CU, then the partial merge)" if R <= 16 else
                               "gemv_kernel<F16,4,1,1,ARGMAX> (LM head %dx%d + fused argmax, %d row(s))")
                              % (d.vocab, d.hidden, R),
                    "bound": "hbm", "achieved": round(lm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(lm_gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "traffic_note": traffic_note,
                    "avg_us": round(lm_us, 2), "algorithmic_bytes": lm_bytes,
                    "timing": "ocrdec_lm_argmax alone, %d calls between HIP events on its stream" % args.lm_iters},
        "step_kernels": main_run.get("kernels"),
        "cpu_baseline": cpu,
        "quantised_head": qhead,
        "kernels": kernels,
        "single_layers": layers1,
        "sink_block": sink,
        "prefill_moe": prefill,
        "prompt_pass": prompt,
        "int8_kv": int8_kv,
        "round": round_line,
        "setup_s": round(t_build, 1),
    }
    print(json.dumps(line), flush=True)


def dominant_roofline(kernels, traffic, traffic_note):
    """Roofline of the kernel kind that takes the most time per step (event
    timing inside the step): algorithmic bytes per launch / average launch
    time (kernel plus the gap before it)."""
    if not kernels:
        return None
    k = next((r for r in kernels if "bytes_per_launch" in r), None)
    if k is None:
        return None
    return {"kernel": k["kernel"], "bound": "hbm", "achieved": k["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": k["frac"], "traffic": (traffic or {}).get(k["kernel"]), "traffic_note": traffic_note,
            "avg_us": k["avg_us"], "launches_per_step": k["launches_per_step"], "share_of_step": k["share_of_step"],
            "algorithmic_bytes": k["bytes_per_launch"],
            "timing": "HIP events recorded on the bench stream before every kernel of the step (ocrdec_profile_set), "
                      "direct launches queued behind a spin kernel, mean of 10 steps; a launch's time is the interval "
                      "to the next event minus the mean per-launch cost of the events and direct launches "
                      "((profiled step - graph step) / launches)"}


def per_call_bandwidth(q, torch, dev, stream, dm, d, layer: int = 1, reps: int = 20, replays: int = 5):
    """Achieved HBM GB/s of the C-ABI calls one MoE layer of the decode step is
    made of, at one row and the step's shapes: each call is captured `reps`
    times in a HIP graph and the graph replayed `replays` times between HIP
    events on its stream (GPU time only; the launch gaps between the captured
    kernels are included, as in the step).  Algorithmic bytes: the weight
    blocks a call must read (for the MoE layer the router, the 6 routed experts
    the row takes and the 2 shared experts), the KV window for attention."""
    import synth
    lay, L = dm.src_layers[layer], dm.layers[layer]
    H, NH, D, HD = d.hidden, d.n_heads, d.head_dim, d.n_heads * d.head_dim

    def nb(m):
        return {0: 2.0, 1: 34 / 32, 2: 18 / 32, 3: 36 / 32}[m.fmt] * m.n * m.k
    x = torch.from_numpy(synth.normal_f16(synth.stream_id(SEED, "kern_x"), (1, H)).view(np.int16)).to(dev)
    o16 = torch.from_numpy(synth.normal_f16(synth.stream_id(SEED, "kern_o"), (1, HD)).view(np.int16)).to(dev)
    qkv = torch.zeros((1, 3 * HD), dtype=torch.float32, device=dev)
    y = torch.zeros((1, H), dtype=torch.float32, device=dev)
    # attention over a full window: prefix 1100 + the whole 128-slot ring
    st = synth.make_state(d, SEED, [d.prefix_cap], [2 * d.ring_cap])
    ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
    att_out = torch.zeros((1, HD), dtype=torch.int16, device=dev)
    a = q.AttnArgs(1, NH, D, qkv.data_ptr(), 3 * HD, ds.k_cache[layer].data_ptr(), ds.v_cache[layer].data_ptr(),
                   d.prefix_cap, d.ring_cap, ds.prefix_len.data_ptr(), ds.gen_index.data_ptr(), None,
                   d.rope_theta, 1.0 / np.sqrt(D), att_out.data_ptr(), HD, None, None)
    a_wsb = q.ocrdec_attn_workspace_bytes(a)
    a_ws = torch.zeros(a_wsb, dtype=torch.uint8, device=dev)
    h16 = torch.zeros((1, H), dtype=torch.int16, device=dev)
    m_wsb = q.ocrdec_moe_workspace_bytes(L.moe, 1)
    m_ws = torch.zeros(m_wsb, dtype=torch.uint8, device=dev)
    keys = d.prefix_cap + d.ring_cap
    per_expert = nb(lay.exp_gate_up) / d.n_experts + nb(lay.exp_down) / d.n_experts
    calls = [
        ("ocrdec_gemv_q: QKV projection, Q8_0 %dx%d" % (3 * HD, H), nb(lay.wqkv),
         lambda s: q.ocrdec_gemv_q(L.wqkv, 1, x, H, qkv, q.OCRDEC_OUT_F32, 3 * HD, stream=s)),
        ("ocrdec_attn_decode: %d heads x %d over %d keys (prefix %d + full ring)" % (NH, D, keys, d.prefix_cap),
         keys * NH * D * 2 * 2.0, lambda s: q.ocrdec_attn_decode(a, a_ws, a_wsb, stream=s)),
        ("ocrdec_gemv_q: O projection, Q8_0 %dx%d" % (H, HD), nb(lay.wo),
         lambda s: q.ocrdec_gemv_q(L.wo, 1, o16, HD, y, q.OCRDEC_OUT_F32, H, stream=s)),
        ("ocrdec_moe_layer: router + %d routed + %d shared Q4_0 experts of %d" % (d.top_k, d.n_shared, d.expert_ff),
         nb(lay.router) + d.top_k * per_expert + nb(lay.sh_gate_up) + nb(lay.sh_down),
         lambda s: q.ocrdec_moe_layer(L.moe, 1, x, h16, True, ws=m_ws, ws_bytes=m_wsb, stream=s)),
    ]
    out = []
    with torch.cuda.stream(stream):
        for name, byt, fn in calls:
            for _ in range(3):
                fn(stream)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for _ in range(reps):
                    fn(torch.cuda.current_stream())
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(replays):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000.0 / (reps * replays)
            gbs = byt / (us * 1e-6) / 1e9
            out.append({"call": name, "us": round(us, 2), "algorithmic_bytes": round(byt), "GBps": round(gbs, 1),
                        "frac": round(gbs / HBM_PEAK_GBS, 4)})
            del g
    return {"rows": 1, "layer": "MoE layer %d of the 12-layer decoder" % layer, "peak_GBps": HBM_PEAK_GBS,
            "calls": out}


def _graph_time_us(torch, stream, fn, reps: int = 20, replays: int = 5) -> float:
    """Microseconds per call of fn(stream): `reps` calls captured in a graph,
    replayed `replays` times between HIP events on the stream."""
    with torch.cuda.stream(stream):
        for _ in range(3):
            fn(stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(reps):
                fn(torch.cuda.current_stream())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1000.0 / (reps * replays)


def single_layers(q, torch, dev, stream):
    """One decoder layer, one decode step at one row: the dense fp16 layer
    (256 cached positions + the new token, SwiGLU 3584, seed 1001) and the Q8_0
    MoE layer (prefix 1100 + a full 128-slot ring, seed 1002).  The hidden
    state goes in and comes out (no embedding, no LM head).  Algorithmic bytes:
    every weight block once (the MoE layer's 6 routed experts of the row and
    the 2 shared ones) plus the KV window."""
    import synth
    out = []
    for name, d, seed, pl, gi in (("dense fp16 layer: 1 row, 10x128 MHA over 256 cached + 1 new, SwiGLU 3584",
                                   synth.dims_dense_layer(), 1001, 256, 0),
                                  ("MoE Q8_0 layer: 1 row, prefix 1100 + full 128-slot ring, 64 routed top-6 + 2 "
                                   "shared experts of 896", synth.dims_moe_layer(), 1002, 1100, 128)):
        model = synth.make_model(d, seed, with_embed=False, with_lm=False)
        st = synth.make_state(d, seed, [pl], [gi])
        dm = q.DeviceModel(model)
        ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
        dm.bind_caches(ds.k_cache, ds.v_cache)
        wsb = q.ocrdec_step_workspace_bytes(dm.desc, ds.desc)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        h0 = synth.normal_f16(synth.stream_id(seed, "h0"), (1, d.hidden))
        hidden = torch.from_numpy(h0.astype(np.float32)).to(dev)
        us = _graph_time_us(torch, stream, lambda s: q.ocrdec_decode_step(dm.desc, ds.desc, None, hidden, None, None,
                                                                          None, ws, wsb, stream=s))

        def nb(m):
            return {0: 2.0, 1: 34 / 32, 2: 18 / 32, 3: 36 / 32}[m.fmt] * m.n * m.k
        lay = model.layers[0]
        byt = nb(lay.wqkv) + nb(lay.wo) + 4 * d.hidden
        if lay.is_moe:
            byt += nb(lay.router) + d.top_k * (nb(lay.exp_gate_up) + nb(lay.exp_down)) / d.n_experts
            byt += nb(lay.sh_gate_up) + nb(lay.sh_down)
            keys = pl + d.ring_cap
        else:
            byt += nb(lay.dense_gate_up) + nb(lay.dense_down)
            keys = pl + 1
        byt += 2 * d.n_heads * d.head_dim * 2 * keys
        gbs = byt / (us * 1e-6) / 1e9
        out.append({"workload": name, "us_per_step": round(us, 2), "rows_steps_per_s": round(1e6 / us, 1),
                    "algorithmic_MB": round(byt / 1e6, 2), "GBps": round(gbs, 1),
                    "frac": round(gbs / HBM_PEAK_GBS, 4)})
        del dm, ds, ws
    return out


def sink_blocks(q, torch, dev, stream, seed: int = 1004):
    """The sink-augmented attention block with int8-asymmetric projections:
    x [R][512] -> U8A_G32 QKV GEMV -> RoPE(64), new key at index L, attention
    over the sink (index 0), the L cached and the new key (8 heads, q/k 65
    lanes folded to 64 + a sink logit, v 64) -> U8A_G32 O GEMV.  Three C-ABI
    calls per block.  Algorithmic bytes: the weights (0.885 + 0.295 MB) and
    the KV of the L + 1 attended keys."""
    import synth
    H, NH, D = 512, 8, 64
    wqkv = synth.random_qmat(synth.U8A_G32, synth.stream_id(seed, "wqkv"), 3 * H, H)
    wo = synth.random_qmat(synth.U8A_G32, synth.stream_id(seed, "wo"), H, H)
    dq, do = q.DeviceQMat(wqkv), q.DeviceQMat(wo)
    sink = torch.from_numpy(synth.normal_f64(synth.stream_id(seed, "sink"), (NH,)).astype(np.float16)
                            .astype(np.float32)).to(dev)
    wbytes = (3 * H * H + H * H) * 36 / 32
    out = []
    for L in (350, 3000):
        for R in (1, 6, 12, 24):
            cap = L + 1
            x = torch.from_numpy(synth.normal_f16(synth.stream_id(seed, "x", R), (R, H)).view(np.int16)).to(dev)
            kc = torch.from_numpy(synth.normal_f16(synth.stream_id(seed, "kc", L), (R, NH, cap, D)).view(np.int16)).to(dev)
            vc = torch.from_numpy(synth.normal_f16(synth.stream_id(seed, "vc", L), (R, NH, cap, D)).view(np.int16)).to(dev)
            kc[:, :, 0] = 0
            vc[:, :, 0] = 0
            qkv = torch.zeros((R, 3 * H), dtype=torch.float32, device=dev)
            o = torch.zeros((R, H), dtype=torch.int16, device=dev)
            y = torch.zeros((R, H), dtype=torch.int16, device=dev)
            pl = torch.full((R,), L, dtype=torch.int32, device=dev)
            a = q.AttnArgs(R, NH, D, qkv.data_ptr(), 3 * H, kc.data_ptr(), vc.data_ptr(), cap, 0, pl.data_ptr(), None,
                           sink.data_ptr(), 10000.0, 1.0 / 8.0, o.data_ptr(), H, None, None)
            wsb = q.ocrdec_attn_workspace_bytes(a)
            ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

            def block(s):
                q.ocrdec_gemv_q(dq.desc, R, x, H, qkv, q.OCRDEC_OUT_F32, 3 * H, stream=s)
                q.ocrdec_attn_decode(a, ws, wsb, stream=s)
                q.ocrdec_gemv_q(do.desc, R, o, H, y, q.OCRDEC_OUT_F16, H, stream=s)
            us = _graph_time_us(torch, stream, block)
            byt = wbytes + R * NH * (L + 1) * D * 2 * 2.0
            gbs = byt / (us * 1e-6) / 1e9
            out.append({"rows": R, "cached": L, "us_per_block": round(us, 2),
                        "rows_blocks_per_s": round(R * 1e6 / us, 1), "algorithmic_MB": round(byt / 1e6, 3),
                        "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)})
            del kc, vc, ws
    return {"workload": "sink-augmented attention block: hidden 512, 8 heads (q/k 64 lanes + sink logit, v 64), "
                        "U8A_G32 QKV and O projections, fp16 KV cache with the sink at index 0",
            "runs": out}


PREFILL_SEED = 1005
PROMPT_SEED = 1006
ROUND_SEED = 1007
PREFILL_TOKENS = 2048


def prefill_moe(args, q, torch, dev, stream):
    """The prefill-shaped MoE layer: 2048 tokens, router bias ~N(0,1) (skewed
    expert loads), 64 routed top-6 + 2 shared Q4_0 SwiGLU experts of 896.
    Returns its time per call and the MFMA-path throughput (useful flops: every
    routed and shared expert product, 2 flop per multiply-add)."""
    import synth

    class _Lay:
        pass
    d = synth.Dims(fmt_router=synth.Q8_0, fmt_expert=synth.Q4_0, fmt_shared=synth.Q4_0)
    lay = _Lay()
    for k_, v_ in synth.make_moe_weights(d, PREFILL_SEED, 0, with_bias=True).items():
        setattr(lay, k_, v_)
    T = PREFILL_TOKENS
    x = synth.normal_f16(synth.stream_id(PREFILL_SEED, "x"), (T, d.hidden))
    w, keep = q.moe_weights(lay, d.hidden, d.top_k)
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    out = torch.zeros((T, d.hidden), dtype=torch.int16, device=dev)
    wsb = q.ocrdec_moe_workspace_bytes(w, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    with torch.cuda.stream(stream):
        for _ in range(3):
            q.ocrdec_moe_layer(w, T, xd, out, False, None, None, ws, wsb, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.prefill_iters):
            q.ocrdec_moe_layer(w, T, xd, out, False, None, None, ws, wsb, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / args.prefill_iters
    H, F, K, S = d.hidden, d.expert_ff, d.top_k, d.n_shared
    flops = 2.0 * T * (K + S) * (2 * F * H + H * F) + 2.0 * T * d.n_experts * H
    wbytes = sum(m.data.size for m in (lay.exp_gate_up, lay.exp_down, lay.sh_gate_up, lay.sh_down, lay.router))
    return {"mode": "prefill", "workload": "prefill-shaped MoE layer: 2048 tokens x 1280, router bias ~N(0,1), "
            "64 routed top-6 + 2 shared Q4_0 SwiGLU experts of 896", "bound": "mfma", "peak_TFLOPs": 2500.0,
            "tokens": T, "us_per_layer": round(us, 2), "gflop": round(flops / 1e9, 2),
            "tflops": round(flops / (us * 1e-6) / 1e12, 2), "frac_of_fp16_mfma_peak": round(flops / (us * 1e-6) / 2.5e15, 4),
            "weight_MB": round(wbytes / 1e6, 1)}


def prompt_pass(args, q, torch, dev, stream, dm, d):
    """The prompt pass (prefill) of one row through the 12-layer model: 1100
    positions of fp16 input features ~N(0,1) (the image and prompt features
    the decode's prefix stands for), causal attention, keys and values written
    to the row's cache prefix, the LM-head argmax at the last position.
    Useful flops count every projection, expert and attention product once
    (2 flop per multiply-add; the causal half of the score and value products)."""
    import synth
    P = d.prefix_cap
    st = synth.make_state(d, PROMPT_SEED, [0], [0])
    ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
    dm.bind_caches(ds.k_cache, ds.v_cache)
    emb = torch.from_numpy(synth.normal_f16(synth.stream_id(PROMPT_SEED, "features"), (P, d.hidden)).view(np.int16)).to(dev)
    tok_out = torch.zeros(1, dtype=torch.int32, device=dev)
    wsb = q.ocrdec_prefill_workspace_bytes(dm.desc, ds.desc, P)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    with torch.cuda.stream(stream):
        for _ in range(2):
            q.ocrdec_prefill(dm.desc, ds.desc, 0, P, emb=emb, tok_out=tok_out, ws=ws, ws_bytes=wsb, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.prompt_iters):
            q.ocrdec_prefill(dm.desc, ds.desc, 0, P, emb=emb, tok_out=tok_out, ws=ws, ws_bytes=wsb, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.prompt_iters
    H, HD, NH, D = d.hidden, d.n_heads * d.head_dim, d.n_heads, d.head_dim

    def useful_flops(n_seq):
        f = 0.0
        for lay in dm.src_layers:
            f += n_seq * (2.0 * P * H * 3 * HD + 2.0 * P * HD * H + 2.0 * 2 * D * NH * P * (P + 1) / 2)
            if lay.is_moe:
                f += n_seq * (2.0 * P * H * d.n_experts + 2.0 * P * (d.top_k + d.n_shared) * 3 * H * d.expert_ff)
            else:
                f += n_seq * 2.0 * P * 3 * H * d.dense_ff
        return f + n_seq * 2.0 * d.vocab * H
    flops = useful_flops(1)
    tf = flops / (ms * 1e-3) / 1e12
    # the same prompt in 8 rows at once (ocrdec_prefill_batch)
    NB = 8
    st8 = synth.make_state(d, PROMPT_SEED, [0] * NB, [0] * NB)
    ds8 = q.DeviceState(st8, d.prefix_cap, d.ring_cap)
    dm.bind_caches(ds8.k_cache, ds8.v_cache)
    emb8 = emb.repeat(NB, 1)
    tok8 = torch.zeros(NB, dtype=torch.int32, device=dev)
    rows8, P8 = list(range(NB)), [P] * NB
    wsb8 = q.ocrdec_prefill_batch_workspace_bytes(dm.desc, ds8.desc, rows8, P8)
    ws8 = torch.empty(wsb8, dtype=torch.uint8, device=dev)
    with torch.cuda.stream(stream):
        q.ocrdec_prefill_batch(dm.desc, ds8.desc, rows8, P8, emb=emb8, tok_out=tok8, ws=ws8, ws_bytes=wsb8,
                               stream=stream)
        e0.record(stream)
        for _ in range(2):
            q.ocrdec_prefill_batch(dm.desc, ds8.desc, rows8, P8, emb=emb8, tok_out=tok8, ws=ws8, ws_bytes=wsb8,
                                   stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
    ms8 = e0.elapsed_time(e1) / 2
    tf8 = useful_flops(NB) / (ms8 * 1e-3) / 1e12
    del ws8
    return {"workload": "prompt pass of the 12-layer mixed-Q4_0 MoE decoder: 1 row, %d positions of fp16 input "
                        "features, causal attention, cache prefix written, LM-head argmax at the last position" % P,
            "positions": P, "ms": round(ms, 3), "positions_per_s": round(P / (ms * 1e-3), 1),
            "gflop": round(flops / 1e9, 1), "tflops": round(tf, 1), "bound": "mfma", "peak_TFLOPs": 2500.0,
            "frac_of_fp16_mfma_peak": round(tf / 2500.0, 4),
            "batch_of_8": {"ms": round(ms8, 3), "positions_per_s": round(NB * P / (ms8 * 1e-3), 1),
                           "tflops": round(tf8, 1), "frac_of_fp16_mfma_peak": round(tf8 / 2500.0, 4)}}


def round_queue(args, q, torch, dev, stream, dm, d, n_req: int = 48, rows: int = 24, P: int = 1100,
                max_new: int = 64):
    """A queue of requests through ocrdec_run_round: 48 requests of 1100
    positions of fp16 input features each, 64 generated tokens each (no EOS),
    served by 24 rows.  Reports generated tokens/s and requests/s of the whole
    queue (prompt passes and decode steps, one host read of the tokens per
    step)."""
    import ctypes
    import synth
    st = synth.make_state(d, ROUND_SEED, [0] * rows, [0] * rows)
    ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
    dm.bind_caches(ds.k_cache, ds.v_cache)
    feats = torch.from_numpy(synth.normal_f16(synth.stream_id(ROUND_SEED, "features"), (8, P, d.hidden))
                             .view(np.int16)).to(dev)
    reqs = (q.Request * n_req)()
    outs = []
    for i in range(n_req):
        reqs[i].tokens, reqs[i].features = None, feats[i % 8].data_ptr()
        reqs[i].P, reqs[i].max_new = P, max_new
        o = (ctypes.c_int32 * max_new)()
        outs.append(o)
        reqs[i].out = ctypes.cast(o, ctypes.c_void_p)
    wsb = q.ocrdec_round_workspace_bytes(dm.desc, ds.desc, P)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    q.ocrdec_run_round(dm.desc, ds.desc, reqs, ws=ws, ws_bytes=wsb, stream=stream)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    q.ocrdec_run_round(dm.desc, ds.desc, reqs, ws=ws, ws_bytes=wsb, stream=stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    gen = sum(r.n_out for r in reqs)
    assert gen == n_req * max_new
    return {"workload": "%d requests x (%d positions of fp16 input features, %d generated tokens) on %d rows of the "
                        "12-layer decoder, no EOS" % (n_req, P, max_new, rows),
            "s": round(dt, 3), "generated_tokens_per_s": round(gen / dt, 1), "requests_per_s": round(n_req / dt, 2)}


def lm_only(args, dm, d, q, torch, dev, stream):
    """The LM-head argmax kernel alone, then a device-to-device copy of a known
    size (its FETCH_SIZE/WRITE_SIZE calibrate the counters)."""
    import synth
    R = args.rows
    x = torch.from_numpy(synth.normal_f16(synth.stream_id(SEED, "lm_x"), (R, d.hidden)).view(np.int16)).to(dev)
    tok_out = torch.zeros(R, dtype=torch.int32, device=dev)
    wsb = q.ocrdec_lm_argmax_workspace_bytes(dm.lm_head.desc, R)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    with torch.cuda.stream(stream):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q.ocrdec_lm_argmax(dm.lm_head.desc, R, x, tok_out, None, ws, wsb, stream=stream)
        e0.record(stream)
        for _ in range(args.lm_iters):
            q.ocrdec_lm_argmax(dm.lm_head.desc, R, x, tok_out, None, ws, wsb, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        n = args.copy_mb * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / args.lm_iters
    print(json.dumps({"mode": "lm", "rows": R, "lm_avg_us_incl_merge": round(us, 2),
                      "copy_bytes": n, "copy_launches": 3}), flush=True)


def cpu_baseline(model, d, budget_s: float, T0: int, rows: int = 1, threads: int = 0):
    """The oracle, as it stands, on `rows` rows of the same workload: as many
    whole steps as fit in the budget (at least one); with `threads`, its BLAS
    limited to that many threads."""
    if threads:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=threads):
            return cpu_baseline(model, d, budget_s, T0, rows)
    import synth
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    st = synth.make_state(d, SEED, [d.prefix_cap] * rows, [T0] * rows)
    tok = synth.first_tokens(d, SEED, rows)
    steps = 0
    t0 = time.time()
    while True:
        res = O.decode_step(model, st, tok_in=tok)
        tok = res.tok
        steps += 1
        if time.time() - t0 >= budget_s:
            break
    el = time.time() - t0
    return {"value": round(rows * steps / el, 4), "unit": "rows\u00b7steps/s", "cores": int(cores), "kind": "oracle",
            "sample": "%d step(s) of %d row(s) of the same 12-layer workload (prefix 1100, ring from t=%d), "
                      "numpy float64, %.1f s" % (steps, rows, T0, el)}


if __name__ == "__main__":
    main()
