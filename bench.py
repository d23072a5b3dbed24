"""Decode benchmark of the persistent megakernel on one MI355X.

Workload (default): the synthetic 30B-total / ~3B-active parallel-transformer MoE
(48 layers, hidden 2048, 32 q / 4 kv heads of 128, 128 experts top-8 with SwiGLU
inter 768, tied 151552 x 2048 embedding), bf16 random weights, batch 1 with 8192
cached tokens (random K/V) in shuffled 16-token pages, greedy decoding: each step
feeds the argmax of the previous step's logits at the next position.

One JSON line is printed.  `value` is decode tokens/s over the timed steps; the
roofline block prices the step kernel against MI355X's 8 TB/s HBM with the
algorithmic bytes of each step (active weights actually selected + KV read), and
cpu_baseline times the CPU reference on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
COPY_BYTES = 1 << 30  # bytes read (and written) by one calibration copy
METRIC = "decode tok/s + achieved HBM TB/s (% of SoL), 30B-A3B MoE bs1 @8K ctx"


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_megakernel_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".h", ".cpp")):
            continue  # built objects
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(geom, seq_lens, n_distinct_experts):
    """Bytes a decode step must move at least once: every weight it uses (dense
    projections, the distinct experts selected in each layer, the LM head, one
    embedding row per token, the norm vectors) and every cached K/V it attends to.
    n_distinct_experts: [n_layers] distinct experts selected by the batch."""
    H, hd, nq, nkv = geom.hidden, geom.head_dim, geom.n_q_heads, geom.n_kv_heads
    bf = 2
    dense = (geom.qkv_rows * H + H * nq * hd + geom.n_experts * H + H) * bf
    expert = (2 * geom.moe_inter * H + H * geom.moe_inter) * bf
    window, every = getattr(geom, "attn_window", 0), getattr(geom, "full_every", 1)
    total = 0
    for layer in range(geom.n_layers):
        # a local-attention layer reads the last `window` positions of each sequence
        local = window > 0 and (layer + 1) % every != 0
        kv_per_layer = sum(min(s + 1, window) if local else s + 1 for s in seq_lens) * nkv * hd * 2 * bf
        total += dense + n_distinct_experts[layer] * expert + kv_per_layer
    total += geom.vocab * H * bf + H * bf + len(seq_lens) * H * bf
    return total


def cpu_baseline(wl, n_layers_sample=2, reps=2):
    """The CPU reference as it stands, timed on this host on a bounded sample: the
    layer function on layers 0..n-1 of the workload (weights and that layer's KV
    materialised on the host beforehand, untimed) and the final norm + LM head.
    Scaled to one full step: t = n_layers * mean(t_layer) + t_lm_head."""
    import numpy as np

    import oracle
    import synth

    g = wl.geom
    H = g.hidden
    pt = synth.page_tables(wl)
    toks = synth.host_tokens(wl)
    numel = g.tensor_numel()
    per_layer = {k: numel[k] // g.n_layers for k in ("w_qkv", "w_o", "w_router", "w_gate_up", "w_down")}
    t_layers = []
    h = oracle.bf16_to_f32(synth.host_weight(wl, "embed", int(toks[0]) * H, H)).reshape(1, H).copy()
    for layer in range(n_layers_sample):
        Wl = {k: synth.host_weight(wl, k, layer * n, n) for k, n in per_layer.items()}
        gamma = synth.host_weight(wl, "norm", layer * H, H)
        kv0 = synth.host_kv_layer(wl, layer)
        for _ in range(reps):
            kv = kv0.copy()
            hh = h.copy()
            t0 = time.perf_counter()
            oracle.layer(g, wl.seq_lens, pt, kv, wl.n_pages, gamma, Wl["w_qkv"], Wl["w_o"], Wl["w_router"],
                         Wl["w_gate_up"], Wl["w_down"], hh)
            t_layers.append(time.perf_counter() - t0)
        h = hh
        del Wl, kv0
    embed = synth.host_weight(wl, "embed")
    gamma = synth.host_weight(wl, "norm", g.n_layers * H, H)
    t_lm = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.lm_head(g, h, gamma, embed)
        t_lm.append(time.perf_counter() - t0)
    t_step = g.n_layers * float(np.mean(t_layers)) + float(np.mean(t_lm))
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {
        "value": wl.batch / t_step,
        "unit": "tok/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"layer function on {n_layers_sample} of {g.n_layers} layers x {reps} reps "
                  f"({float(np.mean(t_layers)) * 1e3:.1f} ms/layer) + final norm and LM head "
                  f"({float(np.mean(t_lm)) * 1e3:.1f} ms), scaled to one {g.n_layers}-layer step "
                  f"of batch {wl.batch} at context {wl.seq_lens[0]}",
        "ms_per_step": t_step * 1e3,
    }


ORDERS = {"default": 0, "attention-first": 1, "moe-first": 2, "interleaved": 3}
PLACEMENTS = {"round-robin": 0, "xcd": 1}


def run(args):
    import numpy as np
    import torch

    import decode_megakernel_amd as mkd
    import synth
    from synth import device as sdev

    torch.cuda.set_device(0)
    ctx, batch = args.ctx, args.batch
    total_steps = args.warmup + args.steps
    wl = synth.full_workload(ctx=ctx, batch=batch, steps=min(total_steps, args.max_positions))
    if args.layers:
        import dataclasses
        wl = dataclasses.replace(wl, geom=dataclasses.replace(wl.geom, n_layers=args.layers))
    if args.window:
        import dataclasses
        wl = dataclasses.replace(wl, geom=dataclasses.replace(wl.geom, attn_window=args.window,
                                                              full_every=args.full_every))
    g = wl.geom
    t_setup = time.perf_counter()
    W = sdev.device_weights(wl)
    pool = sdev.device_kv_pool(wl)
    inp = sdev.device_step_inputs(wl)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    eng = mkd.Engine(g, 0, max_batch=batch, max_pages_per_seq=wl.max_pages)
    eng.load_weights(W)
    eng.set_mode(mkd.MODE_OP_PER_KERNEL if args.mode == "ablation" else mkd.MODE_MEGAKERNEL)
    eng.set_schedule(ORDERS[args.order], PLACEMENTS[args.placement])
    if args.window:
        eng.set_attention_window(args.window, args.full_every)
    stream = torch.cuda.current_stream()
    logits = torch.empty((batch, g.vocab), dtype=torch.float32, device="cuda")
    tokens = inp["tokens"].clone()
    base_lens = inp["h_seq_lens"].copy()
    seq_lens = inp["seq_lens"].clone()
    h_pt = inp["h_page_table"]

    def step(s, ev=None):
        # positions advance one per step and wrap after max_positions tokens
        off = s % args.max_positions
        h_lens = base_lens + off
        seq_lens.copy_(torch.from_numpy(h_lens), non_blocking=False) if off == 0 else seq_lens.add_(1)
        if ev is not None:
            ev[0].record(stream)
        eng.decode_step(tokens, seq_lens, h_lens, inp["page_table"], pool, wl.n_pages, logits,
                        stream=stream.cuda_stream)
        if ev is not None:
            ev[1].record(stream)
        torch.argmax(logits, dim=-1, out=tokens_i64)
        tokens.copy_(tokens_i64)

    tokens_i64 = torch.empty(batch, dtype=torch.int64, device="cuda")
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    eng.sync_status()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    eng.sync_status()
    launch_ms = np.array([a.elapsed_time(b) for a, b in events])
    elapsed = t1 - t0
    ms_per_step = elapsed / args.steps * 1e3
    value = batch * args.steps / elapsed
    # algorithmic bytes of each timed step (batch 1: top-k picks k distinct experts)
    ids = eng.debug_read(mkd.DEBUG_TOPK_IDS, batch)
    distinct = [len(np.unique(ids[l])) for l in range(g.n_layers)]
    step_bytes = []
    for i in range(args.steps):
        off = (args.warmup + i) % args.max_positions
        step_bytes.append(algorithmic_bytes(g, [s + off for s in wl.seq_lens], distinct))
    mean_bytes = float(np.mean(step_bytes))
    achieved = mean_bytes / (float(np.mean(launch_ms)) * 1e-3) / 1e9
    sol_ms = mean_bytes / (PEAK_HBM_GBS * 1e9) * 1e3
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"synthetic 30B-total/~3B-active parallel-transformer MoE, {g.n_layers} layers, "
                        f"batch {batch}, {ctx} cached tokens, greedy decode",
            "batch": batch, "context": ctx, "layers": g.n_layers, "experts": g.n_experts, "top_k": g.top_k,
            "mode": "megakernel" if args.mode != "ablation" else "op-per-kernel",
            "order": args.order, "placement": args.placement,
            **({"attn_window": args.window, "full_every": args.full_every} if args.window else {}),
        },
        "achieved_TBps": round(mean_bytes / (ms_per_step * 1e-3) / 1e12, 4),
        "sol_fraction": round(sol_ms / ms_per_step, 4),
        "sol_tok_s": round(batch / (sol_ms * 1e-3), 1),
        "bytes_per_step": int(mean_bytes),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None,
            "kernel": "mk_persistent" if args.mode != "ablation" else "all step kernels",
            "launch_ms_mean": round(float(np.mean(launch_ms)), 4),
            "launch_ms_p10": round(float(np.percentile(launch_ms, 10)), 4),
            "launch_ms_p90": round(float(np.percentile(launch_ms, 90)), 4),
        },
        "setup_s": round(setup_s, 2),
        "kernel_source": kernel_source_hash(),
    }
    pmc = os.path.join(ROOT, "profiles", "mk_persistent_full_b1_ctx8k_traffic.json")
    if (os.path.exists(pmc) and args.mode != "ablation" and batch == 1 and ctx == 8192 and not args.layers
            and not args.window):
        with open(pmc) as f:
            rec = json.load(f)
        if rec.get("kernel_source") == out["kernel_source"]:
            out["roofline"]["traffic"] = rec.get("traffic_bytes_per_launch")
    if args.trace:
        # one more step with the per-task trace on (not part of the timed region)
        from decode_megakernel_amd import trace as mtrace
        desc, _ = eng.plan(torch.cuda.get_device_properties(0).multi_processor_count)
        buf = torch.zeros((desc.shape[0], 4), dtype=torch.int64, device="cuda")
        eng.set_trace(buf)
        step(args.warmup + args.steps)
        torch.cuda.synchronize()
        eng.sync_status()
        eng.set_trace(None)
        rec = mtrace.decode(desc, buf.cpu().numpy())
        del buf
        summ = mtrace.summarize(rec)
        if args.chrome:
            mtrace.chrome_trace(rec, args.trace + ".chrome.json")
        with open(args.trace, "w") as f:
            json.dump(summ, f, indent=1)
        out["trace_summary"] = {k: summ[k] for k in ("span_us", "layer_span_us_median",
                                                      "workgroup_busy_fraction_mean")}
        if args.tile_report:
            # the traced step's positions and the experts it selected
            off = (args.warmup + args.steps) % args.max_positions
            tids = eng.debug_read(mkd.DEBUG_TOPK_IDS, batch)
            out["tile_report"] = mtrace.tile_report(rec, g, [s + off for s in wl.seq_lens],
                                                    [len(np.unique(tids[l])) for l in range(g.n_layers)])
    # Release every device resource before returning: the engine (its handle; the
    # workspace and weight references it holds), the weights, the KV pool and the step
    # buffers, then return the caching allocator's blocks to the driver.  Nothing is left
    # for C++ static destructors to free inside exit(), where a profiler that has already
    # finalized its own state intercepts the calls.
    torch.cuda.synchronize()
    eng.close()
    del eng, W, pool, inp, logits, tokens, seq_lens, tokens_i64
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if args.calibrate_copy:
        # plain device-to-device copies of a known size, for scaling the HBM byte counters
        # (FETCH_SIZE / WRITE_SIZE) that a profiler reads for the step kernel
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 2.0, out=dst)  # an elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    return out, wl


def run_continuous(args):
    """Continuous batching on the full model through the library's decode loop
    (mkd_server_*): up to 16 live sequences with cached lengths uniform in [512, 32768],
    each generating 8..64 greedy tokens; finished sequences retire and new ones join, over
    `steps` steps.  The KV pool holds seeded N(0, 1) K/V in every page, so a joining
    sequence's cached pages are ready.  A first, untimed pass records each step's batch
    and the experts its tokens selected (the algorithmic bytes: distinct experts per
    layer, every cached K/V read); the timed pass repeats the same steps (the kernel is
    deterministic, the loop's decisions depend only on lengths) without synchronising."""
    import numpy as np
    import torch

    import decode_megakernel_amd as mkd
    import synth
    from synth import device as sdev

    torch.cuda.set_device(0)
    g, B = synth.FULL, 16
    max_pages = -(-(32768 + 64 + 1) // g.page_size) + 1
    n_pages = B * max_pages
    wl = synth.make_workload("continuous", g, [0], spare_pages=n_pages - 1, max_pages=max_pages)
    seqs = synth.continuous_sequences(4 * B + args.steps, g.vocab)
    W = sdev.device_weights(wl)
    pool = sdev.device_kv_pool(wl)
    eng = mkd.Engine(g, 0, max_batch=B, max_pages_per_seq=max_pages)
    eng.load_weights(W)
    eng.set_schedule(ORDERS[args.order], PLACEMENTS[args.placement])
    torch.cuda.synchronize()

    def one_pass(record):
        srv = mkd.Server(eng, n_pages, max_live=B)
        pending, log, tokens = list(seqs), [], 0
        for _ in range(args.steps):
            while pending and srv.try_join(*pending[0]) is not None:
                pending.pop(0)
            n = srv.step(pool)
            tokens += n
            if record:
                st = srv.last_step()
                ids = eng.debug_read(mkd.DEBUG_TOPK_IDS, n)
                log.append((st["seq_lens"].tolist(), [len(np.unique(ids[l])) for l in range(g.n_layers)]))
        torch.cuda.synchronize()
        srv.close()
        return tokens, log

    _, log = one_pass(True)
    eng.sync_status()
    t0 = time.perf_counter()
    tokens, _ = one_pass(False)
    elapsed = time.perf_counter() - t0
    eng.sync_status()
    step_bytes = [algorithmic_bytes(g, lens, distinct) for lens, distinct in log]
    batches = [len(lens) for lens, _ in log]
    ms_per_step = elapsed / args.steps * 1e3
    achieved = float(np.sum(step_bytes)) / elapsed / 1e9
    out = {
        "metric": "continuous-batching decode tok/s + achieved HBM GB/s (algorithmic bytes)",
        "value": round(tokens / elapsed, 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "full synthetic 30B-total/~3B-active MoE, 48 layers; up to 16 live sequences, "
                               "cached lengths U[512, 32768], 8..64 greedy tokens each, joining and retiring "
                               f"over {args.steps} steps through the library's decode loop",
                   "sequences_available": len(seqs), "order": args.order, "placement": args.placement},
        "batch_mean": round(float(np.mean(batches)), 2), "batch_min": int(np.min(batches)),
        "tokens": tokens, "bytes_per_step_mean": int(np.mean(step_bytes)),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "whole loop (step kernel, token gather, sampling)"},
        "kernel_source": kernel_source_hash(),
    }
    eng.close()
    del eng, W, pool
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def read_counter_csv(path, counter):
    """{kernel name: [value per dispatch]} of one counter from a rocprofv3 counter CSV."""
    import csv
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def traffic_from_counters(fetch_csv, write_csv, kernel="mk_persistent"):
    """HBM bytes per launch of the step kernel from two rocprofv3 --pmc runs (FETCH_SIZE,
    then WRITE_SIZE, KiB per dispatch), each scaled by the reading for the calibration
    kernel (an elementwise multiply reading and writing COPY_BYTES):
    bytes = counter * COPY_BYTES / counter(calibration)."""
    import numpy as np
    res = {}
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        vals = read_counter_csv(path, counter)
        step = [v for k, vs in vals.items() if kernel in k for v in vs]
        copy = [v for k, vs in vals.items() if "MulFunctor" in k for v in vs]
        if not step or not copy:
            raise SystemExit(f"{path}: no {kernel} or calibration copy dispatches for {counter}")
        scale = COPY_BYTES / float(np.median(copy))
        res[name] = {"counter_kib_median": float(np.median(step)), "copy_kib_median": float(np.median(copy)),
                     "bytes_per_count": scale, "bytes": float(np.median(step)) * scale}
    res["traffic_bytes_per_launch"] = res["fetch"]["bytes"] + res["write"]["bytes"]
    return res


def sq_summary(csv_paths, kernel="mk_persistent", n_cu=256, waves_per_cu=8):
    """Per-dispatch medians of the SQ counters that rocprofv3 --pmc wrote for the step kernel
    (several CSVs, one per pass), and the ratios that describe where its waves' cycles go.
    SQ_WAVE_CYCLES and the SQ_WAIT_* / SQ_ACTIVE_INST_* counters are summed over waves (in
    units of 4 cycles on this part, the same unit for all of them, so ratios are exact);
    SQ_INSTS_* count wave instructions."""
    import numpy as np
    med = {}
    for path in csv_paths:
        import csv
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if kernel in row["Kernel_Name"]:
                    vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
        med.update({k: float(np.median(v)) for k, v in vals.items()})
    out = {"counters_median_per_dispatch": med}
    wc = med.get("SQ_WAVE_CYCLES")
    if wc:
        for key in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                    "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM"):
            if key in med:
                out[key.lower() + "_per_wave_cycle"] = round(med[key] / wc, 4)
    if "SQ_INSTS_LDS" in med and "SQ_LDS_BANK_CONFLICT" in med and "SQ_LDS_IDX_ACTIVE" in med:
        out["lds_bank_conflict_per_active_cycle"] = round(med["SQ_LDS_BANK_CONFLICT"] / max(med["SQ_LDS_IDX_ACTIVE"], 1), 4)
    if "SQ_INSTS_VALU" in med and "SQ_INSTS_VMEM" in med:
        out["valu_per_vmem_inst"] = round(med["SQ_INSTS_VALU"] / max(med["SQ_INSTS_VMEM"], 1), 2)
    if "SQ_INSTS_LDS" in med and "SQ_INSTS_VMEM" in med:
        out["lds_per_vmem_inst"] = round(med["SQ_INSTS_LDS"] / max(med["SQ_INSTS_VMEM"], 1), 2)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--ctx", type=int, default=8192)
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (diagnostics)")
    ap.add_argument("--window", type=int, default=0,
                    help="local-attention layers: attend to the last WINDOW positions (0: all layers full)")
    ap.add_argument("--full-every", type=int, default=1,
                    help="with --window: layer l is full attention when (l + 1) %% FULL_EVERY == 0")
    ap.add_argument("--mode", choices=["megakernel", "ablation"], default="megakernel")
    ap.add_argument("--max-positions", type=int, default=128)
    ap.add_argument("--workload", choices=["step", "continuous"], default="step",
                    help="step: the fixed batch of --batch sequences at --ctx (the headline); continuous: "
                         "16 ragged sequences joining and retiring through the library's decode loop")
    ap.add_argument("--order", choices=list(ORDERS), default="default",
                    help="wave order of the task lists (the scheduler's named orders)")
    ap.add_argument("--placement", choices=list(PLACEMENTS), default="round-robin",
                    help="placement of the global task order onto workgroups")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trace", default="", help="write a per-task trace summary (JSON) here")
    ap.add_argument("--chrome", action="store_true", help="with --trace: also write the Chrome trace")
    ap.add_argument("--tile-report", action="store_true",
                    help="with --trace: per-operation bandwidth of the traced step (phase GB/s, per-CU GB/s)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the run, multiply 1 GiB into another 1 GiB buffer three times "
                         "(calibration of the HBM byte counters)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="reduce two rocprofv3 counter CSVs to HBM bytes per step launch and write "
                         "profiles/mk_persistent_full_b1_ctx8k_traffic.json (no GPU run)")
    ap.add_argument("--counters", nargs="+", metavar="CSV",
                    help="reduce rocprofv3 SQ counter CSVs of the step kernel to per-dispatch medians "
                         "and wait/active ratios, printed as JSON (no GPU run)")
    args = ap.parse_args()
    if args.counters:
        print(json.dumps(sq_summary(args.counters), indent=1))
        return
    if args.traffic:
        res = traffic_from_counters(*args.traffic)
        res["kernel_source"] = kernel_source_hash()
        res["sources"] = list(args.traffic)
        with open(os.path.join(ROOT, "profiles", "mk_persistent_full_b1_ctx8k_traffic.json"), "w") as f:
            json.dump(res, f, indent=1)
        print(json.dumps(res))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU sharding is a design "
                                   "note, not an implemented path", "n_gpus": args.gpus}))
        sys.exit(2)
    libs = [os.path.join(ROOT, "decode_megakernel_amd", "libmkd.so"), os.path.join(ROOT, "synth", "libsynth_gpu.so"),
            os.path.join(ROOT, "synth", "libsynth_host.so"), os.path.join(ROOT, "oracle", "liboracle.so")]
    if not all(os.path.exists(p) for p in libs):
        import __graft_entry__
        __graft_entry__.build()
    if args.workload == "continuous":
        print(json.dumps(run_continuous(args)), flush=True)
        return
    out, wl = run(args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
