"""Decode the per-task trace of a megakernel step (see mkd_set_trace in include/mkd.h).

Each task record holds the 100 MHz wall-clock time it started, the time its first
wait on input data (tagged words) completed, the time it ended, and its opcode / workgroup / number of
claimed items.  `summarize` reports, per opcode, the time spent waiting for inputs
and working, per layer the span between its first start and last end, and per
workgroup the idle time; `chrome_trace` writes the timeline in the Chrome /
Perfetto trace-event format.
"""
from __future__ import annotations

import json

import numpy as np

OPNAMES = {0: "nop", 1: "embed", 2: "qkv", 3: "router", 4: "attn", 5: "moe_up", 6: "out", 7: "lm_head", 8: "moe_down"}
TICK_US = 0.01  # 100 MHz


def decode(desc: np.ndarray, trace: np.ndarray) -> dict:
    """desc: [n][32] descriptors (any order, field 7 = global index); trace: [>=n][4] uint64."""
    gidx = desc[:, 7]  # descriptor word D_GIDX
    order = np.argsort(gidx)
    d = desc[order]
    t = trace[: len(d)].astype(np.int64)
    valid = t[:, 2] > 0
    t0 = t[valid, 0].min()
    return {
        "op": d[:, 0],
        "layer": d[:, 1],
        "gidx": d[:, 7],
        "start": (t[:, 0] - t0) * TICK_US,
        "ready": (t[:, 1] - t0) * TICK_US,
        "end": (t[:, 2] - t0) * TICK_US,
        "wg": ((t[:, 3] >> 8) & 0xFFF).astype(np.int64),
        "items": ((t[:, 3] >> 20) & 0xFFF).astype(np.int64),
        "staged": (t[:, 0] - t0 + ((t[:, 3] >> 32) & 0xFFFF)) * TICK_US,
        "done": (t[:, 0] - t0 + ((t[:, 3] >> 48) & 0xFFFF)) * TICK_US,
        "valid": valid,
    }


def summarize(rec: dict) -> dict:
    v = rec["valid"]
    span = float(rec["end"][v].max() - rec["start"][v].min())
    per_op = {}
    for op in np.unique(rec["op"][v]):
        m = v & (rec["op"] == op)
        wait = rec["ready"][m] - rec["start"][m]
        work = rec["end"][m] - rec["ready"][m]
        has = m & (rec["staged"] > rec["start"]) & (rec["done"] > rec["start"])
        per_op[OPNAMES.get(int(op), str(op))] = {
            "tasks": int(m.sum()),
            "wait_us_total": round(float(wait.sum()), 1),
            "work_us_total": round(float(work.sum()), 1),
            "work_us_mean": round(float(work.mean()), 2),
            "items": int(rec["items"][m].sum()),
            # single-tile tasks: ready -> inputs staged, staged -> compute done, done -> end;
            # output tasks: ready (attention combined) -> expert up tiles done, -> last GEMV
            # done, -> end; attention claimers: ready -> first queries staged, -> last
            # partial published, -> end (the combine, when this claimer was last)
            "stage_us_median": round(float(np.median(rec["staged"][has] - rec["ready"][has])), 2) if has.any() else None,
            "compute_us_median": round(float(np.median(rec["done"][has] - rec["staged"][has])), 2) if has.any() else None,
            "epilogue_us_median": round(float(np.median(rec["end"][has] - rec["done"][has])), 2) if has.any() else None,
        }
    layers = {}
    for layer in np.unique(rec["layer"][v]):
        m = v & (rec["layer"] == layer)
        layers[int(layer)] = round(float(rec["end"][m].max() - rec["start"][m].min()), 2)
    n_wg = int(rec["wg"][v].max()) + 1
    busy = np.zeros(n_wg)
    for w in range(n_wg):
        m = v & (rec["wg"] == w)
        busy[w] = float((rec["end"][m] - rec["ready"][m]).sum())
    lay = np.array(list(layers.values()))
    return {
        "span_us": round(span, 1),
        "per_op": per_op,
        "layer_span_us_median": round(float(np.median(lay)), 2) if len(lay) else 0.0,
        "workgroup_busy_fraction_mean": round(float(busy.mean() / span), 4) if span > 0 else 0.0,
        "layers": layers,
        "layer_phases": layer_phases(rec, int(np.median(rec["layer"][v]))) if v.any() else {},
    }


def layer_phases(rec: dict, layer: int) -> dict:
    """Per opcode of one layer: [min, median, max] of task start, input-ready and end
    times (us, relative to the layer's first task start), and the median work time."""
    v = rec["valid"] & (rec["layer"] == layer)
    if not v.any():
        return {}
    t0 = rec["start"][v].min()
    out = {"layer": int(layer)}
    for op in np.unique(rec["op"][v]):
        m = v & (rec["op"] == op)
        q = lambda x: [round(float(x.min() - t0), 1), round(float(np.median(x) - t0), 1), round(float(x.max() - t0), 1)]
        out[OPNAMES.get(int(op), str(op))] = {
            "n": int(m.sum()), "start": q(rec["start"][m]), "ready": q(rec["ready"][m]), "end": q(rec["end"][m]),
            "work_median": round(float(np.median(rec["end"][m] - rec["ready"][m])), 2)}
    return out


def chrome_trace(rec: dict, path: str) -> None:
    ev = []
    v = rec["valid"]
    for i in np.nonzero(v)[0]:
        name = f"{OPNAMES.get(int(rec['op'][i]), '?')} L{int(rec['layer'][i])}"
        wg = int(rec["wg"][i])
        if rec["ready"][i] > rec["start"][i]:
            ev.append({"name": "wait", "ph": "X", "pid": 0, "tid": wg, "ts": float(rec["start"][i]),
                       "dur": float(rec["ready"][i] - rec["start"][i]), "cat": "wait"})
        ev.append({"name": name, "ph": "X", "pid": 0, "tid": wg, "ts": float(rec["ready"][i]),
                   "dur": float(max(rec["end"][i] - rec["ready"][i], 0.0)), "cat": "work",
                   "args": {"gidx": int(rec["gidx"][i]), "items": int(rec["items"][i]),
                            "staged": round(float(rec["staged"][i]), 3), "done": round(float(rec["done"][i]), 3)}})
    with open(path, "w") as f:
        json.dump({"traceEvents": ev, "displayTimeUnit": "ns"}, f)


def op_bytes(geom, seq_lens, n_distinct) -> dict:
    """Algorithmic bytes each operation of one layer streams (bf16 weights, cached K/V):
    QKV rows, router rows, every cached K and V of the batch, gate/up rows of the distinct
    selected experts, O-proj plus their down rows."""
    H, I, hd, nq, nkv, bf = geom.hidden, geom.moe_inter, geom.head_dim, geom.n_q_heads, geom.n_kv_heads, 2
    return {
        "qkv": geom.qkv_rows * H * bf,
        "router": geom.n_experts * H * bf,
        "attn": sum(s + 1 for s in seq_lens) * nkv * hd * 2 * bf,
        "moe_up": n_distinct * 2 * I * H * bf,
        "out": (H * nq * hd + n_distinct * H * I) * bf,
    }


def tile_report(rec: dict, geom, seq_lens, distinct) -> dict:
    """Per operation, the median over layers 1 .. L-1 of: the phase bandwidth (its bytes
    over the span from its first input-ready time to its last end) and the per-CU rate (its
    bytes over the summed work time of its tasks, i.e. the rate of one CU while it works on
    that operation); distinct[l] = distinct experts selected in layer l."""
    v = rec["valid"]
    names = {2: "qkv", 3: "router", 4: "attn", 5: "moe_up", 6: "out"}
    rows = {n: {"phase": [], "per_cu": [], "span_us": [], "bytes": []} for n in names.values()}
    for layer in range(1, geom.n_layers):
        ob = op_bytes(geom, seq_lens, distinct[layer])
        for op, name in names.items():
            m = v & (rec["layer"] == layer) & (rec["op"] == op)
            if not m.any():
                continue
            span = float(rec["end"][m].max() - rec["ready"][m].min())
            work = float((rec["end"][m] - rec["ready"][m]).sum())
            b = ob[name]
            rows[name]["phase"].append(b / (span * 1e-6) / 1e9 if span > 0 else 0.0)
            rows[name]["per_cu"].append(b / (work * 1e-6) / 1e9 if work > 0 else 0.0)
            rows[name]["span_us"].append(span)
            rows[name]["bytes"].append(b)
    out = {}
    for name, r in rows.items():
        if r["phase"]:
            out[name] = {"bytes_per_layer": int(np.median(r["bytes"])),
                         "phase_span_us": round(float(np.median(r["span_us"])), 2),
                         "phase_GBps": round(float(np.median(r["phase"])), 1),
                         "per_cu_GBps": round(float(np.median(r["per_cu"])), 2)}
    return out
