"""Decode and summarise the task trace written by libpmk (pmk_trace_attach).

Each record is one task run by one persistent workgroup, with the 100 MHz
device clock at seven points: taken, input event satisfied, inputs staged,
weights streamed by wave 0 (attention: wave 0's positions done), partial sums
reduced (attention: every wave done), outputs stored (attention: issued),
notified. The summary gives, per stage of a layer, when the first workgroup
started it and the last one finished, and how the tasks' time splits over
those phases, averaged over layers: where a step's time goes between the
HBM-bound work and the synchronisation around it.
"""
from __future__ import annotations

import numpy as np

TICK_US = 0.01     # 100 MHz
TASK_NAMES = {1: "qkv", 2: "attn", 3: "o", 4: "gate_up", 5: "down", 6: "router", 7: "route", 8: "moe_gate_up",
              9: "moe_down", 10: "combine", 11: "attn_s", 12: "norm1", 13: "norm2", 14: "rope", 15: "append",
              16: "merge"}
PHASES = ("t0", "ready", "staged", "streamed", "reduced", "stored", "t1")
WORDS = 8


def decode(buf: np.ndarray) -> np.ndarray:
    """buf: uint32 [grid][cap][8] -> structured records (wg, type, layer, coord, t0 .. t1) in microseconds from
    the earliest record (the 32-bit clock may wrap once within the traced step). A phase a task does not have
    takes the previous phase's clock."""
    buf = np.asarray(buf, dtype=np.uint32).reshape(buf.shape[0], -1, WORDS)
    grid, cap, _ = buf.shape
    rows = []
    for w in range(grid):
        n = int(buf[w, 0, 0])
        for i in range(1, min(n, cap - 1) + 1):
            e = buf[w, i]
            rows.append([w, int(e[0]) & 0xff, (int(e[0]) >> 8) & 0xff, int(e[0]) >> 16] + [int(x) for x in e[1:8]])
    dt = np.dtype([("wg", "i4"), ("type", "i4"), ("layer", "i4"), ("coord", "i4")] + [(p, "f8") for p in PHASES])
    rec = np.zeros(len(rows), dtype=dt)
    if not rows:
        return rec
    arr = np.array(rows, dtype=np.int64)
    ref = arr[0, 4]
    rel = ((arr[:, 4:11] - ref + (1 << 31)) % (1 << 32)) - (1 << 31)   # signed distance from the first record
    rel = np.maximum.accumulate(rel, axis=1)                            # phases in order
    rel -= rel[:, 0].min()
    for j, p in enumerate(PHASES):
        rec[p] = rel[:, j] * TICK_US
    for j, f in enumerate(("wg", "type", "layer", "coord")):
        rec[f] = arr[:, j]
    return rec


def summary(rec: np.ndarray) -> str:
    """Per-stage table averaged over layers: span from the stage's first ready task to its last finish, the gap
    after the previous stage's last finish, and the mean split of a task's time over its phases."""
    if len(rec) == 0:
        return "no trace records"
    lines = []
    total = rec["t1"].max() - rec["t0"].min()
    lines.append(f"records {len(rec)}, workgroups {len(np.unique(rec['wg']))}, layers "
                 f"{rec['layer'].max() + 1}, first take to last finish {total:.1f} us")
    cols = ("wait", "stage", "stream", "reduce", "store", "notify")
    lines.append(f"{'stage':<12}{'tasks':>7}{'span us':>9}{'gap us':>8}" + "".join(f"{c:>8}" for c in cols) +
                 f"{'max work':>10}")
    layers = np.unique(rec["layer"])
    types = [t for t in TASK_NAMES if np.any(rec["type"] == t)]
    for i, t in enumerate(types):
        spans, gaps, counts, wmax = [], [], [], []
        parts = {c: [] for c in cols}
        for l in layers:
            r = rec[(rec["type"] == t) & (rec["layer"] == l)]
            if len(r) == 0:
                continue
            counts.append(len(r))
            ready = r["ready"].min()
            spans.append(r["t1"].max() - ready)
            wmax.append(float(np.max(r["t1"] - r["ready"])))
            for c, (p0, p1) in zip(cols, zip(PHASES[:-1], PHASES[1:])):
                parts[c].append(float(np.mean(r[p1] - r[p0])))
            if i > 0:
                p = rec[(rec["type"] == types[i - 1]) & (rec["layer"] == l)]
                if len(p):
                    gaps.append(ready - p["t1"].max())
        lines.append(f"{TASK_NAMES[t]:<12}{np.mean(counts):>7.0f}{np.mean(spans):>9.2f}"
                     f"{(np.mean(gaps) if gaps else 0.0):>8.2f}" +
                     "".join(f"{np.mean(parts[c]):>8.2f}" for c in cols) + f"{np.mean(wmax):>10.2f}")
    per_layer = [rec[rec["layer"] == l]["t1"].max() - rec[rec["layer"] == l]["t0"].min() for l in layers]
    lines.append(f"layer span (first take to last finish): mean {np.mean(per_layer):.2f} us")
    s = sync_overhead(rec)
    lines.append(f"event waits: {s['wait_us']:.1f} us per workgroup ({100 * s['wait_frac']:.1f} % of its span), "
                 f"{s['spin_total_us']:.0f} workgroup-us in all; between tasks {s['between_us']:.1f} us per workgroup")
    return "\n".join(lines)


def sync_overhead(rec: np.ndarray) -> dict:
    """Synchronisation cost of a traced step, per workgroup: the time its tasks spent between being taken and
    their input event being seen (spinning, with their weight loads in flight), and the time outside any task,
    against the workgroup's span from its first take to its last finish."""
    waits, spans, between = [], [], []
    for w in np.unique(rec["wg"]):
        r = rec[rec["wg"] == w]
        span = float(r["t1"].max() - r["t0"].min())
        waits.append(float(np.sum(r["ready"] - r["t0"])))
        between.append(span - float(np.sum(r["t1"] - r["t0"])))
        spans.append(span)
    return {"wait_us": float(np.mean(waits)), "wait_frac": float(np.sum(waits) / max(np.sum(spans), 1e-9)),
            "spin_total_us": float(np.sum(waits)), "between_us": float(np.mean(between))}
