"""Decode and summarise the task trace written by libpmk (pmk_trace_attach).

Each record is one task run by one persistent workgroup: when it was taken,
when its input event was satisfied, and when it had finished and notified, in
ticks of the device's 100 MHz clock. The summary gives, per stage of a layer,
when the first workgroup took the stage, when the last one finished, and how
long the tasks spent waiting and working, averaged over layers; this is where a
step's time goes between the HBM-bound work and the synchronisation.
"""
from __future__ import annotations

import numpy as np

TICK_US = 0.01     # 100 MHz
TASK_NAMES = {1: "qkv", 2: "attn", 3: "o", 4: "gate_up", 5: "down", 6: "router", 7: "route", 8: "moe_gate_up",
              9: "moe_down", 10: "combine"}


def decode(buf: np.ndarray) -> np.ndarray:
    """buf: uint32 [grid][cap][4] -> structured records (wg, type, layer, coord, t0, tw, t1) in microseconds
    from the earliest record (the 32-bit clock may wrap once within the traced step)."""
    buf = np.asarray(buf, dtype=np.uint32)
    grid, cap, _ = buf.shape
    rows = []
    for w in range(grid):
        n = int(buf[w, 0, 0])
        for i in range(1, min(n, cap - 1) + 1):
            e = buf[w, i]
            rows.append((w, int(e[0]) & 0xff, (int(e[0]) >> 8) & 0xff, int(e[0]) >> 16, int(e[1]), int(e[2]),
                         int(e[3])))
    dt = np.dtype([("wg", "i4"), ("type", "i4"), ("layer", "i4"), ("coord", "i4"), ("t0", "f8"), ("tw", "f8"),
                   ("t1", "f8")])
    rec = np.zeros(len(rows), dtype=dt)
    if not rows:
        return rec
    arr = np.array(rows, dtype=np.int64)
    # signed 32-bit distance from the first record, so one clock wrap inside a
    # step does not reorder records; then shift the earliest to zero
    ref = arr[0, 4]
    rel = {f: ((arr[:, j] - ref + (1 << 31)) % (1 << 32)) - (1 << 31) for j, f in ((4, "t0"), (5, "tw"), (6, "t1"))}
    base = rel["t0"].min()
    for f in ("t0", "tw", "t1"):
        rec[f] = (rel[f] - base) * TICK_US
    for j, f in enumerate(("wg", "type", "layer", "coord")):
        rec[f] = arr[:, j]
    return rec


def summary(rec: np.ndarray) -> str:
    """Per-stage table averaged over layers (span = first take to last finish)."""
    if len(rec) == 0:
        return "no trace records"
    lines = []
    total = rec["t1"].max() - rec["t0"].min()
    lines.append(f"records {len(rec)}, workgroups {len(np.unique(rec['wg']))}, layers "
                 f"{rec['layer'].max() + 1}, first take to last finish {total:.1f} us")
    lines.append(f"{'stage':<12}{'tasks/layer':>12}{'ready->done us':>16}{'wait us':>10}{'work us':>10}"
                 f"{'work max':>10}{'gap us':>9}")
    layers = np.unique(rec["layer"])
    types = [t for t in TASK_NAMES if np.any(rec["type"] == t)]
    for i, t in enumerate(types):
        spans, waits, works, wmax, gaps, counts = [], [], [], [], [], []
        for l in layers:
            r = rec[(rec["type"] == t) & (rec["layer"] == l)]
            if len(r) == 0:
                continue
            counts.append(len(r))
            ready = r["tw"].min()
            spans.append(r["t1"].max() - ready)
            waits.append(float(np.mean(r["tw"] - r["t0"])))
            works.append(float(np.mean(r["t1"] - r["tw"])))
            wmax.append(float(np.max(r["t1"] - r["tw"])))
            if i > 0:
                p = rec[(rec["type"] == types[i - 1]) & (rec["layer"] == l)]
                if len(p):
                    # from the previous stage's last finish to this stage's first start
                    gaps.append(ready - p["t1"].max())
        lines.append(f"{TASK_NAMES[t]:<12}{np.mean(counts):>12.1f}{np.mean(spans):>16.2f}{np.mean(waits):>10.2f}"
                     f"{np.mean(works):>10.2f}{np.mean(wmax):>10.2f}{(np.mean(gaps) if gaps else 0.0):>9.2f}")
    per_layer = []
    for l in layers:
        r = rec[rec["layer"] == l]
        per_layer.append(r["t1"].max() - r["t0"].min())
    lines.append(f"layer span (first take to last finish): mean {np.mean(per_layer):.2f} us")
    return "\n".join(lines)
