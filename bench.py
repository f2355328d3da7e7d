"""Decode throughput of the persistent decode megakernel on one MI355X.

One step = one call of ``decode_step`` (dense stack) or ``moe_layer_step`` (MoE
layer) through the C ABI of libpmk.so over one batch of seeded synthetic input
already resident in HBM: a queue/event prologue launch and one persistent
kernel launch that runs every layer.

Default workload: the Llama-3.1-8B-shaped 32-layer bf16 stack at batch 1 with
512 cached positions, advancing one position per step (steps 0..K-1 attend over
512+i+1 entries), a fresh N(0,1) input row per step.

Printed (rank 0, one JSON line): tokens/s, ms per step, and
  roofline      algorithmic HBM bytes of one persistent-kernel launch divided by
                that launch's average duration (HIP events recorded on the
                launch stream by the library around that launch only), against
                8 TB/s; ``traffic`` is the measured HBM bytes per launch from the
                committed rocprofv3 counter summary when it was taken on the
                current kernel source, else null;
  cpu_baseline  the CPU oracle (plain C, double precision, OpenMP) timed on this
                host's cores on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--batch B] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
METRIC = "decode tokens/s + achieved HBM GB/s (% of 8 TB/s peak), 8B-shaped, batch 1–128"
KERNEL_SOURCES = ["persistent_megakernel_04_amd/csrc/pmk_kernels.hip",
                  "persistent_megakernel_04_amd/csrc/pmk_device.h",
                  "persistent_megakernel_04_amd/csrc/pmk_internal.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# Algorithmic bytes: what one step must move at the least. Each weight byte is
# read once per step whatever the batch; each cached K/V entry of each request
# is read once; the new K/V entry of each request is written once. Activations
# (a few KB per request per layer) are not counted.
# ---------------------------------------------------------------------------
def step_bytes(w, lens, experts_touched=None) -> dict:
    eb = w.elem_bytes
    H, d, Hq, Hkv = w.hidden, w.head_dim, w.n_q_heads, w.n_kv_heads
    attn_w = (w.qkv_rows * H + H * Hq * d) * eb + 2 * H * 4
    if w.n_experts:
        E, Fe = w.n_experts, w.expert_ffn_dim
        touched = E if experts_touched is None else experts_touched
        ffn_w = E * H * eb + touched * 3 * H * Fe * eb
    else:
        ffn_w = 3 * H * w.ffn_dim * eb
    kv_row = 2 * Hkv * d * eb                       # K and V of one position, one layer
    kv_read = sum(int(s) for s in lens) * kv_row * w.n_layers
    kv_write = len(lens) * kv_row * w.n_layers
    weights = (attn_w + ffn_w) * w.n_layers
    return {"weights": weights, "kv_read": kv_read, "kv_write": kv_write, "total": weights + kv_read + kv_write}


# ---------------------------------------------------------------------------
# Measured HBM traffic, from the committed rocprofv3 counter summary
# ---------------------------------------------------------------------------
def committed_traffic(workload: str, batch: int):
    """HBM bytes per persistent-kernel launch from profiles/traffic_pmk_main_<workload>_b<batch>.md,
    if that summary was taken on the current kernel source (its 'kernel source' line)."""
    path = os.path.join(ROOT, "profiles", f"traffic_pmk_main_{workload}_b{batch}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"kernel source:\s*`?([0-9a-f]{16})", txt)
    m_b = re.search(r"hbm bytes per launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------
def cpu_baseline(case, budget_s: float = 12.0) -> dict:
    import numpy as np

    import oracle
    from _cases import to_np

    w = case.w
    B = int(case.hidden.shape[0])
    oracle.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    desc = oracle.make_desc(w, case.max_batch, case.max_seq, n_layers=1)
    hidden = to_np(case.hidden).astype(np.float64)
    lens = to_np(case.seq_lens)
    t_compute = 0.0
    layers_done = 0
    for l in range(case.n_layers):
        layer = {k: to_np(v) for k, v in case.layers[l].items()}
        kv_l = np.ascontiguousarray(to_np(case.kv[l]))
        t0 = time.perf_counter()
        hidden = oracle.decode_layer(desc, layer, kv_l, lens, hidden)
        t_compute += time.perf_counter() - t0
        layers_done += 1
        del layer, kv_l
        if t_compute >= budget_s:
            break
    per_step = t_compute / layers_done * case.n_layers
    return {"value": round(B / per_step, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"oracle decode_layer on layers 0..{layers_done - 1} of {case.n_layers} for one step at "
                       f"batch {B} (lengths {lens.tolist()[:4]}{'...' if B > 4 else ''}), {t_compute:.2f} s of "
                       f"compute, extrapolated to the full stack; host copies excluded")}


class RowMajorLayers:
    """Layer l's row-major tensors, regenerated on demand from the same seeds."""

    def __init__(self, w, device):
        self.w, self.device = w, device

    def __getitem__(self, l):
        import synth
        return synth.make_layer_weights(self.w, l, device=self.device)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2_8b_b1")
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-probe", action="store_true", help="first run a plain 2 GiB device-to-device copy "
                    "(a kernel of known traffic, for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--schedule", default="fused", choices=["fused", "layer", "stage", "barrier"],
                    help="fused: the whole stack in one persistent launch per step (the default); layer / stage: "
                    "an ablation that puts a kernel boundary after every layer / every stage of a layer; barrier: "
                    "one launch with a grid-wide barrier after every stage")
    ap.add_argument("--moe-scheduler", default="static", choices=["static", "dynamic"],
                    help="MoE workloads: grouped expert tasks as fixed per-workgroup shares (static) or popped from "
                    "a per-layer queue (dynamic)")
    ap.add_argument("--flush-cache", action="store_true",
                    help="between timed steps, write a 1 GiB buffer so that no weight stays in the 256 MB "
                    "memory-side cache (for working sets that fit it, e.g. the MoE layer at one token); the "
                    "roofline then rests on the persistent kernel's own launch times, which exclude the writes")
    ap.add_argument("--seq-range", type=int, nargs=2, default=None, metavar=("LO", "HI"),
                    help="cached lengths uniform on [LO, HI] instead of the workload's own (e.g. batches beyond 128, "
                    "whose cache at the sweep's lengths would not fit in HBM)")
    ap.add_argument("--weight-layout", default="auto", choices=["auto", "rows", "tiles"],
                    help="weights row-major, or (bfloat16) packed layer by layer, before timing, into the tile "
                    "layout: 16 x 32 tiles, each a contiguous 1 KiB block that one wave-wide load reads, streamed "
                    "non-temporally; auto: tiles for bfloat16 workloads")
    ap.add_argument("--trace", default=None, help="after the timed steps, run one traced step and write a "
                    "per-stage summary of the task trace to this file")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path here has no multi-GPU mode "
              f"(--gpus {args.gpus} requested). Each GPU would run its own share of the requests "
              f"with replicated weights; run one process per GPU.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")

    import numpy as np
    import torch

    import synth
    from _cases import Case

    from persistent_megakernel_04_amd import DecodeModel
    from persistent_megakernel_04_amd.model import pack_layers

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU (the HIP library has no CPU path)")
    dev = "cuda"
    if args.copy_probe:
        src = torch.empty(1 << 29, dtype=torch.float32, device=dev).fill_(1.0)   # 2 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: 3 x copy of 2 GiB (reads 2 GiB, writes 2 GiB each)")
        del src, dst
    w = synth.get_workload(args.workload)
    B = args.batch if args.batch is not None else w.batches[0]
    K, W = args.steps, args.warmup
    # per-step lengths: request b holds lens0[b] + i cached entries at step i
    if args.seq_range is not None:
        lo, hi = args.seq_range
        if not 0 <= lo <= hi:
            sys.exit("--seq-range needs 0 <= LO <= HI")
        lens0 = synth.ragged_lengths(B, lo, hi, (w.name, "lens", B, lo, hi))
    elif w.seq_lo == w.seq_hi:
        lens0 = np.full(B, w.seq_lo, np.int32)
    else:
        lens0 = synth.ragged_lengths(B, w.seq_lo, w.seq_hi, (w.name, "lens", B))
    max_seq = int(lens0.max()) + max(K, W) + 1
    L = w.n_layers
    log(f"workload {w.name}: L={L} H={w.hidden} Hq/Hkv={w.n_q_heads}/{w.n_kv_heads} d={w.head_dim} "
        f"F={w.ffn_dim} E={w.n_experts} dtype={w.dtype} B={B} max_seq={max_seq} steps={K} warmup={W}")

    t0 = time.perf_counter()
    layout = args.weight_layout
    if layout == "auto":
        layout = "tiles" if w.dtype == "bf16" else "rows"
    if layout == "tiles":
        # each layer packed as it is generated; the row-major copy is dropped
        # (the 70B-shaped stack would not fit twice)
        layers = [pack_layers([synth.make_layer_weights(w, l, device=dev)])[0] for l in range(L)]
    else:
        layers = [synth.make_layer_weights(w, l, device=dev) for l in range(L)]
    kv = synth.make_kv_cache(w, B, max_seq, device=dev, n_layers=L)
    hid = torch.stack([synth.make_hidden(w, B, i, device=dev) for i in range(max(K, W, 1))])   # [steps][B][H]
    steps_lens = torch.tensor(np.stack([lens0 + i for i in range(max(K, W, 1))]), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB resident)")

    cpu_case = None
    if not args.no_cpu_baseline:
        # the oracle's sample sees step 0's inputs, taken before any GPU step
        # the oracle takes row-major layers: regenerated one at a time (same seeds) when packed
        cpu_layers = layers if layout == "rows" else RowMajorLayers(w, dev)
        cpu_case = Case(w, L, cpu_layers, kv, hid[0].clone(), steps_lens[0].clone(), B, max_seq)

    model = DecodeModel.from_workload(w, layers, B, max_seq, weight_layout=layout, pack=False)
    log(f"weight layout: {layout}")
    model.set_schedule(args.schedule)
    if w.n_experts:
        model.set_moe_scheduler(args.moe_scheduler)
    stages_per_layer = 8 if w.n_experts else 5
    launches = {"fused": 2, "barrier": 2, "layer": 1 + L, "stage": 1 + L * stages_per_layer}[args.schedule]
    info = model.info()
    log(f"handle: grid={info['grid']} block={info['block']} lds={info['lds_bytes']} "
        f"workspace={info['workspace_bytes'] / 2**20:.1f} MiB")
    hid_work = hid.clone()

    for i in range(W):
        model.step(hid_work[i], kv, steps_lens[i])
    torch.cuda.synchronize()
    if model.device_error() != 0:
        sys.exit("device error during warm-up")

    hid_work.copy_(hid)
    torch.cuda.synchronize()
    model.timing_enable(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev) if args.flush_cache else None
    # per-step events around each call (prologue + persistent kernel), for the spread of step times
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    e0.record()
    h0 = time.perf_counter()
    for i in range(K):
        if flush is not None:
            flush.fill_(float(i))
        marks[i][0].record()
        model.step(hid_work[i], kv, steps_lens[i])
        marks[i][1].record()
    host_us = (time.perf_counter() - h0) / K * 1e6   # host time to submit a step (the launches are asynchronous)
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    step_ms = sorted(a.elapsed_time(b) for a, b in marks)
    main_ms, timed_steps = model.timing_read()
    model.timing_enable(False)
    err = model.device_error()
    if err != 0:
        sys.exit(f"device error {err} during the timed steps")
    assert timed_steps == K, (timed_steps, K)
    ms_per_step = total_ms / K
    avg_main_ms = main_ms / timed_steps

    # algorithmic bytes: average over the K steps (lengths grow by one per step;
    # a MoE step reads the experts its tokens selected, taken from an untimed
    # replay of each step's routing)
    touched = [None] * K
    if w.n_experts:
        topk = torch.empty((B, w.top_k), dtype=torch.int32, device=dev)
        for i in range(K):
            replay = hid[i].clone()
            model.step(replay, kv, steps_lens[i], routing={"topk_idx": topk})
            torch.cuda.synchronize()
            touched[i] = int(torch.unique(topk).numel())
        log(f"experts touched per step: {touched[:8]}{'...' if K > 8 else ''}")
    by = [step_bytes(w, (lens0 + i).tolist(), touched[i]) for i in range(K)]
    bytes_avg = sum(b["total"] for b in by) / K
    achieved = bytes_avg / (avg_main_ms * 1e-3) / 1e9
    step_gbs = bytes_avg / (ms_per_step * 1e-3) / 1e9
    traffic = committed_traffic(w.name, B)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "pmk_main", "kernel_ms": round(avg_main_ms, 4),
                "algorithmic_bytes_per_launch": int(bytes_avg), "step_GBps": round(step_gbs, 1)}
    if args.trace:
        from persistent_megakernel_04_amd import trace as ptrace
        cap = 4096
        tbuf = torch.zeros((info["grid"], cap, 8), dtype=torch.int32, device=dev)
        model.trace_attach(tbuf, cap)
        model.step(hid_work[0], kv, steps_lens[0])
        torch.cuda.synchronize()
        model.trace_attach(None)
        rec = ptrace.decode(tbuf.cpu().numpy().view(np.uint32))
        txt = ptrace.summary(rec)
        with open(args.trace, "w") as f:
            f.write(f"workload {w.name} batch {B} lengths {lens0.tolist()[:8]}\n{txt}\n")
        np.save(args.trace + ".npy", rec)
        log("trace summary:\n" + txt)
    log(f"{K} steps in {total_ms:.2f} ms: {ms_per_step:.4f} ms/step, persistent kernel {avg_main_ms:.4f} ms, "
        f"{achieved:.0f} GB/s ({100 * achieved / HBM_PEAK_GBS:.1f} % of 8 TB/s); step incl. prologue "
        f"{step_gbs:.0f} GB/s")
    model.close()
    del hid_work

    cpu = None
    if cpu_case is not None:
        log("timing the CPU oracle on a sample of the same workload")
        cpu = cpu_baseline(cpu_case, args.cpu_budget)
        log(f"cpu baseline: {cpu}")

    out = {"metric": METRIC, "value": round(B * K / (total_ms * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1,
           "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
           # the projections' matrix-core arithmetic: bf16 operands (activations as bf16 hi + lo pairs)
           # with float32 accumulation for bf16 weights; float32 throughout for float32 weights
           "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
           "data": "synthetic (seeded N(0,0.02) weights, N(0,1) KV cache and inputs)",
           "config": {"workload": w.name, "layers": L, "hidden": w.hidden, "q_heads": w.n_q_heads,
                      "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "ffn": w.ffn_dim,
                      "experts": w.n_experts, "global_batch": B,
                      "seq_len_start": [int(x) for x in lens0[:8]],
                      **({"seq_range": list(args.seq_range)} if args.seq_range is not None else {}),
                      "weights": w.dtype, "kv_cache": w.dtype,
                      "accumulate": "f32", "parallelism": "single GPU", "schedule": args.schedule,
                      "weight_layout": layout,
                      "host_submit_us_per_step": round(host_us, 1), "cache_flushed": bool(args.flush_cache),
                      **({"moe_scheduler": args.moe_scheduler} if w.n_experts else {}),
                      "launches_per_step": launches},
           "roofline": roofline, "cpu_baseline": cpu,
           "step_ms_stats": {"median": round(step_ms[len(step_ms) // 2], 4), "min": round(step_ms[0], 4),
                             "max": round(step_ms[-1], 4)}}
    if w.n_experts:
        # the grouped expert GEMMs' arithmetic (gate, up, down: 2 flops per multiply-add) against the bf16
        # matrix cores' dense peak, over the persistent kernel's time
        flops = 2.0 * B * w.top_k * 3 * w.hidden * w.expert_ffn_dim
        out["moe_mfma"] = {"expert_tflop_per_step": round(flops / 1e12, 5),
                           "achieved_tflops": round(flops / (avg_main_ms * 1e-3) / 1e12, 3),
                           "peak_tflops": 2500.0,
                           "util": round(flops / (avg_main_ms * 1e-3) / 2.5e15, 6)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
