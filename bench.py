"""Benchmark of the tile-aligned W4/W8 x A8 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one pass of the whole hot path over one batch of synthetic input:
  decode  : activation quantization + decode linear for the four
            Llama-3.2-3B-shaped projections (fused qkv 5120x3072, o 3072x3072,
            fused gate_up 16384x3072, down 3072x8192; 25% INT8 tiles) at
            M = 1, 4 and 16 tokens (12 calls); every call reads a different
            copy of the packed weights (24 copies, 1.6 GB) so the weights
            come from HBM, not from the 256 MB last-level cache;
  prefill : activation quantization + prefill linear for the four
            Qwen3-4B-shaped projections (qkv 6144x2560, o 2560x4096,
            gate_up 19456x2560, down 2560x9728; 30% INT8 tiles in bands) at
            M = 2048 tokens.
Inputs are resident in HBM before the timed region.

Timed region: W warm-up steps, then the work of K steps whose launches are
all enqueued while a GPU spin kernel holds the stream (the hold is sized from
the measured host enqueue time, and the line reports whether the host stayed
ahead), so the device runs them back to back as a captured runtime would;
the pages time theirs under CUDA Graph, Table 22.  The K decode segments run
first, then the K prefill segments: the work per step is unchanged, and a
prefill's ~250 MB of FP32 outputs are not still being written back to HBM
while the next decode segment streams its weights (interleaved, that
write-back costs the decode calls about 2 us each).  The region is bracketed
by device synchronizations.  HIP events between the groups (decode
activation quantization, the 12 decode linears, prefill activation
quantization, the 4 prefill linears) time the segments and the back-to-back
linear calls; a linear kernel's average duration is its group's span over
the number of calls.  ms_per_step is the events' span over K.

The JSON line: value = decode HBM GB/s over the decode segment (algorithmic
bytes: packed weights with per-row scales, labels, row offsets, INT8
activations and their scales, FP32 outputs; activation quantization time is
inside the segment); prefill.value = INT8 TOPS over the prefill segment
(2 M N K per call); roofline objects for the decode kernel (HBM-bound) and
the prefill kernel (MFMA-bound) from the per-call event durations;
cpu_baseline = the CPU oracle on a bounded sample, single-threaded.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode linear HBM GB/s (% of peak) + prefill int8 TOPS (% MFMA peak)"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0      # MI355X dense INT8 MFMA, published (no sparsity)
DECODE_M = (1, 4, 16)
PREFILL_M = 2048
N_COPIES = 24


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-models", action="store_true",
                    help="skip the whole-model fields (8B-class decode steps, Qwen3-14B-shaped chunk and step)")
    ap.add_argument("--no-fp32-decode", action="store_true",
                    help="skip the decode segment from FP32 activations (profiles of the timed region)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes three times (the "
                         "known-size reference for the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--split-comparison", action="store_true",
                    help="only time the decode linears of the Llama-3.2-3B shapes with the adaptive "
                         "split and with every fixed split, and print a markdown table")
    ap.add_argument("--grouped", action="store_true",
                    help="only time the App. B.3 grouped-activation route (quantization + decode on "
                         "the Llama-3.2-3B shapes, prefill on the Qwen3-4B shapes) beside the per-token "
                         "route, and print a markdown table")
    ap.add_argument("--pack-and-group", action="store_true",
                    help="only time packing with absmax vs fitted (eq. 7) scales, and decode of "
                         "input-sharing projections called separately vs packed as one group (App. E.4), "
                         "on 8B-class shapes, and print a markdown table")
    ap.add_argument("--transformed", action="store_true",
                    help="only time the App. B.1 block transforms around the linear (X V before "
                         "quantization, Y~ U after it) on the Llama-3.2-3B decode and Qwen3-4B prefill "
                         "shapes, and print a markdown table")
    ap.add_argument("--model-step", action="store_true",
                    help="only time whole decode steps of the 8B-class model (36 layers x 4 packed "
                         "projections resident in HBM; quantization + linear per projection) at "
                         "M = 1, 8, 32, 64: enqueued ahead, captured in a HIP graph, and host-paced "
                         "wall-clock; print a markdown table")
    ap.add_argument("--model-14b", action="store_true",
                    help="only time the Qwen3-14B-shaped model workload (40 layers x 4 packed projections): "
                         "a 65536-token prompt prefilled in 8 chunks of 8192 through all 160 projections, "
                         "with the long-prompt operands built per call or prepared once and kept resident, "
                         "then one batch-32 decode step; print a markdown table")
    ap.add_argument("--chunked-prefill", action="store_true",
                    help="only time a long prompt prefilled in chunks through Qwen3-14B-shaped projections: "
                         "the temporary INT8 operand prepared with every chunk (aq_linear_prefill) or once "
                         "(aq_prefill_prepare + aq_linear_prefill_prepared); print a markdown table")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure reference ceilings with library kernels on this GPU: streaming "
                         "read and copy bandwidth by size, back-to-back launch floor, and hipBLASLt INT8 "
                         "GEMM rate (torch._int_mm) on the prefill shapes and a large square; print a "
                         "markdown table")
    ap.add_argument("--trace-summary", metavar="DB",
                    help="print the per-call kernel times of the timed region from a rocprofv3 "
                         "--kernel-trace database of a default bench run (run with --no-fp32-decode)")
    ap.add_argument("--traffic-summary", nargs=4, metavar="CSV",
                    help="print the per-launch HBM traffic summary from four rocprofv3 counter "
                         "CSVs: bench FETCH_SIZE, bench WRITE_SIZE, copy FETCH_SIZE, copy WRITE_SIZE")
    return ap.parse_args()


def linear_bytes(plan, M: int) -> int:
    """Algorithmic bytes of one linear call: the packed projection with
    per-row scales, INT8 activations + FP32 scales, FP32 outputs."""
    packed = (plan.labels_bytes + 2 * plan.offs_bytes + plan.w4_bytes + plan.w8_bytes
              + plan.s4_bytes + plan.s8_bytes)
    return int(packed + M * plan.K + 4 * M + 4 * M * plan.N)


def clone_packed(aq, pw):
    """A second device copy of a packed projection (same bytes)."""
    t = {k: getattr(pw, k).clone() for k in ("labels", "row_off4", "row_off8", "w4", "w8", "s4", "s8")}
    d = aq.AqPacked(pw.plan.N, pw.plan.K, pw.plan.bN, pw.plan.bK, pw.plan.T4, pw.plan.T8,
                    *(t[k].data_ptr() for k in ("labels", "row_off4", "row_off8", "w4", "w8", "s4", "s8")),
                    pw.desc.meta_host)
    return aq.PackedWeights(plan=pw.plan, labels_host=pw.labels_host, desc=d, meta_host=pw.meta_host, **t)


def setup(aq, gen, torch):
    dev = torch.device("cuda", 0)
    dec = []   # (name, [packed copies], {M: X}, {M: (qx, sx, Y)})
    for proj, N, K in gen.LLAMA3B:
        d = gen.llama3b_decode(proj, max(DECODE_M))
        labels = aq.aq_labels_from_map(d["zmap"].astype(np.uint8))
        pw = aq.aq_pack_weights(torch.from_numpy(d["W"]).to(dev), labels, 64, 128)
        copies = [pw] + [clone_packed(aq, pw) for _ in range(N_COPIES - 1)]
        xs, bufs = {}, {}
        for M in DECODE_M:
            x = gen.llama3b_decode(proj, M)["X"]
            xs[M] = torch.from_numpy(x).to(dev)
            bufs[M] = (torch.empty((M, K), dtype=torch.int8, device=dev),
                       torch.empty((M,), dtype=torch.float32, device=dev),
                       torch.empty((M, N), dtype=torch.float32, device=dev))
        dec.append((proj, copies, xs, bufs))
    ws_need = max(aq.aq_workspace_bytes(c[1][0], M, ph) for c in dec for M in DECODE_M
                  for ph in (aq.AQ_PHASE_DECODE, aq.AQ_PHASE_DECODE_FP32))
    ws = torch.zeros(max(ws_need, 16), dtype=torch.uint8, device=dev)  # counters start at zero
    pre = []
    for proj, N, K in gen.QWEN4B:
        d = gen.qwen4b_prefill(proj, PREFILL_M)
        labels = aq.aq_labels_from_map(d["zmap"].astype(np.uint8))
        pw = aq.aq_pack_weights(torch.from_numpy(d["W"]).to(dev), labels, 64, 128)
        x = torch.from_numpy(d["X"]).to(dev)
        bufs = (torch.empty((PREFILL_M, K), dtype=torch.int8, device=dev),
                torch.empty((PREFILL_M,), dtype=torch.float32, device=dev),
                torch.empty((PREFILL_M, N), dtype=torch.float32, device=dev))
        pre.append((proj, pw, x, bufs))
    torch.cuda.synchronize()
    return dec, ws, pre


def decode_quant(aq, dec):
    """Activation quantization of the 12 decode calls (4 projections x 3 M)."""
    for M in DECODE_M:
        for proj, copies, xs, bufs in dec:
            qx, sx, _ = bufs[M]
            aq.aq_quant_act(xs[M], qx, sx)


def decode_linears(aq, i, dec, ws):
    """The 12 decode linear calls; step i reads weight copies 3i .. 3i+2 (mod 24)."""
    for mi, M in enumerate(DECODE_M):
        c = (i * len(DECODE_M) + mi) % N_COPIES
        for proj, copies, xs, bufs in dec:
            qx, sx, Y = bufs[M]
            aq.aq_linear_decode(copies[c], qx, sx, None, 0, Y, ws)


def decode_fp32_calls(aq, i, dec, ws, two_launch=False):
    """The 12 decode calls from the FP32 activations: aq_linear_decode_fp32
    (one kernel where the tokens fit, else the quantizer into the workspace,
    then the linear), or with two_launch the quantizer and the linear per
    call; same weight copies as decode_linears."""
    for mi, M in enumerate(DECODE_M):
        c = (i * len(DECODE_M) + mi) % N_COPIES
        for proj, copies, xs, bufs in dec:
            qx, sx, Y = bufs[M]
            if two_launch:
                aq.aq_quant_act(xs[M], qx, sx)
                aq.aq_linear_decode(copies[c], qx, sx, None, 0, Y, ws)
            else:
                aq.aq_linear_decode_fp32(copies[c], xs[M], None, 0, Y, ws)


def fp32_decode_segment(aq, torch, dec, ws, steps: int, first: int) -> dict:
    """The decode segment as a caller holding FP32 activations runs it, call
    by call, both ways, each behind its own GPU hold: the quantizer and the
    linear per call, then aq_linear_decode_fp32.  GB/s over the same
    algorithmic bytes as the main line."""
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    cyc = sleep_cycles_per_us(torch)
    dbytes1, _ = step_bytes_ops(dec, [])
    out = {}
    for name, two in (("quant_then_linear", True), ("fp32_entry", False)):
        decode_fp32_calls(aq, first, dec, ws, two)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        decode_fp32_calls(aq, first, dec, ws, two)
        host_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        a, b = E(), E()
        torch.cuda._sleep(int(cyc * (2.0 * host_us * (steps + 1) + 2000.0)))
        a.record()
        for i in range(steps):
            decode_fp32_calls(aq, first + i, dec, ws, two)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        out[name] = {"segment_ms_per_step": round(ms, 4), "GB/s": round(dbytes1 / (ms * 1e-3) / 1e9, 1),
                     "us_per_call": round(ms * 1e3 / (len(DECODE_M) * len(dec)), 3)}
    out["note"] = ("12 calls per step (M = 1, 4, 16); aq_linear_decode_fp32 runs one kernel for "
                   "M*K <= 8192 (here the M = 1 calls of qkv, o, gate_up and down), else the same "
                   "two launches")
    return out


def prefill_quant(aq, pre):
    for proj, pw, x, (qx, sx, Y) in pre:
        aq.aq_quant_act(x, qx, sx)


def prefill_linears(aq, pre):
    for proj, pw, x, (qx, sx, Y) in pre:
        aq.aq_linear_prefill(pw, qx, sx, None, Y)


def run_step(aq, i, dec, ws, pre):
    decode_quant(aq, dec)
    decode_linears(aq, i, dec, ws)
    prefill_quant(aq, pre)
    prefill_linears(aq, pre)


def step_bytes_ops(dec, pre):
    dbytes = sum(linear_bytes(copies[0].plan, M) for M in DECODE_M for _, copies, _, _ in dec)
    pops = sum(2 * PREFILL_M * pw.plan.N * pw.plan.K for _, pw, _, _ in pre)
    return dbytes, pops


# ---------------------------------------------------------------- HBM traffic
# The roofline's traffic figure comes from rocprofv3 counter runs whose summary
# is committed under profiles/ (with the commands that made it); it is
# reported only while the kernel sources still hash to what was profiled.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_llama3b_decode_qwen4b_prefill.md")
KERNEL_SOURCES = {
    "decode": ["aq_decode.hip", "aq_device.h"],
    "prefill": ["aq_expand.hip", "aq_prefill_dense.hip", "aq_prefill_big.hip", "aq_device.h"],
}


def sources_sha(kind: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "mixed_precision_int_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic() -> dict:
    """{kind: bytes per launch} from the committed counter summary, for the
    kinds whose kernel sources are unchanged since it was taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
        blob = json.loads(text.split("```json")[1].split("```")[0])
    except (OSError, IndexError, ValueError):
        return {}
    out = {}
    for kind, rec in blob.get("kernels", {}).items():
        if kind in KERNEL_SOURCES and rec.get("sources_sha") == sources_sha(kind):
            out[kind] = rec["hbm_bytes_per_call"]
    return out


def traffic_summary(paths) -> dict:
    """Per-call HBM bytes of the decode and prefill linears from the counter
    CSVs of a bench run (every dispatch of the run, warm-up included,
    averaged per call), each counter scaled by bytes / counter of a plain
    copy of known size."""
    import csv

    def read(path):
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(open(path))]

    def copy_factor(path, nbytes):
        vals = sorted(v for name, v in read(path) if "copy" in name.lower() or "elementwise" in name.lower())
        return nbytes / (vals[len(vals) // 2] * 1024.0)

    cal_bytes = int(os.environ.get("AQ_COPY_MB", "512")) << 20
    f_fetch, f_write = copy_factor(paths[2], cal_bytes), copy_factor(paths[3], cal_bytes)
    kinds = {"decode": (("decode_kernel",), ("decode_kernel",)),
             "prefill": (("prefill_dense_kernel", "prefill_big_kernel", "prefill_kernel", "expand_kernel"),
                         ("prefill_dense_kernel", "prefill_big_kernel", "prefill_kernel"))}
    res = {}
    for kind, (members, calls) in kinds.items():
        fetch = sum(v for n, v in read(paths[0]) if any(k in n for k in members)) * 1024.0 * f_fetch
        write = sum(v for n, v in read(paths[1]) if any(k in n for k in members)) * 1024.0 * f_write
        ncalls = max(1, sum(1 for n, _ in read(paths[0]) if any(k in n for k in calls)))
        res[kind] = dict(hbm_bytes_per_call=int((fetch + write) / ncalls),
                         fetch_bytes_per_call=int(fetch / ncalls), write_bytes_per_call=int(write / ncalls),
                         calls=ncalls, sources_sha=sources_sha(kind))
    return dict(copy_calibration=dict(bytes=cal_bytes, fetch_factor=round(f_fetch, 4),
                                      write_factor=round(f_write, 4)), kernels=res)


def trace_summary(db_path: str) -> str:
    """Per-call kernel times of the timed region from a rocprofv3 kernel-trace
    database (its `kernels` view) of a bench run made with --no-fp32-decode:
    the dispatches after the last spin kernel (the hold that opens the timed
    region), which runs the decode segments of all steps, then the prefill
    segments.  Decode calls are averaged per position in the step (M, then
    projection, as decode_linears issues them); GB/s and fractions use the
    bench's algorithmic bytes (plans from the same seeded maps, on the host)
    and 2MNK."""
    import sqlite3
    from mixed_precision_int_amd import binding as aqb
    from workloads import gen

    rows = sqlite3.connect(db_path).execute("select name, start, end from kernels order by start").fetchall()
    last = max(i for i, r in enumerate(rows) if "spin_kernel" in r[0])
    tr = [(n, (e - b) / 1000.0) for n, b, e in rows[last + 1:]]
    dec = [d for n, d in tr if "decode_kernel" in n]
    ncall = len(DECODE_M) * len(gen.LLAMA3B)
    steps = len(dec) // ncall
    plans = {}
    for proj, N, K in gen.LLAMA3B:
        z = gen.llama3b_decode(proj, 1)["zmap"]
        plans[proj] = aqb.aq_plan_pack(N, K, 64, 128, aqb.aq_labels_from_map(z.astype(np.uint8)))
    out = [f"Timed region: {steps} steps.", "",
           "| decode call | µs | GB/s |", "|---|---|---|"]
    per_m = {}
    for mi, M in enumerate(DECODE_M):
        for pi, (proj, N, K) in enumerate(gen.LLAMA3B):
            k = mi * len(gen.LLAMA3B) + pi
            us = float(np.mean([dec[s * ncall + k] for s in range(steps)]))
            b = linear_bytes(plans[proj], M)
            per_m.setdefault(M, [0, 0.0])
            per_m[M][0] += b
            per_m[M][1] += us
            out.append(f"| {proj} {N}x{K} M={M} | {us:.2f} | {b / us / 1e3:.0f} |")
    out += ["", "| M | algorithmic MB | kernel µs | GB/s | fraction of 8 TB/s |", "|---|---|---|---|---|"]
    tb, tu = 0, 0.0
    for M, (b, us) in per_m.items():
        tb, tu = tb + b, tu + us
        out.append(f"| {M} | {b / 1e6:.2f} | {us:.2f} | {b / us / 1e3:.0f} | {b / us / 1e3 / 8000:.3f} |")
    out.append(f"| all | {tb / 1e6:.2f} | {tu:.2f} | {tb / tu / 1e3:.0f} | {tb / tu / 1e3 / 8000:.3f} |")
    out.append(f"\nDecode mean per call: {tu / ncall:.2f} µs.")
    pre = [(n, d) for n, d in tr if "expand_kernel" in n or "prefill_big" in n or "prefill_dense" in n]
    gemm = [(n, d) for n, d in pre if "expand_kernel" not in n]
    exp_ = [d for n, d in pre if "expand_kernel" in n]
    nproj = len(gen.QWEN4B)
    psteps = len(gemm) // nproj
    out += ["", "| prefill call | expansion µs | GEMM kernel | GEMM µs | GEMM only | expansion + GEMM |",
            "|---|---|---|---|---|---|"]
    tops, tg, te = 0, 0.0, 0.0
    for pi, (proj, N, K) in enumerate(gen.QWEN4B):
        g = float(np.mean([gemm[s * nproj + pi][1] for s in range(psteps)]))
        e = float(np.mean([exp_[s * nproj + pi] for s in range(psteps)])) if len(exp_) == len(gemm) else 0.0
        kname = gemm[pi][0].replace("void aq::(anonymous namespace)::", "").split("(")[0]
        ops = 2 * PREFILL_M * N * K
        tops, tg, te = tops + ops, tg + g, te + e
        out.append(f"| {proj} {N}x{K} | {e:.2f} | `{kname}` | {g:.2f} | {ops / g / 1e6 / 5000:.3f} | "
                   f"{ops / (g + e) / 1e6 / 5000:.3f} |")
    out.append(f"| all four ({tops / 1e9:.1f} G-ops) | {te:.2f} | | {tg:.2f} | {tops / tg / 1e6 / 5000:.3f} | "
               f"{tops / (tg + te) / 1e6 / 5000:.3f} |")
    out.append(f"\nPrefill mean per call (expansion + GEMM): {(tg + te) / nproj:.2f} µs.")
    return "\n".join(out)


def sleep_cycles_per_us(torch):
    """Rate of torch.cuda._sleep (a spinning kernel), measured with HIP events."""
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    torch.cuda._sleep(20_000_000)
    b.record()
    torch.cuda.synchronize()
    return 20_000_000 / (a.elapsed_time(b) * 1e3)


def cpu_baseline(budget_s: float):
    """The CPU oracle as it stands, single-threaded, on a bounded sample:
    decode linears of the Llama-3.2-3B shapes (activation quantization, INT32
    tile products, FP64 rescale) at M = 1, 4, 16, repeated until the budget;
    prefill on 64 token rows x all outputs of each Qwen3-4B-shaped
    projection."""
    from threadpoolctl import threadpool_limits
    from oracle import aq_oracle as O
    from workloads import gen

    with threadpool_limits(limits=1):
        prep = []
        for proj, N, K in gen.LLAMA3B:
            d = gen.llama3b_decode(proj, max(DECODE_M))
            codes, sW = O.quant_weights(d["W"], d["zmap"], 64, 128)
            pk_bytes = O.packed_bytes_rowscale(int((d["zmap"] == 4).sum()), int((d["zmap"] == 8).sum()),
                                               N // 64, K // 128, 64, 128)
            xs = {M: gen.llama3b_decode(proj, M)["X"] for M in DECODE_M}
            prep.append((N, K, codes, sW, pk_bytes, xs))
        nbytes, t_dec, reps = 0, 0.0, 0
        while t_dec < budget_s * 0.6 or reps == 0:
            for N, K, codes, sW, pk_bytes, xs in prep:
                for M in DECODE_M:
                    t0 = time.perf_counter()
                    qx, sx = O.quant_act(xs[M])
                    O.linear_from_partials(O.tile_partials(qx, codes, 128), sx, sW)
                    t_dec += time.perf_counter() - t0
                    nbytes += pk_bytes + M * K + 4 * M + 4 * M * N
            reps += 1
        ops, t_pre = 0, 0.0
        for proj, N, K in gen.QWEN4B:
            d = gen.qwen4b_prefill(proj, 64)
            codes, sW = O.quant_weights(d["W"], d["zmap"], 64, 128)
            t0 = time.perf_counter()
            qx, sx = O.quant_act(d["X"])
            O.linear_from_partials(O.tile_partials(qx, codes, 128), sx, sW)
            t_pre += time.perf_counter() - t0
            ops += 2 * 64 * N * K
    dec_bps, pre_ops = nbytes / t_dec, ops / t_pre
    return dict(
        value=round(dec_bps / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
        sample=(f"decode linears of the 4 Llama-3.2-3B-shaped projections at M=1,4,16, "
                f"{reps} pass(es), {t_dec:.1f} s; numpy FP64 oracle, 1 thread"),
        prefill=dict(value=round(pre_ops / 1e12, 6), unit="TOPS",
                     sample=f"64 token rows x all outputs of the 4 Qwen3-4B-shaped projections, {t_pre:.1f} s"),
        extrapolated_s=oracle_full_config_seconds(dec_bps, pre_ops),
        cpu_model=cpu_model(),
        host_cores_available=len(os.sched_getaffinity(0)),
    )


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_full_config_seconds(dec_bps: float, pre_ops: float) -> dict:
    """Time the single-threaded oracle would take on the whole of each larger
    workload, extrapolated (not run) from the rates measured on the sample:
    decode by algorithmic bytes, prefill by integer operations.  Bytes count
    the packed weights with their scales and metadata (eq. 18 with per-row
    scales), the INT8 activations and their scales, and the FP32 outputs."""
    from oracle import aq_oracle as O
    from workloads import gen

    def step_bytes(geometry, maps, M):
        total = 0
        for layer in maps:
            for (name, N, K), z in zip(geometry, layer):
                t4, t8 = int((z == 4).sum()), int((z == 8).sum())
                total += O.packed_bytes_rowscale(t4, t8, N // 64, K // 128, 64, 128) + M * K + 4 * M + 4 * M * N
        return total

    m8, m14 = gen.dense8b_maps(), gen.qwen14b_maps()
    q4_ops = sum(2 * PREFILL_M * N * K for _, N, K in gen.QWEN4B)
    q14_ops = sum(2 * 65536 * N * K for _, N, K in gen.QWEN14B) * len(m14)
    out = {"qwen3_4b_prefill_m2048": round(q4_ops / pre_ops, 1)}
    for M in (1, 8, 32, 64):
        out[f"dense8b_decode_step_m{M}"] = round(step_bytes(gen.DENSE8B, m8, M) / dec_bps, 1)
    out["qwen14b_prefill_64k"] = round(q14_ops / pre_ops, 1)
    out["qwen14b_decode_step_m32"] = round(step_bytes(gen.QWEN14B, m14, 32) / dec_bps, 1)
    return out


def split_comparison(aq, torch, dec, ws, reps: int = 48):
    """Adaptive against fixed decode splits (the kernel-level analogue of the
    pages' fixed-vs-adaptive split ablation, Table 22): per call, the average
    over `reps` back-to-back calls behind a GPU hold, each call on the next
    of the 24 weight copies; the weight bytes come from HBM."""
    def timed(calls):
        for f in calls:  # untimed pass: first launches and cold caches stay out of the average
            f()
        torch.cuda.synchronize()
        torch.cuda._sleep(30_000_000)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for f in calls:
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / len(calls)

    splits = (16, 8, 4)
    rows = ["| projection | M | adaptive S | adaptive µs | " + " | ".join(f"S = {s} µs" for s in splits)
            + " | adaptive vs best fixed |", "|---" * (5 + len(splits)) + "|"]
    for proj, copies, xs, bufs in dec:
        for M in DECODE_M:
            qx, sx, Y = bufs[M]
            aq.aq_quant_act(xs[M], qx, sx)
            res = {}
            for s in (0,) + splits:
                calls = [(lambda c=c, s=s: aq.aq_linear_decode(copies[c % N_COPIES], qx, sx, None, s, Y, ws))
                         for c in range(reps)]
                timed(calls[:4])
                res[s] = timed(calls)
            best = min(res[s] for s in splits)
            p = copies[0].plan
            rows.append(f"| {proj} {p.N}x{p.K} | {M} | {aq.aq_decode_split(copies[0], M)} | {res[0]:.2f} | "
                        + " | ".join(f"{res[s]:.2f}" for s in splits) + f" | {best / res[0]:.3f} |")
    print("\n".join(rows))


def grouped_comparison(aq, torch, dec, ws, pre, reps: int = 48):
    """The pages' activation quantizer (App. B.3 groups) against the per-token
    route: per call, quantization and linear separately, decode on the 24
    weight copies (HBM-resident weights), prefill on one copy."""
    def timed(calls):
        for f in calls:  # untimed pass: first launches and cold caches stay out of the average
            f()
        torch.cuda.synchronize()
        torch.cuda._sleep(30_000_000)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for f in calls:
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / len(calls)

    rows = ["| call | M | per-token quant µs | per-token linear µs | grouped quant µs | grouped linear µs "
            "| grouped linear rate |", "|---|---|---|---|---|---|---|"]
    for proj, copies, xs, bufs in dec:
        for M in DECODE_M:
            qx, sx, Y = bufs[M]
            X = xs[M]
            qg, sg = aq.aq_quant_act_grouped(X)
            t = [timed([(lambda: aq.aq_quant_act(X, qx, sx))] * 16),
                 timed([(lambda c=c: aq.aq_linear_decode(copies[c % N_COPIES], qx, sx, None, 0, Y, ws))
                        for c in range(reps)]),
                 timed([(lambda: aq.aq_quant_act_grouped(X, qg, sg))] * 16),
                 timed([(lambda c=c: aq.aq_linear_decode_grouped(copies[c % N_COPIES], qg, sg, None, 0, Y, ws))
                        for c in range(reps)])]
            p = copies[0].plan
            rate = linear_bytes(p, M) / t[3] / 1e3
            rows.append(f"| decode {proj} {p.N}x{p.K} | {M} | " + " | ".join(f"{v:.2f}" for v in t)
                        + f" | {rate:.0f} GB/s |")
    for proj, pw, x, (qx, sx, Y) in pre:
        qg, sg = aq.aq_quant_act_grouped(x)
        pws = torch.empty(max(16, aq.aq_workspace_bytes(pw, PREFILL_M, aq.AQ_PHASE_PREFILL)), dtype=torch.uint8,
                          device=x.device)
        gws = torch.zeros(max(16, aq.aq_workspace_bytes(pw, PREFILL_M, aq.AQ_PHASE_PREFILL_GROUPED)),
                          dtype=torch.uint8, device=x.device)
        t = [timed([(lambda: aq.aq_quant_act(x, qx, sx))] * 4),
             timed([(lambda: aq.aq_linear_prefill(pw, qx, sx, None, Y, pws))] * 4),
             timed([(lambda: aq.aq_quant_act_grouped(x, qg, sg))] * 4),
             timed([(lambda: aq.aq_linear_prefill_grouped(pw, qg, sg, None, Y, gws))] * 4)]
        ops = 2 * PREFILL_M * pw.plan.N * pw.plan.K
        rows.append(f"| prefill {proj} {pw.plan.N}x{pw.plan.K} | {PREFILL_M} | " + " | ".join(f"{v:.2f}" for v in t)
                    + f" | {ops / t[3] / 1e6:.0f} TOPS |")
    print("\n".join(rows))


def transformed_comparison(aq, gen, torch, dec, ws, pre, reps: int = 48):
    """Cost of the online App. B.1 transforms: per call the transform of the
    activations (X V), quantization, both in one pass, the linear, the
    output transform (Y~ U) alone, and the linear with Y~ U applied in its
    epilogue (decode and long-prompt GEMM), each timed alone; "added" is (one
    pass - quantization + the fused linear's excess over the plain one) over
    the untransformed quantization + linear.
    Decode runs on the 24 weight copies (HBM-resident weights); the linear's
    time does not depend on the weight values, so the untransformed packed
    copies stand in for packed W~."""
    tables = aq.transform_tables(*gen.transform_tables())

    def timed(calls):
        for f in calls:  # untimed pass: first launches and cold caches stay out of the average
            f()
        torch.cuda.synchronize()
        torch.cuda._sleep(30_000_000)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for f in calls:
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / len(calls)

    rows = ["| call | M | X V µs | quant µs | X V + quant in one pass µs | linear µs | Y~ U µs "
            "| linear with Y~ U in its epilogue µs | added by the transforms | X V rate | one-pass rate "
            "| Y~ U rate |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    rng = np.random.default_rng(77)
    # the transformed decode hands tile rows over through its own (larger) workspace
    xws = torch.zeros(max(16, max(aq.aq_workspace_bytes(copies[0], M, aq.AQ_PHASE_DECODE_TRANSFORMED)
                                  for _, copies, _, _ in dec for M in DECODE_M)), dtype=torch.uint8,
                      device=dec[0][2][DECODE_M[0]].device)
    todo = [(f"decode {proj}", copies, xs[M], bufs[M], M,
             lambda c, q, s, Y, copies=copies: aq.aq_linear_decode(copies[c % N_COPIES], q, s, None, 0, Y, ws), reps,
             lambda c, q, s, us, Y, copies=copies: aq.aq_linear_decode_transformed(
                 copies[c % N_COPIES], q, s, us, tables, out=Y, ws=xws))
            for proj, copies, xs, bufs in dec for M in DECODE_M]
    for proj, pw, x, bufs in pre:
        pws = torch.empty(max(16, aq.aq_workspace_bytes(pw, PREFILL_M, aq.AQ_PHASE_PREFILL)), dtype=torch.uint8,
                          device=x.device)
        todo.append((f"prefill {proj}", [pw], x, bufs, PREFILL_M,
                     lambda c, q, s, Y, pw=pw, pws=pws: aq.aq_linear_prefill(pw, q, s, None, Y, pws), 8,
                     lambda c, q, s, us, Y, pw=pw, pws=pws: aq.aq_linear_prefill_transformed(pw, q, s, us, tables,
                                                                                           out=Y, ws=pws)))
    for name, copies, X, (qx, sx, Y), M, lin, n, fused in todo:
        N, K = copies[0].plan.N, copies[0].plan.K
        vs = torch.from_numpy(gen.transform_seeds(rng, K // 64)).to(X.device)
        us = torch.from_numpy(gen.transform_seeds(rng, N // 64)).to(X.device)
        Xt = torch.empty_like(X)
        t = [timed([(lambda: aq.aq_transform_rows(X, vs, tables, out=Xt))] * n),
             timed([(lambda: aq.aq_quant_act(Xt, qx, sx))] * n),
             timed([(lambda: aq.aq_quant_act_transformed(X, vs, tables, qx, sx))] * n),
             timed([(lambda c=c: lin(c, qx, sx, Y)) for c in range(n)]),
             timed([(lambda: aq.aq_transform_out(Y, us, tables, out=Y))] * n)]
        tf = timed([(lambda c=c: fused(c, qx, sx, us, Y)) for c in range(n)]) if fused else None
        # with the fused epilogue, the output transform's cost is its excess over the plain linear
        added = (t[2] - t[1] + (tf - t[3] if fused else t[4])) / (t[1] + t[3])
        rows.append(f"| {name} {N}x{K} | {M} | " + " | ".join(f"{v:.2f}" for v in t)
                    + f" | {'%.2f' % tf if fused else '-'} | {100 * added:.1f} % | {8 * M * K / t[0] / 1e3:.0f} GB/s"
                    f" | {5 * M * K / t[2] / 1e3:.0f} GB/s | {8 * M * N / t[4] / 1e3:.0f} GB/s |")
    print("\n".join(rows))


def model_step(aq, gen, torch, reps: int = 10):
    """Whole decode steps of the 8B-class model: all 144 projections (36
    layers x qkv 6144x4096, o 4096x4096, gate_up 28672x4096, down 4096x14336;
    per-layer INT8 fraction ~ U(0.15, 0.45)), packed and resident (about
    5.4 GB, far beyond the last-level cache). A step quantizes each
    projection's activations and runs its decode linear. Three timings:
    launches enqueued behind a GPU hold (device back to back), the step
    captured once as a HIP graph and replayed, and host-paced wall-clock
    (each step enqueued and synchronized). The graph's outputs are checked
    against the eager step's, bit for bit."""
    from mixed_precision_int_amd.model import pack_model
    dev = torch.device("cuda", 0)
    maps = gen.dense8b_maps()
    model = pack_model(gen.DENSE8B, maps, lambda l, name, N, K: gen.device_weights(N, K, gen.seed_for(4, l, name)))
    torch.cuda.synchronize()
    per_us = sleep_cycles_per_us(torch)
    rows = [f"Packed model: {model.nbytes() / 1e9:.3f} GB resident.", "",
            "| M | algorithmic GB / step | enqueued ahead ms | GB/s | HIP graph ms | GB/s | host-paced ms "
            "| graph = eager |", "|---|---|---|---|---|---|---|---|"]
    for M in (1, 8, 32, 64):
        xs = {name: gen.device_acts_outliers(M, K, gen.act_seed(4, 0, name, M)) for name, N, K in gen.DENSE8B}
        bufs = {name: (torch.empty((M, K), dtype=torch.int8, device=dev), torch.empty((M,), dtype=torch.float32, device=dev),
                       torch.empty((M, N), dtype=torch.float32, device=dev)) for name, N, K in gen.DENSE8B}
        need = max(aq.aq_workspace_bytes(pw, M, aq.AQ_PHASE_DECODE) for _, _, pw in model)
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
        nbytes = sum(linear_bytes(pw.plan, M) for _, _, pw in model)

        def step():
            for l, name, pw in model:
                qx, sx, Y = bufs[name]
                aq.aq_quant_act(xs[name], qx, sx)
                aq.aq_linear_decode(pw, qx, sx, None, 0, Y, ws)

        step()
        torch.cuda.synchronize()
        eager = {name: b[2].clone() for name, b in bufs.items()}
        t0 = time.perf_counter()
        step()
        host_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        # enqueued ahead behind a hold
        a, b = E(), E()
        torch.cuda._sleep(int(per_us * (host_us * reps * 1.5 + 2000)))
        a.record()
        for _ in range(reps):
            step()
        b.record()
        torch.cuda.synchronize()
        t_ahead = a.elapsed_time(b) / reps
        # HIP graph
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for Y in bufs.values():
            Y[2].zero_()
        g.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(bufs[name][2], eager[name]) for name in bufs)
        a, b = E(), E()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        same = same and all(torch.equal(bufs[name][2], eager[name]) for name in bufs)
        t_graph = a.elapsed_time(b) / reps
        # host-paced wall-clock
        walls = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            step()
            torch.cuda.synchronize()
            walls.append((time.perf_counter() - t0) * 1e3)
        t_wall = float(np.median(walls))
        rows.append(f"| {M} | {nbytes / 1e9:.3f} | {t_ahead:.3f} | {nbytes / t_ahead / 1e6:.0f} | {t_graph:.3f} | "
                    f"{nbytes / t_graph / 1e6:.0f} | {t_wall:.3f} | {same} |")
        print(rows[-1], flush=True)
        del g, xs, bufs, eager, ws
    print("\n".join(rows))


def model_14b(aq, gen, torch):
    """The Qwen3-14B-shaped workload: 40 layers x (qkv 7168x5120, o 5120x5120,
    gate_up 34816x5120, down 5120x17408), model-wide 30% INT8 tiles, packed
    and resident.  Prefill: 8 chunks of 8192 tokens, chunk-major (each chunk
    through all 160 projections, as a chunked prompt runs), per call the
    activation quantization and the prefill linear; the long-prompt operands
    are either built by every call or prepared once for all 160 projections
    and kept resident (memory the 288 GB of HBM has room for), the
    preparation timed on its own.  Then one batch-32 decode step over the
    160 projections.  Launches are enqueued back to back; HIP events time
    each part.  The prepared route's last outputs are compared bit for bit
    with the per-call route's."""
    from mixed_precision_int_amd.model import pack_model
    dev = torch.device("cuda", 0)
    maps = gen.qwen14b_maps()
    model = pack_model(gen.QWEN14B, maps, lambda l, name, N, K: gen.device_weights(N, K, gen.seed_for(5, l, name)))
    torch.cuda.synchronize()
    print(f"packed model {model.nbytes() / 1e9:.3f} GB", flush=True)
    M, chunks = 8192, 8
    xs = {name: gen.device_acts_heavy_tail(M, K, seed=gen.act_seed(5, 0, name, 0)) for name, N, K in gen.QWEN14B}
    q = {name: (torch.empty((M, K), dtype=torch.int8, device=dev), torch.empty((M,), dtype=torch.float32, device=dev))
         for name, N, K in gen.QWEN14B}
    ys = {name: torch.empty((M, N), dtype=torch.float32, device=dev) for name, N, K in gen.QWEN14B}
    need = max(aq.aq_workspace_bytes(pw, M, aq.AQ_PHASE_PREFILL) for _, _, pw in model)
    shared_ws = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
    ops = chunks * sum(2 * M * pw.N * pw.K for _, _, pw in model)

    def timed(fn):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def prefill_per_call():
        for _ in range(chunks):
            for l, name, pw in model:
                qx, sx = q[name]
                aq.aq_quant_act(xs[name], qx, sx)
                aq.aq_linear_prefill(pw, qx, sx, None, ys[name], shared_ws)

    t_a = timed(prefill_per_call)
    last_a = ys["down"].clone()
    print(f"prefill, operand per call: {t_a:.1f} ms", flush=True)
    wss = {}
    for l, name, pw in model:
        n = aq.aq_workspace_bytes(pw, M, aq.AQ_PHASE_PREFILL)
        wss[(l, name)] = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
    resident = sum(w.numel() for w in wss.values() if w is not None)

    def prepare_all():
        for l, name, pw in model:
            if wss[(l, name)] is not None:
                aq.aq_prefill_prepare(pw, wss[(l, name)])

    def prefill_prepared():
        for _ in range(chunks):
            for l, name, pw in model:
                qx, sx = q[name]
                aq.aq_quant_act(xs[name], qx, sx)
                aq.aq_linear_prefill_prepared(pw, qx, sx, wss[(l, name)], None, ys[name])

    t_p = timed(prepare_all)
    t_b = timed(prefill_prepared)
    same = bool(torch.equal(ys["down"], last_a))
    print(f"prefill, prepared once: {t_p:.1f} + {t_b:.1f} ms", flush=True)
    del wss, xs, q, ys, shared_ws
    torch.cuda.empty_cache()
    Md = 32
    xd = {name: gen.device_acts_outliers(Md, K, seed=gen.act_seed(5, 0, name, 9)) for name, N, K in gen.QWEN14B}
    qd = {name: aq.aq_quant_act(xd[name]) for name, N, K in gen.QWEN14B}
    yd = {name: torch.empty((Md, N), dtype=torch.float32, device=dev) for name, N, K in gen.QWEN14B}
    dneed = max(aq.aq_workspace_bytes(pw, Md, aq.AQ_PHASE_DECODE) for _, _, pw in model)
    dws = torch.zeros(max(16, dneed), dtype=torch.uint8, device=dev)
    dbytes = sum(linear_bytes(pw.plan, Md) for _, _, pw in model)

    def decode_step():
        for l, name, pw in model:
            qx, sx = qd[name]
            aq.aq_quant_act(xd[name], qx, sx)
            aq.aq_linear_decode(pw, qx, sx, None, 0, yd[name], dws)

    decode_step()
    t_d = min(timed(decode_step) for _ in range(3))
    rows = [f"Packed model: {model.nbytes() / 1e9:.3f} GB resident; prepared operands: {resident / 1e9:.2f} GB.", "",
            "| part | ms | rate |", "|---|---|---|",
            f"| 65536-token prefill, 8 x 8192 chunks, operand built by every call | {t_a:.1f} | {ops / t_a / 1e9:.0f} TOPS |",
            f"| operands of all 160 projections prepared once | {t_p:.1f} | |",
            f"| 65536-token prefill over the prepared operands | {t_b:.1f} | {ops / t_b / 1e9:.0f} TOPS |",
            f"| prepared total (preparation + prefill); outputs equal to the per-call route: {same} | {t_p + t_b:.1f} | "
            f"{ops / (t_p + t_b) / 1e9:.0f} TOPS |",
            f"| batch-32 decode step, 160 projections (best of 3) | {t_d:.3f} | {dbytes / t_d / 1e6:.0f} GB/s |"]
    print("\n".join(rows))


def model_fields(aq, gen, torch, reps: int = 5) -> dict:
    """Compact whole-model figures for the bench line (after the timed
    region, outside ms_per_step): the 8B-class model's decode step over all
    144 resident projections at M = 1 and 64 (launches enqueued behind a GPU
    hold, mean of `reps` steps), then the Qwen3-14B-shaped model's one
    8192-token prefill chunk through all 160 projections (operand built by
    every call) and one batch-32 decode step (best of 3).  Each step
    quantizes every projection's activations and runs its linear (the 8B
    M = 1 step also through aq_linear_decode_fp32, which quantizes inside the
    linear's kernel where the tokens fit); rates are algorithmic bytes or
    2MNK operations over the step."""
    from mixed_precision_int_amd.model import pack_model
    dev = torch.device("cuda", 0)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    per_us = sleep_cycles_per_us(torch)
    out = {}

    def timed_ahead(step, n):
        step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step()
        host_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        a, b = E(), E()
        torch.cuda._sleep(int(per_us * (host_us * n * 1.5 + 2000)))
        a.record()
        for _ in range(n):
            step()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def decode_step_fn(model, geometry, M, seed_cfg, salt, fp32=False):
        xs = {name: gen.device_acts_outliers(M, K, gen.act_seed(seed_cfg, 0, name, salt)) for name, N, K in geometry}
        bufs = {name: (torch.empty((M, K), dtype=torch.int8, device=dev),
                       torch.empty((M,), dtype=torch.float32, device=dev),
                       torch.empty((M, N), dtype=torch.float32, device=dev)) for name, N, K in geometry}
        need = max(aq.aq_workspace_bytes(pw, M, ph) for _, _, pw in model
                   for ph in (aq.AQ_PHASE_DECODE, aq.AQ_PHASE_DECODE_FP32))
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)

        def step():
            for _, name, pw in model:
                qx, sx, Y = bufs[name]
                if fp32:  # the quantization inside the linear's kernel where the tokens fit
                    aq.aq_linear_decode_fp32(pw, xs[name], None, 0, Y, ws)
                else:
                    aq.aq_quant_act(xs[name], qx, sx)
                    aq.aq_linear_decode(pw, qx, sx, None, 0, Y, ws)
        return step, sum(linear_bytes(pw.plan, M) for _, _, pw in model)

    model = pack_model(gen.DENSE8B, gen.dense8b_maps(),
                       lambda l, name, N, K: gen.device_weights(N, K, gen.seed_for(4, l, name)))
    torch.cuda.synchronize()
    d8 = {"workload": "8B-class dense model (hidden 4096, FFN 14336, 36 layers), all 144 projections resident, "
                      "one decode step", "packed_gb": round(model.nbytes() / 1e9, 3)}
    for M, fp32 in ((1, False), (1, True), (64, False)):
        step, nbytes = decode_step_fn(model, gen.DENSE8B, M, 4, M, fp32)
        ms = timed_ahead(step, reps)
        d8[f"M{M}" + ("_fp32_entry" if fp32 else "")] = {
            "ms_per_step": round(ms, 3), "GB/s": round(nbytes / ms / 1e6, 1),
            "frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
        del step
    out["dense8b_decode"] = d8
    del model
    torch.cuda.empty_cache()

    model = pack_model(gen.QWEN14B, gen.qwen14b_maps(),
                       lambda l, name, N, K: gen.device_weights(N, K, gen.seed_for(5, l, name)))
    torch.cuda.synchronize()
    q14 = {"workload": "Qwen3-14B-shaped model (hidden 5120, FFN 17408, 40 layers), all 160 projections "
                       "resident", "packed_gb": round(model.nbytes() / 1e9, 3)}
    M = 8192
    xs = {name: gen.device_acts_heavy_tail(M, K, seed=gen.act_seed(5, 0, name, 0)) for name, N, K in gen.QWEN14B}
    q = {name: (torch.empty((M, K), dtype=torch.int8, device=dev), torch.empty((M,), dtype=torch.float32, device=dev))
         for name, N, K in gen.QWEN14B}
    ys = {name: torch.empty((M, N), dtype=torch.float32, device=dev) for name, N, K in gen.QWEN14B}
    need = max(aq.aq_workspace_bytes(pw, M, aq.AQ_PHASE_PREFILL) for _, _, pw in model)
    pws = torch.zeros(max(16, need), dtype=torch.uint8, device=dev)
    ops = sum(2 * M * pw.N * pw.K for _, _, pw in model)

    def chunk():
        for _, name, pw in model:
            qx, sx = q[name]
            aq.aq_quant_act(xs[name], qx, sx)
            aq.aq_linear_prefill(pw, qx, sx, None, ys[name], pws)

    chunk()
    torch.cuda.synchronize()
    a, b = E(), E()
    a.record()
    chunk()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    q14["prefill_chunk_8192"] = {"ms": round(ms, 2), "TOPS": round(ops / ms / 1e9, 1),
                                 "frac": round(ops / ms / 1e9 / INT8_PEAK_TOPS, 4)}
    del xs, q, ys, pws
    torch.cuda.empty_cache()
    step, nbytes = decode_step_fn(model, gen.QWEN14B, 32, 5, 9)
    ms = min(timed_ahead(step, 1) for _ in range(3))
    q14["decode_step_M32"] = {"ms": round(ms, 3), "GB/s": round(nbytes / ms / 1e6, 1),
                              "frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
    out["qwen14b"] = q14
    del model, step
    torch.cuda.empty_cache()
    return out


def chunked_prefill(aq, gen, torch):
    """A 16K-token prompt prefilled in chunks of 1024 or 8192 tokens through
    Qwen3-14B-shaped projections (30% INT8 tiles in bands): the long-prompt
    operand (App. E.3 Prefill) prepared with every chunk, or once for all of
    them (it depends on the weights only).  Outputs compared bit for bit."""
    dev = torch.device("cuda", 0)

    def span(fn, n=1):
        torch.cuda.synchronize()
        torch.cuda._sleep(20_000_000)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    total = 16384
    rows = ["| projection | chunk | chunks | operand prepared per chunk µs | prepared once µs | saved | equal |",
            "|---|---|---|---|---|---|---|"]
    for name, N, K in (("gate_up", 34816, 5120), ("down", 5120, 17408), ("o", 5120, 5120)):
        rng = np.random.default_rng(N + K)
        z = gen.map_bands(rng, N // 64, K // 128, 0.30)
        W = gen.device_weights(N, K, seed=N + K, device=dev)
        pw = aq.aq_pack_weights(W, aq.aq_labels_from_map(z.astype(np.uint8)), 64, 128)
        del W
        ws = torch.empty(max(16, aq.aq_workspace_bytes(pw, 1024, aq.AQ_PHASE_PREFILL)), dtype=torch.uint8, device=dev)
        for chunk in (1024, 8192):
            n = total // chunk
            X = gen.device_acts_heavy_tail(chunk, K, seed=5, device=dev)
            qx, sx = aq.aq_quant_act(X)
            del X
            Ya = torch.empty((chunk, N), dtype=torch.float32, device=dev)
            Yb = torch.empty_like(Ya)

            def per_chunk():
                for _ in range(n):
                    aq.aq_linear_prefill(pw, qx, sx, None, Ya, ws)

            def once():
                aq.aq_prefill_prepare(pw, ws)
                for _ in range(n):
                    aq.aq_linear_prefill_prepared(pw, qx, sx, ws, None, Yb)

            per_chunk(); once()
            ta, tb = span(per_chunk), span(once)
            same = bool(torch.equal(Ya, Yb))
            rows.append(f"| {name} {N}x{K} | {chunk} | {n} | {ta:.0f} | {tb:.0f} | {100 * (ta - tb) / ta:.1f} % | {same} |")
            print(rows[-1], flush=True)
            del qx, sx, Ya, Yb
        del pw, ws
        torch.cuda.empty_cache()
    print("\n".join(rows))


def ceilings(torch):
    """Reference ceilings measured with library kernels (not this library's):
    HBM streaming read (a sum over int64 words) and copy, cycling over
    distinct buffers of at least 1 GiB in total so the 256 MB last-level
    cache does not serve them; the back-to-back floor of a tiny kernel; and
    hipBLASLt INT8 GEMM (torch._int_mm, INT32 out, no rescale, no INT4)."""
    dev = torch.device("cuda", 0)

    def span(fns):
        torch.cuda.synchronize()
        torch.cuda._sleep(20_000_000)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for f in fns:
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / len(fns)

    rows = ["| size MB | read by torch.sum GB/s | copy GB/s (read + write) |", "|---|---|---|"]
    for mb in (6, 16, 32, 64, 256, 1024):
        n = max(1, (1024 + mb - 1) // mb + 1)
        nbytes = mb << 20
        bufs = [torch.ones(nbytes // 8, dtype=torch.int64, device=dev) for _ in range(n)]
        outs = [torch.empty_like(b) for b in bufs]
        reps = max(2 * n, 8)
        for b in bufs:
            b.sum()
        tr = span([(lambda k=k: bufs[k % n].sum()) for k in range(reps)])
        tc = span([(lambda k=k: outs[k % n].copy_(bufs[k % n])) for k in range(reps)])
        rows.append(f"| {mb} | {nbytes / tr / 1e3:.0f} | {2 * nbytes / tc / 1e3:.0f} |")
        del bufs, outs
        torch.cuda.empty_cache()
    one = torch.zeros(1, device=dev)
    for _ in range(3):
        one.add_(1.0)
    tl = span([(lambda: one.add_(1.0))] * 200)
    rows += ["", f"Back-to-back floor of a one-element kernel: {tl:.2f} µs per launch.", "",
             "| INT8 GEMM (hipBLASLt via torch._int_mm) | µs | TOPS |", "|---|---|---|"]
    for M, N, K in ((2048, 6144, 2560), (2048, 2560, 4096), (2048, 19456, 2560), (2048, 2560, 9728),
                    (8192, 34816, 5120), (8192, 8192, 8192)):
        a = torch.randint(-128, 127, (M, K), dtype=torch.int8, device=dev)
        b = torch.randint(-128, 127, (N, K), dtype=torch.int8, device=dev).t()
        torch._int_mm(a, b)
        n = 6 if M * N * K < 2 ** 38 else 3
        t = span([(lambda: torch._int_mm(a, b))] * n)
        rows.append(f"| M {M} x N {N} x K {K} | {t:.1f} | {2 * M * N * K / t / 1e6:.0f} |")
        del a, b
        torch.cuda.empty_cache()
    print("\n".join(rows))


def pack_and_group(aq, gen, torch, reps: int = 24):
    """Pack time with absmax and with eq. 7 fitted scales; decode of the 8B
    attention inputs (q 4096, k 1024, v 1024 rows) and MLP inputs (gate, up
    14336 rows each), K = 4096, called per member or as one packed group
    (App. E.4), each behind one quantization of the shared input."""
    from mixed_precision_int_amd.model import pack_group
    dev = torch.device("cuda", 0)

    def span(fn, n):
        torch.cuda.synchronize()
        torch.cuda._sleep(30_000_000)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    rows = ["| projection | absmax pack ms | eq. 7 pack ms |", "|---|---|---|"]
    for N, K in ((4096, 4096), (28672, 4096), (4096, 14336)):
        rng = np.random.default_rng(N + K)
        lab = aq.aq_labels_from_map(gen.map_uniform(rng, N // 64, K // 128, 0.3).astype(np.uint8))
        W = gen.device_weights(N, K, N + K, device=dev)
        aq.aq_pack_weights(W, lab, 64, 128)
        aq.aq_pack_weights(W, lab, 64, 128, mse=True)
        ta = span(lambda: aq.aq_pack_weights(W, lab, 64, 128), 3) / 1e3
        tm = span(lambda: aq.aq_pack_weights(W, lab, 64, 128, mse=True), 3) / 1e3
        rows.append(f"| {N}x{K} | {ta:.2f} | {tm:.2f} |")
        del W
    rows += ["", "| group | M | members called one by one µs | one grouped call µs |", "|---|---|---|---|"]
    for names, Ns in ((("q", "k", "v"), (4096, 1024, 1024)), (("gate", "up"), (14336, 14336))):
        K = 4096
        rng = np.random.default_rng(len(names))
        ws = [gen.device_weights(N, K, 50 + i, device=dev) for i, N in enumerate(Ns)]
        zs = [gen.map_uniform(rng, N // 64, K // 128, 0.3) for N in Ns]
        members = [aq.aq_pack_weights(w, aq.aq_labels_from_map(z.astype(np.uint8)), 64, 128) for w, z in zip(ws, zs)]
        grp = pack_group(list(names), ws, zs)
        del ws
        for M in (1, 16):
            x = gen.device_acts_outliers(M, K, seed=7, device=dev)
            qx, sx = aq.aq_quant_act(x)
            outs = [torch.empty((M, pw.N), dtype=torch.float32, device=dev) for pw in members]
            Yg = torch.empty((M, grp.packed.N), dtype=torch.float32, device=dev)

            def separate():
                aq.aq_quant_act(x, qx, sx)
                for pw, Y in zip(members, outs):
                    aq.aq_linear_decode(pw, qx, sx, None, 0, Y)

            def grouped():
                aq.aq_quant_act(x, qx, sx)
                aq.aq_linear_decode(grp.packed, qx, sx, None, 0, Yg)

            separate(); grouped()
            rows.append(f"| {'/'.join(names)} {'+'.join(map(str, Ns))}x{K} | {M} | {span(separate, reps):.2f} | "
                        f"{span(grouped, reps):.2f} |")
    print("\n".join(rows))


def _med_min(v):
    return {"median": round(float(np.median(v)), 4), "min": round(float(np.min(v)), 4)}


def main():
    args = parse()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.traffic_summary:
        print(json.dumps(traffic_summary(args.traffic_summary), indent=1))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU sharding is a "
                                   "design note, not implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import mixed_precision_int_amd as aq
    from workloads import gen

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}))
        return
    if args.ceilings:
        ceilings(torch)
        return
    aq.lib()
    if args.model_14b:
        model_14b(aq, gen, torch)
        return
    if args.chunked_prefill:
        chunked_prefill(aq, gen, torch)
        return
    if args.model_step:
        model_step(aq, gen, torch)
        return
    if args.pack_and_group:
        pack_and_group(aq, gen, torch)
        return
    dec, ws, pre = setup(aq, gen, torch)
    if args.split_comparison:
        split_comparison(aq, torch, dec, ws)
        return
    if args.grouped:
        grouped_comparison(aq, torch, dec, ws, pre)
        return
    if args.transformed:
        transformed_comparison(aq, gen, torch, dec, ws, pre)
        return

    t_host = 0.0
    for i in range(args.warmup):
        t = time.perf_counter()
        run_step(aq, i, dec, ws, pre)
        t_host = max(t_host, time.perf_counter() - t)   # host enqueue time of one step
        torch.cuda.synchronize()

    # ---- timed region: K steps enqueued behind a GPU hold, so the device
    # runs them back to back: the K decode segments, then the K prefill
    # segments (each step's work is unchanged; grouping the phases keeps the
    # write-back of a prefill's outputs out of the next step's decode reads);
    # HIP events on the launch stream bracket every group
    K = args.steps
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    d_seg, d_call = [E() for _ in range(K + 1)], [E() for _ in range(K)]
    p_seg, p_call = [E() for _ in range(K + 1)], [E() for _ in range(K)]
    hold_us = 2.0 * t_host * 1e6 * (K + 1) + 2000.0
    cyc = sleep_cycles_per_us(torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(int(hold_us * cyc))
    d_seg[0].record()
    for i in range(K):
        decode_quant(aq, dec)
        d_call[i].record()
        decode_linears(aq, args.warmup + i, dec, ws)
        d_seg[i + 1].record()
    p_seg[0].record()
    for i in range(K):
        prefill_quant(aq, pre)
        p_call[i].record()
        prefill_linears(aq, pre)
        p_seg[i + 1].record()
    t_enq = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dseg = d_seg[0].elapsed_time(d_seg[K])                                   # ms
    dcall = sum(d_call[i].elapsed_time(d_seg[i + 1]) for i in range(K))
    pseg = p_seg[0].elapsed_time(p_seg[K])
    pcall = sum(p_call[i].elapsed_time(p_seg[i + 1]) for i in range(K))
    gpu_ms = d_seg[0].elapsed_time(p_seg[K])
    ncalls_d = K * len(DECODE_M) * len(dec)
    ncalls_p = K * len(pre)
    dbytes1, pops1 = step_bytes_ops(dec, pre)
    dbytes, pops = dbytes1 * K, pops1 * K
    decode_gbs = dbytes / (dseg * 1e-3) / 1e9
    prefill_tops = pops / (pseg * 1e-3) / 1e12
    dk_gbs = dbytes / (dcall * 1e-3) / 1e9
    pk_tops = pops / (pcall * 1e-3) / 1e12
    traffic = load_traffic()
    out = {
        "metric": METRIC,
        "value": round(decode_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(gpu_ms / args.steps, 4),
        "wall_ms_incl_hold": round(wall * 1e3, 2),
        "host_enqueued_ahead": bool(t_enq * 1e6 < hold_us),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded random weights and activations of the stated shapes)",
        "config": {
            "workload": ("decode: Llama-3.2-3B-shaped linears qkv 5120x3072, o 3072x3072, "
                         "gate_up 16384x3072, down 3072x8192, 25% INT8 tiles, M in {1,4,16}; "
                         "prefill: Qwen3-4B-shaped linears qkv 6144x2560, o 2560x4096, "
                         "gate_up 19456x2560, down 2560x9728, 30% INT8 tiles, M=2048"),
            "tile": [64, 128],
            "decode_weight_copies": N_COPIES,
        },
        "roofline": {
            "kernel": "aq_linear_decode",
            "bound": "hbm",
            "achieved": round(dk_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dk_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic.get("decode"),
            "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes_per_call": dbytes1 // (len(DECODE_M) * len(dec)),
            "avg_call_us": round(dcall * 1e3 / max(ncalls_d, 1), 3),
            "bytes_per_step": dbytes // args.steps,
        },
        "prefill": {
            "value": round(prefill_tops, 2),
            "unit": "TOPS",
            "roofline": {
                "kernel": "aq_linear_prefill",
                "bound": "mfma",
                "achieved": round(pk_tops, 2),
                "peak": INT8_PEAK_TOPS,
                "unit": "TOPS",
                "frac": round(pk_tops / INT8_PEAK_TOPS, 4),
                "traffic": traffic.get("prefill"),
                "traffic_unit": "HBM bytes per call",
                "avg_call_us": round(pcall * 1e3 / max(ncalls_p, 1), 3),
            },
        },
        "segments_ms_per_step": {"decode": round(dseg / args.steps, 4),
                                 "prefill": round(pseg / args.steps, 4)},
        # per-step spread (median and minimum over the K timed steps)
        "step_stats": {
            "decode_linear_us_per_call": _med_min([d_call[i].elapsed_time(d_seg[i + 1]) * 1e3
                                                   / (len(DECODE_M) * len(dec)) for i in range(K)]),
            "prefill_linear_us_per_call": _med_min([p_call[i].elapsed_time(p_seg[i + 1]) * 1e3 / len(pre)
                                                    for i in range(K)]),
            "decode_segment_ms": _med_min([d_seg[i].elapsed_time(d_seg[i + 1]) for i in range(K)]),
            "prefill_segment_ms": _med_min([p_seg[i].elapsed_time(p_seg[i + 1]) for i in range(K)]),
        },
    }
    if not args.no_fp32_decode:
        try:  # after the timed region, outside ms_per_step
            out["decode_fp32"] = fp32_decode_segment(aq, torch, dec, ws, args.steps, args.warmup + args.steps)
        except Exception as e:  # the headline line is printed regardless
            out["decode_fp32"] = {"error": f"{type(e).__name__}: {e}"}
    if not args.no_models:
        try:
            out["models"] = model_fields(aq, gen, torch)
        except Exception as e:  # the headline line is printed regardless
            out["models"] = {"error": f"{type(e).__name__}: {e}"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
