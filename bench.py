"""Benchmark of the gated delta-rule hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic inputs:
  * prefill: gdn_chunk_prefill on the single-sequence layer workload
    (T = 32768 tokens, 32 value / 16 key heads, d = 128, bf16 q/k/v/z, chunk
    64, zero initial state, gated-RMSNorm tail, bf16 output [T, 4096]);
  * decode:  gdn_decode_step on the batched-decode workload (256 sequences x
    one token, 32 value / 16 key heads, fp32 state [256, 32, 128, 128]
    updated in place, fused tail).
Inputs are generated on the GPU before timing (resident in HBM).  Each leg is
timed with HIP events recorded on the stream its kernels are launched on.

Prints one JSON line: `value` is prefill tokens/s; the `roofline` object is
for the prefill call (the dominant cost: its chunk-map, prep and scan
launches, timed together; the scan applies the gated-RMSNorm tail itself); the `decode` object carries the decode step's
state-update bandwidth and its own roofline; `traffic` fields are HBM bytes
per call, and `busy_frac_counter` / `executed_flops_counter` the matrix-core
busy fraction and executed flops, from the committed counter summaries in
profiles/ (null when a summary was taken on other kernel sources); `cpu_baseline` is the fp64 oracle
timed on this host's cores over a bounded sample of the same prefill
workload.  After the timed steps, two neighbours of the path are timed on
their own, outside the step: one multi-token decode call (256 sequences x 4
tokens, the shape of speculative verification) in `decode_tokens`, and the
convolution prologue of the 32768-token layer in `prologue`.  The other
two prefill workloads are timed the same way as extra legs in
`prefill_legs`: the 4096-token 8-head layer and the packed batch of 8
sequences (131048 tokens, carried state, tail).  Before every timed prefill
a 512 MiB scratch buffer is overwritten (outside the timed events), so that
inputs come from HBM rather than from the 256 MB last-level cache.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("GDN prefill tokens/s (MFMA util) + decode state-update GB/s vs "
          "HBM peak")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_bench_legs.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_counters_bench_legs.txt")
CSRC = os.path.join(ROOT, "gated_deltanet_recurrence_delta_amd", "csrc")


# HIP sources each measured leg's kernels are built from.  Hardware byte
# counts recorded for a leg describe the kernels of those sources; they are
# reported only while the sources are unchanged.
_COMMON = ["gdn_device.h", "gdn_internal.h"]
TRAFFIC_SOURCES = {
    "prefill": ["prefill_bf16.hip", "gdn_seqmap.h"] + _COMMON,
    "decode": ["decode.hip"] + _COMMON,
    "decode_tokens": ["decode.hip"] + _COMMON,
    "prologue": ["prologue.hip", "gdn_seqmap.h"] + _COMMON,
    "out_proj": ["proj.hip", "gemm.hip", "gdn_proj.h", "gdn_device.h"],
}


def kernel_source_hash(group: str) -> str:
    """Hash of the HIP sources of one measured leg."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(TRAFFIC_SOURCES[group]):
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _recorded(path, suffixes):
    """`<leg>_<suffix>` entries of a committed counter summary whose leg's
    sources still hash to the recorded `<group>_source_hash`."""
    vals = {}
    try:
        with open(path) as f:
            for line in f:
                line = line.split("#", 1)[0].strip()
                if ":" in line:
                    k, v = line.split(":", 1)
                    vals[k.strip()] = v.strip()
    except OSError:
        return {}
    out = {}
    for k, v in vals.items():
        if not k.endswith(suffixes):
            continue
        group = next((g for g in TRAFFIC_SOURCES if k.startswith(g + "_")
                      and not (g == "decode" and k.startswith("decode_tokens"))),
                     None)
        if group and vals.get(group + "_source_hash") == kernel_source_hash(group):
            out[k] = float(v)
    return out


def recorded_mfma():
    """Matrix-core busy fraction and executed flops per call, from the
    committed SQ_VALU_MFMA_BUSY_CYCLES / SQ_INSTS_VALU_MFMA_MOPS_* summary,
    when it was taken on the current kernel sources."""
    return _recorded(MFMA_FILE, ("_mfma_busy_frac", "_mfma_exec_flops"))


def recorded_traffic():
    """HBM bytes per call measured with FETCH_SIZE / WRITE_SIZE counter runs
    (scaled by a plain-copy calibration), from the committed summary, when
    it was taken on the current kernel sources."""
    return _recorded(TRAFFIC_FILE, ("_traffic_bytes",))


HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
FP4_PEAK_TFLOPS = 10100.0    # MI355X dense fp4 (MXFP4) MFMA


def prefill_algorithmic(wl, chunk):
    """Algorithmic FLOPs and bytes of one prefill of workload wl.
    FLOPs per token: h_v (4 C d_v + 6 d_k d_v) + h_k 4 C d_k -- the Grams
    (K K^T, Q K^T), T R, P U, K S^T, Q S^T and U^T K of the chunked form.
    Bytes: every input read once, every output written once, states once."""
    T, hk, hv, dk, dv = wl.total_tokens, wl.h_k, wl.h_v, wl.d_k, wl.d_v
    flops = T * (hv * (4 * chunk * dv + 6 * dk * dv) + hk * 4 * chunk * dk)
    io = 2 if wl.io == "bf16" else 4
    per_tok = (2 * hk * dk * io + hv * dv * io + 2 * hv * 4)  # q, k, v, g, b
    if wl.tail:
        per_tok += hv * dv * io * 2                            # z in, out
    else:
        per_tok += hv * dv * io                                # o out
    state = wl.n_seqs * hv * dv * dk * 4
    nbytes = T * per_tok + state * (2 if wl.s0_std is not None else 1)
    return flops, nbytes


def decode_algorithmic(wl):
    """Bytes of one decode step: the fp32 state read once and written once,
    plus q, k, v, z, gates and the output."""
    N, hk, hv, dk, dv = wl.n_seqs, wl.h_k, wl.h_v, wl.d_k, wl.d_v
    io = 2 if wl.io == "bf16" else 4
    state = N * hv * dv * dk * 4 * 2
    small = N * (2 * hk * dk * io + hv * dv * io * (3 if wl.tail else 2)
                 + 2 * hv * 4)
    flops = N * hv * 6 * dk * dv
    return flops, state + small


def decode_tokens_algorithmic(N, T, hk, hv, d):
    """Bytes of one multi-token decode call (bf16 io, tail): the fp32 state
    read once and written once, plus q, k, v, z, gates and the output of
    every token."""
    state = N * hv * d * d * 4 * 2
    per_tok = 2 * hk * d * 2 + 3 * hv * d * 2 + 2 * hv * 4
    return state + N * T * per_tok


def cpu_baseline(wl, x, budget_s=12.0):
    """Time the fp64 oracle on a bounded sample of the prefill workload:
    the first T' tokens of every value head (tail included), T' grown until
    one timed run takes about budget_s.  Reported in tokens/s of the full
    layer (all value heads)."""
    import numpy as np
    from oracle import oracle as O
    O.build()
    threads = O.max_threads()
    T = wl.total_tokens
    cols = {k: getattr(x, k) for k in ("q", "k", "v", "g", "beta", "z")}
    host = {k: v.float().cpu().numpy() for k, v in cols.items()}
    A, D = x.A_log.cpu().numpy(), x.dt_bias.cpu().numpy()
    w = x.w.cpu().numpy()

    def run(tp):
        t0 = time.perf_counter()
        o, _ = O.prefill(host["q"][:tp], host["k"][:tp], host["v"][:tp],
                         host["g"][:tp], host["beta"][:tp], A, D,
                         n_threads=threads)
        O.tail(o, host["z"][:tp], w, x.eps)
        return time.perf_counter() - t0

    tp = 256
    dt = run(tp)
    while dt < budget_s / 4 and tp < T:
        tp = min(T, int(tp * max(2.0, min(8.0, budget_s / 2 / max(dt, 1e-3)))))
        dt = run(tp)
    return {"value": tp / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "first %d of %d tokens, all %d value heads, fp64 "
                      "token-by-token recurrence + tail, %.1f s"
                      % (tp, T, wl.h_v, dt)}


def prefill_leg(G, I, name, dev, stream, steps, warmup, traffic, mfma,
                flush):
    """One prefill workload timed on its own: `steps` calls, each preceded by
    the cache flush and bracketed by HIP events on the launch stream."""
    import torch
    wl = I.WORKLOADS[name]
    x = I.make_inputs(wl, device=dev)
    shape = ((wl.total_tokens, wl.h_v * wl.d_v) if wl.tail
             else (wl.total_tokens, wl.h_v, wl.d_v))
    out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    fin = torch.empty(wl.n_seqs, wl.h_v, wl.d_v, wl.d_k, dtype=torch.float32,
                      device=dev)
    kw = dict(cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_list,
              initial_state=x.s0, final_state=fin, z=x.z if wl.tail else None,
              norm_weight=x.w if wl.tail else None, eps=x.eps,
              chunk_size=wl.chunk, out=out)
    a, keep = G.binding.make_prefill_args(
        x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias, num_seqs=wl.n_seqs,
        **kw)
    ws_bytes = G.binding.gdn_prefill_workspace_size(a)
    del keep
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def fn():
        G.gdn_chunk_prefill(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
                            workspace=ws, **kw)

    ms = time_launches(fn, stream, steps, warmup, flush=flush)
    t = sum(ms) / len(ms) * 1e-3
    flops, nbytes = prefill_algorithmic(wl, wl.chunk)
    gbs = nbytes / t / 1e9
    tf = flops / t / 1e12
    key = "prefill_" + name.replace("prefill_", "")
    return {"workload": name, "tokens": wl.total_tokens, "seqs": wl.n_seqs,
            "h_v": wl.h_v, "h_k": wl.h_k, "tail": wl.tail,
            "value": wl.total_tokens / t, "unit": "tokens/s",
            "launch_ms": sum(ms) / len(ms), "launch_ms_min": min(ms),
            "launch_ms_median": sorted(ms)[len(ms) // 2], "ws_bytes": ws_bytes,
            "roofline": {"bound": "hbm", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": traffic.get(key + "_traffic_bytes"),
                         "kernel": "gdn_chunk_prefill (chunk map, prep and scan"
                                   + (" with the fused tail" if wl.tail else "")
                                   + " launches)",
                         "algorithmic_bytes": nbytes},
            "mfma": {"algorithmic_flops": flops, "achieved_tflops": tf,
                     "peak_tflops": BF16_PEAK_TFLOPS,
                     "frac_algorithmic": tf / BF16_PEAK_TFLOPS,
                     "busy_frac_counter": mfma.get(key + "_mfma_busy_frac"),
                     "executed_flops_counter": mfma.get(key + "_mfma_exec_flops")}}


def time_launches(fn, stream, steps, warmup, back_to_back=False, flush=None):
    """Per-launch milliseconds of fn() from HIP events on its stream: one
    event pair per launch, or (back_to_back) one pair around `steps`
    launches issued without waiting, the average returned `steps` times --
    for calls so short that a lone launch's event gap is mostly launch
    latency."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if back_to_back:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) / steps] * steps
    ms = []
    for _ in range(steps):
        if flush is not None:
            flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return ms


def out_proj_legs(G, I, dev, stream, steps, warmup, traffic, mfma):
    """The ssm_out projection after the tail (4096 -> 2048): the 32768-token
    prefill with a dense bf16, a packed Q4_K, an FP8 (W8A8) and an MXFP4
    (W4A4) weight, the 256-token decode batch with Q4_K and MXFP4, and a
    single token with Q4_K; bf16 activations and output (FP8 / MXFP4 calls
    include quantizing the activations).  Matrix-core legs report
    algorithmic flops 2 M K N against the dense peak of the dtype the
    products run in (bf16 for bf16 and Q4_K, fp8, fp4); the single token
    reports weight + activation bytes against HBM.
    Each leg's launches are timed back to back (`launch_ms` is their mean)."""
    import torch
    K, N = 4096, 2048
    weights = {"q4k": (I.q4k_weight(N, K, seed=90, device=dev), None),
               "bf16": (I.dense_weight(N, K, seed=91, device=dev), None),
               "fp8": I.fp8_weight(N, K, seed=92, device=dev),
               "mxfp4": I.mxfp4_weight(N, K, seed=93, device=dev)}
    wbytes_of = {"q4k": N * (K // 256) * 144, "bf16": N * K * 2,
                 "fp8": N * K + N * 4, "mxfp4": N * K // 2 + N * K // 32}
    peak_of = {"q4k": BF16_PEAK_TFLOPS, "bf16": BF16_PEAK_TFLOPS,
               "fp8": FP8_PEAK_TFLOPS, "mxfp4": FP4_PEAK_TFLOPS}
    legs = {}
    for name, M, fmt in (("prefill_bf16", 32768, "bf16"),
                         ("prefill_q4k", 32768, "q4k"),
                         ("prefill_fp8", 32768, "fp8"),
                         ("prefill_mxfp4", 32768, "mxfp4"),
                         ("decode_q4k", 256, "q4k"),
                         ("decode_mxfp4", 256, "mxfp4"),
                         ("token_q4k", 1, "q4k")):
        gen = torch.Generator(device=dev).manual_seed(M)
        x = torch.randn(M, K, generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        w, wsc = weights[fmt]
        a = G.binding.make_out_proj_args(x, w, N, weight_format=fmt,
                                         weight_scale=wsc, out=y)
        ws_n = G.binding.gdn_out_proj_workspace_size(a)
        ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
        fn = lambda: G.gdn_out_proj(x, w, N, weight_format=fmt,
                                    weight_scale=wsc, out=y, workspace=ws)
        ms = time_launches(fn, stream, steps, warmup, back_to_back=True)
        t = sum(ms) / len(ms) * 1e-3
        flops = 2.0 * M * K * N
        nbytes = wbytes_of[fmt] + M * K * 2 + M * N * 2
        leg = {"rows": M, "weight": fmt, "launch_ms": t * 1e3,
               "ws_bytes": ws_n,
               "value": M / t, "unit": "tokens/s",
               "algorithmic_flops": flops, "algorithmic_bytes": nbytes}
        if M >= 256:
            tf = flops / t / 1e12
            peak = peak_of[fmt]
            leg["roofline"] = {"bound": "mfma", "achieved": tf,
                               "peak": peak, "unit": "TFLOP/s",
                               "frac": tf / peak,
                               "traffic": traffic.get(
                                   "out_proj_%s_traffic_bytes" % name),
                               "busy_frac_counter": mfma.get(
                                   "out_proj_%s_mfma_busy_frac" % name),
                               "kernel": "gdn_out_proj"}
        else:
            gbs = nbytes / t / 1e9
            leg["roofline"] = {"bound": "hbm", "achieved": gbs,
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": gbs / HBM_PEAK_GBS,
                               "traffic": traffic.get(
                                   "out_proj_%s_traffic_bytes" % name),
                               "kernel": "gdn_out_proj"}
        if name == "prefill_bf16":
            # The vendor GEMM on the same problem, for context only.
            wt = w.t().contiguous()
            yr = torch.empty_like(y)
            ref_ms = time_launches(lambda: torch.matmul(x, wt, out=yr),
                                   stream, steps, warmup, back_to_back=True)
            leg["torch_matmul_ms"] = sum(ref_ms) / len(ref_ms)
            del wt, yr
        legs[name] = leg
        del x, y
    return legs


# ------------------------------------------------------------------------
# Counter summaries.  `bench.py --summarize KIND DIR...` turns rocprofv3
# --pmc output of a bench run into the text summaries kept in profiles/
# (the numbers bench.py reports as `traffic` and `busy_frac_counter`).

# Prefill workloads of the bench in the order it runs them; a prefill call is
# told apart by its prep kernel's grid (chunk slots x value heads x 256).
PREFILL_LEGS = (("prefill", "prefill_t32768_hv32_tail"),
                ("prefill_t4096_h8", "prefill_t4096_h8"),
                ("prefill_varlen_8seq_hv32", "varlen_8seq_hv32"))


def _pmc_dispatches(d):
    """Dispatches of a rocprofv3 --pmc csv directory, in order: kernel
    name, grid size, duration (ns) and the counter values."""
    import csv
    import glob
    rows = {}
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                              recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                e = rows.setdefault(int(r["Dispatch_Id"]), {
                    "kernel": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                    "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                    "c": {}})
                e["c"][r["Counter_Name"]] = (e["c"].get(r["Counter_Name"], 0.0)
                                             + float(r["Counter_Value"]))
    return [rows[k] for k in sorted(rows)]


def _short(kernel):
    """Kernel name without namespaces and parameter list."""
    k = kernel.replace("(anonymous namespace)::", "").replace("void ", "")
    return k.split("(")[0].replace("gdn::", "")


def _classify(dispatches):
    """Leg of each library dispatch of a `--prefill-only --no-out-proj` run
    (prefill legs by their prep grid, the convolution prologue, the plain
    copy of --copy-calibration); other dispatches map to None."""
    from gated_deltanet_recurrence_delta_amd import inputs as I
    by_grid = {}
    for leg, name in PREFILL_LEGS:
        wl = I.WORKLOADS[name]
        by_grid[(wl.total_tokens // 64 + wl.n_seqs) * wl.h_v * 256] = leg
    legs, cur, pending = [], None, []
    for i, d in enumerate(dispatches):
        k = _short(d["kernel"])
        leg = None
        if k == "chunk_map_kernel":
            pending.append(i)
        elif k == "prep_kernel":
            cur = by_grid.get(d["grid"])
            for j in pending:
                legs[j] = cur
            pending = []
            leg = cur
        elif k.startswith("scan_kernel"):
            leg = cur
        elif k.startswith("prologue_kernel"):
            leg = "prologue"
        elif "copyBuffer" in k or "copy_kernel" in k:
            leg = "copy"
        legs.append(leg)
    return legs


def scan_breakdown(dirs):
    """Where the scan kernel's cycles go on the 32768-token layer (the
    `prefill` leg), from counter runs that each hold some of: GRBM_GUI_ACTIVE,
    SQ_WAVE_CYCLES, SQ_BUSY_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY,
    SQ_ACTIVE_INST_*, SQ_WAIT_INST_LDS, SQ_INSTS_*, SQ_LDS_BANK_CONFLICT,
    SQ_LDS_IDX_ACTIVE,
    SQ_VALU_MFMA_BUSY_CYCLES.  Per-wave SQ counters are summed over waves;
    they are reported as fractions of SQ_WAVE_CYCLES (same units), and
    instruction counts per chunk step of one workgroup."""
    from gated_deltanet_recurrence_delta_amd import inputs as I
    wl = I.WORKLOADS["prefill_t32768_hv32_tail"]
    wgs = wl.n_seqs * wl.h_v * 8            # one workgroup per 16-row slice
    chunks = wl.total_tokens // 64          # chunk steps of each workgroup
    c, ns, n = {}, [], {}
    for d in dirs:
        ds = _pmc_dispatches(d)
        for disp, leg in zip(ds, _classify(ds)):
            if leg != "prefill" or not _short(disp["kernel"]).startswith("scan_kernel"):
                continue
            ns.append(disp["ns"])
            for k, v in disp["c"].items():
                c[k] = c.get(k, 0.0) + v
                n[k] = n.get(k, 0) + 1
    avg = {k: c[k] / n[k] for k in c}
    out = ["# scan_kernel on the 32768-token layer (%d workgroups of 11 waves, "
           "%d chunk steps each); %d dispatches over the runs, mean %.1f us"
           % (wgs, chunks, len(ns), sum(ns) / len(ns) / 1e3)]
    cyc = avg.get("GRBM_GUI_ACTIVE", 0.0) / 8
    if cyc:
        out.append("scan_cycles: %.0f   # GRBM_GUI_ACTIVE / 8 XCDs" % cyc)
        out.append("scan_cycles_per_chunk: %.0f" % (cyc / chunks))
    wc = avg.get("SQ_WAVE_CYCLES")
    if wc:
        for k in ("SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                  "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS",
                  "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_SCA",
                  "SQ_ACTIVE_INST_MISC"):
            if k in avg:
                out.append("scan_%s_per_wave_cycle: %.4f" % (k[3:].lower(), avg[k] / wc))
    if "SQ_LDS_BANK_CONFLICT" in avg and "SQ_LDS_IDX_ACTIVE" in avg:
        out.append("scan_lds_bank_conflict_frac: %.4f   # of SQ_LDS_IDX_ACTIVE"
                   % (avg["SQ_LDS_BANK_CONFLICT"] / avg["SQ_LDS_IDX_ACTIVE"]))
    if cyc and "SQ_LDS_IDX_ACTIVE" in avg:
        out.append("scan_lds_active_frac: %.4f   # SQ_LDS_IDX_ACTIVE / (cycles x 256 CUs)"
                   % (avg["SQ_LDS_IDX_ACTIVE"] / (cyc * 256)))
    if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        out.append("scan_mfma_busy_frac: %.4f   # SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)"
                   % (avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 1024)))
    for k in ("SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR", "SQ_INSTS_MFMA",
              "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_SMEM"):
        if k in avg:
            out.append("scan_%s_per_chunk_per_wg: %.1f" % (k[9:].lower(),
                                                           avg[k] / wgs / chunks))
    for k in ("SQ_VMEM_TA_CMD_FIFO_FULL", "SQ_LDS_DATA_FIFO_FULL"):
        if k in avg and cyc:
            out.append("scan_%s_per_cu_cycle: %.4f" % (k[3:].lower(),
                                                       avg[k] / (cyc * 256)))
    return out


def summarize(kind, dirs, prev=None):
    """Text of one summary in profiles/ (see the --summarize help)."""
    groups = {"prefill": "prefill", "prefill_t4096_h8": "prefill",
              "prefill_varlen_8seq_hv32": "prefill", "prologue": "prologue"}
    lines = []
    measured = set()          # groups this run measured besides the prefill legs
    if kind == "traffic":
        fetch, write = _pmc_dispatches(dirs[0]), _pmc_dispatches(dirs[1])
        legs = _classify(fetch)
        assert legs == _classify(write), "the two runs dispatched differently"
        cal = [(f["c"]["FETCH_SIZE"], w["c"]["WRITE_SIZE"], f["grid"])
               for f, w, l in zip(fetch, write, legs) if l == "copy"]
        # The 1 GiB copy: the largest copy dispatch of the run.
        cf, cw, _ = max(cal, key=lambda c: c[1])
        sf, sw = (1 << 20) / cf, (1 << 20) / cw
        lines.append("# Calibration: a plain 1 GiB device copy (bench.py "
                     "--copy-calibration) reads FETCH_SIZE %.1f KiB and "
                     "WRITE_SIZE %.1f KiB -> scale %.4f and %.4f." % (cf, cw, sf, sw))
        for g in sorted(set(groups.values())):
            lines.append("%s_source_hash: %s" % (g, kernel_source_hash(g)))
        for leg in ("prefill", "prefill_t4096_h8", "prefill_varlen_8seq_hv32",
                    "prologue"):
            idx = [i for i, l in enumerate(legs) if l == leg]
            calls = sum(1 for i in idx if _short(fetch[i]["kernel"]) in
                        ("prep_kernel",) or leg == "prologue")
            per = {}
            for i in idx:
                k = _short(fetch[i]["kernel"])
                a = per.setdefault(k, [0.0, 0.0, 0])
                a[0] += fetch[i]["c"]["FETCH_SIZE"] * 1024 * sf
                a[1] += write[i]["c"]["WRITE_SIZE"] * 1024 * sw
                a[2] += 1
            tf = tw = 0.0
            for k, (f, w, n) in per.items():
                lines.append("# %-40s fetch %12.0f B  write %12.0f B  (%d dispatches)"
                             % (k, f / calls, w / calls, n))
                tf += f / calls
                tw += w / calls
            lines.append("%s_fetch_bytes: %.0f" % (leg, tf))
            lines.append("%s_write_bytes: %.0f" % (leg, tw))
            lines.append("%s_traffic_bytes: %.0f" % (leg, tf + tw))
        # A full bench run also holds the decode step (decode_kernel, one
        # dispatch per call) and the multi-token decode (decode_tokens_kernel).
        for leg, kname in (("decode", "decode_kernel<"),
                           ("decode_tokens", "decode_tokens_kernel<")):
            idx = [i for i, d in enumerate(fetch) if _short(d["kernel"]).startswith(kname)]
            if not idx:
                continue
            tf = sum(fetch[i]["c"]["FETCH_SIZE"] for i in idx) * 1024 * sf / len(idx)
            tw = sum(write[i]["c"]["WRITE_SIZE"] for i in idx) * 1024 * sw / len(idx)
            measured.add(leg)
            lines.insert(1, "%s_source_hash: %s" % (leg, kernel_source_hash(leg)))
            lines.append("# %-40s fetch %12.0f B  write %12.0f B  (%d dispatches)"
                         % (kname.rstrip("<"), tf, tw, len(idx)))
            lines.append("%s_fetch_bytes: %.0f" % (leg, tf))
            lines.append("%s_write_bytes: %.0f" % (leg, tw))
            lines.append("%s_traffic_bytes: %.0f" % (leg, tf + tw))
    elif kind == "mfma":
        ds = _pmc_dispatches(dirs[0])
        legs = _classify(ds)
        for g in sorted(set(groups.values())):
            lines.append("%s_source_hash: %s" % (g, kernel_source_hash(g)))
        for leg in ("prefill", "prefill_t4096_h8", "prefill_varlen_8seq_hv32"):
            idx = [i for i, l in enumerate(legs) if l == leg]
            calls = sum(1 for i in idx if _short(ds[i]["kernel"]) == "prep_kernel")
            per = {}
            for i in idx:
                k = _short(ds[i]["kernel"])
                a = per.setdefault(k, [0.0, 0.0, 0.0])
                a[0] += ds[i]["c"].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
                a[1] += ds[i]["c"].get("GRBM_GUI_ACTIVE", 0.0) / 8 * 1024
                a[2] += ds[i]["c"].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
            b = c = f = 0.0
            for k, (bb, cc, ff) in per.items():
                if cc > 0:
                    lines.append("# %-24s busy %.4f  exec bf16 flops per call %.4g"
                                 % (k, bb / cc, ff / calls))
                b, c, f = b + bb, c + cc, f + ff
            lines.append("%s_mfma_busy_frac: %.5f" % (leg, b / c if c else 0.0))
            lines.append("%s_mfma_exec_flops: %.6g" % (leg, f / calls))
    elif kind == "scan":
        lines += scan_breakdown(dirs)
    elif kind == "stats":
        # Per-leg kernel durations from the kernel trace of a default run
        # (prefill kernels told apart by their prep grid, as above).
        import csv
        import glob
        f = sorted(glob.glob(os.path.join(dirs[0], "**", "*kernel_trace.csv"),
                             recursive=True))[0]
        with open(f) as fh:
            ds = [{"kernel": r["Kernel_Name"], "grid": int(r["Grid_Size_X"]),
                   "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                   "id": int(r["Dispatch_Id"])} for r in csv.DictReader(fh)]
        ds.sort(key=lambda d: d["id"])
        legs = _classify(ds)
        agg = {}
        for d, leg in zip(ds, legs):
            k = _short(d["kernel"])
            if not k or k.startswith(("at::", "__amd", "Cijk")):
                continue
            a = agg.setdefault((leg or "-", k), [])
            a.append(d["ns"] / 1e3)
        lines.append("%-26s %-46s %6s %10s %10s %10s" % (
            "leg", "kernel", "calls", "avg_us", "min_us", "max_us"))
        for (leg, k), v in sorted(agg.items(), key=lambda kv: -sum(kv[1]) / len(kv[1])):
            lines.append("%-26s %-46s %6d %10.1f %10.1f %10.1f" % (
                leg, k[:46], len(v), sum(v) / len(v), min(v), max(v)))
    else:
        raise SystemExit("unknown summary kind %r" % kind)
    if prev:
        # Legs this run did not measure (decode, multi-token decode, output
        # projection) keep their lines from the previous summary while their
        # kernel sources hash as recorded there.
        with open(prev) as fh:
            old = [ln.rstrip("\n") for ln in fh]
        hashes = {ln.split(":")[0][:-len("_source_hash")]: ln.split(":")[1].strip()
                  for ln in old if ln.split(":")[0].endswith("_source_hash")}
        kept, pending = [], []
        for ln in old:
            if ln.startswith("# ") and (" fetch " in ln or " busy " in ln):
                pending.append(ln)
                continue
            key = ln.split(":")[0].strip() if ":" in ln and not ln.startswith("#") else None
            grp = None
            if key:
                grp = max((g for g in TRAFFIC_SOURCES if key.startswith(g + "_")),
                          key=len, default=None)
            if (grp and grp not in ("prefill", "prologue") and grp not in measured
                    and hashes.get(grp) == kernel_source_hash(grp)):
                if key.endswith("_source_hash"):
                    lines.insert(0, ln)
                else:
                    kept.extend(pending)
                    kept.append(ln)
            if key or not ln.startswith("# "):
                pending = []
        if kept:
            lines += ["# Kept from the previous summary (legs not in this run, "
                      "kernel sources unchanged):"] + kept
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true")
    ap.add_argument("--decode-only", action="store_true")
    ap.add_argument("--no-decode-tokens", action="store_true",
                    help="skip the multi-token decode measurement")
    ap.add_argument("--no-prologue", action="store_true",
                    help="skip the convolution prologue measurement")
    ap.add_argument("--no-out-proj", action="store_true",
                    help="skip the output projection measurements")
    ap.add_argument("--no-extra-prefill", action="store_true",
                    help="skip the 4096-token and packed-batch prefill legs")
    ap.add_argument("--extra-prefill-only", action="store_true",
                    help="time only the 4096-token and packed-batch legs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for scaling "
                         "hardware byte counters)")
    ap.add_argument("--summarize", nargs="+", metavar="ARG",
                    help="KIND DIR... [--prev FILE]: print the profiles/ "
                         "summary of rocprofv3 --pmc output of a bench run "
                         "(traffic: FETCH_SIZE dir, WRITE_SIZE dir; mfma: "
                         "one dir) and exit")
    ap.add_argument("--prev", help="with --summarize: previous summary whose "
                                   "entries for unmeasured, unchanged legs "
                                   "are kept")
    args = ap.parse_args()
    if args.summarize:
        sys.stdout.write(summarize(args.summarize[0], args.summarize[1:],
                                   args.prev))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the path has no multi-GPU "
              "component (the per-GPU kernel is what is timed); run with "
              "--gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_recurrence_delta_amd as G
    from gated_deltanet_recurrence_delta_amd import inputs as I

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    wl_p = I.WORKLOADS["prefill_t32768_hv32_tail"]
    wl_d = I.WORKLOADS["decode_n256_hv32"]
    do_p = not args.decode_only and not args.extra_prefill_only
    do_d = not args.prefill_only and not args.extra_prefill_only
    do_x = not (args.decode_only or args.no_extra_prefill)
    # Overwritten before every timed prefill so that its inputs come from HBM.
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush = lambda: scratch.fill_(1)

    xp = I.make_inputs(wl_p, device=dev) if do_p else None
    xd = I.make_inputs(wl_d, device=dev) if do_d else None
    if do_p:
        out_p = torch.empty(wl_p.total_tokens, wl_p.h_v * wl_p.d_v,
                            dtype=torch.bfloat16, device=dev)
        fin_p = torch.empty(1, wl_p.h_v, wl_p.d_v, wl_p.d_k,
                            dtype=torch.float32, device=dev)
        a, keep = G.binding.make_prefill_args(
            xp.q, xp.k, xp.v, xp.g, xp.beta, xp.A_log, xp.dt_bias,
            cu_seqlens=xp.cu_seqlens, cu_seqlens_host=xp.cu_list,
            final_state=fin_p, z=xp.z, norm_weight=xp.w, eps=xp.eps,
            chunk_size=wl_p.chunk, out=out_p)
        ws_bytes = G.binding.gdn_prefill_workspace_size(a)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    if do_d:
        state = xd.s0.clone()
        out_d = torch.empty(wl_d.n_seqs, wl_d.h_v * wl_d.d_v,
                            dtype=torch.bfloat16, device=dev)

    def prefill():
        G.gdn_chunk_prefill(
            xp.q, xp.k, xp.v, xp.g, xp.beta, xp.A_log, xp.dt_bias,
            cu_seqlens=xp.cu_seqlens, cu_seqlens_host=xp.cu_list,
            final_state=fin_p, z=xp.z, norm_weight=xp.w, eps=xp.eps,
            chunk_size=wl_p.chunk, out=out_p, workspace=ws)

    def decode():
        G.gdn_decode_step(xd.q, xd.k, xd.v, xd.g, xd.beta, xd.A_log,
                          xd.dt_bias, state, z=xd.z, norm_weight=xd.w,
                          eps=xd.eps, out=out_d)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        if do_p:
            prefill()
        if do_d:
            decode()
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)
    p_ms, d_ms = [], []
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for _ in range(args.steps):
        if do_p:
            flush()
            e0, e1 = ev(), ev()
            e0.record(stream)
            prefill()
            e1.record(stream)
        if do_d:
            if not do_p:
                flush()   # otherwise the prefill keeps the GPU busy meanwhile
            e2, e3 = ev(), ev()
            e2.record(stream)
            decode()
            e3.record(stream)
        torch.cuda.synchronize()
        if do_p:
            p_ms.append(e0.elapsed_time(e1))
        if do_d:
            d_ms.append(e2.elapsed_time(e3))
    wall = time.perf_counter() - t_wall

    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded; inputs resident in HBM)"}
    mean = lambda v: sum(v) / len(v)
    res["ms_per_step"] = (mean(p_ms) if p_ms else 0.0) + (
        mean(d_ms) if d_ms else 0.0)
    res["wall_ms_per_step"] = 1e3 * wall / args.steps
    if not (do_p or do_d):
        res["ms_per_step"] = None
    cfg = {"workload": []}
    traffic = recorded_traffic()
    mfma = recorded_mfma()
    if do_p:
        t = mean(p_ms) * 1e-3
        flops, nbytes = prefill_algorithmic(wl_p, wl_p.chunk)
        res["value"] = wl_p.total_tokens / t
        res["unit"] = "tokens/s"
        gbs = nbytes / t / 1e9
        res["roofline"] = {
            "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": traffic.get("prefill_traffic_bytes"),
            "kernel": "gdn_chunk_prefill (chunk map, prep and scan with the "
                      "fused tail launches)",
            "algorithmic_bytes": nbytes, "launch_ms": mean(p_ms),
            "launch_ms_min": min(p_ms),
            "launch_ms_median": sorted(p_ms)[len(p_ms) // 2]}
        tf = flops / t / 1e12
        res["mfma"] = {"algorithmic_flops": flops, "achieved_tflops": tf,
                       "peak_tflops": BF16_PEAK_TFLOPS,
                       "frac_algorithmic": tf / BF16_PEAK_TFLOPS,
                       "busy_frac_counter": mfma.get("prefill_mfma_busy_frac"),
                       "executed_flops_counter": mfma.get("prefill_mfma_exec_flops")}
        cfg["workload"].append(wl_p.name)
        cfg.update({"prefill_tokens": wl_p.total_tokens, "h_v": wl_p.h_v,
                    "h_k": wl_p.h_k, "d": wl_p.d_k, "chunk": wl_p.chunk,
                    "ws_bytes": ws_bytes})
    if do_d:
        t = mean(d_ms) * 1e-3
        flops, nbytes = decode_algorithmic(wl_d)
        gbs = nbytes / t / 1e9
        res["decode"] = {
            "value": gbs, "unit": "GB/s", "launch_ms": mean(d_ms),
            "launch_ms_min": min(d_ms),
            "roofline": {"bound": "hbm", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": traffic.get("decode_traffic_bytes"),
                         "kernel": "gdn_decode_step (one launch)",
                         "algorithmic_bytes": nbytes}}
        cfg["workload"].append(wl_d.name)
        cfg["decode_seqs"] = wl_d.n_seqs
        if not do_p:
            res["value"], res["unit"] = gbs, "GB/s"
            res["roofline"] = dict(res["decode"]["roofline"],
                                   kernel="decode (gdn_decode_step)")
    if do_d and not args.no_decode_tokens:
        # Multi-token decode (speculative verification of 4 draft tokens per
        # sequence), timed on its own after the step: 256 sequences x 4
        # tokens, same heads, bf16, fused tail, no snapshots.
        NS, TT = wl_d.n_seqs, 4
        del xd
        xt = I.random_case(T_list=[TT] * NS, h_k=wl_d.h_k, h_v=wl_d.h_v,
                           d_k=wl_d.d_k, d_v=wl_d.d_v, io="bf16", seed=12,
                           tail=True, s0_std=0.05, device=dev)
        st_t = xt.s0.clone()
        out_t = torch.empty(NS * TT, wl_d.h_v * wl_d.d_v, dtype=torch.bfloat16,
                            device=dev)

        def decode_tokens():
            G.gdn_decode_tokens(xt.q, xt.k, xt.v, xt.g, xt.beta, xt.A_log,
                                xt.dt_bias, st_t, tokens_per_seq=TT, z=xt.z,
                                norm_weight=xt.w, eps=xt.eps, out=out_t)

        for _ in range(args.warmup):
            decode_tokens()
        torch.cuda.synchronize()
        t_ms = []
        for _ in range(args.steps):
            # The flush keeps the GPU busy while the call is enqueued (as in
            # the prefill legs), so the events bracket the kernel, not the
            # host-side launch.
            flush()
            e4, e5 = ev(), ev()
            e4.record(stream)
            decode_tokens()
            e5.record(stream)
            torch.cuda.synchronize()
            t_ms.append(e4.elapsed_time(e5))
        t = mean(t_ms) * 1e-3
        nbytes = decode_tokens_algorithmic(NS, TT, wl_d.h_k, wl_d.h_v, wl_d.d_k)
        gbs = nbytes / t / 1e9
        res["decode_tokens"] = {
            "value": NS * TT / t, "unit": "tokens/s", "seqs": NS,
            "tokens_per_seq": TT, "launch_ms": mean(t_ms),
            "launch_ms_min": min(t_ms),
            "roofline": {"bound": "hbm", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": traffic.get("decode_tokens_traffic_bytes"),
                         "kernel": "gdn_decode_tokens (one launch, T = 4)",
                         "algorithmic_bytes": nbytes}}
    if do_p and not args.no_prologue:
        # Convolution prologue of the 32768-token layer (q, k, v channels,
        # C = 8192, width 4, bf16 in and out), timed on its own after the
        # step.  HBM-bound: x read once, q/k/v written once.
        Tp, Cp, Wp = wl_p.total_tokens, 2 * wl_p.h_k * wl_p.d_k + wl_p.h_v * wl_p.d_v, 4
        gen = torch.Generator(device=dev).manual_seed(40)
        xc = torch.randn(Tp, Cp, generator=gen, device=dev).to(torch.bfloat16)
        wc = torch.randn(Cp, Wp, generator=gen, device=dev) / 2.0
        bc = 0.1 * torch.randn(Cp, generator=gen, device=dev)
        qo = torch.empty(Tp, wl_p.h_k, wl_p.d_k, dtype=torch.bfloat16, device=dev)
        ko = torch.empty_like(qo)
        vo = torch.empty(Tp, wl_p.h_v, wl_p.d_v, dtype=torch.bfloat16, device=dev)

        def prologue():
            G.gdn_conv_prologue(xc, wc, bc, h_k=wl_p.h_k, h_v=wl_p.h_v,
                                d_k=wl_p.d_k, d_v=wl_p.d_v, q=qo, k=ko, v=vo)

        for _ in range(args.warmup):
            prologue()
        torch.cuda.synchronize()
        c_ms = []
        for _ in range(args.steps):
            e6, e7 = ev(), ev()
            e6.record(stream)
            prologue()
            e7.record(stream)
            torch.cuda.synchronize()
            c_ms.append(e6.elapsed_time(e7))
        t = mean(c_ms) * 1e-3
        nbytes = 2 * Tp * Cp * 2 + Cp * (Wp + 1) * 4
        gbs = nbytes / t / 1e9
        res["prologue"] = {
            "value": Tp / t, "unit": "tokens/s", "width": Wp, "channels": Cp,
            "launch_ms": mean(c_ms), "launch_ms_min": min(c_ms),
            "roofline": {"bound": "hbm", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": traffic.get("prologue_traffic_bytes"),
                         "kernel": "gdn_conv_prologue (one launch)",
                         "algorithmic_bytes": nbytes}}
    if do_x:
        res["prefill_legs"] = {
            name: prefill_leg(G, I, name, dev, stream, args.steps, args.warmup,
                              traffic, mfma, flush)
            for name in ("prefill_t4096_h8", "varlen_8seq_hv32")}
        if not (do_p or do_d):
            leg = res["prefill_legs"]["varlen_8seq_hv32"]
            res["value"], res["unit"] = leg["value"], leg["unit"]
            res["roofline"] = leg["roofline"]
            cfg["workload"].append("varlen_8seq_hv32")
    if do_p and not args.no_out_proj:
        res["out_proj"] = out_proj_legs(G, I, dev, stream, args.steps,
                                        args.warmup, traffic, mfma)
    cfg["workload"] = " + ".join(cfg["workload"])
    res["config"] = cfg
    if do_p and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl_p, xp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
