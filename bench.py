"""Benchmark of the gated delta rule hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  gdn_gate + gdn_prefill on the chunked-prefill workload
      (B=4 x S=4096 packed, Hq=16, Hv=32, Dk=Dv=128, bf16, qwen gates), then
  gdn_decode on the slot-pool decode workload
      (pool [1024, 32, 128, 128] fp32, B=256 rows with 26 skipped, T=1, bf16).
A 1 GiB buffer is written before the prefill and before the decode so that
neither reads its inputs out of the 256 MB last-level cache.  Kernel times come
from HIP events recorded on the launch stream; `value` is prefill tokens/s
(16384 tokens over the gate + prefill time).

Beside the step, the other workloads are timed the same way (flush, then the
launch; median of the timed runs): the single-head scan (B2 x S64, d16, fp32:
launch latency), the ragged fp32 prefill (8 requests, Hv32, d128, initial
state; bound by the fp32 matrix rate) and the multi-token decode (pool
[512, 16, 64, 128], B64, T4, n2, per-token scatter), plus a plain 1 GiB
device copy as the achievable-bandwidth reference.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--only prefill|decode] [--copy-calib]
    python bench.py --summarize-traffic FETCH.csv WRITE.csv   (no GPU)

Prints one JSON line.

HBM traffic.  `roofline.traffic` and `decode.traffic` come from two
rocprofv3 counter runs of this script with --copy-calib (one collecting
FETCH_SIZE, one WRITE_SIZE); each counter is scaled by what it reads for a
plain 1 GiB streaming pass (torch.neg: 1 GiB read, 1 GiB written).  --summarize-traffic
turns the two counter CSVs into profiles/hbm_traffic_prefill_b4s4096_decode_b256_conv1d_b4s4096.json, stamped with a hash
of the kernel sources; a later run reports the traffic only while that hash
still matches, and null otherwise.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
FP32_MATRIX_PEAK_TFLOPS = 157.3  # MI355X fp32 matrix, TFLOP/s

METRIC = "GDN prefill tokens/s (B4×S4096,Hv32,d128) + decode state HBM GB/s % of peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_prefill_b4s4096_decode_b256_conv1d_b4s4096.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_prefill_b4s4096.json")
CALIB_BYTES = 2 * (1 << 30)   # the calibration copy reads 1 GiB and writes 1 GiB
PREFILL_KERNEL = "prefill_pair_kernel<128,false,false,false,false>"


def kernel_source_hash() -> str:
    """sha256 over the kernel sources of libgdn (.hip, .hpp; the host-only
    argument validation in .cpp does not change a kernel).  Any change
    invalidates the stored counter figures."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_deltanet_state_delta_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


# The kernels each traffic figure belongs to, by the instantiation the timed
# workloads launch (demangled or mangled, as the profiler prints them).
KERNEL_KEYS = (
    ("prefill", ("prefill_pair_kernel<128, false, false, false, false>", "prefill_pair_kernelILi128ELb0ELb0ELb0ELb0E")),
    ("decode", ("decode_kernel<__bf16, 128, 128, 32>", "decode_kernelIDF16bLi128ELi128ELi32E")),
    # extra workloads: the multi-token decode (B64 T4 n2, dv 64), the ragged
    # fp32 prefill (general kernel, 32-token chunks), the per-key-decay prefill
    ("decode_mtp", ("decode_kernel<__bf16, 128, 64, 32>", "decode_kernelIDF16bLi128ELi64ELi32E")),
    ("prefill_f32", ("prefill_kernel<float, 128, 64, 32, false>", "prefill_kernelIfLi128ELi64ELi32ELb0E")),
    ("prefill_pk", ("prefill_pk_kernel<__bf16, 128, 64, false>", "prefill_pk_kernelIDF16bLi128ELi64ELb0E")),
    ("gate", ("gate_kernel",)),
    ("conv1d_out", ("conv1d_out_kernel<__bf16, 4, 16>", "conv1d_out_kernelIDF16bLi4ELi16E")),
    ("conv1d_state", ("conv1d_state_kernel<__bf16, 4>", "conv1d_state_kernelIDF16bLi4E")),
    ("copy", ("neg_kernel",)),
)


def _kernel_key(name):
    for key, pats in KERNEL_KEYS:
        if any(p in name for p in pats):
            return key
    return None


def _counter_means(path, counter):
    """Mean counter value (KiB for FETCH_SIZE/WRITE_SIZE) per kernel family."""
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = _kernel_key(r["Kernel_Name"])
        if key is None:
            continue
        vals.setdefault(key, []).append(float(r["Counter_Value"]))
    out = {k: statistics.mean(v) for k, v in vals.items() if k != "copy"}
    if "copy" in vals:
        out["copy"] = max(vals["copy"])
    return out


# Instantiations that only the extra workloads launch: their counter means
# come from a run of every workload; the headline kernels' from a run of the
# headline step alone (extras reuse some headline instantiations on other
# shapes, e.g. the long request's serial walk).
EXTRA_KEYS = ("decode_mtp", "prefill_f32", "prefill_pk")


def summarize_traffic(fetch_csv, write_csv, fetch_all_csv=None, write_all_csv=None):
    """HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE (KiB) counter runs,
    each scaled by what the same counter reads for the run's calibration copy
    of known size."""
    def run(fc, wc):
        f = _counter_means(fc, "FETCH_SIZE")
        w = _counter_means(wc, "WRITE_SIZE")
        # the copy reads and writes 1 GiB each: scale each counter separately
        return f, w, (CALIB_BYTES / 2) / (f["copy"] * 1024.0), (CALIB_BYTES / 2) / (w["copy"] * 1024.0)
    f, w, f_scale, w_scale = run(fetch_csv, write_csv)
    res = {"source_hash": kernel_source_hash(), "calibration_copy_bytes": CALIB_BYTES,
           "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    def put(k, f, w, fs, ws):
        rb = f[k] * 1024.0 * fs
        wb = w[k] * 1024.0 * ws
        res["kernels"][k] = {"fetch_kib_raw": f[k], "write_kib_raw": w[k],
                             "read_bytes": rb, "write_bytes": wb, "bytes": rb + wb}
    for k in ("prefill", "decode", "gate", "conv1d_out", "conv1d_state"):
        if k in f and k in w:
            put(k, f, w, f_scale, w_scale)
    if fetch_all_csv and write_all_csv:
        fa, wa, fa_scale, wa_scale = run(fetch_all_csv, write_all_csv)
        res["all_workload_run"] = {"fetch_scale": fa_scale, "write_scale": wa_scale}
        for k in EXTRA_KEYS:
            if k in fa and k in wa:
                put(k, fa, wa, fa_scale, wa_scale)
    if "conv1d_out" in res["kernels"]:
        # one conv1d call = the output launch + the write-back launch
        parts = [res["kernels"][k] for k in ("conv1d_out", "conv1d_state") if k in res["kernels"]]
        res["kernels"]["conv1d"] = {n: sum(p[n] for p in parts)
                                    for n in ("read_bytes", "write_bytes", "bytes")}
    return res


def summarize_mfma(csv_path, all_csv_path=None):
    """MfmaUtil (% of SIMD cycles the MFMA unit is busy) and MfmaFlopsBF16 of
    the headline prefill kernel (from a run of the headline step), averaged
    over its dispatches; the same for the extra workloads' own prefill
    kernels (under "others", from a run of every workload)."""
    def read(path):
        vals = {}
        for r in csv.DictReader(open(path)):
            key = _kernel_key(r["Kernel_Name"])
            if key is not None:
                vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        return vals
    vals = read(csv_path)
    for k in EXTRA_KEYS:
        vals.pop(k, None)
    if all_csv_path:
        va = read(all_csv_path)
        for k in EXTRA_KEYS:
            if k in va:
                vals[k] = va[k]
    def one(v):
        return {"dispatches": len(v.get("MfmaUtil", [])),
                "mfma_util_pct": statistics.mean(v["MfmaUtil"]) if "MfmaUtil" in v else None,
                "mfma_flops_bf16": statistics.mean(v["MfmaFlopsBF16"]) if "MfmaFlopsBF16" in v else None}
    res = {"source_hash": kernel_source_hash(), "kernel": PREFILL_KERNEL}
    res.update(one(vals["prefill"]))
    res["others"] = {k: one(v) for k, v in vals.items() if k in ("prefill_f32", "prefill_pk")}
    return res


def load_mfma(kernel="prefill"):
    try:
        m = json.load(open(MFMA_FILE))
    except (OSError, ValueError):
        return None
    if m.get("source_hash") != kernel_source_hash():
        return None
    return m if kernel == "prefill" else m.get("others", {}).get(kernel)


def load_traffic(kernel):
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k["bytes"]


def prefill_algorithmic(T, hq, hv, dk, dv, n_seqs, chunk, io_bytes=2):
    """Bytes and flops one prefill launch must move / compute.

    Bytes: q, k, v, out and the fp32 gates once per token, the final states
    once.  Flops: the GEMM work of the chunked WY form, per token -- per q/k
    head the chunk's Gram products K K^T and Q K^T (4 C dk); per value head
    the WY transform W = T diag(beta Gam) K (2 C dk), U~ = T diag(beta) V and
    the intra-chunk (M o Q K^T) U (4 C dv), and the state pass [Q; W] S0 plus
    the state update K^T U (6 dk dv)."""
    per_token_bytes = (hq * dk * io_bytes * 2          # q, k
                       + hv * dv * io_bytes * 2        # v, out
                       + hv * 4 * 2)                   # log-decay, beta (fp32)
    state_bytes = n_seqs * hv * dv * dk * 4            # final state (no initial state)
    bytes_ = T * per_token_bytes + state_bytes
    flops_per_token = hq * 4 * chunk * dk + hv * (2 * chunk * dk + 4 * chunk * dv + 6 * dk * dv)
    return bytes_, T * flops_per_token


def prefill_flops_substitution_form(T, hq, hv, dk, dv, chunk):
    """Flops of the same chunk in the substitution form, which never forms W:
    X = beta (V - Gam K S0) is solved for U by block forward substitution,
    so the 2 C dk per value head of the WY transform of K drop out."""
    return T * (hq * 4 * chunk * dk + hv * (6 * dk * dv + 4 * chunk * dv))


def decode_algorithmic(x):
    """Bytes one decode launch must move: per active (row, head) its state read
    once and written once per required slot, plus the row's activations."""
    import torch
    B, T, n = x["batch"], x["T"], x["n_hh"]
    hq, hv, dk, dv = x["hq"], x["hv"], x["dk"], x["dv"]
    active = int(((x["read_idx"] >= 0) & (x["read_idx"] < x["pool_size"])).sum())
    st = dv * dk * 4
    if x["scatter_idx"] is not None:
        sc = x["scatter_idx"][(x["read_idx"] >= 0)]
        writes = int(((sc >= 0) & (sc < x["pool_size"])).sum()) * hv * st
    else:
        wr = x["write_idx"][(x["read_idx"] >= 0)]
        writes = int(((wr >= 0) & (wr < x["pool_size"])).sum()) * hv * st
    reads = active * hv * st
    e = 2 if x["dtype"] == "bf16" else 4
    act = active * T * (hq * dk + n * hq * dk + n * hv * dv + hv + n * hv + hv * dv) * e
    return reads + writes + act


def conv1d_algorithmic(x):
    """HBM bytes a conv1d call must move: x read and out written once, the
    weights read once, and each sequence's K-1 saved inputs per channel read
    and written back."""
    es = 2 if x["dtype"] == "bf16" else 4
    T, C, K = x["T"], x["conv_dim"], x["K"]
    n = len(x["lengths"])
    return es * (2 * T * C + C * K + 2 * n * C * (K - 1)) + 4 * (2 * n + 1)


def cpu_baseline_prefill(x, budget_units=None):
    """The fp64 oracle on the prefill workload (all of it unless budget_units)."""
    import oracle
    import torch
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    g, _, beta = oracle.gate(x["A_log"], x["dt_bias"], x["a"], x["b"])
    T = x["T"]
    if budget_units is None:
        oracle.prefill(x["q"], x["k"], x["v"], g, beta, n_seqs=x["n_seqs"], seq_len=x["seq_len"],
                       scale=x["scale"], nthreads=threads)
        tokens = T
        sample = "whole workload: gate + prefill of all 4 requests x 32 value heads"
    else:
        raise NotImplementedError
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": dt}


def _time_launches(torch, fn, warmup=3, runs=20, flush=None):
    """Median milliseconds of `fn` over `runs` launches, each after a cache flush."""
    stream = torch.cuda.current_stream()
    ts = []
    for i in range(warmup + runs):
        if flush is not None:
            flush.zero_()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        if i >= warmup:
            ts.append((a, b))
    torch.cuda.synchronize()
    return statistics.median(x.elapsed_time(y) for x, y in ts)


def _progress(what):
    """One progress line per workload on stderr (stdout carries only the JSON line)."""
    print("[bench] %s" % what, file=sys.stderr, flush=True)


def extra_workloads(torch, gdn, synth, dev):
    """The other workloads of the scope table, each timed on its own."""
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    out = {}

    # plain device copy: the achievable streaming bandwidth on this machine
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    cm = _time_launches(torch, lambda: dst.copy_(src), flush=flush)
    _progress("copy_1gib")
    out["copy_1gib"] = {"ms": cm, "gbs": 2 * (1 << 30) / (cm * 1e-3) / 1e9}
    del src, dst

    # the chunked-prefill workload with the gate fused into the prefill and the
    # in-kernel q/k L2 norm (one launch instead of gate + prefill)
    px = synth.chunked_prefill_b4_s4096()
    B, S = px["n_seqs"], px["seq_len"]
    q = px["q"].to(dev).view(B, S, px["hq"], px["dk"])
    k = px["k"].to(dev).view(B, S, px["hq"], px["dk"])
    v = px["v"].to(dev).view(B, S, px["hv"], px["dv"])
    A_log, dt_bias = px["A_log"].to(dev), px["dt_bias"].to(dev)
    a = px["a"].to(dev).view(B, S, -1)
    b = px["b"].to(dev).view(B, S, -1)
    o2 = torch.empty_like(v)
    f2 = torch.empty(B, px["hv"], px["dv"], px["dk"], dtype=torch.float32, device=dev)
    # the same gates computed inside the prefill kernel: one launch for the
    # headline step's gate + prefill (the same arithmetic, g and beta never
    # stored)
    fn = lambda: gdn.prefill(q, k, v, None, None, scale=px["scale"], out=o2, final_state=f2,
                             A_log=A_log, dt_bias=dt_bias, a=a, b=b)
    ms = _time_launches(torch, fn, flush=flush)
    _progress("chunked_prefill_fused_gate")
    out["chunked_prefill_fused_gate"] = {"ms": ms, "tokens_per_s": px["T"] / (ms * 1e-3)}
    fn = lambda: gdn.prefill(q, k, v, None, None, scale=px["scale"], out=o2, final_state=f2,
                             A_log=A_log, dt_bias=dt_bias, a=a, b=b, qk_l2norm=True)
    ms = _time_launches(torch, fn, flush=flush)
    _progress("chunked_prefill_fused_gate_qk_l2norm")
    out["chunked_prefill_fused_gate_qk_l2norm"] = {"ms": ms, "tokens_per_s": px["T"] / (ms * 1e-3)}
    del q, k, v, o2, f2

    # single-head scan: B2 x S64, d16, fp32 (launch latency)
    x = synth.single_head_scan()
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    gam, bet = x["gamma"].to(dev), x["beta"].to(dev)
    o1 = torch.empty_like(v)
    f1 = torch.empty(x["n_seqs"], 1, x["dv"], x["dk"], device=dev)
    B1, S1 = x["n_seqs"], x["seq_len"]
    fn = lambda: gdn.prefill(q.view(B1, S1, 1, -1), k.view(B1, S1, 1, -1), v.view(B1, S1, 1, -1),
                             gam.view(B1, S1, 1), bet.view(B1, S1, 1), decay_kind="gamma",
                             scale=x["scale"], out=o1.view(B1, S1, 1, -1), final_state=f1)
    _progress("single_head_scan_b2_s64_d16_f32")
    out["single_head_scan_b2_s64_d16_f32"] = {"ms": _time_launches(torch, fn, runs=50)}

    # ragged fp32 prefill: 8 requests, initial state, gamma gates
    x = synth.ragged_prefill_8req()
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    gam, bet, cu = x["gamma"].to(dev), x["beta"].to(dev), x["cu_seqlens"].to(dev)
    init = x["initial_state"].to(dev)
    o3 = torch.empty_like(v)
    f3 = torch.empty_like(init)
    fn = lambda: gdn.prefill(q, k, v, gam, bet, decay_kind="gamma", cu_seqlens=cu,
                             initial_state=init, scale=x["scale"], out=o3, final_state=f3)
    ms = _time_launches(torch, fn, flush=flush)
    T = x["T"]
    nb, nf = prefill_algorithmic(T, x["hq"], x["hv"], x["dk"], x["dv"], x["n_seqs"], 64, io_bytes=4)
    nb += x["n_seqs"] * x["hv"] * x["dv"] * x["dk"] * 4  # the initial state is read too
    mf = load_mfma("prefill_f32")
    _progress("ragged_prefill_8req_hv32_d128_f32")
    out["ragged_prefill_8req_hv32_d128_f32"] = {
        "ms": ms, "tokens": T, "tokens_per_s": T / (ms * 1e-3),
        "algorithmic_bytes": nb, "algorithmic_flops": nf,
        "gbs": nb / (ms * 1e-3) / 1e9, "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "fp32_matrix_tflops": nf / (ms * 1e-3) / 1e12,
        "fp32_matrix_frac": nf / (ms * 1e-3) / 1e12 / FP32_MATRIX_PEAK_TFLOPS,
        "traffic": load_traffic("prefill_f32"),
        "mfma_util_counter_pct": None if mf is None else mf["mfma_util_pct"]}
    del q, k, v, o3, f3, init

    # multi-token decode: pool [512, 16, 64, 128], B64, T4, n2, scatter
    x = synth.mtp_decode_b64_t4()
    t = {n: x[n].to(dev) for n in ("q", "k", "v", "A_log", "dt_bias", "a", "b", "pool",
                                   "read_idx", "scatter_idx")}
    o5 = torch.zeros(x["batch"], x["T"], x["hv"], x["dv"], dtype=torch.bfloat16, device=dev)
    fn = lambda: gdn.decode(t["q"], t["k"], t["v"], t["A_log"], t["dt_bias"], t["a"], t["b"],
                            t["pool"], t["read_idx"], scatter_idx=t["scatter_idx"],
                            scale=x["scale"], out=o5, use_qk_l2norm=False)
    ms = _time_launches(torch, fn, flush=flush)
    by = decode_algorithmic(x)
    _progress("mtp_decode_b64_t4_n2_h16_dv64_bf16")
    out["mtp_decode_b64_t4_n2_h16_dv64_bf16"] = {
        "ms": ms, "algorithmic_bytes": by, "gbs": by / (ms * 1e-3) / 1e9,
        "hbm_frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": load_traffic("decode_mtp")}
    del t, o5

    # multi-token decode batches (B64, n1) with 16 and 64 tokens per row: the
    # decode entry point runs them in the chunked form over the pool
    for T16 in (16, 64):
        x = synth.decode_inputs(9, pool_size=256, batch=64, T=T16, n_hh=1, hq=16, hv=32, dk=128,
                                dv=128, dtype="bf16", write_slots=True)
        t = {n: x[n].to(dev) for n in ("q", "k", "v", "A_log", "dt_bias", "a", "b", "pool",
                                       "read_idx", "write_idx")}
        o6 = torch.zeros(x["batch"], T16, x["hv"], x["dv"], dtype=torch.bfloat16, device=dev)
        fn = lambda: gdn.decode(t["q"], t["k"], t["v"], t["A_log"], t["dt_bias"], t["a"], t["b"],
                                t["pool"], t["read_idx"], write_idx=t["write_idx"],
                                scale=x["scale"], out=o6, use_qk_l2norm=False)
        ms = _time_launches(torch, fn, flush=flush)
        by = decode_algorithmic(x)
        out["mtp_decode_b64_t%d_h32_d128_bf16" % T16] = {
            "ms": ms, "tokens_per_s": x["batch"] * T16 / (ms * 1e-3), "algorithmic_bytes": by,
            "gbs": by / (ms * 1e-3) / 1e9, "hbm_frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del t, o6

    # the chunked-prefill shape with a per-key decay ([T, hv, dk] log-decay,
    # the separate 16-token-chunk kernel)
    px = synth.chunked_prefill_b4_s4096()
    g = torch.Generator().manual_seed(12)
    q, k, v = (px[n].to(dev) for n in ("q", "k", "v"))
    T, hv, dk = px["T"], px["hv"], px["dk"]
    dec = (-torch.rand(T, hv, dk, generator=g) * 0.5).to(dev)
    bet = torch.rand(T, hv, generator=g).to(dev)
    cu = torch.arange(px["n_seqs"] + 1, dtype=torch.int32, device=dev) * px["seq_len"]
    o8 = torch.empty_like(v)
    f8 = torch.empty(px["n_seqs"], hv, px["dv"], dk, device=dev)
    fn = lambda: gdn.prefill(q, k, v, dec, bet, cu_seqlens=cu, scale=px["scale"], out=o8,
                             final_state=f8, decay_per_key=True)
    ms = _time_launches(torch, fn, flush=flush, runs=5)
    nb, _ = prefill_algorithmic(T, px["hq"], hv, dk, px["dv"], px["n_seqs"], 16)
    nb += T * hv * dk * 4 - T * hv * 4  # the decay is per key
    mf = load_mfma("prefill_pk")
    _progress("chunked_prefill_per_key_decay_b4_s4096_bf16")
    out["chunked_prefill_per_key_decay_b4_s4096_bf16"] = {
        "ms": ms, "tokens_per_s": T / (ms * 1e-3), "algorithmic_bytes": nb,
        "gbs": nb / (ms * 1e-3) / 1e9, "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "traffic": load_traffic("prefill_pk"),
        "mfma_util_counter_pct": None if mf is None else mf["mfma_util_pct"]}
    del q, k, v, dec, bet, o8, f8

    # one long request with few heads (1 x 65536 tokens, Hq 2, Hv 4, d 128):
    # the scan over segment maps (local pass, combine, rerun, with a
    # preallocated workspace) against the serial walk of the same call
    x = synth.long_request_b1_s65536_hv4()
    q, k, v, cu = (x[n].to(dev) for n in ("q", "k", "v", "cu_seqlens"))
    g9, _, b9 = gdn.gate(x["A_log"].to(dev), x["dt_bias"].to(dev), x["a"].to(dev), x["b"].to(dev))
    o9 = torch.empty_like(v)
    f9 = torch.empty(1, x["hv"], x["dv"], x["dk"], device=dev)
    need = gdn.prefill_workspace_size(q, k, v, g9, b9, cu_seqlens=cu)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    fn_scan = lambda: gdn.prefill(q, k, v, g9, b9, cu_seqlens=cu, scale=x["scale"], out=o9,
                                  final_state=f9, workspace=ws)
    fn_serial = lambda: gdn.prefill(q, k, v, g9, b9, cu_seqlens=cu, scale=x["scale"], out=o9,
                                    final_state=f9, scan=False)
    ms_scan = _time_launches(torch, fn_scan, flush=flush)
    ms_serial = _time_launches(torch, fn_serial, flush=flush, runs=5)
    T = x["T"]
    _progress("long_request_b1_s65536_hq2_hv4_d128_bf16")
    out["long_request_b1_s65536_hq2_hv4_d128_bf16"] = {
        "ms_scan": ms_scan, "ms_serial": ms_serial, "speedup": ms_serial / ms_scan,
        "segments": need // (x["hv"] * x["dk"] * (2 * x["dv"] + x["dk"]) * 4),
        "workspace_bytes": need, "tokens_per_s_scan": T / (ms_scan * 1e-3),
        "tokens_per_s_serial": T / (ms_serial * 1e-3)}
    del q, k, v, g9, b9, o9, f9, ws

    # causal conv1d over the QKV rows with the conv-state pool: the prefill
    # batch (B4 x S4096, 8192 channels) and one decode step (256 x 1 row)
    for name, make in (("conv1d_prefill_b4_s4096_c8192_k4_bf16", synth.conv1d_prefill_b4_s4096),
                       ("conv1d_decode_b256_c8192_k4_bf16", synth.conv1d_decode_b256)):
        x = make()
        xd, wd, pool = x["x"].to(dev), x["weight"].to(dev), x["conv_state"].to(dev)
        sl = x["slot_idx"].to(torch.int32).to(dev)
        off = x["row_offsets"].to(torch.int32).to(dev)
        oc = torch.empty_like(xd)
        fn = lambda: gdn.conv1d(xd, wd, pool, sl, off, out=oc)
        ms = _time_launches(torch, fn, flush=flush)
        by = conv1d_algorithmic(x)
        _progress(name)
        out[name] = {"ms": ms, "tokens": x["T"], "algorithmic_bytes": by,
                     "gbs": by / (ms * 1e-3) / 1e9, "hbm_frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del xd, wd, pool, oc
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "conv1d"], nargs="+", default=None,
                    help="parts of the step to run (default: prefill and decode); conv1d adds "
                         "the causal conv1d over the prefill batch's QKV rows")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--summarize-traffic", nargs="+", metavar="CSV",
                    help="FETCH.csv WRITE.csv of the headline run [FETCH.csv WRITE.csv of an all-workload run]")
    ap.add_argument("--summarize-mfma", nargs="+", metavar="CSV",
                    help="MFMA.csv of the headline run [MFMA.csv of an all-workload run]")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the single-head, ragged-fp32 and multi-token-decode timings")
    args = ap.parse_args()
    if args.summarize_traffic:
        if len(args.summarize_traffic) not in (2, 4):
            ap.error("--summarize-traffic takes 2 or 4 CSV files")
        print(json.dumps(summarize_traffic(*args.summarize_traffic), indent=1))
        return
    if args.summarize_mfma:
        if len(args.summarize_mfma) not in (1, 2):
            ap.error("--summarize-mfma takes 1 or 2 CSV files")
        print(json.dumps(summarize_mfma(*args.summarize_mfma), indent=1))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_state_delta_amd as gdn
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)

    parts = set(args.only or ("prefill", "decode"))
    do_prefill, do_decode, do_conv = ("prefill" in parts), ("decode" in parts), ("conv1d" in parts)

    # ---------------------------------------------------------------- inputs
    px = synth.chunked_prefill_b4_s4096()
    B, S = px["n_seqs"], px["seq_len"]
    q = px["q"].to(dev).view(B, S, px["hq"], px["dk"])
    k = px["k"].to(dev).view(B, S, px["hq"], px["dk"])
    v = px["v"].to(dev).view(B, S, px["hv"], px["dv"])
    A_log, dt_bias = px["A_log"].to(dev), px["dt_bias"].to(dev)
    a, b = px["a"].to(dev), px["b"].to(dev)
    out = torch.empty_like(v)
    fin = torch.empty(B, px["hv"], px["dv"], px["dk"], dtype=torch.float32, device=dev)
    g_buf = torch.empty(px["T"], px["hv"], dtype=torch.float32, device=dev)
    b_buf = torch.empty_like(g_buf)

    dx = synth.decode_pool_b256()
    pool = dx["pool"].to(dev)
    dq, dk_, dv_ = dx["q"].to(dev), dx["k"].to(dev), dx["v"].to(dev)
    dA, ddt, da, db = dx["A_log"].to(dev), dx["dt_bias"].to(dev), dx["a"].to(dev), dx["b"].to(dev)
    rd, wr = dx["read_idx"].to(dev), dx["write_idx"].to(dev)
    dout = torch.zeros(dx["batch"], 1, dx["hv"], dx["dv"], dtype=torch.bfloat16, device=dev)

    if do_conv:
        cx = synth.conv1d_prefill_b4_s4096()
        c_x, c_w, c_pool = cx["x"].to(dev), cx["weight"].to(dev), cx["conv_state"].to(dev)
        c_sl = cx["slot_idx"].to(torch.int32).to(dev)
        c_off = cx["row_offsets"].to(torch.int32).to(dev)
        c_out = torch.empty_like(c_x)

    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    stream = torch.cuda.current_stream()

    def run_gate():
        gdn.gate(A_log, dt_bias, a, b, log_decay_out=g_buf, beta_out=b_buf)

    def run_prefill():
        gdn.prefill(q, k, v, g_buf.view(B, S, -1), b_buf.view(B, S, -1), scale=px["scale"],
                    out=out, final_state=fin)

    def run_decode():
        gdn.decode(dq, dk_, dv_, dA, ddt, da, db, pool, rd, write_idx=wr, scale=dx["scale"],
                   out=dout, use_qk_l2norm=False)

    def run_conv():
        gdn.conv1d(c_x, c_w, c_pool, c_sl, c_off, out=c_out)

    E = lambda: torch.cuda.Event(enable_timing=True)
    n_ev = args.warmup + args.steps
    ev = [[E() for _ in range(7)] for _ in range(n_ev)]

    def step(i):
        e = ev[i]
        if do_prefill:
            flush.zero_()
            e[0].record(stream)
            run_gate()
            e[1].record(stream)
            run_prefill()
            e[2].record(stream)
        if do_decode:
            flush.zero_()
            e[3].record(stream)
            run_decode()
            e[4].record(stream)
        if do_conv:
            flush.zero_()
            e[5].record(stream)
            run_conv()
            e[6].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, n_ev):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    if args.copy_calib:
        # a plain streaming pass over known bytes: reads 1 GiB, writes 1 GiB
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()

    timed = ev[args.warmup:]
    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "chunked_prefill_b4_s4096_hq16_hv32_d128_bf16 + "
                                  "decode_pool1024_b256_t1_hq16_hv32_d128_bf16",
                      "prefill_tokens": px["T"], "chunk": 64, "decode_rows": dx["batch"],
                      "decode_active_rows": int((dx["read_idx"] >= 0).sum()),
                      "device": props.name, "cus": props.multi_processor_count}}

    if do_prefill:
        gate_ms = [e[0].elapsed_time(e[1]) for e in timed]
        pre_ms = [e[1].elapsed_time(e[2]) for e in timed]
        tot = statistics.median(g_ + p_ for g_, p_ in zip(gate_ms, pre_ms))
        pb, pf = prefill_algorithmic(px["T"], px["hq"], px["hv"], px["dk"], px["dv"], B, 64)
        pm = statistics.median(pre_ms)
        res["value"] = px["T"] / (tot * 1e-3)
        res["unit"] = "tokens/s"
        gbs = pb / (pm * 1e-3) / 1e9
        tfl = pf / (pm * 1e-3) / 1e12
        pf_sub = prefill_flops_substitution_form(px["T"], px["hq"], px["hv"], px["dk"], px["dv"], 64)
        res["roofline"] = {"kernel": PREFILL_KERNEL, "bound": "hbm",
                           "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": gbs / HBM_PEAK_GBS, "traffic": load_traffic("prefill"),
                           "algorithmic_bytes": pb, "algorithmic_flops": pf,
                           "mfma_tflops": tfl, "mfma_peak_tflops": BF16_PEAK_TFLOPS,
                           "mfma_frac": tfl / BF16_PEAK_TFLOPS,
                           "algorithmic_flops_substitution_form": pf_sub,
                           "mfma_frac_substitution_form": pf_sub / (pm * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                           "avg_ms": pm}
        mf = load_mfma()
        # counter view of the same kernel (rocprofv3 MfmaUtil / MfmaFlopsBF16), or
        # null once the kernels have changed since it was taken
        res["roofline"]["mfma_util_counter_pct"] = None if mf is None else mf["mfma_util_pct"]
        res["roofline"]["mfma_flops_executed"] = None if mf is None else mf["mfma_flops_bf16"]
        res["prefill"] = {"gate_ms": statistics.median(gate_ms), "prefill_ms": pm,
                          "prefill_ms_min": min(pre_ms), "tokens_per_s": res["value"]}
    if do_decode:
        dec_ms = [e[3].elapsed_time(e[4]) for e in timed]
        dm = statistics.median(dec_ms)
        db_ = decode_algorithmic(dx)
        gbs = db_ / (dm * 1e-3) / 1e9
        res["decode"] = {"kernel": "decode_kernel<bf16,128,128,32>", "bound": "hbm",
                         "ms": dm, "ms_min": min(dec_ms), "algorithmic_bytes": db_,
                         "traffic": load_traffic("decode"),
                         "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS}
        if not do_prefill:
            res["value"] = gbs
            res["unit"] = "GB/s"
            res["roofline"] = dict(res["decode"])
    if do_conv:
        c_ms = [e[5].elapsed_time(e[6]) for e in timed]
        cm = statistics.median(c_ms)
        cb = conv1d_algorithmic(cx)
        gbs = cb / (cm * 1e-3) / 1e9
        res["conv1d"] = {"kernel": "conv1d_out_kernel<bf16,4,16> + conv1d_state_kernel<bf16,4>",
                         "workload": "conv1d_prefill_b4_s4096_c8192_k4_bf16", "bound": "hbm",
                         "ms": cm, "ms_min": min(c_ms), "algorithmic_bytes": cb,
                         "traffic": load_traffic("conv1d"), "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}
        if not (do_prefill or do_decode):
            res["value"] = gbs
            res["unit"] = "GB/s"
            res["roofline"] = dict(res["conv1d"])

    if not args.no_extra and args.only is None:
        del pool, flush
        torch.cuda.empty_cache()
        res["extra"] = extra_workloads(torch, gdn, synth, dev)
        # rates against the measured plain-copy bandwidth of this machine
        copy_gbs = res["extra"]["copy_1gib"]["gbs"]
        for part in ("roofline", "decode", "conv1d"):
            if part in res and res[part].get("unit") == "GB/s":
                res[part]["frac_of_measured_copy"] = res[part]["achieved"] / copy_gbs

    if not args.no_cpu_baseline and do_prefill:
        res["cpu_baseline"] = cpu_baseline_prefill(px)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
