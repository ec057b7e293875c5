"""The benchmark's roofline accounting, on the CPU: the algorithmic bytes and
flops of the headline prefill and decode workloads, written out term by term
from the tensors each launch must touch, and the HBM-traffic summary of
rocprofv3 counter files (calibration by a copy of known size, attribution by
kernel instantiation) on small synthetic counter files."""
import csv

import pytest

import bench


def test_prefill_algorithmic_bytes_and_flops():
    T, hq, hv, dk, dv, n, C = 16384, 16, 32, 128, 128, 4, 64
    by, fl = bench.prefill_algorithmic(T, hq, hv, dk, dv, n, C)
    q_k = 2 * T * hq * dk * 2              # bf16 q and k, read once
    v_out = 2 * T * hv * dv * 2            # bf16 v read, out written
    gates = 2 * T * hv * 4                 # fp32 log-decay and beta
    final = n * hv * dv * dk * 4           # fp32 final states, written once
    assert by == q_k + v_out + gates + final == 415236096
    # Gram tiles K K^T and Q K^T (2 C dk flops each per token and q/k head),
    # and per value head: W = T diag(beta Gam) K (2 C dk), U~ = T diag(beta) V
    # and (M o Q K^T) U (2 C dv each), [Q; W] S0 (4 dk dv) and the state
    # update K^T U (2 dk dv): 5 242 880 flops per token, 85.9 GFLOP in all
    gram = T * hq * 4 * C * dk
    wy = T * hv * 2 * C * dk
    state = T * hv * (6 * dk * dv + 4 * C * dv)
    assert fl == gram + wy + state == 85899345920
    assert fl // T == 5242880
    # the substitution form (no explicit W) drops the WY term of K
    assert bench.prefill_flops_substitution_form(T, hq, hv, dk, dv, C) == gram + state == 77309411328


def test_decode_algorithmic_bytes():
    import synth
    x = synth.decode_pool_b256()
    active = int(((x["read_idx"] >= 0) & (x["read_idx"] < x["pool_size"])).sum())
    assert 0 < active < x["batch"]
    by = bench.decode_algorithmic(x)
    st = x["dv"] * x["dk"] * 4
    # every active (row, head) state read once and written once, plus the
    # row's activations; skipped rows move nothing of the pool
    assert by >= active * x["hv"] * 2 * st
    assert by < active * x["hv"] * 2 * st * 1.02


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, val in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val})


def test_traffic_summary_calibration_and_attribution(tmp_path):
    kib = bench.CALIB_BYTES / 2 / 1024.0          # the copy's read (and written) KiB
    fetch = [("void at::native::neg_kernel(...)", kib / 2),   # FETCH_SIZE reads half
             ("void gdn::prefill_pair_kernel<128, false, false, false, false>(gdn::PrefillParams)", 1000.0),
             ("void gdn::prefill_pair_kernel<128, false, false, false, false>(gdn::PrefillParams)", 1200.0),
             ("_ZN3gdn13decode_kernelIDF16bLi128ELi128ELi32EEEvNS_12DecodeParamsE", 500.0),
             ("void gdn::decode_kernel<__bf16, 128, 64, 32>(gdn::DecodeParams)", 700.0),
             ("void gdn::prefill_pair_kernel<128, true, true, false, false>(gdn::PrefillParams)", 9999.0),
             ("void gdn::prefill_pair_kernel<128, false, false, true, false>(gdn::PrefillParams)", 8888.0)]
    write = [("void at::native::neg_kernel(...)", kib),
             ("void gdn::prefill_pair_kernel<128, false, false, false, false>(gdn::PrefillParams)", 300.0),
             ("_ZN3gdn13decode_kernelIDF16bLi128ELi128ELi32EEEvNS_12DecodeParamsE", 400.0),
             ("void gdn::decode_kernel<__bf16, 128, 64, 32>(gdn::DecodeParams)", 800.0)]
    fp, wp = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_counters(fp, "FETCH_SIZE", fetch)
    _write_counters(wp, "WRITE_SIZE", write)
    t = bench.summarize_traffic(str(fp), str(wp))
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    pre = t["kernels"]["prefill"]
    # the mean over the headline instantiation's dispatches only (the fused,
    # normed instantiation is another workload)
    assert pre["fetch_kib_raw"] == pytest.approx(1100.0)
    assert pre["read_bytes"] == pytest.approx(1100.0 * 1024 * 2)
    assert pre["write_bytes"] == pytest.approx(300.0 * 1024)
    dec = t["kernels"]["decode"]
    assert dec["bytes"] == pytest.approx(500.0 * 1024 * 2 + 400.0 * 1024)
    # an extra workload's own kernel is taken from the all-workload run only,
    # scaled by that run's own calibration copy
    assert "decode_mtp" not in t["kernels"]
    fa, wa = tmp_path / "fetch_all.csv", tmp_path / "write_all.csv"
    _write_counters(fa, "FETCH_SIZE", [("void at::native::neg_kernel(...)", kib / 4),
                                       ("void gdn::decode_kernel<__bf16, 128, 64, 32>(gdn::DecodeParams)", 350.0)])
    _write_counters(wa, "WRITE_SIZE", [("void at::native::neg_kernel(...)", kib),
                                       ("void gdn::decode_kernel<__bf16, 128, 64, 32>(gdn::DecodeParams)", 800.0)])
    t = bench.summarize_traffic(str(fp), str(wp), str(fa), str(wa))
    assert t["kernels"]["prefill"]["fetch_kib_raw"] == pytest.approx(1100.0)
    assert t["all_workload_run"]["fetch_scale"] == pytest.approx(4.0)
    assert t["kernels"]["decode_mtp"]["bytes"] == pytest.approx(350.0 * 1024 * 4 + 800.0 * 1024)
