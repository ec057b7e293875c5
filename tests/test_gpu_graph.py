"""Every libgdn call can be captured in a HIP graph: no call reads device data
on the host, synchronises or allocates.  The calls (gate; prefill with the
pair-role and general kernels and an update_rule that reads the per-device
gate constant; decode with the token loop and the chunked form; conv1d; the
per-key prefill and the chunked per-key decode) are captured once into a
torch CUDA graph and replayed three times, with eager work in between; every
replay must reproduce the eager results bit for bit.
States updated in place (pools) are reset eagerly before each replay.
"""
import pytest
import torch

import gated_deltanet_state_delta_amd as gdn
import synth
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _inputs():
    dev = "cuda"
    px = synth.prefill_inputs(800, lengths=[70, 0, 130], hq=2, hv=4, dk=128, dv=128, dtype="bf16",
                              gate="qwen")
    pf = synth.prefill_inputs(801, lengths=[50, 33], hq=1, hv=2, dk=64, dv=32, dtype="f32",
                              gate="qwen", init_std=0.05)
    d1 = synth.decode_inputs(802, pool_size=24, batch=6, T=1, n_hh=1, hq=2, hv=4, dk=128, dv=64,
                             dtype="bf16", skip_rows=1, write_slots=True)
    d16 = synth.decode_inputs(803, pool_size=24, batch=6, T=16, n_hh=1, hq=2, hv=4, dk=64, dv=64,
                              dtype="bf16", skip_rows=1, write_slots=True)
    cx = synth.conv1d_inputs(804, lengths=[40, 1, 77], conv_dim=256, kernel_size=4, max_slots=8,
                             dtype="bf16")
    pk = synth.prefill_inputs(805, lengths=[45, 0, 20], hq=1, hv=2, dk=64, dv=64, dtype="bf16", gate="log",
                              init_std=0.05)
    dpk = synth.decode_inputs(806, pool_size=24, batch=6, T=16, n_hh=1, hq=2, hv=4, dk=64, dv=64,
                              dtype="bf16", skip_rows=1, write_slots=True)
    g = torch.Generator().manual_seed(807)
    t = {}
    for name, x in (("p", px), ("f", pf)):
        for k in ("q", "k", "v", "A_log", "dt_bias", "a", "b", "cu_seqlens", "initial_state"):
            if x.get(k) is not None:
                t[name + k] = x[k].to(dev)
    for name, x in (("d1", d1), ("d16", d16)):
        for k in ("q", "k", "v", "A_log", "dt_bias", "a", "b", "read_idx", "write_idx", "pool"):
            t[name + k] = x[k].to(dev)
        t[name + "scale"] = x["scale"]
    for k in ("x", "weight", "conv_state"):
        t["c" + k] = cx[k].to(dev)
    for k in ("q", "k", "v", "beta", "cu_seqlens", "initial_state"):
        t["k" + k] = pk[k].to(dev)
    t["kdec"] = (-torch.rand(pk["T"], 2, 64, generator=g) * 0.5).to(dev)
    t["kscale"] = pk["scale"]
    for k in ("q", "k", "v", "b", "read_idx", "write_idx", "pool"):
        t["e" + k] = dpk[k].to(dev)
    t["edec"] = (-torch.rand(6, 16, 4, 64, generator=g) * 0.5).to(dev)
    t["escale"] = dpk["scale"]
    t["cslot"] = cx["slot_idx"].to(torch.int32).to(dev)
    t["coff"] = cx["row_offsets"].to(torch.int32).to(dev)
    T, hv = px["T"], px["hv"]
    out = dict(
        g=torch.empty(T, hv, device=dev), beta=torch.empty(T, hv, device=dev),
        po=torch.empty(T, hv, 128, dtype=torch.bfloat16, device=dev),
        pfin=torch.empty(3, hv, 128, 128, device=dev),
        fo=torch.empty(pf["T"], 2, 32, device=dev), ffin=torch.empty(2, 2, 32, 64, device=dev),
        d1o=torch.zeros(6, 1, 4, 64, dtype=torch.bfloat16, device=dev),
        d16o=torch.zeros(6, 16, 4, 64, dtype=torch.bfloat16, device=dev),
        co=torch.zeros(cx["T"], 256, dtype=torch.bfloat16, device=dev),
        ko=torch.empty(pk["T"], 2, 64, dtype=torch.bfloat16, device=dev),
        kfin=torch.empty(3, 2, 64, 64, device=dev),
        eo=torch.zeros(6, 16, 4, 64, dtype=torch.bfloat16, device=dev))
    return t, out, px["scale"], pf["scale"]


def _calls(t, o, ps, fs):
    gdn.gate(t["pA_log"], t["pdt_bias"], t["pa"], t["pb"], log_decay_out=o["g"], beta_out=o["beta"])
    gdn.prefill(t["pq"], t["pk"], t["pv"], o["g"], o["beta"], cu_seqlens=t["pcu_seqlens"], scale=ps,
                out=o["po"], final_state=o["pfin"])
    # general kernel, gated rule: no beta input (reads the gate constant)
    gdn.prefill(t["fq"], t["fk"], t["fv"], None, None, A_log=t["fA_log"], dt_bias=t["fdt_bias"],
                a=t["fa"], cu_seqlens=t["fcu_seqlens"], initial_state=t["finitial_state"],
                scale=fs, out=o["fo"], final_state=o["ffin"], update_rule="gated")
    for n in ("d1", "d16"):
        gdn.decode(t[n + "q"], t[n + "k"], t[n + "v"], t[n + "A_log"], t[n + "dt_bias"], t[n + "a"],
                   t[n + "b"], t[n + "pool"], t[n + "read_idx"], write_idx=t[n + "write_idx"],
                   scale=t[n + "scale"], out=o[n + "o"], use_qk_l2norm=False)
    gdn.conv1d(t["cx"], t["cweight"], t["cconv_state"], t["cslot"], t["coff"], out=o["co"])
    # per-key decay: prefill, and the chunked multi-token decode over a pool
    gdn.prefill(t["kq"], t["kk"], t["kv"], t["kdec"], t["kbeta"], cu_seqlens=t["kcu_seqlens"],
                initial_state=t["kinitial_state"], scale=t["kscale"], out=o["ko"], final_state=o["kfin"],
                decay_per_key=True)
    gdn.decode(t["eq"], t["ek"], t["ev"], None, None, None, t["eb"], t["epool"], t["eread_idx"],
               write_idx=t["ewrite_idx"], scale=t["escale"], out=o["eo"], decay_per_key=t["edec"], use_qk_l2norm=False)


STATEFUL = ("d1pool", "d16pool", "cconv_state", "epool")


def test_all_calls_replay_from_a_graph():
    t, o, ps, fs = _inputs()
    saved = {k: t[k].clone() for k in STATEFUL}
    # eager reference (this also takes the gate-constant address once)
    _calls(t, o, ps, fs)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in o.items()}
    ref.update({k: t[k].clone() for k in STATEFUL})
    for k in STATEFUL:
        t[k].copy_(saved[k])
    for v in o.values():
        v.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _calls(t, o, ps, fs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for k in STATEFUL:
            t[k].copy_(saved[k])
        for v in o.values():
            v.zero_()
        junk.mul_(1.0001).add_(0.5)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in o.items():
            assert torch.equal(v, ref[k]), "replay %d: %s differs from the eager run" % (rep, k)
        for k in STATEFUL:
            assert torch.equal(t[k], ref[k]), "replay %d: %s differs from the eager run" % (rep, k)
