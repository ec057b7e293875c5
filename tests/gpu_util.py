"""Shared helpers for the GPU tests: device checks, comparison, oracle runners."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}  # max |gpu - oracle| / max |oracle|


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_state_delta_amd._lib as L
    L.load()


def rel_err(gpu, ref) -> float:
    """max |gpu - ref| / max |ref|; with max |ref| == 0 it is max |gpu| (must be 0)."""
    g = gpu.detach().to("cpu", torch.float64).numpy() if hasattr(gpu, "detach") else np.asarray(gpu)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU values"
    m = np.abs(ref).max() if ref.size else 0.0
    d = np.abs(g - ref).max() if ref.size else 0.0
    return float(d / m) if m > 0 else float(d)


def assert_close(gpu, ref, dtype, what=""):
    e = rel_err(gpu, ref)
    assert e <= TOL[dtype], "%s: normalised max error %.3e > %.1e" % (what, e, TOL[dtype])
    return e


def to_dev(x, dev="cuda"):
    return None if x is None else x.to(dev)


def oracle_prefill_from(x, gate_out=None):
    """Oracle prefill for a synth.prefill_inputs dict (gates in fp64 for qwen)."""
    if x["gate"] == "qwen":
        g, _, beta = oracle.gate(x["A_log"], x["dt_bias"], x["a"], x["b"])
        dec, is_gamma = g, False
    elif x["gate"] == "gamma":
        dec, beta, is_gamma = x["gamma"], x["beta"], True
    else:
        dec, beta, is_gamma = x["log_decay"], x["beta"], False
    kw = dict(decay_is_gamma=is_gamma, initial_state=x["initial_state"], scale=x["scale"])
    if x["cu_seqlens"] is not None:
        kw["cu_seqlens"] = x["cu_seqlens"]
    else:
        kw["n_seqs"], kw["seq_len"] = x["n_seqs"], x["seq_len"]
    return oracle.prefill(x["q"], x["k"], x["v"], dec, beta, **kw)


def gpu_prefill_from(x, chunk_size=0, dev="cuda", out=None, final_state=None, initial_state=None):
    """GPU prefill for a synth.prefill_inputs dict (qwen gates through gdn_gate)."""
    import gated_deltanet_state_delta_amd as gdn
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    if x["gate"] == "qwen":
        dec, _, beta = gdn.gate(to_dev(x["A_log"]), to_dev(x["dt_bias"]), to_dev(x["a"]),
                                to_dev(x["b"]))
        kind = "log"
    elif x["gate"] == "gamma":
        dec, beta, kind = to_dev(x["gamma"]), to_dev(x["beta"]), "gamma"
    else:
        dec, beta, kind = to_dev(x["log_decay"]), to_dev(x["beta"]), "log"
    init = to_dev(x["initial_state"]) if initial_state is None else initial_state
    cu = to_dev(x["cu_seqlens"])
    if cu is None and x["n_seqs"] > 1:
        B, S = x["n_seqs"], x["seq_len"]
        o, f = gdn.prefill(q.view(B, S, *q.shape[1:]), k.view(B, S, *k.shape[1:]),
                           v.view(B, S, *v.shape[1:]), dec, beta, decay_kind=kind,
                           initial_state=init, scale=x["scale"], chunk_size=chunk_size,
                           out=out, final_state=final_state)
        return o.view(B * S, *o.shape[2:]), f
    return gdn.prefill(q, k, v, dec, beta, decay_kind=kind, cu_seqlens=cu, initial_state=init,
                       scale=x["scale"], chunk_size=chunk_size, out=out, final_state=final_state)
