"""Seeded synthetic inputs for the gated delta rule workloads.

This module is shared by the tests, the benchmark and the smoke check, and by
both sides of every parity comparison (the HIP path and the fp64 oracle).  It
holds none of the method's arithmetic: it only draws random tensors with a
seeded CPU ``torch.Generator`` and shapes them.  Keys are L2-normalised in
fp32 before the cast to the input dtype, as the "Gated DeltaNet State Update"
constraints require (keys unit-normalised before conversion, not renormalised
afterwards); fp32 -> bf16 casts round to nearest even (torch's default).

Draw order inside one generator: lengths (ragged workloads only), then q, k,
v, then gate inputs, then initial state / pool, then slot indices.
"""
from __future__ import annotations

import math

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    """Normalise the last dimension to unit L2 norm (fp32), as an input recipe."""
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def _randn(g, shape, std=1.0):
    return torch.randn(*shape, generator=g, dtype=torch.float32) * std


def _uniform(g, shape, lo, hi):
    return torch.rand(*shape, generator=g, dtype=torch.float32) * (hi - lo) + lo


def prefill_inputs(seed: int, *, lengths=None, n_seqs=None, seq_len=None, hq=1, hv=1,
                   dk=16, dv=16, dtype="f32", gate="gamma", gamma_range=(0.9, 1.0),
                   init_std=None, scale=None):
    """Inputs for one prefill call (all CPU tensors).

    Either ``lengths`` (a list of per-request token counts, packed back to back
    via cu_seqlens) or ``n_seqs`` x ``seq_len`` (uniform packing, no
    cu_seqlens) selects the request layout.  ``gate`` selects the decay input:
      * "gamma": gamma ~ U[gamma_range], beta ~ U[0, 1]  (decay passed as gamma)
      * "log":   log of such a gamma (decay passed in log space)
      * "qwen":  raw A_log ~ U[0, ln 16], dt_bias ~ N(0, 0.5) [hv] and
                 a, b ~ N(0, 1) [T, hv] in the io dtype (gates computed by the
                 fused gate call)
    """
    g = _gen(seed)
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        T = sum(lengths)
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
        n = len(lengths)
    else:
        T = n_seqs * seq_len
        cu = None
        n = n_seqs
    dt = DTYPES[dtype]
    q = _randn(g, (T, hq, dk)).to(dt)
    k = _unit_rows(_randn(g, (T, hq, dk))).to(dt)
    v = _randn(g, (T, hv, dv)).to(dt)
    out = dict(q=q, k=k, v=v, cu_seqlens=cu, n_seqs=n, seq_len=seq_len, T=T,
               hq=hq, hv=hv, dk=dk, dv=dv, dtype=dtype, gate=gate,
               scale=(1.0 / math.sqrt(dk)) if scale is None else float(scale))
    if gate in ("gamma", "log"):
        gam = _uniform(g, (T, hv), gamma_range[0], gamma_range[1])
        beta = _uniform(g, (T, hv), 0.0, 1.0)
        out["beta"] = beta
        if gate == "gamma":
            out["gamma"] = gam
        else:
            out["log_decay"] = torch.log(gam)
    elif gate == "qwen":
        out["A_log"] = _uniform(g, (hv,), 0.0, math.log(16.0))
        out["dt_bias"] = _randn(g, (hv,), 0.5)
        out["a"] = _randn(g, (T, hv)).to(dt)
        out["b"] = _randn(g, (T, hv)).to(dt)
    else:
        raise ValueError(gate)
    out["initial_state"] = None if init_std is None else _randn(g, (n, hv, dv, dk), init_std)
    return out


def decode_inputs(seed: int, *, pool_size, batch, T=1, n_hh=1, hq, hv, dk, dv,
                  dtype="bf16", skip_rows=0, write_slots=True, scatter=False,
                  pool_std=0.05, scale=None, materialize_pool=True):
    """Inputs for one decode call (all CPU tensors).

    Slots come from one randperm of the pool: read = perm[:B]; then either
    write = perm[B:2B] (write_slots=True), or scatter = perm[B:B+B*T] as [B, T]
    (scatter=True).  ``skip_rows`` seeded rows get read = -1 with their write
    slot left valid.  With materialize_pool=False the pool is not drawn and
    the returned "pool" is None.
    """
    g = _gen(seed)
    dt = DTYPES[dtype]
    q = _randn(g, (batch, T, hq, dk)).to(dt)
    k = _unit_rows(_randn(g, (batch, T, n_hh, hq, dk))).to(dt)
    v = _randn(g, (batch, T, n_hh, hv, dv)).to(dt)
    A_log = _uniform(g, (hv,), 0.0, math.log(16.0))
    dt_bias = _randn(g, (hv,), 0.5)
    a = _randn(g, (batch, T, hv)).to(dt)
    b = _randn(g, (batch, T, n_hh, hv)).to(dt)
    pool = _randn(g, (pool_size, hv, dv, dk), pool_std) if materialize_pool else None
    need = batch + (batch * T if scatter else (batch if write_slots else 0))
    if need > pool_size:
        raise ValueError("pool too small for distinct slots")
    perm = torch.randperm(pool_size, generator=g).to(torch.int32)
    read = perm[:batch].clone()
    write = None
    scat = None
    if scatter:
        scat = perm[batch:batch + batch * T].clone().view(batch, T)
    elif write_slots:
        write = perm[batch:2 * batch].clone()
    if skip_rows:
        rows = torch.randperm(batch, generator=g)[:skip_rows]
        read[rows] = -1
    return dict(q=q, k=k, v=v, A_log=A_log, dt_bias=dt_bias, a=a, b=b, pool=pool,
                read_idx=read, write_idx=write, scatter_idx=scat, batch=batch, T=T,
                n_hh=n_hh, hq=hq, hv=hv, dk=dk, dv=dv, dtype=dtype, pool_size=pool_size,
                scale=(1.0 / math.sqrt(dk)) if scale is None else float(scale))


# --------------------------------------------------------------------------
# The five named workloads.  Seeds are the workload numbers 1..5.
# --------------------------------------------------------------------------

def single_head_scan():
    """B=2, S=64, one head, Dk=Dv=16, fp32; gamma ~ U[0.9,1], beta ~ U[0,1];
    zero initial state; scale 1."""
    return prefill_inputs(1, n_seqs=2, seq_len=64, hq=1, hv=1, dk=16, dv=16, dtype="f32",
                          gate="gamma", gamma_range=(0.9, 1.0), scale=1.0)


def chunked_prefill_b4_s4096():
    """B=4 x S=4096 packed, Hq=16, Hv=32, Dk=Dv=128, bf16 q/k/v; qwen gates
    from A_log ~ U[0, ln 16], dt_bias ~ N(0, 0.5), a, b ~ N(0, 1) bf16;
    scale 1/sqrt(128); zero initial state."""
    return prefill_inputs(2, n_seqs=4, seq_len=4096, hq=16, hv=32, dk=128, dv=128,
                          dtype="bf16", gate="qwen")


def ragged_prefill_lengths(seed: int = 30, n: int = 8, max_len: int = 8192):
    g = _gen(seed)
    lengths = torch.randint(1, max_len + 1, (n,), generator=g)
    zero = int(torch.randint(0, n, (1,), generator=g))
    lengths[zero] = 0
    return [int(x) for x in lengths], g


def ragged_prefill_8req():
    """8 ragged requests, lengths U{1..8192} with one forced to 0, via
    cu_seqlens; Hq=16, Hv=32, Dk=Dv=128, fp32; initial state ~ N(0, 0.05);
    gamma ~ U[0.8, 1] passed as gamma, beta ~ U[0, 1]; scale 1/sqrt(128)."""
    lengths, _ = ragged_prefill_lengths()
    return prefill_inputs(3, lengths=lengths, hq=16, hv=32, dk=128, dv=128, dtype="f32",
                          gate="gamma", gamma_range=(0.8, 1.0), init_std=0.05)


def decode_pool_b256(materialize_pool=True):
    """Pool [1024, 32, 128, 128] fp32 ~ N(0, 0.05); B=256 rows, 26 skipped;
    T=1, n=1; Hq=16, Hv=32; bf16 activations; qwen gates; distinct read and
    write slots."""
    return decode_inputs(4, pool_size=1024, batch=256, T=1, n_hh=1, hq=16, hv=32, dk=128,
                         dv=128, dtype="bf16", skip_rows=26, write_slots=True,
                         materialize_pool=materialize_pool)


def mtp_decode_b64_t4():
    """Pool [512, 16, 64, 128] fp32 ~ N(0, 0.05); B=64, T=4, n=2; H=Hv=16,
    Dk=128, Dv=64; bf16 activations; per-token scatter slots [64, 4]."""
    return decode_inputs(5, pool_size=512, batch=64, T=4, n_hh=2, hq=16, hv=16, dk=128,
                         dv=64, dtype="bf16", scatter=True)


def long_request_b1_s65536_hv4():
    """One request of 65536 tokens with few heads: Hq=2, Hv=4, Dk=Dv=128,
    bf16 q/k/v, qwen gates drawn as for the chunked-prefill workload, zero
    initial state, scale 1/sqrt(128).  Its serial walk fills only 8
    workgroups; it is the case the scan over segment maps is for."""
    return prefill_inputs(13, lengths=[65536], hq=2, hv=4, dk=128, dv=128, dtype="bf16",
                          gate="qwen")


def conv1d_inputs(seed: int, *, lengths, conv_dim, kernel_size=4, max_slots=8, dtype="bf16",
                  slots=None, state_std=1.0, x_std=1.0):
    """Inputs for one conv1d call (all CPU tensors), after the page example of
    "gated_delta_conv1d_fwd": x [T, conv_dim], weight [conv_dim, K] and the
    pool [max_slots, conv_dim, K-1] all standard normal (scaled by x_std /
    state_std), in the io dtype.  ``lengths`` lists the per-sequence row
    counts, packed back to back (row_offsets uint32-valued, held as int64).
    ``slots`` None draws distinct slots (a random choice without replacement
    from the pool); otherwise the given list is used as is."""
    g = _gen(seed)
    lengths = [int(x) for x in lengths]
    n = len(lengths)
    T = sum(lengths)
    off = torch.zeros(n + 1, dtype=torch.int64)
    off[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0)
    dt = DTYPES[dtype]
    K = int(kernel_size)
    x = _randn(g, (T, conv_dim), x_std).to(dt)
    w = _randn(g, (conv_dim, K)).to(dt)
    st = _randn(g, (max_slots, conv_dim, K - 1), state_std).to(dt)
    if slots is None:
        if n > max_slots:
            raise ValueError("distinct slots need n_seqs <= max_slots")
        slot = torch.randperm(max_slots, generator=g)[:n].to(torch.int64)
    else:
        slot = torch.tensor([int(v) for v in slots], dtype=torch.int64)
    return dict(x=x, weight=w, conv_state=st, slot_idx=slot, row_offsets=off, T=T,
                conv_dim=conv_dim, K=K, dtype=dtype, lengths=lengths)


def conv1d_prefill_b4_s4096():
    """The prefill batch's QKV projection ahead of the delta rule: B=4 x S=4096
    packed, conv_dim = 2*16*128 + 32*128 = 8192 (q, k of Hq=16 and v of Hv=32
    heads of size 128), K=4, bf16; pool of 64 slots, 4 distinct slots."""
    return conv1d_inputs(6, lengths=[4096] * 4, conv_dim=8192, kernel_size=4, max_slots=64,
                         dtype="bf16")


def conv1d_decode_b256():
    """One decode step's QKV rows: 256 sequences of length 1, conv_dim 8192,
    K=4, bf16; pool of 1024 slots, 256 distinct slots."""
    return conv1d_inputs(7, lengths=[1] * 256, conv_dim=8192, kernel_size=4, max_slots=1024,
                         dtype="bf16")


WORKLOADS = {
    "single_head_scan_b2_s64_d16_f32": single_head_scan,
    "chunked_prefill_b4_s4096_hv32_d128_bf16": chunked_prefill_b4_s4096,
    "ragged_prefill_8req_hv32_d128_f32": ragged_prefill_8req,
    "decode_pool1024_b256_hv32_d128_bf16": decode_pool_b256,
    "mtp_decode_b64_t4_n2_h16_dv64_bf16": mtp_decode_b64_t4,
}
