"""Prefill over a slot-indexed state pool (the decode's pool layout) through
the C ABI, against the fp64 oracle.

Request r starts from pool[read_slot[r]] (zeros for a slot outside the pool)
and stores its final state to pool[write_slot[r]] (the read slot when
write_slot is None; nothing for a slot outside the pool).  The expected pool
is built on the host from the oracle's final states; slots nobody writes
must keep their bits.  A multi-token decode batch run as a pooled prefill
(one request per batch row, fused gate) must match the decode kernel and the
decode oracle.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_state_delta_amd as gdn
import oracle
import synth
from gpu_util import assert_close, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


LENGTHS = [70, 0, 129, 33, 1]
READ = [3, 5, -1, 7, 9]       # request 2 starts from zeros
WRITE = [3, 11, 0, -1, 2]     # request 0 reads and writes slot 3; request 3 stores nothing


def _expected(x, pool0, read, write):
    P = pool0.shape[0]
    init = np.zeros((len(read), *pool0.shape[1:]))
    for r, s in enumerate(read):
        if 0 <= s < P:
            init[r] = pool0[s]
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], x["log_decay"], x["beta"],
                            cu_seqlens=x["cu_seqlens"], initial_state=init, scale=x["scale"])
    pool = pool0.astype(np.float64).copy()
    written = set()
    for r in range(len(read)):
        s = (write[r] if write is not None else read[r])
        if 0 <= s < P:
            pool[s] = rf[r]
            written.add(s)
    return ro, pool, written


@pytest.mark.parametrize("cfg", [("bf16", 128, 128, 0), ("bf16", 64, 64, 0), ("f32", 64, 64, 32),
                                 ("bf16", 32, 32, 16)],
                         ids=["pair_d128", "pair_d64", "general_f32_c32", "general_d32_c16"])
@pytest.mark.parametrize("write_given", [True, False], ids=["write_slots", "write_is_read"])
def test_pooled_prefill_matches_oracle(cfg, write_given):
    dt, dk, dv, chunk = cfg
    x = synth.prefill_inputs(410, lengths=LENGTHS, hq=2, hv=4, dk=dk, dv=dv, dtype=dt,
                             gate="log", gamma_range=(0.85, 1.0))
    g = torch.Generator().manual_seed(411)
    pool0 = torch.randn(12, 4, dv, dk, generator=g) * 0.05
    read = torch.tensor(READ, dtype=torch.int32)
    write = torch.tensor(WRITE, dtype=torch.int32) if write_given else None
    if not write_given:
        read = torch.tensor([3, 5, -1, 7, 20], dtype=torch.int32)  # distinct; one outside the pool
    pool = to_dev(pool0.clone())
    o, p_out = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["log_decay"]),
                           to_dev(x["beta"]), cu_seqlens=to_dev(x["cu_seqlens"]),
                           scale=x["scale"], chunk_size=chunk, state_pool=pool,
                           read_slot=to_dev(read), write_slot=to_dev(write))
    torch.cuda.synchronize()
    assert p_out is pool
    ro, rpool, written = _expected(x, pool0.numpy(), read.tolist(),
                                   None if write is None else write.tolist())
    assert_close(o, ro, dt, "pooled prefill out")
    got = pool.cpu().double().numpy()
    for s in range(12):
        if s in written:
            assert_close(got[s], rpool[s], dt, "slot %d" % s)
        else:
            np.testing.assert_array_equal(got[s], pool0[s].double().numpy())


def test_pooled_prefill_with_padded_pool_strides():
    """Slot and head strides larger than the dense extents (multiples of 4)."""
    x = synth.prefill_inputs(412, lengths=[40, 90], hq=1, hv=2, dk=64, dv=64, dtype="bf16",
                             gate="log")
    g = torch.Generator().manual_seed(413)
    base = torch.zeros(6 * (2 * (64 * 64 + 8) + 12))
    pool = base.as_strided((6, 2, 64, 64), (2 * (64 * 64 + 8) + 12, 64 * 64 + 8, 64, 1))
    pool.copy_(torch.randn(6, 2, 64, 64, generator=g) * 0.05)
    dbase = to_dev(base.clone())
    dpool = dbase.as_strided(pool.shape, pool.stride())
    read = torch.tensor([1, 4], dtype=torch.int32)
    write = torch.tensor([2, 5], dtype=torch.int32)
    o, _ = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["log_decay"]),
                       to_dev(x["beta"]), cu_seqlens=to_dev(x["cu_seqlens"]), scale=x["scale"],
                       state_pool=dpool, read_slot=to_dev(read), write_slot=to_dev(write))
    torch.cuda.synchronize()
    ro, rpool, written = _expected(x, pool.numpy(), read.tolist(), write.tolist())
    assert_close(o, ro, "bf16", "padded-pool out")
    got = dpool.cpu().double().numpy()
    for s in range(6):
        if s in written:
            assert_close(got[s], rpool[s], "bf16", "slot %d" % s)
        else:
            np.testing.assert_array_equal(got[s], pool[s].double().numpy())
    # the padding between heads and slots is never written
    db = dbase.cpu()
    mask = torch.ones_like(base, dtype=torch.bool)
    mask[torch.as_strided(torch.arange(base.numel()), pool.shape, pool.stride()).reshape(-1)] = False
    assert torch.all(db[mask] == 0)


@pytest.mark.parametrize("T", [4, 9, 33])
def test_multi_token_decode_as_pooled_prefill(T):
    """One request per batch row over the decode's pool with the fused gate:
    the chunked form equals the decode kernel's token loop (n = 1, no scatter)."""
    d = synth.decode_inputs(420 + T, pool_size=40, batch=12, T=T, n_hh=1, hq=2, hv=4, dk=128,
                            dv=128, dtype="bf16", skip_rows=0, write_slots=True)
    B, hq, hv, dk, dv = 12, 2, 4, 128, 128
    t = {n: to_dev(d[n]) for n in ("q", "k", "v", "A_log", "dt_bias", "a", "b", "read_idx",
                                   "write_idx")}
    pool_a = to_dev(d["pool"].clone())
    od, _ = gdn.decode(t["q"], t["k"], t["v"], t["A_log"], t["dt_bias"], t["a"], t["b"], pool_a,
                       t["read_idx"], write_idx=t["write_idx"], scale=d["scale"], use_qk_l2norm=False)
    pool_b = to_dev(d["pool"].clone())
    cu = torch.arange(B + 1, dtype=torch.int32, device="cuda") * T
    op, _ = gdn.prefill(t["q"].reshape(B * T, hq, dk), t["k"].reshape(B * T, hq, dk),
                        t["v"].reshape(B * T, hv, dv), None, None, A_log=t["A_log"],
                        dt_bias=t["dt_bias"], a=t["a"].reshape(B * T, hv),
                        b=t["b"].reshape(B * T, hv), cu_seqlens=cu, scale=d["scale"],
                        state_pool=pool_b, read_slot=t["read_idx"], write_slot=t["write_idx"])
    torch.cuda.synchronize()
    ro, rpool = oracle.decode(d["q"], d["k"], d["v"], d["A_log"], d["dt_bias"], d["a"], d["b"],
                              d["pool"], d["read_idx"], write_idx=d["write_idx"], scale=d["scale"])
    assert_close(op.view(B, T, hv, dv), ro, "bf16", "chunked decode out")
    assert_close(od, ro, "bf16", "decode out")
    assert_close(pool_b, rpool, "bf16", "chunked decode pool")
    assert_close(pool_a, rpool, "bf16", "decode pool")
