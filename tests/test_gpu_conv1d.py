"""Causal depthwise conv1d with a slot-indexed conv-state pool
("gated_delta_conv1d_fwd") through the C ABI, against the fp64 oracle.

Outputs are compared at the io dtype's tolerance (fp32 accumulation, one
rounding to the io dtype).  The pool after the call must equal the oracle's
bit for bit: the new window is a copy of io-dtype values, no arithmetic.
Cases cover every kernel_size template (1..8), both io dtypes, channel counts
whose 16-byte groups do not fill a wave, ragged sequences that start and end
inside the kernel's 32-row runs and 8-row unrolled blocks, sequences shorter
than the window, empty sequences, out-of-range and negative slots, rows no
sequence covers, write_state off, strided rows, split calls, and the two full
workloads the benchmark times.
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


RAGGED = [1, 0, 37, 100, 2, 64, 33, 3, 200]


def _state_np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _run(x, *, write_state=True, out_init=None, slot_override=None, offsets_override=None):
    slots = x["slot_idx"] if slot_override is None else slot_override
    offs = x["row_offsets"] if offsets_override is None else offsets_override
    pool = to_dev(x["conv_state"].clone()) if x["K"] > 1 else None
    out = None if out_init is None else to_dev(out_init.clone())
    o = gdn.conv1d(to_dev(x["x"]), to_dev(x["weight"]), pool, to_dev(slots), to_dev(offs),
                   write_state=write_state, out=out)
    ro, rst = oracle.conv1d(x["x"], x["weight"], x["conv_state"], slots.numpy(), offs.numpy(),
                            write_state=write_state,
                            out_init=None if out_init is None else out_init)
    torch.cuda.synchronize()
    return o, pool, ro, rst


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 6, 7, 8])
def test_ragged_all_kernel_sizes(dtype, K):
    x = synth.conv1d_inputs(100 + K, lengths=RAGGED, conv_dim=264, kernel_size=K, max_slots=12,
                            dtype=dtype)
    o, pool, ro, rst = _run(x)
    # rows of the empty sequence are covered by no one: none here (all packed)
    assert_close(o, ro, dtype, "conv1d out K=%d" % K)
    if K > 1:
        np.testing.assert_array_equal(_state_np(pool), rst)


# short sequences: the kernel then gives each thread 1, 2 or 4 rows (from the
# mean length), so sequences longer than that span threads and their windows
# are written by the second launch, while the others are written in place
SHORT = {
    "decode_len1": [1] * 40,
    "mixed_short": [1, 1, 3, 1, 2, 0, 1, 5, 1, 1, 2, 7],
    "mtp_len4": [4] * 16,
    "len3_rows2": [3] * 11,
    "one_long_among_short": [1] * 20 + [90] + [1] * 5,
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name", list(SHORT))
def test_short_sequences(name, dtype):
    lengths = SHORT[name]
    x = synth.conv1d_inputs(200 + len(lengths), lengths=lengths, conv_dim=136, kernel_size=4,
                            max_slots=len(lengths) + 3, dtype=dtype)
    o, pool, ro, rst = _run(x)
    assert_close(o, ro, dtype, "conv1d out %s" % name)
    np.testing.assert_array_equal(_state_np(pool), rst)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_write_state_off_leaves_pool(dtype):
    x = synth.conv1d_inputs(11, lengths=RAGGED, conv_dim=512, kernel_size=4, max_slots=16,
                            dtype=dtype)
    o, pool, ro, rst = _run(x, write_state=False)
    assert_close(o, ro, dtype, "conv1d out, write_state off")
    np.testing.assert_array_equal(_state_np(pool), _state_np(x["conv_state"]))
    np.testing.assert_array_equal(rst, _state_np(x["conv_state"]))


def test_out_of_range_and_negative_slots():
    lengths = [5, 40, 1, 70]
    x = synth.conv1d_inputs(12, lengths=lengths, conv_dim=128, kernel_size=4, max_slots=6,
                            dtype="f32")
    slots = torch.tensor([6, 2, -1, 2**32 - 1], dtype=torch.int64)
    o, pool, ro, rst = _run(x, slot_override=slots)
    assert_close(o, ro, "f32", "conv1d out, skipped slots")
    # only slot 2 is written
    before = _state_np(x["conv_state"])
    after = _state_np(pool)
    np.testing.assert_array_equal(after, rst)
    keep = [s for s in range(6) if s != 2]
    np.testing.assert_array_equal(after[keep], before[keep])


def test_uncovered_rows_keep_out():
    x = synth.conv1d_inputs(13, lengths=[50, 90, 20], conv_dim=256, kernel_size=4,
                            max_slots=4, dtype="bf16")
    T = x["T"]
    offs = torch.tensor([7, 50, 50, T - 9], dtype=torch.int64)  # rows 0..6 and T-9..T-1 uncovered
    init = torch.full((T, 256), 7.0).to(torch.bfloat16)
    o, pool, ro, rst = _run(x, out_init=init, offsets_override=offs)
    assert_close(o, ro, "bf16", "conv1d out, uncovered rows")
    assert torch.all(o[:7].cpu() == 7.0) and torch.all(o[T - 9:].cpu() == 7.0)
    np.testing.assert_array_equal(_state_np(pool), rst)


def test_offsets_past_the_end_are_clamped():
    x = synth.conv1d_inputs(14, lengths=[30, 30], conv_dim=64, kernel_size=3, max_slots=3,
                            dtype="f32")
    offs = torch.tensor([0, 45, 10**6], dtype=torch.int64)
    o, pool, ro, rst = _run(x, offsets_override=offs)
    assert_close(o, ro, "f32", "conv1d out, clamped offsets")
    np.testing.assert_array_equal(_state_np(pool), rst)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strided_rows(dtype):
    x = synth.conv1d_inputs(15, lengths=[70, 1, 129], conv_dim=192, kernel_size=4, max_slots=5,
                            dtype=dtype)
    dt = synth.DTYPES[dtype]
    T = x["T"]
    wide = torch.zeros(T, 192 + 64, dtype=dt)
    wide[:, 32:224] = x["x"]
    xin = to_dev(wide)[:, 32:224]
    big_out = torch.full((T, 320), -3.0, dtype=dt, device="cuda")
    out = big_out[:, 64:256]
    pool = to_dev(x["conv_state"].clone())
    gdn.conv1d(xin, to_dev(x["weight"]), pool, to_dev(x["slot_idx"]), to_dev(x["row_offsets"]),
               out=out)
    ro, rst = oracle.conv1d(x["x"], x["weight"], x["conv_state"], x["slot_idx"].numpy(),
                            x["row_offsets"].numpy())
    torch.cuda.synchronize()
    assert_close(out, ro, dtype, "conv1d strided out")
    assert torch.all(big_out[:, :64].cpu() == -3.0) and torch.all(big_out[:, 256:].cpu() == -3.0)
    np.testing.assert_array_equal(_state_np(pool), rst)


def test_split_calls_equal_one_call():
    """A sequence fed in pieces (each call writing its window back) gives the
    same outputs and final window as one call over the whole sequence."""
    x = synth.conv1d_inputs(16, lengths=[300], conv_dim=256, kernel_size=4, max_slots=2,
                            dtype="f32")
    xd, wd = to_dev(x["x"]), to_dev(x["weight"])
    slot = torch.tensor([1], device="cuda")
    pool_a = to_dev(x["conv_state"].clone())
    whole = gdn.conv1d(xd, wd, pool_a, slot, torch.tensor([0, 300], device="cuda"))
    pool_b = to_dev(x["conv_state"].clone())
    parts = []
    for a, b in ((0, 1), (1, 2), (2, 77), (77, 300)):
        parts.append(gdn.conv1d(xd[a:b].contiguous(), wd, pool_b, slot,
                                torch.tensor([0, b - a], device="cuda")))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(torch.cat(parts).cpu().numpy(), whole.cpu().numpy())
    np.testing.assert_array_equal(pool_a.cpu().numpy(), pool_b.cpu().numpy())
    ro, rst = oracle.conv1d(x["x"], x["weight"], x["conv_state"], np.array([1]), np.array([0, 300]))
    assert_close(whole, ro, "f32", "conv1d whole")
    np.testing.assert_array_equal(_state_np(pool_a), rst)


def test_no_sequences_and_no_tokens_are_noops():
    x = synth.conv1d_inputs(17, lengths=[4], conv_dim=64, kernel_size=4, max_slots=2,
                            dtype="bf16")
    pool = to_dev(x["conv_state"].clone())
    out = torch.full((4, 64), 5.0, dtype=torch.bfloat16, device="cuda")
    gdn.conv1d(to_dev(x["x"]), to_dev(x["weight"]), pool, torch.zeros(0, dtype=torch.int32, device="cuda"),
               torch.zeros(1, dtype=torch.int32, device="cuda"), out=out)
    gdn.conv1d(to_dev(x["x"][:0]), to_dev(x["weight"]), pool, torch.tensor([0], device="cuda"),
               torch.tensor([0, 0], device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(out.cpu() == 5.0)
    np.testing.assert_array_equal(_state_np(pool), _state_np(x["conv_state"]))


@pytest.mark.parametrize("make", [synth.conv1d_prefill_b4_s4096, synth.conv1d_decode_b256],
                         ids=["prefill_b4_s4096_c8192", "decode_b256_c8192"])
def test_full_workloads(make):
    """The benchmark's two conv1d workloads at full size, every element."""
    x = make()
    o, pool, ro, rst = _run(x)
    assert_close(o, ro, x["dtype"], "conv1d full workload")
    np.testing.assert_array_equal(_state_np(pool), rst)
