"""The C ABI on the host (no GPU needed): exports and host-side validation.

Every symbol include/libgdn.h declares must be exported by libgdn.so, and every
argument error the header documents must be returned before anything is
launched -- these calls never reach the device, so they run without a GPU.
"""
import ctypes
import os
import re

import pytest

import gated_deltanet_state_delta_amd._lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libgdn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from gated_deltanet_state_delta_amd import build
        build.build()
    return L.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_exported_set(lib):
    names = declared_functions()
    assert names == sorted(L.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), "libgdn.so does not export %s" % n


def test_version_and_error_text(lib):
    assert re.match(r"^\d+\.\d+\.\d+$", lib.gdn_version().decode())
    st = lib.gdn_gate(None, None, None, None, 9, 1, 1, None, None, None, None)
    assert st == 3  # GDN_ERR_DTYPE
    assert b"ab_dtype" in lib.gdn_last_error()


FAKE = 0x10000  # a 16-byte-aligned address that is never dereferenced on the host


def _prefill(**over):
    a = L.PrefillArgs()
    a.n_seqs, a.seq_len, a.total_tokens = 2, 8, 16
    a.hq, a.hv, a.dk, a.dv = 2, 4, 64, 64
    a.io_dtype, a.decay_kind, a.chunk_size, a.scale = L.GDN_BF16, L.GDN_DECAY_LOG, 0, 0.125
    a.q, a.q_stride_token, a.q_stride_head = FAKE, 128, 64
    a.k, a.k_stride_token, a.k_stride_head = FAKE * 2, 128, 64
    a.v, a.v_stride_token, a.v_stride_head = FAKE * 3, 256, 64
    a.out, a.out_stride_token, a.out_stride_head = FAKE * 4, 256, 64
    a.decay, a.beta = FAKE * 5, FAKE * 6
    a.cu_seqlens = None
    a.initial_state = None
    a.final_state = FAKE * 7
    for k, v in over.items():
        setattr(a, k, v)
    return a


def _decode(**over):
    d = L.DecodeArgs()
    d.batch, d.T, d.n_householder = 4, 2, 2
    d.hq, d.hv, d.dk, d.dv = 2, 4, 128, 64
    d.io_dtype, d.disable_state_update, d.scale = L.GDN_BF16, 0, 0.1
    d.q, d.k, d.v, d.A_log, d.dt_bias, d.a, d.b = (FAKE * i for i in range(1, 8))
    d.pool, d.pool_size, d.pool_slot_stride, d.pool_head_stride = FAKE * 8, 10, 4 * 64 * 128, 64 * 128
    d.read_idx, d.write_idx, d.scatter_idx, d.out = FAKE * 9, None, None, FAKE * 10
    for k, v in over.items():
        setattr(d, k, v)
    return d


PREFILL_ERRORS = [
    (dict(io_dtype=5), 3),
    (dict(decay_kind=2), 3),
    (dict(hq=3), 2),                      # hv % hq != 0
    (dict(dk=48), 5),
    (dict(dv=256), 5),
    (dict(chunk_size=8), 5),
    (dict(seq_len=7), 2),                 # n_seqs * seq_len != total_tokens
    (dict(final_state=None), 1),
    (dict(q=None), 1),
    (dict(beta=None), 1),
    (dict(q=FAKE + 8), 4),                # misaligned pointer
    (dict(v_stride_head=68), 4),          # stride not a multiple of 8
    (dict(q_stride_token=64), 4),         # token stride smaller than heads * dk
    (dict(v_stride_token=1 << 25), 4),    # stride too large for 32-bit in-chunk offsets
    (dict(q_stride_token=1 << 23), 4),    # the first stride past the 32-bit offset range
    (dict(out_stride_head=1 << 23), 4),
    (dict(initial_state=FAKE * 7 + 1024), 4),  # partial overlap with final_state
    (dict(n_seqs=-1), 2),
    # update_rule and the gate inputs it takes
    (dict(update_rule=4), 3),
    (dict(update_rule=1), 2),                          # gated takes no beta
    (dict(update_rule=1, beta=None, decay=None), 1),   # gated needs a decay
    (dict(update_rule=2), 2),                          # delta takes no decay
    (dict(update_rule=2, beta=None, decay=None), 1),   # delta needs a beta
    (dict(update_rule=3, beta=None), 2),               # linear takes no decay
    (dict(update_rule=3, decay=None), 2),              # ... and no beta
    (dict(update_rule=3, decay=None, beta=None, gate_a=FAKE * 8, A_log=FAKE * 9,
          dt_bias=FAKE * 10), 2),                      # linear takes no fused decay
    (dict(update_rule=3, decay=None, beta=None, gate_b=FAKE * 11), 2),  # ... and no fused beta
    (dict(gate_a=FAKE * 8, A_log=FAKE * 9, dt_bias=FAKE * 10), 2),  # decay and gate_a
    (dict(gate_b=FAKE * 8), 2),                        # beta and gate_b
    (dict(decay=None, gate_a=FAKE * 8, A_log=None, dt_bias=FAKE * 10, beta=None,
          gate_b=FAKE * 11), 1),                       # gate_a without A_log
    (dict(total_tokens=1 << 27, seq_len=1 << 26, hv=16, v_stride_token=1 << 24,
          out_stride_token=1 << 24), 2),               # total_tokens * hv >= 2^31
    # state pool
    (dict(final_state=None, state_pool=FAKE * 13, pool_size=10, pool_slot_stride=4 * 64 * 64, pool_head_stride=64 * 64, initial_state=FAKE * 14), 2),            # pool and initial_state
    (dict(state_pool=FAKE * 13, pool_size=10, pool_slot_stride=4 * 64 * 64,
          pool_head_stride=64 * 64), 2),                # pool and final_state
    (dict(final_state=None, state_pool=FAKE * 13, pool_size=-1, pool_slot_stride=4 * 64 * 64,
          pool_head_stride=64 * 64), 2),
    (dict(final_state=None, state_pool=FAKE * 13 + 8, pool_size=10, pool_slot_stride=4 * 64 * 64,
          pool_head_stride=64 * 64), 4),                # misaligned pool
    (dict(final_state=None, state_pool=FAKE * 13, pool_size=10, pool_slot_stride=4 * 64 * 64,
          pool_head_stride=64 * 64 - 4), 4),            # heads overlap
    (dict(final_state=None, state_pool=FAKE * 13, pool_size=10, pool_slot_stride=3 * 64 * 64,
          pool_head_stride=64 * 64), 4),                # slots overlap
    (dict(final_state=None, state_pool=FAKE * 13, pool_size=10, pool_slot_stride=4 * 64 * 64 + 2,
          pool_head_stride=64 * 64), 4),                # stride not a multiple of 4
    (dict(read_slot=FAKE * 15), 2),                     # slots without a pool
    (dict(decay_per_key=1, decay=None, beta=None, gate_a=FAKE * 8, A_log=FAKE * 9,
          dt_bias=FAKE * 10, gate_b=FAKE * 11), 5),      # per-key decay takes a given decay
    (dict(decay_per_key=1, decay=None, gate_a=FAKE * 8, A_log=FAKE * 9, dt_bias=FAKE * 10), 5),
    (dict(decay_per_key=1, update_rule=2, decay=None), 2),  # per-key decay with a rule without decay
    (dict(decay_per_key=1, update_rule=3, decay=None, beta=None), 2),
]


@pytest.mark.parametrize("over,status", PREFILL_ERRORS)
def test_prefill_rejects(lib, over, status):
    a = _prefill(**over)
    assert lib.gdn_prefill(ctypes.byref(a), None) == status
    assert lib.gdn_last_error()


def test_prefill_stride_limit_matches_the_kernel_offset_range(lib):
    """The kernels form a row's byte offset inside a chunk (up to 63 rows of
    one stride, elements of at most 4 bytes, plus the row's own extent) in
    32-bit signed arithmetic.  The validator's limit must keep that below
    2^31: the largest stride it accepts passes validation (on a host without
    a GPU the call then fails at the launch, GDN_ERR_HIP), the next multiple
    of 8 is refused, and the worst offset at the accepted stride fits."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("an accepted call would launch on the fake pointers of this test")
    limit = 1 << 23
    for field in ("q_stride_token", "k_stride_token", "v_stride_token", "out_stride_token",
                  "q_stride_head", "out_stride_head"):
        assert lib.gdn_prefill(ctypes.byref(_prefill(**{field: limit})), None) == 4
        st = lib.gdn_prefill(ctypes.byref(_prefill(**{field: limit - 8})), None)
        assert st in (0, 6), (field, st, lib.gdn_last_error())
    worst = 63 * (limit - 8) * 4 + 128 * 4
    assert worst < (1 << 31)


def test_prefill_rule_inputs_accepted_before_launch(lib):
    """Each rule with exactly its inputs passes validation: checked with
    tokens present (so the gate checks run) but n_seqs = 0 through
    cu_seqlens, where a valid request returns OK without launching."""
    base = dict(n_seqs=0, seq_len=0, total_tokens=16, cu_seqlens=FAKE * 12)
    assert lib.gdn_prefill(ctypes.byref(_prefill(**base)), None) == 0
    for rule, dec, bet in ((1, FAKE * 5, None), (2, None, FAKE * 6), (3, None, None)):
        a = _prefill(update_rule=rule, decay=dec, beta=bet, **base)
        assert lib.gdn_prefill(ctypes.byref(a), None) == 0, lib.gdn_last_error()


def test_prefill_mixed_gate_sources_accepted_before_launch(lib):
    """"com.microsoft.GatedDeltaNet", Attributes: gate_activation and
    beta_activation are separate, so a fused decay with a given beta and a
    given decay with a fused beta both pass validation (n_seqs = 0 through
    cu_seqlens: nothing is launched); so does a per-key decay with a fused
    beta."""
    base = dict(n_seqs=0, seq_len=0, total_tokens=16, cu_seqlens=FAKE * 12)
    a = _prefill(decay=None, gate_a=FAKE * 8, A_log=FAKE * 9, dt_bias=FAKE * 10, **base)
    assert lib.gdn_prefill(ctypes.byref(a), None) == 0, lib.gdn_last_error()
    a = _prefill(beta=None, gate_b=FAKE * 8, **base)
    assert lib.gdn_prefill(ctypes.byref(a), None) == 0, lib.gdn_last_error()
    a = _prefill(beta=None, gate_b=FAKE * 8, decay_per_key=1, **base)
    assert lib.gdn_prefill(ctypes.byref(a), None) == 0, lib.gdn_last_error()


def test_prefill_pool_mode_accepted_before_launch(lib):
    a = _prefill(n_seqs=0, seq_len=0, total_tokens=16, cu_seqlens=FAKE * 12, final_state=None,
                 state_pool=FAKE * 13, pool_size=10, pool_slot_stride=4 * 64 * 64 + 64,
                 pool_head_stride=64 * 64 + 16, read_slot=FAKE * 15, write_slot=FAKE * 16)
    assert lib.gdn_prefill(ctypes.byref(a), None) == 0, lib.gdn_last_error()


def test_prefill_workspace_size(lib):
    """0 for calls that run as serial walks; for one long request with few
    heads the scan's workspace n_seqs * nseg * hv * dk * (2 dv + dk) * 4 bytes,
    with nseg from the sizes alone (about 512 local-pass workgroups, segments
    of 16 chunks or more, 4 <= nseg <= 64)."""
    assert lib.gdn_prefill_workspace_size(None) == 0
    assert lib.gdn_prefill_workspace_size(ctypes.byref(_prefill())) == 0
    def one_long(**over):
        kw = dict(n_seqs=1, seq_len=65536, total_tokens=65536, hq=2, hv=4, dk=128, dv=128,
                  q_stride_token=256, k_stride_token=256, q_stride_head=128, k_stride_head=128,
                  v_stride_token=512, out_stride_token=512, v_stride_head=128, out_stride_head=128)
        kw.update(over)
        return lib.gdn_prefill_workspace_size(ctypes.byref(_prefill(**kw)))
    # 512 / (1 * 4 * (256 / 64)) = 32 segments of 32 chunks
    assert one_long() == 1 * 32 * 4 * 128 * (2 * 128 + 128) * 4
    # dk = dv = 64: 512 / (4 * 2) = 64 segments
    assert one_long(dk=64, dv=64) == 1 * 64 * 4 * 64 * (2 * 64 + 64) * 4
    # shorter request: segments of at least 16 chunks -> 8192 / 64 / 16 = 8
    assert one_long(seq_len=8192, total_tokens=8192) == 8 * 4 * 128 * 384 * 4
    # too short for 4 segments, too many heads, fp32, per-key decay, a chunk hint,
    # mixed gates: serial walks, no workspace
    assert one_long(seq_len=2048, total_tokens=2048) == 0
    # Hv = 32: the serial walk fills 64 workgroups, 4 segments still pay;
    # Hv = 64 fills 128 and keeps the serial walk
    assert one_long(hv=32, hq=16, q_stride_token=2048, k_stride_token=2048,
                    v_stride_token=4096, out_stride_token=4096) == 4 * 32 * 128 * 384 * 4
    assert one_long(hv=64, hq=16, q_stride_token=2048, k_stride_token=2048,
                    v_stride_token=8192, out_stride_token=8192) == 0
    assert one_long(io_dtype=L.GDN_F32) == 0
    assert one_long(decay_per_key=1) == 0
    assert one_long(chunk_size=32) == 0
    assert one_long(beta=None, gate_b=FAKE * 8) == 0
    # the size is at most about 25 MiB whenever it is not 0
    for hv in (1, 2, 4, 8):
        for d in (64, 128):
            for n in (1, 2):
                sz = one_long(hv=hv, dk=d, dv=d, n_seqs=n, seq_len=65536 // n,
                              q_stride_token=hv * d, k_stride_token=hv * d,
                              q_stride_head=d, k_stride_head=d, hq=hv,
                              v_stride_token=hv * d, out_stride_token=hv * d,
                              v_stride_head=d, out_stride_head=d)
                assert sz <= 26 * 1024 * 1024


def test_prefill_noalloc_host_checks(lib):
    """gdn_prefill_noalloc refuses what gdn_prefill refuses, before any
    launch, and every call the scan plan can choose fits its static array."""
    assert lib.gdn_prefill_noalloc(None, None) == 1
    assert b"gdn_prefill_noalloc" in lib.gdn_last_error()
    for over, status in PREFILL_ERRORS:
        assert lib.gdn_prefill_noalloc(ctypes.byref(_prefill(**over)), None) == status
    a = _prefill(n_seqs=0, seq_len=0, total_tokens=0)
    assert lib.gdn_prefill_noalloc(ctypes.byref(a), None) == 0
    for hv in (1, 2, 4, 8, 16, 32):
        for d in (64, 128):
            for n in (1, 2, 3):
                a = _prefill(n_seqs=n, seq_len=(1 << 20) // n, total_tokens=((1 << 20) // n) * n,
                             hq=hv, hv=hv, dk=d, dv=d, q_stride_token=hv * d, k_stride_token=hv * d,
                             q_stride_head=d, k_stride_head=d, v_stride_token=hv * d,
                             out_stride_token=hv * d, v_stride_head=d, out_stride_head=d)
                assert lib.gdn_prefill_workspace_size(ctypes.byref(a)) <= L.NOALLOC_SCRATCH_BYTES


def test_wait_timeouts_null(lib):
    """gdn_wait_timeouts refuses a NULL count before touching the device."""
    assert lib.gdn_wait_timeouts(None, 0) == 1
    assert b"gdn_wait_timeouts" in lib.gdn_last_error()


def test_prefill_null_args_and_noop(lib):
    assert lib.gdn_prefill(None, None) == 1
    a = _prefill(n_seqs=0, seq_len=0, total_tokens=0)
    assert lib.gdn_prefill(ctypes.byref(a), None) == 0  # nothing to do, nothing launched


DECODE_ERRORS = [
    (dict(io_dtype=2), 3),
    (dict(T=0), 2),
    (dict(T=65), 5),
    (dict(n_householder=0), 5),
    (dict(n_householder=5), 5),
    (dict(hq=3), 2),
    (dict(hq=1, hv=65537), 5),   # in-kernel offsets of a pass stay 32-bit
    (dict(dk=96), 5),
    (dict(scatter_idx=FAKE * 11, disable_state_update=1), 5),
    (dict(pool=None), 1),
    (dict(read_idx=None), 1),
    (dict(pool=FAKE + 4), 4),
    (dict(pool_head_stride=64 * 128 + 2), 4),
    (dict(pool_slot_stride=64 * 128), 4),   # slots overlap the heads
    (dict(q=FAKE + 2), 4),
    (dict(pool_size=-1), 2),
]


@pytest.mark.parametrize("over,status", DECODE_ERRORS)
def test_decode_rejects(lib, over, status):
    d = _decode(**over)
    assert lib.gdn_decode(ctypes.byref(d), None) == status
    assert lib.gdn_last_error()


def test_decode_null_args_and_noop(lib):
    assert lib.gdn_decode(None, None) == 1
    d = _decode(batch=0)
    assert lib.gdn_decode(ctypes.byref(d), None) == 0


def test_gate_rejects(lib):
    assert lib.gdn_gate(None, None, None, None, 1, -1, 4, None, None, None, None) == 2
    assert lib.gdn_gate(None, None, None, None, 1, 4, 0, None, None, None, None) == 2
    assert lib.gdn_gate(None, None, None, FAKE, 1, 4, 4, FAKE, None, None, None) == 1  # decay w/o a
    assert lib.gdn_gate(None, None, FAKE, None, 1, 4, 4, None, None, FAKE, None) == 1  # beta w/o b
    assert lib.gdn_gate(None, None, FAKE, None, 1, 4, 4, FAKE, None, None, None) == 1  # a w/o A_log
    assert lib.gdn_gate(None, None, None, None, 1, 0, 4, None, None, None, None) == 0  # n == 0


def _conv1d(**over):
    c = L.Conv1dArgs()
    c.total_tokens, c.conv_dim, c.kernel_size, c.n_seqs = 64, 256, 4, 3
    c.io_dtype, c.write_state, c.max_slots = L.GDN_BF16, 1, 8
    c.x, c.x_stride_token = FAKE, 256
    c.weight, c.conv_state, c.slot_idx, c.row_offsets = FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5
    c.out, c.out_stride_token = FAKE * 6, 256
    for k, v in over.items():
        setattr(c, k, v)
    return c


CONV1D_ERRORS = [
    (dict(io_dtype=3), 3),
    (dict(total_tokens=-1), 2),
    (dict(conv_dim=0), 2),
    (dict(n_seqs=-2), 2),
    (dict(max_slots=-1), 2),
    (dict(kernel_size=0), 5),
    (dict(kernel_size=9), 5),
    (dict(conv_dim=252, x_stride_token=252, out_stride_token=252), 4),  # not a multiple of 8 bf16
    (dict(x=None), 1),
    (dict(weight=None), 1),
    (dict(conv_state=None), 1),           # required for kernel_size > 1
    (dict(slot_idx=None), 1),
    (dict(row_offsets=None), 1),
    (dict(out=None), 1),
    (dict(x=FAKE + 8), 4),                # not 16-byte aligned
    (dict(conv_state=FAKE * 3 + 4), 4),
    (dict(out_stride_token=200), 4),      # smaller than conv_dim
    (dict(x_stride_token=260), 4),        # not a multiple of 8 elements
    (dict(out=FAKE + 256 * 2 * 10), 4),   # out overlaps x
]


@pytest.mark.parametrize("over,status", CONV1D_ERRORS)
def test_conv1d_rejects(lib, over, status):
    c = _conv1d(**over)
    assert lib.gdn_conv1d(ctypes.byref(c), None) == status
    assert lib.gdn_last_error()


def test_conv1d_null_args_and_noop(lib):
    assert lib.gdn_conv1d(None, None) == 1
    assert lib.gdn_conv1d(ctypes.byref(_conv1d(n_seqs=0)), None) == 0
    assert lib.gdn_conv1d(ctypes.byref(_conv1d(total_tokens=0)), None) == 0
    # kernel_size 1 needs no conv state; nothing to do without sequences
    assert lib.gdn_conv1d(ctypes.byref(_conv1d(kernel_size=1, conv_state=None, n_seqs=0)), None) == 0


@pytest.mark.parametrize("cname,pycls", [("gdn_prefill_args", "PrefillArgs"), ("gdn_decode_args", "DecodeArgs"),
                                         ("gdn_conv1d_args", "Conv1dArgs")])
def test_struct_layout_matches_the_binding(cname, pycls, tmp_path):
    """Every field of the argument structs sits at the same offset in C (gcc
    on the header) and in the Python binding's ctypes mirror."""
    import subprocess
    cls = getattr(L, pycls)
    fields = [f[0] for f in cls._fields_]
    src = tmp_path / "layout.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "libgdn.h"', "int main(void) {",
             '  printf("%%zu\\n", sizeof(%s));' % cname]
    lines += ['  printf("%%zu\\n", offsetof(%s, %s));' % (cname, f) for f in fields]
    lines += ["  return 0;", "}"]
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    want = [ctypes.sizeof(cls)] + [getattr(cls, f).offset for f in fields]
    assert got == want
