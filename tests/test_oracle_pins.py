"""Pins for the fp64 oracle, each against something other than the oracle.

CPU only.  Every check here is fixed by the pages or by mathematics:
  * the three worked examples printed on "Gated DeltaNet State Update";
  * invariants the recurrence implies (beta=0/gamma=1 identity, gamma=0 reset,
    unit-key overwrite, linearity in (V, S0));
  * a brute-force product of explicit Dk x Dk per-step matrices, as the page's
    hints suggest (identity matrix, batched matmul, broadcast outer products),
    and a tree reduction of the per-step affine maps;
  * a closed form: one-hot keys turn every state row into a scalar EMA;
  * contract identities from the ONNX card and the FlashInfer page (ragged ==
    separate calls, cu_seqlens clamping, empty-request copy, GVA == explicit
    head repeat, split/resume, decode == prefill, Householder sub-steps ==
    expanded tokens, slot skip / scatter / disable rules);
  * library routines for the gate (torch softplus with threshold 20, sigmoid).
A plausible slip in the oracle (dropped term, wrong sign, transposed operand,
wrong head map, readout before the update, decay applied per sub-step) fails
at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _bsd_to_tokens(x):
    """(B, S, D) -> (B*S, 1, D): one head, requests packed back to back."""
    x = np.asarray(x, dtype=np.float64)
    return x.reshape(x.shape[0] * x.shape[1], 1, x.shape[2])


# ----------------------------------------------------------------------------
# worked examples ("Gated DeltaNet State Update", Examples)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("idx", [0, 1, 2])
def test_worked_examples(idx):
    ex = json.load(open(GOLDEN))["examples"][idx]
    q = _bsd_to_tokens(ex["q"])
    k = _bsd_to_tokens(ex["k"])
    v = _bsd_to_tokens(ex["v"])
    B, S = len(ex["q"]), len(ex["q"][0])
    gam = np.asarray(ex["gamma"], dtype=np.float64).reshape(B * S, 1)
    beta = np.asarray(ex["beta"], dtype=np.float64).reshape(B * S, 1)
    out, fin = oracle.prefill(q, k, v, gam, beta, decay_is_gamma=True, n_seqs=B, seq_len=S,
                              scale=1.0)
    want_out = np.asarray(ex["outputs"], dtype=np.float64)
    want_fin = np.asarray(ex["final_state"], dtype=np.float64)  # (B, Dk, Dv) K-major
    np.testing.assert_array_equal(out.reshape(want_out.shape), want_out)
    # oracle final state is V-major (B, H, Dv, Dk)
    np.testing.assert_array_equal(fin[:, 0].transpose(0, 2, 1), want_fin)


# ----------------------------------------------------------------------------
# brute force with explicit per-step matrices
# ----------------------------------------------------------------------------

def _bruteforce(q, k, v, gam, beta, S0, scale):
    """S_t = M_t S_{t-1} + beta_t k_t v_t^T with M_t = gamma_t (I - beta_t k_t k_t^T),
    y_t = scale * q_t^T S_t; single head, K-major state."""
    dk = q.shape[1]
    S = S0.copy()
    ys = []
    I = np.eye(dk)
    for t in range(q.shape[0]):
        M = gam[t] * (I - beta[t] * np.outer(k[t], k[t]))
        S = M @ S + beta[t] * np.outer(k[t], v[t])
        ys.append(scale * (q[t] @ S))
    return np.array(ys), S


def _affine_tree(k, v, gam, beta, S0):
    """Final state via a balanced tree reduction of the affine maps S -> M S + B."""
    dk = k.shape[1]
    maps = [(gam[t] * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])), beta[t] * np.outer(k[t], v[t]))
            for t in range(k.shape[0])]
    while len(maps) > 1:
        nxt = []
        for i in range(0, len(maps) - 1, 2):
            (M1, B1), (M2, B2) = maps[i], maps[i + 1]  # apply 1, then 2
            nxt.append((M2 @ M1, M2 @ B1 + B2))
        if len(maps) % 2:
            nxt.append(maps[-1])
        maps = nxt
    M, Bm = maps[0]
    return M @ S0 + Bm


@pytest.mark.parametrize("seed,dk,dv,S", [(0, 2, 3, 5), (1, 4, 4, 17), (2, 8, 5, 32), (3, 7, 8, 9)])
def test_bruteforce_explicit_matrices(seed, dk, dv, S):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, dk))
    k = rng.standard_normal((S, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((S, dv))
    gam = rng.uniform(0.0, 1.0, S)
    beta = rng.uniform(0.0, 1.0, S)
    S0 = rng.standard_normal((dk, dv))
    scale = 0.7
    y_bf, S_bf = _bruteforce(q, k, v, gam, beta, S0, scale)
    out, fin = oracle.prefill(q[:, None], k[:, None], v[:, None], gam[:, None], beta[:, None],
                              decay_is_gamma=True, n_seqs=1, seq_len=S,
                              initial_state=S0.T[None, None], scale=scale)
    np.testing.assert_allclose(out[:, 0], y_bf, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0].T, S_bf, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0].T, _affine_tree(k, v, gam, beta, S0), rtol=1e-11, atol=1e-11)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

def test_beta0_gamma1_leaves_state_unchanged():
    rng = np.random.default_rng(5)
    dk, dv, S = 6, 5, 11
    q = rng.standard_normal((S, 1, dk))
    k = rng.standard_normal((S, 1, dk))
    v = rng.standard_normal((S, 1, dv))
    S0 = rng.standard_normal((1, 1, dv, dk))
    out, fin = oracle.prefill(q, k, v, np.ones((S, 1)), np.zeros((S, 1)), decay_is_gamma=True,
                              n_seqs=1, seq_len=S, initial_state=S0, scale=2.0)
    np.testing.assert_array_equal(fin, S0)
    np.testing.assert_allclose(out[:, 0], 2.0 * q[:, 0] @ S0[0, 0].T, rtol=1e-13)


def test_gamma0_gives_rank_one_state():
    rng = np.random.default_rng(6)
    dk, dv, S = 5, 7, 9
    q = rng.standard_normal((S, 1, dk))
    k = rng.standard_normal((S, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((S, 1, dv))
    gam = rng.uniform(0.2, 1.0, (S, 1))
    gam[-1] = 0.0
    beta = rng.uniform(0.0, 1.0, (S, 1))
    S0 = rng.standard_normal((1, 1, dv, dk))
    _, fin = oracle.prefill(q, k, v, gam, beta, decay_is_gamma=True, n_seqs=1, seq_len=S,
                            initial_state=S0)
    want = beta[-1, 0] * np.outer(k[-1, 0], v[-1, 0])  # K-major
    np.testing.assert_allclose(fin[0, 0].T, want, rtol=1e-14, atol=1e-15)
    # the same reset through the log-space input (log 0 = -inf)
    with np.errstate(divide="ignore"):
        logd = np.log(gam)
    _, fin2 = oracle.prefill(q, k, v, logd, beta, n_seqs=1, seq_len=S, initial_state=S0)
    np.testing.assert_array_equal(fin2, fin)


def test_unit_key_beta1_overwrites_its_direction():
    rng = np.random.default_rng(7)
    dk, dv = 8, 6
    S0 = rng.standard_normal((dk, dv))
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(dv)
    g = 0.6
    out, fin = oracle.prefill(np.zeros((1, 1, dk)), k[None, None], v[None, None],
                              np.array([[g]]), np.array([[1.0]]), decay_is_gamma=True,
                              n_seqs=1, seq_len=1, initial_state=S0.T[None, None])
    S1 = fin[0, 0].T
    np.testing.assert_allclose(S1.T @ k, v, rtol=1e-13, atol=1e-13)  # retrieves exactly v
    P = np.eye(dk) - np.outer(k, k)
    np.testing.assert_allclose(P @ S1, g * (P @ S0), rtol=1e-13, atol=1e-13)  # rest only decays


def test_linear_in_values_and_initial_state():
    rng = np.random.default_rng(8)
    T, dk, dv = 40, 6, 5
    q = rng.standard_normal((T, 1, dk))
    k = rng.standard_normal((T, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    gam = rng.uniform(0.5, 1.0, (T, 1))
    beta = rng.uniform(0.0, 1.0, (T, 1))
    v1, v2 = rng.standard_normal((2, T, 1, dv))
    s1, s2 = rng.standard_normal((2, 1, 1, dv, dk))
    a, b = 1.7, -0.4
    run = lambda v, s: oracle.prefill(q, k, v, gam, beta, decay_is_gamma=True, n_seqs=1,
                                      seq_len=T, initial_state=s)
    o1, f1 = run(v1, s1)
    o2, f2 = run(v2, s2)
    o3, f3 = run(a * v1 + b * v2, a * s1 + b * s2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(f3, a * f1 + b * f2, rtol=1e-11, atol=1e-11)


def test_onehot_keys_closed_form():
    """k_t = e_{i_t}: row i_t follows S <- gamma (1 - beta) S + beta v, every
    other row S <- gamma S; outputs read row i of the state through q."""
    rng = np.random.default_rng(9)
    T, dk, dv = 300, 32, 24
    idx = rng.integers(0, dk, T)
    k = np.zeros((T, 1, dk))
    k[np.arange(T), 0, idx] = 1.0
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    gam = rng.uniform(0.8, 1.0, (T, 1))
    beta = rng.uniform(0.0, 1.0, (T, 1))
    S0 = rng.standard_normal((dk, dv))
    out, fin = oracle.prefill(q, k, v, gam, beta, decay_is_gamma=True, n_seqs=1, seq_len=T,
                              initial_state=S0.T[None, None], scale=0.5)
    S = S0.copy()
    for t in range(T):
        i = idx[t]
        S *= gam[t, 0]                                              # every row decays
        S[i] = (1.0 - beta[t, 0]) * S[i] + beta[t, 0] * v[t, 0]     # addressed row: EMA
        np.testing.assert_allclose(out[t, 0], 0.5 * q[t, 0] @ S, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(fin[0, 0].T, S, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------
# contract identities: ragged / empty / clamped / GVA / split-resume
# ----------------------------------------------------------------------------

def _small(seed, lengths, hq=2, hv=4, dk=8, dv=6, init=True, gate="gamma"):
    return synth.prefill_inputs(seed, lengths=lengths, hq=hq, hv=hv, dk=dk, dv=dv,
                                dtype="f32", gate=gate, gamma_range=(0.5, 1.0),
                                init_std=0.3 if init else None)


def _run(x, **kw):
    dec = x.get("gamma", x.get("log_decay"))
    args = dict(decay_is_gamma="gamma" in x, cu_seqlens=x["cu_seqlens"],
                initial_state=x["initial_state"], scale=x["scale"])
    args.update(kw)
    return oracle.prefill(x["q"], x["k"], x["v"], dec, x["beta"], **args)


def test_ragged_equals_separate_requests():
    lengths = [5, 0, 13, 1, 9]
    x = _small(11, lengths)
    out, fin = _run(x)
    cu = x["cu_seqlens"].tolist()
    for r, L in enumerate(lengths):
        s, e = cu[r], cu[r + 1]
        dec = x["gamma"][s:e]
        o_r, f_r = oracle.prefill(x["q"][s:e], x["k"][s:e], x["v"][s:e], dec, x["beta"][s:e],
                                  decay_is_gamma=True, n_seqs=1, seq_len=L,
                                  initial_state=x["initial_state"][r:r + 1], scale=x["scale"])
        np.testing.assert_array_equal(out[s:e], o_r)
        np.testing.assert_array_equal(fin[r], f_r[0])
    # the empty request copies its incoming state bit for bit
    np.testing.assert_array_equal(fin[1], x["initial_state"][1].double().numpy())


def test_empty_request_without_initial_state_is_zero():
    x = _small(12, [4, 0, 3], init=False)
    _, fin = _run(x)
    assert np.all(fin[1] == 0.0)


def test_cu_seqlens_clamped_and_decreasing():
    x = _small(13, [6, 6, 6])
    T = x["T"]
    cu = torch.tensor([0, 6, 3, T + 50], dtype=torch.int32)  # decreasing, then past the end
    out, fin = _run(x, cu_seqlens=cu)
    # request 1 is [6, 3) -> empty: copies its state
    np.testing.assert_array_equal(fin[1], x["initial_state"][1].double().numpy())
    # request 2 is clamped to [3, T)
    ref_o, ref_f = oracle.prefill(x["q"][3:], x["k"][3:], x["v"][3:], x["gamma"][3:],
                                  x["beta"][3:], decay_is_gamma=True, n_seqs=1, seq_len=T - 3,
                                  initial_state=x["initial_state"][2:3], scale=x["scale"])
    np.testing.assert_array_equal(fin[2], ref_f[0])
    # rows 3..5 lie in requests 0 and 2 at once: which request's output they
    # end up holding is unspecified (units run in parallel); rows 6.. are
    # request 2's alone, rows 0..2 request 0's alone
    np.testing.assert_array_equal(out[6:], ref_o[3:])
    ref0, _ = oracle.prefill(x["q"][:6], x["k"][:6], x["v"][:6], x["gamma"][:6], x["beta"][:6],
                             decay_is_gamma=True, n_seqs=1, seq_len=6,
                             initial_state=x["initial_state"][0:1], scale=x["scale"])
    np.testing.assert_array_equal(out[:3], ref0[:3])


def test_gva_equals_explicit_head_repeat():
    x = _small(14, [7, 12], hq=2, hv=6)
    out, fin = _run(x)
    rep = 6 // 2
    q = x["q"].repeat_interleave(rep, dim=1)
    k = x["k"].repeat_interleave(rep, dim=1)
    out2, fin2 = oracle.prefill(q, k, x["v"], x["gamma"], x["beta"], decay_is_gamma=True,
                                cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
                                scale=x["scale"])
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(fin, fin2)
    # and value head h really reads q/k head h*hq/hv: swapping the q/k heads changes heads 0..2 only
    q_sw = x["q"].flip(1)
    out3, _ = oracle.prefill(q_sw, x["k"], x["v"], x["gamma"], x["beta"], decay_is_gamma=True,
                             cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
                             scale=x["scale"])
    assert not np.allclose(out3[:, 0], out[:, 0])


def test_split_resume():
    x = _small(15, [40], hq=1, hv=2)
    out, fin = _run(x)
    n = 17
    o1, f1 = oracle.prefill(x["q"][:n], x["k"][:n], x["v"][:n], x["gamma"][:n], x["beta"][:n],
                            decay_is_gamma=True, n_seqs=1, seq_len=n,
                            initial_state=x["initial_state"], scale=x["scale"])
    o2, f2 = oracle.prefill(x["q"][n:], x["k"][n:], x["v"][n:], x["gamma"][n:], x["beta"][n:],
                            decay_is_gamma=True, n_seqs=1, seq_len=40 - n, initial_state=f1,
                            scale=x["scale"])
    np.testing.assert_allclose(np.concatenate([o1, o2]), out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(f2, fin, rtol=1e-12, atol=1e-13)


def test_log_and_gamma_inputs_agree():
    x = _small(16, [9, 4])
    out, fin = _run(x)
    out2, fin2 = oracle.prefill(x["q"], x["k"], x["v"], torch.log(x["gamma"].double()), x["beta"],
                                cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
                                scale=x["scale"])
    np.testing.assert_allclose(out2, out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(fin2, fin, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------
# gate vs library routines
# ----------------------------------------------------------------------------

def test_gate_against_torch_routines():
    rng = np.random.default_rng(17)
    hv = 5
    A_log = rng.uniform(-2.0, 3.0, hv)
    dt_bias = rng.normal(0.0, 0.5, hv)
    a = np.concatenate([rng.normal(0.0, 4.0, (40, hv)),
                        np.array([[20.0, 20.0 + 1e-9, 19.999, 25.0, -30.0]]) - dt_bias])
    b = rng.normal(0.0, 3.0, (41, hv))
    g, gam, beta = oracle.gate(A_log, dt_bias, a, b)
    x = torch.tensor(a + dt_bias, dtype=torch.float64)
    sp = torch.nn.functional.softplus(x, beta=1.0, threshold=20.0).numpy()
    want_g = -np.exp(A_log) * sp
    np.testing.assert_allclose(g, want_g, rtol=1e-14, atol=0)
    np.testing.assert_allclose(gam, np.exp(want_g), rtol=1e-14, atol=0)
    np.testing.assert_allclose(beta, torch.sigmoid(torch.tensor(b)).numpy(), rtol=1e-15, atol=0)


def test_gate_special_values():
    g, gam, beta = oracle.gate([-math.inf, 0.0], [0.0, 0.0], [[3.0, 0.0]], [[0.0, 0.0]])
    assert gam[0, 0] == 1.0                       # A_log = -inf: no decay
    assert g[0, 1] == -math.log(2.0)              # softplus(0) = ln 2
    assert beta[0, 0] == 0.5                      # sigmoid(0)
    # threshold: identity strictly above 20, log1p(exp(x)) at and below
    g2, _, _ = oracle.gate([0.0], [0.0], [[20.5], [20.0]], None)
    assert g2[0, 0] == -20.5
    assert g2[1, 0] == -math.log1p(math.exp(20.0))


# ----------------------------------------------------------------------------
# decode identities
# ----------------------------------------------------------------------------

def _dec(seed, **kw):
    args = dict(pool_size=12, batch=3, T=3, n_hh=1, hq=2, hv=4, dk=8, dv=6, dtype="f32")
    args.update(kw)
    return synth.decode_inputs(seed, **args)


def _run_dec(x, **kw):
    args = dict(write_idx=x["write_idx"], scatter_idx=x["scatter_idx"], scale=x["scale"])
    args.update(kw)
    return oracle.decode(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"], x["b"],
                         x["pool"], x["read_idx"], **args)


def test_decode_equals_prefill_with_slot_state():
    x = _dec(21, T=5)
    out, pool = _run_dec(x)
    g, _, beta = oracle.gate(x["A_log"], x["dt_bias"], x["a"], x["b"][:, :, 0])
    for b in range(x["batch"]):
        rd, wr = int(x["read_idx"][b]), int(x["write_idx"][b])
        o, f = oracle.prefill(x["q"][b], x["k"][b, :, 0], x["v"][b, :, 0], g[b], beta[b],
                              n_seqs=1, seq_len=x["T"], initial_state=x["pool"][rd:rd + 1],
                              scale=x["scale"])
        np.testing.assert_allclose(out[b], o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(pool[wr], f[0], rtol=1e-12, atol=1e-13)


def test_householder_substeps_equal_expanded_tokens():
    """n sub-steps per token == gated delta over T*n tokens whose decay is the
    token's gamma on its first sub-step and 1 on the others, read out on the
    last sub-step."""
    x = _dec(22, T=3, n_hh=3)
    out, pool = _run_dec(x)
    T, n = x["T"], x["n_hh"]
    g, _, _ = oracle.gate(x["A_log"], x["dt_bias"], x["a"], None)
    _, _, beta = oracle.gate(x["A_log"], x["dt_bias"], None, x["b"])  # [B,T,n,hv]
    for b in range(x["batch"]):
        rd, wr = int(x["read_idx"][b]), int(x["write_idx"][b])
        kk = x["k"][b].reshape(T * n, x["hq"], x["dk"])
        vv = x["v"][b].reshape(T * n, x["hv"], x["dv"])
        qq = x["q"][b].repeat_interleave(n, dim=0)  # same q on every sub-step
        dec = np.zeros((T, n, x["hv"]))
        dec[:, 0] = g[b]
        bb = beta[b].reshape(T * n, x["hv"])
        o, f = oracle.prefill(qq, kk, vv, dec.reshape(T * n, -1), bb, n_seqs=1, seq_len=T * n,
                              initial_state=x["pool"][rd:rd + 1], scale=x["scale"])
        o = o.reshape(T, n, x["hv"], x["dv"])[:, -1]
        np.testing.assert_allclose(out[b], o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(pool[wr], f[0], rtol=1e-12, atol=1e-13)


def test_decode_skip_write_scatter_disable_rules():
    x = _dec(23, batch=4, T=2, pool_size=20)
    pool0 = x["pool"].double().numpy()
    read = x["read_idx"].clone()
    write = x["write_idx"].clone()
    read[1] = -1          # skipped row
    read[2] = 20          # out of range: skipped as well
    write[3] = -5         # row 3 computes its output but writes nothing back
    sentinel = np.full((4, 2, x["hv"], x["dv"]), 7.25)
    out, pool = oracle.decode(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"], x["b"],
                              x["pool"], read, write_idx=write, scale=x["scale"], out_init=sentinel)
    assert np.all(out[1] == 7.25) and np.all(out[2] == 7.25)
    assert not np.any(out[3] == 7.25) and not np.any(out[0] == 7.25)
    changed = {int(write[0])}
    for s in range(20):
        if s not in changed:
            np.testing.assert_array_equal(pool[s], pool0[s])
    assert not np.array_equal(pool[int(write[0])], pool0[int(write[0])])
    # disable_state_update: outputs identical, pool untouched
    out_d, pool_d = oracle.decode(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"],
                                  x["b"], x["pool"], read, write_idx=write, scale=x["scale"],
                                  out_init=sentinel, disable_state_update=True)
    np.testing.assert_array_equal(out_d, out)
    np.testing.assert_array_equal(pool_d, pool0)
    # scatter: state after each token to its slot, negative entries skipped, no end writeback
    sc = torch.tensor([[10, 11], [12, 13], [14, 15], [-1, 16]], dtype=torch.int32)
    out_s, pool_s = oracle.decode(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"],
                                  x["b"], x["pool"], read, write_idx=write, scatter_idx=sc,
                                  scale=x["scale"], out_init=sentinel)
    np.testing.assert_array_equal(out_s, out)
    np.testing.assert_array_equal(pool_s[11], pool[int(write[0])])  # last token of row 0
    for s in (12, 13, 14, 15):  # rows 1 and 2 are skipped entirely
        np.testing.assert_array_equal(pool_s[s], pool0[s])
    np.testing.assert_array_equal(pool_s[int(write[0])], pool0[int(write[0])])
    with pytest.raises(ValueError):
        oracle.decode(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"], x["b"], x["pool"],
                      read, scatter_idx=sc, disable_state_update=True)


def test_decode_scatter_first_token_equals_one_token_call():
    x = _dec(24, batch=2, T=2, pool_size=10, write_slots=False, scatter=True)
    out, pool = _run_dec(x)
    x1 = dict(x)
    for key in ("q", "k", "v", "a", "b"):
        x1[key] = x[key][:, :1]
    sc1 = x["scatter_idx"][:, :1]
    out1, pool1 = oracle.decode(x1["q"], x1["k"], x1["v"], x["A_log"], x["dt_bias"], x1["a"],
                                x1["b"], x["pool"], x["read_idx"], scatter_idx=sc1,
                                scale=x["scale"])
    np.testing.assert_array_equal(out[:, 0], out1[:, 0])
    for b in range(2):
        s = int(sc1[b, 0])
        np.testing.assert_array_equal(pool[s], pool1[s])


# ----------------------------------------------------------------------------
# in-kernel q/k L2 norm and the fused gate inside prefill (the ONNX card's
# qk_l2_norm attribute; the FlashInfer page's use_qk_l2norm and fused gate)
# ----------------------------------------------------------------------------

def _raw_qk(seed, T=40, hq=2, dk=8):
    """q and k that are far from unit length (norms spread over 0.2 .. 5)."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(T, hq, dk, generator=g, dtype=torch.float64)
    k = torch.randn(T, hq, dk, generator=g, dtype=torch.float64)
    s = torch.rand(T, hq, 1, generator=g, dtype=torch.float64) * 4.8 + 0.2
    return (q * s).numpy(), (k / s).numpy()


def test_qk_l2norm_invariant_to_rescaling_q_and_k():
    """With the norm on (eps = 0), scaling any q or k head vector by a positive
    factor changes nothing; with it off the outputs change."""
    x = synth.prefill_inputs(60, lengths=[40], hq=2, hv=4, dk=8, dv=6, gate="gamma",
                             gamma_range=(0.6, 1.0), init_std=0.3)
    q, k = _raw_qk(61)
    g = torch.Generator().manual_seed(62)
    cq = (torch.rand(40, 2, 1, generator=g, dtype=torch.float64) * 3 + 0.1).numpy()
    ck = (torch.rand(40, 2, 1, generator=g, dtype=torch.float64) * 3 + 0.1).numpy()
    kw = dict(decay_is_gamma=True, cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
              scale=0.7)
    o1, f1 = oracle.prefill(q, k, x["v"], x["gamma"], x["beta"], qk_l2norm_eps=0.0, **kw)
    o2, f2 = oracle.prefill(q * cq, k * ck, x["v"], x["gamma"], x["beta"], qk_l2norm_eps=0.0, **kw)
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(f2, f1, rtol=1e-11, atol=1e-12)
    o3, _ = oracle.prefill(q * cq, k * ck, x["v"], x["gamma"], x["beta"], **kw)
    assert np.abs(o3 - o1).max() > 1e-3


def test_qk_l2norm_equals_prenormalised_inputs():
    """The norm is x / sqrt(sum x^2 + eps): the same as normalising the inputs
    with numpy (eps folded into the norm) and running without it."""
    x = synth.prefill_inputs(63, lengths=[17, 0, 23], hq=1, hv=2, dk=16, dv=8, gate="log",
                             gamma_range=(0.5, 1.0))
    q, k = _raw_qk(64, T=40, hq=1, dk=16)
    eps = 0.25  # large enough to matter
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + eps)
    kn = k / np.sqrt(np.einsum("thd,thd->th", k, k)[..., None] + eps)
    kw = dict(cu_seqlens=x["cu_seqlens"], scale=0.5)
    o1, f1 = oracle.prefill(q, k, x["v"], x["log_decay"], x["beta"], qk_l2norm_eps=eps, **kw)
    o2, f2 = oracle.prefill(qn, kn, x["v"], x["log_decay"], x["beta"], **kw)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(f1, f2, rtol=1e-12, atol=1e-13)


def test_qk_l2norm_of_a_zero_vector_is_zero():
    """eps > 0 keeps an all-zero key finite: it normalises to zero, so the
    token writes nothing and only decays the state."""
    x = synth.prefill_inputs(65, n_seqs=1, seq_len=6, hq=1, hv=1, dk=4, dv=3, gate="gamma",
                             gamma_range=(0.5, 0.9), init_std=1.0)
    k = x["k"].clone().double()
    k[2] = 0.0
    q = x["q"].clone().double()
    q[2] = 0.0
    out, fin = oracle.prefill(q, k, x["v"], x["gamma"], x["beta"], decay_is_gamma=True,
                              n_seqs=1, seq_len=6, initial_state=x["initial_state"],
                              qk_l2norm_eps=1e-12)
    assert np.isfinite(out).all() and np.isfinite(fin).all()
    assert np.abs(out[2]).max() == 0.0
    # the state after token 2 is the state after token 1 times gamma_2
    _, f1 = oracle.prefill(q[:2], k[:2], x["v"][:2], x["gamma"][:2], x["beta"][:2],
                           decay_is_gamma=True, n_seqs=1, seq_len=2,
                           initial_state=x["initial_state"], qk_l2norm_eps=1e-12)
    _, f2 = oracle.prefill(q[:3], k[:3], x["v"][:3], x["gamma"][:3], x["beta"][:3],
                           decay_is_gamma=True, n_seqs=1, seq_len=3,
                           initial_state=x["initial_state"], qk_l2norm_eps=1e-12)
    np.testing.assert_allclose(f2, f1 * float(x["gamma"][2, 0]), rtol=1e-13, atol=1e-15)


def test_fused_gate_prefill_equals_gate_then_prefill():
    """Gates computed inside the prefill (qwen gate, sigmoid beta) equal the
    separate gate call (itself pinned to torch's routines above)."""
    x = synth.prefill_inputs(66, lengths=[30, 11], hq=2, hv=4, dk=8, dv=8, gate="qwen",
                             init_std=0.2)
    g, _, beta = oracle.gate(x["A_log"], x["dt_bias"], x["a"], x["b"])
    kw = dict(cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"], scale=0.3)
    o1, f1 = oracle.prefill(x["q"], x["k"], x["v"], g, beta, **kw)
    o2, f2 = oracle.prefill(x["q"], x["k"], x["v"], None, None, A_log=x["A_log"],
                            dt_bias=x["dt_bias"], a=x["a"], b=x["b"], **kw)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)


def test_decode_qk_l2norm_invariance_and_prenormalised_inputs():
    x = _dec(67, T=3, n_hh=2, dk=8)
    g = torch.Generator().manual_seed(68)
    cq = (torch.rand(*x["q"].shape[:3], 1, generator=g, dtype=torch.float64) * 3 + 0.1)
    ck = (torch.rand(*x["k"].shape[:4], 1, generator=g, dtype=torch.float64) * 3 + 0.1)
    o1, p1 = _run_dec(x, qk_l2norm_eps=0.0)
    y = dict(x)
    y["q"] = x["q"].double() * cq
    y["k"] = x["k"].double() * ck
    o2, p2 = _run_dec(y, qk_l2norm_eps=0.0)
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(p2, p1, rtol=1e-11, atol=1e-12)
    eps = 0.5
    z = dict(y)
    qd, kd = y["q"].numpy(), y["k"].numpy()
    z["q"] = qd / np.sqrt((qd * qd).sum(-1, keepdims=True) + eps)
    z["k"] = kd / np.sqrt((kd * kd).sum(-1, keepdims=True) + eps)
    o3, p3 = _run_dec(y, qk_l2norm_eps=eps)
    o4, p4 = _run_dec(z)
    np.testing.assert_allclose(o3, o4, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p3, p4, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# causal conv1d with a slot-indexed conv-state pool ("gated_delta_conv1d_fwd")
# ----------------------------------------------------------------------------

def test_conv1d_page_example_invariants():
    """The page's example: two sequences (lengths 3 and 2) on slots 2 and 0
    of a 3-slot pool, K = 4: afterwards slot 2 holds the first sequence's
    three inputs, slot 0 holds the last three entries of its window, slot 1
    is unchanged.  Inputs drawn as the example draws them."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 8), dtype=np.float32)
    w = rng.standard_normal((8, 4), dtype=np.float32)
    st = rng.standard_normal((3, 8, 3), dtype=np.float32)
    out, st2 = oracle.conv1d(x, w, st, np.array([2, 0]), np.array([0, 3, 5]))
    np.testing.assert_array_equal(st2[2], x[0:3].T)
    np.testing.assert_array_equal(st2[0][:, 1:], x[3:5].T)
    np.testing.assert_array_equal(st2[0][:, 0], st[0][:, 2])
    np.testing.assert_array_equal(st2[1], st[1])
    assert out.shape == (5, 8) and np.isfinite(out).all()


def test_conv1d_against_torch_grouped_conv():
    """Each sequence equals torch's depthwise conv1d (groups = channels) over
    its slot's saved inputs followed by its own."""
    g = torch.Generator().manual_seed(90)
    T, C, K = 37, 12, 4
    x = torch.randn(T, C, generator=g, dtype=torch.float64)
    w = torch.randn(C, K, generator=g, dtype=torch.float64)
    st = torch.randn(5, C, K - 1, generator=g, dtype=torch.float64)
    offs = np.array([0, 10, 10, 29, 37])
    slots = np.array([3, 1, 4, 0])
    out, _ = oracle.conv1d(x, w, st, slots, offs)
    for b in range(4):
        s0, s1 = offs[b], offs[b + 1]
        if s1 == s0:
            continue
        inp = torch.cat([st[slots[b]], x[s0:s1].T], dim=1)[None]  # [1, C, K-1+len]
        ref = torch.nn.functional.conv1d(inp, w[:, None, :], groups=C)[0].T
        np.testing.assert_allclose(out[s0:s1], ref.numpy(), rtol=1e-13, atol=1e-13)


def test_conv1d_split_calls_equal_one_call():
    g = torch.Generator().manual_seed(91)
    T, C, K = 50, 6, 4
    x = torch.randn(T, C, generator=g, dtype=torch.float64).numpy()
    w = torch.randn(C, K, generator=g, dtype=torch.float64).numpy()
    st = torch.randn(2, C, K - 1, generator=g, dtype=torch.float64).numpy()
    out, st_end = oracle.conv1d(x, w, st, np.array([1]), np.array([0, T]))
    for cut in (1, 2, 3, 17):
        o1, s1 = oracle.conv1d(x[:cut], w, st, np.array([1]), np.array([0, cut]))
        o2, s2 = oracle.conv1d(x[cut:], w, s1, np.array([1]), np.array([0, T - cut]))
        np.testing.assert_array_equal(np.concatenate([o1, o2]), out)
        np.testing.assert_array_equal(s2, st_end)


def test_conv1d_delay_weights_closed_form_and_write_state_flag():
    """A one-hot weight at tap K-1-d delays the input by d (the saved inputs
    supply the first d outputs); write_state=False leaves the pool alone."""
    g = torch.Generator().manual_seed(92)
    T, C, K = 9, 5, 4
    x = torch.randn(T, C, generator=g, dtype=torch.float64).numpy()
    st = torch.randn(1, C, K - 1, generator=g, dtype=torch.float64).numpy()
    for d in range(K):
        w = np.zeros((C, K))
        w[:, K - 1 - d] = 1.0
        out, st2 = oracle.conv1d(x, w, st, np.array([0]), np.array([0, T]), write_state=False)
        hist = np.concatenate([st[0].T, x])  # [K-1+T, C]
        np.testing.assert_array_equal(out, hist[K - 1 - d:K - 1 - d + T])
        np.testing.assert_array_equal(st2, st)


def test_conv1d_out_of_range_slot_reads_zeros_and_writes_nothing():
    g = torch.Generator().manual_seed(93)
    x = torch.randn(6, 3, generator=g, dtype=torch.float64).numpy()
    w = torch.randn(3, 3, generator=g, dtype=torch.float64).numpy()
    st = torch.randn(2, 3, 2, generator=g, dtype=torch.float64).numpy()
    out, st2 = oracle.conv1d(x, w, st, np.array([7]), np.array([0, 6]))
    out0, _ = oracle.conv1d(x, w, np.zeros_like(st), np.array([0]), np.array([0, 6]))
    np.testing.assert_array_equal(out, out0)
    np.testing.assert_array_equal(st2, st)


# ---------------------------------------------------------------------------
# update_rule variants ("com.microsoft.GatedDeltaNet", update_rule attribute)


def _rule_inputs(seed, lengths=(5, 0, 12), hq=2, hv=4, dk=6, dv=5):
    g = torch.Generator().manual_seed(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    q = torch.randn(T, hq, dk, generator=g, dtype=torch.float64).numpy()
    k = torch.randn(T, hq, dk, generator=g, dtype=torch.float64).numpy() * 0.4
    v = torch.randn(T, hv, dv, generator=g, dtype=torch.float64).numpy()
    logd = -torch.rand(T, hv, generator=g, dtype=torch.float64).numpy() * 0.5
    beta = torch.rand(T, hv, generator=g, dtype=torch.float64).numpy()
    init = torch.randn(len(lengths), hv, dv, dk, generator=g, dtype=torch.float64).numpy()
    return dict(q=q, k=k, v=v, logd=logd, beta=beta, init=init, cu=cu, hq=hq, hv=hv)


def _masked_form(x, decayed, scale):
    """Y = scale (D o (Q K^T)) V + scale diag(e^G) Q S0 and S = e^{G_T} S0 +
    K^T diag(e^{G_T - G}) V per (request, head): the matrix form of linear
    attention (D = causal ones) and of its decayed variant (D_ts = e^{G_t -
    G_s}, s <= t), with no retrieval term."""
    q, k, v, cu, hq, hv = x["q"], x["k"], x["v"], x["cu"], x["hq"], x["hv"]
    T = q.shape[0]
    out = np.full((T, hv, v.shape[2]), np.nan)
    fin = np.zeros_like(x["init"])
    for r in range(len(cu) - 1):
        a, b = cu[r], cu[r + 1]
        for h in range(hv):
            qh = h * hq // hv
            Q, K, V = q[a:b, qh], k[a:b, qh], v[a:b, h]
            S0 = x["init"][r, h].T  # K-major [dk, dv]
            G = np.cumsum(x["logd"][a:b, h]) if decayed else np.zeros(b - a)
            D = np.tril(np.exp(G[:, None] - G[None, :]))
            out[a:b, h] = scale * ((D * (Q @ K.T)) @ V + np.exp(G)[:, None] * (Q @ S0))
            GT = G[-1] if b > a else 0.0
            S = np.exp(GT) * S0 + K.T @ (np.exp(GT - G)[:, None] * V)
            fin[r, h] = S.T
    return out, fin


@pytest.mark.parametrize("rule", ["linear", "gated"])
def test_rules_without_retrieval_match_the_masked_matrix_form(rule):
    x = _rule_inputs(101)
    dec = x["logd"] if rule == "gated" else None
    out, fin = oracle.prefill(x["q"], x["k"], x["v"], dec, None, cu_seqlens=x["cu"],
                              initial_state=x["init"], scale=0.7, update_rule=rule)
    ref_o, ref_f = _masked_form(x, rule == "gated", 0.7)
    np.testing.assert_allclose(out, ref_o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin, ref_f, rtol=1e-12, atol=1e-12)


def test_delta_rule_with_one_hot_keys_is_a_per_row_ema():
    """delta: S <- S + k (beta (v - S^T k))^T.  With one-hot keys e_i the
    update touches row i only: row_i <- (1 - beta) row_i + beta v."""
    g = torch.Generator().manual_seed(102)
    T, dk, dv = 40, 5, 3
    idx = torch.randint(0, dk, (T,), generator=g).numpy()
    k = np.zeros((T, 1, dk))
    k[np.arange(T), 0, idx] = 1.0
    q = torch.randn(T, 1, dk, generator=g, dtype=torch.float64).numpy()
    v = torch.randn(T, 1, dv, generator=g, dtype=torch.float64).numpy()
    beta = torch.rand(T, 1, generator=g, dtype=torch.float64).numpy()
    init = torch.randn(1, 1, dv, dk, generator=g, dtype=torch.float64).numpy()
    out, fin = oracle.prefill(q, k, v, None, beta, n_seqs=1, seq_len=T, initial_state=init,
                              scale=1.0, update_rule="delta")
    S = init[0, 0].T.copy()  # rows = keys
    for t in range(T):
        i = idx[t]
        S[i] = (1.0 - beta[t, 0]) * S[i] + beta[t, 0] * v[t, 0]
        np.testing.assert_allclose(out[t, 0], q[t, 0] @ S, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(fin[0, 0], S.T, rtol=1e-13, atol=1e-13)


def test_delta_equals_gated_delta_without_decay():
    """The ONNX card's step form (delta) and the problem statement's
    Householder form (gated_delta at gamma = 1) agree."""
    x = _rule_inputs(103)
    o1, f1 = oracle.prefill(x["q"], x["k"], x["v"], None, x["beta"], cu_seqlens=x["cu"],
                            initial_state=x["init"], scale=0.5, update_rule="delta")
    o2, f2 = oracle.prefill(x["q"], x["k"], x["v"], np.zeros_like(x["beta"]), x["beta"],
                            cu_seqlens=x["cu"], initial_state=x["init"], scale=0.5)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f1, f2, rtol=1e-12, atol=1e-12)


def test_rules_ignore_the_inputs_they_drop_and_fuse_per_input():
    """Rules read only their own inputs; the fused decay (a) and the fused
    beta (b) each equal the separate gate's output."""
    x = _rule_inputs(104)
    g = torch.Generator().manual_seed(105)
    T, hv = x["v"].shape[0], x["hv"]
    A_log = torch.rand(hv, generator=g, dtype=torch.float64).numpy()
    dt_bias = torch.randn(hv, generator=g, dtype=torch.float64).numpy() * 0.5
    a = torch.randn(T, hv, generator=g, dtype=torch.float64).numpy()
    b = torch.randn(T, hv, generator=g, dtype=torch.float64).numpy()
    gd, _, gb = oracle.gate(A_log, dt_bias, a, b)
    kw = dict(cu_seqlens=x["cu"], initial_state=x["init"], scale=0.9)
    args = (x["q"], x["k"], x["v"])
    # gated: beta is never read; fused a == separate gate
    o1, f1 = oracle.prefill(*args, gd, None, update_rule="gated", **kw)
    o2, f2 = oracle.prefill(*args, gd, np.full_like(gd, 7.0), update_rule="gated", **kw)
    o3, f3 = oracle.prefill(*args, None, None, A_log=A_log, dt_bias=dt_bias, a=a,
                            update_rule="gated", **kw)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_allclose(o1, o3, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f1, f3, rtol=1e-12, atol=1e-12)
    # delta: decay is never read; fused b == separate sigmoid
    o1, _ = oracle.prefill(*args, None, gb, update_rule="delta", **kw)
    o2, _ = oracle.prefill(*args, np.full_like(gb, -3.0), gb, update_rule="delta", **kw)
    o3, _ = oracle.prefill(*args, None, None, b=b, update_rule="delta", **kw)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_allclose(o1, o3, rtol=1e-12, atol=1e-12)
    # gated_delta with the decay fused and beta given == both given
    o1, _ = oracle.prefill(*args, gd, gb, **kw)
    o2, _ = oracle.prefill(*args, None, gb, A_log=A_log, dt_bias=dt_bias, a=a, **kw)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    # a rule missing an input it needs is an argument error
    with pytest.raises(ValueError):
        oracle.prefill(*args, None, gb, **kw)
    with pytest.raises(ValueError):
        oracle.prefill(*args, gd, None, update_rule="delta", **kw)


# ---------------------------------------------------------------------------
# per-key decay ("com.microsoft.GatedDeltaNet", decay input: the per-key-
# dimension spelling (..., num_heads_v, head_size_qk)): exp(g_t) scales the
# key rows of S elementwise in the card's recurrence


def _pk_inputs(seed, T=23, dk=5, dv=4, hv=2):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(T, 1, dk, generator=g, dtype=torch.float64).numpy()
    k = torch.randn(T, 1, dk, generator=g, dtype=torch.float64).numpy()
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = torch.randn(T, hv, dv, generator=g, dtype=torch.float64).numpy()
    gk = -torch.rand(T, hv, dk, generator=g, dtype=torch.float64).numpy() * 0.6
    beta = torch.rand(T, hv, generator=g, dtype=torch.float64).numpy()
    init = torch.randn(1, hv, dv, dk, generator=g, dtype=torch.float64).numpy()
    return q, k, v, gk, beta, init


def test_per_key_decay_equal_across_keys_is_scalar_decay():
    q, k, v, gk, beta, init = _pk_inputs(120)
    gs = gk[:, :, 0]
    gk_eq = np.repeat(gs[:, :, None], gk.shape[2], axis=2)
    T = q.shape[0]
    for rule in ("gated_delta", "gated"):
        bet = beta if rule == "gated_delta" else None
        o1, f1 = oracle.prefill(q, k, v, gk_eq, bet, n_seqs=1, seq_len=T, initial_state=init,
                                scale=0.8, update_rule=rule, decay_per_key=True)
        o2, f2 = oracle.prefill(q, k, v, gs, bet, n_seqs=1, seq_len=T, initial_state=init,
                                scale=0.8, update_rule=rule)
        np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(f1, f2, rtol=1e-12, atol=1e-12)


def test_per_key_decay_brute_force_matrices():
    """S_t = (I - beta k k^T) diag(alpha_t) S_{t-1} + beta k v^T with explicit
    dk x dk matrices, y_t = scale S_t^T q_t."""
    q, k, v, gk, beta, init = _pk_inputs(121)
    T, hv = v.shape[0], v.shape[1]
    out, fin = oracle.prefill(q, k, v, gk, beta, n_seqs=1, seq_len=T, initial_state=init,
                              scale=0.5, decay_per_key=True)
    for h in range(hv):
        S = init[0, h].T.copy()
        for t in range(T):
            kt = k[t, 0][:, None]
            M = (np.eye(kt.shape[0]) - beta[t, h] * kt @ kt.T) @ np.diag(np.exp(gk[t, h]))
            S = M @ S + beta[t, h] * kt @ v[t, h][None, :]
            np.testing.assert_allclose(out[t, h], 0.5 * S.T @ q[t, 0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(fin[0, h], S.T, rtol=1e-12, atol=1e-12)


def test_per_key_decay_one_hot_keys_closed_form():
    """One-hot keys e_i: key row i is written, (1 - beta) alpha_i S[i] + beta v;
    every other row only decays by its own factor."""
    g = torch.Generator().manual_seed(122)
    T, dk, dv = 40, 6, 3
    idx = torch.randint(0, dk, (T,), generator=g).numpy()
    k = np.zeros((T, 1, dk))
    k[np.arange(T), 0, idx] = 1.0
    q = torch.randn(T, 1, dk, generator=g, dtype=torch.float64).numpy()
    v = torch.randn(T, 1, dv, generator=g, dtype=torch.float64).numpy()
    gk = -torch.rand(T, 1, dk, generator=g, dtype=torch.float64).numpy()
    beta = torch.rand(T, 1, generator=g, dtype=torch.float64).numpy()
    init = torch.randn(1, 1, dv, dk, generator=g, dtype=torch.float64).numpy()
    out, fin = oracle.prefill(q, k, v, gk, beta, n_seqs=1, seq_len=T, initial_state=init,
                              scale=1.0, decay_per_key=True)
    S = init[0, 0].T.copy()
    for t in range(T):
        a = np.exp(gk[t, 0])
        S = a[:, None] * S
        i = idx[t]
        S[i] = (1.0 - beta[t, 0]) * S[i] + beta[t, 0] * v[t, 0]
        np.testing.assert_allclose(out[t, 0], q[t, 0] @ S, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(fin[0, 0], S.T, rtol=1e-13, atol=1e-13)


def test_per_key_gated_rule_masked_form():
    """gated rule with per-key decay: y_t = (q_t o Gam_t)^T S0 +
    sum_{s<=t} ((q_t o Gam_t / Gam_s) . k_s) v_s with Gam_t the running
    product of the per-key factors (no retrieval term)."""
    q, k, v, gk, beta, init = _pk_inputs(123)
    T, hv = v.shape[0], v.shape[1]
    out, fin = oracle.prefill(q, k, v, gk, None, n_seqs=1, seq_len=T, initial_state=init,
                              scale=1.0, update_rule="gated", decay_per_key=True)
    for h in range(hv):
        G = np.cumsum(gk[:, h], axis=0)          # [T, dk]
        S0 = init[0, h].T                        # [dk, dv]
        for t in range(T):
            y = (q[t, 0] * np.exp(G[t])) @ S0
            for s in range(t + 1):
                y = y + ((q[t, 0] * np.exp(G[t] - G[s])) @ k[s, 0]) * v[s, h]
            np.testing.assert_allclose(out[t, h], y, rtol=1e-11, atol=1e-11)
        S = np.exp(G[-1])[:, None] * S0 + sum(np.outer(k[s, 0] * np.exp(G[-1] - G[s]), v[s, h])
                                              for s in range(T))
        np.testing.assert_allclose(fin[0, h], S.T, rtol=1e-11, atol=1e-11)


def test_per_key_decay_decode_equals_prefill_from_the_slot():
    q, k, v, gk, beta_raw, init = _pk_inputs(124, T=6)
    T, hv, dv, dk = v.shape[0], v.shape[1], v.shape[2], k.shape[2]
    g = torch.Generator().manual_seed(125)
    b = torch.randn(T, hv, generator=g, dtype=torch.float64).numpy()
    beta = 1.0 / (1.0 + np.exp(-b))
    pool = np.concatenate([np.zeros((1, hv, dv, dk)), init])  # slot 1 holds the state
    ro, rp = oracle.decode(q[None], k[None, :, None], v[None, :, None], np.zeros(hv), np.zeros(hv),
                           np.zeros((1, T, hv)), b[None, :, None], pool, np.array([1]),
                           scale=0.7, decay_per_key=gk[None])
    po, pf = oracle.prefill(q, k, v, gk, beta, n_seqs=1, seq_len=T, initial_state=init, scale=0.7,
                            decay_per_key=True)
    np.testing.assert_allclose(ro[0], po, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rp[1], pf[0], rtol=1e-12, atol=1e-12)
