"""Pins of the fp64 oracle against things other than itself.

Each test fixes some part of the oracle by a closed form, a hand-evaluated
example, a special case that reduces to a library routine, brute force with
explicit transition matrices, or an invariant of the mathematics, chosen so that
a dropped term, a wrong sign, a wrong index or a transposed operand anywhere in
the oracle fails at least one of them.  The rule itself is the gated delta rule
(Yang, Kautz & Hatamizadeh, ICLR 2025); checkpoint / rollback semantics follow the
onnxruntime-genai pull request "Run chained MTP drafting in the batch Engine",
section "Correctness fix".
"""
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from gateddeltanet_linear_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def rand_case(seed, L, Hqk=1, Hv=1, dk=16, dv=16, gate_shift=0.0, s0_scale=1.0):
    """Random fp64 inputs (not bf16 rounded: the oracle is exact in any case)."""
    rng = np.random.default_rng(seed)
    N = int(np.sum(L))
    q = rng.standard_normal((N, Hqk, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True) * np.sqrt(dk)
    k = rng.standard_normal((N, Hqk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, Hv, dv))
    a = rng.standard_normal((N, Hv)) + gate_shift
    b = rng.standard_normal((N, Hv))
    A_log = rng.uniform(0.0, np.log(16.0), Hv)
    dt_bias = 0.1 * rng.standard_normal(Hv)
    S0 = s0_scale * rng.standard_normal((len(L), Hv, dv, dk))
    return dict(q=q, k=k, v=v, a=a, b=b, A_log=A_log, dt_bias=dt_bias, S0=S0)


def lib_gates(a, b, A_log, dt_bias):
    """Gates through library routines: softplus = logaddexp(0, x), sigmoid = expit."""
    alpha = np.exp(-np.exp(A_log) * np.logaddexp(0.0, a + dt_bias))
    return alpha, expit(b)


def brute_force_unit(S0, q, k, v, alpha, beta):
    """States and outputs of one (row, head) by explicit d_k x d_k transition matrices:
    S_t = S_0 M_1 ... M_t + sum_{s<=t} beta_s v_s k_s^T M_{s+1} ... M_t,
    M_s = alpha_s (I - beta_s k_s k_s^T).  Returns (states [T][dv][dk], o [T][dv])."""
    T, dk = k.shape
    I = np.eye(dk)
    M = [alpha[s] * (I - beta[s] * np.outer(k[s], k[s])) for s in range(T)]
    states, outs = [], []
    for t in range(T):
        P = I.copy()
        for s in range(t + 1):
            P = P @ M[s]
        St = S0 @ P
        for s in range(t + 1):
            tail = I.copy()
            for m in range(s + 1, t + 1):
                tail = tail @ M[m]
            St = St + beta[s] * np.outer(v[s], k[s]) @ tail
        states.append(St)
        outs.append(St @ q[t])
    return np.array(states), np.array(outs)


def rel(x, ref):
    return np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300)


# ---------------------------------------------------------------- gates

def test_gate_special_points():
    # A_log = 0 and a + dt_bias = 0: softplus(0) = ln 2, so alpha = exp(-ln 2) = 1/2
    al, be = oracle.gates([0.0, 0.25], [0.0, 0.0], 0.0, -np.array(0.0))
    assert abs(al[0] - 0.5) < 1e-15 and abs(be[0] - 0.5) < 1e-15
    # very negative logit: softplus -> 0, alpha -> 1 (no decay); b -> -inf: beta -> 0
    al, be = oracle.gates([-1000.0], [-1000.0], np.log(8.0), 0.3)
    assert al[0] == 1.0 and be[0] == 0.0
    # b -> +inf: beta -> 1; large positive logit: softplus(x) ~ x
    al, be = oracle.gates([30.0], [1000.0], np.log(2.0), 0.0)
    assert be[0] == 1.0
    assert abs(np.log(al[0]) - (-2.0 * 30.0)) < 1e-9
    # sigmoid symmetry beta(b) + beta(-b) = 1
    bs = np.linspace(-20, 20, 41)
    _, b1 = oracle.gates(np.zeros_like(bs), bs, 0.0, 0.0)
    _, b2 = oracle.gates(np.zeros_like(bs), -bs, 0.0, 0.0)
    assert np.max(np.abs(b1 + b2 - 1.0)) < 1e-15


def test_gates_match_library_routines():
    rng = np.random.default_rng(1)
    for A_log, dt in [(0.0, 0.0), (np.log(16.0), -0.2), (1.3, 0.05)]:
        a = np.concatenate([rng.standard_normal(200), [-60, -30, -5, 5, 30, 60]])
        b = np.concatenate([rng.standard_normal(200), [-60, -30, -5, 5, 30, 60]])
        al, be = oracle.gates(a, b, A_log, dt)
        al_ref, be_ref = lib_gates(a, b, A_log, dt)
        assert np.max(np.abs(al - al_ref) / np.maximum(al_ref, 1e-300)) < 1e-12
        assert np.max(np.abs(be - be_ref) / be_ref) < 1e-14


# ---------------------------------------------------------------- worked examples

def test_hand_worked_2x2_example():
    rows = []
    with open(os.path.join(GOLDEN, "hand_2x2.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append([float(x) for x in line.replace("|", " ").split()])
    g = np.array(rows)
    T = g.shape[0]
    a, b = g[:, 0:1], g[:, 1:2]
    k, v, q = g[:, 2:4], g[:, 4:6], g[:, 6:8]
    o_exp, S_exp = g[:, 8:10], g[:, 10:14].reshape(T, 2, 2)
    S_fin, ckpt, o = oracle.run_sequential(
        [T], q[:, None, :], k[:, None, :], v[:, None, :], a, b, [0.0], [0.0],
        n_tail=[T], n_slot=T)
    assert np.max(np.abs(o[:, 0, :] - o_exp)) < 1e-12
    assert np.max(np.abs(ckpt[0, :, 0] - S_exp)) < 1e-12
    assert np.max(np.abs(S_fin[0, 0] - S_exp[-1])) < 1e-12


def test_scalar_closed_form():
    # d = 1, k = q = v = 1, alpha = beta = 1/2: S_t = S_{t-1}/4 + 1/2 = (2/3)(1 - 4^-t)
    T = 12
    one = np.ones((T, 1, 1))
    _, ckpt, o = oracle.run_sequential([T], one, one, one, np.zeros((T, 1)), np.zeros((T, 1)),
                                       [0.0], [0.0], n_tail=[T], n_slot=T)
    t = np.arange(1, T + 1)
    exp = (2.0 / 3.0) * (1.0 - 0.25 ** t)
    assert np.max(np.abs(o[:, 0, 0] - exp)) < 1e-15
    assert np.max(np.abs(ckpt[0, :, 0, 0, 0] - exp)) < 1e-15


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("Hqk,Hv,dk,dv,L", [
    (1, 1, 16, 16, [12]),          # the tiny single-head shape
    (2, 4, 16, 8, [5, 1, 9]),      # d_k != d_v catches a transposed operand; ragged rows
    (1, 3, 6, 10, [4, 7]),         # three v-heads share one qk-head
])
def test_brute_force_transition_matrices(Hqk, Hv, dk, dv, L):
    c = rand_case(7 + dk + Hv, L, Hqk, Hv, dk, dv)
    n_tail = [min(x, 3) for x in L]
    S_fin, ckpt, o = oracle.run_sequential(L, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                                           c["dt_bias"], c["S0"], n_tail=n_tail, n_slot=4)
    cu = np.concatenate([[0], np.cumsum(L)])
    group = Hv // Hqk
    for r in range(len(L)):
        sl = slice(cu[r], cu[r + 1])
        for h in range(Hv):
            hq = h // group
            alpha, beta = lib_gates(c["a"][sl, h], c["b"][sl, h], c["A_log"][h], c["dt_bias"][h])
            states, outs = brute_force_unit(c["S0"][r, h], c["q"][sl, hq], c["k"][sl, hq],
                                            c["v"][sl, h], alpha, beta)
            assert rel(S_fin[r, h], states[-1]) < 1e-12
            assert np.max(np.abs(o[sl, h] - outs)) < 1e-12 * max(1.0, np.abs(outs).max())
            for j in range(n_tail[r]):
                assert rel(ckpt[r, j, h], states[L[r] - n_tail[r] + j]) < 1e-12
            for j in range(n_tail[r], 4):
                assert np.all(np.isnan(ckpt[r, j, h])), "unrequested checkpoint slot was written"


# ---------------------------------------------------------------- special cases / invariants

def test_beta_zero_is_pure_decay():
    L = [6]
    c = rand_case(3, L)
    c["b"][:] = -1000.0  # beta = 0 exactly
    S_fin, _, o = oracle.run_sequential(L, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                                        c["dt_bias"], c["S0"])
    alpha, _ = lib_gates(c["a"][:, 0], c["b"][:, 0], c["A_log"][0], c["dt_bias"][0])
    assert rel(S_fin[0, 0], np.prod(alpha) * c["S0"][0, 0]) < 1e-13
    assert rel(o[0, 0], alpha[0] * c["S0"][0, 0] @ c["q"][0, 0]) < 1e-13


def test_beta_one_overwrites_the_key_slot():
    # beta = 1, unit key: whatever alpha and history, S_t k_t = v_t
    L = [9]
    c = rand_case(4, L, s0_scale=3.0)
    c["b"][:] = 1000.0
    _, ckpt, _ = oracle.run_sequential(L, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                                       c["dt_bias"], c["S0"], n_tail=L, n_slot=9)
    for t in range(9):
        assert np.max(np.abs(ckpt[0, t, 0] @ c["k"][t, 0] - c["v"][t, 0])) < 1e-12


def test_orthonormal_keys_store_and_recall():
    # no decay (alpha = 1), beta = 1, keys e_0..e_{d-1}: S = sum_i v_i e_i^T, and q = e_j recalls v_j
    d = 8
    L = [d]
    k = np.eye(d)[:, None, :]
    rng = np.random.default_rng(5)
    v = rng.standard_normal((d, 1, d))
    q = np.roll(np.eye(d), 1, axis=0)[:, None, :]  # token t queries key t-1 (t=0 queries e_{d-1}, not yet stored)
    a = np.full((d, 1), -1000.0)
    b = np.full((d, 1), 1000.0)
    S_fin, _, o = oracle.run_sequential(L, q, k, v, a, b, [0.0], [0.0])
    assert np.max(np.abs(S_fin[0, 0] - v[:, 0, :].T)) < 1e-15
    assert np.max(np.abs(o[0, 0])) < 1e-15
    for t in range(1, d):
        assert np.max(np.abs(o[t, 0] - v[t - 1, 0])) < 1e-15


def test_frobenius_norm_bound():
    # for unit k and beta in [0,1], I - beta k k^T has spectral norm <= 1, so
    # ||S_t||_F <= alpha_t ||S_{t-1}||_F + beta_t ||v_t||
    L = [20]
    c = rand_case(6, L, gate_shift=-3.0)
    _, ckpt, _ = oracle.run_sequential(L, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                                       c["dt_bias"], c["S0"], n_tail=L, n_slot=20)
    alpha, beta = lib_gates(c["a"][:, 0], c["b"][:, 0], c["A_log"][0], c["dt_bias"][0])
    prev = np.linalg.norm(c["S0"][0, 0])
    for t in range(20):
        cur = np.linalg.norm(ckpt[0, t, 0])
        assert cur <= alpha[t] * prev + beta[t] * np.linalg.norm(c["v"][t, 0]) + 1e-12
        prev = cur


def test_value_channel_permutation_equivariance():
    L = [7]
    c = rand_case(8, L, dk=6, dv=9)
    perm = np.random.default_rng(0).permutation(9)
    base = oracle.run_sequential(L, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                                 c["dt_bias"], c["S0"])
    permd = oracle.run_sequential(L, c["q"], c["k"], c["v"][:, :, perm], c["a"], c["b"], c["A_log"],
                                  c["dt_bias"], c["S0"][:, :, perm, :])
    assert np.array_equal(base[0][:, :, perm, :], permd[0])
    assert np.array_equal(base[2][:, :, perm], permd[2])


def test_homogeneity_in_state_and_values():
    L = [10]
    c = rand_case(9, L)
    base = oracle.run_sequential(L, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                                 c["dt_bias"], c["S0"])
    scaled = oracle.run_sequential(L, c["q"], c["k"], 4.0 * c["v"], c["a"], c["b"], c["A_log"],
                                   c["dt_bias"], 4.0 * c["S0"])
    assert rel(scaled[0], 4.0 * base[0]) < 1e-14
    assert rel(scaled[2], 4.0 * base[2]) < 1e-14


def test_rows_and_heads_are_independent():
    L = [3, 8, 1, 5]
    c = rand_case(10, L, Hqk=2, Hv=4, dk=8, dv=8)
    S_fin, ckpt, o = oracle.run_sequential(L, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                                           c["dt_bias"], c["S0"], n_tail=[1, 4, 1, 2], n_slot=4)
    cu = np.concatenate([[0], np.cumsum(L)])
    for r in range(len(L)):
        sl = slice(cu[r], cu[r + 1])
        s1, k1, o1 = oracle.run_sequential([L[r]], c["q"][sl], c["k"][sl], c["v"][sl], c["a"][sl],
                                           c["b"][sl], c["A_log"], c["dt_bias"], c["S0"][r:r + 1],
                                           n_tail=[[1, 4, 1, 2][r]], n_slot=4)
        assert np.array_equal(s1[0], S_fin[r])
        assert np.array_equal(o1, o[sl])
        assert np.array_equal(np.nan_to_num(k1[0], nan=7.0), np.nan_to_num(ckpt[r], nan=7.0))


def test_thread_count_does_not_change_bits():
    L = [4, 9, 2]
    c = rand_case(11, L, Hqk=2, Hv=4, dk=16, dv=16)
    r1 = oracle.run_sequential(L, **{k: c[k] for k in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "S0")},
                               n_tail=[2, 2, 2], n_slot=2, n_threads=1)
    r4 = oracle.run_sequential(L, **{k: c[k] for k in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "S0")},
                               n_tail=[2, 2, 2], n_slot=2, n_threads=4)
    for x, y in zip(r1, r4):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------- chunked form

@pytest.mark.parametrize("chunk", [1, 3, 8, 64])
@pytest.mark.parametrize("gate_shift", [0.0, -8.0])
def test_chunked_form_equals_sequential(chunk, gate_shift):
    L = [1, 5, 64, 65, 130]
    n_tail = [1, 4, 4, 2, 4]  # tails of 65 (with chunk 64) straddle the chunk boundary
    c = rand_case(12, L, Hqk=1, Hv=2, dk=12, dv=10, gate_shift=gate_shift)
    seq = oracle.run_sequential(L, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"], c["dt_bias"],
                                c["S0"], n_tail=n_tail, n_slot=4)
    chk = oracle.run_chunked(L, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"], c["dt_bias"],
                             c["S0"], n_tail=n_tail, n_slot=4, chunk=chunk)
    assert rel(chk[0], seq[0]) < 1e-12
    assert np.max(np.abs(chk[2] - seq[2])) < 1e-12 * max(1.0, np.abs(seq[2]).max())
    for r in range(len(L)):
        for j in range(n_tail[r]):
            assert rel(chk[1][r, j], seq[1][r, j]) < 1e-12
        assert np.all(np.isnan(chk[1][r, n_tail[r]:]))


def test_chunked_form_at_full_head_width():
    L = [130]
    c = rand_case(13, L, Hqk=1, Hv=2, dk=128, dv=128)
    seq = oracle.run_sequential(L, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"], c["dt_bias"],
                                c["S0"], n_tail=[4], n_slot=4)
    chk = oracle.run_chunked(L, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"], c["dt_bias"],
                             c["S0"], n_tail=[4], n_slot=4, chunk=64)
    assert rel(chk[0], seq[0]) < 1e-12
    assert rel(chk[1], seq[1]) < 1e-12
    assert rel(chk[2], seq[2]) < 1e-12


# ---------------------------------------------------------------- checkpoints, verify, commit

def test_checkpoint_i_is_the_state_after_i_steps():
    L = [7]
    c = rand_case(14, L, Hqk=1, Hv=2, dk=8, dv=8)
    _, ckpt, _ = oracle.run_sequential(L, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                                       c["dt_bias"], c["S0"], n_tail=L, n_slot=7)
    for i in range(1, 8):
        sl = slice(0, i)
        S_i, _, _ = oracle.run_sequential([i], c["q"][sl], c["k"][sl], c["v"][sl], c["a"][sl],
                                          c["b"][sl], c["A_log"], c["dt_bias"], c["S0"])
        assert np.array_equal(ckpt[0, i - 1], S_i[0])


@pytest.mark.parametrize("accepted", [0, 1, 2, 3])
def test_commit_then_continue_equals_accepted_prefix(accepted):
    """Rollback leaves no trace: after a K=3 window and commit(a), decoding on gives the
    same as running the previous bonus token, the a accepted drafts and then the next
    tokens, with the rejected drafts never seen."""
    shape = synth.HeadShape(2, 4, 16)
    g = synth.streams(99, 2)
    A_log, dt_bias = synth.head_params(g[0], shape)
    win = synth.tokens(g[1], shape, 4)
    nxt = synth.tokens(g[1], shape, 3)
    S0 = np.random.default_rng(1).standard_normal((1, 4, 16, 16))
    ckpt, o = oracle.verify_window([4], win.q, win.k, win.v, win.a, win.b, A_log, dt_bias, S0)
    S_c = oracle.commit(ckpt, [4], [accepted])
    S_after, _, o_after = oracle.run_sequential([3], nxt.q, nxt.k, nxt.v, nxt.a, nxt.b, A_log,
                                                dt_bias, S_c)
    keep = win.slice(0, accepted + 1)
    ref = synth.Tokens.concat([keep, nxt])
    S_ref, _, o_ref = oracle.run_sequential([ref.n], ref.q, ref.k, ref.v, ref.a, ref.b, A_log,
                                            dt_bias, S0)
    assert rel(S_after, S_ref) < 1e-13
    assert np.max(np.abs(o_after - o_ref[accepted + 1:])) < 1e-13
    # the window's outputs for the kept tokens are those of the prefix run
    assert np.max(np.abs(o[:accepted + 1] - o_ref[:accepted + 1])) < 1e-15


def test_commit_rejects_out_of_range():
    ckpt = np.zeros((1, 4, 1, 2, 2))
    with pytest.raises(ValueError):
        oracle.commit(ckpt, [2], [2])
    with pytest.raises(ValueError):
        oracle.commit(ckpt, [4], [-1])


def test_oracle_rejects_bad_arguments():
    c = rand_case(15, [3])
    with pytest.raises(ValueError):  # n_tail larger than the row
        oracle.run_sequential([3], c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"], c["dt_bias"],
                              c["S0"], n_tail=[4], n_slot=4)


# ---------------------------------------------------------------- token trees

TREES = [[-1, 0, 0, 1], [-1, -1, 1, 0], [-1, 0, 1, 2], [-1, -1, -1, -1], [-1, 0, 0], [-1]]


def test_tree_nodes_match_brute_force_on_their_paths():
    """Node states and outputs against the explicit transition-matrix evaluation of
    each node's root path, on grouped heads with d_k != d_v."""
    Hqk, Hv, dk, dv = 1, 2, 6, 5
    T = [len(p) for p in TREES]
    parents = np.concatenate([np.array(p) for p in TREES])
    c = rand_case(91, T, Hqk, Hv, dk, dv)
    ckpt, o = oracle.verify_tree(T, parents, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                                 c["dt_bias"], c["S0"])
    cu = np.concatenate([[0], np.cumsum(T)])
    for r, par in enumerate(TREES):
        for t in range(len(par)):
            path, x = [], t
            while x >= 0:
                path.append(x)
                x = par[x]
            idx = cu[r] + np.array(path[::-1])
            for h in range(Hv):
                alpha, beta = lib_gates(c["a"][idx, h], c["b"][idx, h], c["A_log"][h], c["dt_bias"][h])
                states, outs = brute_force_unit(c["S0"][r, h], c["q"][idx, 0], c["k"][idx, 0], c["v"][idx, h],
                                                alpha, beta)
                assert rel(ckpt[r, t, h], states[-1]) < 1e-12
                assert np.max(np.abs(o[cu[r] + t, h] - outs[-1])) < 1e-12 * max(1.0, np.abs(outs).max())
        assert np.all(np.isnan(ckpt[r, len(par):]))


def test_chain_tree_is_the_verify_window():
    T = [4, 2, 3]
    parents = np.concatenate([np.arange(t) - 1 for t in T])
    c = rand_case(92, T, 2, 4, 16, 16)
    ck_t, o_t = oracle.verify_tree(T, parents, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                                   c["dt_bias"], c["S0"])
    ck_w, o_w = oracle.verify_window(T, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"], c["dt_bias"], c["S0"])
    for r, t in enumerate(T):
        assert np.array_equal(ck_t[r, :t], ck_w[r, :t])
    assert np.array_equal(o_t, o_w)


def test_star_tree_is_independent_single_steps():
    T = [4]
    c = rand_case(93, T, 1, 2, 8, 8)
    ck, o = oracle.verify_tree(T, [-1, -1, -1, -1], c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                               c["dt_bias"], c["S0"])
    for t in range(4):
        S1, o1 = oracle.decode_step(c["q"][t:t + 1], c["k"][t:t + 1], c["v"][t:t + 1], c["a"][t:t + 1],
                                    c["b"][t:t + 1], c["A_log"], c["dt_bias"], c["S0"])
        assert np.array_equal(ck[0, t], S1[0]) and np.array_equal(o[t], o1[0])


def test_tree_rejects_bad_parents():
    c = rand_case(94, [3], 1, 1, 4, 4)
    for bad in ([0, 0, 1], [-1, 1, 0], [-1, 0, 2], [-1, -2, 0]):
        with pytest.raises(ValueError):
            oracle.verify_tree([3], bad, c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"], c["dt_bias"], c["S0"])


# ------------------------------------------------------------ fused input normalisation

def test_l2norm_hand_example():
    """Pythagorean vectors, worked by hand: |(3, 4, 0, 0)| = 5 and |(1, 2, 2, 0)| = 3,
    d = 4 so the query scale is 1/2.  The eps under the root moves the results by
    less than eps / (2 |x|^2) relative."""
    q = np.array([[[1.0, 2.0, 2.0, 0.0]]])
    k = np.array([[[3.0, 4.0, 0.0, 0.0]]])
    qh, kh = oracle.l2norm_qk(q, k)
    np.testing.assert_allclose(kh[0, 0], [0.6, 0.8, 0.0, 0.0], rtol=1e-7, atol=0)
    np.testing.assert_allclose(qh[0, 0], [1 / 6, 1 / 3, 1 / 3, 0.0], rtol=1e-7, atol=0)


def test_l2norm_unit_vectors_per_token_and_head():
    """Every (token, head) vector of k_hat has norm 1 and of q_hat norm d^-1/2, each
    pointing the way its input does (a normalisation over the wrong axis, a missing or
    misplaced 1/sqrt(d) or a sign slip fails here)."""
    g = np.random.default_rng(7)
    d = 128
    q = g.standard_normal((5, 3, d)) * g.uniform(0.1, 10.0, (5, 3, 1))
    k = g.standard_normal((5, 3, d)) * g.uniform(0.1, 10.0, (5, 3, 1))
    qh, kh = oracle.l2norm_qk(q, k)
    np.testing.assert_allclose(np.linalg.norm(kh, axis=-1), 1.0, rtol=1e-6)
    np.testing.assert_allclose(np.linalg.norm(qh, axis=-1), d ** -0.5, rtol=1e-6)
    assert np.all((kh * k).sum(-1) > 0) and np.all((qh * q).sum(-1) > 0)
    # parallel to the input: the cross terms vanish
    np.testing.assert_allclose(kh * np.linalg.norm(k, axis=-1, keepdims=True), k, rtol=1e-6, atol=1e-12)


def test_l2norm_zero_vector_stays_zero():
    qh, kh = oracle.l2norm_qk(np.zeros((1, 1, 16)), np.zeros((1, 1, 16)))
    assert np.all(qh == 0) and np.all(kh == 0)


def test_rule_on_normalised_inputs_ignores_input_scale():
    """With the normalisation in front, scaling the raw q and k by any positive
    factor leaves states and outputs unchanged (up to eps / |x|^2)."""
    shape = synth.HeadShape(2, 4, 16)
    g = synth.streams(31, 2)
    A_log, dt_bias = synth.head_params(g[0], shape)
    tok = synth.tokens(g[1], shape, 12, raw_qk=True)
    outs = []
    for c in (1.0, 8.0):
        qh, kh = oracle.l2norm_qk(c * tok.q.astype(np.float64), c * tok.k.astype(np.float64))
        S, _, o = oracle.run_sequential(np.array([12]), qh, kh, tok.v, tok.a, tok.b, A_log, dt_bias)
        outs.append((S, o))
    np.testing.assert_allclose(outs[1][0], outs[0][0], rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(outs[1][1], outs[0][1], rtol=1e-6, atol=1e-9)


def test_raw_tokens_share_the_stream_layout():
    """raw_qk draws the same number of values as the normalised recipe, so v and the
    gate logits of a workload are the same in both modes."""
    shape = synth.FULL
    t0 = synth.tokens(np.random.default_rng(3), shape, 5)
    t1 = synth.tokens(np.random.default_rng(3), shape, 5, raw_qk=True)
    assert np.array_equal(t0.v, t1.v) and np.array_equal(t0.a, t1.a) and np.array_equal(t0.b, t1.b)
    np.testing.assert_allclose(np.linalg.norm(t0.k.astype(np.float64), axis=-1), 1.0, rtol=1e-2)
    assert np.linalg.norm(t1.k.astype(np.float64), axis=-1).mean() > 5
