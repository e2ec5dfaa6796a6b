"""GPU checks of rollback from delta checkpoints (gdn_verify_window_delta, then
gdn_commit_delta), through the C ABI.

Each step of the rule is a rank-1 update applied elementwise, S_t = fmaf(c, k_t,
alpha_t S_{t-1}), so storing (c, alpha_t) per window token is an exact, compact form
of the checkpoints the pages publish for rollback (onnxruntime-genai pull request
"Run chained MTP drafting in the batch Engine", section "Correctness fix").  Checked:

* the folded state is bit-identical to checkpoint slot a_r of a checkpointing verify
  of the same window (so to gdn_commit_accepted), for every (T, a) pair and three
  head shapes; verify with delta checkpoints writes the same outputs bit for bit and
  never writes the pool;
* in-place commit, bad accepted counts (row untouched, status bit set), zero source
  state, rows spread over two launches;
* the batch-1 and concurrency-16 workloads run in delta mode against the oracle.
"""
import numpy as np
import pytest

from gateddeltanet_linear_attention_amd import binding as gb
from gateddeltanet_linear_attention_amd import synth
from tests.gpu_common import assert_same_bits, bits, dev_params, dev_tokens, dims_of, say
from tests.test_gpu_recurrent import run_verify_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _pool(n_slots, Hv, d, seed, scale=0.3):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (scale * torch.randn(n_slots, Hv, d, d, generator=g)).cuda()


@pytest.mark.parametrize("raw_qk", [False, True], ids=["given_qk", "fused_l2norm"])
@pytest.mark.parametrize("shape", [synth.FULL, synth.TINY, synth.HeadShape(2, 6, 128)],
                         ids=["h16x32_d128", "h1_d16", "h2x6_d128"])
def test_delta_commit_equals_checkpoint_commit_bitwise(shape, raw_qk):
    """With GDN_QK_L2NORM the fold re-scales each raw key by the factor the verify
    stored, so the bits still agree."""
    dims = dims_of(shape, raw_qk=raw_qk)
    Hv, d = shape.n_v_heads, shape.d
    pairs = [(t, a) for t in range(1, 5) for a in range(t)]
    T = np.array([t for t, _ in pairs], np.int32)
    B = T.size
    g = synth.streams(51, 2)
    A_log, dt_bias = synth.head_params(g[0], shape)
    P = dev_params(A_log, dt_bias)
    td = dev_tokens(synth.tokens(g[1], shape, int(T.sum()), raw_qk=raw_qk))
    acc = torch.tensor([a for _, a in pairs], dtype=torch.int32, device="cuda")
    rows = np.arange(B, dtype=np.int32)
    pool = _pool(3 * B, Hv, d, 11)
    before = pool.clone()
    N = int(T.sum())
    o_ck = torch.empty(N, Hv, d, dtype=torch.bfloat16, device="cuda")
    o_dl = torch.empty_like(o_ck)
    ckpt = torch.empty(B, 4, Hv, d, d, device="cuda")
    delta = torch.empty(gb.delta_shape(dims, B), device="cuda")
    status = torch.zeros((B + 31) // 32, dtype=torch.int32, device="cuda")
    gb.gdn_verify_window(dims, T, **td, **P, state_pool=pool, src_slot=rows, ckpt=ckpt, o=o_ck)
    gb.gdn_commit_accepted(dims, T, ckpt, acc, pool, dst_slot=rows + B, status=status)
    gb.gdn_verify_window_delta(dims, T, **td, **P, state_pool=pool, src_slot=rows, delta=delta, o=o_dl)
    gb.gdn_commit_delta(dims, T, td["k"], delta, acc, pool, src_slot=rows, dst_slot=rows + 2 * B, status=status)
    torch.cuda.synchronize()
    assert int(status.abs().sum()) == 0
    assert_same_bits(o_ck, o_dl, "o_ck vs o_dl")
    assert_same_bits(pool[:B], before[:B], "verify wrote the committed pool")
    for r in range(B):
        assert_same_bits(pool[2 * B + r], pool[B + r],
                         "row %d (T=%d, a=%d): delta fold differs from checkpoint commit" % (r, T[r], pairs[r][1]))


def test_delta_in_place_flags_bad_counts_zero_source_and_spans_launches():
    shape = synth.FULL
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    B = 70
    rng = np.random.default_rng(7)
    T = rng.integers(1, 5, size=B).astype(np.int32)
    g = synth.streams(53, 3)
    A_log, dt_bias = synth.head_params(g[0], shape)
    P = dev_params(A_log, dt_bias)
    td = dev_tokens(synth.tokens(g[1], shape, int(T.sum())))
    acc_np = np.array([g[2].integers(0, t) for t in T], np.int32)
    acc_np[5] = T[5]
    acc_np[67] = -3
    acc = torch.from_numpy(acc_np).cuda()
    src = np.arange(B, dtype=np.int32)
    src[[2, 40]] = -1  # zero source states
    pool = _pool(B, Hv, d, 12, scale=0.1)
    ref = pool.clone()
    ckpt = torch.empty(B, 4, Hv, d, d, device="cuda")
    delta = torch.empty(gb.delta_shape(dims, B), device="cuda")
    o = torch.empty(int(T.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    st_ref = torch.zeros(3, dtype=torch.int32, device="cuda")
    st = torch.zeros(3, dtype=torch.int32, device="cuda")
    gb.gdn_verify_window(dims, T, **td, **P, state_pool=ref, src_slot=src, ckpt=ckpt, o=o)
    gb.gdn_commit_accepted(dims, T, ckpt, acc, ref, dst_slot=np.arange(B), status=st_ref)
    gb.gdn_verify_window_delta(dims, T, **td, **P, state_pool=pool, src_slot=src, delta=delta, o=o)
    gb.gdn_commit_delta(dims, T, td["k"], delta, acc, pool, src_slot=src, dst_slot=np.arange(B), status=st)
    torch.cuda.synchronize()
    expect = [0, 0, 0]
    for r in (5, 67):
        expect[r // 32] |= 1 << (r % 32)
    assert [int(x) & 0xFFFFFFFF for x in st.cpu()] == expect
    assert torch.equal(st, st_ref)
    assert_same_bits(pool, ref, "delta fold differs from checkpoint commit")


def test_batch1_workload_in_delta_mode():
    w = synth.verify_workload("batch1", n_windows=64)
    say("batch1 delta worst:", run_verify_workload(w, n_windows=w.n_windows, check_every=16, mode="delta"))


def test_conc16_workload_in_delta_mode():
    w = synth.verify_workload("conc16", n_windows=128)
    say("conc16 delta worst:", run_verify_workload(w, n_windows=w.n_windows, check_every=32, mode="delta"))


# ---------------------------------------------------------------- fold into the next verify

@pytest.mark.parametrize("raw_qk", [False, True], ids=["given_qk", "fused_l2norm"])
def test_folded_verify_equals_commit_then_verify_bitwise(raw_qk):
    """gdn_verify_window_delta_fold == gdn_commit_delta(previous window) followed by
    gdn_verify_window_delta (new window), bit for bit: pool, outputs and factors;
    a row with a bad previous accepted count is left untouched and flagged."""
    shape = synth.FULL
    dims = dims_of(shape, raw_qk=raw_qk)
    Hv, d = shape.n_v_heads, shape.d
    B = 6
    T1 = np.array([4, 3, 2, 4, 1, 4], np.int32)
    T2 = np.array([2, 4, 4, 1, 3, 4], np.int32)
    g = synth.streams(55, 4)
    A_log, dt_bias = synth.head_params(g[0], shape)
    P = dev_params(A_log, dt_bias)
    w1 = dev_tokens(synth.tokens(g[1], shape, int(T1.sum()), raw_qk=raw_qk))
    w2 = dev_tokens(synth.tokens(g[2], shape, int(T2.sum()), raw_qk=raw_qk))
    acc_np = np.array([g[3].integers(0, t) for t in T1], np.int32)
    acc_np[4] = 1  # out of range for a 1-token window: row 4 must stay untouched
    acc = torch.from_numpy(acc_np).cuda()
    rows = np.arange(B, dtype=np.int32)
    base = _pool(B, Hv, d, 13, scale=0.1)
    d1 = torch.empty(gb.delta_shape(dims, B), device="cuda")
    o1 = torch.empty(int(T1.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    gb.gdn_verify_window_delta(dims, T1, **w1, **P, state_pool=base, src_slot=rows, delta=d1, o=o1)
    # reference: commit, then verify (two launches)
    ref = base.clone()
    st_ref = torch.zeros(1, dtype=torch.int32, device="cuda")
    gb.gdn_commit_delta(dims, T1, w1["k"], d1, acc, ref, src_slot=rows, dst_slot=rows, status=st_ref)
    d2_ref = torch.zeros(gb.delta_shape(dims, B), device="cuda")
    o2_ref = torch.zeros(int(T2.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    gb.gdn_verify_window_delta(dims, T2, **w2, **P, state_pool=ref, src_slot=rows, delta=d2_ref, o=o2_ref)
    # folded: one launch
    pool = base.clone()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    d2 = torch.zeros(gb.delta_shape(dims, B), device="cuda")
    o2 = torch.zeros(int(T2.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    gb.gdn_verify_window_delta_fold(dims, T2, **w2, **P, state_pool=pool, slot=rows, delta=d2, o=o2,
                                    prev_row_tokens=T1, prev_k=w1["k"], prev_delta=d1, prev_accepted=acc, status=st)
    torch.cuda.synchronize()
    assert int(st[0]) == 1 << 4 and int(st_ref[0]) == 1 << 4
    cu2 = np.concatenate([[0], np.cumsum(T2)])
    for r in range(B):
        if r == 4:
            assert_same_bits(pool[r], base[r], "flagged row was folded")
            assert not bool(o2[cu2[r]:cu2[r + 1]].view(torch.int16).any()), "flagged row wrote outputs"
            continue
        assert_same_bits(pool[r], ref[r], "row %d: folded state differs" % r)
        assert_same_bits(o2[cu2[r]:cu2[r + 1]], o2_ref[cu2[r]:cu2[r + 1]], "row %d: folded verify outputs" % r)
        assert_same_bits(d2[r, :T2[r]], d2_ref[r, :T2[r]], "row %d: factors differ" % r)


def test_conc16_workload_with_folded_verify():
    """The concurrency-16 chain of windows where each verify commits the previous
    window itself; the pool is checked against the oracle's committed states."""
    import oracle
    from tests.gpu_common import assert_o, assert_state, host, index_tokens
    w = synth.verify_workload("conc16", n_windows=48)
    dims = dims_of(w.shape)
    B, Hv, d = w.n_rows, w.shape.n_v_heads, w.shape.d
    P = dev_params(w.A_log, w.dt_bias)
    rows = np.arange(B, dtype=np.int32)
    warm = w.warm_tokens()
    wt = dev_tokens(warm)
    cu = np.concatenate([[0], np.cumsum(w.warm_lens)]).astype(np.int64)
    pool = torch.zeros(B, Hv, d, d, device="cuda")
    for t in range(int(w.warm_lens.max())):
        act = rows[w.warm_lens > t]
        o_step = torch.empty(len(act), Hv, d, dtype=torch.bfloat16, device="cuda")
        src = act if t > 0 else np.full(len(act), -1, np.int32)
        gb.gdn_decode_step(dims, **index_tokens(wt, cu[act] + t), **P, state_pool=pool, src_slot=src,
                           dst_slot=act, o=o_step)
    S_ref, _, _ = oracle.run_sequential(w.warm_lens, warm.q, warm.k, warm.v, warm.a, warm.b, w.A_log, w.dt_bias)
    T = w.window_lens
    deltas = [torch.empty(gb.delta_shape(dims, B), device="cuda") for _ in range(2)]
    o_win = torch.empty(int(T.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    prev = None
    S_prev_committed = S_ref
    for i in range(w.n_windows):
        win, acc = w.window_tokens(i), w.accepted(i)
        wd = dev_tokens(win)
        dl = deltas[i % 2]
        if prev is None:
            gb.gdn_verify_window_delta(dims, T, **wd, **P, state_pool=pool, src_slot=rows, delta=dl, o=o_win)
        else:
            gb.gdn_verify_window_delta_fold(dims, T, **wd, **P, state_pool=pool, slot=rows, delta=dl, o=o_win,
                                            prev_row_tokens=T, prev_k=prev[0], prev_delta=prev[1],
                                            prev_accepted=prev[2], status=status)
        ck_o, o_o = oracle.verify_window(T, win.q, win.k, win.v, win.a, win.b, w.A_log, w.dt_bias, S_prev_committed)
        assert_o(host(o_win), o_o, "folded-verify window %d outputs" % i)
        if i % 16 == 15:  # the pool holds the state committed after window i - 1
            assert_state(host(pool), S_prev_committed, "committed state before window %d" % i)
        S_prev_committed = np.stack([ck_o[r, acc[r]] for r in range(B)])
        prev = (wd["k"], dl, torch.from_numpy(acc).cuda())
    gb.gdn_commit_delta(dims, T, prev[0], prev[1], prev[2], pool, src_slot=rows, dst_slot=rows, status=status)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    assert_state(host(pool), S_prev_committed, "final committed state")
