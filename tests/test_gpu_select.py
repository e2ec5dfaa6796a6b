"""GPU checks of rollback by checkpoint select (gdn_verify_window_select, then
gdn_commit_select), through the C ABI.

The checkpoints are written into the state pool (two banks of k_max + 1 slots per
row, used alternately) and the commit only updates a device slot table, so the state
after the accepted prefix becomes the committed state where it is.  Checked:

* window after window, the selected slot holds bit for bit the state that
  gdn_commit_accepted copies, and the outputs equal the checkpoint path's, with
  q/k given or normalised in the kernels;
* a source slot inside a bank of the call, or outside the pool, leaves the row
  untouched and sets its status bit; a bad accepted count leaves the table entry;
* the batch-1 and concurrency-16 workloads in select mode against the oracle, with the
  commit its own launch and with it inside the next window's verify;
* the commit inside the verify against the two separate calls, bit for bit.
"""
import numpy as np
import pytest

from gateddeltanet_linear_attention_amd import binding as gb
from gateddeltanet_linear_attention_amd import synth
from tests.gpu_common import assert_same_bits, bits, dev_params, dev_tokens, dims_of, say
from tests.test_gpu_recurrent import run_verify_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

POISON = 0x7FC0DEAD


@pytest.mark.parametrize("B", [6, 20], ids=["rows6_one_row_per_lane", "rows20_two_rows_per_lane"])
@pytest.mark.parametrize("raw_qk", [False, True], ids=["given_qk", "fused_l2norm"])
def test_select_equals_checkpoint_commit_window_after_window(raw_qk, B):
    shape = synth.FULL
    dims = dims_of(shape, raw_qk=raw_qk)
    Hv, d = shape.n_v_heads, shape.d
    n_windows = 5
    g = synth.streams(101, 2 + 2 * n_windows)
    A_log, dt_bias = synth.head_params(g[0], shape)
    P = dev_params(A_log, dt_bias)
    rows = np.arange(B, dtype=np.int32)
    gen = torch.Generator(device="cpu").manual_seed(101)
    start = (0.2 * torch.randn(B, Hv, d, d, generator=gen)).cuda()
    dense = start.clone()
    sel = torch.zeros(9 * B, Hv, d, d, device="cuda")
    sel[8 * B:] = start
    table = torch.arange(8 * B, 9 * B, dtype=torch.int32, device="cuda")
    ckpt = torch.empty(B, 4, Hv, d, d, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i in range(n_windows):
        T = g[1].integers(1, 5, size=B).astype(np.int32)
        tok = dev_tokens(synth.tokens(g[2 + i], shape, int(T.sum()), raw_qk=raw_qk))
        acc = torch.from_numpy(np.array([g[2 + n_windows + i].integers(0, t) for t in T], np.int32)).cuda()
        o_d = torch.zeros(int(T.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
        o_s = torch.zeros_like(o_d)
        gb.gdn_verify_window(dims, T, **tok, **P, state_pool=dense, src_slot=rows, ckpt=ckpt, o=o_d)
        gb.gdn_commit_accepted(dims, T, ckpt, acc, dense, dst_slot=rows, status=st)
        bank = 2 * rows + (i % 2)
        gb.gdn_verify_window_select(dims, T, **tok, **P, state_pool=sel, slot_table=table, bank=bank, o=o_s,
                                    status=st)
        gb.gdn_commit_select(dims, T, acc, bank, sel, table, st)
        torch.cuda.synchronize()
        assert int(st[0]) == 0
        assert_same_bits(o_s, o_d, "window %d: outputs differ" % i)
        expect = (bank * 4 + acc.cpu().numpy()).astype(np.int32)
        assert np.array_equal(table.cpu().numpy(), expect), "window %d: slot table" % i
        assert_same_bits(sel[table.long()], dense, "window %d: selected states differ" % i)
    say("select == checkpoint commit over %d windows" % n_windows)


def test_select_refuses_sources_inside_banks_and_bad_accepted_counts():
    shape = synth.HeadShape(2, 4, 128)
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    B = 4
    T = np.array([4, 3, 2, 4], np.int32)
    g = synth.streams(103, 2)
    A_log, dt_bias = synth.head_params(g[0], shape)
    P = dev_params(A_log, dt_bias)
    tok = dev_tokens(synth.tokens(g[1], shape, int(T.sum())))
    pool = torch.empty(8 * B + 1, Hv, d, d, device="cuda")
    pool.view(torch.int32).fill_(POISON)
    gen = torch.Generator(device="cpu").manual_seed(3)
    pool[8 * B] = 0.1 * torch.randn(Hv, d, d, generator=gen).cuda()
    bank = np.array([0, 2, 4, 6], np.int32)
    # row 1 starts inside row 2's bank, row 3 outside the pool; rows 0 and 2 are fine
    table = torch.tensor([8 * B, 4 * 4 + 1, 8 * B, 9 * B], dtype=torch.int32, device="cuda")
    before = pool.clone()
    o = torch.empty(int(T.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    o.view(torch.int16).fill_(0x7FC1)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    gb.gdn_verify_window_select(dims, T, **tok, **P, state_pool=pool, slot_table=table, bank=bank, o=o, status=st)
    torch.cuda.synchronize()
    assert int(st[0]) == (1 << 1) | (1 << 3)
    cu = np.concatenate([[0], np.cumsum(T)])
    for r in (1, 3):
        assert bool((o[cu[r]:cu[r + 1]].view(torch.int16) == 0x7FC1).all()), "refused row %d wrote outputs" % r
        lo = 4 * bank[r]
        assert_same_bits(pool[lo:lo + 4], before[lo:lo + 4], "refused row %d wrote its bank" % r)
    for r in (0, 2):
        lo = 4 * bank[r]
        assert not bool((bits(pool[lo:lo + T[r]]) == POISON).any()), "row %d: checkpoints missing" % r
        assert_same_bits(pool[lo + T[r]:lo + 4], before[lo + T[r]:lo + 4], "row %d: extra slot" % r)
    # commit: row 2's accepted count is past its window; its entry stays
    acc = torch.tensor([1, 0, 2, 3], dtype=torch.int32, device="cuda")
    st2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    old = table.clone()
    gb.gdn_commit_select(dims, T, acc, bank, pool, table, st2)
    torch.cuda.synchronize()
    assert int(st2[0]) == 1 << 2
    expect = old.cpu().numpy().copy()
    for r in (0, 1, 3):
        expect[r] = 4 * bank[r] + int(acc[r])
    assert np.array_equal(table.cpu().numpy(), expect)


def test_batch1_workload_in_select_mode():
    w = synth.verify_workload("batch1", n_windows=64)
    worst = run_verify_workload(w, n_windows=w.n_windows, check_every=16, mode="select")
    say("batch1 select worst:", worst)


def test_conc16_workload_in_select_mode():
    w = synth.verify_workload("conc16", n_windows=128)
    worst = run_verify_workload(w, n_windows=w.n_windows, check_every=32, mode="select")
    say("conc16 select worst:", worst)


def test_batch1_workload_with_the_commit_inside_the_next_verify():
    w = synth.verify_workload("batch1", n_windows=64)
    worst = run_verify_workload(w, n_windows=w.n_windows, check_every=16, mode="select_commit")
    say("batch1 select-commit worst:", worst)


def test_conc16_workload_with_the_commit_inside_the_next_verify():
    """The headline form (one gdn_verify_window_select_commit launch per window) on the
    concurrency-16 workload (warm rows, K_r in {1, 2, 3}) against the oracle."""
    w = synth.verify_workload("conc16", n_windows=128)
    worst = run_verify_workload(w, n_windows=w.n_windows, check_every=32, mode="select_commit")
    say("conc16 select-commit worst:", worst)


@pytest.mark.parametrize("B", [1, 16], ids=["batch1", "rows16"])
def test_commit_inside_verify_equals_commit_then_verify(B):
    """gdn_verify_window_select_commit is gdn_commit_select followed by
    gdn_verify_window_select, bit for bit: outputs every window, table and selected states
    at the end, including a row whose accepted count is out of range (its table entry is
    kept, its status bit set, and its window runs from the kept entry)."""
    shape = synth.FULL
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    n_windows = 6
    g = synth.streams(131, 2 + 2 * n_windows)
    A_log, dt_bias = synth.head_params(g[0], shape)
    P = dev_params(A_log, dt_bias)
    rows = np.arange(B, dtype=np.int32)
    gen = torch.Generator(device="cpu").manual_seed(131)
    start = (0.2 * torch.randn(B, Hv, d, d, generator=gen)).cuda()
    pools = [torch.zeros(9 * B, Hv, d, d, device="cuda") for _ in range(2)]
    tables = [torch.arange(8 * B, 9 * B, dtype=torch.int32, device="cuda") for _ in range(2)]
    sts = [torch.zeros((B + 31) // 32, dtype=torch.int32, device="cuda") for _ in range(2)]
    for p in pools:
        p[8 * B:] = start
    prev = None  # (T, bank, accepted) of the previous window, for the folded calls
    for i in range(n_windows):
        T = g[1].integers(1, 5, size=B).astype(np.int32)
        tok = dev_tokens(synth.tokens(g[2 + i], shape, int(T.sum())))
        acc_h = np.array([g[2 + n_windows + i].integers(0, t) for t in T], np.int32)
        if i == 3:
            acc_h[B // 2] = T[B // 2]  # out of range: the commit is refused for that row
        acc = torch.from_numpy(acc_h).cuda()
        bank = 2 * rows + (i % 2)
        outs = []
        for path in (0, 1):
            o = torch.zeros(int(T.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
            if path == 0 or prev is None:
                gb.gdn_verify_window_select(dims, T, **tok, **P, state_pool=pools[path], slot_table=tables[path],
                                            bank=bank, o=o, status=sts[path])
            else:
                gb.gdn_verify_window_select_commit(dims, T, prev[0], prev[1], prev[2], **tok, **P,
                                                   state_pool=pools[path], slot_table=tables[path], bank=bank,
                                                   o=o, status=sts[path])
            if path == 0:
                gb.gdn_commit_select(dims, T, acc, bank, pools[0], tables[0], sts[0])
            outs.append(o)
        torch.cuda.synchronize()
        assert_same_bits(outs[0], outs[1], "window %d: outputs differ" % i)
        prev = (T, bank, acc)
    gb.gdn_commit_select(dims, prev[0], prev[2], prev[1], pools[1], tables[1], sts[1])  # the last window's commit
    torch.cuda.synchronize()
    assert torch.equal(tables[0], tables[1]), "slot tables differ"
    assert torch.equal(sts[0], sts[1]), "status words differ"
    assert int(sts[0][0]) & (1 << (B // 2)), "refused commit not flagged"
    assert_same_bits(pools[1][tables[1].long()], pools[0][tables[0].long()], "committed states differ")
    say("commit inside verify == commit then verify, %d rows, %d windows" % (B, n_windows))
