"""GPU checks of rollback by replay (gdn_verify_window without checkpoints, then
gdn_commit_replay), through the C ABI.

The pull request thread "Run chained MTP drafting in the batch Engine" closes by
replacing dense recurrent checkpoints with a replay of the state; the reading
taken here: verification computes the window's outputs from the committed state
and stores no checkpoint, and commit re-runs the accepted prefix (the previous
bonus token and a_r drafts) from the committed state.  Checked:

* the replayed state is bit-identical to checkpoint slot a_r of a checkpointing
  verify of the same window (so to gdn_commit_accepted and to a_r + 1 decode
  calls), for every accepted count and three head shapes;
* verify without checkpoints writes the same outputs bit for bit and never writes
  the pool;
* in-place replay, bad accepted counts (row untouched, status bit set), rows
  spread over more than one launch;
* the batch-1 and concurrency-16 workloads run in replay mode against the oracle.
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


def _case(shape, T, seed, raw_qk=False):
    g = synth.streams(seed, 3)
    A_log, dt_bias = synth.head_params(g[0], shape)
    tok = synth.tokens(g[1], shape, int(np.sum(T)), raw_qk=raw_qk)
    acc = np.array([g[2].integers(0, t) for t in T], np.int32)
    return dev_params(A_log, dt_bias), dev_tokens(tok), acc


@pytest.mark.parametrize("raw_qk", [False, True], ids=["given_qk", "fused_l2norm"])
@pytest.mark.parametrize("shape", [synth.FULL, synth.TINY, synth.HeadShape(2, 6, 128)],
                         ids=["h16x32_d128", "h1_d16", "h2x6_d128"])
def test_replay_equals_checkpoint_commit_bitwise(shape, raw_qk):
    dims = dims_of(shape, raw_qk=raw_qk)
    Hv, d = shape.n_v_heads, shape.d
    # every (T, a) pair with 1 <= T <= 4, 0 <= a < T
    pairs = [(t, a) for t in range(1, 5) for a in range(t)]
    T = np.array([t for t, _ in pairs], np.int32)
    B = T.size
    P, td, _ = _case(shape, T, 41, raw_qk)
    acc = torch.tensor([a for _, a in pairs], dtype=torch.int32, device="cuda")
    rows = np.arange(B, dtype=np.int32)
    pool = _pool(3 * B, Hv, d, 7)
    before = pool.clone()
    N = int(T.sum())
    o_ck = torch.empty(N, Hv, d, dtype=torch.bfloat16, device="cuda")
    o_nock = torch.empty_like(o_ck)
    ckpt = torch.empty(B, 4, Hv, d, d, device="cuda")
    status = torch.zeros((B + 31) // 32, dtype=torch.int32, device="cuda")
    # checkpointing verify + commit into slots B..2B-1
    gb.gdn_verify_window(dims, T, **td, **P, state_pool=pool, src_slot=rows, ckpt=ckpt, o=o_ck)
    gb.gdn_commit_accepted(dims, T, ckpt, acc, pool, dst_slot=rows + B, status=status)
    # verify without checkpoints + replay into slots 2B..3B-1
    gb.gdn_verify_window(dims, T, **td, **P, state_pool=pool, src_slot=rows, ckpt=None, o=o_nock)
    gb.gdn_commit_replay(dims, T, **td, **P, accepted=acc, state_pool=pool, src_slot=rows,
                         dst_slot=rows + 2 * B, status=status)
    torch.cuda.synchronize()
    assert int(status.abs().sum()) == 0
    assert_same_bits(o_ck, o_nock, "o_ck vs o_nock")
    assert_same_bits(pool[:B], before[:B], "verify wrote the committed pool")
    for r in range(B):
        assert_same_bits(pool[2 * B + r], pool[B + r],
                         "row %d (T=%d, a=%d): replay differs from checkpoint commit" % (r, T[r], pairs[r][1]))


def test_replay_in_place_flags_bad_counts_and_spans_launches():
    shape = synth.FULL
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    B = 70  # more rows than one launch carries
    g = np.random.default_rng(5)
    T = g.integers(1, 5, size=B).astype(np.int32)
    P, td, acc_np = _case(shape, T, 43)
    acc_np[3] = T[3]      # one past the window
    acc_np[66] = -1       # negative, in the second launch
    acc = torch.from_numpy(acc_np).cuda()
    rows = np.arange(B, dtype=np.int32)
    pool = _pool(B, Hv, d, 8, scale=0.1)
    ref = pool.clone()
    ckpt = torch.empty(B, 4, Hv, d, d, device="cuda")
    o = torch.empty(int(T.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    status_ref = torch.zeros(3, dtype=torch.int32, device="cuda")
    status = torch.zeros(3, dtype=torch.int32, device="cuda")
    gb.gdn_verify_window(dims, T, **td, **P, state_pool=ref, src_slot=rows, ckpt=ckpt, o=o)
    gb.gdn_commit_accepted(dims, T, ckpt, acc, ref, dst_slot=rows, status=status_ref)
    gb.gdn_commit_replay(dims, T, **td, **P, accepted=acc, state_pool=pool, src_slot=rows,
                         dst_slot=rows, status=status)
    torch.cuda.synchronize()
    expect = [0, 0, 0]
    for r in (3, 66):
        expect[r // 32] |= 1 << (r % 32)
    assert [int(x) & 0xFFFFFFFF for x in status.cpu()] == expect
    assert torch.equal(status, status_ref)
    assert_same_bits(pool, ref, "in-place replay differs from checkpoint commit")


def test_replay_zero_source_state():
    shape = synth.FULL
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    T = np.array([4, 2, 3], np.int32)
    P, td, acc_np = _case(shape, T, 47)
    acc = torch.from_numpy(acc_np).cuda()
    pool = _pool(6, Hv, d, 9)
    ckpt = torch.empty(3, 4, Hv, d, d, device="cuda")
    o = torch.empty(int(T.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    src = np.array([-1, -1, -1], np.int32)
    gb.gdn_verify_window(dims, T, **td, **P, state_pool=pool, src_slot=src, ckpt=ckpt, o=o)
    gb.gdn_commit_accepted(dims, T, ckpt, acc, pool, dst_slot=[0, 1, 2], status=status)
    gb.gdn_commit_replay(dims, T, **td, **P, accepted=acc, state_pool=pool, src_slot=src,
                         dst_slot=[3, 4, 5], status=status)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    assert_same_bits(pool[3:], pool[:3], "pool[3:] vs pool[:3]")


def test_batch1_workload_in_replay_mode():
    w = synth.verify_workload("batch1", n_windows=64)
    worst = run_verify_workload(w, n_windows=w.n_windows, check_every=16, mode="replay")
    say("batch1 replay worst:", worst)


def test_conc16_workload_in_replay_mode():
    w = synth.verify_workload("conc16", n_windows=128)
    worst = run_verify_workload(w, n_windows=w.n_windows, check_every=32, mode="replay")
    say("conc16 replay worst:", worst)
