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
from tests.gpu_common import bits, dev_params, dev_tokens, dims_of, say
from tests.test_gpu_recurrent import run_verify_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _pool(n_slots, Hv, d, seed, scale=0.3):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (scale * torch.randn(n_slots, Hv, d, d, generator=g)).cuda()


@pytest.mark.parametrize("shape", [synth.FULL, synth.TINY, synth.HeadShape(2, 6, 128)],
                         ids=["h16x32_d128", "h1_d16", "h2x6_d128"])
def test_delta_commit_equals_checkpoint_commit_bitwise(shape):
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    pairs = [(t, a) for t in range(1, 5) for a in range(t)]
    T = np.array([t for t, _ in pairs], np.int32)
    B = T.size
    g = synth.streams(51, 2)
    A_log, dt_bias = synth.head_params(g[0], shape)
    P = dev_params(A_log, dt_bias)
    td = dev_tokens(synth.tokens(g[1], shape, int(T.sum())))
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
    assert torch.equal(o_ck.view(torch.int16), o_dl.view(torch.int16))
    assert torch.equal(bits(pool[:B]), bits(before[:B])), "verify wrote the committed pool"
    for r in range(B):
        assert torch.equal(bits(pool[2 * B + r]), bits(pool[B + r])), \
            "row %d (T=%d, a=%d): delta fold differs from checkpoint commit" % (r, T[r], pairs[r][1])


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
    assert torch.equal(bits(pool), bits(ref)), "delta fold differs from checkpoint commit"


def test_batch1_workload_in_delta_mode():
    w = synth.verify_workload("batch1", n_windows=64)
    say("batch1 delta worst:", run_verify_workload(w, n_windows=w.n_windows, check_every=16, mode="delta"))


def test_conc16_workload_in_delta_mode():
    w = synth.verify_workload("conc16", n_windows=128)
    say("conc16 delta worst:", run_verify_workload(w, n_windows=w.n_windows, check_every=32, mode="delta"))
