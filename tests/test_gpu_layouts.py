"""The recurrent kernel runs in two lane layouts: one state row per lane for
launches that store dense checkpoints (and small launches), two rows per lane for
wide launches that store none (verify without checkpoints, replay, delta verify,
folded verify, decode).  Each state row keeps its lanes, columns and reduction order
in both, so results must agree bit for bit.  A 20-row launch of 32 value heads
takes the two-row layout; the one-row results it is compared with come from the
checkpointing verify, which always takes the one-row layout."""
import numpy as np
import pytest

from gateddeltanet_linear_attention_amd import binding as gb
from gateddeltanet_linear_attention_amd import synth
from tests.gpu_common import assert_same_bits, bits, dev_params, dev_tokens, dims_of, index_tokens

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

B = 20  # rows x 32 heads >= 512: the two-row layout


def _setup(raw_qk, seed):
    shape = synth.FULL
    dims = dims_of(shape, raw_qk=raw_qk)
    g = synth.streams(seed, 5)
    T1 = g[0].integers(1, 5, size=B).astype(np.int32)
    T2 = g[0].integers(1, 5, size=B).astype(np.int32)
    A_log, dt_bias = synth.head_params(g[1], shape)
    P = dev_params(A_log, dt_bias)
    w1 = dev_tokens(synth.tokens(g[2], shape, int(T1.sum()), raw_qk=raw_qk))
    w2 = dev_tokens(synth.tokens(g[3], shape, int(T2.sum()), raw_qk=raw_qk))
    acc = np.array([g[4].integers(0, t) for t in T1], np.int32)
    gen = torch.Generator(device="cpu").manual_seed(seed)
    pool = (0.2 * torch.randn(B, shape.n_v_heads, shape.d, shape.d, generator=gen)).cuda()
    return dims, T1, T2, P, w1, w2, acc, pool


def _o(T, Hv=32, d=128):
    return torch.zeros(int(np.sum(T)), Hv, d, dtype=torch.bfloat16, device="cuda")


@pytest.mark.parametrize("raw_qk", [False, True], ids=["given_qk", "fused_l2norm"])
def test_two_row_layout_matches_one_row_layout_bitwise(raw_qk):
    dims, T1, T2, P, w1, w2, acc_np, base = _setup(raw_qk, 81)
    rows = np.arange(B, dtype=np.int32)
    acc = torch.from_numpy(acc_np).cuda()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    # reference: checkpointing verify (one-row layout) and its commit
    ckpt = torch.empty(B, 4, 32, 128, 128, device="cuda")
    o_ck = _o(T1)
    gb.gdn_verify_window(dims, T1, **w1, **P, state_pool=base, src_slot=rows, ckpt=ckpt, o=o_ck)
    committed = base.clone()
    gb.gdn_commit_accepted(dims, T1, ckpt, acc, committed, dst_slot=rows, status=st)
    # verify without checkpoints, then replay in place
    o_nock = _o(T1)
    pool_r = base.clone()
    gb.gdn_verify_window(dims, T1, **w1, **P, state_pool=pool_r, src_slot=rows, ckpt=None, o=o_nock)
    gb.gdn_commit_replay(dims, T1, **w1, **P, accepted=acc, state_pool=pool_r, src_slot=rows, dst_slot=rows,
                         status=st)
    # delta verify, fold commit
    d1 = torch.empty(gb.delta_shape(dims, B), device="cuda")
    o_dl = _o(T1)
    pool_d = base.clone()
    gb.gdn_verify_window_delta(dims, T1, **w1, **P, state_pool=pool_d, src_slot=rows, delta=d1, o=o_dl)
    pool_f = pool_d.clone()
    gb.gdn_commit_delta(dims, T1, w1["k"], d1, acc, pool_d, src_slot=rows, dst_slot=rows, status=st)
    # the next window: checkpointing verify from the committed state (one-row layout)
    # against the folded verify from the uncommitted pool (two-row layout)
    ck2 = torch.empty(B, 4, 32, 128, 128, device="cuda")
    o2_ck = _o(T2)
    gb.gdn_verify_window(dims, T2, **w2, **P, state_pool=committed, src_slot=rows, ckpt=ck2, o=o2_ck)
    d2 = torch.empty(gb.delta_shape(dims, B), device="cuda")
    o2_f = _o(T2)
    gb.gdn_verify_window_delta_fold(dims, T2, **w2, **P, state_pool=pool_f, slot=rows, delta=d2, o=o2_f,
                                    prev_row_tokens=T1, prev_k=w1["k"], prev_delta=d1, prev_accepted=acc, status=st)
    # decode of each row's first new token (two-row layout) against checkpoint slot 0
    cu2 = np.concatenate([[0], np.cumsum(T2)])
    pool_dec = committed.clone()
    o_dec = _o(np.ones(B))
    gb.gdn_decode_step(dims, **index_tokens(w2, cu2[:-1]), **P, state_pool=pool_dec, src_slot=rows,
                       dst_slot=rows, o=o_dec)
    torch.cuda.synchronize()
    assert int(st[0]) == 0
    i16 = lambda t: t.view(torch.int16)
    assert torch.equal(i16(o_nock), i16(o_ck)), "verify without checkpoints: outputs differ"
    assert torch.equal(i16(o_dl), i16(o_ck)), "delta verify: outputs differ"
    assert_same_bits(pool_r, committed, "replay commit differs from the checkpoint commit")
    assert_same_bits(pool_d, committed, "fold commit differs from the checkpoint commit")
    assert torch.equal(i16(o2_f), i16(o2_ck)), "folded verify: outputs differ"
    assert_same_bits(pool_f, committed, "folded verify: committed state differs")
    assert_same_bits(pool_dec, ck2[:, 0], "decode differs from checkpoint slot 0")
    assert torch.equal(i16(o_dec), i16(o2_ck[torch.as_tensor(cu2[:-1], device="cuda")]))
