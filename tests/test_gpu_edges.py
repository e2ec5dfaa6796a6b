"""Edge cases through the C ABI on the GPU.

* Zero rows: every entry point returns without launching or writing anything.
* The largest head count (H_v = 1024) with pool offsets past 2^31 elements, against the
  oracle, through verify, commit, decode and the chunked prefill.
* Degenerate gates and vectors, against the oracle: write strength beta -> 1 (the
  delta-rule overwrite) and -> 0 (pure decay), decay alpha -> 0 (state reset) and
  -> 1 (no decay), zero keys, zero values and zero queries, with q/k given or
  normalised in the kernels (a zero raw vector stays zero), through the recurrent
  kernel and the chunked form.
"""
import numpy as np
import pytest

import oracle
from gateddeltanet_linear_attention_amd import binding as gb
from gateddeltanet_linear_attention_amd import synth
from tests.gpu_common import (assert_o, assert_same_bits, assert_state, bits, dev_params, dev_tokens, dims_of,
                              host, ref_qk)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

POISON = 0x7FC0DEAD


def test_zero_row_calls_write_nothing():
    shape = synth.FULL
    dims = dims_of(shape)
    Hv, d, Hq = shape.n_v_heads, shape.d, shape.n_qk_heads
    pool = torch.empty(2, Hv, d, d, device="cuda")
    pool.view(torch.int32).fill_(POISON)
    before = pool.clone()
    e16 = lambda h: torch.empty(0, h, d, dtype=torch.bfloat16, device="cuda")
    ef = torch.empty(0, Hv, device="cuda")
    P = dev_params(np.zeros(Hv, np.float32), np.zeros(Hv, np.float32))
    tok = dict(q=e16(Hq), k=e16(Hq), v=e16(Hv), a=ef, b=ef.clone())
    none = np.zeros(0, np.int32)
    ckpt = torch.empty(0, 4, Hv, d, d, device="cuda")
    o = e16(Hv)
    acc = torch.empty(0, dtype=torch.int32, device="cuda")
    st = torch.zeros(0, dtype=torch.int32, device="cuda")  # status words for zero rows
    delta = torch.empty(gb.delta_shape(dims, 0), device="cuda")
    gb.gdn_decode_step(dims, **tok, **P, state_pool=pool, src_slot=none, dst_slot=none, o=o)
    gb.gdn_verify_window(dims, none, **tok, **P, state_pool=pool, src_slot=none, ckpt=ckpt, o=o)
    gb.gdn_verify_window(dims, none, **tok, **P, state_pool=pool, src_slot=none, ckpt=None, o=o)
    gb.gdn_verify_tree(dims, none, none, **tok, **P, state_pool=pool, src_slot=none, ckpt=ckpt, o=o)
    gb.gdn_commit_accepted(dims, none, ckpt, acc, pool, dst_slot=none, status=st)
    gb.gdn_commit_replay(dims, none, **tok, **P, accepted=acc, state_pool=pool, src_slot=none, dst_slot=none,
                         status=st)
    gb.gdn_verify_window_delta(dims, none, **tok, **P, state_pool=pool, src_slot=none, delta=delta, o=o)
    gb.gdn_commit_delta(dims, none, tok["k"], delta, acc, pool, src_slot=none, dst_slot=none, status=st)
    gb.gdn_verify_window_delta_fold(dims, none, **tok, **P, state_pool=pool, slot=none, delta=delta, o=o,
                                    prev_row_tokens=none, prev_k=tok["k"], prev_delta=delta.clone(),
                                    prev_accepted=acc, status=st)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    assert gb.gdn_chunked_workspace_bytes(dims, none) == 0
    gb.gdn_chunked_prefill_with_checkpoints(dims, none, none, **tok, **P, state_pool=pool, src_slot=none,
                                            dst_slot=none, ckpt=ckpt, o=o, workspace=ws)
    gb.gdn_run_transaction(dims, none, none, **tok, **P, state_pool=pool, src_slot=none, dst_slot=none,
                           ckpt=ckpt, o=o, workspace=ws)
    torch.cuda.synchronize()
    assert_same_bits(pool, before, "pool vs before")


def _degenerate_tokens(shape, raw_qk, seed):
    """8 rows x 4 tokens; row r carries one extreme case on every token."""
    g = synth.streams(seed, 2)
    tok = synth.tokens(g[0], shape, 32, raw_qk=raw_qk)
    q, k, v, a, b = (x.copy() for x in (tok.q, tok.k, tok.v, tok.a, tok.b))
    rows = lambda r: slice(4 * r, 4 * r + 4)
    b[rows(0)] = 60.0    # beta = 1: the key's old value is overwritten
    b[rows(1)] = -60.0   # beta ~ 1e-26: pure decay
    a[rows(2)] = 60.0    # alpha = exp(-exp(A_log) * 60) ~ 0: the state is reset
    a[rows(3)] = -60.0   # alpha ~ 1: no decay
    k[rows(4)] = 0.0     # zero keys
    v[rows(5)] = 0.0     # zero values
    q[rows(6)] = 0.0     # zero queries: zero outputs
    a[rows(7)] = 88.0    # both gates saturated at once
    b[rows(7)] = 88.0
    return synth.Tokens(q, k, v, a, b), *synth.head_params(g[1], shape)


@pytest.mark.parametrize("raw_qk", [False, True], ids=["given_qk", "fused_l2norm"])
def test_degenerate_gates_and_vectors_match_the_oracle(raw_qk):
    shape = synth.HeadShape(2, 4, 128)
    dims = dims_of(shape, raw_qk=raw_qk)
    Hv, d = shape.n_v_heads, shape.d
    tok, A_log, dt_bias = _degenerate_tokens(shape, raw_qk, 95)
    B, T = 8, np.full(8, 4, np.int32)
    gen = torch.Generator(device="cpu").manual_seed(95)
    pool = (0.3 * torch.randn(B, Hv, d, d, generator=gen)).cuda()
    td, P = dev_tokens(tok), dev_params(A_log, dt_bias)
    ckpt = torch.empty(B, 4, Hv, d, d, device="cuda")
    o = torch.empty(32, Hv, d, dtype=torch.bfloat16, device="cuda")
    gb.gdn_verify_window(dims, T, **td, **P, state_pool=pool, src_slot=np.arange(B), ckpt=ckpt, o=o)
    # the same rows through the chunked form, from the same states, into fresh slots
    pool2 = torch.cat([pool, torch.zeros_like(pool)])
    ck_c = torch.empty_like(ckpt)
    o_c = torch.empty_like(o)
    ws = torch.empty(gb.gdn_chunked_workspace_bytes(dims, T), dtype=torch.uint8, device="cuda")
    gb.gdn_chunked_prefill_with_checkpoints(dims, T, T, **td, **P, state_pool=pool2, src_slot=np.arange(B),
                                            dst_slot=np.arange(B, 2 * B), ckpt=ck_c, o=o_c, workspace=ws)
    qo, ko = ref_qk(tok, raw_qk)
    ck_o, o_o = oracle.verify_window(T, qo, ko, tok.v, tok.a, tok.b, A_log, dt_bias, host(pool))
    torch.cuda.synchronize()
    for name, oo, cc in (("recurrent", o, ckpt), ("chunked", o_c, ck_c)):
        assert bool(torch.isfinite(cc).all()) and bool(torch.isfinite(oo.float()).all()), name
        assert_o(host(oo), o_o, name + " outputs")
        for r in range(B):
            assert_state(host(cc[r]), ck_o[r], "%s row %d checkpoints" % (name, r))
    assert not bool(o[24:28].view(torch.int16).any()), "zero queries must give zero outputs"


def test_readme_example_runs_and_matches_the_oracle():
    """The usage example of the README, as written, against the oracle."""
    import re
    import os
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", src, re.S)
    assert len(blocks) == 2
    env = {}
    torch.manual_seed(0)
    exec(compile(blocks[0], "README.md", "exec"), env)
    torch.cuda.synchronize()
    host_ = lambda t: t.float().cpu().numpy().astype(np.float64)
    qh, kh = host_(env["q"]), host_(env["k"])
    ck_o, o_o = oracle.verify_window(env["T"], qh, kh, host_(env["v"]), host_(env["a"]), host_(env["b"]),
                                     host_(env["A_log"]), host_(env["dt_bias"]), np.zeros((16, 32, 128, 128)))
    assert_o(host(env["o"]), o_o, "README example outputs")
    assert_state(host(env["pool"]), oracle.commit(ck_o, env["T"], np.full(16, 3)), "README example commit")
    assert int(env["status"][0]) == 0
    # the second example: four windows of the same tokens, each committing 3 drafts
    exec(compile(blocks[1], "README.md", "exec"), env)
    torch.cuda.synchronize()
    S = np.zeros((16, 32, 128, 128))
    for _ in range(4):
        ck_s, o_s = oracle.verify_window(env["T"], qh, kh, host_(env["v"]), host_(env["a"]), host_(env["b"]),
                                         host_(env["A_log"]), host_(env["dt_bias"]), S)
        S = oracle.commit(ck_s, env["T"], np.full(16, 3))
    assert_o(host(env["o"]), o_s, "README select example outputs (last window)")
    assert_state(host(env["committed"]), S, "README select example committed states")
    assert int(env["status"][0]) == 0


def test_largest_head_count_with_slot_offsets_past_2_31_elements():
    """H_v = 1024 (the largest supported), H_qk = 512, d = 128, in a 132-slot pool: one
    slot is 2^24 floats, so the source and destination slots used here (128..131) lie
    past 2^31 elements.  A verify window with every checkpoint, the copy commit, an
    in-place decode step, and a 130-token chunked prefill (two full chunks and a partial
    one) with four tail checkpoints, each against the oracle."""
    shape = synth.HeadShape(512, 1024, 128)
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    g = synth.streams(177, 5)
    A_log, dt_bias = synth.head_params(g[0], shape)
    P = dev_params(A_log, dt_bias)
    n_slots = 132
    pool = torch.zeros(n_slots, Hv, d, d, device="cuda")  # 8.6 GB
    gen = torch.Generator(device="cpu").manual_seed(177)
    S0 = 0.2 * torch.randn(2, Hv, d, d, generator=gen)
    src = np.array([131, 129], np.int32)
    pool[torch.as_tensor(src.astype(np.int64), device="cuda")] = S0.cuda()
    S0 = S0.numpy().astype(np.float64)

    # verify window (T = 4, 3) with checkpoints, then the copy commit into slots 130, 128
    T = np.array([4, 3], np.int32)
    win = synth.tokens(g[1], shape, int(T.sum()))
    ckpt = torch.full((2, 4, Hv, d, d), float("nan"), device="cuda")
    o = torch.empty(int(T.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    gb.gdn_verify_window(dims, T, **dev_tokens(win), **P, state_pool=pool, src_slot=src, ckpt=ckpt, o=o)
    ck_o, o_o = oracle.verify_window(T, win.q, win.k, win.v, win.a, win.b, A_log, dt_bias, S0)
    torch.cuda.synchronize()
    assert_o(host(o), o_o, "H_v 1024 verify outputs")
    for r in range(2):
        assert_state(host(ckpt[r, :T[r]]), ck_o[r, :T[r]], "H_v 1024 verify row %d checkpoints" % r)
    acc = np.array([3, 1], np.int32)
    dst = np.array([130, 128], np.int32)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gb.gdn_commit_accepted(dims, T, ckpt, torch.from_numpy(acc).cuda(), pool, dst_slot=dst, status=status)
    S1 = oracle.commit(ck_o, T, acc)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    assert_state(host(pool[torch.as_tensor(dst.astype(np.int64), device="cuda")]), S1, "H_v 1024 committed states")

    # one decode step in place on the committed slots
    dec = synth.tokens(g[2], shape, 2)
    od = torch.empty(2, Hv, d, dtype=torch.bfloat16, device="cuda")
    gb.gdn_decode_step(dims, **dev_tokens(dec), **P, state_pool=pool, src_slot=dst, dst_slot=dst, o=od)
    S2, od_ref = oracle.decode_step(dec.q, dec.k, dec.v, dec.a, dec.b, A_log, dt_bias, S1)
    torch.cuda.synchronize()
    assert_o(host(od), od_ref, "H_v 1024 decode outputs")
    assert_state(host(pool[torch.as_tensor(dst.astype(np.int64), device="cuda")]), S2, "H_v 1024 decode states")

    # chunked prefill of 130 tokens from slot 131 into slot 129, last four checkpoints
    L = np.array([130], np.int32)
    n_tail = np.array([4], np.int32)
    pre = synth.tokens(g[3], shape, 130)
    ck_c = torch.full((1, 4, Hv, d, d), float("nan"), device="cuda")
    o_c = torch.empty(130, Hv, d, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gb.gdn_chunked_workspace_bytes(dims, L), dtype=torch.uint8, device="cuda")
    gb.gdn_chunked_prefill_with_checkpoints(dims, L, n_tail, **dev_tokens(pre), **P, state_pool=pool,
                                            src_slot=[131], dst_slot=[129], ckpt=ck_c, o=o_c, workspace=ws)
    S_f, ck_f, o_f = oracle.run_sequential(L, pre.q, pre.k, pre.v, pre.a, pre.b, A_log, dt_bias, S0[:1],
                                           n_tail=n_tail, n_slot=4)
    torch.cuda.synchronize()
    assert_o(host(o_c), o_f, "H_v 1024 chunked outputs")
    assert_state(host(pool[129:130]), S_f, "H_v 1024 chunked final state")
    assert_state(host(ck_c[0]), ck_f[0], "H_v 1024 chunked tail checkpoints")
    assert_same_bits(ck_c[0, 3], pool[129], "last checkpoint != published state")
