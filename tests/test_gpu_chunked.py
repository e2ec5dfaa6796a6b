"""GPU parity of the chunked prefill (with tail checkpoints) and of mixed ragged
transactions, against the fp64 oracle's sequential definition, through the C ABI.

* one 2048-token prefill at the full head shape, chunk 64, checkpoints at the last 4
  positions: outputs, final state and checkpoints vs the token-by-token recurrence;
* ragged rows whose tails straddle chunk boundaries, zero and non-zero start states,
  both head widths, a slow-decay stress case;
* a 16-row transaction mixing 4 long prefills and 12 K=3 verify windows: every
  verify row gets its per-token checkpoints although long prefills share the step
  (the fault of the onnxruntime-genai pull request "Run chained MTP drafting in the
  batch Engine", section "Correctness fix"), then commit and 64 decode-only windows;
* verify rows of a transaction are bit-identical to gdn_verify_window;
* a prefill published on one stream is seen by a verify on another after an event
  ("Native three-step MTP", section "What changed": publish pending prefill state
  before a dependent verification).
"""
import numpy as np
import pytest

import oracle
from gateddeltanet_linear_attention_amd import binding as gb
from gateddeltanet_linear_attention_amd import synth
from tests.gpu_common import (assert_o, assert_same_bits, assert_state, bits, dev_params, dev_tokens, dims_of,
                              host, index_tokens, ref_qk, say)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

POISON = 0x7FC0DEAD


def _poison(shape):
    t = torch.empty(shape, dtype=torch.float32, device="cuda")
    t.view(torch.int32).fill_(POISON)
    return t


def _ws(dims, lens):
    nb = gb.gdn_chunked_workspace_bytes(dims, lens)
    return torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")


def run_chunked_case(shape, lens, n_tail, src_kind, seed, gate_shift=0.0, what="", raw_qk=False):
    dims = dims_of(shape, raw_qk=raw_qk)
    B, Hv, d = len(lens), shape.n_v_heads, shape.d
    lens = np.asarray(lens, np.int32)
    n_tail = np.asarray(n_tail, np.int32)
    g = synth.streams(seed, 3)
    A_log, dt_bias = synth.head_params(g[0], shape)
    tok = synth.tokens(g[1], shape, int(lens.sum()), gate_shift, raw_qk=raw_qk)
    n_slots = 2 * B
    gen = torch.Generator(device="cpu").manual_seed(seed)
    pool = (0.3 * torch.randn(n_slots, Hv, d, d, generator=gen)).cuda()
    src = np.arange(B, dtype=np.int32) if src_kind == "state" else np.full(B, -1, np.int32)
    if src_kind == "mixed":
        src[::2] = np.arange(B, dtype=np.int32)[::2]
    dst = np.arange(B, 2 * B, dtype=np.int32)
    before = pool.clone()
    ckpt = _poison((B, 4, Hv, d, d))
    o = torch.empty(int(lens.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    gb.gdn_chunked_prefill_with_checkpoints(dims, lens, n_tail, **dev_tokens(tok), **dev_params(A_log, dt_bias),
                                            state_pool=pool, src_slot=src, dst_slot=dst, ckpt=ckpt, o=o,
                                            workspace=_ws(dims, lens))
    S0 = host(before[:B])
    S0[src < 0] = 0.0
    S_ref, ck_ref, o_ref = oracle.run_sequential(lens, *ref_qk(tok, raw_qk), tok.v, tok.a, tok.b, A_log, dt_bias,
                                                 S0, n_tail=n_tail, n_slot=4)
    torch.cuda.synchronize()
    mo = assert_o(host(o), o_ref, what + " outputs")
    ms = assert_state(host(pool[B:]), S_ref, what + " final states")
    for r in range(B):
        if n_tail[r]:
            ms = max(ms, assert_state(host(ckpt[r, :n_tail[r]]), ck_ref[r, :n_tail[r]],
                                      what + " row %d checkpoints" % r))
        assert bool((bits(ckpt[r, n_tail[r]:]) == POISON).all()), what + " row %d: extra slot written" % r
    assert_same_bits(pool[:B], before[:B], what + ": a source slot was written")
    say("%s: max |do| %.2e, state rel %.2e" % (what, mo, ms))


@pytest.mark.parametrize("raw_qk", [False, True], ids=["given_qk", "fused_l2norm"])
def test_prefill_2048_tokens_with_last_four_checkpoints(raw_qk):
    w = synth.prefill_workload(raw_qk=raw_qk)
    dims = dims_of(w.shape, raw_qk=raw_qk)
    Hv, d = w.shape.n_v_heads, w.shape.d
    tok = w.tokens()
    L = int(w.lens[0])
    pool = torch.zeros(1, Hv, d, d, device="cuda")
    ckpt = _poison((1, 4, Hv, d, d))
    o = torch.empty(L, Hv, d, dtype=torch.bfloat16, device="cuda")
    gb.gdn_chunked_prefill_with_checkpoints(dims, w.lens, w.n_tail, **dev_tokens(tok),
                                            **dev_params(w.A_log, w.dt_bias), state_pool=pool,
                                            src_slot=[-1], dst_slot=[0], ckpt=ckpt, o=o,
                                            workspace=_ws(dims, w.lens))
    S_ref, ck_ref, o_ref = oracle.run_sequential(w.lens, *ref_qk(tok, raw_qk), tok.v, tok.a, tok.b, w.A_log,
                                                 w.dt_bias, n_tail=w.n_tail, n_slot=4)
    torch.cuda.synchronize()
    mo = assert_o(host(o), o_ref, "prefill outputs")
    ms = assert_state(host(pool), S_ref, "prefill final state")
    ms = max(ms, assert_state(host(ckpt[0]), ck_ref[0], "prefill checkpoints (last 4 positions)"))
    # checkpoint 3 is the final state (bit for bit); checkpoint j is the state after L-3+j tokens
    assert_same_bits(ckpt[0, 3], pool[0], "last checkpoint differs from the final state")
    say("prefill 2048: max |do| %.2e, state rel %.2e" % (mo, ms))


@pytest.mark.parametrize("src_kind", ["zero", "state", "mixed"])
def test_ragged_rows_tails_straddling_chunks(src_kind):
    lens = [1, 5, 63, 64, 65, 66, 130, 200]
    n_tail = [1, 4, 4, 3, 4, 4, 4, 2]
    run_chunked_case(synth.HeadShape(2, 4, 128), lens, n_tail, src_kind, 61, what="ragged/" + src_kind)


@pytest.mark.parametrize("n_qk,n_v", [(8, 32), (8, 8), (4, 16)], ids=["group4_8qk", "group1_8qk", "group4_4qk"])
def test_head_groupings(n_qk, n_v):
    """Value heads per qk-head other than 2, with qk-head counts that do (8) and do not (4)
    take the prep kernel's chiplet-grouped block order."""
    run_chunked_case(synth.HeadShape(n_qk, n_v, 128), [130, 64, 3], [4, 2, 3], "mixed", 72 + n_v,
                     what="%d qk / %d v heads" % (n_qk, n_v))


def test_tiny_head_width():
    run_chunked_case(synth.TINY, [8, 70, 129], [4, 4, 1], "mixed", 62, what="d16")


def test_ragged_rows_with_fused_normalisation():
    lens = [1, 5, 63, 64, 65, 130, 200]
    n_tail = [1, 4, 4, 3, 4, 4, 2]
    run_chunked_case(synth.HeadShape(2, 4, 128), lens, n_tail, "mixed", 66, what="ragged/fused", raw_qk=True)
    run_chunked_case(synth.TINY, [8, 70, 129], [4, 4, 1], "mixed", 67, what="d16/fused", raw_qk=True)


def test_slow_decay_long_memory():
    run_chunked_case(synth.HeadShape(1, 2, 128), [300, 257], [4, 0], "state", 63, gate_shift=-8.0,
                     what="slow decay")


def test_streamed_workspace_with_fp32_w_at_the_tiny_head_width():
    """A call whose workspace with W in parts would pass 160 MiB streams it, with W in fp32
    (its parts formed in the chain kernel): 64 value heads of width 16 over 68 chunks.  The
    transaction tests cover that form at d = 128."""
    shape = synth.HeadShape(32, 64, 16)
    lens, chunks = [2176, 2150], 68
    assert ws_bytes_d16(chunks, fp32_w=False) > (160 << 20)
    assert gb.gdn_chunked_workspace_bytes(dims_of(shape), lens) == ws_bytes_d16(chunks, fp32_w=True)
    run_chunked_case(shape, lens, [4, 3], "mixed", 69, what="streamed d16")


def ws_bytes_d16(chunks, fp32_w):
    """Workspace bytes at d = 16 with 64 value heads over 32 qk-heads: per (chunk, value
    head) W (3072 floats in parts, 2048 in fp32), P 4608, U' 1024 and 6 * 64 factor floats;
    per (chunk, qk-head) Q 1024 and K^T 512 floats."""
    unit = (2048 if fp32_w else 3072) + 4608 + 1024 + 6 * 64
    return chunks * (64 * unit + 32 * (1024 + 512)) * 4


def compare_rows_alone_and_together(shape, lens, n_tail, raw_qk, seed, what):
    """Rows are independent, so the same row gives the same bits in any call: run the
    rows together and each alone, from random start states, and compare every row's
    outputs, final state and tail checkpoints bit for bit."""
    import torch
    dims = dims_of(shape, raw_qk=raw_qk)
    Hv, d = shape.n_v_heads, shape.d
    g = synth.streams(seed, 3)
    A_log, dt_bias = synth.head_params(g[0], shape)
    tok = synth.tokens(g[1], shape, int(lens.sum()), raw_qk=raw_qk)
    t, p = dev_tokens(tok), dev_params(A_log, dt_bias)
    gen = torch.Generator(device="cpu").manual_seed(seed)
    start = (0.3 * torch.randn(len(lens), Hv, d, d, generator=gen)).cuda()

    def run(rows):
        B = len(rows)
        tk = index_tokens(t, np.concatenate([np.arange(lens[:r].sum(), lens[:r + 1].sum()) for r in rows]))
        pool = torch.cat([start[list(rows)], torch.zeros(B, Hv, d, d, device="cuda")])
        ckpt = _poison((B, 4, Hv, d, d))
        o = torch.empty(int(lens[list(rows)].sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
        gb.gdn_chunked_prefill_with_checkpoints(dims, lens[list(rows)], n_tail[list(rows)], **tk, **p,
                                                state_pool=pool, src_slot=np.arange(B, dtype=np.int32),
                                                dst_slot=np.arange(B, 2 * B, dtype=np.int32), ckpt=ckpt, o=o,
                                                workspace=_ws(dims, lens[list(rows)]))
        return o, pool[B:], ckpt

    o2, s2, c2 = run(list(range(len(lens))))
    for r in range(len(lens)):
        o1, s1, c1 = run([r])
        o_rows = o2[int(lens[:r].sum()):int(lens[:r + 1].sum())]
        assert_same_bits(o_rows, o1, "row %d outputs, %s" % (r, what))
        assert_same_bits(s2[r:r + 1], s1, "row %d final state, %s" % (r, what))
        assert_same_bits(c2[r:r + 1, :n_tail[r]], c1[:, :n_tail[r]], "row %d checkpoints, %s" % (r, what))
    say("%s (%s): bit-identical" % (what, "fused" if raw_qk else "given q/k"))


@pytest.mark.parametrize("raw_qk", [False, True], ids=["given_qk", "fused_l2norm"])
def test_streamed_and_cached_workspaces_agree_bit_for_bit(raw_qk):
    """Two rows together pass 160 MiB of workspace (streamed: W in fp32); each alone stays
    under it (cached: W in bf16 parts).  Outputs, final states and tail checkpoints must
    agree bit for bit."""
    shape = synth.HeadShape(32, 64, 16)
    lens, n_tail = np.array([2176, 2176], np.int32), np.array([4, 3], np.int32)
    dims = dims_of(shape, raw_qk=raw_qk)
    assert gb.gdn_chunked_workspace_bytes(dims, lens) == ws_bytes_d16(68, fp32_w=True)     # streamed: fp32 W
    assert gb.gdn_chunked_workspace_bytes(dims, lens[:1]) == ws_bytes_d16(34, fp32_w=False)  # cached: parts
    compare_rows_alone_and_together(shape, lens, n_tail, raw_qk, 71, "streamed vs cached workspace")


@pytest.mark.parametrize("raw_qk", [False, True], ids=["given_qk", "fused_l2norm"])
def test_one_and_two_state_tiles_per_chain_block_agree_bit_for_bit(raw_qk):
    """At d = 128 the chain kernel holds two 16-channel state tiles per block when a launch
    has more (row, value head, tile) chains than the chip's 256 CUs, one otherwise: one row
    of 32 value heads (256 chains) runs with one tile per block, two rows (512) with two.
    Rows are independent, so both forms must give the same bits."""
    shape = synth.FULL
    lens, n_tail = np.array([300, 191], np.int32), np.array([4, 3], np.int32)
    assert len(lens) * shape.n_v_heads * (shape.d // 16) == 512
    compare_rows_alone_and_together(shape, lens, n_tail, raw_qk, 73, "one vs two tiles per chain block")


def test_more_than_64_chunked_rows_span_launches():
    """70 rows: the library splits a call into launches of at most 64 rows and numbers
    workspace chunks across them; tails straddle chunk boundaries, sources are mixed."""
    rng = np.random.default_rng(68)
    lens = rng.integers(65, 201, size=70).astype(np.int32)
    lens[:6] = [65, 127, 128, 129, 191, 200]
    n_tail = np.minimum(rng.integers(0, 5, size=70), lens).astype(np.int32)
    run_chunked_case(synth.HeadShape(1, 2, 128), lens, n_tail, "mixed", 68, what="70 rows")


def test_transaction_of_140_rows_mixing_routes():
    """140 rows alternating K<=3 verify windows and 65-300-token prefills: both routes
    take two launches each; every row's outputs, checkpoints and final state vs the
    oracle, verify rows' pool slots untouched."""
    shape = synth.HeadShape(1, 2, 128)
    dims = dims_of(shape)
    B, Hv, d = 140, shape.n_v_heads, shape.d
    rng = np.random.default_rng(69)
    is_pf = np.arange(B) % 2 == 1
    lens = np.where(is_pf, rng.integers(65, 301, size=B), rng.integers(1, 5, size=B)).astype(np.int32)
    n_ck = np.where(is_pf, rng.integers(0, 5, size=B), lens).astype(np.int32)
    n_ck = np.minimum(n_ck, lens).astype(np.int32)
    assert np.array_equal(gb.gdn_plan_transaction(dims, lens),
                          np.where(is_pf, gb.ROUTE_CHUNKED, gb.ROUTE_RECURRENT))
    g = synth.streams(69, 3)
    A_log, dt_bias = synth.head_params(g[0], shape)
    tok = synth.tokens(g[1], shape, int(lens.sum()))
    gen = torch.Generator(device="cpu").manual_seed(69)
    pool = (0.3 * torch.randn(2 * B, Hv, d, d, generator=gen)).cuda()
    src = np.arange(B, dtype=np.int32)
    src[is_pf & (np.arange(B) % 4 == 1)] = -1
    dst = np.where(is_pf, B + np.arange(B), -1).astype(np.int32)
    before = pool.clone()
    ckpt = _poison((B, 4, Hv, d, d))
    o = torch.empty(int(lens.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    say("transaction of 140 rows: %d chunked, %d recurrent" % (is_pf.sum(), (~is_pf).sum()))
    gb.gdn_run_transaction(dims, lens, n_ck, **dev_tokens(tok), **dev_params(A_log, dt_bias), state_pool=pool,
                           src_slot=src, dst_slot=dst, ckpt=ckpt, o=o, workspace=_ws(dims, lens[is_pf]))
    S0 = host(before[:B])
    S0[src < 0] = 0.0
    S_ref, ck_ref, o_ref = oracle.run_sequential(lens, tok.q, tok.k, tok.v, tok.a, tok.b, A_log, dt_bias, S0,
                                                 n_tail=n_ck, n_slot=4)
    torch.cuda.synchronize()
    mo = assert_o(host(o), o_ref, "140-row transaction outputs")
    pf_i = torch.as_tensor(np.nonzero(is_pf)[0], device="cuda")
    vf_i = torch.as_tensor(np.nonzero(~is_pf)[0], device="cuda")
    ms = assert_state(host(pool[B:].index_select(0, pf_i)), S_ref[is_pf], "140-row transaction final states")
    ck_h = host(ckpt)
    for r in range(B):
        if n_ck[r]:
            ms = max(ms, assert_state(ck_h[r, :n_ck[r]], ck_ref[r, :n_ck[r]], "row %d checkpoints" % r))
        assert bool((bits(ckpt[r, n_ck[r]:]) == POISON).all()), "row %d: extra checkpoint slot written" % r
    assert_same_bits(pool[:B], before[:B], "a source slot was written")
    assert_same_bits(pool[B:].index_select(0, vf_i), before[B:].index_select(0, vf_i), "a verify row published a state")
    say("140-row transaction: max |do| %.2e, state rel %.2e" % (mo, ms))


def test_chunked_matches_verify_within_tolerance_and_commit_works_on_it():
    """Commit is path-agnostic: tail slots of a chunked row mean what verify slots mean."""
    shape = synth.FULL
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    g = synth.streams(64, 2)
    A_log, dt_bias = synth.head_params(g[0], shape)
    P = dev_params(A_log, dt_bias)
    tok = synth.tokens(g[1], shape, 4)
    td = dev_tokens(tok)
    gen = torch.Generator(device="cpu").manual_seed(3)
    pool = (0.3 * torch.randn(3, Hv, d, d, generator=gen)).cuda()
    ck_v = torch.empty(1, 4, Hv, d, d, device="cuda")
    ck_c = torch.empty(1, 4, Hv, d, d, device="cuda")
    o_v = torch.empty(4, Hv, d, dtype=torch.bfloat16, device="cuda")
    o_c = torch.empty_like(o_v)
    gb.gdn_verify_window(dims, [4], **td, **P, state_pool=pool, src_slot=[0], ckpt=ck_v, o=o_v)
    gb.gdn_chunked_prefill_with_checkpoints(dims, [4], [4], **td, **P, state_pool=pool, src_slot=[0],
                                            dst_slot=[1], ckpt=ck_c, o=o_c, workspace=_ws(dims, [4]))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gb.gdn_commit_accepted(dims, [4], ck_c, torch.tensor([2], dtype=torch.int32, device="cuda"), pool,
                           dst_slot=[2], status=status)
    torch.cuda.synchronize()
    assert_state(host(ck_c[0]), host(ck_v[0]), "chunked vs verify checkpoints")
    assert_o(host(o_c), host(o_v), "chunked vs verify outputs")
    assert_same_bits(pool[2], ck_c[0, 2], "pool[2] vs ck_c[0, 2]")
    assert_same_bits(pool[1], ck_c[0, 3], "pool[1] vs ck_c[0, 3]")


# ---------------------------------------------------------------- mixed transaction

def test_mixed_transaction_then_decode_only_windows():
    run_mixed(synth.mixed_workload())


def test_mixed_transaction_with_fused_normalisation():
    run_mixed(synth.mixed_workload(n_windows=8, raw_qk=True))


def run_mixed(m: synth.MixedWorkload):
    """Warm the verify rows, run the packed transaction (prefills + K=3 windows), commit,
    then m.n_windows decode-only windows, each against the oracle."""
    raw = m.raw_qk
    shape = m.shape
    dims = dims_of(shape, raw_qk=raw)
    B, Hv, d = m.n_rows, shape.n_v_heads, shape.d
    P = dev_params(m.A_log, m.dt_bias)
    rows = np.arange(B, dtype=np.int32)
    is_pf = m.is_prefill
    pool = torch.zeros(B, Hv, d, d, device="cuda")

    # warm the verify rows (zero state, chunked prefill without checkpoints)
    warm = m.warm_tokens()
    wrows = rows[~is_pf]
    wl = m.warm_lens[~is_pf]
    ow = torch.empty(warm.n, Hv, d, dtype=torch.bfloat16, device="cuda")
    gb.gdn_chunked_prefill_with_checkpoints(dims, wl, np.zeros_like(wl), **dev_tokens(warm), **P,
                                            state_pool=pool, src_slot=np.full(len(wrows), -1), dst_slot=wrows,
                                            ckpt=torch.empty(len(wrows), 4, Hv, d, d, device="cuda"), o=ow,
                                            workspace=_ws(dims, wl))
    S_w, _, o_wref = oracle.run_sequential(wl, *ref_qk(warm, raw), warm.v, warm.a, warm.b, m.A_log, m.dt_bias)
    S_o = np.zeros((B, Hv, d, d))
    S_o[wrows] = S_w
    torch.cuda.synchronize()
    assert_o(host(ow), o_wref, "warm-up outputs")
    assert_state(host(pool), S_o, "warmed states")

    # the transaction: 4 prefills from zero (publish final state), 12 K=3 windows (checkpoints)
    lens = m.transaction_lens()
    assert np.array_equal(gb.gdn_plan_transaction(dims, lens),
                          np.where(is_pf, gb.ROUTE_CHUNKED, gb.ROUTE_RECURRENT))
    n_ck = np.where(is_pf, 0, 4).astype(np.int32)
    src = np.where(is_pf, -1, rows).astype(np.int32)
    dst = np.where(is_pf, rows, -1).astype(np.int32)
    tx = m.transaction_tokens()
    ckpt = _poison((B, 4, Hv, d, d))
    o = torch.empty(tx.n, Hv, d, dtype=torch.bfloat16, device="cuda")
    ws = _ws(dims, lens)
    gb.gdn_run_transaction(dims, lens, n_ck, **dev_tokens(tx), **P, state_pool=pool, src_slot=src,
                           dst_slot=dst, ckpt=ckpt, o=o, workspace=ws)
    acc = m.transaction_accepted()
    vrows = rows[~is_pf]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gb.gdn_commit_accepted(dims, np.full(len(vrows), 4), ckpt[torch.as_tensor(vrows, device="cuda")].contiguous(),
                           torch.from_numpy(acc[vrows]).cuda(), pool, dst_slot=vrows, status=status)
    S0 = S_o.copy()
    S_t, ck_t, o_t = oracle.run_sequential(lens, *ref_qk(tx, raw), tx.v, tx.a, tx.b, m.A_log, m.dt_bias, S0,
                                           n_tail=n_ck, n_slot=4)
    torch.cuda.synchronize()
    assert_o(host(o), o_t, "transaction outputs")
    for r in vrows:  # every verify row got all four checkpoints, and they are right
        assert_state(host(ckpt[r]), ck_t[r], "transaction verify row %d checkpoints" % r)
    for r in rows[is_pf]:
        assert bool((bits(ckpt[r]) == POISON).all()), "prefill row %d wrote checkpoints it did not ask for" % r
    S_o[is_pf] = S_t[is_pf]
    for r in vrows:
        S_o[r] = ck_t[r, acc[r]]
    assert int(status[0]) == 0
    assert_state(host(pool), S_o, "committed states after the transaction")
    say("mixed transaction ok; prefill lengths %s" % m.prefill_lens[is_pf].tolist())

    # 64 decode-only K=3 windows over all 16 rows
    T = np.full(B, 4, np.int32)
    ckw = torch.empty(B, 4, Hv, d, d, device="cuda")
    ow = torch.empty(4 * B, Hv, d, dtype=torch.bfloat16, device="cuda")
    out = dict(S_final=np.zeros_like(S_o), ckpt=np.zeros((B, 4, Hv, d, d)), o=np.zeros((4 * B, Hv, d)))
    S_bufs, cur = [S_o, np.zeros_like(S_o)], 0
    worst = 0.0
    for i in range(m.n_windows):
        win = m.window_tokens(i)
        a = m.accepted(i)
        gb.gdn_verify_window(dims, T, **dev_tokens(win), **P, state_pool=pool, src_slot=rows, ckpt=ckw, o=ow)
        gb.gdn_commit_accepted(dims, T, ckw, torch.from_numpy(a).cuda(), pool, dst_slot=rows, status=status)
        ck_o, o_o = oracle.verify_window(T, *ref_qk(win, raw), win.v, win.a, win.b, m.A_log, m.dt_bias,
                                         S_bufs[cur], nan_fill=False, out=out)
        cur = 1 - cur
        for r in range(B):
            S_bufs[cur][r] = ck_o[r, a[r]]
        worst = max(worst, assert_o(host(ow), o_o, "decode-only window %d" % i))
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    e = assert_state(host(pool), S_bufs[cur], "states after %d decode-only windows" % m.n_windows)
    say("decode-only windows ok: max |do| %.2e, state rel %.2e" % (worst, e))


@pytest.mark.parametrize("raw_qk", [False, True], ids=["given_qk", "fused_l2norm"])
def test_transaction_verify_rows_bit_identical_to_verify_window(raw_qk):
    shape = synth.FULL
    dims = dims_of(shape, raw_qk=raw_qk)
    Hv, d = shape.n_v_heads, shape.d
    lens = np.array([4, 300, 2, 1, 3, 130], np.int32)
    n_ck = np.array([4, 0, 2, 1, 3, 4], np.int32)
    B = len(lens)
    g = synth.streams(65, 2)
    A_log, dt_bias = synth.head_params(g[0], shape)
    P = dev_params(A_log, dt_bias)
    tok = synth.tokens(g[1], shape, int(lens.sum()), raw_qk=raw_qk)
    td = dev_tokens(tok)
    gen = torch.Generator(device="cpu").manual_seed(4)
    pool = (0.3 * torch.randn(B, Hv, d, d, generator=gen)).cuda()
    ckpt = _poison((B, 4, Hv, d, d))
    o = torch.empty(int(lens.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    gb.gdn_run_transaction(dims, lens, n_ck, **td, **P, state_pool=pool, src_slot=np.arange(B),
                           dst_slot=np.full(B, -1), ckpt=ckpt, o=o, workspace=_ws(dims, lens))
    short = np.nonzero(lens <= 4)[0]
    cu = np.concatenate([[0], np.cumsum(lens)])
    idx = np.concatenate([np.arange(cu[r], cu[r + 1]) for r in short])
    ck2 = _poison((len(short), 4, Hv, d, d))
    o2 = torch.empty(len(idx), Hv, d, dtype=torch.bfloat16, device="cuda")
    gb.gdn_verify_window(dims, lens[short], **index_tokens(td, idx), **P, state_pool=pool,
                         src_slot=short.astype(np.int32), ckpt=ck2, o=o2)
    torch.cuda.synchronize()
    for j, r in enumerate(short):
        assert_same_bits(ckpt[r, :n_ck[r]], ck2[j, lens[r] - n_ck[r]:lens[r]],
                         "row %d: transaction checkpoints vs the verify window's" % r)
    assert_same_bits(o[torch.as_tensor(idx, device="cuda")], o2, "o[torch.as_tensor(idx, device='cuda')] vs o2")
    # the long rows' checkpoints are the oracle's
    S_ref, ck_ref, o_ref = oracle.run_sequential(lens, *ref_qk(tok, raw_qk), tok.v, tok.a, tok.b, A_log, dt_bias,
                                                 host(pool), n_tail=n_ck, n_slot=4)
    assert_o(host(o), o_ref, "transaction outputs")
    assert_state(host(ckpt[5, :4]), ck_ref[5, :4], "chunked row checkpoints")


def test_prefill_published_on_one_stream_is_seen_by_verify_on_another():
    shape = synth.HeadShape(2, 4, 128)
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    g = synth.streams(66, 3)
    A_log, dt_bias = synth.head_params(g[0], shape)
    P = dev_params(A_log, dt_bias)
    pre = dev_tokens(synth.tokens(g[1], shape, 1000))
    win = dev_tokens(synth.tokens(g[2], shape, 4))
    ws = _ws(dims, [1000])

    def run(two_streams):
        pool = torch.zeros(1, Hv, d, d, device="cuda")
        o_p = torch.empty(1000, Hv, d, dtype=torch.bfloat16, device="cuda")
        ck = torch.empty(1, 4, Hv, d, d, device="cuda")
        o_v = torch.empty(4, Hv, d, dtype=torch.bfloat16, device="cuda")
        s1 = torch.cuda.Stream()
        s2 = torch.cuda.Stream() if two_streams else s1
        torch.cuda.synchronize()
        gb.gdn_chunked_prefill_with_checkpoints(dims, [1000], [0], **pre, **P, state_pool=pool, src_slot=[-1],
                                                dst_slot=[0], ckpt=ck, o=o_p, workspace=ws, stream=s1)
        if two_streams:
            ev = torch.cuda.Event()
            ev.record(s1)
            s2.wait_event(ev)
        gb.gdn_verify_window(dims, [4], **win, **P, state_pool=pool, src_slot=[0], ckpt=ck, o=o_v, stream=s2)
        torch.cuda.synchronize()
        return ck.clone(), o_v.clone()

    a = run(False)
    b = run(True)
    assert_same_bits(a[0], b[0], "a[0] vs b[0]")
    assert_same_bits(a[1], b[1], "a[1] vs b[1]")


def test_chunked_errors_write_nothing():
    shape = synth.HeadShape(1, 2, 128)
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    g = synth.streams(67, 2)
    A_log, dt_bias = synth.head_params(g[0], shape)
    td = dev_tokens(synth.tokens(g[1], shape, 100))
    pool = torch.zeros(2, Hv, d, d, device="cuda")
    ckpt = _poison((1, 4, Hv, d, d))
    o = torch.empty(100, Hv, d, dtype=torch.bfloat16, device="cuda")
    ws = _ws(dims, [100])
    small = torch.empty(ws.numel() - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(gb.GdnError) as e:  # workspace too small
        gb.gdn_chunked_prefill_with_checkpoints(dims, [100], [4], **td, **dev_params(A_log, dt_bias),
                                                state_pool=pool, src_slot=[-1], dst_slot=[0], ckpt=ckpt,
                                                o=o, workspace=small)
    assert e.value.code == -6
    with pytest.raises(gb.GdnError) as e:  # more tail checkpoints than slots
        gb.gdn_chunked_prefill_with_checkpoints(dims, [100], [5], **td, **dev_params(A_log, dt_bias),
                                                state_pool=pool, src_slot=[-1], dst_slot=[0], ckpt=ckpt,
                                                o=o, workspace=ws)
    assert e.value.code == -3
    torch.cuda.synchronize()
    assert float(pool.abs().sum()) == 0.0
    assert bool((bits(ckpt) == POISON).all())
