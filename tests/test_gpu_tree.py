"""GPU checks of token-tree verification (gdn_verify_tree) through the C ABI.

A draft tree replaces the chain: window token t runs from its parent's state
(parent -1: the committed state), checkpoint slot t holds node t's state, and the
accepted path's last node is committed with gdn_commit_accepted.  The pages run
chains only and refuse tree shapes ("Occamy 1.0 MTP", section "MTP1 runtime");
this is the extension listed after the chain path.  Checked:

* every 4-node tree shape (24 parent lists) at d = 16, and random trees at the full
  head shape, against the fp64 oracle (tolerances of tests/gpu_common.py);
* a chain-shaped tree is bit-identical to gdn_verify_window;
* each node equals GPU decode calls along its root path, bit for bit, and committing
  a node then decoding on leaves no trace of the other branches;
* unwritten checkpoint slots keep their contents; the pool is only read.
"""
import itertools

import numpy as np
import pytest

import oracle
from gateddeltanet_linear_attention_amd import binding as gb
from gateddeltanet_linear_attention_amd import synth
from tests.gpu_common import (assert_o, assert_same_bits, assert_state, bits, dev_params, dev_tokens, dims_of,
                              host, index_tokens)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

POISON = 0x7FC0DEAD


def _case(shape, parents_by_row, seed, raw_qk=False):
    T = np.array([len(p) for p in parents_by_row], np.int32)
    g = synth.streams(seed, 2)
    A_log, dt_bias = synth.head_params(g[0], shape)
    tok = synth.tokens(g[1], shape, int(T.sum()), raw_qk=raw_qk)
    parents = np.concatenate([np.asarray(p, np.int32) for p in parents_by_row])
    return T, parents, tok, A_log, dt_bias


def _run_tree(shape, T, parents, tok, A_log, dt_bias, pool, raw_qk=False):
    dims = dims_of(shape, raw_qk=raw_qk)
    B, Hv, d = len(T), shape.n_v_heads, shape.d
    ckpt = torch.empty(B, 4, Hv, d, d, device="cuda")
    ckpt.view(torch.int32).fill_(POISON)
    o = torch.empty(int(T.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
    gb.gdn_verify_tree(dims, T, parents, **dev_tokens(tok), **dev_params(A_log, dt_bias), state_pool=pool,
                       src_slot=np.arange(B), ckpt=ckpt, o=o)
    return ckpt, o


def _random_trees(rng, B):
    out = []
    for _ in range(B):
        n = int(rng.integers(1, 5))
        out.append([-1] + [int(rng.integers(-1, t)) for t in range(1, n)])
    return out


def test_every_four_node_tree_against_the_oracle_d16():
    shape = synth.TINY
    trees = [[-1, p1, p2, p3] for p1 in (-1, 0) for p2 in (-1, 0, 1) for p3 in (-1, 0, 1, 2)]
    assert len(trees) == 24
    T, parents, tok, A_log, dt_bias = _case(shape, trees, 71)
    g = torch.Generator(device="cpu").manual_seed(3)
    pool = (0.3 * torch.randn(len(T), 1, 16, 16, generator=g)).cuda()
    before = pool.clone()
    ckpt, o = _run_tree(shape, T, parents, tok, A_log, dt_bias, pool)
    torch.cuda.synchronize()
    ck_o, o_o = oracle.verify_tree(T, parents, tok.q, tok.k, tok.v, tok.a, tok.b, A_log, dt_bias, host(before))
    assert_o(host(o), o_o, "tree outputs (d=16)")
    assert_state(host(ckpt), ck_o, "tree node states (d=16)")
    assert_same_bits(pool, before, "pool vs before")


def test_random_trees_full_shape_against_the_oracle():
    shape = synth.FULL
    trees = _random_trees(np.random.default_rng(72), 16)
    T, parents, tok, A_log, dt_bias = _case(shape, trees, 73)
    g = torch.Generator(device="cpu").manual_seed(4)
    pool = (0.05 * torch.randn(len(T), 32, 128, 128, generator=g)).cuda()
    ckpt, o = _run_tree(shape, T, parents, tok, A_log, dt_bias, pool)
    torch.cuda.synchronize()
    ck_o, o_o = oracle.verify_tree(T, parents, tok.q, tok.k, tok.v, tok.a, tok.b, A_log, dt_bias, host(pool))
    assert_o(host(o), o_o, "tree outputs")
    for r, t in enumerate(T):
        assert_state(host(ckpt[r, :t]), ck_o[r, :t], "row %d node states" % r)
        assert bool((bits(ckpt[r, t:]) == POISON).all()), "row %d: slot >= T_r written" % r


@pytest.mark.parametrize("raw_qk", [False, True], ids=["given_qk", "fused_l2norm"])
@pytest.mark.parametrize("shape", [synth.FULL, synth.TINY], ids=["h16x32_d128", "h1_d16"])
def test_chain_shaped_tree_is_bit_identical_to_the_window(shape, raw_qk):
    dims = dims_of(shape, raw_qk=raw_qk)
    T = np.array([4, 3, 1, 2, 4], np.int32)
    parents = np.concatenate([np.arange(t) - 1 for t in T]).astype(np.int32)
    _, _, tok, A_log, dt_bias = _case(shape, [list(range(-1, t - 1)) for t in T], 74, raw_qk)
    g = torch.Generator(device="cpu").manual_seed(5)
    pool = (0.2 * torch.randn(len(T), shape.n_v_heads, shape.d, shape.d, generator=g)).cuda()
    ck_t, o_t = _run_tree(shape, T, parents, tok, A_log, dt_bias, pool, raw_qk)
    ck_w = torch.empty_like(ck_t)
    ck_w.view(torch.int32).fill_(POISON)
    o_w = torch.empty_like(o_t)
    gb.gdn_verify_window(dims, T, **dev_tokens(tok), **dev_params(A_log, dt_bias), state_pool=pool,
                         src_slot=np.arange(len(T)), ckpt=ck_w, o=o_w)
    torch.cuda.synchronize()
    assert_same_bits(ck_t, ck_w, "ck_t vs ck_w")
    assert_same_bits(o_t, o_w, "o_t vs o_w")


def test_nodes_equal_decode_along_their_paths_and_commit_leaves_no_trace():
    shape = synth.FULL
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    trees = [[-1, 0, 0, 1], [-1, -1, 1, 0], [-1, 0, 1]]
    T, parents, tok, A_log, dt_bias = _case(shape, trees, 75)
    P = dev_params(A_log, dt_bias)
    td = dev_tokens(tok)
    g = torch.Generator(device="cpu").manual_seed(6)
    pool = (0.1 * torch.randn(len(T), Hv, d, d, generator=g)).cuda()
    ckpt, o = _run_tree(shape, T, parents, tok, A_log, dt_bias, pool)
    cu = np.concatenate([[0], np.cumsum(T)])
    work = torch.empty(1, Hv, d, d, device="cuda")
    o1 = torch.empty(1, Hv, d, dtype=torch.bfloat16, device="cuda")
    for r, par in enumerate(trees):
        for t in range(len(par)):
            path, x = [], t
            while x >= 0:
                path.append(x)
                x = par[x]
            work.copy_(pool[r:r + 1])
            for x in path[::-1]:
                gb.gdn_decode_step(dims, **index_tokens(td, [cu[r] + x]), **P, state_pool=work, src_slot=[0],
                                   dst_slot=[0], o=o1)
            torch.cuda.synchronize()
            assert_same_bits(work[0], ckpt[r, t], "row %d node %d differs from its path" % (r, t))
            assert_same_bits(o1[0], o[cu[r] + t], "row %d node %d output" % (r, t))
    # commit node 3 of row 0 (path 0 -> 1 -> 3) and node 2 of row 1 (path 1 -> 2)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc = torch.tensor([3, 2, 0], dtype=torch.int32, device="cuda")
    gb.gdn_commit_accepted(dims, T, ckpt, acc, pool, dst_slot=[0, 1, 2], status=status)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    for r, a in enumerate([3, 2, 0]):
        assert_same_bits(pool[r], ckpt[r, a], "row %d: committed node %d" % (r, a))
