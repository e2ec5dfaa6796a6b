"""HIP graph capture of whole verification steps through the C ABI.

The library allocates nothing and never synchronises the host, so a step (every
layer's verify window, then every layer's commit) can be captured once on a stream
and replayed, which removes the per-call host launch cost that dominates at batch 1.
Each replay is checked bit for bit against the same step run eagerly on a copy of the
buffers, with eager work and device synchronisation between replays; the checkpoint
and replay commits are covered, and the folded delta mode (one launch per layer and
step, a graph of two steps alternating the two factor buffers).  The checkpoint-select
loop (batch 1 and 16 rows, the commit inside the next verify or its own launch) is
checked against the oracle instead: new windows and accepted counts are copied into the
graph's input buffers between replays, and every replay's outputs and committed states
are compared with the oracle's sequential run.
"""
import numpy as np
import pytest

from gateddeltanet_linear_attention_amd import binding as gb
from gateddeltanet_linear_attention_amd import synth
from tests.gpu_common import assert_same_bits, bits, dev_params, dev_tokens, dims_of, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


class Layer:
    """One layer's buffers and its prepared verify / commit calls on `stream`."""

    def __init__(self, dims, T, tok, P, acc, pool, replay, stream, folded=False):
        B = len(T)
        Hv, d = dims.n_v_heads, dims.d_k
        rows = np.arange(B, dtype=np.int32)
        self.inputs = (tok, P, acc)  # the prepared calls hold these too
        self.pool = pool
        self.o = torch.zeros(int(np.sum(T)), Hv, d, dtype=torch.bfloat16, device="cuda")
        self.status = torch.zeros((B + 31) // 32, dtype=torch.int32, device="cuda")
        self.ckpt, self.deltas = None, None
        if folded:
            self.deltas = [torch.zeros(gb.delta_shape(dims, B), device="cuda") for _ in range(2)]
            self.first = gb.prepare_verify_window_delta(dims, T, **tok, **P, state_pool=pool, src_slot=rows,
                                                        delta=self.deltas[0], o=self.o, stream=stream)
            self.fold = [gb.prepare_verify_window_delta_fold(
                dims, T, **tok, **P, state_pool=pool, slot=rows, delta=self.deltas[1 - j], o=self.o,
                prev_row_tokens=T, prev_k=tok["k"], prev_delta=self.deltas[j], prev_accepted=acc,
                status=self.status, stream=stream) for j in (0, 1)]
        elif replay:
            self.ckpt = None
            self.verify = gb.prepare_verify_window(dims, T, **tok, **P, state_pool=pool, src_slot=rows,
                                                   ckpt=None, o=self.o, stream=stream)
            self.commit = gb.prepare_commit_replay(dims, T, **tok, **P, accepted=acc, state_pool=pool,
                                                   src_slot=rows, dst_slot=rows, status=self.status,
                                                   stream=stream)
        else:
            self.ckpt = torch.zeros(B, 4, Hv, d, d, device="cuda")
            self.verify = gb.prepare_verify_window(dims, T, **tok, **P, state_pool=pool, src_slot=rows,
                                                   ckpt=self.ckpt, o=self.o, stream=stream)
            self.commit = gb.prepare_commit_accepted(dims, T, self.ckpt, acc, pool, dst_slot=rows,
                                                     status=self.status, stream=stream)


def _step(layers):
    for l in layers:
        l.verify()
    for l in layers:
        l.commit()


@pytest.mark.parametrize("replay", [False, True], ids=["checkpoint_commit", "replay_commit"])
def test_captured_step_replays_match_eager_steps(replay):
    shape = synth.FULL
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    T = np.array([4, 3, 2, 4, 1], np.int32)
    n_layers, n_replays = 3, 4
    cap = torch.cuda.Stream()
    graph_layers, eager_layers = [], []
    for li in range(n_layers):
        g = synth.streams(60 + li, 3)
        A_log, dt_bias = synth.head_params(g[0], shape)
        P = dev_params(A_log, dt_bias)
        tok = dev_tokens(synth.tokens(g[1], shape, int(T.sum())))
        acc = torch.from_numpy(synth.accepted_counts(g[2], T - 1)).cuda()
        gen = torch.Generator(device="cpu").manual_seed(li)
        pool = (0.1 * torch.randn(len(T), Hv, d, d, generator=gen)).cuda()
        graph_layers.append(Layer(dims, T, tok, P, acc, pool.clone(), replay, cap))
        eager_layers.append(Layer(dims, T, tok, P, acc, pool.clone(), replay, torch.cuda.current_stream()))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        _step(graph_layers)
    torch.cuda.synchronize()
    # capture records the launches without running them: both sides start equal
    for gl, el in zip(graph_layers, eager_layers):
        assert_same_bits(gl.pool, el.pool, "gl.pool vs el.pool")
    for k in range(n_replays):
        graph.replay()
        _step(eager_layers)
        torch.cuda.synchronize()
        for li, (gl, el) in enumerate(zip(graph_layers, eager_layers)):
            assert_same_bits(gl.pool, el.pool, "replay %d layer %d: state differs" % (k, li))
            assert_same_bits(gl.o, el.o, "replay %d layer %d: o" % (k, li))
            if gl.ckpt is not None:
                assert_same_bits(gl.ckpt, el.ckpt, "replay %d layer %d: checkpoints" % (k, li))
            assert int(gl.status.abs().sum()) == 0
    say("graph replays match eager steps (%s)" % ("replay" if replay else "checkpoint"))


def test_captured_folded_steps_match_eager_steps():
    shape = synth.FULL
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    T = np.array([4, 3, 2, 4, 1, 4], np.int32)
    n_layers, n_replays = 3, 4
    cap = torch.cuda.Stream()
    graph_layers, eager_layers = [], []
    for li in range(n_layers):
        g = synth.streams(70 + li, 3)
        A_log, dt_bias = synth.head_params(g[0], shape)
        P = dev_params(A_log, dt_bias)
        tok = dev_tokens(synth.tokens(g[1], shape, int(T.sum())))
        acc = torch.from_numpy(synth.accepted_counts(g[2], T - 1)).cuda()
        gen = torch.Generator(device="cpu").manual_seed(li)
        pool = (0.1 * torch.randn(len(T), Hv, d, d, generator=gen)).cuda()
        graph_layers.append(Layer(dims, T, tok, P, acc, pool.clone(), False, cap, folded=True))
        eager_layers.append(Layer(dims, T, tok, P, acc, pool.clone(), False, torch.cuda.current_stream(),
                                  folded=True))
    for l in graph_layers + eager_layers:  # the first window has no previous one to commit
        l.first()
    torch.cuda.synchronize()

    def two_steps(layers):
        for j in (0, 1):
            for l in layers:
                l.fold[j]()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        two_steps(graph_layers)
    torch.cuda.synchronize()
    for k in range(n_replays):
        graph.replay()
        two_steps(eager_layers)
        torch.cuda.synchronize()
        for li, (gl, el) in enumerate(zip(graph_layers, eager_layers)):
            assert_same_bits(gl.pool, el.pool, "replay %d layer %d: state differs" % (k, li))
            assert_same_bits(gl.o, el.o, "replay %d layer %d: o" % (k, li))
            for j in (0, 1):
                assert_same_bits(gl.deltas[j], el.deltas[j], "replay %d layer %d: factors" % (k, li))
            assert int(gl.status.abs().sum()) == 0 and int(el.status.abs().sum()) == 0
    say("graph replays of folded steps match eager steps")


@pytest.mark.parametrize("B", [1, 16], ids=["batch1", "rows16"])
@pytest.mark.parametrize("form", ["commit_inside_verify", "commit_then_verify"])
def test_decode_loop_from_a_graph_against_the_oracle(form, B):
    """A speculative decoding loop of K=3 windows (B rows) through 3 layers, captured once
    as a HIP graph of two windows per layer (checkpoint select: each row's two pool banks
    alternate) and replayed 4 times.  Between replays the next windows' tokens and accepted
    counts (Binomial(3, 0.85) per row) are copied into the device buffers the graph reads;
    after every replay each layer's outputs of both windows and its committed states are
    checked against the oracle's sequential run of the same windows and accepted prefixes.
    Forms: the previous window's commit inside the verify (one launch per layer and
    window), and gdn_commit_select then gdn_verify_window_select."""
    import oracle
    from tests.gpu_common import assert_o, assert_state, host
    shape = synth.FULL
    dims = dims_of(shape)
    Hv, d = shape.n_v_heads, shape.d
    n_layers, n_replays = 3, 4
    n_win = 1 + 2 * n_replays
    rows = np.arange(B, dtype=np.int32)
    T = np.full(B, 4, np.int32)
    banks = [2 * rows + j for j in (0, 1)]
    cap = torch.cuda.Stream()
    layers = []
    for li in range(n_layers):
        g = synth.streams(140 + li, 3)
        A_log, dt_bias = synth.head_params(g[0], shape)
        wins = [synth.tokens(g[1], shape, 4 * B) for _ in range(n_win)]
        accs = np.stack([synth.accepted_counts(g[2], np.full(B, 3)) for _ in range(n_win)]).astype(np.int32)
        gen = torch.Generator(device="cpu").manual_seed(140 + li)
        start = (0.2 * torch.randn(B, Hv, d, d, generator=gen)).cuda()
        pool = torch.zeros(9 * B, Hv, d, d, device="cuda")
        pool[8 * B:] = start
        L = dict(P=dev_params(A_log, dt_bias), wins=wins, accs=accs, pool=pool, A_log=A_log, dt_bias=dt_bias,
                 table=torch.arange(8 * B, 9 * B, dtype=torch.int32, device="cuda"),
                 status=torch.zeros((B + 31) // 32, dtype=torch.int32, device="cuda"),
                 tok=[dev_tokens(wins[1]), dev_tokens(wins[2])],
                 acc=[torch.zeros(B, dtype=torch.int32, device="cuda") for _ in range(2)],
                 o=[torch.zeros(4 * B, Hv, d, dtype=torch.bfloat16, device="cuda") for _ in range(2)])
        # the oracle's run: committed states before each window, outputs of each window
        S = host(start)
        L["S_before"], L["o_ref"] = [], []
        for w in range(n_win):
            L["S_before"].append(S)
            ck, o_ref = oracle.verify_window(T, wins[w].q, wins[w].k, wins[w].v, wins[w].a, wins[w].b, A_log,
                                             dt_bias, S)
            L["o_ref"].append(o_ref)
            S = oracle.commit(ck, T, accs[w])
        L["S_after"] = S
        # window 0, eagerly, into bank 0 of every row
        o0 = torch.zeros(4 * B, Hv, d, dtype=torch.bfloat16, device="cuda")
        gb.gdn_verify_window_select(dims, T, **dev_tokens(wins[0]), **L["P"], state_pool=pool,
                                    slot_table=L["table"], bank=banks[0], o=o0, status=L["status"])
        torch.cuda.synchronize()
        assert_o(host(o0), L["o_ref"][0], "layer %d window 0 outputs" % li)
        # the graph's calls: window j of a replay verifies into bank 1 - j, committing the
        # previous window (bank j, counts acc[j]) first
        calls = [[], []]
        for j in (0, 1):
            if form == "commit_inside_verify":
                calls[j].append(gb.prepare_verify_window_select_commit(
                    dims, T, T, banks[j], L["acc"][j], **L["tok"][j], **L["P"], state_pool=pool,
                    slot_table=L["table"], bank=banks[1 - j], o=L["o"][j], status=L["status"], stream=cap))
            else:
                calls[j].append(gb.prepare_commit_select(dims, T, L["acc"][j], banks[j], pool, L["table"],
                                                         L["status"], stream=cap))
                calls[j].append(gb.prepare_verify_window_select(dims, T, **L["tok"][j], **L["P"], state_pool=pool,
                                                                slot_table=L["table"], bank=banks[1 - j],
                                                                o=L["o"][j], status=L["status"], stream=cap))
        L["calls"] = calls
        layers.append(L)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for j in (0, 1):
            for L in layers:
                for c in L["calls"][j]:
                    c()
    for i in range(n_replays):
        w1, w2 = 1 + 2 * i, 2 + 2 * i
        for L in layers:  # eager copies of the next inputs between replays
            for j, w in ((0, w1), (1, w2)):
                src = dev_tokens(L["wins"][w])
                for key in src:
                    L["tok"][j][key].copy_(src[key])
            L["acc"][0].copy_(torch.from_numpy(L["accs"][w1 - 1]))
            L["acc"][1].copy_(torch.from_numpy(L["accs"][w2 - 1]))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for li, L in enumerate(layers):
            assert int(L["status"].abs().sum()) == 0, "layer %d replay %d: status set" % (li, i)
            assert_o(host(L["o"][0]), L["o_ref"][w1], "layer %d window %d outputs" % (li, w1))
            assert_o(host(L["o"][1]), L["o_ref"][w2], "layer %d window %d outputs" % (li, w2))
            # committed states: window w1's accepted checkpoints (the graph committed them)
            expect = 4 * banks[1] + L["accs"][w1]
            assert np.array_equal(L["table"].cpu().numpy(), expect), "layer %d: table entries" % li
            assert_state(host(L["pool"][L["table"].long()]), L["S_before"][w2], "layer %d committed states" % li)
    for li, L in enumerate(layers):  # the last window's commit, eagerly: the oracle's final states
        gb.gdn_commit_select(dims, T, torch.from_numpy(L["accs"][-1]).cuda(), banks[0], L["pool"], L["table"],
                             L["status"])
        torch.cuda.synchronize()
        assert_state(host(L["pool"][L["table"].long()]), L["S_after"], "layer %d final committed states" % li)
    say("decode loop from a graph (%s, %d rows): %d replays x 2 windows x %d layers vs the oracle"
        % (form, B, n_replays, n_layers))
