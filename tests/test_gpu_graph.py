"""HIP graph capture of whole verification steps through the C ABI.

The library allocates nothing and never synchronises the host, so a step (every
layer's verify window, then every layer's commit) can be captured once on a stream
and replayed, which removes the per-call host launch cost that dominates at batch 1.
Each replay is checked bit for bit against the same step run eagerly on a copy of the
buffers, with eager work and device synchronisation between replays; the checkpoint
and replay commits are covered, and the folded delta mode (one launch per layer and
step, a graph of two steps alternating the two factor buffers).
"""
import numpy as np
import pytest

from gateddeltanet_linear_attention_amd import binding as gb
from gateddeltanet_linear_attention_amd import synth
from tests.gpu_common import bits, dev_params, dev_tokens, dims_of, say

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
        assert torch.equal(bits(gl.pool), bits(el.pool))
    for k in range(n_replays):
        graph.replay()
        _step(eager_layers)
        torch.cuda.synchronize()
        for li, (gl, el) in enumerate(zip(graph_layers, eager_layers)):
            assert torch.equal(bits(gl.pool), bits(el.pool)), "replay %d layer %d: state differs" % (k, li)
            assert torch.equal(gl.o.view(torch.int16), el.o.view(torch.int16)), "replay %d layer %d: o" % (k, li)
            if gl.ckpt is not None:
                assert torch.equal(bits(gl.ckpt), bits(el.ckpt)), "replay %d layer %d: checkpoints" % (k, li)
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
            assert torch.equal(bits(gl.pool), bits(el.pool)), "replay %d layer %d: state differs" % (k, li)
            assert torch.equal(gl.o.view(torch.int16), el.o.view(torch.int16)), "replay %d layer %d: o" % (k, li)
            for j in (0, 1):
                assert torch.equal(bits(gl.deltas[j]), bits(el.deltas[j])), "replay %d layer %d: factors" % (k, li)
            assert int(gl.status.abs().sum()) == 0 and int(el.status.abs().sum()) == 0
    say("graph replays of folded steps match eager steps")
