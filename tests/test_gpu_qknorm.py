"""GPU parity of the fused input side (GDN_QK_L2NORM): q and k arrive as raw
projections and the library normalises them -- k to unit norm, q to norm
1/sqrt(d_k) -- before the rule runs.  The oracle normalises the same raw inputs
itself in fp64 (oracle.l2norm_qk).  Checked here:

* the tiny, batch-1 and concurrency-16 workloads with raw q/k in the checkpoint,
  replay and delta modes against the oracle;
* the result does not depend on the scale of the raw inputs.

The bit-exact properties in this mode (checkpoint j == j+1 decode calls, replay and
delta commits == checkpoint commit, folded verify, chain-shaped trees, transaction
rows == verify, the chunked path's last checkpoint == its final state) are covered
by the fused_l2norm cases of the other GPU test files.
"""
import numpy as np
import pytest

import oracle
from gateddeltanet_linear_attention_amd import binding as gb
from gateddeltanet_linear_attention_amd import synth
from tests.gpu_common import assert_o, assert_state, dev_params, dev_tokens, dims_of, host, say, state_err
from tests.test_gpu_recurrent import run_verify_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("mode", ["checkpoint", "replay", "delta"])
def test_tiny_workload_fused(mode):
    w = synth.verify_workload("tiny", raw_qk=True)
    worst = run_verify_workload(w, n_windows=w.n_windows, check_every=1, mode=mode)
    say("tiny fused %s worst:" % mode, worst)


@pytest.mark.parametrize("mode", ["checkpoint", "replay", "delta"])
def test_batch1_workload_fused(mode):
    w = synth.verify_workload("batch1", n_windows=32, raw_qk=True)
    worst = run_verify_workload(w, n_windows=w.n_windows, check_every=8, mode=mode)
    say("batch1 fused %s worst:" % mode, worst)


@pytest.mark.parametrize("mode", ["checkpoint", "delta"])
def test_conc16_workload_fused(mode):
    w = synth.verify_workload("conc16", n_windows=32, raw_qk=True)
    worst = run_verify_workload(w, n_windows=w.n_windows, check_every=8, mode=mode)
    say("conc16 fused %s worst:" % mode, worst)


def test_fused_result_does_not_depend_on_input_scale():
    """Raw q and k times 4 (exact in bf16) give the same states and outputs up to
    the eps under the root and fp32 rounding; both match the oracle."""
    shape = synth.FULL
    dims = dims_of(shape, raw_qk=True)
    Hv, d = shape.n_v_heads, shape.d
    T = np.array([4, 3, 2, 1, 4, 4], np.int32)
    B = T.size
    g = synth.streams(91, 2)
    A_log, dt_bias = synth.head_params(g[0], shape)
    P = dev_params(A_log, dt_bias)
    tok = synth.tokens(g[1], shape, int(T.sum()), raw_qk=True)
    gen = torch.Generator(device="cpu").manual_seed(9)
    pool = (0.2 * torch.randn(B, Hv, d, d, generator=gen)).cuda()
    res = []
    for c in (1.0, 4.0):
        td = dev_tokens(tok)
        td["q"] = td["q"] * c
        td["k"] = td["k"] * c
        ck = torch.empty(B, 4, Hv, d, d, device="cuda")
        o = torch.empty(int(T.sum()), Hv, d, dtype=torch.bfloat16, device="cuda")
        gb.gdn_verify_window(dims, T, **td, **P, state_pool=pool, src_slot=np.arange(B), ckpt=ck, o=o)
        res.append((ck, o))
    torch.cuda.synchronize()
    qh, kh = oracle.l2norm_qk(tok.q, tok.k)
    ck_o, o_o = oracle.verify_window(T, qh, kh, tok.v, tok.a, tok.b, A_log, dt_bias, host(pool))
    for ck, o in res:
        assert_o(host(o), o_o, "fused outputs")
        for r in range(B):
            assert_state(host(ck[r, :T[r]]), ck_o[r, :T[r]], "fused row %d checkpoints" % r)
    for r in range(B):
        e = state_err(host(res[1][0][r, :T[r]]), host(res[0][0][r, :T[r]]))
        assert e <= 1e-5, "row %d: scaled inputs moved the checkpoints by %.2e" % (r, e)
