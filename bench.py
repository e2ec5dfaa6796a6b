#!/usr/bin/env python3
"""Throughput of the K=3 draft-verification step of the gated delta rule on one MI355X.

A step is one speculative-decoding verification round of a batch through L
GatedDeltaNet layers, in the order a target model runs it: one
gdn_verify_window_select_commit launch per layer.  Each row first commits its
previous window (rollback to the accepted length: the row's entry of the device
slot table is pointed at that window's accepted checkpoint, accepted counts ~
Binomial(3, 0.85) resident on the device; nothing is copied), then runs its previous
bonus token and 3 drafts from that state, publishing the state after every token
into the row's other bank of pool slots.  The same step as two launches per layer
(gdn_verify_window_select for every layer, then gdn_commit_select) is a side line, and so
is the headline step replayed from a HIP graph (the launch gaps removed).
Inputs are synthetic (seeded), at the head shape of a hybrid GatedDeltaNet layer:
16 q/k heads, 32 value heads, d_k = d_v = 128, fp32 128x128 state per value head,
bf16 q/k/v/o.

Workload of the headline line: 16 concurrent requests, every row K=3 (4 tokens per
window): 16 x 32 x 4 = 2048 head-token updates per layer, L = 12 layers per step
by default.  Every layer has its own state pool, checkpoints and tokens (160 MiB),
so a step touches 1.9 GB and the state a verify reads was written a whole step
earlier: it streams from HBM, not from the 256 MB last-level cache.  `roofline` is
the verify launch's algorithmic bytes over its mean duration (HIP events on the
launch stream), with the calibrated HBM traffic from the committed rocprofv3
counter summary when it was taken on the current kernel sources.

Reported beside the headline, on the same synthetic data: the same step with dense
checkpoints in a separate buffer and a copy commit (gdn_verify_window +
gdn_commit_accepted), batch 1 (eager and HIP-graph steps), mixed draft lengths, the
other rollback forms (replay, delta checkpoints with a fold commit or folded into the
next verify),
token trees, raw q/k normalised in the kernels, the in-place decode step, the
2048-token chunked prefill, the mixed ragged transaction (4 prefill rows and 12
verify rows planned per row in one call), the streaming-bandwidth ceilings of a plain
kernel with the verify's and the commit's traffic (context; the roofline's peak stays
8 TB/s), and the fp64 oracle timed on the host cores.

Prints one JSON line (see --help).  --gpus N>1 is refused: the path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN verify head-token updates/s + HBM GB/s vs peak, K=3, batch 1 and 16"
HBM_PEAK_GBPS = 8000.0
STATE_BYTES = 128 * 128 * 4          # one value head's fp32 state
TOKEN_BYTES = 776                    # per head-token: q,k (shared by 2 v-heads) 256 + v 256 + a,b 8 + o 256
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "verify_select_conc16_k3_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "gateddeltanet_linear_attention_amd", "csrc", f)
                  for f in ("gdn_recurrent.hip", "gdn_internal.h", "gdn_device.h")]
V_HEADS = 32


def verify_bytes(row_tokens) -> int:
    """Algorithmic HBM bytes of one verify launch: per (row, v-head) unit, read the
    committed state once, write T_r checkpoints, and move 776 B of token I/O per token."""
    return sum(V_HEADS * ((1 + int(T)) * STATE_BYTES + TOKEN_BYTES * int(T)) for T in row_tokens)


def commit_bytes(n_units: int) -> int:
    return n_units * 2 * STATE_BYTES


TREE4 = [-1, 0, 0, 1]      # draft tree of the tree line: the bonus token, two children, one grandchild
REPLAY_TOKEN_BYTES = 392  # per head-token replayed: k (shared by 2 v-heads) 128 + v 256 + a,b 8


def verify_nockpt_bytes(row_tokens) -> int:
    """Verify without checkpoints: read the committed state, token I/O incl. outputs."""
    return sum(V_HEADS * (STATE_BYTES + TOKEN_BYTES * int(T)) for T in row_tokens)


DELTA_TOKEN_BYTES = (128 + 4) * 4   # delta checkpoint per (token, v-head): c (d_v floats) + alpha + pad


def verify_delta_bytes(row_tokens) -> int:
    """Verify with delta checkpoints: read the state, token I/O, write the factors."""
    return sum(V_HEADS * (STATE_BYTES + (TOKEN_BYTES + DELTA_TOKEN_BYTES) * int(T)) for T in row_tokens)


def fold_bytes(accepted) -> int:
    """Fold commit: read and write the state, read a_r + 1 tokens' keys (128 B per v-head)
    and delta checkpoints."""
    return sum(V_HEADS * (2 * STATE_BYTES + (128 + DELTA_TOKEN_BYTES) * (int(a) + 1)) for a in accepted)


def folded_verify_bytes(row_tokens, accepted) -> int:
    """Verify that first folds the previous window: read the state, write the folded
    state back, read the previous window's a_r + 1 keys and delta checkpoints, token
    I/O and the new window's delta checkpoints."""
    return sum(V_HEADS * (2 * STATE_BYTES + (TOKEN_BYTES + DELTA_TOKEN_BYTES) * int(T)
                          + (128 + DELTA_TOKEN_BYTES) * (int(a) + 1)) for T, a in zip(row_tokens, accepted))


def replay_bytes(accepted) -> int:
    """Replay commit: read and write the state, re-read a_r + 1 tokens' inputs."""
    return sum(V_HEADS * (2 * STATE_BYTES + REPLAY_TOKEN_BYTES * (int(a) + 1)) for a in accepted)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(n_launch_bytes: int):
    """HBM bytes per verify launch from the committed counter summary, or None when
    it is missing or was taken on a different kernel source."""
    try:
        with open(PROFILE_COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


class VerifySet:
    """One buffer set: state pool, checkpoints, a window of tokens, accepted counts,
    and the two prepared C-ABI calls of a step."""

    def __init__(self, gb, synth, dims, Ts, seed, stream, replay=False, parents=None, delta=False,
                 folded=False, select=False, two_sets=False, select_commit=False):
        select = select or select_commit
        raw_qk = bool(dims.flags & gb.QK_L2NORM)
        import numpy as np
        import torch
        shape = synth.FULL
        Hv, d = shape.n_v_heads, shape.d
        Ts = np.asarray(Ts, np.int32)
        B, N = int(Ts.size), int(Ts.sum())
        g = synth.streams(seed, 3)
        A_log, dt_bias = synth.head_params(g[0], shape)
        tok = synth.tokens(g[1], shape, N, raw_qk=raw_qk)
        acc = synth.accepted_counts(g[2], Ts - 1)
        dev = "cuda"
        self.t = dict(q=torch.from_numpy(tok.q).to(torch.bfloat16).to(dev),
                      k=torch.from_numpy(tok.k).to(torch.bfloat16).to(dev),
                      v=torch.from_numpy(tok.v).to(torch.bfloat16).to(dev),
                      a=torch.from_numpy(tok.a).to(dev), b=torch.from_numpy(tok.b).to(dev),
                      A_log=torch.from_numpy(A_log).to(dev), dt_bias=torch.from_numpy(dt_bias).to(dev))
        gen = torch.Generator(device="cpu").manual_seed(seed)
        self.pool = (0.05 * torch.randn(B, Hv, d, d, generator=gen)).to(dev)
        self.ckpt = None if (replay or delta or folded or select) else torch.empty(B, 4, Hv, d, d, device=dev)
        self.o = torch.empty(N, Hv, d, dtype=torch.bfloat16, device=dev)
        self.acc = torch.from_numpy(acc).to(dev)
        self.status = torch.zeros((B + 31) // 32, dtype=torch.int32, device=dev)
        rows = np.arange(B, dtype=np.int32)
        if select:  # checkpoints into two pool banks per row, used alternately; commit selects
            start = self.pool
            self.pool = torch.empty(9 * B, Hv, d, d, device=dev)
            self.pool[8 * B:] = start
            self.table = torch.arange(8 * B, 9 * B, dtype=torch.int32, device=dev)
            banks = [2 * rows + j for j in (0, 1)]
            sv = [gb.prepare_verify_window_select(dims, Ts, **self.t, state_pool=self.pool, slot_table=self.table,
                                                  bank=banks[j], o=self.o, status=self.status, stream=stream)
                  for j in (0, 1)]
            sc = [gb.prepare_commit_select(dims, Ts, self.acc, banks[j], self.pool, self.table, self.status,
                                           stream=stream) for j in (0, 1)]
            phase = [0]

            def verify():
                sv[phase[0]]()

            def commit():
                sc[phase[0]]()
                phase[0] ^= 1
            self.verify, self.commit = verify, commit
            if select_commit:  # the previous window's select inside the next verify: no commit launch
                svc = [gb.prepare_verify_window_select_commit(
                    dims, Ts, Ts, banks[j], self.acc, **self.t, state_pool=self.pool, slot_table=self.table,
                    bank=banks[1 - j], o=self.o, status=self.status, stream=stream) for j in (0, 1)]
                cphase = [None]

                def verify_commit():
                    if cphase[0] is None:
                        sv[0]()
                        cphase[0] = 0
                    else:
                        svc[cphase[0]]()
                        cphase[0] ^= 1
                self.verify, self.commit = verify_commit, (lambda: None)
        elif folded:  # each verify first folds the previous window's accepted prefix: no commit launch
            self.deltas = [torch.empty(gb.delta_shape(dims, B), device=dev) for _ in range(2)]
            first = gb.prepare_verify_window_delta(dims, Ts, **self.t, state_pool=self.pool, src_slot=rows,
                                                   delta=self.deltas[0], o=self.o, stream=stream)
            fold = [gb.prepare_verify_window_delta_fold(dims, Ts, **self.t, state_pool=self.pool, slot=rows,
                                                        delta=self.deltas[1 - j], o=self.o, prev_row_tokens=Ts,
                                                        prev_k=self.t["k"], prev_delta=self.deltas[j],
                                                        prev_accepted=self.acc, status=self.status,
                                                        stream=stream) for j in (0, 1)]
            phase = [None]

            def verify():
                if phase[0] is None:
                    first()
                    phase[0] = 0
                else:
                    fold[phase[0]]()
                    phase[0] ^= 1
            self.verify = verify
            self.commit = lambda: None
        elif delta:  # delta checkpoints: commit folds the accepted prefix in place
            self.delta = torch.empty(gb.delta_shape(dims, B), device=dev)
            self.verify = gb.prepare_verify_window_delta(dims, Ts, **self.t, state_pool=self.pool, src_slot=rows,
                                                         delta=self.delta, o=self.o, stream=stream)
            self.commit = gb.prepare_commit_delta(dims, Ts, self.t["k"], self.delta, self.acc, self.pool,
                                                  src_slot=rows, dst_slot=rows, status=self.status, stream=stream)
        elif replay and two_sets:  # replay from one slot set into the other, the sets alternating
            self.ckpt = None
            start = self.pool
            self.pool = torch.empty(2 * B, Hv, d, d, device=dev)
            self.pool[:B] = start
            tin = {k: v for k, v in self.t.items()}
            sv = [gb.prepare_verify_window(dims, Ts, **self.t, state_pool=self.pool, src_slot=rows + B * j,
                                           ckpt=None, o=self.o, stream=stream) for j in (0, 1)]
            sc = [gb.prepare_commit_replay(dims, Ts, **tin, accepted=self.acc, state_pool=self.pool,
                                           src_slot=rows + B * j, dst_slot=rows + B * (1 - j), status=self.status,
                                           stream=stream) for j in (0, 1)]
            phase = [0]

            def verify():
                sv[phase[0]]()

            def commit():
                sc[phase[0]]()
                phase[0] ^= 1
            self.verify, self.commit = verify, commit
        elif replay:  # no checkpoints: commit re-runs the accepted prefix in place
            self.ckpt = None
            self.verify = gb.prepare_verify_window(dims, Ts, **self.t, state_pool=self.pool, src_slot=rows,
                                                   ckpt=None, o=self.o, stream=stream)
            tin = {k: v for k, v in self.t.items()}
            self.commit = gb.prepare_commit_replay(dims, Ts, **tin, accepted=self.acc, state_pool=self.pool,
                                                   src_slot=rows, dst_slot=rows, status=self.status,
                                                   stream=stream)
        elif parents is not None:  # a draft tree per row; commit the accepted path's last node
            self.verify = gb.prepare_verify_tree(dims, Ts, np.tile(parents, B), **self.t, state_pool=self.pool,
                                                 src_slot=rows, ckpt=self.ckpt, o=self.o, stream=stream)
            self.commit = gb.prepare_commit_accepted(dims, Ts, self.ckpt, self.acc, self.pool, dst_slot=rows,
                                                     status=self.status, stream=stream)
        else:
            self.verify = gb.prepare_verify_window(dims, Ts, **self.t, state_pool=self.pool, src_slot=rows,
                                                   ckpt=self.ckpt, o=self.o, stream=stream)
            self.commit = gb.prepare_commit_accepted(dims, Ts, self.ckpt, self.acc, self.pool, dst_slot=rows,
                                                     status=self.status, stream=stream)
        self.acc_host = acc
        self.select = select
        # the window's tokens, for the CPU baseline
        self.tok, self.A_log, self.dt_bias, self.T, self.B = tok, A_log, dt_bias, Ts, B

    def committed_states(self):
        """The rows' committed states (checkpoint select: the pool slots the table names)."""
        return self.pool[self.table.long()] if self.select else self.pool


def run_steps(layers, steps, warmup, stream, torch):
    """Warm-up, then `steps` timed steps, bracketed by synchronisation.  A step runs
    every layer's verify back to back, then every layer's commit.  Events recorded
    on the launch stream around each step's run of verify launches, and of commit
    launches, give the mean launch durations (their span / L)."""
    def step():
        for s in layers:
            s.verify()
        for s in layers:
            s.commit()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        for s in layers:
            s.verify()
        ev[i][1].record(stream)
        for s in layers:
            s.commit()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    verify_ms = [a.elapsed_time(b) / len(layers) for a, b, _ in ev]
    commit_ms = [b.elapsed_time(c) / len(layers) for _, b, c in ev]
    return wall, verify_ms, commit_ms


def measure_graph(gb, synth, torch, Ts, steps, warmup, n_layers, seed0, replay=False, folded=False,
                  select=False, select_commit=False):
    """The same step captured once as a HIP graph on a side stream and replayed:
    wall time per step (launch costs of the 2 L calls removed from the host side).
    folded: one launch per layer and step (the previous window's commit inside the
    next verify); folded and select graphs hold two steps, so the two factor buffers
    (pool banks) alternate as they do in a real decode loop."""
    dims = gb.Dims(16, 32, 128, 128, 3)
    cap = torch.cuda.Stream()
    sets = [VerifySet(gb, synth, dims, Ts, seed0 + i, cap, replay, folded=folded, select=select,
                      select_commit=select_commit) for i in range(n_layers)]
    per_replay = 2 if (folded or select or select_commit) else 1

    def step():
        for s in sets:
            s.verify()
        for s in sets:
            s.commit()
    with torch.cuda.stream(cap):
        for _ in range(3):
            step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for _ in range(per_replay):
            step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for s in sets:
        assert int(s.status.abs().sum()) == 0
    upd = int(sum(Ts)) * V_HEADS * n_layers * steps * per_replay
    return {"ms_per_layer": 1e3 * wall / (steps * per_replay) / n_layers, "head_token_updates_per_s": upd / wall}


def decode_bytes(n_rows: int) -> int:
    """One decode launch: read and write each (row, head) state once, 776 B of token I/O."""
    return n_rows * V_HEADS * (2 * STATE_BYTES + TOKEN_BYTES)


def measure_decode(gb, synth, torch, B, steps, warmup, n_layers, stream, seed0, two_sets=False):
    """Decode of one token per row through n_layers layers (each with its own state
    pool and tokens), HIP events around each step's run of launches.  In place by
    default; two_sets: each layer's pool holds two slot sets and the steps alternate
    between them (new state to the other set, twice the state memory)."""
    import numpy as np
    dims = gb.Dims(16, 32, 128, 128, 3)
    rows = np.arange(B, dtype=np.int32)
    calls, keep = [], []
    for li in range(n_layers):
        g = synth.streams(seed0 + li, 2)
        A_log, dt_bias = synth.head_params(g[0], synth.FULL)
        tok = synth.tokens(g[1], synth.FULL, B)
        t = dict(q=torch.from_numpy(tok.q).to(torch.bfloat16).cuda(), k=torch.from_numpy(tok.k).to(torch.bfloat16).cuda(),
                 v=torch.from_numpy(tok.v).to(torch.bfloat16).cuda(), a=torch.from_numpy(tok.a).cuda(),
                 b=torch.from_numpy(tok.b).cuda(), A_log=torch.from_numpy(A_log).cuda(),
                 dt_bias=torch.from_numpy(dt_bias).cuda())
        gen = torch.Generator(device="cpu").manual_seed(seed0 + li)
        pool = (0.05 * torch.randn((2 if two_sets else 1) * B, 32, 128, 128, generator=gen)).cuda()
        o = torch.empty(B, 32, 128, dtype=torch.bfloat16, device="cuda")
        if two_sets:
            calls.append([gb.prepare_decode_step(dims, **t, state_pool=pool, src_slot=rows + B * j,
                                                 dst_slot=rows + B * (1 - j), o=o, stream=stream) for j in (0, 1)])
        else:
            c = gb.prepare_decode_step(dims, **t, state_pool=pool, src_slot=rows, dst_slot=rows, o=o, stream=stream)
            calls.append([c, c])
        keep.append((t, pool, o))
    for i in range(warmup):
        for c in calls:
            c[i % 2]()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        for c in calls:
            c[(warmup + i) % 2]()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / (steps * n_layers)
    nb = decode_bytes(B)
    return {"rows": B, "in_place": not two_sets, "decode_us_mean": us, "algorithmic_bytes_per_launch": nb,
            "gbps": nb / (us * 1e-6) / 1e9, "frac_of_hbm_peak": nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "head_token_updates_per_s": B * V_HEADS * n_layers * steps / wall}


def measure_transaction(gb, synth, torch, stream, reps):
    """The mixed ragged transaction (16 rows in one packed batch: 4 prefills of
    U{256..4096} tokens from the zero state, 12 K=3 verify windows with all four
    checkpoints), planned per row and launched by gdn_run_transaction on both routes;
    events on the launch stream around `reps` back-to-back transactions.  Also the
    host planner's own time per call."""
    import numpy as np
    m = synth.mixed_workload()
    dims = gb.Dims(16, 32, 128, 128, 3)
    B, Hv, d = m.n_rows, 32, 128
    lens = m.transaction_lens()
    rows = np.arange(B, dtype=np.int32)
    is_pf = m.is_prefill
    n_ck = np.where(is_pf, 0, 4).astype(np.int32)
    src = np.where(is_pf, -1, rows).astype(np.int32)
    dst = np.where(is_pf, rows, -1).astype(np.int32)
    tx = m.transaction_tokens()
    dev = "cuda"
    t = dict(q=torch.from_numpy(tx.q).to(torch.bfloat16).to(dev), k=torch.from_numpy(tx.k).to(torch.bfloat16).to(dev),
             v=torch.from_numpy(tx.v).to(torch.bfloat16).to(dev), a=torch.from_numpy(tx.a).to(dev),
             b=torch.from_numpy(tx.b).to(dev), A_log=torch.from_numpy(m.A_log).to(dev),
             dt_bias=torch.from_numpy(m.dt_bias).to(dev))
    gen = torch.Generator(device="cpu").manual_seed(1005)
    pool = (0.05 * torch.randn(B, Hv, d, d, generator=gen)).to(dev)
    ckpt = torch.empty(B, 4, Hv, d, d, device=dev)
    o = torch.empty(int(lens.sum()), Hv, d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(gb.gdn_chunked_workspace_bytes(dims, lens), dtype=torch.uint8, device=dev)

    def call():
        gb.gdn_run_transaction(dims, lens, n_ck, **t, state_pool=pool, src_slot=src, dst_slot=dst, ckpt=ckpt,
                               o=o, workspace=ws, stream=stream)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        call()
    ev[1].record(stream)
    torch.cuda.synchronize()
    us = 1e3 * ev[0].elapsed_time(ev[1]) / reps
    n_plan = 2000
    t0 = time.perf_counter()
    for _ in range(n_plan):
        gb.gdn_plan_transaction(dims, lens)
    plan_us = 1e6 * (time.perf_counter() - t0) / n_plan
    n_tok = int(lens.sum())
    return {"workload": "mixed_transaction_4_prefills_12_verify_rows", "row_tokens": [int(x) for x in lens],
            "us_per_transaction": us, "tokens": n_tok, "head_token_updates_per_s": n_tok * Hv / (us * 1e-6),
            "planner_host_us_per_call": plan_us,
            "planner_note": "host time of the Python binding call (marshalling included)"}


def measure_ceilings(torch, stream, sets: int = 12, reps: int = 240):
    """Streaming ceilings for context, in the same process: a plain kernel that reads
    32 MiB once and writes it to 4 copies (the verify's 1 read : 4 writes of state, none
    of its work) and to 1 copy (a plain copy, the commit's traffic), over `sets` rotating
    buffer sets so that every launch streams from HBM; HIP events on the launch stream."""
    import ctypes
    path = os.path.join(ROOT, "gateddeltanet_linear_attention_amd", "libgdn_probe.so")
    if not os.path.exists(path):
        raise RuntimeError("%s is missing: run python -m gateddeltanet_linear_attention_amd.build" % path)
    lib = ctypes.CDLL(path)
    lib.gdn_probe_stream.restype = ctypes.c_int
    lib.gdn_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_void_p]
    n = 32 << 20  # bytes read per launch
    src = [torch.zeros(n // 4, device="cuda") for _ in range(sets)]          # 32 MiB of fp32
    dst = [torch.empty(4 * (n // 4), device="cuda") for _ in range(sets)]    # room for 4 copies
    shapes = {0: "512x2", 1: "256x2_prio", 2: "256x4_prio"}
    out = {}
    for n_out, name in ((4, "stream_1r4w_32MiB"), (1, "copy_1r1w_32MiB")):
        per = {}
        for shape, sname in shapes.items():
            def launch(i):
                rc = lib.gdn_probe_stream(src[i % sets].data_ptr(), dst[i % sets].data_ptr(), n, n_out, shape,
                                          ctypes.c_void_p(stream.cuda_stream))
                if rc != 0:
                    raise RuntimeError("gdn_probe_stream returned %d" % rc)
            for i in range(2 * sets):
                launch(i)
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for i in range(reps):
                launch(i)
            ev[1].record(stream)
            torch.cuda.synchronize()
            per[sname] = 1e3 * ev[0].elapsed_time(ev[1]) / reps
        best = min(per, key=per.get)
        us = per[best]
        gbps = (1 + n_out) * n / (us * 1e-6) / 1e9
        out[name] = {"us": us, "gbps": gbps, "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS, "schedule": best,
                     "us_per_schedule": per}
    del src, dst
    torch.cuda.empty_cache()
    return out


def cpu_baseline(s: "VerifySet", seconds: float, seconds_1thread: float):
    """The fp64 oracle on the host, on the same window as the GPU step (a bounded
    sample: repeated windows for about `seconds` of work), with every host core the
    oracle uses and again on one thread."""
    import numpy as np
    import oracle
    tok = s.tok
    S0 = s.committed_states().double().cpu().numpy()
    out = dict(S_final=np.zeros(S0.shape), ckpt=np.zeros((s.B, 4) + S0.shape[1:]),
               o=np.zeros((int(s.T.sum()),) + S0.shape[1:3]))

    def rate(budget, n_threads):
        oracle.verify_window(s.T, tok.q, tok.k, tok.v, tok.a, tok.b, s.A_log, s.dt_bias, S0,
                             n_threads=n_threads, nan_fill=False, out=out)  # untimed first pass
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.verify_window(s.T, tok.q, tok.k, tok.v, tok.a, tok.b, s.A_log, s.dt_bias, S0,
                                 n_threads=n_threads, nan_fill=False, out=out)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return n, el, n * int(s.T.sum()) * S0.shape[1] / el

    n, el, value = rate(seconds, None)
    cores = oracle.threads_used()
    n1, el1, value1 = rate(seconds_1thread, 1)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": value, "unit": "head-token updates/s", "cores": cores,
            "kind": "oracle",
            "sample": "%d repetitions of one %d-row K=%d verify window (%d head-token updates each), "
                      "fp64, %.1f s" % (n, s.B, int(s.T[0]) - 1, int(s.T.sum()) * S0.shape[1], el),
            "value_1thread": value1,
            "sample_1thread": "%d repetitions, %.1f s" % (n1, el1),
            "cpu_model": cpu_model}


MFMA_F32_PEAK_TFLOPS = 157.3


def prefill_flops(L: int, n_heads: int = 32, d: int = 128, C: int = 64) -> float:
    """Algorithmic flops of the chunked prefill, every chunk contraction counted as a
    dense 64-token tile: KK^T, QK^T, W = T K, U' = T V (4 x 2 C^2 d), W S^T, Q S^T,
    U^T K (3 x 2 C d^2) and P U (2 C^2 d) per (chunk, value head)."""
    per_chunk = 4 * 2 * C * C * d + 3 * 2 * C * d * d + 2 * C * C * d
    return float((L + C - 1) // C) * n_heads * per_chunk


def measure_prefill(gb, synth, torch, stream, reps, raw_qk=False):
    """The 2048-token chunked prefill (1 row, 32 value heads, chunk 64, checkpoints at
    the last 4 positions), timed with events on the launch stream.  raw_qk: q and k
    unnormalised, normalised inside the kernels (GDN_QK_L2NORM)."""
    w = synth.prefill_workload(raw_qk=raw_qk)
    dims = gb.Dims(16, 32, 128, 128, 3, gb.QK_L2NORM if raw_qk else 0)
    tok = w.tokens()
    dev = "cuda"
    t = dict(q=torch.from_numpy(tok.q).to(torch.bfloat16).to(dev),
             k=torch.from_numpy(tok.k).to(torch.bfloat16).to(dev),
             v=torch.from_numpy(tok.v).to(torch.bfloat16).to(dev),
             a=torch.from_numpy(tok.a).to(dev), b=torch.from_numpy(tok.b).to(dev),
             A_log=torch.from_numpy(w.A_log).to(dev), dt_bias=torch.from_numpy(w.dt_bias).to(dev))
    L = int(w.lens[0])
    pool = torch.zeros(1, 32, 128, 128, device=dev)
    ckpt = torch.empty(1, 4, 32, 128, 128, device=dev)
    o = torch.empty(L, 32, 128, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(gb.gdn_chunked_workspace_bytes(dims, w.lens), dtype=torch.uint8, device=dev)

    def call():
        gb.gdn_chunked_prefill_with_checkpoints(dims, w.lens, w.n_tail, **t, state_pool=pool, src_slot=[-1],
                                                dst_slot=[0], ckpt=ckpt, o=o, workspace=ws, stream=stream)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * a.elapsed_time(b) / reps
    fl = prefill_flops(L)
    return {"workload": "prefill_2048_chunk64_tail4", "tokens": L, "us_per_call": us,
            "head_token_updates_per_s": L * 32 / (us * 1e-6),
            "algorithmic_tflops": fl / (us * 1e-6) / 1e12, "mfma_f32_peak_tflops": MFMA_F32_PEAK_TFLOPS,
            "frac_of_mfma_f32_peak": fl / (us * 1e-6) / 1e12 / MFMA_F32_PEAK_TFLOPS,
            "algorithmic_flops_per_call": fl}


def measure(gb, synth, torch, Ts, steps, warmup, n_layers, stream, seed0, replay=False, parents=None,
            delta=False, folded=False, raw_qk=False, select=False, two_sets=False, select_commit=False):
    """Steps over n_layers layers of windows with per-row token counts Ts (replay:
    verify without checkpoints, commit by replay; parents: one draft tree per row;
    delta: delta checkpoints folded by a commit launch; folded: folded by the next
    verify, one launch per layer per step; raw_qk: q and k normalised inside the kernels)."""
    dims = gb.Dims(16, 32, 128, 128, 3, gb.QK_L2NORM if raw_qk else 0)
    sets = [VerifySet(gb, synth, dims, Ts, seed0 + i, stream, replay, parents, delta, folded, select, two_sets,
                      select_commit) for i in range(n_layers)]
    wall, verify_ms, commit_ms = run_steps(sets, steps, warmup, stream, torch)
    for s in sets:
        assert int(s.status.abs().sum()) == 0
    units = len(Ts) * V_HEADS
    upd_per_layer = int(sum(Ts)) * V_HEADS
    if folded:
        vb = sum(folded_verify_bytes(Ts, s.acc_host) for s in sets) / len(sets)
        cb = 0
    elif select or select_commit:  # same verify traffic; the commit moves no state
        vb = verify_bytes(Ts)
        cb = 0
    elif delta:
        vb = verify_delta_bytes(Ts)
        cb = sum(fold_bytes(s.acc_host) for s in sets) / len(sets)
    elif replay:
        vb = verify_nockpt_bytes(Ts)
        cb = sum(replay_bytes(s.acc_host) for s in sets) / len(sets)
    else:
        vb = verify_bytes(Ts)
        cb = commit_bytes(units)
    vms = sum(verify_ms) / len(verify_ms)
    cms = sum(commit_ms) / len(commit_ms)
    srt = sorted(verify_ms)
    return sets, {
        "ms_per_step": 1e3 * wall / steps,
        "updates_per_s": upd_per_layer * n_layers * steps / wall,
        "verify_ms_mean": vms,
        "verify_ms_p10": srt[len(srt) // 10],
        "verify_ms_p50": srt[len(srt) // 2],
        "verify_ms_p90": srt[(9 * len(srt)) // 10],
        "verify_updates_per_s": upd_per_layer / (vms * 1e-3),
        "verify_bytes": vb,
        "verify_gbps": vb / (vms * 1e-3) / 1e9,
        "commit_ms_mean": cms,
        "commit_bytes": cb,
        "commit_gbps": cb / (cms * 1e-3) / 1e9 if cb else None,
        "step_gbps": (vb + cb) * n_layers * steps / wall / 1e9,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=12,
                    help="GatedDeltaNet layers per step, each with its own 160 MiB of buffers")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-seconds-1thread", type=float, default=4.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batch1", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-mixed", action="store_true")
    ap.add_argument("--no-replay", action="store_true")
    ap.add_argument("--no-tree", action="store_true")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the line with q/k normalised inside the kernels")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replays of the batch-1 step")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the 2048-token chunked prefill and print its figures")
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--transaction-only", action="store_true",
                    help="time only the mixed ragged transaction and print its figures")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode lines (16 rows in place, into a second slot set, batch 1)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the streaming-bandwidth ceilings (plain 1:4 and 1:1 streams) reported for context")
    ap.add_argument("--no-transaction", action="store_true",
                    help="skip the mixed ragged transaction (4 prefills + 12 verify rows); --no-prefill skips it too")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode side lines")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline step and the copy-commit step (whose commit kernel, a plain copy "
                         "of known size, calibrates the HBM counters); every other line is skipped")
    args = ap.parse_args()
    if args.headline_only:
        for flag in ("no_cpu_baseline", "no_batch1", "no_mixed", "no_prefill", "no_replay", "no_tree", "no_fused",
                     "no_graph", "no_ceilings", "no_transaction", "no_decode"):
            setattr(args, flag, True)
    if args.gpus != 1:
        print("bench.py: this path runs on one GPU; --gpus %d is not supported "
              "(rows and heads are independent, see the design notes on sharding)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gateddeltanet_linear_attention_amd import binding as gb
    from gateddeltanet_linear_attention_amd import synth
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    gb.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    if args.prefill_only:
        print(json.dumps(measure_prefill(gb, synth, torch, stream, args.prefill_reps)), flush=True)
        return
    if args.transaction_only:
        print(json.dumps(measure_transaction(gb, synth, torch, stream, args.prefill_reps)), flush=True)
        return
    if args.decode_only:
        print(json.dumps({
            "conc16": measure_decode(gb, synth, torch, 16, args.steps, args.warmup, args.layers, stream, 900),
            "conc16_two_slot_sets": measure_decode(gb, synth, torch, 16, args.steps, args.warmup, args.layers,
                                                   stream, 900, two_sets=True),
            "batch1": measure_decode(gb, synth, torch, 1, args.steps, args.warmup, args.layers, stream, 950)}),
            flush=True)
        return

    import numpy as np
    sets_sel, rs = measure(gb, synth, torch, [4] * 16, args.steps, args.warmup, args.layers, stream, 500,
                           select_commit=True)
    rsel = None
    if not args.headline_only:
        _, rsel = measure(gb, synth, torch, [4] * 16, args.steps, args.warmup, args.layers, stream, 500,
                          select=True)
    _, r16 = measure(gb, synth, torch, [4] * 16, args.steps, args.warmup, args.layers, stream, 500)

    def side(r, Ts):
        return {"row_tokens": [int(t) for t in Ts],
                "head_token_updates_per_s": r["updates_per_s"],
                "ms_per_layer": r["ms_per_step"] / args.layers,
                "verify_us_mean": 1e3 * r["verify_ms_mean"], "verify_us_p50": 1e3 * r["verify_ms_p50"],
                "verify_gbps": r["verify_gbps"], "verify_frac_of_hbm_peak": r["verify_gbps"] / HBM_PEAK_GBPS,
                "commit_us_mean": 1e3 * r["commit_ms_mean"], "commit_gbps": r["commit_gbps"]}
    out_copy = side(r16, [4] * 16)
    out_copy["mode"] = ("dense checkpoints in a separate buffer (gdn_verify_window), commit copies the accepted "
                        "one into the row's pool slot (gdn_commit_accepted)")
    out_sel = None
    if rsel is not None:
        out_sel = side(rsel, [4] * 16)
        out_sel["mode"] = ("checkpoint select, the commit its own launch (gdn_verify_window_select, then "
                           "gdn_commit_select): two launches per layer-step")
    out_graph16 = None
    if not (args.no_graph or args.headline_only):
        g16 = measure_graph(gb, synth, torch, [4] * 16, args.steps, args.warmup, args.layers, 500,
                            select_commit=True)
        out_graph16 = {"mode": "the headline step replayed from a HIP graph (two steps per replay, banks "
                               "alternating)", "ms_per_layer": g16["ms_per_layer"],
                       "head_token_updates_per_s": g16["head_token_updates_per_s"]}
    out_b1 = out_mixed = None
    if not args.no_batch1:
        _, r1s = measure(gb, synth, torch, [4], args.steps, args.warmup, args.layers, stream, 600,
                         select_commit=True)
        _, r1t = measure(gb, synth, torch, [4], args.steps, args.warmup, args.layers, stream, 600, select=True)
        _, r1 = measure(gb, synth, torch, [4], args.steps, args.warmup, args.layers, stream, 600)
        out_b1 = side(r1s, [4])
        out_b1["mode"] = "as the headline: checkpoint select, the commit inside the next verify"
        out_b1["select_two_launches"] = side(r1t, [4])
        out_b1["copy_commit"] = side(r1, [4])
        if not args.no_graph:
            out_b1["graph"] = measure_graph(gb, synth, torch, [4], args.steps, args.warmup, args.layers, 600,
                                            select_commit=True)
            out_b1["graph_select_two_launches"] = measure_graph(gb, synth, torch, [4], args.steps, args.warmup,
                                                                args.layers, 600, select=True)
            out_b1["graph_copy_commit"] = measure_graph(gb, synth, torch, [4], args.steps, args.warmup,
                                                        args.layers, 600)
            out_b1["graph_replay_mode"] = measure_graph(gb, synth, torch, [4], args.steps, args.warmup,
                                                        args.layers, 600, replay=True)
            if not args.no_replay:
                out_b1["graph_folded_delta_mode"] = measure_graph(gb, synth, torch, [4], args.steps, args.warmup,
                                                                  args.layers, 600, folded=True)
    if not args.no_mixed:
        Ts = (synth.verify_workload("conc16").draft_lens + 1).astype(np.int32)
        _, rm = measure(gb, synth, torch, Ts, args.steps, args.warmup, args.layers, stream, 700)
        out_mixed = side(rm, Ts)
    out_replay = None
    if not args.no_replay:
        _, rr = measure(gb, synth, torch, [4] * 16, args.steps, args.warmup, args.layers, stream, 500,
                        replay=True)
        out_replay = {"mode": "verify without checkpoints + commit by replay of the accepted prefix",
                      "head_token_updates_per_s": rr["updates_per_s"],
                      "ms_per_layer": rr["ms_per_step"] / args.layers,
                      "verify_us_mean": 1e3 * rr["verify_ms_mean"], "verify_gbps": rr["verify_gbps"],
                      "replay_us_mean": 1e3 * rr["commit_ms_mean"], "replay_gbps": rr["commit_gbps"],
                      "step_gbps": rr["step_gbps"],
                      "step_algorithmic_bytes_per_layer": rr["verify_bytes"] + rr["commit_bytes"]}
        _, rr2 = measure(gb, synth, torch, [4] * 16, args.steps, args.warmup, args.layers, stream, 500,
                         replay=True, two_sets=True)
        out_replay["two_slot_sets"] = {
            "mode": "the replay writes into a second slot set, the two sets used alternately (twice the state memory)",
            "head_token_updates_per_s": rr2["updates_per_s"], "ms_per_layer": rr2["ms_per_step"] / args.layers,
            "verify_us_mean": 1e3 * rr2["verify_ms_mean"], "replay_us_mean": 1e3 * rr2["commit_ms_mean"],
            "replay_gbps": rr2["commit_gbps"]}
    out_delta = None
    if not args.no_replay:
        _, rd = measure(gb, synth, torch, [4] * 16, args.steps, args.warmup, args.layers, stream, 500, delta=True)
        out_delta = {"mode": "verify storing each step's rank-1 factors + commit by folding them",
                     "head_token_updates_per_s": rd["updates_per_s"],
                     "ms_per_layer": rd["ms_per_step"] / args.layers,
                     "verify_us_mean": 1e3 * rd["verify_ms_mean"], "verify_gbps": rd["verify_gbps"],
                     "fold_us_mean": 1e3 * rd["commit_ms_mean"], "fold_gbps": rd["commit_gbps"],
                     "step_gbps": rd["step_gbps"],
                     "step_algorithmic_bytes_per_layer": rd["verify_bytes"] + rd["commit_bytes"]}
    out_folded = None
    if not args.no_replay:
        _, rf = measure(gb, synth, torch, [4] * 16, args.steps, args.warmup, args.layers, stream, 500,
                        folded=True)
        out_folded = {"mode": "delta checkpoints; each verify first folds the previous window's accepted "
                              "prefix (one launch per layer per step)",
                      "head_token_updates_per_s": rf["updates_per_s"],
                      "ms_per_layer": rf["ms_per_step"] / args.layers,
                      "verify_us_mean": 1e3 * rf["verify_ms_mean"], "verify_us_p50": 1e3 * rf["verify_ms_p50"],
                      "verify_gbps": rf["verify_gbps"],
                      "verify_frac_of_hbm_peak": rf["verify_gbps"] / HBM_PEAK_GBPS,
                      "step_algorithmic_bytes_per_layer": rf["verify_bytes"]}
    out_fused = None
    if not args.no_fused:
        _, rq = measure(gb, synth, torch, [4] * 16, args.steps, args.warmup, args.layers, stream, 500,
                        raw_qk=True)
        out_fused = side(rq, [4] * 16)
        out_fused["mode"] = ("raw q/k normalised inside the kernels (GDN_QK_L2NORM), checkpoint verify + "
                             "commit; same algorithmic bytes as the headline")
        # what the fusion removes: a separate pass reading raw bf16 q and k and writing
        # them back normalised, per layer-step
        out_fused["saved_pass_bytes_per_layer"] = 2 * 2 * 16 * 4 * 16 * 128 * 2
        if not args.no_prefill:
            out_fused["prefill_us_per_call"] = measure_prefill(gb, synth, torch, stream, args.prefill_reps,
                                                               raw_qk=True)["us_per_call"]
    decode = None if args.no_decode else {"conc16": measure_decode(gb, synth, torch, 16, args.steps, args.warmup, args.layers, stream, 900),
              "conc16_two_slot_sets": measure_decode(gb, synth, torch, 16, args.steps, args.warmup, args.layers,
                                                     stream, 900, two_sets=True),
              "batch1": measure_decode(gb, synth, torch, 1, args.steps, args.warmup, args.layers, stream, 950)}
    out_tree = None
    if not args.no_tree:
        tree = np.array(TREE4, np.int32)
        _, rt = measure(gb, synth, torch, [4] * 16, args.steps, args.warmup, args.layers, stream, 800,
                        parents=tree)
        out_tree = side(rt, [4] * 16)
        out_tree["parents"] = TREE4
    prefill = None if args.no_prefill else measure_prefill(gb, synth, torch, stream, args.prefill_reps)
    ceilings = None
    if not args.no_ceilings:
        ceilings = measure_ceilings(torch, stream)
        # ceiling time / kernel time: 1 means the kernel runs as fast as the best plain stream
        ceilings["verify_frac_of_1r4w_ceiling"] = ceilings["stream_1r4w_32MiB"]["us"] / (1e3 * rs["verify_ms_mean"])
        ceilings["commit_frac_of_copy_ceiling"] = ceilings["copy_1r1w_32MiB"]["us"] / (1e3 * r16["commit_ms_mean"])
    transaction = None
    if not (args.no_prefill or args.no_transaction):
        transaction = measure_transaction(gb, synth, torch, stream, args.prefill_reps)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(sets_sel[0], args.cpu_seconds, args.cpu_seconds_1thread)

    traffic = traffic_from_profile(rs["verify_bytes"])
    line = {
        "metric": METRIC,
        "value": rs["updates_per_s"],
        "unit": "head-token updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rs["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": "conc16_k3_verify_select_commit", "rows": 16, "drafts_per_row": 3,
                   "tokens_per_window": 4, "qk_heads": 16, "v_heads": 32, "d_k": 128, "d_v": 128,
                   "state": "fp32", "io": "bf16", "layers_per_step": args.layers},
        "roofline": {"bound": "hbm", "achieved": rs["verify_gbps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": rs["verify_gbps"] / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     "kernel": "recurrent_kernel<128,16,1,4,select,stream,ntload> (gdn_verify_window_select_commit)",
                     "algorithmic_bytes_per_launch": rs["verify_bytes"],
                     "launch_us_mean": 1e3 * rs["verify_ms_mean"],
                     "launch_us_p10": 1e3 * rs["verify_ms_p10"],
                     "launch_us_p50": 1e3 * rs["verify_ms_p50"],
                     "launch_us_p90": 1e3 * rs["verify_ms_p90"]},
        "ms_per_layer": rs["ms_per_step"] / args.layers,
        "verify_head_token_updates_per_s": rs["verify_updates_per_s"],
        "commit_us_mean": 1e3 * rs["commit_ms_mean"],
        "step_gbps": rs["step_gbps"],
        "conc16_k3_copy_commit": out_copy,
        "conc16_k3_select_two_launches": out_sel,
        "conc16_k3_graph": out_graph16,
        "batch1": out_b1,
        "conc16_mixed_k": out_mixed,
        "conc16_k3_replay": out_replay,
        "conc16_tree4": out_tree,
        "conc16_k3_delta": out_delta,
        "conc16_k3_delta_folded": out_folded,
        "conc16_k3_fused_qk_norm": out_fused,
        "decode": decode,
        "prefill": prefill,
        "mixed_transaction": transaction,
        "streaming_ceilings": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
