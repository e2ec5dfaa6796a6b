"""CPU tests of the C ABI: the library loads, exports every entry point that
include/gdn.h declares, and its host-side validation fails closed.

Every call here is built to be rejected by host validation before any launch
(it never reaches a kernel).  As a guard these tests do not run where a GPU is
visible: there the GPU tests cover the same paths with real buffers.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from gateddeltanet_linear_attention_amd import binding as gb

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "gdn.h")


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


no_gpu = pytest.mark.skipif(_gpu_visible(), reason="host-validation probes run only where no kernel can launch")


def declared_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"gdn_decode_step", "gdn_verify_window", "gdn_commit_accepted",
            "gdn_chunked_prefill_with_checkpoints", "gdn_chunked_workspace_bytes",
            "gdn_plan_transaction", "gdn_run_transaction", "gdn_status_str", "gdn_version",
            "gdn_commit_replay", "gdn_verify_tree", "gdn_verify_window_delta",
            "gdn_commit_delta", "gdn_verify_window_delta_fold", "gdn_verify_window_select",
            "gdn_commit_select", "gdn_chunked_prefill_with_checkpoints_static",
            "gdn_verify_window_select_commit"} <= set(names)
    lib = gb.lib()
    import gateddeltanet_linear_attention_amd as pkg
    for n in names:
        assert hasattr(lib, n), "libgdn.so does not export %s" % n
        assert callable(getattr(pkg, n, None)), "the package does not export %s" % n


def test_bandwidth_probe_library_loads_and_refuses_bad_arguments():
    """The benchmark's streaming-ceiling probe is a library of its own beside libgdn.so;
    its argument checks run on the host, so bad calls return -1 without a GPU."""
    path = os.path.join(os.path.dirname(os.path.abspath(gb.__file__)), "libgdn_probe.so")
    lib = ctypes.CDLL(path)
    f = lib.gdn_probe_stream
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_void_p]
    a, b = 1 << 40, 2 << 40  # never dereferenced: every call below fails its checks first
    assert f(None, b, 1024, 4, 0, None) == -1
    assert f(a, b, 0, 4, 0, None) == -1
    assert f(a, b, 1000, 4, 0, None) == -1   # not a multiple of 16
    assert f(a, b, 1024, 0, 0, None) == -1
    assert f(a, b, 1024, 9, 0, None) == -1
    assert f(a + 4, b, 1024, 4, 0, None) == -1  # misaligned
    assert f(a, b, 1024, 4, 3, None) == -1   # no such schedule


def test_version_and_status_strings():
    m = re.search(r"#define GDN_VERSION (\d+)", open(HEADER).read())
    assert gb.gdn_version() == int(m.group(1))
    for code in range(-7, 1):
        assert gb.gdn_status_str(code) and gb.gdn_status_str(code) != "unknown status"
    assert gb.gdn_status_str(-99) == "unknown status"


@pytest.mark.parametrize("k_max", [0, 1, 2, 3])
def test_planner_routes_short_rows_to_the_recurrent_kernel(k_max):
    dims = gb.Dims(16, 32, 128, 128, k_max)
    lens = np.arange(1, 200)
    route = gb.gdn_plan_transaction(dims, lens)
    assert np.array_equal(route, np.where(lens <= k_max + 1, gb.ROUTE_RECURRENT, gb.ROUTE_CHUNKED))


def test_planner_is_per_row_on_a_mixed_batch():
    dims = gb.Dims(16, 32, 128, 128, 3)
    lens = [4, 883, 4, 1, 3702, 2, 3]
    route = gb.gdn_plan_transaction(dims, lens)
    assert route.tolist() == [0, 1, 0, 0, 1, 0, 0]
    with pytest.raises(gb.GdnError) as e:
        gb.gdn_plan_transaction(dims, [4, 0, 2])
    assert e.value.code == -3


# ---------------------------------------------------------------- raw-ABI validation

class Bufs:
    """Synthetic, far-apart, 16-byte-aligned addresses standing in for device
    pointers (1 TiB apart, so no two claimed buffers overlap).  Never dereferenced:
    every call below is rejected by host validation before a launch."""

    def __init__(self):
        self._next = 1 << 44

    def ptr(self, nbytes=256, misalign=0):
        p = self._next
        self._next += 1 << 40
        return ctypes.c_void_p(p + misalign)


def _dims(**kw):
    d = dict(n_qk_heads=16, n_v_heads=32, d_k=128, d_v=128, k_max=3)
    d.update(kw)
    return gb._Dims(d["n_qk_heads"], d["n_v_heads"], d["d_k"], d["d_v"], d["k_max"])


def _i32(x):
    arr = np.ascontiguousarray(np.asarray(x, np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _verify(dims, T, src, n_slots=8, bufs=None, ckpt=None, pool=None, misalign=0, null_q=False):
    bufs = bufs or Bufs()
    Ta, Tp = _i32(T)
    sa, sp = _i32(src)
    toks = [ctypes.c_void_p(0) if null_q else bufs.ptr(misalign=misalign)] + [bufs.ptr() for _ in range(6)]
    return gb.lib().gdn_verify_window(ctypes.byref(dims), len(Ta), Tp, *toks,
                                      pool or bufs.ptr(), n_slots, sp, ckpt or bufs.ptr(), bufs.ptr(),
                                      ctypes.c_void_p(0))


@no_gpu
def test_verify_validation_codes():
    d = _dims()
    assert _verify(_dims(d_k=64, d_v=64), [1], [0]) == -2          # unsupported width
    assert _verify(_dims(d_k=128, d_v=16), [1], [0]) == -2         # d_k != d_v
    assert _verify(_dims(n_v_heads=30), [1], [0]) == -2            # H_v % H_qk != 0
    assert _verify(_dims(n_v_heads=2048), [1], [0]) == -2          # H_v > GDN_MAX_V_HEADS
    assert _verify(_dims(n_qk_heads=1024, n_v_heads=1024), [5], [0]) == -3  # H_v 1024 passes the shape check
    assert _verify(_dims(k_max=4), [1], [0]) == -2                 # k_max > 3
    assert _verify(d, [1, 5], [0, 1]) == -3                        # T_r > k_max + 1
    assert _verify(d, [1, 0], [0, 1]) == -3                        # T_r < 1
    assert _verify(_dims(k_max=1), [3], [0]) == -3                 # T_r > k_max + 1 (k_max 1)
    assert _verify(d, [2, 2], [0, 8]) == -3                        # slot >= n_slots
    assert _verify(d, [2, 2], [0, -2]) == -3                       # slot < -1
    assert _verify(d, [2], [0], misalign=8) == -5                  # misaligned q
    assert _verify(d, [2], [0], null_q=True) == -1                 # NULL q
    assert gb.lib().gdn_verify_window(None, 1, None, *[None] * 8, 1, None, None, None, None) == -1
    # checkpoint buffer overlapping the state pool
    b = Bufs()
    p = b.ptr(1 << 20)
    assert _verify(d, [2], [0], bufs=b, pool=p, ckpt=ctypes.c_void_p(p.value + 4096)) == -4


@no_gpu
def test_zero_rows_is_a_no_op():
    assert _verify(_dims(), [], []) == 0


@no_gpu
def test_decode_and_commit_validation_codes():
    lib = gb.lib()
    b = Bufs()
    d = _dims()

    def decode(src, dst, n_slots=8):
        sa, sp = _i32(src)
        da, dp = _i32(dst)
        return lib.gdn_decode_step(ctypes.byref(d), len(sa), *[b.ptr() for _ in range(7)], b.ptr(),
                                   n_slots, sp, dp, b.ptr(), ctypes.c_void_p(0))

    assert decode([0, 1], [1, 1]) == -4      # two rows write one slot
    assert decode([0, 1], [1, 0]) == -4      # row 0 writes the slot row 1 reads
    assert decode([0, 1], [0, 8]) == -3      # dst out of range
    assert decode([0, 1], [0, -1]) == -3     # decode must publish its state

    def commit(T, dst, n_slots=8, ckpt=None, pool=None):
        Ta, Tp = _i32(T)
        da, dp = _i32(dst)
        return lib.gdn_commit_accepted(ctypes.byref(d), len(Ta), Tp, ckpt or b.ptr(), b.ptr(),
                                       pool or b.ptr(), n_slots, dp, b.ptr(), ctypes.c_void_p(0))

    assert commit([4, 4], [3, 3]) == -4      # duplicate destination
    assert commit([4, 5], [1, 2]) == -3      # T_r > k_max + 1
    assert commit([4, 2], [1, 9]) == -3      # slot out of range
    p = b.ptr(1 << 20)
    assert commit([4], [0], pool=p, ckpt=p) == -4  # checkpoint buffer is the pool


@no_gpu
def test_verify_without_checkpoints_and_replay_validation_codes():
    lib = gb.lib()
    b = Bufs()
    d = _dims()
    NULL = ctypes.c_void_p(0)

    def verify_nock(T, o=None, misalign=0):
        Ta, Tp = _i32(T)
        sa, sp = _i32(list(range(len(T))))
        return lib.gdn_verify_window(ctypes.byref(d), len(Ta), Tp, *[b.ptr() for _ in range(7)], b.ptr(), 8,
                                     sp, NULL, o if o is not None else b.ptr(misalign=misalign), NULL)

    assert verify_nock([4, 2], o=NULL) == -1          # outputs are still required
    assert verify_nock([4, 2], misalign=2) == -5      # misaligned o
    assert verify_nock([4, 5]) == -3                  # T_r > k_max + 1
    # a valid call passes validation; with no GPU here the launch itself fails
    assert verify_nock([4, 2]) == -7

    def replay(T, src, dst, accepted=True, status=True, n_slots=8, misalign=0):
        Ta, Tp = _i32(T)
        sa, sp = _i32(src)
        da, dp = _i32(dst)
        toks = [b.ptr(misalign=misalign)] + [b.ptr() for _ in range(6)]
        return lib.gdn_commit_replay(ctypes.byref(d), len(Ta), Tp, *toks,
                                     b.ptr() if accepted else NULL, b.ptr(), n_slots, sp, dp,
                                     b.ptr() if status else NULL, NULL)

    assert replay([4, 2], [0, 1], [2, 3], accepted=False) == -1   # no accepted counts
    assert replay([4, 2], [0, 1], [2, 3], status=False) == -1     # no status word
    assert replay([4, 2], [0, 1], [2, -1]) == -3                  # replay must publish its state
    assert replay([4, 2], [0, 1], [2, 8]) == -3                   # dst out of range
    assert replay([4, 5], [0, 1], [2, 3]) == -3                   # T_r > k_max + 1
    assert replay([4, 2], [0, 1], [2, 2]) == -4                   # two rows write one slot
    assert replay([4, 2], [0, 1], [1, 3]) == -4                   # row 0 writes row 1's source
    assert replay([4, 2], [0, 1], [2, 3], misalign=8) == -5       # misaligned q
    assert replay([4, 2], [0, 1], [0, 1]) == -7                   # in place passes validation
    assert replay([], [], []) == 0


@no_gpu
def test_verify_tree_validation_codes():
    lib = gb.lib()
    b = Bufs()
    d = _dims()
    NULL = ctypes.c_void_p(0)

    def tree(T, parents, ckpt=True, par_null=False):
        Ta, Tp = _i32(T)
        pa, pp = _i32(parents)
        sa, sp = _i32(list(range(len(T))))
        return lib.gdn_verify_tree(ctypes.byref(d), len(Ta), Tp, None if par_null else pp,
                                   *[b.ptr() for _ in range(7)], b.ptr(), 8, sp,
                                   b.ptr() if ckpt else NULL, b.ptr(), NULL)

    assert tree([4], [-1, 0, 0, 1], par_null=True) == -1   # parents required
    assert tree([4], [-1, 0, 0, 1], ckpt=False) == -1      # checkpoints required
    assert tree([4], [0, 0, 0, 1]) == -3                   # first token must follow the committed state
    assert tree([4], [-1, 1, 0, 1]) == -3                  # a parent must be an earlier node
    assert tree([4], [-1, 0, 3, 1]) == -3
    assert tree([4], [-1, -2, 0, 1]) == -3                 # below -1
    assert tree([5], [-1, 0, 1, 2, 3]) == -3               # T_r > k_max + 1
    assert tree([2, 2], [-1, 0, -1, 1]) == -3              # second row: parent 1 of node 1
    assert tree([4, 2], [-1, 0, 0, 1, -1, -1]) == -7       # valid: passes validation, no GPU here


@no_gpu
def test_delta_validation_codes():
    lib = gb.lib()
    b = Bufs()
    d = _dims()
    NULL = ctypes.c_void_p(0)

    def verify(T, delta=True):
        Ta, Tp = _i32(T)
        sa, sp = _i32(list(range(len(T))))
        return lib.gdn_verify_window_delta(ctypes.byref(d), len(Ta), Tp, *[b.ptr() for _ in range(7)], b.ptr(), 8,
                                           sp, b.ptr() if delta else NULL, b.ptr(), NULL)

    def commit(T, src, dst, k=True, accepted=True, misalign=0):
        Ta, Tp = _i32(T)
        sa, sp = _i32(src)
        da, dp = _i32(dst)
        return lib.gdn_commit_delta(ctypes.byref(d), len(Ta), Tp, b.ptr() if k else NULL, b.ptr(misalign=misalign),
                                    b.ptr() if accepted else NULL, b.ptr(), 8, sp, dp, b.ptr(), NULL)

    assert verify([4, 2], delta=False) == -1
    assert verify([4, 5]) == -3
    assert verify([4, 2]) == -7                      # valid: passes validation, no GPU here
    assert commit([4, 2], [0, 1], [2, 3], k=False) == -1
    assert commit([4, 2], [0, 1], [2, 3], accepted=False) == -1
    assert commit([4, 2], [0, 1], [2, -1]) == -3
    assert commit([4, 2], [0, 1], [2, 2]) == -4
    assert commit([4, 2], [0, 1], [1, 3]) == -4
    assert commit([4, 2], [0, 1], [2, 3], misalign=4) == -5
    assert commit([4, 2], [0, 1], [0, 1]) == -7      # in place passes validation


@no_gpu
def test_select_validation_codes():
    lib = gb.lib()
    b = Bufs()
    d = _dims()
    NULL = ctypes.c_void_p(0)

    def verify(T, bank, n_slots=16, table=True, status=True):
        Ta, Tp = _i32(T)
        ba, bp = _i32(bank)
        return lib.gdn_verify_window_select(ctypes.byref(d), len(Ta), Tp, *[b.ptr() for _ in range(7)], b.ptr(),
                                            n_slots, b.ptr() if table else NULL, bp, b.ptr(),
                                            b.ptr() if status else NULL, NULL)

    def commit(T, bank, n_slots=16):
        Ta, Tp = _i32(T)
        ba, bp = _i32(bank)
        return lib.gdn_commit_select(ctypes.byref(d), len(Ta), Tp, b.ptr(), bp, n_slots, b.ptr(), b.ptr(), NULL)

    assert verify([4, 2], [0, 1], table=False) == -1
    assert verify([4, 2], [0, 1], status=False) == -1
    assert verify([4, 5], [0, 1]) == -3               # window too long
    assert verify([4, 2], [0, 4]) == -3               # bank 4 ends past 16 slots
    assert verify([4, 2], [-1, 1]) == -3
    assert verify([4, 2], [1, 1]) == -4               # two rows on one bank
    assert verify([1] * 65, list(range(65)), n_slots=4 * 65) == -3  # more rows than one launch
    assert verify([4, 2], [0, 3]) == -7               # valid: passes validation, no GPU here
    assert commit([4, 2], [0, 1]) == -7
    assert commit([4, 2], [2, 2]) == -4
    assert commit([4, 0], [0, 1]) == -3
    assert verify([], []) == 0 and commit([], []) == 0


@no_gpu
def test_select_commit_validation_codes():
    lib = gb.lib()
    b = Bufs()
    d = _dims()

    def call(T, PT, PB, bank, n_slots=72, acc=None):
        Ta, Tp = _i32(T)
        pa, pp = _i32(PT)
        ba, bp = _i32(PB)
        ka, kp = _i32(bank)
        return lib.gdn_verify_window_select_commit(
            ctypes.byref(d), len(Ta), Tp, pp, bp, acc if acc is not None else b.ptr(), *[b.ptr() for _ in range(7)],
            b.ptr(), n_slots, b.ptr(), kp, b.ptr(), b.ptr(), ctypes.c_void_p(0))

    assert call([4, 4], [4, 4], [0, 1], [2, 3], acc=ctypes.c_void_p(0)) == -1   # no accepted counts
    assert call([4, 4], [5, 4], [0, 1], [2, 3]) == -3                           # previous window too long
    assert call([4, 4], [4, 0], [0, 1], [2, 3]) == -3                           # previous window empty
    assert call([4, 4], [4, 4], [0, 18], [2, 3]) == -3                          # previous bank past the pool
    assert call([4, 4], [4, 4], [0, 0], [2, 3]) == -4                           # two rows share a previous bank
    assert call([4, 4], [4, 4], [0, 3], [2, 3]) == -4                           # a previous bank is written now
    assert call([4, 4], [4, 4], [0, 1], [2, 3], acc=b.ptr(misalign=2)) == -5    # misaligned counts


@no_gpu
def test_unknown_dims_flags_are_refused():
    lib = gb.lib()
    b = Bufs()
    src, src_p = _i32([0])
    dst, dst_p = _i32([1])
    for flags, expect in ((2, -2), (0x80000000, -2), (gb.QK_L2NORM, -7)):
        d = gb._Dims(16, 32, 128, 128, 3, flags)
        rc = lib.gdn_decode_step(ctypes.byref(d), 1, *[b.ptr() for _ in range(7)], b.ptr(), 4,
                                 src_p, dst_p, b.ptr(), None)
        assert rc == expect, (flags, rc)  # -7: valid, refused only for want of a GPU


@no_gpu
def test_folded_verify_validation_codes():
    lib = gb.lib()
    b = Bufs()
    d = _dims()
    NULL = ctypes.c_void_p(0)

    def fold(T, slots, pT, prev_k=True, same_delta=False):
        Ta, Tp = _i32(T)
        sa, sp = _i32(slots)
        pa, pp = _i32(pT)
        dl = b.ptr()
        return lib.gdn_verify_window_delta_fold(ctypes.byref(d), len(Ta), Tp, *[b.ptr() for _ in range(7)], b.ptr(), 8,
                                                sp, dl, b.ptr(), pp, b.ptr() if prev_k else NULL,
                                                dl if same_delta else b.ptr(), b.ptr(), b.ptr(), NULL)

    assert fold([4, 2], [0, 1], [4, 4], prev_k=False) == -1
    assert fold([4, 2], [0, -1], [4, 4]) == -3       # the folded state needs a slot
    assert fold([4, 2], [0, 1], [4, 5]) == -3        # previous window too long
    assert fold([4, 2], [0, 1], [0, 4]) == -3        # previous window empty
    assert fold([4, 2], [1, 1], [4, 4]) == -4        # two rows on one slot
    assert fold([4, 2], [0, 1], [4, 4], same_delta=True) == -4  # new factors would overwrite the pending ones
    assert fold([4, 2], [0, 1], [4, 4]) == -7        # valid: passes validation, no GPU here


@no_gpu
def test_binding_rejects_host_tensors_before_the_library():
    torch = pytest.importorskip("torch")
    dims = gb.Dims(1, 1, 16, 16, 3)
    t = torch.zeros(1, 1, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gb.gdn_decode_step(dims, t, t, t, torch.zeros(1, 1), torch.zeros(1, 1), torch.zeros(1),
                           torch.zeros(1), torch.zeros(1, 1, 16, 16), [0], [0], t)


@no_gpu
def test_chunked_and_transaction_validation_codes():
    lib = gb.lib()
    b = Bufs()
    d = _dims()
    need = gb.gdn_chunked_workspace_bytes(gb.Dims(16, 32, 128, 128, 3), [100, 64, 1])
    # per (chunk, value head): W parts 48 KiB, the six nonzero P blocks in parts 18, U' 32
    # KiB, 1.5 KiB of factors; per (chunk, qk-head): Q 16 KiB, K^T 16
    def ws(chunks, w_kib):
        return chunks * (32 * ((w_kib + 18 + 32) * 1024 + 1536) + 16 * (16 + 16) * 1024)
    assert need == ws(2 + 1 + 1, 48)
    # past 160 MiB with W in parts the workspace is streamed and holds W in fp32 (32 KiB)
    assert ws(44, 48) <= (160 << 20) < ws(45, 48)
    assert gb.gdn_chunked_workspace_bytes(gb.Dims(16, 32, 128, 128, 3), [64 * 45]) == ws(45, 32)
    assert gb.gdn_chunked_workspace_bytes(gb.Dims(16, 32, 128, 128, 3), [64 * 44]) == ws(44, 48)  # W in parts
    assert gb.gdn_chunked_workspace_bytes(gb.Dims(16, 32, 128, 128, 3), [64 * 44 + 1]) == ws(45, 32)
    # one qk-head for all value heads: one Q/K^T unit per chunk
    assert gb.gdn_chunked_workspace_bytes(gb.Dims(1, 32, 128, 128, 3), [64]) == \
        32 * ((48 + 18 + 32) * 1024 + 1536) + 32 * 1024
    assert gb.gdn_chunked_workspace_bytes(gb.Dims(16, 32, 128, 128, 3), [100], chunk=32) == 0
    assert gb.gdn_chunked_workspace_bytes(gb.Dims(16, 32, 128, 128, 3), [0]) == 0

    def chunked(L, nt, src, dst, chunk=64, ws=None, ws_bytes=1 << 40, ckpt=None, pool=None):
        La, Lp = _i32(L)
        na, np_ = _i32(nt)
        sa, sp = _i32(src)
        da, dp = _i32(dst)
        return lib.gdn_chunked_prefill_with_checkpoints(
            ctypes.byref(d), len(La), Lp, chunk, np_, *[b.ptr() for _ in range(7)], pool or b.ptr(), 8, sp, dp,
            ckpt or b.ptr(), b.ptr(), ws if ws is not None else b.ptr(), ws_bytes, ctypes.c_void_p(0))

    assert chunked([100], [4], [0], [1], chunk=32) == -2        # chunk size other than 64
    assert chunked([100], [5], [0], [1]) == -3                  # n_tail > k_max + 1
    assert chunked([3], [4], [0], [1]) == -3                    # n_tail > L
    assert chunked([0], [0], [0], [1]) == -3                    # empty row
    assert chunked([100, 50], [0, 0], [0, 1], [1, 2]) == -4     # row 0 writes row 1's source
    assert chunked([100, 50], [0, 0], [0, 1], [3, 3]) == -4     # duplicate destination
    assert chunked([100], [0], [0], [1], ws_bytes=16) == -6     # workspace too small
    assert chunked([100], [0], [0], [1], ws=ctypes.c_void_p(0)) == -6
    p = b.ptr(1 << 20)
    assert chunked([100], [4], [0], [1], pool=p, ckpt=ctypes.c_void_p(p.value + 256)) == -4

    def tx(L, nc, src, dst, ws=None, ws_bytes=1 << 40):
        La, Lp = _i32(L)
        na, np_ = _i32(nc)
        sa, sp = _i32(src)
        da, dp = _i32(dst)
        return lib.gdn_run_transaction(ctypes.byref(d), len(La), Lp, np_, *[b.ptr() for _ in range(7)], b.ptr(), 8,
                                       sp, dp, b.ptr(), b.ptr(), ws if ws is not None else b.ptr(), ws_bytes,
                                       ctypes.c_void_p(0))

    def static(L, nt, src, dst, chunk=64):
        La, Lp = _i32(L)
        na, np_ = _i32(nt)
        sa, sp = _i32(src)
        da, dp = _i32(dst)
        return lib.gdn_chunked_prefill_with_checkpoints_static(
            ctypes.byref(d), len(La), Lp, chunk, np_, *[b.ptr() for _ in range(7)], b.ptr(), 8, sp, dp,
            b.ptr(), b.ptr(), ctypes.c_void_p(0))

    # the no-allocation form: the same checks, then a hard cap at the static array's size
    # (refused before the array is looked up, so nothing here needs a GPU)
    m = re.search(r"#define GDN_STATIC_WS_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    cap = int(m.group(1)) << int(m.group(2))
    assert cap == gb.STATIC_WS_BYTES
    assert static([100], [4], [0], [1], chunk=32) == -2
    assert static([100], [5], [0], [1]) == -3
    assert static([100, 50], [0, 0], [0, 1], [3, 3]) == -4
    big = [2048] * 4
    assert gb.gdn_chunked_workspace_bytes(gb.Dims(16, 32, 128, 128, 3), big) > cap
    assert static(big, [0] * 4, [0, 1, 2, 3], [4, 5, 6, 7]) == -6

    assert tx([4, 100], [4, 0], [0, -1], [-1, 1], ws_bytes=100) == -6  # the long row needs workspace
    assert tx([4, 100], [5, 0], [0, -1], [-1, 1]) == -3                # checkpoints > k_max + 1
    assert tx([4, 100], [4, 0], [0, -1], [-1, 0]) == -4                # prefill row overwrites a verify source

    # at most GDN_MAX_CHUNK_UNITS (chunk, value head) units per call: 2^24 / 32 heads = 2^19 chunks
    m = re.search(r"#define GDN_MAX_CHUNK_UNITS \(\(int64_t\)1 << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) == 24
    at, past = 64 << 19, (64 << 19) + 1                               # 2^19 chunks, one token more
    assert gb.gdn_chunked_workspace_bytes(gb.Dims(16, 32, 128, 128, 3), [at]) > 0
    assert gb.gdn_chunked_workspace_bytes(gb.Dims(16, 32, 128, 128, 3), [past]) == 0
    assert chunked([at], [0], [0], [1]) == -6        # within the limit: only the 1 TiB workspace is short
    assert chunked([past], [0], [0], [1]) == -3
    assert tx([4, past], [4, 0], [0, -1], [-1, 1]) == -3


@no_gpu
def test_header_compiles_as_c_and_a_c_program_links_the_library(tmp_path):
    """include/gdn.h is a C header: a C11 program includes it, links libgdn.so and
    calls it (validation paths only: no GPU here)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi_c.c"
    src.write_text(r"""
#include <stdio.h>
#include "gdn.h"
int main(void) {
  gdn_dims d = {16, 32, 128, 128, 3, 0};
  gdn_dims bad = {16, 32, 64, 64, 3, 0};
  int32_t T[1] = {4}, src[1] = {0};
  if (gdn_version() != GDN_VERSION) return 1;
  if (gdn_verify_window(&d, 0, T, 0, 0, 0, 0, 0, 0, 0, 0, 1, src, 0, 0, 0) != GDN_OK) return 2;
  if (gdn_verify_window(&bad, 1, T, 0, 0, 0, 0, 0, 0, 0, 0, 1, src, 0, 0, 0) != GDN_E_UNSUPPORTED) return 3;
  if (gdn_verify_window(&d, 1, T, 0, 0, 0, 0, 0, 0, 0, 0, 1, src, 0, 0, 0) != GDN_E_NULL) return 4;
  printf("%s\n", gdn_status_str(GDN_E_ALIAS));
  return 0;
}
""")
    exe = tmp_path / "abi_c"
    lib_dir = os.path.dirname(gb.LIB_PATH)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe),
                    "-L", lib_dir, "-lgdn", "-Wl,-rpath," + lib_dir], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert r.stdout.strip()
