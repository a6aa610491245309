"""The C ABI on the host: the library loads, exports every declared entry point,
and rejects bad arguments before any HIP call (so no GPU is needed here).
Pointers passed below are fake but aligned addresses; every call shown returns
an error status from host-side validation and launches nothing."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qknr.h")
BENCH_HEADER = os.path.join(ROOT, "include", "qknr_bench.h")


@pytest.fixture(scope="module")
def L():
    import qk_norm_rope_amd.build as b
    if not os.path.exists(b.LIB):
        b.build()
    import qk_norm_rope_amd as q
    return q.lib


def declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qknr_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("qknr_fwd", "qknr_bwd", "qknr_bwd_workspace_bytes", "qknr_status_string"):
        assert n in names


def exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return set(re.findall(r" T (qknr_\w+)", out))


def test_library_exports_every_declared_symbol(L):
    import qk_norm_rope_amd as q
    missing = [n for n in declared_functions() if n not in exported(q.lib_path)]
    assert not missing, missing
    for n in declared_functions():
        getattr(L, n)


@pytest.fixture(scope="module")
def LB():
    import qk_norm_rope_amd.build as b
    if not os.path.exists(b.BENCH_LIB):
        b.build()
    from qk_norm_rope_amd import bench_helpers
    return bench_helpers


def test_bench_library_exports_its_header(LB):
    names = declared_functions(BENCH_HEADER)
    assert names == ["qknr_bench_copy", "qknr_bench_empty", "qknr_bench_flush", "qknr_bench_stream2"]
    assert not [n for n in names if n not in exported(LB.lib_path)]
    # the operation's library carries none of the measurement helpers
    import qk_norm_rope_amd as q
    assert not [n for n in names if n in exported(q.lib_path)]


def test_stream_helpers_validate(LB):
    # no-op, null, misaligned pointer, bytes not a multiple of 16: no launch
    L = LB.lib
    for f, args in ((L.qknr_bench_copy, (A, A)), (L.qknr_bench_stream2, (A, A, A))):
        assert f(*args, 0, None) == 0
        assert f(*((None,) + args[1:]), 16, None) == 1
        assert f(*(args[:-1] + (A + 4,)), 16, None) == 3
        assert f(*args, 24, None) == 3
    assert L.qknr_bench_flush(None, 16, 0, None) == 1
    assert L.qknr_bench_flush(A + 8, 16, 0, None) == 3


def test_status_strings(L):
    import qk_norm_rope_amd as q
    assert q.qknr_status_string(0) == "ok"
    for s in range(1, 6):
        assert q.qknr_status_string(s) not in ("ok", "unknown status")
    assert q.qknr_status_string(99) == "unknown status"


A = 0x10000  # fake, 16-byte aligned address: never dereferenced (validation fails first)


def fwd(L, **kw):
    a = dict(q=A, k=A, wq=A, wk=A, pos=A, tokens=8, hq=4, hkv=2, D=64, R=64, eps=1e-6, theta=1e4,
             dtype=1, qo=A, ko=A)
    a.update(kw)
    return L.qknr_fwd(a["q"], a["k"], a["wq"], a["wk"], a["pos"], a["tokens"], a["hq"], a["hkv"],
                      a["D"], a["R"], a["eps"], a["theta"], a["dtype"], a["qo"], a["ko"], None)


def bwd(L, **kw):
    a = dict(q=A, k=A, wq=A, wk=A, pos=A, tokens=8, hq=4, hkv=2, D=64, R=64, eps=1e-6, theta=1e4,
             dtype=1, dqo=A, dko=A, dq=A, dk=A, dwq=A, dwk=A, ws=A, wsb=1 << 20)
    a.update(kw)
    return L.qknr_bwd(a["q"], a["k"], a["wq"], a["wk"], a["pos"], a["tokens"], a["hq"], a["hkv"],
                      a["D"], a["R"], a["eps"], a["theta"], a["dtype"], a["dqo"], a["dko"], a["dq"],
                      a["dk"], a["dwq"], a["dwk"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("call", [fwd, bwd])
def test_argument_errors(L, call):
    INV, UNS, MIS = 1, 2, 3
    assert call(L, tokens=-1) == INV
    assert call(L, hq=0) == INV
    assert call(L, hkv=0) == INV
    assert call(L, hq=2000) == INV
    assert call(L, eps=0.0) == INV
    assert call(L, eps=-1.0) == INV
    assert call(L, eps=float("nan")) == INV
    assert call(L, theta=0.0) == INV
    assert call(L, theta=float("inf")) == INV
    assert call(L, D=96) == UNS
    assert call(L, D=32) == UNS
    assert call(L, R=8) == UNS
    assert call(L, R=80) == UNS
    assert call(L, R=-16) == UNS
    assert call(L, dtype=7) == UNS
    assert call(L, q=None) == INV
    assert call(L, pos=None) == INV
    assert call(L, k=A + 8) == MIS
    assert call(L, wq=A + 2) == MIS
    assert call(L, pos=A + 2) == MIS
    # tokens == 0 is a no-op that inspects no pointer
    assert call(L, tokens=0, q=None, k=None, pos=None) == 0


def test_fwd_output_errors(L):
    assert fwd(L, qo=None) == 1
    assert fwd(L, ko=A + 4) == 3


def test_bwd_specific_errors(L):
    assert bwd(L, dq=None) == 1
    assert bwd(L, dwk=None) == 1
    assert bwd(L, dko=A + 2) == 3
    assert bwd(L, ws=None) == 4
    need = L.qknr_bwd_workspace_bytes(8, 4, 2, 64, 1)
    assert need > 0
    assert bwd(L, wsb=need - 1) == 4
    assert bwd(L, ws=A + 4, wsb=need) == 3


def test_workspace_bytes(L):
    f = L.qknr_bwd_workspace_bytes
    assert f(0, 4, 2, 64, 1) == 0
    assert f(-5, 4, 2, 64, 1) == 0
    assert f(100, 4, 2, 96, 1) == 0
    # one [4, D] fp32 partial (dwq, dwk, dbq, dbk) per backward workgroup (4
    # waves; at most 512).  A wave owns blocks of whole tokens: as many as fit
    # in one group of 64 / (D / E) rows (E = 8 for bf16, 4 for fp32), at least one.
    def expect(wgs, D):
        return wgs * 4 * D * 4
    assert f(1, 4, 2, 64, 1) == expect(1, 64)          # bf16 D=64: 8 rows/group -> 1 token/block
    assert f(17, 4, 2, 128, 0) == expect(5, 128)       # f32 D=128: 2 rows/group -> 17 blocks
    assert f(100, 1, 1, 64, 1) == expect(7, 64)        # 4 tokens/block -> 25 blocks -> 7 workgroups
    assert f(32768, 14, 2, 64, 1) == expect(512, 64)
    assert f(10 ** 7, 64, 8, 256, 1) == expect(512, 256)


# ---- extended entry points ---------------------------------------------------

class Layout(ctypes.Structure):
    _fields_ = [("q_stride", ctypes.c_int64), ("k_stride", ctypes.c_int64),
                ("q_out_stride", ctypes.c_int64), ("k_out_stride", ctypes.c_int64),
                ("dq_out_stride", ctypes.c_int64), ("dk_out_stride", ctypes.c_int64),
                ("k_out_slots", ctypes.c_void_p), ("k_out_rows", ctypes.c_int64)]


def test_layout_struct_matches_header():
    src = open(HEADER).read()
    body = re.search(r"typedef struct qknr_layout \{(.*?)\} qknr_layout;", src, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"\b(\w+);", body)
    assert fields == [f for f, _ in Layout._fields_]
    import qk_norm_rope_amd as q
    assert [f for f, _ in q.QknrLayout._fields_] == fields
    assert ctypes.sizeof(q.QknrLayout) == ctypes.sizeof(Layout) == 64


def dense(hq=4, hkv=2, D=64, **kw):
    import qk_norm_rope_amd as q
    lay = q.QknrLayout(hq * D, hkv * D, hq * D, hkv * D, hq * D, hkv * D, None, 0)
    for k_, v in kw.items():
        setattr(lay, k_, v)
    return lay


def fwd_ex(L, flags=0, layout="dense", **kw):
    a = dict(q=A, k=A, wq=A, wk=A, pos=A, tokens=8, hq=4, hkv=2, D=64, R=64, eps=1e-6, theta=1e4,
             dtype=1, qo=A, ko=A)
    a.update(kw)
    lay = dense(a["hq"], a["hkv"], a["D"]) if layout == "dense" else layout
    return L.qknr_fwd_ex(a["q"], a["k"], a["wq"], a["wk"], a["pos"], a["tokens"], a["hq"],
                         a["hkv"], a["D"], a["R"], ctypes.c_float(a["eps"]),
                         ctypes.c_double(a["theta"]), a["dtype"], ctypes.c_uint32(flags),
                         None if lay is None else ctypes.byref(lay), a["qo"], a["ko"], None)


def bwd_ex(L, flags=0, layout="dense", **kw):
    a = dict(q=A, k=A, wq=A, wk=A, pos=A, tokens=8, hq=4, hkv=2, D=64, R=64, eps=1e-6, theta=1e4,
             dtype=1, dqo=A, dko=A, dq=A, dk=A, dwq=A, dwk=A, ws=A, wsb=1 << 20)
    a.update(kw)
    lay = dense(a["hq"], a["hkv"], a["D"]) if layout == "dense" else layout
    return L.qknr_bwd_ex(a["q"], a["k"], a["wq"], a["wk"], a["pos"], a["tokens"], a["hq"],
                         a["hkv"], a["D"], a["R"], ctypes.c_float(a["eps"]),
                         ctypes.c_double(a["theta"]), a["dtype"], ctypes.c_uint32(flags),
                         None if lay is None else ctypes.byref(lay), a["dqo"], a["dko"], a["dq"],
                         a["dk"], a["dwq"], a["dwk"], a["ws"], ctypes.c_size_t(a["wsb"]), None)


@pytest.fixture(scope="module")
def Lx(L):
    import qk_norm_rope_amd as q
    return q.lib   # argtypes for the _ex entry points are set by the binding


@pytest.mark.parametrize("call", [fwd_ex, bwd_ex])
def test_ex_flag_and_stride_errors(Lx, call):
    INV, MIS = 1, 3
    assert call(Lx, flags=32) == INV                    # unknown flag bit
    assert call(Lx, flags=1 << 31) == INV
    # strides: at least heads * D, whole 16-byte chunks (8 bf16 elements)
    assert call(Lx, layout=dense(q_stride=4 * 64 - 8)) == INV
    assert call(Lx, layout=dense(k_stride=2 * 64 + 4)) == MIS
    assert call(Lx, layout=dense(k_out_stride=-128)) == INV
    assert call(Lx, layout=dense(q_out_stride=1 << 41)) == INV
    # fp32 chunks are 4 elements: stride 132 is aligned but a later check fails
    assert call(Lx, layout=dense(k_stride=2 * 64 + 4), dtype=0, q=None) == INV
    # weights are required without QKNR_FLAG_NO_WEIGHT ...
    assert call(Lx, wq=None) == INV
    assert call(Lx, wk=A + 2) == MIS
    # ... and neither read nor checked with it (a later check reports instead)
    assert call(Lx, flags=4, wq=None, wk=None, layout=dense(k_stride=2 * 64 + 4)) == MIS
    assert call(Lx, flags=4, wq=A + 2, wk=A + 6, layout=dense(k_stride=2 * 64 + 4)) == MIS
    assert call(Lx, tokens=0, q=None, layout=None) == 0


def test_ex_fwd_specific_errors(Lx):
    INV, MIS = 1, 3
    lay = dense()
    lay.k_out_slots = A + 4                              # int64 slots: 8-byte aligned
    lay.k_out_rows = 100
    assert fwd_ex(Lx, layout=lay) == MIS
    assert fwd_ex(Lx, qo=None) == INV
    # slots need the row count of the K output they index (the kernels skip
    # any slot outside [0, k_out_rows), so a bad slot is never written)
    for rows in (0, -1, -(1 << 40)):
        lay = dense(k_out_slots=A, k_out_rows=rows)
        assert fwd_ex(Lx, layout=lay) == INV
    lay = dense(k_out_slots=A, k_out_rows=1)
    assert fwd_ex(Lx, layout=lay, qo=None) == INV         # valid; a later check reports
    # without slots k_out_rows is not used
    assert fwd_ex(Lx, layout=dense(k_out_rows=-7), qo=None) == INV


def test_ex_bwd_specific_errors(Lx):
    INV, MIS, WS = 1, 3, 4
    lay = dense()
    lay.k_out_slots = A                                  # a forward-only option
    assert bwd_ex(Lx, layout=lay) == INV
    assert bwd_ex(Lx, layout=dense(dq_out_stride=100)) == INV   # < 4 * 64
    assert bwd_ex(Lx, layout=dense(dk_out_stride=2 * 64 + 2)) == MIS
    assert bwd_ex(Lx, dwq=None) == INV
    # dw is neither written nor checked without weights: the workspace check reports
    assert bwd_ex(Lx, flags=4, wq=None, wk=None, dwq=None, dwk=None, ws=None) == WS


# ---- entry points with every option ---------------------------------------------

class Options(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("layout", ctypes.c_void_p),
                ("bq", ctypes.c_void_p), ("bk", ctypes.c_void_p),
                ("inv_freq", ctypes.POINTER(ctypes.c_double)),
                ("attention_factor", ctypes.c_double),
                ("norm_group_q", ctypes.c_int32), ("norm_group_k", ctypes.c_int32)]


def test_options_struct_matches_header():
    src = open(HEADER).read()
    body = re.search(r"typedef struct qknr_options \{(.*?)\} qknr_options;", src, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"\b(\w+)(?:,|;)", body)
    assert fields == [f for f, _ in Options._fields_]
    import qk_norm_rope_amd as q
    assert [f for f, _ in q.QknrOptions._fields_] == fields
    assert ctypes.sizeof(q.QknrOptions) == ctypes.sizeof(Options) == 56


def opts(flags=0, bq=None, bk=None, table=None, attn=0.0):
    import qk_norm_rope_amd as q
    o = q.QknrOptions()
    o.flags = flags
    o.bq, o.bk = bq, bk
    keep = None
    if table is not None:
        keep = (ctypes.c_double * len(table))(*table)
        o.inv_freq = ctypes.cast(keep, ctypes.POINTER(ctypes.c_double))
    o.attention_factor = attn
    return o, keep


def fwd_opt(L, o, **kw):
    a = dict(q=A, k=A, wq=A, wk=A, pos=A, tokens=8, hq=4, hkv=2, D=64, R=64, eps=1e-6, theta=1e4,
             dtype=1, qo=A, ko=A)
    a.update(kw)
    return L.qknr_fwd_opt(a["q"], a["k"], a["wq"], a["wk"], a["pos"], a["tokens"], a["hq"],
                          a["hkv"], a["D"], a["R"], a["eps"], a["theta"], a["dtype"],
                          None if o is None else ctypes.byref(o), a["qo"], a["ko"], None)


def bwd_opt(L, o, **kw):
    a = dict(q=A, k=A, wq=A, wk=A, pos=A, tokens=8, hq=4, hkv=2, D=64, R=64, eps=1e-6, theta=1e4,
             dtype=1, dqo=A, dko=A, dq=A, dk=A, dwq=A, dwk=A, dbq=None, dbk=None, ws=A, wsb=1 << 20)
    a.update(kw)
    return L.qknr_bwd_opt(a["q"], a["k"], a["wq"], a["wk"], a["pos"], a["tokens"], a["hq"],
                          a["hkv"], a["D"], a["R"], a["eps"], a["theta"], a["dtype"],
                          None if o is None else ctypes.byref(o), a["dqo"], a["dko"], a["dq"],
                          a["dk"], a["dwq"], a["dwk"], a["dbq"], a["dbk"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("call", [fwd_opt, bwd_opt])
def test_opt_errors(Lx, call):
    INV, MIS, WS = 1, 3, 4
    # every failing case is rejected on the host; the passing ones get a
    # failing workspace (backward) or output (forward) check after it
    late = dict(ws=None) if call is bwd_opt else dict(qo=None)
    late_code = WS if call is bwd_opt else INV
    o, _ = opts(flags=32)
    assert call(Lx, o) == INV                                 # unknown flag bit
    o, _ = opts(bq=A)
    assert call(Lx, o) == INV                                 # one bias only
    o, _ = opts(bq=A, bk=A + 4)
    assert call(Lx, o) == MIS                                 # misaligned bias
    o, keep = opts(table=[1.0] * 31 + [float("nan")])
    assert call(Lx, o) == INV                                 # non-finite frequency
    o, _ = opts(attn=float("inf"))
    assert call(Lx, o) == INV                                 # non-finite factor
    o, keep = opts(flags=8, bq=A, bk=A, table=[0.5] * 32, attn=1.3)
    assert call(Lx, o, **late) == late_code                   # all valid
    assert call(Lx, None, **late) == late_code                # NULL options = defaults
    o, keep = opts(table=[1.0] * 8)                           # R = 16: 8 values read
    assert call(Lx, o, R=16, **late) == late_code
    # head_dim, rotary_dim and dtype are checked before the table is read: an
    # unsupported rotary_dim gives UNSUPPORTED, not the INVALID_ARG a read of
    # the non-finite entries would give, and an absurd one reads nothing
    UNS = 2
    o, keep = opts(table=[float("nan")] * 16)
    assert call(Lx, o, R=24) == UNS
    assert call(Lx, o, R=1 << 30) == UNS
    assert call(Lx, o, R=-16) == UNS
    assert call(Lx, o, D=96, R=32) == UNS
    assert call(Lx, o, dtype=7) == UNS


def test_opt_bwd_bias_grad_errors(Lx):
    INV, MIS = 1, 3
    assert bwd_opt(Lx, None, dbq=A) == INV                    # one bias gradient only
    assert bwd_opt(Lx, None, dbq=A, dbk=A + 8) == MIS
    assert bwd_opt(Lx, None, dbq=A, dbk=A, ws=None) == 4


def test_opt_norm_group_errors(Lx):
    INV, UNS = 1, 2
    o, _ = opts()
    o.norm_group_q = 3                                        # does not divide hq = 4
    assert fwd_opt(Lx, o) == INV
    o, _ = opts()
    o.norm_group_k = -1
    assert bwd_opt(Lx, o) == INV
    lay = dense()
    lay.k_out_slots = A                                       # slots: forward only
    o, _ = opts()
    o.norm_group_q = 2
    o.layout = ctypes.pointer(lay)
    assert bwd_opt(Lx, o) == INV
    o, _ = opts(flags=16)                                     # [H, D] weights, token too large
    assert fwd_opt(Lx, o, hq=1024, hkv=1024, D=256) == UNS
    assert bwd_opt(Lx, o, hq=512, hkv=64, D=128) == UNS
    # just past the limits: 136 bf16 rows of 128 = 34 KiB > 32 KiB (forward),
    # 104 rows = 26 KiB > 24 KiB (backward, bf16), 72 fp32 rows of 64 = 18 KiB >
    # 16 KiB (backward, fp32)
    assert fwd_opt(Lx, o, hq=128, hkv=8, D=128) == UNS
    assert bwd_opt(Lx, o, hq=96, hkv=8, D=128) == UNS
    assert bwd_opt(Lx, o, hq=64, hkv=8, D=64, dtype=0) == UNS


def test_opt_workspace_bytes(Lx):
    import qk_norm_rope_amd as q
    f = q.qknr_bwd_opt_workspace_bytes
    # default options: the plain workspace
    assert f(1000, 4, 2, 64, 64, 1) == q.qknr_bwd_workspace_bytes(1000, 4, 2, 64, 1)
    # [H, D] weights, bf16, D = 64: a wave instruction holds 8 rows, so a
    # token of 6 rows fits the 16 rows of a stage twice -> blocks of 2 tokens,
    # 4 per workgroup (one per wave): ceil(1000 / 2 / 4) = 125 workgroups (at
    # most 512), each a partial row of 2 (hq + hkv) D fp32 columns (dw and db)
    assert f(1000, 4, 2, 64, 64, 1, flags=16) == 125 * 2 * 6 * 64 * 4
    assert f(100, 4, 2, 64, 64, 1, flags=16) == 13 * 2 * 6 * 64 * 4
    assert f(100000, 4, 2, 64, 64, 1, flags=16) == 512 * 2 * 6 * 64 * 4
    # fp32: 4 rows per instruction, 8 per stage -> 1 token per block, 250
    # workgroups
    assert f(1000, 4, 2, 64, 64, 0, flags=16) == 250 * 2 * 6 * 64 * 4
    # norm groups with [D] weights: as above, 125 workgroups of 4 D columns
    assert f(1000, 4, 2, 64, 64, 1, norm_groups=(2, 1)) == 125 * 4 * 64 * 4
    # 18 rows span two 16-row stages, per-head norms lie in one: (token,
    # stage) pairs 2000 -> 500 workgroups (an even count of waves per stage)
    assert f(1000, 16, 2, 64, 64, 1, flags=16) == 500 * 2 * 18 * 64 * 4
    # q groups of 5 heads, one of them across the two stages: the whole-token
    # kernel, 1536 chunk slots / (22 rows * 8 chunks) = 8 tokens per iteration
    # -> 125 workgroups
    assert f(1000, 20, 2, 64, 64, 1, flags=16, norm_groups=(5, 2)) == 125 * 2 * 22 * 64 * 4
    assert f(1000, 20, 2, 64, 64, 1, flags=16, norm_groups=(4, 2)) == 500 * 2 * 22 * 64 * 4
    # [D] weights (4 D columns), 14 + 4 heads: k groups of 2 stay in the second
    # stage (two stages per token, 500 workgroups); one k group of 4 crosses
    # into it (whole tokens: 1536 / (18 * 8) = 10 tokens per iteration)
    assert f(1000, 14, 4, 64, 64, 1, norm_groups=(7, 2)) == 500 * 4 * 64 * 4
    assert f(1000, 14, 4, 64, 64, 1, norm_groups=(7, 4)) == 100 * 4 * 64 * 4
    assert f(10, 512, 64, 128, 128, 1, flags=16) == 0          # a token too large
    assert f(10, 4, 2, 64, 64, 1, norm_groups=(3, 1)) == 0       # 3 does not divide 4
    assert f(10, 4, 2, 64, 24, 1) == 0 and f(10, 4, 2, 64, 1 << 30, 1) == 0
    assert f(10, 4, 2, 96, 32, 1) == 0 and f(10, 4, 2, 64, 64, 7) == 0


# ---- Best-Fit-Decreasing packing ---------------------------------------------------

def bfd(L, **kw):
    a = dict(len=A, n=10, cap=64, mb=4, ds=A, pos=A, cu=A, cnt=A, st=A, ws=A, wsb=1 << 20)
    a.update(kw)
    return L.qknr_bfd_pack(a["len"], a["n"], a["cap"], a["mb"], a["ds"], a["pos"], a["cu"],
                           a["cnt"], a["st"], a["ws"], a["wsb"], None)


def test_bfd_argument_errors(Lx):
    INV, MIS, WS = 1, 3, 4
    assert bfd(Lx, n=-1) == INV
    assert bfd(Lx, n=(1 << 22) + 1) == INV
    assert bfd(Lx, cap=0) == INV
    assert bfd(Lx, mb=0) == INV
    assert bfd(Lx, mb=4097) == INV
    assert bfd(Lx, cap=1 << 20, mb=4096) == INV             # max_bins * capacity >= 2^31
    assert bfd(Lx, len=None) == INV
    assert bfd(Lx, cnt=None) == INV
    assert bfd(Lx, pos=A + 2) == MIS
    assert bfd(Lx, ws=None) == WS
    assert bfd(Lx, wsb=Lx.qknr_bfd_workspace_bytes(10, 4) - 1) == WS
    assert bfd(Lx, ws=A + 8) == MIS


def test_bfd_workspace_bytes(Lx):
    f = Lx.qknr_bfd_workspace_bytes
    # 8-byte sort keys for the next power of two of ndocs, then rank [ndocs] and
    # three [max_bins] arrays, each part rounded up to 16 bytes
    assert f(400, 16) == 512 * 8 + 1600 + 3 * 64
    assert f(0, 1) == 16 + 16 + 3 * 16          # 8 bytes of keys round up to 16
    assert f(-1, 4) == 0 and f(10, 0) == 0 and f(10, 5000) == 0
