"""The C ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments with the documented status codes before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _header_text():
    with open(HEADER, encoding="utf-8") as f:
        return f.read()


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def _defines():
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(FA_\w+)\s+(-?\d+)", _header_text())}


@pytest.fixture(scope="module")
def fa():
    import exact_tiled_attention_06_amd as fa
    return fa


@pytest.fixture(scope="module")
def lib(fa):
    return ctypes.CDLL(fa.LIBRARY)


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert "fa_fwd" in names and "fa_status_string" in names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in include/fa.h but not exported"


def test_binding_constants_match_header(fa):
    for name, value in _defines().items():
        assert getattr(fa, name) == value, name


def test_status_strings(fa):
    codes = [v for k, v in _defines().items() if k.startswith("FA_ERR_") or k == "FA_OK"]
    seen = set()
    for c in codes:
        s = fa.fa_status_string(c)
        assert s and s != "unknown status", c
        seen.add(s)
    assert len(seen) == len(codes)
    assert fa.fa_status_string(12345) == "unknown status"


# fake, never-dereferenced addresses: every case below fails validation first
P = 1 << 20
ARGS = dict(q=P, k=2 * P, v=3 * P, o=4 * P, lse=5 * P, B=1, H=1, S=64, D=64, causal=0,
            scale=0.125, dtype=1, stream=0)


def call(fa, **over):
    a = dict(ARGS, **over)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S"], a["D"],
                     a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(B=-1), "FA_ERR_SHAPE"),
    (dict(H=-2), "FA_ERR_SHAPE"),
    (dict(S=-64), "FA_ERR_SHAPE"),
    (dict(D=48), "FA_ERR_HEAD_DIM"),
    (dict(D=256), "FA_ERR_HEAD_DIM"),
    (dict(D=0), "FA_ERR_HEAD_DIM"),
    (dict(dtype=3), "FA_ERR_DTYPE"),
    (dict(dtype=-1), "FA_ERR_DTYPE"),
    (dict(causal=2), "FA_ERR_CAUSAL"),
    (dict(scale=0.0), "FA_ERR_SCALE"),
    (dict(scale=-0.5), "FA_ERR_SCALE"),
    (dict(scale=float("inf")), "FA_ERR_SCALE"),
    (dict(scale=float("nan")), "FA_ERR_SCALE"),
    (dict(q=0), "FA_ERR_NULL_POINTER"),
    (dict(lse=0), "FA_ERR_NULL_POINTER"),
    (dict(o=0), "FA_ERR_NULL_POINTER"),
    (dict(o=P + 64), "FA_ERR_ALIAS"),             # o inside q
    (dict(lse=4 * P + 1024), "FA_ERR_ALIAS"),     # lse inside o
    (dict(o=2 * P), "FA_ERR_ALIAS"),              # o == k
    (dict(q=P + 8), "FA_ERR_ALIGNMENT"),
    (dict(o=4 * P + 2), "FA_ERR_ALIGNMENT"),
    (dict(lse=5 * P + 2), "FA_ERR_ALIGNMENT"),
    (dict(B=1 << 31), "FA_ERR_TOO_LARGE"),
    (dict(S=1 << 31), "FA_ERR_TOO_LARGE"),
    (dict(B=1 << 20, H=1 << 20), "FA_ERR_TOO_LARGE"),
    (dict(S=1 << 23, D=128), "FA_ERR_TOO_LARGE"),   # one head's K is 2 GiB: beyond a buffer extent
])
def test_rejects_bad_arguments(fa, over, code):
    assert call(fa, **over) == _defines()[code]


def test_first_failed_check_wins(fa):
    assert call(fa, B=-1, D=48, dtype=7) == fa.FA_ERR_SHAPE
    assert call(fa, D=48, dtype=7) == fa.FA_ERR_HEAD_DIM


@pytest.mark.parametrize("over", [dict(B=0), dict(H=0), dict(S=0)])
def test_empty_problem_is_a_no_op(fa, over):
    # nothing to compute: OK without touching the (null) pointers or the device
    assert call(fa, q=0, k=0, v=0, o=0, lse=0, **over) == fa.FA_OK


def test_q_k_v_may_alias(fa):
    # read-only inputs may share storage; only the output checks reject overlaps,
    # so this call fails later, at the null lse check
    assert call(fa, k=P, v=P, lse=0) == fa.FA_ERR_NULL_POINTER


def test_python_errors_map(fa):
    with pytest.raises(ValueError):
        fa.check(fa.FA_ERR_HEAD_DIM)
    with pytest.raises(RuntimeError):
        fa.check(fa.FA_ERR_LAUNCH)
    fa.check(fa.FA_OK)


# ---- fa_bwd: the same checks, over its ten buffers
BARGS = dict(q=P, k=2 * P, v=3 * P, o=4 * P, dout=5 * P, lse=6 * P, dq=7 * P, dk=8 * P, dv=9 * P,
             delta=10 * P, B=1, H=1, S=64, D=64, causal=0, scale=0.125, dtype=1, stream=0)


def bcall(fa, **over):
    a = dict(BARGS, **over)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                     a["delta"], a["B"], a["H"], a["S"], a["D"], a["causal"], a["scale"], a["dtype"],
                     a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(B=-1), "FA_ERR_SHAPE"),
    (dict(D=96), "FA_ERR_HEAD_DIM"),
    (dict(dtype=0), "FA_ERR_DTYPE"),              # fp32 has no backward
    (dict(dtype=5), "FA_ERR_DTYPE"),
    (dict(causal=-1), "FA_ERR_CAUSAL"),
    (dict(scale=float("nan")), "FA_ERR_SCALE"),
    (dict(dout=0), "FA_ERR_NULL_POINTER"),
    (dict(delta=0), "FA_ERR_NULL_POINTER"),
    (dict(dv=0), "FA_ERR_NULL_POINTER"),
    (dict(dq=P), "FA_ERR_ALIAS"),                  # dq == q
    (dict(dk=7 * P + 512), "FA_ERR_ALIAS"),        # dk inside dq
    (dict(delta=6 * P + 64), "FA_ERR_ALIAS"),      # delta inside lse
    (dict(delta=9 * P + 4), "FA_ERR_ALIAS"),       # delta inside dv (and 4-byte aligned)
    (dict(dv=5 * P), "FA_ERR_ALIAS"),              # dv == dout
    (dict(dout=5 * P + 8), "FA_ERR_ALIGNMENT"),
    (dict(dk=8 * P + 4), "FA_ERR_ALIGNMENT"),
    (dict(delta=10 * P + 2), "FA_ERR_ALIGNMENT"),
    (dict(S=1 << 23, D=128), "FA_ERR_TOO_LARGE"),
])
def test_bwd_rejects_bad_arguments(fa, over, code):
    assert bcall(fa, **over) == _defines()[code]


def test_bwd_first_failed_check_wins(fa):
    assert bcall(fa, B=-1, D=48, dtype=0) == fa.FA_ERR_SHAPE
    assert bcall(fa, D=48, dtype=0) == fa.FA_ERR_HEAD_DIM
    assert bcall(fa, dtype=0, causal=3) == fa.FA_ERR_DTYPE


@pytest.mark.parametrize("over", [dict(B=0), dict(H=0), dict(S=0)])
def test_bwd_empty_problem_is_a_no_op(fa, over):
    nulls = {n: 0 for n in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "delta")}
    assert bcall(fa, **nulls, **over) == fa.FA_OK


def test_bwd_inputs_may_alias(fa):
    # q, k, v, o, dout share storage: only outputs are checked, so this fails
    # at the null-pointer check that follows the input checks
    assert bcall(fa, k=P, v=P, o=P, dout=P, delta=0) == fa.FA_ERR_NULL_POINTER


# ---- fa_fwd_ex / fa_bwd_ex: grouped heads, query and key lengths, windows
XARGS = dict(ARGS, Hkv=1, wl=-1, wr=-1)


def xcall(fa, **over):
    a = dict(XARGS, **over)
    sq, sk = a.get("Sq", a["S"]), a.get("Sk", a["S"])
    return fa.fa_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], sq, sk, a["D"],
                        a["causal"], a["wl"], a["wr"], a["scale"], a["dtype"], a["stream"])


def xbcall(fa, **over):
    a = dict(BARGS, Hkv=1, wl=-1, wr=-1)
    a.update(over)
    sq, sk = a.get("Sq", a["S"]), a.get("Sk", a["S"])
    return fa.fa_bwd_ex(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                        a["delta"], a["B"], a["H"], a["Hkv"], sq, sk, a["D"], a["causal"], a["wl"], a["wr"],
                        a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(H=6, Hkv=4), "FA_ERR_SHAPE"),       # H not a multiple of H_kv
    (dict(Hkv=0), "FA_ERR_SHAPE"),
    (dict(Hkv=-1), "FA_ERR_SHAPE"),
    (dict(wl=-2), "FA_ERR_WINDOW"),
    (dict(wr=-7), "FA_ERR_WINDOW"),
    (dict(q=0, wl=3), "FA_ERR_NULL_POINTER"),
    (dict(H=4, Hkv=2, o=2 * P + 8192), "FA_ERR_ALIAS"),  # o overlaps k (k is 2 heads long)
])
def test_ex_rejects_bad_arguments(fa, over, code):
    assert xcall(fa, **over) == _defines()[code]
    if "o" not in over:  # the backward's o is an input: overlapping it is no error
        assert xbcall(fa, **over) == _defines()[code]


def test_ex_defaults_reach_the_plain_checks(fa):
    # H_kv = H and no window: the extended entries check exactly as the plain ones
    for over, code in [(dict(D=48), "FA_ERR_HEAD_DIM"), (dict(scale=-1.0), "FA_ERR_SCALE"),
                       (dict(lse=0), "FA_ERR_NULL_POINTER")]:
        assert xcall(fa, **over) == call(fa, **over) == _defines()[code]
    assert xbcall(fa, dtype=0) == fa.FA_ERR_DTYPE


@pytest.mark.parametrize("over", [dict(B=0), dict(S=0)])
def test_ex_empty_problem_is_a_no_op(fa, over):
    assert xcall(fa, q=0, k=0, v=0, o=0, lse=0, wl=5, **over) == fa.FA_OK


@pytest.mark.parametrize("over,code", [
    (dict(Sq=-1), "FA_ERR_SHAPE"),
    (dict(Sk=-3), "FA_ERR_SHAPE"),
    (dict(Sq=64, Sk=256, k=0), "FA_ERR_NULL_POINTER"),   # keys exist: k is needed
    (dict(Sq=256, Sk=64, v=0), "FA_ERR_NULL_POINTER"),
    (dict(Sq=64, Sk=1 << 24, D=128), "FA_ERR_TOO_LARGE"),  # one head's K: S_k * D * 2 bytes >= 2^31
])
def test_ex_query_and_key_lengths_checked(fa, over, code):
    # (only rejected calls: an accepted one would launch on these fake pointers)
    assert xcall(fa, **over) == _defines()[code]


def test_ex_rectangular_alias_uses_both_lengths(fa):
    # q, o: B*H*Sq*D*2 = 1*4*64*64*2 = 32 KiB; k, v: B*Hkv*Sk*D*2 = 1*1*1024*64*2 = 128 KiB
    base = dict(B=1, H=4, Hkv=1, Sq=64, Sk=1024, D=64, dtype=1)
    q, k, v, o, lse = P, 2 * P, 3 * P, 4 * P, 5 * P
    assert xcall(fa, q=q, k=k, v=v, o=k + 96 * 1024, lse=lse, **base) == fa.FA_ERR_ALIAS  # inside k's 128 KiB
    assert xcall(fa, q=q, k=k, v=v, o=o, lse=q + 16 * 1024, **base) == fa.FA_ERR_ALIAS  # lse inside q
    assert xbcall(fa, dk=v + 120 * 1024, Sq=64, Sk=1024, H=4) == fa.FA_ERR_ALIAS  # dk inside v's 128 KiB


def test_ex_no_query_rows_is_a_no_op_forward(fa):
    # S_q = 0: the forward has no row to write (pointers may be NULL)
    assert xcall(fa, q=0, k=0, v=0, o=0, lse=0, Sq=0, Sk=512) == fa.FA_OK
    assert xbcall(fa, q=0, k=0, v=0, o=0, dout=0, lse=0, dq=0, dk=0, dv=0, delta=0, Sq=0, Sk=0) == fa.FA_OK
    # the backward still owes dK = dV = 0 for the keys
    assert xbcall(fa, q=0, o=0, dout=0, lse=0, dq=0, delta=0, dk=0, Sq=0, Sk=512) == fa.FA_ERR_NULL_POINTER


# ---- the microbenchmark library (include/fa_micro.h) --------------------------

MICRO_HEADER = os.path.join(ROOT, "include", "fa_micro.h")


def test_micro_exports_and_rejects_bad_arguments():
    """libfa_micro.so exports every function fa_micro.h declares, its constants
    match the binding's, and out-of-range arguments fail before any HIP call."""
    from exact_tiled_attention_06_amd import micro
    with open(MICRO_HEADER, encoding="utf-8") as f:
        text = f.read()
    lib = micro.library()
    for name in set(re.findall(r"\b(fa_micro\w*)\s*\(", re.sub(r"/\*.*?\*/", "", text, flags=re.S))):
        assert hasattr(lib, name), f"{name} declared in include/fa_micro.h but not exported"
    defs = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(FA_MICRO_\w+)\s+(-?\d+)", text)}
    assert defs["FA_MICRO_OP_EXP"] == micro.OP_EXP and defs["FA_MICRO_OP_MAX3"] == micro.OP_MAX3
    assert defs["FA_MICRO_MIXED"] == micro.MIXED and defs["FA_MICRO_SPLIT"] == micro.SPLIT
    err = defs["FA_MICRO_ERR_ARG"]
    out = 1 << 20  # never dereferenced: every call below fails validation first
    assert lib.fa_micro(99, 4, 0, micro.MIXED, 4, 10, out, None) == err      # op
    assert lib.fa_micro(micro.OP_EXP, 3, 0, micro.MIXED, 4, 10, out, None) == err   # k
    assert lib.fa_micro(micro.OP_EXP, 4, 2, micro.MIXED, 4, 10, out, None) == err   # agpr
    assert lib.fa_micro(micro.OP_EXP, 4, 0, 7, 4, 10, out, None) == err             # mode
    assert lib.fa_micro(micro.OP_EXP, 4, 0, micro.SPLIT, 4, 10, out, None) == err   # split needs 8 waves
    assert lib.fa_micro(micro.OP_EXP, 4, 0, micro.MIXED, 9, 10, out, None) == err   # waves
    assert lib.fa_micro(micro.OP_EXP, 4, 0, micro.MIXED, 4, 0, out, None) == err    # iters
    assert lib.fa_micro(micro.OP_EXP, 4, 0, micro.MIXED, 4, 10, None, None) == err  # cycles


def test_bwd_noalloc_rejects_oversized_problem(fa):
    """fa_bwd_noalloc refuses B * H * S_q beyond its static workspace (4,194,304
    rows) with FA_ERR_WORKSPACE, before any HIP call."""
    st = fa.fa_bwd_noalloc(P, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P, 7 * P, 8 * P, 9 * P, 1, 1, 1, 4194305, 64, 64,
                           0, -1, -1, 0.125, fa.FA_DTYPE_F16, 0)
    assert st == fa.FA_ERR_WORKSPACE
    # the argument checks of fa_bwd_ex come first: a bad head dim wins
    st = fa.fa_bwd_noalloc(P, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P, 7 * P, 8 * P, 9 * P, 1, 1, 1, 4194305, 64, 48,
                           0, -1, -1, 0.125, fa.FA_DTYPE_F16, 0)
    assert st == fa.FA_ERR_HEAD_DIM


@pytest.mark.parametrize("over", [dict(dtype=0), dict(D=16), dict(D=128), dict(B=1, H=1, S=64)])
def test_single_buffered_unsupported_problems(fa, over):
    """The race-check entry exists only where fa_fwd runs the two-block kernel;
    elsewhere it returns FA_ERR_UNSUPPORTED before any HIP call."""
    G = 1 << 32  # fake, never-dereferenced buffers far enough apart not to overlap
    a = dict(ARGS, q=G, k=2 * G, v=3 * G, o=4 * G, lse=5 * G, B=4, H=16, S=4096, D=64)
    a.update(over)
    st = fa.fa_fwd_single_buffered(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S"], a["D"],
                                   a["causal"], a["scale"], a["dtype"], a["stream"])
    assert st == fa.FA_ERR_UNSUPPORTED


# ---- fa_fwd_workspace_bytes / fa_fwd_ws: the key split of the longest causal blocks

def test_fwd_workspace_bytes_closed_form(fa):
    """The split's workspace: (ceil(S/BM) / 2) blocks per head, two key halves
    each, BM rows of D fp32 values plus the lse; only for the problems the
    split runs on (causal, no window, S_q = S_k, fp16 / bf16, a grid of at
    most 512 workgroups of BM rows on the two-block kernel, BM = 256, or the
    one-block kernel, BM = 128).  A pure size computation: no HIP call."""
    def ws(B=8, H=1, Hkv=1, Sq=16384, Sk=16384, D=64, causal=1, wl=-1, wr=-1, dtype=1):
        return fa.fa_fwd_workspace_bytes(B, H, Hkv, Sq, Sk, D, causal, wl, wr, dtype)
    assert ws() == (64 // 2) * 8 * 2 * 256 * (64 + 1) * 4 == 34_078_720
    assert ws(D=32, dtype=2) == 32 * 8 * 2 * 256 * 33 * 4
    assert ws(Sq=16383, Sk=16383) == ws()                       # a ragged last block: same 64 blocks
    assert ws(B=4, H=2, Hkv=1) == ws()                          # grouped K/V heads: B * H = 8 query heads
    assert ws(B=2, H=16, Hkv=4, Sq=4096, Sk=4096) == 8 * 32 * 2 * 256 * 65 * 4  # 16 blocks x 32 heads
    # the one-block kernel: 128-row workgroups at D = 128 (between the key-split
    # kernel and the 256-row tile, at most one per CU) and at D = 16 (512)
    assert ws(D=128, Sq=4096, Sk=4096, dtype=2) == 16 * 8 * 2 * 128 * 129 * 4
    assert ws(D=128, Sq=8192, Sk=8192) == 0    # 512 workgroups of 128 rows: two per CU, no gain measured
    assert ws(D=16, Sq=8192, Sk=8192) == 32 * 8 * 2 * 128 * 17 * 4
    assert ws(D=128, Sq=2048, Sk=2048) == 0    # the key-split kernel (64-row grid below 512)
    assert ws(D=16, Sq=4096, Sk=4096) == 0     # 256 workgroups: the key-split kernel
    assert ws(D=128, B=16, Sq=8192, Sk=8192) == 0  # 1024 workgroups of 128 rows: not resident at once
    for over in [dict(causal=0), dict(D=128), dict(D=16), dict(dtype=0), dict(wl=1000), dict(wr=0),
                 dict(Sk=8192), dict(B=16), dict(B=4), dict(D=48), dict(Hkv=3), dict(dtype=7),
                 dict(B=0), dict(Sq=-1, Sk=-1)]:
        assert ws(**over) == 0, over
    # a window bound of max(S_q, S_k) or more is no window
    assert ws(wl=16384, wr=1 << 40) == ws()


def wscall(fa, ws, ws_bytes, **over):
    a = dict(XARGS, **over)
    sq, sk = a.get("Sq", a["S"]), a.get("Sk", a["S"])
    return fa.fa_fwd_ws(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], sq, sk, a["D"],
                        a["causal"], a["wl"], a["wr"], a["scale"], a["dtype"], ws, ws_bytes, a["stream"])


def test_fwd_ws_rejects_bad_workspace(fa):
    """fa_fwd_ws checks its workspace after fa_fwd_ex's checks and before any
    HIP call: a negative size, a misaligned or an overlapping workspace."""
    W = 64 * P  # far from the fake tensors at P .. 5P
    assert wscall(fa, W, -1) == fa.FA_ERR_WORKSPACE
    assert wscall(fa, W + 4, 1024) == fa.FA_ERR_ALIGNMENT
    assert wscall(fa, P + 64, 1024) == fa.FA_ERR_ALIAS             # inside q
    assert wscall(fa, 5 * P - 64, 1024) == fa.FA_ERR_ALIAS         # runs into lse
    # fa_fwd_ex's own checks come first
    assert wscall(fa, W, -1, D=48) == fa.FA_ERR_HEAD_DIM
    assert wscall(fa, W + 4, 1024, q=0) == fa.FA_ERR_NULL_POINTER
    # an empty problem is a no-op whatever the workspace
    assert wscall(fa, 0, 0, B=0, q=0, k=0, v=0, o=0, lse=0) == fa.FA_OK
