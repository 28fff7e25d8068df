"""GPU parity of the forward's key split (fa_fwd_ws with the workspace that
fa_fwd_workspace_bytes sizes) against the float64 oracle and against
fa_fwd_ex.

With the workspace, the longer half of every head's causal query blocks runs
as two workgroups over the two halves of the block's keys; a second kernel
merges the two partial results (O_i, lse_i) by the log-sum-exp rule ("T5 讲解：
FlashAttention forward", section ⑥; "Inside FlashAttention", section 2.4).
Each half keeps its own running maximum, so its softmax weights are rounded to
the input type against a different reference than fa_fwd_ex's: the results
agree with fa_fwd_ex to within the weights' rounding, not bit for bit, and both
meet the oracle's tolerance.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import DT, O_ABS_TOL, check_lse, check_o, sample_rows, to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import exact_tiled_attention_06_amd as fa  # noqa: E402

fa.library()  # fails loudly when libfa.so is missing

DEV = "cuda:0"


def fp32(x):
    return float(torch.tensor(x, dtype=torch.float32))


def ws_bytes(B, H, Hkv, S, D, dtype):
    return fa.fa_fwd_workspace_bytes(B, H, Hkv, S, S, D, 1, -1, -1, fa.DTYPE_CODES[DT[dtype]])


def run(q, k, v, scale, ws=None, nbytes=0):
    """fa_fwd_ws (fa_fwd_ex when ws is None) on device copies; causal, no window."""
    B, H, S, D = q.shape
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    code = fa.DTYPE_CODES[q.dtype]
    if ws is None:
        st = fa.fa_fwd_ex(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                          k.shape[1], S, S, D, 1, -1, -1, scale, code, stream)
    else:
        st = fa.fa_fwd_ws(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                          k.shape[1], S, S, D, 1, -1, -1, scale, code, ws.data_ptr(), nbytes, stream)
    fa.check(st)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def inputs(B, H, Hkv, S, D, dtype, seed):
    q, _, _ = workloads.make_inputs(B, H, S, D, dtype, seed)
    _, k, v = workloads.make_inputs(B, Hkv, S, D, dtype, seed + 1)
    return q, k, v


# grids the split runs on: B * H * ceil(S / 256) = 512 at D = 32, 64 (the
# two-block kernel); B * H * ceil(S / 128) = 512 at D = 16 and 256 at D = 128
# (the one-block kernel)
SPLIT_CASES = [
    (2, 16, 2, 4096, 64, "f16"),     # 16 blocks per head, 8 split; grouped K/V heads
    (16, 16, 16, 512, 64, "bf16"),   # 2 blocks per head, the last one split
    (8, 16, 16, 1000, 64, "f16"),    # ragged last block (232 rows), 2 of 4 split
    (4, 16, 4, 2048, 32, "bf16"),    # D = 32, grouped K/V heads
    (8, 8, 8, 2000, 32, "f16"),      # D = 32, ragged
    (2, 4, 4, 4096, 128, "bf16"),    # D = 128: 32 blocks of 128 rows per head, 16 split
    (1, 16, 4, 2000, 128, "f16"),    # D = 128, ragged (80-row last block), grouped K/V heads
    (16, 8, 8, 512, 16, "f16"),      # D = 16: 4 blocks of 128 rows per head, 2 split
    (8, 8, 2, 1000, 16, "bf16"),     # D = 16, ragged, grouped K/V heads
]


def test_split_matches_oracle_and_fa_fwd_ex():
    """Every element of O and lse against the oracle, for each case in turn on
    one shared workspace (first filled with NaN, then reused with the previous
    case's contents: the call must read none of it), and against fa_fwd_ex."""
    need = max(ws_bytes(B, H, Hkv, S, D, dt) for B, H, Hkv, S, D, dt in SPLIT_CASES)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)
    for i, (B, H, Hkv, S, D, dtype) in enumerate(SPLIT_CASES):
        bm = 256 if D in (32, 64) else 128
        n_qblk = -(-S // bm)
        nbytes = ws_bytes(B, H, Hkv, S, D, dtype)
        assert nbytes == (n_qblk // 2) * B * H * 2 * bm * (D + 1) * 4
        q, k, v = inputs(B, H, Hkv, S, D, dtype, 8100 + 7 * i)
        scale = fp32(1 / math.sqrt(D))
        what = f"{dtype} B={B} H={H} Hkv={Hkv} S={S} D={D}"
        print(f"\nsplit case {what}", flush=True)
        o, lse = run(q, k, v, scale, ws, nbytes)
        o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), True, scale)
        e = check_o(to_f64(o), o_ref, dtype, f"O {what}")
        check_lse(to_f64(lse), l_ref, f"lse {what}")
        o_ex, lse_ex = run(q, k, v, scale)
        d = float((o.double() - o_ex.double()).abs().max())
        dl = float((lse.double() - lse_ex.double()).abs().max())
        print(f"  max|dO| vs oracle {e:.3e}, vs fa_fwd_ex {d:.3e}; max|dlse| vs fa_fwd_ex {dl:.3e}", flush=True)
        assert d <= O_ABS_TOL[dtype]
        assert dl <= 1e-4 * max(1.0, float(lse_ex.abs().max()))
        # causal row 0 sees key 0 alone: O = V[0] exactly (row 0 is in no split block)
        assert torch.equal(o[:, :, 0], v.repeat_interleave(H // Hkv, dim=1)[:, :, 0])


def test_short_workspace_runs_fa_fwd_ex():
    """A workspace below fa_fwd_workspace_bytes, or none, runs fa_fwd_ex's
    kernel: the same bits."""
    B, H, Hkv, S, D, dtype = 16, 16, 16, 512, 64, "f16"
    q, k, v = inputs(B, H, Hkv, S, D, dtype, 8200)
    scale = fp32(1 / math.sqrt(D))
    nbytes = ws_bytes(B, H, Hkv, S, D, dtype)
    ws = torch.zeros(nbytes // 4, dtype=torch.float32, device=DEV)
    o_ex, lse_ex = run(q, k, v, scale)
    for short in (nbytes - 16, 0):
        o, lse = run(q, k, v, scale, ws, short)
        assert torch.equal(o, o_ex) and torch.equal(lse, lse_ex), short


def test_no_split_problem_ignores_workspace():
    """Where fa_fwd_workspace_bytes is 0 (here a non-causal problem), a given
    workspace changes nothing."""
    B, H, S, D = 8, 16, 1000, 64
    q, k, v = inputs(B, H, H, S, D, "f16", 8300)
    scale = fp32(1 / math.sqrt(D))
    assert fa.fa_fwd_workspace_bytes(B, H, H, S, S, D, 0, -1, -1, fa.FA_DTYPE_F16) == 0
    ws = torch.zeros(1 << 20, dtype=torch.float32, device=DEV)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    outs = []
    for use_ws in (False, True):
        o = torch.empty_like(qd)
        lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
        stream = torch.cuda.current_stream().cuda_stream
        args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H, S, S, D, 0,
                -1, -1, scale, fa.FA_DTYPE_F16)
        st = (fa.fa_fwd_ws(*args, ws.data_ptr(), ws.numel() * 4, stream) if use_ws
              else fa.fa_fwd_ex(*args, stream))
        fa.check(st)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("name", ["sweep_D64_S16384", "sweep_D32_S16384", "sweep_D128_S4096",
                                  "sweep_D16_S8192"])
def test_full_size_sampled_rows(name):
    """At the full B=8 H=1 size of the sweep points that split: the oracle row
    by row on the first and last rows of every head, rows on both sides of
    block boundaries (the split blocks' included) and random rows."""
    w = workloads.BY_NAME[name]
    q, k, v = workloads.workload_inputs(w)
    scale = fp32(1 / math.sqrt(w.D))
    nbytes = ws_bytes(w.B, w.H, w.kv_heads, w.S, w.D, w.dtype)
    assert nbytes > 0
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=DEV)
    o, lse = run(q, k, v, scale, ws, nbytes)
    rows = sample_rows(w.B, w.H, w.S, 256, seed=8400)
    o_ref, l_ref = oracle.attention_rows(to_f64(q), to_f64(k), to_f64(v), True, scale, rows)
    of = to_f64(o).reshape(-1, w.D)[rows]
    lf = to_f64(lse).reshape(-1)[rows]
    check_o(of, np.asarray(o_ref).reshape(of.shape), w.dtype, f"O {name}")
    check_lse(lf, np.asarray(l_ref).reshape(lf.shape), f"lse {name}")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_split_under_graph_capture_replays():
    """forward() on a split shape captured in a HIP graph (its workspace then
    comes from the graph's own memory pool) and replayed several times, with
    eager work and synchronisation between the replays: every replay equals
    the eager result bit for bit (the split path records no memset)."""
    B, H, S, D = 16, 16, 512, 64
    q, k, v = (x.to(DEV) for x in inputs(B, H, H, S, D, "f16", 8600))
    scale = fp32(1 / math.sqrt(D))
    assert ws_bytes(B, H, H, S, D, "f16") > 0
    o_ref, l_ref = fa.forward(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        fa.forward(q, k, v, causal=True, scale=scale, out=o, lse=lse)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fa.forward(q, k, v, causal=True, scale=scale, out=o, lse=lse)
    for rep in range(4):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"replay {rep}"
        # eager work between the replays (another forward on the same shape)
        o2, _ = fa.forward(k, q, v, causal=True, scale=scale)
        torch.cuda.synchronize()
        assert torch.isfinite(o2.float()).all()
