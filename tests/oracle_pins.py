"""Pins that tie the CPU oracle to facts other than its own code.

Each ``pin_*`` function takes an oracle handle (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with the page, a closed form, an
invariant of exact softmax attention, or an independent library evaluation.
``test_oracle.py`` runs them on the real oracle; ``test_oracle_mutants.py``
runs them on deliberately broken copies of the oracle source and requires every
mutant to fail at least one of them.
"""
from __future__ import annotations

import math
import os
from decimal import Decimal, getcontext

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TIGHT = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max scaled error {err:.3e} > {tol:.1e}"


def load_worked_example():
    """Parse the worked-example fixture: dict of name -> list of floats."""
    out = {}
    with open(os.path.join(GOLDEN, "t5_worked_example.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = [float(x) for x in vals]
    return out


def online_blocked(scores, values, block_n):
    """The page's streaming update for one query row, in plain Python floats.

    Running max m, running denominator l and running numerator u; each block of
    ``block_n`` keys rescales the old state by alpha = exp(m_old - m_new)
    ("从零训练语言模型（第二部分）", section "安全 / 在线 softmax").  Returns
    (o, lse, alphas) with one alpha per block.
    """
    m, l, u = -math.inf, 0.0, 0.0
    alphas = []
    for start in range(0, len(scores), block_n):
        blk = scores[start:start + block_n]
        vb = values[start:start + block_n]
        m_new = max(m, max(blk))
        alpha = math.exp(m - m_new)
        p = [math.exp(s - m_new) for s in blk]
        l = alpha * l + sum(p)
        u = alpha * u + sum(pi * vi for pi, vi in zip(p, vb))
        m = m_new
        alphas.append(alpha)
    return u / l, m + math.log(l), alphas


def _decimal_softmax_average(scores, values, digits=40):
    """sum_j e^{s_j} v_j / sum_j e^{s_j} and ln sum_j e^{s_j}, in `digits`-digit decimal arithmetic."""
    getcontext().prec = digits
    w = [Decimal(s).exp() for s in scores]
    den = sum(w)
    num = sum(wi * Decimal(vi) for wi, vi in zip(w, values))
    return float(num / den), float(den.ln())


# ---------------------------------------------------------------- the pins


def pin_worked_example(orc):
    """"T5 讲解", section ④: scores [1,2,3,0], v [10,20,30,40], BLOCK_N=2, round-1 alpha = 0."""
    ex = load_worked_example()
    scores, values = ex["scores"], ex["values"]
    block_n = int(ex["block_n"][0])
    # realise the scores with D = 1, q = 1, k_j = s_j, scale = 1
    q = np.ones((1, 1, 1, 1))
    k = np.array(scores).reshape(1, 1, 4, 1)
    v = np.array(values).reshape(1, 1, 4, 1)
    # one query against four keys: pad Q to four identical rows so the shapes agree
    q4 = np.repeat(q, 4, axis=2)
    o, lse = orc.attention(q4, k, v, False, 1.0)
    o_blk, lse_blk, alphas = online_blocked(scores, values, block_n)
    assert alphas[0] == ex["alpha_round1"][0], f"round-1 alpha {alphas[0]} != page's 0"
    o_dec, lse_dec = _decimal_softmax_average(scores, values)
    for row in range(4):
        _close(o[0, 0, row, 0], o_dec, TIGHT, "worked example O vs decimal")
        _close(o[0, 0, row, 0], o_blk, TIGHT, "worked example O vs blocked recurrence")
        _close(lse[0, 0, row], lse_dec, TIGHT, "worked example lse vs decimal")
        _close(lse[0, 0, row], lse_blk, TIGHT, "worked example lse vs blocked recurrence")
    # the natural-log lse, not the base-2 lse some kernels store internally
    base2 = max(scores) / math.log(2) + math.log2(sum(math.exp(s - max(scores)) for s in scores))
    assert abs(lse[0, 0, 0] - base2) > 1.0


def _rand(shape, seed, scale=1.0):
    return _rng(seed).standard_normal(shape) * scale


def _scores(q, k, scale):
    # independent evaluation of the score matrix (numpy matmul)
    return scale * np.matmul(q, np.swapaxes(k, -1, -2))


def _mask(S, causal):
    if not causal:
        return np.ones((S, S), dtype=bool)
    return np.tril(np.ones((S, S), dtype=bool))


def pin_normalisation(orc):
    """sum_{j in J} exp(s_j - lse_i) = 1 for every row (pins p and lse together)."""
    for causal in (False, True):
        B, H, S, D = 2, 3, 37, 8
        q, k, v = (_rand((B, H, S, D), 10 + t) for t in range(3))
        scale = 0.3
        _, lse = orc.attention(q, k, v, causal, scale)
        s = _scores(q, k, scale)
        w = np.exp(s - lse[..., None]) * _mask(S, causal)
        _close(w.sum(-1), np.ones((B, H, S)), 1e-12, f"row sums (causal={causal})")


def pin_convex_hull(orc):
    """Each o[i,d] lies between the min and max of v[j,d] over attended j."""
    for causal in (False, True):
        B, H, S, D = 1, 2, 29, 5
        q, k, v = (_rand((B, H, S, D), 20 + t, 2.0) for t in range(3))
        o, _ = orc.attention(q, k, v, causal, 0.7)
        for i in range(S):
            vis = v[:, :, : i + 1, :] if causal else v
            lo, hi = vis.min(axis=2), vis.max(axis=2)
            assert np.all(o[:, :, i, :] >= lo - 1e-12) and np.all(o[:, :, i, :] <= hi + 1e-12), \
                f"row {i} outside the convex hull (causal={causal})"


def pin_permutation(orc):
    """Non-causal O and lse are unchanged by a joint permutation of the K and V rows."""
    B, H, S, D = 2, 2, 23, 6
    q, k, v = (_rand((B, H, S, D), 30 + t) for t in range(3))
    perm = _rng(39).permutation(S)
    o1, l1 = orc.attention(q, k, v, False, 0.5)
    o2, l2 = orc.attention(q, k[:, :, perm], v[:, :, perm], False, 0.5)
    _close(o1, o2, 1e-12, "O under K/V permutation")
    _close(l1, l2, 1e-12, "lse under K/V permutation")


def pin_key_shift(orc):
    """Adding u to every key row leaves O unchanged and shifts lse_i by scale * <q_i, u>."""
    for causal in (False, True):
        B, H, S, D = 1, 2, 19, 4
        q, k, v = (_rand((B, H, S, D), 40 + t) for t in range(3))
        u = _rand((D,), 44, 1.5)
        scale = 0.6
        o1, l1 = orc.attention(q, k, v, causal, scale)
        o2, l2 = orc.attention(q, k + u, v, causal, scale)
        _close(o2, o1, 1e-11, "O under key shift")
        _close(l2, l1 + scale * (q @ u), 1e-11, "lse under key shift")


def pin_uniform_scores(orc):
    """Q = 0 makes every score 0: O is the mean of the attended V rows, lse = ln|J|."""
    B, H, S, D = 2, 1, 17, 3
    v = _rand((B, H, S, D), 50)
    k = _rand((B, H, S, D), 51)
    q = np.zeros((B, H, S, D))
    o, lse = orc.attention(q, k, v, False, 0.9)
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), 1e-12, "uniform O")
    _close(lse, np.full((B, H, S), math.log(S)), 1e-12, "uniform lse")
    o, lse = orc.attention(q, k, v, True, 0.9)
    prefix = np.cumsum(v, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    _close(o, prefix, 1e-12, "causal uniform O (prefix mean)")
    _close(lse, np.broadcast_to(np.log(np.arange(1, S + 1)), (B, H, S)), 1e-12, "causal uniform lse")


def pin_causal_row0(orc):
    """Causal row 0 sees only key 0: O[0] = V[0] and lse[0] = scale * <q_0, k_0>."""
    B, H, S, D = 2, 2, 11, 7
    q, k, v = (_rand((B, H, S, D), 60 + t) for t in range(3))
    o, lse = orc.attention(q, k, v, True, 0.45)
    _close(o[:, :, 0], v[:, :, 0], 1e-12, "causal row 0 O")
    _close(lse[:, :, 0], 0.45 * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), 1e-12, "causal row 0 lse")


def pin_single_key(orc):
    """S = 1: O = V and lse = scale * <q, k>, causal or not."""
    for causal in (False, True):
        q, k, v = (_rand((3, 2, 1, 5), 70 + t) for t in range(3))
        o, lse = orc.attention(q, k, v, causal, 1.3)
        _close(o, v, 1e-12, "S=1 O")
        _close(lse, 1.3 * np.sum(q * k, axis=-1), 1e-12, "S=1 lse")


def pin_last_row_agrees(orc):
    """Row S-1 attends to every key with or without the causal mask."""
    B, H, S, D = 2, 2, 33, 6
    q, k, v = (_rand((B, H, S, D), 80 + t) for t in range(3))
    o1, l1 = orc.attention(q, k, v, False, 0.4)
    o2, l2 = orc.attention(q, k, v, True, 0.4)
    _close(o2[:, :, -1], o1[:, :, -1], 1e-13, "last row O, causal vs not")
    _close(l2[:, :, -1], l1[:, :, -1], 1e-13, "last row lse, causal vs not")


def pin_torch_reference(orc):
    """Tiny shapes against torch's float64 softmax and logsumexp on an explicitly masked score matrix."""
    seed = 90
    for causal in (False, True):
        for (B, H, S, D) in [(1, 1, 1, 1), (1, 2, 3, 2), (2, 1, 5, 3), (1, 3, 8, 4), (2, 2, 7, 4)]:
            q, k, v = (_rand((B, H, S, D), seed + t) for t in range(3))
            seed += 3
            scale = 1.0 / math.sqrt(D)
            o, lse = orc.attention(q, k, v, causal, scale)
            tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
            s = torch.matmul(tq, tk.transpose(-1, -2)) * scale
            if causal:
                s = s.masked_fill(~torch.from_numpy(_mask(S, True)), float("-inf"))
            ref_o = torch.matmul(torch.softmax(s, dim=-1), tv).numpy()
            ref_l = torch.logsumexp(s, dim=-1).numpy()
            _close(o, ref_o, 1e-12, f"O vs torch {B,H,S,D} causal={causal}")
            _close(lse, ref_l, 1e-12, f"lse vs torch {B,H,S,D} causal={causal}")


def pin_large_scores(orc):
    """Scores of magnitude ~1e3 must not overflow: compare with torch's stable float64 softmax."""
    for causal in (False, True):
        B, H, S, D = 1, 2, 12, 4
        q, k, v = (_rand((B, H, S, D), 120 + t) for t in range(3))
        scale = 400.0
        o, lse = orc.attention(q, k, v, causal, scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        s = torch.matmul(tq, tk.transpose(-1, -2)) * scale
        if causal:
            s = s.masked_fill(~torch.from_numpy(_mask(S, True)), float("-inf"))
        _close(o, torch.matmul(torch.softmax(s, dim=-1), tv).numpy(), 1e-12, "large-score O")
        _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12, "large-score lse")


def pin_heads_independent(orc):
    """Each (b, h) slice of a [B,H,S,D] call equals a call on that slice alone."""
    for causal in (False, True):
        B, H, S, D = 2, 3, 9, 4
        q, k, v = (_rand((B, H, S, D), 130 + t) for t in range(3))
        o, lse = orc.attention(q, k, v, causal, 0.5)
        for b in range(B):
            for h in range(H):
                sl = (slice(b, b + 1), slice(h, h + 1))
                o1, l1 = orc.attention(q[sl], k[sl], v[sl], causal, 0.5)
                _close(o[sl], o1, 0.0, f"head ({b},{h}) O")
                _close(lse[sl], l1, 0.0, f"head ({b},{h}) lse")


def pin_rows_entry(orc):
    """The row-sampling entry point returns exactly the rows of the full call, in the order asked."""
    for causal in (False, True):
        B, H, S, D = 2, 2, 21, 5
        q, k, v = (_rand((B, H, S, D), 140 + t) for t in range(3))
        o, lse = orc.attention(q, k, v, causal, 0.8)
        rows = np.array([0, 5, B * H * S - 1, 22, 41, 20, 63], dtype=np.int64)
        orow, lrow = orc.attention_rows(q, k, v, causal, 0.8, rows)
        _close(orow, o.reshape(-1, D)[rows], 0.0, "rows entry O")
        _close(lrow, lse.reshape(-1)[rows], 0.0, "rows entry lse")


def pin_one_hot(orc):
    """A key aligned with the query and scaled up dominates: O -> that key's value row."""
    S, D = 6, 4
    k = _rand((1, 1, S, D), 150, 0.1)
    k[0, 0, 3] = np.eye(D)[0]
    v = _rand((1, 1, S, D), 151)
    q = np.zeros((1, 1, S, D))
    q[0, 0, :, :] = k[0, 0, 3, :] * 50.0  # every query points at key 3
    o, _ = orc.attention(q, k, v, False, 1.0)
    gap = 50.0 * (np.sum(k[0, 0, 3] ** 2) - np.max(np.delete(k[0, 0] @ k[0, 0, 3], 3)))
    assert gap > 40.0
    _close(o[0, 0], np.broadcast_to(v[0, 0, 3], (S, D)), 1e-12, "one-hot O")



# ------------------------------------------------------------------ backward pins
# The gradients are pinned to the forward oracle (already pinned above) through
# finite differences, to invariants of exact softmax attention that hold for any
# input, and to torch's float64 autograd of an explicitly written forward.


def _loss_fd(orc, q, k, v, dout, causal, scale, name, h=1e-5):
    """Central differences of L = sum(dout * O) with respect to q, k or v."""
    base = {"q": q, "k": k, "v": v}
    x = base[name]
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        vals = []
        for step in (h, -h):
            xs = x.copy()
            xs[idx] += step
            args = dict(base)
            args[name] = xs
            o, _ = orc.attention(args["q"], args["k"], args["v"], causal, scale)
            vals.append(float(np.sum(o * dout)))
        g[idx] = (vals[0] - vals[1]) / (2 * h)
    return g


def pin_bwd_finite_differences(orc):
    """dQ, dK, dV equal central differences of sum(dO * O) taken through the forward
    oracle (truncation ~h^2, rounding ~1e-16/h: agreement to 1e-7)."""
    for causal in (False, True):
        B, H, S, D = 1, 2, 6, 3
        q, k, v, dout = (_rand((B, H, S, D), 200 + t) for t in range(4))
        scale = 0.7
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal, scale)
        for name, got in (("q", dq), ("k", dk), ("v", dv)):
            fd = _loss_fd(orc, q, k, v, dout, causal, scale, name)
            _close(got, fd, 1e-7, f"d{name} vs finite differences (causal={causal})")


def pin_bwd_key_shift(orc):
    """Adding one vector to every key leaves every row's softmax unchanged, so the
    key gradients of a head sum to zero (causal too: row i's visible keys all shift)."""
    for causal in (False, True):
        B, H, S, D = 2, 2, 17, 5
        q, k, v, dout = (_rand((B, H, S, D), 210 + t) for t in range(4))
        _, dk, _ = orc.attention_bwd(q, k, v, dout, causal, 0.6)
        _close(dk.sum(axis=2), np.zeros((B, H, D)), 1e-12, f"sum_j dK_j (causal={causal})")


def pin_bwd_dv_mass(orc):
    """Each row of P sums to one, so sum_j dV_j = sum_i dO_i."""
    for causal in (False, True):
        B, H, S, D = 1, 3, 15, 4
        q, k, v, dout = (_rand((B, H, S, D), 220 + t) for t in range(4))
        _, _, dv = orc.attention_bwd(q, k, v, dout, causal, 0.8)
        _close(dv.sum(axis=2), dout.sum(axis=2), 1e-12, f"sum_j dV_j (causal={causal})")


def pin_bwd_euler(orc):
    """Scores are bilinear in q and k, so sum_i <dQ_i, Q_i> = sum_j <dK_j, K_j>
    (both equal sum_ij dS_ij s_ij); catches a gradient routed to the wrong operand."""
    for causal in (False, True):
        B, H, S, D = 2, 1, 13, 6
        q, k, v, dout = (_rand((B, H, S, D), 230 + t) for t in range(4))
        dq, dk, _ = orc.attention_bwd(q, k, v, dout, causal, 0.5)
        lhs = np.sum(dq * q, axis=(2, 3))
        rhs = np.sum(dk * k, axis=(2, 3))
        _close(lhs, rhs, 1e-12, f"Euler identity (causal={causal})")


def pin_bwd_single_key(orc):
    """S = 1: P = 1, so dV = dO and dS = 0 (dQ = dK = 0)."""
    for causal in (False, True):
        q, k, v, dout = (_rand((2, 2, 1, 4), 240 + t) for t in range(4))
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal, 1.1)
        _close(dv, dout, 1e-15, "S=1 dV")
        _close(dq, np.zeros_like(dq), 1e-15, "S=1 dQ")
        _close(dk, np.zeros_like(dk), 1e-15, "S=1 dK")


def pin_bwd_torch_autograd(orc):
    """Small shapes against torch float64 autograd of softmax(scale Q K^T + mask) V."""
    seed = 250
    for causal in (False, True):
        for (B, H, S, D) in [(1, 1, 3, 2), (1, 2, 9, 4), (2, 1, 16, 8)]:
            q, k, v, dout = (_rand((B, H, S, D), seed + t) for t in range(4))
            seed += 4
            scale = 1.0 / math.sqrt(D)
            tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
            s = torch.matmul(tq, tk.transpose(-1, -2)) * scale
            if causal:
                s = s.masked_fill(~torch.from_numpy(_mask(S, True)), float("-inf"))
            o = torch.matmul(torch.softmax(s, dim=-1), tv)
            o.backward(torch.from_numpy(dout))
            dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal, scale)
            for name, got, ref in (("dq", dq, tq.grad), ("dk", dk, tk.grad), ("dv", dv, tv.grad)):
                _close(got, ref.numpy(), 1e-12, f"{name} vs torch autograd {B,H,S,D} causal={causal}")


def pin_bwd_rows_entry(orc):
    """The sampled entry point returns dQ of query t and dK, dV of key t exactly as the full call."""
    for causal in (False, True):
        B, H, S, D = 2, 2, 19, 3
        q, k, v, dout = (_rand((B, H, S, D), 270 + t) for t in range(4))
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal, 0.9)
        rows = np.array([0, 7, 18, 19, 40, B * H * S - 1, 57], dtype=np.int64)
        rq, rk, rv = orc.attention_bwd_rows(q, k, v, dout, causal, 0.9, rows)
        _close(rq, dq.reshape(-1, D)[rows], 1e-13, "rows entry dQ")
        _close(rk, dk.reshape(-1, D)[rows], 1e-13, "rows entry dK")
        _close(rv, dv.reshape(-1, D)[rows], 1e-13, "rows entry dV")


# ------------------------------------------- grouped heads and sliding windows
# Grouped heads (GQA / MQA) and window_size = (left, right) ("Inside
# FlashAttention", section 6.1): query head h reads key/value head h // G,
# query i sees keys i - left .. i + right (and j <= i when causal).


def _band(S, causal, window):
    wl, wr = window
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    m = np.ones((S, S), dtype=bool)
    if causal:
        m &= j <= i
    if wl >= 0:
        m &= j >= i - wl
    if wr >= 0:
        m &= j <= i + wr
    return m


def pin_gqa_equals_replication(orc):
    """Grouped heads give exactly what K/V replicated to every query head give;
    dK, dV of a shared head are the sums over its query heads."""
    for causal in (False, True):
        B, H, Hkv, S, D = 2, 6, 2, 11, 4
        q, dout = _rand((B, H, S, D), 300), _rand((B, H, S, D), 301)
        k, v = _rand((B, Hkv, S, D), 302), _rand((B, Hkv, S, D), 303)
        kr, vr = np.repeat(k, H // Hkv, axis=1), np.repeat(v, H // Hkv, axis=1)
        o1, l1 = orc.attention(q, k, v, causal, 0.6)
        o2, l2 = orc.attention(q, kr, vr, causal, 0.6)
        _close(o1, o2, 1e-14, "GQA O vs replicated K/V")
        _close(l1, l2, 1e-14, "GQA lse vs replicated K/V")
        g1 = orc.attention_bwd(q, k, v, dout, causal, 0.6)
        g2 = orc.attention_bwd(q, kr, vr, dout, causal, 0.6)
        _close(g1[0], g2[0], 1e-13, "GQA dQ")
        for a, b, nm in ((g1[1], g2[1], "dK"), (g1[2], g2[2], "dV")):
            _close(a, b.reshape(B, Hkv, H // Hkv, S, D).sum(axis=2), 1e-13, f"GQA {nm} = group sum")


def pin_window_torch_reference(orc):
    """Windowed (and grouped) attention against torch float64 softmax of a band-masked
    score matrix, and its gradients against torch autograd."""
    seed = 310
    for causal, window in [(True, (3, -1)), (False, (2, 4)), (False, (0, 0)), (True, (0, 0)), (False, (-1, 1))]:
        B, H, Hkv, S, D = 1, 4, 2, 12, 3
        q, dout = _rand((B, H, S, D), seed), _rand((B, H, S, D), seed + 1)
        k, v = _rand((B, Hkv, S, D), seed + 2), _rand((B, Hkv, S, D), seed + 3)
        seed += 4
        o, lse = orc.attention(q, k, v, causal, 0.7, window)
        tq = torch.from_numpy(q.copy()).requires_grad_(True)
        tk = torch.from_numpy(k.copy()).requires_grad_(True)
        tv = torch.from_numpy(v.copy()).requires_grad_(True)
        ke = tk.repeat_interleave(H // Hkv, dim=1)
        ve = tv.repeat_interleave(H // Hkv, dim=1)
        sc = torch.matmul(tq, ke.transpose(-1, -2)) * 0.7
        sc = sc.masked_fill(~torch.from_numpy(_band(S, causal, window)), float("-inf"))
        ref_o = torch.matmul(torch.softmax(sc, dim=-1), ve)
        _close(o, ref_o.detach().numpy(), 1e-12, f"windowed O causal={causal} window={window}")
        _close(lse, torch.logsumexp(sc, dim=-1).detach().numpy(), 1e-12, f"windowed lse {window}")
        ref_o.backward(torch.from_numpy(dout))
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal, 0.7, window)
        for nm, got, ref in (("dQ", dq, tq.grad), ("dK", dk, tk.grad), ("dV", dv, tv.grad)):
            _close(got, ref.numpy(), 1e-12, f"windowed {nm} causal={causal} window={window}")


def pin_window_limits(orc):
    """A window wider than the sequence changes nothing; window (0, 0) leaves each
    query its own key: O = V, lse = scale <q, k>, dV = dO, dQ = dK = 0."""
    B, H, S, D = 2, 2, 9, 4
    q, k, v, dout = (_rand((B, H, S, D), 330 + t) for t in range(4))
    for causal in (False, True):
        o1, l1 = orc.attention(q, k, v, causal, 0.5)
        o2, l2 = orc.attention(q, k, v, causal, 0.5, (S, S))
        _close(o2, o1, 0.0, "window wider than S, O")
        _close(l2, l1, 0.0, "window wider than S, lse")
        o, lse = orc.attention(q, k, v, causal, 0.5, (0, 0))
        _close(o, v, 1e-15, "window (0,0) O = V")
        _close(lse, 0.5 * np.sum(q * k, axis=-1), 1e-14, "window (0,0) lse")
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal, 0.5, (0, 0))
        _close(dv, dout, 1e-15, "window (0,0) dV = dO")
        _close(dq, np.zeros_like(dq), 1e-15, "window (0,0) dQ")
        _close(dk, np.zeros_like(dk), 1e-15, "window (0,0) dK")


def pin_window_reversal(orc):
    """Reversing the sequence turns a (left, right) window into (right, left)."""
    B, H, S, D = 1, 2, 14, 3
    q, k, v = (_rand((B, H, S, D), 340 + t) for t in range(3))
    o1, l1 = orc.attention(q, k, v, False, 0.8, (2, 5))
    rev = (slice(None), slice(None), slice(None, None, -1))
    o2, l2 = orc.attention(q[rev], k[rev], v[rev], False, 0.8, (5, 2))
    _close(o2[rev], o1, 1e-13, "reversed window O")
    _close(l2[rev], l1, 1e-13, "reversed window lse")


def pin_window_finite_differences(orc):
    """Windowed, grouped gradients against central differences of sum(dO * O)."""
    B, H, Hkv, S, D = 1, 2, 1, 7, 2
    q, dout = _rand((B, H, S, D), 350), _rand((B, H, S, D), 351)
    k, v = _rand((B, Hkv, S, D), 352), _rand((B, Hkv, S, D), 353)
    window, h = (2, 1), 1e-5
    dq, dk, dv = orc.attention_bwd(q, k, v, dout, False, 0.9, window)
    for name, x, got in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            vals = []
            for step in (h, -h):
                xs = x.copy()
                xs[idx] += step
                args = {"q": q, "k": k, "v": v}
                args[name] = xs
                o, _ = orc.attention(args["q"], args["k"], args["v"], False, 0.9, window)
                vals.append(float(np.sum(o * dout)))
            fd[idx] = (vals[0] - vals[1]) / (2 * h)
        _close(got, fd, 1e-7, f"windowed grouped d{name} vs finite differences")


def pin_ex_rows_entries(orc):
    """With grouped heads and a window, the row entries equal the full entries
    (dK, dV addressed by key/value rows)."""
    B, H, Hkv, S, D = 2, 4, 2, 13, 3
    q, dout = _rand((B, H, S, D), 360), _rand((B, H, S, D), 361)
    k, v = _rand((B, Hkv, S, D), 362), _rand((B, Hkv, S, D), 363)
    for causal, window in ((True, (4, -1)), (False, (3, 2))):
        o, lse = orc.attention(q, k, v, causal, 0.4, window)
        rows = np.array([0, 5, 12, 13, 30, B * H * S - 1], dtype=np.int64)
        orow, lrow = orc.attention_rows(q, k, v, causal, 0.4, rows, window)
        _close(orow, o.reshape(-1, D)[rows], 0.0, "ex rows O")
        _close(lrow, lse.reshape(-1)[rows], 0.0, "ex rows lse")
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal, 0.4, window)
        krows = np.array([0, 3, 12, 20, B * Hkv * S - 1], dtype=np.int64)
        rq, rk, rv = orc.attention_bwd_rows(q, k, v, dout, causal, 0.4, rows, krows, window)
        _close(rq, dq.reshape(-1, D)[rows], 1e-13, "ex rows dQ")
        _close(rk, dk.reshape(-1, D)[krows], 1e-13, "ex rows dK")
        _close(rv, dv.reshape(-1, D)[krows], 1e-13, "ex rows dV")

# ------------------------------------------------ queries and keys of different length
# Sq queries and Sk keys (the CS336 write-up's forward kernel: N_QUERIES and
# N_KEYS, keys at or past N_KEYS absent, causal compares absolute positions,
# so query i sees keys 0..min(i, Sk-1)).


def _rect_band(Sq, Sk, causal, window=(-1, -1)):
    wl, wr = window
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    m = np.ones((Sq, Sk), dtype=bool)
    if causal:
        m &= j <= i
    if wl >= 0:
        m &= j >= i - wl
    if wr >= 0:
        m &= j <= i + wr
    return m


def pin_rect_sdpa(orc):
    """Sq != Sk against torch's float64 scaled_dot_product_attention (its causal
    mask is the top-left lower triangle of the [Sq, Sk] score matrix) and the
    logsumexp of the masked scores."""
    seed = 400
    for (B, H, Sq, Sk, D) in [(1, 2, 5, 9, 4), (2, 1, 9, 4, 3), (1, 1, 1, 6, 2), (1, 1, 6, 1, 2)]:
        for causal in (False, True):
            q = _rand((B, H, Sq, D), seed)
            k, v = _rand((B, H, Sk, D), seed + 1), _rand((B, H, Sk, D), seed + 2)
            seed += 3
            o, lse = orc.attention(q, k, v, causal, 0.45)
            tq, tk, tv = (torch.from_numpy(x.copy()) for x in (q, k, v))
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.45)
            _close(o, ref.numpy(), 1e-12, f"rect O {B,H,Sq,Sk,D} causal={causal}")
            sc = (torch.matmul(tq, tk.transpose(-1, -2)) * 0.45).masked_fill(
                ~torch.from_numpy(_rect_band(Sq, Sk, causal)), float("-inf"))
            _close(lse, torch.logsumexp(sc, dim=-1).numpy(), 1e-12, f"rect lse {B,H,Sq,Sk,D} causal={causal}")


def pin_rect_prefix(orc):
    """Sq < Sk: the queries are the first Sq rows of a square problem over the same
    keys, so O, lse and dQ equal that problem's first Sq rows."""
    B, H, Sq, Sk, D = 2, 2, 5, 13, 3
    qf, doutf = _rand((B, H, Sk, D), 420), _rand((B, H, Sk, D), 421)
    k, v = _rand((B, H, Sk, D), 422), _rand((B, H, Sk, D), 423)
    for causal in (False, True):
        o1, l1 = orc.attention(qf[:, :, :Sq], k, v, causal, 0.7)
        o2, l2 = orc.attention(qf, k, v, causal, 0.7)
        _close(o1, o2[:, :, :Sq], 1e-15, f"rect prefix O causal={causal}")
        _close(l1, l2[:, :, :Sq], 1e-15, f"rect prefix lse causal={causal}")
        dq1 = orc.attention_bwd(qf[:, :, :Sq], k, v, doutf[:, :, :Sq], causal, 0.7)[0]
        dq2 = orc.attention_bwd(qf, k, v, doutf, causal, 0.7)[0]
        _close(dq1, dq2[:, :, :Sq], 1e-14, f"rect prefix dQ causal={causal}")


def pin_rect_rows_past_keys(orc):
    """Sq > Sk, causal: rows i >= Sk - 1 see every key (they equal the non-causal
    rows) and rows i < Sk are the square causal problem on the first Sk queries."""
    B, H, Sq, Sk, D = 1, 3, 11, 4, 5
    q = _rand((B, H, Sq, D), 430)
    k, v = _rand((B, H, Sk, D), 431), _rand((B, H, Sk, D), 432)
    oc, lc = orc.attention(q, k, v, True, 0.8)
    on, ln = orc.attention(q, k, v, False, 0.8)
    _close(oc[:, :, Sk - 1:], on[:, :, Sk - 1:], 1e-15, "causal rows past the keys O")
    _close(lc[:, :, Sk - 1:], ln[:, :, Sk - 1:], 1e-15, "causal rows past the keys lse")
    os_, ls_ = orc.attention(q[:, :, :Sk], k, v, True, 0.8)
    _close(oc[:, :, :Sk], os_, 1e-15, "causal rows below Sk O")
    _close(lc[:, :, :Sk], ls_, 1e-15, "causal rows below Sk lse")


def pin_rect_empty_rows(orc):
    """A window can leave a query with no key when Sq > Sk: such a row has O = 0,
    lse = -inf, dQ = 0 and adds nothing to dK, dV (the gradients equal those of
    the problem without those rows)."""
    B, H, Sq, Sk, D = 1, 2, 7, 3, 2
    q, dout = _rand((B, H, Sq, D), 440), _rand((B, H, Sq, D), 441)
    k, v = _rand((B, H, Sk, D), 442), _rand((B, H, Sk, D), 443)
    for causal in (False, True):
        window = (1, 0)  # rows 4..6 see keys i-1..i, all past Sk - 1 = 2
        o, lse = orc.attention(q, k, v, causal, 0.6, window)
        _close(o[:, :, 4:], np.zeros((B, H, 3, D)), 0.0, f"empty rows O causal={causal}")
        assert np.all(np.isneginf(lse[:, :, 4:])), f"empty rows lse must be -inf, got {lse[:, :, 4:]}"
        assert np.all(np.isfinite(lse[:, :, :4])), "rows with keys must have finite lse"
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal, 0.6, window)
        _close(dq[:, :, 4:], np.zeros((B, H, 3, D)), 0.0, f"empty rows dQ causal={causal}")
        dq4, dk4, dv4 = orc.attention_bwd(q[:, :, :4], k, v, dout[:, :, :4], causal, 0.6, window)
        _close(dq[:, :, :4], dq4, 1e-15, "rows with keys dQ")
        _close(dk, dk4, 1e-15, "empty rows add nothing to dK")
        _close(dv, dv4, 1e-15, "empty rows add nothing to dV")


def pin_rect_bwd_torch_autograd(orc):
    """Sq != Sk gradients (with grouped heads and a window) against torch float64
    autograd of softmax over the masked [Sq, Sk] score matrix."""
    seed = 450
    cases = [(1, 2, 2, 5, 9, 3, False, (-1, -1)), (1, 2, 1, 9, 5, 2, True, (-1, -1)),
             (2, 4, 2, 6, 11, 2, True, (2, -1)), (1, 2, 2, 10, 7, 3, False, (3, 1))]
    for (B, H, Hkv, Sq, Sk, D, causal, window) in cases:
        q, dout = _rand((B, H, Sq, D), seed), _rand((B, H, Sq, D), seed + 1)
        k, v = _rand((B, Hkv, Sk, D), seed + 2), _rand((B, Hkv, Sk, D), seed + 3)
        seed += 4
        tq = torch.from_numpy(q.copy()).requires_grad_(True)
        tk = torch.from_numpy(k.copy()).requires_grad_(True)
        tv = torch.from_numpy(v.copy()).requires_grad_(True)
        ke = tk.repeat_interleave(H // Hkv, dim=1)
        ve = tv.repeat_interleave(H // Hkv, dim=1)
        sc = (torch.matmul(tq, ke.transpose(-1, -2)) * 0.5).masked_fill(
            ~torch.from_numpy(_rect_band(Sq, Sk, causal, window)), float("-inf"))
        ref_o = torch.matmul(torch.softmax(sc, dim=-1), ve)
        o, lse = orc.attention(q, k, v, causal, 0.5, window)
        _close(o, ref_o.detach().numpy(), 1e-12, f"rect O {Sq, Sk} causal={causal} window={window}")
        ref_o.backward(torch.from_numpy(dout))
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal, 0.5, window)
        for nm, got, ref in (("dQ", dq, tq.grad), ("dK", dk, tk.grad), ("dV", dv, tv.grad)):
            _close(got, ref.numpy(), 1e-12, f"rect {nm} {Sq, Sk} causal={causal} window={window}")


def pin_rect_rows_entries(orc):
    """With Sq != Sk the row entries index query rows by Sq and key rows by Sk and
    return exactly the full entries' rows."""
    B, H, Hkv, Sq, Sk, D = 2, 2, 1, 6, 10, 3
    q, dout = _rand((B, H, Sq, D), 470), _rand((B, H, Sq, D), 471)
    k, v = _rand((B, Hkv, Sk, D), 472), _rand((B, Hkv, Sk, D), 473)
    for causal, window in ((False, (-1, -1)), (True, (-1, -1)), (False, (2, 3))):
        o, lse = orc.attention(q, k, v, causal, 0.4, window)
        rows = np.array([0, 5, 6, 13, B * H * Sq - 1], dtype=np.int64)
        ro, rl = orc.attention_rows(q, k, v, causal, 0.4, rows, window)
        _close(ro, o.reshape(-1, D)[rows], 0.0, "rect rows entry O")
        _close(rl, lse.reshape(-1)[rows], 0.0, "rect rows entry lse")
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal, 0.4, window)
        krows = np.array([0, 9, 10, 17, B * Hkv * Sk - 1], dtype=np.int64)
        rq, rk, rv = orc.attention_bwd_rows(q, k, v, dout, causal, 0.4, rows, krows, window)
        _close(rq, dq.reshape(-1, D)[rows], 1e-13, "rect rows entry dQ")
        _close(rk, dk.reshape(-1, D)[krows], 1e-13, "rect rows entry dK")
        _close(rv, dv.reshape(-1, D)[krows], 1e-13, "rect rows entry dV")


ALL_PINS = [
    pin_worked_example,
    pin_normalisation,
    pin_convex_hull,
    pin_permutation,
    pin_key_shift,
    pin_uniform_scores,
    pin_causal_row0,
    pin_single_key,
    pin_last_row_agrees,
    pin_torch_reference,
    pin_large_scores,
    pin_heads_independent,
    pin_rows_entry,
    pin_one_hot,
    pin_bwd_finite_differences,
    pin_bwd_key_shift,
    pin_bwd_dv_mass,
    pin_bwd_euler,
    pin_bwd_single_key,
    pin_bwd_torch_autograd,
    pin_bwd_rows_entry,
    pin_gqa_equals_replication,
    pin_window_torch_reference,
    pin_window_limits,
    pin_window_reversal,
    pin_window_finite_differences,
    pin_ex_rows_entries,
    pin_rect_sdpa,
    pin_rect_prefix,
    pin_rect_rows_past_keys,
    pin_rect_empty_rows,
    pin_rect_bwd_torch_autograd,
    pin_rect_rows_entries,
]
