"""The seeded shape generators of the random-shape tests: host arithmetic
only (numpy), shared by the GPU parity tests and the CPU check that every
case lands in the kernel-selection regime it was drawn for."""
import numpy as np

FULL_GRID = 512  # workgroups that fill the GPU twice over (the dispatch's threshold)


def cdiv(a, b):
    return -(-a // b)


def heads(rng, need_bh, max_b=8):
    """(B, H, H_kv) with H = G * H_kv, G in {1, 2, 4}, and B * H >= need_bh."""
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4]))
    h = hkv * g
    b = max(1, cdiv(need_bh, h))
    while b > max_b:  # too many batches: widen the heads instead
        hkv *= 2
        h = hkv * g
        b = max(1, cdiv(need_bh, h))
    return b, h, hkv


def window_of(rng):
    return tuple(int(x) for x in rng.choice([-1, 0, 3, 17, 64, 200, 700], size=2))


def make_cases():
    rng = np.random.default_rng(20261202)
    cases = []
    # large grids: the two-block kernel (D = 32, 64: 256 rows), the one-block
    # kernel on 128 rows (D = 16) and on 8-wave 256-row workgroups (D = 128)
    for i in range(8):
        D = [32, 64, 16, 128][i % 4]
        S = int(rng.integers(500, 2200))
        rows = 128 if D == 16 else 256
        B, H, Hkv = heads(rng, cdiv(FULL_GRID, cdiv(S, rows)))
        win = window_of(rng) if i >= 6 else None
        cases.append(dict(kind="large", B=B, H=H, Hkv=Hkv, Sq=S, Sk=S, D=D, dtype=["f16", "bf16"][i % 2],
                          causal=bool(rng.integers(0, 2)) or i < 2, window=win))
    # the key split's grids: causal, no window, S_q = S_k, the whole grid
    # resident: n query blocks x B*H = 512 at D = 16, 32, 64; at D = 128,
    # n 128-row blocks x B*H = 256 with 64-row blocks reaching 512 (S in the
    # upper half of its last 128-row block)
    for i, (D, n) in enumerate([(64, 2), (64, 8), (32, 4), (32, 16), (16, 4), (16, 16), (128, 8), (128, 16)]):
        rows = 128 if D in (16, 128) else 256
        lo = (n - 1) * rows + (65 if D == 128 else 1)
        S = int(rng.integers(lo, n * rows + 1))
        bh = (FULL_GRID if D != 128 else 256) // n
        hkv = int(rng.choice([1, 2]))
        H = 2 * hkv if bh % (2 * hkv) == 0 else hkv
        cases.append(dict(kind="split", B=bh // H, H=H, Hkv=hkv, Sq=S, Sk=S, D=D, dtype=["f16", "bf16"][i % 2],
                          causal=True, window=None))
    # D = 128 grids between the key split and the large tile (128 rows)
    for i in range(2):
        S = int(rng.integers(2100, 4000))
        bh = int(rng.integers(cdiv(FULL_GRID, cdiv(S, 64)), cdiv(FULL_GRID, cdiv(S, 256))))
        cases.append(dict(kind="mid128", B=bh, H=1, Hkv=1, Sq=S, Sk=S, D=128, dtype=["bf16", "f16"][i],
                          causal=bool(i), window=None))
    # thin grids (keys split across the waves of a workgroup), fp32 included
    for i in range(10):
        D = int(rng.choice([16, 32, 64, 128]))
        B, H, Hkv = heads(rng, int(rng.integers(1, 9)), max_b=2)
        S = int(rng.integers(1, 3000))
        cases.append(dict(kind="thin", B=B, H=H, Hkv=Hkv, Sq=S, Sk=S, D=D, dtype=["f16", "bf16", "f32"][i % 3],
                          causal=bool(i % 2), window=window_of(rng) if i % 4 == 3 else None))
    # queries and keys of different length, with and without windows
    for i in range(8):
        D = int(rng.choice([16, 32, 64, 128]))
        B, H, Hkv = heads(rng, int(rng.integers(1, 33)), max_b=4)
        Sq, Sk = (int(x) for x in rng.integers(1, 1800, size=2))
        cases.append(dict(kind="rect", B=B, H=H, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, dtype=["f16", "bf16", "f32"][i % 3],
                          causal=bool(i % 2), window=window_of(rng) if i >= 4 else None))
    return cases


def make_bwd_cases():
    rng = np.random.default_rng(20261203)
    cases = []
    for i in range(10):
        D = [16, 32, 64, 128][i % 4]
        if i < 4:  # grids of at least 512 dK/dV workgroups (128 keys each)
            S = int(rng.integers(300, 1300))
            B, H, Hkv = heads(rng, cdiv(FULL_GRID, cdiv(S, 128)))
            # K/V heads set the dK/dV grid: widen B until it is full
            while B * Hkv * cdiv(S, 128) < FULL_GRID:
                B += 1
            Sq = Sk = S
        else:
            B, H, Hkv = heads(rng, int(rng.integers(1, 17)), max_b=4)
            Sq = int(rng.integers(1, 1500))
            Sk = Sq if i < 7 else int(rng.integers(1, 1500))
        cases.append(dict(kind="bwd", B=B, H=H, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, dtype=["f16", "bf16"][i % 2],
                          causal=bool(rng.integers(0, 2)), window=window_of(rng) if i in (5, 8) else None))
    return cases


CASES = make_cases()
BWD_CASES = make_bwd_cases()


def case_id(c):
    w = "" if c["window"] is None else f"-w{c['window'][0]}_{c['window'][1]}"
    return (f"{c['kind']}-{c['dtype']}-B{c['B']}H{c['H']}kv{c['Hkv']}-S{c['Sq']}x{c['Sk']}-D{c['D']}"
            f"-{'c' if c['causal'] else 'n'}{w}")
