"""The random-shape cases land in the kernel-selection regime each was drawn
for (host arithmetic only, no GPU): the key split's cases are exactly those
for which the library sizes a workspace, and every family is present."""
import exact_tiled_attention_06_amd as fa
from fuzz_cases import BWD_CASES, CASES, case_id
from parity_util import DT


def test_cases_reach_every_regime():
    kinds = {c["kind"] for c in CASES}
    assert kinds == {"large", "split", "mid128", "thin", "rect"}
    for c in CASES:
        code = fa.DTYPE_CODES[DT[c["dtype"]]]
        wl, wr = (-1, -1) if c["window"] is None else c["window"]
        nb = fa.fa_fwd_workspace_bytes(c["B"], c["H"], c["Hkv"], c["Sq"], c["Sk"], c["D"], int(c["causal"]), wl, wr,
                                       code)
        assert (nb > 0) == (c["kind"] == "split"), case_id(c)
        assert c["H"] % c["Hkv"] == 0


def test_backward_cases():
    """Half of the backward cases fill the dK/dV grid (K/V heads x 128-key
    blocks >= 512 workgroups), the rest are thin; every head count divides."""
    full = [c for c in BWD_CASES if c["B"] * c["Hkv"] * -(-c["Sk"] // 128) >= 512]
    assert len(full) >= 4
    assert all(c["H"] % c["Hkv"] == 0 and c["dtype"] in ("f16", "bf16") for c in BWD_CASES)
    assert len({case_id(c) for c in CASES + BWD_CASES}) == len(CASES) + len(BWD_CASES)
