"""CPU model of the fp32 attention kernel's index arithmetic (attn_f32_kernel):
the key groups' tile dealing, the tile loads and LDS stores, the merge state
and the query rows, checked for coverage and bounds on seeded segment lists.

The kernel's shape constants are read from kernels.hip, so a change there is
checked by the same model; the formulas below restate the kernel's."""
import os
import re

import numpy as np
import pytest

from conftest import ROOT

SRC = open(os.path.join(ROOT, "bounded_kv_block_amd", "csrc", "kernels.hip")).read()
F32 = SRC[SRC.index("void attn_f32_kernel(AttnArgs a)"):SRC.index("// ------------------------------------------------------------------ ConvKV gather")]
LAUNCH = SRC[SRC.index("attn_f32_kernel<64><<<") - 200:SRC.index("attn_f32_kernel<128><<<") + 80]


def shape(D):
    """(G, LG, QPB, KG, BNF, NL, threads, queries per workgroup in the launch)"""
    def pick(name):
        m = re.search(rf"constexpr int {name} = D == 64 \? (\d+) : (\d+);", F32)
        return int(m.group(1) if D == 64 else m.group(2))
    G, LG, KG, BNF = D // 8, pick("LG"), pick("KG"), pick("BNF")
    QPB = LG // G
    NL = BNF * D // 4 // LG
    m = re.search(rf"const int nwg = \(\(a\.T \+ (\d+)\) / (\d+)\) \* a\.H;[^\n]*\n\s*attn_f32_kernel<{D}><<<nwg, (\d+)",
                  LAUNCH)
    assert m, f"launch of attn_f32_kernel<{D}> not found"
    assert int(m.group(1)) + 1 == int(m.group(2))
    return G, LG, QPB, KG, BNF, NL, int(m.group(3)), int(m.group(2))


@pytest.mark.parametrize("D", [64, 128])
def test_launch_matches_kernel_shape(D):
    """Threads = KG groups of LG lanes (within the launch bound and the
    1024-thread limit); the launch's queries per workgroup are the kernel's;
    both LDS tile sets and the merge states fit the 160 KiB of a CU."""
    G, LG, QPB, KG, BNF, NL, threads, qpw = shape(D)
    assert threads == KG * LG <= 1024
    assert qpw == QPB
    bound = int(re.search(r"__launch_bounds__\(D == 64 \? (\d+) : (\d+)\) void attn_f32_kernel", SRC)
                .group(1 if D == 64 else 2))
    assert threads <= bound
    assert LG % 64 == 0 and LG % G == 0            # groups are whole waves of whole queries
    assert NL * LG * 4 == BNF * D                  # the loads cover a tile exactly
    assert 2 * KG * BNF * D * 4 + 4096 <= 160 * 1024
    assert KG == 1 or (KG - 1) * 10 * LG <= KG * BNF * D


def deal(ns, KG, BNF):
    """The kernel's cursors: tiles in segment order, group g starts at tile g
    and moves KG tiles per round; returns, per round, each group's tile or None."""
    nseg = len(ns)

    def skip_empty(sg, j0):
        while sg < nseg and j0 >= ns[sg]:
            sg, j0 = sg + 1, 0
        return sg, j0

    def advance(sg, j0, k):
        i = 0
        while i < k and sg < nseg:
            sg, j0 = skip_empty(sg, j0 + BNF)
            i += 1
        return sg, j0

    ntiles = sum((n + BNF - 1) // BNF for n in ns)
    rounds = (ntiles + KG - 1) // KG
    cur = [advance(*skip_empty(0, 0), g) for g in range(KG)]
    out = []
    for _ in range(rounds):
        out.append([c if c[0] < nseg else None for c in cur])
        cur = [advance(sg, j0, KG) for sg, j0 in cur]
    return out, ntiles


@pytest.mark.parametrize("D", [64, 128])
def test_key_groups_visit_every_tile_once(D):
    """Every context tile (empty and ragged segments included) is run by exactly
    one group in exactly one round, and each group runs its tiles in order."""
    _, _, _, KG, BNF, _, _, _ = shape(D)
    rng = np.random.default_rng(7)
    cases = [[1], [BNF], [BNF + 1], [0, 5, 0], [3 * BNF, 0, 1, BNF - 1, 2 * BNF + 7]]
    cases += [list(rng.integers(0, 5 * BNF, size=rng.integers(1, 21))) for _ in range(200)]
    for ns in cases:
        rounds, ntiles = deal(ns, KG, BNF)
        want = [(sg, j0) for sg, n in enumerate(ns) for j0 in range(0, n, BNF)]
        got = [t for r in rounds for t in r if t is not None]
        assert sorted(got) == want and len(got) == ntiles, ns
        assert len(rounds) == (ntiles + KG - 1) // KG
        for g in range(KG):
            seq = [r[g] for r in rounds if r[g] is not None]
            assert seq == sorted(seq), (ns, g)


@pytest.mark.parametrize("D", [64, 128])
def test_tile_loads_and_stores_cover_the_tile(D):
    """Each lane's float4 loads read K rows and V^T columns of the tile only
    (row r < BNF, channel d < D), every 16-byte chunk of K and every four keys
    of a V^T row exactly once; the XOR placement puts a key row's chunks at
    distinct positions of its LDS row."""
    G, LG, QPB, KG, BNF, NL, _, _ = shape(D)
    NC = D // 4
    kseen = np.zeros((BNF, NC), int)
    vseen = np.zeros((D, BNF // 4), int)
    for gt in range(LG):
        for it in range(NL):
            idx = it * LG + gt
            r, c4 = divmod(idx, NC)
            assert r < BNF
            kseen[r, c4] += 1
            d, q = divmod(idx, BNF // 4)
            jj = 4 * q
            assert d < D and jj + 3 < BNF
            vseen[d, q] += 1
    assert (kseen == 1).all() and (vseen == 1).all()
    for j in range(BNF):
        pos = [(qc ^ (j & (NC - 1))) for qc in range(NC)]
        assert sorted(pos) == list(range(NC))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 7, 8, 9, 128, 257, 3510])
def test_query_rows_cover_the_block(D, T):
    """qrow = qt * QPB + lane / G over nqt = ceil(T / QPB) workgroups of a head
    covers every query once; rows past T only exist in the last workgroup."""
    G, LG, QPB, KG, BNF, NL, _, qpw = shape(D)
    nqt = (T + qpw - 1) // qpw
    rows = [qt * QPB + gt // G for qt in range(nqt) for gt in range(0, LG, G)]
    assert sorted(r for r in rows if r < T) == list(range(T))
    assert all(r < nqt * QPB for r in rows)
