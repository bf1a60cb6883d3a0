"""Bank model of the k-row weight tiles (stated [K][N] weight layout).

The GEMM kernel stores 16-byte chunk c of contraction row k of a weight tile
at chunk c ^ key(k) and reads MFMA fragments with gfx950's transposing LDS
loads (bf16: 8 bytes per lane, lanes m of a 16-lane group addressing rows
k0 + m / 4, columns 4 (m % 4)..; FP8: rows k0 + m / 2, columns 8 (m % 2)..;
fp32: one element per lane).  With 64 banks of 4 bytes, serving 8-byte reads
32 lanes at a time and 4-byte reads 64 at a time, the keys the kernel uses
(kn_key in csrc/gemm.hip) must let every read touch each bank at most once
per pass.  The same model shows the unswizzled layout 4 to 16 times slower.
"""
import pytest


def key(es, hb, k):
    # the kernel's kn_key: bf16, FP8 and fp32 k-row tiles
    if es == 2:
        return ((k << 2) ^ (k >> 2)) if hb >= 256 else (k ^ (k >> 1))
    if es == 1:
        return k ^ (k >> 2) ^ (k >> 3)
    return k


def phys(es, hb, k, byte, swizzle=True):
    ch = byte // 16
    if swizzle:
        ch = (ch ^ key(es, hb, k)) & (hb // 16 - 1)
    return k * hb + ch * 16 + byte % 16


def passes(addrs, width):
    lanes = {4: 64, 8: 32}[width]
    total = 0
    for p in range(0, 64, lanes):
        banks = {}
        for a in addrs[p:p + lanes]:
            for w in range(0, width, 4):
                d = (a + w) // 4
                banks.setdefault(d % 64, set()).add(d)
        total += max(len(v) for v in banks.values())
    return total


def fragment_reads(es, hb, cols, swizzle=True):
    """(addresses, bytes per lane) of every weight-fragment read of one stage
    for fragments starting at the given tile columns"""
    out = []
    for c0 in cols:
        if es == 2:  # two k-steps of 32, two 4-row reads each
            for kk in range(2):
                for r in range(2):
                    a = [phys(es, hb, 32 * kk + 8 * (l // 16) + 4 * r + (l % 16) // 4,
                              (c0 + 4 * (l % 4)) * 2, swizzle) for l in range(64)]
                    out.append((a, 8))
        elif es == 1:  # 32 rows per lane, four 8-row reads
            for r in range(4):
                a = [phys(es, hb, 32 * (l // 16) + 8 * r + (l % 16) // 2,
                          c0 + 8 * (l % 2), swizzle) for l in range(64)]
                out.append((a, 8))
        else:  # four single-element reads, rows 4 lg + u
            for u in range(4):
                a = [phys(es, hb, 4 * (l // 16) + u, (c0 + l % 16) * 4, swizzle)
                     for l in range(64)]
                out.append((a, 4))
    return out


# (element bytes, row bytes of a half tile, fragment column starts of a wave)
CASES = [(2, 256, [0, 16]), (2, 512, [0, 16, 32, 48]), (2, 128, [0, 16]), (2, 256, [0, 32]),
         (1, 128, [0, 16]), (1, 256, [0, 16, 32, 48]), (4, 256, [0, 16]), (4, 512, [0, 16])]


@pytest.mark.parametrize("es,hb,cols", CASES)
def test_kn_fragment_reads_are_conflict_free(es, hb, cols):
    reads = fragment_reads(es, hb, cols)
    ideal = sum({4: 1, 8: 2}[w] for _, w in reads)
    assert sum(passes(a, w) for a, w in reads) == ideal
    plain = fragment_reads(es, hb, cols, swizzle=False)
    assert sum(passes(a, w) for a, w in plain) >= 4 * ideal


@pytest.mark.parametrize("es,hb,cols", CASES)
def test_kn_swizzle_is_a_permutation_of_each_row(es, hb, cols):
    # the DMA writes physical chunk p from logical chunk p ^ key: every
    # logical chunk of a row lands exactly once
    nch = hb // 16
    for k in range(128):
        assert sorted((c ^ key(es, hb, k)) & (nch - 1) for c in range(nch)) == list(range(nch))
