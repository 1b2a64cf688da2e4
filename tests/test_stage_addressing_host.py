"""Host model of the prefill kernel's bias-stage loads (relative_position_bias_paged_amd/csrc/prefill_bf16.hip).

Each wave stages, for a key tile s0 in its band, 64 consecutive bias
distances of each of its 32 query rows, through a buffer resource based on
one row of its own and per-lane byte offsets.  The hardware reads memory
only for offsets below the resource's record count and returns zeros above
it.  The model repeats the kernel's work-group layout (heads per work-group,
query blocks, waves past the sequence), its band and edge-wave tests and the
offsets, and checks on the CPU that:

* every access the range check lets through lies inside the bias tensor,
  including for waves wholly past a short last sequence;
* every row of a query inside the sequence reads bias[token, head, d] for
  the first distance d of its 8-element run, i.e. the element the layout
  [total_tokens][Hq][rel_extent] puts there;
* basing a wave's resource on its first query's row, which lies past the
  sequence for such waves, fails the first check (the model can tell).

For the variant that forms the bias in the kernel, a second model follows
one band tile's product through the stage: the 16-byte stores stay aligned
and inside the stage part, and every element a lane reads back was written
by exactly one lane, with the value its query and distance name.  Without
the product's row permutation, the read-back fails.
"""
import random

import numpy as np
import pytest

BN = 64                  # keys per tile
STAGE_PAST = 0xC0000000  # offset given to rows of queries past the sequence


def _heads_per_wg(G, NW):
    hpw = 1
    while hpw * 2 <= NW and G % (hpw * 2) == 0:
        hpw *= 2
    return hpw


def stage_accesses(Hq, Hkv, R, W, lens, new, base_on_first_query=False):
    """Yield (lane row index array, in-range mask, byte address, expected
    element or -1) for every (wave, tile) that stages bias."""
    G = Hq // Hkv
    NW = 4 if W > 0 else 8               # wave count of the streamed-bias kernel
    hpw = _heads_per_wg(G, NW)
    QM = 32 * (NW // hpw)
    Ls = list(new) if new is not None else list(lens)
    cu = np.concatenate([[0], np.cumsum(Ls)]).astype(np.int64)
    elems = int(cu[-1]) * Hq * R
    nrec = min((31 * Hq * R + R + 256) * 2, 2**31 - 1)
    lane = np.arange(64)
    col = lane & 31
    rq = 8 * np.arange(4)[:, None] + (lane >> 3)[None, :]        # stage write k, lane
    chunk = (lane & 7)[None, :] ^ ((rq >> 1) & 7)
    for b, L in enumerate(Ls):
        n_k = lens[b]
        hist = n_k - L
        tok0 = int(cu[b])
        for qt in range(-(-max(Ls) // QM)):
            t0 = qt * QM
            if t0 >= L:
                continue
            for kvh in range(Hkv):
                for hg in range(G // hpw):
                    for wave in range(NW):
                        h = kvh * G + hg * hpw + wave % hpw
                        tq0 = t0 + 32 * (wave // hpw)
                        pq0 = hist + tq0
                        t = tq0 + col
                        row_off = ((tok0 + np.where(t < L, t, 0)) * Hq + h).astype(np.int64) * R
                        if np.any((row_off < 1024) | (elems - row_off < R + 1024)):
                            continue             # edge wave: element reads, no stage
                        wide = W <= 0 or W > R
                        s_band = pq0 - (BN - 2) - R - (0 if wide else 1)
                        s_lo = pq0 - (BN - 1) - W if W > 0 else -2**31
                        lo = max(s_lo, s_band, -1)
                        span = max(pq0 + 31 - lo, 0)
                        tq = tq0 + rq
                        valid = tq < L
                        tq_base = tq0 if base_on_first_query else min(tq0, L - 1)
                        srow0 = (tok0 + tq_base) * Hq + h
                        base = (srow0 * R - 128) * 2
                        run0 = hist + tq - (BN - 1) + 8 * chunk      # first distance of tile 0
                        if base_on_first_query:
                            sofs = (np.where(valid, rq * Hq, 0) * R + 128 + run0) * 2
                        else:
                            sofs = np.where(valid, ((tq - tq_base) * Hq * R + 128 + run0) * 2, STAGE_PAST)
                        for s0 in range(0, n_k, BN):
                            if not (s0 - lo - 1) % 2**32 < span:
                                continue
                            off = (sofs - 2 * s0) % 2**32
                            d = run0 - s0
                            expect = np.where(valid, ((tok0 + tq) * Hq + h) * R + d, -1)
                            yield valid, off < nrec, base + off, expect


def check(Hq, Hkv, R, W, lens, new, **kw):
    nbytes = sum(new if new is not None else lens) * Hq * R * 2
    outside = loads = 0
    for valid, inrange, addr, expect in stage_accesses(Hq, Hkv, R, W, lens, new, **kw):
        loads += int(inrange.sum())
        outside += int((inrange & ((addr < 0) | (addr + 16 > nbytes))).sum())
        if not kw:
            # rows inside the sequence read their own element; the others nothing
            assert np.all(inrange == valid)
            assert np.array_equal(addr[valid], 2 * expect[valid])
    return outside, loads


# the clamp-only grouping cases of the prefill GPU tests, GQA and MHA pools
CASES = [
    (8, 2, 64, 0, [1000, 65, 700, 129], None),
    (8, 2, 100, 0, [513, 300, 64], None),
    (4, 1, 32, 0, [900, 257], None),
    (16, 2, 128, 0, [2000], None),
    (8, 2, 64, 0, [1500, 700], [333, 64]),
    (8, 2, 128, 128, [4096, 700], [512, 64]),
    (8, 4, 256, 1000, [3000, 40], [3000, 40]),
]


@pytest.mark.parametrize("Hq,Hkv,R,W,lens,new", CASES)
@pytest.mark.parametrize("mha", [False, True])
def test_stage_reads_stay_inside_the_bias(Hq, Hkv, R, W, lens, new, mha):
    outside, loads = check(Hq, Hq if mha else Hkv, R, W, lens, new)
    assert loads > 0 and outside == 0


def test_stage_reads_random_layouts():
    rng = random.Random(5)
    for _ in range(40):
        Hkv = rng.choice([1, 2, 4])
        Hq = Hkv * rng.choice([1, 2, 3, 4, 8])
        R = rng.choice([8, 16, 32, 64, 100, 128, 256])
        W = rng.choice([0, 0, 16, 64, 100, 128, 300, 1000])
        new = [rng.randint(1, 700) for _ in range(rng.randint(1, 4))]
        lens = [n + rng.choice([0, 0, rng.randint(0, 900)]) for n in new]
        assert check(Hq, Hkv, R, W, lens, new)[0] == 0, (Hq, Hkv, R, W, lens, new)


def test_model_catches_a_resource_past_the_sequence():
    # MHA over a 64-query last sequence: waves 2-7 of its 256-query
    # work-group lie wholly past it, so a resource on their first query's row
    # starts past the tensor
    outside, _ = check(8, 8, 64, 0, [1500, 700], [333, 64], base_on_first_query=True)
    assert outside > 0


# ---- fused variant: the stage the bias product is written to and read from ----
# (prefill_bf16.hip: rows of 105 elements; part 1 of a separate 4 KiB slice 16
# elements in, else 16 rows after part 0; lane m of the product loads W^T row
# sigma(m), sigma swapping bits 2 and 3; 16-byte stores of 8 consecutive
# indices; 8-element runs read back as five 4-byte words shifted by the row
# start's parity.)
FUSED_ROW, FUSED_PART1, SLICE = 105, 16, 2048


def _sigma(m):
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1)


def fused_stage_model(alias):
    """Simulate one band tile's stage writes and reads for the 64 lanes of a
    wave. Returns (per part: element -> every (query, idx) written there,
    the runs each lane reads, the store addresses)."""
    parts = [dict(), dict()]
    stores = []
    for lane in range(64):
        col, half = lane & 31, lane >> 5
        hi = col >> 4
        frow = (col & 15) if alias else col
        part = hi if alias else 0
        fw_off = 32 + (FUSED_ROW - 1) * frow + ((FUSED_PART1 - 16) * hi if alias else 0) + 8 * half
        for b in range(3):
            for k in range(2):
                base = fw_off + 32 * b + 16 * k
                stores.append((part, base))
                for x in range(8):
                    # register 8k + x of block b: output row m = 8i + 4*half + j,
                    # which the lane loaded from W^T row sigma(m)
                    i, j = 2 * k + x // 4, x % 4
                    idx = 32 * b + _sigma(8 * i + 4 * half + j)
                    parts[part].setdefault(base + x, []).append((col, idx))
    reads = {}
    for lane in range(64):
        col, half = lane & 31, lane >> 5
        hi = col >> 4
        frow = (col & 15) if alias else col
        part = hi if alias else 0
        fr_off = 32 + FUSED_ROW * frow + (FUSED_PART1 * hi if alias else 0)
        for p in range(4):
            word = fr_off // 2 + (7 - half - 2 * p) * 4
            shift = fr_off & 1                      # elements shifted out
            elems = [2 * word + shift + x for x in range(8)]
            reads[(lane, p)] = (part, elems, [parts[part].get(e, []) for e in elems])
    return parts, reads, stores


@pytest.mark.parametrize("alias", [True, False])
def test_fused_stage_layout(alias):
    parts, reads, stores = fused_stage_model(alias)
    limit = SLICE if alias else 32 + 32 * FUSED_ROW
    for part, base in stores:
        assert base % 8 == 0                        # 16-byte aligned stores
        assert 0 <= base and base + 8 <= limit
    for (lane, p), (part, elems, got) in reads.items():
        col, half = lane & 31, lane >> 5
        assert 0 <= min(elems) and max(elems) // 2 * 2 + 2 <= limit   # five words inside
        # run p holds distance indices e = 63 - 8*half - 16p - 7 .. - 0 of the
        # lane's query row, i.e. product index idx = e + q (ascending)
        e0 = (7 - half - 2 * p) * 8
        # exactly one lane writes each element read, with the right value
        assert got == [[(col, e0 + x + col)] for x in range(8)], (lane, p)


def test_fused_stage_model_catches_a_wrong_row_order():
    # without the bit swap the product rows' order no longer matches the
    # 16-byte stores: the reads then return other indices
    global _sigma
    keep = _sigma
    _sigma = lambda m: m
    try:
        with pytest.raises(AssertionError):
            test_fused_stage_layout(True)
    finally:
        _sigma = keep
