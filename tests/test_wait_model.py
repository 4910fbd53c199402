"""CPU model of the vector-memory queue of one wave of the persistent dgrad
kernel (`dgrad_igemm` in convolution_backward_amd/csrc/dgrad_kernels.hip).

The kernel's slice loads are direct-to-LDS buffer loads written as inline
assembly, so the compiler does not wait for them: before computing a slice,
each wave waits with a fixed `s_waitcnt vmcnt(N)`. A wave's vector-memory
operations retire in issue order, so vmcnt(N) guarantees that every operation
except the last N issued has completed. The kernel is correct only if, at
every such wait, all loads of the slice about to be computed are older than
the last N operations.

This model replays the kernel's issue order for one wave (two slice requests
ahead of the matrix cores; zero stripes riding with each request; an
epilogue of z loads and dx stores, with companion zero stores, after each
tile's last slice; standalone zero chunks at the end) over many tile-length
sequences and checks each wait the kernel performs:
  * safety: the slice's loads are complete when the wait returns;
  * tightness: allowing one more operation would release some slice early
    in some sequence, i.e. the fixed counts are the largest safe ones for the
    cases they cover (except where the kernel is stricter on purpose).
Stream-K launches are not modelled: a share that leaves partial sums drains
its queue with vmcnt(0), and a completing share's partial-sum loads are
waited for by the compiler before the epilogue, so both only make the next
waits stricter.
"""
import itertools

import pytest

K_MAX_ZERO_PER_SLICE = 4          # dgrad_internal.h: zero stores per slice request
K_ZERO_CHUNK_STRIPES = 8          # dgrad_internal.h: stores per standalone zero chunk
CONFIGS = [(128, 128, 2, 2), (256, 64, 4, 1), (128, 64, 2, 2), (64, 64, 2, 2), (256, 128, 4, 2), (128, 256, 2, 4)]
BK = 64


def constants(BM, BN, WM, WN):
    """The kernel's per-wave operation counts for one tile configuration."""
    NW = WM * WN
    a_instr = BM * 2 * BK // 1024 // NW
    b_instr = BK * BN * 2 // 1024 // NW
    LD = a_instr + b_instr
    TM, TN = BM // WM, BN // WN
    FM, FN = TM // 32, TN // 32
    CH = TN // 8
    EST = 32 // (64 // CH)
    return {"LD": LD, "EPI_STORES": FM * EST, "Z_LOADS": FM * FN * 4}


def wait_count(k, inflight, post_epi, zw_active):
    """The kernel's wait at the top of a slice (the branch structure of the
    slice loop): LD loads of the next request, both requests' zero stores in
    zero-work launches, and the last epilogue's stores in the two slices after it."""
    if inflight >= 2:
        n = k["LD"]
        if zw_active:
            n += 2 * K_MAX_ZERO_PER_SLICE
        if post_epi > 0:
            n += k["EPI_STORES"]
        return n
    return 0


def replay(k, tiles, zps, ncomp, fused, chunks, slack=0):
    """Issue order of one wave over its GEMM tiles (slice counts in `tiles`),
    then `chunks` standalone zero chunks. Returns a list of (required, n):
    at each wait, the number of operations issued after the computed slice's
    last load (`required` must be >= n for safety) and the count n used,
    plus `slack` extra (to probe tightness)."""
    queue = []                          # tags of issued operations, oldest first
    stream = [t for t, n in enumerate(tiles) for _ in range(n)]   # tile of each slice
    last_load = {}                      # slice index -> queue position of its last load
    nxt = 0                             # next slice to request

    def request():
        nonlocal nxt
        if nxt >= len(stream):
            return False
        queue.extend(["load"] * k["LD"])
        last_load[nxt] = len(queue) - 1
        queue.extend(["zero"] * zps)
        nxt += 1
        return True

    inflight = 0
    post_epi = 0
    if request():
        inflight += 1
    if request():
        inflight += 1
    checks = []
    for s, tile in enumerate(stream):
        n = wait_count(k, inflight, post_epi, zps != 0) + slack
        after = len(queue) - 1 - last_load[s]   # operations issued after the slice's last load
        checks.append((after, n))
        post_epi = max(post_epi - 1, 0)
        # barrier, then compute with the next request's loads issued in parts
        if not request():
            inflight -= 1
        if s + 1 == len(stream) or stream[s + 1] != tile:     # the tile's last slice: epilogue
            if fused:
                queue.extend(["zload"] * k["Z_LOADS"])
            queue.extend(["store"] * (k["EPI_STORES"] * (1 + ncomp)))
            post_epi = 2
    for _ in range(chunks):
        queue.extend(["zero"] * K_ZERO_CHUNK_STRIPES)
    return checks


def tile_sequences():
    """Every sequence of up to four tiles of 1-4 slices, plus longer tiles."""
    seqs = []
    for ntiles in range(1, 5):
        seqs.extend(itertools.product(range(1, 5), repeat=ntiles))
    seqs.extend([(8,), (9, 9, 9), (72, 72), (2, 4, 4, 8), (18, 1, 18)])
    return seqs


CASES = [  # (zps, ncomp, fused): plain, companion, zero-work, fused epilogue
    (0, 0, False), (0, 3, False), (0, 0, True), (K_MAX_ZERO_PER_SLICE, 0, False), (K_MAX_ZERO_PER_SLICE, 0, True),
]


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: "%dx%d_%dx%d" % c)
def test_waits_never_release_a_slice_early(cfg):
    k = constants(*cfg)
    assert k["LD"] + 2 * K_MAX_ZERO_PER_SLICE + k["EPI_STORES"] < 64, "vmcnt holds at most 63"
    for zps, ncomp, fused in CASES:
        for seq in tile_sequences():
            for after, n in replay(k, seq, zps, ncomp, fused, chunks=2):
                assert after >= n, (cfg, zps, ncomp, fused, seq, after, n)


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: "%dx%d_%dx%d" % c)
def test_wait_counts_are_tight(cfg):
    """For each branch of the wait (steady state; after an epilogue; with zero
    stripes), some sequence has exactly as many operations after the slice as
    the count allows, so one more would release the slice early."""
    k = constants(*cfg)
    tight = set()
    for zps, ncomp, fused in [(0, 0, False), (K_MAX_ZERO_PER_SLICE, 0, False)]:
        for seq in tile_sequences():
            checks = replay(k, seq, zps, ncomp, fused, chunks=0)
            stream_len = sum(seq)
            for s, (after, n) in enumerate(checks):
                if after == n and n > 0:
                    branch = (zps != 0, n > k["LD"] + (2 * K_MAX_ZERO_PER_SLICE if zps else 0))
                    tight.add(branch)
            assert len(checks) == stream_len
    assert tight == {(False, False), (False, True), (True, False), (True, True)}, tight


def test_one_slice_too_long_fails():
    """A wait that allowed one more slice request (LD more operations) would
    release a slice before its loads land: the model catches it."""
    k = constants(256, 128, 4, 2)
    bad = [after < n for seq in tile_sequences() for after, n in replay(k, seq, 0, 0, False, 0, slack=k["LD"])]
    assert any(bad)
