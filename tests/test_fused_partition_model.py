"""A CPU model of the fused launch's partition (trellis_gemv_fused): layers' units (one 16-tile step
of one 128-output block) in layer, block, step order; workgroup w takes [w*upw, (w+1)*upw). The
model replays the host's choice of upw and the kernel's segment and contributor arithmetic, and
checks that every unit is decoded exactly once, that a run crosses at most one layer boundary (the
kernel keeps two layers' inputs in LDS), that each block's contributor indices are 0..count-1
with count <= the workspace's max_contrib, and that exactly one contributor finishes each block."""
import numpy as np


def lds_bytes(n, int8=False):
    """The fused kernel's dynamic LDS: two layers' x~ areas, the output buffer, flags (+ int8 side arrays)."""
    nbp = ((n // 128) + 1) & ~1
    return 2 * nbp * 128 * 4 + 128 * 4 + 16 + (2 * nbp * 9 * 4 if int8 else 0)


def default_target(total, n, int8=False):
    """The host's default workgroup count: two per compute unit where each still gets at least 16
    units and two workgroups fit 160 KB of LDS, else one."""
    return 512 if total >= 512 * 16 and 2 * lds_bytes(n, int8) <= 160 * 1024 else 256


def geometry(ms, n, target=None):
    nb = n // 128
    spr = (nb + 1) // 2
    units = [(m // 128) * spr for m in ms]
    unit0 = np.concatenate([[0], np.cumsum(units)[:-1]]).astype(int)
    total = sum(units)
    if target is None:
        target = default_target(total, n)
    upw = max(1, min(-(-total // target), min(units)))
    grid = -(-total // upw)
    maxc = 1
    for l, m in enumerate(ms):
        for ob in range(m // 128):
            b0 = unit0[l] + ob * spr
            maxc = max(maxc, (b0 + spr - 1) // upw - b0 // upw + 1)
    return spr, unit0, total, upw, grid, maxc


def replay(ms, n, target=None):
    spr, unit0, total, upw, grid, maxc = geometry(ms, n, target)
    covered = np.zeros(total, int)
    contributors = {}
    for w in range(grid):
        u0, u1 = w * upw, min((w + 1) * upw, total)
        layers = {int(np.searchsorted(unit0, u, side="right") - 1) for u in range(u0, u1)}
        assert len(layers) <= 2 and max(layers) - min(layers) <= 1, (w, layers)
        u = u0
        while u < u1:
            l = int(np.searchsorted(unit0, u, side="right") - 1)
            ob = (u - unit0[l]) // spr
            seg_u0 = unit0[l] + ob * spr
            seg_end = min(seg_u0 + spr, u1)
            covered[u:seg_end] += 1
            first, last = seg_u0 // upw, (seg_u0 + spr - 1) // upw
            count = last - first + 1
            assert count <= maxc
            contributors.setdefault((l, ob), []).append((w - first, count))
            u = seg_end
    assert (covered == 1).all()
    for key, lst in contributors.items():
        counts = {c for _, c in lst}
        assert len(counts) == 1 and sorted(i for i, _ in lst) == list(range(counts.pop())), key
    return upw, grid, maxc


def test_decoder_layer_groups():
    assert replay([8192, 1024, 1024], 8192) == (10, 256, 4)      # q/k/v: 2560 units, 10 per workgroup
    assert replay([28672, 28672], 8192) == (28, 512, 2)          # gate/up: 14336 units, 28 per workgroup
    assert default_target(14336, 16384) == 256                   # 16384 inputs: one workgroup's x~ fills the LDS
    assert default_target(14336, 8192, int8=True) == 512


def test_random_tables_and_forced_counts():
    rng = np.random.default_rng(3)
    for _ in range(200):
        n = 128 * int(rng.integers(1, 129))
        ms = [128 * int(rng.integers(1, 65)) for _ in range(int(rng.integers(1, 9)))]
        replay(ms, n, target=int(rng.integers(1, 700)))


def issue_replay(ms, n, K, target=None, pf=2):
    """The fused kernel's code prefetch, replayed: the issue position (output block, step) advances
    by one unit per issue with a block wrap and one switch of code pointer where the run enters its
    second layer, and every issue inside the run must address the code words the unit's own
    (layer, block, step) names, for every tile row (wave) of the block."""
    spr, unit0, total, upw, grid, _ = geometry(ms, n, target)
    n16 = n // 16
    step_words = 16 * 8 * K
    layer_of = lambda u: int(np.searchsorted(unit0, u, side="right") - 1)
    for w in range(grid):
        u0, u1 = w * upw, min((w + 1) * upw, total)
        lay0, lay1 = layer_of(u0), layer_of(u1 - 1)
        for wave in range(8):
            inext = unit0[lay1] if lay1 != lay0 else 1 << 62
            iu, icodes = u0, lay0
            rel = u0 - unit0[lay0]
            iob, ist = rel // spr, rel % spr
            ibase = ((iob * 8 + wave) * n16 + ist * 16) * (8 * K)
            for _ in range(u1 - u0 + pf):
                if iu < u1:
                    l = layer_of(iu)
                    r = iu - unit0[l]
                    want = (l, ((r // spr * 8 + wave) * n16 + (r % spr) * 16) * (8 * K))
                    assert (icodes, ibase) == want, (ms, n, K, w, wave, iu)
                    assert ist == r % spr                     # the ragged-step test uses ist
                iu += 1
                ibase += step_words
                ist += 1
                if ist == spr:
                    ist = 0
                    iob += 1
                    if iu == inext:
                        iob, icodes, inext = 0, lay1, 1 << 62
                    ibase = (iob * 8 + wave) * n16 * (8 * K)


def test_prefetch_position_replay():
    issue_replay([8192, 1024, 1024], 8192, 2)
    issue_replay([28672, 28672], 8192, 2)
    rng = np.random.default_rng(5)
    for _ in range(60):
        n = 128 * int(rng.integers(1, 40))
        ms = [128 * int(rng.integers(1, 12)) for _ in range(int(rng.integers(1, 5)))]
        issue_replay(ms, n, int(rng.integers(1, 9)), target=int(rng.integers(1, 300)))


def needed_blocks_replay(ms, n, target=None):
    """The fused kernel transforms only the input blocks its run reads: in its first layer the
    nn0 blocks from 2 * (first unit's step) on, in the second the nn1 blocks from 0 on (modulo
    the padded block count). Every block a unit of the run reads (two per step) must be among
    them."""
    spr, unit0, total, upw, grid, _ = geometry(ms, n, target)
    nbp = 2 * spr
    layer_of = lambda u: int(np.searchsorted(unit0, u, side="right") - 1)
    for w in range(grid):
        u0, u1 = w * upw, min((w + 1) * upw, total)
        lay0, lay1 = layer_of(u0), layer_of(u1 - 1)
        end0 = unit0[lay1] if lay1 != lay0 else u1
        step0 = (u0 - unit0[lay0]) % spr
        nn0 = min(nbp, 2 * (end0 - u0))
        nn1 = min(nbp, 2 * (u1 - unit0[lay1]))
        done = {lay0: {(2 * step0 + i) % nbp for i in range(nn0)}}
        if lay1 != lay0:
            done[lay1] = {i % nbp for i in range(nn1)}
        for u in range(u0, u1):
            l = layer_of(u)
            s = (u - unit0[l]) % spr
            assert {2 * s, 2 * s + 1} <= done[l], (ms, n, w, u)


def test_needed_input_blocks():
    needed_blocks_replay([8192, 1024, 1024], 8192)
    needed_blocks_replay([28672, 28672], 8192)
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = 128 * int(rng.integers(1, 129))
        ms = [128 * int(rng.integers(1, 65)) for _ in range(int(rng.integers(1, 9)))]
        needed_blocks_replay(ms, n, target=int(rng.integers(1, 700)))
