"""A CPU model of the grouped launch's split choice and each workgroup's input and code loads.

The host picks one split count S for the whole launch from the widest layer of the table
(the grid is selections x largest block count x S). Each workgroup then runs its selected
layer with min(S, that layer's 128-block count) input chunks and leaves if its split index
is past them, so no chunk is ever empty. The model replays the host's choice of S and the
kernel's chunk bounds over random tables that mix shapes, and checks that every input,
sign-word, gated-input and code-word index a workgroup loads lies inside its layer's arrays.
It also checks that running every layer with the launch's S (the earlier rule) would load
outside them for the tables where that went wrong, so the test is not vacuous."""
import numpy as np

KBLOCK = 128
MAX_CHUNK_BLOCKS = 64
WAVES = 8


def split_for_target(nb, target):
    steps = nb // 2
    if steps < 1:
        return 1
    best = 1
    for s in range(1, steps + 1):
        if steps % s:
            continue
        d, bd = abs(s - target), abs(best - target)
        if d < bd or (d == bd and s > best):
            best = s
    return best


def grouped_splits(layers, n_sel):
    """The host's split count (grouped_geometry in api.hip, no override)."""
    max_ob = max(m for m, n, k in layers) // KBLOCK
    max_nb = max(n for m, n, k in layers) // KBLOCK
    per = n_sel * max_ob
    s = split_for_target(max_nb, 1 if per >= 256 else 256 // per)
    while s > 1 and s * per > 256:
        s -= 1
    s = max(s, -(-max_nb // MAX_CHUNK_BLOCKS))
    return max(1, min(s, max_nb))


def workgroup_loads(layer, ob, split, S, per_layer_splits=True):
    """Index ranges one workgroup loads, or None if it leaves at once.

    Returns (x_lo, x_hi, sign_words, code_lo, code_hi) over all its lanes."""
    m, n, k = layer
    if ob >= m // KBLOCK:
        return None
    nb = n // KBLOCK
    s_l = min(S, nb) if per_layer_splits else S
    if split >= s_l:
        return None
    blk0, blk1 = split * nb // s_l, (split + 1) * nb // s_l
    cb = blk1 - blk0
    ntiles, nsteps = cb * 8, (cb + 1) // 2
    xlo, xhi, sw = 1 << 62, -(1 << 62), set()
    for wave in range(WAVES):
        for lane in range(64):
            xb, xs = 8 * wave + (lane >> 3), lane & 7
            first = (blk0 + (xb if xb < cb else cb - 1)) * KBLOCK + 16 * xs
            xlo, xhi = min(xlo, first), max(xhi, first + 15)
            sw.add(first >> 5)
    n16, wpt = n // 16, 8 * k
    rw, lane, st = np.meshgrid(np.arange(8), np.arange(64), np.arange(nsteps), indexing="ij")
    valid = st * 16 + (lane >> 2) < ntiles           # the kernel loads a dummy line otherwise
    tile = (ob * 8 + rw) * n16 + blk0 * 8 + st * 16 + (lane >> 2)
    word = (tile * wpt + (lane % 4) * 2 * k)[valid]
    if word.size == 0:                               # an empty chunk loads only the dummy line
        return xlo, xhi, sw, 0, 0
    return xlo, xhi, sw, int(word.min()), int(word.max()) + 2 * k - 1


def check_table(layers, n_sel, rng, per_layer_splits=True):
    """True iff every load of every working workgroup stays inside its layer."""
    S = grouped_splits(layers, n_sel)
    max_ob = max(m for m, n, k in layers) // KBLOCK
    sel = rng.integers(0, len(layers), size=n_sel)
    for e in range(n_sel):
        layer = layers[int(sel[e])]
        m, n, k = layer
        for ob in range(max_ob):
            for split in range(S):
                r = workgroup_loads(layer, ob, split, S, per_layer_splits)
                if r is None:
                    continue
                xlo, xhi, sw, clo, chi = r
                if xlo < 0 or xhi >= n or min(sw) < 0 or max(sw) >= (n + 31) // 32:
                    return False
                if clo < 0 or chi >= (m // 16) * (n // 16) * 8 * k:
                    return False
    return True


def test_mixed_tables_in_bounds():
    rng = np.random.default_rng(11)
    for _ in range(60):
        nl = int(rng.integers(1, 5))
        layers = [(128 * int(rng.integers(1, 17)), 128 * int(rng.integers(1, 97)), int(rng.integers(1, 9)))
                  for _ in range(nl)]
        n_sel = int(rng.integers(1, 9))
        assert check_table(layers, n_sel, rng), (layers, n_sel)


def test_expert_tables_in_bounds():
    rng = np.random.default_rng(12)
    for layers in ([(768, 2048, 2), (2048, 768, 3)], [(128, 128, 1), (128, 8192, 2)],
                   [(1024, 8192, 2), (8192, 8192, 2)]):
        for n_sel in (1, 2, 8):
            assert check_table(layers, n_sel, rng), (layers, n_sel)


def test_launch_wide_split_count_would_read_outside():
    """Running every layer with the launch's S leaves empty chunks whose loads start at
    index -128 (the tables found by the review)."""
    rng = np.random.default_rng(13)
    assert grouped_splits([(768, 2048, 2), (2048, 768, 2)], 2) == 8
    r = workgroup_loads((2048, 768, 2), 0, 0, 8, per_layer_splits=False)   # down: 6 blocks, 8 splits
    assert r is not None and r[0] == -128
    assert workgroup_loads((2048, 768, 2), 0, 0, 8)[0] == 0
    assert check_table([(768, 2048, 2), (2048, 768, 2)], 2, rng)
    assert grouped_splits([(128, 128, 1), (128, 8192, 2)], 1) == 32
    r = workgroup_loads((128, 128, 1), 0, 1, 32, per_layer_splits=False)
    assert r is not None and r[0] < 0
    assert workgroup_loads((128, 128, 1), 0, 1, 32) is None
    assert check_table([(128, 128, 1), (128, 8192, 2)], 1, rng)
