"""GPU parity: decoded fp16 weights and the code table, bit-exact against the oracle."""
import numpy as np
import pytest

from gpu_common import device, say
from oracle import code as ocode
from oracle import gemv as ogemv
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu


def test_code_table_bit_exact():
    dev = device()
    say("code table")
    t = tg.code_table(dev).cpu().numpy().view(np.uint16)
    assert np.array_equal(t, ocode.table())


@pytest.mark.parametrize("k", range(1, 9))
@pytest.mark.parametrize("m,n", [(16, 16), (48, 32), (128, 384), (256, 128)])
def test_decode_small_bit_exact(k, m, n):
    dev = device()
    arr = inputs.make_layer(m, n, k, 1000 + k, tensor=m + n)
    L = tg.DeviceLayer(arr, dev)
    say("decode", m, n, k)
    w = tg.trellis_decode(L).cpu().numpy().view(np.uint16)
    assert np.array_equal(w, ogemv.decode_layer(arr))


@pytest.mark.parametrize("cfg,tensor", [(1, "linear"), (2, "down"), (3, "k"), (3, "gate"), (4, "gate")])
def test_decode_config_tensors(cfg, tensor):
    """Workload tensors at full size: the GPU decodes everything, the oracle re-decodes sampled tile rows."""
    dev = device()
    wl = inputs.WORKLOADS[cfg]
    m, n, k = wl.tensors[tensor]
    idx = list(wl.tensors).index(tensor)
    arr = inputs.make_layer(m, n, k, wl.seed, tensor=idx)
    L = tg.DeviceLayer(arr, dev)
    say("decode config", cfg, tensor, m, n, k)
    w = tg.trellis_decode(L).cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(cfg)
    trows = sorted({0, m // 16 - 1, int(rng.integers(0, m // 16))}) if m > 256 else list(range(m // 16))
    ref = ogemv.decode_layer(arr, trows)
    got = np.concatenate([w[16 * r:16 * r + 16] for r in trows])
    assert np.array_equal(got, ref)


def test_decode_moe_experts():
    dev = device()
    wl = inputs.CFG5
    for e in (0, 77, 127):
        for which in ("gate", "up", "down"):
            arr = wl.layer(e, which)
            say("decode moe", e, which, arr.k_bits)
            w = tg.trellis_decode(tg.DeviceLayer(arr, dev)).cpu().numpy().view(np.uint16)
            assert np.array_equal(w[:64], ogemv.decode_layer(arr, [0, 1, 2, 3]))
