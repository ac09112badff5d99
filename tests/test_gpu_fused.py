"""GPU parity of trellis_gemv_fused (layers that share one input vector, one launch, the work split
evenly over the workgroups) against the oracle, through the C ABI."""
import numpy as np
import pytest

from gpu_common import REL_TOL, device, full_size_case, rel_err, say
from oracle import gemv as ogemv
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu


def _run(arrays, x_bits, dev, flags=0, splits=0, ws=None):
    import torch
    layers = [tg.DeviceLayer(a, dev, flags=flags, splits=splits) for a in arrays]
    ys = tg.trellis_gemv_fused(layers, tg.fp16_tensor(x_bits, dev), ws=ws)
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


@pytest.mark.parametrize("code_id,flags", [(0, 0), (1, 0), (0, tg.TG_FLAG_ROUND_WEIGHTS), (1, tg.TG_FLAG_ROUND_WEIGHTS)])
@pytest.mark.parametrize("splits", [0, 7, 37, 160])
def test_fused_small_layers_every_output(code_id, flags, splits):
    """Three layers of different heights on one input; forced workgroup counts give runs that
    start and end inside blocks and cross layers (up to a dozen contributors per block)."""
    dev = device()
    n = 1024
    arrays = [inputs.make_layer(m, n, 3, 5000 + m, code_id=code_id) for m in (512, 128, 256)]
    x = inputs.make_x(n, 5001)
    say("fused small", code_id, flags, splits)
    ys = _run(arrays, x, dev, flags, splits)
    for a, y in zip(arrays, ys):
        assert rel_err(y, ogemv.gemv(a, x)) <= REL_TOL


@pytest.mark.parametrize("n,k", [(128, 1), (384, 2), (1152, 5), (16384, 2)])
def test_fused_odd_block_counts_and_widths(n, k):
    """n/128 odd (a half step closes each block row), a single block, and the widest input (two
    transform passes)."""
    dev = device()
    arrays = [inputs.make_layer(256, n, k, 5100 + n), inputs.make_layer(128, n, k, 5101 + n)]
    x = inputs.make_x(n, 5102 + n)
    say("fused widths", n, k)
    ys = _run(arrays, x, dev, splits=13)
    for a, y in zip(arrays, ys):
        assert rel_err(y, ogemv.gemv(a, x)) <= REL_TOL


def test_fused_one_layer_equals_gemv_and_repeats():
    """One layer through the fused launch against trellis_gemv; two calls on one workspace give the same
    bits, and the ticket counters end each call on a call boundary."""
    dev = device()
    import torch
    arr = inputs.make_layer(1024, 4096, 2, 5200)
    x = inputs.make_x(4096, 5200)
    L = tg.DeviceLayer(arr, dev)
    ws = tg.fused_workspace([L], dev)
    say("fused one layer")
    xt = tg.fp16_tensor(x, dev)
    y1 = tg.trellis_gemv_fused([L], xt, ws=ws)[0].clone()
    y2 = tg.trellis_gemv_fused([L], xt, ws=ws)[0].clone()
    ref = tg.trellis_gemv(L, xt)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert rel_err(y1.cpu().numpy(), ref.cpu().numpy()) <= 2e-4
    tickets = ws[256: 256 + 8 * 4].view(torch.int32)
    assert ((tickets & 0xFFFF) == 0).all()
    assert tg.workspace_status(ws) == 0


@pytest.mark.parametrize("group,code_id", [(("q", "k", "v"), 0), (("gate", "up"), 0), (("q", "k", "v"), 1)])
def test_fused_decoder_layer_full_size(group, code_id):
    """The 70B-shaped layer's fused launches in the bench's configuration; two outputs of every
    128-output block of every layer against stored oracle outputs."""
    dev = device()
    cases = [full_size_case(f"w3f_{name}_c{code_id}") for name in group]
    x = cases[0][1]
    assert all(np.array_equal(c[1], x) for c in cases)        # one shared input vector
    say("fused full size", group, code_id)
    ys = _run([c[0] for c in cases], x, dev)
    for name, c, y in zip(group, cases, ys):
        assert np.isfinite(y).all()
        assert rel_err(y[c[2]], c[4][0]) <= REL_TOL, name
