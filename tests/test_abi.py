"""C-ABI checks that need no GPU: the library loads, exports what the header declares, and rejects bad
arguments on the host before anything is enqueued (so these calls never reach the device)."""
import ctypes
import os
import re

import pytest

from trellis_coded_gemv_amd import binding as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "trellis_gemv.h")

# fake device addresses: never dereferenced, every call below fails validation first
A16 = 0x10000
A4 = 0x20004


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def _layer(**kw):
    d = dict(m=256, n=512, k_bits=2, code_id=0, flags=0, splits=0, codes=A16, scales=A16, sign_in=A16,
             sign_out=A16)
    d.update(kw)
    return tg.TgLayer(**d)


def test_library_loads_and_exports_every_declared_symbol():
    L = tg.lib()
    declared = _declared_functions()
    assert set(declared) == set(tg.EXPORTS), declared
    for name in declared:
        assert hasattr(L, name), name
    assert L.tg_abi_version() == 4
    from trellis_coded_gemv_amd.build import source_hash
    assert L.tg_build_id().decode() == source_hash()


def test_struct_layout_matches_header():
    assert ctypes.sizeof(tg.TgLayer) == 56
    assert tg.TgLayer.codes.offset == 24 and tg.TgLayer.sign_out.offset == 48


def test_status_strings():
    L = tg.lib()
    for code in range(-8, 1):
        assert L.tg_status_str(code).decode().startswith(tg.STATUS[code])
    assert L.tg_status_str(-99) == b"unknown tg_status"


@pytest.mark.parametrize("kw,status", [
    (dict(k_bits=0), -3), (dict(k_bits=9), -3), (dict(m=100), -2), (dict(n=0), -2), (dict(m=-128), -2),
    (dict(code_id=4), -6), (dict(code_id=-1), -6), (dict(flags=4), -8), (dict(flags=2), -8), (dict(splits=-1), -8), (dict(splits=65536), -8), (dict(codes=0), -1),
    (dict(sign_out=0), -1), (dict(codes=A16 + 8), -4), (dict(scales=A16 + 1), -4), (dict(sign_in=A4 + 2), -4)])
def test_gemv_layer_validation(kw, status):
    d = _layer(**kw)
    assert tg.lib().trellis_gemv(ctypes.byref(d), A16, A16, A16, 1 << 30, None) == status


def test_gemv_argument_validation():
    L = tg.lib()
    d = _layer()
    assert L.trellis_gemv(None, A16, A16, A16, 1 << 30, None) == -1
    assert L.trellis_gemv(ctypes.byref(d), 0, A16, A16, 1 << 30, None) == -1
    assert L.trellis_gemv(ctypes.byref(d), A16, A16 + 2, A16, 1 << 30, None) == -4
    need = L.tg_workspace_size(ctypes.byref(d), 1)
    assert need > 0
    assert L.trellis_gemv(ctypes.byref(d), A16, A16, 0, need, None) == -5
    assert L.trellis_gemv(ctypes.byref(d), A16, A16, A16, 255, None) == -5
    assert L.trellis_gemv(ctypes.byref(d), A16, A16, A16 + 16, need, None) == -4


def test_workspace_size_queries():
    L = tg.lib()
    d = _layer()
    assert L.tg_workspace_size(None, 1) == 0
    assert L.tg_workspace_size(ctypes.byref(d), 0) == 0
    assert L.tg_workspace_size(ctypes.byref(d), 65) == 0
    assert L.tg_workspace_size(ctypes.byref(_layer(k_bits=9)), 1) == 0
    for M in (1, 2, 16, 17, 64):
        assert L.tg_workspace_size(ctypes.byref(d), M) % 256 == 0


def test_gemm_small_validation():
    L = tg.lib()
    d = _layer()
    ws = 1 << 34
    assert L.trellis_gemm_small(ctypes.byref(d), 0, A16, 512, A16, 256, A16, ws, None) == -2
    assert L.trellis_gemm_small(ctypes.byref(d), 65, A16, 512, A16, 256, A16, ws, None) == -2
    assert L.trellis_gemm_small(ctypes.byref(d), 4, A16, 511, A16, 256, A16, ws, None) == -8
    assert L.trellis_gemm_small(ctypes.byref(d), 4, A16, 512, A16, 255, A16, ws, None) == -8
    assert L.trellis_gemm_small(ctypes.byref(d), 4, 0, 512, A16, 256, A16, ws, None) == -1
    assert L.trellis_gemm_small(ctypes.byref(d), 4, A16, 512, A16, 256, A16, 16, None) == -5


def test_rht_validation():
    L = tg.lib()
    assert L.rht_apply(100, 1, A16, A16, A16, 0, None) == -2
    assert L.rht_apply(128, 0, A16, A16, A16, 0, None) == -2
    assert L.rht_apply(128, 70000, A16, A16, A16, 0, None) == -2
    assert L.rht_apply(128, 1, 0, A16, A16, 0, None) == -1
    assert L.rht_apply(128, 1, A16, A16 + 2, A16, 0, None) == -4


def test_decode_and_table_validation():
    L = tg.lib()
    assert L.trellis_decode(None, A16, None) == -1
    assert L.trellis_decode(ctypes.byref(_layer(m=24)), A16, None) == -2
    assert L.trellis_decode(ctypes.byref(_layer(k_bits=0)), A16, None) == -3
    assert L.trellis_decode(ctypes.byref(_layer()), 0, None) == -1
    assert L.tg_code_table(4, A16, None) == -6
    assert L.tg_code_table(0, 0, None) == -1


def test_grouped_validation():
    L = tg.lib()
    arr = (tg.TgLayer * 2)(_layer(), _layer(m=128, k_bits=3))
    assert L.tg_grouped_workspace_size(arr, 2, 4) > 0
    assert L.tg_grouped_workspace_size(arr, 0, 4) == 0
    bad = (tg.TgLayer * 2)(_layer(), _layer(k_bits=11))
    ws = 1 << 34
    assert L.trellis_gemv_grouped(bad, A16, 2, A16, 4, A16, 0, A16, 256, A16, ws, None) == -3
    mixed = (tg.TgLayer * 2)(_layer(), _layer(flags=1))
    assert L.trellis_gemv_grouped(mixed, A16, 2, A16, 4, A16, 0, A16, 256, A16, ws, None) == -8
    assert L.trellis_gemv_grouped(arr, 0, 2, A16, 4, A16, 0, A16, 256, A16, ws, None) == -1
    assert L.trellis_gemv_grouped(arr, A16, 2, A16, 4, A16, 100, A16, 256, A16, ws, None) == -8
    assert L.trellis_gemv_grouped(arr, A16, 2, A16, 4, A16, 0, A16, 255, A16, ws, None) == -8
    assert L.trellis_gemv_grouped(arr, A16, 2, A16, 4, A16, 0, A16, 256, A16, 64, None) == -5


def test_pair_code_passes_layer_validation():
    """code_id 1 is accepted: the call gets past the layer checks and stops at the missing workspace."""
    L = tg.lib()
    d = _layer(code_id=1)
    assert L.tg_workspace_size(ctypes.byref(d), 1) > 0
    assert L.trellis_gemv(ctypes.byref(d), A16, A16, 0, 1 << 30, None) == -5
    assert L.trellis_gemm_small(ctypes.byref(d), 16, A16, 512, A16, 256, 0, 1 << 30, None) == -5
    assert L.tg_code_table(1, 0, None) == -1
    assert L.trellis_decode(ctypes.byref(d), 0, None) == -1


def test_encode_argument_validation():
    L = tg.lib()
    assert L.tg_encode_workspace_size(4, 2, 0) > 0
    assert L.tg_encode_workspace_size(0, 2, 0) == 0
    assert L.tg_encode_workspace_size(4, 9, 0) == 0
    assert L.tg_encode_workspace_size(4, 5, 1) == 0           # pair code: at most 4 bits (8 per step)
    assert L.tg_encode_workspace_size(4, 2, 4) == 0
    assert L.tg_encode_workspace_size(4, 8, 2) > 0            # mul1: one state per weight, like code 0
    need = L.tg_encode_workspace_size(4, 2, 0)
    assert L.trellis_encode(4, 2, 0, 0.75, A16, A16, A16, 0, need, None) == -5
    assert L.trellis_encode(4, 2, 0, 0.75, 0, A16, A16, A16, need, None) == -1
    assert L.trellis_encode(4, 2, 0, -1.0, A16, A16, A16, A16, need, None) == -8
    assert L.trellis_encode(4, 2, 0, float("nan"), A16, A16, A16, A16, need, None) == -8
    assert L.trellis_encode(4, 0, 0, 0.75, A16, A16, A16, A16, need, None) == -3
    assert L.trellis_encode(4, 2, 4, 0.75, A16, A16, A16, A16, need, None) == -6
    assert L.trellis_encode(0, 2, 0, 0.75, A16, A16, A16, A16, need, None) == -2
    assert L.trellis_encode(4, 2, 0, 0.75, A16 + 2, A16, A16, A16, need, None) == -4
    assert L.trellis_encode(4, 2, 0, 0.75, A16, A16, A16, A16 + 16, need, None) == -4


def test_prefill_argument_validation():
    L = tg.lib()
    d = _layer()
    need = L.tg_prefill_workspace_size(ctypes.byref(d), 100)
    assert need == 100 * 512 * 2           # the transformed input rows only: the weights are never stored
    assert L.tg_prefill_workspace_size(ctypes.byref(d), 0) == 0
    assert L.tg_prefill_workspace_size(ctypes.byref(d), 65536) == 0
    assert L.trellis_gemm_prefill(ctypes.byref(d), 100, A16, 512, A16, 256, 0, need, None) == -5
    assert L.trellis_gemm_prefill(ctypes.byref(d), 100, A16, 511, A16, 256, A16, need, None) == -8
    assert L.trellis_gemm_prefill(ctypes.byref(d), 0, A16, 512, A16, 256, A16, need, None) == -2
    assert L.trellis_gemm_prefill(ctypes.byref(d), 100, 0, 512, A16, 256, A16, need, None) == -1
    assert L.trellis_gemm_prefill(ctypes.byref(d), 100, A16, 512, A16, 256, A16 + 16, need, None) == -4
    bad = _layer(k_bits=0)
    assert L.trellis_gemm_prefill(ctypes.byref(bad), 100, A16, 512, A16, 256, A16, need, None) == -3


def test_moe_block_argument_validation():
    L = tg.lib()
    gu = (tg.TgLayer * 4)(*[_layer(m=256, n=512) for _ in range(4)])
    dn = (tg.TgLayer * 2)(*[_layer(m=512, n=256) for _ in range(2)])
    need = L.tg_moe_workspace_size(gu, 4, dn, 2, 2)
    assert need > 0
    assert L.tg_moe_workspace_size(gu, 3, dn, 2, 2) == 0            # gate/up table must be twice the down table
    assert L.tg_moe_workspace_size(gu, 4, dn, 2, 3) == 0            # top_k above the expert count
    bad = (tg.TgLayer * 2)(*[_layer(m=512, n=384) for _ in range(2)])
    assert L.tg_moe_workspace_size(gu, 4, bad, 2, 2) == 0           # down must be hidden x inter
    args = [gu, A16, 4, dn, A16, 2, A16, A16, 2, A16, A16]
    assert L.trellis_moe_block(*args, 0, need, None) == -5
    assert L.trellis_moe_block(*args, A16, need - 1, None) == -5
    assert L.trellis_moe_block(gu, A16, 4, dn, A16, 2, 0, A16, 2, A16, A16, A16, need, None) == -1
    assert L.trellis_moe_block(gu, A16, 4, dn, A16, 2, A16, A16, 0, A16, A16, A16, need, None) == -8


def test_trellis_linear_dispatch():
    """Row counts map to the entry points the dense-linear wrapper documents."""
    from trellis_coded_gemv_amd.binding import TrellisLinear
    assert TrellisLinear.path_for_rows(1) == "gemv"
    assert TrellisLinear.path_for_rows(2) == "small" and TrellisLinear.path_for_rows(64) == "small"
    assert TrellisLinear.path_for_rows(65) == "small_chunked" and TrellisLinear.path_for_rows(127) == "small_chunked"
    assert TrellisLinear.path_for_rows(128) == "prefill" and TrellisLinear.path_for_rows(4096) == "prefill"
    assert TrellisLinear.path_for_rows(100, prefill_min_rows=65) == "prefill"
    with pytest.raises(ValueError):
        TrellisLinear.path_for_rows(0)


def test_huge_shapes_rejected_before_launch():
    """The dense decode hook caps the weight count (2^38); the grouped grid must fit 31 bits; a
    batch-1 layer whose input chunks overflow the workspace's slot area (2048 block-chunk pairs) is
    refused, while the same layer's small-batch and prefill workspace sizes are still defined (the
    prefill path never stores decoded weights)."""
    L = tg.lib()
    big = _layer(m=1 << 22, n=1 << 22)
    assert L.trellis_gemv(ctypes.byref(big), A16, A16, A16, 1 << 40, None) == -2
    assert L.tg_workspace_size(ctypes.byref(big), 16) > 0
    assert L.trellis_decode(ctypes.byref(big), A16, None) == -2
    assert L.tg_prefill_workspace_size(ctypes.byref(big), 16) == 16 * (1 << 22) * 2
    table = (tg.TgLayer * 1)(_layer(m=1 << 22, n=1 << 22))
    assert L.tg_grouped_workspace_size(table, 1, 65536) == 0


def test_status_query_and_splits_validation():
    L = tg.lib()
    word = ctypes.c_uint32(7)
    assert L.tg_workspace_status(None, 0, ctypes.byref(word), None) == -1
    assert L.tg_workspace_status(A16, 0, None, None) == -1
    assert L.tg_workspace_status(A16 + 16, 0, ctypes.byref(word), None) == -4
    mixed = (tg.TgLayer * 2)(_layer(), _layer(splits=4))
    assert L.tg_grouped_workspace_size(mixed, 2, 4) == 0          # a table shares one splits value
    same = (tg.TgLayer * 2)(_layer(splits=4), _layer(splits=4))
    assert L.tg_grouped_workspace_size(same, 2, 4) > 0


def test_decode_ceiling_validation():
    L = tg.lib()
    assert L.tg_decode_ceiling(0, 0, 0, 1, 1, A16, None) == -3
    assert L.tg_decode_ceiling(2, 4, 0, 1, 1, A16, None) == -6
    assert L.tg_decode_ceiling(2, 0, 2, 1, 1, A16, None) == -8     # the int8 loop is mul1's
    assert L.tg_decode_ceiling(2, 2, 4, 1, 1, A16, None) == -8
    assert L.tg_decode_ceiling(2, 0, 0, 0, 1, A16, None) == -8
    assert L.tg_decode_ceiling(2, 0, 0, 1, 0, A16, None) == -8
    assert L.tg_decode_ceiling(2, 0, 0, 1, 1, 0, None) == -1
    assert L.tg_decode_ceiling(2, 2, 2, 1, 1, A16 + 2, None) == -4


def test_fused_validation():
    L = tg.lib()
    arr = (tg.TgLayer * 3)(_layer(m=512, n=1024), _layer(m=128, n=1024), _layer(m=256, n=1024))
    need = L.tg_fused_workspace_size(arr, 3)
    assert need >= 256 and need % 256 == 0
    assert L.tg_fused_workspace_size(arr, 0) == 0 and L.tg_fused_workspace_size(arr, 9) == 0
    ys = (ctypes.c_void_p * 3)(A16, A16, A16)
    assert L.trellis_gemv_fused(arr, 3, A16, ys, 0, need, None) == -5
    assert L.trellis_gemv_fused(arr, 3, A16, ys, A16, need - 1, None) == -5
    assert L.trellis_gemv_fused(arr, 3, 0, ys, A16, need, None) == -1
    assert L.trellis_gemv_fused(arr, 3, A16, None, A16, need, None) == -1
    assert L.trellis_gemv_fused(arr, 3, A16 + 1, ys, A16, need, None) == -4
    bad_y = (ctypes.c_void_p * 3)(A16, 0, A16)
    assert L.trellis_gemv_fused(arr, 3, A16, bad_y, A16, need, None) == -1
    mixed_n = (tg.TgLayer * 2)(_layer(n=1024), _layer(n=2048))
    assert L.tg_fused_workspace_size(mixed_n, 2) == 0
    mixed_k = (tg.TgLayer * 2)(_layer(n=1024), _layer(n=1024, k_bits=3))
    assert L.tg_fused_workspace_size(mixed_k, 2) == 0
    too_wide = (tg.TgLayer * 1)(_layer(n=16384 + 128))
    assert L.tg_fused_workspace_size(too_wide, 1) == 0


def test_mul1_and_int8_flag_validation():
    """code_id 2 passes the layer checks everywhere; TG_FLAG_INT8_ACT only with code_id 2 and only on the
    batch-1, no-allocation and fused entry points."""
    L = tg.lib()
    d = _layer(code_id=2)
    i8 = _layer(code_id=2, flags=2)
    ws = 1 << 34
    assert L.tg_workspace_size(ctypes.byref(d), 1) > 0
    assert L.trellis_gemv(ctypes.byref(d), A16, A16, 0, 1 << 30, None) == -5
    assert L.trellis_gemv(ctypes.byref(i8), A16, A16, 0, 1 << 30, None) == -5      # past the layer checks
    assert L.trellis_gemv(ctypes.byref(_layer(flags=2)), A16, A16, 0, 1 << 30, None) == -8
    assert L.trellis_gemv(ctypes.byref(_layer(code_id=1, flags=2)), A16, A16, 0, 1 << 30, None) == -8
    assert L.trellis_gemv_noalloc(ctypes.byref(_layer(flags=2)), A16, A16, None) == -8
    assert L.trellis_gemm_small(ctypes.byref(d), 16, A16, 512, A16, 256, 0, 1 << 30, None) == -5
    assert L.trellis_gemm_small(ctypes.byref(i8), 16, A16, 512, A16, 256, A16, ws, None) == -8
    assert L.trellis_gemm_prefill(ctypes.byref(i8), 16, A16, 512, A16, 256, A16, ws, None) == -8
    arr = (tg.TgLayer * 2)(i8, i8)
    assert L.tg_grouped_workspace_size(arr, 2, 4) == 0
    assert L.trellis_gemv_grouped(arr, A16, 2, A16, 4, A16, 0, A16, 256, A16, ws, None) == -8
    fz = (tg.TgLayer * 2)(_layer(code_id=2, flags=2, n=1024), _layer(code_id=2, flags=2, m=128, n=1024))
    need = L.tg_fused_workspace_size(fz, 2)
    assert need > 0
    ys = (ctypes.c_void_p * 2)(A16, A16)
    assert L.trellis_gemv_fused(fz, 2, A16, ys, 0, need, None) == -5
    mixed = (tg.TgLayer * 2)(_layer(code_id=2, n=1024), _layer(code_id=2, flags=2, n=1024))
    assert L.tg_fused_workspace_size(mixed, 2) == 0
    assert L.tg_code_table(2, 0, None) == -1
    assert L.trellis_decode(ctypes.byref(d), 0, None) == -1


def test_mcg_validation():
    """code_id 3 (MCG) passes the layer checks on every path, with or without the rounded form;
    the int8-activation flag stays mul1's."""
    L = tg.lib()
    d = _layer(code_id=3)
    r = _layer(code_id=3, flags=1)
    assert L.tg_workspace_size(ctypes.byref(d), 1) > 0
    assert L.trellis_gemv(ctypes.byref(d), A16, A16, 0, 1 << 30, None) == -5      # past the layer checks
    assert L.trellis_gemv(ctypes.byref(r), A16, A16, 0, 1 << 30, None) == -5
    assert L.trellis_gemv(ctypes.byref(_layer(code_id=3, flags=2)), A16, A16, 0, 1 << 30, None) == -8
    assert L.trellis_gemm_small(ctypes.byref(d), 16, A16, 512, A16, 256, 0, 1 << 30, None) == -5
    assert L.tg_encode_workspace_size(4, 8, 3) == L.tg_encode_workspace_size(4, 8, 0) > 0
    assert L.tg_code_table(3, 0, None) == -1
    assert L.trellis_decode(ctypes.byref(d), 0, None) == -1
    fz = (tg.TgLayer * 2)(_layer(code_id=3, n=1024), _layer(code_id=3, m=128, n=1024))
    assert L.tg_fused_workspace_size(fz, 2) > 0
    mixed = (tg.TgLayer * 2)(_layer(code_id=3, n=1024), _layer(code_id=0, n=1024))
    assert L.tg_fused_workspace_size(mixed, 2) == 0
    assert L.tg_grouped_workspace_size((tg.TgLayer * 2)(d, _layer(code_id=0)), 2, 4) > 0
