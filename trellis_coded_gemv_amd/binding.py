"""ctypes binding of libtrellis_gemv.so -- argument marshalling only.

Every step of the computation runs in the library's HIP kernels; PyTorch is
used only to own device memory and to supply the current HIP stream. The
functions mirror the C ABI of include/trellis_gemv.h name for name. If the
library is missing or fails to load, every entry point raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtrellis_gemv.so")

TG_FLAG_ROUND_WEIGHTS = 1
TG_FLAG_INT8_ACT = 2
TG_STATUS_SPLITK_TIMEOUT = 1
ABI_VERSION = 4

STATUS = {0: "TG_OK", -1: "TG_ERR_NULL", -2: "TG_ERR_SHAPE", -3: "TG_ERR_KBITS", -4: "TG_ERR_ALIGN",
          -5: "TG_ERR_WORKSPACE", -6: "TG_ERR_CODE_ID", -7: "TG_ERR_LAUNCH", -8: "TG_ERR_ARG"}

# every symbol the header declares
EXPORTS = ("tg_abi_version", "tg_build_id", "tg_workspace_status", "tg_status_str", "tg_workspace_size",
           "trellis_gemv", "trellis_gemv_noalloc", "tg_noalloc_scratch_bytes", "trellis_gemv_fused",
           "tg_fused_workspace_size", "trellis_gemm_small",
           "tg_decode_ceiling",
           "rht_apply", "trellis_gemv_grouped", "tg_grouped_workspace_size", "trellis_decode", "tg_code_table",
           "trellis_encode", "tg_encode_workspace_size", "trellis_gemm_prefill", "tg_prefill_workspace_size",
           "trellis_moe_block", "tg_moe_workspace_size")


class TgLayer(ctypes.Structure):
    """Mirror of tg_layer."""
    _fields_ = [("m", ctypes.c_int32), ("n", ctypes.c_int32), ("k_bits", ctypes.c_int32),
                ("code_id", ctypes.c_int32), ("flags", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("sign_in", ctypes.c_void_p), ("sign_out", ctypes.c_void_p)]


class TgError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_status_str(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it is not built, or was built from other sources
    than the ones in this tree (its tg_build_id differs from their hash)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m trellis_coded_gemv_amd.build`")
    from .build import source_hash
    L = ctypes.CDLL(LIB_PATH)
    L.tg_build_id.restype = ctypes.c_char_p
    L.tg_build_id.argtypes = []
    built, want = L.tg_build_id().decode(), source_hash()
    if built != want:
        raise RuntimeError(f"{LIB_PATH} was built from other sources (build id {built}, sources {want}): "
                           "rebuild it with `python -m trellis_coded_gemv_amd.build`")
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    LP = ctypes.POINTER(TgLayer)
    sig = {
        "tg_abi_version": (I32, []),
        "tg_build_id": (ctypes.c_char_p, []),
        "tg_workspace_status": (I32, [P, I32, ctypes.POINTER(ctypes.c_uint32), P]),
        "tg_status_str": (ctypes.c_char_p, [I32]),
        "tg_workspace_size": (SZ, [LP, I32]),
        "trellis_gemv": (I32, [LP, P, P, P, SZ, P]),
        "trellis_gemv_noalloc": (I32, [LP, P, P, P]),
        "trellis_gemv_fused": (I32, [LP, I32, P, P, P, SZ, P]),
        "tg_fused_workspace_size": (SZ, [LP, I32]),
        "tg_noalloc_scratch_bytes": (SZ, []),
        "trellis_gemm_small": (I32, [LP, I32, P, I64, P, I64, P, SZ, P]),
        "rht_apply": (I32, [I32, I32, P, P, P, I32, P]),
        "trellis_gemv_grouped": (I32, [LP, P, I32, P, I32, P, I64, P, I64, P, SZ, P]),
        "tg_grouped_workspace_size": (SZ, [LP, I32, I32]),
        "trellis_decode": (I32, [LP, P, P]),
        "tg_code_table": (I32, [I32, P, P]),
        "tg_decode_ceiling": (I32, [I32, I32, I32, I32, I32, P, P]),
        "trellis_encode": (I32, [I32, I32, I32, ctypes.c_float, P, P, P, P, SZ, P]),
        "tg_encode_workspace_size": (SZ, [I32, I32, I32]),
        "trellis_gemm_prefill": (I32, [LP, I32, P, I64, P, I64, P, SZ, P]),
        "tg_prefill_workspace_size": (SZ, [LP, I32]),
        "trellis_moe_block": (I32, [LP, P, I32, LP, P, I32, P, P, I32, P, P, P, SZ, P]),
        "tg_moe_workspace_size": (SZ, [LP, I32, LP, I32, I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    if L.tg_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {L.tg_abi_version()}, the binding expects {ABI_VERSION}")
    _lib = L
    return L


def _status_str(status: int) -> str:
    try:
        return lib().tg_status_str(status).decode()
    except Exception:  # noqa: BLE001 - message only
        return "?"


def _check(status: int, where: str) -> None:
    if status != 0:
        raise TgError(status, where)


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class DeviceLayer:
    """A layer's arrays in device memory plus its tg_layer descriptor."""

    def __init__(self, arrays, device="cuda", flags: int = 0, splits: int = 0):
        torch = _torch()
        self.m, self.n, self.k_bits = int(arrays.m), int(arrays.n), int(arrays.k_bits)
        self.code_id, self.flags, self.splits = int(getattr(arrays, "code_id", 0)), int(flags), int(splits)
        self.codes = torch.from_numpy(np.ascontiguousarray(arrays.codes).view(np.int32)).to(device)
        self.scales = torch.from_numpy(np.ascontiguousarray(arrays.scales).view(np.int16)).to(device)
        self.sign_in = torch.from_numpy(np.ascontiguousarray(arrays.sign_in).view(np.int32)).to(device)
        self.sign_out = torch.from_numpy(np.ascontiguousarray(arrays.sign_out).view(np.int32)).to(device)

    def desc(self) -> TgLayer:
        return TgLayer(self.m, self.n, self.k_bits, self.code_id, self.flags, self.splits,
                       self.codes.data_ptr(), self.scales.data_ptr(),
                       self.sign_in.data_ptr(), self.sign_out.data_ptr())

    @property
    def code_bytes(self) -> int:
        return self.codes.numel() * 4


def fp16_tensor(bits: np.ndarray, device="cuda"):
    """Host uint16 fp16 patterns -> device float16 tensor (same bits)."""
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.float16)).to(device)


def build_id() -> str:
    return lib().tg_build_id().decode()


def workspace_status(ws, clear: bool = False, stream=None) -> int:
    """The workspace's status word (TG_STATUS_* bits); waits for the stream."""
    word = ctypes.c_uint32(0)
    _check(lib().tg_workspace_status(_ptr(ws), int(clear), ctypes.byref(word), _stream(stream)), "tg_workspace_status")
    return int(word.value)


def workspace_size(layer: DeviceLayer, M: int = 1) -> int:
    d = layer.desc()
    return int(lib().tg_workspace_size(ctypes.byref(d), M))


def workspace(layer: DeviceLayer, M: int = 1, device="cuda"):
    """Zero-filled workspace for trellis_gemv (M == 1) / trellis_gemm_small."""
    size = workspace_size(layer, M)
    if size == 0:
        raise TgError(-8, "tg_workspace_size")
    return _torch().zeros(size, dtype=_torch().uint8, device=device)


def trellis_gemv(layer: DeviceLayer, x, y=None, ws=None, stream=None):
    """y = W x for fp16 x [n] on the device; returns fp32 y [m]."""
    torch = _torch()
    if y is None:
        y = torch.empty(layer.m, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(layer, 1, x.device)
    d = layer.desc()
    _check(lib().trellis_gemv(ctypes.byref(d), _ptr(x), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)),
           "trellis_gemv")
    return y


def _layer_array(layers):
    arr = (TgLayer * len(layers))(*[L.desc() for L in layers])
    return arr


def fused_workspace(layers, device="cuda"):
    """Zero-filled workspace for trellis_gemv_fused over these layers."""
    size = int(lib().tg_fused_workspace_size(_layer_array(layers), len(layers)))
    if size == 0:
        raise TgError(-8, "tg_fused_workspace_size")
    return _torch().zeros(size, dtype=_torch().uint8, device=device)


def trellis_gemv_fused(layers, x, ys=None, ws=None, stream=None):
    """y_l = W_l x for layers that share the fp16 input x [n]; returns the list of fp32 outputs."""
    torch = _torch()
    if ys is None:
        ys = [torch.empty(L.m, dtype=torch.float32, device=x.device) for L in layers]
    if ws is None:
        ws = fused_workspace(layers, x.device)
    arr = _layer_array(layers)
    yp = (ctypes.c_void_p * len(layers))(*[y.data_ptr() for y in ys])
    _check(lib().trellis_gemv_fused(arr, len(layers), _ptr(x), yp, _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)), "trellis_gemv_fused")
    return ys


def trellis_gemm_small(layer: DeviceLayer, X, Y=None, ws=None, stream=None):
    """Y[r] = W X[r] for fp16 X [M, n] (row stride X.stride(0)); returns fp32 Y [M, m]."""
    torch = _torch()
    M = X.shape[0]
    if Y is None:
        Y = torch.empty(M, layer.m, dtype=torch.float32, device=X.device)
    if ws is None:
        ws = workspace(layer, M, X.device)
    d = layer.desc()
    ldx = X.stride(0) if M > 1 else X.shape[1]      # a single row's stride is meaningless (may be 0)
    ldy = Y.stride(0) if M > 1 else Y.shape[1]
    _check(lib().trellis_gemm_small(ctypes.byref(d), M, _ptr(X), ldx, _ptr(Y), ldy,
                                    _ptr(ws), ws.numel(), _stream(stream)), "trellis_gemm_small")
    return Y


def rht_apply(x, signs, inverse: bool = False, out=None, stream=None):
    """Randomized Hadamard transform on 128-blocks of fp16 rows x [rows, n] -> fp32."""
    torch = _torch()
    x2 = x.reshape(-1, x.shape[-1])
    if out is None:
        out = torch.empty(x2.shape, dtype=torch.float32, device=x.device)
    _check(lib().rht_apply(x2.shape[1], x2.shape[0], _ptr(x2), _ptr(out), _ptr(signs), int(bool(inverse)),
                           _stream(stream)), "rht_apply")
    return out.reshape(x.shape)


class LayerTable:
    """Host and device copies of an array of tg_layer descriptors (for the grouped path)."""

    def __init__(self, layers: Sequence[DeviceLayer], device="cuda"):
        torch = _torch()
        self.layers = list(layers)
        self.host = (TgLayer * len(self.layers))(*[l.desc() for l in self.layers])
        raw = np.frombuffer(bytes(self.host), dtype=np.uint8)
        self.device = torch.from_numpy(raw.copy()).to(device)

    def __len__(self):
        return len(self.layers)


def grouped_workspace(table: LayerTable, n_sel: int, device="cuda"):
    size = int(lib().tg_grouped_workspace_size(table.host, len(table), n_sel))
    if size == 0:
        raise TgError(-8, "tg_grouped_workspace_size")
    return _torch().zeros(size, dtype=_torch().uint8, device=device)


def trellis_gemv_grouped(table: LayerTable, sel, X, x_stride: int, Y, y_stride: int, ws=None, stream=None):
    """For each e < len(sel): Y[e*y_stride : ...][:m] = W_{sel[e]} X[e*x_stride : ...] (x_stride 0 = shared x)."""
    n_sel = int(sel.numel())
    if ws is None:
        ws = grouped_workspace(table, n_sel, X.device)
    _check(lib().trellis_gemv_grouped(table.host, _ptr(table.device), len(table), _ptr(sel), n_sel,
                                      _ptr(X), x_stride, _ptr(Y), y_stride, _ptr(ws), ws.numel(), _stream(stream)),
           "trellis_gemv_grouped")
    return Y


def trellis_decode(layer: DeviceLayer, out=None, stream=None):
    """All decoded weights as fp16 patterns, int16 tensor [m, n]."""
    torch = _torch()
    if out is None:
        out = torch.empty(layer.m, layer.n, dtype=torch.int16, device=layer.codes.device)
    d = layer.desc()
    _check(lib().trellis_decode(ctypes.byref(d), _ptr(out), _stream(stream)), "trellis_decode")
    return out


def decode_ceiling(k_bits: int, code_id: int, workgroups: int, steps: int, out=None, stream=None, flags: int = 0):
    """Launch the decode-only rate probe; returns its fp32 output [workgroups * 512]."""
    torch = _torch()
    if out is None:
        out = torch.empty(workgroups * 512, dtype=torch.float32, device="cuda")
    _check(lib().tg_decode_ceiling(k_bits, code_id, int(flags), workgroups, steps, _ptr(out), _stream(stream)),
           "tg_decode_ceiling")
    return out


def code_table(device="cuda", code_id: int = 0, stream=None):
    """The code for all 65536 states: int16 [65536] (code 0) or [65536, 2] (pair code)."""
    torch = _torch()
    shape = (1 << 16, 2) if code_id == 1 else (1 << 16,)
    out = torch.empty(shape, dtype=torch.int16, device=device)
    _check(lib().tg_code_table(int(code_id), _ptr(out), _stream(stream)), "tg_code_table")
    return out


def encode_workspace(n_tiles: int, k_bits: int, code_id: int = 0, device="cuda"):
    torch = _torch()
    n = lib().tg_encode_workspace_size(int(n_tiles), int(k_bits), int(code_id))
    if n == 0:
        raise TgError(-8, "tg_encode_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def trellis_encode(targets, k_bits: int, code_id: int = 0, scale: float = 1.0, codes=None, sq_err=None, ws=None,
                   stream=None):
    """Viterbi-encode tiles: targets fp32 [n_tiles, 256] (sequence order) -> (codes int32 [n_tiles, 8K], sq_err)."""
    torch = _torch()
    if targets.dtype != torch.float32 or not targets.is_contiguous() or targets.shape[-1] != 256:
        raise ValueError("targets must be a contiguous float32 tensor [n_tiles, 256]")
    n_tiles = int(targets.shape[0])
    dev = targets.device
    if codes is None:
        codes = torch.empty(n_tiles, 8 * k_bits, dtype=torch.int32, device=dev)
    if sq_err is None:
        sq_err = torch.empty(n_tiles, dtype=torch.float32, device=dev)
    if ws is None:
        ws = encode_workspace(n_tiles, k_bits, code_id, dev)
    _check(lib().trellis_encode(n_tiles, int(k_bits), int(code_id), float(scale), _ptr(targets),
                                _ptr(codes), _ptr(sq_err), _ptr(ws), ws.numel(), _stream(stream)), "trellis_encode")
    return codes, sq_err


def prefill_workspace(layer: DeviceLayer, M: int, device="cuda"):
    torch = _torch()
    d = layer.desc()
    n = lib().tg_prefill_workspace_size(ctypes.byref(d), int(M))
    if n == 0:
        raise TgError(-2, "tg_prefill_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def trellis_gemm_prefill(layer: DeviceLayer, X, Y=None, ws=None, stream=None):
    """Y [M, m] fp32 = W X[r] for every row of fp16 X [M, n] (row stride X.stride(0)); each weight decoded once per 512 rows into MFMA operands."""
    torch = _torch()
    M = int(X.shape[0])
    if Y is None:
        Y = torch.empty(M, layer.m, dtype=torch.float32, device=X.device)
    if ws is None:
        ws = prefill_workspace(layer, M, X.device)
    d = layer.desc()
    ldx = X.stride(0) if M > 1 else X.shape[1]
    ldy = Y.stride(0) if M > 1 else Y.shape[1]
    _check(lib().trellis_gemm_prefill(ctypes.byref(d), M, _ptr(X), ldx, _ptr(Y), ldy, _ptr(ws), ws.numel(),
                                      _stream(stream)), "trellis_gemm_prefill")
    return Y


def moe_workspace(gate_up: "LayerTable", down: "LayerTable", top_k: int, device="cuda"):
    torch = _torch()
    n = lib().tg_moe_workspace_size(gate_up.host, len(gate_up), down.host, len(down), int(top_k))
    if n == 0:
        raise TgError(-8, "tg_moe_workspace_size")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def trellis_moe_block(gate_up: "LayerTable", down: "LayerTable", sel, weights, x, y=None, ws=None, stream=None):
    """y [hidden] fp32 = sum_i w_i down_{sel_i}(fp16(silu(gate(x)) * up(x))); sel int32 / weights fp32 on device."""
    torch = _torch()
    top_k = int(sel.numel())
    hidden = down.layers[0].m
    if y is None:
        y = torch.empty(hidden, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = moe_workspace(gate_up, down, top_k, x.device)
    _check(lib().trellis_moe_block(gate_up.host, _ptr(gate_up.device), len(gate_up), down.host, _ptr(down.device),
                                   len(down), _ptr(sel), _ptr(weights), top_k, _ptr(x), _ptr(y), _ptr(ws),
                                   ws.numel(), _stream(stream)), "trellis_moe_block")
    return y


class TrellisLinear:
    """A trellis-coded linear layer used like a dense one: y = W x over the last axis.

    `forward(x)` takes fp16 activations [..., n] on the device and returns fp32 [..., m]. It
    picks the entry point by the number of rows R (the product of the leading axes), as the
    pages' drop-in linear does for its batch sizes ("Trellis Quantization" lecture, Part
    eleven: small batches decode per call, prefill decodes once):
      R == 1                 -> trellis_gemv
      R <= 64                -> trellis_gemm_small
      R <  prefill_min_rows  -> trellis_gemm_small on row chunks of 64
      otherwise              -> trellis_gemm_prefill (decode once per 512 rows into MFMA operands)
    The default threshold (128 rows) sits at the measured crossover of the last two on the
    8192 -> 28672 gate shape (96 rows: chunked small batch faster; 128: prefill faster). Workspaces are allocated on first use of each path and kept
    (the prefill one grows with the largest row count seen); calls are ordered on one stream.
    """

    SMALL_MAX_ROWS = 64

    def __init__(self, layer: DeviceLayer, prefill_min_rows: int = 128):
        self.layer = layer
        self.prefill_min_rows = int(prefill_min_rows)
        self._ws = None
        self._prefill_ws, self._prefill_rows = None, 0

    @classmethod
    def path_for_rows(cls, rows: int, prefill_min_rows: int = 128) -> str:
        if rows < 1:
            raise ValueError("no rows")
        if rows == 1:
            return "gemv"
        if rows <= cls.SMALL_MAX_ROWS:
            return "small"
        return "small_chunked" if rows < prefill_min_rows else "prefill"

    def _layer_ws(self, device):
        if self._ws is None:   # one buffer for every row count up to 64 (the split count varies with it)
            size = max(workspace_size(self.layer, M) for M in range(1, self.SMALL_MAX_ROWS + 1))
            self._ws = _torch().zeros(size, dtype=_torch().uint8, device=device)
        return self._ws

    def forward(self, x, stream=None):
        torch = _torch()
        n, m = self.layer.n, self.layer.m
        if x.dtype != torch.float16 or x.shape[-1] != n:
            raise ValueError(f"expected float16 activations [..., {n}], got {tuple(x.shape)} {x.dtype}")
        lead = tuple(x.shape[:-1])
        X = x.reshape(-1, n).contiguous()
        rows = X.shape[0]
        path = self.path_for_rows(rows, self.prefill_min_rows)
        Y = torch.empty(rows, m, dtype=torch.float32, device=x.device)
        if path == "gemv":
            trellis_gemv(self.layer, X[0], Y[0], self._layer_ws(x.device), stream)
        elif path == "prefill":
            if rows > self._prefill_rows:
                self._prefill_ws, self._prefill_rows = prefill_workspace(self.layer, rows, x.device), rows
            trellis_gemm_prefill(self.layer, X, Y, self._prefill_ws, stream)
        else:
            ws = self._layer_ws(x.device)
            for r0 in range(0, rows, self.SMALL_MAX_ROWS):
                r1 = min(rows, r0 + self.SMALL_MAX_ROWS)
                trellis_gemm_small(self.layer, X[r0:r1], Y[r0:r1], ws, stream)
        return Y.reshape(lead + (m,))

    __call__ = forward
