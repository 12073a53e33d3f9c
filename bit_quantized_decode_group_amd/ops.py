"""Thin Python binding over libqgemv.so (declared in include/qgemv.h).

Argument marshalling only: every function takes torch CUDA tensors, checks
that their dtypes / element sizes / contiguity match what the C ABI expects,
allocates outputs that were not passed in, and hands raw device pointers and
torch's current HIP stream to the library.  All arithmetic runs in the HIP
kernels.  There is no fallback: if the library was not built, the first call
raises.

Tensor conventions (bit patterns are what the ABI sees):
  bf16 data   torch.bfloat16 (or int16/uint16 holding bf16 bits)
  affine4     codes int32/uint32 [N, K/8]; scales, biases bf16 [N, K/64]
  Q4_K        uint8 [..., K/256, 144] (any leading shape; row-major blocks)
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "qgemv.h")

QG_OK, QG_EINVAL, QG_EALIAS, QG_EUNSUPPORTED, QG_EHIP = 0, -1, -2, -3, -4

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
_WS = [_P, _Z]  # (ws, ws_bytes)
_SIGS = {
    "qgemv_affine4": [_P, _P, _P, _P, _P, _I, _I, _I] + _WS + [_P],
    "qg_affine4_valu": [_P, _P, _P, _P, _P, _I, _I, _I] + _WS + [_P],
    "qgemv_q4k": [_P, _P, _P, _I, _I, _I] + _WS + [_P],
    "qgemv_affine4_rht": [_P, _P, _I, _P, _P, _P, _P, _I, _I, _I] + _WS + [_P],
    "affine4_tile_pack": [_P, _P, _P, _P, _P, _I, _I, _P],
    "qgemv_affine4_tiled": [_P, _P, _P, _P, _I, _I, _I] + _WS + [_P],
    "lmhead_argmax_tiled": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I] + _WS + [_P],
    "qg_check_affine4_tile_pack": [_P, _P, _P, _P, _P, _I, _I],
    "qg_check_qgemv_affine4_tiled": [_P, _P, _P, _P, _I, _I, _I] + _WS,
    "qg_check_lmhead_argmax_tiled": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I] + _WS,
    "qg_check_qgemv_affine4_rht": [_P, _P, _I, _P, _P, _P, _P, _I, _I, _I] + _WS,
    "qgemv_affine8": [_P, _P, _P, _P, _P, _I, _I, _I] + _WS + [_P],
    "qgemv_q6k": [_P, _P, _P, _I, _I, _I] + _WS + [_P],
    "qg_check_qgemv_q6k": [_P, _P, _P, _I, _I, _I] + _WS,
    "mlp_block_affine4_tiled": [_P, _P, _F, _P, _P, _P, _P, _P, _P, _I, _I, _I] + _WS + [_P],
    "qg_check_mlp_block_affine4_tiled": [_P, _P, _F, _P, _P, _P, _P, _P, _P, _I, _I, _I] + _WS,
    "qg_check_qgemv_affine8": [_P, _P, _P, _P, _P, _I, _I, _I] + _WS,
    "rmsnorm_gateup_swiglu_tiled": [_P, _P, _F, _P, _P, _P, _I, _I, _I] + _WS + [_P],
    "qg_check_rmsnorm_gateup_swiglu_tiled": [_P, _P, _F, _P, _P, _P, _I, _I, _I] + _WS,
    "rmsnorm_gateup_swiglu": [_P, _P, _F, _P, _P, _P, _P, _I, _I, _I] + _WS + [_P],
    "moe_expert_qgemv": [_P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I] + _WS + [_P],
    "lmhead_argmax": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I] + _WS + [_P],
    "lmhead_topk": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I] + _WS + [_P],
    "qg_check_qgemv_affine4": [_P, _P, _P, _P, _P, _I, _I, _I] + _WS,
    "qg_check_qgemv_q4k": [_P, _P, _P, _I, _I, _I] + _WS,
    "qg_check_rmsnorm_gateup_swiglu": [_P, _P, _F, _P, _P, _P, _P, _I, _I, _I] + _WS,
    "qg_check_moe_expert_qgemv": [_P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I] + _WS,
    "qg_check_lmhead_argmax": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I] + _WS,
    "qg_check_lmhead_topk": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I] + _WS,
    "lmhead_topk_tiled": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I] + _WS + [_P],
    "qg_check_lmhead_topk_tiled": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I] + _WS,
    "mlp_block_affine4_tiled_failures": [_P, _P],
    "lmhead_argmax_static": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P],
    "mlp_stack_affine4_tiled": [_P, _P, _F, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I] + _WS + [_P],
    "qg_check_mlp_stack_affine4_tiled": [_P, _P, _F, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I] + _WS,
}
# size queries: name -> shape arguments (all int); they return size_t
_QUERIES = {
    "qgemv_affine4_workspace": 3, "qg_affine4_valu_workspace": 3, "qgemv_affine8_workspace": 3,
    "qgemv_affine4_rht_workspace": 3, "qgemv_affine4_tiled_workspace": 3, "qgemv_q4k_workspace": 3,
    "qgemv_q6k_workspace": 3, "rmsnorm_gateup_swiglu_workspace": 3, "rmsnorm_gateup_swiglu_tiled_workspace": 3,
    "lmhead_argmax_workspace": 3, "lmhead_argmax_tiled_workspace": 3, "lmhead_topk_workspace": 5,
    "lmhead_topk_tiled_workspace": 5,
    "moe_expert_qgemv_workspace": 4, "mlp_block_affine4_tiled_workspace": 3,
    "mlp_stack_affine4_tiled_workspace": 3,
}


class QgError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


def lib():
    """Load libqgemv.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m bit_quantized_decode_group_amd.build` "
                "(there is no CPU fallback)")
        l = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int32
        for name, n in _QUERIES.items():
            fn = getattr(l, name)
            fn.argtypes = [_I] * n
            fn.restype = ctypes.c_size_t
        l.qg_workspace_header_bytes.argtypes = []
        l.qg_workspace_header_bytes.restype = ctypes.c_size_t
        l.qg_status_string.argtypes = [ctypes.c_int32]
        l.qg_status_string.restype = ctypes.c_char_p
        l.qg_last_error.argtypes = []
        l.qg_last_error.restype = ctypes.c_char_p
        _lib = l
    return _lib


def _raise_on(status: int, where: str):
    if status != QG_OK:
        l = lib()
        detail = l.qg_last_error().decode() or l.qg_status_string(status).decode()
        raise QgError(status, where, detail)


def _ptr(t):
    return None if t is None else _P(t.data_ptr())


def _stream():
    return _P(torch.cuda.current_stream().cuda_stream)


# ------------------------------------------------------------ workspaces --
# The library takes its scratch memory from the caller.  Every function below
# accepts `ws` (a workspace from `workspace()`); without one it uses a
# workspace this module keeps per (device, stream).  Workspaces are zeroed
# once when created (a fill kernel, no memset node) and are never freed while
# cached: a HIP graph captured earlier may still hold a pointer into one, so a
# cache that must grow adds a larger workspace and keeps the old ones.

def workspace(nbytes, device=None):
    """A zeroed workspace of at least nbytes bytes (uint8 CUDA tensor, 256-byte aligned)."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    n = max(int(nbytes), 1)
    t = torch.zeros(n + 256, dtype=torch.uint8, device=dev)
    off = (-t.data_ptr()) % 256
    return t[off:off + n]


@functools.lru_cache(maxsize=4096)
def _ws_query(entry: str, shape: tuple) -> int:
    return int(getattr(lib(), entry + "_workspace")(*shape))


def workspace_bytes(entry: str, *shape) -> int:
    """Bytes of workspace `entry` (e.g. "lmhead_argmax") needs for this shape (0: none)."""
    return _ws_query(entry, tuple(int(v) for v in shape))


_ws_cache = {}


def _default_ws(need, device):
    if need == 0:
        return None
    key = (device.index if device.index is not None else torch.cuda.current_device(),
           torch.cuda.current_stream(device).cuda_stream)
    held = _ws_cache.setdefault(key, [])
    if not held or held[-1].numel() < need:
        held.append(workspace(max(need, 2 * (held[-1].numel() if held else 0), 1 << 20), device))
    return held[-1]


def release_workspaces():
    """Drop the cached default workspaces (only when no captured graph still uses them)."""
    _ws_cache.clear()


def _ws_args(entry, shape, ws, device):
    need = workspace_bytes(entry, *shape)
    if ws is None:
        ws = _default_ws(need, device)
    if ws is None:
        return None, 0
    _need(ws, "ws", 1, device)
    return _P(ws.data_ptr()), ws.numel()


def _need(t, name, esize, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.element_size() != esize:
        raise TypeError(f"{name}: element size {t.element_size()} != {esize}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _dims2(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return t.shape[0], t.shape[1]


def qgemv_affine4(x, codes, scales, biases, y=None, ws=None):
    """Y[M,N] (bf16) = X[M,K] . dequant(W)[N,K]^T for affine-4 weights."""
    M, K = _dims2(x, "x")
    N = codes.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    for t, n, e in ((x, "x", 2), (codes, "codes", 4), (scales, "scales", 2), (biases, "biases", 2), (y, "y", 2)):
        _need(t, n, e, x.device)
    wsp, wsn = _ws_args("qgemv_affine4", (M, N, K), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().qgemv_affine4(_ptr(x), _ptr(codes), _ptr(scales), _ptr(biases), _ptr(y), M, N, K, wsp, wsn, _stream()),
                  "qgemv_affine4")
    return y


def affine4_valu(x, codes, scales, biases, y=None, ws=None):
    """Measurement aid: qgemv_affine4 with the products on the vector ALU (qg_affine4_valu)."""
    M, K = _dims2(x, "x")
    N = codes.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    for t, n, e in ((x, "x", 2), (codes, "codes", 4), (scales, "scales", 2), (biases, "biases", 2), (y, "y", 2)):
        _need(t, n, e, x.device)
    wsp, wsn = _ws_args("qg_affine4_valu", (M, N, K), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().qg_affine4_valu(_ptr(x), _ptr(codes), _ptr(scales), _ptr(biases), _ptr(y), M, N, K,
                                        wsp, wsn, _stream()), "qg_affine4_valu")
    return y


def qgemv_affine4_rht(x, signs, had, codes, scales, biases, y=None, ws=None):
    """Y[M,N] (bf16) = RHT(X)[M,K] . dequant(W)[N,K]^T; signs int8 [K], had a power of two dividing K."""
    M, K = _dims2(x, "x")
    N = codes.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    for t, n, e in ((x, "x", 2), (signs, "signs", 1), (codes, "codes", 4), (scales, "scales", 2),
                    (biases, "biases", 2), (y, "y", 2)):
        _need(t, n, e, x.device)
    if signs.numel() != K:
        raise ValueError("signs must hold K values")
    wsp, wsn = _ws_args("qgemv_affine4_rht", (M, N, K), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().qgemv_affine4_rht(_ptr(x), _ptr(signs), int(had), _ptr(codes), _ptr(scales), _ptr(biases),
                                          _ptr(y), M, N, K, wsp, wsn, _stream()), "qgemv_affine4_rht")
    return y


def tiled_bytes(N, K):
    """(codes bytes, scale/bias bytes) of the tile-order copy of an [N, K] affine-4 matrix."""
    l = lib()
    l.qg_tiled_bytes.argtypes = [_I, _I, ctypes.POINTER(ctypes.c_size_t)]
    l.qg_tiled_bytes.restype = ctypes.c_size_t
    sbb = ctypes.c_size_t(0)
    cb = int(l.qg_tiled_bytes(int(N), int(K), ctypes.byref(sbb)))
    if cb == 0:
        raise ValueError("tile order needs N >= 1 and K % 512 == 0")
    return cb, int(sbb.value)


def tile_pack(codes, scales, biases):
    """Tile-order copies (codes_t int32, sb_t bf16) of canonical affine-4 weights [N, K] (K % 512 == 0)."""
    N = codes.shape[0]
    K = codes.shape[1] * 8
    l = lib()
    cb, sbb = tiled_bytes(N, K)
    sbb = ctypes.c_size_t(sbb)
    codes_t = torch.empty(cb // 4, dtype=torch.int32, device=codes.device)
    sb_t = torch.empty(sbb.value // 2, dtype=torch.bfloat16, device=codes.device)
    for t, n, e in ((codes, "codes", 4), (scales, "scales", 2), (biases, "biases", 2)):
        _need(t, n, e, codes.device)
    with torch.cuda.device(codes.device):
        _raise_on(l.affine4_tile_pack(_ptr(codes), _ptr(scales), _ptr(biases), _ptr(codes_t), _ptr(sb_t), N, K,
                                      _stream()), "affine4_tile_pack")
    return codes_t, sb_t


def qgemv_affine8(x, codes, scales, biases, y=None, ws=None):
    """Y = X . dequant8(W)^T: codes int32 [N, K/4] (four 8-bit codes per word), scales/biases bf16 [N, K/64]."""
    M, K = _dims2(x, "x")
    N = codes.shape[0]
    if codes.dim() != 2 or codes.shape[1] * 4 != K:
        raise ValueError(f"codes must be [N, K/4] = [N, {K // 4}], got {tuple(codes.shape)}")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    for t, n, e in ((x, "x", 2), (codes, "codes", 4), (scales, "scales", 2), (biases, "biases", 2), (y, "y", 2)):
        _need(t, n, e, x.device)
    wsp, wsn = _ws_args("qgemv_affine8", (M, N, K), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().qgemv_affine8(_ptr(x), _ptr(codes), _ptr(scales), _ptr(biases), _ptr(y), M, N, K, wsp, wsn, _stream()),
                  "qgemv_affine8")
    return y


def mlp_block_affine4_tiled(x, gamma, eps, gu_t, dn_t, D, I, h=None, y=None, ws=None):
    """The MLP block (RMSNorm -> gate/up -> SwiGLU -> down) in one persistent launch on tile-order
    weights: gu_t = tile_pack of the [2I, D] gate-then-up matrix, dn_t = tile_pack of [D, I].
    Returns (h, y)."""
    M, K = _dims2(x, "x")
    if K != D:
        raise ValueError(f"x has {K} columns, D = {D}")
    if h is None:
        h = torch.empty((M, I), dtype=torch.bfloat16, device=x.device)
    if y is None:
        y = torch.empty((M, D), dtype=torch.bfloat16, device=x.device)
    for t, n, e in ((x, "x", 2), (gamma, "gamma", 2), (gu_t[0], "gu_codes_t", 4), (gu_t[1], "gu_sb_t", 2),
                    (dn_t[0], "dn_codes_t", 4), (dn_t[1], "dn_sb_t", 2), (h, "h", 2), (y, "y", 2)):
        _need(t, n, e, x.device)
    wsp, wsn = _ws_args("mlp_block_affine4_tiled", (M, D, I), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().mlp_block_affine4_tiled(_ptr(x), _ptr(gamma), float(eps), _ptr(gu_t[0]), _ptr(gu_t[1]),
                                                _ptr(dn_t[0]), _ptr(dn_t[1]), _ptr(h), _ptr(y), M, D, I, wsp, wsn, _stream()),
                  "mlp_block_affine4_tiled")
    return h, y


def mlp_stack_affine4_tiled(x, gamma, eps, gu_codes_t, gu_sb_t, dn_codes_t, dn_sb_t, L, D, I, h=None, ys=None,
                            ws=None):
    """L MLP blocks in one persistent launch on stacked tile-order weights: gamma [L, D];
    gu_codes_t / gu_sb_t and dn_codes_t / dn_sb_t hold the L layers' tile_pack outputs one after
    the other.  Returns (h [M, I] of the last layer, ys [L, M, D] = every layer's output)."""
    M, K = _dims2(x, "x")
    if K != D:
        raise ValueError(f"x has {K} columns, D = {D}")
    if h is None:
        h = torch.empty((M, I), dtype=torch.bfloat16, device=x.device)
    if ys is None:
        ys = torch.empty((L, M, D), dtype=torch.bfloat16, device=x.device)
    for t, n, e in ((x, "x", 2), (gamma, "gamma", 2), (gu_codes_t, "gu_codes_t", 4), (gu_sb_t, "gu_sb_t", 2),
                    (dn_codes_t, "dn_codes_t", 4), (dn_sb_t, "dn_sb_t", 2), (h, "h", 2), (ys, "ys", 2)):
        _need(t, n, e, x.device)
    gcb, gsb = tiled_bytes(2 * I, D)
    dcb, dsb = tiled_bytes(D, I)
    for t, n, b in ((gamma, "gamma", L * D * 2), (gu_codes_t, "gu_codes_t", L * gcb), (gu_sb_t, "gu_sb_t", L * gsb),
                    (dn_codes_t, "dn_codes_t", L * dcb), (dn_sb_t, "dn_sb_t", L * dsb), (h, "h", M * I * 2),
                    (ys, "ys", L * M * D * 2)):
        if t.numel() * t.element_size() != b:
            raise ValueError(f"{n} holds {t.numel() * t.element_size()} bytes, L={L} layers need {b}")
    wsp, wsn = _ws_args("mlp_stack_affine4_tiled", (M, D, I), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().mlp_stack_affine4_tiled(_ptr(x), _ptr(gamma), float(eps), _ptr(gu_codes_t), _ptr(gu_sb_t),
                                                _ptr(dn_codes_t), _ptr(dn_sb_t), _ptr(h), _ptr(ys), int(L), M, D, I,
                                                wsp, wsn, _stream()), "mlp_stack_affine4_tiled")
    return h, ys


def mlp_failures(ws):
    """Diagnostic: synchronises the current stream; how many persistent-MLP calls on workspace ws had a
    barrier wait give up since the last query (the count is reset)."""
    with torch.cuda.device(ws.device):
        return int(lib().mlp_block_affine4_tiled_failures(_ptr(ws), _stream()))


def qgemv_q6k(x, blocks, y=None, ws=None):
    """Y = X . dequant(W)^T for GGUF Q6_K blocks: uint8 [N, K/256, 210] (or [N, K/256*210])."""
    M, K = _dims2(x, "x")
    N = blocks.shape[0]
    if blocks.numel() != N * (K // 256) * 210 or K % 256:
        raise ValueError(f"blocks must hold N x K/256 Q6_K blocks of 210 bytes, got {tuple(blocks.shape)}")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    for t, n, e in ((x, "x", 2), (blocks, "blocks", 1), (y, "y", 2)):
        _need(t, n, e, x.device)
    wsp, wsn = _ws_args("qgemv_q6k", (M, N, K), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().qgemv_q6k(_ptr(x), _ptr(blocks), _ptr(y), M, N, K, wsp, wsn, _stream()), "qgemv_q6k")
    return y


def qgemv_affine4_tiled(x, codes_t, sb_t, N, y=None, ws=None):
    """qgemv_affine4 on tile-order weights (from tile_pack) of an [N, K] matrix."""
    M, K = _dims2(x, "x")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    for t, n, e in ((x, "x", 2), (codes_t, "codes_t", 4), (sb_t, "sb_t", 2), (y, "y", 2)):
        _need(t, n, e, x.device)
    wsp, wsn = _ws_args("qgemv_affine4_tiled", (M, N, K), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().qgemv_affine4_tiled(_ptr(x), _ptr(codes_t), _ptr(sb_t), _ptr(y), M, N, K, wsp, wsn, _stream()),
                  "qgemv_affine4_tiled")
    return y


def rmsnorm_gateup_swiglu_tiled(x, gamma, eps, codes_t, sb_t, I, h=None, ws=None):
    """rmsnorm_gateup_swiglu on the tile-order copy of the [2I, K] gate-then-up matrix."""
    M, K = _dims2(x, "x")
    if h is None:
        h = torch.empty((M, I), dtype=torch.bfloat16, device=x.device)
    for t, n, e in ((x, "x", 2), (gamma, "gamma", 2), (codes_t, "codes_t", 4), (sb_t, "sb_t", 2), (h, "h", 2)):
        _need(t, n, e, x.device)
    wsp, wsn = _ws_args("rmsnorm_gateup_swiglu_tiled", (M, I, K), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().rmsnorm_gateup_swiglu_tiled(_ptr(x), _ptr(gamma), float(eps), _ptr(codes_t),
                                                    _ptr(sb_t), _ptr(h), M, I, K, wsp, wsn, _stream()),
                  "rmsnorm_gateup_swiglu_tiled")
    return h


def lmhead_argmax_tiled(x, codes_t, sb_t, V, draft=None, logits=None, want_logits=False, ids=None, accepted=None,
                        ws=None):
    """lmhead_argmax on tile-order weights.  Returns (ids, accepted, logits or None)."""
    M, K = _dims2(x, "x")
    if logits is None and want_logits:
        logits = torch.empty((M, V), dtype=torch.float32, device=x.device)
    if ids is None:
        ids = torch.empty(M, dtype=torch.int32, device=x.device)
    if accepted is None:
        accepted = torch.empty(1, dtype=torch.int32, device=x.device)
    for t, n, e in ((x, "x", 2), (codes_t, "codes_t", 4), (sb_t, "sb_t", 2), (logits, "logits", 4),
                    (ids, "ids", 4), (draft, "draft", 4), (accepted, "accepted", 4)):
        _need(t, n, e, x.device)
    wsp, wsn = _ws_args("lmhead_argmax_tiled", (M, V, K), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().lmhead_argmax_tiled(_ptr(x), _ptr(codes_t), _ptr(sb_t), _ptr(logits), _ptr(ids), _ptr(draft),
                                            _ptr(accepted), M, V, K, wsp, wsn, _stream()), "lmhead_argmax_tiled")
    return ids, accepted, logits


def qgemv_q4k(x, blocks, y=None, ws=None):
    """Y[M,N] (bf16) = X[M,K] . dequant(W)[N,K]^T for Q4_K blocks [N, K/256, 144]."""
    M, K = _dims2(x, "x")
    N = blocks.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    for t, n, e in ((x, "x", 2), (blocks, "blocks", 1), (y, "y", 2)):
        _need(t, n, e, x.device)
    if blocks.numel() != N * (K // 256) * 144:
        raise ValueError("blocks must hold N * K/256 * 144 bytes")
    wsp, wsn = _ws_args("qgemv_q4k", (M, N, K), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().qgemv_q4k(_ptr(x), _ptr(blocks), _ptr(y), M, N, K, wsp, wsn, _stream()), "qgemv_q4k")
    return y


def rmsnorm_gateup_swiglu(x, gamma, eps, codes_gu, scales_gu, biases_gu, h=None, ws=None):
    """h[M,I] (bf16) = silu(xn.Wg^T) * (xn.Wu^T), xn = RMSNorm(x; gamma, eps)."""
    M, K = _dims2(x, "x")
    I = codes_gu.shape[0] // 2
    if h is None:
        h = torch.empty((M, I), dtype=torch.bfloat16, device=x.device)
    for t, n, e in ((x, "x", 2), (gamma, "gamma", 2), (codes_gu, "codes_gu", 4), (scales_gu, "scales_gu", 2),
                    (biases_gu, "biases_gu", 2), (h, "h", 2)):
        _need(t, n, e, x.device)
    wsp, wsn = _ws_args("rmsnorm_gateup_swiglu", (M, I, K), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().rmsnorm_gateup_swiglu(_ptr(x), _ptr(gamma), float(eps), _ptr(codes_gu), _ptr(scales_gu),
                                              _ptr(biases_gu), _ptr(h), M, I, K, wsp, wsn, _stream()),
                  "rmsnorm_gateup_swiglu")
    return h


def moe_expert_qgemv(x, router_logits, top_k, w_gu, w_down, y=None, out_ids=None, out_w=None, ws=None):
    """One token through the top-k routed Q4_K SwiGLU experts.  Returns (y, ids, w)."""
    D = x.numel()
    E = router_logits.numel()
    I = w_down.numel() // (E * D * 144) * 256
    if y is None:
        y = torch.empty((1, D), dtype=torch.bfloat16, device=x.device)
    if out_ids is None:
        out_ids = torch.empty(top_k, dtype=torch.int32, device=x.device)
    if out_w is None:
        out_w = torch.empty(top_k, dtype=torch.float32, device=x.device)
    for t, n, e in ((x, "x", 2), (router_logits, "router_logits", 4), (w_gu, "w_gu", 1), (w_down, "w_down", 1),
                    (y, "y", 2), (out_ids, "out_ids", 4), (out_w, "out_w", 4)):
        _need(t, n, e, x.device)
    wsp, wsn = _ws_args("moe_expert_qgemv", (top_k, E, D, I), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().moe_expert_qgemv(_ptr(x), _ptr(router_logits), int(top_k), _ptr(w_gu), _ptr(w_down), _ptr(y),
                                         _ptr(out_ids), _ptr(out_w), E, D, I, wsp, wsn, _stream()), "moe_expert_qgemv")
    return y, out_ids, out_w


def lmhead_argmax(x, codes, scales, biases, draft=None, logits=None, want_logits=False, ids=None, accepted=None,
                  ws=None):
    """Greedy readout.  Returns (ids int32 [M], accepted int32 [1], logits fp32 [M,V] or None)."""
    M, K = _dims2(x, "x")
    V = codes.shape[0]
    if logits is None and want_logits:
        logits = torch.empty((M, V), dtype=torch.float32, device=x.device)
    if ids is None:
        ids = torch.empty(M, dtype=torch.int32, device=x.device)
    if accepted is None:
        accepted = torch.empty(1, dtype=torch.int32, device=x.device)
    for t, n, e in ((x, "x", 2), (codes, "codes", 4), (scales, "scales", 2), (biases, "biases", 2),
                    (logits, "logits", 4), (ids, "ids", 4), (draft, "draft", 4), (accepted, "accepted", 4)):
        _need(t, n, e, x.device)
    if draft is not None and draft.numel() < M:
        raise ValueError("draft must hold at least M ids")
    wsp, wsn = _ws_args("lmhead_argmax", (M, V, K), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().lmhead_argmax(_ptr(x), _ptr(codes), _ptr(scales), _ptr(biases), _ptr(logits), _ptr(ids),
                                      _ptr(draft), _ptr(accepted), M, V, K, wsp, wsn, _stream()), "lmhead_argmax")
    return ids, accepted, logits


def lmhead_argmax_static(x, codes, scales, biases, draft=None, logits=None, want_logits=False, ids=None,
                         accepted=None):
    """lmhead_argmax with the library's static scratch (no workspace; the call allocates nothing on the device).
    Returns (ids int32 [M], accepted int32 [1], logits fp32 [M,V] or None)."""
    M, K = _dims2(x, "x")
    V = codes.shape[0]
    if logits is None and want_logits:
        logits = torch.empty((M, V), dtype=torch.float32, device=x.device)
    if ids is None:
        ids = torch.empty(M, dtype=torch.int32, device=x.device)
    if accepted is None:
        accepted = torch.empty(1, dtype=torch.int32, device=x.device)
    for t, n, e in ((x, "x", 2), (codes, "codes", 4), (scales, "scales", 2), (biases, "biases", 2),
                    (logits, "logits", 4), (ids, "ids", 4), (draft, "draft", 4), (accepted, "accepted", 4)):
        _need(t, n, e, x.device)
    if draft is not None and draft.numel() < M:
        raise ValueError("draft must hold at least M ids")
    with torch.cuda.device(x.device):
        _raise_on(lib().lmhead_argmax_static(_ptr(x), _ptr(codes), _ptr(scales), _ptr(biases), _ptr(logits),
                                             _ptr(ids), _ptr(draft), _ptr(accepted), M, V, K, _stream()),
                  "lmhead_argmax_static")
    return ids, accepted, logits


def lmhead_topk(x, codes, scales, biases, k, logits=None, want_logits=False, ids=None, vals=None, want_vals=True,
                ws=None):
    """Top-k readout.  Returns (ids int32 [M,k], vals fp32 [M,k] or None, logits fp32 [M,V] or None)."""
    M, K = _dims2(x, "x")
    V = codes.shape[0]
    if logits is None and want_logits:
        logits = torch.empty((M, V), dtype=torch.float32, device=x.device)
    if ids is None:
        ids = torch.empty((M, k), dtype=torch.int32, device=x.device)
    if vals is None and want_vals:
        vals = torch.empty((M, k), dtype=torch.float32, device=x.device)
    for t, n, e in ((x, "x", 2), (codes, "codes", 4), (scales, "scales", 2), (biases, "biases", 2),
                    (logits, "logits", 4), (ids, "ids", 4), (vals, "vals", 4)):
        _need(t, n, e, x.device)
    wsp, wsn = _ws_args("lmhead_topk", (M, V, K, k, logits is not None), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().lmhead_topk(_ptr(x), _ptr(codes), _ptr(scales), _ptr(biases), _ptr(logits), _ptr(ids),
                                    _ptr(vals), M, V, K, int(k), wsp, wsn, _stream()), "lmhead_topk")
    return ids, vals, logits


def lmhead_topk_tiled(x, codes_t, sb_t, V, k, logits=None, want_logits=False, ids=None, vals=None, want_vals=True,
                      ws=None):
    """lmhead_topk on tile-order weights.  Returns (ids [M,k], vals [M,k] or None, logits [M,V] or None)."""
    M, K = _dims2(x, "x")
    if logits is None and want_logits:
        logits = torch.empty((M, V), dtype=torch.float32, device=x.device)
    if ids is None:
        ids = torch.empty((M, k), dtype=torch.int32, device=x.device)
    if vals is None and want_vals:
        vals = torch.empty((M, k), dtype=torch.float32, device=x.device)
    for t, n, e in ((x, "x", 2), (codes_t, "codes_t", 4), (sb_t, "sb_t", 2), (logits, "logits", 4),
                    (ids, "ids", 4), (vals, "vals", 4)):
        _need(t, n, e, x.device)
    wsp, wsn = _ws_args("lmhead_topk_tiled", (M, V, K, k, logits is not None), ws, x.device)
    with torch.cuda.device(x.device):
        _raise_on(lib().lmhead_topk_tiled(_ptr(x), _ptr(codes_t), _ptr(sb_t), _ptr(logits), _ptr(ids), _ptr(vals),
                                          M, V, K, int(k), wsp, wsn, _stream()), "lmhead_topk_tiled")
    return ids, vals, logits


def stream_read(buf):
    """Measurement aid: one streaming read of a contiguous CUDA tensor's bytes."""
    _need(buf, "buf", buf.element_size(), buf.device)
    sink = torch.empty(1, dtype=torch.int32, device=buf.device)
    l = lib()
    l.qg_stream_read.argtypes = [_P, ctypes.c_size_t, _P, _P]
    l.qg_stream_read.restype = ctypes.c_int32
    with torch.cuda.device(buf.device):
        _raise_on(l.qg_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream()),
                  "qg_stream_read")


# ------------------------------------------------------------- host checks --
# The qg_check_* twins run the entry points' argument checks on the host only
# (no GPU, no launch); they take raw addresses so tests can probe the rules.

def check(name: str, *args) -> int:
    """Call qg_check_<name>(*args) with integer addresses; returns the status."""
    fn = getattr(lib(), "qg_check_" + name)
    conv = []
    for a, ty in zip(args, fn.argtypes):
        conv.append(_P(a) if ty is _P else a)
    return int(fn(*conv))


def last_error() -> str:
    return lib().qg_last_error().decode()
