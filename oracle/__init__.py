"""Plain fp64 CPU oracle for the 4-bit quantized decode projections.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the GPU library (``bit_quantized_decode_group_amd``): the arithmetic
lives in ``oracle.c`` (plain C, double precision, ascending summation order),
and this module only marshals numpy arrays into it.

Which step of the method each function follows is documented in ``oracle.h``
next to its declaration (O0-O15), with the page and section it comes from.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_MT_PATH = os.path.join(_HERE, "liboracle_mt.so")
_lib = None
_mt = False  # which build _lib is


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` with gcc (-O2, no fast-math, no FMA contraction)
    into ``liboracle.so`` (single-threaded, what the tests use) and
    ``liboracle_mt.so`` (the same code with OpenMP: output rows split over
    threads, every row's sum unchanged; only for timing the oracle on all host
    cores).  Returns the path of the single-threaded library."""
    src = os.path.join(_HERE, "oracle.c")
    for path, extra in ((_LIB_PATH, []), (_MT_PATH, ["-fopenmp"])):
        if force or not os.path.exists(path) or os.path.getmtime(path) < max(
            os.path.getmtime(src), os.path.getmtime(os.path.join(_HERE, "oracle.h"))
        ):
            tmp = path + ".tmp%d" % os.getpid()
            subprocess.check_call(
                ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                 "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unknown-pragmas", *extra, "-o", tmp, src, "-lm"],
                cwd=_HERE,
            )
            os.replace(tmp, path)
    return _LIB_PATH


def use_threads(n: int) -> int:
    """Run the following oracle calls on n host threads (n > 1: the OpenMP
    build; n <= 1: the single-threaded build).  Returns the threads in use."""
    global _lib, _mt
    want_mt = n > 1
    if _lib is not None and _mt != want_mt:
        _lib = None
    _mt = want_mt
    return int(_load().oracle_set_threads(int(n)))


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_MT_PATH if _mt else _LIB_PATH)
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = ctypes.c_int
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        D = ctypes.c_double
        lib.o_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.o_bf16_to_f64.restype = D
        lib.o_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.o_f16_to_f64.restype = D
        lib.o_f64_to_bf16_rne.argtypes = [D]
        lib.o_f64_to_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_dequant_affine4.argtypes = [P, P, P, I64, I64, I64, I64, P]
        lib.oracle_dequant_q4k.argtypes = [P, I64, I64, I64, I64, P]
        lib.oracle_qgemv_affine4.argtypes = [P, P, P, P, I, I64, I64, P]
        lib.oracle_qgemv_affine4_f64x.argtypes = [P, P, P, P, I, I64, I64, P]
        lib.oracle_dequant_affine8.argtypes = [P, P, P, I64, I64, I64, I64, P]
        lib.oracle_qgemv_affine8.argtypes = [P, P, P, P, I, I64, I64, P]
        lib.oracle_dequant_q6k.argtypes = [P, I64, I64, I64, I64, P]
        lib.oracle_qgemv_q6k.argtypes = [P, P, I, I64, I64, P]
        lib.oracle_qgemv_q4k.argtypes = [P, P, I, I64, I64, P]
        lib.oracle_rmsnorm.argtypes = [P, P, D, I, I64, P]
        lib.oracle_silu.argtypes = [D]
        lib.oracle_silu.restype = D
        lib.oracle_rmsnorm_gateup_swiglu.argtypes = [P, P, D, P, P, P, I, I64, I64, P]
        lib.oracle_mlp_block.argtypes = [P, P, D, P, P, P, P, P, P, I, I64, I64, P]
        lib.oracle_moe.argtypes = [P, P, I, P, P, I, I64, I64, P, P, P]
        lib.oracle_lmhead.argtypes = [P, P, P, P, I, I64, I64, P, P, P, P, P]
        lib.oracle_lmhead_topk.argtypes = [P, P, P, P, I, I64, I64, I, P, P]
        lib.oracle_rht.argtypes = [P, P, I, I, I64, P]
        lib.oracle_qgemv_affine4_rht.argtypes = [P, P, I, P, P, P, I, I64, I64, P]
        for name in ("oracle_dequant_affine4", "oracle_dequant_q4k", "oracle_qgemv_affine4",
                     "oracle_qgemv_affine4_f64x", "oracle_qgemv_q4k", "oracle_rmsnorm",
                     "oracle_rmsnorm_gateup_swiglu", "oracle_mlp_block", "oracle_moe",
                     "oracle_lmhead", "oracle_lmhead_topk", "oracle_rht", "oracle_qgemv_affine4_rht",
                     "oracle_dequant_affine8", "oracle_qgemv_affine8", "oracle_dequant_q6k", "oracle_qgemv_q6k"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle: {name} rejected its arguments")


# -------------------------------------------------------------------- O0 --
def bf16_to_f64(h: int) -> float:
    return _load().o_bf16_to_f64(int(h))


def f16_to_f64(h: int) -> float:
    return _load().o_f16_to_f64(int(h))


def f64_to_bf16_rne(v: float) -> int:
    return int(_load().o_f64_to_bf16_rne(float(v)))


def bf16_array_to_f64(h) -> np.ndarray:
    lib = _load()
    h = np.asarray(h, dtype=np.uint16)
    return np.array([lib.o_bf16_to_f64(int(v)) for v in h.reshape(-1)], dtype=np.float64).reshape(h.shape)


# -------------------------------------------------------------------- O1/O2 --
def dequant_affine4(codes, scales, biases, rows=None) -> np.ndarray:
    codes, pc = _c(codes, np.uint32)
    scales, ps = _c(scales, np.uint16)
    biases, pb = _c(biases, np.uint16)
    N = codes.shape[0]
    K = codes.shape[1] * 8
    n0, nr = (0, N) if rows is None else rows
    w = np.empty((nr, K), dtype=np.float64)
    _check(_load().oracle_dequant_affine4(pc, ps, pb, N, K, n0, nr, w.ctypes.data_as(ctypes.c_void_p)),
           "dequant_affine4")
    return w


def dequant_q4k(blocks, rows=None) -> np.ndarray:
    """blocks: uint8 [N][K/256][144] (or [N][K/256*144])."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    N = blocks.shape[0]
    K = (blocks.size // N) // 144 * 256
    n0, nr = (0, N) if rows is None else rows
    w = np.empty((nr, K), dtype=np.float64)
    _check(_load().oracle_dequant_q4k(blocks.ctypes.data_as(ctypes.c_void_p), N, K, n0, nr,
                                      w.ctypes.data_as(ctypes.c_void_p)), "dequant_q4k")
    return w


# -------------------------------------------------------------------- O3 --
def qgemv_affine4(x, codes, scales, biases) -> np.ndarray:
    x, px = _c(x, np.uint16)
    codes, pc = _c(codes, np.uint32)
    _, ps = _c(scales, np.uint16)
    _, pb = _c(biases, np.uint16)
    M, K = x.shape
    N = codes.shape[0]
    assert codes.shape[1] * 8 == K
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_qgemv_affine4(px, pc, ps, pb, M, N, K, y.ctypes.data_as(ctypes.c_void_p)),
           "qgemv_affine4")
    return y


def dequant_affine8(codes, scales, biases) -> np.ndarray:
    """O12: the whole affine-8 matrix as fp64 [N, K]."""
    codes, pc = _c(codes, np.uint32)
    _, ps = _c(scales, np.uint16)
    _, pb = _c(biases, np.uint16)
    N, K = codes.shape[0], codes.shape[1] * 4
    w = np.empty((N, K), dtype=np.float64)
    _check(_load().oracle_dequant_affine8(pc, ps, pb, N, K, 0, N, w.ctypes.data_as(ctypes.c_void_p)),
           "dequant_affine8")
    return w


def qgemv_affine8(x, codes, scales, biases) -> np.ndarray:
    """O13: Y = X . dequant8(W)^T in fp64."""
    x, px = _c(x, np.uint16)
    codes, pc = _c(codes, np.uint32)
    _, ps = _c(scales, np.uint16)
    _, pb = _c(biases, np.uint16)
    M, K = x.shape
    N = codes.shape[0]
    assert codes.shape[1] * 4 == K
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_qgemv_affine8(px, pc, ps, pb, M, N, K, y.ctypes.data_as(ctypes.c_void_p)),
           "qgemv_affine8")
    return y


def dequant_q6k(blocks) -> np.ndarray:
    """O14: a Q6_K matrix [N, K/256, 210] bytes as fp64 [N, K]."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    N, K = blocks.shape[0], blocks.shape[1] * 256
    w = np.empty((N, K), dtype=np.float64)
    _check(_load().oracle_dequant_q6k(blocks.ctypes.data_as(ctypes.c_void_p), N, K, 0, N,
                                      w.ctypes.data_as(ctypes.c_void_p)), "dequant_q6k")
    return w


def qgemv_q6k(x, blocks) -> np.ndarray:
    """O15: Y = X . dequant_q6k(W)^T in fp64."""
    x, px = _c(x, np.uint16)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    M, K = x.shape
    N = blocks.shape[0]
    assert blocks.shape[1] * 256 == K and blocks.shape[2] == 210
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_qgemv_q6k(px, blocks.ctypes.data_as(ctypes.c_void_p), M, N, K,
                                    y.ctypes.data_as(ctypes.c_void_p)), "qgemv_q6k")
    return y


def qgemv_affine4_f64x(x, codes, scales, biases) -> np.ndarray:
    x, px = _c(x, np.float64)
    codes, pc = _c(codes, np.uint32)
    _, ps = _c(scales, np.uint16)
    _, pb = _c(biases, np.uint16)
    M, K = x.shape
    N = codes.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_qgemv_affine4_f64x(px, pc, ps, pb, M, N, K, y.ctypes.data_as(ctypes.c_void_p)),
           "qgemv_affine4_f64x")
    return y


def qgemv_q4k(x, blocks) -> np.ndarray:
    x, px = _c(x, np.uint16)
    blocks, pb = _c(blocks, np.uint8)
    M, K = x.shape
    N = blocks.shape[0]
    assert (blocks.size // N) == K // 256 * 144
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_qgemv_q4k(px, pb, M, N, K, y.ctypes.data_as(ctypes.c_void_p)), "qgemv_q4k")
    return y


# -------------------------------------------------------------------- O4-O6 --
def rmsnorm(x, gamma, eps=1e-6) -> np.ndarray:
    x, px = _c(x, np.uint16)
    _, pg = _c(gamma, np.uint16)
    M, K = x.shape
    xn = np.empty((M, K), dtype=np.float64)
    _check(_load().oracle_rmsnorm(px, pg, float(eps), M, K, xn.ctypes.data_as(ctypes.c_void_p)), "rmsnorm")
    return xn


def silu(g: float) -> float:
    return _load().oracle_silu(float(g))


def rmsnorm_gateup_swiglu(x, gamma, eps, codes_gu, scales_gu, biases_gu) -> np.ndarray:
    x, px = _c(x, np.uint16)
    _, pg = _c(gamma, np.uint16)
    codes_gu, pc = _c(codes_gu, np.uint32)
    _, ps = _c(scales_gu, np.uint16)
    _, pb = _c(biases_gu, np.uint16)
    M, K = x.shape
    I = codes_gu.shape[0] // 2
    h = np.empty((M, I), dtype=np.float64)
    _check(_load().oracle_rmsnorm_gateup_swiglu(px, pg, float(eps), pc, ps, pb, M, I, K,
                                                h.ctypes.data_as(ctypes.c_void_p)), "rmsnorm_gateup_swiglu")
    return h


def mlp_block(x, gamma, eps, codes_gu, scales_gu, biases_gu, codes_d, scales_d, biases_d) -> np.ndarray:
    x, px = _c(x, np.uint16)
    _, pg = _c(gamma, np.uint16)
    codes_gu, pc = _c(codes_gu, np.uint32)
    _, ps = _c(scales_gu, np.uint16)
    _, pb = _c(biases_gu, np.uint16)
    _, pcd = _c(codes_d, np.uint32)
    _, psd = _c(scales_d, np.uint16)
    _, pbd = _c(biases_d, np.uint16)
    M, K = x.shape
    I = codes_gu.shape[0] // 2
    y = np.empty((M, K), dtype=np.float64)
    _check(_load().oracle_mlp_block(px, pg, float(eps), pc, ps, pb, pcd, psd, pbd, M, I, K,
                                    y.ctypes.data_as(ctypes.c_void_p)), "mlp_block")
    return y


# -------------------------------------------------------------------- O7 --
def moe(x, logits, top_k, w_gu, w_down, E, D, I):
    """Returns (y fp64 [D], ids int32 [top_k], p fp64 [top_k])."""
    x, px = _c(np.asarray(x).reshape(-1), np.uint16)
    logits, pl = _c(np.asarray(logits).reshape(-1), np.float32)
    w_gu, pgu = _c(w_gu, np.uint8)
    w_down, pdn = _c(w_down, np.uint8)
    assert w_gu.size == E * 2 * I * (D // 256) * 144
    assert w_down.size == E * D * (I // 256) * 144
    y = np.empty(D, dtype=np.float64)
    ids = np.empty(top_k, dtype=np.int32)
    p = np.empty(top_k, dtype=np.float64)
    _check(_load().oracle_moe(px, pl, int(top_k), pgu, pdn, int(E), int(D), int(I),
                              y.ctypes.data_as(ctypes.c_void_p), ids.ctypes.data_as(ctypes.c_void_p),
                              p.ctypes.data_as(ctypes.c_void_p)), "moe")
    return y, ids, p


# -------------------------------------------------------------------- O8 --
def lmhead(x, codes, scales, biases, draft=None, want_logits=True):
    """Returns (logits fp64 [M,V] or None, ids int32 [M], gap fp64 [M], accepted int)."""
    x, px = _c(x, np.uint16)
    codes, pc = _c(codes, np.uint32)
    _, ps = _c(scales, np.uint16)
    _, pb = _c(biases, np.uint16)
    M, K = x.shape
    V = codes.shape[0]
    logits = np.empty((M, V), dtype=np.float64) if want_logits else None
    ids = np.empty(M, dtype=np.int32)
    gap = np.empty(M, dtype=np.float64)
    acc = np.zeros(1, dtype=np.int32)
    pd = None
    if draft is not None:
        draft, pd = _c(np.asarray(draft).reshape(-1)[:M], np.int32)
    _check(_load().oracle_lmhead(px, pc, ps, pb, M, V, K,
                                 logits.ctypes.data_as(ctypes.c_void_p) if logits is not None else None,
                                 ids.ctypes.data_as(ctypes.c_void_p), gap.ctypes.data_as(ctypes.c_void_p),
                                 pd, acc.ctypes.data_as(ctypes.c_void_p)), "lmhead")
    return logits, ids, gap, int(acc[0])


# -------------------------------------------------------------------- O9 --
def lmhead_topk(x, codes, scales, biases, k):
    """Returns (ids int32 [M,k], vals fp64 [M,k]): the k largest logits of each
    row, larger first, equal logits by lower index, NaN above every number."""
    x, px = _c(x, np.uint16)
    codes, pc = _c(codes, np.uint32)
    _, ps = _c(scales, np.uint16)
    _, pb = _c(biases, np.uint16)
    M, K = x.shape
    V = codes.shape[0]
    ids = np.empty((M, k), dtype=np.int32)
    vals = np.empty((M, k), dtype=np.float64)
    _check(_load().oracle_lmhead_topk(px, pc, ps, pb, M, V, K, int(k), ids.ctypes.data_as(ctypes.c_void_p),
                                      vals.ctypes.data_as(ctypes.c_void_p)), "lmhead_topk")
    return ids, vals


def rht(x, signs, had) -> np.ndarray:
    """O10: blockwise (1/sqrt(had)) H_had . diag(s) . x of every bf16 row; fp64 [M, K]."""
    x, px = _c(x, np.uint16)
    signs, ps = _c(signs, np.int8)
    M, K = x.shape
    xr = np.empty((M, K), dtype=np.float64)
    _check(_load().oracle_rht(px, ps, int(had), M, K, xr.ctypes.data_as(ctypes.c_void_p)), "rht")
    return xr


def qgemv_affine4_rht(x, signs, had, codes, scales, biases) -> np.ndarray:
    """O11: dequant(W) . RHT(x) in fp64."""
    x, px = _c(x, np.uint16)
    signs, psg = _c(signs, np.int8)
    codes, pc = _c(codes, np.uint32)
    _, ps = _c(scales, np.uint16)
    _, pb = _c(biases, np.uint16)
    M, K = x.shape
    N = codes.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_qgemv_affine4_rht(px, psg, int(had), pc, ps, pb, M, N, K,
                                           y.ctypes.data_as(ctypes.c_void_p)), "qgemv_affine4_rht")
    return y
