"""Seeded synthetic inputs for the decode projections.

This module is the only code shared by the GPU path's tests/bench and the CPU
oracle's tests.  It draws random numbers and stores them in the byte formats
the two sides consume; it holds none of the method's arithmetic (no dequant,
no dot products, no norm, no routing).

Recipe (one numpy PCG64 generator per seed; values drawn in fp64, then rounded
to nearest-even into bf16 / fp16):
  * activations        X ~ N(0, 1) -> bf16
  * affine-4 weights   codes: uniform random 32-bit words, i.e. every 4-bit
                       code ~ U{0..15}; scale ~ U(0.005, 0.02) -> bf16; bias
                       ~ U(-0.1, 0.1) -> bf16, one per (row, group of 64)
  * Q4_K weights       every 144-byte block is uniform random bytes (codes
                       ~ U{0..15}, 6-bit scales and mins ~ U{0..63}), then the
                       two fp16 super-scales d, dmin ~ U(1e-3, 1e-2) are written
                       over the first four bytes
  * RMSNorm gain       gamma ~ U(0.8, 1.2) -> bf16
  * verify blocks      row 0 ~ N(0,1); every element of rows 1.. copies row 0's
                       element with probability 0.9, else a fresh N(0,1) draw
  * router logits      ~ N(0, 1) fp32
  * draft ids          ~ U{0..V-1} int32
"""
from __future__ import annotations

import numpy as np

AFFINE_GROUP = 64
Q4K_BLOCK_WEIGHTS = 256
Q4K_BLOCK_BYTES = 144


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(int(seed))


def to_bf16_bits(a) -> np.ndarray:
    """fp64 values -> bf16 bit patterns (uint16), round to nearest even via fp32."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = (((u[nan] >> 16) & 0x8000) | 0x7FC0).astype(np.uint16)
    return r.reshape(np.shape(a))


def to_f16_bits(a) -> np.ndarray:
    """fp64 values -> fp16 bit patterns (uint16), numpy's round to nearest even."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float16)).view(np.uint16)


def normal_bf16(g: np.random.Generator, shape) -> np.ndarray:
    return to_bf16_bits(g.standard_normal(shape))


def uniform_bf16(g: np.random.Generator, lo: float, hi: float, shape) -> np.ndarray:
    return to_bf16_bits(g.uniform(lo, hi, shape))


def shared_rows_bf16(g: np.random.Generator, M: int, K: int, share: float = 0.9) -> np.ndarray:
    """Verify-block activations: rows 1.. copy row 0 elementwise with probability `share`."""
    x = g.standard_normal((M, K))
    copy = g.random((M, K)) < share
    copy[0, :] = True
    x = np.where(copy, x[0:1, :], x)
    return to_bf16_bits(x)


def affine4_matrix(g: np.random.Generator, N: int, K: int, s_lo=0.005, s_hi=0.02, b_lo=-0.1, b_hi=0.1):
    """Returns dict(codes uint32 [N, K/8], scales uint16 [N, K/64], biases uint16 [N, K/64])."""
    assert K % AFFINE_GROUP == 0
    codes = g.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    scales = uniform_bf16(g, s_lo, s_hi, (N, K // AFFINE_GROUP))
    biases = uniform_bf16(g, b_lo, b_hi, (N, K // AFFINE_GROUP))
    return {"codes": codes, "scales": scales, "biases": biases}


def affine8_matrix(g: np.random.Generator, N: int, K: int, s_lo=0.0003, s_hi=0.0012, b_lo=-0.1, b_hi=0.1):
    """8-bit affine weights: dict(codes uint32 [N, K/4] of uniform random bytes, scales and biases
    uint16 [N, K/64]); scales span the same weight range as the 4-bit matrices' over 255 steps."""
    assert K % AFFINE_GROUP == 0
    codes = g.integers(0, 2**32, size=(N, K // 4), dtype=np.uint64).astype(np.uint32)
    scales = uniform_bf16(g, s_lo, s_hi, (N, K // AFFINE_GROUP))
    biases = uniform_bf16(g, b_lo, b_hi, (N, K // AFFINE_GROUP))
    return {"codes": codes, "scales": scales, "biases": biases}


def single_projection8(M=1, N=3072, K=1024, seed=1006):
    """X[M,K] ~ N(0,1) bf16 and an 8-bit affine W[N,K] (group 64)."""
    g = rng(seed)
    x = normal_bf16(g, (M, K))
    return {"x": x, **affine8_matrix(g, N, K), "M": M, "N": N, "K": K, "seed": seed}


def q6k_matrix(g: np.random.Generator, N: int, K: int, d_lo=1e-3, d_hi=1e-2) -> np.ndarray:
    """Returns uint8 [N, K/256, 210] Q6_K blocks: uniform random bytes (codes and int8 scales),
    fp16 d ~ U(d_lo, d_hi) written over bytes 208..209."""
    assert K % 256 == 0
    nb = K // 256
    blocks = g.integers(0, 256, size=(N, nb, 210), dtype=np.uint8)
    d = to_f16_bits(g.uniform(d_lo, d_hi, (N, nb)))
    blocks[..., 208] = (d & 0xFF).astype(np.uint8)
    blocks[..., 209] = (d >> 8).astype(np.uint8)
    return blocks


def single_projection_q6k(M=1, N=3072, K=1024, seed=1007):
    """X[M,K] ~ N(0,1) bf16 and a Q6_K W[N,K]."""
    g = rng(seed)
    x = normal_bf16(g, (M, K))
    return {"x": x, "blocks": q6k_matrix(g, N, K), "M": M, "N": N, "K": K, "seed": seed}


def q4k_matrix(g: np.random.Generator, N: int, K: int, d_lo=1e-3, d_hi=1e-2) -> np.ndarray:
    """Returns uint8 [N, K/256, 144] Q4_K blocks."""
    assert K % Q4K_BLOCK_WEIGHTS == 0
    nb = K // Q4K_BLOCK_WEIGHTS
    blocks = g.integers(0, 256, size=(N, nb, Q4K_BLOCK_BYTES), dtype=np.uint16).astype(np.uint8)
    d = to_f16_bits(g.uniform(d_lo, d_hi, (N, nb)))
    dmin = to_f16_bits(g.uniform(d_lo, d_hi, (N, nb)))
    blocks[:, :, 0:2] = d.reshape(N, nb, 1).view(np.uint8).reshape(N, nb, 2)
    blocks[:, :, 2:4] = dmin.reshape(N, nb, 1).view(np.uint8).reshape(N, nb, 2)
    return blocks


# ------------------------------------------------------------ workloads --
# Seeds 1001..1005, one per workload.

def single_projection(M=1, N=3072, K=1024, seed=1001):
    """Qwen3-0.6B-shaped single projection: X[M,1024] x W[3072,1024] affine-4."""
    g = rng(seed)
    x = normal_bf16(g, (M, K))
    w = affine4_matrix(g, N, K)
    return {"x": x, **w, "M": M, "N": N, "K": K, "seed": seed}


def mlp_block(M=1, D=1024, I=3072, seed=1002, shared=False):
    """Fused MLP block: RMSNorm(eps 1e-6) -> gate/up [2I, D] -> SwiGLU -> down [D, I]."""
    g = rng(seed)
    x = shared_rows_bf16(g, M, D) if shared else normal_bf16(g, (M, D))
    gamma = uniform_bf16(g, 0.8, 1.2, (D,))
    gu = affine4_matrix(g, 2 * I, D)
    dn = affine4_matrix(g, D, I)
    return {"x": x, "gamma": gamma, "eps": 1e-6,
            "codes_gu": gu["codes"], "scales_gu": gu["scales"], "biases_gu": gu["biases"],
            "codes_d": dn["codes"], "scales_d": dn["scales"], "biases_d": dn["biases"],
            "M": M, "D": D, "I": I, "seed": seed}


def verify_block(M=8, D=2560, I=12800, seed=1003):
    """4B-class speculative verify block: X[8,2560] rows sharing 90% of values."""
    return mlp_block(M=M, D=D, I=I, seed=seed, shared=True)


def moe_token(E=128, D=2048, I=768, top_k=8, seed=1004, n_logit_sets=1):
    """Q4_K MoE decode token: x[1,2048], experts gate/up [2I, D] and down [D, I]."""
    g = rng(seed)
    x = normal_bf16(g, (1, D))
    w_gu = q4k_matrix(g, E * 2 * I, D).reshape(E, 2 * I, D // 256, 144)
    w_down = q4k_matrix(g, E * D, I).reshape(E, D, I // 256, 144)
    logits = g.standard_normal((n_logit_sets, E)).astype(np.float32)
    return {"x": x, "w_gu": w_gu, "w_down": w_down, "logits": logits, "E": E, "D": D, "I": I,
            "top_k": top_k, "seed": seed}


def lm_head(M=8, V=151936, K=1024, seed=1005):
    """Untied LM head: X[M,1024] x W[151936,1024] affine-4, plus 8 seeded draft ids."""
    g = rng(seed)
    x = normal_bf16(g, (M, K))
    w = affine4_matrix(g, V, K)
    draft = g.integers(0, V, size=8, dtype=np.int64).astype(np.int32)
    return {"x": x, **w, "draft": draft, "M": M, "V": V, "K": K, "seed": seed}
