"""CPU oracle for the quantized GEMV / mmq path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's ``cpu_baseline`` leg may import
this package.  The product path (``gemm_gguf_block_amd``) never touches it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over
output rows).  This module builds it with gcc and marshals numpy arrays.
Every function follows a plain definition: dequantize both operands exactly to
double, then dot (see the header comment of ``oracle.c`` for the formats).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q8_0_BYTES, Q8_1_BYTES, Q4_K_BYTES, Q6_K_BYTES, Q5_K_BYTES = 34, 36, 144, 210, 176
Q4_0_BYTES, Q5_0_BYTES = 18, 22
FMT_CODE = {"q8_0": 0, "q4_k": 1, "q6_k": 2, "q5_k": 3, "q4_0": 4, "q5_0": 5}


def build() -> str:
    """Compile oracle.c into liboracle.so (no fast-math, no FP contraction)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int64


def _declare(L):
    L.orc_set_threads.restype = None
    L.orc_set_threads.argtypes = [ctypes.c_int]
    L.orc_max_threads.restype = ctypes.c_int
    L.orc_max_threads.argtypes = []
    L.orc_f16_to_f32.restype = ctypes.c_float
    L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.orc_f32_to_f16.restype = ctypes.c_uint16
    L.orc_f32_to_f16.argtypes = [ctypes.c_float]
    for name, args in {
        "orc_f16_to_f32_n": [_P, _P, _I],
        "orc_f32_to_f16_n": [_P, _P, _I],
        "orc_quantize_q8_1": [_P, _P, _I, _I],
        "orc_rms_scale": [_P, _P, _I, _I, ctypes.c_double],
        "orc_unpack_q4_k": [_P, _P, _P, _P, _P, _P],
        "orc_unpack_q5_k": [_P, _P, _P, _P, _P, _P],
        "orc_unpack_q6_k": [_P, _P, _P, _P],
        "orc_unpack_q4_0": [_P, _P, _P],
        "orc_unpack_q5_0": [_P, _P, _P],
        "orc_dequant_q4_0": [_P, _P, _I, _I],
        "orc_dequant_q5_0": [_P, _P, _I, _I],
        "orc_qgemv_q4_0": [_P, _P, _P, _I, _I, _P, _I],
        "orc_qgemv_q5_0": [_P, _P, _P, _I, _I, _P, _I],
        "orc_blockdots_q4_0": [_P, _P, _P, _I, _I],
        "orc_blockdots_q5_0": [_P, _P, _P, _I, _I],
        "orc_qgemm_q4_0": [_P, _P, _P, _I, _I, _I, _P, _I],
        "orc_qgemm_q5_0": [_P, _P, _P, _I, _I, _I, _P, _I],
        "orc_blockdots_q4_0_mmq": [_P, _P, _P, _I, _I, _I],
        "orc_blockdots_q5_0_mmq": [_P, _P, _P, _I, _I, _I],
        "orc_dequant_q8_0": [_P, _P, _I, _I],
        "orc_dequant_q8_1": [_P, _P, _I, _I],
        "orc_dequant_q4_k": [_P, _P, _I, _I],
        "orc_dequant_q5_k": [_P, _P, _I, _I],
        "orc_dequant_q6_k": [_P, _P, _I, _I],
        "orc_qgemv_q8_0": [_P, _P, _P, _I, _I, _P, _I],
        "orc_qgemv_q4_k": [_P, _P, _P, _I, _I, _P, _I],
        "orc_qgemv_q5_k": [_P, _P, _P, _I, _I, _P, _I],
        "orc_qgemv_q6_k": [_P, _P, _P, _I, _I, _P, _I],
        "orc_blockdots_q8_0": [_P, _P, _P, _I, _I],
        "orc_blockdots_q4_k": [_P, _P, _P, _P, _I, _I],
        "orc_blockdots_q5_k": [_P, _P, _P, _P, _I, _I],
        "orc_blockdots_q6_k": [_P, _P, _P, _I, _I],
        "orc_qgemv_factored": [ctypes.c_int, _P, _P, _P, _I, _I],
        "orc_qgemm_q4_k": [_P, _P, _P, _I, _I, _I, _P, _I],
        "orc_qgemm_q6_k": [_P, _P, _P, _I, _I, _I, _P, _I],
        "orc_qgemm_q5_k": [_P, _P, _P, _I, _I, _I, _P, _I],
        "orc_qgemm_q8_0": [_P, _P, _P, _I, _I, _I, _P, _I],
        "orc_blockdots_q4_k_mmq": [_P, _P, _P, _I, _I, _I],
        "orc_blockdots_q6_k_mmq": [_P, _P, _P, _I, _I, _I],
        "orc_blockdots_q5_k_mmq": [_P, _P, _P, _I, _I, _I],
        "orc_blockdots_q8_0_mmq": [_P, _P, _P, _I, _I, _I],
        "orc_moe_q4_k": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P],
        "orc_router_logits": [_P, _P, _P, _I, _I, _I],
        "orc_route_topk": [_P, _P, _P, _I, _I, _I],
    }.items():
        fn = getattr(L, name)
        fn.restype = None
        fn.argtypes = args


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- fp16 codec
def set_threads(n):
    """OpenMP threads of the oracle's routines (for the CPU-baseline timing)."""
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


def f16_bits_to_f32(bits):
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().orc_f16_to_f32_n(_ptr(bits), _ptr(out), bits.size)
    return out


def f32_to_f16_bits(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_f16_n(_ptr(x), _ptr(out), x.size)
    return out


# ------------------------------------------------------------------ quantize
def quantize_q8_1(x):
    """f32 [rows][k] (k % 32 == 0) -> Q8_1 bytes [rows][k/32*36]."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, k = x.shape
    out = np.empty((rows, (k // 32) * Q8_1_BYTES), np.uint8)
    lib().orc_quantize_q8_1(_ptr(x), _ptr(out), rows, k)
    return out


def rms_scale(x, eps):
    """r = 1/sqrt(mean(x^2) + eps) per row of f32 x ([rows][k] or [k]), in double."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, k = x.shape
    r = np.empty(rows, np.float64)
    lib().orc_rms_scale(_ptr(x), _ptr(r), rows, k, float(eps))
    return r


# -------------------------------------------------------------------- decode
def unpack_q4_k(block):
    block = _c(block, np.uint8)
    d = np.zeros(1, np.float32)
    dmin = np.zeros(1, np.float32)
    sc = np.zeros(8, np.int32)
    m = np.zeros(8, np.int32)
    q = np.zeros(256, np.int32)
    lib().orc_unpack_q4_k(_ptr(block), _ptr(d), _ptr(dmin), _ptr(sc), _ptr(m), _ptr(q))
    return float(d[0]), float(dmin[0]), sc, m, q


def unpack_q5_k(block):
    """(d, dmin, sc[8], m[8], q[256]) of one Q5_K superblock, q in 0..31."""
    block = _c(block, np.uint8)
    d = np.zeros(1, np.float32)
    dmin = np.zeros(1, np.float32)
    sc = np.zeros(8, np.int32)
    m = np.zeros(8, np.int32)
    q = np.zeros(256, np.int32)
    lib().orc_unpack_q5_k(_ptr(block), _ptr(d), _ptr(dmin), _ptr(sc), _ptr(m), _ptr(q))
    return float(d[0]), float(dmin[0]), sc, m, q


def unpack_q6_k(block):
    block = _c(block, np.uint8)
    d = np.zeros(1, np.float32)
    sc = np.zeros(16, np.int32)
    q = np.zeros(256, np.int32)
    lib().orc_unpack_q6_k(_ptr(block), _ptr(d), _ptr(sc), _ptr(q))
    return float(d[0]), sc, q


def unpack_legacy(fmt, block):
    """(d, q[32]) of one Q4_0 (q in 0..15) or Q5_0 (q in 0..31) block."""
    block = _c(block, np.uint8)
    d = np.zeros(1, np.float32)
    q = np.zeros(32, np.int32)
    getattr(lib(), "orc_unpack_" + fmt)(_ptr(block), _ptr(d), _ptr(q))
    return float(d[0]), q


def dequant(fmt, w, rows, k):
    """Dequantize `rows` rows of format fmt ('q8_0','q8_1','q4_k','q5_k','q6_k',
    'q4_0','q5_0') to f64."""
    w = _c(w, np.uint8)
    out = np.empty((rows, k), np.float64)
    getattr(lib(), "orc_dequant_" + fmt)(_ptr(w), _ptr(out), rows, k)
    return out


# ---------------------------------------------------------------------- GEMV
def qgemv(fmt, w, xq, n, k, rows=None):
    """Plain-definition GEMV in double; `rows` optionally selects output rows."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    sel = None if rows is None else _c(rows, np.int64)
    cnt = n if sel is None else sel.size
    y = np.empty(cnt, np.float64)
    getattr(lib(), "orc_qgemv_" + fmt)(_ptr(w), _ptr(xq), _ptr(y), n, k, _ptr(sel),
                                       0 if sel is None else sel.size)
    return y


def blockdots(fmt, w, xq, n, k):
    """Per-block int32 dots.  q8_0, q4_0, q5_0: D[n][k/32]; q4_k, q5_k:
    (D[n][k/32], S[k/32]); q6_k: D[n][k/16]."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    if fmt in ("q8_0", "q4_0", "q5_0"):
        D = np.empty((n, k // 32), np.int32)
        getattr(lib(), "orc_blockdots_" + fmt)(_ptr(w), _ptr(xq), _ptr(D), n, k)
        return D
    if fmt in ("q4_k", "q5_k"):
        D = np.empty((n, k // 32), np.int32)
        S = np.empty(k // 32, np.int32)
        getattr(lib(), "orc_blockdots_" + fmt)(_ptr(w), _ptr(xq), _ptr(D), _ptr(S), n, k)
        return D, S
    if fmt == "q6_k":
        D = np.empty((n, k // 16), np.int32)
        lib().orc_blockdots_q6_k(_ptr(w), _ptr(xq), _ptr(D), n, k)
        return D
    raise ValueError(fmt)


def qgemv_factored(fmt, w, xq, n, k):
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    y = np.empty(n, np.float64)
    lib().orc_qgemv_factored(FMT_CODE[fmt], _ptr(w), _ptr(xq), _ptr(y), n, k)
    return y


# ----------------------------------------------------------------------- mmq
def qgemm(fmt, w, aq, m, n, k, pairs=None):
    """C[m][n] = sum_k a^[m,k] w^[n,k] in double, for fmt 'q4_k', 'q5_k', 'q6_k',
    'q8_0', 'q4_0' or 'q5_0' weights.  `pairs` (array [P][2] of (m, n)) selects entries; then a
    1-D array of P values is returned."""
    fn = getattr(lib(), "orc_qgemm_" + fmt)
    w = _c(w, np.uint8)
    aq = _c(aq, np.uint8)
    if pairs is None:
        c = np.empty((m, n), np.float64)
        fn(_ptr(w), _ptr(aq), _ptr(c), m, n, k, None, 0)
        return c
    sel = _c(pairs, np.int64).reshape(-1, 2)
    c = np.empty(sel.shape[0], np.float64)
    fn(_ptr(w), _ptr(aq), _ptr(c), m, n, k, _ptr(sel), sel.shape[0])
    return c


def qgemm_q4_k(w, aq, m, n, k, pairs=None):
    return qgemm("q4_k", w, aq, m, n, k, pairs)


def blockdots_mmq(fmt, w, aq, m, n, k):
    """[m][n][k/32] block dots (Q6_K: [m][n][k/16] sub-block dots)."""
    w = _c(w, np.uint8)
    aq = _c(aq, np.uint8)
    D = np.empty((m, n, k // (16 if fmt == "q6_k" else 32)), np.int32)
    getattr(lib(), f"orc_blockdots_{fmt}_mmq")(_ptr(w), _ptr(aq), _ptr(D), m, n, k)
    return D


def blockdots_q4_k_mmq(w, aq, m, n, k):
    return blockdots_mmq("q4_k", w, aq, m, n, k)


# -------------------------------------------------------------------- router
def router_logits(wr, x):
    """logits[t][e] = Wr[e] . x[t] in double; wr f32 [E][H], x f32 [T][H]."""
    wr = _c(wr, np.float32)
    x = _c(x, np.float32)
    E, H = wr.shape
    T = x.shape[0]
    out = np.empty((T, E), np.float64)
    lib().orc_router_logits(_ptr(wr), _ptr(x), _ptr(out), T, E, H)
    return out


def route_topk(logits, k):
    """(ids int32 [T][k], weights f64 [T][k]) from f32 logits [T][E]: the k
    largest, larger first, ties to the lower expert; softmax over those k."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().orc_route_topk(_ptr(logits), _ptr(ids), _ptr(w), T, E, k)
    return ids, w


# ----------------------------------------------------------------------- MoE
def moe_q4_k(w_gu, w_down, xq, ids, weights, n_tok, top_k, n_expert, n_ff, n_embd, hq_in=None):
    """Returns dict(out [T][H] f64, gu [P][2F] f64, hq [P][F/32*36] u8)."""
    w_gu = _c(w_gu, np.uint8)
    w_down = _c(w_down, np.uint8)
    xq = _c(xq, np.uint8)
    ids = _c(ids, np.int32)
    weights = _c(weights, np.float32)
    P = n_tok * top_k
    out = np.empty((n_tok, n_embd), np.float64)
    gu = np.empty((P, 2 * n_ff), np.float64)
    hq = np.empty((P, (n_ff // 32) * Q8_1_BYTES), np.uint8)
    hin = None if hq_in is None else _c(hq_in, np.uint8)
    lib().orc_moe_q4_k(_ptr(w_gu), _ptr(w_down), _ptr(xq), _ptr(ids), _ptr(weights),
                       n_tok, top_k, n_expert, n_ff, n_embd, _ptr(gu), _ptr(hq), _ptr(hin), _ptr(out))
    return {"out": out, "gu": gu, "hq": hq}
