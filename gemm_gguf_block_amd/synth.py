"""Seeded synthetic inputs for the quantized GEMV / mmq path.

This module is the only code that the HIP path's callers (bench, tests) and the
CPU oracle's callers share.  It makes *inputs*: f32 tensors drawn from seeded
normals, weight matrices quantized from them into GGUF blocks, fully random
block bytes, and MoE routing tables.  It holds none of the path's arithmetic:
it never quantizes activations to Q8_1, never dequantizes and never dots.

Weight quantization here is data generation only -- the path consumes weights
that are already quantized.  The fitting rules are the plainest ones the
workload descriptions support (GGUF byte layouts, since the pages name the
types -- blazr README, "Model Formats > GGUF" -- but give no layout):

* Q8_0: per 32 values, d = amax/127, q = round(w/d).
* Q4_K: per 32-value sub-block, lo = min(0, min w), hi = max w,
  scale = (hi-lo)/15, min = -lo; d = max(scale)/63, dmin = max(min)/63;
  6-bit sc = round(scale/d), m = round(min/dmin); q = round((w + dmin*m)/(d*sc))
  clamped to [0, 15], using the fp16-rounded d and dmin.
* Q5_K: as Q4_K with 32 levels: scale = (hi-lo)/31, q clamped to [0, 31].
* Q6_K: per 16-value sub-block, scale = amax/31; d = max(scale)/127;
  int8 sc = round(scale/d); q = round(w/(d*sc)) + 32 clamped to [0, 63].
* Q4_0 / Q5_0: per 32 values, v = the value of largest magnitude (sign kept),
  d = v/-8 (Q4_0) or v/-16 (Q5_0), so that v takes the lowest code;
  q = round(w/d) + 8 (+ 16) clamped to [0, 15] ([0, 31]), from the
  fp16-rounded d.

"round" is half away from zero.  Shapes and distributions of the five
workloads (``WORKLOADS``) follow the workload descriptions: weights N(0, 0.02),
activations N(0, 1).
"""
from __future__ import annotations

import numpy as np

Q8_0_BYTES, Q8_1_BYTES, Q4_K_BYTES, Q6_K_BYTES, Q5_K_BYTES = 34, 36, 144, 210, 176
Q4_0_BYTES, Q5_0_BYTES = 18, 22
BLOCK_BYTES = {"q8_0": Q8_0_BYTES, "q8_1": Q8_1_BYTES, "q4_k": Q4_K_BYTES, "q6_k": Q6_K_BYTES, "q5_k": Q5_K_BYTES,
               "q4_0": Q4_0_BYTES, "q5_0": Q5_0_BYTES}
BLOCK_ELEMS = {"q8_0": 32, "q8_1": 32, "q4_k": 256, "q6_k": 256, "q5_k": 256, "q4_0": 32, "q5_0": 32}

# tensor ids within a workload seed
T_W, T_X, T_ROUTE, T_WDOWN = 0, 1, 2, 3

WORKLOADS = {
    # name: shape parameters, seed
    "q8_0_gemv": dict(fmt="q8_0", n=4096, k=4096, seed=1000),
    "q4_k_gemv": dict(fmt="q4_k", n=14336, k=4096, seed=1001),
    "q6_k_gemv": dict(fmt="q6_k", n=128256, k=4096, seed=1002),
    # the Llama-3-8B FFN shape in Q5_K (Q5_K_M files)
    "q5_k_gemv": dict(fmt="q5_k", n=14336, k=4096, seed=1008),
    "q4_k_mmq": dict(fmt="q4_k", m=512, n=4096, k=4096, seed=1003),
    "moe_q4_k": dict(fmt="q4_k", n_expert=128, n_ff=768, n_embd=2048, n_tok=16, top_k=8, seed=1004),
    # prefill with the other two integer-dot types: a Q6_K ffn_down of the
    # Llama-3-8B shape (Q4_K_M files keep part of ffn_down in Q6_K) and a Q8_0
    # 4096 x 4096 projection, both at 512 tokens
    "q6_k_mmq": dict(fmt="q6_k", m=512, n=4096, k=14336, seed=1005),
    "q8_0_mmq": dict(fmt="q8_0", m=512, n=4096, k=4096, seed=1006),
    "q5_k_mmq": dict(fmt="q5_k", m=512, n=4096, k=4096, seed=1009),
    # the 32-value types of Q4_0 / Q5_0 files at the Llama-3-8B FFN shape, and
    # their prefill at 512 tokens
    "q4_0_gemv": dict(fmt="q4_0", n=14336, k=4096, seed=1011),
    "q5_0_gemv": dict(fmt="q5_0", n=14336, k=4096, seed=1012),
    "q4_0_mmq": dict(fmt="q4_0", m=512, n=4096, k=4096, seed=1013),
    "q5_0_mmq": dict(fmt="q5_0", m=512, n=4096, k=4096, seed=1014),
    # the activation prologue of a 512-token prefill at hidden size 4096
    "rmsnorm_q8_1": dict(rows=512, k=4096, eps=1e-5, seed=1007),
    # the router in front of the MoE FFN above: f32 [128][2048] router, 16
    # tokens, 8 experts each
    "router_topk": dict(n_expert=128, n_embd=2048, n_tok=16, top_k=8, seed=1010),
}


def row_bytes(fmt: str, k: int) -> int:
    return (k // BLOCK_ELEMS[fmt]) * BLOCK_BYTES[fmt]


def rng(seed: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([seed, tensor])


def normal(seed: int, tensor: int, shape, std: float = 1.0) -> np.ndarray:
    x = rng(seed, tensor).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _round_away(v: np.ndarray) -> np.ndarray:
    t = np.trunc(v)
    return t + np.where(np.abs(v - t) >= 0.5, np.sign(v), 0).astype(v.dtype)


def _div(a, b):
    """a / b where b != 0, else 0 (no warnings)."""
    out = np.zeros(np.broadcast(a, b).shape, dtype=np.float32)
    np.divide(a, b, out=out, where=(b != 0))
    return out


def _f16_bytes(v: np.ndarray) -> np.ndarray:
    """float32 array [...] -> uint8 [..., 2] little-endian binary16 (RNE)."""
    return np.ascontiguousarray(v.astype(np.float16)).view(np.uint8).reshape(v.shape + (2,))


def _f16_val(v: np.ndarray) -> np.ndarray:
    return v.astype(np.float16).astype(np.float32)


# ------------------------------------------------------------ weight quantizers
def _rows_in_chunks(W, per_row_fn, out_row_bytes, chunk_rows=4096):
    n = W.shape[0]
    out = np.empty((n, out_row_bytes), np.uint8)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        out[r0:r1] = per_row_fn(np.asarray(W[r0:r1], dtype=np.float32)).reshape(r1 - r0, out_row_bytes)
    return out


def quantize_weights_q8_0(W: np.ndarray) -> np.ndarray:
    n, k = W.shape
    assert k % 32 == 0

    def conv(X):
        X = X.reshape(-1, 32)
        amax = np.abs(X).max(axis=1)
        d = amax / np.float32(127)
        q = np.clip(_round_away(_div(X, d[:, None])), -127, 127).astype(np.int8)
        blk = np.empty((X.shape[0], Q8_0_BYTES), np.uint8)
        blk[:, 0:2] = _f16_bytes(d)
        blk[:, 2:] = q.view(np.uint8)
        return blk

    return _rows_in_chunks(W, conv, row_bytes("q8_0", k))


def pack_q4_k(d16: np.ndarray, dmin16: np.ndarray, sc: np.ndarray, m: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Pack Q4_K fields into 144-byte superblocks.

    d16, dmin16: uint16 bit patterns [B]; sc, m: 6-bit ints [B][8];
    q: 4-bit codes [B][256] in element order.
    """
    B = q.shape[0]
    sc = sc.astype(np.uint8)
    m = m.astype(np.uint8)
    blk = np.zeros((B, Q4_K_BYTES), np.uint8)
    blk[:, 0:2] = d16.astype(np.uint16).view(np.uint8).reshape(B, 2)
    blk[:, 2:4] = dmin16.astype(np.uint16).view(np.uint8).reshape(B, 2)
    s = blk[:, 4:16]
    s[:, 0:4] = (sc[:, 0:4] & 63) | ((sc[:, 4:8] >> 4) << 6)
    s[:, 4:8] = (m[:, 0:4] & 63) | ((m[:, 4:8] >> 4) << 6)
    s[:, 8:12] = (sc[:, 4:8] & 15) | ((m[:, 4:8] & 15) << 4)
    qq = q.astype(np.uint8).reshape(B, 4, 2, 32)  # [group][low/high half][l]
    blk[:, 16:] = (qq[:, :, 0, :] | (qq[:, :, 1, :] << 4)).reshape(B, 128)
    return blk


def quantize_weights_q4_k(W: np.ndarray) -> np.ndarray:
    n, k = W.shape
    assert k % 256 == 0

    def conv(X):
        X = X.reshape(-1, 8, 32)
        lo = np.minimum(X.min(axis=2), 0)
        hi = X.max(axis=2)
        scale = (hi - lo) / np.float32(15)
        minv = -lo
        d = scale.max(axis=1) / np.float32(63)
        dmin = minv.max(axis=1) / np.float32(63)
        sc = np.clip(_round_away(_div(scale, d[:, None])), 0, 63)
        m = np.clip(_round_away(_div(minv, dmin[:, None])), 0, 63)
        eff = _f16_val(d)[:, None] * sc
        mm = _f16_val(dmin)[:, None] * m
        q = np.clip(_round_away(_div(X + mm[:, :, None], eff[:, :, None])), 0, 15)
        return pack_q4_k(d.astype(np.float16).view(np.uint16), dmin.astype(np.float16).view(np.uint16),
                         sc.astype(np.int32), m.astype(np.int32), q.reshape(-1, 256).astype(np.int32))

    return _rows_in_chunks(W, conv, row_bytes("q4_k", k))


def pack_q5_k(d16: np.ndarray, dmin16: np.ndarray, sc: np.ndarray, m: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Pack Q5_K fields into 176-byte superblocks: Q4_K's 16-byte header, then
    qh[32] (bit j of qh[l] = fifth bit of element 32j + l), then the low
    nibbles packed as Q4_K's qs.  q: 5-bit codes [B][256] in element order."""
    q = q.astype(np.int32)
    p4 = pack_q4_k(d16, dmin16, sc, m, q & 15)
    B = q.shape[0]
    hb = ((q >> 4) & 1).reshape(B, 8, 32).astype(np.uint8)  # [sub-block j][l]
    qh = np.zeros((B, 32), np.uint8)
    for j in range(8):
        qh |= hb[:, j, :] << j
    blk = np.empty((B, Q5_K_BYTES), np.uint8)
    blk[:, 0:16] = p4[:, 0:16]
    blk[:, 16:48] = qh
    blk[:, 48:] = p4[:, 16:]
    return blk


def quantize_weights_q5_k(W: np.ndarray) -> np.ndarray:
    n, k = W.shape
    assert k % 256 == 0

    def conv(X):
        X = X.reshape(-1, 8, 32)
        lo = np.minimum(X.min(axis=2), 0)
        hi = X.max(axis=2)
        scale = (hi - lo) / np.float32(31)
        minv = -lo
        d = scale.max(axis=1) / np.float32(63)
        dmin = minv.max(axis=1) / np.float32(63)
        sc = np.clip(_round_away(_div(scale, d[:, None])), 0, 63)
        m = np.clip(_round_away(_div(minv, dmin[:, None])), 0, 63)
        eff = _f16_val(d)[:, None] * sc
        mm = _f16_val(dmin)[:, None] * m
        q = np.clip(_round_away(_div(X + mm[:, :, None], eff[:, :, None])), 0, 31)
        return pack_q5_k(d.astype(np.float16).view(np.uint16), dmin.astype(np.float16).view(np.uint16),
                         sc.astype(np.int32), m.astype(np.int32), q.reshape(-1, 256).astype(np.int32))

    return _rows_in_chunks(W, conv, row_bytes("q5_k", k))


def pack_q6_k(d16: np.ndarray, sc: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Pack Q6_K fields into 210-byte superblocks.

    d16: uint16 bit patterns [B]; sc: int8 scales [B][16]; q: 6-bit codes
    [B][256] in element order (element 128h + 32g + l).
    """
    B = q.shape[0]
    q = q.astype(np.uint8).reshape(B, 2, 4, 32)  # [h][g][l]
    blk = np.zeros((B, Q6_K_BYTES), np.uint8)
    ql = blk[:, 0:128].reshape(B, 2, 2, 32)  # [h][which 32-byte run][l]
    ql[:, :, 0, :] = (q[:, :, 0, :] & 15) | ((q[:, :, 2, :] & 15) << 4)
    ql[:, :, 1, :] = (q[:, :, 1, :] & 15) | ((q[:, :, 3, :] & 15) << 4)
    qh = blk[:, 128:192].reshape(B, 2, 32)
    qh[:] = ((q[:, :, 0, :] >> 4) | ((q[:, :, 1, :] >> 4) << 2) |
             ((q[:, :, 2, :] >> 4) << 4) | ((q[:, :, 3, :] >> 4) << 6))
    blk[:, 192:208] = sc.astype(np.int8).view(np.uint8)
    blk[:, 208:210] = d16.astype(np.uint16).view(np.uint8).reshape(B, 2)
    return blk


def quantize_weights_q6_k(W: np.ndarray) -> np.ndarray:
    n, k = W.shape
    assert k % 256 == 0

    def conv(X):
        X = X.reshape(-1, 16, 16)
        amax = np.abs(X).max(axis=2)
        scale = amax / np.float32(31)
        d = scale.max(axis=1) / np.float32(127)
        sc = np.clip(_round_away(_div(scale, d[:, None])), 0, 127)
        eff = _f16_val(d)[:, None] * sc
        q = np.clip(_round_away(_div(X, eff[:, :, None])) + 32, 0, 63)
        return pack_q6_k(d.astype(np.float16).view(np.uint16), sc.astype(np.int32),
                         q.reshape(-1, 256).astype(np.int32))

    return _rows_in_chunks(W, conv, row_bytes("q6_k", k))


def pack_q4_0(d16: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Pack Q4_0 fields into 18-byte blocks: d16 [nb] fp16 bits, q [nb][32]
    codes 0..15; byte 2 + j holds q[j] (low nibble) and q[j + 16] (high)."""
    q = np.asarray(q, dtype=np.int64)
    nb = q.shape[0]
    blk = np.zeros((nb, Q4_0_BYTES), np.uint8)
    blk[:, 0:2] = np.asarray(d16, np.uint16).reshape(nb).view(np.uint8).reshape(nb, 2)
    blk[:, 2:18] = ((q[:, :16] & 15) | ((q[:, 16:] & 15) << 4)).astype(np.uint8)
    return blk


def pack_q5_0(d16: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Pack Q5_0 fields into 22-byte blocks: d16 [nb] fp16 bits, q [nb][32]
    codes 0..31; bytes 2..5 hold the fifth bits (bit i of that little-endian
    word for q[i]), bytes 6..21 the low nibbles as in Q4_0."""
    q = np.asarray(q, dtype=np.int64)
    nb = q.shape[0]
    blk = np.zeros((nb, Q5_0_BYTES), np.uint8)
    blk[:, 0:2] = np.asarray(d16, np.uint16).reshape(nb).view(np.uint8).reshape(nb, 2)
    qh = (((q >> 4) & 1) << np.arange(32, dtype=np.int64)[None, :]).sum(axis=1).astype(np.uint32)
    blk[:, 2:6] = qh.astype("<u4").view(np.uint8).reshape(nb, 4)
    blk[:, 6:22] = ((q[:, :16] & 15) | ((q[:, 16:] & 15) << 4)).astype(np.uint8)
    return blk


def _quantize_weights_legacy(W: np.ndarray, bits: int) -> np.ndarray:
    n, k = W.shape
    assert k % 32 == 0
    half = 1 << (bits - 1)
    fmt = "q4_0" if bits == 4 else "q5_0"

    def conv(X):
        X = X.reshape(-1, 32)
        v = X[np.arange(X.shape[0]), np.abs(X).argmax(axis=1)]
        d = _f16_val(v / np.float32(-half))
        q = np.clip(_round_away(_div(X, d[:, None])) + half, 0, 2 * half - 1)
        pack = pack_q4_0 if bits == 4 else pack_q5_0
        return pack(d.astype(np.float16).view(np.uint16), q.astype(np.int64))

    return _rows_in_chunks(W, conv, row_bytes(fmt, k))


def quantize_weights_q4_0(W: np.ndarray) -> np.ndarray:
    return _quantize_weights_legacy(W, 4)


def quantize_weights_q5_0(W: np.ndarray) -> np.ndarray:
    return _quantize_weights_legacy(W, 5)


QUANTIZE_WEIGHTS = {"q8_0": quantize_weights_q8_0, "q4_k": quantize_weights_q4_k, "q6_k": quantize_weights_q6_k,
                    "q5_k": quantize_weights_q5_k, "q4_0": quantize_weights_q4_0, "q5_0": quantize_weights_q5_0}


def weights(fmt: str, n: int, k: int, seed: int, tensor: int = T_W, std: float = 0.02,
            chunk_rows: int = 4096, threads: int = 0) -> np.ndarray:
    """N(0, std) f32 [n][k] quantized to `fmt`.  Row chunks are drawn in order
    from one generator (the values equal one [n][k] draw) and quantized in a
    thread pool; the result does not depend on the thread count."""
    import concurrent.futures as cf
    import os

    g = rng(seed, tensor)
    out = np.empty((n, row_bytes(fmt, k)), np.uint8)
    workers = threads or min(16, os.cpu_count() or 1)
    conv = QUANTIZE_WEIGHTS[fmt]

    def job(r0, W):
        out[r0:r0 + W.shape[0]] = conv(W)

    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        pending = []
        for r0 in range(0, n, chunk_rows):
            r1 = min(n, r0 + chunk_rows)
            W = g.standard_normal((r1 - r0, k), dtype=np.float32)
            W *= np.float32(std)
            pending.append(ex.submit(job, r0, W))
            if len(pending) >= 2 * workers:  # bound the chunks held in memory
                pending.pop(0).result()
        for f in pending:
            f.result()
    return out


# ------------------------------------------------------------ random block bytes
def random_f16_bits(g: np.random.Generator, size, lo_exp: int = -24, hi_exp: int = 15) -> np.ndarray:
    """Random finite binary16 bit patterns (either sign, exponents within range)."""
    x = g.uniform(0.5, 1.0, size) * np.exp2(g.integers(lo_exp, hi_exp + 1, size))
    x *= np.where(g.integers(0, 2, size) == 0, 1.0, -1.0)
    h = x.astype(np.float16)
    h[~np.isfinite(h)] = np.float16(1.0)
    return h.view(np.uint16)


def random_blocks(fmt: str, rows: int, k: int, seed: int, tensor: int = T_W,
                  lo_exp: int = -20, hi_exp: int = 4) -> np.ndarray:
    """Uniformly random block bytes with every fp16 field set to a random finite
    value (exponents 2^lo_exp..2^hi_exp, either sign, subnormals included)."""
    g = rng(seed, tensor)
    nb = k // BLOCK_ELEMS[fmt]
    blk = g.integers(0, 256, (rows * nb, BLOCK_BYTES[fmt]), dtype=np.uint8)
    offs = {"q8_0": [0], "q8_1": [0, 2], "q4_k": [0, 2], "q6_k": [208], "q5_k": [0, 2], "q4_0": [0],
            "q5_0": [0]}[fmt]
    for o in offs:
        bits = random_f16_bits(g, rows * nb, lo_exp, hi_exp)
        blk[:, o:o + 2] = bits.view(np.uint8).reshape(-1, 2)
    return blk.reshape(rows, nb * BLOCK_BYTES[fmt])


# ---------------------------------------------------------------------- routing
def routing(seed: int, n_tok: int, n_expert: int, top_k: int):
    """Per token: top_k distinct experts drawn uniformly without replacement,
    and softmax weights over top_k N(0,1) logits (selection ignores logits)."""
    g = rng(seed, T_ROUTE)
    ids = np.empty((n_tok, top_k), np.int32)
    w = np.empty((n_tok, top_k), np.float32)
    for t in range(n_tok):
        ids[t] = g.choice(n_expert, top_k, replace=False)
        logits = g.standard_normal(top_k)
        e = np.exp(logits - logits.max())
        w[t] = (e / e.sum()).astype(np.float32)
    return ids, w


# ------------------------------------------------------------ whole workloads
def workload(name: str, **override):
    """Inputs of one named workload as numpy arrays (host memory)."""
    p = dict(WORKLOADS[name])
    p.update(override)
    seed = p["seed"]
    if name.endswith("_gemv"):
        return dict(p, w=weights(p["fmt"], p["n"], p["k"], seed),
                    x=normal(seed, T_X, (p["k"],)))
    if name.endswith("_mmq"):
        return dict(p, w=weights(p["fmt"], p["n"], p["k"], seed),
                    a=normal(seed, T_X, (p["m"], p["k"])))
    if name == "moe_q4_k":
        E, F, H = p["n_expert"], p["n_ff"], p["n_embd"]
        w_gu = weights("q4_k", E * 2 * F, H, seed, T_W)
        w_dn = weights("q4_k", E * H, F, seed, T_WDOWN)
        ids, rw = routing(seed, p["n_tok"], E, p["top_k"])
        return dict(p, w_gu=w_gu.reshape(E, -1), w_down=w_dn.reshape(E, -1),
                    x=normal(seed, T_X, (p["n_tok"], H)), ids=ids, weights=rw)
    if name == "router_topk":
        E, H, T = p["n_expert"], p["n_embd"], p["n_tok"]
        return dict(p, w_router=normal(seed, T_W, (E, H), std=0.02), x=normal(seed, T_X, (T, H)))
    raise KeyError(name)
