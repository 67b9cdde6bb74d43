"""Python binding of libqgguf.so -- argument marshalling only.

Every entry point has the name of its C-ABI function (declared in
``include/qgguf.h``) and takes torch tensors that live on the GPU: it checks
dtypes and sizes, passes ``data_ptr()`` values and the current HIP stream, and
raises ``QGError`` on a non-zero status.  All work runs in the HIP kernels of
libqgguf.so; there is no other code path.  If the library has not been built,
the first call raises -- there is no fallback.

The seeded input generators live in the separate module ``.synth``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgguf.so")

Q8_0_BYTES, Q8_1_BYTES, Q4_K_BYTES, Q6_K_BYTES = 34, 36, 144, 210
_BLOCK = {"q8_0": (32, Q8_0_BYTES), "q8_1": (32, Q8_1_BYTES), "q4_k": (256, Q4_K_BYTES), "q6_k": (256, Q6_K_BYTES),
          "q5_k": (256, 176), "q4_0": (32, 18), "q5_0": (32, 22)}

STATUS = {0: "QG_OK", 1: "QG_ERR_NULL", 2: "QG_ERR_SHAPE", 3: "QG_ERR_ALIGN", 4: "QG_ERR_WORKSPACE",
          5: "QG_ERR_NO_DEVICE", 6: "QG_ERR_ARCH", 7: "QG_ERR_LAUNCH"}

# C-ABI signatures: name -> argument types (restype is qg_status unless noted)
_P, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "quantize_q8_1": [_P, _P, _I, _I, _P],
    "qgemv_q8_0": [_P, _P, _P, _I, _I, _P],
    "qgemv_q4_k": [_P, _P, _P, _I, _I, _P],
    "qgemv_q6_k": [_P, _P, _P, _I, _I, _P],
    "qgemv_q5_k": [_P, _P, _P, _I, _I, _P],
    "qgemv_q4_0": [_P, _P, _P, _I, _I, _P],
    "qgemv_q5_0": [_P, _P, _P, _I, _I, _P],
    "rmsnorm_quantize_q8_1": [_P, _P, ctypes.c_float, _P, _P, _I, _I, _P],
    "qgemv_q8_0_batch": [_P, _P, _P, _I, _I, _I, _P],
    "qgemv_q4_k_batch": [_P, _P, _P, _I, _I, _I, _P],
    "qgemv_q6_k_batch": [_P, _P, _P, _I, _I, _I, _P],
    "qgemm_q8_0_mmq": [_P, _P, _P, _I, _I, _I, _P],
    "qgemm_q4_k_mmq": [_P, _P, _P, _I, _I, _I, _P],
    "qgemm_q6_k_mmq": [_P, _P, _P, _I, _I, _I, _P],
    "qgemm_q5_k_mmq": [_P, _P, _P, _I, _I, _I, _P],
    "qgemm_q4_0_mmq": [_P, _P, _P, _I, _I, _I, _P],
    "qgemm_q5_0_mmq": [_P, _P, _P, _I, _I, _I, _P],
    "moe_qgemv_q4_k_workspace_size": [_I, _I, _I, _I, _I],
    "moe_router_topk": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P],
    "moe_qgemv_q4_k": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P],
    "qg_status_str": [ctypes.c_int],
    "qg_blockdots_q8_0": [_P, _P, _P, _I, _I, _P],
    "qg_blockdots_q4_k": [_P, _P, _P, _P, _I, _I, _P],
    "qg_blockdots_q5_k": [_P, _P, _P, _P, _I, _I, _P],
    "qg_blockdots_q6_k": [_P, _P, _P, _I, _I, _P],
    "qg_blockdots_q8_0_mmq": [_P, _P, _P, _I, _I, _I, _P],
    "qg_blockdots_q4_k_mmq": [_P, _P, _P, _I, _I, _I, _P],
    "qg_blockdots_q6_k_mmq": [_P, _P, _P, _I, _I, _I, _P],
    "qg_blockdots_q5_k_mmq": [_P, _P, _P, _I, _I, _I, _P],
    "qg_blockdots_q4_0": [_P, _P, _P, _I, _I, _P],
    "qg_blockdots_q5_0": [_P, _P, _P, _I, _I, _P],
    "qg_blockdots_q4_0_mmq": [_P, _P, _P, _I, _I, _I, _P],
    "qg_blockdots_q5_0_mmq": [_P, _P, _P, _I, _I, _I, _P],
    "qg_blockdots_q8_0_batch": [_P, _P, _P, _I, _I, _I, _P],
    "qg_blockdots_q4_k_batch": [_P, _P, _P, _I, _I, _I, _P],
    "qg_blockdots_q6_k_batch": [_P, _P, _P, _I, _I, _I, _P],
    "moe_qgemv_q4_k_noalloc": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P],
    "moe_qgemv_q4_k_noalloc_max_workspace": [],
    "qg_blockdots_moe_q4_k": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P, _P, _P],
    "qg_moe_q4_k_launches": [_I, _I, _I, _I, _I],
    "qg_peak_read": [_P, _I, _P, _I, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P],
    "qg_peak_mfma_i8": [_P, _I, _I, _P, _P],
}


class QGError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({status_str(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqgguf.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python __graft_entry__.py build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_qgemv_q4_k_workspace_size.restype = ctypes.c_size_t
        L.moe_qgemv_q4_k_noalloc_max_workspace.restype = ctypes.c_size_t
        L.qg_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().qg_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise QGError(fn, status)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, nbytes: int, name: str):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")
    return t.data_ptr()


def row_bytes(fmt: str, k: int) -> int:
    e, b = _BLOCK[fmt]
    return (k // e) * b


def _empty(shape, dtype, like):
    import torch
    return torch.empty(shape, dtype=dtype, device=like.device)


# ----------------------------------------------------------------- entry points
def quantize_q8_1(x, xq=None, stream=None):
    """x: f32 [rows][k] (or [k]) -> Q8_1 bytes uint8 [rows][k/32*36]."""
    import torch
    rows, k = (1, x.shape[0]) if x.dim() == 1 else (x.shape[0], x.shape[1])
    if xq is None:
        xq = _empty((rows, row_bytes("q8_1", k)), torch.uint8, x)
    px = _need(x, torch.float32, rows * k * 4, "x")
    pq = _need(xq, torch.uint8, rows * row_bytes("q8_1", k), "xq")
    _check("quantize_q8_1", lib().quantize_q8_1(px, pq, rows, k, _stream(stream)))
    return xq


def _gemv(fmt, w, xq, n, k, y, stream):
    import torch
    if y is None:
        y = _empty((n,), torch.float32, w)
    pw = _need(w, torch.uint8, n * row_bytes(fmt, k), "w")
    pq = _need(xq, torch.uint8, row_bytes("q8_1", k), "xq")
    py = _need(y, torch.float32, n * 4, "y")
    name = "qgemv_" + fmt
    _check(name, getattr(lib(), name)(pw, pq, py, n, k, _stream(stream)))
    return y


def qgemv_q8_0(w, xq, n, k, y=None, stream=None):
    return _gemv("q8_0", w, xq, n, k, y, stream)


def qgemv_q4_k(w, xq, n, k, y=None, stream=None):
    return _gemv("q4_k", w, xq, n, k, y, stream)


def qgemv_q6_k(w, xq, n, k, y=None, stream=None):
    return _gemv("q6_k", w, xq, n, k, y, stream)


def qgemv_q5_k(w, xq, n, k, y=None, stream=None):
    return _gemv("q5_k", w, xq, n, k, y, stream)


def qgemv_q4_0(w, xq, n, k, y=None, stream=None):
    return _gemv("q4_0", w, xq, n, k, y, stream)


def qgemv_q5_0(w, xq, n, k, y=None, stream=None):
    return _gemv("q5_0", w, xq, n, k, y, stream)


def _gemv_batch(fmt, w, xq, b, n, k, y, stream):
    import torch
    if y is None:
        y = _empty((b, n), torch.float32, w)
    pw = _need(w, torch.uint8, n * row_bytes(fmt, k), "w")
    pq = _need(xq, torch.uint8, b * row_bytes("q8_1", k), "xq")
    py = _need(y, torch.float32, b * n * 4, "y")
    name = "qgemv_" + fmt + "_batch"
    _check(name, getattr(lib(), name)(pw, pq, py, b, n, k, _stream(stream)))
    return y


def qgemv_q8_0_batch(w, xq, b, n, k, y=None, stream=None):
    """b (<= 8) Q8_1 rows xq [b][k/32*36] against Q8_0 weights -> y f32 [b][n]."""
    return _gemv_batch("q8_0", w, xq, b, n, k, y, stream)


def qgemv_q4_k_batch(w, xq, b, n, k, y=None, stream=None):
    return _gemv_batch("q4_k", w, xq, b, n, k, y, stream)


def qgemv_q6_k_batch(w, xq, b, n, k, y=None, stream=None):
    return _gemv_batch("q6_k", w, xq, b, n, k, y, stream)


def rmsnorm_quantize_q8_1(x, gamma, eps, xq=None, r=None, stream=None):
    """x: f32 [rows][k] (or [k]) -> Q8_1 bytes of (x * r) * gamma per row, with
    r = 1/sqrt(mean(x^2) + eps).  Returns (xq, r) when r (f32 [rows]) is given,
    else xq."""
    import torch
    rows, k = (1, x.shape[0]) if x.dim() == 1 else (x.shape[0], x.shape[1])
    if xq is None:
        xq = _empty((rows, row_bytes("q8_1", k)), torch.uint8, x)
    px = _need(x, torch.float32, rows * k * 4, "x")
    pg = _need(gamma, torch.float32, k * 4, "gamma")
    pq = _need(xq, torch.uint8, rows * row_bytes("q8_1", k), "xq")
    pr = None if r is None else _need(r, torch.float32, rows * 4, "r")
    _check("rmsnorm_quantize_q8_1", lib().rmsnorm_quantize_q8_1(px, pg, float(eps), pq, pr, rows, k,
                                                                 _stream(stream)))
    return xq if r is None else (xq, r)


def _mmq(fmt, w, aq, m, n, k, c, stream):
    import torch
    if c is None:
        c = _empty((m, n), torch.float32, w)
    pw = _need(w, torch.uint8, n * row_bytes(fmt, k), "w")
    pa = _need(aq, torch.uint8, m * row_bytes("q8_1", k), "aq")
    pc = _need(c, torch.float32, m * n * 4, "c")
    name = f"qgemm_{fmt}_mmq"
    _check(name, getattr(lib(), name)(pw, pa, pc, m, n, k, _stream(stream)))
    return c


def qgemm_q4_k_mmq(w, aq, m, n, k, c=None, stream=None):
    return _mmq("q4_k", w, aq, m, n, k, c, stream)


def qgemm_q6_k_mmq(w, aq, m, n, k, c=None, stream=None):
    return _mmq("q6_k", w, aq, m, n, k, c, stream)


def qgemm_q8_0_mmq(w, aq, m, n, k, c=None, stream=None):
    return _mmq("q8_0", w, aq, m, n, k, c, stream)


def qgemm_q5_k_mmq(w, aq, m, n, k, c=None, stream=None):
    return _mmq("q5_k", w, aq, m, n, k, c, stream)


def qgemm_q4_0_mmq(w, aq, m, n, k, c=None, stream=None):
    return _mmq("q4_0", w, aq, m, n, k, c, stream)


def qgemm_q5_0_mmq(w, aq, m, n, k, c=None, stream=None):
    return _mmq("q5_0", w, aq, m, n, k, c, stream)


def moe_router_topk(w_router, x, top_k, ids=None, weights=None, logits=None, stream=None):
    """(ids int32 [T][top_k], weights f32 [T][top_k]) for x f32 [T][H] and the
    router f32 [E][H]; the logits (f32 [T][E]) are written to `logits`, which is
    allocated when not given."""
    import torch
    E, H = w_router.shape
    T = x.shape[0]
    if ids is None:
        ids = _empty((T, top_k), torch.int32, x)
    if weights is None:
        weights = _empty((T, top_k), torch.float32, x)
    if logits is None:
        logits = _empty((T, E), torch.float32, x)
    pl = _need(logits, torch.float32, T * E * 4, "logits")
    _check("moe_router_topk", lib().moe_router_topk(
        _need(w_router, torch.float32, E * H * 4, "w_router"), _need(x, torch.float32, T * H * 4, "x"),
        _need(ids, torch.int32, T * top_k * 4, "ids"), _need(weights, torch.float32, T * top_k * 4, "weights"),
        pl, T, E, H, top_k, _stream(stream)))
    return ids, weights


def moe_qgemv_q4_k_workspace_size(n_tok, top_k, n_expert, n_ff, n_embd) -> int:
    return int(lib().moe_qgemv_q4_k_workspace_size(n_tok, top_k, n_expert, n_ff, n_embd))


def moe_qgemv_q4_k(w_gate_up, w_down, xq, ids, weights, n_tok, top_k, n_expert, n_ff, n_embd,
                   out=None, workspace=None, stream=None):
    import torch
    ws_bytes = moe_qgemv_q4_k_workspace_size(n_tok, top_k, n_expert, n_ff, n_embd)
    if out is None:
        out = _empty((n_tok, n_embd), torch.float32, xq)
    if workspace is None:
        workspace = _empty((max(ws_bytes, 1),), torch.uint8, xq)
    pgu = _need(w_gate_up, torch.uint8, n_expert * 2 * n_ff * row_bytes("q4_k", n_embd), "w_gate_up")
    pdn = _need(w_down, torch.uint8, n_expert * n_embd * row_bytes("q4_k", n_ff), "w_down")
    pq = _need(xq, torch.uint8, n_tok * row_bytes("q8_1", n_embd), "xq")
    pid = _need(ids, torch.int32, n_tok * top_k * 4, "ids")
    pwt = _need(weights, torch.float32, n_tok * top_k * 4, "weights")
    po = _need(out, torch.float32, n_tok * n_embd * 4, "out")
    pws = _need(workspace, torch.uint8, ws_bytes, "workspace")
    _check("moe_qgemv_q4_k", lib().moe_qgemv_q4_k(pgu, pdn, pq, pid, pwt, po, n_tok, top_k, n_expert, n_ff, n_embd,
                                                  pws, workspace.numel(), _stream(stream)))
    return out


def moe_qgemv_q4_k_noalloc(w_gate_up, w_down, xq, ids, weights, n_tok, top_k, n_expert, n_ff, n_embd, out=None,
                           stream=None):
    """moe_qgemv_q4_k on the library's own per-GPU workspace: no allocation
    beyond `out` (none when `out` is given)."""
    import torch
    if out is None:
        out = _empty((n_tok, n_embd), torch.float32, xq)
    pgu = _need(w_gate_up, torch.uint8, n_expert * 2 * n_ff * row_bytes("q4_k", n_embd), "w_gate_up")
    pdn = _need(w_down, torch.uint8, n_expert * n_embd * row_bytes("q4_k", n_ff), "w_down")
    pq = _need(xq, torch.uint8, n_tok * row_bytes("q8_1", n_embd), "xq")
    pid = _need(ids, torch.int32, n_tok * top_k * 4, "ids")
    pwt = _need(weights, torch.float32, n_tok * top_k * 4, "weights")
    po = _need(out, torch.float32, n_tok * n_embd * 4, "out")
    _check("moe_qgemv_q4_k_noalloc", lib().moe_qgemv_q4_k_noalloc(pgu, pdn, pq, pid, pwt, po, n_tok, top_k, n_expert,
                                                                  n_ff, n_embd, _stream(stream)))
    return out


def moe_qgemv_q4_k_noalloc_max_workspace() -> int:
    return int(lib().moe_qgemv_q4_k_noalloc_max_workspace())


def moe_workspace_regions(workspace, n_tok, top_k, n_ff, n_embd):
    """Views of the first three MoE workspace regions: (h^ Q8_1 [P][n_ff/32*36]
    uint8, g|u f32 [P][2*n_ff], weighted down f32 [P][n_embd]) -- the
    documented layout."""
    import torch

    def up(v):
        return (v + 255) & ~255

    P = n_tok * top_k
    hq_bytes = P * row_bytes("q8_1", n_ff)
    gu_off = up(hq_bytes)
    z_off = gu_off + up(P * 2 * n_ff * 4)
    hq = workspace[:hq_bytes].view(P, row_bytes("q8_1", n_ff))
    gu = workspace[gu_off:gu_off + P * 2 * n_ff * 4].view(torch.float32).view(P, 2 * n_ff)
    z = workspace[z_off:z_off + P * n_embd * 4].view(torch.float32).view(P, n_embd)
    return hq, gu, z


# ------------------------------------------------------- per-block dots (tests)
def _blockdots_32(fmt, w, xq, n, k, stream):
    import torch
    D = _empty((n, k // 32), torch.int32, w)
    name = f"qg_blockdots_{fmt}"
    _check(name, getattr(lib(), name)(
        _need(w, torch.uint8, n * row_bytes(fmt, k), "w"), _need(xq, torch.uint8, row_bytes("q8_1", k), "xq"),
        _need(D, torch.int32, D.numel() * 4, "D"), n, k, _stream(stream)))
    return D


def blockdots_q8_0(w, xq, n, k, stream=None):
    return _blockdots_32("q8_0", w, xq, n, k, stream)


def blockdots_q4_0(w, xq, n, k, stream=None):
    return _blockdots_32("q4_0", w, xq, n, k, stream)


def blockdots_q5_0(w, xq, n, k, stream=None):
    return _blockdots_32("q5_0", w, xq, n, k, stream)


def _blockdots_kmin(fmt, w, xq, n, k, stream):
    import torch
    D = _empty((n, k // 32), torch.int32, w)
    S = _empty((k // 32,), torch.int32, w)
    name = f"qg_blockdots_{fmt}"
    _check(name, getattr(lib(), name)(
        _need(w, torch.uint8, n * row_bytes(fmt, k), "w"), _need(xq, torch.uint8, row_bytes("q8_1", k), "xq"),
        _need(D, torch.int32, D.numel() * 4, "D"), _need(S, torch.int32, S.numel() * 4, "S"), n, k,
        _stream(stream)))
    return D, S


def blockdots_q4_k(w, xq, n, k, stream=None):
    return _blockdots_kmin("q4_k", w, xq, n, k, stream)


def blockdots_q5_k(w, xq, n, k, stream=None):
    return _blockdots_kmin("q5_k", w, xq, n, k, stream)


def blockdots_q6_k(w, xq, n, k, stream=None):
    import torch
    D = _empty((n, k // 16), torch.int32, w)
    _check("qg_blockdots_q6_k", lib().qg_blockdots_q6_k(
        _need(w, torch.uint8, n * row_bytes("q6_k", k), "w"), _need(xq, torch.uint8, row_bytes("q8_1", k), "xq"),
        _need(D, torch.int32, D.numel() * 4, "D"), n, k, _stream(stream)))
    return D


def _blockdots_mmq(fmt, w, aq, m, n, k, stream):
    import torch
    D = _empty((m, n, k // (16 if fmt == "q6_k" else 32)), torch.int32, w)
    name = f"qg_blockdots_{fmt}_mmq"
    _check(name, getattr(lib(), name)(
        _need(w, torch.uint8, n * row_bytes(fmt, k), "w"), _need(aq, torch.uint8, m * row_bytes("q8_1", k), "aq"),
        _need(D, torch.int32, D.numel() * 4, "D"), m, n, k, _stream(stream)))
    return D


def blockdots_q4_k_mmq(w, aq, m, n, k, stream=None):
    return _blockdots_mmq("q4_k", w, aq, m, n, k, stream)


def blockdots_q6_k_mmq(w, aq, m, n, k, stream=None):
    """[m][n][k/16]: the exact dot of every 16-value sub-block."""
    return _blockdots_mmq("q6_k", w, aq, m, n, k, stream)


def blockdots_q8_0_mmq(w, aq, m, n, k, stream=None):
    return _blockdots_mmq("q8_0", w, aq, m, n, k, stream)


def blockdots_q4_0_mmq(w, aq, m, n, k, stream=None):
    return _blockdots_mmq("q4_0", w, aq, m, n, k, stream)


def blockdots_q5_0_mmq(w, aq, m, n, k, stream=None):
    return _blockdots_mmq("q5_0", w, aq, m, n, k, stream)


def blockdots_q5_k_mmq(w, aq, m, n, k, stream=None):
    return _blockdots_mmq("q5_k", w, aq, m, n, k, stream)


def blockdots_batch(fmt, w, xq, b, n, k, stream=None):
    """[b][n][k/32] (Q6_K: [b][n][k/16]) exact dots from the kernel that
    qgemv_<fmt>_batch runs for b rows, on its launch grid."""
    import torch
    D = _empty((b, n, k // (16 if fmt == "q6_k" else 32)), torch.int32, w)
    name = f"qg_blockdots_{fmt}_batch"
    _check(name, getattr(lib(), name)(
        _need(w, torch.uint8, n * row_bytes(fmt, k), "w"), _need(xq, torch.uint8, b * row_bytes("q8_1", k), "xq"),
        _need(D, torch.int32, D.numel() * 4, "D"), b, n, k, _stream(stream)))
    return D


# ------------------------------------------------ measurement references (bench)
def peak_read(src, grid, threads, loads, nontemporal, sink, stream=None):
    """Streaming read of every 16-byte word of the uint8 tensor src (its whole
    size, a multiple of 16); sink: uint32/int32 tensor of >= grid entries."""
    import torch
    nbytes = src.numel() * src.element_size()
    _check("qg_peak_read", lib().qg_peak_read(
        _need(src, src.dtype, nbytes, "src"), nbytes, _need(sink, sink.dtype, grid * 4, "sink"), sink.numel(),
        grid, threads, loads, int(bool(nontemporal)), _stream(stream)))


def peak_mfma_i8(iters, sink, stream=None):
    """Loop of int8 MFMAs; returns the int8 operation count of the launch.
    sink: int32 tensor of >= 8 * CUs entries."""
    import torch
    ops = ctypes.c_int64(0)
    _check("qg_peak_mfma_i8", lib().qg_peak_mfma_i8(_need(sink, torch.int32, 4, "sink"), sink.numel(), iters,
                                                    ctypes.byref(ops), _stream(stream)))
    return ops.value


def blockdots_moe_q4_k(w_gate_up, w_down, xq, ids, weights, n_tok, top_k, n_expert, n_ff, n_embd, workspace,
                       stream=None):
    """Exact dots of the MoE call's expert GEMVs, from their dump instances:
    (D_gu int32 [P][2*n_ff][n_embd/32], D_dn int32 [P][n_embd][n_ff/32]).
    The gate/up product runs first (its g|u feeds the down dump); the
    workspace then holds h^ as the product call would.  Rows of pairs with an
    out-of-range id are not written."""
    import torch
    P = n_tok * top_k
    D_gu = torch.zeros((P, 2 * n_ff, n_embd // 32), dtype=torch.int32, device=xq.device)
    D_dn = torch.zeros((P, n_embd, n_ff // 32), dtype=torch.int32, device=xq.device)
    ws_bytes = moe_qgemv_q4_k_workspace_size(n_tok, top_k, n_expert, n_ff, n_embd)
    _check("qg_blockdots_moe_q4_k", lib().qg_blockdots_moe_q4_k(
        _need(w_gate_up, torch.uint8, n_expert * 2 * n_ff * row_bytes("q4_k", n_embd), "w_gate_up"),
        _need(w_down, torch.uint8, n_expert * n_embd * row_bytes("q4_k", n_ff), "w_down"),
        _need(xq, torch.uint8, n_tok * row_bytes("q8_1", n_embd), "xq"), _need(ids, torch.int32, P * 4, "ids"),
        _need(weights, torch.float32, P * 4, "weights"), n_tok, top_k, n_expert, n_ff, n_embd,
        _need(workspace, torch.uint8, ws_bytes, "workspace"), workspace.numel(),
        _need(D_gu, torch.int32, D_gu.numel() * 4, "D_gu"), _need(D_dn, torch.int32, D_dn.numel() * 4, "D_dn"),
        _stream(stream)))
    return D_gu, D_dn


def moe_launches(n_tok, top_k, n_expert, n_ff, n_embd) -> int:
    """Kernel launches moe_qgemv_q4_k makes for this shape (2 or 4)."""
    return int(lib().qg_moe_q4_k_launches(n_tok, top_k, n_expert, n_ff, n_embd))
