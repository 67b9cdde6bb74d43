"""C-ABI checks that need no GPU: the library loads, exports every function
include/qgguf.h declares, and rejects invalid arguments before any HIP call
(no kernel is launched and no pointer is dereferenced on these paths)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgguf.h")

OK, NULL, SHAPE, ALIGN, WORKSPACE, NO_DEVICE = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:qg_status|size_t|char|int)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import gemm_gguf_block_amd as qg
    return qg.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ["quantize_q8_1", "qgemv_q8_0", "qgemv_q4_k", "qgemv_q6_k", "qgemv_q5_k", "qgemm_q4_k_mmq",
                 "qgemm_q6_k_mmq", "qgemm_q8_0_mmq", "qgemm_q5_k_mmq", "rmsnorm_quantize_q8_1", "moe_router_topk",
                 "qgemv_q8_0_batch", "qgemv_q4_k_batch", "qgemv_q6_k_batch", "qgemv_q4_0", "qgemv_q5_0",
                 "qgemm_q4_0_mmq", "qgemm_q5_0_mmq",
                 "moe_qgemv_q4_k", "moe_qgemv_q4_k_workspace_size", "qg_status_str"]:
        assert want in names


def test_library_exports_every_declared_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    # nothing else leaks out of the library
    assert exported == set(declared_functions())


def test_binding_names_match_the_header():
    import gemm_gguf_block_amd as qg
    assert set(qg.SIGNATURES) == set(declared_functions())


def test_status_strings(lib):
    import gemm_gguf_block_amd as qg
    for code in range(8):
        assert qg.status_str(code)
    assert qg.status_str(99) == "unknown status"


P = ctypes.c_void_p
A16 = P(1 << 20)       # 16-byte aligned fake device addresses: never dereferenced
A16b = P((1 << 20) + 4096)
MIS = P((1 << 20) + 4)  # 4-byte aligned only


def test_quantize_validation(lib):
    assert lib.quantize_q8_1(None, A16, 1, 32, None) == NULL
    assert lib.quantize_q8_1(A16, None, 1, 32, None) == NULL
    assert lib.quantize_q8_1(A16, A16b, 1, 33, None) == SHAPE
    assert lib.quantize_q8_1(A16, A16b, -1, 32, None) == SHAPE
    assert lib.quantize_q8_1(A16, A16b, 1, -32, None) == SHAPE
    assert lib.quantize_q8_1(MIS, A16b, 1, 32, None) == ALIGN
    assert lib.quantize_q8_1(A16, MIS, 1, 32, None) == ALIGN
    # empty problems are a no-op that never reaches the runtime
    assert lib.quantize_q8_1(A16, A16b, 0, 32, None) == OK
    assert lib.quantize_q8_1(A16, A16b, 5, 0, None) == OK


@pytest.mark.parametrize("name,kmult", [("qgemv_q8_0", 32), ("qgemv_q4_k", 256), ("qgemv_q6_k", 256),
                                        ("qgemv_q5_k", 256), ("qgemv_q4_0", 64), ("qgemv_q5_0", 64)])
def test_gemv_validation(lib, name, kmult):
    f = getattr(lib, name)
    y = P((1 << 20) + 8192)
    assert f(None, A16b, y, 4, kmult, None) == NULL
    assert f(A16, None, y, 4, kmult, None) == NULL
    assert f(A16, A16b, None, 4, kmult, None) == NULL
    assert f(A16, A16b, y, 4, kmult + 16, None) == SHAPE
    assert f(A16, A16b, y, -1, kmult, None) == SHAPE
    assert f(A16, A16b, y, 4, -kmult, None) == SHAPE
    assert f(A16, A16b, y, 1 << 31, kmult, None) == SHAPE
    assert f(A16, A16b, y, 4, kmult * (1 << 25), None) == SHAPE
    assert f(MIS, A16b, y, 4, kmult, None) == ALIGN
    assert f(A16, MIS, y, 4, kmult, None) == ALIGN
    assert f(A16, A16b, P((1 << 20) + 2), 4, kmult, None) == ALIGN
    assert f(A16, A16b, y, 0, kmult, None) == OK
    if kmult == 64:
        assert f(A16, A16b, y, 4, 96, None) == SHAPE   # an odd block count: the kernel reads block pairs


@pytest.mark.parametrize("name,kmult", [("qgemv_q8_0_batch", 32), ("qgemv_q4_k_batch", 256),
                                        ("qgemv_q6_k_batch", 256)])
def test_gemv_batch_validation(lib, name, kmult):
    f = getattr(lib, name)
    y = P((1 << 20) + 8192)
    assert f(None, A16b, y, 2, 4, kmult, None) == NULL
    assert f(A16, None, y, 2, 4, kmult, None) == NULL
    assert f(A16, A16b, None, 2, 4, kmult, None) == NULL
    assert f(A16, A16b, y, 9, 4, kmult, None) == SHAPE      # more than 8 activation rows
    assert f(A16, A16b, y, -1, 4, kmult, None) == SHAPE
    assert f(A16, A16b, y, 2, 4, kmult + 16, None) == SHAPE
    assert f(A16, A16b, y, 2, -1, kmult, None) == SHAPE
    assert f(A16, A16b, y, 8, 1 << 29, kmult, None) == SHAPE  # b * n beyond 2^31 - 1
    assert f(A16, A16b, y, 2, 4, kmult * (1 << 25), None) == SHAPE
    assert f(MIS, A16b, y, 2, 4, kmult, None) == ALIGN
    assert f(A16, MIS, y, 2, 4, kmult, None) == ALIGN
    assert f(A16, A16b, P((1 << 20) + 2), 2, 4, kmult, None) == ALIGN
    assert f(A16, A16b, y, 0, 4, kmult, None) == OK
    assert f(A16, A16b, y, 3, 0, kmult, None) == OK


def test_mmq_validation(lib):
    c = P((1 << 20) + 8192)
    f = lib.qgemm_q4_k_mmq
    assert f(None, A16b, c, 4, 4, 256, None) == NULL
    assert f(A16, A16b, c, 4, 4, 128, None) == SHAPE
    assert f(A16, A16b, c, -4, 4, 256, None) == SHAPE
    assert f(A16, MIS, c, 4, 4, 256, None) == ALIGN
    assert f(A16, A16b, c, 0, 4, 256, None) == OK
    assert f(A16, A16b, c, 4, 0, 256, None) == OK
    # the dot dump refuses outputs it would not be asked to hold
    assert lib.qg_blockdots_q4_k_mmq(A16, A16b, c, 1 << 14, 1 << 14, 4096, None) == SHAPE


@pytest.mark.parametrize("fmt,kmult", [("q6_k", 256), ("q8_0", 32), ("q5_k", 256), ("q4_0", 32), ("q5_0", 32)])
def test_mmq_validation_other_formats(lib, fmt, kmult):
    c = P((1 << 20) + 8192)
    f = getattr(lib, f"qgemm_{fmt}_mmq")
    assert f(None, A16b, c, 4, 4, kmult, None) == NULL
    assert f(A16, A16b, c, 4, 4, kmult // 2, None) == SHAPE
    assert f(A16, A16b, c, 4, 4, kmult + kmult // 2, None) == SHAPE
    assert f(A16, A16b, c, 4, -1, kmult, None) == SHAPE
    assert f(MIS, A16b, c, 4, 4, kmult, None) == ALIGN
    assert f(A16, A16b, P((1 << 20) + 2), 4, 4, kmult, None) == ALIGN
    assert f(A16, A16b, c, 0, 4, kmult, None) == OK
    assert f(A16, A16b, c, 4, 0, kmult, None) == OK
    d = getattr(lib, f"qg_blockdots_{fmt}_mmq")
    assert d(A16, A16b, None, 4, 4, kmult, None) == NULL
    # dump limit m * n * (dots per row) <= 2^28; Q6_K has one dot per 16 values
    per = 16 if fmt == "q6_k" else 32
    assert d(A16, A16b, c, 1 << 10, 1 << 10, 256 * per, None) != SHAPE  # at the limit (then: no device here)
    assert d(A16, A16b, c, 1 << 10, 1 << 10, 512 * per, None) == SHAPE


def test_moe_validation(lib):
    T, K, E, F, H = 16, 8, 128, 768, 2048
    need = lib.moe_qgemv_q4_k_workspace_size(T, K, E, F, H)
    P_ = T * K
    assert need >= P_ * (F // 32) * 36 + P_ * 2 * F * 4 + P_ * H * 4
    assert need % 256 == 0
    ws = P(1 << 24)
    ids, wts, out = P((1 << 20) + 64), P((1 << 20) + 128), P((1 << 20) + 256)
    f = lib.moe_qgemv_q4_k

    def call(**kw):
        a = dict(wgu=A16, wdn=A16b, xq=A16, ids=ids, wts=wts, out=out, T=T, K=K, E=E, F=F, H=H, ws=ws, wsb=need)
        a.update(kw)
        return f(a["wgu"], a["wdn"], a["xq"], a["ids"], a["wts"], a["out"], a["T"], a["K"], a["E"], a["F"], a["H"],
                 a["ws"], a["wsb"], None)

    assert call(ids=None) == NULL
    assert call(ws=None) == NULL
    assert call(F=700) == SHAPE
    assert call(H=1000) == SHAPE
    assert call(K=0) == SHAPE
    assert call(E=0) == SHAPE
    assert call(T=-1) == SHAPE
    assert call(ws=P((1 << 24) + 16)) == ALIGN
    assert call(ids=P((1 << 20) + 66)) == ALIGN
    assert call(wsb=need - 1) == WORKSPACE
    assert call(T=0, wsb=0) == OK


def test_no_device_status_without_a_gpu():
    """With valid arguments and no GPU visible the call reports QG_ERR_NO_DEVICE
    (run in a child process so the HIP runtime is not initialised here)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    code = (
        "import ctypes, gemm_gguf_block_amd as qg\n"
        "L = qg.lib()\n"
        "print(L.qgemv_q4_k(ctypes.c_void_p(1<<20), ctypes.c_void_p((1<<20)+4096), "
        "ctypes.c_void_p((1<<20)+8192), 4, 256, None))\n"
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, cwd=ROOT,
                       env=dict(os.environ, HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", "")))
    assert r.returncode == 0, r.stderr
    assert int(r.stdout.strip().splitlines()[-1]) == NO_DEVICE


def test_rmsnorm_quantize_validation(lib):
    f = lib.rmsnorm_quantize_q8_1
    f.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_int64, ctypes.c_int64, P]
    xq = P((1 << 20) + 8192)
    assert f(None, A16b, 1e-5, xq, None, 2, 64, None) == NULL
    assert f(A16, None, 1e-5, xq, None, 2, 64, None) == NULL
    assert f(A16, A16b, 1e-5, None, None, 2, 64, None) == NULL
    assert f(A16, A16b, 1e-5, xq, None, 2, 48, None) == SHAPE
    assert f(A16, A16b, 1e-5, xq, None, -1, 64, None) == SHAPE
    assert f(A16, A16b, -1.0, xq, None, 2, 64, None) == SHAPE
    assert f(A16, A16b, float("nan"), xq, None, 2, 64, None) == SHAPE
    assert f(MIS, A16b, 1e-5, xq, None, 2, 64, None) == ALIGN
    assert f(A16, A16b, 1e-5, xq, P((1 << 20) + 2), 2, 64, None) == ALIGN
    assert f(A16, A16b, 1e-5, xq, None, 0, 64, None) == OK
    assert f(A16, A16b, 1e-5, xq, None, 2, 0, None) == OK


def test_router_validation(lib):
    f = lib.moe_router_topk
    o = P((1 << 20) + 8192)
    assert f(None, A16b, o, o, o, 2, 128, 2048, 8, None) == NULL
    assert f(A16, A16b, None, o, o, 2, 128, 2048, 8, None) == NULL
    assert f(A16, A16b, o, o, None, 2, 128, 2048, 8, None) == NULL       # logits are required
    assert f(A16, A16b, o, o, o, 2, 300, 2048, 8, None) == SHAPE         # more than 256 experts
    assert f(A16, A16b, o, o, o, 2, 128, 2048, 65, None) == SHAPE        # top_k above 64
    assert f(A16, A16b, o, o, o, 2, 4, 2048, 5, None) == SHAPE           # top_k above n_expert
    assert f(A16, A16b, o, o, o, 2, 128, 2050, 8, None) == SHAPE         # n_embd not a multiple of 4
    assert f(A16, A16b, o, o, o, 2, 128, 1 << 17, 8, None) == SHAPE      # n_embd above 65536
    assert f(MIS, A16b, o, o, o, 2, 128, 2048, 8, None) == ALIGN
    assert f(A16, A16b, P((1 << 20) + 2), o, o, 2, 128, 2048, 8, None) == ALIGN
    assert f(A16, A16b, o, o, P((1 << 20) + 2), 2, 128, 2048, 8, None) == ALIGN
    assert f(A16, None, None, None, None, 0, 128, 2048, 8, None) == OK    # nothing to do
