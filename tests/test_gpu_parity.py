"""GPU parity: every HIP entry point against the CPU oracle on the same seeded
inputs.  Q8_1 bytes and per-block int32 dots must match exactly; f32 outputs
within REL_TOL under the max(|r|, rms(r))-floored relative metric."""
from fractions import Fraction

import numpy as np
import pytest

from _util import REL_TOL, read_golden, rel_err
from gemm_gguf_block_amd import synth

pytestmark = pytest.mark.gpu

GEMV = {"q8_0": "qgemv_q8_0", "q4_k": "qgemv_q4_k", "q6_k": "qgemv_q6_k", "q5_k": "qgemv_q5_k", "q4_0": "qgemv_q4_0",
        "q5_0": "qgemv_q5_0"}
ALL_GEMV = list(GEMV)


@pytest.fixture(scope="module")
def env():
    import torch

    import gemm_gguf_block_amd as qg
    import oracle
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    return qg, oracle, torch, dev


def _gpu(torch, dev, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ------------------------------------------------------------------- quantize
def test_quantize_q8_1_hand_vectors(env):
    qg, orc, torch, dev = env
    fx = read_golden("q8_1_vectors.txt")
    for xs, bs in zip(fx["x"], fx["bytes"]):
        x = np.array([float.fromhex(t) for t in xs.split()], np.float32)
        got = _host(qg.quantize_q8_1(_gpu(torch, dev, x)))
        assert got.tobytes() == bytes.fromhex(bs)


# A block whose s = d*sum(q) (d = fl(2.4586923/127), sum = 729) is an fp32
# product that sits exactly on a binary16 tie: rounding it to fp32 first and
# then to fp16 gives 14.11, one fused rounding would give 14.12.
DOUBLE_ROUNDING_BLOCK = ("0x1.3ab66ep+1 " + " ".join(["0x1.78a9f8p-2"] * 5) + " " +
                         " ".join(["0x1.8c7d04p-2", "0x1.78a9f8p-2"] * 13))


def test_quantize_q8_1_s_rounds_the_fp32_product(env):
    qg, orc, torch, dev = env
    x = np.array([float.fromhex(t) for t in DOUBLE_ROUNDING_BLOCK.split()], np.float32)
    assert x.size == 32
    got = _host(qg.quantize_q8_1(_gpu(torch, dev, x)))[0]
    want = orc.quantize_q8_1(x[None])[0]
    q = want[4:].view(np.int8).astype(np.int64)
    d = np.float32(np.abs(x).max() / np.float32(127))
    assert q.sum() == 729
    s16 = np.float32(d * np.float32(q.sum())).astype(np.float16)
    assert want[2:4].copy().view(np.float16)[0] == s16
    assert np.array_equal(got, want)


@pytest.mark.parametrize("rows,k,scale", [(1, 32, 1.0), (1, 4096, 1.0), (3, 768, 1.0), (7, 4096, 1e-6),
                                          (5, 2048, 3e4), (33, 96, 1.0), (512, 4096, 1.0), (16, 2048, 1.0)])
def test_quantize_q8_1_bytes_exact(env, rows, k, scale):
    qg, orc, torch, dev = env
    x = synth.normal(300 + rows, 1, (rows, k), std=scale)
    x[0, :32] = 0.0                       # an all-zero block
    if k >= 64:
        x[-1, 32:64] = np.float32(1e-30)  # amax far below binary16 range
    got = _host(qg.quantize_q8_1(_gpu(torch, dev, x)))
    want = orc.quantize_q8_1(x)
    assert np.array_equal(got, want)


# ----------------------------------------------------------- GEMV block dots
# (7, 17152) and (5, 33536) span two and three of the 16384-value activation
# chunks a workgroup stages in LDS, the last one partial
SHAPES = [(1, 256), (3, 512), (65, 256), (130, 768), (257, 2048), (64, 4096), (33, 14336), (7, 17152), (5, 33536)]


@pytest.mark.parametrize("fmt", ALL_GEMV)
@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("data", ["random_bytes", "weights"])
def test_gemv_block_dots_exact(env, fmt, n, k, data):
    qg, orc, torch, dev = env
    if data == "random_bytes":
        w = synth.random_blocks(fmt, n, k, seed=n * 7 + k)
        xq = synth.random_blocks("q8_1", 1, k, seed=n + k)
    else:
        w = synth.weights(fmt, n, k, seed=n + 3 * k)
        xq = orc.quantize_q8_1(synth.normal(n + k, 1, (1, k)))
    W, X = _gpu(torch, dev, w), _gpu(torch, dev, xq)
    if fmt in ("q4_k", "q5_k"):
        D, S = getattr(qg, "blockdots_" + fmt)(W, X, n, k)
        Dr, Sr = orc.blockdots(fmt, w, xq, n, k)
        assert np.array_equal(_host(S), Sr)
    else:
        D = getattr(qg, "blockdots_" + fmt)(W, X, n, k)
        Dr = orc.blockdots(fmt, w, xq, n, k)
    assert np.array_equal(_host(D), Dr)


def test_q8_0_block_dots_odd_block_count(env):
    """Rows of an odd number of 34-byte blocks start at 2-byte offsets."""
    qg, orc, torch, dev = env
    for n, k in [(5, 32), (9, 96), (64, 4064), (3, 2080)]:
        w = synth.random_blocks("q8_0", n, k, seed=k)
        xq = synth.random_blocks("q8_1", 1, k, seed=k + 1)
        D = qg.blockdots_q8_0(_gpu(torch, dev, w), _gpu(torch, dev, xq), n, k)
        assert np.array_equal(_host(D), orc.blockdots("q8_0", w, xq, n, k))


# ---------------------------------------------------------------- GEMV values
@pytest.mark.parametrize("fmt", ALL_GEMV)
@pytest.mark.parametrize("n,k", SHAPES + [(1, 4096), (511, 1024), (1000, 4096)])
def test_gemv_values(env, fmt, n, k):
    qg, orc, torch, dev = env
    w = synth.weights(fmt, n, k, seed=11 * n + k)
    x = synth.normal(n + 5 * k, 1, (k,))
    X = qg.quantize_q8_1(_gpu(torch, dev, x))
    y = getattr(qg, GEMV[fmt])(_gpu(torch, dev, w), X, n, k)
    xq = orc.quantize_q8_1(x[None])[0]
    assert np.array_equal(_host(X).ravel(), xq)
    assert rel_err(_host(y), orc.qgemv(fmt, w, xq, n, k)) <= REL_TOL


@pytest.mark.parametrize("fmt", ALL_GEMV)
def test_gemv_values_random_bytes(env, fmt):
    qg, orc, torch, dev = env
    n, k = 300, 1024
    w = synth.random_blocks(fmt, n, k, seed=77, lo_exp=-14, hi_exp=2)
    xq = synth.random_blocks("q8_1", 1, k, seed=78, lo_exp=-14, hi_exp=2)
    y = getattr(qg, GEMV[fmt])(_gpu(torch, dev, w), _gpu(torch, dev, xq), n, k)
    assert rel_err(_host(y), orc.qgemv(fmt, w, xq, n, k)) <= REL_TOL


def test_q8_0_values_odd_block_count(env):
    qg, orc, torch, dev = env
    n, k = 77, 4064
    w = synth.weights("q8_0", n, k, seed=5)
    xq = orc.quantize_q8_1(synth.normal(6, 1, (1, k)))
    y = qg.qgemv_q8_0(_gpu(torch, dev, w), _gpu(torch, dev, xq), n, k)
    assert rel_err(_host(y), orc.qgemv("q8_0", w, xq[0], n, k)) <= REL_TOL


def _hand_activation(k):
    nb = k // 32
    blk = np.zeros((nb, 36), np.uint8)
    blk[:, 0:2] = np.frombuffer(np.float16(0.125).tobytes(), np.uint8)
    qa = np.array([(i % 7) - 3 for i in range(k)], np.int64)
    blk[:, 4:] = qa.reshape(nb, 32).astype(np.int8).view(np.uint8)
    return blk.reshape(1, -1), qa


def test_gemv_hand_superblock_exact(env):
    """Every intermediate is exactly representable in fp32, so y must equal the
    hand-computed dot bit for bit (any summation order)."""
    qg, orc, torch, dev = env
    xq, qa = _hand_activation(256)
    X = _gpu(torch, dev, xq)
    fx = read_golden("q4_k_superblock.txt")
    blk = np.frombuffer(bytes.fromhex(fx["bytes"][0]), np.uint8)
    q = [int(t) for t in fx["q"][0].split()]
    sc = [int(t) for t in fx["sc"][0].split()]
    m = [int(t) for t in fx["m"][0].split()]
    exact = sum((Fraction(1, 16) * sc[i // 32] * q[i] - Fraction(1, 32) * m[i // 32]) * Fraction(1, 8) * qa[i]
                for i in range(256))
    y = _host(qg.qgemv_q4_k(_gpu(torch, dev, np.tile(blk, (5, 1))), X, 5, 256))
    assert all(Fraction(float(v)) == exact for v in y)
    fx = read_golden("q5_k_superblock.txt")
    blk = np.frombuffer(bytes.fromhex(fx["bytes"][0]), np.uint8)
    q = [int(t) for t in fx["q"][0].split()]
    sc = [int(t) for t in fx["sc"][0].split()]
    m = [int(t) for t in fx["m"][0].split()]
    exact = sum((Fraction(1, 16) * sc[i // 32] * q[i] - Fraction(1, 32) * m[i // 32]) * Fraction(1, 8) * qa[i]
                for i in range(256))
    y = _host(qg.qgemv_q5_k(_gpu(torch, dev, np.tile(blk, (6, 1))), X, 6, 256))
    assert all(Fraction(float(v)) == exact for v in y)
    fx = read_golden("q6_k_superblock.txt")
    blk = np.frombuffer(bytes.fromhex(fx["bytes"][0]), np.uint8)
    q = [int(t) for t in fx["q"][0].split()]
    sc = [int(t) for t in fx["scales"][0].split()]
    exact = sum(Fraction(1, 256) * sc[i // 16] * (q[i] - 32) * Fraction(1, 8) * qa[i] for i in range(256))
    y = _host(qg.qgemv_q6_k(_gpu(torch, dev, np.tile(blk, (3, 1))), X, 3, 256))
    assert all(Fraction(float(v)) == exact for v in y)
    blk = np.frombuffer(bytes.fromhex(read_golden("q8_0_block.txt")["bytes"][0]), np.uint8)
    exact = sum(Fraction((i % 32) - 16, 4) * Fraction(1, 8) * qa[i] for i in range(256))
    y = _host(qg.qgemv_q8_0(_gpu(torch, dev, np.tile(blk, (2, 8))), X, 2, 256))
    assert all(Fraction(float(v)) == exact for v in y)
    for fmt, d, off in (("q4_0", Fraction(-1, 8), 8), ("q5_0", Fraction(1, 32), 16)):
        fx = read_golden(f"{fmt}_block.txt")
        blk = np.frombuffer(bytes.fromhex(fx["bytes"][0]), np.uint8)
        q = [int(t) for t in fx["q"][0].split()]
        exact = sum(d * (q[i % 32] - off) * Fraction(1, 8) * qa[i] for i in range(256))
        y = _host(getattr(qg, GEMV[fmt])(_gpu(torch, dev, np.tile(blk, (7, 8))), X, 7, 256))
        assert all(Fraction(float(v)) == exact for v in y), fmt


def test_gemv_empty_and_zero_k(env):
    qg, orc, torch, dev = env
    X = torch.zeros(288, dtype=torch.uint8, device=dev)
    y = torch.full((8,), 7.0, device=dev)
    for fn in (qg.qgemv_q8_0, qg.qgemv_q4_k, qg.qgemv_q6_k, qg.qgemv_q5_k, qg.qgemv_q4_0, qg.qgemv_q5_0):
        fn(torch.zeros(16, dtype=torch.uint8, device=dev), X, 0, 256, y=y)   # n = 0: nothing written
        assert np.all(_host(y) == 7.0)
        fn(torch.zeros(16, dtype=torch.uint8, device=dev), X, 8, 0, y=y)     # k = 0: zeros
        assert np.all(_host(y) == 0.0)
        y.fill_(7.0)


# ------------------------------------------------------------ small-batch GEMV
GEMV_BATCH = {f: GEMV[f] + "_batch" for f in ("q8_0", "q4_k", "q6_k")}
# k = 17152 and 33536 span several activation chunks for every batch template
BATCH_SHAPES = [(1, 256), (3, 512), (65, 256), (130, 768), (64, 4096), (33, 14336), (7, 17152), (5, 33536)]


@pytest.mark.parametrize("fmt", ["q8_0", "q4_k", "q6_k"])
@pytest.mark.parametrize("b", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("n,k", BATCH_SHAPES)
def test_gemv_batch_values(env, fmt, b, n, k):
    """Each of the b rows against the oracle's batch-1 GEMV of that row."""
    qg, orc, torch, dev = env
    w = synth.weights(fmt, n, k, seed=13 * n + k)
    x = synth.normal(n + 7 * k + b, 1, (b, k))
    X = qg.quantize_q8_1(_gpu(torch, dev, x))
    y = _host(getattr(qg, GEMV_BATCH[fmt])(_gpu(torch, dev, w), X, b, n, k))
    xq = orc.quantize_q8_1(x)
    assert np.array_equal(_host(X), xq)
    assert y.shape == (b, n)
    for i in range(b):
        assert rel_err(y[i], orc.qgemv(fmt, w, xq[i], n, k)) <= REL_TOL, f"row {i}"


@pytest.mark.parametrize("b", [2, 4, 5, 8])
@pytest.mark.parametrize("n,k", [(9, 96), (70, 800), (33, 4128), (40, 320), (33, 4160)])
def test_gemv_batch_q8_0_block_counts(env, b, n, k):
    """Q8_0 rows whose block count is odd take the single-block path, and an
    even count that is not a multiple of 8 the block-pair path at every b (the
    matrix-core kernel needs k to be a multiple of 256): values against the
    oracle and exact dots."""
    qg, orc, torch, dev = env
    assert (k // 32) % 8 != 0
    w = synth.weights("q8_0", n, k, seed=5 * n + k)
    x = synth.normal(3 * n + k + b, 1, (b, k))
    X = qg.quantize_q8_1(_gpu(torch, dev, x))
    W = _gpu(torch, dev, w)
    y = _host(qg.qgemv_q8_0_batch(W, X, b, n, k))
    xq = orc.quantize_q8_1(x)
    for i in range(b):
        assert rel_err(y[i], orc.qgemv("q8_0", w, xq[i], n, k)) <= REL_TOL, f"row {i}"
    D = _host(qg.blockdots_batch("q8_0", W, X, b, n, k))
    for i in range(b):
        assert np.array_equal(D[i], orc.blockdots("q8_0", w, xq[i], n, k)), f"activation row {i}"


@pytest.mark.parametrize("fmt", ["q8_0", "q4_k", "q6_k"])
def test_gemv_batch_values_random_bytes(env, fmt):
    qg, orc, torch, dev = env
    b, n, k = 6, 300, 1024
    w = synth.random_blocks(fmt, n, k, seed=177, lo_exp=-14, hi_exp=2)
    xq = synth.random_blocks("q8_1", b, k, seed=178, lo_exp=-14, hi_exp=2)
    y = _host(getattr(qg, GEMV_BATCH[fmt])(_gpu(torch, dev, w), _gpu(torch, dev, xq), b, n, k))
    for i in range(b):
        assert rel_err(y[i], orc.qgemv(fmt, w, xq[i], n, k)) <= REL_TOL, f"row {i}"


# b = 2: Q4_K on the matrix cores, Q6_K on v_dot4; b = 3 and 5: both on the matrix cores
@pytest.mark.parametrize("b", [2, 3, 5])
def test_gemv_batch_hand_superblock_exact(env, b):
    """Rows with different power-of-two d_a and shifted codes: every
    intermediate is exact in fp32, so each y[i] equals its hand-computed dot."""
    qg, orc, torch, dev = env
    k = 256
    xq = np.zeros((b, k // 32, 36), np.uint8)
    qa = np.zeros((b, k), np.int64)
    for i in range(b):
        xq[i, :, 0:2] = np.frombuffer(np.float16(2.0 ** (i - 3)).tobytes(), np.uint8)
        qa[i] = [((j + i) % 7) - 3 for j in range(k)]
        xq[i, :, 4:] = qa[i].reshape(k // 32, 32).astype(np.int8).view(np.uint8)
    X = _gpu(torch, dev, xq.reshape(b, -1))
    da = [Fraction(2) ** (i - 3) for i in range(b)]
    fx = read_golden("q4_k_superblock.txt")
    blk = np.frombuffer(bytes.fromhex(fx["bytes"][0]), np.uint8)
    q = [int(t) for t in fx["q"][0].split()]
    sc = [int(t) for t in fx["sc"][0].split()]
    m = [int(t) for t in fx["m"][0].split()]
    y = _host(qg.qgemv_q4_k_batch(_gpu(torch, dev, np.tile(blk, (5, 1))), X, b, 5, k))
    for i in range(b):
        exact = sum((Fraction(1, 16) * sc[j // 32] * q[j] - Fraction(1, 32) * m[j // 32]) * da[i] * qa[i][j]
                    for j in range(k))
        assert all(Fraction(float(v)) == exact for v in y[i])
    fx = read_golden("q6_k_superblock.txt")
    blk = np.frombuffer(bytes.fromhex(fx["bytes"][0]), np.uint8)
    q = [int(t) for t in fx["q"][0].split()]
    sc = [int(t) for t in fx["scales"][0].split()]
    y = _host(qg.qgemv_q6_k_batch(_gpu(torch, dev, np.tile(blk, (3, 1))), X, b, 3, k))
    for i in range(b):
        exact = sum(Fraction(1, 256) * sc[j // 16] * (q[j] - 32) * da[i] * qa[i][j] for j in range(k))
        assert all(Fraction(float(v)) == exact for v in y[i])
    blk = np.frombuffer(bytes.fromhex(read_golden("q8_0_block.txt")["bytes"][0]), np.uint8)
    y = _host(qg.qgemv_q8_0_batch(_gpu(torch, dev, np.tile(blk, (2, 8))), X, b, 2, k))
    for i in range(b):
        exact = sum(Fraction((j % 32) - 16, 4) * da[i] * qa[i][j] for j in range(k))
        assert all(Fraction(float(v)) == exact for v in y[i])


def test_gemv_batch_empty_and_zero_k(env):
    qg, orc, torch, dev = env
    X = torch.zeros(8 * 288, dtype=torch.uint8, device=dev)
    y = torch.full((4, 8), 7.0, device=dev)
    for fmt, fn in GEMV_BATCH.items():
        f = getattr(qg, fn)
        W = torch.zeros(8 * qg.row_bytes(fmt, 256), dtype=torch.uint8, device=dev)
        f(W, X, 4, 0, 256, y=y)   # n = 0: nothing written
        f(W, X, 0, 8, 256, y=y)   # b = 0: nothing written
        assert np.all(_host(y) == 7.0)
        f(W, X, 4, 8, 0, y=y)     # k = 0: zeros
        assert np.all(_host(y) == 0.0)
        y.fill_(7.0)


def _blockdots_ref(orc, fmt, w, xq, n, k):
    D = orc.blockdots(fmt, w, xq, n, k)
    return D[0] if fmt in ("q4_k", "q5_k") else D


@pytest.mark.parametrize("fmt", ["q8_0", "q4_k", "q6_k"])
@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n,k", [(65, 256), (130, 768), (33, 14336), (5, 33536)])
def test_gemv_batch_block_dots_exact(env, fmt, b, n, k):
    """Exact int32 dots of the kernel each b dispatches to (matrix cores from 2
    rows for Q4_K, from 3 for Q6_K and from 5 for Q8_0, v_dot4 below), on fully
    random bytes."""
    qg, orc, torch, dev = env
    w = synth.random_blocks(fmt, n, k, seed=7 * n + b)
    xq = synth.random_blocks("q8_1", b, k, seed=11 * n + b)
    D = _host(qg.blockdots_batch(fmt, _gpu(torch, dev, w), _gpu(torch, dev, xq), b, n, k))
    for i in range(b):
        assert np.array_equal(D[i], _blockdots_ref(orc, fmt, w, xq[i], n, k)), f"activation row {i}"


@pytest.mark.big
@pytest.mark.parametrize("name,b", [("q8_0_gemv", 8), ("q4_k_gemv", 8), ("q4_k_gemv", 3), ("q6_k_gemv", 4),
                                    ("q6_k_gemv", 8)])
def test_gemv_batch_full_size(env, name, b):
    """The workload shapes with b activation rows: every output against the
    oracle, and the exact dots of the whole product from its launch grid."""
    qg, orc, torch, dev = env
    p = synth.WORKLOADS[name]
    fmt, n, k = p["fmt"], p["n"], p["k"]
    w = synth.weights(fmt, n, k, p["seed"])
    x = synth.normal(p["seed"], synth.T_X, (b, k))
    X = qg.quantize_q8_1(_gpu(torch, dev, x))
    W = _gpu(torch, dev, w)
    y = _host(getattr(qg, GEMV_BATCH[fmt])(W, X, b, n, k))
    xq = orc.quantize_q8_1(x)
    for i in range(b):
        assert rel_err(y[i], orc.qgemv(fmt, w, xq[i], n, k)) <= REL_TOL, f"activation row {i}"
    D = qg.blockdots_batch(fmt, W, X, b, n, k)
    for i in range(b):
        assert np.array_equal(_host(D[i]), _blockdots_ref(orc, fmt, w, xq[i], n, k)), f"activation row {i}"


@pytest.mark.big
@pytest.mark.parametrize("name", ["q8_0_gemv", "q4_k_gemv", "q6_k_gemv", "q5_k_gemv", "q4_0_gemv", "q5_0_gemv"])
def test_gemv_full_size(env, name):
    """The full workload sizes in the launch configuration the bench times:
    every output row against the oracle, and the exact dots of the whole
    matrix from a dump that runs on the product launch's grid."""
    qg, orc, torch, dev = env
    p = synth.WORKLOADS[name]
    fmt, n, k = p["fmt"], p["n"], p["k"]
    w = synth.weights(fmt, n, k, p["seed"])
    x = synth.normal(p["seed"], synth.T_X, (k,))
    X = qg.quantize_q8_1(_gpu(torch, dev, x))
    W = _gpu(torch, dev, w)
    y = _host(getattr(qg, GEMV[fmt])(W, X, n, k))
    xq = orc.quantize_q8_1(x[None])[0]
    assert np.array_equal(_host(X).ravel(), xq)
    assert rel_err(y, orc.qgemv(fmt, w, xq, n, k)) <= REL_TOL
    D = getattr(qg, "blockdots_" + fmt)(W, X, n, k)
    D = D[0] if fmt in ("q4_k", "q5_k") else D
    assert np.array_equal(_host(D), _blockdots_ref(orc, fmt, w, xq, n, k))


@pytest.mark.big
@pytest.mark.parametrize("fmt,n", [("q4_k", 10000), ("q5_k", 10000), ("q6_k", 52000)])
def test_gemv_chunked_k_multi_round(env, fmt, n):
    """k = 20480 runs the activation in two LDS chunks (16384 + 4096 values),
    and n is large enough that the persistent workgroups take more than one
    round of row groups (at most 6 resident per CU by LDS, 4 or 16 rows per
    group, Q6_K on twice the resident grid), so a workgroup restages chunk 0
    after chunk 1 of its previous round.  Every row and every block dot."""
    qg, orc, torch, dev = env
    k = 20480
    w = synth.random_blocks(fmt, n, k, seed=n + 3)
    x = synth.normal(n + 4, synth.T_X, (k,))
    X = qg.quantize_q8_1(_gpu(torch, dev, x))
    xq = orc.quantize_q8_1(x[None])[0]
    W = _gpu(torch, dev, w)
    y = _host(getattr(qg, GEMV[fmt])(W, X, n, k))
    assert rel_err(y, orc.qgemv(fmt, w, xq, n, k)) <= REL_TOL
    D = getattr(qg, "blockdots_" + fmt)(W, X, n, k)
    D = D[0] if fmt in ("q4_k", "q5_k") else D
    assert np.array_equal(_host(D), _blockdots_ref(orc, fmt, w, xq, n, k))


# ------------------------------------------------------------------------ mmq
@pytest.mark.parametrize("m,n,k", [(1, 1, 256), (32, 32, 256), (64, 64, 512), (70, 100, 512), (130, 65, 768),
                                   (3, 200, 1024)])
def test_mmq_block_dots_exact(env, m, n, k):
    qg, orc, torch, dev = env
    w = synth.random_blocks("q4_k", n, k, seed=m + n)
    aq = synth.random_blocks("q8_1", m, k, seed=m * n + k)
    D = qg.blockdots_q4_k_mmq(_gpu(torch, dev, w), _gpu(torch, dev, aq), m, n, k)
    assert np.array_equal(_host(D), orc.blockdots_q4_k_mmq(w, aq, m, n, k))


@pytest.mark.parametrize("m,n,k", [(1, 1, 256), (1, 64, 4096), (64, 64, 256), (100, 130, 512), (33, 4096, 256),
                                   (257, 70, 1024), (512, 256, 4096)])
def test_mmq_values(env, m, n, k):
    qg, orc, torch, dev = env
    w = synth.weights("q4_k", n, k, seed=m + 2 * n + k)
    a = synth.normal(m + n, 1, (m, k))
    AQ = qg.quantize_q8_1(_gpu(torch, dev, a))
    C = _host(qg.qgemm_q4_k_mmq(_gpu(torch, dev, w), AQ, m, n, k))
    aq = orc.quantize_q8_1(a)
    assert np.array_equal(_host(AQ), aq)
    assert rel_err(C, orc.qgemm_q4_k(w, aq, m, n, k)) <= REL_TOL


def test_mmq_hand_superblock_exact(env):
    qg, orc, torch, dev = env
    fx = read_golden("q4_k_superblock.txt")
    blk = np.frombuffer(bytes.fromhex(fx["bytes"][0]), np.uint8)
    q = [int(t) for t in fx["q"][0].split()]
    sc = [int(t) for t in fx["sc"][0].split()]
    m = [int(t) for t in fx["m"][0].split()]
    xq, qa = _hand_activation(256)
    exact = sum((Fraction(1, 16) * sc[i // 32] * q[i] - Fraction(1, 32) * m[i // 32]) * Fraction(1, 8) * qa[i]
                for i in range(256))
    C = _host(qg.qgemm_q4_k_mmq(_gpu(torch, dev, np.tile(blk, (70, 1))), _gpu(torch, dev, np.tile(xq, (40, 1))),
                                40, 70, 256))
    assert all(Fraction(float(v)) == exact for v in C.ravel())


@pytest.mark.big
def test_mmq_full_size(env):
    qg, orc, torch, dev = env
    p = synth.WORKLOADS["q4_k_mmq"]
    m, n, k = p["m"], p["n"], p["k"]
    w = synth.weights("q4_k", n, k, p["seed"])
    a = synth.normal(p["seed"], synth.T_X, (m, k))
    AQ = qg.quantize_q8_1(_gpu(torch, dev, a))
    C = _host(qg.qgemm_q4_k_mmq(_gpu(torch, dev, w), AQ, m, n, k))
    aq = orc.quantize_q8_1(a)
    assert np.array_equal(_host(AQ), aq)
    assert rel_err(C, orc.qgemm_q4_k(w, aq, m, n, k)) <= REL_TOL
    # the exact dots of the whole product (m * n * k/32 = 2^28), same grid
    D = _host(qg.blockdots_q4_k_mmq(_gpu(torch, dev, w), AQ, m, n, k))
    assert np.array_equal(D, orc.blockdots_q4_k_mmq(w, aq, m, n, k))


# ------------------------------------------------- activation prologue fusion
def _gamma(k, seed):
    return (1.0 + 0.25 * synth.normal(seed, 5, (k,))).astype(np.float32)


def _check_rmsnorm_stagewise(orc, x, gamma, eps, xq_gpu, r_gpu):
    """r within 1e-6 of the double oracle; the bytes exactly the oracle's
    quantization of (x * r) * gamma formed in fp32 from the GPU's own r."""
    r_ref = orc.rms_scale(x, eps)
    assert np.max(np.abs(r_gpu.astype(np.float64) - r_ref) / r_ref) <= 1e-6
    v = (x * r_gpu[:, None].astype(np.float32)) * gamma[None, :]
    assert v.dtype == np.float32
    assert np.array_equal(xq_gpu, orc.quantize_q8_1(v))


# k <= 4096 keeps the row in registers; 4128 and up read it again, 4128 with a
# remainder past the four-load rounds of the first step
@pytest.mark.parametrize("rows,k,std", [(1, 32, 1.0), (2, 64, 1.0), (3, 4096, 1.0), (2, 4128, 1.0),
                                        (2, 14336, 1e-3), (5, 768, 30.0), (2, 33536, 1.0)])
def test_rmsnorm_quantize_stagewise(env, rows, k, std):
    qg, orc, torch, dev = env
    x = synth.normal(rows + k, 4, (rows, k), std=std)
    gamma = _gamma(k, k)
    r = torch.empty(rows, device=dev)
    XQ, r = qg.rmsnorm_quantize_q8_1(_gpu(torch, dev, x), _gpu(torch, dev, gamma), 1e-5, r=r)
    _check_rmsnorm_stagewise(orc, x, gamma, 1e-5, _host(XQ), _host(r))


def test_rmsnorm_quantize_zero_row(env):
    """An all-zero row gives r = 1/sqrt(eps) and all-zero blocks."""
    qg, orc, torch, dev = env
    x = np.zeros((2, 256), np.float32)
    x[1] = synth.normal(3, 4, (256,))
    gamma = _gamma(256, 9)
    r = torch.empty(2, device=dev)
    XQ, r = qg.rmsnorm_quantize_q8_1(_gpu(torch, dev, x), _gpu(torch, dev, gamma), 1e-4, r=r)
    _check_rmsnorm_stagewise(orc, x, gamma, 1e-4, _host(XQ), _host(r))
    assert np.all(_host(XQ)[0] == 0)


# ------------------------------------------- mmq with the other weight types
MMQ_SHAPES = [(1, 1, 256), (32, 32, 256), (70, 100, 512), (130, 65, 768), (3, 200, 1024), (64, 128, 2048)]
# Q8_0 rows need k % 32 only: a ragged last 256-wide step, with an odd block
# count (rows at 2-byte offsets) or an even one (dword-aligned block pairs)
MMQ_Q80_RAGGED = [(5, 7, 32), (33, 70, 96), (64, 128, 288), (65, 129, 4128), (33, 70, 320), (17, 40, 64)]


@pytest.mark.parametrize("fmt,m,n,k", [("q6_k",) + s for s in MMQ_SHAPES] + [("q5_k",) + s for s in MMQ_SHAPES] +
                         [(f,) + s for f in ("q8_0", "q4_0", "q5_0") for s in MMQ_SHAPES + MMQ_Q80_RAGGED])
def test_mmq_block_dots_exact_other_formats(env, fmt, m, n, k):
    """Random bytes: the matrix-core dots equal the oracle's block dots
    (per 16 values for Q6_K)."""
    qg, orc, torch, dev = env
    w = synth.random_blocks(fmt, n, k, seed=m + n + 7)
    aq = synth.random_blocks("q8_1", m, k, seed=m * n + k + 7)
    D = getattr(qg, f"blockdots_{fmt}_mmq")(_gpu(torch, dev, w), _gpu(torch, dev, aq), m, n, k)
    assert np.array_equal(_host(D), orc.blockdots_mmq(fmt, w, aq, m, n, k))


@pytest.mark.parametrize("fmt,m,n,k", [("q6_k",) + s for s in MMQ_SHAPES + [(1, 64, 4096), (257, 70, 1024)]] +
                         [("q5_k",) + s for s in MMQ_SHAPES + [(257, 70, 1024)]] +
                         [(f,) + s for f in ("q8_0", "q4_0", "q5_0")
                          for s in MMQ_SHAPES + MMQ_Q80_RAGGED + [(257, 70, 1024)]])
def test_mmq_values_other_formats(env, fmt, m, n, k):
    qg, orc, torch, dev = env
    w = synth.weights(fmt, n, k, seed=m + 2 * n + k)
    a = synth.normal(m + n, 1, (m, k))
    AQ = qg.quantize_q8_1(_gpu(torch, dev, a))
    C = _host(getattr(qg, f"qgemm_{fmt}_mmq")(_gpu(torch, dev, w), AQ, m, n, k))
    aq = orc.quantize_q8_1(a)
    assert np.array_equal(_host(AQ), aq)
    assert rel_err(C, orc.qgemm(fmt, w, aq, m, n, k)) <= REL_TOL


@pytest.mark.parametrize("fmt", ["q6_k", "q8_0", "q5_k", "q4_0", "q5_0"])
def test_mmq_values_random_bytes_other_formats(env, fmt):
    qg, orc, torch, dev = env
    m, n, k = 70, 130, 512
    w = synth.random_blocks(fmt, n, k, seed=191, lo_exp=-14, hi_exp=2)
    aq = synth.random_blocks("q8_1", m, k, seed=192, lo_exp=-14, hi_exp=2)
    C = _host(getattr(qg, f"qgemm_{fmt}_mmq")(_gpu(torch, dev, w), _gpu(torch, dev, aq), m, n, k))
    assert rel_err(C, orc.qgemm(fmt, w, aq, m, n, k)) <= REL_TOL


def test_mmq_hand_blocks_exact_other_formats(env):
    """Hand-built Q6_K superblock and Q8_0 blocks against d_a = 1/8: every
    intermediate is exact in fp32, so C equals the hand-computed dot."""
    qg, orc, torch, dev = env
    xq, qa = _hand_activation(256)
    A = _gpu(torch, dev, np.tile(xq, (40, 1)))
    fx = read_golden("q6_k_superblock.txt")
    blk = np.frombuffer(bytes.fromhex(fx["bytes"][0]), np.uint8)
    q = [int(t) for t in fx["q"][0].split()]
    sc = [int(t) for t in fx["scales"][0].split()]
    exact = sum(Fraction(1, 256) * sc[i // 16] * (q[i] - 32) * Fraction(1, 8) * qa[i] for i in range(256))
    C = _host(qg.qgemm_q6_k_mmq(_gpu(torch, dev, np.tile(blk, (70, 1))), A, 40, 70, 256))
    assert all(Fraction(float(v)) == exact for v in C.ravel())
    blk = np.frombuffer(bytes.fromhex(read_golden("q8_0_block.txt")["bytes"][0]), np.uint8)
    exact = sum(Fraction((i % 32) - 16, 4) * Fraction(1, 8) * qa[i] for i in range(256))
    C = _host(qg.qgemm_q8_0_mmq(_gpu(torch, dev, np.tile(blk, (70, 8))), A, 40, 70, 256))
    assert all(Fraction(float(v)) == exact for v in C.ravel())
    fx = read_golden("q5_k_superblock.txt")
    blk = np.frombuffer(bytes.fromhex(fx["bytes"][0]), np.uint8)
    q = [int(t) for t in fx["q"][0].split()]
    sc = [int(t) for t in fx["sc"][0].split()]
    m = [int(t) for t in fx["m"][0].split()]
    exact = sum((Fraction(1, 16) * sc[i // 32] * q[i] - Fraction(1, 32) * m[i // 32]) * Fraction(1, 8) * qa[i]
                for i in range(256))
    C = _host(qg.qgemm_q5_k_mmq(_gpu(torch, dev, np.tile(blk, (70, 1))), A, 40, 70, 256))
    assert all(Fraction(float(v)) == exact for v in C.ravel())
    for fmt, d, off in (("q4_0", Fraction(-1, 8), 8), ("q5_0", Fraction(1, 32), 16)):
        fx = read_golden(f"{fmt}_block.txt")
        blk = np.frombuffer(bytes.fromhex(fx["bytes"][0]), np.uint8)
        q = [int(t) for t in fx["q"][0].split()]
        exact = sum(d * (q[i % 32] - off) * Fraction(1, 8) * qa[i] for i in range(256))
        C = _host(getattr(qg, f"qgemm_{fmt}_mmq")(_gpu(torch, dev, np.tile(blk, (70, 8))), A, 40, 70, 256))
        assert all(Fraction(float(v)) == exact for v in C.ravel()), fmt


def test_mmq_empty_other_formats(env):
    qg, orc, torch, dev = env
    A = torch.zeros(4 * 288, dtype=torch.uint8, device=dev)
    for fmt, k in (("q6_k", 256), ("q8_0", 32), ("q5_k", 256), ("q4_0", 32), ("q5_0", 32)):
        W = torch.zeros(4 * qg.row_bytes(fmt, 256), dtype=torch.uint8, device=dev)
        c = torch.full((4, 4), 7.0, device=dev)
        f = getattr(qg, f"qgemm_{fmt}_mmq")
        f(W, A, 0, 4, k, c=c)   # m = 0: nothing written
        f(W, A, 4, 0, k, c=c)   # n = 0: nothing written
        assert np.all(_host(c) == 7.0)
        f(W, A, 4, 4, 0, c=c)   # k = 0: zeros
        assert np.all(_host(c) == 0.0)


@pytest.mark.big
@pytest.mark.parametrize("name", ["q6_k_mmq", "q8_0_mmq", "q5_k_mmq", "q4_0_mmq", "q5_0_mmq"])
def test_mmq_full_size_other_formats(env, name):
    qg, orc, torch, dev = env
    p = synth.WORKLOADS[name]
    fmt, m, n, k = p["fmt"], p["m"], p["n"], p["k"]
    w = synth.weights(fmt, n, k, p["seed"])
    a = synth.normal(p["seed"], synth.T_X, (m, k))
    AQ = qg.quantize_q8_1(_gpu(torch, dev, a))
    C = _host(getattr(qg, f"qgemm_{fmt}_mmq")(_gpu(torch, dev, w), AQ, m, n, k))
    aq = orc.quantize_q8_1(a)
    assert np.array_equal(_host(AQ), aq)
    assert rel_err(C, orc.qgemm(fmt, w, aq, m, n, k)) <= REL_TOL
    # exact dots of every token row against the first 512 weight rows: the
    # workgroups of the first four column tiles of the launch, whole
    nd = 512
    D = _host(getattr(qg, f"blockdots_{fmt}_mmq")(_gpu(torch, dev, w[:nd]), AQ, m, nd, k))
    assert np.array_equal(D, orc.blockdots_mmq(fmt, w[:nd], aq, m, nd, k))


# --------------------------------------------------------------------- router
def _router_case(seed, T, E, H):
    g = np.random.default_rng(seed)
    wr = (0.02 * g.standard_normal((E, H))).astype(np.float32)
    x = g.standard_normal((T, H)).astype(np.float32)
    return wr, x


def _check_router_stagewise(orc, wr, x, k, ids, w, logits):
    """logits within 1e-5 of the double oracle; ids exactly and weights within
    1e-6 of the oracle's selection from the GPU's own f32 logits."""
    ref = orc.router_logits(wr, x)
    assert rel_err(logits, ref) <= 1e-5
    ids_ref, w_ref = orc.route_topk(logits, k)
    assert np.array_equal(ids, ids_ref)
    assert np.max(np.abs(w.astype(np.float64) - w_ref)) <= 1e-6


@pytest.mark.parametrize("T,E,H,k", [(1, 8, 4, 1), (16, 128, 2048, 8), (33, 64, 256, 2), (5, 256, 8192, 64),
                                     (7, 40, 1024, 40), (3, 128, 2048, 1), (9, 7, 512, 3), (2, 16, 16384, 4),
                                     (130, 128, 2048, 8)])
def test_router_topk_stagewise(env, T, E, H, k):
    qg, orc, torch, dev = env
    wr, x = _router_case(T * E + H, T, E, H)
    logits = torch.empty((T, E), device=dev)
    ids, w = qg.moe_router_topk(_gpu(torch, dev, wr), _gpu(torch, dev, x), k, logits=logits)
    _check_router_stagewise(orc, wr, x, k, _host(ids), _host(w), _host(logits))


def test_router_topk_exact_ties(env):
    """Duplicated router rows give bit-equal logits: the lower expert wins."""
    qg, orc, torch, dev = env
    T, E, H, k = 9, 96, 512, 6
    wr, x = _router_case(5, T, E, H)
    wr[50] = wr[3]
    wr[77] = wr[3]
    wr[60] = wr[10]
    x[2] = 0.0                                             # an all-zero row: every logit equal
    logits = torch.empty((T, E), device=dev)
    ids, w = qg.moe_router_topk(_gpu(torch, dev, wr), _gpu(torch, dev, x), k, logits=logits)
    L, I = _host(logits), _host(ids)
    assert np.array_equal(L[:, 50], L[:, 3]) and np.array_equal(L[:, 77], L[:, 3])
    assert I[2].tolist() == list(range(k))
    _check_router_stagewise(orc, wr, x, k, I, _host(w), L)


def test_router_feeds_moe(env):
    """The router's table drives the expert FFN as is: the stage-wise MoE
    check passes on the ids and weights the router wrote."""
    qg, orc, torch, dev = env
    E, F, H, T, K = 6, 256, 512, 5, 2
    w_gu, w_dn, _, _, x = _moe_case(97, E, F, H, T, K)
    wr, _ = _router_case(98, 1, E, H)
    ids, rw = qg.moe_router_topk(_gpu(torch, dev, wr), _gpu(torch, dev, x), K)
    ids, rw = _host(ids), _host(rw)
    assert ids.dtype == np.int32 and rw.dtype == np.float32
    _run_moe_stagewise(env, w_gu, w_dn, ids, rw, x, E, F, H, T, K)


def test_router_empty(env):
    qg, orc, torch, dev = env
    wr, _ = _router_case(1, 1, 8, 16)
    x = torch.zeros((0, 16), device=dev)
    ids, w = qg.moe_router_topk(_gpu(torch, dev, wr), x, 2)
    assert ids.shape == (0, 2) and w.shape == (0, 2)


# ------------------------------------------------------------------------ MoE
def _moe_case(seed, E, F, H, T, K):
    w_gu = synth.weights("q4_k", E * 2 * F, H, seed, synth.T_W).reshape(E, -1)
    w_dn = synth.weights("q4_k", E * H, F, seed, synth.T_WDOWN).reshape(E, -1)
    ids, rw = synth.routing(seed, T, E, K)
    x = synth.normal(seed, synth.T_X, (T, H))
    return w_gu, w_dn, ids, rw, x


def _run_moe_stagewise(env, w_gu, w_dn, ids, rw, x, E, F, H, T, K):
    qg, orc, torch, dev = env
    XQ = qg.quantize_q8_1(_gpu(torch, dev, x))
    xq = orc.quantize_q8_1(x)
    assert np.array_equal(_host(XQ), xq)
    ws = torch.empty(qg.moe_qgemv_q4_k_workspace_size(T, K, E, F, H), dtype=torch.uint8, device=dev)
    WGU, WDN = _gpu(torch, dev, w_gu), _gpu(torch, dev, w_dn)
    IDS, RW = _gpu(torch, dev, ids), _gpu(torch, dev, rw)
    out = _host(qg.moe_qgemv_q4_k(WGU, WDN, XQ, IDS, RW, T, K, E, F, H, workspace=ws))
    hq_g, gu_g, _ = qg.moe_workspace_regions(ws, T, K, F, H)
    hq_g, gu_g = _host(hq_g), _host(gu_g)
    ref = orc.moe_q4_k(w_gu, w_dn, xq, ids, rw, T, K, E, F, H)
    valid = (ids.ravel() >= 0) & (ids.ravel() < E)
    # stage 1: gate/up values
    assert rel_err(gu_g[valid], ref["gu"][valid]) <= REL_TOL
    # exact dots of both expert GEMVs, every valid pair, from the call's own
    # kernels (dump instances on the product's grids): gate/up against the
    # token's Q8_1 row, down against the pair's h^ as the call formed it
    ws2 = torch.empty_like(ws)
    D_gu, D_dn = qg.blockdots_moe_q4_k(WGU, WDN, XQ, IDS, RW, T, K, E, F, H, ws2)
    hq_d = _host(qg.moe_workspace_regions(ws2, T, K, F, H)[0])
    assert np.array_equal(hq_d[valid], hq_g[valid])
    D_gu, D_dn = _host(D_gu), _host(D_dn)
    for p in np.flatnonzero(valid):
        e, t = ids.ravel()[p], p // K
        assert np.array_equal(D_gu[p], orc.blockdots("q4_k", w_gu[e], xq[t], 2 * F, H)[0]), f"gate/up pair {p}"
        assert np.array_equal(D_dn[p], orc.blockdots("q4_k", w_dn[e], hq_g[p], H, F)[0]), f"down pair {p}"
    ref_own = orc.moe_q4_k(w_gu, w_dn, xq, ids, rw, T, K, E, F, H, hq_in=hq_g)
    assert rel_err(out, ref_own["out"]) <= REL_TOL
    # Against the oracle's own h^: the GPU sums g and u in another fp32 order,
    # so a value on a rounding boundary of its block can land one code away.
    # Every such difference must be a tie of the quantizer under the oracle's
    # own h (|h/d| within 1e-3 of k + 1/2), and a stored d that differs must be
    # a tie of its binary16 rounding; the end-to-end error is then held to
    # REL_TOL plus the oracle's own measure of what those tie-breaks change.
    stats = _check_hq_ties(orc, ref, hq_g, valid, F)
    e2e = rel_err(out, ref["out"])
    tie_effect = rel_err(ref_own["out"], ref["out"])
    assert e2e <= REL_TOL + tie_effect, (e2e, tie_effect, stats)
    if stats["code_flips"] == 0 and stats["d_flips"] == 0:
        assert e2e <= REL_TOL
    return dict(stats, e2e_rel_err=e2e, tie_effect=tie_effect)


def _check_hq_ties(orc, ref, hq_g, valid, F):
    """Compares the GPU's h^ with the oracle's block by block; see the caller."""
    g_blk = hq_g[valid].reshape(-1, F // 32, 36)
    r_blk = ref["hq"][valid].reshape(-1, F // 32, 36)
    dq = g_blk[..., 4:].view(np.int8).astype(np.int32) - r_blk[..., 4:].view(np.int8).astype(np.int32)
    assert np.abs(dq).max(initial=0) <= 1
    gd = g_blk[..., 0:2].copy().view(np.uint16).astype(np.int32)[..., 0]
    rd = r_blk[..., 0:2].copy().view(np.uint16).astype(np.int32)[..., 0]
    assert np.abs(gd - rd).max(initial=0) <= 1  # d >= 0: bit patterns are ordered like the values
    # the oracle's h (double silu(g) * u rounded once to f32) and its fp32 d
    gu = ref["gu"][valid]
    g, u = gu[:, :F], gu[:, F:]
    h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32).reshape(-1, F // 32, 32)
    d32 = (np.abs(h).max(axis=2) / np.float32(127.0)).astype(np.float32)
    where = np.argwhere(dq != 0)
    for pi, b, i in where:
        x = abs(float(np.float32(h[pi, b, i]) / d32[pi, b]))
        assert abs(x - np.floor(x) - 0.5) <= 1e-3, f"h^ code differs off a tie: pair {pi} block {b} value {i}: {x}"
    for pi, b in np.argwhere(gd != rd):
        dv = float(d32[pi, b])
        lo = float(np.float16(dv))
        hi = float(np.nextafter(np.float16(dv), np.float16(np.inf if lo <= dv else -np.inf)))
        ulp = abs(hi - lo)
        assert abs(abs(dv - lo) - ulp / 2) <= 1e-2 * ulp, f"d differs off a binary16 tie: pair {pi} block {b}"
    return {"code_flips": int(len(where)), "codes": int(dq.size), "d_flips": int(np.count_nonzero(gd != rd)),
            "blocks": int(gd.size)}


def _record(name, rec):
    """Keeps a parity measurement: as a JSON file in the repository's run-output
    folder when that folder exists, and as a warning (pytest prints those in
    its summary)."""
    import json
    import os
    import warnings
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = os.path.join(root, "gpurun_out")
    if os.path.isdir(out):
        with open(os.path.join(out, f"parity_{name}.json"), "w") as f:
            json.dump(rec, f)
    warnings.warn(f"{name}: {json.dumps(rec)}")


def test_moe_small(env):
    E, F, H, T, K = 6, 256, 512, 5, 3
    case = _moe_case(61, E, F, H, T, K)
    _run_moe_stagewise(env, *case, E, F, H, T, K)


def test_moe_invalid_ids_skipped(env):
    E, F, H, T, K = 5, 256, 768, 4, 2
    w_gu, w_dn, ids, rw, x = _moe_case(62, E, F, H, T, K)
    ids = ids.copy()
    ids[0, 1] = E + 3
    ids[3, 0] = -7
    _run_moe_stagewise(env, w_gu, w_dn, ids, rw, x, E, F, H, T, K)


def test_moe_token_without_valid_slots_and_repeated_experts(env):
    """A token whose slots are all out of range gets zeros (no slot arrives
    for it); a token routed twice to one expert counts both slots."""
    E, F, H, T, K = 5, 256, 512, 4, 2
    w_gu, w_dn, ids, rw, x = _moe_case(66, E, F, H, T, K)
    ids = ids.copy()
    ids[2, :] = [-1, E]
    ids[1, :] = [3, 3]
    qg = env[0]
    assert qg.moe_launches(T, K, E, F, H) == 2
    _run_moe_stagewise(env, w_gu, w_dn, ids, rw, x, E, F, H, T, K)


@pytest.mark.parametrize("E,F,H,T,K,launches", [(6, 1536, 512, 5, 3, 2),    # 24 down units: 8 lanes x 3 units
                                                (3, 8192, 256, 2, 2, 2),    # 128 down units: 64 lanes x 2 units
                                                (4, 1280, 512, 3, 2, 4)])   # 20 down units: the four-kernel path
def test_moe_down_row_splits(env, E, F, H, T, K, launches):
    """Down rows of n_ff/64 units split over L lanes with 1, 2 or 3 units each
    (two kernels), or not at all (four kernels)."""
    qg = env[0]
    assert qg.moe_launches(T, K, E, F, H) == launches
    case = _moe_case(67 + F, E, F, H, T, K)
    _run_moe_stagewise(env, *case, E, F, H, T, K)


def test_moe_shared_experts(env):
    """Several tokens on one expert: the expert's rows are reused across pairs."""
    E, F, H, T, K = 3, 512, 256, 9, 2
    w_gu, w_dn, ids, rw, x = _moe_case(63, E, F, H, T, K)
    _run_moe_stagewise(env, w_gu, w_dn, ids, rw, x, E, F, H, T, K)


@pytest.mark.parametrize("E,T,K,H", [(160, 6, 3, 512),    # experts past 128: four words of routing state
                                     (8, 40, 4, 512),     # 160 pairs: four words of routing state
                                     (8, 70, 4, 512),     # 280 pairs: the (expert x tile) grid form
                                     (8, 20, 4, 2048)])   # token rows past the 40 KB staging: unstaged gate/up
def test_moe_routing_table_sizes(env, E, T, K, H):
    """The persistent form keeps two words of ids and touched-expert bitmap per
    lane up to 128 pairs and 128 experts, four words up to 256; larger tables
    run the grid form (four kernels).  The gate/up call stages the token rows
    in LDS when they fit in 40 KB.  Each case against the oracle, stage by
    stage."""
    F = 256
    assert env[0].moe_launches(T, K, E, F, H) == (2 if T * K <= 256 else 4)
    case = _moe_case(65 + E + T, E, F, H, T, K)
    _run_moe_stagewise(env, *case, E, F, H, T, K)


@pytest.mark.big
def test_moe_full_size(env):
    p = synth.WORKLOADS["moe_q4_k"]
    E, F, H, T, K = p["n_expert"], p["n_ff"], p["n_embd"], p["n_tok"], p["top_k"]
    assert env[0].moe_launches(T, K, E, F, H) == 2
    case = _moe_case(p["seed"], E, F, H, T, K)
    rec = _run_moe_stagewise(env, *case, E, F, H, T, K)
    _record("moe_full_size", rec)


# ---------------------------------------------------------------- HIP graphs
def test_graph_replay_matches_eager(env):
    """The bench replays captured HIP graphs: every entry point captured in one
    graph must reproduce the eager results bit for bit on every replay, with
    other eager work and synchronizations between the replays."""
    qg, orc, torch, dev = env
    n, k, m = 300, 1024, 70
    E, F, H, T, K = 4, 256, 512, 5, 2
    x = _gpu(torch, dev, synth.normal(91, 1, (k,)))
    a = _gpu(torch, dev, synth.normal(92, 1, (m, k)))
    Ws = {f: _gpu(torch, dev, synth.weights(f, n, k, seed=93)) for f in ("q8_0", "q4_k", "q6_k")}
    w_gu, w_dn, ids, rw, xm = _moe_case(94, E, F, H, T, K)
    WGU, WDN, IDS, RW, XM = (_gpu(torch, dev, v) for v in (w_gu, w_dn, ids, rw, xm))
    xb = _gpu(torch, dev, synth.normal(95, 1, (5, k)))
    xbq = torch.empty((5, k // 32 * 36), dtype=torch.uint8, device=dev)
    ybs = {f: torch.empty((5, n), device=dev) for f in Ws}
    xq = torch.empty(k // 32 * 36, dtype=torch.uint8, device=dev)
    aq = torch.empty((m, k // 32 * 36), dtype=torch.uint8, device=dev)
    xmq = torch.empty((T, H // 32 * 36), dtype=torch.uint8, device=dev)
    ys = {f: torch.empty(n, device=dev) for f in Ws}
    c = torch.empty((m, n), device=dev)
    c6 = torch.empty((m, n), device=dev)
    c8 = torch.empty((m, n), device=dev)
    out = torch.empty((T, H), device=dev)
    ws = torch.empty(qg.moe_qgemv_q4_k_workspace_size(T, K, E, F, H), dtype=torch.uint8, device=dev)
    gam = _gpu(torch, dev, _gamma(k, 96))
    xnq = torch.empty((5, k // 32 * 36), dtype=torch.uint8, device=dev)
    rr = torch.empty(5, device=dev)
    wr_h, xr_h = _router_case(99, 16, 128, 2048)
    WR, XR = _gpu(torch, dev, wr_h), _gpu(torch, dev, xr_h)
    rids = torch.empty((16, 8), dtype=torch.int32, device=dev)
    rws = torch.empty((16, 8), device=dev)
    rlg = torch.empty((16, 128), device=dev)
    Wl = {f: _gpu(torch, dev, synth.weights(f, n, k, seed=97)) for f in ("q4_0", "q5_0")}
    yl = {f: torch.empty(n, device=dev) for f in Wl}
    cl = {f: torch.empty((m, n), device=dev) for f in Wl}

    def work():
        qg.rmsnorm_quantize_q8_1(xb, gam, 1e-5, xq=xnq, r=rr)
        qg.moe_router_topk(WR, XR, 8, ids=rids, weights=rws, logits=rlg)
        qg.quantize_q8_1(x, xq)
        for f, W in Ws.items():
            getattr(qg, GEMV[f])(W, xq, n, k, y=ys[f])
        qg.quantize_q8_1(xb, xbq)
        for f, W in Ws.items():
            getattr(qg, GEMV_BATCH[f])(W, xbq, 5, n, k, y=ybs[f])
        qg.quantize_q8_1(a, aq)
        qg.qgemm_q4_k_mmq(Ws["q4_k"], aq, m, n, k, c=c)
        qg.qgemm_q6_k_mmq(Ws["q6_k"], aq, m, n, k, c=c6)
        qg.qgemm_q8_0_mmq(Ws["q8_0"], aq, m, n, k, c=c8)
        for f, W in Wl.items():
            getattr(qg, GEMV[f])(W, xq, n, k, y=yl[f])
            getattr(qg, f"qgemm_{f}_mmq")(W, aq, m, n, k, c=cl[f])
        qg.quantize_q8_1(XM, xmq)
        qg.moe_qgemv_q4_k(WGU, WDN, xmq, IDS, RW, T, K, E, F, H, out=out, workspace=ws)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (xq, *ys.values(), xbq, *ybs.values(), aq, c, c6, c8, xmq, out, xnq, rr,
                                    rids, rws, rlg, *yl.values(), *cl.values())]

    work()
    eager = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        work()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            work()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (xq, *ys.values(), xbq, *ybs.values(), aq, c, c6, c8, xmq, out, xnq, rr, rids, rws, rlg,
                  *yl.values(), *cl.values()):
            t.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for e, r in zip(eager, got):
            assert torch.equal(e, r), f"replay {rep} differs"


@pytest.mark.parametrize("F,H", [(256, 4608), (512, 8448)])
def test_moe_long_rows(env, F, H):
    """Rows of 72 and 132 lane units: the two-units-per-lane and the reload-per-
    pair paths of the expert GEMV."""
    E, T, K = 3, 4, 2
    case = _moe_case(64 + F, E, F, H, T, K)
    _run_moe_stagewise(env, *case, E, F, H, T, K)
