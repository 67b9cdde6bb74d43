"""moe_qgemv_q4_k_noalloc (the MoE call on the library's own per-GPU
workspace) against moe_qgemv_q4_k with a caller workspace, through the C ABI:
two calls in a row, the second smaller, each bit-identical to the workspace
call on the same inputs (the kernels are the same), and a shape whose
workspace exceeds the library's maximum refused with QG_ERR_WORKSPACE."""
import numpy as np
import pytest

from _util import REL_TOL, rel_err
from gemm_gguf_block_amd import synth

pytestmark = pytest.mark.gpu


def _case(qg, torch, dev, seed, E, F, H, T, K):
    w_gu = synth.weights("q4_k", E * 2 * F, H, seed, synth.T_W).reshape(E, -1)
    w_dn = synth.weights("q4_k", E * H, F, seed, synth.T_WDOWN).reshape(E, -1)
    ids, rw = synth.routing(seed, T, E, K)
    x = synth.normal(seed, synth.T_X, (T, H))
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return g(w_gu), g(w_dn), qg.quantize_q8_1(g(x)), g(ids), g(rw), (w_gu, w_dn, x, ids, rw)


def test_noalloc_matches_the_workspace_call():
    import torch

    import gemm_gguf_block_amd as qg
    import oracle
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # the workload shape (128 experts, 768 x 2048, 16 tokens, top-8), then a
    # smaller one that reuses the same scratch right after it
    for seed, E, F, H, T, K in ((1004, 128, 768, 2048, 16, 8), (77, 6, 256, 512, 5, 3)):
        WGU, WDN, XQ, IDS, RW, host = _case(qg, torch, dev, seed, E, F, H, T, K)
        ws = torch.empty(qg.moe_qgemv_q4_k_workspace_size(T, K, E, F, H), dtype=torch.uint8, device=dev)
        ref = qg.moe_qgemv_q4_k(WGU, WDN, XQ, IDS, RW, T, K, E, F, H, workspace=ws)
        out = torch.full((T, H), float("nan"), device=dev)
        qg.moe_qgemv_q4_k_noalloc(WGU, WDN, XQ, IDS, RW, T, K, E, F, H, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"shape E={E} F={F} H={H} T={T} K={K}"
        # and the product itself, against the oracle through the call's own h^
        w_gu, w_dn, x, ids, rw = host
        hq = qg.moe_workspace_regions(ws, T, K, F, H)[0].cpu().numpy()
        r = oracle.moe_q4_k(w_gu, w_dn, oracle.quantize_q8_1(x), ids, rw, T, K, E, F, H, hq_in=hq)["out"]
        assert rel_err(out.cpu().numpy(), r) <= REL_TOL


def test_noalloc_refuses_shapes_past_its_workspace():
    import torch

    import gemm_gguf_block_amd as qg
    dev = torch.device("cuda:0")
    E, F, H, K = 4, 256, 4096, 8
    T = 1
    while qg.moe_qgemv_q4_k_workspace_size(T, K, E, F, H) <= qg.moe_qgemv_q4_k_noalloc_max_workspace():
        T *= 2
    assert T * K <= 1 << 20
    u8 = lambda n: torch.zeros(n, dtype=torch.uint8, device=dev)
    WGU = u8(E * 2 * F * qg.row_bytes("q4_k", H))
    WDN = u8(E * H * qg.row_bytes("q4_k", F))
    XQ = u8(T * qg.row_bytes("q8_1", H))
    IDS = torch.zeros((T, K), dtype=torch.int32, device=dev)
    RW = torch.zeros((T, K), dtype=torch.float32, device=dev)
    out = torch.full((T, H), 7.0, device=dev)
    with pytest.raises(qg.QGError) as e:
        qg.moe_qgemv_q4_k_noalloc(WGU, WDN, XQ, IDS, RW, T, K, E, F, H, out=out)
    assert e.value.status == 4  # QG_ERR_WORKSPACE
    assert torch.all(out == 7.0)
