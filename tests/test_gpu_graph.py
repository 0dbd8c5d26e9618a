"""The library's calls captured in a HIP graph: every replay must equal the
eager result bit for bit (the kernels clear nothing with memset nodes and keep
no state between calls).  Replays are interleaved with eager work on the same
buffers and synchronizations, and the inputs change between replays."""
import numpy as np
import pytest

from block_scaled_fp4_act_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")


def test_graph_replays_match_eager():
    import torch
    import block_scaled_fp4_act_amd as rs
    M, N, K = 4, 512, 1024
    W = torch.from_numpy(inputs.weights(N, K, 3)).cuda()
    blob_nv = rs.prepack_weights(W, 0)
    blob_mx = rs.prepack_weights(W, 1)
    masks = rs.kext_select(rs.channel_abs_sum(torch.randn(32, K, device="cuda")), 2)
    blob_kx = rs.prepack_weights_kext(W, 0, masks, 2)
    KE = rs.kext_dim(K, 2)
    # attention: 2 sequences in a small paged cache, 3 splits (partials + combine)
    H_q, H_kv, D = 16, 2, 128
    lens = [70, 45]
    pages = torch.arange(6, dtype=torch.int32, device="cuda").view(2, 3)
    cache = torch.zeros(6 * rs.kv_page_bytes(H_kv, D), dtype=torch.uint8, device="cuda")
    slots = torch.cat([pages[b, torch.arange(L, device="cuda") // 32] * 32 + torch.arange(L, device="cuda") % 32
                       for b, L in enumerate(lens)]).to(torch.int32)
    kv = torch.randn(sum(lens), H_kv, D, device="cuda").to(torch.bfloat16)
    rs.kv_cache_write(kv, kv.flip(0).contiguous(), slots, cache)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")

    x = torch.empty(M, K, device="cuda", dtype=torch.bfloat16)
    q = torch.empty(2 * H_q, D, device="cuda", dtype=torch.bfloat16)
    act_nv = torch.empty(rs.packed_act_bytes(0, M, K, True), dtype=torch.uint8, device="cuda")
    act_mx = torch.empty(rs.packed_act_bytes(1, M, K, True), dtype=torch.uint8, device="cuda")
    act_kx = torch.empty(rs.packed_act_bytes(0, M, KE, False), dtype=torch.uint8, device="cuda")
    act_q = torch.empty(rs.packed_act_bytes(0, 2 * H_q, D, True), dtype=torch.uint8, device="cuda")
    outs = [torch.empty(M, N, device="cuda") for _ in range(3)] + [torch.empty(2, H_q, D, device="cuda")]
    ws = torch.empty(rs.lib().rsfp4_resattn_workspace_bytes(2, H_q, D, 3), dtype=torch.uint8, device="cuda")

    def work():
        rs.quantize_act_with_residue(x, 0, True, out=act_nv)
        rs.fp4_linear_compensated(act_nv, blob_nv, M, N, K, 0, out=outs[0])
        rs.quantize_act_with_residue(x, 1, True, out=act_mx)
        rs.fp4_linear_compensated(act_mx, blob_mx, M, N, K, 1, out=outs[1])
        rs.quantize_act_kext(x, 0, masks, 2, out=act_kx)
        rs.fp4_linear(act_kx, blob_kx, M, N, KE, 0, out=outs[2])
        rs.quantize_act_with_residue(q, 0, True, out=act_q)
        rs.resattn_decode(act_q, cache, pages, seq, 96, 2, H_q, H_kv, D, splits=3, out=outs[3], ws=ws)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    x.copy_(torch.randn(M, K, device="cuda"))
    q.copy_(torch.randn(2 * H_q, D, device="cuda"))
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()                                   # warm-up outside the capture
        with torch.cuda.graph(g, stream=s):
            work()
    torch.cuda.synchronize()
    for rep in range(3):
        torch.manual_seed(100 + rep)
        x.copy_(torch.randn(M, K, device="cuda") * (1 + rep))
        q.copy_(torch.randn(2 * H_q, D, device="cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        for o in outs:
            o.fill_(float("nan"))                # eager work between replays
        work()
        torch.cuda.synchronize()
        for a, b in zip(got, outs):
            assert torch.equal(a, b), f"replay {rep} differs from the eager result"
