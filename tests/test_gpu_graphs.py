"""The decode step captured as one HIP graph with two branches, as the benchmark replays it: the
CSA layer (kv_compress of the newest group into the row cache and the indexer keys, index_topk,
csa_attend) on the capturing stream and the HCA layer (kv_compress at m = 128, hca_attend) on a
second stream. Every replay, with the program's own eager work and synchronisations between
replays and every output overwritten before it, must give bitwise the eager results."""
import pytest
import torch

import long_context_attention_03_amd as L
from long_context_attention_03_amd import synth
from helpers import say

pytestmark = pytest.mark.gpu


def test_two_branch_step_graph_replays_match_eager():
    dev = torch.device("cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    # 4 sequences at 131,072 tokens: 32,768 CSA entries, 1,024 HCA entries, top-1024
    B, CTX, HI, dI, k, H, D, W = 4, 131072, 4, 128, 1024, 64, 512, 128
    N, NH = CTX // 4, CTX // 128

    def rnd_bytes(shape, lo, hi):
        return torch.randint(lo, hi, shape, dtype=torch.uint8, device=dev, generator=g)

    kc, ks = rnd_bytes((B, N, dI // 2), 0, 256), rnd_bytes((B, N, dI // 32), 124, 129)
    iqc, iqs = rnd_bytes((B, 1, HI, dI // 2), 0, 256), rnd_bytes((B, 1, HI, dI // 32), 125, 128)
    rows = rnd_bytes((B, N, 576), 0, 256) & 0x77  # finite E4M3 bytes and bf16 values
    hrows = rnd_bytes((B, NH, 576), 0, 256) & 0x77
    win, hwin = rnd_bytes((B, W, 576), 0, 256) & 0x77, rnd_bytes((B, W, 576), 0, 256) & 0x77
    q = torch.randn((B, 1, H, D), generator=g, device=dev).to(torch.bfloat16)
    hq = torch.randn((B, 1, H, D), generator=g, device=dev).to(torch.bfloat16)
    sink = torch.randn((H,), generator=g, device=dev)
    pos = torch.full((B,), CTX - 1, dtype=torch.int64, device=dev)
    d = synth.Draws(78, dev)
    xt, xit = d.normal((B, 4, D), dtype=torch.bfloat16), d.normal((B, 4, dI))
    hxt = d.normal((B, 128, D), dtype=torch.bfloat16)
    w_csa, b_csa = synth.compressor_params(D, 4, d)
    w_idx, b_idx = synth.compressor_params(dI, 4, d)
    w_hca, b_hca = synth.compressor_params(D, 128, d)

    idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    o, lse = torch.empty((B, 1, H, D), device=dev), torch.empty((B, 1, H), device=dev)
    ho, hlse = torch.empty((B, 1, H, D), device=dev), torch.empty((B, 1, H), device=dev)
    ws_idx = torch.empty(L.index_topk_workspace(B, 1, N, k, HI, dI), dtype=torch.uint8, device=dev)
    ws_csa = torch.empty(max(256, L.attend_workspace(B, 1, H, D, k + W)), dtype=torch.uint8,
                         device=dev)
    ws_hca = torch.empty(max(256, L.attend_workspace(B, 1, H, D, NH + W)), dtype=torch.uint8,
                         device=dev)
    side = torch.cuda.Stream()
    scale = D ** -0.5

    def csa_layer():
        L.kv_compress(xt, 4, w_csa, b_csa, L.FMT_ROW_E4M3_BF16, out_rows=rows[:, N - 1:N])
        L.kv_compress(xit, 4, w_idx, b_idx, L.FMT_FP4_E8M0, out_rows=kc[:, N - 1:N],
                      out_scales=ks[:, N - 1:N])
        L.index_topk(iqc, iqs, kc, ks, pos, 4, k, want_scores=False, ws=ws_idx, idx_out=idx)
        L.csa_attend(q, rows, idx, win, W, pos, sink, scale, ws=ws_csa, out=o, lse=lse)

    def hca_layer():
        L.kv_compress(hxt, 128, w_hca, b_hca, L.FMT_ROW_E4M3_BF16, out_rows=hrows[:, NH - 1:NH])
        L.hca_attend(hq, hrows, 128, hwin, W, pos, sink, scale, ws=ws_hca, out=ho, lse=hlse)

    def step():
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        csa_layer()
        with torch.cuda.stream(side):
            hca_layer()
        cur.wait_stream(side)

    say("[graphs] eager step: 4 x 131072 tokens, CSA + HCA layers on two streams")
    step()
    torch.cuda.synchronize()
    written = (rows[:, N - 1:N], kc[:, N - 1:N], ks[:, N - 1:N], hrows[:, NH - 1:NH])
    outs = (idx, o, lse, ho, hlse)
    ref = [t.clone() for t in written + outs]
    assert (idx >= 0).all()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    names = ["rows entry", "key codes entry", "key scales entry", "hca entry", "idx", "csa out",
             "csa lse", "hca out", "hca lse"]
    for r in range(3):
        # eager work between replays: overwrite everything the graph writes, and run the library
        # eagerly on other inputs
        for t in written:
            t.fill_(0x55)
        idx.fill_(-7)
        for t in (o, lse, ho, hlse):
            t.fill_(float("nan"))
        L.index_topk(iqc[:1], iqs[:1], kc[:1, :4096], ks[:1, :4096], pos[:1] // 32, 4, 64)
        torch.cuda.synchronize()
        say(f"[graphs] replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, ref, written + outs):
            a = a.view(torch.int32) if a.dtype == torch.float32 else a
            b = b.view(torch.int32) if b.dtype == torch.float32 else b
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager step"
