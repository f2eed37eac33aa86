"""csah_csa_attend_noalloc (partials in the library's static scratch) against csah_csa_attend
(partials in a caller workspace): bitwise-equal outputs on two calls in a row, the second smaller,
and the clear error for a call that needs more scratch than there is."""
import pytest
import torch

import long_context_attention_03_amd as L
from helpers import say

pytestmark = pytest.mark.gpu


def _rows(shape, g):
    """N(0,1) values quantised to E4M3 + bf16 rows by the library (m = 1 is its quantiser)."""
    x = torch.randn(shape, generator=g, device="cuda")
    w = torch.zeros(shape[-1], device="cuda")
    beta = torch.zeros(1, device="cuda")
    rows, _ = L.kv_compress(x, 1, w, beta, L.FMT_ROW_E4M3_BF16)
    return rows


def _inputs(B, N, k, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    rows = _rows((B, N, 512), g)
    win = _rows((B, 128, 512), g)
    q = torch.randn((B, 1, 64, 512), generator=g, device="cuda").to(torch.bfloat16)
    sink = torch.randn((64,), generator=g, device="cuda")
    idx = torch.stack([torch.randperm(N, generator=g, device="cuda")[:k] for _ in range(B)])
    idx = idx.to(torch.int32).view(B, 1, k)
    idx[:, :, ::7] = -1  # some empty slots
    pos = torch.full((B,), 4 * N - 1, dtype=torch.int64, device="cuda")
    return rows, win, q, sink, idx, pos


def test_noalloc_matches_workspace_call_twice_second_smaller():
    for B, N, k, seed in ((16, 65536, 1024, 1), (3, 4096, 200, 2)):
        say(f"[csa_attend_noalloc] B={B} N={N} k={k}")
        rows, win, q, sink, idx, pos = _inputs(B, N, k, seed)
        need = L.attend_workspace(B, 1, 64, 512, k + 128)
        assert 0 < need <= L.NOALLOC_SCRATCH_BYTES
        o1, l1 = L.csa_attend(q, rows, idx, win, 128, pos, sink, 512 ** -0.5)
        o2, l2 = L.csa_attend_noalloc(q, rows, idx, win, 128, pos, sink, 512 ** -0.5)
        torch.cuda.synchronize()
        assert torch.isfinite(o1).all()
        assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), "out differs"
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "lse differs"


def test_noalloc_rejects_a_call_beyond_its_scratch():
    # 32 sequences split 8 ways: 32 x 8 x 64 partial rows of 2,064 bytes, more than 32 MiB
    B, Q, N, k = 32, 1, 2048, 1024
    need = L.attend_workspace(B, Q, 64, 512, k + 128)
    assert need > L.NOALLOC_SCRATCH_BYTES
    rows = torch.zeros((B, N, 576), dtype=torch.uint8, device="cuda")
    win = torch.zeros((B, 128, 576), dtype=torch.uint8, device="cuda")
    q = torch.zeros((B, Q, 64, 512), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((B, Q, k), dtype=torch.int32, device="cuda")
    pos = torch.full((B,), 4 * N - 1, dtype=torch.int64, device="cuda")
    out = torch.full((B, Q, 64, 512), 7.0, device="cuda")
    with pytest.raises(L.CsahError) as e:
        L.csa_attend_noalloc(q, rows, idx, win, 128, pos, None, 1.0, out=out)
    assert e.value.status == L.SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert (out == 7.0).all()  # nothing was enqueued
