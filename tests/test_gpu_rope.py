"""GPU parity of RoPE (csah_rope, csah_kv_compress_rope, csah_kv_compress_paged_rope) against the
oracle's fp64 rotation.

csah_rope computes angles, sines, cosines and the rotation in fp64 and rounds once, as the oracle
does. Both sides take the angle p * base^(-2j/R) to within a few units of fp64 round-off of p (the
last-ulp error of base^(-2j/R), scaled by the position), so their turned values may differ by
(p + 1) 2^-48 times the pair's size. bf16 rows must match the oracle's rounding bit for bit except
where the oracle's value lies within that bound of a rounding midpoint; f32 rows must lie within
half a binary32 ulp plus that bound of the oracle's value. Compression with RoPE pools in fp32 as
csah_kv_compress does; its rotated dims are checked with the pooling bound of both dims of their
pair plus the binary32 rounding of the rotation.
"""
import numpy as np
import pytest
import torch

import long_context_attention_03_amd as L
import oracle as O
from helpers import (angle_bound, assert_close, bf16_bits, check_bf16, check_f32,
                     check_rows_e4m3_bf16, check_rows_fp4, dev, gather_pages, oracle_bf16,
                     paginate, pooling_tolerance, rope_tolerance, say)
from long_context_attention_03_amd import synth

pytestmark = pytest.mark.gpu


def _q(shape, seed, bf16=True):
    d = synth.Draws(seed)
    return d.normal(shape, dtype=torch.bfloat16 if bf16 else torch.float32)


def _run_rope(x, pos, R, base=10000.0, inverse=False):
    xg = x.cuda().contiguous()
    pg = torch.from_numpy(np.asarray(pos, np.int64)).cuda()
    L.rope(xg, pg, R, base, inverse)
    torch.cuda.synchronize()
    return xg.cpu()


def test_decode_queries_bf16_at_1m():
    """16 sequences x 64 heads x 512 (the last 64 dims rotary), positions around 2^20."""
    x = _q((16, 1, 64, 512), 101)
    pos = 1048576 - 1 + np.arange(16, dtype=np.int64) * 977
    say("[rope] decode queries bf16 [16,1,64,512] R=64 at ~1M")
    got = bf16_bits(_run_rope(x, pos, 64))
    ref = O.rope(bf16_bits(x), pos, 64)
    np.testing.assert_array_equal(got[..., :448], bf16_bits(x)[..., :448])
    check_bf16(got[..., 448:], ref[..., 448:], angle_bound(x.float().numpy(), pos, 64),
                "rotary dims")


def test_prefill_queries_bf16():
    """One sequence's 4096-query chunk at position 2^20: rows (b, i) at pos + i."""
    x = _q((1, 4096, 64, 512), 102)
    pos = np.array([1048576], np.int64)
    say("[rope] prefill queries bf16 [1,4096,64,512] R=64")
    got = bf16_bits(_run_rope(x, pos, 64))
    ref = O.rope(bf16_bits(x), pos, 64)
    np.testing.assert_array_equal(got[..., :448], bf16_bits(x)[..., :448])
    check_bf16(got[..., 448:], ref[..., 448:], angle_bound(x.float().numpy(), pos, 64),
                "rotary dims")


def test_inverse_on_f32_attention_output():
    x = _q((16, 1, 64, 512), 103, bf16=False)
    pos = 1048576 + np.arange(16, dtype=np.int64) * 31
    say("[rope] inverse on f32 output [16,1,64,512]")
    got = _run_rope(x, pos, 64, inverse=True).numpy()
    ref = O.rope(x.numpy(), pos, 64, inverse=True)
    np.testing.assert_array_equal(got[..., :448], x.numpy()[..., :448])
    check_f32(got[..., 448:], ref[..., 448:], angle_bound(x.numpy(), pos, 64), "rotary dims")


def test_forward_then_inverse_restores_f32_rows():
    x = _q((2, 3, 8, 128), 104, bf16=False)
    pos = np.array([5, 2000000], np.int64)
    xg = x.cuda()
    pg = torch.from_numpy(pos).cuda()
    L.rope(xg, pg, 64)
    L.rope(xg, pg, 64, inverse=True)
    torch.cuda.synchronize()
    assert_close(xg.cpu().numpy(), x.numpy(), "round trip", atol=1e-6, rtol=1e-6)


@pytest.mark.parametrize("B,Q,H,D,R,bf16", [
    (3, 5, 4, 128, 64, True), (3, 5, 4, 128, 64, False), (2, 3, 1, 64, 64, True),
    (1, 2, 3, 1024, 1024, False), (2, 1, 8, 256, 2, True), (1, 7, 5, 96, 32, True),
    (4, 1, 64, 512, 128, False),
])
def test_shapes(B, Q, H, D, R, bf16):
    rng = np.random.default_rng(B * 1000 + Q * 100 + D + R)
    x = _q((B, Q, H, D), 105 + R, bf16)
    pos = rng.integers(0, 2 ** 31 - 64, size=B).astype(np.int64)
    pos[0] = 0
    say(f"[rope] shape B={B} Q={Q} H={H} D={D} R={R} bf16={bf16}")
    out = _run_rope(x, pos, R, base=500000.0)
    ref = O.rope(bf16_bits(x) if bf16 else x.numpy(), pos, R, base=500000.0)
    tol = angle_bound(x.float().numpy(), pos, R)
    if bf16:
        got = bf16_bits(out)
        np.testing.assert_array_equal(got[..., :D - R], bf16_bits(x)[..., :D - R])
        check_bf16(got[..., D - R:], ref[..., D - R:], tol, "rotary dims")
        # position 0 of sequence 0 is the identity rotation for query 0
        np.testing.assert_array_equal(got[0, 0], bf16_bits(x)[0, 0])
    else:
        got = out.numpy()
        np.testing.assert_array_equal(got[..., :D - R], x.numpy()[..., :D - R])
        check_f32(got[..., D - R:], ref[..., D - R:], tol, "rotary dims")


def test_bf16_special_values():
    """Rows whose turned values fall below the bf16 normal range (subnormal inputs), overflow it
    (inputs near the bf16 maximum) or are not finite: the same IEEE results as the oracle's fp64
    rotation rounded to bf16 (NaN compared as NaN, whatever its payload)."""
    rng = np.random.default_rng(9)
    H, D = 6, 64
    vals = np.zeros((1, 3, H, D), np.float32)
    vals[..., 0, :] = rng.normal(size=(1, 3, D)) * 1e-39           # subnormal range
    vals[..., 1, :] = rng.choice([-1, 1], size=(1, 3, D)) * 3.0e38  # turned values may overflow
    vals[..., 2, :] = rng.normal(size=(1, 3, D)) * 2.0 ** -120      # results near 2^-126
    vals[..., 3, :] = rng.normal(size=(1, 3, D))
    vals[..., 3, ::7] = np.inf
    vals[..., 4, :] = rng.normal(size=(1, 3, D))
    vals[..., 4, 1::9] = np.nan
    vals[..., 5, :] = 0.0
    vals[..., 5, ::2] = -0.0
    x = torch.from_numpy(vals).to(torch.bfloat16)
    pos = np.array([3], np.int64)
    say("[rope] bf16 special values")
    got = bf16_bits(_run_rope(x, pos, 64))
    ref = O.rope(bf16_bits(x), pos, 64)
    want = oracle_bf16(np.nan_to_num(ref, nan=0.0))
    nan_ref = np.isnan(ref)
    gv = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(np.isnan(gv), nan_ref)
    assert np.array_equal(got[~nan_ref], want[~nan_ref])


def test_no_rows_is_a_no_op():
    x = torch.empty((0, 1, 64, 512), dtype=torch.bfloat16, device="cuda")
    L.rope(x, torch.empty(0, dtype=torch.int64, device="cuda"), 64)
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------- compression
def _gpu_compress_rope(x, m, w, beta, fmt, tok, R, span=None, skip=0):
    rows, sc = L.kv_compress_rope(x.cuda(), m, dev(w), dev(beta), fmt,
                                  torch.from_numpy(np.asarray(tok, np.int64)).cuda(), R,
                                  span=span, skip=skip)
    torch.cuda.synchronize()
    return rows.cpu().numpy(), None if sc is None else sc.cpu().numpy()


@pytest.mark.parametrize("m", [1, 4, 128])
def test_compress_prefill_chunk_e4m3_bf16_rows(m):
    """The prefill chunk's caches (window rows m = 1, CSA m = 4, HCA m = 128) with RoPE at the
    chunk's position 2^20."""
    wl = synth.WORKLOADS["prefill"]
    raw = synth.raw_tokens(wl, 4096)
    x = raw["x"]
    w = raw["w_hca" if m == 128 else "w_csa"].numpy()
    beta = raw["b_hca" if m == 128 else "b_csa"].numpy()[:m]
    tok = np.array([1048576], np.int64)
    say(f"[kv_compress_rope] prefill chunk m={m} -> E4M3+bf16 rows, R=64")
    rows, _ = _gpu_compress_rope(x, m, w, beta, O.FMT_ROW_E4M3_BF16, tok, 64)
    ref = O.kv_compress(bf16_bits(x), O.DT_BF16, m, w, beta, O.FMT_ROW_E4M3_BF16, tok_pos=tok,
                        rope_dims=64)
    tol = rope_tolerance(pooling_tolerance(x.float().numpy(), m, ref["pre"]), ref["pre"], 512,
                          64)
    nd = check_rows_e4m3_bf16(rows, ref["rows"], ref["pre"], tol)
    say(f"  {nd} elements differ, all within fp32 round-off of a rounding midpoint")


def test_compress_indexer_keys_fp4():
    wl = synth.WORKLOADS["prefill"]
    raw = synth.raw_tokens(wl, 4096)
    xi = raw["xi"]
    w, beta = raw["w_idx"].numpy(), raw["b_idx"].numpy()
    tok = np.array([1048576], np.int64)
    say("[kv_compress_rope] indexer keys FP4, D=128, R=64")
    rows, sc = _gpu_compress_rope(xi, 4, w, beta, O.FMT_FP4_E8M0, tok, 64)
    ref = O.kv_compress(xi.numpy(), O.DT_F32, 4, w, beta, O.FMT_FP4_E8M0, tok_pos=tok,
                        rope_dims=64)
    tol = rope_tolerance(pooling_tolerance(xi.numpy(), 4, ref["pre"]), ref["pre"], 128, 64)
    nd = check_rows_fp4(rows, sc, ref["rows"], ref["scales"], ref["pre"], tol)
    say(f"  {nd} codes differ, all at a rounding midpoint")


@pytest.mark.parametrize("D,m,R", [(64, 4, 64), (64, 1, 16), (128, 4, 64), (256, 8, 64),
                                   (1024, 128, 64), (512, 32, 512)])
def test_compress_f32_rows(D, m, R):
    """Every lane layout: a pair across two lanes (D = 64), two to sixteen dims per lane, one
    wavefront per entry and four (m > 16)."""
    d = synth.Draws(200 + D + m)
    x = d.normal((3, 16 * m, D))
    w = d.normal((D,), 0.02).numpy()
    beta = d.normal((m,), 0.1).numpy()
    tok = np.array([0, 77777, 1 << 20], np.int64)
    say(f"[kv_compress_rope] f32 rows D={D} m={m} R={R}")
    rows, _ = _gpu_compress_rope(x, m, w, beta, O.FMT_ROW_F32, tok, R)
    ref = O.kv_compress(x.numpy(), O.DT_F32, m, w, beta, O.FMT_ROW_F32, tok_pos=tok, rope_dims=R)
    got = rows.view(np.float32).reshape(ref["pre"].shape)
    assert_close(got, ref["pre"], f"D={D} m={m} R={R}", atol=1e-4, rtol=1e-4)


def test_compress_overlapping_span_with_context_groups():
    """Entries of 8 tokens at stride 4 after one context group: entry g (of raw's groups g >= 1)
    sits at tok_pos + 4(g+1) - 1."""
    d = synth.Draws(300)
    x = d.normal((2, 4 * 65, 512), dtype=torch.bfloat16)
    w = d.normal((512,), 0.02).numpy()
    beta = d.normal((8,), 0.1).numpy()
    tok = np.array([1048576 - 4, 12], np.int64)
    say("[kv_compress_rope] span 8 stride 4, skip 1, E4M3+bf16")
    rows, _ = _gpu_compress_rope(x, 4, w, beta, O.FMT_ROW_E4M3_BF16, tok, 64, span=8, skip=1)
    ref = O.kv_compress(bf16_bits(x), O.DT_BF16, 4, w, beta, O.FMT_ROW_E4M3_BF16, span=8, skip=1,
                        tok_pos=tok, rope_dims=64)
    tol = rope_tolerance(pooling_tolerance(x.float().numpy(), 4, ref["pre"], span=8, skip=1),
                          ref["pre"], 512, 64)
    check_rows_e4m3_bf16(rows, ref["rows"], ref["pre"], tol)


def test_compress_paged_equals_contiguous():
    """RoPE compression into shuffled pages writes exactly the bytes of the contiguous call."""
    d = synth.Draws(301)
    B, T, m, P = 3, 4 * 300, 4, 16
    x = d.normal((B, T, 512), dtype=torch.bfloat16)
    w = d.normal((512,), 0.02).numpy()
    beta = d.normal((m,), 0.1).numpy()
    tok = np.array([1048576, 4096, 0], np.int64)
    rng = np.random.default_rng(5)
    say("[kv_compress_paged_rope] 300 entries per sequence into 16-entry pages")
    rows, _ = _gpu_compress_rope(x, m, w, beta, O.FMT_ROW_E4M3_BF16, tok, 64)
    first = 7
    S = first + T // m
    empty = np.full((B, S, 576), 0xAB, np.uint8)
    pool, table = paginate(empty, P, rng)
    pool_g = dev(pool)
    L.kv_compress_paged_rope(x.cuda(), m, dev(w), dev(beta), O.FMT_ROW_E4M3_BF16, pool_g,
                             dev(table), P, torch.from_numpy(tok).cuda(), 64, first_entry=first)
    torch.cuda.synchronize()
    got = gather_pages(pool_g.cpu().numpy(), table, S)
    np.testing.assert_array_equal(got[:, first:], rows)
    np.testing.assert_array_equal(got[:, :first], empty[:, :first])
