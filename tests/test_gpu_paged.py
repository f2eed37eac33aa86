"""GPU parity of the paged-cache calls: caches scattered over a shuffled page pool, read and
written through a block table. Each result must match the oracle on the logical cache (indices and
scores bit-exact, attention within atol = rtol = 1e-3) and be bit-identical to the contiguous
call's result on the same cache."""
import numpy as np
import pytest
import torch

import long_context_attention_03_amd as L
import oracle as O
from helpers import (DecodeCase, assert_close, bf16_bits, check_rows_e4m3_bf16, check_rows_fp4,
                     dev, gather_pages, paginate, pooling_tolerance, say)
from long_context_attention_03_amd import synth

pytestmark = pytest.mark.gpu


# ---- indexer -------------------------------------------------------------------------------
def _index_both(kc, ks, qc, qs, pos, m, k, P, seed):
    rng = np.random.default_rng(seed)
    N = kc.shape[1]
    pool_c, table = paginate(kc, P, rng)
    pool_s, _ = paginate(ks, P, np.random.default_rng(seed))  # same draws: same table
    gi, gs = L.index_topk_paged(dev(qc), dev(qs), dev(pool_c), dev(pool_s), dev(table), P, N,
                                dev(pos), m, k)
    ci, cs = L.index_topk(dev(qc), dev(qs), dev(kc), dev(ks), dev(pos), m, k)
    torch.cuda.synchronize()
    return gi.cpu().numpy(), gs.cpu().numpy(), ci.cpu().numpy(), cs.cpu().numpy()


def _check_index(name, kc, ks, qc, qs, pos, m, k, P, seed=0):
    say(f"[index_topk_paged] {name}: B={qc.shape[0]} Q={qc.shape[1]} N={kc.shape[1]} k={k} P={P}")
    gi, gs, ci, cs = _index_both(kc, ks, qc, qs, pos, m, k, P, seed)
    assert np.array_equal(gi, ci) and np.array_equal(gs, cs), "paged differs from contiguous"
    ri, rs, ex = O.index_topk(qc, qs, kc, ks, pos, m, k)
    assert ex.all()
    assert np.array_equal(gi, ri), f"{name}: {int((gi != ri).sum())} index mismatches"
    assert np.array_equal(gs, rs.astype(np.float32)), f"{name}: score mismatch"
    return ri


@pytest.mark.parametrize("P", [1, 16, 64, 4096])
def test_index_decode_page_sizes(P):
    """One query per sequence (the VALU scan). P = 4096 is larger than a scan chunk, so chunks
    start inside a page; P = 1 puts every entry on its own page."""
    rng = np.random.default_rng(80 + P)
    B, N, m, k = 3, 9001, 4, 512
    kc, ks = O.encode_rows(rng.normal(size=(B, N, 128)), O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, 1, 4, 128)), O.FMT_FP4_E8M0)
    pos = np.array([N * m - 1, 4 * 3000 + 2, 4 * 700 - 1], np.int64)
    _check_index("decode", kc, ks, qc, qs, pos, m, k, P, seed=P)


def test_index_decode_one_entry_pages_1m_keys():
    """One entry per page over 1,048,576 keys: a scan range may span at most 1024 pages, so the
    decode schedule runs its largest number of ranges (1024, with the shortest published lists)."""
    rng = np.random.default_rng(83)
    B, N, m, k = 1, 1 << 20, 4, 1024
    kc, ks = O.encode_rows(rng.normal(size=(B, N, 128)), O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, 1, 4, 128)), O.FMT_FP4_E8M0)
    pos = np.array([N * m - 1], np.int64)
    _check_index("decode P=1 1M", kc, ks, qc, qs, pos, m, k, 1, seed=3)


@pytest.mark.parametrize("P", [4, 128])
def test_index_multi_query_page_sizes(P):
    """5 queries per sequence (one MFMA pass over paged keys, scores stored)."""
    rng = np.random.default_rng(70 + P)
    B, Q, N, m, k = 2, 5, 20000, 4, 256
    kc, ks = O.encode_rows(rng.normal(size=(B, N, 128)), O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, Q, 4, 128)), O.FMT_FP4_E8M0)
    pos = np.array([N * m - Q, 4 * 9000 - 3], np.int64)
    _check_index("multi-query", kc, ks, qc, qs, pos, m, k, P, seed=P)


@pytest.mark.parametrize("P", [8, 256])
def test_index_prefill_schedule_page_sizes(P):
    """40 queries per sequence (the scaled-FP4-MFMA schedule); P = 8 shrinks the key ranges to
    1024 pages each."""
    rng = np.random.default_rng(90 + P)
    B, Q, N, m, k = 2, 40, 40000, 4, 256
    kc, ks = O.encode_rows(rng.normal(size=(B, N, 128)), O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, Q, 4, 128)), O.FMT_FP4_E8M0)
    pos = np.array([N * m - Q - 37, 4 * 20000 - 1], np.int64)
    _check_index("prefill", kc, ks, qc, qs, pos, m, k, P, seed=P)


def test_index_prefill_tie_list_overflow_paged():
    """Prefill queries whose threshold bin overflows the tie list (zero query codes: every score
    ties), finished by the re-scan through the block table, next to ordinary queries."""
    rng = np.random.default_rng(97)
    B, Q, N, m, k = 2, 32, 20000, 4, 500
    kc, ks = O.encode_rows(rng.normal(size=(B, N, 128)), O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, Q, 4, 128)), O.FMT_FP4_E8M0)
    qc[:, 20:] = 0
    pos = np.array([N * m - Q, 4 * 12000 - 1], np.int64)
    _check_index("prefill overflow", kc, ks, qc, qs, pos, m, k, 16, seed=97)


# ---- attention -----------------------------------------------------------------------------
def _pages(c, P, seed):
    pool, table = paginate(c.cache, P, np.random.default_rng(seed))
    return dev(pool), dev(table)


def _idx(B, Q, N, k, seed, empty_frac=0.1):
    rng = np.random.default_rng(seed)
    idx = np.stack([np.stack([rng.permutation(N)[:k] for _ in range(Q)]) for _ in range(B)])
    idx = idx.astype(np.int32)
    idx[rng.random(idx.shape) < empty_frac] = -1
    return idx


def _csa_both(c, idx, P, seed):
    q, cache, win, pos, sink = c.gpu("q", "cache", "window", "pos", "sink")
    pool, table = _pages(c, P, seed)
    ix = dev(idx)
    o, l = L.csa_attend_paged(q, pool, table, P, c.N, ix, win, c.wl.w, pos, sink, c.scale)
    co, cl = L.csa_attend(q, cache, ix, win, c.wl.w, pos, sink, c.scale)
    torch.cuda.synchronize()
    o, l, co, cl = (t.cpu().numpy() for t in (o, l, co, cl))
    assert np.array_equal(o, co) and np.array_equal(l, cl), "paged differs from contiguous"
    return o, l


def _hca_both(c, m, P, seed):
    q, cache, win, pos, sink = c.gpu("q", "cache", "window", "pos", "sink")
    pool, table = _pages(c, P, seed)
    o, l = L.hca_attend_paged(q, pool, table, P, c.N, m, win, c.wl.w, pos, sink, c.scale)
    co, cl = L.hca_attend(q, cache, m, win, c.wl.w, pos, sink, c.scale)
    torch.cuda.synchronize()
    o, l, co, cl = (t.cpu().numpy() for t in (o, l, co, cl))
    assert np.array_equal(o, co) and np.array_equal(l, cl), "paged differs from contiguous"
    return o, l


@pytest.mark.parametrize("P", [1, 32])
def test_csa_attend_paged(P):
    """Three queries per sequence with causal windows, 10 % empty slots, early positions."""
    c = DecodeCase("csa128k", B=3, N=5000, Q=3, pos=[4 * 5000 - 3, 300, 60])
    say(f"[csa_attend_paged] B={c.B} Q=3 N={c.N} P={P}")
    idx = _idx(c.B, 3, c.N, c.wl.k, 100 + P)
    o, l = _csa_both(c, idx, P, P)
    ro, rl = O.csa_attend(c.q, c.cache, c.fmt, idx, c.window, c.wl.w, c.pos, c.sink, c.scale)
    assert_close(o, ro, "paged csa out")
    assert_close(l, rl, "paged csa lse")


@pytest.mark.parametrize("P", [4, 64])
def test_hca_attend_paged(P):
    """Dense attention over a paged HCA cache, one sequence seeing only part of it."""
    c = DecodeCase("hca1m", B=3, N=3000, Q=2, pos=[128 * 3000 - 2, 128 * 1234 + 5, 100])
    say(f"[hca_attend_paged] B={c.B} Q=2 N={c.N} P={P}")
    o, l = _hca_both(c, 128, P, P)
    ro, rl = O.hca_attend(c.q, c.cache, c.fmt, 128, c.window, c.wl.w, c.pos, c.sink, c.scale)
    assert_close(o, ro, "paged hca out")
    assert_close(l, rl, "paged hca lse")


@pytest.mark.parametrize("P", [16])
def test_hca_attend_paged_prefill_grid(P):
    """512 queries of one sequence over about 3,000 paged entries: one split of 98 tiles per
    query on 512 workgroups, the two-per-CU build that leaves the lo term of P out of tiles whose
    weights are all small. Paged equals contiguous bit for bit; sampled queries match the oracle."""
    Q = 512
    c = DecodeCase("hca1m", B=1, N=3000, Q=Q, pos=128 * 3000 - Q)
    say(f"[hca_attend_paged] prefill grid B=1 Q={Q} N={c.N} P={P}")
    o, l = _hca_both(c, 128, P, P)
    w = c.wl.w
    for i in (0, 1, 127, 128, 300, Q - 1):
        ro, rl = O.hca_attend(c.q[:, i:i + 1], c.cache, c.fmt, 128, c.window[:, i:i + w], w,
                              c.pos + i, c.sink, c.scale)
        assert_close(o[:, i:i + 1], ro, f"paged hca prefill grid out, query {i}")
        assert_close(l[:, i:i + 1], rl, f"paged hca prefill grid lse, query {i}")


def test_fp32_rows_paged():
    """The tiny fp32-row configuration (D = 128) through both paged attention calls."""
    c = DecodeCase("tiny")
    say("[attend_paged] tiny fp32 rows P=8")
    idx = _idx(c.B, 1, c.N, c.wl.k, 7)
    o, l = _csa_both(c, idx, 8, 8)
    ro, rl = O.csa_attend(c.q, c.cache, c.fmt, idx, c.window, c.wl.w, c.pos, c.sink, c.scale)
    assert_close(o, ro, "tiny paged csa out")
    assert_close(l, rl, "tiny paged csa lse")
    h = DecodeCase("tiny", N=32)
    h.pos = np.array([4095], np.int64)
    o, l = _hca_both(h, 128, 8, 9)
    ro, rl = O.hca_attend(h.q, h.cache, h.fmt, 128, h.window, h.wl.w, h.pos, h.sink, h.scale)
    assert_close(o, ro, "tiny paged hca out")
    assert_close(l, rl, "tiny paged hca lse")


def test_csa_decode_1m_full_size_paged():
    """The 1M CSA decode step with every cache paged (64 entries = 256 tokens per page): indexer
    over 4 x 262,144 FP4 keys, top-1024, then sparse attention of 64 heads."""
    c = DecodeCase("csa1m")
    P = 64
    say(f"[paged 1M] B={c.B} N={c.N} P={P}")
    ri = _check_index("csa1m", c.kc, c.ks, c.qc, c.qs, c.pos, c.m, c.wl.k, P, seed=11)
    o, l = _csa_both(c, ri, P, 12)
    ro, rl = O.csa_attend(c.q, c.cache, c.fmt, ri, c.window, c.wl.w, c.pos, c.sink, c.scale)
    assert_close(o, ro, "csa1m paged out")
    assert_close(l, rl, "csa1m paged lse")


# ---- compression into pages -----------------------------------------------------------------
def test_kv_compress_into_pages():
    """Entries appended from logical entry 100 (inside a page) of a 64-entry-page cache: the
    prefill chunk's E4M3 rows (m = 4, and 8-token entries at stride 4) and FP4 keys. Rows land
    where the table says, match the contiguous call byte for byte, and nothing else is touched."""
    wl = synth.WORKLOADS["prefill"]
    raw = synth.raw_tokens(wl, 4096)
    x, xi = raw["x"], raw["xi"]
    P, first, S = 64, 100, 100 + 1024 + 60
    rng = np.random.default_rng(5)
    say(f"[kv_compress_paged] prefill chunk -> pages of {P} from entry {first}")
    for span in (None, 8):
        skip = 0 if span is None else 1
        G = 4096 // 4 - skip
        beta = raw["b_csa"].numpy() if span is None else rng.normal(0, 0.1, 8).astype(np.float32)
        blank = np.full((1, S, 576), 0xAB, np.uint8)
        pool, table = paginate(blank, P, np.random.default_rng(span or 4), fill=0xCD)
        pool_t = dev(pool)
        L.kv_compress_paged(x.cuda(), 4, dev(raw["w_csa"].numpy()), dev(beta),
                            O.FMT_ROW_E4M3_BF16, pool_t, dev(table), P, first, span=span,
                            skip=skip)
        ref_rows, _ = L.kv_compress(x.cuda(), 4, dev(raw["w_csa"].numpy()), dev(beta),
                                    O.FMT_ROW_E4M3_BF16, span=span, skip=skip)
        torch.cuda.synchronize()
        got_pool = pool_t.cpu().numpy()
        got = gather_pages(got_pool, table, S)
        assert np.array_equal(got[:, first:first + G], ref_rows.cpu().numpy())
        assert (got[:, :first] == 0xAB).all() and (got[:, first + G:] == 0xAB).all()
        used = np.zeros(pool.shape[0], bool)
        used[table.reshape(-1)] = True
        assert (got_pool[~used] == 0xCD).all(), "a page outside the table was written"
        ref = O.kv_compress(bf16_bits(x), O.DT_BF16, 4, raw["w_csa"].numpy(), beta,
                            O.FMT_ROW_E4M3_BF16, span=span, skip=skip)
        tol = pooling_tolerance(x.float().numpy(), 4, ref["pre"], span=span, skip=skip)
        check_rows_e4m3_bf16(got[:, first:first + G], ref["rows"], ref["pre"], tol)
    # FP4 indexer keys with their scale pool
    blank_c = np.zeros((1, S, 64), np.uint8)
    blank_s = np.zeros((1, S, 4), np.uint8)
    pc, table = paginate(blank_c, P, np.random.default_rng(3))
    ps, _ = paginate(blank_s, P, np.random.default_rng(3))
    pc_t, ps_t = dev(pc), dev(ps)
    L.kv_compress_paged(xi.cuda(), 4, dev(raw["w_idx"].numpy()), dev(raw["b_idx"].numpy()),
                        O.FMT_FP4_E8M0, pc_t, dev(table), P, first, scale_pool=ps_t)
    torch.cuda.synchronize()
    got_c = gather_pages(pc_t.cpu().numpy(), table, S)[:, first:first + 1024]
    got_s = gather_pages(ps_t.cpu().numpy(), table, S)[:, first:first + 1024]
    ref = O.kv_compress(xi.numpy(), O.DT_F32, 4, raw["w_idx"].numpy(), raw["b_idx"].numpy(),
                        O.FMT_FP4_E8M0)
    check_rows_fp4(got_c, got_s, ref["rows"], ref["scales"], ref["pre"],
                   pooling_tolerance(xi.numpy(), 4, ref["pre"]))
