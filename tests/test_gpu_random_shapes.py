"""Randomised parity: every call on seeded random shapes inside the supported ranges (sequence,
query, head and entry counts, widths, group sizes, windows, sinks, positions near the start of
the sequence, contiguous and paged caches), each checked against the oracle. The seeds are fixed,
so every run sees the same cases."""
import numpy as np
import pytest
import torch

import long_context_attention_03_amd as L
import oracle as O
from helpers import (angle_bound, assert_close, check_bf16, check_f32, check_rows_e4m3_bf16,
                     check_rows_fp4, dev, gather_pages, paginate, pooling_tolerance,
                     rope_tolerance, say)

pytestmark = pytest.mark.gpu


def _bf16(rng, shape):
    x = torch.from_numpy(rng.normal(size=shape).astype(np.float32)).to(torch.bfloat16)
    return x, x.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("seed", range(40))
def test_index_topk_random(seed):
    rng = np.random.default_rng(1000 + seed)
    Q = int(rng.choice([1, 1, 2, 3, 5, 9, 15, 16, 21]))
    dI = 128 if Q >= 3 else int(rng.choice([32, 64, 128]))
    HI = int(rng.integers(1, 17))
    B = int(rng.integers(1, 4))
    N = int(rng.integers(1, 6000))
    k = int(rng.integers(1, 700))
    m = int(rng.choice([1, 2, 4, 8]))
    pos = rng.integers(0, N * m + 8, size=B).astype(np.int64)
    pos[0] = N * m - Q  # one sequence where the last query sees every entry
    kv = rng.normal(size=(B, N, dI))
    if rng.random() < 0.3:
        kv = np.round(kv)  # coarse keys: many ties
    kc, ks = O.encode_rows(kv, O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, Q, HI, dI)), O.FMT_FP4_E8M0)
    paged = rng.random() < 0.4
    say(f"[random index] seed={seed} B={B} Q={Q} HI={HI} dI={dI} N={N} k={k} m={m} paged={paged}")
    if paged:
        P = int(rng.choice([1, 4, 16, 64, 512]))
        pc, table = paginate(kc, P, np.random.default_rng(seed))
        ps, _ = paginate(ks, P, np.random.default_rng(seed))
        gi, gs = L.index_topk_paged(dev(qc), dev(qs), dev(pc), dev(ps), dev(table), P, N, dev(pos),
                                    m, k)
    else:
        gi, gs = L.index_topk(dev(qc), dev(qs), dev(kc), dev(ks), dev(pos), m, k)
    torch.cuda.synchronize()
    ri, rs, ex = O.index_topk(qc, qs, kc, ks, pos, m, k)
    assert ex.all()
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy()
    assert np.array_equal(gi, ri), f"{int((gi != ri).sum())} index mismatches"
    assert np.array_equal(gs, rs.astype(np.float32))


@pytest.mark.parametrize("seed", range(24))
def test_index_topk_random_mfma_scan(seed):
    """One or two queries per sequence with 128-dim keys and 1-4 indexer heads: the scan whose
    scores come from the scaled FP4 MFMA (heads as columns, zero columns past the head count)."""
    rng = np.random.default_rng(3000 + seed)
    Q = int(rng.choice([1, 2]))
    HI = int(rng.integers(1, 5))
    B = int(rng.integers(1, 5))
    N = int(rng.integers(1, 40000))
    k = int(rng.integers(1, 1500))
    m = int(rng.choice([1, 4, 8]))
    pos = rng.integers(0, N * m + 8, size=B).astype(np.int64)
    pos[0] = N * m - Q
    kv = rng.normal(size=(B, N, 128))
    if rng.random() < 0.3:
        kv = np.round(kv)
    kc, ks = O.encode_rows(kv, O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, Q, HI, 128)), O.FMT_FP4_E8M0)
    paged = rng.random() < 0.4
    say(f"[random mfma scan] seed={seed} B={B} Q={Q} HI={HI} N={N} k={k} m={m} paged={paged}")
    if paged:
        P = int(rng.choice([1, 16, 64, 256]))
        pc, table = paginate(kc, P, np.random.default_rng(seed))
        ps, _ = paginate(ks, P, np.random.default_rng(seed))
        gi, gs = L.index_topk_paged(dev(qc), dev(qs), dev(pc), dev(ps), dev(table), P, N, dev(pos),
                                    m, k)
    else:
        gi, gs = L.index_topk(dev(qc), dev(qs), dev(kc), dev(ks), dev(pos), m, k)
    torch.cuda.synchronize()
    ri, rs, ex = O.index_topk(qc, qs, kc, ks, pos, m, k)
    assert ex.all()
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy()
    assert np.array_equal(gi, ri), f"{int((gi != ri).sum())} index mismatches"
    assert np.array_equal(gs, rs.astype(np.float32))


@pytest.mark.parametrize("seed", range(30))
def test_attend_random(seed):
    rng = np.random.default_rng(2000 + seed)
    B = int(rng.integers(1, 4))
    Q = int(rng.choice([1, 1, 2, 4]))
    H = int(rng.choice([16, 24, 64, 72, 128]))
    D = 512
    N = int(rng.integers(1, 2500))
    w = int(rng.choice([0, 1, 17, 128]))
    k = int(rng.integers(1, 400))
    m = int(rng.choice([1, 4, 128]))
    pos = rng.integers(0, max(1, N * m), size=B).astype(np.int64)
    if w == 0:
        pos[:] = np.maximum(pos, m)  # keep some entries visible when there is no window
    with_sink = rng.random() < 0.7
    cache, _ = O.encode_rows(rng.normal(size=(B, N, D)), O.FMT_ROW_E4M3_BF16)
    win, _ = O.encode_rows(rng.normal(size=(B, max(w - 1 + Q, 1), D)), O.FMT_ROW_E4M3_BF16)
    q_t, q_bits = _bf16(rng, (B, Q, H, D))
    sink = rng.normal(size=H).astype(np.float32) if with_sink else None
    idx = rng.integers(-1, N, size=(B, Q, k)).astype(np.int32)  # repeats and empty slots
    scale = D ** -0.5
    paged = rng.random() < 0.4
    say(f"[random attend] seed={seed} B={B} Q={Q} H={H} N={N} w={w} k={k} m={m} sink={with_sink}"
        f" paged={paged}")
    qd, wd, pd, sd = q_t.cuda(), dev(win), dev(pos), None if sink is None else dev(sink)
    if paged:
        P = int(rng.choice([1, 8, 64]))
        pool, table = paginate(cache, P, np.random.default_rng(seed))
        o1, l1 = L.csa_attend_paged(qd, dev(pool), dev(table), P, N, dev(idx), wd, w, pd, sd,
                                    scale)
        o2, l2 = L.hca_attend_paged(qd, dev(pool), dev(table), P, N, m, wd, w, pd, sd, scale)
    else:
        cd = dev(cache)
        o1, l1 = L.csa_attend(qd, cd, dev(idx), wd, w, pd, sd, scale)
        o2, l2 = L.hca_attend(qd, cd, m, wd, w, pd, sd, scale)
    torch.cuda.synchronize()
    r1, rl1 = O.csa_attend(q_bits, cache, O.FMT_ROW_E4M3_BF16, idx, win, w, pos, sink, scale)
    r2, rl2 = O.hca_attend(q_bits, cache, O.FMT_ROW_E4M3_BF16, m, win, w, pos, sink, scale)
    assert_close(o1.cpu().numpy(), r1, "csa out")
    assert_close(l1.cpu().numpy(), rl1, "csa lse")
    assert_close(o2.cpu().numpy(), r2, "hca out")
    assert_close(l2.cpu().numpy(), rl2, "hca lse")


@pytest.mark.parametrize("seed", range(24))
def test_kv_compress_random(seed):
    rng = np.random.default_rng(3000 + seed)
    B = int(rng.integers(1, 4))
    m = int(rng.choice([1, 2, 3, 4, 8, 128]))
    span = m * int(rng.choice([1, 1, 2, 3]))
    skip = int(rng.integers(0, 3)) if span > m else 0
    G = int(rng.integers(1, 40))
    T = (G + skip) * m
    fmt = int(rng.choice([O.FMT_ROW_F32, O.FMT_ROW_E4M3_BF16, O.FMT_FP4_E8M0]))
    D = 512 if fmt == O.FMT_ROW_E4M3_BF16 else int(rng.choice([64, 128, 256, 512, 1024]))
    bf16_raw = rng.random() < 0.5
    say(f"[random compress] seed={seed} B={B} T={T} D={D} m={m} span={span} skip={skip} fmt={fmt}"
        f" bf16={bf16_raw}")
    w = rng.normal(0, 0.05, D).astype(np.float32)
    beta = rng.normal(0, 0.3, span).astype(np.float32)
    if bf16_raw:
        x_t, x_np = _bf16(rng, (B, T, D))
        xf = x_t.float().numpy()
        ref = O.kv_compress(x_np, O.DT_BF16, m, w, beta, fmt, span=span, skip=skip)
    else:
        xf = rng.normal(size=(B, T, D)).astype(np.float32)
        x_t = torch.from_numpy(xf)
        ref = O.kv_compress(xf, O.DT_F32, m, w, beta, fmt, span=span, skip=skip)
    rows, sc = L.kv_compress(x_t.cuda(), m, dev(w), dev(beta), fmt, span=span if span > m else None,
                             skip=skip)
    torch.cuda.synchronize()
    rows = rows.cpu().numpy()
    tol = pooling_tolerance(xf, m, ref["pre"], span=span, skip=skip)
    if fmt == O.FMT_ROW_F32:
        got = rows.view(np.float32).reshape(ref["pre"].shape)
        assert_close(got, ref["pre"], "pooled", atol=1e-4, rtol=1e-4)
    elif fmt == O.FMT_ROW_E4M3_BF16:
        check_rows_e4m3_bf16(rows, ref["rows"], ref["pre"], tol)
    else:
        check_rows_fp4(rows, sc.cpu().numpy(), ref["rows"], ref["scales"], ref["pre"], tol)


@pytest.mark.parametrize("seed", range(20))
def test_rope_random(seed):
    """csah_rope on random widths (vector and one-pair-per-thread kernels), heads, positions up
    to 2^31, bases, both directions and both row types."""
    rng = np.random.default_rng(4000 + seed)
    B, Q, H = int(rng.integers(1, 4)), int(rng.integers(1, 7)), int(rng.integers(1, 70))
    D = int(rng.choice([64, 96, 128, 200, 256, 512, 1024]))
    R = 2 * int(rng.integers(1, D // 2 + 1))
    if rng.random() < 0.5:
        R = min(D, 8 * int(rng.integers(1, 9)))  # whole 16-byte vectors
    bf16 = rng.random() < 0.6
    base = float(rng.choice([10000.0, 500000.0, 1e6, 2.5]))
    inverse = bool(rng.random() < 0.4)
    pos = rng.integers(0, 2 ** 31 - 64, size=B).astype(np.int64)
    if rng.random() < 0.5:
        pos = rng.integers(0, 1 << 21, size=B).astype(np.int64)
    say(f"[random rope] seed={seed} B={B} Q={Q} H={H} D={D} R={R} bf16={bf16} base={base} "
        f"inverse={inverse}")
    if bf16:
        x_t, x_np = _bf16(rng, (B, Q, H, D))
    else:
        x_np = rng.normal(size=(B, Q, H, D)).astype(np.float32)
        x_t = torch.from_numpy(x_np)
    xg = x_t.cuda()
    L.rope(xg, torch.from_numpy(pos).cuda(), R, base, inverse)
    torch.cuda.synchronize()
    out = xg.cpu()
    ref = O.rope(x_np, pos, R, base, inverse)
    tol = angle_bound(x_t.float().numpy(), pos, R)
    if bf16:
        got = out.view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got[..., :D - R], x_np[..., :D - R])
        check_bf16(got[..., D - R:], ref[..., D - R:], tol, "rotary dims")
    else:
        got = out.numpy()
        assert np.array_equal(got[..., :D - R], x_np[..., :D - R])
        check_f32(got[..., D - R:], ref[..., D - R:], tol, "rotary dims")


@pytest.mark.parametrize("seed", range(16))
def test_kv_compress_rope_random(seed):
    """csah_kv_compress_rope / csah_kv_compress_paged_rope on random group sizes, spans, context
    groups, widths, rotary widths, positions and formats."""
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 4))
    m = int(rng.choice([1, 2, 4, 8, 128]))
    span = m * int(rng.choice([1, 1, 2]))
    skip = int(rng.integers(0, 3)) if span > m else 0
    G = int(rng.integers(1, 30))
    T = (G + skip) * m
    fmt = int(rng.choice([O.FMT_ROW_F32, O.FMT_ROW_E4M3_BF16, O.FMT_FP4_E8M0]))
    D = 512 if fmt == O.FMT_ROW_E4M3_BF16 else int(rng.choice([64, 128, 256, 512, 1024]))
    R = 64 if fmt == O.FMT_ROW_E4M3_BF16 and rng.random() < 0.6 else 2 * int(rng.integers(1, D // 2 + 1))
    base = float(rng.choice([10000.0, 1e6]))
    tok = rng.integers(0, 1 << 22, size=B).astype(np.int64)
    paged = rng.random() < 0.3
    say(f"[random compress rope] seed={seed} B={B} T={T} D={D} m={m} span={span} skip={skip} "
        f"fmt={fmt} R={R} paged={paged}")
    w = rng.normal(0, 0.05, D).astype(np.float32)
    beta = rng.normal(0, 0.3, span).astype(np.float32)
    xf = rng.normal(size=(B, T, D)).astype(np.float32)
    ref = O.kv_compress(xf, O.DT_F32, m, w, beta, fmt, span=span, skip=skip, tok_pos=tok,
                        rope_dims=R, rope_base=base)
    x_g, tok_g = torch.from_numpy(xf).cuda(), torch.from_numpy(tok).cuda()
    if paged:
        P = int(rng.choice([1, 4, 16]))
        rb = L.row_bytes(fmt, D)
        empty = np.zeros((B, G, rb), np.uint8)
        pool, table = paginate(empty, P, rng)
        spool = None
        if fmt == O.FMT_FP4_E8M0:  # the scale pool shares the block table
            spool = dev(np.zeros((pool.shape[0], P, D // 32), np.uint8))
        pool_g = dev(pool)
        L.kv_compress_paged_rope(x_g, m, dev(w), dev(beta), fmt, pool_g, dev(table), P, tok_g, R,
                                 base, scale_pool=spool, span=span if span > m else None,
                                 skip=skip)
        torch.cuda.synchronize()
        rows = gather_pages(pool_g.cpu().numpy(), table, G)
        sc = None if spool is None else gather_pages(spool.cpu().numpy(), table, G)
    else:
        rows_t, sc_t = L.kv_compress_rope(x_g, m, dev(w), dev(beta), fmt, tok_g, R, base,
                                          span=span if span > m else None, skip=skip)
        torch.cuda.synchronize()
        rows, sc = rows_t.cpu().numpy(), None if sc_t is None else sc_t.cpu().numpy()
    tol = rope_tolerance(pooling_tolerance(xf, m, ref["pre"], span=span, skip=skip), ref["pre"],
                         D, R)
    if fmt == O.FMT_ROW_F32:
        got = rows.view(np.float32).reshape(ref["pre"].shape)
        assert_close(got, ref["pre"], "pooled and turned", atol=1e-4, rtol=1e-4)
    elif fmt == O.FMT_ROW_E4M3_BF16:
        check_rows_e4m3_bf16(rows, ref["rows"], ref["pre"], tol)
    else:
        check_rows_fp4(rows, sc, ref["rows"], ref["scales"], ref["pre"], tol)
