"""GPU parity of csah_index_topk against the oracle: indices and scores must be bit-exact."""
import numpy as np
import pytest
import torch

import long_context_attention_03_amd as L
import oracle as O
from helpers import DecodeCase, dev, say

pytestmark = pytest.mark.gpu


def _run(case_kc, case_ks, qc, qs, pos, m, k, N=None):
    idx, sc = L.index_topk(dev(qc), dev(qs), dev(case_kc), dev(case_ks), dev(pos), m, k, N=N)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def _compare(name, kc, ks, qc, qs, pos, m, k, N=None):
    say(f"[index_topk] {name}: B={qc.shape[0]} Q={qc.shape[1]} N={kc.shape[1]} k={k}")
    gi, gs = _run(kc, ks, qc, qs, pos, m, k, N)
    ri, rs, ex = O.index_topk(qc, qs, kc, ks, pos, m, k, N=N)
    assert ex.all(), "inputs outside the fp32-exact domain"
    assert np.array_equal(gi, ri), f"{name}: {int((gi != ri).sum())} index mismatches"
    assert np.array_equal(gs, rs.astype(np.float32)), f"{name}: score mismatch"


def test_tiny_workload():
    c = DecodeCase("tiny")
    _compare("tiny", c.kc, c.ks, c.qc, c.qs, c.pos, c.m, c.wl.k)


def test_csa128k_shape_subset():
    c = DecodeCase("csa128k", B=4)
    _compare("csa128k B=4", c.kc, c.ks, c.qc, c.qs, c.pos, c.m, c.wl.k)


def test_csa1m_full_size():
    """The 1M-context CSA decode step at its full size: 4 x 262,144 entries, top-1024."""
    c = DecodeCase("csa1m")
    _compare("csa1m full", c.kc, c.ks, c.qc, c.qs, c.pos, c.m, c.wl.k)


def test_decode_step_launch_shape_16_sequences():
    """The index call as the decode step runs it: 16 sequences x 262,144 entries, top-1024 (the
    candidate-list scan with 2048-key ranges over 2048 workgroups, then one top-k workgroup per
    sequence). Codes are random bytes and scales a narrow band, which keeps every score exact."""
    rng = np.random.default_rng(22)
    B, N, HI, dI, m, k = 16, 262144, 4, 128, 4, 1024
    kc = rng.integers(0, 256, size=(B, N, dI // 2), dtype=np.uint8)
    ks = rng.integers(124, 129, size=(B, N, dI // 32), dtype=np.uint8)
    qc = rng.integers(0, 256, size=(B, 1, HI, dI // 2), dtype=np.uint8)
    qs = rng.integers(125, 128, size=(B, 1, HI, dI // 32), dtype=np.uint8)
    pos = np.full(B, N * m - 1, np.int64)
    pos[3] -= m * 5000  # one sequence sees fewer entries
    _compare("decode-step shape", kc, ks, qc, qs, pos, m, k)


def test_long_key_ranges_several_stage_windows():
    """2 x (2^22 + 777) keys, beyond the candidate-list schedule's 2^22 per sequence, so the
    stored-score schedule runs: each scan workgroup streams 17,408 keys, four full 4096-score
    stage windows and a partial one; the last range of each sequence is ragged,
    and the second sequence sees 999 groups fewer. Codes and scales are random bytes (scales in a
    narrow band keep every score exact)."""
    rng = np.random.default_rng(12)
    B, N, HI, dI, m, k = 2, (1 << 22) + 777, 4, 128, 4, 1024
    kc = rng.integers(0, 256, size=(B, N, dI // 2), dtype=np.uint8)
    ks = rng.integers(124, 129, size=(B, N, dI // 32), dtype=np.uint8)
    qc = rng.integers(0, 256, size=(B, 1, HI, dI // 2), dtype=np.uint8)
    qs = rng.integers(125, 128, size=(B, 1, HI, dI // 32), dtype=np.uint8)
    pos = np.array([N * m - 1, N * m - 1 - m * 999], np.int64)
    _compare("long ranges", kc, ks, qc, qs, pos, m, k)


@pytest.mark.parametrize("HI,Q", [(4, 1), (5, 1), (4, 5), (6, 5)])
def test_clustered_top_entries_are_scored_again(HI, Q):
    """The relevant entries cluster. In sequence 0 the 1,500 entries from 30,000 on have every
    block scale raised by 2^4, so nearly all of the top-1024 lie in a few adjacent scan ranges,
    far more than any range publishes; sequence 1 has two such clusters, at the start and at the
    ragged end. The top-k kernel must score those ranges again. One query: 4 heads take the MFMA
    scan, 5 the vector scan; five queries take the multi-query pass, whose per-query lists the
    top-k re-scores with the one-query code (MFMA for 4 heads, vector for 6). Indices and scores
    stay bit-exact."""
    rng = np.random.default_rng(61 + HI + Q)
    B, N, dI, m, k = 2, 100003, 128, 4, 1024
    kc, ks = O.encode_rows(rng.normal(size=(B, N, dI)), O.FMT_FP4_E8M0)
    ks = ks.copy()
    ks[0, 30000:31500] += 4
    ks[1, :700] += 4
    ks[1, N - 800:] += 4
    qc, qs = O.encode_rows(rng.normal(size=(B, Q, HI, dI)), O.FMT_FP4_E8M0)
    pos = np.full(B, N * m - Q, np.int64)
    _compare(f"clustered HI={HI} Q={Q}", kc, ks, qc, qs, pos, m, k)


@pytest.mark.parametrize("Q,coarse", [(1, False), (1, True), (5, False), (16, False), (16, True)])
def test_largest_k(Q, coarse):
    """k = 4096, the largest supported: all three schedules (one query, the multi-query scan, the
    prefill schedule), and coarse keys whose tie list pushes the candidates of the last two past
    the 4096-key sort capacity onto the radix-select path."""
    rng = np.random.default_rng(40 + Q)
    B, N, HI, dI, m, k = 2, 70001, 4, 128, 4, 4096
    kv = rng.normal(size=(B, N, dI))
    if coarse:
        kv = np.round(kv * 0.7)
    kc, ks = O.encode_rows(kv, O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, Q, HI, dI)), O.FMT_FP4_E8M0)
    pos = np.array([N * m - Q, 4 * 5000 + 3], np.int64)  # the second sees about 5000 entries
    _compare(f"k=4096 Q={Q} coarse={coarse}", kc, ks, qc, qs, pos, m, k)


def test_ties_multi_query_causal_and_ragged():
    """Coarse keys (many equal scores), 3 queries per sequence with causal visibility, ragged N."""
    rng = np.random.default_rng(7)
    B, Q, N, HI, dI, m, k = 2, 3, 20011, 4, 128, 4, 1024
    kc, ks = O.encode_rows(np.round(rng.normal(size=(B, N, dI))), O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(np.round(rng.normal(size=(B, Q, HI, dI))), O.FMT_FP4_E8M0)
    pos = np.array([N * m - Q, 4 * 5000 + 1], np.int64)
    _compare("ties", kc, ks, qc, qs, pos, m, k)


def test_all_equal_scores_take_lowest_indices():
    """Zero keys: every score ties, so the top-k is the k lowest indices. No range can publish
    its one full bin, so every range's bound reaches the threshold and is scored again."""
    B, N, dI = 1, 50000, 64
    kc = np.zeros((B, N, dI // 2), np.uint8)
    ks = np.full((B, N, dI // 32), 127, np.uint8)
    rng = np.random.default_rng(8)
    qc, qs = O.encode_rows(rng.normal(size=(B, 1, 4, dI)), O.FMT_FP4_E8M0)
    pos = np.array([N * 4 - 1], np.int64)
    _compare("all-equal", kc, ks, qc, qs, pos, 4, 1000)
    gi, _ = _run(kc, ks, qc, qs, pos, 4, 1000)
    assert list(gi[0, 0]) == list(range(1000))


def test_fewer_visible_than_k_and_none_visible():
    rng = np.random.default_rng(9)
    B, N, dI = 3, 300, 128
    kc, ks = O.encode_rows(rng.normal(size=(B, N, dI)), O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, 1, 4, dI)), O.FMT_FP4_E8M0)
    pos = np.array([4 * 200 + 3, 2, 10 ** 6], np.int64)  # 201 visible, none, clamped to N
    _compare("short", kc, ks, qc, qs, pos, 4, 256)
    gi, gs = _run(kc, ks, qc, qs, pos, 4, 256)
    assert (gi[0, 0, 201:] == -1).all() and (gi[1, 0] == -1).all() and (gi[2, 0] >= 0).all()
    assert np.isneginf(gs[1, 0]).all()


def test_n_limits_visibility_below_stride():
    rng = np.random.default_rng(10)
    B, S, N, dI = 2, 4096, 3000, 64
    kc, ks = O.encode_rows(rng.normal(size=(B, S, dI)), O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, 1, 4, dI)), O.FMT_FP4_E8M0)
    pos = np.array([4 * S - 1, 4 * S - 1], np.int64)
    _compare("N<stride", kc, ks, qc, qs, pos, 4, 128, N=N)


@pytest.mark.parametrize("HI,dI", [(1, 128), (8, 64), (16, 32), (5, 128)])
def test_decode_head_counts_and_key_widths(HI, dI):
    """One query per sequence with other indexer shapes: heads beyond the first MFMA row group
    (summed across lane rows), and 64- / 32-dim keys (zero-padded operand blocks)."""
    rng = np.random.default_rng(40 + HI + dI)
    B, N, m, k = 3, 9001, 4, 512
    kc, ks = O.encode_rows(rng.normal(size=(B, N, dI)), O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, 1, HI, dI)), O.FMT_FP4_E8M0)
    pos = np.array([N * m - 1, 4 * 3000 + 2, 4 * 700 - 1], np.int64)
    _compare(f"decode HI={HI} dI={dI}", kc, ks, qc, qs, pos, m, k)


# ---- many queries per sequence (prefill chunks): the scaled-FP4-MFMA schedule ----------------
def _fp4_inputs(rng, B, Q, N, HI, dI=128, coarse=False):
    kv = rng.normal(size=(B, N, dI))
    kc, ks = O.encode_rows(np.round(kv) if coarse else kv, O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, Q, HI, dI)), O.FMT_FP4_E8M0)
    return kc, ks, qc, qs


@pytest.mark.parametrize("HI", [3, 4, 8])
def test_prefill_schedule_blocks_ranges_and_causality(HI):
    """40 queries (3 blocks of 16, the last partial) over 40,000 keys (3 key ranges, the last
    ragged); sequence 1's queries see 20,000..20,010 entries, so visibility changes inside a
    block. HI = 3 pads the MFMA operands with a zero head."""
    rng = np.random.default_rng(20 + HI)
    B, Q, N, m, k = 2, 40, 40000, 4, 256
    kc, ks, qc, qs = _fp4_inputs(rng, B, Q, N, HI)
    pos = np.array([N * m - Q - 37, 4 * 20000 - 1], np.int64)
    _compare(f"prefill HI={HI}", kc, ks, qc, qs, pos, m, k)


def test_prefill_schedule_ties_and_fewer_visible_than_k():
    """Coarse keys (many equal scores); the first queries see fewer entries than k."""
    rng = np.random.default_rng(31)
    B, Q, N, m, k = 1, 48, 2000, 4, 256
    kc, ks, qc, qs = _fp4_inputs(rng, B, Q, N, 4, coarse=True)
    pos = np.array([4 * 100 - 5], np.int64)  # query i sees floor((396 + i) / 4) = 99..110 entries
    _compare("prefill ties/short", kc, ks, qc, qs, pos, m, k)
    gi, _ = _run(kc, ks, qc, qs, pos, m, k)
    assert (gi[0, 0, 99:] == -1).all() and (gi[0, 0, :99] >= 0).all()


def test_prefill_schedule_all_equal_scores():
    """Zero keys: every one of the 20,000 keys reaches the estimate, more than the 8192-key list
    holds, so every query is finished by the re-scan (radix select on the index bits alone)."""
    rng = np.random.default_rng(32)
    B, Q, N, m, k = 1, 16, 20000, 4, 1000
    kc = np.zeros((B, N, 64), np.uint8)
    ks = np.full((B, N, 4), 127, np.uint8)
    qc, qs = O.encode_rows(rng.normal(size=(B, Q, 4, 128)), O.FMT_FP4_E8M0)
    pos = np.array([N * m - Q], np.int64)
    _compare("prefill all-equal", kc, ks, qc, qs, pos, m, k)
    gi, _ = _run(kc, ks, qc, qs, pos, m, k)
    assert (gi[0, :, :] == np.arange(k)).all()


def _one_bin_inputs(rng, B, Q, N, HI):
    """Scores that differ but share one 11-bit histogram bin: key block 0 is all 4.0 and query
    block 0 all 1.0, 128 per head, so each score starts at 128 HI (a power of two for HI = 4, 8);
    the other blocks add a non-negative term below 36 * 96 * HI / 256, under a quarter of that
    (positive codes, keys scaled by 2^-8), so every score lies in the first quarter of its
    binade: one bin."""
    kc = np.zeros((B, N, 64), np.uint8)
    kc[:, :, :16] = 0x66
    kc[:, :, 16:] = rng.integers(0, 8, size=(B, N, 48)) | (rng.integers(0, 8, size=(B, N, 48)) << 4)
    ks = np.full((B, N, 4), 119, np.uint8)
    ks[:, :, 0] = 127
    qc = np.zeros((B, Q, HI, 64), np.uint8)
    qc[..., :16] = 0x22
    qc[..., 16:] = rng.integers(0, 8, size=(B, Q, HI, 48)) | (rng.integers(0, 8, size=(B, Q, HI, 48)) << 4)
    qs = np.full((B, Q, HI, 4), 127, np.uint8)
    return kc, ks, qc, qs


@pytest.mark.parametrize("HI", [4, 8])
def test_prefill_tie_list_overflow_distinct_scores_in_one_bin(HI):
    """30,000 keys whose scores all fall in one 11-bit histogram bin, mostly distinct (with some
    ties): the threshold estimate and the ranking must split them on score bits, then on index
    bits. 20 queries (a partial second block) with causal visibility changing inside the
    blocks."""
    rng = np.random.default_rng(40 + HI)
    B, Q, N, m, k = 1, 20, 30000, 4, 1024
    kc, ks, qc, qs = _one_bin_inputs(rng, B, Q, N, HI)
    pos = np.array([N * m - Q - 37], np.int64)
    _compare(f"prefill one-bin HI={HI}", kc, ks, qc, qs, pos, m, k)


def test_prefill_tie_list_overflow_mixed_with_normal_queries():
    """Two sequences x 32 queries over 20,000 normal keys; in each sequence queries 16..31 have
    zero codes (every score 0: every key reaches the estimate and the list overflows) while
    queries 0..15 take the ordinary path, so both finishers run in one call."""
    rng = np.random.default_rng(43)
    B, Q, N, m, k = 2, 32, 20000, 4, 777
    kc, ks, qc, qs = _fp4_inputs(rng, B, Q, N, 4)
    qc[:, 16:] = 0
    pos = np.array([N * m - Q, 4 * 15000 - 1], np.int64)
    _compare("prefill overflow mixed", kc, ks, qc, qs, pos, m, k)


def _sampled_positions(nvmin: int) -> np.ndarray:
    """The keys the prefill schedule samples for a query block whose first query sees nvmin keys:
    64 segments of 128 keys spread evenly (all of them, contiguous, up to 8192)."""
    if nvmin <= 8192:
        return np.arange(nvmin)
    stride = nvmin // 64
    return (np.arange(64)[:, None] * stride + np.arange(128)[None, :]).ravel()


@pytest.mark.parametrize("sampled", ["high", "low"])
def test_prefill_estimate_misled_by_the_sample(sampled):
    """The threshold estimate comes from a sample of each query block's keys. Here the sampled
    keys are built to mislead it: scored above every other key ("high": the estimate lands far
    above the true kk-th key, too few candidates reach it) or below every other key ("low": nearly
    all keys reach it, more than the list holds). Either way the re-scan must finish every query
    exactly. 16 queries over 40,000 keys, 4 heads."""
    rng = np.random.default_rng(50 if sampled == "high" else 51)
    B, Q, N, m, k, HI = 1, 16, 40000, 4, 1024, 4
    kc, ks, qc, qs = _fp4_inputs(rng, B, Q, N, HI)
    pos = np.array([N * m - Q], np.int64)
    smp = _sampled_positions((N * m - Q + 1) // m)
    qc[..., :16] = 0x22  # query block 0 all 1.0: key block 0 decides the sampled keys' scores
    qs[..., 0] = 127
    kc[0, smp, :16] = 0x66 if sampled == "high" else 0xEE  # +4.0 or -4.0 throughout block 0
    ks[0, smp, 0] = 127
    _compare(f"prefill sample {sampled}", kc, ks, qc, qs, pos, m, k)


def test_prefill_chunk_full_size_sampled_queries():
    """The prefill chunk at full size: 4096 queries at positions 1,048,576 + i over 263,168 FP4
    keys (262,144 cached + 1,024 from the chunk), top-1024 each. All queries run on the GPU;
    sampled rows (chunk edges, group boundaries, random) are checked against the oracle, which
    scores one query at a time."""
    rng = np.random.default_rng(5)
    B, Q, N, m, k, HI = 1, 4096, 262144 + 1024, 4, 1024, 4
    kc, ks, qc, qs = _fp4_inputs(rng, B, Q, N, HI)
    pos0 = 1 << 20
    say(f"[index_topk] prefill full: Q={Q} N={N} k={k}")
    gi, gs = _run(kc, ks, qc, qs, np.array([pos0], np.int64), m, k)
    sample = sorted({0, 1, 2, 3, 4, 127, 128, 2047, 4094, 4095,
                     *rng.choice(Q, size=6, replace=False).tolist()})
    for i in sample:
        ri, rs, ex = O.index_topk(qc[:, i:i + 1], qs[:, i:i + 1], kc, ks,
                                  np.array([pos0 + i], np.int64), m, k)
        assert ex.all()
        assert np.array_equal(gi[:, i:i + 1], ri), f"query {i}: index mismatch"
        assert np.array_equal(gs[:, i:i + 1], rs.astype(np.float32)), f"query {i}: score mismatch"
    say(f"  {len(sample)} sampled queries bit-exact")


@pytest.mark.parametrize("HI,Q", [(4, 2), (8, 7), (16, 15), (3, 5)])
def test_multi_query_scan_shapes(HI, Q):
    """2 to 15 queries per sequence (one MFMA pass, stored scores): head counts that pad the MFMA
    operands, a ragged key count, and visibility that changes inside the query block (sequence 1's
    queries see 4,000..4,003 entries, fewer than k for none; sequence 2's see 50..53 < k)."""
    rng = np.random.default_rng(50 + HI + Q)
    B, N, m, k = 3, 30011, 4, 512
    kc, ks, qc, qs = _fp4_inputs(rng, B, Q, N, HI)
    pos = np.array([N * m - Q, 4 * 4000 - 2, 4 * 50 - 1], np.int64)
    _compare(f"multi-query HI={HI} Q={Q}", kc, ks, qc, qs, pos, m, k)


def test_multi_query_scan_ties():
    """Coarse keys (many equal scores) with 4 queries per sequence, and all-zero keys (every score
    ties: more candidates than the sort buffer)."""
    rng = np.random.default_rng(57)
    B, Q, N, m, k = 2, 4, 12000, 4, 1000
    kc, ks, qc, qs = _fp4_inputs(rng, B, Q, N, 4, coarse=True)
    pos = np.array([N * m - Q, 4 * 3000], np.int64)
    _compare("multi-query ties", kc, ks, qc, qs, pos, m, k)
    kz = np.zeros_like(kc)
    kzs = np.full_like(ks, 127)
    _compare("multi-query all-equal", kz, kzs, qc, qs, pos, m, k)
    gi, _ = _run(kz, kzs, qc, qs, pos, m, k)
    assert (gi[0] == np.arange(k)).all()


def test_multi_query_decode_1m_five_drafts():
    """Speculative verification: 5 query tokens per sequence at the end of a 1M context
    (positions L-5 .. L-1), 262,144 FP4 keys, top-1024 each; every query on the oracle."""
    rng = np.random.default_rng(60)
    B, Q, N, m, k = 2, 5, 262144, 4, 1024
    kc, ks, qc, qs = _fp4_inputs(rng, B, Q, N, 4)
    pos = np.full(B, N * m - Q, np.int64)
    _compare("decode Q=5 at 1M", kc, ks, qc, qs, pos, m, k)


def _sure_count(scores: np.ndarray, k: int, bin_shift: int = 20) -> tuple[int, int]:
    """(entries in histogram bins above the k-th largest score's bin, entries in that bin) for
    scores sorted descending; a bin is the top 32 - bin_shift bits of the score's order key."""
    u = scores.astype(np.float32).view(np.uint32)
    key = np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)
    b = key >> bin_shift
    t = b[k - 1]
    return int((b > t).sum()), int((b == t).sum())


def test_rank_sure_tie_boundaries():
    """One query per sequence (the candidate-list schedule) around the sure/tie boundaries of the
    stored-score ranking: cases put the boundary at every offset within a group of four, at 63, 0
    and 1 past a multiple of 64, at 0 and 1, and cut the tie bin at various points. The boundary
    is moved by raising the block scales of a few low-ranked keys by 2^10, which lifts them above
    every threshold. The multi-query test below reaches the ranking kernel itself."""
    rng = np.random.default_rng(21)
    B, N, HI, dI, m = 1, 24000, 4, 128, 4
    kc0, ks0 = O.encode_rows(rng.normal(size=(B, N, dI)), O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, 1, HI, dI)), O.FMT_FP4_E8M0)
    pos = np.array([N * m - 1], np.int64)
    order, _, _ = O.index_topk(qc, qs, kc0, ks0, pos, m, N)
    seen = []
    for lift, k in [(0, 1), (0, 3), (0, 20), (0, 100), (0, 500), (0, 1024), (51, 1075),
                    (52, 1076), (53, 1077), (0, 2000), (0, 2200), (0, 3900)]:
        ks = ks0.copy()
        ks[0, order[0, 0, 5000:5000 + lift]] += 10  # positive scores, ranked far below k
        _, rs, ex = O.index_topk(qc, qs, kc0, ks, pos, m, N)
        assert ex.all()
        ns, nt = _sure_count(rs[0, 0], k)
        assert ns + nt <= 4096, "the counting path, not the radix-select fallback"
        seen.append(ns)
        _compare(f"boundary ns={ns} nt={nt} k={k}", kc0, ks, qc, qs, pos, m, k)
    assert {s % 4 for s in seen} == {0, 1, 2, 3}
    assert {s % 64 for s in seen if s >= 64} >= {63, 0, 1}
    assert 0 in seen and 1 in seen


def test_multi_query_rank_sure_tie_boundaries():
    """The ranking kernel of the 3-15-query schedule counts entries above the threshold bin
    ("sure") and in it ("tie") separately and holds four candidates per lane group, 64 per
    workgroup. Three copies of one query (the last sees all 24,000 entries); cases are chosen from
    the oracle's own ranking so that the sure count lands on every offset within a group of four,
    on 63, 0 and 1 past a multiple of 64, and on 0 and 1 (2048-bin histogram: 11-bit bins). Lifting
    L low-ranked keys by 2^10 puts them above every threshold, so with k the sure count is L plus
    the original sure count at k - L."""
    rng = np.random.default_rng(23)
    B, Q, N, HI, dI, m = 1, 3, 24000, 4, 128, 4
    kc0, ks0 = O.encode_rows(rng.normal(size=(B, N, dI)), O.FMT_FP4_E8M0)
    q1c, q1s = O.encode_rows(rng.normal(size=(B, 1, HI, dI)), O.FMT_FP4_E8M0)
    qc, qs = np.repeat(q1c, Q, axis=1), np.repeat(q1s, Q, axis=1)
    pos = np.array([N * m - Q], np.int64)  # query 2 sees every entry, queries 0 and 1 one fewer
    last = np.array([N * m - 1], np.int64)
    order, rs0, _ = O.index_topk(q1c, q1s, kc0, ks0, last, m, 4096)
    u = rs0[0, 0].astype(np.float32).view(np.uint32)
    bins = (np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32) >> 21).astype(np.int64)
    sure = np.array([int((bins > bins[j]).sum()) for j in range(4096)])  # sure count at k = j + 1
    ties = np.array([int((bins == bins[j]).sum()) for j in range(4096)])
    want = {("mod4", r) for r in range(4)} | {("mod64", r) for r in (63, 0, 1)} | {("abs", 0), ("abs", 1)}
    cases = {}
    for k in range(1, 3000):
        for L in range(0, 64):
            j = k - L - 1
            if j < 0 or L + sure[j] + ties[j] > 4000:
                continue
            ns = L + int(sure[j])
            for tag in (("mod4", ns % 4), ("abs", ns)) + ((("mod64", ns % 64),) if ns >= 64 else ()):
                if tag in want and tag not in cases:
                    cases[tag] = (L, k)
        if len(cases) == len(want):
            break
    assert len(cases) == len(want), sorted(want - set(cases))
    # and wide tie bins cut at various points
    wide = [(0, k) for k in (500, 1024, 2000, 3500) if sure[k - 1] + ties[k - 1] <= 4000]
    seen = []
    for L, k in sorted(set(cases.values()) | set(wide)):
        ks = ks0.copy()
        ks[0, order[0, 0, 3000:3000 + L]] += 10  # positive scores, ranked far below k
        _, rs, ex = O.index_topk(q1c, q1s, kc0, ks, last, m, k)
        assert ex.all()
        ns, nt = _sure_count(rs[0, 0], k, bin_shift=21) if k < 4096 else (None, None)
        seen.append(ns)
        _compare(f"multi-query boundary L={L} k={k} ns={ns} nt={nt}", kc0, ks, qc, qs, pos, m, k)
    assert {s % 4 for s in seen} == {0, 1, 2, 3}
    assert {s % 64 for s in seen if s >= 64} >= {63, 0, 1}
    assert 0 in seen and 1 in seen


@pytest.mark.parametrize("HI", [4, 5])
def test_decode_scan_wide_exponent_range(HI):
    """Each key's four block scales shifted by the same offset in [-90, 90]: key magnitudes span
    2^-90 to 2^90, every score stays exact and in the fp32 normal range; k = N ranks (and
    compares) every score, the smallest included. 4 heads take the MFMA scan (E8M0 scales as
    MFMA operands), 5 the vector scan."""
    rng = np.random.default_rng(31)
    B, N, dI, m, k = 2, 4000, 128, 4, 4000
    kc, ks = O.encode_rows(rng.normal(size=(B, N, dI)), O.FMT_FP4_E8M0)
    off = rng.integers(-90, 91, size=(B, N, 1))
    ks = np.clip(ks.astype(np.int64) + off, 1, 254).astype(np.uint8)
    qc, qs = O.encode_rows(rng.normal(size=(B, 1, HI, dI)), O.FMT_FP4_E8M0)
    pos = np.array([N * m - 1, N * m // 2], np.int64)
    _compare(f"wide exponents HI={HI}", kc, ks, qc, qs, pos, m, k)


def test_many_sequences_small_caches():
    """700 sequences of 1,500 entries (one scan workgroup per sequence, 700 slots deep grids),
    causal positions drawn per sequence, 4 heads x 128 (the MFMA scan)."""
    rng = np.random.default_rng(41)
    B, N, HI, dI, m, k = 700, 1500, 4, 128, 4, 100
    kc, ks = O.encode_rows(rng.normal(size=(B, N, dI)), O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(rng.normal(size=(B, 1, HI, dI)), O.FMT_FP4_E8M0)
    pos = rng.integers(0, N * m, size=B).astype(np.int64)
    _compare("many sequences", kc, ks, qc, qs, pos, m, k)


def test_csa128k_full_shape_index_then_attention():
    """The 128K CSA decode configuration at its own shape: 16 sequences x 32,768 entries (131,072
    tokens at m = 4), top-1024 over 4 x 128 FP4 indexer heads, then sparse attention of 64 heads
    x 512 over the selected rows + 128-token window + sink. Indices and scores bit-exact, the
    attention output and lse within 1e-3 of the oracle on the GPU's own selection."""
    from helpers import assert_close
    c = DecodeCase("csa128k")
    assert (c.B, c.N, c.wl.k) == (16, 32768, 1024)
    _compare("csa128k full", c.kc, c.ks, c.qc, c.qs, c.pos, c.m, c.wl.k)
    gi, _ = _run(c.kc, c.ks, c.qc, c.qs, c.pos, c.m, c.wl.k)
    say("[csa_attend] csa128k full: 16 x (1024 + 128) rows")
    q, cache, win, pos, sink = c.gpu("q", "cache", "window", "pos", "sink")
    out, lse = L.csa_attend(q, cache, dev(gi), win, c.wl.w, pos, sink, c.scale)
    torch.cuda.synchronize()
    ro, rl = O.csa_attend(c.q, c.cache, c.fmt, gi, c.window, c.wl.w, c.pos, c.sink, c.scale)
    assert_close(out.cpu().numpy(), ro, "csa128k out")
    assert_close(lse.cpu().numpy(), rl, "csa128k lse")
