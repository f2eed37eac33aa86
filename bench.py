#!/usr/bin/env python3
"""Benchmark of the compress-then-sparsify decode hot path on one MI355X.

One step = one decode token for 16 sequences at 1,048,576 tokens of context through one CSA layer
and one HCA layer, i.e. every row of the decode hot path:
  1. kv_compress of the newest complete groups of every sequence: CSA K=V (m=4, E4M3+bf16 rows),
     indexer keys (m=4, FP4+E8M0) and HCA K=V (m=128), written at the caches' append position.
     This runs every step, an upper bound (in steady state it is due every 4th / 128th token).
  2. CSA layer, all 16 sequences in one call: index_topk over 262,144 FP4 indexer entries per
     sequence -> top-1024, then csa_attend (64 heads x 512, top-1024 entries + 128-token window
     + sink).
  3. HCA layer, the same 16 sequences: hca_attend over 8,192 entries + window + sink; it runs
     on a second stream, concurrently with the CSA layer (the two are independent).
The CSA decode step of the 4-sequence 1M configuration (index_topk + csa_attend on 4 of the
sequences) is timed separately and reported with its fraction of peak HBM bandwidth, both on one
replica (whose 71 MB of keys stay in the 256 MB last-level cache between replays) and rotating
through 16 disjoint 4-sequence replicas (1.14 GB of keys). The 128K configuration (16 sequences x
32,768 entries) is timed the same way over 8 disjoint slices of the 1M caches. Every figure is the
median (with p10 / p90) of per-replay times over at least 200 replays.
Inputs are seeded synthetic values (~N(0,1) before quantisation) generated and encoded on the
GPU with the library's own kv_compress (m = 1 is its quantiser). The step's working set is
~2.8 GB, so consecutive steps stream from HBM rather than from the 256 MB last-level cache.

The timed region replays a HIP graph of the step (the eager launch path is CPU-bound); value is
queries (sequences) per second. The roofline object reports the kernel that moves most of the
step's algorithmic HBM bytes (the indexer scan), timed with HIP events attached to its dispatch
on the library's stream (csah_profile_next_call); the "kernels" object gives the same figures for
every stage. The
cpu_baseline object times the CPU oracle on one sequence of each layer; prefill.cpu_baseline times
it on a sample of the prefill chunk's query rows (extrapolated to the chunk, and labelled so).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import long_context_attention_03_amd as L  # noqa: E402
from long_context_attention_03_amd import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0
METRIC = "CSA+HCA decode queries/sec at 1M ctx; achieved HBM GB/s vs peak"
CTX = 1 << 20
N_CSA = CTX // 4       # 262,144 entries
N_HCA = CTX // 128     # 8,192 entries
B_STEP = 16      # sequences per decode step (both layers)
B_CSA4 = 4       # the 1M-context CSA decode configuration
MTP_Q = 5        # draft tokens verified per sequence in the multi-query decode measurement
H, D, HI, DI, K, W = 64, 512, 4, 128, 1024, 128
ROW = 576
SCAN_BYTES_PER_SEQ = N_CSA * (DI // 2 + DI // 32)   # 17,825,792 B of FP4 keys + E8M0 scales


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def encode(values, m, fmt, rows=None, scales=None):
    """Quantise [B, T, D] fp32 values with the library (m=1 compression is the identity)."""
    w = torch.zeros(values.shape[-1], dtype=torch.float32, device=values.device)
    b = torch.zeros(m, dtype=torch.float32, device=values.device)
    return L.kv_compress(values, m, w, b, fmt, out_rows=rows, out_scales=scales)


class DecodeStep:
    """The decode step's inputs, workspaces and calls (one CSA and one HCA layer, 16 sequences)."""

    def __init__(self, seed: int = 4):
        dev = torch.device("cuda")
        self.scale = D ** -0.5
        self.pos = torch.full((B_STEP,), CTX - 1, dtype=torch.int64, device=dev)
        d = synth.Draws(seed, dev)
        cache = torch.empty((B_STEP, N_CSA, ROW), dtype=torch.uint8, device=dev)
        kc = torch.empty((B_STEP, N_CSA, DI // 2), dtype=torch.uint8, device=dev)
        ks = torch.empty((B_STEP, N_CSA, DI // 32), dtype=torch.uint8, device=dev)
        step = 1 << 16
        for b in range(B_STEP):
            for r0 in range(0, N_CSA, step):
                encode(d.normal((1, step, D)), 1, L.FMT_ROW_E4M3_BF16,
                       rows=cache[b:b + 1, r0:r0 + step])
                encode(d.normal((1, step, DI)), 1, L.FMT_FP4_E8M0,
                       rows=kc[b:b + 1, r0:r0 + step], scales=ks[b:b + 1, r0:r0 + step])
        win, _ = encode(d.normal((B_STEP, W, D)), 1, L.FMT_ROW_E4M3_BF16)
        iqc, iqs = encode(d.normal((B_STEP, HI, DI)), 1, L.FMT_FP4_E8M0)
        self.csa = dict(
            cache=cache, kc=kc, ks=ks, win=win,
            iqc=iqc.view(B_STEP, 1, HI, DI // 2), iqs=iqs.view(B_STEP, 1, HI, DI // 32),
            q=d.normal((B_STEP, 1, H, D), dtype=torch.bfloat16),
            xt=d.normal((B_STEP, 4, D), dtype=torch.bfloat16),
            xit=d.normal((B_STEP, 4, DI)),
            idx=torch.empty((B_STEP, 1, K), dtype=torch.int32, device=dev),
            out=torch.empty((B_STEP, 1, H, D), dtype=torch.float32, device=dev),
            lse=torch.empty((B_STEP, 1, H), dtype=torch.float32, device=dev))
        self.sink = d.normal((H,))
        self.w_csa, self.b_csa = synth.compressor_params(D, 4, d)
        self.w_idx, self.b_idx = synth.compressor_params(DI, 4, d)
        self.w_hca, self.b_hca = synth.compressor_params(D, 128, d)
        hcache = torch.empty((B_STEP, N_HCA, ROW), dtype=torch.uint8, device=dev)
        encode(d.normal((B_STEP, N_HCA, D)), 1, L.FMT_ROW_E4M3_BF16, rows=hcache)
        hwin, _ = encode(d.normal((B_STEP, W, D)), 1, L.FMT_ROW_E4M3_BF16)
        self.hca = dict(cache=hcache, win=hwin, q=d.normal((B_STEP, 1, H, D), dtype=torch.bfloat16),
                        xt=d.normal((B_STEP, 128, D), dtype=torch.bfloat16),
                        out=torch.empty((B_STEP, 1, H, D), dtype=torch.float32, device=dev),
                        lse=torch.empty((B_STEP, 1, H), dtype=torch.float32, device=dev))
        self.ws_idx = torch.empty(L.index_topk_workspace(B_STEP, 1, N_CSA, K, HI, DI),
                                  dtype=torch.uint8, device=dev)
        self.ws_csa = torch.empty(max(256, L.attend_workspace(B_STEP, 1, H, D, K + W),
                                      L.attend_workspace(B_CSA4, 1, H, D, K + W)),
                                  dtype=torch.uint8, device=dev)
        self.ws_hca = torch.empty(max(256, L.attend_workspace(B_STEP, 1, H, D, N_HCA + W)),
                                  dtype=torch.uint8, device=dev)
        # The two layers' streams, created back to back (default priority); the step runs with
        # `main` current. HIP maps streams onto the device's few hardware queues in turn, and two
        # streams on one queue run one after the other: with the HCA layer on the queue of the
        # stream that runs the CSA layer the step serializes (measured 179 against 137 us, for
        # every fourth stream created beside the default stream). Two streams created in a row
        # never share a queue.
        self.main = torch.cuda.Stream(device=dev)
        self.side = torch.cuda.Stream(device=dev)
        # speculative verification: 5 query tokens per sequence for the first 4 sequences
        QM, BM = MTP_Q, B_CSA4
        self.pos_m = torch.full((BM,), CTX - QM, dtype=torch.int64, device=dev)
        iqc5, iqs5 = encode(d.normal((BM * QM, HI, DI)), 1, L.FMT_FP4_E8M0)
        win5, _ = encode(d.normal((BM, W - 1 + QM, D)), 1, L.FMT_ROW_E4M3_BF16)
        hwin5, _ = encode(d.normal((BM, W - 1 + QM, D)), 1, L.FMT_ROW_E4M3_BF16)
        self.mtp = dict(
            iqc=iqc5.view(BM, QM, HI, DI // 2), iqs=iqs5.view(BM, QM, HI, DI // 32),
            q=d.normal((BM, QM, H, D), dtype=torch.bfloat16), win=win5, hwin=hwin5,
            idx=torch.empty((BM, QM, K), dtype=torch.int32, device=dev),
            out=torch.empty((BM, QM, H, D), dtype=torch.float32, device=dev),
            lse=torch.empty((BM, QM, H), dtype=torch.float32, device=dev),
            hout=torch.empty((BM, QM, H, D), dtype=torch.float32, device=dev),
            hlse=torch.empty((BM, QM, H), dtype=torch.float32, device=dev),
            ws_idx=torch.empty(L.index_topk_workspace(BM, QM, N_CSA, K, HI, DI),
                               dtype=torch.uint8, device=dev),
            ws_att=torch.empty(max(256, L.attend_workspace(BM, QM, H, D, K + W)),
                               dtype=torch.uint8, device=dev),
            ws_hatt=torch.empty(max(256, L.attend_workspace(BM, QM, H, D, N_HCA + W)),
                                dtype=torch.uint8, device=dev))
        torch.cuda.synchronize()

    def mtp_csa(self):
        """Verification of 5 draft tokens for 4 sequences, CSA layer: each query gets its own
        causal top-k and sparse attention (the CSA caches of sequences 0-3)."""
        c, t = self.csa_slice(B_CSA4), self.mtp
        L.index_topk(t["iqc"], t["iqs"], c["kc"], c["ks"], self.pos_m, 4, K, want_scores=False,
                     ws=t["ws_idx"], idx_out=t["idx"])
        L.csa_attend(t["q"], c["cache"], t["idx"], t["win"], W, self.pos_m, self.sink, self.scale,
                     ws=t["ws_att"], out=t["out"], lse=t["lse"])

    def mtp_hca(self):
        """The same 5 x 4 queries through the HCA layer: dense attention (own workspace, so that
        the two layers can run on two streams)."""
        t = self.mtp
        L.hca_attend(t["q"], self.hca["cache"][:B_CSA4], 128, t["hwin"], W, self.pos_m, self.sink,
                     self.scale, ws=t["ws_hatt"], out=t["hout"], lse=t["hlse"])

    def mtp_step(self):
        self.mtp_csa()
        self.mtp_hca()

    def csa_slice(self, nb):
        """The first nb sequences of the CSA layer (views; nothing is copied)."""
        return {k: v[:nb] for k, v in self.csa.items()}

    # ---- the stages of one step
    def compress_csa(self):
        c = self.csa
        L.kv_compress(c["xt"], 4, self.w_csa, self.b_csa, L.FMT_ROW_E4M3_BF16,
                      out_rows=c["cache"][:, N_CSA - 1:N_CSA])
        L.kv_compress(c["xit"], 4, self.w_idx, self.b_idx, L.FMT_FP4_E8M0,
                      out_rows=c["kc"][:, N_CSA - 1:N_CSA], out_scales=c["ks"][:, N_CSA - 1:N_CSA])

    def compress_hca(self):
        h = self.hca
        L.kv_compress(h["xt"], 128, self.w_hca, self.b_hca, L.FMT_ROW_E4M3_BF16,
                      out_rows=h["cache"][:, N_HCA - 1:N_HCA])

    def index(self, c=None, ev=None):
        c = self.csa if c is None else c
        if ev is not None:
            L.profile_next_call(*ev)
        L.index_topk(c["iqc"], c["iqs"], c["kc"], c["ks"], self.pos[:c["kc"].shape[0]], 4, K,
                     want_scores=False, ws=self.ws_idx, idx_out=c["idx"])

    def csa_attend(self, c=None, ev=None):
        c = self.csa if c is None else c
        if ev is not None:
            L.profile_next_call(*ev)
        L.csa_attend(c["q"], c["cache"], c["idx"], c["win"], W, self.pos[:c["q"].shape[0]],
                     self.sink, self.scale, ws=self.ws_csa, out=c["out"], lse=c["lse"])

    def hca_attend(self, ev=None):
        h = self.hca
        if ev is not None:
            L.profile_next_call(*ev)
        L.hca_attend(h["q"], h["cache"], 128, h["win"], W, self.pos, self.sink, self.scale,
                     ws=self.ws_hca, out=h["out"], lse=h["lse"])

    def csa_branch(self):
        self.compress_csa()
        self.index()
        self.csa_attend()

    def hca_branch(self):
        self.compress_hca()
        self.hca_attend()

    def step(self):
        """Eager step: the HCA branch on the side stream beside the CSA branch on the current
        stream (run it with `main` current). The CSA branch (the longer chain) is enqueued first;
        the side stream forks from the point before it."""
        main = torch.cuda.current_stream()
        self.side.wait_stream(main)
        self.csa_branch()
        with torch.cuda.stream(self.side):
            self.hca_branch()
        main.wait_stream(self.side)

    def csa4_step(self):
        """The 1M-context CSA decode step of 4 sequences: index_topk + csa_attend."""
        c = self.csa_slice(B_CSA4)
        self.index(c)
        self.csa_attend(c)

    def make_paged(self, page: int, seed: int = 41):
        """The 4-sequence CSA caches (rows and FP4 keys) copied into page pools of `page` entries,
        pages handed out in a shuffled order, plus the int32 block table (setup, not timed)."""
        c = self.csa_slice(B_CSA4)
        per = N_CSA // page
        g = torch.Generator(device="cpu").manual_seed(seed)
        perm = torch.randperm(B_CSA4 * per, generator=g).to(torch.int32)
        table = perm.view(B_CSA4, per).cuda()
        inv = torch.empty_like(perm)
        inv[perm.long()] = torch.arange(B_CSA4 * per, dtype=torch.int32)
        src = inv.long().cuda()  # pool page p holds logical page src[p]

        def pool(t):
            return t.reshape(B_CSA4 * per, page, t.shape[-1])[src].contiguous()

        self.paged = dict(P=page, table=table, cache=pool(c["cache"]), kc=pool(c["kc"]),
                          ks=pool(c["ks"]), idx=torch.empty_like(c["idx"]),
                          out=torch.empty_like(c["out"]), lse=torch.empty_like(c["lse"]))
        torch.cuda.synchronize()

    def index_paged(self, ev=None):
        c, p = self.csa_slice(B_CSA4), self.paged
        if ev is not None:
            L.profile_next_call(*ev)
        L.index_topk_paged(c["iqc"], c["iqs"], p["kc"], p["ks"], p["table"], p["P"], N_CSA,
                           self.pos[:B_CSA4], 4, K, want_scores=False, ws=self.ws_idx,
                           idx_out=p["idx"])

    def csa_attend_paged(self, ev=None):
        c, p = self.csa_slice(B_CSA4), self.paged
        if ev is not None:
            L.profile_next_call(*ev)
        L.csa_attend_paged(c["q"], p["cache"], p["table"], p["P"], N_CSA, p["idx"], c["win"], W,
                           self.pos[:B_CSA4], self.sink, self.scale, ws=self.ws_csa,
                           out=p["out"], lse=p["lse"])

    def csa4_paged_step(self):
        """The same 4-sequence CSA step with both caches paged."""
        self.index_paged()
        self.csa_attend_paged()


class StepGraphs:
    """The step as one HIP graph with two branches, captured across the step's two streams, so
    that the HCA branch (compress + dense attention, bound by the matrix cores) runs concurrently
    with the CSA branch (compress + index scan, bound by HBM, then sparse attention). The layers
    are independent. (csa_fn, hca_fn) default to the decode step's branches; the multi-query step
    passes its own. One graph launch measured 133 against 137 us for one graph per layer on the
    two streams (one launch and no cross-stream waits at replay)."""

    def __init__(self, ws: "DecodeStep", csa_fn=None, hca_fn=None):
        self.ws = ws
        csa_fn, hca_fn = csa_fn or ws.csa_branch, hca_fn or ws.hca_branch

        def both():
            # the CSA branch (the longer chain) first; the side stream forks from the point
            # before it and joins after it
            cur = torch.cuda.current_stream()
            ws.side.wait_stream(cur)
            csa_fn()
            with torch.cuda.stream(ws.side):
                hca_fn()
            cur.wait_stream(ws.side)

        self.g = capture(both)

    def replay(self):
        self.g.replay()



def event_pair():
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()  # materialise the underlying hipEvent_t
    return a, b


# Algorithmic HBM bytes and flops per launch of each stage's dominant kernel: what the method must
# move (selected rows, not the whole cache) and compute (QK and PV, 2 flops per MAC).
#   index_scan: 16 sequences x 262,144 FP4 keys x (64 B codes + 4 B scales); 512 MAC per key, on
#               the scaled FP4 MFMA (4 heads as the columns of one 16 x 16 x 128 product).
#   csa_attend: 16 x [(1024 + 128) rows x 576 B + 1024 ids x 4 B + q 64x512 bf16 + out 64x512 fp32
#               + lse 64 fp32] + sink; 64 heads x 1152 rows x 512 x 4 flops.
#   hca_attend: 16 x [(8192 + 128) rows x 576 B + q + out + lse] + sink; 64 x 8320 x 512 x 4 flops.
CSA_SEQ_BYTES = (K + W) * ROW + K * 4 + H * D * 2 + H * D * 4 + H * 4
KERNELS = {
    "index_scan": dict(per_step=1, bytes=B_STEP * SCAN_BYTES_PER_SEQ,
                       flops=B_STEP * N_CSA * 512 * 2, peak_flops=10.1e15,
                       name="index_cand_scan_kernel (csah_index_topk)", source="index_cand.hip",
                       profile="index_cand_scan_csa1m_b16"),
    "csa_attend": dict(per_step=1, bytes=B_STEP * CSA_SEQ_BYTES + H * 4,
                       flops=B_STEP * H * (K + W) * D * 4, peak_flops=2.5e15,
                       name="attend_x_kernel (csah_csa_attend)", source="attend.hip",
                       profile="csa_attend_csa1m_b16"),
    "hca_attend": dict(per_step=1,
                       bytes=B_STEP * ((N_HCA + W) * ROW + H * D * 2 + H * D * 4 + H * 4) + H * 4,
                       flops=B_STEP * H * (N_HCA + W) * D * 4, peak_flops=2.5e15,
                       name="attend_x_kernel (csah_hca_attend)", source="attend.hip",
                       profile="hca_attend_hca1m_b16"),
}
# The 1M-context CSA decode step of 4 sequences (index_topk + csa_attend): what the method must
# move per sequence is its FP4 keys, the selected rows, the window, q and the output.
CSA4_BYTES = B_CSA4 * (SCAN_BYTES_PER_SEQ + CSA_SEQ_BYTES) + H * 4
# The 128K CSA decode configuration: 16 sequences x 32,768 entries (131,072 tokens, m = 4).
N_128K = 32768
CSA128K_BYTES = B_STEP * (N_128K * (DI // 2 + DI // 32) + CSA_SEQ_BYTES) + H * 4
# All the decode step moves: every stage's algorithmic bytes (compression's few rows aside).
STEP_BYTES = sum(k["bytes"] * k["per_step"] for k in KERNELS.values())


def kernel_times(ws: DecodeStep, reps: int):
    """Average duration (ms) of each stage's dominant kernel, from events attached to its dispatch."""
    evs = {k: [] for k in KERNELS}
    for _ in range(reps):
        e = event_pair()
        ws.index(ev=e)
        evs["index_scan"].append(e)
        e = event_pair()
        ws.csa_attend(ev=e)
        evs["csa_attend"].append(e)
        e = event_pair()
        ws.hca_attend(e)
        evs["hca_attend"].append(e)
    torch.cuda.synchronize()
    return {k: statistics.mean(a.elapsed_time(b) for a, b in v) for k, v in evs.items()}


def paged_measure(ws: DecodeStep, args, ms4_contiguous):
    """The 4-sequence 1M CSA step with paged caches (64 entries = 256 tokens per page): step time
    and the two kernels' times next to the contiguous ones, and a check that both layouts give
    the same indices and outputs."""
    P = 64
    ws.make_paged(P)
    g = None if args.no_graph else capture(ws.csa4_paged_step)
    ms = time_replays(g, ws.csa4_paged_step, args.steps)
    c = ws.csa_slice(B_CSA4)
    ws.csa4_step()
    torch.cuda.synchronize()
    same = bool(torch.equal(ws.paged["idx"], c["idx"]) and torch.equal(ws.paged["out"], c["out"]))
    ev = {"index_scan": [], "csa_attend": [], "index_scan_paged": [], "csa_attend_paged": []}
    for _ in range(args.kernel_reps):
        for name, fn in (("index_scan", lambda e: ws.index(c, ev=e)),
                         ("csa_attend", lambda e: ws.csa_attend(c, ev=e)),
                         ("index_scan_paged", lambda e: ws.index_paged(ev=e)),
                         ("csa_attend_paged", lambda e: ws.csa_attend_paged(ev=e))):
            e = event_pair()
            fn(e)
            ev[name].append(e)
    torch.cuda.synchronize()
    kt = {k: statistics.mean(a.elapsed_time(b) for a, b in v) * 1e3 for k, v in ev.items()}
    log(f"  paged CSA step (P={P}): {ms * 1e3:.1f} us; kernels (us): "
        + ", ".join(f"{k} {v:.2f}" for k, v in kt.items()) + f"; same results: {same}")
    return {
        "what": f"csa_decode_1m_b4 with both caches paged: {P} entries ({4 * P} tokens) per page, "
                "pages in shuffled order, int32 block table",
        "page_entries": P, "us_per_step": ms * 1e3,
        "us_per_step_contiguous": None if ms4_contiguous is None else ms4_contiguous * 1e3,
        "achieved_GBps": CSA4_BYTES / (ms * 1e-3) / 1e9,
        "kernel_us": kt, "identical_to_contiguous": same,
    }


def capture(fn):
    """A HIP graph of fn() (warmed up on a scratch stream first), replayed a few times on the
    current stream."""
    cur = torch.cuda.current_stream()
    s = torch.cuda.Stream()
    s.wait_stream(cur)
    with torch.cuda.stream(s):
        fn()
    cur.wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    return g


def time_replays(g, fn, steps):
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        if g is not None:
            g.replay()
        else:
            fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def replay_stats(replays, n: int):
    """Per-replay times (us) of n calls: replays(i) runs replay i (graphs rotate by i). Events
    bracket each replay on the current stream; returns median, p10, p90 and mean."""
    evs = []
    for i in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        replays(i)
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    v = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return {"median_us": v[n // 2], "p10_us": v[n // 10], "p90_us": v[(9 * n) // 10],
            "mean_us": statistics.mean(v), "replays": n}


class Replicas:
    """Disjoint copies of a CSA decode configuration (index_topk + csa_attend), one HIP graph
    each, replayed in rotation so that consecutive replays read different keys and rows and the
    last-level cache holds none of them. make(r) -> dict(iqc, iqs, kc, ks, cache, win, q, pos)."""

    def __init__(self, ws: "DecodeStep", make, count: int, k: int = K):
        self.ws, self.graphs, self.keep = ws, [], []
        for r in range(count):
            c = make(r)
            B = c["kc"].shape[0]
            dev = c["kc"].device
            c["idx"] = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
            c["out"] = torch.empty((B, 1, H, D), dtype=torch.float32, device=dev)
            c["lse"] = torch.empty((B, 1, H), dtype=torch.float32, device=dev)
            N = c["kc"].shape[1]
            c["ws_idx"] = torch.empty(L.index_topk_workspace(B, 1, N, k, HI, DI),
                                      dtype=torch.uint8, device=dev)
            c["ws_att"] = torch.empty(max(256, L.attend_workspace(B, 1, H, D, k + W)),
                                      dtype=torch.uint8, device=dev)

            def fn(c=c):
                L.index_topk(c["iqc"], c["iqs"], c["kc"], c["ks"], c["pos"], 4, k,
                             want_scores=False, ws=c["ws_idx"], idx_out=c["idx"])
                L.csa_attend(c["q"], c["cache"], c["idx"], c["win"], W, c["pos"], ws.sink,
                             ws.scale, ws=c["ws_att"], out=c["out"], lse=c["lse"])
            self.keep.append(c)
            self.graphs.append(capture(fn))

    def stats(self, n: int, rotate: bool):
        return replay_stats(lambda i: self.graphs[i % len(self.graphs) if rotate else 0].replay(),
                            n)


def csa4_replicas(ws: "DecodeStep", count: int = 16, seed: int = 77):
    """16 disjoint 4-sequence replicas of the 1M CSA decode step: sequences 4r..4r+3 of the
    decode step's caches for r < 4, then 12 more sets of FP4 keys (N(0,1) before quantisation)
    over the same rows (each replica's own keys select its own rows)."""
    d = synth.Draws(seed, torch.device("cuda"))
    extra = []
    step = 1 << 16
    for r in range(4, count):
        kc = torch.empty((B_CSA4, N_CSA, DI // 2), dtype=torch.uint8, device="cuda")
        ks = torch.empty((B_CSA4, N_CSA, DI // 32), dtype=torch.uint8, device="cuda")
        for b in range(B_CSA4):
            for r0 in range(0, N_CSA, step):
                encode(d.normal((1, step, DI)), 1, L.FMT_FP4_E8M0,
                       rows=kc[b:b + 1, r0:r0 + step], scales=ks[b:b + 1, r0:r0 + step])
        extra.append((kc, ks))
    c = ws.csa

    def make(r):
        g = r % 4
        sl = slice(B_CSA4 * g, B_CSA4 * (g + 1))
        kc, ks = (c["kc"][sl], c["ks"][sl]) if r < 4 else extra[r - 4]
        return dict(iqc=c["iqc"][sl], iqs=c["iqs"][sl], kc=kc, ks=ks, cache=c["cache"][sl],
                    win=c["win"][sl], q=c["q"][sl], pos=ws.pos[sl])
    return Replicas(ws, make, count)


def csa128k_replicas(ws: "DecodeStep", count: int = 8):
    """The 128K configuration (16 sequences x 32,768 entries, 131,072 tokens at m = 4) as 8
    disjoint 32,768-entry slices of the 1M caches: 8 x 35.7 MB of keys and 8 x 302 MB of rows."""
    c = ws.csa
    pos = torch.full((B_STEP,), 4 * N_128K - 1, dtype=torch.int64, device="cuda")

    def make(r):
        sl = slice(N_128K * r, N_128K * (r + 1))
        return dict(iqc=c["iqc"], iqs=c["iqs"], kc=c["kc"][:, sl], ks=c["ks"][:, sl],
                    cache=c["cache"][:, sl], win=c["win"], q=c["q"], pos=pos)
    return Replicas(ws, make, count)


HCA_BYTES = KERNELS["hca_attend"]["bytes"]


class HcaReplicas:
    """The 1M HCA decode configuration (16 sequences x 8,192 entries + window + sink) as one HIP
    graph per replica: replica 0 is the decode step's own HCA cache, the others are disjoint
    8,192-entry slices of the CSA cache (rows of the same format and distribution), so that the
    rotation reads 15 x 75.5 MB = 1.13 GB of rows and the last-level cache holds none of them.
    Replays are serialized on one stream, so the replicas share the workspace and outputs."""

    def __init__(self, ws: "DecodeStep", count: int = 15):
        h, c = ws.hca, ws.csa
        self.out = torch.empty((B_STEP, 1, H, D), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((B_STEP, 1, H), dtype=torch.float32, device="cuda")
        self.ws_att = torch.empty(max(256, L.attend_workspace(B_STEP, 1, H, D, N_HCA + W)),
                                  dtype=torch.uint8, device="cuda")
        self.graphs = []
        for r in range(count):
            cache = h["cache"] if r == 0 else c["cache"][:, N_HCA * (r - 1):N_HCA * r]

            def fn(cache=cache):
                L.hca_attend(h["q"], cache, 128, h["win"], W, ws.pos, ws.sink, ws.scale,
                             N=N_HCA, ws=self.ws_att, out=self.out, lse=self.lse)
            self.graphs.append(capture(fn))

    def stats(self, n: int, rotate: bool):
        return replay_stats(lambda i: self.graphs[i % len(self.graphs) if rotate else 0].replay(),
                            n)


def tiny_measure(steps: int):
    """The tiny configuration (1 sequence, 4,096 tokens, 8 heads x 128, fp32 rows and queries,
    indexer 4 x 64, top-64, window 128): its caches compressed from raw tokens by the library
    (m = 4 rows and FP4 indexer keys, m = 128 rows), then one decode step (index_topk,
    csa_attend, hca_attend) as a HIP graph. The whole working set is a few MB and stays in L2,
    so this line measures launch and latency, not bandwidth."""
    wl = synth.WORKLOADS["tiny"]
    dev = torch.device("cuda")
    raw = synth.raw_tokens(wl, wl.L, dev)
    v = synth.decode_inputs(wl, dev)
    rows4, _ = L.kv_compress(raw["x"], 4, raw["w_csa"], raw["b_csa"], L.FMT_ROW_F32)
    rows128, _ = L.kv_compress(raw["x"], 128, raw["w_hca"], raw["b_hca"], L.FMT_ROW_F32)
    kc, ks = L.kv_compress(raw["xi"], 4, raw["w_idx"], raw["b_idx"], L.FMT_FP4_E8M0)
    iqc, iqs = encode(v["iq"].view(1, wl.HI, wl.dI), 1, L.FMT_FP4_E8M0)
    iqc, iqs = iqc.view(1, 1, wl.HI, wl.dI // 2), iqs.view(1, 1, wl.HI, wl.dI // 32)
    win, _ = encode(v["window"], 1, L.FMT_ROW_F32)
    q, sink = v["q"], v["sink"]
    pos = torch.full((1,), wl.L - 1, dtype=torch.int64, device=dev)
    idx = torch.empty((1, 1, wl.k), dtype=torch.int32, device=dev)
    o1, l1 = torch.empty((1, 1, wl.H, wl.D), device=dev), torch.empty((1, 1, wl.H), device=dev)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    wsi = torch.empty(L.index_topk_workspace(1, 1, kc.shape[1], wl.k, wl.HI, wl.dI),
                      dtype=torch.uint8, device=dev)
    wsa = torch.empty(max(256, L.attend_workspace(1, 1, wl.H, wl.D, wl.k + wl.w)),
                      dtype=torch.uint8, device=dev)
    wsh = torch.empty(max(256, L.attend_workspace(1, 1, wl.H, wl.D, rows128.shape[1] + wl.w)),
                      dtype=torch.uint8, device=dev)

    def step():
        L.index_topk(iqc, iqs, kc, ks, pos, 4, wl.k, want_scores=False, ws=wsi, idx_out=idx)
        L.csa_attend(q, rows4, idx, win, wl.w, pos, sink, wl.scale, ws=wsa, out=o1, lse=l1)
        L.hca_attend(q, rows128, 128, win, wl.w, pos, sink, wl.scale, ws=wsh, out=o2, lse=l2)
    g = capture(step)
    st = replay_stats(lambda i: g.replay(), max(200, steps))
    return {"what": "tiny configuration: 1 sequence at 4,096 tokens, 8 heads x 128 (fp32), "
                    "index_topk over 1,024 FP4 keys (4 x 64) -> top-64, csa_attend, hca_attend "
                    "over 32 entries, window 128, sink; one graph per step",
            "replays": st, "queries_per_s": 1e6 / st["median_us"]}


def source_hash(path: str) -> str:
    """First 16 hex digits of the sha256 of a kernel source's code together with the local headers
    it includes (recursively, looked up beside it and in include/): comments and whitespace are
    dropped first, so that documentation edits do not invalidate counters taken from the code,
    while a change in any header the kernels are built from does."""
    import hashlib
    import re
    dirs = [os.path.dirname(os.path.abspath(path)), os.path.join(ROOT, "include")]
    order = []

    def visit(p):
        if p in order:
            return
        order.append(p)
        for inc in re.findall(r'#include\s+"([^"]+)"', open(p).read()):
            for d in dirs:
                q = os.path.join(d, inc)
                if os.path.exists(q):
                    visit(q)
                    break

    visit(os.path.abspath(path))
    h = hashlib.sha256()
    for p in order:
        text = open(p).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str):
    """HBM bytes per launch from the committed counter summary, if it matches the kernel's source.

    profiles/<kernel>_<workload>_counters.txt holds `key = value` lines written from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE) scaled by a copy-kernel calibration; its source_sha256_16 is
    source_hash() of the .hip file the kernel was built from when the counters were taken.
    """
    path = os.path.join(ROOT, "profiles", f"{KERNELS[kernel]['profile']}_counters.txt")
    try:
        rec = {}
        with open(path) as f:
            for ln in f:
                if "=" in ln and not ln.lstrip().startswith("#"):
                    k, v = ln.split("=", 1)
                    rec[k.strip()] = v.strip()
        src = os.path.join(ROOT, "long_context_attention_03_amd", "csrc", KERNELS[kernel]["source"])
        if rec.get("source_sha256_16") != source_hash(src):
            return None
        return float(rec["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(reps: int = 3):
    """A plain device copy of known size (1 GiB read + 1 GiB written per launch), for scaling the
    FETCH_SIZE / WRITE_SIZE counters of a --pmc run to bytes."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} launches of neg() over {n * 4} bytes in, {n * 4} bytes out")


def cpu_baseline(min_seconds: float):
    """The oracle on one sequence of each layer at 1M context (index + attention + compression)."""
    import numpy as np

    import oracle as O
    d = synth.Draws(99)
    kc, ks = O.encode_rows(d.normal((1, N_CSA, DI)).numpy(), O.FMT_FP4_E8M0)
    qc, qs = O.encode_rows(d.normal((1, 1, HI, DI)).numpy(), O.FMT_FP4_E8M0)
    # the CSA cache only needs real rows where the selection lands; rows are drawn in full
    cache, _ = O.encode_rows(d.normal((1, N_CSA, D)).numpy(), O.FMT_ROW_E4M3_BF16)
    win, _ = O.encode_rows(d.normal((1, W, D)).numpy(), O.FMT_ROW_E4M3_BF16)
    hcache, _ = O.encode_rows(d.normal((1, N_HCA, D)).numpy(), O.FMT_ROW_E4M3_BF16)
    q = d.normal((1, 1, H, D), dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    sink = d.normal((H,)).numpy()
    xt = d.normal((1, 128, D)).numpy()
    xit = d.normal((1, 4, DI)).numpy()
    w512, b4, b128 = d.normal((D,), 0.02).numpy(), d.normal((4,), 0.1).numpy(), \
        d.normal((128,), 0.1).numpy()
    w128 = d.normal((DI,), 0.02).numpy()
    pos = np.array([CTX - 1], np.int64)
    times = []
    t_end = time.perf_counter() + min_seconds
    while len(times) < 3 or time.perf_counter() < t_end:
        t0 = time.perf_counter()
        O.kv_compress(xt[:, -4:], O.DT_F32, 4, w512, b4, O.FMT_ROW_E4M3_BF16)
        O.kv_compress(xit, O.DT_F32, 4, w128, b4, O.FMT_FP4_E8M0)
        O.kv_compress(xt, O.DT_F32, 128, w512, b128, O.FMT_ROW_E4M3_BF16)
        idx, _, _ = O.index_topk(qc, qs, kc, ks, pos, 4, K)
        O.csa_attend(q, cache, O.FMT_ROW_E4M3_BF16, idx, win, W, pos, sink, D ** -0.5)
        O.hca_attend(q, hcache, O.FMT_ROW_E4M3_BF16, 128, win, W, pos, sink, D ** -0.5)
        times.append(time.perf_counter() - t0)
        if len(times) >= 50:
            break
    t = statistics.median(times)
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": 1.0 / t, "unit": "queries/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"one sequence through one CSA and one HCA layer at 1M context (compress the "
                      f"newest groups, exact FP4 index over 262,144 entries + top-1024, CSA and HCA "
                      f"attention, 64 heads, fp64), median of {len(times)} runs, "
                      f"{t * 1e3:.0f} ms each, CPU: {cpu}"}


# ---- prefill chunk: 4096 new tokens appended to a 1,048,576-token cache ---------------------------
PF_Q = 4096
PF_POS0 = CTX                       # query i sits at position 1,048,576 + i
PF_N_CSA = N_CSA + PF_Q // 4        # 263,168 entries once the chunk is compressed
PF_N_HCA = N_HCA + PF_Q // 128      # 8,224
PF_PEAK_BF16, PF_PEAK_FP4 = 2.5e15, 10.1e15


def prefill_cpu_baseline():
    """The oracle on a seeded sample of the prefill chunk's query rows (positions 1,048,576 + i),
    each through the CSA layer (exact FP4 index over the 263,168 entries it sees + top-1024, CSA
    attention) and the HCA layer (dense over 8,224 entries), plus the chunk's compression once;
    the chunk's time is extrapolated to all 4096 rows and labelled so."""
    import numpy as np

    import oracle as O
    d = synth.Draws(98)
    kc, ks = O.encode_rows(d.normal((1, PF_N_CSA, DI)).numpy(), O.FMT_FP4_E8M0)
    cache, _ = O.encode_rows(d.normal((1, PF_N_CSA, D)).numpy(), O.FMT_ROW_E4M3_BF16)
    hcache, _ = O.encode_rows(d.normal((1, PF_N_HCA, D)).numpy(), O.FMT_ROW_E4M3_BF16)
    win, _ = O.encode_rows(d.normal((1, W - 1 + PF_Q, D)).numpy(), O.FMT_ROW_E4M3_BF16)
    sink = d.normal((H,)).numpy()
    x = d.normal((1, PF_Q, D)).numpy()
    xi = d.normal((1, PF_Q, DI)).numpy()
    w512, b4, b128 = d.normal((D,), 0.02).numpy(), d.normal((4,), 0.1).numpy(), \
        d.normal((128,), 0.1).numpy()
    w128 = d.normal((DI,), 0.02).numpy()
    rows = sorted({0, 1, 3, 4, 127, 128, PF_Q - 1,
                   *np.random.default_rng(98).choice(PF_Q, size=3, replace=False).tolist()})
    t0 = time.perf_counter()
    O.kv_compress(x, O.DT_F32, 4, w512, b4, O.FMT_ROW_E4M3_BF16)
    O.kv_compress(xi, O.DT_F32, 4, w128, b4, O.FMT_FP4_E8M0)
    O.kv_compress(x, O.DT_F32, 128, w512, b128, O.FMT_ROW_E4M3_BF16)
    t_comp = time.perf_counter() - t0
    per_row = []
    for i in rows:
        qc, qs = O.encode_rows(d.normal((1, 1, HI, DI)).numpy(), O.FMT_FP4_E8M0)
        q = d.normal((1, 1, H, D), dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        pos = np.array([PF_POS0 + i], np.int64)
        t0 = time.perf_counter()
        idx, _, _ = O.index_topk(qc, qs, kc, ks, pos, 4, K)
        O.csa_attend(q, cache, O.FMT_ROW_E4M3_BF16, idx, win[:, i:i + W], W, pos, sink, D ** -0.5)
        O.hca_attend(q, hcache, O.FMT_ROW_E4M3_BF16, 128, win[:, i:i + W], W, pos, sink,
                     D ** -0.5)
        per_row.append(time.perf_counter() - t0)
    t_row = statistics.median(per_row)
    t_chunk = t_comp + PF_Q * t_row
    return {"value": PF_Q / t_chunk, "unit": "tokens/s", "cores": O.num_threads(),
            "kind": "oracle", "extrapolated": True,
            "per_query_row_ms": t_row * 1e3, "chunk_compression_ms": t_comp * 1e3,
            "sample": f"{len(rows)} query rows of the chunk (i = {', '.join(map(str, rows))}), each "
                      f"through the CSA layer (exact FP4 index over its visible entries of "
                      f"{PF_N_CSA:,} + top-1024, attention) and the HCA layer ({PF_N_HCA:,} entries), "
                      f"median {t_row * 1e3:.0f} ms per row, plus the chunk's compression "
                      f"({t_comp * 1e3:.0f} ms); tokens/s extrapolated to all {PF_Q} rows"}


def hooked_us(fn, reps: int):
    """Average duration (us) of the dominant kernel of the library call fn(), from events attached
    to its dispatch."""
    evs = []
    for _ in range(reps):
        e = event_pair()
        L.profile_next_call(*e)
        fn()
        evs.append(e)
    torch.cuda.synchronize()
    return statistics.mean(a.elapsed_time(b) for a, b in evs) * 1e3


def rope_decode_measure(ws: DecodeStep, reps: int):
    """RoPE at the decode step's sizes: the 16 queries' rotary dims (64 of 512, 64 heads, bf16),
    the inverse on the f32 attention output, and the newest CSA group's compression with and
    without RoPE."""
    c = ws.csa
    q_us = hooked_us(lambda: L.rope(c["q"], ws.pos, 64), reps)
    o_us = hooked_us(lambda: L.rope(c["out"], ws.pos, 64, inverse=True), reps)
    tok = ws.pos - 3  # the group's first token: its last token is the current position
    comp = lambda: L.kv_compress(c["xt"], 4, ws.w_csa, ws.b_csa, L.FMT_ROW_E4M3_BF16,
                                 out_rows=c["cache"][:, N_CSA - 1:])
    comp_r = lambda: L.kv_compress_rope(c["xt"], 4, ws.w_csa, ws.b_csa, L.FMT_ROW_E4M3_BF16, tok,
                                        64, out_rows=c["cache"][:, N_CSA - 1:])
    cp_us, cr_us = hooked_us(comp, reps), hooked_us(comp_r, reps)
    qb, ob = B_STEP * H * 64 * 2 * 2, B_STEP * H * 64 * 4 * 2
    log(f"  RoPE at decode (us): queries {q_us:.2f}, output inverse {o_us:.2f}, "
        f"compress m=4 {cp_us:.2f} -> with RoPE {cr_us:.2f}")
    return {
        "what": "RoPE at the decode step's sizes: 16 queries x 64 heads, the last 64 of 512 dims "
                "(bf16, turned forward), the f32 attention output (turned back), and the newest "
                "group's m=4 compression with RoPE at the group's last token",
        "q_rope_us": q_us, "q_rope_bytes": qb,
        "out_inverse_us": o_us, "out_inverse_bytes": ob,
        "compress_m4_us": cp_us, "compress_m4_rope_us": cr_us,
    }


class PrefillStep:
    """One prefill chunk through one CSA and one HCA layer.

    Per step: kv_compress the chunk's raw K=V rows (m=4 into the CSA cache, m=128 into the HCA
    cache, m=1 into the window buffer) and raw indexer keys (m=4, FP4), then index_topk for the
    4096 queries (causal top-1024 each), csa_attend and hca_attend (64 heads x 512, window 128,
    sink). Caches and queries are seeded ~N(0,1) values encoded on the GPU by the library.
    """

    def __init__(self, seed: int = 5):
        dev = torch.device("cuda")
        d = synth.Draws(seed, dev)
        self.scale = D ** -0.5
        self.cache = torch.empty((1, PF_N_CSA, ROW), dtype=torch.uint8, device=dev)
        self.kc = torch.empty((1, PF_N_CSA, DI // 2), dtype=torch.uint8, device=dev)
        self.ks = torch.empty((1, PF_N_CSA, DI // 32), dtype=torch.uint8, device=dev)
        step = 1 << 16
        for r0 in range(0, N_CSA, step):
            encode(d.normal((1, step, D)), 1, L.FMT_ROW_E4M3_BF16, rows=self.cache[:, r0:r0 + step])
            encode(d.normal((1, step, DI)), 1, L.FMT_FP4_E8M0, rows=self.kc[:, r0:r0 + step],
                   scales=self.ks[:, r0:r0 + step])
        self.hcache = torch.empty((1, PF_N_HCA, ROW), dtype=torch.uint8, device=dev)
        encode(d.normal((1, N_HCA, D)), 1, L.FMT_ROW_E4M3_BF16, rows=self.hcache[:, :N_HCA])
        # window buffer: the 127 cached tokens before the chunk, then the chunk's own tokens
        self.win = torch.empty((1, W - 1 + PF_Q, ROW), dtype=torch.uint8, device=dev)
        encode(d.normal((1, W - 1, D)), 1, L.FMT_ROW_E4M3_BF16, rows=self.win[:, :W - 1])
        self.x = d.normal((1, PF_Q, D), dtype=torch.bfloat16)       # chunk K=V tokens
        self.xi = d.normal((1, PF_Q, DI))                           # chunk indexer-key tokens
        self.q = d.normal((1, PF_Q, H, D), dtype=torch.bfloat16)
        iqc, iqs = encode(d.normal((PF_Q, HI, DI)), 1, L.FMT_FP4_E8M0)
        self.iqc, self.iqs = iqc.view(1, PF_Q, HI, DI // 2), iqs.view(1, PF_Q, HI, DI // 32)
        self.sink = d.normal((H,))
        self.w_csa, self.b_csa = synth.compressor_params(D, 4, d)
        self.w_idx, self.b_idx = synth.compressor_params(DI, 4, d)
        self.w_hca, self.b_hca = synth.compressor_params(D, 128, d)
        self.w_one, self.b_one = torch.zeros(D, device=dev), torch.zeros(1, device=dev)
        self.pos = torch.full((1,), PF_POS0, dtype=torch.int64, device=dev)
        self.idx = torch.empty((1, PF_Q, K), dtype=torch.int32, device=dev)
        self.out = torch.empty((1, PF_Q, H, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((1, PF_Q, H), dtype=torch.float32, device=dev)
        self.ws_idx = torch.empty(L.index_topk_workspace(1, PF_Q, PF_N_CSA, K, HI, DI),
                                  dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def compress(self):
        L.kv_compress(self.x, 4, self.w_csa, self.b_csa, L.FMT_ROW_E4M3_BF16,
                      out_rows=self.cache[:, N_CSA:])
        L.kv_compress(self.xi, 4, self.w_idx, self.b_idx, L.FMT_FP4_E8M0,
                      out_rows=self.kc[:, N_CSA:], out_scales=self.ks[:, N_CSA:])
        L.kv_compress(self.x, 128, self.w_hca, self.b_hca, L.FMT_ROW_E4M3_BF16,
                      out_rows=self.hcache[:, N_HCA:])
        L.kv_compress(self.x, 1, self.w_one, self.b_one, L.FMT_ROW_E4M3_BF16,
                      out_rows=self.win[:, W - 1:])

    def index(self, ev=None):
        if ev is not None:
            L.profile_next_call(*ev)
        L.index_topk(self.iqc, self.iqs, self.kc, self.ks, self.pos, 4, K, want_scores=False,
                     ws=self.ws_idx, idx_out=self.idx)

    def csa(self, ev=None):
        if ev is not None:
            L.profile_next_call(*ev)
        L.csa_attend(self.q, self.cache, self.idx, self.win, W, self.pos, self.sink, self.scale,
                     out=self.out, lse=self.lse)

    def hca(self, ev=None):
        if ev is not None:
            L.profile_next_call(*ev)
        L.hca_attend(self.q, self.hcache, 128, self.win, W, self.pos, self.sink, self.scale,
                     out=self.out, lse=self.lse)

    def step(self):
        self.compress()
        self.index()
        self.csa()
        self.hca()


def prefill_measure(steps: int, warmup: int):
    """Whole-chunk time and the dominant kernel of each stage against its MFMA roofline."""
    ps = PrefillStep()
    for _ in range(warmup):
        ps.step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        ps.step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    ev = {"index_select": [], "csa_attend": [], "hca_attend": []}
    for _ in range(max(1, steps // 2)):
        ps.compress()
        e = event_pair()
        ps.index(e)
        ev["index_select"].append(e)
        e = event_pair()
        ps.csa(e)
        ev["csa_attend"].append(e)
        e = event_pair()
        ps.hca(e)
        ev["hca_attend"].append(e)
    torch.cuda.synchronize()
    kt = {k: statistics.mean(a.elapsed_time(b) for a, b in v) for k, v in ev.items()}
    # algorithmic operations: FP4 MACs of the indexer (512 per visible entry per query, one pass),
    # QK + PV flops of the attention over each query's rows (1152 CSA, 8192 + (i+1)//128 + 128 HCA)
    n_vis = sum(min(PF_N_CSA, (PF_POS0 + i + 1) // 4) for i in range(PF_Q))
    hca_rows = sum(min(PF_N_HCA, (PF_POS0 + i + 1) // 128) + W for i in range(PF_Q))
    ops = {"index_select": (2.0 * 512 * n_vis, PF_PEAK_FP4, "fp4"),
           "csa_attend": (4.0 * H * D * PF_Q * (K + W), PF_PEAK_BF16, "bf16"),
           "hca_attend": (4.0 * H * D * hca_rows, PF_PEAK_BF16, "bf16")}
    # overlapping entries (8 tokens each at stride 4) for the chunk: the 4 tokens before it are
    # context; E4M3+bf16 rows and FP4 indexer keys, timed on events around the two calls
    xs = torch.cat([ps.x[:, :4], ps.x], dim=1)
    xis = torch.cat([ps.xi[:, :4], ps.xi], dim=1)
    b8 = torch.zeros(8, device="cuda")
    rows8 = torch.empty((1, PF_Q // 4, ROW), dtype=torch.uint8, device="cuda")
    k8 = torch.empty((1, PF_Q // 4, DI // 2), dtype=torch.uint8, device="cuda")
    s8 = torch.empty((1, PF_Q // 4, DI // 32), dtype=torch.uint8, device="cuda")
    span_ms = []
    for _ in range(max(2, steps)):
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        L.kv_compress(xs, 4, ps.w_csa, b8, L.FMT_ROW_E4M3_BF16, out_rows=rows8, span=8, skip=1)
        L.kv_compress(xis, 4, ps.w_idx, b8, L.FMT_FP4_E8M0, out_rows=k8, out_scales=s8, span=8,
                      skip=1)
        e.record()
        torch.cuda.synchronize()
        span_ms.append(a.elapsed_time(e))
    span_bytes = (PF_Q + 4) * (D * 2 + DI * 4) + (PF_Q // 4) * (ROW + DI // 2 + DI // 32)
    t_span = statistics.median(span_ms[1:]) * 1e-3
    # RoPE on the chunk: the 4096 queries' rotary dims (bf16), the inverse on the f32 output, and
    # the chunk's m=4 compression with and without RoPE
    reps = max(2, steps)
    rq = hooked_us(lambda: L.rope(ps.q, ps.pos, 64), reps)
    ro = hooked_us(lambda: L.rope(ps.out, ps.pos, 64, inverse=True), reps)
    rc = hooked_us(lambda: L.kv_compress(ps.x, 4, ps.w_csa, ps.b_csa, L.FMT_ROW_E4M3_BF16,
                                         out_rows=ps.cache[:, N_CSA:]), reps)
    rcr = hooked_us(lambda: L.kv_compress_rope(ps.x, 4, ps.w_csa, ps.b_csa, L.FMT_ROW_E4M3_BF16,
                                               ps.pos, 64, out_rows=ps.cache[:, N_CSA:]), reps)
    qb, ob = PF_Q * H * 64 * 2 * 2, PF_Q * H * 64 * 4 * 2
    log(f"  RoPE on the chunk (us): queries {rq:.1f} ({qb / rq / 1e3:.0f} GB/s), output inverse "
        f"{ro:.1f} ({ob / ro / 1e3:.0f} GB/s), compress m=4 {rc:.1f} -> with RoPE {rcr:.1f}")
    rope = {
        "what": "RoPE on the chunk: 4096 queries x 64 heads, the last 64 of 512 dims (bf16, "
                "turned forward), the f32 attention output (turned back), and the chunk's m=4 "
                "compression with RoPE; bytes = the rotary dims read and written",
        "q_rope_us": rq, "q_rope_bytes": qb, "q_rope_GBps": qb / rq / 1e3,
        "out_inverse_us": ro, "out_inverse_bytes": ob, "out_inverse_GBps": ob / ro / 1e3,
        "compress_m4_us": rc, "compress_m4_rope_us": rcr,
    }
    kernels = {}
    for k, (fl, peak, dt) in ops.items():
        t = kt[k] * 1e-3
        kernels[k] = {"avg_launch_us": t * 1e6, "algorithmic_ops": fl, "achieved_TFLOPs": fl / t / 1e12,
                      "peak_TFLOPs": peak / 1e12, "frac": fl / t / peak, "dtype": dt}
    dom = max(kernels, key=lambda k: kernels[k]["avg_launch_us"])
    log(f"  prefill chunk: {ms:.3f} ms; " + ", ".join(f"{k} {v['avg_launch_us']:.0f} us"
                                                      for k, v in kernels.items()))
    return {
        "metric": "prefill chunk tokens/s (4096 new tokens on a 1M cache, one CSA + one HCA layer)",
        "value": PF_Q / (ms * 1e-3), "unit": "tokens/s", "ms_per_chunk": ms, "steps": steps,
        "workload": "1 sequence, 1,048,576 cached tokens + 4,096 new: kv_compress of the chunk "
                    "(m=4, FP4 indexer keys, m=128, window rows), per-query causal top-1024 over "
                    "263,168 FP4 entries (scaled FP4 MFMA), CSA and HCA attention, 64 heads x 512",
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": kernels[dom]["achieved_TFLOPs"],
                     "peak": kernels[dom]["peak_TFLOPs"], "unit": "TFLOP/s",
                     "frac": kernels[dom]["frac"]},
        "kernels": kernels,
        "index_workspace_bytes": L.index_topk_workspace(1, PF_Q, PF_N_CSA, K, HI, DI),
        "compress_span8": {
            "what": "the chunk's overlapping entries: 8 tokens each at stride 4 (1024 E4M3+bf16 "
                    "rows and 1024 FP4 indexer keys, the 4 preceding tokens as context)",
            "us": t_span * 1e6, "algorithmic_bytes": span_bytes,
            "achieved_GBps": span_bytes / t_span / 1e9,
        },
        "rope": rope,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead")
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-chunk measurement")
    ap.add_argument("--no-csa4", action="store_true",
                    help="skip the separate 4-sequence CSA step (for counter runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB copy kernel (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    log("building inputs (about 2.8 GB of encoded caches on the GPU)...")
    ws = DecodeStep()
    # everything below runs on the step's main stream, which never shares a hardware queue with
    # the side stream that the HCA layer takes
    torch.cuda.set_stream(ws.main)
    log("warmup...")
    for _ in range(args.warmup):
        ws.step()
    torch.cuda.synchronize()
    graph = None if args.no_graph else StepGraphs(ws)
    log(f"timing {args.steps} steps ({'graph replay' if graph else 'eager'})...")
    ms = time_replays(graph, ws.step, args.steps)
    n_stats = max(200, args.steps)
    step_stats = replay_stats(lambda i: graph.replay() if graph else ws.step(), n_stats)
    log(f"  {ms * 1e3:.1f} us per step (median {step_stats['median_us']:.1f}, p10 "
        f"{step_stats['p10_us']:.1f}, p90 {step_stats['p90_us']:.1f})")
    g4, ms4, rot4, rot128, roth = None, None, None, None, None
    if not args.no_csa4:
        g4 = None if args.no_graph else capture(ws.csa4_step)
        ms4 = time_replays(g4, ws.csa4_step, args.steps)
        log(f"  CSA decode step, 4 sequences at 1M: {ms4 * 1e3:.1f} us")
        if not args.no_graph:
            log("  16 rotated 4-sequence replicas (1.14 GB of keys) and 8 rotated 128K slices...")
            r4 = csa4_replicas(ws)
            rot4 = {"one_replica": r4.stats(n_stats, False), "rotated_16": r4.stats(n_stats, True)}
            del r4
            r128 = csa128k_replicas(ws)
            rot128 = {"one_replica": r128.stats(n_stats, False),
                      "rotated_8": r128.stats(n_stats, True)}
            del r128
            rh = HcaReplicas(ws)
            roth = {"one_replica": rh.stats(n_stats, False), "rotated_15": rh.stats(n_stats, True)}
            del rh
            log(f"  4 x 1M: median {rot4['one_replica']['median_us']:.1f} us on one replica, "
                f"{rot4['rotated_16']['median_us']:.1f} us rotated; 16 x 128K: "
                f"{rot128['one_replica']['median_us']:.1f} / {rot128['rotated_8']['median_us']:.1f} us; "
                f"HCA 16 x 1M: {roth['one_replica']['median_us']:.1f} / "
                f"{roth['rotated_15']['median_us']:.1f} us")
    kt = kernel_times(ws, args.kernel_reps)
    log("  dominant kernels (us): " + ", ".join(f"{k} {v * 1e3:.2f}" for k, v in kt.items()))
    # the roofline object reports the kernel that moves most of the step's algorithmic HBM bytes
    # (the metric is HBM bandwidth): the indexer scan. HCA attention takes about as long per
    # launch but runs beside it on the other stream; every kernel's fraction is in "kernels".
    dom = max(KERNELS, key=lambda k: KERNELS[k]["per_step"] * KERNELS[k]["bytes"])
    kinfo = {}
    for k, spec in KERNELS.items():
        t = kt[k] * 1e-3
        t_hbm, t_mfma = spec["bytes"] / (PEAK_HBM_GBS * 1e9), spec["flops"] / spec["peak_flops"]
        kinfo[k] = {"avg_launch_us": t * 1e6, "launches_per_step": spec["per_step"],
                    "algorithmic_bytes_per_launch": spec["bytes"],
                    "algorithmic_flops_per_launch": spec["flops"],
                    "achieved_GBps": spec["bytes"] / t / 1e9,
                    "achieved_TFLOPs": spec["flops"] / t / 1e12,
                    "roofline_bound": "hbm" if t_hbm >= t_mfma else "compute",
                    "frac_of_roofline": max(t_hbm, t_mfma) / t}
    spec = KERNELS[dom]
    t_dom = kt[dom] * 1e-3
    if spec["bytes"] / (PEAK_HBM_GBS * 1e9) >= spec["flops"] / spec["peak_flops"]:
        roof = {"bound": "hbm", "achieved": spec["bytes"] / t_dom / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma",
                "achieved": spec["flops"] / t_dom / 1e12, "peak": spec["peak_flops"] / 1e12,
                "unit": "TFLOP/s"}
    queries = B_STEP
    line = {
        "metric": METRIC,
        "value": queries / (ms * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "step_replay_us": step_stats,
        "step_algorithmic_bytes": STEP_BYTES,
        "step_frac_of_hbm_peak": STEP_BYTES / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode step, 16 sequences x 1,048,576-token context through one CSA "
                        "layer (FP4 index over 262,144 entries per sequence, top-1024, sparse "
                        "attention + 128-token window + sink) and one HCA layer (dense attention "
                        "over 8,192 entries + window + sink), newest-group kv_compress every "
                        "step; 64 heads x 512 (448 e4m3 + 64 bf16)",
            "global_batch": queries, "seq_len": CTX, "heads": H, "head_dim": D,
            "indexer": "4 heads x 128, FP4 e2m1 + E8M0/32", "top_k": K, "window": W,
            "timing": "hip graph replay" if graph is not None else "eager",
            "compute": "indexer scan fp32 (exact), attention bf16 MFMA with fp32 accumulation",
        },
        "roofline": {
            "kernel": spec["name"],
            **roof,
            "frac": roof["achieved"] / roof["peak"],
            "traffic": traffic_from_profile(dom),
            "algorithmic_bytes_per_launch": spec["bytes"],
            "avg_launch_us": kt[dom] * 1e3,
        },
        "kernels": kinfo,
    }
    if not args.no_csa4:
        if args.no_graph:
            msm = time_replays(None, ws.mtp_step, args.steps)
        else:
            mg = StepGraphs(ws, ws.mtp_csa, ws.mtp_hca)
            for _ in range(args.warmup):
                mg.replay()
            msm = time_replays(None, mg.replay, args.steps)
        log(f"  multi-query decode (4 sequences x {MTP_Q} queries): {msm * 1e3:.1f} us")
        # unique bytes: each sequence's keys and HCA rows once, each query's selected rows, the
        # windows, q and both outputs
        mbytes = (B_CSA4 * (SCAN_BYTES_PER_SEQ + N_HCA * ROW + 2 * (W - 1 + MTP_Q) * ROW)
                  + B_CSA4 * MTP_Q * (K * ROW + K * 4 + 2 * H * D * 2 + 2 * H * D * 4 + 2 * H * 4))
        line["decode_multi_query"] = {
            "what": f"{B_CSA4} sequences x {MTP_Q} query tokens (draft verification) at 1,048,576 "
                    "tokens: per-query causal top-1024 over 262,144 FP4 keys, CSA attention, HCA "
                    "attention over 8,192 entries, window 128, sink",
            "us_per_step": msm * 1e3, "queries_per_s": B_CSA4 * MTP_Q / (msm * 1e-3),
            "unique_bytes": mbytes, "achieved_GBps": mbytes / (msm * 1e-3) / 1e9,
        }
    if ms4 is not None:
        line["csa_decode_1m_b4"] = {
            "what": "index_topk + csa_attend for 4 sequences at 1,048,576 tokens (262,144 FP4 "
                    "keys each, top-1024, window 128, sink)",
            "us_per_step": ms4 * 1e3, "algorithmic_bytes": CSA4_BYTES,
            "achieved_GBps": CSA4_BYTES / (ms4 * 1e-3) / 1e9,
            "frac_of_hbm_peak": CSA4_BYTES / (ms4 * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "queries_per_s": B_CSA4 / (ms4 * 1e-3),
        }
        if rot4 is not None:
            med = rot4["rotated_16"]["median_us"]
            line["csa_decode_1m_b4"].update({
                "replays": rot4,
                "rotated_median_us": med,
                "rotated_frac_of_hbm_peak": CSA4_BYTES / (med * 1e-6) / 1e9 / PEAK_HBM_GBS,
                "rotation": "16 disjoint 4-sequence replicas, 1.14 GB of FP4 keys; one_replica "
                            "replays the same 71 MB of keys, which stay in the 256 MB last-level "
                            "cache",
            })
    if rot128 is not None:
        med = rot128["rotated_8"]["median_us"]
        line["csa_decode_128k_b16"] = {
            "what": "index_topk + csa_attend for 16 sequences at 131,072 tokens (32,768 FP4 keys "
                    "each, top-1024, window 128, sink)",
            "replays": rot128, "rotated_median_us": med, "algorithmic_bytes": CSA128K_BYTES,
            "achieved_GBps": CSA128K_BYTES / (med * 1e-6) / 1e9,
            "frac_of_hbm_peak": CSA128K_BYTES / (med * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "queries_per_s": B_STEP / (med * 1e-6),
            "rotation": "8 disjoint 32,768-entry slices of the 1M caches (285 MB of keys)",
        }
    if roth is not None:
        med = roth["rotated_15"]["median_us"]
        line["hca_decode_1m_b16"] = {
            "what": "hca_attend for 16 sequences at 1,048,576 tokens (8,192 entries each, window "
                    "128, sink)",
            "replays": roth, "rotated_median_us": med, "algorithmic_bytes": HCA_BYTES,
            "achieved_GBps": HCA_BYTES / (med * 1e-6) / 1e9,
            "frac_of_hbm_peak": HCA_BYTES / (med * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "queries_per_s": B_STEP / (med * 1e-6),
            "rotation": "15 replicas: the HCA cache and 14 disjoint 8,192-entry slices of the CSA "
                        "cache (1.13 GB of rows)",
        }
        if rot4 is not None:
            t4, t3 = rot4["rotated_16"]["median_us"], med
            line["one_csa_plus_one_hca_layer_1m"] = {
                "what": "queries/s through one CSA and one HCA layer at 1M context from the two "
                        "rotated configurations timed apart: 1 / (t_csa_4seq / 4 + t_hca_16seq / 16)",
                "t_csa_decode_1m_b4_us": t4, "t_hca_decode_1m_b16_us": t3,
                "queries_per_s": 1e6 / (t4 / B_CSA4 + t3 / B_STEP),
            }
    if not args.no_csa4:
        line["csa_decode_1m_b4_paged"] = paged_measure(ws, args, ms4)
        line["tiny_decode"] = tiny_measure(args.steps)
    line["rope_decode"] = rope_decode_measure(ws, args.kernel_reps)
    if not args.no_prefill:
        log("prefill chunk (4096 tokens on a 1M cache)...")
        del ws, graph, g4
        torch.cuda.empty_cache()
        line["prefill"] = prefill_measure(max(2, min(args.steps, 10)), max(1, min(args.warmup, 2)))
    if args.calibrate_copy:
        copy_calibration()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on one sequence per layer...")
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        if "prefill" in line:
            log("timing the CPU oracle on a sample of the prefill chunk's query rows...")
            line["prefill"]["cpu_baseline"] = prefill_cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
