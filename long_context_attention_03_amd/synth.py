"""Seeded synthetic inputs shared by the GPU path's tests, the oracle's tests and the benchmark.

This module draws random numbers and nothing else: it holds none of the method's arithmetic
(no pooling, no quantisation, no scoring, no attention). Encoding the drawn values into cache
formats is done by the side that consumes them (the oracle's codecs in tests, the library's own
``kv_compress`` with m=1 in the benchmark).

Draws come from ``torch.Generator(device).manual_seed(seed)`` in a fixed order per workload,
so a (workload, seed, device) triple always yields the same tensors. CPU and GPU generators are
different streams; the parity tests draw on the CPU and copy to the GPU.

Workloads (one query token per sequence unless noted):
  tiny      1 x 4096 ctx, 8 heads x 128, fp32 rows; m=4 -> 1024 and m=128 -> 32 entries;
            indexer 4 heads x 64; top-64; window 128; seed 0.
  csa128k   16 x 131072 ctx, 64 heads x 512 (448 e4m3 + 64 bf16), m=4 -> 32768 entries,
            indexer 4 x 128, top-1024, window 128, seed 2.
  hca1m     16 x 1048576 ctx, m=128 -> 8192 entries dense, window 128, seed 3.
  csa1m     4 x 1048576 ctx, m=4 -> 262144 entries, indexer 4 x 128, top-1024, window 128,
            seed 4.
  prefill   1 sequence, 1048576 cached + 4096 new tokens; m=4 and m=128; seed 5.
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int            # sequences
    L: int            # context tokens already cached (decode: position of the query is L-1)
    Q: int            # query tokens per sequence
    H: int            # query heads
    D: int            # shared K=V row width
    row_fmt: int      # 0 = fp32 rows, 1 = e4m3 + bf16 rows
    q_dtype: int      # 0 = fp32, 1 = bf16
    m_csa: int        # CSA group size (0 = no CSA layer in this workload)
    m_hca: int        # HCA group size (0 = no HCA layer)
    HI: int           # indexer heads
    dI: int           # indexer width
    k: int            # top-k
    w: int            # window
    seed: int

    @property
    def n_csa(self) -> int:
        return self.L // self.m_csa if self.m_csa else 0

    @property
    def n_hca(self) -> int:
        return self.L // self.m_hca if self.m_hca else 0

    @property
    def scale(self) -> float:
        return self.D ** -0.5


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4096, 1, 8, 128, 0, 0, 4, 128, 4, 64, 64, 128, 0),
    "csa128k": Workload("csa128k", 16, 131072, 1, 64, 512, 1, 1, 4, 0, 4, 128, 1024, 128, 2),
    "hca1m": Workload("hca1m", 16, 1048576, 1, 64, 512, 1, 1, 0, 128, 4, 128, 0, 128, 3),
    "csa1m": Workload("csa1m", 4, 1048576, 1, 64, 512, 1, 1, 4, 0, 4, 128, 1024, 128, 4),
    "prefill": Workload("prefill", 1, 1048576, 4096, 64, 512, 1, 1, 4, 128, 4, 128, 1024, 128, 5),
}


class Draws:
    """Sequential seeded draws: every call advances the same generator."""

    def __init__(self, seed: int, device: str | torch.device = "cpu"):
        self.device = torch.device(device)
        self.gen = torch.Generator(device=self.device)
        self.gen.manual_seed(int(seed))

    def normal(self, shape, std: float = 1.0, dtype=torch.float32) -> torch.Tensor:
        x = torch.randn(tuple(shape), generator=self.gen, device=self.device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        return x if dtype == torch.float32 else x.to(dtype)

    def integers(self, low: int, high: int, shape) -> torch.Tensor:
        return torch.randint(low, high, tuple(shape), generator=self.gen, device=self.device)


def decode_inputs(wl: Workload, device="cpu", B: int | None = None, n_entries: int | None = None,
                  seed: int | None = None):
    """Pre-encoding values for one decode step of ``wl`` (one query per sequence).

    Draw order: cache rows, window rows, queries, sink, indexer keys, indexer queries.
    Returns a dict of float32 tensors (q is bf16 when the workload's queries are bf16):
      cache [B, N, D], window [B, w, D], q [B, 1, H, D], sink [H],
      ikeys [B, N, dI], iq [B, 1, HI, dI]   (indexer tensors only for CSA workloads)
    ``B`` / ``n_entries`` shrink the workload for tests; shapes and distributions are unchanged.
    """
    B = wl.B if B is None else B
    N = (wl.n_csa or wl.n_hca) if n_entries is None else n_entries
    d = Draws(wl.seed if seed is None else seed, device)
    out = {}
    out["cache"] = d.normal((B, N, wl.D))
    out["window"] = d.normal((B, wl.w - 1 + wl.Q, wl.D))
    out["q"] = d.normal((B, wl.Q, wl.H, wl.D), dtype=torch.bfloat16 if wl.q_dtype else torch.float32)
    out["sink"] = d.normal((wl.H,))
    if wl.m_csa:
        out["ikeys"] = d.normal((B, N, wl.dI))
        out["iq"] = d.normal((B, wl.Q, wl.HI, wl.dI))
    return out


def compressor_params(D: int, m: int, draws: Draws):
    """Gate weights ~N(0, 0.02) and positional biases ~N(0, 0.1)."""
    return draws.normal((D,), 0.02), draws.normal((m,), 0.1)


def raw_tokens(wl: Workload, T: int, device="cpu", seed: int | None = None):
    """Raw per-token rows for compression workloads.

    Draw order: K=V rows [B, T, D] (bf16 for bf16 workloads, else fp32), indexer-key rows
    [B, T, dI], CSA gate (w, beta), HCA gate (w, beta), indexer gate (w, beta).
    """
    d = Draws(wl.seed if seed is None else seed, device)
    out = {}
    dt = torch.bfloat16 if wl.q_dtype else torch.float32
    out["x"] = d.normal((wl.B, T, wl.D), dtype=dt)
    out["xi"] = d.normal((wl.B, T, wl.dI))
    out["w_csa"], out["b_csa"] = compressor_params(wl.D, wl.m_csa or 4, d)
    out["w_hca"], out["b_hca"] = compressor_params(wl.D, wl.m_hca or 128, d)
    out["w_idx"], out["b_idx"] = compressor_params(wl.dI, wl.m_csa or 4, d)
    return out
