"""Seeded synthetic workloads for mixed FP8/TQ3 paged decode.

This module only draws inputs: sequence lengths, which logical pages stay FP8
(anchors), the placement seed of the page allocator, outlier channels, fp32 K/V
rows, bf16 queries and the fp32 softmax scale.  It performs none of the
method's arithmetic (no quantisation, no attention), so the HIP library and the
CPU oracle can both consume exactly the same bits.

Named workloads (shapes of the five evaluation cases of this library):

  tiny        B=1, Hq=8, Hkv=2, d=128, P=16, L=1024; last 16 pages FP8; 256-page
              slabs with a seeded page placement.
  ragged      B=8, Hq=32, Hkv=8, d=128, P=16, L ~ U[2048, 8192]; anchors = pages
              overlapping the last 512 tokens plus a seeded 5% of older pages;
              8192-page slabs.
  long        B=1, Hq=48, Hkv=8, d=128, P=16, L=131072; last 4096 tokens FP8;
              K and V have ceil(2% of d) outlier channels per kv-head scaled x8.
  throughput  B=64, Hq=48, Hkv=8, d=128, P=16, L ~ U[16384, 32768]; anchors =
              pages overlapping the last 1024 tokens; slabs sized to a given
              share of device memory (default 60% of 288 GB).
  sweep(f)    B=4, Hq=16, Hkv=4, d=256, P=64, L = {16384, 16384, 16361, 1}; the
              last ceil(f * pages) pages FP8; K has ceil(2% of d) outlier
              channels per kv-head scaled x20.
  canary(n)   a multi-layer step shaped like the summaries' canary test (two
              59,008-token requests, n = 16 full-attention layers): batch entry
              b = layer * 2 + request, Hq=48, Hkv=8, d=128, P=16; each entry has
              its own K, V and query; anchors = pages overlapping the last 1024
              tokens; K and V outliers as in long.  One decode call over all
              entries is one model step's attention over every layer.

Random streams: numpy PCG64 seeded by SeedSequence(seed), spawned in the fixed
order lengths, placement, anchors, outliers, K, V, Q; K and V streams are split
again per sequence so any one sequence can be regenerated on its own.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

NAMED_SEEDS = {"tiny": 1000, "ragged": 1001, "long": 1002, "throughput": 1003, "sweep": 1004,
               "canary": 1005}
HBM_BYTES_MI355X = 288 * 10**9


def fp8_record_bytes(Hkv: int, P: int, d: int) -> int:
    """Bytes of one FP8 page record (codes, K/V scales, running amax)."""
    return 2 * Hkv * P * d + 16 * Hkv


def tq3_record_bytes(Hkv: int, P: int, d: int) -> int:
    """Bytes of one TQ3 page record (3-bit codes and fp16 group scales)."""
    return Hkv * P * d * 7 // 8


def _bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest even) and return the raw bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    P: int
    lengths: np.ndarray                      # int64 [B]
    anchors: list                            # per sequence: sorted int64 logical pages kept FP8
    fp8_pages: int
    tq3_pages: int
    placement_seed: int
    tau: np.float32
    q_bits: np.ndarray                       # uint16 [B][Hq][d] (bf16)
    k_seeds: list = field(repr=False, default_factory=list)
    v_seeds: list = field(repr=False, default_factory=list)
    k_outliers: np.ndarray | None = None     # int64 [Hkv][n] channels, or None
    k_factor: float = 1.0
    v_outliers: np.ndarray | None = None
    v_factor: float = 1.0

    # ------------------------------------------------------------------ shapes
    def n_pages(self, b: int) -> int:
        return -(-int(self.lengths[b]) // self.P)

    def demote_pages(self, b: int) -> np.ndarray:
        """Logical pages of sequence b that end up TQ3 (all pages not anchored)."""
        keep = set(int(p) for p in self.anchors[b])
        return np.array([p for p in range(self.n_pages(b)) if p not in keep], dtype=np.int64)

    def kv(self, b: int, first: int = 0, count: int | None = None):
        """fp32 K and V rows [count][Hkv][d] of sequence b, tokens first..first+count-1."""
        L = int(self.lengths[b])
        if count is None:
            count = L - first
        k = np.random.Generator(np.random.PCG64(self.k_seeds[b])).standard_normal(
            (L, self.Hkv, self.d), dtype=np.float32)[first:first + count]
        v = np.random.Generator(np.random.PCG64(self.v_seeds[b])).standard_normal(
            (L, self.Hkv, self.d), dtype=np.float32)[first:first + count]
        if self.k_outliers is not None:
            for h in range(self.Hkv):
                k[:, h, self.k_outliers[h]] *= np.float32(self.k_factor)
        if self.v_outliers is not None:
            for h in range(self.Hkv):
                v[:, h, self.v_outliers[h]] *= np.float32(self.v_factor)
        return np.ascontiguousarray(k), np.ascontiguousarray(v)

    def total_tokens(self) -> int:
        return int(np.sum(self.lengths))


def _tail_pages(L: int, P: int, tokens: int) -> list:
    """Logical pages that overlap the last `tokens` tokens of a length-L sequence."""
    n = -(-L // P)
    first = max(0, (L - tokens) // P)
    return list(range(first, n))


def make(name: str, *, B, Hq, Hkv, d, P, seed, lengths, anchor_rule,
         fp8_pages, tq3_pages, outliers=None) -> Workload:
    """Generic seeded workload.

    lengths: callable(rng) -> int array [B], or a sequence of ints.
    anchor_rule: callable(rng, b, L, P) -> iterable of logical pages kept FP8.
    outliers: None or dict(k=(count, factor) or None, v=(count, factor) or None).
    """
    ss = np.random.SeedSequence(seed)
    s_len, s_place, s_anchor, s_out, s_k, s_v, s_q = ss.spawn(7)
    r_len = np.random.Generator(np.random.PCG64(s_len))
    if callable(lengths):
        lens = np.asarray(lengths(r_len), dtype=np.int64)
    else:
        lens = np.asarray(lengths, dtype=np.int64)
    assert lens.shape == (B,) and np.all(lens >= 1)
    placement_seed = int(np.random.Generator(np.random.PCG64(s_place)).integers(1, 2**63 - 1))
    r_anchor = np.random.Generator(np.random.PCG64(s_anchor))
    anchors = []
    for b in range(B):
        a = sorted(set(int(p) for p in anchor_rule(r_anchor, b, int(lens[b]), P)))
        anchors.append(np.array(a, dtype=np.int64))
    r_out = np.random.Generator(np.random.PCG64(s_out))
    k_out = v_out = None
    k_fac = v_fac = 1.0
    if outliers:
        if outliers.get("k"):
            cnt, k_fac = outliers["k"]
            k_out = np.stack([r_out.choice(d, cnt, replace=False) for _ in range(Hkv)])
        if outliers.get("v"):
            cnt, v_fac = outliers["v"]
            v_out = np.stack([r_out.choice(d, cnt, replace=False) for _ in range(Hkv)])
    q = np.random.Generator(np.random.PCG64(s_q)).standard_normal((B, Hq, d), dtype=np.float32)
    return Workload(
        name=name, B=B, Hq=Hq, Hkv=Hkv, d=d, P=P, lengths=lens, anchors=anchors,
        fp8_pages=int(fp8_pages), tq3_pages=int(tq3_pages), placement_seed=placement_seed,
        tau=np.float32(1.0 / math.sqrt(d)), q_bits=_bf16_bits_rne(q),
        k_seeds=s_k.spawn(B), v_seeds=s_v.spawn(B),
        k_outliers=k_out, k_factor=float(k_fac), v_outliers=v_out, v_factor=float(v_fac))


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------
def tiny() -> Workload:
    return make("tiny", B=1, Hq=8, Hkv=2, d=128, P=16, seed=NAMED_SEEDS["tiny"],
                lengths=[1024], anchor_rule=lambda r, b, L, P: range(64 - 16, 64),
                fp8_pages=256, tq3_pages=256)


def ragged() -> Workload:
    def anchor_rule(r, b, L, P):
        tail = _tail_pages(L, P, 512)
        older = tail[0]
        extra = r.choice(older, int(round(0.05 * older)), replace=False) if older else []
        return list(tail) + [int(x) for x in extra]
    return make("ragged", B=8, Hq=32, Hkv=8, d=128, P=16, seed=NAMED_SEEDS["ragged"],
                lengths=lambda r: r.integers(2048, 8192, size=8, endpoint=True),
                anchor_rule=anchor_rule, fp8_pages=8192, tq3_pages=8192)


def long() -> Workload:
    c = math.ceil(0.02 * 128)
    return make("long", B=1, Hq=48, Hkv=8, d=128, P=16, seed=NAMED_SEEDS["long"],
                lengths=[131072], anchor_rule=lambda r, b, L, P: _tail_pages(L, P, 4096),
                fp8_pages=8192, tq3_pages=8192, outliers={"k": (c, 8.0), "v": (c, 8.0)})


def throughput(pool_bytes: int | None = None) -> Workload:
    """B=64 long-context batch.  The two slabs share pool_bytes (default 60% of
    288 GB): 30% FP8, 70% TQ3, so live pages scatter over the whole pool."""
    if pool_bytes is None:
        pool_bytes = int(0.6 * HBM_BYTES_MI355X)
    Hkv, P, d = 8, 16, 128
    fp8 = int(0.3 * pool_bytes) // fp8_record_bytes(Hkv, P, d)
    tq3 = int(0.7 * pool_bytes) // tq3_record_bytes(Hkv, P, d)
    return make("throughput", B=64, Hq=48, Hkv=Hkv, d=d, P=P, seed=NAMED_SEEDS["throughput"],
                lengths=lambda r: r.integers(16384, 32768, size=64, endpoint=True),
                anchor_rule=lambda r, b, L, P: _tail_pages(L, P, 1024),
                fp8_pages=fp8, tq3_pages=tq3)


def sweep(frac: float) -> Workload:
    assert frac in (0.0, 0.1, 0.5, 1.0)

    def anchor_rule(r, b, L, P):
        n = -(-L // P)
        k = math.ceil(frac * n)
        return range(n - k, n)
    c = math.ceil(0.02 * 256)
    return make(f"sweep{int(frac * 100)}", B=4, Hq=16, Hkv=4, d=256, P=64,
                seed=NAMED_SEEDS["sweep"], lengths=[16384, 16384, 16361, 1],
                anchor_rule=anchor_rule, fp8_pages=1024, tq3_pages=1024,
                outliers={"k": (c, 20.0)})


def canary(layers: int = 16, length: int = 59008, requests: int = 2) -> Workload:
    """Multi-layer step: entry b = layer * requests + r (layer-major)."""
    B = layers * requests
    P = 16
    pages = -(-length // P)
    c = math.ceil(0.02 * 128)
    anchors = len(_tail_pages(length, P, 1024))
    return make(f"canary{layers}", B=B, Hq=48, Hkv=8, d=128, P=P, seed=NAMED_SEEDS["canary"],
                lengths=[length] * B, anchor_rule=lambda r, b, L, P: _tail_pages(L, P, 1024),
                fp8_pages=B * anchors + pages + 16, tq3_pages=B * (pages - anchors) + 16,
                outliers={"k": (c, 8.0), "v": (c, 8.0)})


def small(seed: int, *, B=3, Hq=8, Hkv=2, d=128, P=16, lengths=(200, 37, 513),
          anchor_frac=0.25, outliers=None, fp8_pages=None, tq3_pages=None) -> Workload:
    """Small mixed workload for parity tests: several pages per sequence, ragged
    tails, anchors at the tail plus a random scattering."""
    def anchor_rule(r, b, L, P):
        n = -(-L // P)
        tail = list(range(max(0, n - 2), n))
        rest = [p for p in range(n) if p not in tail]
        k = int(round(anchor_frac * len(rest)))
        extra = r.choice(rest, k, replace=False) if k else []
        return tail + [int(x) for x in extra]
    total_pages = sum(-(-L // P) for L in lengths)
    return make(f"small{seed}", B=B, Hq=Hq, Hkv=Hkv, d=d, P=P, seed=seed, lengths=list(lengths),
                anchor_rule=anchor_rule,
                fp8_pages=fp8_pages or 2 * total_pages + 8,
                tq3_pages=tq3_pages or 2 * total_pages + 8, outliers=outliers)
