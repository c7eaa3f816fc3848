"""Build a synthetic mixed-format cache on the GPU through the C-ABI.

For each sequence of a workload: append all of its fp32 K/V rows as FP8 (in
one call or in the given splits), then demote every non-anchor page to TQ3,
the lifecycle the Minima-KV summary describes in "Ancoras em FP8, arquivo em
TQ3".  The comparison caches of the same summary (section "O que as medicoes
mostram", subsection "Memoria e compressao") use the same rows: a dense BF16
control pool (append only), and an all-FP8 mixed pool (append without
demotion).  Pool memory is a torch uint8 tensor, optionally filled with a
poison byte first so that unwritten slots hold NaN patterns (0x7F is E4M3 NaN and
0x7F7F is fp16 NaN).
"""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_mixed_amd as mkv


def pool_desc(wl, *, max_seqs=None, max_batch=None, max_chunks=0, placement_seed=None,
              fp8_pages=None, tq3_pages=None, max_pages_per_seq=None,
              kind: str = "mixed") -> mkv.PoolDesc:
    """kind: "mixed" (FP8/TQ3 slabs of the workload), "bf16" (control pool with
    one slab holding every page) or "fp8" (mixed pool with an FP8 slab large
    enough for every page and no TQ3 slab use)."""
    max_pages = max_pages_per_seq or max(wl.n_pages(b) for b in range(wl.B))
    all_pages = sum(wl.n_pages(b) for b in range(wl.B))
    if kind == "mixed":
        f8, t3, kv_kind = fp8_pages or wl.fp8_pages, tq3_pages or wl.tq3_pages, mkv.KIND_MIXED
    elif kind == "bf16":
        f8, t3, kv_kind = fp8_pages or all_pages, 0, mkv.KIND_BF16
    elif kind == "fp8":
        f8, t3, kv_kind = fp8_pages or all_pages, tq3_pages or 0, mkv.KIND_MIXED
    else:
        raise ValueError(kind)
    return mkv.make_desc(
        num_kv_heads=wl.Hkv, head_dim=wl.d, page_size=wl.P,
        max_seqs=max_seqs or wl.B, max_pages_per_seq=max_pages,
        max_batch=max_batch or wl.B, max_q_heads=wl.Hq,
        fp8_pages=f8, tq3_pages=t3,
        placement_seed=wl.placement_seed if placement_seed is None else placement_seed,
        max_chunks=max_chunks, kv_kind=kv_kind)


class DevicePool:
    """A pool whose device memory is a torch tensor (kept alive with the pool)."""

    def __init__(self, desc: mkv.PoolDesc, poison: int | None = 0x7F, device="cuda"):
        self.desc = desc
        nbytes = mkv.pool_bytes(desc)
        if nbytes == 0:
            raise ValueError("invalid pool descriptor")
        self.mem = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.mem.data_ptr()) % 256
        self.mem = self.mem[off:off + nbytes]
        if poison is not None:
            self.mem.fill_(poison)
        self.handle = mkv.pool_create(desc, self.mem)

    def close(self):
        if self.handle is not None:
            mkv.pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def load_sequence(pool: DevicePool, wl, b: int, seq_id: int | None = None, splits=None,
                  device="cuda", kv=None, demote: bool = True) -> None:
    """Append sequence b of the workload (in `splits` calls if given) and, if
    demote, demote its non-anchor pages.  kv: optional (k, v) fp32 arrays or
    device tensors."""
    seq_id = b if seq_id is None else seq_id
    if kv is None:
        kv = wl.kv(b)
    k, v = kv
    if not isinstance(k, torch.Tensor):
        k = torch.from_numpy(k)
        v = torch.from_numpy(v)
    k = k.to(device=device, dtype=torch.float32).contiguous()
    v = v.to(device=device, dtype=torch.float32).contiguous()
    L = k.shape[0]
    if splits is None:
        splits = [L]
    assert sum(splits) == L
    pos = 0
    for n in splits:
        mkv.append(pool.handle, seq_id, k[pos:pos + n], v[pos:pos + n])
        pos += n
    dem = wl.demote_pages(b)
    if demote and dem.size and pool.desc.kv_kind == mkv.KIND_MIXED:
        mkv.demote(pool.handle, seq_id, dem)


def load_cache(pool: DevicePool, wl, splits=None, device="cuda", demote: bool = True) -> None:
    """demote=False: the all-FP8 cache (mixed pool); control pools never demote."""
    for b in range(wl.B):
        load_sequence(pool, wl, b, splits=None if splits is None else splits[b], device=device,
                      demote=demote)


def q_tensor(wl, device="cuda") -> torch.Tensor:
    q = torch.from_numpy(wl.q_bits.view(np.int16).copy()).view(torch.bfloat16)
    return q.to(device)


def gather_records(pool: DevicePool, seq_id: int, n_pages: int, device="cuda") -> np.ndarray:
    """Records of logical pages 0..n_pages-1 as a uint8 array [n_pages][slot]."""
    slot = max(mkv.record_bytes(pool.desc, f) for f in (mkv.FMT_FP8, mkv.FMT_TQ3, mkv.FMT_BF16))
    dst = torch.empty(n_pages * slot, dtype=torch.uint8, device=device)
    mkv.debug_gather(pool.handle, seq_id, 0, n_pages, dst)
    torch.cuda.synchronize()
    return dst.cpu().numpy().reshape(n_pages, slot)


class AnchorPolicy:
    """Caller-side anchor policy of a decode loop ("Ancoras em FP8, arquivo em
    TQ3": recent and protected pages stay FP8, older pages are converted).  A
    page is demoted once every one of its tokens is older than the last
    `window` tokens of its sequence, unless it is protected.  The policy keeps
    its own record of demoted pages, so its decisions depend only on lengths,
    the window and the protected sets (the same on any implementation).

    protected: per sequence, logical pages that stay FP8 (e.g. attention sinks
    or pages the caller marks).  demoted: per sequence, pages already TQ3."""

    def __init__(self, P: int, window: int, protected, demoted):
        self.P = P
        self.window = window
        self.protected = [set(int(x) for x in p) for p in protected]
        self.demoted = [set(int(x) for x in d) for d in demoted]
        self.seen = [0] * len(self.demoted)     # pages below this were already decided

    def step(self, seq: int, length: int) -> list:
        """Pages of `seq` to demote now that it holds `length` tokens."""
        full = max(0, (length - self.window) // self.P)      # pages wholly outside the window
        new = [lp for lp in range(self.seen[seq], full)
               if lp not in self.demoted[seq] and lp not in self.protected[seq]]
        self.seen[seq] = max(self.seen[seq], full)
        self.demoted[seq].update(new)
        return new
