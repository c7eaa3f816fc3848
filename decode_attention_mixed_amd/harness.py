"""Build a synthetic mixed-format cache on the GPU through the C-ABI.

For each sequence of a workload: append all of its fp32 K/V rows as FP8 (in
one call or in the given splits), then demote every non-anchor page to TQ3,
the lifecycle the Minima-KV summary describes in "Ancoras em FP8, arquivo em
TQ3".  Pool memory is a torch uint8 tensor, optionally filled with a poison
byte first so that unwritten slots hold NaN patterns (0x7F is E4M3 NaN and
0x7F7F is fp16 NaN).
"""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_mixed_amd as mkv


def pool_desc(wl, *, max_seqs=None, max_batch=None, max_chunks=0, placement_seed=None,
              fp8_pages=None, tq3_pages=None, max_pages_per_seq=None) -> mkv.PoolDesc:
    max_pages = max_pages_per_seq or max(wl.n_pages(b) for b in range(wl.B))
    return mkv.make_desc(
        num_kv_heads=wl.Hkv, head_dim=wl.d, page_size=wl.P,
        max_seqs=max_seqs or wl.B, max_pages_per_seq=max_pages,
        max_batch=max_batch or wl.B, max_q_heads=wl.Hq,
        fp8_pages=fp8_pages or wl.fp8_pages, tq3_pages=tq3_pages or wl.tq3_pages,
        placement_seed=wl.placement_seed if placement_seed is None else placement_seed,
        max_chunks=max_chunks)


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
                  device="cuda", kv=None) -> None:
    """Append sequence b of the workload (in `splits` calls if given) and demote
    its non-anchor pages.  kv: optional (k, v) fp32 arrays or device tensors."""
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
    if dem.size:
        mkv.demote(pool.handle, seq_id, dem)


def load_cache(pool: DevicePool, wl, splits=None, device="cuda") -> None:
    for b in range(wl.B):
        load_sequence(pool, wl, b, splits=None if splits is None else splits[b], device=device)


def q_tensor(wl, device="cuda") -> torch.Tensor:
    q = torch.from_numpy(wl.q_bits.view(np.int16).copy()).view(torch.bfloat16)
    return q.to(device)


def gather_records(pool: DevicePool, seq_id: int, n_pages: int, device="cuda") -> np.ndarray:
    """Records of logical pages 0..n_pages-1 as a uint8 array [n_pages][slot]."""
    slot = max(mkv.record_bytes(pool.desc, mkv.FMT_FP8), mkv.record_bytes(pool.desc, mkv.FMT_TQ3))
    dst = torch.empty(n_pages * slot, dtype=torch.uint8, device=device)
    mkv.debug_gather(pool.handle, seq_id, 0, n_pages, dst)
    torch.cuda.synchronize()
    return dst.cpu().numpy().reshape(n_pages, slot)
