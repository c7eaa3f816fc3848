"""mkv_decode_static (partial states in the library's fixed per-GPU workspace,
no device allocation) against mkv_decode on the same pool and batch.

Both run the same schedule through the same kernels, so the outputs must
agree bit for bit (stricter than the oracle tolerance of the parity tests).
The second call of each pair takes a smaller batch than the first, so it
reads a workspace that still holds the first call's states."""
import numpy as np
import pytest
import torch

import decode_attention_mixed_amd as mkv
from decode_attention_mixed_amd import harness as H
from decode_attention_mixed_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _decode(fn, pool, wl, ids):
    q = H.q_tensor(wl)[ids].contiguous()
    out = torch.full((len(ids), wl.Hq, wl.d), float("nan"), device="cuda")
    lse = torch.full((len(ids), wl.Hq), float("nan"), device="cuda")
    fn(pool.handle, ids, q, float(wl.tau), out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def test_static_workspace_decode_matches_pool_decode():
    wl = W.ragged()
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_cache(pool, wl)
    for ids in ([0, 1, 2, 3, 4, 5, 6, 7], [5, 2, 7]):
        print(f"[no-alloc] ragged ids={ids}", flush=True)
        o_s, l_s = _decode(mkv.decode_static, pool, wl, ids)
        o_p, l_p = _decode(mkv.decode, pool, wl, ids)
        assert np.isfinite(o_s).all() and np.isfinite(l_s).all()
        assert np.array_equal(o_s, o_p) and np.array_equal(l_s, l_p), ids
        info = mkv.debug_schedule(pool.handle, arrays=False)
        print(f"[no-alloc] chunks={info['n_chunks']}", flush=True)
    pool.close()


def test_static_workspace_rejects_an_oversized_batch():
    # d = 256, Hq = 64 and 256 chunks (the split-K floor of a 4096-page batch)
    # need 256 * 64 * 258 * 4 bytes of partial states: more than the 16 MiB
    # workspace.
    Hkv, Hq, d, P, L, B = 4, 64, 256, 16, 16384, 4
    desc = mkv.make_desc(num_kv_heads=Hkv, head_dim=d, page_size=P, max_seqs=B,
                         max_pages_per_seq=L // P, max_batch=B, max_q_heads=Hq,
                         fp8_pages=B * L // P, tq3_pages=16)
    pool = H.DevicePool(desc)
    g = torch.Generator(device="cuda").manual_seed(7)
    for s in range(B):
        k = torch.randn(L, Hkv, d, device="cuda", generator=g)
        v = torch.randn(L, Hkv, d, device="cuda", generator=g)
        mkv.append(pool.handle, s, k, v)
    q = torch.randn(B, Hq, d, device="cuda", generator=g).to(torch.bfloat16)
    out = torch.zeros(B, Hq, d, device="cuda")
    lse = torch.zeros(B, Hq, device="cuda")
    with pytest.raises(mkv.MkvError) as e:
        mkv.decode_static(pool.handle, list(range(B)), q, 0.0625, out, lse)
    assert e.value.status == mkv.ERANGE
    torch.cuda.synchronize()
    assert not out.any()                      # nothing was enqueued
    mkv.decode(pool.handle, list(range(B)), q, 0.0625, out, lse)
    torch.cuda.synchronize()
    info = mkv.debug_schedule(pool.handle, arrays=False)
    assert info["n_chunks"] >= 256
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    # a batch of one sequence fits, and matches the pool decode bit for bit
    o1 = torch.zeros(1, Hq, d, device="cuda")
    l1 = torch.zeros(1, Hq, device="cuda")
    mkv.decode_static(pool.handle, [2], q[2:3].contiguous(), 0.0625, o1, l1)
    o2 = torch.zeros(1, Hq, d, device="cuda")
    l2 = torch.zeros(1, Hq, device="cuda")
    mkv.decode(pool.handle, [2], q[2:3].contiguous(), 0.0625, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    pool.close()
