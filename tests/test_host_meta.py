"""CPU tests of the host metadata layer (pool geometry, free lists, page tables,
split-K scheduler, error handling), through the CPU-only test library that is
built from the same C++ source as libmkv.so."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from decode_attention_mixed_amd import PoolDesc, make_desc
from decode_attention_mixed_amd import build as B

OK, EINVAL, ENOMEM, ESTATE, ERANGE = 0, -1, -2, -3, -4


@pytest.fixture(scope="module")
def lib():
    path = B.build_host_test()
    L = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.mkvh_create.argtypes = [ctypes.POINTER(PoolDesc), ctypes.POINTER(P)]
    L.mkvh_destroy.argtypes = [P]
    L.mkvh_append.argtypes = [P, I32, I32, P, I32, ctypes.POINTER(I32)]
    L.mkvh_append_step.argtypes = [P, P, I32, I32, P, I32, ctypes.POINTER(I32)]
    L.mkvh_demote.argtypes = [P, I32, P, I32, P, I32, ctypes.POINTER(I32)]
    L.mkvh_reset.argtypes = [P, I32]
    L.mkvh_seq_len.argtypes = [P, I32]
    L.mkvh_page_table.argtypes = [P, I32, P, I32]
    L.mkvh_free.argtypes = [P, I32]
    L.mkvh_free.restype = I64
    L.mkvh_kv_bytes.argtypes = [P, P, I32]
    L.mkvh_kv_bytes.restype = I64
    L.mkvh_version.argtypes = [P]
    L.mkvh_version.restype = ctypes.c_uint64
    L.mkvh_layout_version.argtypes = [P]
    L.mkvh_layout_version.restype = ctypes.c_uint64
    L.mkvh_schedule.argtypes = [P, P, I32, I32, I32, I32, P, I32, P, I32, P, P]
    L.mkvh_check_schedule.argtypes = [P, P, I32, I32, I32, I32, I32, ctypes.POINTER(I32)]
    L.mkvh_append_rollback.argtypes = [P, I32, I32]
    L.mkvh_demote_rollback.argtypes = [P, I32, P, I32]
    L.mkvh_append_step_rollback.argtypes = [P, P, I32, I32]
    L.mkvh_protect.argtypes = [P, I32, P, I32, I32]
    L.mkvh_policy_pages.argtypes = [P, I32, I32, P, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]
    L.mkvh_policy_pages.restype = None
    L.mkvh_set_policy_next.argtypes = [P, I32, I32]
    L.mkvh_set_policy_next.restype = None
    L.mkvh_last_error.restype = ctypes.c_char_p
    return L


class Host:
    def __init__(self, lib, **kw):
        self.L = lib
        self.h = ctypes.c_void_p()
        self.desc = make_desc(**kw)
        st = lib.mkvh_create(ctypes.byref(self.desc), ctypes.byref(self.h))
        if st:
            raise ValueError(st)

    def close(self):
        self.L.mkvh_destroy(self.h)

    def append(self, seq, n):
        buf = np.zeros((4096, 8), np.int32)
        cnt = ctypes.c_int32()
        st = self.L.mkvh_append(self.h, seq, n, buf.ctypes.data, 4096, ctypes.byref(cnt))
        return st, buf[:cnt.value]

    def append_step(self, ids, pt_stride=64):
        arr = np.asarray(ids, np.int32)
        buf = np.zeros((4096, 8), np.int32)
        cnt = ctypes.c_int32()
        st = self.L.mkvh_append_step(self.h, arr.ctypes.data, arr.size, pt_stride, buf.ctypes.data,
                                     4096, ctypes.byref(cnt))
        return st, buf[:cnt.value]

    def demote(self, seq, lps):
        arr = np.asarray(lps, np.int32)
        buf = np.zeros((4096, 8), np.int32)
        cnt = ctypes.c_int32()
        st = self.L.mkvh_demote(self.h, seq, arr.ctypes.data, arr.size, buf.ctypes.data, 4096,
                                ctypes.byref(cnt))
        return st, buf[:cnt.value]

    def protect(self, seq, lps, on=True):
        arr = np.asarray(lps, np.int32)
        return self.L.mkvh_protect(self.h, seq, arr.ctypes.data, arr.size, 1 if on else 0)

    def policy_pages(self, seq, window):
        buf = np.zeros(4096, np.int32)
        n, nxt = ctypes.c_int32(), ctypes.c_int32()
        self.L.mkvh_policy_pages(self.h, seq, window, buf.ctypes.data, buf.size, ctypes.byref(n),
                                 ctypes.byref(nxt))
        return buf[:n.value].tolist(), nxt.value

    def pt(self, seq):
        buf = np.zeros(1 << 16, np.int32)
        n = self.L.mkvh_page_table(self.h, seq, buf.ctypes.data, buf.size)
        return buf[:n].copy()

    def free(self, fmt):
        return self.L.mkvh_free(self.h, fmt)

    def schedule(self, ids, Hq, chunk_pages=0, target_waves=0):
        ids = np.asarray(ids, np.int32)
        items = np.zeros((1 << 16, 8), np.int32)
        pages = np.zeros(1 << 20, np.int32)
        base = np.zeros(ids.size + 1, np.int32)
        counts = np.zeros(5, np.int32)
        st = self.L.mkvh_schedule(self.h, ids.ctypes.data, ids.size, Hq, chunk_pages, target_waves,
                                  items.ctypes.data, items.shape[0], pages.ctypes.data,
                                  pages.size, base.ctypes.data, counts.ctypes.data)
        if st:
            return st, None
        n8, n3, npg, nch, cp = counts
        return st, dict(items=items[:n8 + n3].copy(), n8=int(n8), n3=int(n3),
                        pages=pages[:npg].copy(), base=base.copy(), n_chunks=int(nch),
                        chunk_pages=int(cp))


def _host(lib, **over):
    kw = dict(num_kv_heads=2, head_dim=128, page_size=16, max_seqs=4, max_pages_per_seq=64,
              max_batch=4, max_q_heads=8, fp8_pages=32, tq3_pages=32, placement_seed=0)
    kw.update(over)
    return Host(lib, **kw)


TQ3_BIT = -2**31


def is_tq3(e):
    return e < 0


def test_descriptor_validation(lib):
    for bad in (dict(head_dim=96), dict(page_size=8), dict(page_size=24), dict(num_kv_heads=0),
                dict(max_q_heads=1, num_kv_heads=2), dict(max_q_heads=64, num_kv_heads=2),
                dict(fp8_pages=0), dict(max_batch=0)):
        with pytest.raises(ValueError):
            _host(lib, **bad)


def test_append_allocates_pages_in_order_without_seed(lib):
    h = _host(lib)
    st, plan = h.append(0, 40)
    assert st == OK
    # pages 0,1,2 touched: rows 0-15, 0-15, 0-7 from source rows 0, 16, 32
    assert plan[:, :5].tolist() == [[0, 0, 0, 16, 0], [1, 1, 0, 16, 16], [2, 2, 0, 8, 32]]
    st, plan = h.append(0, 10)
    assert plan[:, :5].tolist() == [[2, 2, 8, 8, 0], [3, 3, 0, 2, 8]]
    assert h.L.mkvh_seq_len(h.h, 0) == 50
    assert h.pt(0).tolist() == [0, 1, 2, 3]
    h.close()


def test_placement_is_seeded_and_deterministic(lib):
    a, b, c = (_host(lib, placement_seed=s, fp8_pages=64) for s in (7, 7, 8))
    for x in (a, b, c):
        x.append(0, 64 * 16)
    assert a.pt(0).tolist() == b.pt(0).tolist()
    assert a.pt(0).tolist() != c.pt(0).tolist()
    assert sorted(a.pt(0).tolist()) == list(range(64))
    assert a.pt(0).tolist() != list(range(64))
    for x in (a, b, c):
        x.close()


def test_enomem_has_no_partial_effect(lib):
    h = _host(lib, fp8_pages=4, tq3_pages=1)
    assert h.append(0, 48)[0] == OK
    v = h.L.mkvh_version(h.h)
    st, _ = h.append(1, 33)             # needs 3 pages, 1 free
    assert st == ENOMEM
    assert h.free(0) == 1 and h.L.mkvh_seq_len(h.h, 1) == 0 and h.L.mkvh_version(h.h) == v
    st, _ = h.demote(0, [0, 1])         # needs 2 TQ3 pages, 1 free
    assert st == ENOMEM
    assert (h.pt(0) >= 0).all() and h.free(1) == 1
    h.close()


def test_invalid_arguments_and_states(lib):
    h = _host(lib)
    assert h.append(5, 1)[0] == EINVAL
    assert h.append(-1, 1)[0] == EINVAL
    assert h.append(0, -3)[0] == EINVAL
    assert h.append(0, 64 * 16 + 1)[0] == ERANGE
    assert h.append(0, 20)[0] == OK
    assert h.demote(0, [2])[0] == EINVAL      # out of range
    assert h.demote(0, [0, 0])[0] == EINVAL   # duplicate
    assert h.demote(0, [0])[0] == OK
    assert h.demote(0, [0])[0] == ESTATE      # already TQ3
    assert h.demote(0, [1])[0] == OK          # partial tail page: allowed
    assert h.append(0, 1)[0] == ESTATE        # ... and then the sequence is frozen
    assert h.schedule([1], 8)[0] == EINVAL    # empty sequence
    assert h.schedule([0], 5)[0] == EINVAL    # Hq not a multiple of Hkv
    assert h.schedule([0], 10)[0] == ERANGE   # Hq > max_q_heads
    assert h.schedule([0, 0, 0, 0, 0], 8)[0] == ERANGE  # B > max_batch
    assert h.schedule([], 8)[0] == EINVAL     # empty batch
    assert h.schedule([5], 8)[0] == EINVAL    # id past max_seqs
    h.close()


def test_full_tq3_tail_accepts_appends(lib):
    h = _host(lib)
    assert h.append(0, 32)[0] == OK
    assert h.demote(0, [1])[0] == OK
    st, plan = h.append(0, 3)
    assert st == OK and plan[:, :4].tolist() == [[2, plan[0, 1], 0, 3]]
    h.close()


def test_demote_rewrites_entries_and_recycles_fp8_pages(lib):
    h = _host(lib, fp8_pages=8, tq3_pages=8, placement_seed=3)
    h.append(0, 100)
    before = h.pt(0)
    st, plan = h.demote(0, [1, 6])
    assert st == OK
    after = h.pt(0)
    assert is_tq3(after[1]) and is_tq3(after[6])
    assert (after[1] & 0x7FFFFFFF) == plan[0, 2] and plan[0, 1] == before[1]
    assert plan[0, 3] == 16 and plan[1, 3] == 100 - 6 * 16   # ntok of the partial last page
    assert h.free(0) == 8 - 7 + 2 and h.free(1) == 6
    h.L.mkvh_reset(h.h, 0)
    assert h.free(0) == 8 and h.free(1) == 8 and h.pt(0).size == 0
    h.close()


def _check_coverage(h, ids, sched, P):
    items = sched["items"]
    seen = {}
    chunks = set()
    for it in items:
        b, seq, off, npg, last, chunk, fmt, _ = it.tolist()
        assert ids[b] == seq and npg >= 1
        assert chunk not in chunks
        chunks.add(chunk)
        assert sched["base"][b] <= chunk < sched["base"][b + 1]
        pt = h.pt(seq)
        length = h.L.mkvh_seq_len(h.h, seq)
        lps = sched["pages"][off:off + npg]
        assert all(np.diff(lps) > 0)
        for lp in lps:
            assert int(is_tq3(pt[lp])) == fmt
            key = (b, int(lp))
            assert key not in seen
            seen[key] = True
        assert last == min(P, length - int(lps[-1]) * P)
    for b, seq in enumerate(ids):
        n_pages = h.pt(seq).size
        assert all((b, lp) in seen for lp in range(n_pages))
    assert chunks == set(range(sched["n_chunks"]))


def test_schedule_covers_every_page_once_ragged_and_scattered(lib):
    rng = np.random.default_rng(0)
    h = _host(lib, num_kv_heads=8, max_seqs=8, max_pages_per_seq=600, max_batch=8,
              max_q_heads=32, fp8_pages=4096, tq3_pages=4096, placement_seed=11)
    ids = [0, 3, 5, 7]
    for s in ids:
        L = int(rng.integers(1, 9000))
        assert h.append(s, L)[0] == OK
        n = -(-L // 16)
        dem = [p for p in range(n) if rng.random() < 0.8]
        assert h.demote(s, dem)[0] == OK
    for cp in (1, 3, 32, 1000):
        st, sc = h.schedule(ids, 32, chunk_pages=cp)
        assert st == OK
        _check_coverage(h, ids, sc, 16)
        assert sc["chunk_pages"] <= min(cp, 256)
    for waves in (1, 64, 2048, 100000):
        st, sc = h.schedule(ids, 32, target_waves=waves)
        assert st == OK
        _check_coverage(h, ids, sc, 16)
    h.close()


def test_long_context_schedule_is_balanced_for_the_resident_waves(lib):
    # 131072 tokens, last 4096 FP8.  G = 6 puts two kv-heads on a workgroup,
    # so an item takes four 4-wave workgroups for its 8 kv-heads.  The split-K
    # floor keeps at least 256 chunks even where the resident waves (2048
    # here) would give 128; 4096 resident waves (four per SIMD) give 256 too.
    # An FP8 page costs 1.2 TQ3 pages (a wave walks it one kv-head at a time;
    # 1.2 gave the shortest partial kernels in a sweep of the cost).
    h = _host(lib, num_kv_heads=8, max_seqs=1, max_pages_per_seq=8192, max_batch=1,
              max_q_heads=48, fp8_pages=8192, tq3_pages=8192, placement_seed=5)
    assert h.append(0, 131072)[0] == OK
    assert h.demote(0, list(range(8192 - 256)))[0] == OK
    for waves in (2048, 4096):
        st, sc = h.schedule([0], 48, target_waves=waves)
        assert st == OK
        assert 256 <= sc["n_chunks"] <= 264 and sc["n8"] >= 1 and sc["n3"] >= 1
        _check_coverage(h, [0], sc, 16)
        cost = np.array([float(it[3]) * (1.2 if i < sc["n8"] else 1) for i, it in enumerate(sc["items"])])
        assert cost.max() <= 1.15 * (7936 + 1.2 * 256) / 256
    sizes3 = sc["items"][sc["n8"]:, 3]
    assert sizes3.max() - sizes3.min() <= 1
    # algorithmic bytes: 126976 TQ3 tokens * 896 B + 4096 FP8 tokens * 2048 B + 256 pages * 64 B
    ids = np.array([0], np.int32)
    assert h.L.mkvh_kv_bytes(h.h, ids.ctypes.data, 1) == 122175488
    h.close()


def test_split_k_floor_only_for_long_batches(lib):
    # 4 sequences of 64-token pages, 769 pages in all (the d = 256 sweep
    # shape): fewer than 256 * 16 pages, so no floor; one kv-head per wave and
    # Hkv = 4 make an item four 4-wave workgroups, and 2048 resident waves
    # give 128 items
    h = _host(lib, num_kv_heads=4, head_dim=256, page_size=64, max_seqs=4, max_pages_per_seq=256,
              max_batch=4, max_q_heads=16, fp8_pages=1024, tq3_pages=1024)
    for s_, L in enumerate((16384, 16384, 16361, 1)):
        assert h.append(s_, L)[0] == OK
    st, sc = h.schedule([0, 1, 2, 3], 16, target_waves=2048)
    assert st == OK
    assert 120 <= sc["n_chunks"] <= 136
    _check_coverage(h, [0, 1, 2, 3], sc, 64)
    h.close()


def test_schedule_respects_chunk_capacity(lib):
    # chunks hold at most 240 pages: 4 * (2 + ceil(512 / 240)) = 20 is the
    # smallest max_chunks this descriptor accepts
    with pytest.raises(ValueError):
        _host(lib, max_pages_per_seq=512, fp8_pages=2048, max_chunks=19)
    h = _host(lib, max_pages_per_seq=512, fp8_pages=2048, tq3_pages=2048, max_chunks=20)
    for s in range(4):
        h.append(s, 512 * 16)
    st, sc = h.schedule([0, 1, 2, 3], 8, chunk_pages=1)
    assert st == OK and sc["n_chunks"] <= 20
    _check_coverage(h, [0, 1, 2, 3], sc, 16)
    h.close()


def test_chunks_never_exceed_240_pages(lib):
    # (a wave of the partial kernel then spans at most 64 pages)
    h = _host(lib, max_pages_per_seq=1024, fp8_pages=1024, tq3_pages=1024, max_seqs=2)
    h.append(0, 1000 * 16 + 3)
    assert h.demote(0, list(range(0, 900)))[0] == OK
    st, sc = h.schedule([0], 8, chunk_pages=4096)
    assert st == OK and sc["chunk_pages"] <= 240
    assert sc["n3"] == 4 and sc["n8"] == 1          # ceil(900 / 240), ceil(101 / 240)
    assert sc["items"][:, 3].max() <= 240
    _check_coverage(h, [0], sc, 16)
    h.close()


def test_host_metadata_under_asan_ubsan(tmp_path, repo_root):
    """Randomised append/demote/reset/schedule sequence in a sanitizer build."""
    import shutil
    if not shutil.which("g++"):
        pytest.skip("no host compiler")
    csrc = os.path.join(repo_root, "decode_attention_mixed_amd", "csrc")
    exe = str(tmp_path / "meta_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", csrc, os.path.join(csrc, "mkv_meta.cpp"),
           os.path.join(repo_root, "tests", "meta_fuzz.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout


# ------------------------------------------------------------ BF16 control pools
def test_bf16_control_pool_metadata(lib):
    """A control pool (kv_kind = MKV_KIND_BF16) has one slab, counts 4*Hkv*d
    bytes per token, never converts pages, and schedules every page as one
    format."""
    with pytest.raises(ValueError):
        _host(lib, kv_kind=1)                    # a TQ3 slab is not allowed
    with pytest.raises(ValueError):
        _host(lib, kv_kind=2, tq3_pages=0)       # unknown kind
    h = _host(lib, kv_kind=1, tq3_pages=0, fp8_pages=40)
    st, plan = h.append(0, 100)
    assert st == 0 and len(plan) == 7
    ids = np.array([0], np.int32)
    assert h.L.mkvh_kv_bytes(h.h, ids.ctypes.data, 1) == 100 * 4 * 2 * 128
    v0 = h.L.mkvh_version(h.h)
    st, _ = h.demote(0, [0])
    assert st == -3                              # MKV_ESTATE
    assert h.L.mkvh_version(h.h) == v0 and not any(is_tq3(e) for e in h.pt(0))
    st, sch = h.schedule([0], Hq=8)
    assert st == 0 and sch["n3"] == 0 and sch["n8"] >= 1
    assert sorted(p for p in sch["pages"].tolist() if p >= 0) == list(range(7))   # -1: spare room
    h.close()


# ------------------------------------------------------------ decode-step appends
def test_append_step_plans_and_page_table_patches(lib):
    """One token per sequence: row b goes to ids[b]; a sequence whose last page
    is full (or which is empty) opens a page and its plan carries the device
    page-table slot seq * pt_stride + lp and the new entry."""
    h = _host(lib, fp8_pages=40)
    assert h.append(0, 16)[0] == 0 and h.append(1, 5)[0] == 0
    st, plan = h.append_step([1, 0, 2], pt_stride=64)
    assert st == 0 and len(plan) == 3
    pt0, pt1, pt2 = h.pt(0), h.pt(1), h.pt(2)
    # seq 1: row 5 of its page 0, no new page
    assert list(plan[0]) == [0, pt1[0] & 0x7FFFFFFF, 5, 1, 0, -1, 0, 0]
    # seq 0: page 0 was full -> page 1 opened
    assert list(plan[1]) == [1, pt0[1], 0, 1, 1, 0 * 64 + 1, pt0[1], 0]
    # seq 2: empty -> page 0 opened
    assert list(plan[2]) == [0, pt2[0], 0, 1, 2, 2 * 64 + 0, pt2[0], 0]
    assert [h.L.mkvh_seq_len(h.h, s) for s in (0, 1, 2)] == [17, 6, 1]
    h.close()


def test_append_step_is_all_or_nothing(lib):
    h = _host(lib, fp8_pages=3, tq3_pages=4)
    assert h.append(0, 16)[0] == 0 and h.append(1, 16)[0] == 0
    v0 = h.L.mkvh_version(h.h)
    lens = lambda: [h.L.mkvh_seq_len(h.h, s) for s in range(4)]
    assert h.append_step([0, 2, 0])[0] == -1                 # repeated id: EINVAL
    assert h.append_step([0, 9])[0] == -1                    # bad id
    assert h.append_step([0, 1, 2])[0] == -2                 # 3 new pages, 1 free: ENOMEM
    assert lens() == [16, 16, 0, 0] and h.L.mkvh_version(h.h) == v0 and h.free(0) == 1
    assert h.append(2, 3)[0] == 0 and h.demote(2, [0])[0] == 0   # seq 2: partial TQ3 tail
    v1 = h.L.mkvh_version(h.h)
    assert h.append_step([3, 2])[0] == -3                    # frozen tail: ESTATE
    assert lens() == [16, 16, 3, 0] and h.L.mkvh_version(h.h) == v1
    assert h.append_step([3])[0] == 0 and lens()[3] == 1
    h.close()


def test_layout_version_moves_only_when_pages_change(lib):
    """Decode keeps its schedule while only token counts change; the layout
    version must move whenever a page opens, converts or is freed."""
    h = _host(lib, fp8_pages=40)
    ver = lambda: (h.L.mkvh_version(h.h), h.L.mkvh_layout_version(h.h))
    v0, l0 = ver()
    assert h.append(0, 10)[0] == 0                 # opens page 0
    v1, l1 = ver()
    assert v1 > v0 and l1 > l0
    assert h.append(0, 6)[0] == 0                  # fills page 0: lengths only
    v2, l2 = ver()
    assert v2 > v1 and l2 == l1
    assert h.append_step([0])[0] == 0              # opens page 1
    v3, l3 = ver()
    assert v3 > v2 and l3 > l2
    assert h.append_step([0])[0] == 0              # inside page 1
    v4, l4 = ver()
    assert v4 > v3 and l4 == l3
    assert h.demote(0, [0])[0] == 0                # converts page 0
    v5, l5 = ver()
    assert v5 > v4 and l5 > l4
    assert h.L.mkvh_reset(h.h, 0) == 0             # frees pages
    v6, l6 = ver()
    assert v6 > v5 and l6 > l5
    h.close()


# ------------------------------------------------------------ schedule checks and rollback
def test_built_schedules_pass_the_checker(lib):
    """check_schedule (the invariant the sanitizer fuzz also applies to edited
    schedules) accepts every schedule the builder makes: ragged batches,
    repeated sequences, fixed and balanced chunks, split-K floors."""
    rng = np.random.default_rng(3)
    h = _host(lib, num_kv_heads=8, max_seqs=8, max_pages_per_seq=600, max_batch=8,
              max_q_heads=32, fp8_pages=4096, tq3_pages=4096, placement_seed=11)
    for s in range(6):
        L = int(rng.integers(1, 9000))
        assert h.append(s, L)[0] == OK
        n = -(-L // 16)
        assert h.demote(s, [p for p in range(n) if rng.random() < 0.7])[0] == OK
    n = ctypes.c_int32()
    for ids in ([0], [1, 2, 3], [5, 5, 0], [0, 1, 2, 3, 4, 5]):
        arr = np.asarray(ids, np.int32)
        for cp, waves, floor in ((0, 2048, 0), (0, 4096, 256), (3, 0, 0), (0, 64, 1000), (0, 100000, 0)):
            st = h.L.mkvh_check_schedule(h.h, arr.ctypes.data, arr.size, 32, cp, waves, floor, ctypes.byref(n))
            assert st == OK, h.L.mkvh_last_error()
    h.close()


def test_rolled_back_calls_leave_no_trace(lib):
    """A call taken back with its undo record (what the C-ABI does when the
    call's device work cannot be enqueued) leaves page tables, lengths and free
    lists as they were: the next call hands out the very same pages."""
    def state(h):
        return ([h.pt(s).tolist() for s in range(4)], [h.L.mkvh_seq_len(h.h, s) for s in range(4)],
                h.free(0), h.free(1), h.L.mkvh_version(h.h), h.L.mkvh_layout_version(h.h))
    a = _host(lib, fp8_pages=60, tq3_pages=60, placement_seed=9, max_seqs=4)
    b = _host(lib, fp8_pages=60, tq3_pages=60, placement_seed=9, max_seqs=4)
    for h in (a, b):
        assert h.append(0, 40)[0] == OK and h.append(1, 3)[0] == OK
    s0 = state(a)
    assert a.L.mkvh_append_rollback(a.h, 0, 100) == OK
    assert a.L.mkvh_append_step_rollback(a.h, np.asarray([1, 2, 0], np.int32).ctypes.data, 3, 64) == OK
    lps = np.asarray([0, 2], np.int32)
    assert a.L.mkvh_demote_rollback(a.h, 0, lps.ctypes.data, 2) == OK
    assert state(a) == s0
    # the same calls made for real on both pools now give identical results
    for h in (a, b):
        assert h.append(0, 100)[0] == OK
        assert h.demote(0, [0, 2])[0] == OK
        assert h.append_step([1, 2, 0])[0] == OK
    assert state(a) == state(b)
    a.close()
    b.close()


@pytest.mark.parametrize("window", [0, 5, 16, 40])
def test_anchor_policy_matches_the_reference_policy(lib, window):
    """The library's anchor policy (what mkv_decode_step applies after each
    append: policy_pages, the conversion, then the cursor) decides exactly as
    the harness's reference policy over random one-token steps, with pages
    marked before and after they exist, marks cleared, and a sequence reset."""
    from decode_attention_mixed_amd.harness import AnchorPolicy
    rng = np.random.default_rng(100 + window)
    P, S = 16, 4
    h = _host(lib, max_seqs=S, max_pages_per_seq=64, max_batch=S, fp8_pages=256, tq3_pages=256)
    ref = AnchorPolicy(P, window, protected=[[] for _ in range(S)], demoted=[[] for _ in range(S)])
    lens = [0] * S
    for s_ in range(S):
        n = int(rng.integers(1, 90))
        assert h.append(s_, n)[0] == OK
        lens[s_] = n
    assert h.protect(0, [0, 3]) == OK and h.protect(2, [7, 40]) == OK
    ref.protected[0].update([0, 3])
    ref.protected[2].update([7, 40])
    converted = 0
    for step in range(300):
        if step == 120:                                  # unmark one, mark a passed page
            assert h.protect(2, [7], on=False) == OK
            ref.protected[2].discard(7)
            assert h.protect(1, [0]) == OK
            ref.protected[1].add(0)
        if step == 200:                                  # a sequence starts over
            assert lib.mkvh_reset(h.h, 3) == OK
            ref.protected[3].clear()
            ref.demoted[3].clear()
            ref.seen[3] = 0
            lens[3] = 0
        ids = sorted(rng.choice(S, size=int(rng.integers(1, S + 1)), replace=False).tolist())
        st, _ = h.append_step(ids)
        assert st == OK, (step, lib.mkvh_last_error())
        for s_ in ids:
            lens[s_] += 1
            got, nxt = h.policy_pages(s_, window)
            want = ref.step(s_, lens[s_])
            assert got == want, (step, s_, got, want)
            if got:
                assert h.demote(s_, got)[0] == OK
                converted += len(got)
            lib.mkvh_set_policy_next(h.h, s_, nxt)
            assert nxt == max(0, (lens[s_] - window) // P)        # lengths only grow between resets
    assert converted > 0
    for s_ in range(S):
        pt = h.pt(s_)
        full = max(0, (lens[s_] - window) // P)
        for lp in range(full):
            assert is_tq3(pt[lp]) == (lp in ref.demoted[s_]), (s_, lp)
    # marks outside the page-table range, and on a bad sequence, are refused
    assert h.protect(0, [64]) == EINVAL and h.protect(0, [-1]) == EINVAL and h.protect(9, [0]) == EINVAL
    h.close()
