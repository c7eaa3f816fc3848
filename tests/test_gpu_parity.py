"""GPU parity of the HIP path against the CPU oracle, through the C-ABI.

* page records (placement through the page table, FP8 append, TQ3 demote) are
  compared bit for bit with the oracle's records, on every valid byte;
* decode outputs are compared element by element: max |dO| <= 1e-3 and
  max |dLSE| <= 1e-4 (the acceptance bounds of this library).
Pool memory is poisoned with 0x7F before use, so unwritten slots hold NaN
patterns and any unmasked read shows up in the outputs.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import decode_attention_mixed_amd as mkv
from decode_attention_mixed_amd import harness as H
from decode_attention_mixed_amd import workloads as W
from oracle import attention as A
from tests import oracle_side as OS

pytestmark = pytest.mark.gpu

O_TOL = 1e-3
LSE_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _run_decode(pool, wl, seq_ids=None):
    seq_ids = list(range(wl.B)) if seq_ids is None else seq_ids
    q = H.q_tensor(wl)
    out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), device="cuda")
    lse = torch.full((wl.B, wl.Hq), float("nan"), device="cuda")
    mkv.decode(pool.handle, seq_ids, q, float(wl.tau), out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(out, lse, O, L, what):
    assert np.isfinite(out).all() and np.isfinite(lse).all(), what
    do = np.max(np.abs(out - O))
    dl = np.max(np.abs(lse - L))
    print(f"[{what}] max|dO|={do:.3e} max|dLSE|={dl:.3e}", flush=True)
    assert do <= O_TOL, (what, do)
    assert dl <= LSE_TOL, (what, dl)


def _check_records(pool, wl, models, seq_ids=None):
    seq_ids = list(range(wl.B)) if seq_ids is None else seq_ids
    for b, sid in enumerate(seq_ids):
        m = models[b]
        n = len(m.pages)
        recs = H.gather_records(pool, sid, n)
        pt = mkv.page_table(pool.handle, sid)
        anchors = set(int(x) for x in wl.anchors[b])
        for lp in range(n):
            want_tq3 = lp not in anchors
            assert (pt[lp] < 0) == want_tq3, (b, lp)
            ref = m.record(lp)
            mask = m.valid_mask(lp)
            got = recs[lp, :ref.size]
            bad = np.nonzero((got != ref) & mask)[0]
            assert bad.size == 0, f"seq {b} page {lp}: {bad.size} bytes differ, first at {bad[:8]}"


SMALL_CASES = {
    # name: kwargs of workloads.small
    "d128_p16_g4": dict(seed=11, B=3, Hq=8, Hkv=2, d=128, P=16, lengths=(200, 37, 513)),
    "d64_p32_g6": dict(seed=12, B=2, Hq=12, Hkv=2, d=64, P=32, lengths=(1, 650)),
    "d32_p16_g1": dict(seed=13, B=2, Hq=4, Hkv=4, d=32, P=16, lengths=(97, 16)),
    "d256_p64_g4": dict(seed=14, B=3, Hq=16, Hkv=4, d=256, P=64, lengths=(300, 64, 129),
                        outliers={"k": (6, 20.0)}),
    "d128_p16_g16": dict(seed=15, B=2, Hq=32, Hkv=2, d=128, P=16, lengths=(333, 48)),
    "d128_all_fp8": dict(seed=16, B=2, Hq=8, Hkv=2, d=128, P=16, lengths=(300, 17), anchor_frac=1.0),
    "d128_p48_outl": dict(seed=17, B=2, Hq=12, Hkv=2, d=128, P=48, lengths=(500, 95),
                          outliers={"k": (3, 8.0), "v": (3, 8.0)}),
}


@pytest.mark.parametrize("name", sorted(SMALL_CASES))
def test_small_records_and_decode(name):
    wl = W.small(**SMALL_CASES[name])
    print(f"case {name}: lengths={list(wl.lengths)}", flush=True)
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_cache(pool, wl)
    models = [OS.seq_model(wl, b) for b in range(wl.B)]
    _check_records(pool, wl, models)
    out, lse = _run_decode(pool, wl)
    O, L = OS.decode_all(wl, models)
    _check(out, lse, O, L, name)
    st = mkv.pool_stats(pool.handle)
    from oracle import pool_model as PM
    assert st["kv_bytes"] == sum(PM.kv_bytes(m) for m in models)
    assert st["dense_shadow_bytes"] == 0 and st["dense_fallbacks"] == 0
    assert st["ratio_vs_bf16"] == pytest.approx(2 * st["ratio_vs_fp8"])
    pool.close()


@pytest.mark.parametrize("name", sorted(n for n in SMALL_CASES if n != "d128_all_fp8"))
def test_batches_without_tq3_pages(name):
    """Every page anchored (FP8): a batch with no TQ3 item, for each head dim
    and kv-heads-per-wave case of the partial kernel."""
    wl = W.small(**{**SMALL_CASES[name], "anchor_frac": 1.0})
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_cache(pool, wl)
    models = [OS.seq_model(wl, b) for b in range(wl.B)]
    assert all(p.fmt == 0 for m in models for p in m.pages)
    out, lse = _run_decode(pool, wl)
    _check(out, lse, *OS.decode_all(wl, models), f"{name} all FP8")
    pool.close()


def test_all_tq3_with_partial_tail_and_single_token():
    wl = W.small(seed=21, B=3, Hq=8, Hkv=2, d=128, P=16, lengths=(77, 1, 16), anchor_frac=0.0)
    wl.anchors = [np.zeros(0, np.int64) for _ in range(wl.B)]       # every page TQ3
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_cache(pool, wl)
    models = [OS.seq_model(wl, b) for b in range(wl.B)]
    _check_records(pool, wl, models)
    out, lse = _run_decode(pool, wl)
    _check(out, lse, *OS.decode_all(wl, models), "all_tq3")
    with pytest.raises(mkv.MkvError) as e:                           # frozen partial TQ3 tail
        mkv.append(pool.handle, 0, torch.zeros(1, 2, 128, device="cuda"),
                   torch.zeros(1, 2, 128, device="cuda"))
    assert e.value.status == mkv.ESTATE
    pool.close()


def test_append_in_pieces_rescales_bit_exactly():
    wl = W.small(seed=31, B=2, Hq=8, Hkv=2, d=128, P=16, lengths=(150, 70))
    splits = [[1, 5, 10, 3, 40, 1, 90], [16, 16, 7, 31]]
    # make later rows raise the running amax so earlier rows get re-encoded
    kvs = []
    for b in range(wl.B):
        k, v = wl.kv(b)
        k[3::7] *= 3.0
        v[5::11] *= 5.0
        kvs.append((k, v))
    pool = H.DevicePool(H.pool_desc(wl))
    for b in range(wl.B):
        H.load_sequence(pool, wl, b, splits=splits[b], kv=kvs[b])
    models = [OS.seq_model(wl, b, splits=splits[b], kv=kvs[b]) for b in range(wl.B)]
    _check_records(pool, wl, models)
    out, lse = _run_decode(pool, wl)
    _check(out, lse, *OS.decode_all(wl, models), "append_pieces")
    pool.close()


def test_schedule_is_rebuilt_after_metadata_changes():
    wl = W.small(seed=41, B=2, Hq=8, Hkv=2, d=128, P=16, lengths=(64, 40))
    pool = H.DevicePool(H.pool_desc(wl, max_seqs=3, fp8_pages=64, tq3_pages=64,
                                    max_pages_per_seq=16))
    H.load_cache(pool, wl)
    models = [OS.seq_model(wl, b) for b in range(wl.B)]
    out, lse = _run_decode(pool, wl)
    _check(out, lse, *OS.decode_all(wl, models), "before")
    # grow sequence 1 and decode again: the cached schedule must be replaced
    extra = np.random.default_rng(5).standard_normal((30, 2, 128)).astype(np.float32)
    mkv.append(pool.handle, 1, torch.from_numpy(extra).cuda(), torch.from_numpy(extra).cuda())
    models[1].append(extra, extra)
    out, lse = _run_decode(pool, wl)
    O = np.zeros((2, 8, 128))
    L = np.zeros((2, 8))
    for b in range(2):
        O[b], L[b] = A.decode_seq(models[b], wl.q_bits[b], wl.tau)
    _check(out, lse, O, L, "after_append")
    # reordered batch and a repeated sequence
    q = H.q_tensor(wl)
    out2 = torch.zeros(2, 8, 128, device="cuda")
    lse2 = torch.zeros(2, 8, device="cuda")
    mkv.decode(pool.handle, [1, 1], q, float(wl.tau), out2, lse2)
    torch.cuda.synchronize()
    for b in range(2):
        Ob, Lb = A.decode_seq(models[1], wl.q_bits[b], wl.tau)
        assert np.max(np.abs(out2[b].cpu().numpy() - Ob)) <= O_TOL
        assert np.max(np.abs(lse2[b].cpu().numpy() - Lb)) <= LSE_TOL
    pool.close()


def test_error_paths_through_the_abi():
    wl = W.small(seed=51, B=1, Hq=8, Hkv=2, d=128, P=16, lengths=(40,))
    pool = H.DevicePool(H.pool_desc(wl, max_seqs=2, fp8_pages=3, tq3_pages=2))
    H.load_cache(pool, wl)
    q = H.q_tensor(wl)
    out = torch.zeros(1, 8, 128, device="cuda")
    lse = torch.zeros(1, 8, device="cuda")
    with pytest.raises(mkv.MkvError) as e:
        mkv.decode(pool.handle, [1], q, 0.1, out, lse)              # empty sequence
    assert e.value.status == mkv.EINVAL
    big = torch.zeros(100, 2, 128, device="cuda")
    with pytest.raises(mkv.MkvError) as e:
        mkv.append(pool.handle, 1, big, big)                         # needs 7 pages, 1 free...
    assert e.value.status in (mkv.ENOMEM, mkv.ERANGE)
    assert mkv.seq_info(pool.handle, 1) == (0, 0)                    # no partial effect
    with pytest.raises(mkv.MkvError) as e:
        mkv.demote(pool.handle, 0, [0])                              # page 0 is already TQ3
    assert e.value.status == mkv.ESTATE
    buf = torch.zeros(q.numel() + 8, dtype=q.dtype, device="cuda")
    q_odd = buf[1:1 + q.numel()].view(q.shape)                       # 2-byte offset
    q_odd.copy_(q)
    with pytest.raises(mkv.MkvError) as e:
        mkv.decode(pool.handle, [0], q_odd, 0.1, out, lse)
    assert e.value.status == mkv.EINVAL
    pool.close()


@pytest.mark.parametrize("narrow_max", ["0", "1000"])
def test_both_merge_kernels(monkeypatch, narrow_max):
    """The per-lane merge (few chunks per entry) and the workgroup-reduced merge
    (many), each forced through MKV_MERGE_NARROW_MAX on a schedule of one page
    per chunk (up to 38 chunks per sequence, 1 for the 33-token one)."""
    monkeypatch.setenv("MKV_MERGE_NARROW_MAX", narrow_max)
    monkeypatch.setenv("MKV_CHUNK_PAGES", "1")
    wl = W.small(seed=61, B=3, Hq=8, Hkv=2, d=128, P=16, lengths=(600, 33, 257))
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_cache(pool, wl)
    models = [OS.seq_model(wl, b) for b in range(wl.B)]
    out, lse = _run_decode(pool, wl)
    _check(out, lse, *OS.decode_all(wl, models), f"merge_narrow_max={narrow_max}")
    pool.close()


def test_graph_replays_of_the_decode(monkeypatch):
    """A decode captured in a graph (partial kernel and merge; the schedule
    cached by an eager call first, so capture records no upload) replays to
    the eager result bit for bit, replay after replay, with eager decodes of
    another pool in between."""
    monkeypatch.setenv("MKV_MERGE_NARROW_MAX", "0")
    wl = W.small(seed=65, B=3, Hq=8, Hkv=2, d=128, P=16, lengths=(900, 45, 333))
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_cache(pool, wl)
    q = H.q_tensor(wl)
    ids = list(range(wl.B))
    out = torch.zeros((wl.B, wl.Hq, wl.d), device="cuda")
    lse = torch.zeros((wl.B, wl.Hq), device="cuda")
    mkv.decode(pool.handle, ids, q, float(wl.tau), out, lse)
    torch.cuda.synchronize()
    want = (out.clone(), lse.clone())
    other = H.DevicePool(H.pool_desc(wl))
    H.load_cache(other, wl)
    o2 = torch.zeros_like(out)
    l2 = torch.zeros_like(lse)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mkv.decode(pool.handle, ids, q, float(wl.tau), out, lse)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want[0]) and torch.equal(lse, want[1]), f"replay {rep}"
        mkv.decode(other.handle, ids, q, float(wl.tau), o2, l2)
        torch.cuda.synchronize()
        assert torch.equal(o2, want[0]) and torch.equal(l2, want[1]), f"eager after replay {rep}"
    del g
    other.close()
    pool.close()


def test_paced_priorities_change_no_bits(monkeypatch):
    """Progress-paced wave priorities (on for launches whose workgroups are all
    resident at once, as here) only reorder instruction issue: the results are
    bit-identical to those of unpaced launches, and within tolerance of the
    oracle."""
    wl = W.small(seed=67, B=3, Hq=16, Hkv=4, d=128, P=16, lengths=(2000, 700, 1333))
    res = {}
    for pace in ("0", "1"):
        monkeypatch.setenv("MKV_PACE", pace)
        pool = H.DevicePool(H.pool_desc(wl))
        H.load_cache(pool, wl)
        res[pace] = _run_decode(pool, wl)
        pool.close()
    assert np.array_equal(res["0"][0], res["1"][0]) and np.array_equal(res["0"][1], res["1"][1])
    models = [OS.seq_model(wl, b) for b in range(wl.B)]
    _check(*res["1"], *OS.decode_all(wl, models), "paced")


NAMED = ["tiny", "ragged", "sweep0", "sweep10", "sweep50", "sweep100"]


def _named(name):
    if name.startswith("sweep"):
        return W.sweep(int(name[5:]) / 100.0)
    return getattr(W, name)()


@pytest.mark.parametrize("name", NAMED)
def test_named_workloads_full_parity(name):
    wl = _named(name)
    print(f"workload {name}: B={wl.B} lengths={list(wl.lengths)}", flush=True)
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_cache(pool, wl)
    models = [OS.seq_model(wl, b) for b in range(wl.B)]
    _check_records(pool, wl, models)
    out, lse = _run_decode(pool, wl)
    _check(out, lse, *OS.decode_all(wl, models), name)
    pool.close()


# ------------------------------------------------------------ BF16 control pools
def _control_splits(wl):
    """Append each sequence in two calls (the second starting mid-page)."""
    return [[int(L) // 3, int(L) - int(L) // 3] if L >= 3 else [int(L)] for L in wl.lengths]


@pytest.mark.parametrize("name", sorted(SMALL_CASES))
def test_bf16_control_records_and_decode(name):
    """Control pools: bf16 records bit for bit (valid rows) and decode against
    the oracle on the bf16-rounded rows."""
    wl = W.small(**SMALL_CASES[name])
    print(f"control case {name}: lengths={list(wl.lengths)}", flush=True)
    pool = H.DevicePool(H.pool_desc(wl, kind="bf16"))
    splits = _control_splits(wl)
    H.load_cache(pool, wl, splits=splits)
    models = [OS.bf16_model(wl, b, splits[b]) for b in range(wl.B)]
    for b, m in enumerate(models):
        n = len(m.bits)
        recs = H.gather_records(pool, b, n)
        pt = mkv.page_table(pool.handle, b)
        assert np.all(np.asarray(pt[:n]) >= 0)
        for lp in range(n):
            ref, mask = m.record(lp), m.valid_mask(lp)
            got = recs[lp, :ref.size]
            bad = np.nonzero((got != ref) & mask)[0]
            assert bad.size == 0, f"seq {b} page {lp}: {bad.size} bytes differ, first at {bad[:8]}"
    out, lse = _run_decode(pool, wl)
    _check(out, lse, *OS.decode_all(wl, models), f"bf16 {name}")
    st = mkv.pool_stats(pool.handle)
    from oracle import pool_model as PM
    assert st["kv_bytes"] == sum(PM.bf16_kv_bytes(m) for m in models)
    assert st["ratio_vs_bf16"] == pytest.approx(1.0) and st["tq3_pages_live"] == 0
    with pytest.raises(mkv.MkvError) as e:
        mkv.demote(pool.handle, 0, np.array([0], np.int32))
    assert e.value.status == mkv.ESTATE
    pool.close()


def test_bf16_control_decode_steps():
    """One-token appends to every sequence of a control pool (mkv_append_step,
    pages opened on the way), decoded and gathered against the oracle."""
    wl = W.small(seed=71, B=3, Hq=8, Hkv=2, d=64, P=16, lengths=(30, 16, 1))
    pool = H.DevicePool(H.pool_desc(wl, kind="bf16", max_pages_per_seq=8, fp8_pages=40))
    H.load_cache(pool, wl)
    models = [OS.bf16_model(wl, b) for b in range(wl.B)]
    rng = np.random.default_rng(72)
    ids = [2, 0, 1]                                   # any order of distinct sequences
    for step in range(20):
        k = rng.standard_normal((3, wl.Hkv, wl.d)).astype(np.float32)
        v = rng.standard_normal((3, wl.Hkv, wl.d)).astype(np.float32)
        mkv.append_step(pool.handle, ids, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        for row, b in enumerate(ids):
            models[b].append(k[row:row + 1], v[row:row + 1])
        if step in (0, 1, 14, 19):
            out, lse = _run_decode(pool, wl)
            _check(out, lse, *OS.decode_all(wl, models), f"control step {step}")
    for b in range(wl.B):
        recs = H.gather_records(pool, b, len(models[b].bits))
        for lp in range(len(models[b].bits)):
            ref, mask = models[b].record(lp), models[b].valid_mask(lp)
            assert np.array_equal(recs[lp, :ref.size][mask], ref[mask]), (b, lp)
    pool.close()


def test_bf16_control_long_context_parity():
    """The 131072-token Hq=48/Hkv=8 shape as a BF16 control cache, decoded in
    the launch configuration the benchmark times for the control."""
    wl = W.long()
    model = OS.bf16_model(wl, 0)
    O, L = A.decode_seq(model, wl.q_bits[0], wl.tau)
    pool = H.DevicePool(H.pool_desc(wl, kind="bf16"))
    H.load_cache(pool, wl)
    recs = H.gather_records(pool, 0, len(model.bits))
    for lp in (0, 1, 4000, 8191):
        ref, mask = model.record(lp), model.valid_mask(lp)
        assert np.array_equal(recs[lp, :ref.size][mask], ref[mask])
    out, lse = _run_decode(pool, wl)
    _check(out[0], lse[0], O, L, "bf16 long")
    pool.close()
    del pool
    torch.cuda.empty_cache()


def test_materialising_profile_records_and_decode():
    """mkv_materialize expands every page of a mixed pool (FP8 anchors, TQ3
    archive, partial tails, a 1-token sequence) into a control pool: records bit
    for bit against the oracle's materialised rows, then the control pool's
    decode against the oracle on those rows; the source pool is untouched and
    a second materialisation into a non-empty sequence is refused."""
    wl = W.small(seed=41, B=3, Hq=12, Hkv=2, d=128, P=16, lengths=(410, 1, 77),
                 outliers={"k": (3, 8.0), "v": (3, 8.0)})
    src = H.DevicePool(H.pool_desc(wl))
    H.load_cache(src, wl)
    dst = H.DevicePool(H.pool_desc(wl, kind="bf16"))
    for b in range(wl.B):
        mkv.materialize(src.handle, b, dst.handle, b)
    from oracle import pool_model as PM
    models = [PM.materialise(OS.seq_model(wl, b)) for b in range(wl.B)]
    for b, m in enumerate(models):
        recs = H.gather_records(dst, b, len(m.bits))
        for lp in range(len(m.bits)):
            ref, mask = m.record(lp), m.valid_mask(lp)
            bad = np.nonzero((recs[lp, :ref.size] != ref) & mask)[0]
            assert bad.size == 0, f"seq {b} page {lp}: {bad.size} bytes differ"
    out, lse = _run_decode(dst, wl)
    _check(out, lse, *OS.decode_all(wl, models), "materialised")
    out_src, lse_src = _run_decode(src, wl)
    _check(out_src, lse_src, *OS.decode_all(wl, [OS.seq_model(wl, b) for b in range(wl.B)]), "source")
    with pytest.raises(mkv.MkvError) as e:
        mkv.materialize(src.handle, 0, dst.handle, 0)
    assert e.value.status == mkv.ESTATE
    with pytest.raises(mkv.MkvError) as e:
        mkv.materialize(dst.handle, 0, src.handle, 1)
    assert e.value.status == mkv.EINVAL
    dst.close()
    src.close()


def test_multi_layer_step_in_one_call():
    """Per-layer caches as sequences of one pool (entry = layer * 2 + request):
    one decode call over all layers and layer-by-layer calls both match the
    oracle for every (layer, request)."""
    wl = W.canary(layers=3, length=2000)
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_cache(pool, wl)
    models = [OS.seq_model(wl, b) for b in range(wl.B)]
    O, L = OS.decode_all(wl, models)
    out, lse = _run_decode(pool, wl)
    _check(out, lse, O, L, "all layers in one call")
    q = H.q_tensor(wl)
    for layer in range(3):
        ids = [2 * layer, 2 * layer + 1]
        o = torch.empty(2, wl.Hq, wl.d, device="cuda")
        l = torch.empty(2, wl.Hq, device="cuda")
        mkv.decode(pool.handle, ids, q[ids[0]:ids[1] + 1].contiguous(), float(wl.tau), o, l)
        torch.cuda.synchronize()
        _check(o.cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64),
               O[ids[0]:ids[1] + 1], L[ids[0]:ids[1] + 1], f"layer {layer}")
    pool.close()


def test_decode_steps_with_appends_and_demotions():
    """A decode loop: each step appends one token to every sequence with one
    mkv_append_step call, demotes the pages an anchor policy releases (recency
    window of 40 tokens, the workload's older anchors protected) and decodes; the
    oracle replays the same appends and demotions.  Decodes along the way and
    every record at the end are checked."""
    wl = W.small(seed=51, B=3, Hq=8, Hkv=2, d=128, P=16, lengths=(100, 37, 250),
                 outliers={"k": (3, 8.0)})
    pool = H.DevicePool(H.pool_desc(wl, max_pages_per_seq=32))
    H.load_cache(pool, wl)
    models = [OS.seq_model(wl, b) for b in range(wl.B)]
    # anchors older than the window stay protected; the tail anchors are just
    # the recent pages and age out
    protected = [[a for a in wl.anchors[b] if (a + 1) * wl.P <= int(wl.lengths[b]) - 40]
                 for b in range(wl.B)]
    policy = H.AnchorPolicy(wl.P, 40, protected=protected,
                            demoted=[wl.demote_pages(b) for b in range(wl.B)])
    rng = np.random.default_rng(52)
    ids = list(range(wl.B))
    lengths = [int(x) for x in wl.lengths]
    n_demoted = 0
    for step in range(40):
        k = rng.standard_normal((wl.B, wl.Hkv, wl.d)).astype(np.float32)
        v = (rng.standard_normal((wl.B, wl.Hkv, wl.d)) * (1.0 + step % 3)).astype(np.float32)
        mkv.append_step(pool.handle, ids, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        for b in ids:
            models[b].append(k[b:b + 1], v[b:b + 1])
            lengths[b] += 1
            pages = policy.step(b, lengths[b])
            if pages:
                mkv.demote(pool.handle, b, np.asarray(pages, np.int32))
                for lp in pages:
                    models[b].demote(lp)
                n_demoted += len(pages)
        if step < 6 or step % 10 == 9:      # early steps mostly fill existing pages
            out, lse = _run_decode(pool, wl)
            _check(out, lse, *OS.decode_all(wl, models), f"step {step}")
    assert n_demoted >= 3
    for b in ids:
        pt = mkv.page_table(pool.handle, b)
        recs = H.gather_records(pool, b, len(models[b].pages))
        for lp, page in enumerate(models[b].pages):
            assert (pt[lp] < 0) == (page.fmt == 1), (b, lp)
            ref, mask = models[b].record(lp), models[b].valid_mask(lp)
            bad = np.nonzero((recs[lp, :ref.size] != ref) & mask)[0]
            assert bad.size == 0, f"seq {b} page {lp}: {bad.size} bytes differ"
    pool.close()


@pytest.mark.parametrize("case", ["window40", "window0", "batch36"])
def test_decode_step_appends_converts_and_decodes_in_one_call(case):
    """mkv_decode_step over 40 steps (one token per sequence, the anchor
    policy's conversions with the older anchors protected, the decode): each
    step's output against the oracle replaying the same appends and the
    reference policy's conversions, then every record and format.  window40
    takes the one-launch path; window0 converts, in the step that fills it,
    the page the step appended to (the path with separate launches); batch36
    has more pages than one launch's arguments hold (batched uploads).  A call
    with a bad Hq, and one whose conversions do not fit the TQ3 slab, change
    nothing."""
    window = {"window40": 40, "window0": 0, "batch36": 16}[case]
    if case == "batch36":
        lens = tuple(int(x) for x in np.random.default_rng(55).integers(20, 120, 36))
        wl = W.small(seed=56, B=36, Hq=4, Hkv=2, d=64, P=16, lengths=lens)
    else:
        wl = W.small(seed=51, B=3, Hq=8, Hkv=2, d=128, P=16, lengths=(100, 37, 250),
                     outliers={"k": (3, 8.0)})
    pool = H.DevicePool(H.pool_desc(wl, max_pages_per_seq=32))
    H.load_cache(pool, wl)
    models = [OS.seq_model(wl, b) for b in range(wl.B)]
    protected = [[a for a in wl.anchors[b] if (a + 1) * wl.P <= int(wl.lengths[b]) - window]
                 for b in range(wl.B)]
    policy = H.AnchorPolicy(wl.P, window, protected=protected,
                            demoted=[wl.demote_pages(b) for b in range(wl.B)])
    mkv.set_anchor_window(pool.handle, window)
    for b in range(wl.B):
        mkv.protect_pages(pool.handle, b, protected[b])
    rng = np.random.default_rng(53)
    ids = list(range(wl.B))
    lengths = [int(x) for x in wl.lengths]
    q = H.q_tensor(wl)
    out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), device="cuda")
    lse = torch.full((wl.B, wl.Hq), float("nan"), device="cuda")
    n_demoted = 0
    for step in range(40):
        k = rng.standard_normal((wl.B, wl.Hkv, wl.d)).astype(np.float32)
        v = (rng.standard_normal((wl.B, wl.Hkv, wl.d)) * (1.0 + step % 3)).astype(np.float32)
        mkv.decode_step(pool.handle, ids, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), q,
                        float(wl.tau), out, lse)
        torch.cuda.synchronize()
        for b in ids:
            models[b].append(k[b:b + 1], v[b:b + 1])
            lengths[b] += 1
            for lp in policy.step(b, lengths[b]):
                models[b].demote(lp)
                n_demoted += 1
        if step < 6 or step % 5 == 4:
            _check(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                   *OS.decode_all(wl, models), f"decode_step {step}")
    assert n_demoted >= 3
    for b in ids:
        pt = mkv.page_table(pool.handle, b)
        recs = H.gather_records(pool, b, len(models[b].pages))
        for lp, page in enumerate(models[b].pages):
            assert (pt[lp] < 0) == (page.fmt == 1), (b, lp)
            ref, mask = models[b].record(lp), models[b].valid_mask(lp)
            bad = np.nonzero((recs[lp, :ref.size] != ref) & mask)[0]
            assert bad.size == 0, f"seq {b} page {lp}: {bad.size} bytes differ"
    if case != "window40":
        pool.close()
        return
    # a bad Hq is refused before the append
    kz = torch.zeros(wl.B, wl.Hkv, wl.d, device="cuda")
    ids_arr = (ctypes.c_int32 * wl.B)(*ids)
    st = mkv._load().mkv_decode_step(pool.handle, ids_arr, wl.B, ctypes.c_void_p(kz.data_ptr()),
                                     ctypes.c_void_p(kz.data_ptr()), ctypes.c_void_p(q.data_ptr()), 3,
                                     ctypes.c_float(1.0), ctypes.c_void_p(out.data_ptr()),
                                     ctypes.c_void_p(lse.data_ptr()), None)
    assert st == mkv.EINVAL
    assert [mkv.seq_info(pool.handle, b)[0] for b in ids] == lengths
    pool.close()
    # conversions that do not fit the TQ3 slab: ENOMEM, and the append is taken back
    wl2 = W.small(seed=54, B=1, Hq=4, Hkv=2, d=64, P=16, lengths=(80,))
    n_tq3 = wl2.n_pages(0) - len(wl2.anchors[0])
    pool2 = H.DevicePool(H.pool_desc(wl2, tq3_pages=n_tq3, fp8_pages=wl2.n_pages(0) + 4,
                                     max_pages_per_seq=wl2.n_pages(0) + 4))
    H.load_cache(pool2, wl2)
    mkv.set_anchor_window(pool2.handle, 0)
    L0 = mkv.seq_info(pool2.handle, 0)[0]
    fp8_before = mkv.pool_stats(pool2.handle)["fp8_pages_live"]
    k1 = torch.zeros(1, wl2.Hkv, wl2.d, device="cuda")
    q2 = H.q_tensor(wl2)
    o2 = torch.empty(1, wl2.Hq, wl2.d, device="cuda")
    l2 = torch.empty(1, wl2.Hq, device="cuda")
    with pytest.raises(mkv.MkvError) as e:
        mkv.decode_step(pool2.handle, [0], k1, k1, q2, float(wl2.tau), o2, l2)
    assert e.value.status == mkv.ENOMEM
    assert mkv.seq_info(pool2.handle, 0)[0] == L0
    assert mkv.pool_stats(pool2.handle)["fp8_pages_live"] == fp8_before
    mkv.set_anchor_window(pool2.handle, -1)           # off: the same step goes through
    mkv.decode_step(pool2.handle, [0], k1, k1, q2, float(wl2.tau), o2, l2)
    torch.cuda.synchronize()
    assert mkv.seq_info(pool2.handle, 0)[0] == L0 + 1
    pool2.close()


@pytest.mark.parametrize("B", [3, 40])
def test_append_steps_keep_the_cached_schedule_current(B):
    """Decode after every mkv_append_step.  A step of at most 32 pages carries
    its plan in the kernel arguments and, when it opens no page, brings the
    cached schedule's last-page token counts up to date in the same launch (a
    step that opens a page leaves the rebuild to the decode); larger steps take
    the uploaded plan.  The batch repeats sequence 0 and leaves out the last
    one, and a plain mkv_append between two steps must be picked up too.
    Every fifth step demotes an older FP8 page of sequences 0 and 1, which the
    cached schedule takes in place where it can."""
    rng = np.random.default_rng(60 + B)
    lengths = tuple(int(x) for x in rng.integers(1, 60, B))
    wl = W.small(seed=61 + B, B=B, Hq=4, Hkv=2, d=64, P=16, lengths=lengths)
    n_pages = sum(wl.n_pages(b) for b in range(B))
    pool = H.DevicePool(H.pool_desc(wl, max_pages_per_seq=16, fp8_pages=n_pages + 4 * B + 16))
    H.load_cache(pool, wl)
    models = [OS.seq_model(wl, b) for b in range(B)]
    ids = list(range(B))
    batch = [0] + ids[:-1]
    n_demoted = 0
    q = H.q_tensor(wl)
    out = torch.empty(B, wl.Hq, wl.d, device="cuda")
    lse = torch.empty(B, wl.Hq, device="cuda")
    for step in range(24):
        k = rng.standard_normal((B, wl.Hkv, wl.d)).astype(np.float32)
        v = rng.standard_normal((B, wl.Hkv, wl.d)).astype(np.float32)
        mkv.append_step(pool.handle, ids, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        for b in ids:
            models[b].append(k[b:b + 1], v[b:b + 1])
        if step == 7:
            x = rng.standard_normal((1, wl.Hkv, wl.d)).astype(np.float32)
            mkv.append(pool.handle, 1, torch.from_numpy(x).cuda(), torch.from_numpy(x).cuda())
            models[1].append(x, x)
        if step % 5 == 3:
            # demote the oldest FP8 page outside the last two of sequences 0 and 1
            for sid in (0, 1):
                pages = models[sid].pages
                old = [lp for lp, pg in enumerate(pages[:-2]) if pg.fmt == 0]
                if old:
                    mkv.demote(pool.handle, sid, np.asarray(old[:1], np.int32))
                    models[sid].demote(old[0])
                    n_demoted += 1
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        mkv.decode(pool.handle, batch, q, float(wl.tau), out, lse)
        torch.cuda.synchronize()
        O = np.zeros((B, wl.Hq, wl.d))
        L = np.zeros((B, wl.Hq))
        for b, sid in enumerate(batch):
            O[b], L[b] = A.decode_seq(models[sid], wl.q_bits[b], wl.tau)
        _check(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), O, L,
               f"B={B} step {step}")
    assert n_demoted >= 3
    pool.close()


@pytest.fixture(scope="module")
def long_case():
    wl = W.long()
    model = OS.seq_model(wl, 0)
    O, L = A.decode_seq(model, wl.q_bits[0], wl.tau)
    return wl, model, O, L


def test_long_context_full_parity(long_case):
    """131072-token, Hq=48/Hkv=8 cache, decoded in the launch configuration the
    benchmark times (one sequence per call, default split-K schedule)."""
    wl, model, O, L = long_case
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_cache(pool, wl)
    recs = H.gather_records(pool, 0, len(model.pages))
    for lp in (0, 1, 4000, 7935, 7936, 8191):       # TQ3 and FP8 pages, both ends
        ref = model.record(lp)
        assert np.array_equal(recs[lp, :ref.size][model.valid_mask(lp)], ref[model.valid_mask(lp)])
    out, lse = _run_decode(pool, wl)
    _check(out[0], lse[0], O, L, "long")
    # repeated calls reuse the cached schedule and give identical results
    out2, lse2 = _run_decode(pool, wl)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    pool.close()


def test_throughput_batch_full_parity():
    """The B=64 throughput batch at full size: 16K-32K-token sequences whose
    pages scatter over slabs holding 60% of HBM, decoded in one call over the
    whole batch as the benchmark times it; every sequence is compared element
    by element with the oracle (computed in worker processes)."""
    wl = W.throughput()
    print(f"throughput: B={wl.B} tokens={int(np.sum(wl.lengths))} "
          f"slabs fp8={wl.fp8_pages} tq3={wl.tq3_pages} pages", flush=True)
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_cache(pool, wl)
    print("throughput: cache built", flush=True)
    out, lse = _run_decode(pool, wl)
    pool.close()
    del pool
    torch.cuda.empty_cache()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ref = OS.decode_parallel(("throughput", {}), range(wl.B))
    print("throughput: oracle done", flush=True)
    for b in range(wl.B):
        _check(out[b], lse[b], *ref[b], f"throughput[{b}] L={int(wl.lengths[b])}")


def test_canary16_full_parity():
    """The 16-layer canary step at full size (32 entries of 59008 tokens, each
    layer's cache a sequence of one pool) in one decode call, every entry
    compared with the oracle."""
    wl = W.canary(16)
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_cache(pool, wl)
    print(f"canary16: B={wl.B} cache built", flush=True)
    out, lse = _run_decode(pool, wl)
    pool.close()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ref = OS.decode_parallel(("canary", {"layers": 16}), range(wl.B))
    for b in range(wl.B):
        _check(out[b], lse[b], *ref[b], f"canary16[{b}]")


def _check_schedule_export(pool, ids):
    """The device copy of the cached schedule names every page of the batch's
    sequences exactly once, each by its page-table entry (bit-exact), in items
    of one format whose last page and token count match the sequence."""
    sc = mkv.debug_schedule(pool.handle)
    items, ent = sc["items"], sc["entries"]
    seen = {s: [] for s in ids}
    for it in items:
        b, seq, off, npg, last_ntok, chunk, fmt, last_lp = (int(x) for x in it)
        assert seq == ids[b]
        e = ent[off:off + npg]
        assert npg >= 1 and all((x < 0) == (fmt == 1) for x in e), it
        pt = mkv.page_table(pool.handle, seq)
        assert pt[last_lp] == e[-1], it
        L, n = mkv.seq_info(pool.handle, seq)
        assert last_ntok == (L - pool.desc.page_size * (n - 1) if last_lp == n - 1 else pool.desc.page_size), it
        seen[seq] += [int(x) for x in e]
    for s in ids:
        pt = mkv.page_table(pool.handle, s)
        assert sorted(seen[s]) == sorted(int(x) for x in pt), s
    return sc


def test_schedule_export_matches_page_tables():
    """Schedule built by decode, then edited in place by one-token appends (which
    open pages) and by demotions: after each change the device's schedule
    region agrees with mkv_page_table bit for bit."""
    wl = W.small(seed=41, B=4, Hq=8, Hkv=2, d=128, P=16, lengths=(150, 31, 400, 16), anchor_frac=0.4)
    pool = H.DevicePool(H.pool_desc(wl, max_pages_per_seq=64, fp8_pages=128, tq3_pages=128))
    H.load_cache(pool, wl)
    ids = list(range(wl.B))
    q = H.q_tensor(wl)
    out = torch.empty(wl.B, wl.Hq, wl.d, device="cuda")
    lse = torch.empty(wl.B, wl.Hq, device="cuda")
    mkv.decode(pool.handle, ids, q, float(wl.tau), out, lse)
    torch.cuda.synchronize()
    _check_schedule_export(pool, ids)
    rng = np.random.default_rng(3)
    edits = 0
    for step in range(40):
        k = torch.from_numpy(rng.standard_normal((wl.B, wl.Hkv, wl.d), dtype=np.float32)).cuda()
        mkv.append_step(pool.handle, ids, k, k)
        if step % 10 == 9:
            for s in (0, 2):
                pt = mkv.page_table(pool.handle, s)
                fp8 = [lp for lp in range(len(pt) - 1) if pt[lp] >= 0]
                if fp8:
                    mkv.demote(pool.handle, s, fp8[:2])
        torch.cuda.synchronize()
        try:
            _check_schedule_export(pool, ids)          # the edited schedule, before any rebuild
            edits += 1
        except mkv.MkvError as e:
            assert e.status == mkv.ESTATE               # no schedule cached: the next decode builds one
        mkv.decode(pool.handle, ids, q, float(wl.tau), out, lse)
        torch.cuda.synchronize()
        _check_schedule_export(pool, ids)
    print(f"schedule checked after {edits} in-place edits", flush=True)
    assert edits >= 30
    pool.close()


def test_demote_codes_at_exact_thresholds():
    """TQ3 codes of values on and beside the thresholds b * s: every 32-dim
    group holds +-448 times the page's factor, so the page-head scale is that
    factor exactly (amax / 448) and the group scale is 128 times it; the
    other entries are E4M3 values equal to b * s (b = +-1, +-2, +-3) and their
    E4M3 neighbours.  Four pages at factors 1, 1/2, 2^-10 and 3; all pages
    converted, records bit for bit against the oracle, then the decode with
    the queries scaled by 2^-12 (exactly, in bf16): keys of magnitude up to
    1344 would otherwise put the log-sum-exp in the hundreds, where fp32
    cannot hold it to the absolute tolerance."""
    wl = W.small(seed=47, B=1, Hq=8, Hkv=2, d=128, P=16, lengths=(64,), anchor_frac=0.0)
    wl.anchors = [np.zeros(0, np.int64)]
    base = np.array([448, 384, 352, 416, 256, 240, 288, 128, 120, 144, 0, 64, 8, 192, 320, 448], np.float32)
    vals = np.concatenate([base, -base])                  # 32 values, +-448 included
    rng = np.random.default_rng(9)
    rows = np.empty((64, 2, 2, 128), np.float32)          # token, K/V, kv-head, dim
    for t in range(64):
        for kv in range(2):
            for h in range(2):
                rows[t, kv, h] = np.concatenate([rng.permutation(vals) for _ in range(4)])
    factor = np.repeat(np.array([1.0, 0.5, 2.0 ** -10, 3.0], np.float32), 16)[:, None, None, None]
    rows = rows * factor
    # values at 1/64 of the keys' size (a power of two: their codes sit on
    # the thresholds all the same) keep the outputs small enough for the
    # absolute tolerance
    k, v = rows[:, 0].copy(), rows[:, 1] * np.float32(1.0 / 64.0)
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_sequence(pool, wl, 0, kv=(k, v))
    model = OS.seq_model(wl, 0, kv=(k, v))
    assert all(p.fmt == 1 for p in model.pages)
    _check_records(pool, wl, [model])
    # the exact-tie values reach the packer: group scales 128 x the page factor
    # (keys) and 2 x it (values)
    for kvi, unit in ((0, 128.0), (1, 2.0)):
        scales = np.unique(np.concatenate([p.tscale[kvi, :, :p.ntok].astype(np.float64).ravel()
                                           for p in model.pages]))
        assert set(scales.tolist()) == {unit * f for f in (1.0, 0.5, 2.0 ** -10, 3.0)}
    from oracle import codecs as CD
    from oracle import attention as OA
    qb = CD.bf16_encode(CD.bf16_bits_to_value(wl.q_bits).astype(np.float32) * np.float32(2.0 ** -12))
    q = torch.from_numpy(qb.view(np.int16).copy()).view(torch.bfloat16).cuda()
    out = torch.empty(1, wl.Hq, wl.d, device="cuda")
    lse = torch.empty(1, wl.Hq, device="cuda")
    mkv.decode(pool.handle, [0], q, float(wl.tau), out, lse)
    torch.cuda.synchronize()
    O, L = OA.decode_seq(model, qb[0], wl.tau)
    _check(out[0].cpu().numpy().astype(np.float64), lse[0].cpu().numpy().astype(np.float64), O, L,
           "threshold values")
    pool.close()


def test_edge_values_records_and_decode():
    """Edge values through append, demote and decode: a kv-head whose rows are
    zero on whole pages (FP8 scale 1, TQ3 scale 0), zero groups, groups so small
    that the TQ3 scale is an fp16 subnormal, groups so large that it clamps to
    65504 (records only: their attention outputs exceed what fp32 can hold to
    the absolute tolerance), and queries scaled by 16 and by 1/256."""
    wl = W.small(seed=43, B=3, Hq=8, Hkv=2, d=128, P=16, lengths=(160, 96, 120), anchor_frac=0.3)
    kvs = [wl.kv(b) for b in range(wl.B)]
    k0, v0 = kvs[0]
    k0[16:48, 1, :] = 0.0                          # kv-head 1: pages 1, 2 (TQ3) and the
    v0[16:48, 1, :] = 0.0                          # last page (FP8 anchor) all zero
    k0[144:160, 1, :] = 0.0
    v0[144:160, 1, :] = 0.0
    k0[:, 0, 32:64] = 0.0                          # a zero group in every page of kv-head 0
    v0[64:112, 0, 96:128] = 0.0
    k1, v1 = kvs[1]
    k1[:, 0, 0:32] *= np.float32(3e-6)            # TQ3 scales ~1e-6: fp16 subnormals
    v1[:, 1, 64:96] *= np.float32(2e-7)
    k2, v2 = kvs[2]
    k2[:, 1, 32:64] *= np.float32(4e5)            # TQ3 scales clamp to 65504
    v2[:, 0, 0:32] *= np.float32(5e5)
    pool = H.DevicePool(H.pool_desc(wl))
    for b in range(wl.B):
        H.load_sequence(pool, wl, b, kv=kvs[b])
    models = [OS.seq_model(wl, b, kv=kvs[b]) for b in range(wl.B)]
    _check_records(pool, wl, models)
    # the clamp and subnormal cases really occur in the records
    from oracle import codecs as CD
    from oracle import attention as OA
    scales = np.concatenate([m.pages[lp].tscale[:, :, :m.pages[lp].ntok].astype(np.float64).ravel()
                             for m in models for lp in range(len(m.pages)) if m.pages[lp].fmt == 1])
    assert np.any(scales == 65504.0) and np.any((scales > 0) & (scales < 2.0 ** -14)) and np.any(scales == 0)
    assert any(np.any(m.pages[lp].scale == 1.0) for m in models for lp in range(len(m.pages))
               if m.pages[lp].fmt == 0)            # an all-zero FP8 page-head: sigma = 1
    qf = CD.bf16_bits_to_value(wl.q_bits).astype(np.float32)
    qf[0, :4] *= 16.0                              # sharper softmax on the first 4 query heads
    qf[1, 4:] *= 1.0 / 256.0                       # nearly flat on the others
    qb = CD.bf16_encode(qf)
    q = torch.from_numpy(qb[:2].view(np.int16).copy()).view(torch.bfloat16).cuda()
    out = torch.empty(2, wl.Hq, wl.d, device="cuda")
    lse = torch.empty(2, wl.Hq, device="cuda")
    mkv.decode(pool.handle, [0, 1], q, float(wl.tau), out, lse)
    torch.cuda.synchronize()
    for b in range(2):
        Ob, Lb = OA.decode_seq(models[b], qb[b], wl.tau)
        _check(out[b].cpu().numpy().astype(np.float64), lse[b].cpu().numpy().astype(np.float64), Ob, Lb,
               f"edge values [{b}]")
    pool.close()


@pytest.mark.parametrize("tau_factor", [-1.0, 0.0, -4.0])
def test_negative_and_zero_softmax_scale(tau_factor):
    """The softmax scale is the caller's fp32 factor on <q, k>, any sign: a
    negative scale reverses the order of the scores (the partial kernels fold
    its sign into the query operands) and a zero scale gives uniform weights
    (O = mean of the values, LSE = log of the token count).  Mixed pools with
    partial last tiles on both formats and a one-token sequence."""
    wl = W.small(seed=47, B=3, Hq=12, Hkv=2, d=128, P=16, lengths=(203, 1, 77), anchor_frac=0.3,
                 outliers={"k": (3, 8.0)})
    pool = H.DevicePool(H.pool_desc(wl))
    H.load_cache(pool, wl)
    tau = float(np.float32(wl.tau * tau_factor))
    q = H.q_tensor(wl)
    out = torch.empty(wl.B, wl.Hq, wl.d, device="cuda")
    lse = torch.empty(wl.B, wl.Hq, device="cuda")
    mkv.decode(pool.handle, list(range(wl.B)), q, tau, out, lse)
    torch.cuda.synchronize()
    for b in range(wl.B):
        model = OS.seq_model(wl, b)
        O, L = A.decode_seq(model, wl.q_bits[b], tau)
        _check(out[b].cpu().numpy().astype(np.float64), lse[b].cpu().numpy().astype(np.float64), O, L,
               f"softmax scale x{tau_factor} [{b}]")
    pool.close()
