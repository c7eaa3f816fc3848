"""Pins of the oracle's pool model and attention.

* brute force: pure-Python scalar loops (struct-parsed page records, math.fsum)
  against the numpy oracle;
* partition invariance of partial states + merge;
* all-FP8 / all-TQ3 degenerate caches against torch float64 softmax;
* closed forms (q = 0, L = 1, identical keys);
* append / demote on inputs whose quantisation is exact.
"""
import math
import struct

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import codecs as C
from oracle import pool_model as PM


def _build(rng, Hkv, d, P, L, demote=(), chunks=None, scale=1.0):
    k = (rng.standard_normal((L, Hkv, d)) * scale).astype(np.float32)
    v = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    seq = PM.SeqModel(Hkv, d, P)
    if chunks is None:
        seq.append(k, v)
    else:
        pos = 0
        for n in chunks:
            seq.append(k[pos:pos + n], v[pos:pos + n])
            pos += n
        assert pos == L
    for lp in demote:
        seq.demote(lp)
    return seq, k, v


def _q_bits(rng, Hq, d):
    q = torch.from_numpy(rng.standard_normal((Hq, d)).astype(np.float32)).to(torch.bfloat16)
    return q.view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------- brute force
def _e4m3_scalar(code):
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 15
    m = code & 7
    if e == 0:
        return sign * math.ldexp(m, -9)
    return sign * math.ldexp(8 + m, e - 10)


def _brute_force(seq, q_bits, tau32):
    """Dequantise every valid token from the page *records* with Python scalars,
    then softmax attention with math.fsum."""
    Hkv, P, d = seq.Hkv, seq.P, seq.d
    G32 = d // 32
    rowb = 3 * d // 8
    blk = P * d * 7 // 8
    Ks, Vs = [], []
    for lp, page in enumerate(seq.pages):
        rec = seq.record(lp).tobytes()
        for t in range(page.ntok):
            krow, vrow = [], []
            for h in range(Hkv):
                if page.fmt == PM.FP8:
                    sk, sv = struct.unpack_from("<ff", rec, 2 * Hkv * P * d + 8 * h)
                    kb = (2 * h) * P * d + t * d
                    vb = (2 * h + 1) * P * d + t * d
                    krow.append([_e4m3_scalar(rec[kb + j]) * sk for j in range(d)])
                    vrow.append([_e4m3_scalar(rec[vb + j]) * sv for j in range(d)])
                else:
                    base = h * blk
                    for which, dst in ((0, krow), (1, vrow)):
                        stream = int.from_bytes(rec[base + which * P * rowb + t * rowb:
                                                    base + which * P * rowb + (t + 1) * rowb], "little")
                        soff = base + 2 * P * rowb + which * P * G32 * 2 + t * G32 * 2
                        scales = struct.unpack_from("<%de" % G32, rec, soff)
                        dst.append([(((stream >> (3 * j)) & 7) - 3.5) * scales[j // 32]
                                    for j in range(d)])
            Ks.append(krow)
            Vs.append(vrow)
    Hq = q_bits.shape[0]
    G = Hq // Hkv
    tau = float(np.float32(tau32))
    O = np.zeros((Hq, d))
    lse = np.zeros(Hq)
    for h in range(Hq):
        q = [struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in q_bits[h]]
        s = [tau * math.fsum(q[j] * Ks[t][h // G][j] for j in range(d)) for t in range(len(Ks))]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        Lsum = math.fsum(w)
        for j in range(d):
            O[h, j] = math.fsum(w[t] * Vs[t][h // G][j] for t in range(len(Ks))) / Lsum
        lse[h] = m + math.log(Lsum)
    return O, lse


@pytest.mark.parametrize("L,demote,chunks", [
    (48, (0, 2), None),            # mixed, full pages
    (45, (0, 1, 11), None),        # mixed, partial TQ3 tail page
    (30, (), (7, 1, 22)),          # FP8 only, grown across calls
    (9, (0, 1, 2), None),          # all TQ3
])
def test_oracle_matches_brute_force(L, demote, chunks):
    rng = np.random.default_rng(100 + L)
    Hkv, d, P, Hq = 2, 32, 4, 4
    seq, _, _ = _build(rng, Hkv, d, P, L, demote, chunks)
    qb = _q_bits(rng, Hq, d)
    tau = np.float32(1 / math.sqrt(d))
    O, lse = A.decode_seq(seq, qb, tau)
    Ob, lseb = _brute_force(seq, qb, tau)
    assert np.max(np.abs(O - Ob)) < 1e-12
    assert np.max(np.abs(lse - lseb)) < 1e-12


# ------------------------------------------------------- partition invariance
def test_merge_over_any_page_partition_equals_single_pass():
    rng = np.random.default_rng(21)
    Hkv, d, P, Hq, L = 2, 64, 8, 6, 203
    n_pages = -(-L // P)
    demote = [p for p in range(n_pages) if rng.random() < 0.7]
    seq, _, _ = _build(rng, Hkv, d, P, L, demote, scale=2.0)
    qb = _q_bits(rng, Hq, d)
    tau = np.float32(1 / math.sqrt(d))
    O, lse = A.decode_seq(seq, qb, tau)
    q = C.bf16_bits_to_value(qb)
    K, V = seq.dense()
    starts = np.concatenate([[0], np.cumsum([pg.ntok for pg in seq.pages])])
    partitions = {
        "singletons": [[p] for p in range(n_pages)],
        "format_split": [[p for p in range(n_pages) if seq.pages[p].fmt == f] for f in (0, 1)],
        "with_empty": [[], list(range(0, 10)), [], list(range(10, n_pages)), []],
        "random": None,
    }
    perm = rng.permutation(n_pages)
    cuts = np.sort(rng.choice(np.arange(1, n_pages), 6, replace=False))
    partitions["random"] = [list(x) for x in np.split(perm, cuts)]
    G = Hq // Hkv
    for name, parts in partitions.items():
        for h in range(Hq):
            states = []
            for pages in parts:
                idx = np.concatenate([np.arange(starts[p], starts[p + 1]) for p in pages]) \
                    if pages else np.zeros(0, np.int64)
                states.append(A.partial(q[h], K[idx, h // G], V[idx, h // G], float(tau)))
            Om, lm = A.merge(states)
            assert np.max(np.abs(Om - O[h])) < 1e-12, name
            assert abs(lm - lse[h]) < 1e-12, name


# ------------------------------------------------------ degenerate all-one-format
@pytest.mark.parametrize("fmt", ["fp8", "tq3"])
def test_single_format_cache_equals_dense_softmax(fmt):
    rng = np.random.default_rng(31)
    Hkv, d, P, Hq, L = 2, 128, 16, 8, 300
    n_pages = -(-L // P)
    demote = range(n_pages) if fmt == "tq3" else ()
    seq, _, _ = _build(rng, Hkv, d, P, L, demote)
    assert all(pg.fmt == (PM.TQ3 if fmt == "tq3" else PM.FP8) for pg in seq.pages)
    qb = _q_bits(rng, Hq, d)
    tau = np.float32(1 / math.sqrt(d))
    O, lse = A.decode_seq(seq, qb, tau)
    K, V = (torch.from_numpy(x) for x in seq.dense())
    q = torch.from_numpy(C.bf16_bits_to_value(qb))
    for h in range(Hq):
        s = float(tau) * (K[:, h // 4, :] @ q[h])
        ref_o = torch.softmax(s, 0) @ V[:, h // 4, :]
        assert torch.max(torch.abs(ref_o - torch.from_numpy(O[h]))) < 1e-12
        assert abs(torch.logsumexp(s, 0).item() - lse[h]) < 1e-12


# ----------------------------------------------------------------- closed forms
def test_zero_query_gives_mean_of_values_and_log_length():
    rng = np.random.default_rng(41)
    Hkv, d, P, L = 2, 64, 16, 77
    seq, _, _ = _build(rng, Hkv, d, P, L, demote=(0, 2))
    qb = np.zeros((4, d), np.uint16)
    O, lse = A.decode_seq(seq, qb, np.float32(0.125))
    _, V = seq.dense()
    for h in range(4):
        assert np.max(np.abs(O[h] - V[:, h // 2, :].mean(axis=0))) < 1e-13
    assert np.max(np.abs(lse - math.log(L))) < 1e-13


def test_single_token_sequence():
    rng = np.random.default_rng(43)
    Hkv, d, P = 2, 64, 16
    for demote in ((), (0,)):
        seq, _, _ = _build(rng, Hkv, d, P, 1, demote)
        qb = _q_bits(rng, 4, d)
        tau = np.float32(0.1)
        O, lse = A.decode_seq(seq, qb, tau)
        K, V = seq.dense()
        q = C.bf16_bits_to_value(qb)
        for h in range(4):
            assert np.array_equal(O[h], V[0, h // 2])
            assert abs(lse[h] - float(tau) * float(K[0, h // 2] @ q[h])) < 1e-14


def test_identical_keys_give_uniform_weights():
    # Key values (c - 3.5) * 128 with a 0 or 7 in every group are exact in both
    # FP8 (sigma = 1) and TQ3 (s = 128), so every token has the same dequantised
    # key whatever its page format.
    rng = np.random.default_rng(47)
    Hkv, d, P, L = 2, 64, 8, 50
    c = rng.integers(0, 8, (1, Hkv, d))
    c[..., 0] = 7
    c[..., 32] = 0
    k1 = ((c - 3.5) * 128.0).astype(np.float32)
    k = np.repeat(k1, L, axis=0)
    v = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    seq = PM.SeqModel(Hkv, d, P)
    seq.append(k, v)
    for lp in (1, 3, 6):
        seq.demote(lp)
    qb = _q_bits(rng, 4, d)
    O, lse = A.decode_seq(seq, qb, np.float32(0.2))
    K, V = seq.dense()
    assert np.all(K == K[0])
    for h in range(4):
        assert np.max(np.abs(O[h] - V[:, h // 2].mean(axis=0))) < 1e-13


# ------------------------------------------------------------- append / demote
def test_append_in_calls_equals_one_shot_when_max_comes_first():
    rng = np.random.default_rng(51)
    Hkv, d, P, L = 2, 32, 16, 40
    k = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    k[0] *= 10
    v[0] *= 10
    k[16] *= 10
    v[16] *= 10
    k[32] *= 10
    v[32] *= 10
    a = PM.SeqModel(Hkv, d, P)
    a.append(k, v)
    b = PM.SeqModel(Hkv, d, P)
    for lo, hi in ((0, 3), (3, 17), (17, 20), (20, 40)):
        b.append(k[lo:hi], v[lo:hi])
    for lp in range(3):
        assert np.array_equal(a.record(lp), b.record(lp))


def test_rescale_on_grow_is_exact_for_representable_rows():
    # Rows whose values are E4M3 numbers times 0.5 with amax 224 (sigma 0.5),
    # then a row raising amax to 448 (sigma 1): the re-encoded old rows must be
    # the exact E4M3 codes of their values, as one-shot quantisation gives.
    rng = np.random.default_rng(53)
    Hkv, d, P = 1, 32, 8
    good = C.e4m3_decode(np.arange(0x28, 0x77, dtype=np.uint8))   # 2^-2 .. 224
    first = rng.choice(good, (3, Hkv, d)).astype(np.float32) * np.float32(0.5)
    first[0, 0, 0] = 112.0
    second = rng.choice(good, (2, Hkv, d)).astype(np.float32)
    second[0, 0, 5] = -448.0
    seq = PM.SeqModel(Hkv, d, P)
    seq.append(first, first)
    assert seq.pages[0].scale[0, 0] == np.float32(0.25)
    seq.append(second, second)
    page = seq.pages[0]
    assert page.scale[0, 0] == np.float32(1.0)
    allrows = np.concatenate([first, second])[:, 0, :]
    assert np.array_equal(C.e4m3_decode(page.codes[0, 0, :5]), allrows.astype(np.float64))
    one = PM.SeqModel(Hkv, d, P)
    one.append(np.concatenate([first, second]), np.concatenate([first, second]))
    assert np.array_equal(one.record(0), seq.record(0))


def test_zero_rows_get_unit_scale():
    seq = PM.SeqModel(1, 32, 8)
    z = np.zeros((3, 1, 32), np.float32)
    seq.append(z, z)
    assert np.all(seq.pages[0].scale == 1.0) and np.all(seq.pages[0].codes == 0)


def test_demote_of_representable_page_gives_known_codes():
    # Groups (c - 3.5) * s with s in {128, 64, 32, 16} are E4M3-exact; one group
    # per head reaches 448 so sigma = 1 and FP8 is lossless; demotion must then
    # recover exactly the codes and scales.
    rng = np.random.default_rng(57)
    Hkv, d, P, L = 2, 128, 16, 16
    codes = rng.integers(0, 8, (2, L, Hkv, d)).astype(np.uint8)
    s = rng.choice([128.0, 64.0, 32.0, 16.0], (2, L, Hkv, d // 32))
    codes.reshape(2, L, Hkv, 4, 32)[..., 0] = rng.choice([0, 7], (2, L, Hkv, 4))
    s[:, 0, :, 0] = 128.0
    x = ((codes.astype(np.float64) - 3.5).reshape(2, L, Hkv, 4, 32) * s[..., None]).reshape(2, L, Hkv, d)
    seq = PM.SeqModel(Hkv, d, P)
    seq.append(x[0].astype(np.float32), x[1].astype(np.float32))
    assert np.all(seq.pages[0].scale == 1.0)
    seq.demote(0)
    page = seq.pages[0]
    assert np.array_equal(page.tcodes, np.transpose(codes, (0, 2, 1, 3)))
    assert np.array_equal(page.tscale.astype(np.float64), np.transpose(s, (0, 2, 1, 3)))


def test_append_onto_partial_tq3_tail_is_refused_and_full_tail_is_not():
    rng = np.random.default_rng(59)
    seq, _, _ = _build(rng, 1, 32, 8, 12, demote=(1,))
    with pytest.raises(ValueError):
        seq.append(np.zeros((1, 1, 32), np.float32), np.zeros((1, 1, 32), np.float32))
    seq2, _, _ = _build(rng, 1, 32, 8, 16, demote=(1,))
    seq2.append(np.ones((1, 1, 32), np.float32), np.ones((1, 1, 32), np.float32))
    assert len(seq2.pages) == 3 and seq2.pages[2].fmt == PM.FP8


def test_kv_bytes_hand_count():
    rng = np.random.default_rng(61)
    seq, _, _ = _build(rng, 2, 64, 16, 40, demote=(0,))
    # page 0 TQ3: 16 tok * 2 heads * (K+V) * (64*3/8 + 2*2) B = 1792
    # pages 1, 2 FP8: 24 tok * 2 heads * 2 * 64 B = 6144, + 2 pages * 2 heads * 8 B
    assert PM.kv_bytes(seq) == 1792 + 6144 + 32


def test_record_sizes_and_masks():
    rng = np.random.default_rng(63)
    seq, _, _ = _build(rng, 3, 64, 16, 21, demote=(1,))
    assert seq.record(0).size == PM.fp8_record_bytes(3, 16, 64) == 2 * 3 * 16 * 64 + 48
    assert seq.record(1).size == PM.tq3_record_bytes(3, 16, 64) == 3 * 16 * 64 * 7 // 8
    assert seq.valid_mask(1).size == seq.record(1).size
    # page 1 holds 5 valid rows: K codes of head 0 span 5 * 24 bytes
    m = seq.valid_mask(1)
    assert m[:5 * 24].all() and not m[5 * 24:16 * 24].any()


# ------------------------------------------------------------ BF16 control cache
def test_bf16_control_record_layout_hand_built():
    """Record [Hkv][2][P][d] bf16 little-endian, rows past the valid count zero."""
    Hkv, P, d = 2, 16, 32
    n = 3
    k = np.zeros((n, Hkv, d), np.float32)
    v = np.zeros((n, Hkv, d), np.float32)
    k[1, 1, 5] = 1.0          # bf16 0x3F80
    v[2, 0, 31] = -2.0        # bf16 0xC000
    seq = PM.Bf16SeqModel(Hkv, d, P)
    seq.append(k, v)
    rec = seq.record(0)
    assert rec.size == PM.bf16_record_bytes(Hkv, P, d) == 4 * Hkv * P * d
    off_k = ((1 * 2 + 0) * P + 1) * d * 2 + 5 * 2       # head 1, K, token 1, dim 5
    off_v = ((0 * 2 + 1) * P + 2) * d * 2 + 31 * 2      # head 0, V, token 2, dim 31
    assert rec[off_k] == 0x80 and rec[off_k + 1] == 0x3F
    assert rec[off_v] == 0x00 and rec[off_v + 1] == 0xC0
    nz = np.flatnonzero(rec)
    assert set(nz.tolist()) == {off_k + 1, off_k, off_v + 1}
    assert seq.valid_mask(0).sum() == Hkv * 2 * n * d * 2


def test_bf16_control_dense_and_decode():
    """Values are the bf16 roundings of the rows; with bf16-representable rows
    the control decode equals plain attention on the fp32 rows."""
    rng = np.random.default_rng(8)
    Hkv, P, d, L, Hq = 2, 16, 64, 37, 6
    k = (rng.integers(-64, 64, (L, Hkv, d)) / 16.0).astype(np.float32)   # exact in bf16
    v = (rng.integers(-64, 64, (L, Hkv, d)) / 8.0).astype(np.float32)
    seq = PM.Bf16SeqModel(Hkv, d, P)
    seq.append(k[:20], v[:20])
    seq.append(k[20:], v[20:])
    K, V = seq.dense()
    assert np.array_equal(K, k.astype(np.float64)) and np.array_equal(V, v.astype(np.float64))
    assert len(seq.bits) == 3 and seq.ntok == [16, 16, 5]
    # bytes a decode reads: a hand count (37 tokens x 2 kv-heads x K and V x 64
    # dims x 2 bytes) and the valid bytes of the page records
    assert PM.bf16_kv_bytes(seq) == 18944
    assert PM.bf16_kv_bytes(seq) == sum(int(seq.valid_mask(lp).sum()) for lp in range(len(seq.bits)))
    qb = C.bf16_encode(rng.standard_normal((Hq, d)).astype(np.float32))
    O, lse = A.decode_seq(seq, qb, np.float32(0.125))
    O2, lse2 = A.attend(C.bf16_bits_to_value(qb), k.astype(np.float64), v.astype(np.float64), 0.125)
    assert np.array_equal(O, O2) and np.array_equal(lse, lse2)
    # a non-representable row is rounded to nearest even
    seq2 = PM.Bf16SeqModel(1, 32, 16)
    x = np.full((1, 1, 32), 1.0 + 2.0 ** -8 + 2.0 ** -12, np.float32)
    seq2.append(x, x)
    assert np.all(seq2.dense()[0] == 1.0 + 2.0 ** -7)


def test_materialise_hand_page_and_properties():
    """Materialised rows: FP8 elements are fp32(e4m3(c) * sigma) rounded to bf16,
    TQ3 elements (c - 3.5) * s rounded to bf16; page structure is kept."""
    Hkv, P, d = 1, 16, 32
    k = np.zeros((20, Hkv, d), np.float32)
    v = np.zeros((20, Hkv, d), np.float32)
    k[0, 0, 0] = 448.0          # amax 448: sigma 1, code 0x7E (448)
    k[0, 0, 1] = 1.0 + 2.0 ** -3   # e4m3 exact: 1.125
    v[3, 0, 2] = -3.0
    k[17, 0, 5] = 7.0           # second page: one of its rows
    seq = PM.SeqModel(Hkv, d, P)
    seq.append(k, v)
    m = PM.materialise(seq)
    assert m.ntok == [16, 4] and m.length == 20
    K, V = m.dense()
    assert K[0, 0, 0] == 448.0 and K[0, 0, 1] == 1.125 and V[3, 0, 2] == -3.0 and K[17, 0, 5] == 7.0
    assert np.count_nonzero(K) == 3 and np.count_nonzero(V) == 1
    # demote page 0 to TQ3: the group holding 448 and 1.125 has s = fp16(448/3.5) = 128,
    # so 448 -> code 7 -> 3.5*128 = 448 and 1.125 -> code 4 -> 0.5*128 = 64, zeros -> 64 too
    seq.demote(0)
    K2, _ = PM.materialise(seq).dense()
    assert K2[0, 0, 0] == 448.0 and K2[0, 0, 1] == 64.0 and K2[1, 0, 0] == 0.0
    assert np.all(K2[0, 0, 2:] == 64.0)


def test_materialise_matches_exact_dequantisation_rounded():
    """Against the exact fp64 page values: rounding them to fp32 and then to bf16
    gives the materialised bits (FP8 and TQ3 pages, outlier rows)."""
    rng = np.random.default_rng(31)
    Hkv, P, d, L = 2, 16, 64, 70
    k = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((L, Hkv, d)).astype(np.float32) * np.float32(8.0)
    seq = PM.SeqModel(Hkv, d, P)
    seq.append(k, v)
    for lp in (0, 2):
        seq.demote(lp)
    m = PM.materialise(seq)
    K, V = seq.dense()
    MK, MV = m.dense()
    ref_k = C.bf16_bits_to_value(C.bf16_encode(K.astype(np.float32)))
    ref_v = C.bf16_bits_to_value(C.bf16_encode(V.astype(np.float32)))
    assert np.array_equal(MK, ref_k) and np.array_equal(MV, ref_v)
    # TQ3 values carry at most 14 significant bits, so their fp32 rounding is exact
    tq = K[:16]
    assert np.array_equal(tq.astype(np.float32).astype(np.float64), tq)
