"""CPU model of the paged, mixed-format KV cache: append, demote and page records.

TEST INFRASTRUCTURE.  Part of the CPU oracle; see oracle/__init__.py for who may
use it.  It shares no code with the HIP library.

What it follows
---------------
* Minima-KV summary (brainszone.ai, pt/fr), section "O que os autores propoem":
  the KV cache is a hierarchy of pages and each page is stored in its own
  numeric format.
* Same summary, section "Ancoras em FP8, arquivo em TQ3": recent and anchor
  pages stay FP8; older non-anchor pages are converted to packed TQ3; every
  page of a live request stays addressable (nothing evicted, nothing replaced
  by a proxy).  Conversion therefore re-encodes a page in place of the old one.

Readings where the pages are silent (each is listed in the design notes):
* FP8 pages carry one fp32 scale per (page, kv-head, K-or-V):
  sigma = fp32(amax / 448), or 1.0 when amax == 0; codes = E4M3(fp32(x / sigma)).
* A tail page that grows keeps its running amax.  If new rows raise it, sigma is
  recomputed and the page's existing rows are re-encoded from their dequantised
  fp32 values: E4M3(fp32(fp32(e4m3(c) * sigma_old) / sigma_new)).  A page filled
  by one call therefore equals one-shot quantisation.
* Demotion dequantises each FP8 element to fp32 (x = fp32(e4m3(c) * sigma)) and
  TQ3-encodes every 32-element group of every valid row.

Page records (the byte layout the library stores; the gather check compares
records in logical order).  With Hkv kv-heads, head dim d and P tokens per page:
* FP8 record: codes [Hkv][2 (K, V)][P][d] u8, then scales [Hkv][2] f32, then
  running amax [Hkv][2] f32.  Size 2*Hkv*P*d + 16*Hkv bytes.
* TQ3 record: Hkv blocks of P*d*7/8 bytes; block h holds K codes [P][3d/8]
  (token rows as 3-bit streams), V codes [P][3d/8], K scales [P][d/32] f16 and
  V scales [P][d/32] f16.
Rows at or beyond the page's valid-token count are unspecified in both formats.

The dense BF16 control cache (Bf16SeqModel) is the single-format baseline of the
same summary, section "O que as medicoes mostram", subsection "Memoria e
compressao" (the compression is stated relative to BF16 and to FP8):
every row stored as bf16, record [Hkv][2 (K, V)][P][d] bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import codecs as C

FP8 = 0
TQ3 = 1


def fp8_record_bytes(Hkv: int, P: int, d: int) -> int:
    return 2 * Hkv * P * d + 16 * Hkv


def tq3_record_bytes(Hkv: int, P: int, d: int) -> int:
    return Hkv * P * d * 7 // 8


@dataclass
class Page:
    fmt: int
    ntok: int
    # FP8 fields
    codes: np.ndarray | None = None      # [2][Hkv][P][d] u8 (K, V)
    scale: np.ndarray | None = None      # [2][Hkv] f32
    amax: np.ndarray | None = None       # [2][Hkv] f32
    # TQ3 fields
    tcodes: np.ndarray | None = None     # [2][Hkv][P][d] u8 in 0..7
    tscale: np.ndarray | None = None     # [2][Hkv][P][d/32] f16


@dataclass
class SeqModel:
    Hkv: int
    d: int
    P: int
    pages: list = field(default_factory=list)
    length: int = 0

    # ------------------------------------------------------------------ append
    def append(self, k, v) -> None:
        """Append fp32 rows k, v of shape [n][Hkv][d] as FP8 (rescale-on-grow)."""
        k = np.asarray(k, dtype=np.float32)
        v = np.asarray(v, dtype=np.float32)
        n = k.shape[0]
        assert k.shape == (n, self.Hkv, self.d) and v.shape == k.shape
        if n == 0:
            return
        if self.length % self.P and self.pages[-1].fmt != FP8:
            raise ValueError("tail page is TQ3 and partially filled")
        kv = np.stack([k, v])                    # [2][n][Hkv][d]
        pos = 0
        slot = self.length % self.P
        if slot:                                 # grow the partially filled tail page
            page = self.pages[-1]
            take = min(self.P - slot, n)
            self._fill(page, slot, kv[:, :take])
            page.ntok = slot + take
            self.length += take
            pos = take
        if pos < n:                              # fresh pages: one-shot quantisation each
            self._fill_fresh(kv[:, pos:])
            self.length += n - pos

    def _fill_fresh(self, rows) -> None:
        """Quantise rows [2][m][Hkv][d] into new pages, page by page (vectorised)."""
        P, Hkv, d = self.P, self.Hkv, self.d
        m = rows.shape[1]
        npg = -(-m // P)
        pad = np.zeros((2, npg * P, Hkv, d), np.float32)
        pad[:, :m] = rows
        x = pad.reshape(2, npg, P, Hkv, d).transpose(1, 0, 3, 2, 4)   # [npg][2][Hkv][P][d]
        valid = (np.arange(npg * P) < m).reshape(npg, 1, 1, P, 1)
        amax = np.max(np.abs(x), axis=(3, 4)).astype(np.float32)     # padding rows are 0
        sigma = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
        codes = C.e4m3_encode((x / sigma[..., None, None]).astype(np.float32))
        codes = np.where(valid, codes, np.uint8(0)).astype(np.uint8)
        for i in range(npg):
            ntok = min(P, m - i * P)
            self.pages.append(Page(FP8, ntok, codes=codes[i], scale=sigma[i].copy(),
                                   amax=amax[i].copy()))

    def _fill(self, page: Page, slot: int, rows) -> None:
        new_amax = np.max(np.abs(rows), axis=(1, 3)).astype(np.float32)  # [2][Hkv]
        grown = new_amax > page.amax
        amax = np.where(grown, new_amax, page.amax).astype(np.float32)
        sigma = np.where(amax == 0, np.float32(1.0),
                         amax / np.float32(448.0)).astype(np.float32)
        if slot > 0:
            for kvi in range(2):
                for h in range(self.Hkv):
                    if not grown[kvi, h]:
                        continue
                    old = page.codes[kvi, h, :slot]
                    x_old = (C.e4m3_decode(old).astype(np.float32)
                             * page.scale[kvi, h]).astype(np.float32)
                    page.codes[kvi, h, :slot] = C.e4m3_encode(
                        (x_old / sigma[kvi, h]).astype(np.float32))
        for kvi in range(2):
            for h in range(self.Hkv):
                x = rows[kvi, :, h, :]                        # [take][d]
                page.codes[kvi, h, slot:slot + x.shape[0]] = C.e4m3_encode(
                    (x / sigma[kvi, h]).astype(np.float32))
        page.amax = amax
        page.scale = sigma

    # ------------------------------------------------------------------ demote
    def demote(self, lp: int) -> None:
        """Convert logical page lp from FP8 to TQ3 (valid rows only)."""
        page = self.pages[lp]
        if page.fmt != FP8:
            raise ValueError("page is not FP8")
        n = page.ntok
        G = self.d // C.TQ3_GROUP
        tcodes = np.zeros((2, self.Hkv, self.P, self.d), np.uint8)
        tscale = np.zeros((2, self.Hkv, self.P, G), np.float16)
        x = (C.e4m3_decode(page.codes[:, :, :n, :]).astype(np.float32)
             * page.scale[:, :, None, None]).astype(np.float32)   # [2][Hkv][n][d]
        codes, s = C.tq3_encode_groups(x.reshape(2, self.Hkv, n, G, C.TQ3_GROUP))
        tcodes[:, :, :n, :] = codes.reshape(2, self.Hkv, n, self.d)
        tscale[:, :, :n, :] = s
        self.pages[lp] = Page(TQ3, n, tcodes=tcodes, tscale=tscale)

    # ------------------------------------------------------------- dequantise
    def page_values(self, lp: int):
        """Exact fp64 K, V of the valid rows of page lp: each [ntok][Hkv][d]."""
        page = self.pages[lp]
        n = page.ntok
        if page.fmt == FP8:
            val = C.e4m3_decode(page.codes[:, :, :n, :]) \
                * page.scale.astype(np.float64)[:, :, None, None]
        else:
            G = self.d // C.TQ3_GROUP
            c = page.tcodes[:, :, :n, :].reshape(2, self.Hkv, n, G, C.TQ3_GROUP)
            val = C.tq3_decode(c, page.tscale[:, :, :n, :]).reshape(2, self.Hkv, n, self.d)
        val = np.transpose(val, (0, 2, 1, 3))   # [2][n][Hkv][d]
        return val[0], val[1]

    def dense(self, heads=None):
        """Materialise the whole sequence: K, V fp64 [L][Hkv][d] (or the listed kv-heads)."""
        ks, vs = [], []
        for lp in range(len(self.pages)):
            k, v = self.page_values(lp)
            if heads is not None:
                k, v = k[:, heads], v[:, heads]
            ks.append(k)
            vs.append(v)
        return np.concatenate(ks), np.concatenate(vs)

    # ----------------------------------------------------------------- records
    def record(self, lp: int) -> np.ndarray:
        """Byte record of page lp in the library's layout (invalid rows zero)."""
        page = self.pages[lp]
        Hkv, P, d = self.Hkv, self.P, self.d
        if page.fmt == FP8:
            codes = page.codes.copy()
            codes[:, :, page.ntok:, :] = 0
            body = np.transpose(codes, (1, 0, 2, 3)).reshape(-1)    # [Hkv][2][P][d]
            scales = np.ascontiguousarray(page.scale.T).astype('<f4').view(np.uint8).reshape(-1)
            amax = np.ascontiguousarray(page.amax.T).astype('<f4').view(np.uint8).reshape(-1)
            out = np.concatenate([body, scales, amax])
            assert out.size == fp8_record_bytes(Hkv, P, d)
            return out
        parts = []
        for h in range(Hkv):
            for kvi in range(2):
                rows = page.tcodes[kvi, h].copy()
                rows[page.ntok:] = 0
                parts.append(C.tq3_pack_row(rows).reshape(-1))
            for kvi in range(2):
                sc = page.tscale[kvi, h].copy()
                sc[page.ntok:] = 0
                parts.append(sc.astype('<f2').view(np.uint8).reshape(-1))
        out = np.concatenate(parts)
        assert out.size == tq3_record_bytes(Hkv, P, d)
        return out

    def valid_mask(self, lp: int) -> np.ndarray:
        """Boolean mask over the record bytes of page lp that are specified."""
        page = self.pages[lp]
        Hkv, P, d = self.Hkv, self.P, self.d
        n = page.ntok
        if page.fmt == FP8:
            m = np.zeros((Hkv, 2, P, d), bool)
            m[:, :, :n, :] = True
            return np.concatenate([m.reshape(-1), np.ones(16 * Hkv, bool)])
        G = d // C.TQ3_GROUP
        parts = []
        for _h in range(Hkv):
            for _kvi in range(2):
                r = np.zeros((P, 3 * d // 8), bool)
                r[:n] = True
                parts.append(r.reshape(-1))
            for _kvi in range(2):
                r = np.zeros((P, G * 2), bool)
                r[:n] = True
                parts.append(r.reshape(-1))
        return np.concatenate(parts)


def bf16_record_bytes(Hkv: int, P: int, d: int) -> int:
    return 4 * Hkv * P * d


@dataclass
class Bf16SeqModel:
    """A sequence of the dense BF16 control cache: the single-format baseline the
    summaries compare the mixed cache against (its compression is given relative
    to BF16 in section "O que as medicoes mostram", subsection "Memoria e
    compressao").  Every row is stored as bf16
    (round to nearest even); pages are never converted.
    Record of a page: [Hkv][2 (K, V)][P][d] bf16, little-endian."""
    Hkv: int
    d: int
    P: int
    bits: list = field(default_factory=list)     # per page: [2][Hkv][P][d] u16
    ntok: list = field(default_factory=list)
    length: int = 0

    def append(self, k, v) -> None:
        k = np.asarray(k, dtype=np.float32)
        v = np.asarray(v, dtype=np.float32)
        n = k.shape[0]
        assert k.shape == (n, self.Hkv, self.d) and v.shape == k.shape
        rows = np.stack([C.bf16_encode(k), C.bf16_encode(v)])   # [2][n][Hkv][d]
        for t in range(n):
            slot = self.length % self.P
            if slot == 0:
                self.bits.append(np.zeros((2, self.Hkv, self.P, self.d), np.uint16))
                self.ntok.append(0)
            self.bits[-1][:, :, slot, :] = rows[:, t]
            self.ntok[-1] += 1
            self.length += 1

    def dense(self, heads=None):
        """K, V fp64 [L][Hkv][d] (or the listed kv-heads)."""
        ks, vs = [], []
        for b, n in zip(self.bits, self.ntok):
            val = C.bf16_bits_to_value(b[:, :, :n, :])           # [2][Hkv][n][d]
            val = np.transpose(val, (0, 2, 1, 3))
            if heads is not None:
                val = val[:, :, heads]
            ks.append(val[0])
            vs.append(val[1])
        return np.concatenate(ks), np.concatenate(vs)

    def record(self, lp: int) -> np.ndarray:
        """Byte record of page lp (rows past the valid count zero)."""
        b = self.bits[lp].copy()
        b[:, :, self.ntok[lp]:, :] = 0
        out = np.ascontiguousarray(np.transpose(b, (1, 0, 2, 3))).astype('<u2').view(np.uint8).reshape(-1)
        assert out.size == bf16_record_bytes(self.Hkv, self.P, self.d)
        return out

    def valid_mask(self, lp: int) -> np.ndarray:
        m = np.zeros((self.Hkv, 2, self.P, self.d, 2), bool)
        m[:, :, :self.ntok[lp]] = True
        return m.reshape(-1)


def materialise(seq: SeqModel) -> Bf16SeqModel:
    """The materialising profile of the summary (section "Qualidade em contexto
    longo": the hybrid pages expanded into dense tensors): every valid row of
    every page of a mixed-format sequence, dequantised and stored in a dense
    BF16 control cache with the same page size.  Each element is first the
    fp32 value the decode kernels work with -- fp32(e4m3(c) * sigma) for FP8
    (one rounded fp32 product), (c - 3.5) * s for TQ3 (exact) -- then rounded
    to bf16 (nearest even)."""
    out = Bf16SeqModel(seq.Hkv, seq.d, seq.P)
    for page in seq.pages:
        n = page.ntok
        if page.fmt == FP8:
            x = (C.e4m3_decode(page.codes[:, :, :n, :]).astype(np.float32)
                 * page.scale.astype(np.float32)[:, :, None, None]).astype(np.float32)
        else:
            G = seq.d // C.TQ3_GROUP
            c = page.tcodes[:, :, :n, :].reshape(2, seq.Hkv, n, G, C.TQ3_GROUP)
            x = C.tq3_decode(c, page.tscale[:, :, :n, :]).reshape(2, seq.Hkv, n, seq.d)
            x = x.astype(np.float32)                    # exact: 3-bit level times an fp16 scale
        bits = np.zeros((2, seq.Hkv, seq.P, seq.d), np.uint16)
        bits[:, :, :n, :] = C.bf16_encode(x)
        out.bits.append(bits)
        out.ntok.append(n)
        out.length += n
    return out


def bf16_kv_bytes(seq: Bf16SeqModel) -> int:
    """Bytes a decode step reads for a control sequence: K and V bf16 rows."""
    return seq.length * 4 * seq.Hkv * seq.d


def kv_bytes(seq: SeqModel) -> int:
    """Algorithmic KV bytes a decode step reads for this sequence: codes and
    scales of the valid rows, plus the K and V fp32 scales of each FP8 page-head."""
    total = 0
    for page in seq.pages:
        if page.fmt == FP8:
            total += page.ntok * 2 * seq.Hkv * seq.d + 8 * seq.Hkv
        else:
            total += page.ntok * seq.Hkv * seq.d * 7 // 8     # 3 bits + d/32 fp16 scales, K and V
    return total
