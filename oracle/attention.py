"""Reference decode attention over the mixed-format cache, in fp64 on the CPU.

TEST INFRASTRUCTURE.  Part of the CPU oracle; see oracle/__init__.py.

What it follows
---------------
* Minima-KV summary (brainszone.ai, pt/fr), section "Como os resultados
  parciais sao combinados": each format group's pages yield a partial attention
  state, and a globally normalised online-softmax merge combines the partial
  states; the decode works directly on the heterogeneous cache, without a dense
  single-format copy.  Merging partials is mathematically the same as one
  softmax over all tokens, so the oracle's main entry point computes that plain
  definition on the dequantised cache (the analogue of the summary's
  "materialising profile", section "Qualidade em contexto longo").
* The partial-state and merge functions below restate the merge so tests can
  check that any page partition gives the same result as one pass.

Readings where the pages are silent:
* One query token per sequence; it attends to every token the sequence holds.
* Query head h uses kv-head h // G with G = Hq / Hkv.
* Scores are tau * <q, k> with tau the fp32 softmax scale given by the caller,
  taken exactly; the query is bf16 and taken exactly.
* Outputs: O and the natural-log log-sum-exp LSE = m + ln(sum exp(s - m)).
"""
from __future__ import annotations

import math

import numpy as np

from . import codecs as C


def attend(q, K, V, tau):
    """Single-pass softmax attention for one sequence.

    q: fp64 [Hq][d]; K, V: fp64 [L][Hkv][d]; tau: float.
    Returns O fp64 [Hq][d] and LSE fp64 [Hq]."""
    Hq, d = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    O = np.empty((Hq, d))
    lse = np.empty(Hq)
    for h in range(Hq):
        kvh = h // G
        s = tau * (K[:, kvh, :] @ q[h])            # [L]
        m = np.max(s)
        w = np.exp(s - m)
        Lsum = np.sum(w)
        O[h] = (w @ V[:, kvh, :]) / Lsum
        lse[h] = m + math.log(Lsum)
    return O, lse


def decode_seq(seq, q_bits, tau32):
    """Oracle decode for one sequence of the CPU pool model.

    seq: pool_model.SeqModel; q_bits: uint16 bf16 bits [Hq][d]; tau32: np.float32."""
    q = C.bf16_bits_to_value(q_bits)
    tau = float(np.float32(tau32))
    K, V = seq.dense()
    return attend(q, K, V, tau)


# --------------------------------------------------------------------------
# Partial states and the merge
# --------------------------------------------------------------------------
def partial(q, K, V, tau):
    """Partial state over a subset of tokens for one query head and one kv-head.

    q: [d]; K, V: [n][d].  Returns (m, l, acc): m = max score (-inf if n == 0),
    l = sum exp(s - m), acc = sum exp(s - m) * v."""
    n = K.shape[0]
    if n == 0:
        return -math.inf, 0.0, np.zeros(q.shape[0])
    s = tau * (K @ q)
    m = float(np.max(s))
    w = np.exp(s - m)
    return m, float(np.sum(w)), w @ V


def merge(parts):
    """Globally normalised merge of partial states -> (O, LSE).  Empty partials
    (l == 0) contribute nothing."""
    live = [(m, l, a) for (m, l, a) in parts if l > 0.0]
    M = max(m for (m, _, _) in live)
    Lsum = sum(l * math.exp(m - M) for (m, l, _) in live)
    acc = sum(a * math.exp(m - M) for (m, _, a) in live)
    return acc / Lsum, M + math.log(Lsum)
