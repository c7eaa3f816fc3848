"""Oracle-side helpers for the parity tests: the CPU model of a workload's cache
built from the same seeded inputs (same append splits, same demote list)."""
import numpy as np

from oracle import attention as A
from oracle import pool_model as PM


def seq_model(wl, b, splits=None, kv=None):
    k, v = wl.kv(b) if kv is None else kv
    seq = PM.SeqModel(wl.Hkv, wl.d, wl.P)
    if splits is None:
        seq.append(k, v)
    else:
        pos = 0
        for n in splits:
            seq.append(k[pos:pos + n], v[pos:pos + n])
            pos += n
    for lp in wl.demote_pages(b):
        seq.demote(int(lp))
    return seq


def bf16_model(wl, b, splits=None, kv=None):
    """The dense BF16 control cache of sequence b (same rows, never converted)."""
    k, v = wl.kv(b) if kv is None else kv
    seq = PM.Bf16SeqModel(wl.Hkv, wl.d, wl.P)
    pos = 0
    for n in (splits if splits is not None else [k.shape[0]]):
        seq.append(k[pos:pos + n], v[pos:pos + n])
        pos += n
    return seq


def decode_all(wl, models):
    O = np.zeros((wl.B, wl.Hq, wl.d))
    lse = np.zeros((wl.B, wl.Hq))
    for b in range(wl.B):
        O[b], lse[b] = A.decode_seq(models[b], wl.q_bits[b], wl.tau)
    return O, lse


def _decode_one(spec, b):
    """Oracle output of sequence b of the named workload (run in a worker)."""
    from decode_attention_mixed_amd import workloads as W
    wl = getattr(W, spec[0])(**spec[1])
    return b, A.decode_seq(seq_model(wl, b), wl.q_bits[b], wl.tau)


def decode_parallel(spec, indices, workers=16):
    """{b: (O, lse)} for the listed sequences of workload spec = (factory name,
    kwargs), each built and decoded by the oracle in a separate process (fresh
    interpreters: the workers import no GPU code)."""
    import multiprocessing as mp
    import os
    from concurrent.futures import ProcessPoolExecutor
    indices = list(indices)
    n = max(1, min(workers, len(indices), os.cpu_count() or 1))
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn")) as ex:
        return dict(ex.map(_decode_one, [spec] * len(indices), indices))
