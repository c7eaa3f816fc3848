"""The C-ABI library loads on the CPU and exports every function include/mkv.h
declares (no compute calls: there is no GPU here)."""
import ctypes
import os
import re
import subprocess

import pytest

import decode_attention_mixed_amd as mkv


def _declared(repo_root):
    text = open(os.path.join(repo_root, "include", "mkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mkv_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary(repo_root):
    names = _declared(repo_root)
    for core in ("mkv_pool_create", "mkv_append", "mkv_demote", "mkv_decode"):
        assert core in names
    assert names == sorted(mkv.EXPORTED)


def test_library_exports_every_declared_symbol(repo_root):
    if not os.path.exists(mkv.LIB_PATH):
        pytest.fail("libmkv.so is not built; run python -m decode_attention_mixed_amd.build")
    out = subprocess.run(["nm", "-D", "--defined-only", mkv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(mkv_[a-z_0-9]+)$", out, flags=re.M))
    missing = [n for n in _declared(repo_root) if n not in exported]
    assert not missing, missing


def test_library_loads_and_answers_host_only_queries():
    lib = mkv._load()
    assert isinstance(lib, ctypes.CDLL)
    assert mkv.status_string(mkv.ESTATE).startswith("operation")
    desc = mkv.make_desc(num_kv_heads=8, head_dim=128, page_size=16, max_seqs=1,
                         max_pages_per_seq=8192, max_batch=1, max_q_heads=48,
                         fp8_pages=8192, tq3_pages=8192)
    assert mkv.record_bytes(desc, mkv.FMT_FP8) == 2 * 8 * 16 * 128 + 16 * 8
    assert mkv.record_bytes(desc, mkv.FMT_TQ3) == 8 * 16 * 128 * 7 // 8
    assert mkv.pool_bytes(desc) > 8192 * (32896 + 14336)
    bad = mkv.make_desc(num_kv_heads=8, head_dim=100, page_size=16, max_seqs=1,
                        max_pages_per_seq=8, max_batch=1, max_q_heads=8, fp8_pages=8, tq3_pages=8)
    assert mkv.pool_bytes(bad) == 0


def test_binding_rejects_tensors_of_the_wrong_geometry():
    # shape checks run before any library call or device-pointer check, so a
    # handle that is only registered (never passed to the library) serves
    import torch
    h = ctypes.c_void_p(0x1000)
    mkv._POOL_GEOM[h.value] = (8, 128)
    try:
        bad_q = [torch.zeros(2, 48, 64), torch.zeros(3, 48, 128), torch.zeros(2, 128)]
        for q in bad_q:
            with pytest.raises(ValueError):
                mkv.decode(h, [0, 1], q, 0.1, None, None)
            with pytest.raises(ValueError):
                mkv.decode_static(h, [0, 1], q, 0.1, None, None)
        for k in [torch.zeros(5, 4, 128), torch.zeros(5, 8, 64), torch.zeros(5, 1024)]:
            with pytest.raises(ValueError):
                mkv.append(h, 0, k, k)
        for k in [torch.zeros(2, 8, 64), torch.zeros(3, 8, 128), torch.zeros(2, 4, 128)]:
            with pytest.raises(ValueError):
                mkv.append_step(h, [0, 1], k, k)
        # right shapes pass the shape check and stop at the device-pointer check
        with pytest.raises(TypeError):
            mkv.decode(h, [0, 1], torch.zeros(2, 48, 128, dtype=torch.bfloat16), 0.1, None, None)
        with pytest.raises(TypeError):
            mkv.append(h, 0, torch.zeros(5, 8, 128), torch.zeros(5, 8, 128))
    finally:
        del mkv._POOL_GEOM[h.value]
    with pytest.raises(ValueError):
        mkv.decode(h, [0], torch.zeros(1, 8, 128), 0.1, None, None)
