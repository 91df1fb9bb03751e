"""The C-ABI library loads, exports every symbol include/loftq.h declares, and
rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "loftq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(loftq_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def clib():
    from loftq_qlora_initialization_amd import binding
    return ctypes.CDLL(binding.LIB_PATH)


def test_header_symbols_exported(clib):
    names = _header_functions()
    assert "loftq_init" in names and "loftq_nf4_quantize" in names
    missing = [n for n in names if not hasattr(clib, n)]
    assert not missing, missing


def test_codebook_matches_oracle_bit_for_bit():
    import loftq_qlora_initialization_amd as lq
    lib_cb = np.array(lq.nf4_codebook(), dtype=np.float32)
    assert np.array_equal(lib_cb.view(np.uint32), oracle.nf4_codebook().view(np.uint32))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lower_bit_codebooks_match_oracle_bit_for_bit(bits):
    import loftq_qlora_initialization_amd as lq
    lib_cb = np.array(lq.nf_codebook(bits), dtype=np.float32)
    assert np.array_equal(lib_cb.view(np.uint32), oracle.nf_codebook(bits).view(np.uint32))


def test_status_strings(clib):
    clib.loftq_status_string.restype = ctypes.c_char_p
    assert clib.loftq_status_string(0) == b"ok"
    assert clib.loftq_status_string(3) == b"workspace too small"


def _q(clib, W, wdt, rows, cols, B, A, r, bs, packed, absmax):
    f = clib.loftq_nf4_quantize
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return f(W, wdt, rows, cols, B, A, r, bs, packed, absmax, None)


FAKE = 0x10000  # aligned, never dereferenced: validation fails first


def test_quantize_validation(clib):
    assert _q(clib, FAKE, 1, 64, 64, None, None, 0, 32, FAKE, FAKE) == 2       # blocksize != 64
    assert _q(clib, None, 1, 64, 64, None, None, 0, 64, FAKE, FAKE) == 1       # null W
    assert _q(clib, FAKE + 2, 1, 64, 64, None, None, 0, 64, FAKE, FAKE) == 1   # misaligned
    assert _q(clib, FAKE, 1, 64, 64, FAKE, None, 4, 64, FAKE, FAKE) == 1       # B without A
    assert _q(clib, FAKE, 1, 64, 64, FAKE, FAKE, 0, 64, FAKE, FAKE) == 1       # r = 0 with adapter
    assert _q(clib, FAKE, 7, 64, 64, None, None, 0, 64, FAKE, FAKE) == 1       # bad dtype
    assert _q(clib, FAKE, 1, -1, 64, None, None, 0, 64, FAKE, FAKE) == 1       # negative rows
    assert _q(clib, None, 1, 0, 64, None, None, 0, 64, None, None) == 0        # empty: nothing to do


def test_double_quant_validation(clib):
    f = clib.loftq_double_quant
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert f(FAKE, 10, 128, FAKE, FAKE, None) == 2
    assert f(None, 10, 256, FAKE, FAKE, None) == 1
    assert f(FAKE, -1, 256, FAKE, FAKE, None) == 1
    assert f(None, 0, 256, None, None, None) == 0


def _merge(clib, name, packed, absmax, qa, dqs, rows, cols, bs, dqbs, B, A, r, alpha, po, ao, qo, so):
    f = getattr(clib, name)
    f.restype = ctypes.c_int
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    f.argtypes = [P, P, P, P, I64, I64, I32, I32, P, P, I32, ctypes.c_float, P, P, P, P, P]
    return f(packed, absmax, qa, dqs, rows, cols, bs, dqbs, B, A, r, alpha, po, ao, qo, so, None)


@pytest.mark.parametrize("name", ["loftq_nf4_merge", "loftq_nf4_unmerge"])
def test_merge_validation(clib, name):
    F = FAKE
    ok = (F, F, None, None, 64, 128, 64, 256, F, F, 8, 1.0, F, F, None, None)
    def call(**kw):
        args = list(ok)
        keys = ["packed", "absmax", "qa", "dqs", "rows", "cols", "bs", "dqbs", "B", "A", "r", "alpha", "po", "ao", "qo", "so"]
        for k, v in kw.items():
            args[keys.index(k)] = v
        return _merge(clib, name, *args)
    assert call(bs=32) == 2                                   # blocksize != 64
    assert call(cols=96) == 2                                 # cols % 64 != 0
    assert call(r=65) == 2                                    # r > 64
    assert call(B=None) == 1                                  # B without A
    assert call(absmax=None) == 1                             # no input scales
    assert call(qa=F) == 1                                    # qabsmax without dq_scale
    assert call(qo=F) == 1                                    # qabsmax_out without dq_scale_out
    assert call(qa=F, dqs=F, dqbs=128) == 2                   # dq_blocksize != 256
    assert call(po=None) == 1                                 # no output codes
    assert call(ao=F + 4) == 1                                # misaligned output absmax
    assert call(alpha=float("inf")) == 1                      # non-finite scale
    assert call(rows=0) == 0                                  # empty: nothing to do


def test_qlora_forward_validation(clib):
    f = clib.loftq_qlora_forward
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    f.restype = ctypes.c_int
    f.argtypes = [P, I64, I64, I64, P, P, P, P, I32, P, P, I32, ctypes.c_float, P, P, ctypes.c_size_t, P]
    clib.loftq_qlora_forward_workspace_bytes.restype = ctypes.c_size_t
    clib.loftq_qlora_forward_workspace_bytes.argtypes = [I64, I32]
    F = FAKE
    ws_need = clib.loftq_qlora_forward_workspace_bytes(32, 8)
    assert ws_need >= 32 * 8 * 4 and ws_need % 256 == 0
    keys = ["X", "n", "rows", "cols", "packed", "absmax", "qa", "dqs", "bits", "B", "A", "r", "alpha", "Y", "ws",
            "wsb"]
    ok = (F, 32, 64, 128, F, F, None, None, 4, F, F, 8, 1.0, F, F, ws_need)

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[keys.index(k)] = v
        return f(*args, None)
    assert call(bits=5) == 2                                  # no such codebook
    assert call(cols=96) == 2                                 # rows of the weight split a 64-block
    assert call(r=65) == 2                                    # rank above 64
    assert call(n=1 << 26, r=24) == 2                         # LoRA down beyond 2^32 work-items
    assert call(n=(1 << 31) - 16) == 2                        # even with four token tiles per workgroup
    assert call(n=16, rows=1 << 26) == 2                      # few-token kernel beyond 2^32 work-items
    assert call(n=4096, rows=1 << 30, B=None, A=None) == 2    # tiled kernel beyond 2^32 work-items
    assert call(A=None) == 1                                  # B without A
    assert call(absmax=None) == 1                             # no scales
    assert call(qa=F) == 1                                    # qabsmax without dq_scale
    assert call(X=None) == 1
    assert call(Y=F + 4) == 1                                 # misaligned output
    assert call(alpha=float("nan")) == 1
    assert call(n=-1) == 1
    assert call(wsb=ws_need - 1) == 3                         # workspace too small
    assert call(ws=None) == 1                                 # adapter without workspace
    assert call(n=0) == 0 and call(rows=0) == 0               # empty: nothing to write
