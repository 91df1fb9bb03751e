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


def _deq(clib, packed, absmax, qa, dqs, rows, cols, bs, dqbs, W, wdt, out, sumsq):
    f = clib.loftq_nf4_dequantize
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    f.restype = ctypes.c_int
    f.argtypes = [P, P, P, P, I64, I64, I32, I32, P, ctypes.c_int, P, P, P]
    return f(packed, absmax, qa, dqs, rows, cols, bs, dqbs, W, wdt, out, sumsq, None)


def test_dequantize_validation(clib):
    F = FAKE
    keys = ["packed", "absmax", "qa", "dqs", "rows", "cols", "bs", "dqbs", "W", "wdt", "out", "sumsq"]
    ok = (F, F, None, None, 64, 128, 64, 256, F, 1, F, F)

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[keys.index(k)] = v
        return _deq(clib, *args)
    assert call(bs=128) == 2                                  # blocksize != 64
    assert call(qa=F, dqs=F, absmax=None, dqbs=64) == 2       # dq_blocksize != 256
    assert call(rows=-2) == 1                                 # negative shape
    assert call(wdt=9) == 1                                   # W of an unknown dtype
    assert call(packed=None) == 1                             # no codes
    assert call(out=None) == 1                                # no output
    assert call(absmax=None) == 1                             # no scales at all
    assert call(qa=F) == 1                                    # qabsmax without dq_scale
    assert call(absmax=None, dqs=F) == 1                      # dq_scale without qabsmax
    assert call(packed=F + 8) == 1                            # misaligned codes
    assert call(W=F + 2) == 1                                 # misaligned weight
    assert call(out=F + 4) == 1                               # misaligned output
    assert call(absmax=None, qa=F + 1, dqs=F) == 1            # misaligned qabsmax
    assert call(sumsq=F + 3) == 1                             # misaligned fp64 sum


class _Cfg:
    """loftq_config_t through the binding's ctypes structure."""

    @staticmethod
    def make(**kw):
        from loftq_qlora_initialization_amd import binding
        return binding.default_config(**kw)


def _init(clib, W, wdt, rows, cols, cfg, packed, absmax, qa, dqs, B, A, obj, sigma, ws, wsb):
    from loftq_qlora_initialization_amd import binding
    f = clib.loftq_init
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    f.restype = ctypes.c_int
    f.argtypes = [P, ctypes.c_int, I64, I64, ctypes.POINTER(binding.LoftqConfig), P, P, P, P, P, P, P, P, P,
                  ctypes.c_size_t, P]
    return f(W, wdt, rows, cols, None if cfg is None else ctypes.byref(cfg), packed, absmax, qa, dqs, B, A, obj,
             sigma, ws, wsb, None)


def _init_ws(clib, rows, cols, cfg):
    from loftq_qlora_initialization_amd import binding
    f = clib.loftq_workspace_bytes
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(binding.LoftqConfig)]
    return f(rows, cols, None if cfg is None else ctypes.byref(cfg))


def test_init_validation(clib):
    F = FAKE
    rows, cols = 256, 512
    need = _init_ws(clib, rows, cols, _Cfg.make())
    assert need > 4 * rows * cols and need % 256 == 0
    keys = ["W", "wdt", "rows", "cols", "cfg", "packed", "absmax", "qa", "dqs", "B", "A", "obj", "sigma", "ws",
            "wsb"]

    def call(cfg_kw=None, **kw):
        args = [F, 1, rows, cols, _Cfg.make(**(cfg_kw or {})), F, F, F, F, F, F, F, F, F, need]
        for k, v in kw.items():
            args[keys.index(k)] = v
        return _init(clib, *args)
    # unsupported configurations
    assert call(dict(bits=5)) == 2 and call(dict(bits=1)) == 2
    assert call(dict(blocksize=32)) == 2
    assert call(dict(dq_blocksize=128)) == 2
    assert call(dict(rank=64, oversample=17)) == 2            # sketch width l = 81 > 80
    assert call(dict(rank=65, oversample=0)) == 2             # r > 64 on the randomized path
    assert call(dict(exact_svd=1), rows=640, cols=640, wsb=1 << 40) == 2   # exact SVD beyond 512
    # invalid arguments
    assert call(cfg=None) == 1
    assert call(dict(rank=0)) == 1
    assert call(dict(rank=250, oversample=8)) == 1            # r + p > min(rows, cols) = 256
    assert call(dict(rank=260, exact_svd=1)) == 1             # r > min(rows, cols) (exact)
    assert call(dict(oversample=-1)) == 1
    assert call(dict(power_iters=-1)) == 1 and call(dict(power_iters=65)) == 1
    assert call(dict(iterative_steps=-1)) == 1
    assert call(dict(double_quant=2)) == 1 and call(dict(warm_start=3)) == 1 and call(dict(exact_svd=2)) == 1
    assert call(dict(init_from_BA=-1)) == 1                   # resume count
    assert call(dict(init_from_BA=2, iterative_steps=0)) == 1  # resume with nothing to run
    assert call(wdt=5) == 1
    assert call(rows=0) == 1 and call(cols=-64) == 1
    for k in ("W", "packed", "absmax", "B", "A", "obj", "sigma", "ws"):
        assert call(**{k: None}) == 1, k                      # null pointer
        assert call(**{k: F + 4}) == 1, k                     # misaligned
    assert call(qa=None) == 1 and call(dqs=None) == 1         # double quant without its outputs
    assert call(wsb=need - 1) == 3                            # workspace too small
    # the workspace query rejects what the call rejects
    assert _init_ws(clib, rows, cols, _Cfg.make(bits=5)) == 0
    assert _init_ws(clib, rows, cols, None) == 0
    assert _init_ws(clib, rows, cols, _Cfg.make(rank=250)) == 0


def _svd(clib, E, rows, cols, r, p, q, exact, omega, seed, t, B, A, sigma, ws, wsb):
    f = clib.loftq_lowrank_svd
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    f.restype = ctypes.c_int
    f.argtypes = [P, I64, I64, I32, I32, I32, I32, P, ctypes.c_uint64, I32, P, P, P, P, ctypes.c_size_t, P]
    return f(E, rows, cols, r, p, q, exact, omega, seed, t, B, A, sigma, ws, wsb, None)


def test_lowrank_svd_validation(clib):
    F = FAKE
    ws_q = clib.loftq_lowrank_svd_workspace_bytes
    ws_q.restype = ctypes.c_size_t
    ws_q.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    rows, cols = 300, 200
    need = ws_q(rows, cols, 16, 8, 0)
    assert need > 0 and need % 256 == 0
    assert ws_q(rows, cols, 64, 17, 0) == 0 and ws_q(rows, cols, 0, 8, 0) == 0 and ws_q(600, 600, 4, 0, 1) == 0
    keys = ["E", "rows", "cols", "r", "p", "q", "exact", "omega", "seed", "t", "B", "A", "sigma", "ws", "wsb"]
    ok = (F, rows, cols, 16, 8, 2, 0, None, 42, 1, F, F, F, F, need)

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[keys.index(k)] = v
        return _svd(clib, *args)
    assert call(r=64, p=17) == 2                              # l > 80
    assert call(r=65, p=0) == 2                               # r > 64
    assert call(exact=1, rows=600, cols=600, wsb=1 << 40) == 2   # exact beyond 512
    assert call(r=0) == 1 and call(p=-1) == 1
    assert call(r=190, p=20) == 1                             # l > min(rows, cols)
    assert call(r=201, exact=1) == 1                          # r > min(rows, cols), exact
    assert call(exact=2) == 1
    assert call(q=-1) == 1 and call(q=65) == 1
    assert call(t=0) == 1                                     # alternation numbers start at 1
    assert call(rows=-1) == 1
    for k in ("E", "B", "A", "sigma", "ws"):
        assert call(**{k: None}) == 1, k
        assert call(**{k: F + 8}) == 1, k
    assert call(omega=F + 4) == 1                             # misaligned caller sketch
    assert call(wsb=need - 1) == 3


def test_init_batch_validation(clib):
    """loftq_init_batch checks every matrix and every stream's workspace before enqueueing."""
    from loftq_qlora_initialization_amd import binding
    F = FAKE
    P = ctypes.c_void_p
    cfg = binding.default_config()

    def mat(rows=256, cols=512, **kw):
        m = binding.LoftqMatrix(F, rows, cols, F, F, F, F, F, F, F, F)
        for k, v in kw.items():
            setattr(m, k, v)
        return m
    good = [mat(), mat(512, 256), mat(256, 256)]
    arr = (binding.LoftqMatrix * 3)(*good)
    need = binding._c_batch_ws(arr, 3, ctypes.byref(cfg))
    assert need == max(binding.workspace_bytes(m.rows, m.cols, cfg) for m in good)
    ws = (P * 2)(F, F + 0x100000)
    streams = (P * 2)(None, None)

    def call(mats, n=None, cfg_=cfg, nstreams=2, ws_=ws, wsb=need, wdt=1):
        a = (binding.LoftqMatrix * len(mats))(*mats)
        return binding._c_batch(a, len(mats) if n is None else n, wdt, ctypes.byref(cfg_) if cfg_ else None,
                                nstreams, streams, ws_, wsb)
    assert call(good, wsb=need - 1) == 3                      # one matrix's workspace too small
    assert call(good + [mat(W=None)]) == 1                    # a null weight in the batch
    assert call(good + [mat(sigma=F + 4)]) == 1               # misaligned output
    assert call(good + [mat(qabsmax=None)]) == 1              # double quant without its outputs
    assert call(good + [mat(rows=16, cols=16)]) == 1          # r + p above min(rows, cols)
    assert call(good, cfg_=binding.default_config(bits=7)) == 2
    assert call(good, cfg_=None) == 1
    assert call(good, nstreams=0) == 1 and call(good, nstreams=17) == 1
    assert call(good, ws_=(P * 2)(F, F)) == 1                 # two streams sharing one workspace
    assert call(good, wdt=3) == 1
    assert call(good, n=-1) == 1
    assert call(good, n=0) == 0                               # empty batch: nothing to do
    assert binding._c_batch_ws(arr, 0, ctypes.byref(cfg)) == 0


def test_qlora_forward_noalloc_validation(clib):
    """The allocation-free forward: the scratch limit and the forward's own checks, before any HIP call."""
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    f = clib.loftq_qlora_forward_noalloc
    f.restype = ctypes.c_int
    f.argtypes = [P, I64, I64, I64, P, P, P, P, I32, P, P, I32, ctypes.c_float, P, P]
    clib.loftq_qlora_forward_noalloc_max_bytes.restype = ctypes.c_size_t
    cap = clib.loftq_qlora_forward_noalloc_max_bytes()
    assert cap == 8 << 20
    F = FAKE
    keys = ["X", "n", "rows", "cols", "packed", "absmax", "qa", "dqs", "bits", "B", "A", "r", "alpha", "Y"]
    ok = (F, 32, 64, 128, F, F, None, None, 4, F, F, 8, 1.0, F)

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[keys.index(k)] = v
        return f(*args, None)
    assert call(n=cap // (8 * 4 * 16) + 16, r=16) == 3      # partial products beyond the scratch
    assert call(n=4096, r=65) == 2                          # rank above 64
    assert call(bits=5) == 2
    assert call(cols=96) == 2
    assert call(A=None) == 1 and call(X=None) == 1 and call(Y=F + 4) == 1
    assert call(alpha=float("inf")) == 1 and call(n=-1) == 1
    assert call(n=0) == 0 and call(rows=0) == 0              # empty: nothing to write
