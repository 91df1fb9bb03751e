"""ctypes binding for libloftq: LoftQ initialisation on AMD Instinct MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libloftq.so`` (built in-tree by ``_build.build()``); torch is used
for device memory and the current stream.  Importing this package without the
built library raises ImportError: there is no CPU fallback.

The functions carry the C entry points' names (see include/loftq.h):
    loftq_nf4_quantize, loftq_double_quant, loftq_nf4_dequantize,
    loftq_nf4_merge, loftq_nf4_unmerge, loftq_lowrank_svd, loftq_init,
    loftq_qlora_forward
and return freshly allocated torch tensors on the input's device (or fill the
caller's ``out`` / ``buffers`` where those are given).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libloftq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libloftq.so is not built ({LIB_PATH}); run __graft_entry__.build() first")

_lib = ctypes.CDLL(LIB_PATH)

LOFTQ_F32, LOFTQ_BF16 = 0, 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration", 3: "workspace too small",
          4: "HIP runtime error"}

EXPORTS = ["loftq_init_batch", "loftq_batch_workspace_bytes", "loftq_nf4_quantize", "loftq_double_quant", "loftq_nf4_dequantize", "loftq_nf4_merge",
           "loftq_nf4_unmerge", "loftq_lowrank_svd",
           "loftq_lowrank_svd_workspace_bytes", "loftq_init", "loftq_workspace_bytes", "loftq_default_config",
           "loftq_status_string", "loftq_nf4_codebook", "loftq_nf_codebook", "loftq_qlora_forward",
           "loftq_qlora_forward_workspace_bytes", "loftq_qlora_forward_noalloc", "loftq_qlora_forward_noalloc_max_bytes",
           "loftq_profile_enable", "loftq_profile_collect", "loftq_profile_calibrate"]


class LoftqConfig(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("iterative_steps", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("blocksize", ctypes.c_int32), ("double_quant", ctypes.c_int32), ("dq_blocksize", ctypes.c_int32),
                ("oversample", ctypes.c_int32), ("power_iters", ctypes.c_int32), ("exact_svd", ctypes.c_int32),
                ("warm_start", ctypes.c_int32), ("seed", ctypes.c_uint64), ("init_from_BA", ctypes.c_int32),
                ("materialize_residual", ctypes.c_int32)]


_P, _I64, _I32, _U64, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t


class LoftqMatrix(ctypes.Structure):
    _fields_ = [("W", _P), ("rows", _I64), ("cols", _I64), ("packed", _P), ("absmax", _P), ("qabsmax", _P),
                ("dq_scale", _P), ("B", _P), ("A", _P), ("objective", _P), ("sigma", _P)]


def _sig(name, res, args):
    f = getattr(_lib, name, None)
    if f is None:
        return None
    f.restype, f.argtypes = res, args
    return f


_c_quant = _sig("loftq_nf4_quantize", ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _P, _P, _I32, _I32, _P, _P, _P])
_c_dq = _sig("loftq_double_quant", ctypes.c_int, [_P, _I64, _I32, _P, _P, _P])
_c_deq = _sig("loftq_nf4_dequantize", ctypes.c_int,
              [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _P, ctypes.c_int, _P, _P, _P])
_MERGE_ARGS = [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _P, _I32, ctypes.c_float, _P, _P, _P, _P, _P]
_c_merge = _sig("loftq_nf4_merge", ctypes.c_int, _MERGE_ARGS)
_c_unmerge = _sig("loftq_nf4_unmerge", ctypes.c_int, _MERGE_ARGS)
_c_fwd = _sig("loftq_qlora_forward", ctypes.c_int,
              [_P, _I64, _I64, _I64, _P, _P, _P, _P, _I32, _P, _P, _I32, ctypes.c_float, _P, _P, _SZ, _P])
_c_fwd_ws = _sig("loftq_qlora_forward_workspace_bytes", _SZ, [_I64, _I32])
_c_fwd_na = _sig("loftq_qlora_forward_noalloc", ctypes.c_int,
                 [_P, _I64, _I64, _I64, _P, _P, _P, _P, _I32, _P, _P, _I32, ctypes.c_float, _P, _P])
_c_fwd_na_max = _sig("loftq_qlora_forward_noalloc_max_bytes", _SZ, [])
_c_svd = _sig("loftq_lowrank_svd", ctypes.c_int,
              [_P, _I64, _I64, _I32, _I32, _I32, _I32, _P, _U64, _I32, _P, _P, _P, _P, _SZ, _P])
_c_svd_ws = _sig("loftq_lowrank_svd_workspace_bytes", _SZ, [_I64, _I64, _I32, _I32, _I32])
_c_init = _sig("loftq_init", ctypes.c_int,
               [_P, ctypes.c_int, _I64, _I64, ctypes.POINTER(LoftqConfig), _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                _P])
_c_init_ws = _sig("loftq_workspace_bytes", _SZ, [_I64, _I64, ctypes.POINTER(LoftqConfig)])
_c_batch = _sig("loftq_init_batch", ctypes.c_int,
                [ctypes.POINTER(LoftqMatrix), _I32, ctypes.c_int, ctypes.POINTER(LoftqConfig), _I32,
                 ctypes.POINTER(_P), ctypes.POINTER(_P), _SZ])
_c_batch_ws = _sig("loftq_batch_workspace_bytes", _SZ, [ctypes.POINTER(LoftqMatrix), _I32, ctypes.POINTER(LoftqConfig)])
_c_defaults = _sig("loftq_default_config", None, [ctypes.POINTER(LoftqConfig)])
_c_status = _sig("loftq_status_string", ctypes.c_char_p, [ctypes.c_int])
_c_codebook = _sig("loftq_nf4_codebook", None, [ctypes.POINTER(ctypes.c_float)])
_c_nf_codebook = _sig("loftq_nf_codebook", ctypes.c_int, [_I32, ctypes.POINTER(ctypes.c_float)])
_c_prof_on = _sig("loftq_profile_enable", None, [ctypes.c_int])
_c_prof_get = _sig("loftq_profile_collect", ctypes.c_int, [ctypes.c_int, ctypes.c_char_p, _P, _P])
_c_prof_cal = _sig("loftq_profile_calibrate", ctypes.c_int, [ctypes.c_int, _P])


class LoftqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} (status {status})")


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise LoftqError(fn, st)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _wdtype(W: torch.Tensor) -> int:
    if W.dtype == torch.float32:
        return LOFTQ_F32
    if W.dtype == torch.bfloat16:
        return LOFTQ_BF16
    raise TypeError("W must be float32 or bfloat16")


def _contig(t: torch.Tensor, what: str) -> torch.Tensor:
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous device tensor")
    return t


def exported_symbols():
    """Names from include/loftq.h that the loaded library exports."""
    return [name for name in EXPORTS if hasattr(_lib, name)]


def nf4_codebook() -> list:
    buf = (ctypes.c_float * 16)()
    _c_codebook(buf)
    return list(buf)


def nf_codebook(bits: int) -> list:
    """The 2^bits k-bit NormalFloat levels (bits 2, 3 or 4)."""
    buf = (ctypes.c_float * 16)()
    _check("loftq_nf_codebook", _c_nf_codebook(int(bits), buf))
    return list(buf)[: 1 << int(bits)]


def default_config(**overrides) -> LoftqConfig:
    cfg = LoftqConfig()
    _c_defaults(ctypes.byref(cfg))
    for k, v in overrides.items():
        if not hasattr(cfg, k):
            raise KeyError(k)
        setattr(cfg, k, int(v))
    return cfg


def loftq_nf4_quantize(W: torch.Tensor, B: Optional[torch.Tensor] = None, A: Optional[torch.Tensor] = None,
                       packed: Optional[torch.Tensor] = None, absmax: Optional[torch.Tensor] = None, stream=None):
    """Quantize R = W - B A (or W) to packed NF4 codes and blockwise absmax."""
    _contig(W, "W")
    rows, cols = (W.shape[0], W.shape[1]) if W.dim() == 2 else (1, W.numel())
    n = rows * cols
    r = 0
    if B is not None:
        _contig(B, "B"), _contig(A, "A")
        r = B.shape[1]
    if packed is None:
        packed = torch.empty((n + 1) // 2, dtype=torch.uint8, device=W.device)
    if absmax is None:
        absmax = torch.empty((n + 63) // 64, dtype=torch.float32, device=W.device)
    _check("loftq_nf4_quantize", _c_quant(_ptr(W), _wdtype(W), rows, cols, _ptr(B), _ptr(A), r, 64, _ptr(packed),
                                          _ptr(absmax), _stream(stream)))
    return packed, absmax


def loftq_double_quant(absmax: torch.Tensor, stream=None):
    _contig(absmax, "absmax")
    nb = absmax.numel()
    q = torch.empty(nb, dtype=torch.int8, device=absmax.device)
    s = torch.empty((nb + 255) // 256, dtype=torch.float32, device=absmax.device)
    _check("loftq_double_quant", _c_dq(_ptr(absmax), nb, 256, _ptr(q), _ptr(s), _stream(stream)))
    return q, s


def loftq_nf4_dequantize(packed: torch.Tensor, shape, absmax: Optional[torch.Tensor] = None,
                         qabsmax: Optional[torch.Tensor] = None, dq_scale: Optional[torch.Tensor] = None,
                         W: Optional[torch.Tensor] = None, with_sumsq: bool = False, stream=None):
    """deq(Q), or W - deq(Q) when W is given; optionally also sum of squares (fp64)."""
    rows, cols = shape
    out = torch.empty((rows, cols), dtype=torch.float32, device=packed.device)
    ss = torch.empty(1, dtype=torch.float64, device=packed.device) if with_sumsq else None
    wdt = _wdtype(W) if W is not None else LOFTQ_F32
    _check("loftq_nf4_dequantize",
           _c_deq(_ptr(packed), _ptr(absmax), _ptr(qabsmax), _ptr(dq_scale), rows, cols, 64, 256, _ptr(W), wdt,
                  _ptr(out), _ptr(ss), _stream(stream)))
    return (out, ss) if with_sumsq else out


def _merge_call(fn, c_fn, packed, shape, absmax, qabsmax, dq_scale, B, A, alpha, double_quant, out, stream):
    rows, cols = shape
    n = rows * cols
    r = 0
    if B is not None:
        _contig(B, "B"), _contig(A, "A")
        r = B.shape[1]
    dev = packed.device
    if out is None:
        out = {"packed": torch.empty((n + 1) // 2, dtype=torch.uint8, device=dev),
               "absmax": torch.empty((n + 63) // 64, dtype=torch.float32, device=dev)}
        if double_quant:
            out["qabsmax"] = torch.empty((n + 63) // 64, dtype=torch.int8, device=dev)
            out["dq_scale"] = torch.empty(((n + 63) // 64 + 255) // 256, dtype=torch.float32, device=dev)
    _check(fn, c_fn(_ptr(packed), _ptr(absmax), _ptr(qabsmax), _ptr(dq_scale), rows, cols, 64, 256, _ptr(B), _ptr(A),
                    r, float(alpha), _ptr(out["packed"]), _ptr(out["absmax"]), _ptr(out.get("qabsmax")),
                    _ptr(out.get("dq_scale")), _stream(stream)))
    return out


def loftq_nf4_merge(packed: torch.Tensor, shape, B: Optional[torch.Tensor], A: Optional[torch.Tensor],
                    alpha: float = 1.0, absmax: Optional[torch.Tensor] = None, qabsmax: Optional[torch.Tensor] = None,
                    dq_scale: Optional[torch.Tensor] = None, double_quant: bool = False, out: Optional[dict] = None,
                    stream=None) -> dict:
    """Q' = NF4(deq(Q) + alpha B A): dict of packed, absmax (and qabsmax, dq_scale with double_quant).
    `out` may hold the input tensors themselves (in place)."""
    return _merge_call("loftq_nf4_merge", _c_merge, packed, shape, absmax, qabsmax, dq_scale, B, A, alpha,
                       double_quant, out, stream)


def loftq_nf4_unmerge(packed: torch.Tensor, shape, B: Optional[torch.Tensor], A: Optional[torch.Tensor],
                      alpha: float = 1.0, absmax: Optional[torch.Tensor] = None, qabsmax: Optional[torch.Tensor] = None,
                      dq_scale: Optional[torch.Tensor] = None, double_quant: bool = False, out: Optional[dict] = None,
                      stream=None) -> dict:
    """Q' = NF4(deq(Q) - alpha B A), the reverse of loftq_nf4_merge (not an exact inverse)."""
    return _merge_call("loftq_nf4_unmerge", _c_unmerge, packed, shape, absmax, qabsmax, dq_scale, B, A, alpha,
                       double_quant, out, stream)


def qlora_forward_workspace_bytes(n_tok: int, r: int) -> int:
    return int(_c_fwd_ws(n_tok, r))


def loftq_qlora_forward(X: torch.Tensor, packed: torch.Tensor, shape, absmax: Optional[torch.Tensor] = None,
                        qabsmax: Optional[torch.Tensor] = None, dq_scale: Optional[torch.Tensor] = None,
                        B: Optional[torch.Tensor] = None, A: Optional[torch.Tensor] = None, alpha: float = 1.0,
                        bits: int = 4, out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """Y = X bf16(deq(Q))^T + alpha (X bf16(A)^T) bf16(B)^T for bf16 X (n_tok x cols); Y fp32 n_tok x rows."""
    _contig(X, "X")
    if X.dtype != torch.bfloat16:
        raise TypeError("X must be bfloat16")
    rows, cols = shape
    n_tok = X.shape[0]
    r = 0
    if B is not None:
        _contig(B, "B"), _contig(A, "A")
        r = B.shape[1]
    if out is None:
        out = torch.empty((n_tok, rows), dtype=torch.float32, device=X.device)
    ws_bytes = 0
    if B is not None:
        ws_bytes = qlora_forward_workspace_bytes(n_tok, r)
        if ws is None:
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=X.device)
        else:
            ws_bytes = ws.numel() * ws.element_size()
    _check("loftq_qlora_forward",
           _c_fwd(_ptr(X), n_tok, rows, cols, _ptr(packed), _ptr(absmax), _ptr(qabsmax), _ptr(dq_scale), int(bits),
                  _ptr(B), _ptr(A), r, float(alpha), _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))
    return out


def qlora_forward_noalloc_max_bytes() -> int:
    return int(_c_fwd_na_max())


def loftq_qlora_forward_noalloc(X: torch.Tensor, packed: torch.Tensor, shape, absmax: Optional[torch.Tensor] = None,
                                qabsmax: Optional[torch.Tensor] = None, dq_scale: Optional[torch.Tensor] = None,
                                B: Optional[torch.Tensor] = None, A: Optional[torch.Tensor] = None,
                                alpha: float = 1.0, bits: int = 4, out: Optional[torch.Tensor] = None,
                                stream=None) -> torch.Tensor:
    """loftq_qlora_forward without a workspace: the library's own device scratch holds the
    partial products (no allocation in the call; `out` is allocated here only if not given)."""
    _contig(X, "X")
    if X.dtype != torch.bfloat16:
        raise TypeError("X must be bfloat16")
    rows, cols = shape
    n_tok = X.shape[0]
    r = 0
    if B is not None:
        _contig(B, "B"), _contig(A, "A")
        r = B.shape[1]
    if out is None:
        out = torch.empty((n_tok, rows), dtype=torch.float32, device=X.device)
    _check("loftq_qlora_forward_noalloc",
           _c_fwd_na(_ptr(X), n_tok, rows, cols, _ptr(packed), _ptr(absmax), _ptr(qabsmax), _ptr(dq_scale),
                     int(bits), _ptr(B), _ptr(A), r, float(alpha), _ptr(out), _stream(stream)))
    return out


def lowrank_workspace_bytes(rows: int, cols: int, r: int, oversample: int, exact: bool) -> int:
    return int(_c_svd_ws(rows, cols, r, oversample, int(bool(exact))))


def loftq_lowrank_svd(E: torch.Tensor, r: int, oversample: int = 8, power_iters: int = 2, exact: bool = False,
                      omega: Optional[torch.Tensor] = None, seed: int = 42, t: int = 1, stream=None):
    """Rank-r factors (B, A, sigma) of E by exact or randomized SVD."""
    _contig(E, "E")
    rows, cols = E.shape
    ws_bytes = lowrank_workspace_bytes(rows, cols, r, oversample, exact)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=E.device)
    B = torch.empty((rows, r), dtype=torch.float32, device=E.device)
    A = torch.empty((r, cols), dtype=torch.float32, device=E.device)
    sigma = torch.empty(r, dtype=torch.float32, device=E.device)
    _check("loftq_lowrank_svd",
           _c_svd(_ptr(E), rows, cols, r, oversample, power_iters, int(bool(exact)), _ptr(omega), seed, t, _ptr(B),
                  _ptr(A), _ptr(sigma), _ptr(ws), ws_bytes, _stream(stream)))
    return B, A, sigma


def workspace_bytes(rows: int, cols: int, cfg: LoftqConfig) -> int:
    return int(_c_init_ws(rows, cols, ctypes.byref(cfg)))


class InitBuffers:
    """Caller-owned outputs and workspace for repeated loftq_init calls on one shape."""

    def __init__(self, rows: int, cols: int, cfg: LoftqConfig, device="cuda", workspace: bool = True):
        n = rows * cols
        nb = (n + 63) // 64
        self.cfg = cfg
        self.packed = torch.empty((n + 1) // 2, dtype=torch.uint8, device=device)
        self.absmax = torch.empty(nb, dtype=torch.float32, device=device)
        self.qabsmax = torch.empty(max(nb, 1), dtype=torch.int8, device=device)
        self.dq_scale = torch.empty(max((nb + 255) // 256, 1), dtype=torch.float32, device=device)
        self.B = torch.empty((rows, cfg.rank), dtype=torch.float32, device=device)
        self.A = torch.empty((cfg.rank, cols), dtype=torch.float32, device=device)
        self.sigma = torch.empty(cfg.rank, dtype=torch.float32, device=device)
        self.objective = torch.empty(cfg.iterative_steps + 1, dtype=torch.float64, device=device)
        self.ws_bytes = workspace_bytes(rows, cols, cfg) if workspace else 0
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=device) if workspace else None

    def matrix(self, W: torch.Tensor) -> LoftqMatrix:
        """This buffer set as one loftq_matrix_t of a batch, for weight W."""
        rows, cols = W.shape
        dq = bool(self.cfg.double_quant)
        return LoftqMatrix(W.data_ptr(), rows, cols, self.packed.data_ptr(), self.absmax.data_ptr(),
                           self.qabsmax.data_ptr() if dq else None, self.dq_scale.data_ptr() if dq else None,
                           self.B.data_ptr(), self.A.data_ptr(), self.objective.data_ptr(), self.sigma.data_ptr())


def loftq_init(W: torch.Tensor, cfg: Optional[LoftqConfig] = None, buffers: Optional[InitBuffers] = None,
               stream=None, **overrides):
    """LoftQ initialisation of one matrix; returns a dict of device tensors."""
    _contig(W, "W")
    if cfg is None:
        cfg = default_config(**overrides)
    rows, cols = W.shape
    bufs = buffers if buffers is not None else InitBuffers(rows, cols, cfg, W.device)
    _check("loftq_init",
           _c_init(_ptr(W), _wdtype(W), rows, cols, ctypes.byref(cfg), _ptr(bufs.packed), _ptr(bufs.absmax),
                   _ptr(bufs.qabsmax), _ptr(bufs.dq_scale), _ptr(bufs.B), _ptr(bufs.A), _ptr(bufs.objective),
                   _ptr(bufs.sigma), _ptr(bufs.ws), bufs.ws_bytes, _stream(stream)))
    out = dict(packed=bufs.packed, absmax=bufs.absmax, B=bufs.B, A=bufs.A, sigma=bufs.sigma,
               objective=bufs.objective)
    if cfg.double_quant:
        out.update(qabsmax=bufs.qabsmax, dq_scale=bufs.dq_scale)
    return out


class BatchRunner:
    """Caller-owned outputs, per-stream workspaces and streams for repeated loftq_init_batch
    calls over one list of weights (all of one storage dtype)."""

    def __init__(self, Ws, cfg: LoftqConfig, nstreams: int = 4, device="cuda"):
        self.Ws = list(Ws)
        for W in self.Ws:
            _contig(W, "W")
        self.wdt = _wdtype(self.Ws[0])
        if any(_wdtype(W) != self.wdt for W in self.Ws):
            raise TypeError("every W of a batch must have the same dtype")
        self.cfg = cfg
        self.buffers = [InitBuffers(W.shape[0], W.shape[1], cfg, device, workspace=False) for W in self.Ws]
        n = len(self.Ws)
        self.mats = (LoftqMatrix * n)(*[b.matrix(W) for b, W in zip(self.buffers, self.Ws)])
        self.ws_bytes = int(_c_batch_ws(self.mats, n, ctypes.byref(cfg)))
        if self.ws_bytes == 0:
            raise LoftqError("loftq_batch_workspace_bytes", 1)
        self.nstreams = int(nstreams)
        # streams at the default priority
        self.streams = [torch.cuda.Stream(device=device) for _ in range(self.nstreams)]
        self.ws = [torch.empty(self.ws_bytes, dtype=torch.uint8, device=device) for _ in range(self.nstreams)]
        self._c_streams = (_P * self.nstreams)(*[s.cuda_stream for s in self.streams])
        self._c_ws = (_P * self.nstreams)(*[w.data_ptr() for w in self.ws])

    def run(self):
        """Enqueue the batch; the current stream then waits for every batch stream."""
        cur = torch.cuda.current_stream()
        for s in self.streams:
            s.wait_stream(cur)
        _check("loftq_init_batch", _c_batch(self.mats, len(self.Ws), self.wdt, ctypes.byref(self.cfg),
                                            self.nstreams, self._c_streams, self._c_ws, self.ws_bytes))
        for s in self.streams:
            cur.wait_stream(s)
        return self.buffers


def loftq_init_batch(Ws, cfg: Optional[LoftqConfig] = None, nstreams: int = 4, **overrides):
    """LoftQ initialisation of a list of weights in one batched call; returns one InitBuffers per weight."""
    if cfg is None:
        cfg = default_config(**overrides)
    return BatchRunner(Ws, cfg, nstreams).run()


def profile_enable(on: bool = True) -> None:
    """Bracket every library kernel launch with HIP events on its stream (measurement only)."""
    _c_prof_on(1 if on else 0)


def profile_calibrate(n: int = 256, stream=None) -> None:
    """n bracketed launches of an empty kernel (recorded as "event_overhead" while timing is enabled)."""
    _check("loftq_profile_calibrate", _c_prof_cal(n, _stream(stream)))


def profile_collect(max_entries: int = 64) -> dict:
    """{kernel name: (launches, total milliseconds)} for the launches recorded since the last collect."""
    names = ctypes.create_string_buffer(64 * max_entries)
    launches = (ctypes.c_int64 * max_entries)()
    total = (ctypes.c_double * max_entries)()
    n = _c_prof_get(max_entries, names, ctypes.cast(launches, ctypes.c_void_p), ctypes.cast(total, ctypes.c_void_p))
    out = {}
    for i in range(n):
        nm = names.raw[64 * i:64 * i + 64].split(b"\0", 1)[0].decode()
        out[nm] = (int(launches[i]), float(total[i]))
    return out
