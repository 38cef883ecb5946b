"""CPU oracle for the MLA Prolog (numpy/ctypes front end of ``mlap_oracle.c``).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code
with the HIP path (``mla_prolog_amd``) and never imports it; the only module
both sides use is the seeded input generator ``synth``.

Every function documents the passage of the pages it follows; the arithmetic
itself lives in ``mlap_oracle.c``. Pins: ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mlap_oracle.c")
# MLAP_ORACLE_LIBRARY names another build of the oracle (the sanitizer build of the tests)
_LIB_PATH = os.environ.get("MLAP_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-std=c11", "-Wall", "-Wno-unknown-pragmas"]


# UndefinedBehaviorSanitizer, every finding fatal
UBSAN = ["-fsanitize=undefined", "-fno-sanitize-recover=all", "-g"]


def build(force: bool = True, out: str = None, ubsan: bool = False) -> str:
    """Compile ``liboracle.so`` (or `out`) with gcc (plain C, OpenMP over token rows); with
    `ubsan`, under UndefinedBehaviorSanitizer."""
    out = out or _LIB_PATH
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, *(UBSAN if ubsan else []), _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class _Cfg(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("hidden", "q_lora", "kv_lora", "rope_dim", "nope_dim",
                                          "v_dim", "n_heads", "max_pos")] + \
               [("eps", C.c_float), ("w8a8", C.c_int32), ("norm_rsqrt", C.c_int32),
                ("rope_chunk", C.c_int32), ("q_quant_per_head", C.c_int32),
                ("q_head_norm", C.c_int32), ("mxfp8", C.c_int32)]


class _Inputs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("x", "positions", "w_qa", "w_qb", "w_kva", "w_kvb",
                                          "ws_qa", "ws_qb", "ws_kva", "ws_kvb", "gamma_q",
                                          "gamma_kv", "cos", "sin", "ms_qa", "ms_qb", "ms_kva",
                                          "ms_kvb")]


_OUT_FIELDS = ("q_nope", "q_pe", "kv_norm", "k_pe", "k_nope", "value", "q_norm", "q_i8",
               "q_scale", "kv_i8", "kv_scale")


class _Outputs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in _OUT_FIELDS]


class _Given(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("a", "qn", "kvn", "qraw", "qpe")]


_TAP_FIELDS = ("a_proj", "q_proj", "q_pre")


class _Taps(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in _TAP_FIELDS]


def load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = C.CDLL(_LIB_PATH)
            lib.orc_bf16.restype = C.c_uint16
            lib.orc_bf16.argtypes = [C.c_float]
            lib.orc_bf16_array.argtypes = [C.c_void_p, C.c_void_p, C.c_int64]
            lib.orc_gemm_bf16.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_int64,
                                          C.c_void_p]
            lib.orc_gemm_i8.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_int64,
                                        C.c_void_p]
            lib.orc_gemm_i8.restype = C.c_int
            lib.orc_rmsnorm_row.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_float,
                                            C.c_void_p]
            lib.orc_rope_row.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]
            lib.orc_rmsnorm_row_rsqrt.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_float,
                                                  C.c_void_p]
            lib.orc_rope_row_chunked.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64,
                                                 C.c_int64, C.c_void_p]
            lib.orc_quant_row.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]
            lib.orc_e4m3_value.argtypes = [C.c_uint8]
            lib.orc_e4m3_value.restype = C.c_double
            lib.orc_e4m3_round.argtypes = [C.c_double]
            lib.orc_e4m3_round.restype = C.c_double
            lib.orc_mx_quant_row.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]
            lib.orc_cache_scatter.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p,
                                              C.c_int64, C.c_void_p]
            lib.orc_cache_scatter.restype = C.c_int
            lib.orc_prolog.argtypes = [C.POINTER(_Cfg), C.POINTER(_Inputs), C.c_void_p, C.c_int32,
                                       C.POINTER(_Outputs)]
            lib.orc_prolog.restype = C.c_int
            lib.orc_prolog_staged.argtypes = [C.POINTER(_Cfg), C.POINTER(_Inputs), C.c_void_p,
                                              C.c_int32, C.POINTER(_Given), C.POINTER(_Outputs),
                                              C.POINTER(_Taps)]
            lib.orc_prolog_staged.restype = C.c_int
            lib.orc_num_threads.restype = C.c_int
            lib.orc_set_num_threads.argtypes = [C.c_int]
            lib.orc_set_num_threads.restype = None
            _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _np(t, dtype=None):
    """torch tensor or numpy array -> contiguous numpy array (bf16 -> uint16 bits)."""
    if t is None:
        return None
    if hasattr(t, "detach"):
        import torch
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        t = t.numpy()
    a = np.ascontiguousarray(t)
    if dtype is not None:
        a = a.astype(dtype, copy=False)
    return a


def num_threads() -> int:
    return int(load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's OpenMP loops use from now on."""
    load().orc_set_num_threads(int(n))


# ----------------------------------------------------------------- pieces ----

def bf16(v):
    """fp32 -> bf16 bits, round to nearest even (definition-based; see mlap_oracle.c)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    load().orc_bf16_array(_p(v), _p(out), v.size)
    return out


def f32(b):
    """bf16 bits -> fp32 (exact widening)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def gemm_bf16(X, W):
    """Y = bf16(fp32(sum_k X W^T)) with an fp64 sum; X [M,K], W [N,K] as bf16 bits.

    AT-10 card (matmul with BF16 out, weight [N,K], b_trans) -- "PyPTO-Gym 算子设计模式
    AT-10", sections 二 and 五."""
    X, W = _np(X, np.uint16), _np(W, np.uint16)
    M, K = X.shape
    N, K2 = W.shape
    assert K == K2
    Y = np.empty((M, N), np.uint16)
    load().orc_gemm_bf16(_p(X), _p(W), M, N, K, _p(Y))
    return Y


def gemm_i8(A, B):
    """Exact int32 C = A B^T for int8 A [M,K], B [N,K] (AT-09 INT8 W8A8 matmul, section 四)."""
    A, B = _np(A, np.int8), _np(B, np.int8)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    Cm = np.empty((M, N), np.int32)
    rc = load().orc_gemm_i8(_p(A), _p(B), M, N, K, _p(Cm))
    if rc != 0:
        raise OverflowError("int32 accumulator overflow")
    return Cm


def rmsnorm_row(v, gamma, eps):
    """RMSNorm variant B (sqrt then divide) in fp32, times fp32(gamma), cast to bf16.

    AT-10 card, section 三 (variant B) and section 五 (gamma in fp32, then BF16)."""
    v = _np(v, np.uint16).reshape(-1)
    g = None if gamma is None else _np(gamma, np.uint16).reshape(-1)
    out = np.empty_like(v)
    load().orc_rmsnorm_row(_p(v), _p(g), v.size, C.c_float(eps), _p(out))
    return out


def rmsnorm_row_rsqrt(v, gamma, eps):
    """RMSNorm variant A: sum of squares, times 1/D, + eps, rsqrt (one rounding), times
    fp32(gamma), cast to bf16. AT-10 card, section 三 (variant A)."""
    v = _np(v, np.uint16).reshape(-1)
    g = None if gamma is None else _np(gamma, np.uint16).reshape(-1)
    out = np.empty_like(v)
    load().orc_rmsnorm_row_rsqrt(_p(v), _p(g), v.size, C.c_float(eps), _p(out))
    return out


def rope_row_chunked(u, c, s, chunk=2):
    """The QuantRope3D form: the slice viewed as [R/chunk, chunk], the two axes transposed,
    then rotate-half; output in the transposed order. "PyPTO Operator 深度解析", section 3.3."""
    u = _np(u, np.uint16).reshape(-1)
    c = np.ascontiguousarray(c, np.float32).reshape(-1)
    s = np.ascontiguousarray(s, np.float32).reshape(-1)
    out = np.empty_like(u)
    load().orc_rope_row_chunked(_p(u), _p(c), _p(s), u.size, int(chunk), _p(out))
    return out


def e4m3_value(code):
    """Value of an OCP E4M3FN byte (NaN for 0x7F / 0xFF). grouped_matmul_swiglu_quant page,
    section 算子语义 (MXFP8: E4M3 data)."""
    return load().orc_e4m3_value(int(code) & 0xFF)


def e4m3_round(v):
    """Nearest E4M3 value to v, ties to even, saturating at +-448."""
    return load().orc_e4m3_round(float(v))


def mx_quant_row(v):
    """MX conversion of a bf16 row (length a multiple of 32), block by block: shared exponent
    floor(log2(amax)) - 8, values rounded to E4M3. Returns (dequantised bf16 bits, E8M0 bytes)."""
    v = _np(v, np.uint16).reshape(-1)
    deq = np.empty_like(v)
    sc = np.empty(v.size // 32, np.uint8)
    load().orc_mx_quant_row(_p(v), v.size, _p(deq), _p(sc))
    return deq, sc


def rope_row(u, c, s):
    """Rotate-half RoPE of one slice: x*cos + rotate_half(x)*sin, fp32, back to bf16.

    "PyPTO Operator 深度解析", section 3.3 (QuantRope, RotateHalf)."""
    u = _np(u, np.uint16).reshape(-1)
    c = np.ascontiguousarray(c, np.float32).reshape(-1)
    s = np.ascontiguousarray(s, np.float32).reshape(-1)
    out = np.empty_like(u)
    load().orc_rope_row(_p(u), _p(c), _p(s), u.size, _p(out))
    return out


def quant_row(z):
    """Per-row dynamic symmetric INT8: m = 127/amax, rint(z*m) saturated, scale = amax/127.

    "PyPTO Operator 深度解析", section 3.1 (PrologQuant); grouped_matmul_swiglu_quant
    article, section 实现特点 5."""
    z = _np(z, np.uint16).reshape(-1)
    codes = np.empty(z.size, np.int8)
    sc = np.zeros(1, np.float32)
    load().orc_quant_row(_p(z), z.size, _p(codes), _p(sc))
    return codes, float(sc[0])


def quant_rows(Z):
    """quant_row over each row of a 2-D bf16 array."""
    Z = _np(Z, np.uint16)
    Z2 = Z.reshape(Z.shape[0], -1)
    codes = np.empty(Z2.shape, np.int8)
    scales = np.empty(Z2.shape[0], np.float32)
    for i in range(Z2.shape[0]):
        codes[i], scales[i] = quant_row(Z2[i])
    return codes.reshape(Z.shape), scales


# ----------------------------------------------------------------- prolog ----

def prolog(cfg, inputs, rows=None, q_norm=None, kv_norm=None, a=None, q_raw=None, q_pe_in=None,
           taps=False):
    """Run the whole MLA Prolog for token ``rows`` (default: all) of ``inputs``.

    ``cfg`` is a ``synth.Config`` (or anything with its attributes); ``inputs``
    the dict from ``synth.make_inputs``. Returns a dict of numpy arrays, one row
    per entry of ``rows``: bf16 outputs as uint16 bits, codes int8, scales fp32.
    Staging (each optional, one row per entry of ``rows``, bf16): ``a`` [n, Lq+Lkv+R] replaces
    the down projection, ``q_norm`` / ``kv_norm`` the inputs of the q_b / kv_b projections,
    ``q_raw`` [n, H, Dn+R] the q_b projection (before any per-head norm), ``q_pe_in`` [n, H, R]
    every head's rope slice just before RoPE; everything downstream of a given row is
    computed from it. With ``taps`` the result also holds the oracle's own ``a_proj``,
    ``q_proj`` and ``q_pre`` (the same quantities). Rope slices in these rows are in the
    order the rotate-half takes them (with the QuantRope3D form: already de-interleaved).
    The chain is the V3 MLA Prolog of the AT-10 card, section 五 (q_a -> RMSNorm
    -> *gamma -> bf16 -> q_b; kv_a -> RMSNorm -> *gamma -> bf16), with the kv_b
    stage of the V2-Lite KV Prolog ("DeepSeek-V2-Lite-Chat MLA KV Prolog 迁移指南",
    section 背景) when ``v_dim > 0``, rotate-half RoPE on the rope slices and the
    per-token INT8 quant of q (after RoPE) and of kv_norm.
    """
    T = int(inputs["x"].shape[0])
    rows = np.arange(T, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
    n = int(rows.size)
    H, Dn, R, Dv = cfg.n_heads, cfg.nope_dim, cfg.rope_dim, cfg.v_dim
    Lq, Lkv = cfg.q_lora, cfg.kv_lora
    w8 = bool(cfg.w8a8)
    mx = bool(getattr(cfg, "mxfp8", False))
    wdt = np.int8 if w8 else (np.uint8 if mx else np.uint16)

    arrs = {
        "x": _np(inputs["x"], np.uint16),
        "positions": _np(inputs["positions"], np.int32),
        "gamma_kv": _np(inputs["gamma_kv"], np.uint16),
        "w_kva": _np(inputs["w_kva"], wdt),
        "cos": _np(inputs["cos"], np.float32),
        "sin": _np(inputs["sin"], np.float32),
    }
    for k in ("w_qa", "w_qb", "w_kvb"):
        if k in inputs:
            arrs[k] = _np(inputs[k], wdt)
    if "gamma_q" in inputs:
        arrs["gamma_q"] = _np(inputs["gamma_q"], np.uint16)
    if w8:
        for k in ("w_qa", "w_qb", "w_kva", "w_kvb"):
            if k + "_scale" in inputs:
                arrs["ws" + k[1:]] = _np(inputs[k + "_scale"], np.float32)
    if mx:
        for k in ("w_qa", "w_qb", "w_kva", "w_kvb"):
            if k + "_mxscale" in inputs:
                arrs["ms" + k[1:]] = _np(inputs[k + "_mxscale"], np.uint8)

    outs = {
        "kv_norm": np.empty((n, Lkv), np.uint16),
        "k_pe": np.empty((n, R), np.uint16),
        "kv_i8": np.empty((n, Lkv), np.int8),
        "kv_scale": np.empty((n,), np.float32),
    }
    if Lq > 0:
        outs.update(q_nope=np.empty((n, H, Dn), np.uint16), q_pe=np.empty((n, H, R), np.uint16),
                    q_norm=np.empty((n, Lq), np.uint16), q_i8=np.empty((n, H, Dn + R), np.int8),
                    q_scale=np.empty((n, H) if getattr(cfg, "q_quant_per_head", False) else (n,),
                                     np.float32))
    if Dv > 0:
        outs.update(k_nope=np.empty((n, H, Dn), np.uint16), value=np.empty((n, H, Dv), np.uint16))

    c = _Cfg(cfg.hidden, Lq, Lkv, R, Dn, Dv, H, cfg.max_pos, C.c_float(cfg.eps), int(w8),
             int(getattr(cfg, "norm_rsqrt", False)), 2 if getattr(cfg, "rope_interleaved", False) else 0,
             int(getattr(cfg, "q_quant_per_head", False)), int(getattr(cfg, "q_head_norm", False)),
             int(mx))
    i = _Inputs(**{f: (_p(arrs[f]) if f in arrs else None) for f, _ in _Inputs._fields_})
    o = _Outputs(**{f: (_p(outs[f]) if f in outs else None) for f in _OUT_FIELDS})
    N1 = Lq + Lkv + R
    giv = {"a": None if a is None else _np(a, np.uint16).reshape(n, N1),
           "qn": None if q_norm is None else _np(q_norm, np.uint16).reshape(n, Lq),
           "kvn": None if kv_norm is None else _np(kv_norm, np.uint16).reshape(n, Lkv),
           "qraw": None if q_raw is None else _np(q_raw, np.uint16).reshape(n, H, Dn + R),
           "qpe": None if q_pe_in is None else _np(q_pe_in, np.uint16).reshape(n, H, R)}
    g = _Given(**{k: _p(v) for k, v in giv.items()})
    tp = {}
    if taps:
        tp["a_proj"] = np.empty((n, N1), np.uint16)
        if Lq > 0:
            tp.update(q_proj=np.empty((n, H, Dn + R), np.uint16), q_pre=np.empty((n, H, R), np.uint16))
    t = _Taps(**{f: (_p(tp[f]) if f in tp else None) for f in _TAP_FIELDS})
    rc = load().orc_prolog_staged(C.byref(c), C.byref(i), _p(rows), n, C.byref(g), C.byref(o),
                                  C.byref(t))
    if rc != 0:
        raise ValueError("oracle rejected the inputs (rc=%d)" % rc)
    outs.update(tp)
    return outs


# --------------------------------------------------------------- KV cache ----

# cache name -> the per-token output whose rows it holds
CACHE_OF = {"kv_cache": "kv_norm", "kv_cache_i8": "kv_i8", "kv_cache_scale": "kv_scale",
            "kr_cache": "k_pe"}


def cache_scatter(slots, rows, cache):
    """Row t of ``rows`` into row ``slots[t]`` of ``cache`` (in place) when the slot is in
    [0, len(cache)); other rows untouched. The ScatterUpdate of the prolog's results into
    the K cache ([V32] page, section 2.4; [BLOG] page, step 2). Raises on repeated slots."""
    slots = np.ascontiguousarray(slots, np.int32)
    rows = np.ascontiguousarray(rows)
    assert cache.flags.c_contiguous and cache.dtype == rows.dtype
    assert rows.shape[0] == slots.size and cache.shape[1:] == rows.shape[1:]
    row_bytes = rows.dtype.itemsize * int(np.prod(rows.shape[1:], dtype=np.int64))
    rc = load().orc_cache_scatter(_p(slots), int(slots.size), int(cache.shape[0]), _p(rows),
                                  row_bytes, _p(cache))
    if rc != 0:
        raise ValueError("two tokens share a cache slot")
    return cache


def kv_cache_write(outs, slots, caches):
    """Apply the KV cache write of one run: ``outs`` the oracle's per-token outputs of all
    T tokens (``prolog``), ``caches`` a dict name -> numpy cache (see CACHE_OF), updated in
    place and returned."""
    for name, cache in caches.items():
        cache_scatter(slots, outs[CACHE_OF[name]], cache)
    return caches

