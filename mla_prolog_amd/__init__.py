"""mla_prolog_amd -- Python binding of libmlap.so, the gfx950 MLA Prolog.

Argument marshalling only: every step of the prolog runs in the HIP kernels of
``libmlap.so`` (C ABI in ``include/mlap.h``). PyTorch is used for device memory
and for the current HIP stream. There is no CPU fallback: if the library is not
built, importing this package raises.

    >>> p = Prolog(t_max=256, hidden=7168, q_lora=1536, kv_lora=512, rope_dim=64,
    ...            nope_dim=128, v_dim=0, n_heads=128, max_pos=8192)
    >>> out = p.run(x, positions, weights, cos, sin)      # dict of cuda tensors
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # noqa: F401  -- must precede the library: libmlap binds to torch's HIP runtime

__all__ = ["Prolog", "MlapError", "gemm_i8_i32", "gemm_bf16", "KERNELS", "lib_path", "version", "debug_flags"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLAP_LIBRARY names another build of the same library (the sanitizer build of the tests)
_LIB = os.environ.get("MLAP_LIBRARY") or os.path.join(_HERE, "libmlap.so")

(MLAP_OK, MLAP_ERR_INVALID_ARG, MLAP_ERR_UNSUPPORTED, MLAP_ERR_WORKSPACE, MLAP_ERR_HIP,
 MLAP_ERR_NO_MEMORY) = range(6)
MLAP_W8A8 = 0x1
MLAP_NORM_RSQRT = 0x2        # RMSNorm variant A
MLAP_ROPE_INTERLEAVED = 0x4  # rope slices de-interleaved before rotate-half
MLAP_QUANT_Q_PER_HEAD = 0x8  # q codes / scales per (token, head)
MLAP_Q_HEAD_NORM = 0x10      # RMSNorm of every q head after q_b (the V4-shape prolog)
MLAP_MXFP8 = 0x20            # E4M3 weights with E8M0 scales per 32 of K; MX-converted activations
MLAP_MXFP8_MFMA = 0x40       # ... on the block-scaled MFMA (hardware sums, not exact)
MLAP_STATIC_SCRATCH_BYTES = 64 << 20  # device scratch per GPU behind mlap_run_static

EXPORTS = ("mlap_create", "mlap_workspace_size", "mlap_run", "mlap_run_static", "mlap_destroy", "mlap_status_str",
           "mlap_gemm_i8_i32", "mlap_gemm_bf16", "mlap_gemm_mxfp8_f32", "mlap_timing_begin", "mlap_timing_end",
           "mlap_timing_clock", "mlap_debug_flags",
           "mlap_kernel_name", "mlap_version")


class MlapError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, _lib.mlap_status_str(status).decode(), status))


class _Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("t_max", "hidden", "q_lora", "kv_lora", "rope_dim",
                                          "nope_dim", "v_dim", "n_heads", "max_pos")] + \
               [("eps", C.c_float), ("flags", C.c_uint32)]


class _Inputs(C.Structure):
    _fields_ = [("T", C.c_int32)] + [(n, C.c_void_p) for n in (
        "x", "positions", "w_qa", "w_qb", "w_kva", "w_kvb", "ws_qa", "ws_qb", "ws_kva", "ws_kvb",
        "gamma_q", "gamma_kv", "cos", "sin", "slot_mapping")] + [("cache_slots", C.c_int32)] + \
        [(n, C.c_void_p) for n in ("ms_qa", "ms_qb", "ms_kva", "ms_kvb")]


OUTPUTS = ("q_nope", "q_pe", "kv_norm", "k_pe", "k_nope", "value", "q_norm", "q_i8", "q_scale",
           "kv_i8", "kv_scale")
# KV cache rows written at inputs["slot_mapping"]: [cache_slots, Lkv] bf16, [cache_slots, Lkv]
# int8, [cache_slots] fp32, [cache_slots, R] bf16
CACHES = ("kv_cache", "kv_cache_i8", "kv_cache_scale", "kr_cache")
# diagnostic taps: the down projection as the row stage reads it [T, Lq+Lkv+R] bf16, and (with the
# per-head q norm) the raw q up projection [T, H, Dn+R] bf16
TAPS = ("a_proj", "q_proj")
_DTYPES = {"q_i8": torch.int8, "kv_i8": torch.int8, "q_scale": torch.float32,
           "kv_scale": torch.float32, "kv_cache_i8": torch.int8, "kv_cache_scale": torch.float32}


class _Outputs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in OUTPUTS + CACHES + TAPS]


def _load():
    if not os.path.exists(_LIB):
        raise ImportError("libmlap.so is not built (run `python mla_prolog_amd/build.py`); "
                          "there is no fallback path")
    lib = C.CDLL(_LIB)
    for name in EXPORTS:
        getattr(lib, name)  # raises AttributeError if an ABI symbol is missing
    lib.mlap_create.argtypes = [C.POINTER(_Config), C.POINTER(C.c_void_p)]
    lib.mlap_workspace_size.argtypes = [C.c_void_p, C.c_int32, C.POINTER(C.c_size_t)]
    lib.mlap_run.argtypes = [C.c_void_p, C.c_void_p, C.POINTER(_Inputs), C.POINTER(_Outputs),
                             C.c_void_p, C.c_size_t]
    lib.mlap_run_static.argtypes = [C.c_void_p, C.c_void_p, C.POINTER(_Inputs), C.POINTER(_Outputs)]
    lib.mlap_destroy.argtypes = [C.c_void_p]
    lib.mlap_destroy.restype = None
    lib.mlap_status_str.argtypes = [C.c_int]
    lib.mlap_status_str.restype = C.c_char_p
    lib.mlap_gemm_i8_i32.argtypes = [C.c_void_p] * 4 + [C.c_int32] * 3
    lib.mlap_gemm_bf16.argtypes = [C.c_void_p] * 4 + [C.c_int32] * 3
    lib.mlap_gemm_mxfp8_f32.argtypes = [C.c_void_p] * 6 + [C.c_int32] * 3
    lib.mlap_timing_begin.argtypes = [C.c_void_p, C.c_int32, C.c_int32]
    lib.mlap_timing_end.argtypes = [C.c_void_p, C.POINTER(C.c_float), C.c_int32,
                                    C.POINTER(C.c_int32)]
    lib.mlap_timing_clock.argtypes = [C.c_void_p, C.c_void_p]
    lib.mlap_debug_flags.argtypes = [C.POINTER(C.c_uint32), C.c_int32]
    lib.mlap_kernel_name.argtypes = [C.c_int32]
    lib.mlap_kernel_name.restype = C.c_char_p
    lib.mlap_version.restype = C.c_char_p
    return lib


_lib = _load()


def lib_path() -> str:
    return _LIB


def version() -> str:
    return _lib.mlap_version().decode()


def debug_flags(reset: bool = True):
    """Bits of the debug build's failed bounds checks on the current device since the last
    reset (0: none; see mlap_debug_flags in include/mlap.h), or None for a release build."""
    f = C.c_uint32(0)
    st = _lib.mlap_debug_flags(C.byref(f), 1 if reset else 0)
    if st == MLAP_ERR_UNSUPPORTED:
        return None
    if st != MLAP_OK:
        raise MlapError(st, "mlap_debug_flags")
    return f.value


def _kernels():
    names, i = [], 0
    while True:
        n = _lib.mlap_kernel_name(i)
        if n is None:
            return tuple(names)
        names.append(n.decode())
        i += 1


KERNELS = _kernels()


def _check(status, what):
    if status != MLAP_OK:
        raise MlapError(status, what)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


class Prolog:
    """One MLA Prolog configuration (a host-side handle; holds no device memory)."""

    def __init__(self, t_max, hidden, q_lora, kv_lora, rope_dim, nope_dim, v_dim, n_heads,
                 max_pos, eps=1e-6, w8a8=False, norm_rsqrt=False, rope_interleaved=False,
                 q_quant_per_head=False, q_head_norm=False, mxfp8=False, mxfp8_mfma=False):
        self.cfg = dict(t_max=t_max, hidden=hidden, q_lora=q_lora, kv_lora=kv_lora,
                        rope_dim=rope_dim, nope_dim=nope_dim, v_dim=v_dim, n_heads=n_heads,
                        max_pos=max_pos, eps=eps, w8a8=bool(w8a8), norm_rsqrt=bool(norm_rsqrt),
                        rope_interleaved=bool(rope_interleaved),
                        q_quant_per_head=bool(q_quant_per_head), q_head_norm=bool(q_head_norm),
                        mxfp8=bool(mxfp8), mxfp8_mfma=bool(mxfp8_mfma))
        flags = ((MLAP_W8A8 if w8a8 else 0) | (MLAP_NORM_RSQRT if norm_rsqrt else 0) |
                 (MLAP_ROPE_INTERLEAVED if rope_interleaved else 0) |
                 (MLAP_QUANT_Q_PER_HEAD if q_quant_per_head else 0) |
                 (MLAP_Q_HEAD_NORM if q_head_norm else 0) | (MLAP_MXFP8 if mxfp8 else 0) |
                 (MLAP_MXFP8_MFMA if mxfp8_mfma else 0))
        c = _Config(int(t_max), int(hidden), int(q_lora), int(kv_lora), int(rope_dim),
                    int(nope_dim), int(v_dim), int(n_heads), int(max_pos), C.c_float(eps), flags)
        h = C.c_void_p()
        _check(_lib.mlap_create(C.byref(c), C.byref(h)), "mlap_create")
        self._h = h
        self._ws = None

    @classmethod
    def from_config(cls, cfg, t_max=None):
        """Build from any object with the fields of ``synth.Config``."""
        g = lambda k: bool(getattr(cfg, k, False))
        return cls(t_max or cfg.T, cfg.hidden, cfg.q_lora, cfg.kv_lora, cfg.rope_dim,
                   cfg.nope_dim, cfg.v_dim, cfg.n_heads, cfg.max_pos, cfg.eps, cfg.w8a8,
                   g("norm_rsqrt"), g("rope_interleaved"), g("q_quant_per_head"), g("q_head_norm"),
                   g("mxfp8"), g("mxfp8_mfma"))

    def close(self):
        if getattr(self, "_h", None):
            _lib.mlap_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, T) -> int:
        n = C.c_size_t()
        _check(_lib.mlap_workspace_size(self._h, int(T), C.byref(n)), "mlap_workspace_size")
        return int(n.value)

    def workspace(self, T, device=None):
        """A workspace tensor for T tokens (cached and grown on demand)."""
        n = self.workspace_size(T)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=device or "cuda")
        return self._ws

    def _shapes(self, T, slots=0):
        """Shape of every tensor the run may take, by name: the inputs (``w_*_scale`` for W8A8,
        ``w_*_mxscale`` for MXFP8), the outputs, the caches (``slots`` rows) and the taps."""
        c = self.cfg
        H, Dn, R, Dv, Lq, Lkv, Hd = (c["n_heads"], c["nope_dim"], c["rope_dim"], c["v_dim"],
                                     c["q_lora"], c["kv_lora"], c["hidden"])
        sh = {"x": (T, Hd), "positions": (T,), "slot_mapping": (T,), "gamma_kv": (Lkv,),
              "cos": (c["max_pos"], R), "sin": (c["max_pos"], R),
              "kv_norm": (T, Lkv), "k_pe": (T, R), "kv_i8": (T, Lkv), "kv_scale": (T,),
              "kv_cache": (slots, Lkv), "kv_cache_i8": (slots, Lkv), "kv_cache_scale": (slots,),
              "kr_cache": (slots, R), "a_proj": (T, Lq + Lkv + R)}
        weights = {"w_kva": (Lkv + R, Hd)}
        if Lq > 0:
            weights.update(w_qa=(Lq, Hd), w_qb=(H * (Dn + R), Lq))
            sh.update(gamma_q=(Lq,), q_nope=(T, H, Dn), q_pe=(T, H, R), q_i8=(T, H, Dn + R),
                      q_scale=(T, H) if c["q_quant_per_head"] else (T,), q_norm=(T, Lq),
                      q_proj=(T, H, Dn + R))
        if Dv > 0:
            weights["w_kvb"] = (H * (Dn + Dv), Lkv)
            sh.update(k_nope=(T, H, Dn), value=(T, H, Dv))
        for k, (n, kk) in weights.items():
            sh[k] = (n, kk)
            sh[k + "_scale"] = (n,)
            sh[k + "_mxscale"] = (n, kk // 32)
        return sh

    def alloc_outputs(self, T, device="cuda", want=None):
        """Allocate output tensors; ``want`` selects names (default: all this config makes; the
        optional q_norm and the diagnostic taps a_proj / q_proj only when named)."""
        sh = self._shapes(T)
        names = ["kv_norm", "k_pe", "kv_i8", "kv_scale"]
        if self.cfg["q_lora"] > 0:
            names += ["q_nope", "q_pe", "q_i8", "q_scale"]
        if self.cfg["v_dim"] > 0:
            names += ["k_nope", "value"]
        if want is None:
            want = names
        return {k: torch.empty(sh[k], dtype=_DTYPES.get(k, torch.bfloat16), device=device) for k in want}

    def _check_shapes(self, tensors, T, slots):
        sh = self._shapes(T, slots)
        for k, t in tensors.items():
            if t is None or k not in sh:
                continue
            if tuple(t.shape) != tuple(sh[k]):
                raise ValueError("%s has shape %s, expected %s" % (k, tuple(t.shape), tuple(sh[k])))

    def _marshal(self, inputs, outputs, workspace):
        x = inputs["x"]
        T = int(x.shape[0])
        w8 = self.cfg["w8a8"]
        wdt = torch.int8 if w8 else torch.uint8 if self.cfg["mxfp8"] else torch.bfloat16
        if outputs is None:
            outputs = self.alloc_outputs(T, device=x.device)
        g = inputs.get
        i = _Inputs(T=T, x=_ptr(x, torch.bfloat16, "x"),
                    positions=_ptr(inputs["positions"], torch.int32, "positions"),
                    w_qa=_ptr(g("w_qa"), wdt, "w_qa"), w_qb=_ptr(g("w_qb"), wdt, "w_qb"),
                    w_kva=_ptr(inputs["w_kva"], wdt, "w_kva"), w_kvb=_ptr(g("w_kvb"), wdt, "w_kvb"),
                    ws_qa=_ptr(g("w_qa_scale"), torch.float32, "w_qa_scale"),
                    ws_qb=_ptr(g("w_qb_scale"), torch.float32, "w_qb_scale"),
                    ws_kva=_ptr(g("w_kva_scale"), torch.float32, "w_kva_scale"),
                    ws_kvb=_ptr(g("w_kvb_scale"), torch.float32, "w_kvb_scale"),
                    gamma_q=_ptr(g("gamma_q"), torch.bfloat16, "gamma_q"),
                    gamma_kv=_ptr(inputs["gamma_kv"], torch.bfloat16, "gamma_kv"),
                    cos=_ptr(inputs["cos"], torch.float32, "cos"),
                    sin=_ptr(inputs["sin"], torch.float32, "sin"),
                    slot_mapping=_ptr(g("slot_mapping"), torch.int32, "slot_mapping"),
                    **{"ms_" + k: _ptr(g("w_%s_mxscale" % k), torch.uint8, "w_%s_mxscale" % k)
                       for k in ("qa", "qb", "kva", "kvb")})
        caches = [outputs[k] for k in CACHES if outputs.get(k) is not None]
        if caches:
            i.cache_slots = int(caches[0].shape[0])
            if any(int(c.shape[0]) != i.cache_slots for c in caches):
                raise ValueError("every KV cache must have the same number of rows")
        unknown = set(outputs) - set(OUTPUTS + CACHES + TAPS)
        if unknown:
            raise ValueError("unknown outputs: %s" % sorted(unknown))
        self._check_shapes(inputs, T, i.cache_slots)
        self._check_shapes(outputs, T, i.cache_slots)
        o = _Outputs(**{k: _ptr(outputs.get(k), _DTYPES.get(k, torch.bfloat16), k)
                        for k in OUTPUTS + CACHES + TAPS})
        # workspace False: none (mlap_run_static); None: the cached one, grown on demand
        ws = None if workspace is False else self.workspace(T, device=x.device) if workspace is None else workspace
        return i, o, ws, outputs

    def run(self, inputs, outputs=None, workspace=None, stream=None):
        """Enqueue one prolog run. ``inputs``: dict with x, positions, w_kva, gamma_kv,
        cos, sin and (as configured) w_qa, w_qb, gamma_q, w_kvb, and ``*_scale`` for
        W8A8, ``*_mxscale`` (uint8 E8M0 [N, K/32], with uint8 E4M3 weights) for MXFP8;
        ``slot_mapping`` (int32 [T]) with a KV cache write. ``outputs``: dict of
        preallocated tensors (default: alloc_outputs), plus any of the caches in CACHES
        (rows = cache slots). Returns the outputs dict."""
        i, o, ws, outputs = self._marshal(inputs, outputs, workspace)
        _check(_lib.mlap_run(self._h, _stream(stream), C.byref(i), C.byref(o),
                             C.c_void_p(ws.data_ptr()), C.c_size_t(ws.numel() * ws.element_size())),
               "mlap_run")
        return outputs

    def run_static(self, inputs, outputs=None, stream=None):
        """The same run through mlap_run_static: no workspace and no allocation in the library
        (its device scratch of MLAP_STATIC_SCRATCH_BYTES per GPU is shared by every call on that
        GPU, so overlapping calls race). Returns the outputs dict."""
        i, o, _, outputs = self._marshal(inputs, outputs, workspace=False)
        _check(_lib.mlap_run_static(self._h, _stream(stream), C.byref(i), C.byref(o)), "mlap_run_static")
        return outputs

    def bind(self, inputs, outputs=None, workspace=None, stream=None):
        """Marshal the arguments once; the returned callable enqueues the same run with one
        foreign call (for tight loops and for capture into a HIP graph). The tensors must
        stay alive and in place while it is used."""
        return BoundRun(self, inputs, outputs, workspace, stream)

    # -- per-kernel timing ---------------------------------------------------
    def timing_begin(self, kernel, max_launches):
        kid = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
        _check(_lib.mlap_timing_begin(self._h, kid, int(max_launches)), "mlap_timing_begin")

    def timing_clock(self, counters):
        """Arm (a CUDA int64 tensor of 2, zeroed) or disarm (None) the shader-clock counters of
        the timed kernel; after the run, counters[0] / counters[1] * 100 is its clock in MHz."""
        ptr = None if counters is None else _ptr(counters, torch.int64, "counters")
        _check(_lib.mlap_timing_clock(self._h, ptr), "mlap_timing_clock")

    def timing_end(self, cap=100000):
        buf = (C.c_float * cap)()
        n = C.c_int32()
        _check(_lib.mlap_timing_end(self._h, buf, cap, C.byref(n)), "mlap_timing_end")
        return [float(buf[k]) for k in range(n.value)]


def gemm_i8_i32(A, B, out=None, stream=None):
    """Exact int32 C = A . B^T on the W8A8 MFMA core (test export)."""
    M, K = A.shape
    N = B.shape[0]
    if out is None:
        out = torch.empty(M, N, dtype=torch.int32, device=A.device)
    _check(_lib.mlap_gemm_i8_i32(_stream(stream), C.c_void_p(_ptr(A, torch.int8, "A")),
                                 C.c_void_p(_ptr(B, torch.int8, "B")),
                                 C.c_void_p(_ptr(out, torch.int32, "C")), M, N, K),
           "mlap_gemm_i8_i32")
    return out


def gemm_bf16(A, B, out=None, stream=None):
    """bf16(A . B^T) with fp32 accumulation on the bf16 MFMA core (test export)."""
    M, K = A.shape
    N = B.shape[0]
    if out is None:
        out = torch.empty(M, N, dtype=torch.bfloat16, device=A.device)
    _check(_lib.mlap_gemm_bf16(_stream(stream), C.c_void_p(_ptr(A, torch.bfloat16, "A")),
                               C.c_void_p(_ptr(B, torch.bfloat16, "B")),
                               C.c_void_p(_ptr(out, torch.bfloat16, "C")), M, N, K),
           "mlap_gemm_bf16")
    return out


def gemm_mxfp8_f32(A, A_scale, B, B_scale, out=None, stream=None):
    """sum_k deq(A) deq(B) in fp32 on the block-scaled MFMA core (test export): A [M, K], B [N, K]
    E4M3 bytes (uint8), scales [M, K/32] / [N, K/32] E8M0 bytes."""
    M, K = A.shape
    N = B.shape[0]
    if out is None:
        out = torch.empty(M, N, dtype=torch.float32, device=A.device)
    _check(_lib.mlap_gemm_mxfp8_f32(_stream(stream), C.c_void_p(_ptr(A, torch.uint8, "A")),
                                    C.c_void_p(_ptr(A_scale, torch.uint8, "A_scale")),
                                    C.c_void_p(_ptr(B, torch.uint8, "B")),
                                    C.c_void_p(_ptr(B_scale, torch.uint8, "B_scale")),
                                    C.c_void_p(_ptr(out, torch.float32, "C")), M, N, K),
           "mlap_gemm_mxfp8_f32")
    return out


class BoundRun:
    """A prolog run with its arguments marshalled once (see ``Prolog.bind``)."""

    def __init__(self, prolog, inputs, outputs, workspace, stream):
        self.prolog = prolog
        self._i, self._o, self._ws, self.outputs = prolog._marshal(inputs, outputs, workspace)
        self._keep = (inputs, self.outputs, self._ws)
        self._stream = _stream(stream)
        self._args = (prolog._h, self._stream, C.byref(self._i), C.byref(self._o),
                      C.c_void_p(self._ws.data_ptr()),
                      C.c_size_t(self._ws.numel() * self._ws.element_size()))

    def __call__(self):
        _check(_lib.mlap_run(*self._args), "mlap_run")
        return self.outputs

