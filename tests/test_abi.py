"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, and its host-side validation returns the documented status codes
before touching the GPU (no compute call is made here)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import mla_prolog_amd as mlap
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlap.h")
lib = mlap._lib


def declared_symbols():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"MLAP_API\s+[\w\s\*]+?\b(mlap_\w+)\s*\(", src)))


def test_header_declares_the_abi():
    syms = declared_symbols()
    assert set(syms) == set(mlap.EXPORTS), syms


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", mlap.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mlap_\w+)", out))
    missing = set(declared_symbols()) - exported
    assert not missing, missing
    # internal kernels and helpers stay hidden
    assert all(s.startswith("mlap_") for s in re.findall(r"\bT (\w+)", out) if "mlap" in s)


def test_status_strings_and_kernel_names():
    assert lib.mlap_status_str(mlap.MLAP_ERR_NO_MEMORY) == b"host allocation failed"
    for s in range(6):
        assert lib.mlap_status_str(s)
    assert lib.mlap_status_str(99) == b"unknown status"
    assert mlap.KERNELS == ("act_quant", "gemm_down", "norm_rope", "gemm_up_q", "gemm_up_kv",
                            "quant_q", "q_head_norm", "mx_convert")
    assert mlap.version().startswith("mlap")


def cfg_struct(**kw):
    base = dict(t_max=256, hidden=7168, q_lora=1536, kv_lora=512, rope_dim=64, nope_dim=128,
                v_dim=0, n_heads=128, max_pos=8192, eps=1e-6, flags=0)
    base.update(kw)
    return mlap._Config(*(base[k] for k in ("t_max", "hidden", "q_lora", "kv_lora", "rope_dim",
                                            "nope_dim", "v_dim", "n_heads", "max_pos")),
                        C.c_float(base["eps"]), base["flags"])


def create(**kw):
    h = C.c_void_p()
    rc = lib.mlap_create(C.byref(cfg_struct(**kw)), C.byref(h))
    return rc, h


@pytest.mark.parametrize("kw,status", [
    (dict(), mlap.MLAP_OK),
    (dict(q_lora=0, v_dim=128, n_heads=16, hidden=2048), mlap.MLAP_OK),
    (dict(flags=mlap.MLAP_W8A8), mlap.MLAP_OK),
    (dict(t_max=0), mlap.MLAP_ERR_INVALID_ARG),
    (dict(eps=-1.0), mlap.MLAP_ERR_INVALID_ARG),
    (dict(flags=0x80), mlap.MLAP_ERR_INVALID_ARG),
    (dict(hidden=7000), mlap.MLAP_ERR_UNSUPPORTED),          # not whole 128-byte K tiles
    (dict(hidden=7168 + 64, flags=mlap.MLAP_W8A8), mlap.MLAP_ERR_UNSUPPORTED),
    (dict(rope_dim=24), mlap.MLAP_ERR_UNSUPPORTED),          # RoPE pairs in 8-wide chunks
    (dict(nope_dim=100), mlap.MLAP_ERR_UNSUPPORTED),
    (dict(nope_dim=120, rope_dim=64), mlap.MLAP_ERR_UNSUPPORTED),  # head 184 fits no tile
    (dict(q_lora=16384), mlap.MLAP_ERR_UNSUPPORTED),
    (dict(flags=mlap.MLAP_NORM_RSQRT | mlap.MLAP_ROPE_INTERLEAVED | mlap.MLAP_QUANT_Q_PER_HEAD),
     mlap.MLAP_OK),
    (dict(flags=0x80), mlap.MLAP_ERR_INVALID_ARG),
    (dict(flags=mlap.MLAP_MXFP8_MFMA), mlap.MLAP_ERR_INVALID_ARG),  # needs MLAP_MXFP8
    (dict(flags=mlap.MLAP_MXFP8 | mlap.MLAP_MXFP8_MFMA), mlap.MLAP_OK),
    (dict(flags=mlap.MLAP_MXFP8), mlap.MLAP_OK),
    (dict(flags=mlap.MLAP_MXFP8 | mlap.MLAP_W8A8), mlap.MLAP_ERR_INVALID_ARG),
    (dict(flags=mlap.MLAP_Q_HEAD_NORM, hidden=4096, q_lora=1024, nope_dim=448, n_heads=64), mlap.MLAP_OK),
    (dict(flags=mlap.MLAP_Q_HEAD_NORM | mlap.MLAP_W8A8, hidden=4096, q_lora=1024, nope_dim=448,
          n_heads=64), mlap.MLAP_ERR_UNSUPPORTED),
    (dict(nope_dim=448, n_heads=64), mlap.MLAP_ERR_UNSUPPORTED),  # head 512 without the head norm
    (dict(flags=mlap.MLAP_QUANT_Q_PER_HEAD, n_heads=2048), mlap.MLAP_ERR_UNSUPPORTED),
    (dict(flags=mlap.MLAP_QUANT_Q_PER_HEAD, n_heads=256), mlap.MLAP_ERR_UNSUPPORTED),  # 49152 values
    (dict(rope_dim=8192, nope_dim=64), mlap.MLAP_ERR_UNSUPPORTED),  # the row kernels cover R <= 4096
])
def test_create_validation(kw, status):
    rc, h = create(**kw)
    assert rc == status
    if rc == mlap.MLAP_OK:
        lib.mlap_destroy(h)
    else:
        assert not h.value


def test_create_null_args_and_destroy_null():
    h = C.c_void_p()
    assert lib.mlap_create(None, C.byref(h)) == mlap.MLAP_ERR_INVALID_ARG
    assert lib.mlap_create(C.byref(cfg_struct()), None) == mlap.MLAP_ERR_INVALID_ARG
    lib.mlap_destroy(None)


def test_workspace_size_grows_with_T_and_is_aligned():
    p = mlap.Prolog.from_config(synth.get_config("v3_prefill"))
    sizes = [p.workspace_size(T) for T in (0, 1, 256, 8192)]
    assert sizes == sorted(sizes) and all(s % 256 == 0 for s in sizes)
    # down-projection output + q_norm + partial amax (one per 256-column tile of the
    # 24576-wide q up projection at this batch size: 96)
    T = 8192
    assert sizes[-1] >= T * 2112 * 2 + T * 1536 * 2 + T * 96 * 4
    with pytest.raises(mlap.MlapError):
        p.workspace_size(8193)
    # W8A8 adds the int8 copies of x and q_norm (plus their per-token scales)
    w8 = mlap.Prolog.from_config(synth.get_config("v3_w8a8"))
    T = 8192
    assert w8.workspace_size(T) >= T * 2112 * 2 + T * 1536 * 2 + T * (7168 + 1536)
    # small batches split the down projection over K: fp32 partial sums per split
    dec = mlap.Prolog.from_config(synth.get_config("v3_decode"))
    assert dec.workspace_size(256) >= 2 * 256 * 2112 * 4


def _run_raw(h, inp, out, ws, ws_bytes):
    return lib.mlap_run(h, None, C.byref(inp), C.byref(out), C.c_void_p(ws), C.c_size_t(ws_bytes))


def test_run_argument_errors_return_before_any_launch():
    rc, h = create(t_max=64)
    assert rc == 0
    fake = 0x10000  # never dereferenced: every call below fails validation first
    full = dict(T=8, x=fake, positions=fake, w_qa=fake, w_qb=fake, w_kva=fake, gamma_q=fake,
                gamma_kv=fake, cos=fake, sin=fake)
    ws_need = C.c_size_t()
    assert lib.mlap_workspace_size(h, 8, C.byref(ws_need)) == 0
    out = mlap._Outputs(q_nope=fake, q_pe=fake, q_i8=fake, q_scale=fake)
    # workspace missing / too small / misaligned
    assert _run_raw(h, mlap._Inputs(**full), out, None, 0) == mlap.MLAP_ERR_WORKSPACE
    assert _run_raw(h, mlap._Inputs(**full), out, 0x100000, ws_need.value - 1) == \
        mlap.MLAP_ERR_WORKSPACE
    assert _run_raw(h, mlap._Inputs(**full), out, 0x100010, ws_need.value) == \
        mlap.MLAP_ERR_WORKSPACE
    # T outside [0, t_max]
    assert _run_raw(h, mlap._Inputs(**dict(full, T=65)), out, 0x100000, 1 << 30) == \
        mlap.MLAP_ERR_INVALID_ARG
    assert _run_raw(h, mlap._Inputs(**dict(full, T=-1)), out, 0x100000, 1 << 30) == \
        mlap.MLAP_ERR_INVALID_ARG
    # T == 0 is a no-op that succeeds without touching anything
    assert _run_raw(h, mlap._Inputs(**dict(full, T=0)), out, None, 0) == mlap.MLAP_OK
    # missing required inputs
    for k in ("x", "positions", "w_kva", "gamma_kv", "cos", "sin", "w_qa", "w_qb", "gamma_q"):
        assert _run_raw(h, mlap._Inputs(**dict(full, **{k: None})), out, 0x100000, 1 << 30) == \
            mlap.MLAP_ERR_INVALID_ARG, k
    # outputs of a branch the configuration lacks (no kv_b here)
    assert _run_raw(h, mlap._Inputs(**full), mlap._Outputs(k_nope=fake), 0x100000, 1 << 30) == \
        mlap.MLAP_ERR_INVALID_ARG
    # q codes need the q tensors they are computed from
    assert _run_raw(h, mlap._Inputs(**full), mlap._Outputs(q_i8=fake, q_pe=fake), 0x100000,
                    1 << 30) == mlap.MLAP_ERR_INVALID_ARG
    assert lib.mlap_run(None, None, C.byref(mlap._Inputs(**full)), C.byref(out), None, 0) == \
        mlap.MLAP_ERR_INVALID_ARG
    lib.mlap_destroy(h)


def test_w8a8_run_needs_weight_scales():
    rc, h = create(t_max=64, flags=mlap.MLAP_W8A8)
    assert rc == 0
    fake = 0x10000
    full = dict(T=8, x=fake, positions=fake, w_qa=fake, w_qb=fake, w_kva=fake, gamma_q=fake,
                gamma_kv=fake, cos=fake, sin=fake, ws_qa=fake, ws_qb=fake)
    assert _run_raw(h, mlap._Inputs(**full), mlap._Outputs(), 0x100000, 1 << 30) == \
        mlap.MLAP_ERR_INVALID_ARG  # ws_kva missing
    lib.mlap_destroy(h)


def test_export_gemm_argument_errors():
    assert lib.mlap_gemm_i8_i32(None, None, None, None, 4, 4, 100) == mlap.MLAP_ERR_INVALID_ARG
    assert lib.mlap_gemm_i8_i32(None, 1, 1, 1, 4, 4, 100) == mlap.MLAP_ERR_UNSUPPORTED
    assert lib.mlap_gemm_i8_i32(None, None, None, None, 0, 4, 128) == mlap.MLAP_OK
    assert lib.mlap_gemm_bf16(None, 1, 1, 1, 4, 4, 96) == mlap.MLAP_ERR_UNSUPPORTED
    assert lib.mlap_gemm_bf16(None, 1, 1, 1, 4, 12, 64) == mlap.MLAP_ERR_UNSUPPORTED
    assert lib.mlap_gemm_bf16(None, None, None, None, 4, 4, -1) == mlap.MLAP_ERR_INVALID_ARG


def test_mxfp8_run_needs_aligned_block_scales():
    rc, h = create(t_max=64, flags=mlap.MLAP_MXFP8)
    assert rc == 0
    fake = 0x10000
    full = dict(T=8, x=fake, positions=fake, w_qa=fake, w_qb=fake, w_kva=fake, gamma_q=fake,
                gamma_kv=fake, cos=fake, sin=fake, ms_qa=fake, ms_qb=fake, ms_kva=fake)
    for k in ("ms_qa", "ms_qb", "ms_kva"):
        assert _run_raw(h, mlap._Inputs(**dict(full, **{k: None})), mlap._Outputs(), 0x100000,
                        1 << 30) == mlap.MLAP_ERR_INVALID_ARG, k
        assert _run_raw(h, mlap._Inputs(**dict(full, **{k: fake + 2})), mlap._Outputs(), 0x100000,
                        1 << 30) == mlap.MLAP_ERR_INVALID_ARG, k  # 32-bit scale loads
    lib.mlap_destroy(h)


def test_export_mxfp8_gemm_argument_errors():
    f = lib.mlap_gemm_mxfp8_f32
    assert f(None, None, None, None, None, None, 4, 4, 128) == mlap.MLAP_ERR_INVALID_ARG
    assert f(None, 1, 4, 1, 4, 1, 4, 4, 64) == mlap.MLAP_ERR_UNSUPPORTED    # K not whole stages
    assert f(None, 1, 4, 1, 4, 1, 4, 6, 128) == mlap.MLAP_ERR_UNSUPPORTED   # N % 4
    assert f(None, 1, 5, 1, 4, 1, 4, 4, 128) == mlap.MLAP_ERR_INVALID_ARG   # misaligned scales
    assert f(None, None, None, None, None, None, 0, 4, 128) == mlap.MLAP_OK


@pytest.mark.parametrize("name,var", [("v3_decode", {}), ("v2lite_kv_decode", {}), ("v4_decode", {}),
                                      ("v3_w8a8", {}), ("v3_mxfp8", {}),
                                      ("v3_mxfp8", {"mxfp8_mfma": True}), ("tiny_kv", {"mxfp8": True,
                                                                                      "mxfp8_mfma": True})])
def test_plan_sweep_every_batch_size_has_a_workspace(name, var):
    """The host plan (tile shapes, split counts, head groups) holds for every batch size up to
    a few thousand: the workspace query succeeds, is 256-byte aligned and covers at least the
    down-projection output."""
    cfg = synth.get_config(name, **var)
    p = mlap.Prolog.from_config(cfg, t_max=4096)
    n1 = cfg.q_lora + cfg.kv_lora + cfg.rope_dim
    for T in list(range(1, 300)) + [511, 512, 513, 1000, 1023, 1024, 2047, 2048, 4095, 4096]:
        n = p.workspace_size(T)
        assert n % 256 == 0 and n >= T * n1 * 2, (T, n)


# Every call below must fail validation: with a workspace of None, a check that did not fire
# would return MLAP_ERR_WORKSPACE (not launch), so the fake pointers are never dereferenced.
_IN_PTRS = ("x", "positions", "w_qa", "w_qb", "w_kva", "gamma_q", "gamma_kv", "cos", "sin")


def test_run_rejects_misaligned_tensors():
    rc, h = create(t_max=64)
    assert rc == 0
    fake = 0x10000
    full = dict(T=8, **{k: fake for k in _IN_PTRS})
    outs = dict(q_nope=fake, q_pe=fake, kv_norm=fake, k_pe=fake, q_i8=fake, q_scale=fake,
                kv_i8=fake, kv_scale=fake, q_norm=fake, a_proj=fake)
    assert _run_raw(h, mlap._Inputs(**full), mlap._Outputs(**outs), None, 0) == mlap.MLAP_ERR_WORKSPACE
    for k in _IN_PTRS:
        assert _run_raw(h, mlap._Inputs(**dict(full, **{k: fake + 8})), mlap._Outputs(**outs), None,
                        0) == mlap.MLAP_ERR_INVALID_ARG, k
    for k in outs:
        assert _run_raw(h, mlap._Inputs(**full), mlap._Outputs(**dict(outs, **{k: fake + 4})), None,
                        0) == mlap.MLAP_ERR_INVALID_ARG, k
    lib.mlap_destroy(h)
    # the int32 export too
    assert lib.mlap_gemm_i8_i32(None, fake + 4, fake, fake, 4, 4, 128) == mlap.MLAP_ERR_INVALID_ARG
    assert lib.mlap_gemm_i8_i32(None, fake, fake, fake + 8, 4, 4, 128) == mlap.MLAP_ERR_INVALID_ARG


def test_q_outputs_that_read_the_q_tensors_back_need_them():
    """The per-head q quant reads every head's values back, so even a scale-only run needs both
    q tensors; the per-head norm rewrites the raw heads in place, so any q output needs both;
    the raw-head tap exists with the per-head norm only. All rejected before any launch."""
    fake = 0x10000
    full = dict(T=8, **{k: fake for k in _IN_PTRS})
    rc, h = create(t_max=64, flags=mlap.MLAP_QUANT_Q_PER_HEAD)
    assert rc == 0
    for outs in (dict(q_scale=fake), dict(q_scale=fake, q_pe=fake), dict(q_scale=fake, q_nope=fake)):
        assert _run_raw(h, mlap._Inputs(**full), mlap._Outputs(**outs), None, 0) == \
            mlap.MLAP_ERR_INVALID_ARG, outs
    assert _run_raw(h, mlap._Inputs(**full), mlap._Outputs(q_scale=fake, q_nope=fake, q_pe=fake),
                    None, 0) == mlap.MLAP_ERR_WORKSPACE
    lib.mlap_destroy(h)
    rc, h = create(t_max=64, flags=mlap.MLAP_Q_HEAD_NORM, hidden=4096, q_lora=1024, nope_dim=448,
                   n_heads=64)
    assert rc == 0
    for outs in (dict(q_nope=fake), dict(q_pe=fake), dict(q_scale=fake), dict(q_proj=fake)):
        assert _run_raw(h, mlap._Inputs(**full), mlap._Outputs(**outs), None, 0) == \
            mlap.MLAP_ERR_INVALID_ARG, outs
    assert _run_raw(h, mlap._Inputs(**full), mlap._Outputs(q_nope=fake, q_pe=fake, q_proj=fake),
                    None, 0) == mlap.MLAP_ERR_WORKSPACE
    lib.mlap_destroy(h)
    rc, h = create(t_max=64)
    assert _run_raw(h, mlap._Inputs(**full), mlap._Outputs(q_nope=fake, q_pe=fake, q_proj=fake),
                    None, 0) == mlap.MLAP_ERR_INVALID_ARG  # no per-head norm: no raw-head tap
    lib.mlap_destroy(h)


def test_binding_checks_shapes_against_the_configuration():
    """The binding compares every tensor's shape with the configuration before a pointer
    reaches the library (shape logic only; no tensor is created on a device)."""
    p = mlap.Prolog.from_config(synth.get_config("v3_decode", T=8))
    sh = p._shapes(8, slots=16)
    assert sh["x"] == (8, 7168) and sh["w_qb"] == (128 * 192, 1536) and sh["q_i8"] == (8, 128, 192)
    assert sh["a_proj"] == (8, 2112) and sh["kv_cache"] == (16, 512) and sh["w_qa_mxscale"] == (1536, 224)
    import torch
    ok = {"x": torch.empty(8, 7168), "q_nope": torch.empty(8, 128, 128)}
    p._check_shapes(ok, 8, 0)
    for bad in ({"x": torch.empty(8, 7169)}, {"q_nope": torch.empty(8, 128, 64)},
                {"kv_scale": torch.empty(9)}, {"cos": torch.empty(8192, 32)}):
        with pytest.raises(ValueError):
            p._check_shapes(bad, 8, 0)
    ph = mlap.Prolog.from_config(synth.get_config("v3_decode", T=8, q_quant_per_head=True))
    assert ph._shapes(8)["q_scale"] == (8, 128)


def test_run_static_checks_before_touching_the_device():
    """mlap_run_static rejects a missing handle, a batch past t_max and a batch whose workspace
    exceeds its fixed scratch before any device call (fake pointers, never dereferenced)."""
    rc, h = create(t_max=16384)
    assert rc == 0
    fake = 0x10000
    full = dict(T=16384, **{k: fake for k in _IN_PTRS})
    need = C.c_size_t()
    assert lib.mlap_workspace_size(h, 16384, C.byref(need)) == 0
    assert need.value > mlap.MLAP_STATIC_SCRATCH_BYTES
    run = lambda i: lib.mlap_run_static(h, None, C.byref(mlap._Inputs(**i)), C.byref(mlap._Outputs(kv_norm=fake)))
    assert run(full) == mlap.MLAP_ERR_WORKSPACE
    assert run(dict(full, T=16385)) == mlap.MLAP_ERR_INVALID_ARG
    assert run(dict(full, T=0)) == mlap.MLAP_OK
    assert lib.mlap_run_static(None, None, C.byref(mlap._Inputs(**full)),
                               C.byref(mlap._Outputs(kv_norm=fake))) == mlap.MLAP_ERR_INVALID_ARG
    lib.mlap_destroy(h)


def test_debug_flags_in_release_and_debug_builds():
    """mlap_debug_flags is exported by both builds; the release build reports it unsupported."""
    if mlap.lib_path().endswith("libmlap_debug.so"):
        pytest.skip("running against the debug build")
    assert mlap.debug_flags() is None
    dbg = os.path.join(os.path.dirname(mlap.lib_path()), "libmlap_debug.so")
    if os.path.exists(dbg):
        lib = C.CDLL(dbg)
        for name in mlap.EXPORTS:
            getattr(lib, name)
