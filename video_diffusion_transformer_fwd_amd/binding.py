"""ctypes binding of libh3dit.so: the C ABI of include/h3dit.h under the same names.

Argument marshalling only: tensors become raw device pointers (after checking that they are
on a GPU, with unit inner stride and the dtype the header names), host arrays become ctypes
buffers, error codes become ``H3Error``.  Loading fails loudly when the library has not
been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# H3DIT_LIB names another build of the same library (the host-sanitized copy that the CPU
# tests load); unset, the in-tree build is loaded
LIB_PATH = os.environ.get("H3DIT_LIB") or os.path.join(_PKG, "libh3dit.so")

H3_OK, H3_EINVAL, H3_ESHAPE, H3_EUNSUPPORTED, H3_EWORKSPACE, H3_EHIP = 0, -1, -2, -3, -4, -5
H3_FC2_BF16, H3_FC2_INT8_ROW, H3_FC2_INT8_GROUPED = 0, 1, 2
FC2_MODES = {"bf16": H3_FC2_BF16, "row": H3_FC2_INT8_ROW, "grouped": H3_FC2_INT8_GROUPED}
H3_EPI_NONE, H3_EPI_GELU = 0, 1


class H3Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"h3 error {code}: {msg}")
        self.code = code


class h3_dims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("d_model", "n_heads", "ffn_dim", "ctx_len", "latent_ch", "n_blocks")]


GLOBAL_FIELDS = ("t1_w", "t1_b", "t2_w", "t2_b", "mod_w", "mod_b", "fin_w", "fin_b", "fin_t",
                 "mod_table", "patch_w", "patch_b", "head_w", "head_b")
BLOCK_FIELDS = ("qkvq_w", "qkvq_b", "kc_w", "kc_b", "vc_w", "vc_b", "out_w", "out_b", "outc_b",
                "q_gamma", "k_gamma", "fc1_w", "fc1_b", "fc2_w", "fc2_b", "fc2_q", "fc2_s",
                "qkvq_q", "qkvq_s", "fc1_q", "fc1_s")


class h3_global_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in GLOBAL_FIELDS]


class h3_block_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in BLOCK_FIELDS]


class h3_geom(C.Structure):
    _fields_ = [("f_lat", C.c_int32), ("grid_h", C.c_int32), ("grid_w", C.c_int32),
                ("rope_spatial_scale", C.c_float), ("paired", C.c_int32)]


class h3_run_opts(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("fc2_mode", "fused_gate_adaln", "fused_cross_block", "qk_norm", "token_reduction",
                 "int8_linear", "fused_qk_rope", "store_branches", "fused_head_adaln")]


class h3_ws_layout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in
                ("n1", "qkvq", "attn", "y", "n2", "h", "m", "hq", "hs", "rope", "total")]


_VP, _I32, _I64, _F, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
_PI32, _PF, _PU8, _PU16 = C.POINTER(C.c_int32), C.POINTER(C.c_float), C.POINTER(C.c_uint8), C.POINTER(C.c_uint16)

# name -> (restype, argtypes); every symbol declared in include/h3dit.h
SIGNATURES = {
    "h3_last_error": (C.c_char_p, []),
    "h3_abi_version": (_I32, []),
    "h3_align_frames": (_I32, [_I32, _PI32]),
    "h3_frames_for_seconds": (_I32, [C.c_double, _PI32]),
    "h3_latent_frames": (_I32, [_I32, _PI32]),
    "h3_token_grid": (_I32, [_I32, _I32, _I32, _PI32, _PI32, _PF]),
    "h3_schedule": (_I32, [_I32, _I32, _I32, _PF, _PU8, _PI32]),
    "h3_select_layers": (_I32, [_PU16, _I32, _I32, _I32, _PI32]),
    "h3_token_plan": (_I32, [_I32, _I32, _I32, _I32, _I32, _PI32, _PI32, _PI32, _PI32]),
    "h3_model_create": (_I32, [C.POINTER(h3_dims), C.POINTER(h3_global_weights),
                               C.POINTER(h3_block_weights), _I32, C.POINTER(_VP)]),
    "h3_model_destroy": (None, [_VP]),
    "h3_geom_tokens": (_I32, [C.POINTER(h3_geom), _PI32]),
    "h3_workspace_size": (_I32, [_VP, _I32, C.POINTER(h3_run_opts), C.POINTER(_SZ)]),
    "h3_workspace_layout": (_I32, [_VP, _I32, C.POINTER(h3_run_opts), C.POINTER(h3_ws_layout)]),
    "h3_prepare_context": (_I32, [_VP, _VP, _VP, _VP]),
    "h3_quantize_fc2_weights": (_I32, [_VP, _VP]),
    "h3_quantize_linear_weights": (_I32, [_VP, _VP]),
    "h3_modulation": (_I32, [_VP, _F, _VP, _VP, _VP, _SZ, _VP]),
    "h3_modulation_noalloc": (_I32, [_VP, _F, _VP, _VP, _VP]),
    "h3_dit_block_fwd": (_I32, [_VP, _I32, C.POINTER(h3_geom), C.POINTER(h3_run_opts), _VP, _VP,
                                _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "h3_dit_forward": (_I32, [_VP, C.POINTER(h3_geom), C.POINTER(h3_run_opts), _VP, _F, _PI32,
                              _I32, _I32, _VP, _VP, _VP, _SZ, _VP]),
    "h3_dit_forward_cached": (_I32, [_VP, C.POINTER(h3_geom), C.POINTER(h3_run_opts), _VP, _F, _PI32,
                                     _I32, _I32, _VP, _I32, _VP, _VP, _VP, _SZ, _VP]),
    "h3_euler_step": (_I32, [_VP, _VP, _F, _F, _I64, _VP]),
    "h3_token_reduce": (_I32, [_I32, C.POINTER(h3_geom), _I32, _VP, _VP, _VP, _VP]),
    "h3_gemm_bf16": (_I32, [_VP, _I64, _VP, _I64, _VP, _I64, _I32, _I32, _I32, _VP, _VP, _I32,
                            _I32, _VP]),
    "h3_attention": (_I32, [_VP, _I64, _VP, _I64, _VP, _I64, _VP, _I64, _I32, _I32, _I32, _I32,
                            _VP]),
    "h3_quant_rows": (_I32, [_VP, _VP, _VP, _I32, _I32, _I32, _VP]),
    "h3_gemm_i8": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I32, _I32, _I32, _I32, _I32, _VP]),
    "h3_gate_adaln": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _VP]),
    "h3_gate_adaln_quant": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _VP]),
    "h3_head_adaln_gemm": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _VP]),
    "h3_rope_table": (_I32, [C.POINTER(h3_geom), _I32, _VP, _VP]),
    "h3_qk_norm_rope": (_I32, [_VP, _I64, _I32, _I32, _I32, _VP, _VP, _I32, _VP, _VP]),
    "h3_qkv_gemm": (_I32, [_VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP, _I64, _I32, _I32, _I32, _I32,
                           _VP, _VP, _I32, _VP, _I32, _I32, _PI32, _VP]),
    "h3_mfma_probe": (_I32, [_I32, _I32, _I32, _VP, _VP]),
    "h3_profile_begin": (_I32, [C.c_uint32, _I32]),
    "h3_profile_end": (_I32, [C.POINTER(C.c_double), _PI32]),
}

STAGES = ("modulation", "patch", "adaln", "qkv_gemm", "qk_norm_rope", "self_attn", "cross_attn",
          "out_gemm", "gate_adaln", "fc1_gemm", "fc2_gemm", "fc2_quant", "fc2_i8_gemm",
          "token_reduce", "head", "euler")

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m video_diffusion_transformer_fwd_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(code):
    if code != H3_OK:
        raise H3Error(code, lib().h3_last_error().decode())


_DTYPES = {}


def _dtype(name):
    if not _DTYPES:
        import torch
        _DTYPES.update(bf16=torch.bfloat16, f32=torch.float32, i8=torch.int8)
    return _DTYPES[name]


def ptr(t, dtype=None):
    """Raw device pointer of a tensor (or None).  The library takes bare device addresses and
    cannot check them, so a tensor that is not on a GPU, whose innermost stride is not 1, or
    whose dtype is not ``dtype`` ("bf16", "f32", "i8", or a tuple of them) raises here instead
    of reaching a kernel."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"expected a device tensor, got one on {t.device}")
    if t.dim() > 0 and t.size(-1) > 1 and t.stride(-1) != 1:
        raise ValueError(f"the innermost stride must be 1, got {t.stride(-1)}")
    if dtype is not None:
        names = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in tuple(_dtype(n) for n in names):
            raise TypeError(f"expected {' or '.join(names)}, got {t.dtype}")
    return C.c_void_p(t.data_ptr())


def stream_handle(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ host integer logic
def h3_align_frames(requested: int) -> int:
    out = C.c_int32()
    _check(lib().h3_align_frames(requested, C.byref(out)))
    return out.value


def h3_frames_for_seconds(seconds: float) -> int:
    out = C.c_int32()
    _check(lib().h3_frames_for_seconds(seconds, C.byref(out)))
    return out.value


def h3_latent_frames(frames: int) -> int:
    out = C.c_int32()
    _check(lib().h3_latent_frames(frames, C.byref(out)))
    return out.value


def h3_token_grid(width: int, height: int, reference_rope: bool = False):
    gh, gw, sc = C.c_int32(), C.c_int32(), C.c_float()
    _check(lib().h3_token_grid(width, height, int(reference_rope), C.byref(gh), C.byref(gw), C.byref(sc)))
    return gh.value, gw.value, sc.value


def h3_schedule(steps: int, reuse: int = 1, core_reuse: int = 1):
    sig = np.zeros(max(steps, 0) + 1, dtype=np.float32)
    fresh = np.zeros(max(steps, 1), dtype=np.uint8)
    nf = C.c_int32()
    _check(lib().h3_schedule(steps, reuse, core_reuse, sig.ctypes.data_as(_PF),
                             fresh.ctypes.data_as(_PU8), C.byref(nf)))
    return sig, fresh[:steps], nf.value


def h3_select_layers(mod_table_bf16_bits: np.ndarray, n_active: int):
    t = np.ascontiguousarray(mod_table_bf16_bits, dtype=np.uint16)
    nb, six, d = t.shape
    out = np.zeros(n_active, dtype=np.int32)
    _check(lib().h3_select_layers(t.ctypes.data_as(_PU16), nb, d, n_active, out.ctypes.data_as(_PI32)))
    return [int(v) for v in out]


def h3_token_plan(f_lat, grid_h, grid_w, eval_index, n_active, with_pairs=True):
    ma, rb, nr = C.c_int32(), C.c_int32(), C.c_int32()
    _check(lib().h3_token_plan(f_lat, grid_h, grid_w, eval_index, n_active, C.byref(ma),
                               C.byref(rb), None, C.byref(nr)))
    pairs = None
    if with_pairs:
        buf = np.zeros(2 * nr.value, dtype=np.int32)
        _check(lib().h3_token_plan(f_lat, grid_h, grid_w, eval_index, n_active, C.byref(ma),
                                   C.byref(rb), buf.ctypes.data_as(_PI32), C.byref(nr)))
        pairs = buf.reshape(-1, 2)
    return dict(merge_after=ma.value, restore_before=rb.value, pairs=pairs, n_reduced=nr.value)


def make_geom(f_lat, grid_h, grid_w, scale, paired=0):
    return h3_geom(f_lat, grid_h, grid_w, scale, paired)


def h3_geom_tokens(geom: h3_geom) -> int:
    n = C.c_int32()
    _check(lib().h3_geom_tokens(C.byref(geom), C.byref(n)))
    return n.value


def make_opts(fc2_mode="bf16", fused_gate_adaln=True, fused_cross_block=True, qk_norm=True,
              token_reduction=False, int8_linear=False, fused_qk_rope=True, store_branches=False,
              fused_head_adaln=False):
    return h3_run_opts(FC2_MODES[fc2_mode] if isinstance(fc2_mode, str) else fc2_mode,
                       int(fused_gate_adaln), int(fused_cross_block), int(qk_norm),
                       int(token_reduction), int(int8_linear), int(fused_qk_rope),
                       int(store_branches), int(fused_head_adaln))


# ------------------------------------------------------------------ model
def h3_model_create(dims: h3_dims, g: h3_global_weights, blocks) -> C.c_void_p:
    arr = (h3_block_weights * len(blocks))(*blocks)
    out = C.c_void_p()
    _check(lib().h3_model_create(C.byref(dims), C.byref(g), arr, len(blocks), C.byref(out)))
    return out


def h3_model_destroy(m):
    lib().h3_model_destroy(m)


def h3_workspace_size(m, n_tokens, opts) -> int:
    out = C.c_size_t()
    _check(lib().h3_workspace_size(m, n_tokens, C.byref(opts), C.byref(out)))
    return out.value


def h3_workspace_layout(m, n_tokens, opts) -> h3_ws_layout:
    out = h3_ws_layout()
    _check(lib().h3_workspace_layout(m, n_tokens, C.byref(opts), C.byref(out)))
    return out


def h3_prepare_context(m, ctx, ctx_kv, stream=None):
    _check(lib().h3_prepare_context(m, ptr(ctx, "bf16"), ptr(ctx_kv, "bf16"), stream_handle(stream)))


def h3_quantize_fc2_weights(m, stream=None):
    _check(lib().h3_quantize_fc2_weights(m, stream_handle(stream)))


def h3_quantize_linear_weights(m, stream=None):
    _check(lib().h3_quantize_linear_weights(m, stream_handle(stream)))


def h3_modulation(m, sigma, mod, mod_final, ws, stream=None):
    _check(lib().h3_modulation(m, sigma, ptr(mod, "f32"), ptr(mod_final, "f32"), ptr(ws), ws.numel() * ws.element_size(),
                               stream_handle(stream)))


def h3_modulation_noalloc(m, sigma, mod, mod_final, stream=None):
    _check(lib().h3_modulation_noalloc(m, sigma, ptr(mod, "f32"), ptr(mod_final, "f32"),
                                       stream_handle(stream)))


def h3_dit_block_fwd(m, block, geom, opts, x, n1_in, n1_next, mod, mod_next, ctx_kv, ws, stream=None):
    _check(lib().h3_dit_block_fwd(m, block, C.byref(geom), C.byref(opts), ptr(x, "bf16"), ptr(n1_in),
                                  ptr(n1_next), ptr(mod, "f32"), ptr(mod_next, "f32"),
                                  ptr(ctx_kv, "bf16"), ptr(ws),
                                  ws.numel() * ws.element_size(), stream_handle(stream)))


def h3_dit_forward(m, geom, opts, latent, sigma, active, eval_index, ctx_kv, velocity, ws, stream=None):
    act = np.ascontiguousarray(active, dtype=np.int32)
    _check(lib().h3_dit_forward(m, C.byref(geom), C.byref(opts), ptr(latent, "f32"), sigma,
                                act.ctypes.data_as(_PI32), len(act), eval_index, ptr(ctx_kv, "bf16"),
                                ptr(velocity, "f32"), ptr(ws), ws.numel() * ws.element_size(),
                                stream_handle(stream)))


def h3_dit_forward_cached(m, geom, opts, latent, sigma, active, eval_index, ctx_kv, refresh_core,
                          core_delta, velocity, ws, stream=None):
    act = np.ascontiguousarray(active, dtype=np.int32)
    _check(lib().h3_dit_forward_cached(m, C.byref(geom), C.byref(opts), ptr(latent, "f32"), sigma,
                                       act.ctypes.data_as(_PI32), len(act), eval_index,
                                       ptr(ctx_kv, "bf16"), int(refresh_core), ptr(core_delta, "f32"),
                                       ptr(velocity, "f32"), ptr(ws),
                                       ws.numel() * ws.element_size(), stream_handle(stream)))


def h3_euler_step(latent, velocity, sigma_cur, sigma_next, stream=None):
    _check(lib().h3_euler_step(ptr(latent, "f32"), ptr(velocity, "f32"), sigma_cur, sigma_next, latent.numel(),
                               stream_handle(stream)))


def h3_token_reduce(direction, geom, d_model, src, bypass, dst, stream=None):
    _check(lib().h3_token_reduce(direction, C.byref(geom), d_model, ptr(src, "bf16"), ptr(bypass, "bf16"),
                                 ptr(dst, "bf16"),
                                 stream_handle(stream)))


# ------------------------------------------------------------------ single operations
def h3_gemm_bf16(A, B, C_out, bias=None, bias2=None, epilogue=H3_EPI_NONE, lda=None, ldb=None,
                 ldc=None, M=None, N=None, K=None, stream=None):
    M = M if M is not None else A.shape[0]
    K = K if K is not None else A.shape[1]
    N = N if N is not None else B.shape[0]
    out_f32 = 1 if C_out.dtype.itemsize == 4 else 0
    _check(lib().h3_gemm_bf16(ptr(A, "bf16"), lda or A.stride(0), ptr(B, "bf16"), ldb or B.stride(0),
                              ptr(C_out, ("bf16", "f32")), ldc or C_out.stride(0), M, N, K,
                              ptr(bias, "bf16"), ptr(bias2, "bf16"), epilogue,
                              out_f32, stream_handle(stream)))


def h3_attention(Q, K, V, O, n_q, n_k, n_heads, head_dim, stream=None):
    _check(lib().h3_attention(ptr(Q, "bf16"), Q.stride(0), ptr(K, "bf16"), K.stride(0), ptr(V, "bf16"),
                              V.stride(0), ptr(O, "bf16"), O.stride(0), n_q, n_k, n_heads, head_dim, stream_handle(stream)))


def h3_quant_rows(X, Q, S, group, stream=None):
    rows, K = X.shape
    _check(lib().h3_quant_rows(ptr(X, "bf16"), ptr(Q, "i8"), ptr(S, "f32"), rows, K, group,
                               stream_handle(stream)))


def h3_gemm_i8(QA, SA, QW, SW, bias, C_out, group, epilogue=0, stream=None):
    M, K = QA.shape
    N = QW.shape[0]
    _check(lib().h3_gemm_i8(ptr(QA, "i8"), ptr(SA, "f32"), ptr(QW, "i8"), ptr(SW, "f32"), ptr(bias, "bf16"),
                            ptr(C_out, "bf16"),
                            C_out.stride(0), M, N, K, group, epilogue, stream_handle(stream)))


def h3_qkv_gemm(A, W, bias, C_out, head_dim, q_gamma, k_gamma, qk_norm, table, SA=None, SW=None,
                fused=True, stream=None) -> bool:
    """QKV product + Q/K RMSNorm + RoPE; int8 when A is int8 (SA, SW the scales).  Returns
    whether the fused epilogue ran."""
    import torch
    M, K = A.shape
    d = W.shape[0] // 4
    a_q8 = int(A.dtype == torch.int8)
    used = C.c_int32()
    kind = "i8" if a_q8 else "bf16"
    _check(lib().h3_qkv_gemm(ptr(A, kind), A.stride(0), ptr(SA, "f32"), ptr(W, kind), W.stride(0),
                             ptr(SW, "f32"), ptr(bias, "bf16"), ptr(C_out, "bf16"), C_out.stride(0), M,
                             d, K, head_dim, ptr(q_gamma, "bf16"), ptr(k_gamma, "bf16"), int(qk_norm),
                             ptr(table, "f32"), a_q8, int(fused),
                             C.byref(used), stream_handle(stream)))
    return bool(used.value)


def h3_gate_adaln(x, y, gate, x_out, shift, scale, n_out, stream=None):
    rows, d = x.shape
    _check(lib().h3_gate_adaln(ptr(x, "bf16"), ptr(y, "bf16"), ptr(gate, "f32"), ptr(x_out, "bf16"),
                               ptr(shift, "f32"), ptr(scale, "f32"), ptr(n_out, "bf16"), rows, d,
                               stream_handle(stream)))


def h3_gate_adaln_quant(x, y, gate, x_out, shift, scale, q_out, s_out, stream=None):
    rows, d = x.shape
    _check(lib().h3_gate_adaln_quant(ptr(x, "bf16"), ptr(y, "bf16"), ptr(gate, "f32"),
                                     ptr(x_out, "bf16"), ptr(shift, "f32"), ptr(scale, "f32"),
                                     ptr(q_out, "i8"), ptr(s_out, "f32"), rows, d,
                                     stream_handle(stream)))


def h3_head_adaln_gemm(x, shift, scale, W, bias, out, stream=None):
    rows, d = x.shape
    n_out = W.shape[0]
    # the entry point takes dense rows: x [rows, d], W [n_out, d], out [rows, n_out]
    if x.stride(0) != d or W.shape[1] != d or W.stride(0) != d or tuple(out.shape) != (rows, n_out) \
            or out.stride(0) != n_out:
        raise ValueError("h3_head_adaln_gemm: x, W and out must be dense [rows, d], [n_out, d], [rows, n_out]")
    _check(lib().h3_head_adaln_gemm(ptr(x, "bf16"), ptr(shift, "f32"), ptr(scale, "f32"),
                                    ptr(W, "bf16"), ptr(bias, "bf16"), ptr(out, "f32"), rows, d,
                                    n_out, stream_handle(stream)))


def h3_rope_table(geom, head_dim, table, stream=None):
    _check(lib().h3_rope_table(C.byref(geom), head_dim, ptr(table, "f32"), stream_handle(stream)))


def h3_qk_norm_rope(qkvq, n_tokens, d_model, head_dim, q_gamma, k_gamma, qk_norm, table,
                    stream=None):
    _check(lib().h3_qk_norm_rope(ptr(qkvq, "bf16"), qkvq.stride(0), n_tokens, d_model, head_dim,
                                 ptr(q_gamma, "bf16"), ptr(k_gamma, "bf16"), int(qk_norm), ptr(table, "f32"),
                                 stream_handle(stream)))


def h3_mfma_probe(int8, iters, workgroups, out, stream=None):
    if out.numel() < workgroups * 256:
        raise ValueError("h3_mfma_probe: out needs workgroups * 256 floats")
    _check(lib().h3_mfma_probe(int(int8), iters, workgroups, ptr(out, "f32"), stream_handle(stream)))


def h3_profile_begin(stages, max_launches=100000):
    mask = 0
    for st in stages:
        mask |= 1 << STAGES.index(st)
    _check(lib().h3_profile_begin(mask, max_launches))


def h3_profile_end():
    """{stage: (total_ms, launches)} for the stages that were timed."""
    ms = (C.c_double * len(STAGES))()
    cnt = (C.c_int32 * len(STAGES))()
    _check(lib().h3_profile_end(ms, cnt))
    return {st: (ms[i], cnt[i]) for i, st in enumerate(STAGES) if cnt[i]}
