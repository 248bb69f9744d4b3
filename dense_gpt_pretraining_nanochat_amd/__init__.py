"""Python binding of libnanochat.so, the MI355X training-step library for
nanochat's dense GPT.

Argument marshalling only: every function here forwards to the C entry point
of the same name in ``include/nanochat.h``; all computation runs in the HIP
kernels behind it. Device buffers are torch tensors (torch supplies device
memory and streams, nothing else). There is no fallback: if the library is
not built, or no GPU is present, the compute calls raise.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# NANOCHAT_LIB selects another build of the same library (the host-sanitizer
# build of sanitize.py); by default the in-tree libnanochat.so
LIB_PATH = os.environ.get("NANOCHAT_LIB") or os.path.join(_HERE, "libnanochat.so")

NC_F32, NC_BF16 = 0, 1
NC_OK = 0
NC_ERR = {-1: "NC_ERR_INVALID_CONFIG", -2: "NC_ERR_UNSUPPORTED", -3: "NC_ERR_NULL",
          -4: "NC_ERR_ALIGN", -5: "NC_ERR_WORKSPACE", -6: "NC_ERR_HIP", -7: "NC_ERR_ARG"}
NC_STATUS_TOKEN_RANGE, NC_STATUS_TARGET_RANGE, NC_STATUS_NONFINITE_LOSS = 1, 2, 4
EPI_STORE_T, EPI_STORE_F32, EPI_ADD_F32, EPI_RELU2, EPI_RELU2_BWD = 0, 1, 2, 3, 4


class NcConfig(ctypes.Structure):
    _fields_ = [("depth", ctypes.c_int32), ("vocab_size", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("n_kv_head", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("softcap", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("init_std", ctypes.c_float),
                ("dtype", ctypes.c_int32)]

    def __repr__(self):
        return ("NcConfig(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")")


class NcTensorInfo(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("offset", ctypes.c_uint64),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class NcWsPiece(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("offset", ctypes.c_uint64),
                ("bytes", ctypes.c_uint64)]


class NcOptimConfig(ctypes.Structure):
    _fields_ = [("lr_adamw", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("wd_adamw", ctypes.c_float), ("lr_muon", ctypes.c_float),
                ("momentum", ctypes.c_float), ("wd_muon", ctypes.c_float),
                ("max_grad_norm", ctypes.c_float), ("ns_steps", ctypes.c_int32),
                ("step", ctypes.c_int32)]

    def __repr__(self):
        return ("NcOptimConfig(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")")


class NcError(RuntimeError):
    def __init__(self, code, func, hip=0):
        self.code = code
        super().__init__(f"{func} -> {NC_ERR.get(code, code)}"
                         + (f" (hip error {hip})" if code == -6 else ""))


_lib = None
_P, _I32, _U64, _F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float
_CFG = ctypes.POINTER(NcConfig)
_SIGS = {
    "nc_config_from_depth": [_I32, _I32, _I32, _I32, _I32, _CFG],
    "nc_validate_config": [_CFG],
    "nc_set_lm_chunk_rows": [_I32],
    "nc_lm_chunk_rows": [_CFG, ctypes.POINTER(_I32)],
    "nc_set_gemm_persistent": [_I32],
    "nc_param_count": [_CFG, ctypes.POINTER(_U64)],
    "nc_param_layout": [_CFG, ctypes.POINTER(NcTensorInfo), _I32, ctypes.POINTER(_I32)],
    "nc_workspace_bytes": [_CFG, _I32, ctypes.POINTER(_U64)],
    "nc_token_losses_offset": [_CFG, _I32, ctypes.POINTER(_U64)],
    "nc_workspace_pieces": [_CFG, _I32, ctypes.POINTER(NcWsPiece), _I32, ctypes.POINTER(_I32)],
    "nc_init_params": [_U64, _CFG, _P, _P],
    "nc_forward_loss": [_CFG, _P, _P, _P, _P, _U64, _P, _P],
    "nc_forward_backward": [_CFG, _P, _P, _P, _P, _P, _U64, _P, _P],
    "nc_forward_backward_accumulate": [_CFG, _P, _P, _P, _P, _P, _U64, _P, _P],
    "nc_eval_bpb": [_CFG, _P, _P, _P, _P, _P, _U64, _P, _P, _P],
    "nc_kv_cache_bytes": [_CFG, _I32, ctypes.POINTER(_U64)],
    "nc_infer_workspace_bytes": [_CFG, _I32, ctypes.POINTER(_U64)],
    "nc_prefill": [_CFG, _P, _P, _I32, _P, _I32, _P, _U64, _P, _P],
    "nc_decode_step": [_CFG, _P, _P, _I32, _P, _I32, _P, _U64, _P, _P],
    "nc_optimizer_state_bytes": [_CFG, ctypes.POINTER(_U64)],
    "nc_optimizer_workspace_bytes": [_CFG, ctypes.POINTER(_U64)],
    "nc_optimizer_step": [_CFG, ctypes.POINTER(NcOptimConfig), _P, _P, _P, _P, _U64, _P, _P],
    "nc_read_device_status": [_P, ctypes.POINTER(ctypes.c_uint32), _P],
    "nc_status_string": [ctypes.c_int],
    "nc_last_hip_error": [],
    "nc_op_gemm": [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P],
    "nc_op_wgrad": [_I32, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P],
    "nc_op_gemm_axpby": [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                         ctypes.c_float, ctypes.c_float, _I32, ctypes.c_int64, ctypes.c_int64,
                         ctypes.c_int64, _I32, _P],
    "nc_op_few_rows_scratch_bytes": [_I32, _I32, _I32, _I32, ctypes.POINTER(_U64)],
    "nc_op_few_rows_gemm": [_I32, _P, _I32, _P, _I32, _P, _I32, _I32, _I32, _I32, ctypes.c_float, _P,
                            ctypes.c_float, _P, _P, _I32, _I32, _P, _U64, _P],
    "nc_op_decode_attn": [_I32, _P, _I32, _I32, _I32, _P, _I32, _I32, _P, _P, _I32, _P],
    "nc_op_transpose": [_I32, _P, _I32, _I32, _I32, _P, _I32, _P],
    "nc_op_rmsnorm_fwd": [_I32, _P, _I32, _I32, _F32, _P, _P, _P],
    "nc_op_rmsnorm_bwd": [_I32, _P, _P, _P, _I32, _I32, _P, _I32, _P, _P],
    "nc_op_rope_qknorm_fwd": [_I32, _P, _I32, _I32, _I32, _F32, _F32, _P, _P, _P],
    "nc_op_rope_qknorm_bwd": [_I32, _P, _P, _I32, _I32, _I32, _P, _P, _P],
    "nc_op_attn_fwd": [_I32, _P, _I32, _I32, _I32, _P, _P, _P],
    "nc_op_attn_bwd_scratch_bytes": [_I32, _I32],
    "nc_op_attn_bwd": [_I32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P],
    "nc_op_softcap_ce": [_I32, _P, _P, _I32, _I32, _F32, _F32, _P, _P, _P, _P],
    "nc_op_attn_bwd_noalloc": [_I32, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P],
    "nc_op_attn_bwd_ds_bytes": [_I32, _I32, _I32, _I32],
    "nc_op_attn_bwd_stored_ds": [_I32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P],
}


def lib():
    """Loads the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        # torch first: the library then binds to the HIP runtime torch ships
        # (same sonames), so one runtime serves torch's allocations and
        # streams and these kernels. Loaded the other way round, the system
        # runtime is loaded first and, on the GPU machines used here, calls
        # then fail with hipErrorNoDevice.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = {"nc_status_string": ctypes.c_char_p,
                         "nc_op_attn_bwd_scratch_bytes": ctypes.c_uint64,
                         "nc_op_attn_bwd_ds_bytes": ctypes.c_uint64}.get(name, ctypes.c_int)
        _lib = L
    return _lib


def _check(rc, name):
    if rc != NC_OK:
        raise NcError(rc, name, lib().nc_last_hip_error())


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dt(dtype):
    if isinstance(dtype, int):
        return dtype              # passed through; the library rejects unknown codes
    return {"f32": NC_F32, "bf16": NC_BF16}[dtype]


# ---------------------------------------------------------------- host calls

def nc_config_from_depth(depth, vocab_size, seq_len, batch, dtype="bf16") -> NcConfig:
    cfg = NcConfig()
    _check(lib().nc_config_from_depth(depth, vocab_size, seq_len, batch, _dt(dtype),
                                      ctypes.byref(cfg)), "nc_config_from_depth")
    return cfg


def nc_validate_config(cfg) -> int:
    return lib().nc_validate_config(ctypes.byref(cfg))


def nc_set_lm_chunk_rows(rows: int):
    _check(lib().nc_set_lm_chunk_rows(rows), "nc_set_lm_chunk_rows")


def nc_set_gemm_persistent(on):
    """on: True/False (or the raw 0/1 the C call takes; anything else is refused)."""
    v = int(on) if isinstance(on, bool) else on
    _check(lib().nc_set_gemm_persistent(v), "nc_set_gemm_persistent")


def nc_lm_chunk_rows(cfg) -> int:
    n = _I32()
    _check(lib().nc_lm_chunk_rows(ctypes.byref(cfg), ctypes.byref(n)), "nc_lm_chunk_rows")
    return n.value


def nc_param_count(cfg) -> int:
    n = _U64()
    _check(lib().nc_param_count(ctypes.byref(cfg), ctypes.byref(n)), "nc_param_count")
    return n.value


def nc_param_layout(cfg):
    n = _I32()
    _check(lib().nc_param_layout(ctypes.byref(cfg), None, 0, ctypes.byref(n)), "nc_param_layout")
    arr = (NcTensorInfo * n.value)()
    _check(lib().nc_param_layout(ctypes.byref(cfg), arr, n.value, ctypes.byref(n)), "nc_param_layout")
    return [(t.name.decode(), int(t.offset), int(t.rows), int(t.cols)) for t in arr]


def nc_workspace_bytes(cfg, with_backward=True) -> int:
    n = _U64()
    _check(lib().nc_workspace_bytes(ctypes.byref(cfg), int(with_backward), ctypes.byref(n)),
           "nc_workspace_bytes")
    return n.value


def nc_workspace_pieces(cfg, with_backward=True):
    """[(name, byte offset, bytes)] of the workspace plan, in address order."""
    n = _I32()
    _check(lib().nc_workspace_pieces(ctypes.byref(cfg), int(with_backward), None, 0, ctypes.byref(n)),
           "nc_workspace_pieces")
    arr = (NcWsPiece * n.value)()
    _check(lib().nc_workspace_pieces(ctypes.byref(cfg), int(with_backward), arr, n.value,
                                     ctypes.byref(n)), "nc_workspace_pieces")
    return [(p.name.decode(), int(p.offset), int(p.bytes)) for p in arr]


def nc_token_losses_offset(cfg, with_backward=True) -> int:
    n = _U64()
    _check(lib().nc_token_losses_offset(ctypes.byref(cfg), int(with_backward), ctypes.byref(n)),
           "nc_token_losses_offset")
    return n.value


def nc_status_string(code) -> str:
    return lib().nc_status_string(code).decode()


# ---------------------------------------------------------------- device calls

def nc_init_params(seed, cfg, params, stream=None):
    _check(lib().nc_init_params(seed, ctypes.byref(cfg), _ptr(params), _stream(stream)),
           "nc_init_params")


def nc_forward_loss(cfg, params, tokens, targets, ws, loss, stream=None):
    _check(lib().nc_forward_loss(ctypes.byref(cfg), _ptr(params), _ptr(tokens), _ptr(targets),
                                 _ptr(ws), ws.numel() * ws.element_size(), _ptr(loss),
                                 _stream(stream)), "nc_forward_loss")


def nc_forward_backward(cfg, params, tokens, targets, grads, ws, loss, stream=None):
    _check(lib().nc_forward_backward(ctypes.byref(cfg), _ptr(params), _ptr(tokens), _ptr(targets),
                                     _ptr(grads), _ptr(ws), ws.numel() * ws.element_size(),
                                     _ptr(loss), _stream(stream)), "nc_forward_backward")


def nc_forward_backward_accumulate(cfg, params, tokens, targets, grads, ws, loss, stream=None):
    _check(lib().nc_forward_backward_accumulate(ctypes.byref(cfg), _ptr(params), _ptr(tokens),
                                                _ptr(targets), _ptr(grads), _ptr(ws),
                                                ws.numel() * ws.element_size(), _ptr(loss),
                                                _stream(stream)), "nc_forward_backward_accumulate")


def nc_optimizer_state_bytes(cfg) -> int:
    n = _U64()
    _check(lib().nc_optimizer_state_bytes(ctypes.byref(cfg), ctypes.byref(n)), "nc_optimizer_state_bytes")
    return n.value


def nc_optimizer_workspace_bytes(cfg) -> int:
    n = _U64()
    _check(lib().nc_optimizer_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)),
           "nc_optimizer_workspace_bytes")
    return n.value


def nc_optim_config(lr_adamw, beta1, beta2, eps, wd_adamw, lr_muon, momentum, wd_muon,
                    max_grad_norm, ns_steps, step) -> NcOptimConfig:
    return NcOptimConfig(lr_adamw, beta1, beta2, eps, wd_adamw, lr_muon, momentum, wd_muon,
                         max_grad_norm, ns_steps, step)


def nc_optimizer_step(cfg, optim, params, grads, state, ows, grad_norm, stream=None):
    _check(lib().nc_optimizer_step(ctypes.byref(cfg), ctypes.byref(optim), _ptr(params), _ptr(grads),
                                   _ptr(state), _ptr(ows), ows.numel() * ows.element_size(),
                                   _ptr(grad_norm), _stream(stream)), "nc_optimizer_step")


def nc_eval_bpb(cfg, params, tokens, targets, token_bytes, ws, loss, bpb, stream=None):
    _check(lib().nc_eval_bpb(ctypes.byref(cfg), _ptr(params), _ptr(tokens), _ptr(targets), _ptr(token_bytes),
                             _ptr(ws), ws.numel() * ws.element_size(), _ptr(loss), _ptr(bpb),
                             _stream(stream)), "nc_eval_bpb")


def nc_kv_cache_bytes(cfg, max_seq) -> int:
    n = _U64()
    _check(lib().nc_kv_cache_bytes(ctypes.byref(cfg), max_seq, ctypes.byref(n)), "nc_kv_cache_bytes")
    return n.value


def nc_infer_workspace_bytes(cfg, max_seq) -> int:
    n = _U64()
    _check(lib().nc_infer_workspace_bytes(ctypes.byref(cfg), max_seq, ctypes.byref(n)),
           "nc_infer_workspace_bytes")
    return n.value


def nc_prefill(cfg, params, tokens, T0, kv, max_seq, ws, logits, stream=None):
    _check(lib().nc_prefill(ctypes.byref(cfg), _ptr(params), _ptr(tokens), T0, _ptr(kv), max_seq,
                            _ptr(ws), ws.numel() * ws.element_size(), _ptr(logits), _stream(stream)),
           "nc_prefill")


def nc_decode_step(cfg, params, tokens, pos, kv, max_seq, ws, logits, stream=None):
    _check(lib().nc_decode_step(ctypes.byref(cfg), _ptr(params), _ptr(tokens), pos, _ptr(kv), max_seq,
                                _ptr(ws), ws.numel() * ws.element_size(), _ptr(logits),
                                _stream(stream)), "nc_decode_step")


def nc_read_device_status(ws, stream=None) -> int:
    f = ctypes.c_uint32()
    _check(lib().nc_read_device_status(_ptr(ws), ctypes.byref(f), _stream(stream)),
           "nc_read_device_status")
    return f.value


def nc_op_gemm(dtype, a_kcontig, b_kcontig, epilogue, A, B, C, C2, M, N, K, lda, ldb, ldc,
               stream=None):
    _check(lib().nc_op_gemm(_dt(dtype), int(a_kcontig), int(b_kcontig), epilogue, _ptr(A), _ptr(B),
                            _ptr(C), _ptr(C2), M, N, K, lda, ldb, ldc, _stream(stream)), "nc_op_gemm")


def nc_op_few_rows_scratch_bytes(M, N, K, splits=0) -> int:
    n = _U64()
    _check(lib().nc_op_few_rows_scratch_bytes(M, N, K, splits, ctypes.byref(n)),
           "nc_op_few_rows_scratch_bytes")
    return n.value


def nc_op_few_rows_gemm(epilogue, W, ldw, X, ldx, C, ldc, M, N, K, scratch, cap=0.0, ssq_in=None,
                        eps=0.0, xb=None, ssq_out=None, splits=0, ntile=0, stream=None):
    _check(lib().nc_op_few_rows_gemm(epilogue, _ptr(W), ldw, _ptr(X), ldx, _ptr(C), ldc, M, N, K, cap,
                                     _ptr(ssq_in), eps, _ptr(xb), _ptr(ssq_out), splits, ntile,
                                     _ptr(scratch),
                                     scratch.numel() * scratch.element_size(), _stream(stream)),
           "nc_op_few_rows_gemm")


def nc_op_decode_attn(dtype, qkv, ldq, B, H, cache, max_seq, pos, part, o, ldo, stream=None):
    _check(lib().nc_op_decode_attn(_dt(dtype), _ptr(qkv), ldq, B, H, _ptr(cache), max_seq, pos,
                                   _ptr(part), _ptr(o), ldo, _stream(stream)), "nc_op_decode_attn")


def nc_op_gemm_axpby(dtype, a_kcontig, b_kcontig, out_f32, A, B, C, C2, M, N, K, lda, ldb, ldc, alpha,
                     beta, batch=1, sa=0, sb=0, sc=0, tile=0, stream=None):
    _check(lib().nc_op_gemm_axpby(_dt(dtype), int(a_kcontig), int(b_kcontig), int(out_f32), _ptr(A), _ptr(B),
                                  _ptr(C), _ptr(C2), M, N, K, lda, ldb, ldc, alpha, beta, batch, sa, sb,
                                  sc, tile, _stream(stream)), "nc_op_gemm_axpby")


def nc_op_wgrad(dtype, X1, X2, dW, partial, M, N1, N2, splits, stream=None):
    _check(lib().nc_op_wgrad(_dt(dtype), _ptr(X1), _ptr(X2), _ptr(dW), _ptr(partial), M, N1, N2,
                             splits, _stream(stream)), "nc_op_wgrad")


def nc_op_transpose(dtype, inp, R, C, ld_in, out, ld_out, stream=None):
    _check(lib().nc_op_transpose(_dt(dtype), _ptr(inp), R, C, ld_in, _ptr(out), ld_out,
                                 _stream(stream)), "nc_op_transpose")


def nc_op_rmsnorm_fwd(dtype, x, M, d, eps, y, rinv, stream=None):
    _check(lib().nc_op_rmsnorm_fwd(_dt(dtype), _ptr(x), M, d, eps, _ptr(y), _ptr(rinv),
                                   _stream(stream)), "nc_op_rmsnorm_fwd")


def nc_op_rmsnorm_bwd(dtype, dy, y, rinv, M, d, dx, accumulate, g, stream=None):
    _check(lib().nc_op_rmsnorm_bwd(_dt(dtype), _ptr(dy), _ptr(y), _ptr(rinv), M, d, _ptr(dx),
                                   int(accumulate), _ptr(g), _stream(stream)), "nc_op_rmsnorm_bwd")


def nc_op_rope_qknorm_fwd(dtype, qkv, B, T, H, base, eps, rinv_qk, cs, stream=None):
    _check(lib().nc_op_rope_qknorm_fwd(_dt(dtype), _ptr(qkv), B, T, H, base, eps, _ptr(rinv_qk),
                                       _ptr(cs), _stream(stream)), "nc_op_rope_qknorm_fwd")


def nc_op_rope_qknorm_bwd(dtype, dqkv, qkv, B, T, H, rinv_qk, cs, stream=None):
    _check(lib().nc_op_rope_qknorm_bwd(_dt(dtype), _ptr(dqkv), _ptr(qkv), B, T, H, _ptr(rinv_qk),
                                       _ptr(cs), _stream(stream)), "nc_op_rope_qknorm_bwd")


def nc_op_attn_fwd(dtype, qkv, B, T, H, o, lse, stream=None):
    _check(lib().nc_op_attn_fwd(_dt(dtype), _ptr(qkv), B, T, H, _ptr(o), _ptr(lse),
                                _stream(stream)), "nc_op_attn_fwd")


def nc_op_attn_bwd_scratch_bytes(B, T) -> int:
    return int(lib().nc_op_attn_bwd_scratch_bytes(B, T))


def nc_op_attn_bwd(dtype, qkv, o, dout, lse, delta, B, T, H, dqkv, scratch=None, stream=None):
    """scratch: a device buffer of nc_op_attn_bwd_scratch_bytes(B, T) bytes
    (allocated here through torch when not given; that size is 0, and the
    pointer null, when T <= 2048)."""
    if scratch is None:
        import torch
        scratch = torch.empty(nc_op_attn_bwd_scratch_bytes(B, T), dtype=torch.uint8, device="cuda")
    _check(lib().nc_op_attn_bwd(_dt(dtype), _ptr(qkv), _ptr(o), _ptr(dout), _ptr(lse), _ptr(delta),
                                B, T, H, _ptr(dqkv), _ptr(scratch), _stream(stream)), "nc_op_attn_bwd")


def nc_op_attn_bwd_ds_bytes(dtype, B, T, H) -> int:
    return int(lib().nc_op_attn_bwd_ds_bytes(_dt(dtype), B, T, H))


def nc_op_attn_bwd_stored_ds(dtype, qkv, o, dout, lse, delta, B, T, H, dqkv, scratch=None, ds=None,
                             stream=None):
    """scratch as for nc_op_attn_bwd; ds: a device buffer of nc_op_attn_bwd_ds_bytes
    bytes (allocated here when omitted)."""
    import torch
    if scratch is None and nc_op_attn_bwd_scratch_bytes(B, T) > 0:
        scratch = torch.empty(nc_op_attn_bwd_scratch_bytes(B, T), dtype=torch.uint8, device="cuda")
    if ds is None:
        ds = torch.empty(nc_op_attn_bwd_ds_bytes(dtype, B, T, H), dtype=torch.uint8, device="cuda")
    _check(lib().nc_op_attn_bwd_stored_ds(_dt(dtype), _ptr(qkv), _ptr(o), _ptr(dout), _ptr(lse), _ptr(delta),
                                          B, T, H, _ptr(dqkv), _ptr(scratch), _ptr(ds), _stream(stream)),
           "nc_op_attn_bwd_stored_ds")


def nc_op_attn_bwd_noalloc(dtype, qkv, o, dout, lse, B, T, H, dqkv, stream=None):
    """nc_op_attn_bwd with the library's fixed per-device scratch (no caller
    buffers, no allocation)."""
    _check(lib().nc_op_attn_bwd_noalloc(_dt(dtype), _ptr(qkv), _ptr(o), _ptr(dout), _ptr(lse),
                                        B, T, H, _ptr(dqkv), _stream(stream)),
           "nc_op_attn_bwd_noalloc")


def nc_op_softcap_ce(dtype, logits, targets, R, V, cap, w, loss_rows, dlogits, status, stream=None):
    _check(lib().nc_op_softcap_ce(_dt(dtype), _ptr(logits), _ptr(targets), R, V, cap, w,
                                  _ptr(loss_rows), _ptr(dlogits), _ptr(status), _stream(stream)),
           "nc_op_softcap_ce")


# ---------------------------------------------------------------- buffers

class Decoder:
    """Device buffers for KV-cache inference with ``cfg.batch`` sequences of
    up to ``max_seq`` positions: the cache, scratch and the [batch, V] fp32
    logits. ``params`` is a parameter buffer in the training layout (for
    example a Step's)."""

    def __init__(self, cfg: NcConfig, params, max_seq: int, device="cuda"):
        import torch
        self.cfg, self.params, self.max_seq = cfg, params, max_seq
        self.device = torch.device(device)
        self.kv = torch.zeros(nc_kv_cache_bytes(cfg, max_seq), dtype=torch.uint8, device=self.device)
        self.ws = torch.empty(nc_infer_workspace_bytes(cfg, max_seq), dtype=torch.uint8,
                              device=self.device)
        self.logits = torch.zeros(cfg.batch, cfg.vocab_size, dtype=torch.float32, device=self.device)
        self.pos = 0

    def prefill(self, tokens):
        """tokens: int32 device tensor [batch, T0]; returns the logits of the
        last prompt position."""
        T0 = int(tokens.shape[1])
        nc_prefill(self.cfg, self.params, tokens, T0, self.kv, self.max_seq, self.ws, self.logits)
        self.pos = T0
        return self.logits

    def step(self, tokens):
        """tokens: int32 device tensor [batch] at the next position."""
        nc_decode_step(self.cfg, self.params, tokens, self.pos, self.kv, self.max_seq, self.ws,
                       self.logits)
        self.pos += 1
        return self.logits

    def status(self):
        return nc_read_device_status(self.ws)


class Step:
    """Owns the torch-allocated device buffers of one training-step shape and
    calls the library on them. ``params`` holds nc_param_count elements of the
    config's dtype (bf16 as torch.bfloat16), ``grads`` the fp32 gradient."""

    def __init__(self, cfg: NcConfig, device="cuda", with_backward=True):
        import torch
        self.cfg = cfg
        self.device = torch.device(device)
        n = nc_param_count(cfg)
        pdt = torch.bfloat16 if cfg.dtype == NC_BF16 else torch.float32
        self.params = torch.zeros(n, dtype=pdt, device=self.device)
        self.grads = torch.zeros(n, dtype=torch.float32, device=self.device) if with_backward else None
        self.ws = torch.empty(nc_workspace_bytes(cfg, with_backward), dtype=torch.uint8,
                              device=self.device)
        self.loss = torch.zeros(1, dtype=torch.float32, device=self.device)
        self.with_backward = with_backward
        self.layout = nc_param_layout(cfg)

    def init(self, seed):
        nc_init_params(seed, self.cfg, self.params)

    def forward_loss(self, tokens, targets):
        nc_forward_loss(self.cfg, self.params, tokens, targets, self.ws, self.loss)
        return self.loss

    def forward_backward(self, tokens, targets):
        nc_forward_backward(self.cfg, self.params, tokens, targets, self.grads, self.ws, self.loss)
        return self.loss

    def forward_backward_accumulate(self, tokens, targets):
        nc_forward_backward_accumulate(self.cfg, self.params, tokens, targets, self.grads, self.ws,
                                       self.loss)
        return self.loss

    def eval_bpb(self, tokens, targets, token_bytes):
        """Bits per byte of the batch: a float64 device tensor (nats, bytes,
        bits per byte); the mean loss lands in ``loss``."""
        import torch
        if getattr(self, "bpb", None) is None:
            self.bpb = torch.zeros(3, dtype=torch.float64, device=self.device)
        nc_eval_bpb(self.cfg, self.params, tokens, targets, token_bytes, self.ws, self.loss, self.bpb)
        return self.bpb

    def optimizer_step(self, optim: NcOptimConfig):
        """One optimizer step on params from grads; optimizer state and
        scratch are allocated (zeroed) on first use. Returns the pre-clip
        gradient norm as a one-element device tensor."""
        import torch
        if getattr(self, "opt_state", None) is None:
            self.opt_state = torch.zeros(nc_optimizer_state_bytes(self.cfg) // 4, dtype=torch.float32,
                                         device=self.device)
            self.opt_ws = torch.empty(nc_optimizer_workspace_bytes(self.cfg), dtype=torch.uint8,
                                      device=self.device)
            self.grad_norm = torch.zeros(1, dtype=torch.float32, device=self.device)
        nc_optimizer_step(self.cfg, optim, self.params, self.grads, self.opt_state, self.opt_ws,
                          self.grad_norm)
        return self.grad_norm

    def token_losses(self):
        import torch
        off = nc_token_losses_offset(self.cfg, self.with_backward)
        M = self.cfg.batch * self.cfg.seq_len
        return self.ws[off:off + 4 * M].view(torch.float32).view(self.cfg.batch, self.cfg.seq_len)

    def status(self):
        return nc_read_device_status(self.ws)

    def tensor(self, buf, name):
        for n, off, r, c in self.layout:
            if n == name:
                return buf[off:off + r * c].view(r, c)
        raise KeyError(name)
