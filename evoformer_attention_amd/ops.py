"""Thin torch-tensor binding over libevoattn.so (include/evo_attn.h).

Each function has the name of the C entry point it calls and does argument
marshalling only: shape/dtype/device checks, output allocation through
torch, the data pointers and torch's current HIP stream.  Every step of the
computation runs in the library's kernels.  A missing library is an error
(there is no fallback), and a non-OK status raises EvoAttnError with the
library's message.
"""
import ctypes
import os

import torch

__all__ = ["EvoAttnError", "lib", "evo_abi_version", "evo_attn_fwd",
           "evo_attn_fwd_noalloc", "evo_probe_issue_rate",
           "evo_attn_bwd", "evo_attn_bwd_workspace_bytes",
           "evo_attn_fwd_workspace_bytes", "tri_attn_project",
           "tri_attn_out_project", "tri_attn_module_fwd",
           "tri_attn_workspace_bytes", "tri_attn_proj_bwd_workspace_bytes",
           "tri_attn_out_project_bwd", "tri_attn_project_bwd",
           "tri_attn_bwd_workspace_bytes", "tri_attn_module_bwd",
           "tri_mul_workspace_bytes", "tri_mul_fwd", "pair_transition_fwd",
           "pair_transition_workspace_bytes",
           "outer_product_mean_workspace_bytes", "outer_product_mean_fwd",
           "pair_transition_bwd_workspace_bytes", "pair_transition_bwd",
           "tri_mul_bwd_workspace_bytes", "tri_mul_bwd",
           "outer_product_mean_bwd_workspace_bytes", "outer_product_mean_bwd",
           "LIB_PATH", "EXPORTS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libevoattn.so")

EVO_OK, EVO_EINVAL, EVO_ENOTSUP, EVO_EWORKSPACE, EVO_EHIP, EVO_EINTERNAL = range(6)
EVO_FP32, EVO_BF16 = 0, 1
STATUS_NAMES = {0: "EVO_OK", 1: "EVO_EINVAL", 2: "EVO_ENOTSUP",
                3: "EVO_EWORKSPACE", 4: "EVO_EHIP", 5: "EVO_EINTERNAL"}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t

# Name -> (restype, argtypes), mirroring include/evo_attn.h.
EXPORTS = {
    "evo_abi_version": (_I, []),
    "evo_last_error": (ctypes.c_char_p, []),
    "evo_attn_fwd": (_I, [_I, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P,
                          _P, _I64, _P, _P, _P, _P, _SZ, _P]),
    "evo_attn_fwd_noalloc": (_I, [_I, _I64, _I64, _I64, _I64, _I64, _P, _P, _P,
                                  _P, _P, _I64, _P, _P, _P, _P]),
    "evo_attn_fwd_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I64, _I64]),
    "evo_probe_issue_rate": (_I, [_I, _I, _I, _P, _P]),
    "evo_attn_bwd_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I64, _I64]),
    "evo_attn_bwd": (_I, [_I, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P,
                          _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                          _SZ, _P]),
    "tri_attn_project": (_I, [_I, _I64, _I64, _I64, _I64, _I, _P, _P, _P, _F,
                              _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              _P]),
    "tri_attn_out_project": (_I, [_I, _I64, _I64, _I64, _I64, _I, _P, _P, _P,
                                  _P, _P]),
    "tri_attn_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I64]),
    "tri_attn_module_fwd": (_I, [_I, _I64, _I64, _I64, _I64, _I, _P, _P, _P,
                                 _P, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _P, _SZ, _P]),
    "tri_attn_proj_bwd_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I64]),
    "tri_attn_out_project_bwd": (_I, [_I, _I64, _I64, _I64, _I64, _I, _P, _P,
                                      _P, _P, _P, _P, _P, _SZ, _P]),
    "tri_attn_project_bwd": (_I, [_I, _I64, _I64, _I64, _I64, _I, _P, _P, _P,
                                  _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  _SZ, _P]),
    "tri_attn_bwd_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I64]),
    "tri_attn_module_bwd": (_I, [_I, _I64, _I64, _I64, _I64, _I, _P, _P, _P,
                                 _P, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _SZ, _P]),
    "tri_mul_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64]),
    "tri_mul_fwd": (_I, [_I, _I64, _I64, _I64, _I, _P, _P, _P, _P, _F, _P, _P,
                         _P, _P, _P, _P, _SZ, _P]),
    "pair_transition_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64]),
    "pair_transition_fwd": (_I, [_I, _I64, _I64, _I64, _P, _P, _P, _F, _P, _P,
                                 _P, _P, _P, _SZ, _P]),
    "outer_product_mean_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I64,
                                                 _I64]),
    "pair_transition_bwd_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64]),
    "pair_transition_bwd": (_I, [_I, _I64, _I64, _I64, _P, _P, _P, _F, _P, _P, _P,
                                 _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "outer_product_mean_fwd": (_I, [_I, _I64, _I64, _I64, _I64, _I64, _P, _P,
                                    _P, _F, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "tri_mul_bwd_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64]),
    "outer_product_mean_bwd_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I64, _I64]),
    "outer_product_mean_bwd": (_I, [_I, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _F, _P,
                                    _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "tri_mul_bwd": (_I, [_I, _I64, _I64, _I64, _I, _P, _P, _P, _P, _F, _P, _P,
                         _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
}


class EvoAttnError(RuntimeError):
    def __init__(self, fn, status, message):
        self.status = status
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {message}")


_lib = None


def lib():
    """The loaded library (ctypes.CDLL) with prototypes set."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m evoformer_attention_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(fn, status):
    if status != EVO_OK:
        msg = lib().evo_last_error().decode(errors="replace")
        raise EvoAttnError(fn, status, msg)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return EVO_BF16
    if t.dtype == torch.float32:
        return EVO_FP32
    raise EvoAttnError("binding", EVO_ENOTSUP, f"dtype {t.dtype} not supported")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_meta(name, t, dtype=None, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise EvoAttnError("binding", EVO_EINVAL, f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise EvoAttnError("binding", EVO_EINVAL,
                           f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise EvoAttnError("binding", EVO_EINVAL,
                           f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_dev(name, t):
    if t is None:
        return
    if not t.is_cuda:
        raise EvoAttnError("binding", EVO_EINVAL, f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise EvoAttnError("binding", EVO_EINVAL, f"{name} must be contiguous")


def _dev_tensor(name, t, dtype=None, shape=None):
    """Check one tensor argument: dtype and shape, then device and layout."""
    _check_meta(name, t, dtype, shape)
    _check_dev(name, t)
    return t


def _dev_tensors(specs):
    """Check (name, tensor, dtype, shape) arguments: every dtype and shape
    first, so that a mismatch is reported as such whatever the devices, then
    every device and layout."""
    for name, t, dtype, shape in specs:
        _check_meta(name, t, dtype, shape)
    for name, t, _, _ in specs:
        _check_dev(name, t)


def _pair_rep(name, z):
    """z [N, N, CZ] -> (N, CZ)."""
    if not isinstance(z, torch.Tensor) or z.dim() != 3 or z.shape[0] != z.shape[1]:
        raise EvoAttnError("binding", EVO_EINVAL,
                           f"{name} must be [N, N, c] (got "
                           f"{tuple(z.shape) if isinstance(z, torch.Tensor) else type(z)})")
    return z.shape[0], z.shape[2]


def evo_abi_version():
    return lib().evo_abi_version()


def evo_attn_fwd_workspace_bytes(dtype, B, R, N, H, C):
    code = EVO_BF16 if dtype == torch.bfloat16 else EVO_FP32
    return lib().evo_attn_fwd_workspace_bytes(code, B, R, N, H, C)


def evo_attn_fwd(q, k, v, gate=None, key_mask=None, bias=None, out=None,
                 want_lse=False, workspace=None):
    """Forward of biased gated attention.  q, k, v, gate: [B,R,N,H,C];
    key_mask: uint8 [B,1,N] or [B,R,N]; bias: [B,H,N,N].  Returns out, or
    (out, lse) with lse [B,R,H,N] fp32 when want_lse.  `workspace` (uint8
    device tensor) is allocated here when not given."""
    _dev_tensor("q", q)
    B, R, N, H, C = q.shape
    dt = q.dtype
    _dev_tensor("k", k, dt, q.shape)
    _dev_tensor("v", v, dt, q.shape)
    _dev_tensor("gate", gate, dt, q.shape)
    _dev_tensor("bias", bias, dt, (B, H, N, N))
    mask_rows = 0
    if key_mask is not None:
        _dev_tensor("key_mask", key_mask, torch.uint8)
        if key_mask.dim() != 3 or key_mask.shape[0] != B or key_mask.shape[2] != N:
            raise EvoAttnError("binding", EVO_EINVAL,
                               f"key_mask has shape {tuple(key_mask.shape)}")
        mask_rows = key_mask.shape[1]
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor("out", out, dt, q.shape)
    lse = torch.empty((B, R, H, N), dtype=torch.float32, device=q.device) if want_lse else None
    if workspace is None and (bias is not None or key_mask is not None):
        need = evo_attn_fwd_workspace_bytes(dt, B, R, N, H, C)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().evo_attn_fwd(_dtype_code(q), B, R, N, H, C, _ptr(q), _ptr(k),
                            _ptr(v), _ptr(gate), _ptr(key_mask), mask_rows,
                            _ptr(bias), _ptr(out), _ptr(lse), _ptr(workspace),
                            ws_bytes, _stream(q.device))
    _check("evo_attn_fwd", st)
    return (out, lse) if want_lse else out


def evo_attn_fwd_noalloc(q, k, v, gate=None, key_mask=None, bias=None, out=None,
                         lse=None):
    """evo_attn_fwd through the allocation-free entry point: the library uses
    its static scratch instead of a workspace.  `out` (and `lse` [B,R,H,N]
    fp32, optional) may be passed in; whatever is not given is allocated here
    by torch, not by the library.  Returns out, or (out, lse) when lse is
    given."""
    _dev_tensor("q", q)
    B, R, N, H, C = q.shape
    dt = q.dtype
    _dev_tensor("k", k, dt, q.shape)
    _dev_tensor("v", v, dt, q.shape)
    _dev_tensor("gate", gate, dt, q.shape)
    _dev_tensor("bias", bias, dt, (B, H, N, N))
    mask_rows = 0
    if key_mask is not None:
        _dev_tensor("key_mask", key_mask, torch.uint8)
        if key_mask.dim() != 3 or key_mask.shape[0] != B or key_mask.shape[2] != N:
            raise EvoAttnError("binding", EVO_EINVAL,
                               f"key_mask has shape {tuple(key_mask.shape)}")
        mask_rows = key_mask.shape[1]
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor("out", out, dt, q.shape)
    _dev_tensor("lse", lse, torch.float32, (B, R, H, N))
    st = lib().evo_attn_fwd_noalloc(_dtype_code(q), B, R, N, H, C, _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(gate), _ptr(key_mask), mask_rows,
                                    _ptr(bias), _ptr(out), _ptr(lse), _stream(q.device))
    _check("evo_attn_fwd_noalloc", st)
    return (out, lse) if lse is not None else out


def evo_probe_issue_rate(kind, waves_per_simd, iters, out):
    """Launch the library's issue-rate probe (kind 0 exp, 1 fma, 2 bf16
    MFMA) on torch's current stream; `out` is a float32 device tensor of at
    least 65536 * waves_per_simd elements."""
    _dev_tensor("out", out, torch.float32)
    if out.numel() < 65536 * waves_per_simd:
        raise EvoAttnError("binding", EVO_EINVAL, "out too small")
    st = lib().evo_probe_issue_rate(int(kind), int(waves_per_simd), int(iters), _ptr(out),
                                    _stream(out.device))
    _check("evo_probe_issue_rate", st)


def evo_attn_bwd_workspace_bytes(dtype, B, R, N, H, C):
    code = EVO_BF16 if dtype == torch.bfloat16 else EVO_FP32
    return lib().evo_attn_bwd_workspace_bytes(code, B, R, N, H, C)


def evo_attn_bwd(q, k, v, gate, key_mask, bias, out, lse, dout,
                 want_dbias=True, workspace=None):
    """Backward of evo_attn_fwd.  Returns dq, dk, dv, dgate (None without a
    gate) and dbias ([B,H,N,N] fp32, summed over rows; None unless
    want_dbias)."""
    _dev_tensor("q", q)
    B, R, N, H, C = q.shape
    dt = q.dtype
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        _dev_tensor(name, t, dt, q.shape)
    _dev_tensor("gate", gate, dt, q.shape)
    _dev_tensor("bias", bias, dt, (B, H, N, N))
    _dev_tensor("lse", lse, torch.float32, (B, R, H, N))
    mask_rows = 0
    if key_mask is not None:
        _dev_tensor("key_mask", key_mask, torch.uint8)
        if key_mask.dim() != 3 or key_mask.shape[0] != B or key_mask.shape[2] != N:
            raise EvoAttnError("binding", EVO_EINVAL,
                               f"key_mask has shape {tuple(key_mask.shape)}")
        mask_rows = key_mask.shape[1]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dg = torch.empty_like(q) if gate is not None else None
    db = (torch.empty((B, H, N, N), dtype=torch.float32, device=q.device)
          if want_dbias else None)
    need = evo_attn_bwd_workspace_bytes(dt, B, R, N, H, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib().evo_attn_bwd(_dtype_code(q), B, R, N, H, C, _ptr(q), _ptr(k),
                            _ptr(v), _ptr(gate), _ptr(key_mask), mask_rows,
                            _ptr(bias), _ptr(out), _ptr(lse), _ptr(dout),
                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db),
                            _ptr(workspace), workspace.numel(),
                            _stream(q.device))
    _check("evo_attn_bwd", st)
    return dq, dk, dv, dg, db


def tri_attn_project(z, ln_w, ln_b, eps, w_q, w_k, w_v, w_g, b_g, w_bias, H,
                     C, ending):
    """LayerNorm + projections.  Returns q, k, v, g [1,N,N,H,C] and bias
    [1,H,N,N] in line layout."""
    N, CZ = _pair_rep("z", z)
    dt = z.dtype
    HC = H * C
    _dev_tensors([("z", z, None, None),
                  ("ln_w", ln_w, dt, (CZ,)),
                  ("ln_b", ln_b, dt, (CZ,)),
                  ("w_q", w_q, dt, (HC, CZ)),
                  ("w_k", w_k, dt, (HC, CZ)),
                  ("w_v", w_v, dt, (HC, CZ)),
                  ("w_g", w_g, dt, (HC, CZ)),
                  ("w_bias", w_bias, dt, (H, CZ)),
                  ("b_g", b_g, dt, (HC,))])
    q = torch.empty((1, N, N, H, C), dtype=dt, device=z.device)
    k, v, g = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    bias = torch.empty((1, H, N, N), dtype=dt, device=z.device)
    st = lib().tri_attn_project(_dtype_code(z), N, CZ, H, C, int(ending),
                                _ptr(z), _ptr(ln_w), _ptr(ln_b), float(eps),
                                _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_g),
                                _ptr(b_g), _ptr(w_bias), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(g), _ptr(bias), _stream(z.device))
    _check("tri_attn_project", st)
    return q, k, v, g, bias


def tri_attn_out_project(o, w_o, b_o, CZ, ending):
    """Output projection of o [1,N,N,H,C] (line layout) -> [N,N,CZ]."""
    _dev_tensor("o", o)
    if o.dim() != 5 or o.shape[0] != 1 or o.shape[1] != o.shape[2]:
        raise EvoAttnError("binding", EVO_EINVAL, f"o must be [1, N, N, H, C] (got {tuple(o.shape)})")
    _, N, _, H, C = o.shape
    _dev_tensor("w_o", w_o, o.dtype, (CZ, H * C))
    _dev_tensor("b_o", b_o, o.dtype, (CZ,))
    out = torch.empty((N, N, CZ), dtype=o.dtype, device=o.device)
    st = lib().tri_attn_out_project(_dtype_code(o), N, CZ, H, C, int(ending),
                                    _ptr(o), _ptr(w_o), _ptr(b_o), _ptr(out),
                                    _stream(o.device))
    _check("tri_attn_out_project", st)
    return out


def tri_attn_workspace_bytes(dtype, N, CZ, H, C):
    code = EVO_BF16 if dtype == torch.bfloat16 else EVO_FP32
    return lib().tri_attn_workspace_bytes(code, N, CZ, H, C)


def tri_attn_module_fwd(z, residue_mask, ln_w, ln_b, eps, w_q, w_k, w_v, w_g,
                        b_g, w_bias, w_o, b_o, H, C, ending, workspace=None,
                        out=None):
    """Whole triangle-attention module forward -> [N,N,CZ] update."""
    N, CZ = _pair_rep("z", z)
    dt = z.dtype
    HC = H * C
    _dev_tensors([("z", z, None, None),
                  ("ln_w", ln_w, dt, (CZ,)),
                  ("ln_b", ln_b, dt, (CZ,)),
                  ("w_q", w_q, dt, (HC, CZ)),
                  ("w_k", w_k, dt, (HC, CZ)),
                  ("w_v", w_v, dt, (HC, CZ)),
                  ("w_g", w_g, dt, (HC, CZ)),
                  ("w_bias", w_bias, dt, (H, CZ)),
                  ("w_o", w_o, dt, (CZ, HC)),
                  ("b_g", b_g, dt, (HC,)),
                  ("b_o", b_o, dt, (CZ,)),
                  ("residue_mask", residue_mask, torch.uint8, (N,))])
    need = tri_attn_workspace_bytes(dt, N, CZ, H, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=z.device)
    if out is None:
        out = torch.empty((N, N, CZ), dtype=dt, device=z.device)
    st = lib().tri_attn_module_fwd(_dtype_code(z), N, CZ, H, C, int(ending),
                                   _ptr(z), _ptr(residue_mask), _ptr(ln_w),
                                   _ptr(ln_b), float(eps), _ptr(w_q),
                                   _ptr(w_k), _ptr(w_v), _ptr(w_g), _ptr(b_g),
                                   _ptr(w_bias), _ptr(w_o), _ptr(b_o),
                                   _ptr(out), _ptr(workspace),
                                   workspace.numel(), _stream(z.device))
    _check("tri_attn_module_fwd", st)
    return out


def _f32(shape, device):
    return torch.empty(shape, dtype=torch.float32, device=device)


def tri_attn_proj_bwd_workspace_bytes(dtype, N, CZ, H, C):
    code = EVO_BF16 if dtype == torch.bfloat16 else EVO_FP32
    return lib().tri_attn_proj_bwd_workspace_bytes(code, N, CZ, H, C)


def tri_attn_bwd_workspace_bytes(dtype, N, CZ, H, C):
    code = EVO_BF16 if dtype == torch.bfloat16 else EVO_FP32
    return lib().tri_attn_bwd_workspace_bytes(code, N, CZ, H, C)


def _workspace(need, device, workspace):
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace


def tri_attn_out_project_bwd(o, w_o, dout, ending, workspace=None):
    """Backward of tri_attn_out_project -> (d_o, dw_o fp32, db_o fp32)."""
    _dev_tensor("o", o)
    if o.dim() != 5 or o.shape[0] != 1 or o.shape[1] != o.shape[2]:
        raise EvoAttnError("binding", EVO_EINVAL, f"o must be [1, N, N, H, C] (got {tuple(o.shape)})")
    _, N, _, H, C = o.shape
    dt = o.dtype
    if not isinstance(w_o, torch.Tensor) or w_o.dim() != 2:
        raise EvoAttnError("binding", EVO_EINVAL, "w_o must be [CZ, H*C]")
    CZ = w_o.shape[0]
    _dev_tensor("w_o", w_o, dt, (CZ, H * C))
    _dev_tensor("dout", dout, dt, (N, N, CZ))
    workspace = _workspace(tri_attn_proj_bwd_workspace_bytes(dt, N, CZ, H, C),
                           o.device, workspace)
    d_o = torch.empty_like(o)
    dw_o = _f32((CZ, H * C), o.device)
    db_o = _f32((CZ,), o.device)
    st = lib().tri_attn_out_project_bwd(
        _dtype_code(o), N, CZ, H, C, int(ending), _ptr(o), _ptr(w_o),
        _ptr(dout), _ptr(d_o), _ptr(dw_o), _ptr(db_o), _ptr(workspace),
        workspace.numel(), _stream(o.device))
    _check("tri_attn_out_project_bwd", st)
    return d_o, dw_o, db_o


_PARAM_GRADS = ("dln_w", "dln_b", "dw_q", "dw_k", "dw_v", "dw_g", "db_g",
                "dw_bias")


def _param_grads(CZ, H, C, device):
    HC = H * C
    shapes = dict(dln_w=(CZ,), dln_b=(CZ,), dw_q=(HC, CZ), dw_k=(HC, CZ),
                  dw_v=(HC, CZ), dw_g=(HC, CZ), db_g=(HC,), dw_bias=(H, CZ))
    return {n: _f32(shapes[n], device) for n in _PARAM_GRADS}


def tri_attn_project_bwd(z, ln_w, ln_b, eps, w_q, w_k, w_v, w_g, w_bias, dq,
                         dk, dv, dg, dbias, H, C, ending, workspace=None):
    """Backward of tri_attn_project -> dict with dz and the fp32 parameter
    gradients (dln_w, dln_b, dw_q, dw_k, dw_v, dw_g, db_g, dw_bias)."""
    N, CZ = _pair_rep("z", z)
    dt = z.dtype
    HC = H * C
    _dev_tensors([("z", z, None, None),
                  ("ln_w", ln_w, dt, (CZ,)),
                  ("ln_b", ln_b, dt, (CZ,)),
                  ("w_q", w_q, dt, (HC, CZ)),
                  ("w_k", w_k, dt, (HC, CZ)),
                  ("w_v", w_v, dt, (HC, CZ)),
                  ("w_g", w_g, dt, (HC, CZ)),
                  ("w_bias", w_bias, dt, (H, CZ)),
                  ("dq", dq, dt, (1, N, N, H, C)),
                  ("dk", dk, dt, (1, N, N, H, C)),
                  ("dv", dv, dt, (1, N, N, H, C)),
                  ("dg", dg, dt, (1, N, N, H, C)),
                  ("dbias", dbias, torch.float32, (1, H, N, N))])
    workspace = _workspace(tri_attn_proj_bwd_workspace_bytes(dt, N, CZ, H, C),
                           z.device, workspace)
    res = _param_grads(CZ, H, C, z.device)
    res["dz"] = torch.empty_like(z)
    st = lib().tri_attn_project_bwd(
        _dtype_code(z), N, CZ, H, C, int(ending), _ptr(z), _ptr(ln_w),
        _ptr(ln_b), float(eps), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_g),
        _ptr(w_bias), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbias),
        _ptr(res["dz"]), *(_ptr(res[n]) for n in _PARAM_GRADS),
        _ptr(workspace), workspace.numel(), _stream(z.device))
    _check("tri_attn_project_bwd", st)
    return res


def tri_attn_module_bwd(z, residue_mask, ln_w, ln_b, eps, w_q, w_k, w_v, w_g,
                        b_g, w_bias, w_o, dout, H, C, ending, workspace=None):
    """Gradients of the module forward -> dict with dz and the fp32
    parameter gradients (those of tri_attn_project_bwd plus dw_o, db_o)."""
    N, CZ = _pair_rep("z", z)
    dt = z.dtype
    HC = H * C
    _dev_tensors([("z", z, None, None),
                  ("ln_w", ln_w, dt, (CZ,)),
                  ("ln_b", ln_b, dt, (CZ,)),
                  ("w_q", w_q, dt, (HC, CZ)),
                  ("w_k", w_k, dt, (HC, CZ)),
                  ("w_v", w_v, dt, (HC, CZ)),
                  ("w_g", w_g, dt, (HC, CZ)),
                  ("b_g", b_g, dt, (HC,)),
                  ("w_bias", w_bias, dt, (H, CZ)),
                  ("w_o", w_o, dt, (CZ, HC)),
                  ("dout", dout, dt, (N, N, CZ)),
                  ("residue_mask", residue_mask, torch.uint8, (N,))])
    workspace = _workspace(tri_attn_bwd_workspace_bytes(dt, N, CZ, H, C),
                           z.device, workspace)
    res = _param_grads(CZ, H, C, z.device)
    res["dz"] = torch.empty_like(z)
    res["dw_o"] = _f32((CZ, H * C), z.device)
    res["db_o"] = _f32((CZ,), z.device)
    st = lib().tri_attn_module_bwd(
        _dtype_code(z), N, CZ, H, C, int(ending), _ptr(z), _ptr(residue_mask),
        _ptr(ln_w), _ptr(ln_b), float(eps), _ptr(w_q), _ptr(w_k), _ptr(w_v),
        _ptr(w_g), _ptr(b_g), _ptr(w_bias), _ptr(w_o), _ptr(dout),
        _ptr(res["dz"]), *(_ptr(res[n]) for n in _PARAM_GRADS),
        _ptr(res["dw_o"]), _ptr(res["db_o"]), _ptr(workspace),
        workspace.numel(), _stream(z.device))
    _check("tri_attn_module_bwd", st)
    return res


def tri_mul_workspace_bytes(dtype, N, CZ, C):
    code = EVO_BF16 if dtype == torch.bfloat16 else EVO_FP32
    return lib().tri_mul_workspace_bytes(code, N, CZ, C)


def tri_mul_fwd(z, residue_mask, ln_w, ln_b, eps, w_a, w_b, w_o, b_o,
                outgoing=True, workspace=None, out=None):
    """Triangular multiplicative update -> [N,N,CZ] update."""
    N, CZ = _pair_rep("z", z)
    dt = z.dtype
    if not isinstance(w_a, torch.Tensor) or w_a.dim() != 2:
        raise EvoAttnError("binding", EVO_EINVAL, "w_a must be [C, CZ]")
    C = w_a.shape[0]
    _dev_tensors([("z", z, None, None),
                  ("ln_w", ln_w, dt, (CZ,)),
                  ("ln_b", ln_b, dt, (CZ,)),
                  ("w_a", w_a, dt, (C, CZ)),
                  ("w_b", w_b, dt, (C, CZ)),
                  ("w_o", w_o, dt, (CZ, C)),
                  ("b_o", b_o, dt, (CZ,)),
                  ("residue_mask", residue_mask, torch.uint8, (N,))])
    workspace = _workspace(tri_mul_workspace_bytes(dt, N, CZ, C), z.device, workspace)
    if out is None:
        out = torch.empty((N, N, CZ), dtype=dt, device=z.device)
    st = lib().tri_mul_fwd(_dtype_code(z), N, CZ, C, int(bool(outgoing)),
                           _ptr(z), _ptr(residue_mask), _ptr(ln_w), _ptr(ln_b),
                           float(eps), _ptr(w_a), _ptr(w_b), _ptr(w_o),
                           _ptr(b_o), _ptr(out), _ptr(workspace),
                           workspace.numel(), _stream(z.device))
    _check("tri_mul_fwd", st)
    return out


def pair_transition_workspace_bytes(dtype, N, CZ, HID):
    code = EVO_BF16 if dtype == torch.bfloat16 else EVO_FP32
    return lib().pair_transition_workspace_bytes(code, N, CZ, HID)


def pair_transition_fwd(z, ln_w, ln_b, eps, w_a, w_b, w_o, out=None,
                        workspace=None):
    """LayerNorm + SwiGLU transition of the pair representation -> [N,N,CZ]."""
    N, CZ = _pair_rep("z", z)
    dt = z.dtype
    if not isinstance(w_a, torch.Tensor) or w_a.dim() != 2:
        raise EvoAttnError("binding", EVO_EINVAL, "w_a must be [HID, CZ]")
    HID = w_a.shape[0]
    _dev_tensors([("z", z, None, None),
                  ("ln_w", ln_w, dt, (CZ,)),
                  ("ln_b", ln_b, dt, (CZ,)),
                  ("w_a", w_a, dt, (HID, CZ)),
                  ("w_b", w_b, dt, (HID, CZ)),
                  ("w_o", w_o, dt, (CZ, HID))])
    workspace = _workspace(pair_transition_workspace_bytes(dt, N, CZ, HID),
                           z.device, workspace)
    if out is None:
        out = torch.empty((N, N, CZ), dtype=dt, device=z.device)
    st = lib().pair_transition_fwd(_dtype_code(z), N, CZ, HID, _ptr(z),
                                   _ptr(ln_w), _ptr(ln_b), float(eps),
                                   _ptr(w_a), _ptr(w_b), _ptr(w_o), _ptr(out),
                                   _ptr(workspace), workspace.numel(),
                                   _stream(z.device))
    _check("pair_transition_fwd", st)
    return out


def outer_product_mean_workspace_bytes(dtype, S, N, CM, C, CZ):
    code = EVO_BF16 if dtype == torch.bfloat16 else EVO_FP32
    return lib().outer_product_mean_workspace_bytes(code, S, N, CM, C, CZ)


def outer_product_mean_fwd(m, ln_w, ln_b, eps, w_a, w_b, w_o, b_o, out=None,
                           workspace=None):
    """Outer product mean of the MSA representation m [S,N,CM] -> [N,N,CZ]."""
    if not isinstance(m, torch.Tensor) or m.dim() != 3:
        raise EvoAttnError("binding", EVO_EINVAL, "m must be [S, N, CM]")
    S, N, CM = m.shape
    dt = m.dtype
    for name, t in (("w_a", w_a), ("w_o", w_o)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise EvoAttnError("binding", EVO_EINVAL, f"{name} must be a matrix")
    C, CZ = w_a.shape[0], w_o.shape[0]
    _dev_tensors([("m", m, None, None),
                  ("ln_w", ln_w, dt, (CM,)),
                  ("ln_b", ln_b, dt, (CM,)),
                  ("w_a", w_a, dt, (C, CM)),
                  ("w_b", w_b, dt, (C, CM)),
                  ("w_o", w_o, dt, (CZ, C * C)),
                  ("b_o", b_o, dt, (CZ,))])
    workspace = _workspace(outer_product_mean_workspace_bytes(dt, S, N, CM, C, CZ),
                           m.device, workspace)
    if out is None:
        out = torch.empty((N, N, CZ), dtype=dt, device=m.device)
    st = lib().outer_product_mean_fwd(_dtype_code(m), S, N, CM, C, CZ, _ptr(m),
                                      _ptr(ln_w), _ptr(ln_b), float(eps),
                                      _ptr(w_a), _ptr(w_b), _ptr(w_o), _ptr(b_o),
                                      _ptr(out), _ptr(workspace),
                                      workspace.numel(), _stream(m.device))
    _check("outer_product_mean_fwd", st)
    return out


def pair_transition_bwd_workspace_bytes(dtype, N, CZ, HID):
    code = EVO_BF16 if dtype == torch.bfloat16 else EVO_FP32
    return lib().pair_transition_bwd_workspace_bytes(code, N, CZ, HID)


def pair_transition_bwd(z, ln_w, ln_b, eps, w_a, w_b, w_o, dout, workspace=None):
    """Backward of pair_transition_fwd -> dict of dz (dtype) and the fp32
    parameter gradients dln_w, dln_b, dw_a, dw_b, dw_o."""
    N, CZ = _pair_rep("z", z)
    dt = z.dtype
    if not isinstance(w_a, torch.Tensor) or w_a.dim() != 2:
        raise EvoAttnError("binding", EVO_EINVAL, "w_a must be [HID, CZ]")
    HID = w_a.shape[0]
    _dev_tensors([("z", z, None, None),
                  ("ln_w", ln_w, dt, (CZ,)),
                  ("ln_b", ln_b, dt, (CZ,)),
                  ("w_a", w_a, dt, (HID, CZ)),
                  ("w_b", w_b, dt, (HID, CZ)),
                  ("w_o", w_o, dt, (CZ, HID)),
                  ("dout", dout, dt, (N, N, CZ))])
    workspace = _workspace(pair_transition_bwd_workspace_bytes(dt, N, CZ, HID),
                           z.device, workspace)
    res = {"dz": torch.empty_like(z)}
    for k, shape in (("dln_w", (CZ,)), ("dln_b", (CZ,)), ("dw_a", (HID, CZ)),
                     ("dw_b", (HID, CZ)), ("dw_o", (CZ, HID))):
        res[k] = torch.empty(shape, dtype=torch.float32, device=z.device)
    st = lib().pair_transition_bwd(_dtype_code(z), N, CZ, HID, _ptr(z), _ptr(ln_w),
                                   _ptr(ln_b), float(eps), _ptr(w_a), _ptr(w_b),
                                   _ptr(w_o), _ptr(dout), _ptr(res["dz"]),
                                   _ptr(res["dln_w"]), _ptr(res["dln_b"]),
                                   _ptr(res["dw_a"]), _ptr(res["dw_b"]),
                                   _ptr(res["dw_o"]), _ptr(workspace),
                                   workspace.numel(), _stream(z.device))
    _check("pair_transition_bwd", st)
    return res


def tri_mul_bwd_workspace_bytes(dtype, N, CZ, C):
    code = EVO_BF16 if dtype == torch.bfloat16 else EVO_FP32
    return lib().tri_mul_bwd_workspace_bytes(code, N, CZ, C)


def tri_mul_bwd(z, residue_mask, ln_w, ln_b, eps, w_a, w_b, w_o, dout,
                outgoing=True, workspace=None):
    """Backward of tri_mul_fwd -> dict of dz (dtype) and the fp32 parameter
    gradients dln_w, dln_b, dw_a, dw_b, dw_o, db_o."""
    N, CZ = _pair_rep("z", z)
    dt = z.dtype
    if not isinstance(w_a, torch.Tensor) or w_a.dim() != 2:
        raise EvoAttnError("binding", EVO_EINVAL, "w_a must be [C, CZ]")
    C = w_a.shape[0]
    _dev_tensors([("z", z, None, None),
                  ("ln_w", ln_w, dt, (CZ,)),
                  ("ln_b", ln_b, dt, (CZ,)),
                  ("w_a", w_a, dt, (C, CZ)),
                  ("w_b", w_b, dt, (C, CZ)),
                  ("w_o", w_o, dt, (CZ, C)),
                  ("dout", dout, dt, (N, N, CZ)),
                  ("residue_mask", residue_mask, torch.uint8, (N,))])
    workspace = _workspace(tri_mul_bwd_workspace_bytes(dt, N, CZ, C), z.device, workspace)
    res = {"dz": torch.empty_like(z)}
    for k, shape in (("dln_w", (CZ,)), ("dln_b", (CZ,)), ("dw_a", (C, CZ)),
                     ("dw_b", (C, CZ)), ("dw_o", (CZ, C)), ("db_o", (CZ,))):
        res[k] = torch.empty(shape, dtype=torch.float32, device=z.device)
    st = lib().tri_mul_bwd(_dtype_code(z), N, CZ, C, int(bool(outgoing)), _ptr(z),
                           _ptr(residue_mask), _ptr(ln_w), _ptr(ln_b), float(eps),
                           _ptr(w_a), _ptr(w_b), _ptr(w_o), _ptr(dout), _ptr(res["dz"]),
                           _ptr(res["dln_w"]), _ptr(res["dln_b"]), _ptr(res["dw_a"]),
                           _ptr(res["dw_b"]), _ptr(res["dw_o"]), _ptr(res["db_o"]),
                           _ptr(workspace), workspace.numel(), _stream(z.device))
    _check("tri_mul_bwd", st)
    return res


def outer_product_mean_bwd_workspace_bytes(dtype, S, N, CM, C, CZ):
    code = EVO_BF16 if dtype == torch.bfloat16 else EVO_FP32
    return lib().outer_product_mean_bwd_workspace_bytes(code, S, N, CM, C, CZ)


def outer_product_mean_bwd(m, ln_w, ln_b, eps, w_a, w_b, w_o, dout, workspace=None):
    """Backward of outer_product_mean_fwd -> dict of dm (dtype) and the fp32
    parameter gradients dln_w, dln_b, dw_a, dw_b, dw_o, db_o."""
    if not isinstance(m, torch.Tensor) or m.dim() != 3:
        raise EvoAttnError("binding", EVO_EINVAL, "m must be [S, N, CM]")
    S, N, CM = m.shape
    dt = m.dtype
    for name, t in (("w_a", w_a), ("w_o", w_o)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise EvoAttnError("binding", EVO_EINVAL, f"{name} must be a matrix")
    C, CZ = w_a.shape[0], w_o.shape[0]
    _dev_tensors([("m", m, None, None),
                  ("ln_w", ln_w, dt, (CM,)),
                  ("ln_b", ln_b, dt, (CM,)),
                  ("w_a", w_a, dt, (C, CM)),
                  ("w_b", w_b, dt, (C, CM)),
                  ("w_o", w_o, dt, (CZ, C * C)),
                  ("dout", dout, dt, (N, N, CZ))])
    workspace = _workspace(outer_product_mean_bwd_workspace_bytes(dt, S, N, CM, C, CZ),
                           m.device, workspace)
    res = {"dm": torch.empty_like(m)}
    for k, shape in (("dln_w", (CM,)), ("dln_b", (CM,)), ("dw_a", (C, CM)),
                     ("dw_b", (C, CM)), ("dw_o", (CZ, C * C)), ("db_o", (CZ,))):
        res[k] = torch.empty(shape, dtype=torch.float32, device=m.device)
    st = lib().outer_product_mean_bwd(_dtype_code(m), S, N, CM, C, CZ, _ptr(m), _ptr(ln_w),
                                      _ptr(ln_b), float(eps), _ptr(w_a), _ptr(w_b),
                                      _ptr(w_o), _ptr(dout), _ptr(res["dm"]),
                                      _ptr(res["dln_w"]), _ptr(res["dln_b"]),
                                      _ptr(res["dw_a"]), _ptr(res["dw_b"]),
                                      _ptr(res["dw_o"]), _ptr(res["db_o"]), _ptr(workspace),
                                      workspace.numel(), _stream(m.device))
    _check("outer_product_mean_bwd", st)
    return res
