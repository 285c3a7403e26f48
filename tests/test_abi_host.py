"""C-ABI checks that need no GPU: the library loads, exports every entry
point the header declares, and rejects bad arguments with the documented
status codes before touching the device.  Pointers passed here are never
dereferenced: every call below fails validation (or takes the injected
launch failure) before any HIP call."""
import ctypes
import os
import re
import threading

import pytest
import torch

from evoformer_attention_amd import ops

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "evo_attn.h")
FAKE = 0x10000          # aligned, never dereferenced
MISALIGNED = 0x10004
L = None


@pytest.fixture(autouse=True)
def lib():
    global L
    L = ops.lib()
    yield L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"if", "defined"})


def test_header_functions_are_exported():
    names = declared_functions()
    assert set(names) == set(ops.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_abi_version():
    assert L.evo_abi_version() == 1


def err():
    return L.evo_last_error().decode()


def fwd(**kw):
    a = dict(dt=1, B=1, R=2, N=8, H=2, C=32, q=FAKE, k=FAKE, v=FAKE, g=None,
             m=None, mr=1, bias=None, out=FAKE, lse=None, ws=None, wsb=0)
    a.update(kw)
    return L.evo_attn_fwd(a["dt"], a["B"], a["R"], a["N"], a["H"], a["C"],
                          a["q"], a["k"], a["v"], a["g"], a["m"], a["mr"],
                          a["bias"], a["out"], a["lse"], a["ws"], a["wsb"],
                          None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(C=16), ops.EVO_ENOTSUP, "head dimension"),
    (dict(C=64), ops.EVO_ENOTSUP, "head dimension"),
    (dict(N=0), ops.EVO_EINVAL, "positive"),
    (dict(B=-1), ops.EVO_EINVAL, "positive"),
    (dict(q=None), ops.EVO_EINVAL, "'q' is NULL"),
    (dict(out=None), ops.EVO_EINVAL, "'out' is NULL"),
    (dict(k=MISALIGNED), ops.EVO_ENOTSUP, "'k' is not 16-byte aligned"),
    (dict(m=FAKE, mr=3), ops.EVO_EINVAL, "mask_rows"),
    (dict(bias=FAKE), ops.EVO_EWORKSPACE, "workspace"),
    (dict(m=FAKE, ws=FAKE, wsb=8), ops.EVO_EWORKSPACE, "workspace"),
    (dict(dt=7), ops.EVO_ENOTSUP, "dtype"),
])
def test_fwd_validation(kw, status, needle):
    assert fwd(**kw) == status
    assert needle in err()


def test_fault_injection_reports_hip_error(monkeypatch):
    monkeypatch.setenv("EVO_FAULT_INJECT", "launch")
    assert fwd() == ops.EVO_EHIP
    assert "injected" in err()


def test_last_error_is_thread_local():
    assert fwd(C=16) == ops.EVO_ENOTSUP
    seen = {}

    def other():
        seen["msg"] = L.evo_last_error().decode()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "head dimension" in err()


def test_workspace_queries():
    assert L.evo_attn_fwd_workspace_bytes(1, 1, 768, 768, 4, 32) == 4 * 768 * 768 * 2
    assert L.evo_attn_fwd_workspace_bytes(0, 1, 768, 768, 4, 32) == 4 * 768 * 768 * 4
    assert L.evo_attn_fwd_workspace_bytes(1, 1, 2, 8, 2, 16) == 0
    n = L.evo_attn_bwd_workspace_bytes(1, 1, 512, 512, 4, 32)
    assert n >= 512 * 512 * 128 * 2  # dO = dOut * sigmoid(G) alone
    assert n < 3 * 512 * 512 * 128 * 2  # O(N^2 (H C + H)), no per-line N x N state
    assert L.evo_attn_bwd_workspace_bytes(1, 1, 512, 512, 4, 16) == 0
    assert L.evo_attn_bwd_workspace_bytes(1, 1, 1, 70000, 1, 32) == 0
    t = L.tri_attn_workspace_bytes(1, 768, 128, 4, 32)
    assert t >= 5 * 768 * 768 * 128 * 2 + 4 * 768 * 768 * 2
    assert L.tri_attn_workspace_bytes(1, 768, 100, 4, 32) == 0


def bwd(**kw):
    a = dict(dt=1, B=1, R=2, N=8, H=2, C=32, q=FAKE, k=FAKE, v=FAKE, g=None,
             m=None, mr=1, bias=None, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE,
             dk=FAKE, dv=FAKE, dg=None, db=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return L.evo_attn_bwd(a["dt"], a["B"], a["R"], a["N"], a["H"], a["C"],
                          a["q"], a["k"], a["v"], a["g"], a["m"], a["mr"],
                          a["bias"], a["out"], a["lse"], a["dout"], a["dq"],
                          a["dk"], a["dv"], a["dg"], a["db"], a["ws"],
                          a["wsb"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(g=FAKE), ops.EVO_EINVAL, "dgate"),
    (dict(dg=FAKE), ops.EVO_EINVAL, "dgate"),
    (dict(lse=None), ops.EVO_EINVAL, "'lse' is NULL"),
    (dict(ws=None), ops.EVO_EWORKSPACE, "workspace"),
    (dict(wsb=16), ops.EVO_EWORKSPACE, "workspace"),
    (dict(N=70000, R=1, H=1), ops.EVO_ENOTSUP, "N <= 65536"),
])
def test_bwd_validation(kw, status, needle):
    assert bwd(**kw) == status
    assert needle in err()


def test_module_validation():
    args = [1, 64, 128, 4, 32, 2] + [FAKE] * 2 + [FAKE, FAKE, 1e-5] + \
        [FAKE] * 4 + [None, FAKE, FAKE, None, FAKE, FAKE, 1 << 40, None]
    assert L.tri_attn_module_fwd(*args) == ops.EVO_EINVAL  # ending = 2
    assert "ending" in err()
    args[5] = 1
    args[21] = 10
    assert L.tri_attn_module_fwd(*args) == ops.EVO_EWORKSPACE
    args[2] = 100
    assert L.tri_attn_module_fwd(*args) == ops.EVO_ENOTSUP
    assert "CZ" in err()
    assert L.tri_attn_project(1, 64, 128, 4, 32, 0, FAKE, FAKE, FAKE, -1.0,
                              FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                              FAKE, FAKE, FAKE, None) == ops.EVO_EINVAL
    assert "ln_eps" in err()
    assert L.tri_attn_out_project(1, 64, 128, 4, 32, 0, None, FAKE, None,
                                  FAKE, None) == ops.EVO_EINVAL


def test_binding_rejects_host_tensors_and_raises():
    x = torch.zeros(1, 1, 4, 1, 32)
    with pytest.raises(ops.EvoAttnError, match="GPU tensor"):
        ops.evo_attn_fwd(x, x, x)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(ops, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(ops, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        ops.lib()


def test_module_bwd_workspace_queries():
    p = L.tri_attn_proj_bwd_workspace_bytes(1, 768, 128, 4, 32)
    # chunk partials of the weight gradients only: a fixed number of chunks,
    # so the size does not grow with N
    assert 0 < p < 128 << 20
    assert L.tri_attn_proj_bwd_workspace_bytes(1, 384, 128, 4, 32) == p
    m = L.tri_attn_bwd_workspace_bytes(1, 768, 128, 4, 32)
    # ten activation-sized tensors (q k v g o and their gradients) and more
    assert m >= 10 * 768 * 768 * 128 * 2 + p
    assert m < 12 * 768 * 768 * 128 * 2 + 64 << 20
    assert L.tri_attn_bwd_workspace_bytes(1, 64, 256, 4, 32) == 0   # CZ > 128
    assert L.tri_attn_proj_bwd_workspace_bytes(1, 64, 128, 8, 32) == 0  # H*C > 128
    assert L.tri_attn_bwd_workspace_bytes(1, 64, 96, 2, 16) == 0   # C != 32


def module_bwd(**kw):
    a = dict(dt=1, N=64, CZ=128, H=4, C=32, ending=0, eps=1e-5, ws=FAKE,
             wsb=1 << 40, mask=None, dz=FAKE)
    a.update(kw)
    return L.tri_attn_module_bwd(
        a["dt"], a["N"], a["CZ"], a["H"], a["C"], a["ending"], FAKE, a["mask"],
        FAKE, FAKE, a["eps"], FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
        a["dz"], *([FAKE] * 10), a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(ending=2), ops.EVO_EINVAL, "ending"),
    (dict(eps=0.0), ops.EVO_EINVAL, "ln_eps"),
    (dict(dz=None), ops.EVO_EINVAL, "'dz' is NULL"),
    (dict(dz=MISALIGNED), ops.EVO_ENOTSUP, "aligned"),
    (dict(wsb=10), ops.EVO_EWORKSPACE, "workspace"),
    (dict(CZ=256), ops.EVO_ENOTSUP, "CZ <= 128"),
    (dict(H=8), ops.EVO_ENOTSUP, "H*C <= 128"),
    (dict(dt=7), ops.EVO_ENOTSUP, "dtype"),
])
def test_module_bwd_validation(kw, status, needle):
    assert module_bwd(**kw) == status
    assert needle in err()


def test_project_bwd_validation():
    args = [1, 64, 128, 4, 32, 1, FAKE, FAKE, FAKE, -1.0] + [FAKE] * 10 + \
        [FAKE] * 9 + [FAKE, 1 << 40, None]
    assert L.tri_attn_project_bwd(*args) == ops.EVO_EINVAL
    assert "ln_eps" in err()
    args[9] = 1e-5
    args[19] = None  # dbias
    assert L.tri_attn_project_bwd(*args) == ops.EVO_EINVAL
    assert "'dbias' is NULL" in err()
    args[19] = FAKE
    args[30] = 100
    assert L.tri_attn_project_bwd(*args) == ops.EVO_EWORKSPACE
    assert L.tri_attn_out_project_bwd(1, 64, 128, 4, 32, 0, FAKE, FAKE, FAKE,
                                      FAKE, None, FAKE, FAKE, 1 << 40,
                                      None) == ops.EVO_EINVAL
    assert "'dw_o' is NULL" in err()


def test_module_bwd_fault_injection(monkeypatch):
    monkeypatch.setenv("EVO_FAULT_INJECT", "launch")
    assert module_bwd() == ops.EVO_EHIP
    assert "injected" in err()


def test_trimul_and_transition_validation():
    assert L.tri_mul_workspace_bytes(1, 768, 128, 128) >= 3 * 128 * 768 * 768 * 2
    assert L.tri_mul_workspace_bytes(1, 768, 128, 100) == 0   # C not a multiple of 32
    args = [1, 64, 128, 128, 1, FAKE, None, FAKE, FAKE, 1e-5, FAKE, FAKE, FAKE,
            None, FAKE, FAKE, 1 << 40, None]
    args[4] = 2
    assert L.tri_mul_fwd(*args) == ops.EVO_EINVAL and "outgoing" in err()
    args[4] = 1
    args[16] = 10
    assert L.tri_mul_fwd(*args) == ops.EVO_EWORKSPACE
    args[16] = 1 << 40
    args[3] = 256
    assert L.tri_mul_fwd(*args) == ops.EVO_ENOTSUP
    w = L.pair_transition_workspace_bytes(1, 768, 128, 512)
    assert 0 < w < 1 << 20  # the rearranged weights only, independent of N
    assert L.pair_transition_workspace_bytes(1, 64, 128, 500) == 0  # HID % 64
    targs = [1, 64, 128, 512, FAKE, FAKE, FAKE, 1e-5, FAKE, FAKE, FAKE, FAKE,
             FAKE, 1 << 30, None]
    targs[11] = None
    assert L.pair_transition_fwd(*targs) == ops.EVO_EINVAL and "'out' is NULL" in err()
    targs[11] = FAKE
    targs[13] = 16
    assert L.pair_transition_fwd(*targs) == ops.EVO_EWORKSPACE


def test_opm_validation():
    w = L.outer_product_mean_workspace_bytes(1, 1024, 768, 256, 32, 128)
    M = 768 * 32
    assert w >= M * M * 2 + 2 * M * 1024 * 2  # the product and both projections
    assert L.outer_product_mean_workspace_bytes(1, 1024, 768, 256, 48, 128) == 0  # C % 32
    assert L.outer_product_mean_workspace_bytes(1, 1024, 768, 512, 32, 128) == 0  # CM > 256
    assert L.outer_product_mean_workspace_bytes(1, 8, 2000, 64, 32, 128) == 0  # N*C too big
    assert L.outer_product_mean_workspace_bytes(1, 0, 8, 64, 32, 128) == 0
    args = [1, 16, 8, 64, 32, 64, FAKE, FAKE, FAKE, 1e-5, FAKE, FAKE, FAKE, None,
            FAKE, FAKE, 1 << 30, None]
    args[14] = None
    assert L.outer_product_mean_fwd(*args) == ops.EVO_EINVAL and "'out' is NULL" in err()
    args[14] = FAKE
    args[16] = 64
    assert L.outer_product_mean_fwd(*args) == ops.EVO_EWORKSPACE
    args[16] = 1 << 30
    args[9] = 0.0
    assert L.outer_product_mean_fwd(*args) == ops.EVO_EINVAL and "ln_eps" in err()
    args[9] = 1e-5
    args[3] = 100
    assert L.outer_product_mean_fwd(*args) == ops.EVO_ENOTSUP and "CM=100" in err()


def test_opm_fault_injection(monkeypatch):
    monkeypatch.setenv("EVO_FAULT_INJECT", "launch")
    args = [1, 16, 8, 64, 32, 64, FAKE, FAKE, FAKE, 1e-5, FAKE, FAKE, FAKE, None,
            FAKE, FAKE, 1 << 30, None]
    assert L.outer_product_mean_fwd(*args) == ops.EVO_EHIP
    assert "injected" in err()


def test_transition_bwd_validation():
    assert L.pair_transition_bwd_workspace_bytes(1, 64, 128, 512) > 3 * 64 * 64 * 512 * 2
    assert L.pair_transition_bwd_workspace_bytes(1, 64, 128, 192) == 0  # HID % 128
    args = [1, 16, 64, 256, FAKE, FAKE, FAKE, 1e-5, FAKE, FAKE, FAKE, FAKE, FAKE,
            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 34, None]
    args[12] = None
    assert L.pair_transition_bwd(*args) == ops.EVO_EINVAL and "'dz' is NULL" in err()
    args[12] = FAKE
    args[19] = 128
    assert L.pair_transition_bwd(*args) == ops.EVO_EWORKSPACE
    args[19] = 1 << 34
    args[3] = 192
    assert L.pair_transition_bwd(*args) == ops.EVO_ENOTSUP and "HID=192" in err()


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _module_args(N=8, CZ=32, H=2, C=32):
    HC = H * C
    return dict(z=_bf(N, N, CZ), ln_w=_bf(CZ), ln_b=_bf(CZ), eps=1e-5, w_q=_bf(HC, CZ),
                w_k=_bf(HC, CZ), w_v=_bf(HC, CZ), w_g=_bf(HC, CZ), b_g=_bf(HC),
                w_bias=_bf(H, CZ), w_o=_bf(CZ, HC), b_o=_bf(CZ))


@pytest.mark.parametrize("call,bad,needle", [
    # tri_attn_project: every weight and LayerNorm vector, and z itself
    ("project", dict(z=_bf(8, 7, 32)), "z must be [N, N, c]"),
    ("project", dict(ln_w=_bf(31)), "ln_w has shape"),
    ("project", dict(ln_b=_bf(33)), "ln_b has shape"),
    ("project", dict(w_q=_bf(64, 31)), "w_q has shape"),
    ("project", dict(w_k=_bf(63, 32)), "w_k has shape"),
    ("project", dict(w_v=_bf(64, 33)), "w_v has shape"),
    ("project", dict(w_g=_bf(32, 32)), "w_g has shape"),
    ("project", dict(b_g=_bf(63)), "b_g has shape"),
    ("project", dict(w_bias=_bf(3, 32)), "w_bias has shape"),
    ("module", dict(w_o=_bf(32, 63)), "w_o has shape"),
    ("module", dict(b_o=_bf(31)), "b_o has shape"),
    ("module", dict(residue_mask=torch.ones(7, dtype=torch.uint8)), "residue_mask has shape"),
])
def test_module_bindings_check_shapes(call, bad, needle):
    """A mismatched weight, vector or mask is rejected by the binding with
    EVO_EINVAL before any pointer reaches the library (tensors here are
    host tensors: the shape check comes first)."""
    a = _module_args()
    mask = bad.pop("residue_mask", None)
    a.update(bad)
    with pytest.raises(ops.EvoAttnError) as ei:
        if call == "project":
            ops.tri_attn_project(a["z"], a["ln_w"], a["ln_b"], a["eps"], a["w_q"], a["w_k"],
                                 a["w_v"], a["w_g"], a["b_g"], a["w_bias"], 2, 32, False)
        else:
            ops.tri_attn_module_fwd(a["z"], mask, a["ln_w"], a["ln_b"], a["eps"], a["w_q"],
                                    a["w_k"], a["w_v"], a["w_g"], a["b_g"], a["w_bias"],
                                    a["w_o"], a["b_o"], 2, 32, False)
    assert ei.value.status == ops.EVO_EINVAL
    assert needle in str(ei.value), str(ei.value)


@pytest.mark.parametrize("fn,args,needle", [
    ("tri_mul_fwd", lambda: (_bf(8, 8, 32), None, _bf(32), _bf(32), 1e-5, _bf(16, 32),
                             _bf(16, 31), _bf(32, 16), _bf(32)), "w_b has shape"),
    ("tri_mul_fwd", lambda: (_bf(8, 8, 32), None, _bf(32), _bf(32), 1e-5, _bf(16, 32),
                             _bf(16, 32), _bf(32, 15), _bf(32)), "w_o has shape"),
    ("tri_mul_fwd", lambda: (_bf(8, 8, 32), torch.ones(9, dtype=torch.uint8), _bf(32),
                             _bf(32), 1e-5, _bf(16, 32), _bf(16, 32), _bf(32, 16), _bf(32)),
     "residue_mask has shape"),
    ("pair_transition_fwd", lambda: (_bf(8, 8, 32), _bf(32), _bf(32), 1e-5, _bf(64, 32),
                                     _bf(64, 32), _bf(32, 63)), "w_o has shape"),
    ("pair_transition_fwd", lambda: (_bf(8, 8, 32), _bf(31), _bf(32), 1e-5, _bf(64, 32),
                                     _bf(64, 32), _bf(32, 64)), "ln_w has shape"),
    ("pair_transition_bwd", lambda: (_bf(8, 8, 32), _bf(32), _bf(32), 1e-5, _bf(64, 32),
                                     _bf(65, 32), _bf(32, 64), _bf(8, 8, 32)), "w_b has shape"),
    ("pair_transition_bwd", lambda: (_bf(8, 8, 32), _bf(32), _bf(32), 1e-5, _bf(64, 32),
                                     _bf(64, 32), _bf(32, 64), _bf(8, 7, 32)), "dout has shape"),
    ("outer_product_mean_fwd", lambda: (_bf(4, 8, 16), _bf(16), _bf(16), 1e-5, _bf(8, 16),
                                        _bf(8, 16), _bf(32, 63), _bf(32)), "w_o has shape"),
    ("outer_product_mean_fwd", lambda: (_bf(4, 8, 16), _bf(15), _bf(16), 1e-5, _bf(8, 16),
                                        _bf(8, 16), _bf(32, 64), _bf(32)), "ln_w has shape"),
])
def test_pair_op_bindings_check_shapes(fn, args, needle):
    with pytest.raises(ops.EvoAttnError) as ei:
        getattr(ops, fn)(*args())
    assert ei.value.status == ops.EVO_EINVAL
    assert needle in str(ei.value), str(ei.value)


def test_probe_validation():
    assert L.evo_probe_issue_rate(3, 1, 1, FAKE, None) == ops.EVO_EINVAL
    assert L.evo_probe_issue_rate(0, 9, 1, FAKE, None) == ops.EVO_EINVAL
    assert L.evo_probe_issue_rate(0, 1, 1, None, None) == ops.EVO_EINVAL
