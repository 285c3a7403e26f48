"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle
checks.  This module holds none of the attention arithmetic: it only draws
random tensors, masks and weights (all on the CPU, with a torch.Generator
seeded once per workload and drawn in a fixed order) and rounds them to the
working dtype.

Workloads (shapes after the pages' AlphaFold2 setting: c_z = 128, 4 heads,
bf16, N_res 128..1024, from the memory table of "Evoformer: the memory wall
ZeRO cannot move"):
  core_fp32_small   B=1, R=32,  N=32,  H=4, C=32, fp32, bias, gate, no mask
  msa_row_bf16      B=1, R=128, N=256, H=8, C=32, bf16, bias shared by rows,
                    last 26 residues masked (10% of 256, rounded up)
  tri_start_384     module, starting node, z [384,384,128], no mask
  tri_end_768       module, ending node,  z [768,768,128], 38 random residues
                    masked (5% of 768, rounded down)
  tri_start_512_bwd projection + core forward + core backward, starting node,
                    z [512,512,128], upstream gradient ~ N(0,1)
  trimul_out_768    triangular multiplicative update, outgoing edges,
                    z [768,768,128], 128 channels, 38 random residues masked
  transition_768    LayerNorm + SwiGLU transition, z [768,768,128], hidden
                    width 4 x 128 = 512
  opm_1024x768      outer product mean, m [1024,768,256] (MSA depth 1024 as
                    in the pages' coevolution example, c_m = 8 x 32 as in
                    msa_row_bf16), 32 channels, out [768,768,128]
"""
import math
import torch

__all__ = ["WORKLOADS", "core_inputs", "module_inputs", "round_to",
           "rand_core", "rand_module", "rand_trimul", "trimul_inputs",
           "rand_transition", "transition_inputs", "rand_opm", "opm_inputs"]

WORKLOADS = {
    "core_fp32_small": dict(kind="core", B=1, R=32, N=32, H=4, C=32,
                            dtype="fp32", mask=None, gate=True, bias=True),
    "msa_row_bf16": dict(kind="core", B=1, R=128, N=256, H=8, C=32,
                         dtype="bf16", mask="tail10", gate=True, bias=True),
    "tri_start_384": dict(kind="module", N=384, CZ=128, H=4, C=32,
                          dtype="bf16", ending=False, mask=None),
    "tri_end_768": dict(kind="module", N=768, CZ=128, H=4, C=32,
                        dtype="bf16", ending=True, mask="random5"),
    "tri_start_512_bwd": dict(kind="module_bwd", N=512, CZ=128, H=4, C=32,
                              dtype="bf16", ending=False, mask=None),
    "trimul_out_768": dict(kind="trimul", N=768, CZ=128, C=128, dtype="bf16",
                           outgoing=True, mask="random5"),
    "transition_768": dict(kind="transition", N=768, CZ=128, HID=512, dtype="bf16"),
    "opm_1024x768": dict(kind="opm", S=1024, N=768, CM=256, C=32, CZ=128, dtype="bf16"),
}

_TORCH_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def round_to(t, dtype):
    """Round an fp32 CPU tensor to the working dtype (round-to-nearest-even)."""
    return t.to(_TORCH_DT[dtype])


def _key_mask(rule, N, gen):
    """Keep flags (1 = keep) for the mask rule of a workload."""
    keep = torch.ones(N, dtype=torch.uint8)
    if rule is None:
        return None
    if rule == "tail10":
        n_off = math.ceil(0.10 * N)
        keep[N - n_off:] = 0
    elif rule == "random5":
        n_off = int(0.05 * N)
        keep[torch.randperm(N, generator=gen)[:n_off]] = 0
    else:
        raise ValueError(rule)
    return keep


def rand_core(B, R, N, H, C, dtype, seed=0, gate=True, bias=True, mask=None,
              mask_rows=1, dout=False, scale=1.0):
    """Core attention inputs with N(0,1) entries, drawn in the order
    q, k, v, gate, bias, dout, then the mask.  `mask` is None, a rule name
    ("tail10", "random5") or "random" (each key kept with p = 0.8, per mask
    row).  Returns a dict of CPU tensors in the working dtype; the mask is
    uint8 [B, mask_rows, N]."""
    gen = torch.Generator().manual_seed(seed)
    shp = (B, R, N, H, C)

    def draw(shape):
        return round_to(torch.randn(shape, generator=gen) * scale, dtype)

    d = {"q": draw(shp), "k": draw(shp), "v": draw(shp)}
    d["gate"] = draw(shp) if gate else None
    d["bias"] = draw((B, H, N, N)) if bias else None
    d["dout"] = draw(shp) if dout else None
    if mask is None:
        d["mask"] = None
    elif mask == "random":
        d["mask"] = (torch.rand((B, mask_rows, N), generator=gen) < 0.8).to(
            torch.uint8)
    else:
        km = _key_mask(mask, N, gen)
        d["mask"] = km.expand(B, mask_rows, N).contiguous()
    return d


def rand_module(N, CZ, H, C, dtype, seed=0, mask=None, dout=False,
                ln_affine=False, gate_bias=False, out_bias=False):
    """Module inputs: z ~ N(0,1) [N,N,CZ]; every projection weight
    ~ N(0, 1/fan_in) (standard deviation fan_in^-1/2, fan_in = CZ for the
    input projections and H*C for the output projection), stored [out, in]
    as torch.nn.Linear does; LayerNorm weight 1 and bias 0 unless ln_affine;
    gate/output bias vectors 0 unless requested.  Draw order: z, w_q, w_k,
    w_v, w_g, w_bias, w_o, mask, dout, then the optional affine/bias draws."""
    gen = torch.Generator().manual_seed(seed)
    HC = H * C

    def draw(shape, std=1.0):
        return round_to(torch.randn(shape, generator=gen) * std, dtype)

    d = {"z": draw((N, N, CZ))}
    s_in = CZ ** -0.5
    for name in ("w_q", "w_k", "w_v", "w_g"):
        d[name] = draw((HC, CZ), s_in)
    d["w_bias"] = draw((H, CZ), s_in)
    d["w_o"] = draw((CZ, HC), HC ** -0.5)
    d["mask"] = _key_mask(mask, N, gen) if isinstance(mask, str) else mask
    d["dout"] = draw((1, N, N, H, C)) if dout else None
    d["ln_w"] = draw((CZ,), 0.2) + 1 if ln_affine else round_to(torch.ones(CZ), dtype)
    d["ln_b"] = draw((CZ,), 0.2) if ln_affine else round_to(torch.zeros(CZ), dtype)
    d["b_g"] = draw((HC,), 0.5) if gate_bias else round_to(torch.zeros(HC), dtype)
    d["b_o"] = draw((CZ,), 0.5) if out_bias else round_to(torch.zeros(CZ), dtype)
    d["eps"] = 1e-5
    return d


def core_inputs(name, seed=0, dout=False):
    w = WORKLOADS[name]
    assert w["kind"] == "core"
    return rand_core(w["B"], w["R"], w["N"], w["H"], w["C"], w["dtype"],
                     seed=seed, gate=w["gate"], bias=w["bias"], mask=w["mask"],
                     dout=dout)


def module_inputs(name, seed=0):
    w = WORKLOADS[name]
    return rand_module(w["N"], w["CZ"], w["H"], w["C"], w["dtype"], seed=seed,
                       mask=w["mask"], dout=(w["kind"] == "module_bwd"))


def rand_trimul(N, CZ, C, dtype, seed=0, mask=None, dout=False):
    """Multiplicative-update inputs: z ~ N(0,1) [N,N,CZ]; w_a, w_b [C, CZ]
    ~ N(0, 1/CZ); w_o [CZ, C] ~ N(0, 1/C) / sqrt(N) (the update sums N
    products); LayerNorm weight 1 + N(0, 0.2^2), bias N(0, 0.2^2); b_o
    N(0, 0.5^2); with dout, an upstream gradient ~ N(0,1) [N,N,CZ].  Draw
    order: z, w_a, w_b, w_o, mask, ln_w, ln_b, b_o, dout."""
    gen = torch.Generator().manual_seed(seed)

    def draw(shape, std=1.0):
        return round_to(torch.randn(shape, generator=gen) * std, dtype)

    d = {"z": draw((N, N, CZ))}
    d["w_a"] = draw((C, CZ), CZ ** -0.5)
    d["w_b"] = draw((C, CZ), CZ ** -0.5)
    d["w_o"] = draw((CZ, C), (C * N) ** -0.5)
    d["mask"] = _key_mask(mask, N, gen) if isinstance(mask, str) else mask
    d["ln_w"] = draw((CZ,), 0.2) + 1
    d["ln_b"] = draw((CZ,), 0.2)
    d["b_o"] = draw((CZ,), 0.5)
    d["eps"] = 1e-5
    if dout:
        d["dout"] = draw((N, N, CZ))
    return d


def trimul_inputs(name, seed=0, dout=False):
    w = WORKLOADS[name]
    assert w["kind"] == "trimul"
    return rand_trimul(w["N"], w["CZ"], w["C"], w["dtype"], seed=seed, mask=w["mask"],
                       dout=dout)


def rand_transition(N, CZ, HID, dtype, seed=0, dout=False):
    """Transition inputs: z ~ N(0,1) [N,N,CZ]; w_a, w_b [HID, CZ] ~ N(0,
    1/CZ); w_o [CZ, HID] ~ N(0, 1/HID); LayerNorm weight 1 + N(0, 0.2^2),
    bias N(0, 0.2^2); with dout, an upstream gradient ~ N(0,1) [N,N,CZ].
    Draw order: z, w_a, w_b, w_o, ln_w, ln_b, dout."""
    gen = torch.Generator().manual_seed(seed)

    def draw(shape, std=1.0):
        return round_to(torch.randn(shape, generator=gen) * std, dtype)

    d = {"z": draw((N, N, CZ))}
    d["w_a"] = draw((HID, CZ), CZ ** -0.5)
    d["w_b"] = draw((HID, CZ), CZ ** -0.5)
    d["w_o"] = draw((CZ, HID), HID ** -0.5)
    d["ln_w"] = draw((CZ,), 0.2) + 1
    d["ln_b"] = draw((CZ,), 0.2)
    d["eps"] = 1e-5
    if dout:
        d["dout"] = draw((N, N, CZ))
    return d


def transition_inputs(name, seed=0, dout=False):
    w = WORKLOADS[name]
    assert w["kind"] == "transition"
    return rand_transition(w["N"], w["CZ"], w["HID"], w["dtype"], seed=seed, dout=dout)


def rand_opm(S, N, CM, C, CZ, dtype, seed=0, dout=False):
    """Outer-product-mean inputs: m ~ N(0,1) [S,N,CM]; w_a, w_b [C, CM] ~
    N(0, 1/CM); w_o [CZ, C*C] ~ N(0, S/C^2) (a mean of S products of
    independent unit terms has size 1/sqrt(S), so the projected update is of
    unit size, like b_o); LayerNorm weight 1 + N(0, 0.2^2), bias N(0,
    0.2^2); b_o N(0, 0.5^2); with dout, an upstream gradient ~ N(0,1)
    [N,N,CZ].  Draw order: m, w_a, w_b, w_o, ln_w, ln_b, b_o, dout."""
    gen = torch.Generator().manual_seed(seed)

    def draw(shape, std=1.0):
        return round_to(torch.randn(shape, generator=gen) * std, dtype)

    d = {"m": draw((S, N, CM))}
    d["w_a"] = draw((C, CM), CM ** -0.5)
    d["w_b"] = draw((C, CM), CM ** -0.5)
    d["w_o"] = draw((CZ, C * C), S ** 0.5 / C)
    d["ln_w"] = draw((CM,), 0.2) + 1
    d["ln_b"] = draw((CM,), 0.2)
    d["b_o"] = draw((CZ,), 0.5)
    d["eps"] = 1e-5
    if dout:
        d["dout"] = draw((N, N, CZ))
    return d


def opm_inputs(name, seed=0, dout=False):
    w = WORKLOADS[name]
    assert w["kind"] == "opm"
    return rand_opm(w["S"], w["N"], w["CM"], w["C"], w["CZ"], w["dtype"], seed=seed,
                    dout=dout)
