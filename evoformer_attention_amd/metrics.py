"""Work and traffic counts for the attention path (host-side arithmetic used
by the benchmark; no GPU work).

Flops: 4*L*C for the forward and 2.5 times that for the backward, where
L = B*R*H*N^2 is the number of logits of a call (each logit costs C
multiply-adds for Q.K and C for P.V; masked keys are counted).

Memory: the dense logits a naive implementation would store are N^3*H
elements per triangle attention (one [H, N, N] block per row, N rows), and
the pair representation is N^2*c_z elements ("Evoformer: the memory wall ZeRO
cannot move", section "Where the memory goes" and the table in "The two
tensors").
"""

MI355X_BF16_DENSE_TFLOPS = 2500.0   # dense MFMA, bf16
MI355X_FP32_MFMA_TFLOPS = 157.3
MI355X_HBM_GBS = 8000.0


def n_logits(B, R, N, H):
    return B * R * H * N * N


def fwd_flops(B, R, N, H, C):
    return 4.0 * n_logits(B, R, N, H) * C


def bwd_flops(B, R, N, H, C):
    return 2.5 * fwd_flops(B, R, N, H, C)


def project_flops(N, CZ, H, C):
    """LayerNorm'd pair rep times the four [CZ, H*C] projections and the
    [CZ, H] bias projection."""
    return 2.0 * N * N * CZ * (4 * H * C + H)


def out_project_flops(N, CZ, H, C):
    return 2.0 * N * N * H * C * CZ


def triangle_logit_bytes(N, H, elem_bytes):
    return N ** 3 * H * elem_bytes


def pair_rep_bytes(N, CZ, elem_bytes):
    return N ** 2 * CZ * elem_bytes


def fwd_min_bytes(B, R, N, H, C, elem_bytes, gate=True, bias=True,
                  lse=False, mask_rows=0):
    """Algorithmic HBM bytes of one forward call: Q, K, V (and the gate) read
    once, Out written once, the bias read once per batch, the key mask read
    once, LSE written once when requested."""
    t = B * R * N * H * C * elem_bytes
    n = (3 + (1 if gate else 0) + 1) * t
    if bias:
        n += B * H * N * N * elem_bytes
    if lse:
        n += B * R * H * N * 4
    n += B * mask_rows * N
    return n


def bwd_min_bytes(B, R, N, H, C, elem_bytes, gate=True, bias=True,
                  mask_rows=0):
    """Algorithmic HBM bytes of one backward call: Q, K, V, gate, Out, dOut
    read once; dQ, dK, dV, dGate written once; LSE read once; the bias read
    once per batch and the fp32 dBias written once."""
    t = B * R * N * H * C * elem_bytes
    n_in = 4 + (1 if gate else 0) + 1       # q k v out dout (+gate)
    n_out = 3 + (1 if gate else 0)          # dq dk dv (+dgate)
    n = (n_in + n_out) * t + B * R * H * N * 4
    if bias:
        n += B * H * N * N * elem_bytes + B * H * N * N * 4
    n += B * mask_rows * N
    return n


def module_step_flops(N, CZ, H, C):
    """Counted flops of one training step of the triangle-attention module
    (forward plus backward, recomputation not counted): the projection and
    output-projection GEMMs once forward and twice backward (input and weight
    gradients), the attention 1 + 2.5 times its forward."""
    gemm = project_flops(N, CZ, H, C) + out_project_flops(N, CZ, H, C)
    return 3.0 * gemm + fwd_flops(1, N, N, H, C) + bwd_flops(1, N, N, H, C)


def project_bwd_min_bytes(N, CZ, H, C, elem_bytes):
    """Algorithmic HBM bytes of tri_attn_project_bwd: dq, dk, dv, dg read
    once (working dtype), the fp32 pair-bias gradient read once, z read once
    and dz written once; the fp32 parameter gradients are negligible."""
    t = N * N * H * C * elem_bytes
    return 4 * t + H * N * N * 4 + 2 * pair_rep_bytes(N, CZ, elem_bytes)


def trimul_flops(N, CZ, C):
    """Counted flops of one triangular multiplicative update: the a and b
    projections (2 x C outputs per position), the per-channel products
    (C matrices of N x N times N x N) and the output projection."""
    return 2.0 * N * N * CZ * 2 * C + 2.0 * C * N ** 3 + 2.0 * N * N * C * CZ


def trimul_bwd_flops(N, CZ, C):
    """Counted flops of the multiplicative update's backward: dT = dout . W_o
    and dW_o = dout^T t (2 x 2 N^2 CZ C), the two per-channel products dA and
    dB (2 x 2 C N^3), dx = da . W_a + db . W_b and dW_a, dW_b (4 x 2 N^2 C
    CZ).  The recomputed forward (a, b and t) is not counted."""
    return 4.0 * C * N ** 3 + 12.0 * N * N * C * CZ


def transition_bwd_flops(N, CZ, HID):
    """Counted flops of the transition backward per position: the recomputed
    u, v (2 x 2 HID CZ), dh (2 HID CZ), dx (2 x 2 HID CZ) and the three
    weight-gradient contractions (3 x 2 HID CZ): 16 HID CZ."""
    return 16.0 * N * N * HID * CZ


def opm_bwd_flops(S, N, CM, C, CZ):
    """Counted flops of the outer product mean's backward: dP = dout . W_o and
    dW_o = dout^T P (2 x 2 N^2 CZ C^2), the two products dA = dP . B and
    dB = dP^T . A (2 x 2 (N C)^2 S), dx = da . W_a + db . W_b and dW_a, dW_b
    (4 x 2 S N C CM).  The recomputed forward (a, b and P) is not counted."""
    return (4.0 * N * N * CZ * C * C + 4.0 * (N * C) ** 2 * S
            + 8.0 * S * N * C * CM)


def opm_flops(S, N, CM, C, CZ):
    """Counted flops of one outer product mean: the a and b projections (2 x C
    outputs per sequence-residue position), the product of the [N*C, S] and
    [S, N*C] operand matrices and the [CZ, C*C] output projection per pair."""
    return (2.0 * S * N * CM * 2 * C + 2.0 * (N * C) ** 2 * S
            + 2.0 * N * N * C * C * CZ)


def transition_flops(N, CZ, HID):
    """Counted flops of the LayerNorm + SwiGLU transition: two [HID, CZ]
    projections and the [CZ, HID] output projection per position."""
    return 2.0 * N * N * (2 * HID * CZ + HID * CZ)
