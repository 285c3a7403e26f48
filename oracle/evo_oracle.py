"""Plain fp64 CPU oracle for the Evoformer's biased, gated attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the entry script
and the CPU-baseline leg of the benchmark use it.  It shares no code with the
HIP library and imports nothing from it; both sides receive the same seeded
arrays from a generator module that holds none of the method's arithmetic.

Sources (web pages; cited by title and section):
  [COURSE]  "Evoformer: the memory wall ZeRO cannot move" (DeepSpeed course),
            sections "Where the memory goes" (display equation: logits are
            O(N_res^3 * n_heads)), "The three operations" (triangle attention
            picks the third residue k by attention instead of a uniform sum)
            and "Two properties the tests assert".
  [MEGAFOLD] "MegaFold: Efficient Training of Next-Generation 3D Attention
            Protein Models on Cross-Platform GPUs", section "Methodologie",
            item 1 "EvoFlash-3D": online, numerically stable softmax in the
            forward and backward passes, exact results, and an additively
            broadcast pair bias.

What is computed (the plain reading; the pages never print the formula):
for every attention line (batch b, row r), head h, query q and key k

    s[q,k]  = <Q[q], K[k]> / sqrt(C) + bias[b,h,q,k] + (keep[k] ? 0 : -inf)
    P[q,:]  = softmax_k(s[q,:])
    O[q]    = sum_k P[q,k] V[k]
    Out[q]  = sigmoid(G[q]) * O[q]                  (identity when no gate)
    LSE[q]  = log sum_k exp(s[q,k])                  (natural log)

A line whose keys are all masked has Out = 0, LSE = -inf and zero gradients
(a reading: the pages are silent).  The bias is shared by every row of a
batch ("additively broadcast" in [MEGAFOLD]), so its gradient is the sum over
rows of dS.

Every array is float64; callers pass the exact values the GPU sees (for bf16
runs, the bf16-rounded inputs upcast to float64).  No blocking, fusion or
reordering beyond the definition: each logit block of one (line, head) is
materialised in full before the value product, which is exactly what the GPU
path must avoid doing in HBM.
"""
import numpy as np

__all__ = [
    "sigmoid", "attention_line_probs", "attention_line_forward",
    "attention_forward", "attention_line_backward", "attention_backward",
    "dbias_query_rows", "layer_norm", "tri_project", "tri_out_project",
    "tri_module_forward", "tri_module_lines", "layer_norm_backward",
    "tri_out_project_backward", "tri_project_backward",
    "tri_module_backward", "tri_mul_forward", "tri_mul_entries",
    "tri_mul_backward", "tri_mul_backward_entries",
    "transition_forward", "outer_product_mean", "transition_backward", "transition_weight_grad_units", "outer_product_mean_pairs",
    "outer_product_mean_backward", "outer_product_mean_backward_sampled",
]


def sigmoid(x):
    """Logistic function 1 / (1 + e^-x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def _line_logits(q, k, bias, keep, h):
    """Logits s[q, k] of one (line, head): scaled dot products plus pair bias
    plus the key mask.  q, k: [N, H, C]; bias: [H, N, N] or None; keep: [N]
    bool or None."""
    C = q.shape[-1]
    s = (q[:, h, :] @ k[:, h, :].T) / np.sqrt(C)
    if bias is not None:
        s = s + bias[h]
    if keep is not None:
        s = np.where(keep[None, :], s, -np.inf)
    return s


def attention_line_probs(q, k, bias=None, keep=None):
    """Softmax probabilities P[h, q, k] of one attention line.

    A query whose keys are all masked gets an all-zero row (the reading for a
    fully masked line)."""
    N, H, _ = q.shape
    P = np.zeros((H, N, N))
    for h in range(H):
        s = _line_logits(q, k, bias, keep, h)
        m = s.max(axis=1, keepdims=True)
        live = np.isfinite(m[:, 0])
        e = np.zeros_like(s)
        e[live] = np.exp(s[live] - m[live])
        l = e.sum(axis=1, keepdims=True)
        P[h][live] = e[live] / l[live]
    return P


def attention_line_forward(q, k, v, gate=None, bias=None, keep=None):
    """Forward pass of one attention line (one batch entry b and row r).

    q, k, v, gate: [N, H, C]; bias: [H, N, N]; keep: [N] bool.
    Returns out [N, H, C] and lse [H, N] (natural log; -inf when every key is
    masked)."""
    q = np.asarray(q, np.float64)
    N, H, C = q.shape
    out = np.zeros((N, H, C))
    lse = np.empty((H, N))
    for h in range(H):
        s = _line_logits(q, k, bias, keep, h)
        m = s.max(axis=1)
        live = np.isfinite(m)
        e = np.zeros_like(s)
        e[live] = np.exp(s[live] - m[live, None])
        l = e.sum(axis=1)
        lse[h] = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
        P = np.zeros_like(s)
        P[live] = e[live] / l[live, None]
        o = P @ v[:, h, :]
        if gate is not None:
            o = o * sigmoid(gate[:, h, :])
        out[:, h, :] = o
    return out, lse


def _line_inputs(b, r, gate, key_mask, bias):
    g = None if gate is None else gate[b, r]
    keep = None
    if key_mask is not None:
        mr = key_mask.shape[1]
        keep = key_mask[b, 0 if mr == 1 else r] != 0
    bb = None if bias is None else bias[b]
    return g, keep, bb


def attention_forward(q, k, v, gate=None, key_mask=None, bias=None):
    """Biased gated attention over every line.

    q, k, v, gate: [B, R, N, H, C]; key_mask: [B, MR, N] with MR in {1, R}
    (nonzero = keep); bias: [B, H, N, N] shared by the R rows of a batch.
    Returns out [B, R, N, H, C] and lse [B, R, H, N]."""
    B, R, N, H, C = q.shape
    out = np.zeros((B, R, N, H, C))
    lse = np.zeros((B, R, H, N))
    for b in range(B):
        for r in range(R):
            g, keep, bb = _line_inputs(b, r, gate, key_mask, bias)
            out[b, r], lse[b, r] = attention_line_forward(
                q[b, r], k[b, r], v[b, r], g, bb, keep)
    return out, lse


def attention_line_backward(q, k, v, gate, bias, keep, dout):
    """Gradients of one attention line with respect to Q, K, V, the
    pre-sigmoid gate and this line's contribution to the pair-bias gradient.

    Chain rule through Out = sigmoid(G) * O, O = P V, P = softmax(s):
      dO    = dOut * sigmoid(G)
      dG    = dOut * O * sigmoid(G) * (1 - sigmoid(G))
      dV    = P^T dO,   dP = dO V^T
      dS    = P * (dP - rowsum(P * dP))
      dQ    = dS K / sqrt(C),   dK = dS^T Q / sqrt(C),   dBias = dS
    Returns dq, dk, dv, dg (None when there is no gate) and dbias [H, N, N]."""
    N, H, C = q.shape
    dq = np.zeros((N, H, C))
    dk = np.zeros((N, H, C))
    dv = np.zeros((N, H, C))
    dg = None if gate is None else np.zeros((N, H, C))
    dbias = np.zeros((H, N, N))
    P_all = attention_line_probs(q, k, bias, keep)
    for h in range(H):
        P = P_all[h]
        o = P @ v[:, h, :]
        do_h = dout[:, h, :]
        if gate is not None:
            sg = sigmoid(gate[:, h, :])
            dg[:, h, :] = do_h * o * sg * (1.0 - sg)
            do_h = do_h * sg
        dv[:, h, :] = P.T @ do_h
        dP = do_h @ v[:, h, :].T
        D = (P * dP).sum(axis=1, keepdims=True)
        dS = P * (dP - D)
        dq[:, h, :] = dS @ k[:, h, :] / np.sqrt(C)
        dk[:, h, :] = dS.T @ q[:, h, :] / np.sqrt(C)
        dbias[h] = dS
    return dq, dk, dv, dg, dbias


def attention_backward(q, k, v, gate, key_mask, bias, dout):
    """Backward of attention_forward for every line.

    Returns dq, dk, dv, dgate (None without a gate) shaped like q, and dbias
    [B, H, N, N]: the sum over the R rows of each batch of dS (zeros are
    returned even when no bias was given, since dS does not depend on it)."""
    B, R, N, H, C = q.shape
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros_like(dq)
    dv = np.zeros_like(dq)
    dg = None if gate is None else np.zeros_like(dq)
    dbias = np.zeros((B, H, N, N))
    for b in range(B):
        for r in range(R):
            g, keep, bb = _line_inputs(b, r, gate, key_mask, bias)
            lq, lk, lv, lg, lb = attention_line_backward(
                q[b, r], k[b, r], v[b, r], g, bb, keep, dout[b, r])
            dq[b, r], dk[b, r], dv[b, r] = lq, lk, lv
            if dg is not None:
                dg[b, r] = lg
            dbias[b] += lb
    return dq, dk, dv, dg, dbias


def dbias_query_rows(q, k, v, gate, key_mask, bias, dout, b, picks):
    """dBias[b, h, qi, :] for the (h, qi) pairs in `picks`, summed over every
    row of batch b.  Only the listed query's logits are formed for each row,
    so a few entries of a large problem stay cheap.  Returns [len(picks), N]."""
    _, R, N, H, C = q.shape
    res = np.zeros((len(picks), N))
    for r in range(R):
        g, keep, bb = _line_inputs(b, r, gate, key_mask, bias)
        for t, (h, qi) in enumerate(picks):
            s = (k[b, r, :, h, :] @ q[b, r, qi, h, :]) / np.sqrt(C)
            if bb is not None:
                s = s + bb[h, qi]
            if keep is not None:
                s = np.where(keep, s, -np.inf)
            m = s.max()
            if not np.isfinite(m):
                continue
            e = np.exp(s - m)
            P = e / e.sum()
            do_q = dout[b, r, qi, h, :]
            if g is not None:
                do_q = do_q * sigmoid(g[qi, h, :])
            dP = v[b, r, :, h, :] @ do_q
            D = (P * dP).sum()
            res[t] += P * (dP - D)
    return res


# ----------------------------------------------------------------------------
# Triangle attention module: LayerNorm, projections, core, output projection.
#
# [COURSE] "The three operations": triangle attention updates edge (i, j)
# through third residues k chosen by attention.  [MEGAFOLD] item 3
# "EvoFusion": layer normalisation is followed by linear projections (the
# fusion avoids writing the normalised N x N tensor).  Readings (the pages are
# silent): LayerNorm over c_z with population variance and eps; Q, K, V, gate
# and the per-head pair bias are projections of the same normalised pair
# representation; the gate projection and the output projection carry a
# bias vector, the others do not; the module returns the update only.
#
# Weights follow the torch.nn.Linear convention: W has shape [out, in] and
# y = x . W^T (+ bias vector).
#
# Starting node: line i, query j, key k:
#     s_h(i,j,k) = <q_ij, k_ik>/sqrt(C) + b_jk[h],  out_ij = g_ij * sum_k a v_ik
# Ending node: line j (a column of z), query i, key k:
#     s_h(j,i,k) = <q_ij, k_kj>/sqrt(C) + b_ki[h],  out_ij = g_ij * sum_k a v_kj
# The residue mask removes key k from every line.
# ----------------------------------------------------------------------------

def layer_norm(x, w, b, eps):
    """LayerNorm over the last axis with population variance."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * w + b


def _pair_bias(z, ln_w, ln_b, eps, w_bias):
    """b[j, k, h] = LN(z)[j, k] . w_bias[h, :], computed one z row at a time
    to keep memory at O(N^2 * H)."""
    N = z.shape[0]
    H = w_bias.shape[0]
    out = np.empty((N, N, H))
    for j in range(N):
        out[j] = layer_norm(z[j], ln_w, ln_b, eps) @ w_bias.T
    return out


def _proj(x, w, H, C, bias_vec=None):
    y = x @ w.T
    if bias_vec is not None:
        y = y + bias_vec
    return y.reshape(x.shape[:-1] + (H, C))


def tri_project(z, ln_w, ln_b, eps, w_q, w_k, w_v, w_g, b_g, w_bias, H, C,
                ending, lines=None):
    """First half of the module, in the layout the core attention consumes.

    Returns q, k, v, g as [1, N, N, H, C] (row = attention line, then the
    position along the line) and bias as [1, H, N, N] (bias[h, query, key]).
    Starting node: line i holds z[i, :]; bias[h, j, k] = b_jk[h].
    Ending node: line j holds z[:, j]; bias[h, i, k] = b_ki[h].
    With `lines` given, q, k, v, g hold only those lines ([1, len(lines), N,
    H, C], in the order given); the bias is always complete."""
    z = np.asarray(z, np.float64)
    N = z.shape[0]
    bpair = _pair_bias(z, ln_w, ln_b, eps, w_bias)   # [N, N, H], b_jk[h]
    if ending:
        bias = bpair.transpose(2, 1, 0)     # bias[h, i, k] = b_ki[h]
    else:
        bias = bpair.transpose(2, 0, 1)     # bias[h, j, k] = b_jk[h]
    sel = range(N) if lines is None else lines
    outs = {name: [] for name in ("q", "k", "v", "g")}
    for t in sel:
        # line t: positions (t, j) of z (starting) or (i, t) (ending)
        xl = layer_norm(z[:, t] if ending else z[t], ln_w, ln_b, eps)
        outs["q"].append(_proj(xl, w_q, H, C))
        outs["k"].append(_proj(xl, w_k, H, C))
        outs["v"].append(_proj(xl, w_v, H, C))
        outs["g"].append(_proj(xl, w_g, H, C, b_g))
    q, k, v, g = (np.stack(outs[n])[None] for n in ("q", "k", "v", "g"))
    return q, k, v, g, bias[None]


def tri_out_project(o, w_o, b_o, ending):
    """Output projection: o [1, N, N, H, C] in line layout -> [N, N, CZ] in z
    layout (lines are columns of z for the ending node); w_o is [CZ, H*C]."""
    _, N, _, H, C = o.shape
    y = o[0].reshape(N, N, H * C) @ w_o.T + b_o
    return y.transpose(1, 0, 2) if ending else y


def tri_module_lines(z, residue_mask, ln_w, ln_b, eps, w_q, w_k, w_v, w_g,
                     b_g, w_bias, w_o, b_o, H, C, ending, lines):
    """Module output for selected attention lines, written straight from the
    line-wise definition (not through tri_project).

    Starting node: returns out[i, :, :] for each i in `lines`.
    Ending node:   returns out[:, j, :] for each j in `lines`.
    Result: [len(lines), N, CZ]."""
    z = np.asarray(z, np.float64)
    N = z.shape[0]
    bpair = _pair_bias(z, ln_w, ln_b, eps, w_bias)   # [N, N, H]
    keep = None if residue_mask is None else (np.asarray(residue_mask) != 0)
    res = []
    for t in lines:
        if ending:
            xl = layer_norm(z[:, t], ln_w, ln_b, eps)    # positions (i, t)
            bias = bpair.transpose(2, 1, 0)               # [h, i, k] = b_ki
        else:
            xl = layer_norm(z[t], ln_w, ln_b, eps)        # positions (t, j)
            bias = bpair.transpose(2, 0, 1)               # [h, j, k] = b_jk
        q = _proj(xl, w_q, H, C)
        k = _proj(xl, w_k, H, C)
        v = _proj(xl, w_v, H, C)
        g = _proj(xl, w_g, H, C, b_g)
        o, _ = attention_line_forward(q, k, v, g, bias, keep)
        res.append(o.reshape(N, H * C) @ w_o.T + b_o)
    return np.stack(res)


def tri_module_forward(z, residue_mask, ln_w, ln_b, eps, w_q, w_k, w_v, w_g,
                       b_g, w_bias, w_o, b_o, H, C, ending):
    """Whole module output [N, N, CZ] (the update; no residual add)."""
    N = z.shape[0]
    lines = tri_module_lines(z, residue_mask, ln_w, ln_b, eps, w_q, w_k, w_v,
                             w_g, b_g, w_bias, w_o, b_o, H, C, ending,
                             list(range(N)))
    return lines.transpose(1, 0, 2) if ending else lines


# ----------------------------------------------------------------------------
# Backward of the triangle attention module.
#
# [MEGAFOLD] item 1 trains with the fused kernels in both directions, and
# item 3 fuses the layer normalisation with the projections that follow it;
# the pages print no formula for either backward, so the plain chain rule of
# the forward above is written out here (a reading: the derivative of the
# definition, nothing else).  Weight gradients are summed over every pair
# position; the input gradient is returned in z layout.
# ----------------------------------------------------------------------------

def layer_norm_backward(x, w, eps, dy):
    """Gradients of y = (x - mean) / sqrt(var + eps) * w + b over the last
    axis (population variance).  Returns dx (shaped like x) and dw, db
    summed over every leading axis.  With xhat the normalised input,
    rstd = 1 / sqrt(var + eps) and dxhat = dy * w:
        dx = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat))."""
    x = np.asarray(x, np.float64)
    n = x.shape[-1]
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * rstd
    dxhat = dy * w
    dx = rstd * (dxhat - dxhat.mean(axis=-1, keepdims=True)
                 - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True))
    dw = (dy * xhat).reshape(-1, n).sum(axis=0)
    db = dy.reshape(-1, n).sum(axis=0)
    return dx, dw, db


def _to_lines(t, ending):
    """[N, N, ...] z layout -> line layout (line a, place n): z[a, n] for the
    starting node, z[n, a] for the ending node.  Its own inverse."""
    return t.transpose((1, 0) + tuple(range(2, t.ndim))) if ending else t


def tri_out_project_backward(o, w_o, dout, ending):
    """Backward of tri_out_project.  o [1, N, N, H, C] (line layout),
    w_o [CZ, H*C], dout [N, N, CZ] (z layout).  Returns d_o like o,
    dw_o [CZ, H*C] and db_o [CZ]."""
    _, N, _, H, C = o.shape
    dy = _to_lines(np.asarray(dout, np.float64), ending)   # [line, place, CZ]
    ol = o[0].reshape(N, N, H * C)
    d_o = (dy @ w_o).reshape(1, N, N, H, C)
    CZ = w_o.shape[0]
    dw_o = dy.reshape(-1, CZ).T @ ol.reshape(-1, H * C)
    db_o = dy.reshape(-1, CZ).sum(axis=0)
    return d_o, dw_o, db_o


def tri_project_backward(z, ln_w, ln_b, eps, w_q, w_k, w_v, w_g, w_bias,
                         dq, dk, dv, dg, dbias, ending):
    """Backward of tri_project.  dq, dk, dv, dg: [1, N, N, H, C] (line
    layout), dbias: [1, H, N, N] (bias[h, a, n] is the projection of the
    line-layout position (a, n) in both orientations).  Returns a dict with
    dz [N, N, CZ], dln_w, dln_b [CZ], dw_q, dw_k, dw_v, dw_g [H*C, CZ],
    db_g [H*C] and dw_bias [H, CZ]."""
    z = np.asarray(z, np.float64)
    N, _, CZ = z.shape
    H = w_bias.shape[0]
    HC = w_q.shape[0]
    xl = _to_lines(layer_norm(z, ln_w, ln_b, eps), ending)   # [line, place, CZ]
    flat = {n: t[0].reshape(N, N, HC) for n, t in
            (("q", dq), ("k", dk), ("v", dv), ("g", dg))}
    db = np.moveaxis(dbias[0], 0, -1)                          # [line, place, H]
    dxl = (flat["q"] @ w_q + flat["k"] @ w_k + flat["v"] @ w_v
           + flat["g"] @ w_g + db @ w_bias)
    X = xl.reshape(-1, CZ)
    res = {f"dw_{n}": flat[n].reshape(-1, HC).T @ X for n in "qkvg"}
    res["db_g"] = flat["g"].reshape(-1, HC).sum(axis=0)
    res["dw_bias"] = db.reshape(-1, H).T @ X
    dz, res["dln_w"], res["dln_b"] = layer_norm_backward(
        z, ln_w, eps, _to_lines(dxl, ending))
    res["dz"] = dz
    return res


def tri_module_backward(z, residue_mask, ln_w, ln_b, eps, w_q, w_k, w_v, w_g,
                        b_g, w_bias, w_o, b_o, H, C, ending, dout):
    """Gradients of <dout, tri_module_forward(...)> with respect to z and
    every parameter: the forward recomputed (projections, attention with the
    residue mask on keys), then tri_out_project_backward,
    attention_backward and tri_project_backward.  Returns a dict with the
    entries of tri_project_backward plus dw_o [CZ, H*C] and db_o [CZ]."""
    q, k, v, g, bias = tri_project(z, ln_w, ln_b, eps, w_q, w_k, w_v, w_g,
                                   b_g, w_bias, H, C, ending)
    N = q.shape[1]
    key_mask = (None if residue_mask is None else
                (np.asarray(residue_mask) != 0).astype(np.uint8).reshape(1, 1, N))
    o, _ = attention_forward(q, k, v, g, key_mask, bias)
    d_o, dw_o, db_o = tri_out_project_backward(o, w_o, dout, ending)
    dq, dk, dv, dg, dbias = attention_backward(q, k, v, g, key_mask, bias, d_o)
    res = tri_project_backward(z, ln_w, ln_b, eps, w_q, w_k, w_v, w_g, w_bias,
                               dq, dk, dv, dg, dbias, ending)
    res["dw_o"] = dw_o
    res["db_o"] = db_o
    return res


# ----------------------------------------------------------------------------
# Triangular multiplicative update.
#
# [COURSE] "The three operations": edge (i, j) is updated from every third
# residue k as the sum over k of a_ik * b_jk, channel by channel: O(N^3) time,
# O(N^2) memory.  The pages leave the rest open; the reading taken here is
# the plainest one the module around it supports: a and b are linear
# projections (c channels, no bias) of the layer-normalised pair
# representation, the same normalisation and projection as the
# triangle-attention module; the update is projected back to c_z with an
# output bias.  "Outgoing" sums over edges (i, k) and (j, k); "incoming" over
# (k, i) and (k, j).  A residue mask removes third residues k from the sum.
# ----------------------------------------------------------------------------

def tri_mul_forward(z, residue_mask, ln_w, ln_b, eps, w_a, w_b, w_o, b_o,
                    outgoing=True):
    """z [N, N, CZ]; w_a, w_b [C, CZ]; w_o [CZ, C]; b_o [CZ]; residue_mask
    [N] (nonzero = keep) or None.  Returns the update [N, N, CZ]:
        t[i, j, c] = sum_k keep[k] a[i, k, c] b[j, k, c]   (outgoing)
        t[i, j, c] = sum_k keep[k] a[k, i, c] b[k, j, c]   (incoming)
        out[i, j]  = t[i, j] . w_o^T + b_o,
    with a = LN(z) . w_a^T and b = LN(z) . w_b^T."""
    z = np.asarray(z, np.float64)
    N = z.shape[0]
    x = layer_norm(z, ln_w, ln_b, eps)
    a = x @ w_a.T                        # a[p, q] = projection of edge (p, q)
    b = x @ w_b.T
    keep = (np.ones(N) if residue_mask is None
            else (np.asarray(residue_mask) != 0).astype(np.float64))
    C = a.shape[-1]
    Ac, Bc = _channel_matrices(a, b, outgoing)
    t = np.empty((N, N, C))
    for c in range(C):
        t[:, :, c] = (Ac[c] * keep) @ Bc[c].T
    return t @ w_o.T + b_o


def _channel_matrices(a, b, outgoing):
    """Per channel c the matrices A_c[i, k] and B_c[j, k] of the update:
    a[i, k, c] and b[j, k, c] (edges (i, k), (j, k)) for outgoing, a[k, i, c]
    and b[k, j, c] for incoming; each channel's matrix is a contiguous copy,
    so that the library matrix product serves it."""
    perm = (2, 0, 1) if outgoing else (2, 1, 0)
    return (np.ascontiguousarray(a.transpose(perm)),
            np.ascontiguousarray(b.transpose(perm)))


def tri_mul_entries(z, residue_mask, ln_w, ln_b, eps, w_a, w_b, w_o, b_o,
                    picks, outgoing=True):
    """out[i, j] of tri_mul_forward for the (i, j) pairs in `picks` only: the
    same definition, with the projections formed for the edges those entries
    need (rows i and j for outgoing, columns for incoming), so that a few
    entries of a large problem stay cheap.  Returns [len(picks), CZ]."""
    z = np.asarray(z, np.float64)
    N = z.shape[0]
    keep = (np.ones(N) if residue_mask is None
            else (np.asarray(residue_mask) != 0).astype(np.float64))
    res = []
    for i, j in picks:
        # edges (i, k) and (j, k), or (k, i) and (k, j)
        ei = z[i] if outgoing else z[:, i]
        ej = z[j] if outgoing else z[:, j]
        a = layer_norm(ei, ln_w, ln_b, eps) @ w_a.T       # [N, C]
        b = layer_norm(ej, ln_w, ln_b, eps) @ w_b.T
        t = (keep[:, None] * a * b).sum(axis=0)
        res.append(t @ w_o.T + b_o)
    return np.stack(res)


def tri_mul_backward(z, residue_mask, ln_w, ln_b, eps, w_a, w_b, w_o, b_o,
                     dout, outgoing=True):
    """Gradients of tri_mul_forward for training.  The pages print no backward
    (the update is part of the trained trunk, [COURSE] "The three
    operations"); this is the chain rule of the forward above, nothing else.
    With A_c[i, k] = a[i, k, c] (outgoing; a[k, i, c] incoming), B_c
    likewise, keep the residue mask and dT_c[i, j] = (dout . w_o)[i, j, c]:
        dA_c = (dT_c . B_c) * keep[k],   dB_c = (dT_c^T . A_c) * keep[k],
        dx   = da . w_a + db . w_b,      dz   = LayerNorm backward of dx,
        dw_a = sum_p da[p]^T x[p],  dw_b likewise,
        dw_o = sum_p dout[p]^T t[p],  db_o = sum_p dout[p].
    Returns dict(dz, dln_w, dln_b, dw_a, dw_b, dw_o, db_o)."""
    z = np.asarray(z, np.float64)
    N, _, CZ = z.shape
    dout = np.asarray(dout, np.float64)
    x = layer_norm(z, ln_w, ln_b, eps)
    a = x @ w_a.T
    b = x @ w_b.T
    C = a.shape[-1]
    keep = (np.ones(N) if residue_mask is None
            else (np.asarray(residue_mask) != 0).astype(np.float64))
    dt = dout @ w_o                       # [N, N, C]
    dtc = np.ascontiguousarray(dt.transpose(2, 0, 1))     # dT_c[i, j]
    Ac, Bc = _channel_matrices(a, b, outgoing)            # A_c[i, k], B_c[j, k]
    t = np.empty((N, N, C))
    da = np.empty((N, N, C))
    db = np.empty((N, N, C))
    for c in range(C):
        t[:, :, c] = (Ac[c] * keep) @ Bc[c].T
        dA = (dtc[c] @ Bc[c]) * keep                      # dA[i, k]
        dB = (dtc[c].T @ Ac[c]) * keep                    # dB[j, k]
        da[:, :, c] = dA if outgoing else dA.T
        db[:, :, c] = dB if outgoing else dB.T
    dx = da @ w_a + db @ w_b
    dz, dln_w, dln_b = layer_norm_backward(z, ln_w, eps, dx)
    flat = lambda v: v.reshape(-1, v.shape[-1])
    return dict(dz=dz, dln_w=dln_w, dln_b=dln_b,
                dw_a=flat(da).T @ flat(x), dw_b=flat(db).T @ flat(x),
                dw_o=flat(dout).T @ flat(t), db_o=flat(dout).sum(axis=0))


def tri_mul_backward_entries(z, residue_mask, ln_w, ln_b, eps, w_a, w_b, w_o,
                             dout, picks, outgoing=True):
    """dz[p] of tri_mul_backward at the z positions p = (i, k) in `picks`
    only: the same chain rule with da[p] and db[p] formed for those
    positions alone.  For outgoing, da[i, k] needs dT[i, :] (row i of dout)
    and b on the edges (j, k) for all j; db[i, k] (as B's edge (j=i, k))
    needs dT[:, i] and a on the edges (j, k) ... of every j.  Incoming swaps
    the edge indices.  Returns [len(picks), CZ]."""
    z = np.asarray(z, np.float64)
    N = z.shape[0]
    dout = np.asarray(dout, np.float64)
    keep = (np.ones(N) if residue_mask is None
            else (np.asarray(residue_mask) != 0).astype(np.float64))
    res = []
    for p0, p1 in picks:
        # the edge's (row, third residue) in the A/B matrices
        r, k = (p0, p1) if outgoing else (p1, p0)
        # edges (j, k) for every j: z[j, k] (outgoing) or z[k, j] (incoming)
        ek = z[:, k] if outgoing else z[k, :]
        xk = layer_norm(ek, ln_w, ln_b, eps)              # [N(j), CZ]
        a_k = xk @ w_a.T                                  # A_c[j, k] over j
        b_k = xk @ w_b.T                                  # B_c[j, k] over j
        dT_row = dout[r, :, :] @ w_o                      # dT_c[r, j] over j
        dT_col = dout[:, r, :] @ w_o                      # dT_c[i, r] over i
        da = keep[k] * (dT_row * b_k).sum(axis=0)         # dA_c[r, k]
        db = keep[k] * (dT_col * a_k).sum(axis=0)         # dB_c[r, k]
        dx = da @ w_a + db @ w_b
        zp = z[p0, p1]
        dzp, _, _ = layer_norm_backward(zp[None], ln_w, eps, dx[None])
        res.append(dzp[0])
    return np.stack(res)


# ----------------------------------------------------------------------------
# LayerNorm + linear + SwiGLU transition.
#
# [MEGAFOLD] item 3 "EvoFusion" fuses layer normalisation, the linear
# projections and the SwiGLU activations so that no N x N intermediate is
# written between them.  The pages do not write the transition out; the
# reading taken is the plain SwiGLU feed-forward block on the layer-normalised
# pair representation, without bias vectors:
#     x = LN(z),  h = silu(x . w_a^T) * (x . w_b^T),  out = h . w_o^T
# with silu(u) = u * sigmoid(u) and a hidden width of w_a.shape[0].
# ----------------------------------------------------------------------------

def transition_forward(z, ln_w, ln_b, eps, w_a, w_b, w_o):
    """z [..., CZ]; w_a, w_b [HID, CZ]; w_o [CZ, HID].  Returns [..., CZ]."""
    x = layer_norm(z, ln_w, ln_b, eps)
    u = x @ w_a.T
    h = u * sigmoid(u) * (x @ w_b.T)
    return h @ w_o.T


def transition_backward(z, ln_w, ln_b, eps, w_a, w_b, w_o, dout):
    """Gradients of transition_forward (training, as EvoFusion's scope of
    LayerNorm, projections and SwiGLU implies): the chain rule of
        x = LN(z), u = x w_a^T, v = x w_b^T, h = silu(u) v, out = h w_o^T
    with silu(u) = u sigmoid(u), silu'(u) = sigmoid(u) (1 + u (1 - sigmoid(u))):
        dh = dout w_o,  du = dh v silu'(u),  dv = dh silu(u),
        dx = du w_a + dv w_b,  dz = LayerNorm backward of dx,
        dw_o = sum_p dout^T h,  dw_a = sum_p du^T x,  dw_b = sum_p dv^T x.
    z, dout [..., CZ].  Returns a dict of dz (like z), dln_w, dln_b [CZ],
    dw_a, dw_b [HID, CZ] and dw_o [CZ, HID]."""
    z = np.asarray(z, np.float64)
    dout = np.asarray(dout, np.float64)
    CZ = z.shape[-1]
    x = layer_norm(z, ln_w, ln_b, eps).reshape(-1, CZ)
    dy = dout.reshape(-1, CZ)
    u = x @ w_a.T
    v = x @ w_b.T
    sg = sigmoid(u)
    silu = u * sg
    h = silu * v
    dh = dy @ w_o
    dv = dh * silu
    du = dh * v * sg * (1.0 + u * (1.0 - sg))
    dx = du @ w_a + dv @ w_b
    dz, dln_w, dln_b = layer_norm_backward(z.reshape(-1, CZ), ln_w, eps, dx)
    return dict(dz=dz.reshape(z.shape), dln_w=dln_w, dln_b=dln_b,
                dw_a=du.T @ x, dw_b=dv.T @ x, dw_o=dy.T @ h)


def transition_weight_grad_units(z, ln_w, ln_b, eps, w_a, w_b, w_o, dout, units):
    """Rows dw_a[k], dw_b[k] and columns dw_o[:, k] of transition_backward for
    the hidden units k in `units` only, over every position: each unit's
    u, v and dh are formed for that unit alone (the same chain rule).
    Returns arrays [len(units), CZ] (dw_a, dw_b) and [CZ, len(units)]
    (dw_o)."""
    z = np.asarray(z, np.float64)
    CZ = z.shape[-1]
    x = layer_norm(z, ln_w, ln_b, eps).reshape(-1, CZ)
    dy = np.asarray(dout, np.float64).reshape(-1, CZ)
    ra, rb, ro = [], [], []
    for k in units:
        u = x @ w_a[k]
        v = x @ w_b[k]
        sg = sigmoid(u)
        dh = dy @ w_o[:, k]
        ra.append((dh * v * sg * (1.0 + u * (1.0 - sg))) @ x)
        rb.append((dh * u * sg) @ x)
        ro.append(dy.T @ (u * sg * v))
    return np.stack(ra), np.stack(rb), np.stack(ro, axis=1)


# ----------------------------------------------------------------------------
# Outer product mean.
#
# [COURSE] "The three operations": the bridge from the MSA to the pair
# representation averages, over all sequences, the outer product of MSA
# columns i and j.  Reading (the pages give no formula): the MSA
# representation m [S, N, c_m] is layer-normalised and projected to two
# c-channel vectors per (sequence, residue), a = LN(m) . w_a^T and
# b = LN(m) . w_b^T (no bias); for every residue pair
#     o[i, j, c, d] = (1/S) sum_s a[s, i, c] b[s, j, d],
# flattened with d fastest and projected to c_z with an output bias:
#     out[i, j] = o[i, j].reshape(c*c) . w_o^T + b_o.
# ----------------------------------------------------------------------------

def outer_product_mean(m, ln_w, ln_b, eps, w_a, w_b, w_o, b_o):
    """m [S, N, CM]; w_a, w_b [C, CM]; w_o [CZ, C*C]; b_o [CZ].
    Returns [N, N, CZ]."""
    m = np.asarray(m, np.float64)
    S, N, _ = m.shape
    x = layer_norm(m, ln_w, ln_b, eps)
    a = x @ w_a.T                                   # [S, N, C]
    b = x @ w_b.T
    C = a.shape[-1]
    # o[i, j, c, d]: one residue i at a time (memory N^2 C^2)
    out = np.empty((N, N, w_o.shape[0]))
    for i in range(N):
        o_i = np.einsum("sc,sjd->jcd", a[:, i, :], b) / S   # [N, C, C]
        out[i] = o_i.reshape(N, C * C) @ w_o.T + b_o
    return out


def outer_product_mean_backward(m, ln_w, ln_b, eps, w_a, w_b, w_o, b_o, dout):
    """Gradients of outer_product_mean for training.  The pages print no
    backward (the bridge is part of the trained trunk, [COURSE] "The three
    operations"); this is the chain rule of the forward above, nothing else.
    With P[i, j, c, d] = sum_s a[s, i, c] b[s, j, d] and
    dO[i, j, c, d] = (dout[i, j] . w_o)[c*C + d] / S:
        da[s, i, c] = sum_{j, d} dO[i, j, c, d] b[s, j, d],
        db[s, j, d] = sum_{i, c} dO[i, j, c, d] a[s, i, c],
        dx = da . w_a + db . w_b,  dm = LayerNorm backward of dx,
        dw_a = sum_{s, i} da^T x,  dw_b likewise,
        dw_o = sum_{i, j} dout[i, j]^T flatten(P[i, j]) / S,  db_o = sum dout.
    Returns dict(dm, dln_w, dln_b, dw_a, dw_b, dw_o, db_o)."""
    m = np.asarray(m, np.float64)
    S, N, CM = m.shape
    dout = np.asarray(dout, np.float64)
    x = layer_norm(m, ln_w, ln_b, eps)
    a = x @ w_a.T                                   # [S, N, C]
    b = x @ w_b.T
    C = a.shape[-1]
    CZ = w_o.shape[0]
    dO = (dout @ w_o).reshape(N, N, C, C) / S       # [i, j, c, d]
    # the [N*C, S] operand matrices of the forward: rows (i, c), columns s
    A = a.transpose(1, 2, 0).reshape(N * C, S)
    B = b.transpose(1, 2, 0).reshape(N * C, S)
    dP = dO.transpose(0, 2, 1, 3).reshape(N * C, N * C)   # rows (i, c), cols (j, d)
    dA = dP @ B                                     # [(i, c), s]
    dB = dP.T @ A                                   # [(j, d), s]
    da = dA.reshape(N, C, S).transpose(2, 0, 1)     # [s, i, c]
    db = dB.reshape(N, C, S).transpose(2, 0, 1)
    dx = da @ w_a + db @ w_b
    dm, dln_w, dln_b = layer_norm_backward(m, ln_w, eps, dx)
    P = (A @ B.T).reshape(N, C, N, C).transpose(0, 2, 1, 3)   # [i, j, c, d]
    flat = lambda v: v.reshape(-1, v.shape[-1])
    dw_o = flat(dout).T @ P.reshape(N * N, C * C) / S
    return dict(dm=dm, dln_w=dln_w, dln_b=dln_b,
                dw_a=flat(da).T @ flat(x), dw_b=flat(db).T @ flat(x),
                dw_o=dw_o, db_o=flat(dout).sum(axis=0))


def outer_product_mean_backward_sampled(m, ln_w, ln_b, eps, w_a, w_b, w_o, dout,
                                        dm_picks, wa_rows, wb_rows, wo_cols):
    """Parts of outer_product_mean_backward that a few channels or
    positions determine, each formed from the same chain rule for those
    alone (so that a large problem stays cheap):
      dm[s, i] for (s, i) in dm_picks (da[s, i] needs dO[i, :] and b[s, :],
               db[s, i] needs dO[:, i] and a[s, :]),
      dw_a[c] for c in wa_rows (da[:, :, c] over every (s, i)),
      dw_b[d] for d in wb_rows,
      dw_o[:, c*C + d] for (c, d) in wo_cols (P[:, :, c, d] alone).
    Returns (dm [len(dm_picks), CM], dw_a rows, dw_b rows, dw_o columns
    [CZ, len(wo_cols)])."""
    m = np.asarray(m, np.float64)
    S, N, CM = m.shape
    dout = np.asarray(dout, np.float64)
    x = layer_norm(m, ln_w, ln_b, eps)
    a = x @ w_a.T                                   # [S, N, C]
    b = x @ w_b.T
    C = a.shape[-1]
    wo4 = w_o.reshape(-1, C, C)                     # [CZ, c, d]
    dm = []
    for s_, i in dm_picks:
        dO_row = np.einsum("jz,zcd->jcd", dout[i], wo4) / S     # dO[i, j, c, d]
        dO_col = np.einsum("jz,zcd->jcd", dout[:, i], wo4) / S  # dO[j, i, c, d]
        da = np.einsum("jcd,jd->c", dO_row, b[s_])
        db = np.einsum("jcd,jc->d", dO_col, a[s_])
        dx = da @ w_a + db @ w_b
        g, _, _ = layer_norm_backward(m[s_, i][None], ln_w, eps, dx[None])
        dm.append(g[0])
    xf = x.reshape(-1, CM)
    bf = b.reshape(S, N * C)                        # b[s, (j, d)]
    ra = []
    for c in wa_rows:
        dO_c = (dout @ wo4[:, c, :]) / S            # dO[i, j, c, d] over (i, j, d)
        da_c = bf @ dO_c.reshape(N, N * C).T        # da[s, i, c]: sum over (j, d)
        ra.append(da_c.reshape(-1) @ xf)
    af = a.reshape(S, N * C)                        # a[s, (i, c)]
    rb = []
    for d_ in wb_rows:
        dO_d = (dout @ wo4[:, :, d_]) / S           # dO[i, j, c, d] over (i, j, c)
        dO_t = dO_d.transpose(1, 0, 2).reshape(N, N * C)    # [j, (i, c)]
        db_d = af @ dO_t.T                          # db[s, j, d]: sum over (i, c)
        rb.append(db_d.reshape(-1) @ xf)
    ro = []
    for c, d_ in wo_cols:
        P_cd = a[:, :, c].T @ b[:, :, d_]           # P[i, j, c, d]
        ro.append(dout.reshape(N * N, -1).T @ P_cd.reshape(-1) / S)
    return np.stack(dm), np.stack(ra), np.stack(rb), np.stack(ro, axis=1)


def outer_product_mean_pairs(m, ln_w, ln_b, eps, w_a, w_b, w_o, b_o, picks):
    """out[i, j] of outer_product_mean for the (i, j) pairs in `picks` only,
    with the projections formed for residues i and j alone.  Returns
    [len(picks), CZ]."""
    m = np.asarray(m, np.float64)
    S = m.shape[0]
    res = []
    for i, j in picks:
        a = layer_norm(m[:, i], ln_w, ln_b, eps) @ w_a.T    # [S, C]
        b = layer_norm(m[:, j], ln_w, ln_b, eps) @ w_b.T
        o = a.T @ b / S                                      # [C, C]
        res.append(o.reshape(-1) @ w_o.T + b_o)
    return np.stack(res)
