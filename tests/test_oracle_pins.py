"""Pins for the fp64 oracle: each check ties it to something other than
itself (a library routine, a closed form, an invariant, brute force), and the
mutation tests at the end show that a planted mistake in the oracle fails at
least one of them.  CPU only."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import expit

import oracle.evo_oracle as O


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def core_case(seed, B=2, R=3, N=9, H=2, C=4, mask=True, gate=True, bias=True,
              mask_rows=1):
    rng = np.random.default_rng(seed)
    d = dict(q=rng.standard_normal((B, R, N, H, C)),
             k=rng.standard_normal((B, R, N, H, C)),
             v=rng.standard_normal((B, R, N, H, C)))
    d["gate"] = rng.standard_normal((B, R, N, H, C)) if gate else None
    d["bias"] = rng.standard_normal((B, H, N, N)) if bias else None
    if mask:
        m = (rng.random((B, mask_rows, N)) < 0.7).astype(np.uint8)
        m[..., 0] = 1  # at least one live key per line
        d["key_mask"] = m
    else:
        d["key_mask"] = None
    return d


def fwd(d):
    return O.attention_forward(d["q"], d["k"], d["v"], d["gate"],
                               d["key_mask"], d["bias"])


# ----------------------------------------------------------------- forward

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_probs_rows_sum_to_one_and_masked_keys_zero(seed):
    d = core_case(seed)
    keep = d["key_mask"][0, 0] != 0
    P = O.attention_line_probs(d["q"][0, 0], d["k"][0, 0], d["bias"][0], keep)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-13)
    assert np.all(P[:, :, ~keep] == 0)
    assert np.all(P >= 0)


def test_values_all_one_give_output_one():
    d = core_case(3, gate=False)
    d["v"] = np.ones_like(d["v"])
    out, _ = fwd(d)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("with_bias,with_mask", [(False, False), (True, False),
                                                 (True, True), (False, True)])
def test_matches_torch_sdpa(with_bias, with_mask):
    """Library routine: torch's scaled_dot_product_attention (fp64, CPU)
    adds a float attn_mask [query, key] to QK^T/sqrt(C) before the softmax."""
    d = core_case(4, B=2, R=2, N=11, H=3, C=8, gate=False, bias=with_bias,
                  mask=with_mask, mask_rows=2)
    out, _ = fwd(d)
    B, R, N, H, C = d["q"].shape
    for b in range(B):
        for r in range(R):
            q = torch.tensor(d["q"][b, r]).permute(1, 0, 2)  # [H, N, C]
            k = torch.tensor(d["k"][b, r]).permute(1, 0, 2)
            v = torch.tensor(d["v"][b, r]).permute(1, 0, 2)
            am = torch.zeros(H, N, N, dtype=torch.float64)
            if with_bias:
                am = am + torch.tensor(d["bias"][b])
            if with_mask:
                keep = torch.tensor(d["key_mask"][b, r] != 0)
                am = am.masked_fill(~keep[None, None, :], float("-inf"))
            ref = F.scaled_dot_product_attention(q, k, v, attn_mask=am)
            np.testing.assert_allclose(out[b, r], ref.permute(1, 0, 2).numpy(),
                                       rtol=1e-12, atol=1e-12)


def test_zero_query_log_weight_bias_closed_form():
    """Q = 0 and bias[h,q,k] = ln w_k  =>  O = sum_k w_k V_k / sum_k w_k and
    LSE = ln sum_k w_k."""
    d = core_case(5, gate=False, mask=False)
    B, R, N, H, C = d["q"].shape
    d["q"] = np.zeros_like(d["q"])
    w = np.random.default_rng(5).uniform(0.1, 3.0, (B, H, N))
    d["bias"] = np.broadcast_to(np.log(w)[:, :, None, :], (B, H, N, N)).copy()
    out, lse = fwd(d)
    for b in range(B):
        for h in range(H):
            expect = (w[b, h][None, :, None] * d["v"][b, :, :, h, :]
                      ).sum(1) / w[b, h].sum()               # [R, C]
            np.testing.assert_allclose(out[b, :, :, h, :],
                                       np.broadcast_to(expect[:, None, :],
                                                       (R, N, C)),
                                       rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[b, :, h, :], np.log(w[b, h].sum()),
                                       rtol=1e-13)


def test_zero_query_zero_bias_is_masked_mean():
    d = core_case(6, gate=False, bias=False, mask=True, mask_rows=3)
    d["q"] = np.zeros_like(d["q"])
    out, lse = fwd(d)
    B, R, N, H, C = d["q"].shape
    for b in range(B):
        for r in range(R):
            keep = d["key_mask"][b, r] != 0
            mean = d["v"][b, r][keep].mean(axis=0)            # [H, C]
            np.testing.assert_allclose(out[b, r], np.broadcast_to(mean, (N, H, C)),
                                       rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[b, r], np.log(keep.sum()), rtol=1e-13)


def test_single_live_key_returns_its_value_gated():
    d = core_case(7)
    B, R, N, H, C = d["q"].shape
    m = np.zeros((B, 1, N), np.uint8)
    m[0, 0, 4] = 1
    m[1, 0, 7] = 1
    d["key_mask"] = m
    out, _ = fwd(d)
    for b, kk in ((0, 4), (1, 7)):
        expect = expit(d["gate"][b]) * d["v"][b][:, kk][:, None, :, :]
        np.testing.assert_allclose(out[b], expect, rtol=1e-12, atol=1e-12)


def test_fully_masked_line_is_zero_with_neg_inf_lse():
    d = core_case(8, mask_rows=3)
    d["key_mask"][1, 2, :] = 0
    out, lse = fwd(d)
    assert np.all(out[1, 2] == 0)
    assert np.all(np.isneginf(lse[1, 2]))
    assert np.all(np.isfinite(lse[0]))


def test_key_permutation_with_bias_columns_is_invariant():
    d = core_case(9, mask_rows=3)
    out, lse = fwd(d)
    perm = np.random.default_rng(9).permutation(d["q"].shape[2])
    e = dict(d)
    e["k"] = d["k"][:, :, perm]
    e["v"] = d["v"][:, :, perm]
    e["bias"] = d["bias"][..., perm]
    e["key_mask"] = d["key_mask"][..., perm]
    out2, lse2 = fwd(e)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-12)


def test_query_permutation_with_bias_rows_permutes_output():
    d = core_case(10)
    out, lse = fwd(d)
    perm = np.random.default_rng(10).permutation(d["q"].shape[2])
    e = dict(d)
    e["q"] = d["q"][:, :, perm]
    e["gate"] = d["gate"][:, :, perm]
    e["bias"] = d["bias"][:, :, perm, :]
    out2, lse2 = fwd(e)
    np.testing.assert_allclose(out2, out[:, :, perm], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lse[..., perm], rtol=1e-12, atol=1e-12)


def test_row_permutation_permutes_output():
    """The order of the rows (MSA sequences / pair rows) carries nothing:
    permuting them permutes the output ("Two properties the tests assert")."""
    d = core_case(11, R=4, mask_rows=4)
    out, _ = fwd(d)
    perm = np.array([2, 0, 3, 1])
    e = {k: (None if v is None else v[:, perm] if k != "bias" else v)
         for k, v in d.items()}
    out2, _ = fwd(e)
    np.testing.assert_allclose(out2, out[:, perm], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shift", [3.5, 1e4, -1e4])
def test_softmax_shift_invariance(shift):
    d = core_case(12)
    out, lse = fwd(d)
    e = dict(d)
    sh = shift * (1 + np.random.default_rng(12).random(d["bias"].shape[:3]))
    e["bias"] = d["bias"] + sh[..., None]
    out2, lse2 = fwd(e)
    np.testing.assert_allclose(out2, out, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(lse2 - sh.transpose(0, 1, 2)[:, None],
                               lse, rtol=1e-9, atol=1e-7 * abs(shift))


def test_gate_is_elementwise_sigmoid():
    d = core_case(13)
    out, _ = fwd(d)
    e = dict(d)
    e["gate"] = None
    out_ng, _ = fwd(e)
    np.testing.assert_allclose(out, expit(d["gate"]) * out_ng, rtol=1e-13,
                               atol=1e-14)
    np.testing.assert_allclose(O.sigmoid(np.array([-800.0, 0.0, 800.0])),
                               [0.0, 0.5, 1.0])


# ---------------------------------------------------------------- backward

def loss_and_grads(d, dout):
    out, _ = fwd(d)
    return float((out * dout).sum())


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_central_finite_differences(seed):
    """Brute force: every gradient entry against a central difference of the
    scalar <dOut, Out> (fp64, step 1e-6) on a tiny problem."""
    d = core_case(100 + seed, B=1, R=2, N=5, H=2, C=3, mask_rows=2)
    dout = rnd(200 + seed, *d["q"].shape)
    dq, dk, dv, dg, dbias = O.attention_backward(
        d["q"], d["k"], d["v"], d["gate"], d["key_mask"], d["bias"], dout)
    grads = dict(q=dq, k=dk, v=dv, gate=dg, bias=dbias)
    eps = 1e-6
    for name, g in grads.items():
        base = d[name]
        num = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            e = dict(d)
            plus = base.copy(); plus[idx] += eps
            minus = base.copy(); minus[idx] -= eps
            e[name] = plus
            lp = loss_and_grads(e, dout)
            e[name] = minus
            lm = loss_and_grads(e, dout)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8,
                                   err_msg=f"gradient of {name}")


def test_backward_matches_torch_autograd():
    """Library routine: torch.autograd through softmax/sigmoid (fp64, CPU)."""
    d = core_case(14, B=2, R=3, N=13, H=3, C=8, mask_rows=3)
    dout = rnd(15, *d["q"].shape)
    dq, dk, dv, dg, dbias = O.attention_backward(
        d["q"], d["k"], d["v"], d["gate"], d["key_mask"], d["bias"], dout)
    t = {k: torch.tensor(d[k], requires_grad=True)
         for k in ("q", "k", "v", "gate", "bias")}
    C = d["q"].shape[-1]
    s = torch.einsum("brqhc,brkhc->brhqk", t["q"], t["k"]) / C ** 0.5
    s = s + t["bias"][:, None]
    keep = torch.tensor(d["key_mask"] != 0)[:, :, None, None, :]
    s = s.masked_fill(~keep, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("brhqk,brkhc->brqhc", p, t["v"]) * torch.sigmoid(t["gate"])
    (o * torch.tensor(dout)).sum().backward()
    for name, g in dict(q=dq, k=dk, v=dv, gate=dg, bias=dbias).items():
        np.testing.assert_allclose(g, t[name].grad.numpy(), rtol=1e-10,
                                   atol=1e-12, err_msg=name)


def test_backward_closed_forms():
    """Sum_k dBias[h,q,k] = 0 (softmax Jacobian annihilates constants),
    Sum_k dK[k] = 0 (adding a constant vector to every key shifts each
    query's logits uniformly), Sum_k dV[k] = Sum_q dO_pre[q] (rows of P sum
    to one)."""
    d = core_case(16, B=1, R=4, N=10, H=2, C=4)
    dout = rnd(17, *d["q"].shape)
    dq, dk, dv, dg, dbias = O.attention_backward(
        d["q"], d["k"], d["v"], d["gate"], d["key_mask"], d["bias"], dout)
    np.testing.assert_allclose(dbias.sum(-1), 0, atol=1e-12)
    np.testing.assert_allclose(dk.sum(2), 0, atol=1e-12)
    do_pre = dout * expit(d["gate"])
    np.testing.assert_allclose(dv.sum(2), do_pre.sum(2), rtol=1e-12, atol=1e-12)


def test_dbias_query_rows_matches_full_backward():
    d = core_case(18, B=2, R=3, N=8, H=2, C=4, mask_rows=3)
    dout = rnd(19, *d["q"].shape)
    _, _, _, _, dbias = O.attention_backward(
        d["q"], d["k"], d["v"], d["gate"], d["key_mask"], d["bias"], dout)
    picks = [(0, 0), (1, 5), (0, 7)]
    for b in range(2):
        got = O.dbias_query_rows(d["q"], d["k"], d["v"], d["gate"],
                                 d["key_mask"], d["bias"], dout, b, picks)
        for t, (h, qi) in enumerate(picks):
            np.testing.assert_allclose(got[t], dbias[b, h, qi], rtol=1e-12,
                                       atol=1e-13)


# ------------------------------------------------------------------ module

def module_case(seed, N=7, CZ=12, H=2, C=3, mask=True):
    rng = np.random.default_rng(seed)
    HC = H * C
    d = dict(z=rng.standard_normal((N, N, CZ)),
             ln_w=1 + 0.2 * rng.standard_normal(CZ),
             ln_b=0.2 * rng.standard_normal(CZ), eps=1e-5,
             w_q=rng.standard_normal((HC, CZ)) / CZ ** 0.5,
             w_k=rng.standard_normal((HC, CZ)) / CZ ** 0.5,
             w_v=rng.standard_normal((HC, CZ)) / CZ ** 0.5,
             w_g=rng.standard_normal((HC, CZ)) / CZ ** 0.5,
             b_g=0.3 * rng.standard_normal(HC),
             w_bias=rng.standard_normal((H, CZ)) / CZ ** 0.5,
             w_o=rng.standard_normal((CZ, HC)) / HC ** 0.5,
             b_o=0.3 * rng.standard_normal(CZ), H=H, C=C)
    if mask:
        m = (rng.random(N) < 0.7).astype(np.uint8)
        m[0] = 1
        d["residue_mask"] = m
    else:
        d["residue_mask"] = None
    return d


def module(d, ending, z=None, mask="same"):
    args = dict(d)
    if z is not None:
        args["z"] = z
    if not (isinstance(mask, str) and mask == "same"):
        args["residue_mask"] = mask
    return O.tri_module_forward(ending=ending, **args)


def test_layer_norm_matches_torch():
    x = rnd(20, 5, 6, 17)
    w, b = rnd(21, 17), rnd(22, 17)
    ref = F.layer_norm(torch.tensor(x), (17,), torch.tensor(w), torch.tensor(b),
                       1e-5).numpy()
    np.testing.assert_allclose(O.layer_norm(x, w, b, 1e-5), ref, rtol=1e-12,
                               atol=1e-12)


@pytest.mark.parametrize("masked", [False, True])
def test_ending_node_is_transposed_starting_node(masked):
    """Column-wise reading (line = column j, bias b_ki) agrees with the
    transposition reading: end(z) = T(start(T(z)))."""
    d = module_case(23, mask=masked)
    end = module(d, True)
    zt = d["z"].transpose(1, 0, 2)
    start_t = module(d, False, z=zt)
    np.testing.assert_allclose(end, start_t.transpose(1, 0, 2), rtol=1e-12,
                               atol=1e-12)


@pytest.mark.parametrize("ending", [False, True])
def test_residue_permutation_equivariance(ending):
    """Relabelling residues permutes the output identically, f(P z P^T) =
    P f(z) P^T, with the residue mask permuted alike ("Two properties the
    tests assert": residue-permutation equivariance)."""
    d = module_case(24)
    out = module(d, ending)
    perm = np.random.default_rng(24).permutation(d["z"].shape[0])
    zp = d["z"][perm][:, perm]
    outp = module(d, ending, z=zp, mask=d["residue_mask"][perm])
    np.testing.assert_allclose(outp, out[perm][:, perm], rtol=1e-11,
                               atol=1e-12)


@pytest.mark.parametrize("ending", [False, True])
def test_module_equals_project_core_outproject(ending):
    d = module_case(25)
    H, C = d["H"], d["C"]
    q, k, v, g, bias = O.tri_project(d["z"], d["ln_w"], d["ln_b"], d["eps"],
                                     d["w_q"], d["w_k"], d["w_v"], d["w_g"],
                                     d["b_g"], d["w_bias"], H, C, ending)
    N = d["z"].shape[0]
    km = d["residue_mask"][None, None, :]
    o, _ = O.attention_forward(q, k, v, g, km, bias)
    out = O.tri_out_project(o, d["w_o"], d["b_o"], ending)
    np.testing.assert_allclose(out, module(d, ending), rtol=1e-12, atol=1e-12)
    # and the project layout itself against plain per-position matmuls
    x = O.layer_norm(d["z"], d["ln_w"], d["ln_b"], d["eps"])
    i, j = 2, 5
    qi = (x[i, j] @ d["w_q"].T).reshape(H, C)
    line, pos = (j, i) if ending else (i, j)
    np.testing.assert_allclose(q[0, line, pos], qi, rtol=1e-12, atol=1e-13)
    bij = x[i, j] @ d["w_bias"].T
    # starting: bias[h, j', k'] = b_{j'k'} ; ending: bias[h, i', k'] = b_{k'i'}
    if ending:
        np.testing.assert_allclose(bias[0, :, j, i], bij, rtol=1e-12)
    else:
        np.testing.assert_allclose(bias[0, :, i, j], bij, rtol=1e-12)
    assert N == q.shape[1]


def test_projection_matches_torch_linear():
    """Library routine: torch.nn.functional.layer_norm + linear (fp64)."""
    d = module_case(28)
    H, C = d["H"], d["C"]
    q, k, v, g, bias = O.tri_project(d["z"], d["ln_w"], d["ln_b"], d["eps"],
                                     d["w_q"], d["w_k"], d["w_v"], d["w_g"],
                                     d["b_g"], d["w_bias"], H, C, False)
    z = torch.tensor(d["z"])
    x = F.layer_norm(z, (z.shape[-1],), torch.tensor(d["ln_w"]),
                     torch.tensor(d["ln_b"]), d["eps"])
    N = z.shape[0]
    for got, w, bvec in ((q, "w_q", None), (g, "w_g", "b_g")):
        ref = F.linear(x, torch.tensor(d[w]),
                       None if bvec is None else torch.tensor(d[bvec]))
        np.testing.assert_allclose(got[0].reshape(N, N, H * C), ref.numpy(),
                                   rtol=1e-12, atol=1e-12)
    refb = F.linear(x, torch.tensor(d["w_bias"])).permute(2, 0, 1).numpy()
    np.testing.assert_allclose(bias[0], refb, rtol=1e-12, atol=1e-12)
    o = np.random.default_rng(29).standard_normal((1, N, N, H, C))
    ref = F.linear(torch.tensor(o[0]).reshape(N, N, H * C),
                   torch.tensor(d["w_o"]), torch.tensor(d["b_o"])).numpy()
    np.testing.assert_allclose(O.tri_out_project(o, d["w_o"], d["b_o"], False),
                               ref, rtol=1e-12, atol=1e-12)


def test_module_lines_subset():
    d = module_case(26)
    full = module(d, True)
    sub = O.tri_module_lines(lines=[1, 4], ending=True, **d)
    np.testing.assert_allclose(sub[0], full[:, 1], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(sub[1], full[:, 4], rtol=1e-13, atol=1e-13)


# -------------------------------------------------------- planted mistakes

def _sdpa_pin(monkeypatch=None):
    try:
        test_matches_torch_sdpa(True, True)
        return True
    except AssertionError:
        return False


def test_mutant_scale_omitted_is_caught(monkeypatch):
    orig = O._line_logits

    def no_scale(q, k, bias, keep, h):
        return orig(q * np.sqrt(q.shape[-1]), k, bias, keep, h)
    monkeypatch.setattr(O, "_line_logits", no_scale)
    assert not _sdpa_pin()


def test_mutant_bias_transposed_is_caught(monkeypatch):
    orig = O._line_logits

    def bias_t(q, k, bias, keep, h):
        return orig(q, k, None if bias is None else bias.transpose(0, 2, 1),
                    keep, h)
    monkeypatch.setattr(O, "_line_logits", bias_t)
    assert not _sdpa_pin()
    with pytest.raises(AssertionError):
        test_key_permutation_with_bias_columns_is_invariant()


def test_mutant_mask_ignored_is_caught(monkeypatch):
    orig = O._line_logits
    monkeypatch.setattr(O, "_line_logits",
                        lambda q, k, bias, keep, h: orig(q, k, bias, None, h))
    with pytest.raises(AssertionError):
        test_single_live_key_returns_its_value_gated()


def test_mutant_gate_not_squashed_is_caught(monkeypatch):
    monkeypatch.setattr(O, "sigmoid", lambda x: np.asarray(x, np.float64))
    with pytest.raises(AssertionError):
        test_single_live_key_returns_its_value_gated()


def test_mutant_softmax_over_queries_is_caught(monkeypatch):
    orig = O._line_logits
    monkeypatch.setattr(O, "_line_logits",
                        lambda q, k, bias, keep, h: orig(q, k, bias, keep, h).T)
    assert not _sdpa_pin()


def test_mutant_dbias_one_row_is_caught(monkeypatch):
    orig = O.attention_line_backward
    state = {"n": 0}

    def one_row(*a):
        res = list(orig(*a))
        state["n"] += 1
        if state["n"] > 1:
            res[4] = np.zeros_like(res[4])
        return tuple(res)
    monkeypatch.setattr(O, "attention_line_backward", one_row)
    with pytest.raises(AssertionError):
        test_backward_matches_torch_autograd()


def test_mutant_ending_bias_untransposed_is_caught(monkeypatch):
    orig = O._pair_bias

    def sym(z, ln_w, ln_b, eps, w_bias):
        b = orig(z, ln_w, ln_b, eps, w_bias)
        return b.transpose(1, 0, 2)
    monkeypatch.setattr(O, "_pair_bias", sym)
    with pytest.raises(AssertionError):
        test_module_equals_project_core_outproject(True)
    with pytest.raises(AssertionError):
        test_module_equals_project_core_outproject(False)


def test_module_lines_subset_against_project():
    """Line-wise module (own bias path) against project + core + out-proj."""
    for ending in (False, True):
        d = module_case(27)
        q, k, v, g, bias = O.tri_project(d["z"], d["ln_w"], d["ln_b"],
                                         d["eps"], d["w_q"], d["w_k"],
                                         d["w_v"], d["w_g"], d["b_g"],
                                         d["w_bias"], d["H"], d["C"], ending)
        km = d["residue_mask"][None, None, :]
        o, _ = O.attention_forward(q, k, v, g, km, bias)
        out = O.tri_out_project(o, d["w_o"], d["b_o"], ending)
        sub = O.tri_module_lines(lines=[3], ending=ending, **d)[0]
        ref = out[:, 3] if ending else out[3]
        np.testing.assert_allclose(sub, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- module backward

MODULE_PARAMS = ("z", "ln_w", "ln_b", "w_q", "w_k", "w_v", "w_g", "b_g",
                 "w_bias", "w_o", "b_o")


def module_grads(d, ending, dout):
    g = O.tri_module_backward(ending=ending, dout=dout, **d)
    return {"z": g["dz"], "ln_w": g["dln_w"], "ln_b": g["dln_b"],
            "w_q": g["dw_q"], "w_k": g["dw_k"], "w_v": g["dw_v"],
            "w_g": g["dw_g"], "b_g": g["db_g"], "w_bias": g["dw_bias"],
            "w_o": g["dw_o"], "b_o": g["db_o"]}


def _module_fd_pin(ending, seed=40):
    """Every gradient entry of the module against a central difference of
    <dout, module(...)> (fp64, step 1e-6), residue mask on."""
    d = module_case(seed, N=4, CZ=5, H=2, C=2)
    dout = rnd(seed + 1, 4, 4, 5)
    grads = module_grads(d, ending, dout)
    eps = 1e-6
    for name in MODULE_PARAMS:
        base = d[name]
        num = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            e = dict(d)
            plus = base.copy(); plus[idx] += eps
            minus = base.copy(); minus[idx] -= eps
            e[name] = plus
            lp = float((module(e, ending) * dout).sum())
            e[name] = minus
            lm = float((module(e, ending) * dout).sum())
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grads[name], num, rtol=1e-6, atol=1e-8,
                                   err_msg=f"gradient of {name}")


@pytest.mark.parametrize("ending", [False, True])
def test_module_backward_matches_central_finite_differences(ending):
    _module_fd_pin(ending)


def _torch_module(t, H, C, ending, keep):
    """The module written with torch library routines (fp64): layer_norm,
    linear, softmax, sigmoid; line layout by transposing z for the ending
    node."""
    z = t["z"]
    N, _, CZ = z.shape
    x = F.layer_norm(z, (CZ,), t["ln_w"], t["ln_b"], 1e-5)
    xl = x.transpose(0, 1) if ending else x
    q, k, v = (F.linear(xl, t[w]).reshape(N, N, H, C) for w in ("w_q", "w_k", "w_v"))
    g = F.linear(xl, t["w_g"], t["b_g"]).reshape(N, N, H, C)
    bias = F.linear(xl, t["w_bias"]).permute(2, 0, 1)          # [h, query, key]
    s = torch.einsum("lqhc,lkhc->lhqk", q, k) / C ** 0.5 + bias[None]
    s = s.masked_fill(~keep[None, None, None, :], float("-inf"))
    o = torch.einsum("lhqk,lkhc->lqhc", torch.softmax(s, dim=-1), v)
    y = F.linear((o * torch.sigmoid(g)).reshape(N, N, H * C), t["w_o"], t["b_o"])
    return y.transpose(0, 1) if ending else y


@pytest.mark.parametrize("ending", [False, True])
def test_module_backward_matches_torch_autograd(ending):
    """Library routine: torch.autograd through the module written with
    torch.nn.functional (fp64, CPU)."""
    d = module_case(42, N=9, CZ=12, H=2, C=4)
    dout = rnd(43, 9, 9, 12)
    grads = module_grads(d, ending, dout)
    t = {n: torch.tensor(d[n], requires_grad=True) for n in MODULE_PARAMS}
    keep = torch.tensor(d["residue_mask"] != 0)
    y = _torch_module(t, d["H"], d["C"], ending, keep)
    (y * torch.tensor(dout)).sum().backward()
    for n in MODULE_PARAMS:
        np.testing.assert_allclose(grads[n], t[n].grad.numpy(), rtol=1e-9,
                                   atol=1e-11, err_msg=n)


def test_module_backward_closed_forms():
    """Sum over channels of dz is 0 at every position (LayerNorm is
    invariant to adding a constant to a position's channels), and db_o is the
    sum of dout over positions."""
    d = module_case(44, N=6, CZ=8, H=2, C=3)
    dout = rnd(45, 6, 6, 8)
    for ending in (False, True):
        g = module_grads(d, ending, dout)
        np.testing.assert_allclose(g["z"].sum(-1), 0, atol=1e-12)
        np.testing.assert_allclose(g["b_o"], dout.sum((0, 1)), rtol=1e-12)


def test_layer_norm_backward_matches_torch():
    x = rnd(46, 4, 3, 11)
    w = rnd(47, 11)
    dy = rnd(48, 4, 3, 11)
    tx, tw, tb = (torch.tensor(a, requires_grad=True) for a in (x, w, rnd(49, 11)))
    (F.layer_norm(tx, (11,), tw, tb, 1e-5) * torch.tensor(dy)).sum().backward()
    dx, dw, db = O.layer_norm_backward(x, w, 1e-5, dy)
    for got, ref in ((dx, tx.grad), (dw, tw.grad), (db, tb.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_mutant_layer_norm_backward_without_variance_term_is_caught(monkeypatch):
    def no_var_term(x, w, eps, dy):
        x = np.asarray(x, np.float64)
        n = x.shape[-1]
        mu = x.mean(axis=-1, keepdims=True)
        rstd = 1.0 / np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
        xhat = (x - mu) * rstd
        dxhat = dy * w
        dx = rstd * (dxhat - dxhat.mean(axis=-1, keepdims=True))
        return dx, (dy * xhat).reshape(-1, n).sum(0), dy.reshape(-1, n).sum(0)
    monkeypatch.setattr(O, "layer_norm_backward", no_var_term)
    with pytest.raises(AssertionError):
        _module_fd_pin(False)


def test_mutant_ending_gradient_left_in_line_layout_is_caught(monkeypatch):
    monkeypatch.setattr(O, "_to_lines", lambda t, ending: t)
    _module_fd_pin(False)  # the starting node does not transpose
    with pytest.raises(AssertionError):
        _module_fd_pin(True)


# ------------------------------------------- triangular multiplicative update

def trimul_case(seed, N=6, CZ=8, C=5, mask=True):
    rng = np.random.default_rng(seed)
    d = dict(z=rng.standard_normal((N, N, CZ)),
             ln_w=1 + 0.2 * rng.standard_normal(CZ),
             ln_b=0.2 * rng.standard_normal(CZ), eps=1e-5,
             w_a=rng.standard_normal((C, CZ)) / CZ ** 0.5,
             w_b=rng.standard_normal((C, CZ)) / CZ ** 0.5,
             w_o=rng.standard_normal((CZ, C)) / C ** 0.5,
             b_o=0.3 * rng.standard_normal(CZ))
    m = (rng.random(N) < 0.7).astype(np.uint8)
    m[0] = 1
    d["residue_mask"] = m if mask else None
    return d


@pytest.mark.parametrize("outgoing", [True, False])
def test_trimul_matches_triple_loop(outgoing):
    """Brute force: the sum over the third residue written as explicit loops
    over i, j, k and channels (no matrix products)."""
    d = trimul_case(60)
    got = O.tri_mul_forward(outgoing=outgoing, **d)
    z = d["z"]
    N, _, CZ = z.shape
    mu = z.mean(-1, keepdims=True)
    x = (z - mu) / np.sqrt(((z - mu) ** 2).mean(-1, keepdims=True) + d["eps"])
    x = x * d["ln_w"] + d["ln_b"]
    C = d["w_a"].shape[0]
    ref = np.zeros((N, N, CZ))
    for i in range(N):
        for j in range(N):
            t = np.zeros(C)
            for k in range(N):
                if not d["residue_mask"][k]:
                    continue
                e1, e2 = ((i, k), (j, k)) if outgoing else ((k, i), (k, j))
                for c in range(C):
                    ac = sum(x[e1][q] * d["w_a"][c, q] for q in range(CZ))
                    bc = sum(x[e2][q] * d["w_b"][c, q] for q in range(CZ))
                    t[c] += ac * bc
            for o in range(CZ):
                ref[i, j, o] = sum(t[c] * d["w_o"][o, c] for c in range(C)) + d["b_o"][o]
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_trimul_matches_torch_einsum():
    """Library routines: F.layer_norm, F.linear and torch.einsum (fp64)."""
    d = trimul_case(61, N=9, CZ=12, C=7)
    t = {k: torch.tensor(v) for k, v in d.items() if isinstance(v, np.ndarray)}
    x = F.layer_norm(t["z"], (12,), t["ln_w"], t["ln_b"], 1e-5)
    a, b = F.linear(x, t["w_a"]), F.linear(x, t["w_b"])
    keep = t["residue_mask"].double()
    out = torch.einsum("ikc,jkc,k->ijc", a, b, keep)
    ref_out = F.linear(out, t["w_o"], t["b_o"]).numpy()
    np.testing.assert_allclose(O.tri_mul_forward(outgoing=True, **d), ref_out,
                               rtol=1e-11, atol=1e-12)
    inc = torch.einsum("kic,kjc,k->ijc", a, b, keep)
    ref_in = F.linear(inc, t["w_o"], t["b_o"]).numpy()
    np.testing.assert_allclose(O.tri_mul_forward(outgoing=False, **d), ref_in,
                               rtol=1e-11, atol=1e-12)


def test_trimul_incoming_is_outgoing_of_transpose():
    """Incoming on z equals outgoing on z with its two residue axes swapped
    (edges (k, i) of z are edges (i, k) of the transpose)."""
    d = trimul_case(62)
    e = dict(d)
    e["z"] = d["z"].transpose(1, 0, 2).copy()
    np.testing.assert_allclose(O.tri_mul_forward(outgoing=False, **d),
                               O.tri_mul_forward(outgoing=True, **e),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("outgoing", [True, False])
def test_trimul_residue_permutation_equivariance(outgoing):
    """Relabelling residues permutes the update identically ("Two properties
    the tests assert")."""
    d = trimul_case(63)
    out = O.tri_mul_forward(outgoing=outgoing, **d)
    perm = np.random.default_rng(63).permutation(d["z"].shape[0])
    e = dict(d)
    e["z"] = d["z"][perm][:, perm]
    e["residue_mask"] = d["residue_mask"][perm]
    np.testing.assert_allclose(O.tri_mul_forward(outgoing=outgoing, **e),
                               out[perm][:, perm], rtol=1e-11, atol=1e-12)


def test_trimul_closure_separates_the_broken_variant():
    """The course's counterexample: replacing the sum over the third residue
    by an elementwise product (no k) must give a different answer; the
    correct update depends on edges (i, k) off the (i, j) edge itself."""
    d = trimul_case(64, mask=False)
    out = O.tri_mul_forward(outgoing=True, **d)
    x = O.layer_norm(d["z"], d["ln_w"], d["ln_b"], d["eps"])
    broken = ((x @ d["w_a"].T) * (x @ d["w_b"].T)) @ d["w_o"].T + d["b_o"]
    assert np.abs(out - broken).max() > 0.1
    # changing an edge (i, k) with k != j moves out[i, j] for every j
    e = dict(d)
    e["z"] = d["z"].copy()
    e["z"][1, 3, 0] += 1.0  # one channel (a shift of all channels is normalised away)
    moved = np.abs(O.tri_mul_forward(outgoing=True, **e) - out).max(-1)
    assert (moved[1] > 1e-6).all()


def test_mutant_trimul_without_third_index_is_caught(monkeypatch):
    def broken(z, residue_mask, ln_w, ln_b, eps, w_a, w_b, w_o, b_o, outgoing=True):
        x = O.layer_norm(z, ln_w, ln_b, eps)
        return ((x @ w_a.T) * (x @ w_b.T)) @ w_o.T + b_o
    monkeypatch.setattr(O, "tri_mul_forward", broken)
    with pytest.raises(AssertionError):
        test_trimul_matches_torch_einsum()


@pytest.mark.parametrize("outgoing", [True, False])
def test_trimul_entries_match_full_forward(outgoing):
    d = trimul_case(65, N=7)
    full = O.tri_mul_forward(outgoing=outgoing, **d)
    picks = [(0, 0), (2, 5), (6, 1)]
    got = O.tri_mul_entries(picks=picks, outgoing=outgoing, **d)
    for t, (i, j) in enumerate(picks):
        np.testing.assert_allclose(got[t], full[i, j], rtol=1e-12, atol=1e-12)


TRIMUL_GRADS = (("z", "dz"), ("ln_w", "dln_w"), ("ln_b", "dln_b"), ("w_a", "dw_a"),
                ("w_b", "dw_b"), ("w_o", "dw_o"), ("b_o", "db_o"))


def _trimul_loss(d, dout, outgoing):
    return float((O.tri_mul_forward(outgoing=outgoing, **d) * dout).sum())


@pytest.mark.parametrize("outgoing", [True, False])
def test_trimul_backward_matches_torch_autograd(outgoing):
    """torch.autograd (fp64) of the update written with F.layer_norm,
    F.linear and torch.einsum: every gradient, with a residue mask."""
    d = trimul_case(70, N=6, CZ=8, C=5)
    dout = np.random.default_rng(71).standard_normal((6, 6, 8))
    t = {k: torch.tensor(v, requires_grad=True) for k, v in d.items()
         if isinstance(v, np.ndarray) and k != "residue_mask"}
    keep = torch.tensor(d["residue_mask"] != 0, dtype=torch.float64)
    x = F.layer_norm(t["z"], (8,), t["ln_w"], t["ln_b"], d["eps"])
    a, b = F.linear(x, t["w_a"]), F.linear(x, t["w_b"])
    eq = "ikc,jkc,k->ijc" if outgoing else "kic,kjc,k->ijc"
    out = F.linear(torch.einsum(eq, a, b, keep), t["w_o"], t["b_o"])
    (out * torch.tensor(dout)).sum().backward()
    got = O.tri_mul_backward(dout=dout, outgoing=outgoing, **d)
    for k_t, k_o in TRIMUL_GRADS:
        np.testing.assert_allclose(got[k_o], t[k_t].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=k_o)


@pytest.mark.parametrize("outgoing", [True, False])
@pytest.mark.parametrize("which", ["z", "ln_w", "w_a", "w_b", "w_o", "b_o"])
def test_trimul_backward_matches_central_finite_differences(which, outgoing):
    """The definition of the derivative: central differences of
    sum(out * dout) on a tiny masked case, every element of the input."""
    d = trimul_case(72, N=4, CZ=4, C=3)
    dout = np.random.default_rng(73).standard_normal((4, 4, 4))
    got = O.tri_mul_backward(dout=dout, outgoing=outgoing, **d)["d" + which]
    h = 1e-6
    fd = np.zeros_like(d[which])
    for idx in np.ndindex(d[which].shape):
        e = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d.items()}
        e[which][idx] += h
        fp = _trimul_loss(e, dout, outgoing)
        e[which][idx] -= 2 * h
        fd[idx] = (fp - _trimul_loss(e, dout, outgoing)) / (2 * h)
    np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-8)


def test_trimul_backward_closed_forms():
    """dz sums to zero over a position's channels (LayerNorm ignores a
    shift); db_o is the sum of dout; a masked third residue k receives no
    gradient through a or b on the edges (., k) / (k, .), so with w_o = 0
    (dT = 0) every gradient but dw_o and db_o vanishes."""
    d = trimul_case(74, N=6)
    dout = np.random.default_rng(75).standard_normal((6, 6, 8))
    for outgoing in (True, False):
        g = O.tri_mul_backward(dout=dout, outgoing=outgoing, **d)
        np.testing.assert_allclose(g["dz"].sum(-1), 0.0, atol=1e-12)
        np.testing.assert_allclose(g["db_o"], dout.sum((0, 1)), rtol=1e-12)
        g0 = O.tri_mul_backward(dout=dout, outgoing=outgoing, **dict(d, w_o=0 * d["w_o"]))
        for k in ("dz", "dw_a", "dw_b", "dln_w", "dln_b"):
            np.testing.assert_allclose(g0[k], 0.0, atol=1e-14, err_msg=k)
        assert np.abs(g0["dw_o"]).max() > 1e-3


def test_trimul_backward_planted_mistake_fails():
    """dB taken as dT . A (the transpose of dT dropped), planted in a copy of
    the chain rule, must miss the finite differences of w_b."""
    d = trimul_case(76, N=4, CZ=4, C=3)
    dout = np.random.default_rng(77).standard_normal((4, 4, 4))
    x = O.layer_norm(d["z"], d["ln_w"], d["ln_b"], d["eps"])
    a = x @ d["w_a"].T
    keep = (d["residue_mask"] != 0).astype(float)
    dt = dout @ d["w_o"]
    db_wrong = np.stack([(dt[:, :, c] @ a[:, :, c]) * keep for c in range(3)], -1)
    dw_b_wrong = db_wrong.reshape(-1, 3).T @ x.reshape(-1, 4)
    h = 1e-6
    fd = np.zeros_like(d["w_b"])
    for idx in np.ndindex(d["w_b"].shape):
        e = dict(d, w_b=d["w_b"].copy())
        e["w_b"][idx] += h
        fp = _trimul_loss(e, dout, True)
        e["w_b"][idx] -= 2 * h
        fd[idx] = (fp - _trimul_loss(e, dout, True)) / (2 * h)
    assert np.abs(dw_b_wrong - fd).max() > 1e-3
    np.testing.assert_allclose(O.tri_mul_backward(dout=dout, **d)["dw_b"], fd, rtol=1e-6,
                               atol=1e-8)


@pytest.mark.parametrize("outgoing", [True, False])
def test_trimul_backward_entries_match_full_backward(outgoing):
    d = trimul_case(78, N=7)
    dout = np.random.default_rng(79).standard_normal((7, 7, 8))
    full = O.tri_mul_backward(dout=dout, outgoing=outgoing, **d)
    picks = [(0, 0), (2, 5), (6, 1), (3, 3)]
    e = {k: v for k, v in d.items() if k != "b_o"}
    got = O.tri_mul_backward_entries(dout=dout, picks=picks, outgoing=outgoing, **e)
    for t, (i, j) in enumerate(picks):
        np.testing.assert_allclose(got[t], full["dz"][i, j], rtol=1e-12, atol=1e-12)


# -------------------------------------------- LayerNorm + SwiGLU transition

def transition_case(seed, N=5, CZ=8, HID=12):
    rng = np.random.default_rng(seed)
    return dict(z=rng.standard_normal((N, N, CZ)),
                ln_w=1 + 0.2 * rng.standard_normal(CZ),
                ln_b=0.2 * rng.standard_normal(CZ), eps=1e-5,
                w_a=rng.standard_normal((HID, CZ)) / CZ ** 0.5,
                w_b=rng.standard_normal((HID, CZ)) / CZ ** 0.5,
                w_o=rng.standard_normal((CZ, HID)) / HID ** 0.5)


def test_transition_matches_torch():
    """Library routines: F.layer_norm, F.linear, F.silu (fp64)."""
    d = transition_case(70, N=7, CZ=16, HID=40)
    t = {k: torch.tensor(v) for k, v in d.items() if isinstance(v, np.ndarray)}
    x = F.layer_norm(t["z"], (16,), t["ln_w"], t["ln_b"], 1e-5)
    ref = F.linear(F.silu(F.linear(x, t["w_a"])) * F.linear(x, t["w_b"]), t["w_o"])
    np.testing.assert_allclose(O.transition_forward(**d), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_transition_matches_scalar_loops():
    """Brute force on a tiny case: every sum written as a loop, silu(u) as
    u / (1 + exp(-u))."""
    d = transition_case(71, N=2, CZ=4, HID=3)
    z = d["z"]
    N, _, CZ = z.shape
    HID = d["w_a"].shape[0]
    got = O.transition_forward(**d)
    for i in range(N):
        for j in range(N):
            v = z[i, j]
            mu = sum(v) / CZ
            var = sum((q - mu) ** 2 for q in v) / CZ
            x = [(v[q] - mu) / np.sqrt(var + d["eps"]) * d["ln_w"][q] + d["ln_b"][q]
                 for q in range(CZ)]
            h = []
            for m in range(HID):
                u = sum(x[q] * d["w_a"][m, q] for q in range(CZ))
                b = sum(x[q] * d["w_b"][m, q] for q in range(CZ))
                h.append(u / (1.0 + np.exp(-u)) * b)
            for o in range(CZ):
                ref = sum(h[m] * d["w_o"][o, m] for m in range(HID))
                assert abs(got[i, j, o] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_transition_closed_forms():
    """w_b = 0 or w_a = 0 give 0 (silu(0) = 0); the output is linear in w_o
    and in w_b; a shift of a position's channels leaves it unchanged
    (LayerNorm)."""
    d = transition_case(72)
    out = O.transition_forward(**d)
    e = dict(d, w_b=np.zeros_like(d["w_b"]))
    assert np.abs(O.transition_forward(**e)).max() == 0
    e = dict(d, w_a=np.zeros_like(d["w_a"]))
    assert np.abs(O.transition_forward(**e)).max() == 0
    np.testing.assert_allclose(O.transition_forward(**dict(d, w_o=3 * d["w_o"])), 3 * out,
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(O.transition_forward(**dict(d, w_b=-2 * d["w_b"])), -2 * out,
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(O.transition_forward(**dict(d, z=d["z"] + 5.0)), out,
                               rtol=1e-8, atol=1e-9)


def test_mutant_transition_relu_gate_is_caught(monkeypatch):
    def relu_gate(z, ln_w, ln_b, eps, w_a, w_b, w_o):
        x = O.layer_norm(z, ln_w, ln_b, eps)
        return (np.maximum(x @ w_a.T, 0) * (x @ w_b.T)) @ w_o.T
    monkeypatch.setattr(O, "transition_forward", relu_gate)
    with pytest.raises(AssertionError):
        test_transition_matches_torch()


# ----------------------------------------------- transition backward

def _transition_loss(d, dout):
    return float((O.transition_forward(**d) * dout).sum())


def test_transition_backward_matches_torch_autograd():
    """torch.autograd (fp64) of F.layer_norm, F.linear and F.silu: every
    gradient (input, LayerNorm weight and bias, the three weights)."""
    d = transition_case(90, N=4, CZ=8, HID=12)
    dout = np.random.default_rng(91).standard_normal((4, 4, 8))
    t = {k: torch.tensor(v, requires_grad=True) for k, v in d.items() if isinstance(v, np.ndarray)}
    x = F.layer_norm(t["z"], (8,), t["ln_w"], t["ln_b"], d["eps"])
    out = F.linear(F.silu(F.linear(x, t["w_a"])) * F.linear(x, t["w_b"]), t["w_o"])
    (out * torch.tensor(dout)).sum().backward()
    got = O.transition_backward(dout=dout, **d)
    for k_t, k_o in (("z", "dz"), ("ln_w", "dln_w"), ("ln_b", "dln_b"), ("w_a", "dw_a"),
                     ("w_b", "dw_b"), ("w_o", "dw_o")):
        np.testing.assert_allclose(got[k_o], t[k_t].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=k_o)


@pytest.mark.parametrize("which", ["z", "ln_w", "ln_b", "w_a", "w_b", "w_o"])
def test_transition_backward_matches_central_finite_differences(which):
    """The definition of the derivative: central differences of
    sum(out * dout) on a tiny case, every element of the chosen input."""
    d = transition_case(92, N=2, CZ=4, HID=6)
    dout = np.random.default_rng(93).standard_normal((2, 2, 4))
    got = O.transition_backward(dout=dout, **d)["d" + which]
    h = 1e-6
    fd = np.zeros_like(d[which])
    for idx in np.ndindex(d[which].shape):
        e = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d.items()}
        e[which][idx] += h
        fp = _transition_loss(e, dout)
        e[which][idx] -= 2 * h
        fm = _transition_loss(e, dout)
        fd[idx] = (fp - fm) / (2 * h)
    np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-8)


def test_transition_backward_closed_forms():
    """The LayerNorm ignores a shift of a position's channels, so dz sums to
    zero over channels; with w_b = 0 the hidden layer is zero, so dw_o = 0
    and dw_a = 0 (silu(u) * 0 has no gradient through u)."""
    d = transition_case(94)
    dout = np.random.default_rng(95).standard_normal((5, 5, 8))
    g = O.transition_backward(dout=dout, **d)
    np.testing.assert_allclose(g["dz"].sum(axis=-1), 0.0, atol=1e-12)
    e = dict(d, w_b=np.zeros_like(d["w_b"]))
    g0 = O.transition_backward(dout=dout, **e)
    np.testing.assert_allclose(g0["dw_o"], 0.0, atol=1e-14)
    np.testing.assert_allclose(g0["dw_a"], 0.0, atol=1e-14)
    assert np.abs(g0["dw_b"]).max() > 1e-3


def test_transition_backward_planted_mistake_fails():
    """silu' taken as sigmoid(u) alone (the u sigmoid' term dropped), planted
    in a copy of the oracle, must miss the finite differences."""
    d = transition_case(96, N=2, CZ=4, HID=6)
    dout = np.random.default_rng(97).standard_normal((2, 2, 4))
    x = O.layer_norm(d["z"], d["ln_w"], d["ln_b"], d["eps"]).reshape(-1, 4)
    u = x @ d["w_a"].T
    v = x @ d["w_b"].T
    dh = dout.reshape(-1, 4) @ d["w_o"]
    du_wrong = dh * v * O.sigmoid(u)
    dw_a_wrong = du_wrong.T @ x
    h = 1e-6
    fd = np.zeros_like(d["w_a"])
    for idx in np.ndindex(d["w_a"].shape):
        e = dict(d, w_a=d["w_a"].copy())
        e["w_a"][idx] += h
        fp = _transition_loss(e, dout)
        e["w_a"][idx] -= 2 * h
        fd[idx] = (fp - _transition_loss(e, dout)) / (2 * h)
    assert np.abs(dw_a_wrong - fd).max() > 1e-3
    np.testing.assert_allclose(O.transition_backward(dout=dout, **d)["dw_a"], fd, rtol=1e-6,
                               atol=1e-8)


def test_transition_weight_grad_units_match_full_backward():
    d = transition_case(98, N=4, CZ=8, HID=10)
    dout = np.random.default_rng(99).standard_normal((4, 4, 8))
    full = O.transition_backward(dout=dout, **d)
    units = [0, 3, 9]
    ga, gb, go = O.transition_weight_grad_units(dout=dout, units=units, **d)
    np.testing.assert_allclose(ga, full["dw_a"][units], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gb, full["dw_b"][units], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(go, full["dw_o"][:, units], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- outer product mean

def opm_case(seed, S=4, N=5, CM=6, C=3, CZ=7):
    rng = np.random.default_rng(seed)
    return dict(m=rng.standard_normal((S, N, CM)),
                ln_w=1 + 0.2 * rng.standard_normal(CM),
                ln_b=0.2 * rng.standard_normal(CM), eps=1e-5,
                w_a=rng.standard_normal((C, CM)) / CM ** 0.5,
                w_b=rng.standard_normal((C, CM)) / CM ** 0.5,
                w_o=rng.standard_normal((CZ, C * C)) / C,
                b_o=0.3 * rng.standard_normal(CZ))


def test_opm_matches_torch_einsum():
    """Library routines: F.layer_norm, F.linear, torch.einsum (fp64)."""
    d = opm_case(80, S=6, N=7, CM=10, C=4, CZ=9)
    t = {k: torch.tensor(v) for k, v in d.items() if isinstance(v, np.ndarray)}
    x = F.layer_norm(t["m"], (10,), t["ln_w"], t["ln_b"], 1e-5)
    a, b = F.linear(x, t["w_a"]), F.linear(x, t["w_b"])
    o = torch.einsum("sic,sjd->ijcd", a, b) / 6
    ref = F.linear(o.reshape(7, 7, 16), t["w_o"], t["b_o"])
    np.testing.assert_allclose(O.outer_product_mean(**d), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_opm_matches_scalar_loops():
    d = opm_case(81, S=3, N=3, CM=4, C=2, CZ=3)
    got = O.outer_product_mean(**d)
    m = d["m"]
    S, N, CM = m.shape
    x = np.empty_like(m)
    for s in range(S):
        for n in range(N):
            v = m[s, n]
            mu = sum(v) / CM
            var = sum((q - mu) ** 2 for q in v) / CM
            for q in range(CM):
                x[s, n, q] = (v[q] - mu) / np.sqrt(var + d["eps"]) * d["ln_w"][q] + d["ln_b"][q]
    C = d["w_a"].shape[0]
    for i in range(N):
        for j in range(N):
            o = [[sum(sum(x[s, i, q] * d["w_a"][c, q] for q in range(CM)) *
                      sum(x[s, j, q] * d["w_b"][e, q] for q in range(CM)) for s in range(S)) / S
                  for e in range(C)] for c in range(C)]
            for z in range(d["w_o"].shape[0]):
                ref = sum(o[c][e] * d["w_o"][z, c * C + e] for c in range(C) for e in range(C))
                assert abs(got[i, j, z] - (ref + d["b_o"][z])) < 1e-12


def test_opm_sequence_order_carries_no_information():
    """Permuting the MSA rows leaves the mean unchanged ("Non-query MSA row
    invariance"), and permuting residues permutes both pair axes."""
    d = opm_case(82, S=6, N=5)
    out = O.outer_product_mean(**d)
    e = dict(d, m=d["m"][np.random.default_rng(1).permutation(6)])
    np.testing.assert_allclose(O.outer_product_mean(**e), out, rtol=1e-12, atol=1e-12)
    perm = np.random.default_rng(2).permutation(5)
    e = dict(d, m=d["m"][:, perm])
    np.testing.assert_allclose(O.outer_product_mean(**e), out[perm][:, perm], rtol=1e-12,
                               atol=1e-12)


def test_opm_single_sequence_is_outer_product():
    d = opm_case(83, S=1, N=4, C=3)
    x = O.layer_norm(d["m"][0], d["ln_w"], d["ln_b"], d["eps"])
    a, b = x @ d["w_a"].T, x @ d["w_b"].T
    i, j = 1, 3
    ref = np.outer(a[i], b[j]).reshape(-1) @ d["w_o"].T + d["b_o"]
    np.testing.assert_allclose(O.outer_product_mean(**d)[i, j], ref, rtol=1e-12, atol=1e-12)


def test_opm_pairs_match_full():
    d = opm_case(84, S=5, N=6)
    full = O.outer_product_mean(**d)
    picks = [(0, 0), (2, 5), (5, 1)]
    got = O.outer_product_mean_pairs(picks=picks, **d)
    for t, (i, j) in enumerate(picks):
        np.testing.assert_allclose(got[t], full[i, j], rtol=1e-12, atol=1e-12)


def test_mutant_opm_sum_instead_of_mean_is_caught(monkeypatch):
    orig = O.outer_product_mean

    def summed(m, ln_w, ln_b, eps, w_a, w_b, w_o, b_o):
        S = m.shape[0]
        return (orig(m, ln_w, ln_b, eps, w_a, w_b, w_o, b_o) - b_o) * S + b_o
    monkeypatch.setattr(O, "outer_product_mean", summed)
    with pytest.raises(AssertionError):
        test_opm_matches_torch_einsum()


OPM_GRADS = (("m", "dm"), ("ln_w", "dln_w"), ("ln_b", "dln_b"), ("w_a", "dw_a"),
             ("w_b", "dw_b"), ("w_o", "dw_o"), ("b_o", "db_o"))


def test_opm_backward_matches_torch_autograd():
    """torch.autograd (fp64) of the bridge written with F.layer_norm,
    F.linear and torch.einsum: every gradient."""
    d = opm_case(85, S=6, N=5, CM=10, C=4, CZ=9)
    dout = np.random.default_rng(86).standard_normal((5, 5, 9))
    t = {k: torch.tensor(v, requires_grad=True) for k, v in d.items()
         if isinstance(v, np.ndarray)}
    x = F.layer_norm(t["m"], (10,), t["ln_w"], t["ln_b"], d["eps"])
    a, b = F.linear(x, t["w_a"]), F.linear(x, t["w_b"])
    o = torch.einsum("sic,sjd->ijcd", a, b) / 6
    out = F.linear(o.reshape(5, 5, 16), t["w_o"], t["b_o"])
    (out * torch.tensor(dout)).sum().backward()
    got = O.outer_product_mean_backward(dout=dout, **d)
    for k_t, k_o in OPM_GRADS:
        np.testing.assert_allclose(got[k_o], t[k_t].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=k_o)


def _opm_loss(d, dout):
    return float((O.outer_product_mean(**d) * dout).sum())


@pytest.mark.parametrize("which", ["m", "ln_w", "ln_b", "w_a", "w_b", "w_o", "b_o"])
def test_opm_backward_matches_central_finite_differences(which):
    """The definition of the derivative: central differences of
    sum(out * dout) on a tiny case, every element of the chosen input."""
    d = opm_case(87, S=3, N=3, CM=4, C=2, CZ=3)
    dout = np.random.default_rng(88).standard_normal((3, 3, 3))
    got = O.outer_product_mean_backward(dout=dout, **d)["d" + which]
    h = 1e-6
    fd = np.zeros_like(d[which])
    for idx in np.ndindex(d[which].shape):
        e = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d.items()}
        e[which][idx] += h
        fp = _opm_loss(e, dout)
        e[which][idx] -= 2 * h
        fd[idx] = (fp - _opm_loss(e, dout)) / (2 * h)
    np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-8)


def test_opm_backward_closed_forms():
    """dm sums to zero over each (sequence, residue)'s channels (LayerNorm
    ignores a shift); db_o is the sum of dout; with w_o = 0 only dw_o and
    db_o survive; permuting the sequences permutes dm alike and leaves every
    parameter gradient unchanged."""
    d = opm_case(89, S=5, N=4)
    dout = np.random.default_rng(90).standard_normal((4, 4, 7))
    g = O.outer_product_mean_backward(dout=dout, **d)
    np.testing.assert_allclose(g["dm"].sum(-1), 0.0, atol=1e-12)
    np.testing.assert_allclose(g["db_o"], dout.sum((0, 1)), rtol=1e-12)
    g0 = O.outer_product_mean_backward(dout=dout, **dict(d, w_o=0 * d["w_o"]))
    for k in ("dm", "dw_a", "dw_b", "dln_w", "dln_b"):
        np.testing.assert_allclose(g0[k], 0.0, atol=1e-14, err_msg=k)
    assert np.abs(g0["dw_o"]).max() > 1e-3
    perm = np.random.default_rng(3).permutation(5)
    gp = O.outer_product_mean_backward(dout=dout, **dict(d, m=d["m"][perm]))
    np.testing.assert_allclose(gp["dm"], g["dm"][perm], rtol=1e-12, atol=1e-12)
    for k in ("dw_a", "dw_b", "dw_o", "dln_w", "dln_b"):
        np.testing.assert_allclose(gp[k], g[k], rtol=1e-11, atol=1e-12, err_msg=k)


def test_opm_backward_planted_mistake_fails():
    """The mean's 1/S dropped from dO (the gradient of a sum instead of a
    mean), planted in a copy of the chain rule, must miss the finite
    differences of w_a."""
    d = opm_case(91, S=3, N=3, CM=4, C=2, CZ=3)
    dout = np.random.default_rng(92).standard_normal((3, 3, 3))
    S, N, CM = d["m"].shape
    C = d["w_a"].shape[0]
    x = O.layer_norm(d["m"], d["ln_w"], d["ln_b"], d["eps"])
    b = x @ d["w_b"].T
    dO = (dout @ d["w_o"]).reshape(N, N, C, C)             # no 1/S
    da = np.einsum("ijcd,sjd->sic", dO, b)
    dw_a_wrong = da.reshape(-1, C).T @ x.reshape(-1, CM)
    h = 1e-6
    fd = np.zeros_like(d["w_a"])
    for idx in np.ndindex(d["w_a"].shape):
        e = dict(d, w_a=d["w_a"].copy())
        e["w_a"][idx] += h
        fp = _opm_loss(e, dout)
        e["w_a"][idx] -= 2 * h
        fd[idx] = (fp - _opm_loss(e, dout)) / (2 * h)
    assert np.abs(dw_a_wrong - fd).max() > 1e-3
    np.testing.assert_allclose(O.outer_product_mean_backward(dout=dout, **d)["dw_a"], fd,
                               rtol=1e-6, atol=1e-8)


def test_opm_backward_sampled_matches_full_backward():
    d = opm_case(93, S=5, N=6, CM=8, C=3, CZ=7)
    dout = np.random.default_rng(94).standard_normal((6, 6, 7))
    full = O.outer_product_mean_backward(dout=dout, **d)
    e = {k: v for k, v in d.items() if k != "b_o"}
    dm, ra, rb, ro = O.outer_product_mean_backward_sampled(
        dout=dout, dm_picks=[(0, 0), (4, 5), (2, 3)], wa_rows=[0, 2], wb_rows=[1],
        wo_cols=[(0, 0), (2, 1)], **e)
    np.testing.assert_allclose(dm, full["dm"][[0, 4, 2], [0, 5, 3]], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ra, full["dw_a"][[0, 2]], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rb, full["dw_b"][[1]], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ro, full["dw_o"][:, [0, 2 * 3 + 1]], rtol=1e-12, atol=1e-12)
