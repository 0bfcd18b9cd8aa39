"""Pins of the fp64 backward oracle (oracle_sdpa_bwd) against things other than itself:
central finite differences of the forward oracle, the library's fp64 autograd through its
math-backend SDPA, closed forms and invariants of the softmax Jacobian.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import bernoulli_mask

F64 = torch.float64


def rand(seed, *shape, dtype=F64):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64).to(dtype)


def loss(q, k, v, dout, **kw):
    """<out, dout> with out from the forward oracle: its gradients are the backward's."""
    out, _ = oracle.sdpa_oracle(q, k, v, **kw)
    return float((out * dout.numpy()).sum())


def finite_difference(q, k, v, dout, which, h=1e-6, **kw):
    args = {"q": q, "k": k, "v": v}
    x = args[which]
    grad = np.zeros(tuple(x.shape))
    flat = x.reshape(-1)
    for idx in range(flat.numel()):
        saved = float(flat[idx])
        flat[idx] = saved + h
        up = loss(args["q"], args["k"], args["v"], dout, **kw)
        flat[idx] = saved - h
        dn = loss(args["q"], args["k"], args["v"], dout, **kw)
        flat[idx] = saved
        grad.reshape(-1)[idx] = (up - dn) / (2 * h)
    return grad


CASES = [
    dict(Lq=5, Lk=7, causal=False, mask=None),
    dict(Lq=6, Lk=6, causal=True, mask=None),
    dict(Lq=5, Lk=8, causal=True, mask=None),   # top-left triangle, Lq != Lk
    dict(Lq=6, Lk=5, causal=False, mask="empty_row"),
    dict(Lq=6, Lk=6, causal=True, mask="random"),
]


def make_mask(kind, B, H, Lq, Lk, seed):
    if kind is None:
        return None
    m = bernoulli_mask(seed, (B, H, Lq, Lk), 0.6)
    if kind == "empty_row":
        m[0, 1, 2, :] = False  # one query row sees no key at all
    return m


@pytest.mark.parametrize("case", range(len(CASES)))
def test_bwd_matches_finite_differences(case):
    c = CASES[case]
    B, H, D = 1, 2, 4
    q, k, v = rand(10 + case, B, H, c["Lq"], D), rand(20 + case, B, H, c["Lk"], D), \
        rand(30 + case, B, H, c["Lk"], D)
    dout = rand(40 + case, B, H, c["Lq"], D)
    mask = make_mask(c["mask"], B, H, c["Lq"], c["Lk"], 50 + case)
    kw = dict(is_causal=c["causal"], mask=mask, scale=0.7)
    dq, dk, dv = oracle.sdpa_bwd_oracle(q, k, v, dout, **kw)
    for name, got in (("q", dq), ("k", dk), ("v", dv)):
        fd = finite_difference(q.clone(), k.clone(), v.clone(), dout, name, **kw)
        np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-8, err_msg=f"d{name}")


def test_bwd_matches_library_autograd_fp64():
    """The library's math-backend SDPA in fp64, differentiated by autograd."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    for seed, (B, H, Lq, Lk, D, causal, scale) in enumerate([
            (2, 3, 17, 17, 16, True, None), (1, 2, 9, 23, 8, False, 0.31),
            (2, 1, 33, 12, 32, True, 1.3)]):
        q, k, v = rand(seed, B, H, Lq, D), rand(seed + 100, B, H, Lk, D), \
            rand(seed + 200, B, H, Lk, D)
        dout = rand(seed + 300, B, H, Lq, D)
        dq, dk, dv = oracle.sdpa_bwd_oracle(q, k, v, dout, is_causal=causal, scale=scale)
        qq, kk, vv = (t.clone().requires_grad_() for t in (q, k, v))
        with sdpa_kernel(SDPBackend.MATH):
            out = torch.nn.functional.scaled_dot_product_attention(
                qq, kk, vv, is_causal=causal, scale=scale)
        out.backward(dout)
        np.testing.assert_allclose(dq, qq.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk, kk.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, vv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_bwd_mask_and_empty_rows():
    """A boolean mask (nonzero = visible) against autograd on the visible rows; a row
    with no visible key gets no gradient and passes none to k or v."""
    B, H, Lq, Lk, D = 1, 2, 11, 13, 8
    q, k, v = rand(1, B, H, Lq, D), rand(2, B, H, Lk, D), rand(3, B, H, Lk, D)
    dout = rand(4, B, H, Lq, D)
    mask = bernoulli_mask(5, (B, H, Lq, Lk), 0.5)
    mask[:, :, 0, 0] = True
    mask[0, 1, 4, :] = False
    dq, dk, dv = oracle.sdpa_bwd_oracle(q, k, v, dout, mask=mask)
    assert np.all(dq[0, 1, 4] == 0.0)
    # the same computation with the empty row's upstream gradient zeroed
    dout2 = dout.clone()
    dout2[0, 1, 4] = 0.0
    _, dk2, dv2 = oracle.sdpa_bwd_oracle(q, k, v, dout2, mask=mask)
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)
    # the visible rows agree with autograd through an explicit masked softmax
    qq, kk, vv = (t.clone().requires_grad_() for t in (q, k, v))
    s = (qq @ kk.transpose(-1, -2)) / math.sqrt(D)
    s = s.masked_fill(~mask, float("-inf"))
    p = torch.softmax(s, dim=-1).nan_to_num(0.0)
    (p @ vv).backward(dout2)
    np.testing.assert_allclose(dq, qq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, kk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, vv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_bwd_closed_form_uniform_attention():
    """q = 0: every visible key gets weight 1/n_i, so dV_j = sum over the rows i that see
    key j of dout_i / n_i (n_i = i + 1 under the causal triangle)."""
    B, H, L, D = 1, 1, 9, 5
    q = torch.zeros(B, H, L, D, dtype=F64)
    k, v, dout = rand(1, B, H, L, D), rand(2, B, H, L, D), rand(3, B, H, L, D)
    _, _, dv = oracle.sdpa_bwd_oracle(q, k, v, dout, is_causal=True)
    want = np.zeros((L, D))
    for i in range(L):
        want[: i + 1] += dout[0, 0, i].numpy() / (i + 1)
    np.testing.assert_allclose(dv[0, 0], want, rtol=1e-12, atol=1e-14)


def test_bwd_invariants():
    B, H, Lq, Lk, D = 2, 2, 10, 12, 6
    q, k, v = rand(7, B, H, Lq, D), rand(8, B, H, Lk, D), rand(9, B, H, Lk, D)
    dout = rand(10, B, H, Lq, D)
    dq, dk, dv = oracle.sdpa_bwd_oracle(q, k, v, dout, is_causal=True, scale=0.5)
    # rows of the softmax Jacobian sum to zero, so the key gradients sum to zero
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # shifting every key by one vector changes no output, so no query gradient
    c = rand(11, D)
    dq2, _, dv2 = oracle.sdpa_bwd_oracle(q, k + c, v, dout, is_causal=True, scale=0.5)
    np.testing.assert_allclose(dq2, dq, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv2, dv, rtol=1e-9, atol=1e-11)
    # linear in dout
    dq3, dk3, dv3 = oracle.sdpa_bwd_oracle(q, k, v, 3.0 * dout, is_causal=True, scale=0.5)
    np.testing.assert_allclose(dq3, 3 * dq, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv3, 3 * dv, rtol=1e-12, atol=1e-13)
    # rank 3 is rank 4 with B = 1, bit for bit
    r4 = oracle.sdpa_bwd_oracle(q[:1], k[:1], v[:1], dout[:1], is_causal=True, scale=0.5)
    r3 = oracle.sdpa_bwd_oracle(q[0], k[0], v[0], dout[0], is_causal=True, scale=0.5)
    for a, b in zip(r4, r3):
        np.testing.assert_array_equal(a[0], b)


def test_bwd_reads_bf16_exactly_and_any_strides():
    B, H, Lq, Lk, D = 1, 3, 8, 8, 8
    q, k, v = (rand(s, B, H, n, D, dtype=torch.bfloat16) for s, n in ((1, Lq), (2, Lk), (3, Lk)))
    dout = rand(4, B, H, Lq, D, dtype=torch.bfloat16)
    ref = oracle.sdpa_bwd_oracle(q.double(), k.double(), v.double(), dout.double(),
                                 is_causal=True)
    got = oracle.sdpa_bwd_oracle(q, k, v, dout, is_causal=True)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)
    # a [B,L,H,D] buffer viewed as [B,H,L,D]
    qt = q.transpose(1, 2).contiguous().transpose(1, 2)
    got2 = oracle.sdpa_bwd_oracle(qt, k, v, dout, is_causal=True)
    for a, b in zip(got2, got):
        np.testing.assert_array_equal(a, b)


# ---- the additive mask (bias): a constant added to the scaled scores, -inf hides a key ----

def make_bias(seed, B, H, Lq, Lk, hide=0.15, empty_row=None):
    g = torch.Generator().manual_seed(seed)
    bias = torch.randn(B, H, Lq, Lk, generator=g, dtype=F64) * 1.5
    bias[torch.rand(bias.shape, generator=g) < hide] = float("-inf")
    if empty_row is not None:
        bias[empty_row] = float("-inf")
    return bias


BIAS_CASES = [
    dict(Lq=5, Lk=7, causal=False),
    dict(Lq=6, Lk=6, causal=True),
    dict(Lq=6, Lk=5, causal=False, empty=(0, 1, 2)),
]


@pytest.mark.parametrize("case", range(len(BIAS_CASES)))
def test_bwd_bias_matches_finite_differences(case):
    """Central differences of the forward oracle with the same bias."""
    c = BIAS_CASES[case]
    B, H, D = 1, 2, 4
    q, k, v = rand(60 + case, B, H, c["Lq"], D), rand(70 + case, B, H, c["Lk"], D), \
        rand(80 + case, B, H, c["Lk"], D)
    dout = rand(90 + case, B, H, c["Lq"], D)
    bias = make_bias(95 + case, B, H, c["Lq"], c["Lk"], empty_row=c.get("empty"))
    kw = dict(is_causal=c["causal"], bias=bias, scale=0.6)
    dq, dk, dv = oracle.sdpa_bwd_oracle(q, k, v, dout, **kw)
    for name, got in (("q", dq), ("k", dk), ("v", dv)):
        fd = finite_difference(q.clone(), k.clone(), v.clone(), dout, name, **kw)
        np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-8, err_msg=f"d{name}")
    if "empty" in c:
        assert np.all(dq[c["empty"]] == 0.0)


def test_bwd_bias_matches_library_autograd_fp64():
    """The library's math-backend SDPA in fp64 with a float attn_mask (added to the scaled
    scores), differentiated by autograd; the bias broadcast over heads, -inf entries on
    rows that keep some visible key."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    for seed, (B, H, Lq, Lk, D, causal, scale) in enumerate([
            (2, 3, 13, 13, 16, True, None), (1, 2, 9, 21, 8, False, 0.37)]):
        q, k, v = rand(seed + 400, B, H, Lq, D), rand(seed + 410, B, H, Lk, D), \
            rand(seed + 420, B, H, Lk, D)
        dout = rand(seed + 430, B, H, Lq, D)
        bias = make_bias(seed + 440, B, 1, Lq, Lk)
        bias[..., 0] = 0.0  # key 0 visible to every row
        dq, dk, dv = oracle.sdpa_bwd_oracle(q, k, v, dout, is_causal=causal, scale=scale,
                                            bias=bias)
        qq, kk, vv = (t.clone().requires_grad_() for t in (q, k, v))
        m = bias
        if causal:
            m = bias.masked_fill(~torch.ones(Lq, Lk, dtype=torch.bool).tril(), float("-inf"))
        with sdpa_kernel(SDPBackend.MATH):
            out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m,
                                                                   scale=scale)
        out.backward(dout)
        np.testing.assert_allclose(dq, qq.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk, kk.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, vv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_bwd_bias_special_cases():
    """A zero bias is no bias and a 0 / -inf bias is the boolean mask, bit for bit; a bias
    constant along each row changes no gradient."""
    B, H, Lq, Lk, D = 1, 2, 9, 11, 8
    q, k, v = rand(501, B, H, Lq, D), rand(502, B, H, Lk, D), rand(503, B, H, Lk, D)
    dout = rand(504, B, H, Lq, D)
    ref = oracle.sdpa_bwd_oracle(q, k, v, dout, is_causal=True)
    got = oracle.sdpa_bwd_oracle(q, k, v, dout, is_causal=True,
                                 bias=torch.zeros(B, H, Lq, Lk, dtype=F64))
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)
    mask = bernoulli_mask(505, (B, H, Lq, Lk), 0.5)
    mask[..., 0] = True
    ref = oracle.sdpa_bwd_oracle(q, k, v, dout, mask=mask)
    zb = torch.zeros(B, H, Lq, Lk, dtype=F64).masked_fill(~mask, float("-inf"))
    got = oracle.sdpa_bwd_oracle(q, k, v, dout, bias=zb)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)
    row_const = rand(506, B, H, Lq, 1).expand(B, H, Lq, Lk).contiguous()
    ref = oracle.sdpa_bwd_oracle(q, k, v, dout, is_causal=True)
    got = oracle.sdpa_bwd_oracle(q, k, v, dout, is_causal=True, bias=row_const)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
