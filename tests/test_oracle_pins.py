"""Pins for the fp64 CPU oracle, each against something other than the oracle itself.

- brute force: the five primitive steps of the naive attention module ("Profiling in
  PyTorch (part 3): attention", naive causal attention) written as full-matrix numpy
  fp64 operations, with the math backend's safe softmax for fully masked rows;
- a library routine: PyTorch's own CPU scaled_dot_product_attention pinned to the MATH
  backend (the article's reference backend), in fp64;
- closed forms: V = 1, causal row 0, q = 0 prefix means, Lk = 1, a dominant key;
- invariants: rank-3 == rank-4 with B = 1, K shift, linearity in V, key permutation,
  stride independence, exact bf16 decode, row subsets;
- hand-derived cases in tests/golden/hand_cases.json.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import sdpa_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def naive_five_steps(q, k, v, keep, scale):
    """Full-matrix fp64: scores = q k^T; *scale; hidden -> -inf; safe softmax; attn v."""
    scores = np.matmul(q, np.swapaxes(k, -1, -2))
    scores = scores * scale
    scores = np.where(keep, scores, -np.inf)
    m = scores.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(scores - m)
    l = e.sum(axis=-1, keepdims=True)
    attn = np.where(l > 0, e / np.where(l > 0, l, 1.0), 0.0)
    out = np.matmul(attn, v)
    lse = np.where(l[..., 0] > 0, np.log(np.where(l[..., 0] > 0, l[..., 0], 1.0)) + m[..., 0],
                   -np.inf)
    return out, lse


def visible(Lq, Lk, causal, mask):
    keep = np.ones((Lq, Lk), dtype=bool)
    if causal:
        keep &= np.tril(np.ones((Lq, Lk), dtype=bool))
    if mask is not None:
        keep = keep & mask
    return keep


def rand_case(rng, B, H, Lq, Lk, D, with_mask, p_keep=0.5, empty_rows=0):
    q = rng.standard_normal((B, H, Lq, D))
    k = rng.standard_normal((B, H, Lk, D))
    v = rng.standard_normal((B, H, Lk, D))
    mask = None
    if with_mask:
        mask = rng.random((B, H, Lq, Lk)) < p_keep
        for _ in range(empty_rows):
            mask[rng.integers(B), rng.integers(H), rng.integers(Lq), :] = False
    return q, k, v, mask


@pytest.mark.parametrize("causal,with_mask", [(False, False), (True, False), (False, True),
                                              (True, True)])
def test_brute_force_random_tiny(causal, with_mask):
    rng = np.random.default_rng(1234 + 2 * causal + with_mask)
    for Lq in (1, 2, 3, 5, 9, 17):
        for Lk in (1, 2, 5, 17):
            D = int(rng.choice([1, 2, 4, 8]))
            B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
            q, k, v, mask = rand_case(rng, B, H, Lq, Lk, D, with_mask, empty_rows=2)
            scale = float(rng.uniform(0.1, 1.5))
            out, lse = sdpa_oracle(q, k, v, mask=None if mask is None else torch.from_numpy(mask),
                                   is_causal=causal, scale=scale)
            keep = visible(Lq, Lk, causal, mask)
            ref_out, ref_lse = naive_five_steps(q, k, v, keep, scale)
            np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
            fin = np.isfinite(ref_lse)
            assert np.array_equal(fin, np.isfinite(lse))
            np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=0, atol=1e-12)
            assert np.all(lse[~fin] == -np.inf)
            assert np.all(out[~fin] == 0.0)


def test_library_math_backend_fp64():
    """PyTorch's CPU SDPA, MATH backend, fp64; bool attn_mask True = takes part."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import torch.nn.functional as F
    rng = np.random.default_rng(7)
    for (B, H, Lq, Lk, D, causal, with_mask) in [(2, 3, 33, 33, 16, True, False),
                                                  (1, 2, 20, 45, 8, False, True),
                                                  (2, 2, 31, 17, 4, True, True),
                                                  (1, 1, 64, 64, 64, False, False)]:
        q, k, v, mask = rand_case(rng, B, H, Lq, Lk, D, with_mask, p_keep=0.3)
        scale = 1 / math.sqrt(D)
        keep = visible(Lq, Lk, causal, mask)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        with sdpa_kernel(SDPBackend.MATH):
            ref = F.scaled_dot_product_attention(tq, tk, tv,
                                                 attn_mask=torch.from_numpy(np.broadcast_to(
                                                     keep, (B, H, Lq, Lk)).copy()),
                                                 scale=scale).numpy()
        out, _ = sdpa_oracle(q, k, v, mask=None if mask is None else torch.from_numpy(mask),
                             is_causal=causal, scale=scale)
        rows_ok = keep.any(-1)
        np.testing.assert_allclose(out[..., rows_ok, :], ref[..., rows_ok, :], rtol=0, atol=1e-12)


@pytest.mark.parametrize("D", [32, 96, 256])
def test_brute_force_and_library_at_wide_head_dims(D):
    """The head dims 32, 96 and 256 against the numpy five-step formulation and PyTorch's
    fp64 math backend, causal and masked (the oracle's loops do not depend on D)."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import torch.nn.functional as F
    rng = np.random.default_rng(D)
    for causal, with_mask in [(True, False), (False, True)]:
        q, k, v, mask = rand_case(rng, 1, 2, 9, 13, D, with_mask, empty_rows=1)
        scale = 1 / math.sqrt(D)
        out, lse = sdpa_oracle(q, k, v, mask=None if mask is None else torch.from_numpy(mask),
                               is_causal=causal, scale=scale)
        keep = visible(9, 13, causal, mask)
        ref_out, ref_lse = naive_five_steps(q, k, v, keep, scale)
        np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
        fin = np.isfinite(ref_lse)
        np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=0, atol=1e-12)
        assert np.all(out[~fin] == 0.0) and np.all(lse[~fin] == -np.inf)
        with sdpa_kernel(SDPBackend.MATH):
            lib = F.scaled_dot_product_attention(
                *(torch.from_numpy(x) for x in (q, k, v)),
                attn_mask=torch.from_numpy(np.broadcast_to(keep, (1, 2, 9, 13)).copy()),
                scale=scale).numpy()
        rows_ok = keep.any(-1)
        np.testing.assert_allclose(out[..., rows_ok, :], lib[..., rows_ok, :], rtol=0, atol=1e-12)


def _load_golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_golden(), ids=lambda c: c["name"])
def test_hand_derived_golden(case):
    q, k, v = (torch.tensor(case[n], dtype=torch.float64) for n in ("q", "k", "v"))
    mask = None if case["mask"] is None else torch.tensor(case["mask"], dtype=torch.bool)
    out, lse = sdpa_oracle(q, k, v, mask=mask, is_causal=case["is_causal"],
                           scale=case["scale"])
    exp_out = np.array(case["out"], dtype=np.float64)
    exp_lse = np.array([[(-math.inf if x == "-inf" else x) for x in row] for row in case["lse"]])
    np.testing.assert_allclose(out, exp_out, rtol=0, atol=1e-12)
    fin = np.isfinite(exp_lse)
    assert np.array_equal(np.isfinite(lse), fin)
    np.testing.assert_allclose(lse[fin], exp_lse[fin], rtol=0, atol=1e-12)


def test_rows_sum_to_one_v_ones():
    rng = np.random.default_rng(3)
    q, k, _, mask = rand_case(rng, 2, 2, 40, 40, 8, True, p_keep=0.2, empty_rows=3)
    v = np.ones((2, 2, 40, 8))
    out, lse = sdpa_oracle(q, k, v, mask=torch.from_numpy(mask), is_causal=True, scale=0.7)
    keep = visible(40, 40, True, mask)
    nonempty = keep.any(-1)
    np.testing.assert_allclose(out[nonempty], 1.0, rtol=0, atol=1e-13)
    assert np.all(out[~nonempty] == 0.0)


def test_causal_row0_is_v0():
    rng = np.random.default_rng(4)
    q, k, v, _ = rand_case(rng, 1, 3, 16, 16, 8, False)
    out, lse = sdpa_oracle(q, k, v, is_causal=True, scale=0.3)
    np.testing.assert_array_equal(out[:, :, 0, :], v[:, :, 0, :])
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * np.sum(q[:, :, 0] * k[:, :, 0], -1),
                               rtol=0, atol=1e-13)


def test_zero_query_prefix_mean():
    rng = np.random.default_rng(5)
    _, k, v, _ = rand_case(rng, 1, 2, 50, 50, 4, False)
    q = np.zeros((1, 2, 50, 4))
    out, lse = sdpa_oracle(q, k, v, is_causal=True, scale=1.0)
    prefix = np.cumsum(v, axis=2) / np.arange(1, 51)[None, None, :, None]
    np.testing.assert_allclose(out, prefix, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(np.arange(1, 51))[None, None, :].repeat(2, 1),
                               rtol=0, atol=1e-13)


def test_single_key():
    rng = np.random.default_rng(6)
    q, k, v, _ = rand_case(rng, 2, 2, 7, 1, 8, False)
    out, lse = sdpa_oracle(q, k, v, is_causal=False, scale=0.25)
    np.testing.assert_array_equal(out, np.broadcast_to(v, out.shape))
    np.testing.assert_allclose(lse, 0.25 * np.einsum("bhid,bhjd->bhi", q, k), rtol=0,
                               atol=1e-13)


def test_dominant_key_large_scale():
    """With a large scale and well separated scores the output is v at the argmax."""
    Lk, D = 6, 2
    k = np.array([[[[0.0, 1.0], [1.0, 0.0], [2.0, 0.5], [-1.0, 3.0], [0.5, 0.5], [1.5, -2.0]]]])
    q = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    v = np.arange(Lk * D, dtype=np.float64).reshape(1, 1, Lk, D)
    out, _ = sdpa_oracle(q, k, v, is_causal=False, scale=200.0)
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0, 2], atol=1e-12)  # argmax of k[:,0]
    np.testing.assert_allclose(out[0, 0, 1], v[0, 0, 3], atol=1e-12)  # argmax of k[:,1]


def test_rank3_equals_rank4_b1():
    rng = np.random.default_rng(8)
    q, k, v, mask = rand_case(rng, 1, 3, 21, 13, 8, True, p_keep=0.6, empty_rows=1)
    out4, lse4 = sdpa_oracle(q, k, v, mask=torch.from_numpy(mask), is_causal=True, scale=0.5)
    out3, lse3 = sdpa_oracle(q[0], k[0], v[0], mask=torch.from_numpy(mask[0]), is_causal=True,
                             scale=0.5)
    np.testing.assert_array_equal(out3, out4[0])
    np.testing.assert_array_equal(lse3, lse4[0])


def test_key_shift_invariance():
    rng = np.random.default_rng(9)
    q, k, v, _ = rand_case(rng, 1, 2, 12, 12, 8, False)
    c = rng.standard_normal(8)
    out1, lse1 = sdpa_oracle(q, k, v, is_causal=True, scale=0.4)
    out2, lse2 = sdpa_oracle(q, k + c, v, is_causal=True, scale=0.4)
    np.testing.assert_allclose(out2, out1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse1 + 0.4 * (q @ c), rtol=0, atol=1e-12)


def test_linearity_in_v():
    rng = np.random.default_rng(10)
    q, k, v1, _ = rand_case(rng, 1, 2, 9, 14, 4, False)
    v2 = rng.standard_normal(v1.shape)
    o1, _ = sdpa_oracle(q, k, v1, scale=0.9)
    o2, _ = sdpa_oracle(q, k, v2, scale=0.9)
    o12, _ = sdpa_oracle(q, k, 2.0 * v1 - 3.0 * v2, scale=0.9)
    np.testing.assert_allclose(o12, 2.0 * o1 - 3.0 * o2, rtol=0, atol=1e-12)


def test_joint_key_permutation_noncausal():
    rng = np.random.default_rng(11)
    q, k, v, mask = rand_case(rng, 1, 2, 10, 15, 8, True, p_keep=0.5)
    perm = rng.permutation(15)
    o1, l1 = sdpa_oracle(q, k, v, mask=torch.from_numpy(mask), scale=0.6)
    o2, l2 = sdpa_oracle(q, k[:, :, perm], v[:, :, perm],
                         mask=torch.from_numpy(np.ascontiguousarray(mask[..., perm])), scale=0.6)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    fin = np.isfinite(l1)
    np.testing.assert_allclose(l2[fin], l1[fin], rtol=0, atol=1e-12)


def test_strides_do_not_matter():
    """A [B,L,H,D] buffer viewed as [B,H,L,D] gives the same bits as a contiguous copy."""
    g = torch.Generator().manual_seed(12)
    bufs = [torch.randn(2, 19, 3, 8, generator=g).to(torch.bfloat16) for _ in range(3)]
    views = [b.transpose(1, 2) for b in bufs]
    o1, l1 = sdpa_oracle(*views, is_causal=True)
    o2, l2 = sdpa_oracle(*(x.contiguous() for x in views), is_causal=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_bf16_decoded_exactly():
    """bf16 inputs give the bits of the same values handed over as fp64."""
    g = torch.Generator().manual_seed(13)
    q, k, v = (torch.randn(2, 11, 16, generator=g).to(torch.bfloat16) for _ in range(3))
    o1, l1 = sdpa_oracle(q, k, v, is_causal=True)
    o2, l2 = sdpa_oracle(q.double(), k.double(), v.double(), is_causal=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # a value bf16 cannot hold exactly in fp16: decoding must not pass through fp16
    big = torch.full((1, 1, 2), 2.0 ** 100, dtype=torch.bfloat16)
    o3, _ = sdpa_oracle(torch.zeros(1, 1, 2, dtype=torch.bfloat16),
                        torch.zeros(1, 1, 2, dtype=torch.bfloat16), big)
    assert o3[0, 0, 0] == 2.0 ** 100


def test_row_subset_matches_full():
    rng = np.random.default_rng(14)
    q, k, v, mask = rand_case(rng, 2, 3, 17, 17, 8, True, empty_rows=2)
    o, l = sdpa_oracle(q, k, v, mask=torch.from_numpy(mask), is_causal=True, scale=0.5)
    rows = rng.choice(2 * 3 * 17, size=20, replace=False)
    os_, ls_ = sdpa_oracle(q, k, v, mask=torch.from_numpy(mask), is_causal=True, scale=0.5,
                           rows=rows)
    np.testing.assert_array_equal(os_, o.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(ls_, l.reshape(-1)[rows])


def test_zero_scale_is_uniform_mean():
    rng = np.random.default_rng(15)
    q, k, v, _ = rand_case(rng, 1, 1, 6, 6, 4, False)
    out, lse = sdpa_oracle(q, k, v, scale=0.0)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(v[0, 0].mean(0), (6, 4)), atol=1e-13)
    np.testing.assert_allclose(lse, math.log(6), atol=1e-13)


def test_negative_scale_flips_preference():
    """scale < 0 prefers the key with the smallest dot product."""
    q = np.array([[[[1.0]]]])
    k = np.array([[[[-3.0], [0.0], [3.0]]]])
    v = np.array([[[[10.0], [20.0], [30.0]]]])
    out, _ = sdpa_oracle(q, k, v, scale=-50.0)
    np.testing.assert_allclose(out[0, 0, 0, 0], 10.0, atol=1e-12)


def test_empty_key_set_and_empty_queries():
    q = np.zeros((1, 2, 3, 4))
    k = np.zeros((1, 2, 0, 4))
    out, lse = sdpa_oracle(q, k, k, scale=1.0)
    assert np.all(out == 0.0) and np.all(lse == -np.inf)
    out, lse = sdpa_oracle(np.zeros((1, 2, 0, 4)), np.ones((1, 2, 5, 4)), np.ones((1, 2, 5, 4)))
    assert out.shape == (1, 2, 0, 4) and lse.shape == (1, 2, 0)


def test_fp16_decode_is_exact_for_every_bit_pattern():
    """One key gives weight exactly 1, so out = v: every finite and infinite IEEE binary16
    bit pattern in v must come back as numpy's own float16 -> float64 value."""
    bits = np.arange(65536, dtype=np.uint16)
    halves = bits.view(np.float16)
    keep = ~np.isnan(halves)
    v = torch.from_numpy(halves[keep].copy()).reshape(1, 1, 1, -1)
    D = v.shape[-1]
    q = torch.zeros(1, 1, 1, D, dtype=torch.float16)
    k = torch.zeros(1, 1, 1, D, dtype=torch.float16)
    out, lse = sdpa_oracle(q, k, v)
    want = halves[keep].astype(np.float64)
    assert np.array_equal(out.reshape(-1), want)
    assert lse.reshape(-1)[0] == 0.0


def test_fp16_inputs_match_their_fp64_values():
    g = torch.Generator().manual_seed(77)
    q, k, v = (torch.randn(2, 3, 9, 16, generator=g).to(torch.float16) for _ in range(3))
    a = sdpa_oracle(q, k, v, is_causal=True)
    b = sdpa_oracle(q.double(), k.double(), v.double(), is_causal=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ---- additive float mask (bias) -------------------------------------------------------

def _bias_case(seed=90, B=2, H=3, Lq=11, Lk=13, D=8):
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn(B, H, n, D, generator=g, dtype=torch.float64) for n in (Lq, Lk, Lk))
    bias = torch.randn(B, 1, Lq, Lk, generator=g, dtype=torch.float64) * 2
    return q, k, v, bias


def test_bias_zero_is_no_bias_bitwise():
    q, k, v, bias = _bias_case()
    a = sdpa_oracle(q, k, v, is_causal=True, bias=torch.zeros_like(bias))
    b = sdpa_oracle(q, k, v, is_causal=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_bias_of_zero_and_minus_inf_is_the_bool_mask_bitwise():
    q, k, v, bias = _bias_case()
    m = bias > 0.5
    m[0, 0, 4, :] = False  # an empty row
    minf = torch.where(m, 0.0, float("-inf")).to(torch.float64)
    a = sdpa_oracle(q, k, v, bias=minf)
    b = sdpa_oracle(q, k, v, mask=m)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert np.all(a[0][0, :, 4] == 0) and np.all(a[1][0, :, 4] == -np.inf)


def test_bias_constant_per_row_shifts_only_the_lse():
    q, k, v, _ = _bias_case()
    c = torch.randn(2, 3, 11, 1, generator=torch.Generator().manual_seed(91), dtype=torch.float64)
    a = sdpa_oracle(q, k, v, bias=c.expand(2, 3, 11, 13))
    b = sdpa_oracle(q, k, v)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(a[1], b[1] + c[..., 0].numpy(), rtol=1e-12, atol=1e-12)


def test_bias_matches_library_math_backend_with_float_mask():
    from torch.nn.attention import SDPBackend, sdpa_kernel
    q, k, v, bias = _bias_case(D=16)
    out, lse = sdpa_oracle(q, k, v, bias=bias, scale=0.37)
    with sdpa_kernel(SDPBackend.MATH):
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=bias, scale=0.37)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-11, atol=1e-12)
    s = (q @ k.transpose(-1, -2)) * 0.37 + bias
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def test_bias_with_causal_and_broadcast_strides():
    q, k, v, bias = _bias_case(Lq=9, Lk=9)
    out, lse = sdpa_oracle(q, k, v, bias=bias, is_causal=True)  # bias [B,1,L,L] over 3 heads
    tri = torch.ones(9, 9, dtype=torch.bool).tril()
    s = (q @ k.transpose(-1, -2)) / math.sqrt(8) + bias
    s = s.masked_fill(~tri, float("-inf"))
    np.testing.assert_allclose(out, (torch.softmax(s, -1) @ v).numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=1e-12, atol=1e-12)
