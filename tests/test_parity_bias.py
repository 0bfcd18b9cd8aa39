"""GPU parity of the additive float mask (sdpa_fwd_bias) through the C ABI against the fp64
oracle's bias path: random and ALiBi-style biases, full and head-broadcast layouts, -inf
entries (including whole rows), every causal mode, bf16 / fp16 / fp32, D in {64, 128}, with
the tolerances of test_parity.  The oracle reads the same fp32 bias values in fp64.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import sdpa_oracle
from scaled_dot_product_11_amd import sdpa_fwd, sdpa_fwd_bias
from test_parity import DEV, compare, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def oracle_for(q, k, v, bias, causal, rows=None):
    Lq, Lk = q.shape[-2], k.shape[-2]
    if causal == 2:
        tri = torch.ones(Lq, Lk, dtype=torch.bool).tril(Lk - Lq)
        return sdpa_oracle(q, k, v, mask=tri, bias=bias, rows=rows)
    return sdpa_oracle(q, k, v, is_causal=causal == 1, bias=bias, rows=rows)


def random_bias(seed, shape, inf_frac=0.1):
    g = torch.Generator().manual_seed(seed)
    b = torch.randn(shape, generator=g) * 2
    b[torch.rand(shape, generator=g) < inf_frac] = float("-inf")
    return b


def alibi(H, Lq, Lk, slope0=0.5):
    """Per-head linear distance penalty, slope0 * 2^-h * (j - i) for j <= i, else -|j - i|."""
    i = torch.arange(Lq)[:, None]
    j = torch.arange(Lk)[None, :]
    slopes = slope0 * 2.0 ** -torch.arange(H, dtype=torch.float32)
    return (-slopes[:, None, None] * (i - j).abs()).unsqueeze(0)  # [1, H, Lq, Lk]


SHAPES = [(1, 1), (33, 33), (64, 64), (129, 129), (77, 300), (300, 77)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32],
                         ids=["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [0, 1, 2], ids=["none", "top_left", "bottom_right"])
def test_bias_small(dtype, D, causal):
    for n, (Lq, Lk) in enumerate(SHAPES):
        g = torch.Generator().manual_seed(800 + n + D + causal)
        q, k, v = W.draw_qkv(g, (2, 3, Lq, D), (2, 3, Lk, D), dtype=dtype)
        bias = random_bias(900 + n, (2, 1 if n % 2 else 3, Lq, Lk))
        if Lq > 3:
            bias[0, :, 2, :] = float("-inf")  # a row with every key hidden
        out, lse = sdpa_fwd_bias(to_dev(q), to_dev(k), to_dev(v), to_dev(bias), is_causal=causal)
        torch.cuda.synchronize()
        ro, rl = oracle_for(q, k, v, bias, causal)
        compare(out, lse, ro, rl, dtype, f"bias D={D} causal={causal} Lq={Lq} Lk={Lk}")


def test_bias_zero_minus_inf_equals_bool_mask():
    g = torch.Generator().manual_seed(950)
    q, k, v = W.draw_qkv(g, (2, 2, 200, 128), (2, 2, 200, 128))
    m = torch.rand(2, 2, 200, 200, generator=g) < 0.3
    m[1, 0, 7] = False
    bias = torch.where(m, 0.0, float("-inf"))
    ob, lb = sdpa_fwd_bias(to_dev(q), to_dev(k), to_dev(v), to_dev(bias), is_causal=True)
    om, lm = sdpa_fwd(to_dev(q), to_dev(k), to_dev(v), mask=to_dev(m), is_causal=True)
    torch.cuda.synchronize()
    assert (ob.float() - om.float()).abs().max().item() <= 1e-2
    fin = torch.isfinite(lm)
    assert torch.equal(torch.isfinite(lb), fin)
    assert (lb[fin] - lm[fin]).abs().max().item() <= 1e-4
    ro, rl = sdpa_oracle(q, k, v, mask=m, is_causal=True)
    compare(ob, lb, ro, rl, torch.bfloat16, "0/-inf bias")


def test_bias_alibi_long_sampled():
    """ALiBi-style bias [1, 8, 4096, 4096] broadcast over a batch of 2, causal, D=64."""
    g = torch.Generator().manual_seed(960)
    q, k, v = W.draw_qkv(g, (2, 8, 4096, 64))
    bias = alibi(8, 4096, 4096)
    out, lse = sdpa_fwd_bias(to_dev(q), to_dev(k), to_dev(v), to_dev(bias), is_causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(960)
    rows = np.unique(np.concatenate([[0, 4095, 8 * 4096 - 1, 16 * 4096 - 1],
                                     rng.integers(0, 16 * 4096, size=200)])).astype(np.int64)
    ro, rl = oracle_for(q, k, v, bias, 1, rows=rows)
    idx = torch.from_numpy(rows).to(DEV)
    compare(out.reshape(-1, 64)[idx], lse.reshape(-1)[idx], ro, rl, torch.bfloat16, "alibi")
