"""GPU parity of the key-split tile against the fp64 oracle, with the tolerances of
test_parity.

Small causal 16-bit problems at D <= 64 whose launch lasts as long as their longest items take
the key split: 128 query rows per workgroup, whose two groups of waves walk the two halves of
the item's key tiles, each with its own staged tiles, and merge their row states (output,
exponent reference, row sum) before the rows are stored.  The cases below take that tile (the
plan says so) and cover: both causal alignments, ragged row and key counts, a boolean mask with
fully hidden rows, an additive mask with -inf entries, an item whose second half is empty (a
single key tile to walk), bf16 and fp16, D = 32 and 64; rank-3 and rank-4 inputs of one
problem give the same bits; repeated launches give the same bits.
"""
import numpy as np
import pytest
import torch

from oracle import sdpa_oracle
from scaled_dot_product_11_amd import SDPA_BF16, SDPA_F16, sdpa_fwd, sdpa_fwd_bias, sdpa_plan
from test_parity import DEV, compare, rand_inputs, to_dev

pytestmark = pytest.mark.gpu

CODE = {torch.bfloat16: SDPA_BF16, torch.float16: SDPA_F16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def takes_key_split(B, H, Lq, Lk, D, causal, dtype):
    plan = sdpa_plan(4, B, H, Lq, Lk, D, causal, CODE[dtype])
    return (plan.block_m, plan.threads) == (128, 512)


def oracle(q, k, v, causal, mask=None, bias=None):
    Lq, Lk = q.shape[-2], k.shape[-2]
    if causal == 2:
        tri = torch.ones(Lq, Lk, dtype=torch.bool).tril(Lk - Lq)
        mask = tri if mask is None else (mask & tri)
        return sdpa_oracle(q, k, v, mask=mask, bias=bias)
    return sdpa_oracle(q, k, v, mask=mask, bias=bias, is_causal=causal == 1)


# (B, H, Lq, Lk, causal): one round of items with walks of 1024 keys and more, bottom-right
# alignment with fewer queries than keys, and two single-tile walks (one group walks nothing)
CASES = [(1, 3, 1100, 1100, 1), (1, 2, 700, 2100, 2), (2, 2, 1024, 1024, 1),
         (1, 2, 40, 1100, 1), (1, 1, 130, 1030, 1)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("D", [32, 64])
def test_key_split_no_mask(dtype, D):
    for n, (B, H, Lq, Lk, causal) in enumerate(CASES):
        assert takes_key_split(B, H, Lq, Lk, D, causal, dtype), (B, H, Lq, Lk, causal)
        q, k, v, _ = rand_inputs(5200 + 10 * n + D, B, H, Lq, Lk, D, dtype)
        out, lse = sdpa_fwd(to_dev(q), to_dev(k), to_dev(v), is_causal=causal)
        torch.cuda.synchronize()
        ro, rl = oracle(q, k, v, causal)
        compare(out, lse, ro, rl, dtype, f"key split D={D} {(B, H, Lq, Lk)} causal={causal}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_key_split_masks(dtype):
    D = 64
    for n, (B, H, Lq, Lk, causal) in enumerate(CASES[:3]):
        assert takes_key_split(B, H, Lq, Lk, D, causal, dtype)
        q, k, v, mask = rand_inputs(5300 + n, B, H, Lq, Lk, D, dtype, mask_mode="bcast")
        out, lse = sdpa_fwd(to_dev(q), to_dev(k), to_dev(v), mask=to_dev(mask), is_causal=causal)
        torch.cuda.synchronize()
        ro, rl = oracle(q, k, v, causal, mask=mask)
        compare(out, lse, ro, rl, dtype, f"key split mask {(B, H, Lq, Lk)} causal={causal}")
        g = torch.Generator().manual_seed(5400 + n)
        bias = torch.randn((1, 1, Lq, Lk), generator=g) * 2
        bias[torch.rand(bias.shape, generator=g) < 0.1] = float("-inf")
        bias[..., Lq // 3, :] = float("-inf")  # one fully hidden row
        out, lse = sdpa_fwd_bias(to_dev(q), to_dev(k), to_dev(v), to_dev(bias), is_causal=causal)
        torch.cuda.synchronize()
        ro, rl = oracle(q, k, v, causal, bias=bias)
        compare(out, lse, ro, rl, dtype, f"key split bias {(B, H, Lq, Lk)} causal={causal}")


def test_key_split_rank3_equals_rank4_and_repeats():
    q, k, v, _ = rand_inputs(5500, 1, 3, 1100, 1100, 64, torch.bfloat16, rank=3)
    assert sdpa_plan(3, 1, 3, 1100, 1100, 64, 1, SDPA_BF16).threads == 512
    out3, lse3 = sdpa_fwd(to_dev(q), to_dev(k), to_dev(v), is_causal=True)
    out4, lse4 = sdpa_fwd(to_dev(q[None]), to_dev(k[None]), to_dev(v[None]), is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out3, out4[0]) and torch.equal(lse3, lse4[0])
    for _ in range(3):
        o, l = sdpa_fwd(to_dev(q), to_dev(k), to_dev(v), is_causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o, out3) and torch.equal(l, lse3)
    ro, rl = sdpa_oracle(q, k, v, is_causal=True)
    compare(out3, lse3, ro, rl, torch.bfloat16, "key split rank3")
