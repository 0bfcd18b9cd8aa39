"""GPU parity of the forward at the head dims beyond 64 and 128 (32, 96 and 256) through the
C ABI against the fp64 oracle, with the tolerances of test_parity.

The 16-bit kernel changes shape with D: up to D = 128 a workgroup is 8 waves over 256 query
rows; at D = 256 it is 4 waves over 128 rows, each wave running its matrix and vector work
in turn.  D = 32 and 96 do not split a 64-key tile evenly over the workgroup's threads,
so some staging chunks are idle.  The cases below cross several query tiles of either
shape (rows 1 .. 600) and several key tiles with ragged tails, in every dtype, mask kind
and causal mode, and through the dense, packed and split-key entry points; one larger
problem per head dim is checked on sampled rows.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import sdpa_oracle
from scaled_dot_product_11_amd import (sdpa_fwd, sdpa_fwd_bias, sdpa_fwd_splitkv,
                                       sdpa_fwd_splitkv_workspace, sdpa_fwd_varlen)
from test_parity import DEV, compare, rand_inputs, run_both, to_dev

pytestmark = pytest.mark.gpu

NEW_DIMS = [32, 96, 256]
DTYPES = [torch.bfloat16, torch.float16, torch.float32]
DT_IDS = ["bf16", "f16", "f32"]
DT_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
SHAPES = [(1, 1), (33, 33), (127, 127), (129, 200), (300, 77), (77, 300), (600, 600)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def br_mask(Lq, Lk):
    return torch.ones(Lq, Lk, dtype=torch.bool).tril(Lk - Lq)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", NEW_DIMS)
@pytest.mark.parametrize("mode", ["none", "causal", "mask", "causal_mask"])
def test_head_dims_ragged(dtype, D, mode):
    causal = mode.startswith("causal")
    mask_mode = "full" if mode.endswith("mask") else None
    for n, (Lq, Lk) in enumerate(SHAPES):
        q, k, v, mask = rand_inputs(1000 + 10 * D + n, 1, 2, Lq, Lk, D, dtype,
                                    mask_mode=mask_mode)
        out, lse, ro, rl = run_both(q, k, v, mask, causal)
        compare(out, lse, ro, rl, dtype, f"{mode} D={D} Lq={Lq} Lk={Lk}")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", NEW_DIMS)
def test_head_dims_bottom_right_and_bias(dtype, D):
    for n, (Lq, Lk) in enumerate([(5, 300), (300, 77), (129, 129)]):
        g = torch.Generator().manual_seed(2000 + D + n)
        q, k, v = W.draw_qkv(g, (2, 2, Lq, D), (2, 2, Lk, D), dtype=dtype)
        out, lse = sdpa_fwd(to_dev(q), to_dev(k), to_dev(v), is_causal=2)
        torch.cuda.synchronize()
        ro, rl = sdpa_oracle(q, k, v, mask=br_mask(Lq, Lk))
        compare(out, lse, ro, rl, dtype, f"bottom-right D={D} Lq={Lq} Lk={Lk}")
        bias = torch.randn((2, 1, Lq, Lk), generator=g) * 2
        bias[torch.rand(bias.shape, generator=g) < 0.1] = float("-inf")
        out, lse = sdpa_fwd_bias(to_dev(q), to_dev(k), to_dev(v), to_dev(bias), is_causal=1)
        torch.cuda.synchronize()
        ro, rl = sdpa_oracle(q, k, v, is_causal=True, bias=bias)
        compare(out, lse, ro, rl, dtype, f"bias D={D} Lq={Lq} Lk={Lk}")


@pytest.mark.parametrize("D", NEW_DIMS)
def test_head_dims_rank3_equals_rank4_bitwise(D):
    q, k, v, mask = rand_inputs(3000 + D, 1, 3, 290, 290, D, torch.bfloat16, rank=3)
    out3, lse3, ro, rl = run_both(q, k, v, mask, True)
    compare(out3, lse3, ro, rl, torch.bfloat16, f"rank3 D={D}")
    out4, lse4 = sdpa_fwd(to_dev(q[None]), to_dev(k[None]), to_dev(v[None]), is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out3, out4[0]) and torch.equal(lse3, lse4[0])


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", NEW_DIMS)
def test_head_dims_varlen(dtype, D):
    qlen, klen = [0, 1, 77, 300, 129], [3, 1, 300, 300, 0]
    q, k, v, cq, ck = W.packed(4000 + D, qlen, klen, 3, D, dtype=dtype)
    out = torch.full(q.shape, float("nan"), dtype=dtype, device=DEV)
    out, lse = sdpa_fwd_varlen(to_dev(q), to_dev(k), to_dev(v), to_dev(cq), to_dev(ck),
                               max(qlen), out=out, is_causal=1)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any(), "every output row is written"
    cq_, ck_ = cq.tolist(), ck.tolist()
    out, lse = out.cpu(), lse.cpu()
    for s in range(len(qlen)):
        view = lambda t, a, b: t[a:b].transpose(0, 1).unsqueeze(0)
        qs, ks, vs = view(q, cq_[s], cq_[s + 1]), view(k, ck_[s], ck_[s + 1]), view(v, ck_[s], ck_[s + 1])
        ro, rl = sdpa_oracle(qs, ks, vs, is_causal=True)
        compare(view(out, cq_[s], cq_[s + 1]), lse[:, cq_[s]:cq_[s + 1]][None], ro, rl, dtype,
                f"varlen D={D} seq {s}")


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D", NEW_DIMS)
def test_head_dims_splitkv(dtype, D):
    for n, (Lq, Lk, ns) in enumerate([(1, 700, 0), (16, 3000, 5), (3, 64, 2)]):
        g = torch.Generator().manual_seed(5000 + D + n)
        q, k, v = W.draw_qkv(g, (2, 2, Lq, D), (2, 2, Lk, D), dtype=dtype)
        need = sdpa_fwd_splitkv_workspace(2, 2, Lq, Lk, D, ns, DT_CODE[dtype])
        ws = torch.full((need // 4 + 4,), float("nan"), dtype=torch.float32, device=DEV)
        out = torch.full(q.shape, float("nan"), dtype=dtype, device=DEV)
        out, lse = sdpa_fwd_splitkv(to_dev(q), to_dev(k), to_dev(v), out, is_causal=2,
                                    num_splits=ns, workspace=ws)
        torch.cuda.synchronize()
        ro, rl = sdpa_oracle(q, k, v, mask=br_mask(Lq, Lk))
        compare(out, lse, ro, rl, dtype, f"splitkv D={D} Lq={Lq} Lk={Lk} ns={ns}")


@pytest.mark.parametrize("D", NEW_DIMS)
def test_head_dims_larger_sampled(D):
    """[2, 8, 2048, D] bf16 causal, N(0,1) inputs, scale 1/sqrt(D): sampled rows against the
    oracle (several whole query tiles of either workgroup shape and the last rows)."""
    g = torch.Generator().manual_seed(6000 + D)
    q, k, v = W.draw_qkv(g, (2, 8, 2048, D))
    out, lse = sdpa_fwd(to_dev(q), to_dev(k), to_dev(v), is_causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(D)
    heads = rng.choice(16, size=3, replace=False)
    rows = np.concatenate([h * 2048 + np.r_[0:300, 1900:2048] for h in heads]).astype(np.int64)
    ro, rl = sdpa_oracle(q, k, v, is_causal=True, rows=rows)
    idx = torch.from_numpy(rows).to(DEV)
    compare(out.reshape(-1, D)[idx], lse.reshape(-1)[idx], ro, rl, torch.bfloat16,
            f"[2,8,2048,{D}] sampled")
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
