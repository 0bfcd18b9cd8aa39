"""GPU parity of the row-by-row backward kernels -- fp32 inputs at every head dim, and D = 256
for every input type -- through sdpa_bwd, sdpa_bwd_bias and sdpa_bwd_varlen, against the
fp64 oracle's gradients.

Tolerance (max-abs over each compared block of dq, dk or dv):
    |g - g_oracle| <= TOL * max(1, max |g_oracle|)
with TOL = 1e-2 for bf16 and fp16 inputs (the tiled backward's bound; these kernels keep P
and dS in fp32, so they are closer) and TOL = 1e-4 for fp32 inputs.  The fp32 figure: every
sum runs in fp32 over at most a few hundred terms (relative error a few 1e-5), and delta =
rowsum(dout * out) carries the fp32 forward's output error (2e-5 per element), which reaches
the gradients through dS = P (dP - delta) times scale * |k| or |q|, an order of magnitude
below the bound.  Rows with no visible key and keys no query sees must be exactly zero.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import sdpa_bwd_oracle
from scaled_dot_product_11_amd import (sdpa_bwd, sdpa_bwd_bias, sdpa_bwd_varlen, sdpa_fwd,
                                       sdpa_fwd_bias, sdpa_fwd_varlen)

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2, torch.float16: 1e-2}
WORST = {}  # dtype -> largest normalised error seen (printed by the last test)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def to_dev(t):
    return None if t is None else t.to(DEV)


def nan_like(t):
    return torch.full(t.shape, math.nan, dtype=t.dtype, device=DEV)


def br_mask(Lq, Lk):
    return torch.ones(Lq, Lk, dtype=torch.bool).tril(Lk - Lq)


def visible(B, H, Lq, Lk, causal, mask=None, bias=None):
    vis = torch.ones(B, H, Lq, Lk, dtype=torch.bool)
    if causal == 1:
        vis &= torch.ones(Lq, Lk, dtype=torch.bool).tril()
    elif causal == 2:
        vis &= br_mask(Lq, Lk)
    if mask is not None:
        vis &= mask.expand(B, H, Lq, Lk)
    if bias is not None:
        vis &= torch.isfinite(bias).expand(B, H, Lq, Lk)
    return vis


def compare(got, ref, dtype, where):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.cpu().double().numpy()
        assert g.shape == r.shape, f"{where} {name}: shape"
        if r.size == 0:
            continue
        assert np.all(np.isfinite(g)), f"{where} {name}: non-finite values (unwritten?)"
        scale = max(1.0, float(np.abs(r).max()))
        err = float(np.abs(g - r).max()) / scale
        WORST[dtype] = max(WORST.get(dtype, 0.0), err)
        assert err <= TOL[dtype], f"{where} {name}: normalised max-abs error {err:.3e}"


def exact_zeros(got, vis, where):
    dq, dk, dv = (t.cpu() for t in got)
    assert torch.all(dq[~vis.any(-1)] == 0), f"{where}: dq of rows with no visible key"
    hidden = ~vis.any(-2)
    assert torch.all(dk[hidden] == 0) and torch.all(dv[hidden] == 0), f"{where}: dk, dv"


def oracle_grads(q, k, v, dout, causal, mask=None, bias=None):
    if causal == 2:
        m = br_mask(q.shape[-2], k.shape[-2])
        mask = m if mask is None else mask & m
        return sdpa_bwd_oracle(q, k, v, dout, mask=mask, bias=bias)
    return sdpa_bwd_oracle(q, k, v, dout, mask=mask, is_causal=causal == 1, bias=bias)


SHAPES = [(1, 1), (33, 33), (77, 130), (130, 77), (129, 129)]
CASES = [("none", 0), ("top_left", 1), ("bottom_right", 2), ("mask", 0), ("causal_mask", 1)]


@pytest.mark.parametrize("dtype,D", [(torch.float32, 32), (torch.float32, 64),
                                     (torch.float32, 96), (torch.float32, 128),
                                     (torch.float32, 256), (torch.bfloat16, 256),
                                     (torch.float16, 256)],
                         ids=["f32-32", "f32-64", "f32-96", "f32-128", "f32-256", "bf16-256",
                              "f16-256"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rowwise_bwd_dense(dtype, D, case):
    name, causal = case
    for n, (Lq, Lk) in enumerate(SHAPES):
        g = torch.Generator().manual_seed(3000 + 10 * n + D)
        q, k, v = W.draw_qkv(g, (2, 3, Lq, D), (2, 3, Lk, D), dtype=dtype)
        mask = None
        if "mask" in name:
            mask = torch.rand((2, 1, Lq, Lk), generator=g) < 0.3
            mask[:, :, Lq // 2, :] = False          # a row with no visible key
            mask[:, :, :, Lk // 3] = False          # a key no query sees
        dout = W.upstream_grad(3100 + n, q)
        qd, kd, vd, md = to_dev(q), to_dev(k), to_dev(v), to_dev(mask)
        out, lse = sdpa_fwd(qd, kd, vd, mask=md, is_causal=causal)
        got = sdpa_bwd(qd, kd, vd, out, to_dev(dout), lse, nan_like(q), nan_like(k),
                       nan_like(v), mask=md, is_causal=causal)
        torch.cuda.synchronize()
        where = f"{dtype} D={D} {name} Lq={Lq} Lk={Lk}"
        compare(got, oracle_grads(q, k, v, dout, causal, mask=mask), dtype, where)
        exact_zeros(got, visible(2, 3, Lq, Lk, causal, mask=mask), where)


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.bfloat16, 256)],
                         ids=["f32-64", "bf16-256"])
@pytest.mark.parametrize("causal", [0, 1, 2], ids=["none", "top_left", "bottom_right"])
def test_rowwise_bwd_bias(dtype, D, causal):
    for n, (Lq, Lk) in enumerate([(33, 33), (77, 130), (130, 77)]):
        g = torch.Generator().manual_seed(3200 + n + D)
        q, k, v = W.draw_qkv(g, (2, 3, Lq, D), (2, 3, Lk, D), dtype=dtype)
        bias = torch.randn((2, 3, Lq, Lk), generator=g) * 2
        bias[torch.rand(bias.shape, generator=g) < 0.1] = float("-inf")
        bias[0, :, 2, :] = float("-inf")            # a row with every key hidden
        dout = W.upstream_grad(3300 + n, q)
        qd, kd, vd, bd = to_dev(q), to_dev(k), to_dev(v), to_dev(bias)
        out, lse = sdpa_fwd_bias(qd, kd, vd, bd, is_causal=causal)
        got = sdpa_bwd_bias(qd, kd, vd, out, to_dev(dout), lse, bd, nan_like(q), nan_like(k),
                            nan_like(v), is_causal=causal)
        torch.cuda.synchronize()
        where = f"bias {dtype} D={D} causal={causal} Lq={Lq} Lk={Lk}"
        compare(got, oracle_grads(q, k, v, dout, causal, bias=bias), dtype, where)
        exact_zeros(got, visible(2, 3, Lq, Lk, causal, bias=bias), where)


def seq_view(t, a, b):
    """Rows a..b of a packed [tokens, H, D] tensor as the [1, H, L, D] problem."""
    return t[a:b].transpose(0, 1).unsqueeze(0)


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.float32, 256),
                                     (torch.bfloat16, 256)],
                         ids=["f32-64", "f32-256", "bf16-256"])
@pytest.mark.parametrize("causal", [0, 1, 2], ids=["none", "top_left", "bottom_right"])
def test_rowwise_bwd_varlen(dtype, D, causal):
    ql, kl = [0, 1, 77, 130, 5], [3, 1, 77, 64, 0]
    q, k, v, cq, ck = W.packed(3400 + D + causal, ql, kl, 3, D, dtype=dtype)
    dout = W.upstream_grad(3401 + D, q)
    qd, kd, vd, cqd, ckd = (to_dev(t) for t in (q, k, v, cq, ck))
    out, lse = sdpa_fwd_varlen(qd, kd, vd, cqd, ckd, max(ql), is_causal=causal)
    got = sdpa_bwd_varlen(qd, kd, vd, out, to_dev(dout), lse, cqd, ckd, max(ql), max(kl),
                          nan_like(q), nan_like(k), nan_like(v), is_causal=causal)
    torch.cuda.synchronize()
    dq, dk, dv = (t.cpu() for t in got)
    cq, ck = cq.tolist(), ck.tolist()
    for s in range(len(ql)):
        a, b, c, d = cq[s], cq[s + 1], ck[s], ck[s + 1]
        qs, ds, ks, vs = seq_view(q, a, b), seq_view(dout, a, b), seq_view(k, c, d), seq_view(v, c, d)
        mine = [seq_view(dq, a, b), seq_view(dk, c, d), seq_view(dv, c, d)]
        where = f"varlen {dtype} D={D} causal={causal} seq {s}"
        compare(mine, oracle_grads(qs, ks, vs, ds, causal), dtype, where)
        exact_zeros(mine, visible(1, 3, b - a, d - c, causal), where)


def test_rowwise_rank3_equals_rank4_and_report():
    """A rank-3 fp32 problem is the rank-4 one with B = 1, bit for bit; then the largest
    normalised errors of this file per input type are printed."""
    g = torch.Generator().manual_seed(3500)
    q, k, v = W.draw_qkv(g, (1, 4, 150, 256), dtype=torch.float32)
    dout = W.upstream_grad(3501, q)
    res = []
    for t in ((q, k, v, dout), tuple(x[0] for x in (q, k, v, dout))):
        qd, kd, vd, dd = (to_dev(x) for x in t)
        out, lse = sdpa_fwd(qd, kd, vd, is_causal=True)
        res.append(sdpa_bwd(qd, kd, vd, out, dd, lse, is_causal=True))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a[0], b)
    print("\nrow-by-row backward, largest normalised error per input type:",
          {str(k): f"{v:.2e}" for k, v in WORST.items()})
