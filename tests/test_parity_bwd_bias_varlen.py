"""GPU parity of the backward with an additive mask (sdpa_bwd_bias, the bias held constant)
and of the backward over packed variable-length batches (sdpa_bwd_varlen), through the C
ABI, against the fp64 oracle's gradients (oracle.sdpa_bwd_oracle with bias=...).

Tolerances are those of test_parity_bwd: |g - g_oracle| <= 1e-2 * max(1, max |g_oracle|)
per compared block of dq, dk or dv, and exact zeros where the method defines them (query
rows with no visible key, keys no query sees).  Bottom-right causal visibility is given to
the oracle as the shifted lower triangle (its pinned mask path).  A packed batch is, by
definition, each sequence computed on its own rows: the oracle runs per sequence on
[1, H, L_s, D] views.  Outputs start as NaN so that an element the kernels never write
shows up.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import sdpa_bwd_oracle
from scaled_dot_product_11_amd import (sdpa_bwd, sdpa_bwd_bias, sdpa_bwd_varlen, sdpa_fwd,
                                       sdpa_fwd_bias, sdpa_fwd_varlen)
from test_parity import DEV, to_dev
from test_parity_bwd import compare_grads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def br_mask(Lq, Lk):
    return torch.ones(Lq, Lk, dtype=torch.bool).tril(Lk - Lq)


def nan_like(t):
    return torch.full(t.shape, math.nan, dtype=t.dtype, device=DEV)


def visible(B, H, Lq, Lk, causal, bias=None):
    """Bool [B, H, Lq, Lk]: key j visible to query i (causal mode and -inf bias entries)."""
    vis = torch.ones(B, H, Lq, Lk, dtype=torch.bool)
    if causal == 1:
        vis &= torch.ones(Lq, Lk, dtype=torch.bool).tril()
    elif causal == 2:
        vis &= br_mask(Lq, Lk)
    if bias is not None:
        vis &= torch.isfinite(bias).expand(B, H, Lq, Lk)
    return vis


def assert_exact_zeros(got, vis, where):
    dq, dk, dv = (t.cpu() for t in got)
    assert torch.all(dq[~vis.any(-1)] == 0), f"{where}: dq of rows with no visible key"
    hidden = ~vis.any(-2)
    assert torch.all(dk[hidden] == 0) and torch.all(dv[hidden] == 0), \
        f"{where}: dk, dv of keys no query sees"


# ---------------------------------------------------------------------------------------
# additive mask

def random_bias(seed, shape, inf_frac=0.1):
    g = torch.Generator().manual_seed(seed)
    b = torch.randn(shape, generator=g) * 2
    b[torch.rand(shape, generator=g) < inf_frac] = float("-inf")
    return b


def bias_grads(q, k, v, dout, bias, causal, scale=None):
    qd, kd, vd, bd = to_dev(q), to_dev(k), to_dev(v), to_dev(bias)
    out, lse = sdpa_fwd_bias(qd, kd, vd, bd, is_causal=causal, scale=scale)
    got = sdpa_bwd_bias(qd, kd, vd, out, to_dev(dout), lse, bd, nan_like(q), nan_like(k),
                        nan_like(v), is_causal=causal, scale=scale)
    torch.cuda.synchronize()
    return got


def bias_oracle(q, k, v, dout, bias, causal, scale=None):
    if causal == 2:
        return sdpa_bwd_oracle(q, k, v, dout, mask=br_mask(q.shape[-2], k.shape[-2]),
                               bias=bias, scale=scale)
    return sdpa_bwd_oracle(q, k, v, dout, is_causal=causal == 1, bias=bias, scale=scale)


SHAPES = [(1, 1), (33, 33), (64, 64), (129, 129), (200, 200), (77, 300), (300, 77)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("D", [32, 64, 96, 128])
@pytest.mark.parametrize("causal", [0, 1, 2], ids=["none", "top_left", "bottom_right"])
def test_bwd_bias_small(dtype, D, causal):
    for n, (Lq, Lk) in enumerate(SHAPES):
        g = torch.Generator().manual_seed(1100 + 10 * n + D + causal)
        q, k, v = W.draw_qkv(g, (2, 3, Lq, D), (2, 3, Lk, D), dtype=dtype)
        dout = W.upstream_grad(1200 + n, q)
        # full [B, H] bias on even shapes, head-broadcast [B, 1] on odd ones
        bias = random_bias(1300 + n, (2, 1 if n % 2 else 3, Lq, Lk))
        if Lq > 3:
            bias[0, :, 2, :] = float("-inf")  # a row with every key hidden
        if Lk > 3:
            bias[1, :, :, 1] = float("-inf")  # a key no query of batch 1 sees
        where = f"bias bwd {dtype} D={D} causal={causal} Lq={Lq} Lk={Lk}"
        got = bias_grads(q, k, v, dout, bias, causal)
        compare_grads(got, bias_oracle(q, k, v, dout, bias, causal), where)
        assert_exact_zeros(got, visible(2, 3, Lq, Lk, causal, bias), where)


def test_bwd_bias_zero_is_sdpa_bwd_bitwise():
    """An all-zero bias adds exactly 0 to every base-2 score: the same bits as sdpa_bwd."""
    g = torch.Generator().manual_seed(1400)
    q, k, v = W.draw_qkv(g, (2, 3, 300, 128), (2, 3, 260, 128))
    dout = to_dev(W.upstream_grad(1401, q))
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    for causal in (0, 1, 2):
        out, lse = sdpa_fwd(qd, kd, vd, is_causal=causal)
        zero = torch.zeros(1, 1, 300, 260, device=DEV)
        a = sdpa_bwd_bias(qd, kd, vd, out, dout, lse, zero, is_causal=causal)
        b = sdpa_bwd(qd, kd, vd, out, dout, lse, is_causal=causal)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), causal


def test_bwd_bias_zero_minus_inf_is_bool_mask_bitwise():
    """A 0 / -inf bias hides exactly the keys a False mask entry hides: the same bits as
    sdpa_bwd with that mask, on the same out and lse."""
    g = torch.Generator().manual_seed(1410)
    q, k, v = W.draw_qkv(g, (2, 2, 200, 64), (2, 2, 230, 64))
    m = torch.rand(2, 2, 200, 230, generator=g) < 0.3
    m[1, 0, 7] = False
    bias = torch.where(m, 0.0, float("-inf"))
    dout = to_dev(W.upstream_grad(1411, q))
    qd, kd, vd, md, bd = to_dev(q), to_dev(k), to_dev(v), to_dev(m), to_dev(bias)
    out, lse = sdpa_fwd(qd, kd, vd, mask=md, is_causal=True)
    a = sdpa_bwd_bias(qd, kd, vd, out, dout, lse, bd, is_causal=True)
    b = sdpa_bwd(qd, kd, vd, out, dout, lse, mask=md, is_causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_bias_strided_bias_and_rank3():
    """A bias [Lq, Lk] broadcast over batch and heads (strides 0, 0), and rank-3 inputs
    (the rank-4 problem with B = 1, the same bits)."""
    g = torch.Generator().manual_seed(1420)
    q, k, v = W.draw_qkv(g, (1, 4, 150, 64), (1, 4, 170, 64))
    dout = W.upstream_grad(1421, q)
    bias = random_bias(1422, (150, 170), inf_frac=0.05)
    g4 = bias_grads(q, k, v, dout, bias, 1)
    g3 = bias_grads(q[0], k[0], v[0], dout[0], bias, 1)
    for a, b in zip(g4, g3):
        assert torch.equal(a[0], b)
    compare_grads(g4, bias_oracle(q, k, v, dout, bias[None, None], 1), "broadcast bias")


def test_bwd_bias_alibi_heads():
    """ALiBi-style per-head distance penalties [1, 8, 1024, 1024], batch 2, causal, D=128:
    two whole heads against the oracle, plus sum_j dv_j = sum_i dout_i for every head (each
    row sees key 0, so the rows of P sum to one)."""
    H, L, D = 8, 1024, 128
    g = torch.Generator().manual_seed(1430)
    q, k, v = W.draw_qkv(g, (2, H, L, D))
    dout = W.upstream_grad(1431, q)
    i = torch.arange(L)[:, None]
    j = torch.arange(L)[None, :]
    slopes = 0.5 * 2.0 ** -torch.arange(H, dtype=torch.float32)
    bias = (-slopes[:, None, None] * (i - j).abs()).unsqueeze(0)
    dq, dk, dv = bias_grads(q, k, v, dout, bias, 1)
    sel = lambda t: torch.stack([t[0, 0], t[1, 7]])[None]
    bsel = torch.stack([bias[0, 0], bias[0, 7]])[None]
    ref = sdpa_bwd_oracle(sel(q), sel(k), sel(v), sel(dout), is_causal=True, bias=bsel)
    compare_grads([sel(t) for t in (dq, dk, dv)], ref, "alibi heads (0,0) (1,7)")
    sdv = dv.double().sum(dim=2).cpu()
    sdo = dout.double().sum(dim=2)
    assert float((sdv - sdo).abs().max()) <= 1e-2 * max(1.0, float(sdo.abs().max()))


# ---------------------------------------------------------------------------------------
# packed variable-length batches

def seq_view(t, lo, hi):
    """Rows lo..hi-1 of a packed [tokens, H, D] tensor as the [1, H, L, D] view."""
    return t[lo:hi].transpose(0, 1).unsqueeze(0)


def varlen_grads(q, k, v, dout, cq, ck, causal, max_q=None, max_k=None):
    qd, kd, vd, cqd, ckd = (to_dev(t) for t in (q, k, v, cq, ck))
    lq = (cq[1:] - cq[:-1]).tolist() or [0]
    lk = (ck[1:] - ck[:-1]).tolist() or [0]
    max_q = max(lq) if max_q is None else max_q
    max_k = max(lk) if max_k is None else max_k
    out, lse = sdpa_fwd_varlen(qd, kd, vd, cqd, ckd, max_q, is_causal=causal)
    got = sdpa_bwd_varlen(qd, kd, vd, out, to_dev(dout), lse, cqd, ckd, max_q, max_k,
                          nan_like(q), nan_like(k), nan_like(v), is_causal=causal)
    torch.cuda.synchronize()
    return got


def check_varlen_grads(q, k, v, dout, cq, ck, got, causal, where, seqs=None):
    """Every sequence (or those in `seqs`) against the oracle on its own rows."""
    cq, ck = cq.tolist(), ck.tolist()
    dq, dk, dv = (t.cpu() for t in got)
    for s in range(len(cq) - 1) if seqs is None else seqs:
        a, b, c, d = cq[s], cq[s + 1], ck[s], ck[s + 1]
        Lq, Lk = b - a, d - c
        qs, ds = seq_view(q, a, b), seq_view(dout, a, b)
        ks, vs = seq_view(k, c, d), seq_view(v, c, d)
        mask = br_mask(Lq, Lk) if causal == 2 else None
        ref = sdpa_bwd_oracle(qs, ks, vs, ds, mask=mask, is_causal=causal == 1)
        mine = [seq_view(dq, a, b), seq_view(dk, c, d), seq_view(dv, c, d)]
        compare_grads(mine, ref, f"{where} seq {s} (Lq={Lq}, Lk={Lk})")
        assert_exact_zeros(mine, visible(1, q.shape[1], Lq, Lk, causal), f"{where} seq {s}")


Q_LENGTHS = [0, 1, 77, 256, 300, 5, 129]
K_LENGTHS = [3, 1, 77, 300, 256, 0, 129]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("D", [32, 64, 96, 128])
@pytest.mark.parametrize("causal", [0, 1, 2], ids=["none", "top_left", "bottom_right"])
def test_bwd_varlen_small(dtype, D, causal):
    q, k, v, cq, ck = W.packed(1500 + D + causal, Q_LENGTHS, K_LENGTHS, 3, D, dtype=dtype)
    dout = W.upstream_grad(1501 + D, q)
    got = varlen_grads(q, k, v, dout, cq, ck, causal)
    for name, t in zip(("dq", "dk", "dv"), got):
        assert not torch.isnan(t.float()).any(), f"{name}: every row is written"
    check_varlen_grads(q, k, v, dout, cq, ck, got, causal, f"varlen bwd {dtype} D={D} {causal}")


def test_bwd_varlen_equals_dense_bitwise():
    """Equal lengths: the packed batch [B*L, H, D] is the dense [B, L, H, D] problem viewed
    as [B, H, L, D]; its gradients are the dense backward's, bit for bit."""
    B, L, H, D = 3, 300, 4, 128
    q, k, v, cq, ck = W.packed(1510, [L] * B, [L] * B, H, D)
    dout = W.upstream_grad(1511, q)
    for causal in (0, 1):
        got = varlen_grads(q, k, v, dout, cq, ck, causal)
        dense = [to_dev(t).view(B, L, H, D).transpose(1, 2) for t in (q, k, v, dout)]
        out, lse = sdpa_fwd(*dense[:3], is_causal=causal)
        ref = sdpa_bwd(*dense[:3], out, dense[3], lse, is_causal=causal)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a.view(B, L, H, D), b.transpose(1, 2)), causal


def test_bwd_varlen_strided_from_packed_qkv():
    """q, k, v and dq, dk, dv as slices of [tokens, 3, H, D] buffers (token stride 3*H*D)."""
    lengths = [70, 1, 200]
    T, H, D = sum(lengths), 2, 64
    g = torch.Generator().manual_seed(1520)
    qkv = torch.randn(T, 3, H, D, generator=g).to(torch.bfloat16)
    dout = W.upstream_grad(1521, qkv[:, 0].contiguous())
    cq = torch.tensor([0, 70, 71, 271], dtype=torch.int32)
    qkv_d, cqd = qkv.to(DEV), cq.to(DEV)
    out, lse = sdpa_fwd_varlen(qkv_d[:, 0], qkv_d[:, 1], qkv_d[:, 2], cqd, cqd, 200,
                               is_causal=True)
    grads = torch.full((T, 3, H, D), math.nan, dtype=torch.bfloat16, device=DEV)
    got = sdpa_bwd_varlen(qkv_d[:, 0], qkv_d[:, 1], qkv_d[:, 2], out, to_dev(dout), lse, cqd,
                          cqd, 200, 200, grads[:, 0], grads[:, 1], grads[:, 2], is_causal=True)
    torch.cuda.synchronize()
    assert got[0].data_ptr() == grads[:, 0].data_ptr() and not got[0].is_contiguous()
    check_varlen_grads(qkv[:, 0], qkv[:, 1], qkv[:, 2], dout, cq, cq, got, 1, "packed qkv")


def test_bwd_varlen_documents_sampled():
    """Packed documents, 32768 tokens, H=32, D=128, causal: the five shortest documents in
    full on two heads; the longest through problems the oracle solves exactly (dq of single
    query rows against their visible keys, dk and dv of its last 128 keys, which only its
    last 128 queries see)."""
    wl = W.config_varlen()
    cq = wl.extra["cu_seqlens_q"]
    lengths = wl.extra["lengths"]
    dout = W.upstream_grad(1530, wl.q)
    got = varlen_grads(wl.q, wl.k, wl.v, dout, cq, cq, 1, max(lengths), max(lengths))
    for name, t in zip(("dq", "dk", "dv"), got):
        assert not torch.isnan(t.float()).any(), f"{name}: every row is written"
    heads = [0, 31]
    pick = lambda t: t[:, heads]
    order = np.argsort(lengths)
    check_varlen_grads(pick(wl.q), pick(wl.k), pick(wl.v), pick(dout), cq, cq,
                       [pick(t) for t in got], 1, wl.name + " short docs",
                       seqs=[int(s) for s in order[:5]])
    s = int(order[-1])
    lo, L = int(cq[s]), lengths[s]
    dq, dk, dv = (t.cpu() for t in got)
    rng = np.random.default_rng(1531)
    rows = sorted({0, 1, 127, 128, L - 1} | set(rng.integers(0, L, size=8).tolist()))
    for h in heads:
        for i in rows:
            t = lo + i
            ref = sdpa_bwd_oracle(seq_view(wl.q, t, t + 1)[:, h:h + 1],
                                  seq_view(wl.k, lo, t + 1)[:, h:h + 1],
                                  seq_view(wl.v, lo, t + 1)[:, h:h + 1],
                                  seq_view(dout, t, t + 1)[:, h:h + 1])
            compare_grads([seq_view(dq, t, t + 1)[:, h:h + 1]], ref[:1],
                          f"longest doc h={h} dq row {i}")
    T = 128
    tri = torch.arange(L)[None, :] <= (torch.arange(T)[:, None] + (L - T))
    ref = sdpa_bwd_oracle(pick(seq_view(wl.q, lo + L - T, lo + L)), pick(seq_view(wl.k, lo, lo + L)),
                          pick(seq_view(wl.v, lo, lo + L)),
                          pick(seq_view(dout, lo + L - T, lo + L)), mask=tri[None, None])
    compare_grads([pick(seq_view(dk, lo + L - T, lo + L)), pick(seq_view(dv, lo + L - T, lo + L))],
                  [ref[1][:, :, L - T:], ref[2][:, :, L - T:]], "longest doc last keys",
                  names=("dk", "dv"))
