"""GPU parity: the HIP kernel (through the C ABI) against the fp64 oracle.

Tolerances (max-abs, element by element): out 1e-2 for bf16 (and fp16, read the same way)
and 2e-5 for fp32 inputs,
LSE 1e-3 on finite rows; rows with no visible key must be exactly 0 with LSE -inf on
both sides.  Small problems are compared on every output; the full-size workloads on
sampled rows (the oracle evaluates them one by one) plus properties that hold at any
size.
"""
import math

import numpy as np
import pytest
import torch

import parity_log
import workloads as W
from oracle import sdpa_oracle
from scaled_dot_product_11_amd import (SDPA_BF16, SDPA_F16, SdpaError, sdpa_fwd, sdpa_fwd_bias,
                                      sdpa_fwd_varlen, sdpa_plan)

pytestmark = pytest.mark.gpu

OUT_TOL = {torch.bfloat16: 1e-2, torch.float16: 1e-2, torch.float32: 2e-5}
LSE_TOL = 1e-3
# significand bits of the output format: the bound applies to the value the kernel
# computes, and storing it in the output dtype adds at most half a unit in the last place
OUT_BITS = {torch.bfloat16: 8, torch.float16: 11, torch.float32: 24}
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def to_dev(t):
    if t is None:
        return None
    d = t.to(DEV)
    assert d.stride() == t.stride()
    return d


def half_ulp(x, bits):
    """Half the spacing of `bits`-bit floating-point numbers around |x| (0 at 0)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - bits), 0.0)


def compare(out, lse, ref_out, ref_lse, dtype, where="", literal=False):
    """Element-wise gate: |out - oracle| <= tol + half an output ulp (the bound applies to the
    value the kernel computes; storing it in the output dtype adds at most half an ulp).  With
    literal=True (the five configurations the 1e-2 / 2e-5 criterion is stated for) the raw
    error must also be within tol itself.  Every comparison records the raw max-abs error and
    the number of elements beyond the literal tolerance (printed at the end of the session);
    returns the raw max-abs error."""
    out = out.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    assert out.shape == ref_out.shape and lse.shape == ref_lse.shape
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{where}: empty-row pattern differs"
    assert np.all(lse[~fin] == -np.inf), f"{where}: empty rows need lse = -inf"
    assert np.all(out[~fin] == 0.0), f"{where}: empty rows need out = 0"
    diff = np.abs(out - ref_out)
    mag = np.maximum(np.abs(out), np.abs(ref_out))
    bound = OUT_TOL[dtype] + half_ulp(mag, OUT_BITS[dtype])
    worst = np.max(diff - bound) if out.size else -1.0
    err = float(np.max(diff)) if out.size else 0.0
    beyond = int(np.count_nonzero(diff > OUT_TOL[dtype]))
    lerr = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    parity_log.record(where, str(dtype).replace("torch.", ""), out.size, err, beyond, lerr,
                      literal)
    assert worst <= 0, f"{where}: out error {err:.3e} exceeds tol + half ulp by {worst:.3e}"
    if literal:
        assert err <= OUT_TOL[dtype], f"{where}: out error {err:.3e} beyond {OUT_TOL[dtype]}"
    assert lerr <= LSE_TOL, f"{where}: lse max-abs error {lerr:.3e}"
    return err


def rand_inputs(seed, B, H, Lq, Lk, D, dtype, rank=4, mask_mode=None, p_keep=0.3):
    g = torch.Generator().manual_seed(seed)
    shp_q, shp_k = (B, H, Lq, D), (B, H, Lk, D)
    q, k, v = W.draw_qkv(g, shp_q, shp_k, dtype=dtype)
    mask = None
    if mask_mode is not None:
        mask = torch.rand((B, 1 if mask_mode == "bcast" else H, Lq, Lk), generator=g) < p_keep
        if Lq > 3:  # a few fully hidden rows
            mask[:, :, torch.randperm(Lq, generator=g)[:2], :] = False
    if rank == 3:
        assert B == 1
        q, k, v = q[0], k[0], v[0]
        mask = None if mask is None else mask[0]
    return q, k, v, mask


def run_both(q, k, v, mask, causal, scale=None):
    out, lse = sdpa_fwd(to_dev(q), to_dev(k), to_dev(v), mask=to_dev(mask), is_causal=causal,
                        scale=scale)
    torch.cuda.synchronize()
    ref_out, ref_lse = sdpa_oracle(q, k, v, mask=mask, is_causal=causal, scale=scale)
    return out, lse, ref_out, ref_lse


def test_config1_full():
    wl = W.config1()
    out, lse, ro, rl = run_both(wl.q, wl.k, wl.v, None, True, wl.scale)
    compare(out, lse, ro, rl, torch.float32, "c1", literal=True)


SHAPES = [(1, 1), (33, 33), (64, 64), (127, 127), (129, 129), (200, 200), (77, 300), (300, 77)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32],
                         ids=["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", ["none", "causal", "mask", "causal_mask", "bcast_mask"])
def test_ragged_small(dtype, D, mode):
    causal = mode.startswith("causal")
    mask_mode = {"mask": "full", "causal_mask": "full", "bcast_mask": "bcast"}.get(mode)
    for n, (Lq, Lk) in enumerate(SHAPES):
        q, k, v, mask = rand_inputs(100 + n, 2, 2, Lq, Lk, D, dtype, mask_mode=mask_mode)
        out, lse, ro, rl = run_both(q, k, v, mask, causal)
        compare(out, lse, ro, rl, dtype, f"{mode} D={D} Lq={Lq} Lk={Lk}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("D", [32, 64, 96, 128])
def test_small_problem_tile_equals_two_group_tile(dtype, D):
    """The one-group tile (128 rows, 4 waves) and the two-group tile (256 rows, 8 waves in
    alternating phases) give each 32-row slice the same sequence of operations, so they agree
    bit for bit.  Which tile a launch takes is asserted through sdpa_plan.  At D = 96 and 128
    a 2-head problem runs the one-group tile and a 1040-head problem the two-group tile; their
    shared heads are compared with no mask, both causal alignments, a boolean mask broadcast
    over heads and an additive mask.  At D <= 64 every dense problem runs the one-group tile
    (the 1040-head comparison is then a determinism check), and the two-group side is the same
    two heads packed as one sequence through sdpa_fwd_varlen, which always takes the
    two-group tile (no mask, both causal alignments).  Everything is also checked against the
    oracle."""
    code = {torch.bfloat16: SDPA_BF16, torch.float16: SDPA_F16}[dtype]
    for n, (Lq, Lk) in enumerate([(33, 33), (129, 200), (300, 77), (300, 300)]):
        g = torch.Generator().manual_seed(4100 + n + D)
        q, k, v = W.draw_qkv(g, (1, 1040, Lq, D), (1, 1040, Lk, D), dtype=dtype)
        bmask = torch.rand((1, 1, Lq, Lk), generator=g) < 0.3
        bmask[..., Lq // 2, :] = False  # one fully hidden row
        assert sdpa_plan(4, 1, 2, Lq, Lk, D, 1, code).threads == 256, "2 heads: one-group tile"
        big_threads = sdpa_plan(4, 1, 1040, Lq, Lk, D, 1, code).threads
        assert big_threads == (512 if D >= 96 else 256), (D, Lq, big_threads)
        for mode in (0, 1, 2, "mask"):
            causal = 0 if mode == "mask" else mode
            m = to_dev(bmask) if mode == "mask" else None
            big_o, big_l = sdpa_fwd(to_dev(q), to_dev(k), to_dev(v), mask=m, is_causal=causal)
            small_o, small_l = sdpa_fwd(to_dev(q[:, :2].contiguous()), to_dev(k[:, :2].contiguous()),
                                        to_dev(v[:, :2].contiguous()), mask=m, is_causal=causal)
            torch.cuda.synchronize()
            where = f"D={D} Lq={Lq} Lk={Lk} mode={mode}"
            assert torch.equal(big_o[:, :2], small_o) and torch.equal(big_l[:, :2], small_l), where
            if D <= 64 and mode != "mask":
                # the same two heads packed as one sequence: the two-group tile
                pq, pk, pv = (to_dev(t[0, :2].transpose(0, 1).contiguous()) for t in (q, k, v))
                cq = torch.tensor([0, Lq], dtype=torch.int32, device=DEV)
                ck = torch.tensor([0, Lk], dtype=torch.int32, device=DEV)
                vo, vl = sdpa_fwd_varlen(pq, pk, pv, cq, ck, Lq, is_causal=causal)
                torch.cuda.synchronize()
                assert torch.equal(vo.transpose(0, 1), small_o[0]), where + " varlen"
                assert torch.equal(vl, small_l[0]), where + " varlen lse"
            heads = [0, 1, 263, 1039]
            rows = np.concatenate([h * Lq + np.arange(Lq) for h in heads]).astype(np.int64)
            if mode == 2:
                tri = torch.ones(Lq, Lk, dtype=torch.bool).tril(Lk - Lq)
                ro, rl = sdpa_oracle(q, k, v, mask=tri, rows=rows)
            else:
                ro, rl = sdpa_oracle(q, k, v, mask=bmask if mode == "mask" else None,
                                     is_causal=mode == 1, rows=rows)
            idx = torch.from_numpy(rows).to(DEV)
            compare(big_o.reshape(-1, D)[idx], big_l.reshape(-1)[idx], ro, rl, dtype, where)
        # an additive mask broadcast over heads takes the same two tiles
        bias = torch.randn((1, 1, Lq, Lk), generator=g) * 2
        bias[torch.rand(bias.shape, generator=g) < 0.1] = float("-inf")
        big_o, big_l = sdpa_fwd_bias(to_dev(q), to_dev(k), to_dev(v), to_dev(bias), is_causal=True)
        small_o, small_l = sdpa_fwd_bias(to_dev(q[:, :2].contiguous()), to_dev(k[:, :2].contiguous()),
                                         to_dev(v[:, :2].contiguous()), to_dev(bias), is_causal=True)
        torch.cuda.synchronize()
        where = f"bias D={D} Lq={Lq} Lk={Lk}"
        assert torch.equal(big_o[:, :2], small_o) and torch.equal(big_l[:, :2], small_l), where
        rows = np.concatenate([h * Lq + np.arange(Lq) for h in (0, 1039)]).astype(np.int64)
        ro, rl = sdpa_oracle(q, k, v, is_causal=True, bias=bias, rows=rows)
        idx = torch.from_numpy(rows).to(DEV)
        compare(big_o.reshape(-1, D)[idx], big_l.reshape(-1)[idx], ro, rl, dtype, where)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32],
                         ids=["bf16", "f16", "f32"])
def test_rank3_small_and_equals_rank4(dtype):
    q, k, v, mask = rand_inputs(7, 1, 3, 150, 150, 64, dtype, rank=3, mask_mode="full")
    out3, lse3, ro, rl = run_both(q, k, v, mask, True)
    compare(out3, lse3, ro, rl, dtype, "rank3")
    out4, lse4 = sdpa_fwd(to_dev(q[None]), to_dev(k[None]), to_dev(v[None]),
                          mask=to_dev(mask[None]), is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out3, out4[0]) and torch.equal(lse3, lse4[0])


def test_strided_inputs_and_output():
    """[B,L,H,D] buffers viewed as [B,H,L,D] for q, k, v and out: same bits as contiguous."""
    g = torch.Generator().manual_seed(21)
    bufs = [torch.randn(2, 173, 4, 128, generator=g).to(torch.bfloat16) for _ in range(3)]
    q, k, v = (b.transpose(1, 2) for b in bufs)
    out, lse, ro, rl = run_both(q, k, v, None, True)
    compare(out, lse, ro, rl, torch.bfloat16, "strided")
    out_buf = torch.empty(2, 173, 4, 128, dtype=torch.bfloat16, device=DEV)
    out2, lse2 = sdpa_fwd(*(to_dev(x.contiguous()) for x in (q, k, v)),
                          out=out_buf.transpose(1, 2), is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(lse2, lse)


def test_no_keys_and_no_queries():
    q = torch.randn(1, 2, 40, 64, device=DEV).to(torch.bfloat16)
    kv = torch.empty(1, 2, 0, 64, device=DEV, dtype=torch.bfloat16)
    out, lse = sdpa_fwd(q, kv, kv, is_causal=False)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == -math.inf)
    q0 = torch.empty(1, 2, 0, 64, device=DEV, dtype=torch.bfloat16)
    kk = torch.randn(1, 2, 5, 64, device=DEV).to(torch.bfloat16)
    out, lse = sdpa_fwd(q0, kk, kk)
    assert out.shape == (1, 2, 0, 64)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32],
                         ids=["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [1, 2], ids=["top_left", "bottom_right"])
def test_causal_with_no_keys(dtype, causal):
    """Causal problems with no keys (the one-group tile for 16-bit inputs): every row is
    empty, so out = 0 and lse = -inf, also with an additive mask."""
    q = torch.randn(2, 3, 70, 128, device=DEV).to(dtype)
    kv = torch.empty(2, 3, 0, 128, device=DEV, dtype=dtype)
    out = torch.full(q.shape, float("nan"), device=DEV, dtype=dtype)
    out, lse = sdpa_fwd(q, kv, kv, out, is_causal=causal)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == -math.inf)
    bias = torch.zeros(1, 1, 70, 0, device=DEV)
    out2, lse2 = sdpa_fwd_bias(q, kv, kv, bias, is_causal=causal)
    torch.cuda.synchronize()
    assert torch.all(out2 == 0) and torch.all(lse2 == -math.inf)


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.0])
def test_unusual_scales(scale):
    q, k, v, _ = rand_inputs(31, 1, 2, 90, 90, 64, torch.bfloat16)
    out, lse, ro, rl = run_both(q, k, v, None, True, scale=scale)
    compare(out, lse, ro, rl, torch.bfloat16, f"scale={scale}")


def test_fully_masked_rows_are_zero():
    q, k, v, _ = rand_inputs(41, 1, 2, 130, 130, 128, torch.bfloat16)
    mask = torch.rand(1, 2, 130, 130, generator=torch.Generator().manual_seed(1)) < 0.05
    mask[:, :, ::3, :] = False
    out, lse, ro, rl = run_both(q, k, v, mask, False)
    compare(out, lse, ro, rl, torch.bfloat16, "masked rows")
    assert torch.all(out[:, :, ::3] == 0) and torch.all(lse[:, :, ::3] == -math.inf)


def test_invalid_arguments_raise():
    q = torch.randn(1, 1, 16, 80, device=DEV).to(torch.bfloat16)
    with pytest.raises(SdpaError):
        sdpa_fwd(q, q, q)
    q = torch.randn(1, 1, 16, 64, device=DEV).to(torch.float64)
    with pytest.raises(SdpaError):
        sdpa_fwd(q, q, q)


# ---------------------------------------------------------------------------------------
# Full-size workloads: sampled rows against the oracle, and properties.
# ---------------------------------------------------------------------------------------

def sample_rows(B, H, Lq, n_random, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for bh in {0, B * H - 1, int(rng.integers(B * H))}:
        for i in (0, 1, 63, 64, 127, 128, Lq // 2, Lq - 2, Lq - 1):
            if 0 <= i < Lq:
                rows.add(bh * Lq + i)
    rows.update(rng.choice(B * H * Lq, size=n_random, replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def check_sampled(wl, out, lse, n_random=300, seed=0, extra_rows=None):
    B, H, Lq, Lk, D = wl.shape4()
    rows = sample_rows(B, H, Lq, n_random, seed)
    if extra_rows is not None:
        rows = np.unique(np.concatenate([rows, extra_rows]))
    ro, rl = sdpa_oracle(wl.q, wl.k, wl.v, mask=wl.mask, is_causal=wl.is_causal, scale=wl.scale,
                         rows=rows)
    go = out.reshape(-1, D)[torch.from_numpy(rows).to(out.device)]
    gl = lse.reshape(-1)[torch.from_numpy(rows).to(lse.device)]
    return compare(go, gl, ro, rl, wl.q.dtype, wl.name, literal=True)


def run_wl(wl):
    out, lse = sdpa_fwd(to_dev(wl.q), to_dev(wl.k), to_dev(wl.v), mask=to_dev(wl.mask),
                        is_causal=wl.is_causal, scale=wl.scale)
    torch.cuda.synchronize()
    return out, lse


def test_config2_full_oracle():
    wl = W.config2()
    out, lse = run_wl(wl)
    ro, rl = sdpa_oracle(wl.q, wl.k, wl.v, is_causal=True, scale=wl.scale)
    compare(out, lse, ro, rl, torch.bfloat16, wl.name, literal=True)


def test_config2_fp16_full_oracle():
    """The c2 draws in fp16 (bf16 values are exact in fp16 at these magnitudes)."""
    wl = W.config2()
    q, k, v = (t.to(torch.float16) for t in (wl.q, wl.k, wl.v))
    out, lse = sdpa_fwd(to_dev(q), to_dev(k), to_dev(v), is_causal=True, scale=wl.scale)
    torch.cuda.synchronize()
    ro, rl = sdpa_oracle(q, k, v, is_causal=True, scale=wl.scale)
    compare(out, lse, ro, rl, torch.float16, wl.name + " fp16")


def test_config3_rank3_equals_rank4_bitwise():
    wl3, wl4 = W.config3(rank=3), W.config3(rank=4)
    out3, lse3 = run_wl(wl3)
    out4, lse4 = run_wl(wl4)
    assert torch.equal(out3, out4.reshape(128, 2048, 128))
    assert torch.equal(lse3, lse4.reshape(128, 2048))
    check_sampled(wl3, out3, lse3, seed=3)


def test_config4_strided_long_sequence():
    wl = W.config4()
    out, lse = run_wl(wl)
    check_sampled(wl, out, lse, seed=4)
    # causal row 0 of every head is v[0] exactly (one visible key, weight 1)
    assert torch.equal(out[:, :, 0, :], to_dev(wl.v[:, :, 0, :]))


def test_config5_bool_mask_and_empty_rows():
    wl = W.config5()
    out, lse = run_wl(wl)
    empty = wl.extra["empty_rows"]  # [2, 205] query rows fully hidden per batch entry
    for b in range(2):
        rows = empty[b].to(DEV)
        assert torch.all(out[b][:, rows] == 0)
        assert torch.all(lse[b][:, rows] == -math.inf)
    extra = np.array([(b * 8 + h) * 4096 + int(i) for b in range(2) for h in (0, 7)
                      for i in empty[b][:5]], dtype=np.int64)
    check_sampled(wl, out, lse, seed=5, extra_rows=extra)


def test_rows_sum_to_one_at_size():
    """V = 1 makes every visible row exactly 1 in exact arithmetic."""
    q, k, _, _ = rand_inputs(51, 1, 4, 2048, 2048, 128, torch.bfloat16)
    v = torch.ones_like(k)
    out, _ = sdpa_fwd(to_dev(q), to_dev(k), to_dev(v), is_causal=True)
    torch.cuda.synchronize()
    err = (out.float() - 1).abs().max().item()
    assert err <= OUT_TOL[torch.bfloat16], err


def test_zero_query_prefix_mean_at_size():
    _, k, v, _ = rand_inputs(52, 1, 2, 1024, 1024, 64, torch.bfloat16)
    q = torch.zeros(1, 2, 1024, 64, dtype=torch.bfloat16)
    out, lse = sdpa_fwd(to_dev(q), to_dev(k), to_dev(v), is_causal=True, scale=1.0)
    torch.cuda.synchronize()
    prefix = torch.cumsum(v.double(), dim=2) / torch.arange(1, 1025).double()[None, None, :, None]
    assert (out.cpu().double() - prefix).abs().max().item() <= OUT_TOL[torch.bfloat16]
    ref_lse = torch.log(torch.arange(1, 1025).double())
    assert (lse.cpu().double() - ref_lse).abs().max().item() <= LSE_TOL


def test_deterministic_repeats():
    wl = W.config2()
    out1, lse1 = run_wl(wl)
    for _ in range(3):
        out2, lse2 = run_wl(wl)
        assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
