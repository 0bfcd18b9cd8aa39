"""sdpa_fwd_splitkv_noalloc, the split-key forward whose workspace is the library's static
per-device array (for callers that cannot allocate), through the C ABI: bit for bit what
sdpa_fwd_splitkv computes with a caller workspace and the same split count, and within the
parity tolerances of the fp64 oracle, on two calls in a row (the second smaller, on the
workspace the first one left behind), in every dtype and causal mode; problems needing more
than the static workspace are refused before any launch; the call can be captured into a
graph and replayed.
"""
import pytest
import torch

import workloads as W
from oracle import sdpa_oracle
from scaled_dot_product_11_amd import (SDPA_STATIC_WORKSPACE_BYTES, SdpaError, sdpa_fwd_splitkv,
                                       sdpa_fwd_splitkv_noalloc, sdpa_fwd_splitkv_workspace)
from scaled_dot_product_11_amd._binding import _DTYPES
from test_parity import DEV, compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def oracle_for(q, k, v, causal):
    Lq, Lk = q.shape[-2], k.shape[-2]
    if causal == 2:
        return sdpa_oracle(q, k, v, mask=torch.ones(Lq, Lk, dtype=torch.bool).tril(Lk - Lq))
    return sdpa_oracle(q, k, v, is_causal=causal == 1)


def check_one(seed, B, H, Lq, Lk, D, dtype, causal, splits):
    g = torch.Generator().manual_seed(seed)
    q, k, v = W.draw_qkv(g, (B, H, Lq, D), (B, H, Lk, D), dtype=dtype)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    need = sdpa_fwd_splitkv_workspace(B, H, Lq, Lk, D, splits, _DTYPES[dtype])
    assert need <= SDPA_STATIC_WORKSPACE_BYTES
    out = torch.full(q.shape, float("nan"), dtype=dtype, device=DEV)
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=DEV)
    sdpa_fwd_splitkv_noalloc(qd, kd, vd, out, lse, is_causal=causal, num_splits=splits)
    ref_o, ref_l = sdpa_fwd_splitkv(qd, kd, vd, is_causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    where = f"noalloc {tuple(q.shape)} Lk={Lk} {dtype} causal={causal} splits={splits}"
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), where
    ro, rl = oracle_for(q, k, v, causal)
    compare(out, lse, ro, rl, dtype, where)
    return need


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32],
                         ids=["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [0, 1, 2])
def test_two_calls_in_a_row_match_splitkv(dtype, causal):
    # a large split-key workspace first (about 8.5 MB at D = 128), then a smaller problem
    need1 = check_one(900 + causal, 4, 8, 16, 5000, 128, dtype, causal, 32)
    need2 = check_one(950 + causal, 1, 2, 5, 700, 64, dtype, causal, 0)
    assert need2 < need1


def test_decode_shape_matches_splitkv():
    check_one(990, 8, 32, 1, 8192, 128, torch.bfloat16, 2, 0)


def test_refuses_problems_beyond_the_static_workspace():
    # zero-stride k / v of a long sequence: validation passes, the workspace does not fit
    q = torch.zeros(8, 32, 64, 128, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(1, 1, 1, 128, dtype=torch.bfloat16, device=DEV).expand(8, 32, 65536, 128)
    need = sdpa_fwd_splitkv_workspace(8, 32, 64, 65536, 128, 64, _DTYPES[q.dtype])
    assert need > SDPA_STATIC_WORKSPACE_BYTES
    out = torch.full_like(q, 7.0)
    with pytest.raises(SdpaError) as e:
        sdpa_fwd_splitkv_noalloc(q, kv, kv, out, None, is_causal=2, num_splits=64)
    assert e.value.status == 12
    torch.cuda.synchronize()
    assert torch.all(out == 7.0), "nothing may be written on an error"


def test_graph_capture_and_replay():
    """The call records into a graph (no allocation, no memset) and each replay gives the
    eager result, with eager calls of other sizes on the same workspace in between."""
    g = torch.Generator().manual_seed(995)
    q, k, v = (t.to(DEV) for t in W.draw_qkv(g, (2, 4, 3, 128), (2, 4, 3000, 128)))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
    sdpa_fwd_splitkv_noalloc(q, k, v, out, lse, is_causal=2)  # eager, also the first call
    torch.cuda.synchronize()
    want_o, want_l = out.clone(), lse.clone()
    q2, k2, v2 = (t.to(DEV) for t in W.draw_qkv(g, (1, 2, 7, 64), (1, 2, 900, 64)))
    o2 = torch.empty_like(q2)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            sdpa_fwd_splitkv_noalloc(q, k, v, out, lse, is_causal=2)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        sdpa_fwd_splitkv_noalloc(q2, k2, v2, o2, None, is_causal=1)  # other contents
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_o) and torch.equal(lse, want_l), f"replay {rep}"
