"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle comparisons.

This module only draws numbers and lays them out; it holds none of the attention
arithmetic.  Draws happen on the CPU with a seeded torch.Generator, in the order
q, k, v, then the mask, and the contiguous buffers are then moved to the requested
device, where any view (transpose, reshape, expand) is applied, so that host and device
copies hold identical bits.

The five named workloads follow the configurations this project is measured on: the
pages publish no shapes, so every workload is synthetic, i.i.d. normal, cast to bf16
with round-to-nearest-even where bf16 is named.
"""
import math
from dataclasses import dataclass, field
from typing import Optional

import torch


@dataclass
class Workload:
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    mask: Optional[torch.Tensor]
    is_causal: bool
    scale: float
    description: str
    extra: dict = field(default_factory=dict)

    @property
    def rank(self) -> int:
        return self.q.dim()

    def shape4(self):
        """(B, H, Lq, Lk, D) with rank 3 read as B = 1."""
        if self.q.dim() == 3:
            return 1, self.q.shape[0], self.q.shape[1], self.k.shape[1], self.q.shape[2]
        B, H, Lq, D = self.q.shape
        return B, H, Lq, self.k.shape[2], D


def _randn(g, shape, dtype, mult=1.0):
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if mult != 1.0:
        x = x * mult
    return x.to(dtype)


def draw_qkv(g, q_shape, k_shape=None, dtype=torch.bfloat16, mult=1.0):
    """Three contiguous CPU tensors of i.i.d. N(0, mult^2) drawn from g in the order q, k, v."""
    k_shape = q_shape if k_shape is None else k_shape
    return _randn(g, q_shape, dtype, mult), _randn(g, k_shape, dtype, mult), \
        _randn(g, k_shape, dtype, mult)


def random_qkv(seed, q_shape, k_shape=None, dtype=torch.bfloat16, device="cpu", mult=1.0):
    """draw_qkv from a fresh generator seeded with `seed`, moved to `device`."""
    g = torch.Generator().manual_seed(seed)
    q, k, v = draw_qkv(g, q_shape, k_shape, dtype, mult)
    return q.to(device), k.to(device), v.to(device)


def upstream_grad(seed, like, device="cpu", blhd=False):
    """An upstream gradient dout for an output shaped like `like` (rank 3 or 4): i.i.d.
    N(0,1) in like's dtype from a fresh generator seeded with `seed`.  With blhd (rank 4),
    the draw is a [B,L,H,D] buffer viewed as [B,H,L,D] through a transpose, the layout of
    the long-sequence workload."""
    g = torch.Generator().manual_seed(seed)
    shape = tuple(like.shape)
    if blhd:
        B, H, L, D = shape
        return _randn(g, (B, L, H, D), like.dtype).to(device).transpose(1, 2)
    return _randn(g, shape, like.dtype).to(device)


def bernoulli_mask(seed, shape, p_keep, empty_rows_frac=0.0, device="cpu"):
    """Bool mask [..., Lq, Lk]: True (visible) with probability p_keep; then, per leading
    index, round(empty_rows_frac * Lq) query rows chosen by randperm are set all-False."""
    g = torch.Generator().manual_seed(seed)
    m = torch.rand(shape, generator=g) < p_keep
    n_empty = int(round(empty_rows_frac * shape[-2]))
    if n_empty:
        lead = m.reshape(-1, shape[-2], shape[-1])
        for b in range(lead.shape[0]):
            rows = torch.randperm(shape[-2], generator=g)[:n_empty]
            lead[b, rows, :] = False
    return m.to(device)


def config1(device="cpu"):
    """Rank-3 causal, fp32, [H=4, L=128, D=64], seed 1."""
    q, k, v = random_qkv(1, (4, 128, 64), dtype=torch.float32, device=device)
    return Workload("c1_rank3_fp32_causal_h4_l128_d64", q, k, v, None, True, 1 / math.sqrt(64),
                    "rank-3 causal fp32 [4,128,64]")


def config2(device="cpu"):
    """Rank-4 causal, bf16, [B=4, H=16, L=1024, D=64], contiguous, seed 2."""
    q, k, v = random_qkv(2, (4, 16, 1024, 64), device=device)
    return Workload("c2_rank4_bf16_causal_b4_h16_l1024_d64", q, k, v, None, True,
                    1 / math.sqrt(64), "rank-4 causal bf16 [4,16,1024,64]")


def config3(device="cpu", rank=3):
    """Flattened-batch causal, bf16: rank-4 [8,16,2048,128] drawn with seed 3; the rank-3
    input [128,2048,128] is a reshape of the same storage."""
    q, k, v = random_qkv(3, (8, 16, 2048, 128), device=device)
    if rank == 3:
        q, k, v = (t.reshape(128, 2048, 128) for t in (q, k, v))
    return Workload(f"c3_rank{rank}_bf16_causal_bh128_l2048_d128", q, k, v, None, True,
                    1 / math.sqrt(128), f"rank-{rank} causal bf16 B*H=128 L=2048 D=128")


def config4(device="cpu", D=128):
    """Long-sequence causal, bf16, [1,32,8192,128], entries N(0,1)*0.5, each tensor a
    [B,L,H,D] buffer viewed as [B,H,L,D] through a transpose (non-contiguous).  Another head
    dim D gives the same recipe at [1,32,8192,D] (scale 1/sqrt(D))."""
    g = torch.Generator().manual_seed(4)
    bufs = [_randn(g, (1, 8192, 32, D), torch.bfloat16, 0.5).to(device) for _ in range(3)]
    q, k, v = (b.transpose(1, 2) for b in bufs)
    return Workload(f"c4_rank4_bf16_causal_b1_h32_l8192_d{D}_strided", q, k, v, None, True,
                    1 / math.sqrt(D), f"rank-4 causal bf16 [1,32,8192,{D}], [B,L,H,D] strides")


def config5(device="cpu"):
    """Masked non-causal, bf16, [2,8,4096,64]; bool mask [2,1,4096,4096] with
    P(visible)=0.1 and 5 % of query rows (205 per batch entry) fully masked, expanded over
    heads with stride 0."""
    g = torch.Generator().manual_seed(5)
    q, k, v = draw_qkv(g, (2, 8, 4096, 64))
    m = torch.rand((2, 1, 4096, 4096), generator=g) < 0.1
    empty = []
    for b in range(2):
        rows = torch.randperm(4096, generator=g)[:205]
        m[b, 0, rows, :] = False
        empty.append(rows.sort().values)
    q, k, v, m = q.to(device), k.to(device), v.to(device), m.to(device)
    # the [2,1,L,L] mask is handed over as is: consumers broadcast it over the heads with
    # a zero head stride (moving an expanded view between devices would materialise it)
    return Workload("c5_rank4_bf16_boolmask_b2_h8_l4096_d64", q, k, v, m, False,
                    1 / math.sqrt(64),
                    "rank-4 bool-mask bf16 [2,8,4096,64], p_keep=0.1, 5% empty rows",
                    extra={"empty_rows": torch.stack(empty)})


def doc_lengths(seed, total, lo=128, hi=8192):
    """Document lengths for a packed batch: log-uniform integers in [lo, hi] drawn from a
    generator seeded with `seed` until they sum to `total` (the last one cut to fit)."""
    g = torch.Generator().manual_seed(seed)
    lengths, left = [], total
    while left > 0:
        u = torch.rand((), generator=g).item()
        n = int(round(math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))))
        n = min(max(n, 1), left)
        lengths.append(n)
        left -= n
    return lengths


def packed(seed, q_lengths, k_lengths, H, D, dtype=torch.bfloat16, device="cpu", mult=1.0):
    """Packed variable-length inputs: q [sum q_lengths, H, D], k and v [sum k_lengths, H, D]
    i.i.d. N(0, mult^2) drawn in the order q, k, v, and the int32 offsets cu_seqlens_q,
    cu_seqlens_k (nseq + 1 entries each)."""
    g = torch.Generator().manual_seed(seed)
    tq, tk = sum(q_lengths), sum(k_lengths)
    q, k, v = draw_qkv(g, (tq, H, D), (tk, H, D), dtype=dtype, mult=mult)
    cq = torch.tensor([0] + list(q_lengths), dtype=torch.int64).cumsum(0).to(torch.int32)
    ck = torch.tensor([0] + list(k_lengths), dtype=torch.int64).cumsum(0).to(torch.int32)
    return q.to(device), k.to(device), v.to(device), cq.to(device), ck.to(device)


def config_varlen(device="cpu"):
    """Packed documents, bf16, causal: H=32, D=128, 32768 tokens split into documents of
    log-uniform lengths in [128, 8192] (seed 6), queries and keys of the same documents."""
    lengths = doc_lengths(6, 32768)
    q, k, v, cq, ck = packed(6, lengths, lengths, 32, 128, device=device)
    return Workload("varlen_bf16_causal_h32_d128_t32768", q, k, v, None, True,
                    1 / math.sqrt(128), "packed documents, 32768 tokens, H=32, D=128, causal",
                    extra={"lengths": lengths, "cu_seqlens_q": cq, "cu_seqlens_k": ck})


CONFIGS = {
    "c1": config1,
    "c2": config2,
    "c3": config3,
    "c4": config4,
    "c5": config5,
}

