"""Seeded synthetic inputs for the mixed-head SAF attention layer.

This module is shared by the GPU tests, the benchmark and the oracle checks.  It only draws random
tensors of the shapes and distributions of the workloads; it holds none of the method's arithmetic.

The workloads are the layer shapes the pages report timings for, with synthetic tensors in place of
trained activations (no dataset or checkpoint is used):
  - a 124M-parameter decoder layer: 12 heads of width 64, at 4K and 8K context
    ([Notes §三]; [Paper page] Table 2),
  - one GPU's share of the 1B run at 8K context ([Notes §四.6]; [Paper page] Table 23),
  - causal prefill at batch 64 and at 16K context ([Paper page] Table 29), and at batch 1, where
    the pages see launch overhead dominate ([Notes §四], Appendix D.3),
  - a grouped-query prefill shaped like Qwen3-4B (32 query heads sharing 8 key/value heads of width
    128; [Notes §二.4] and [Paper page] Table 26 run SAF on that model's GQA layers),
plus a tiny fp32 case for exact parity.  Q, K, V and dO are N(0, 1); the replaced heads' a and r are
random preferences in the same position/distance parametrisation as the pages' "structured random"
control ([Notes §二.2]).  Citation keys as in the oracle package.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

SEED0 = 1337  # the pages' first seed ([Notes §三])


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    d: int
    dtype: str            # "f32" or "bf16"
    n_replaced: int
    ar_std: float         # standard deviation of a and r
    backward: bool        # fwd+bwd (True) or forward only
    index: int            # seed offset
    calib_N: int = 0      # > 0: also a calibration over calib_N sequences
    note: str = ""
    Hkv: int = 0          # key/value heads (grouped-query attention); 0 = H

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def kv_heads(self):
        return self.Hkv or self.H

    def replaced(self, placement: str = "interleaved"):
        return replaced_mask(self.H, self.n_replaced, placement)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fwd_f32", 1, 4, 256, 64, "f32", 1, 1.0, False, 0,
                 note="tiny forward, head 3 replaced, fp32"),
        Workload("l124m_t4096", 8, 12, 4096, 64, "bf16", 3, 0.5, True, 1,
                 note="124M-shaped layer at 4K, 25% of heads replaced, fwd+bwd"),
        Workload("l124m_t8192", 4, 12, 8192, 64, "bf16", 6, 0.5, True, 2,
                 note="124M-shaped layer at 8K, 50% of heads replaced, fwd+bwd"),
        Workload("l1b_t8192", 2, 16, 8192, 128, "bf16", 4, 0.5, True, 3, calib_N=32,
                 note="1B-shaped one-GPU share at 8K, 25% replaced, fwd+bwd; calibration N=32"),
        Workload("prefill_b64_t4096", 64, 12, 4096, 64, "bf16", 3, 0.5, False, 4,
                 note="causal prefill, batch 64 at 4K, 25% replaced, forward only"),
        Workload("prefill_b2_t16384", 2, 12, 16384, 64, "bf16", 3, 0.5, False, 5,
                 note="causal prefill, batch 2 at 16K, 25% replaced, forward only"),
        Workload("prefill_b1_t4096", 1, 12, 4096, 64, "bf16", 3, 0.5, False, 6,
                 note="causal prefill, batch 1 at 4K (launch-bound), 25% replaced, forward only"),
        Workload("qwen4b_gqa_t4096", 1, 32, 4096, 128, "bf16", 8, 0.5, False, 7, Hkv=8,
                 note="grouped-query prefill, 32 query heads over 8 key/value heads, 25% replaced"),
    ]
}


def replaced_mask(H: int, R: int, placement: str = "interleaved"):
    """Which heads are replaced: a list of H ints (1 = fixed pattern).

    interleaved: head h is replaced iff h mod (H/R) == H/R - 1 (R divides H), e.g. {3} of 4,
    {3, 7, 11} of 12; contiguous: the last R heads.  The pages pick heads by variance across the
    whole model ([Notes §二.1]); a synthetic layer has no such ranking, so the placement is fixed."""
    if R == 0:
        return [0] * H
    if placement == "interleaved":
        if H % R:
            raise ValueError("interleaved placement needs R to divide H")
        g = H // R
        return [1 if h % g == g - 1 else 0 for h in range(H)]
    if placement == "contiguous":
        return [1 if h >= H - R else 0 for h in range(H)]
    if placement == "all":
        return [1] * H
    raise ValueError(placement)


@dataclass
class LayerInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    dout: torch.Tensor | None
    a: torch.Tensor
    r: torch.Tensor
    replaced: list = field(default_factory=list)


def layer_inputs(B, H, T, d, dtype, replaced, ar_std=0.5, seed=SEED0, backward=True,
                 pat_len=None, device="cpu", Hkv=None, draw_on=None):
    """Draw Q, K, V, dO ~ N(0,1) (Q, dO [B,H,T,d]; K, V [B,Hkv,T,d], Hkv = H unless given; then
    cast to dtype) and a, r ~ N(0, ar_std^2) ([H, pat_len] fp32), in that order, from a CPU
    generator seeded with `seed` (the values the oracle checks see).  draw_on="cuda" draws them
    with a generator on the GPU instead: the same distributions, other values, and no host work
    (for timing runs of large shapes)."""
    gdev = "cpu" if draw_on is None else draw_on
    g = torch.Generator(device=gdev).manual_seed(seed)
    P = T if pat_len is None else pat_len
    shape = (B, H, T, d)
    kvshape = (B, H if Hkv is None else Hkv, T, d)
    q = torch.randn(shape, generator=g, device=gdev).to(dtype)
    k = torch.randn(kvshape, generator=g, device=gdev).to(dtype)
    v = torch.randn(kvshape, generator=g, device=gdev).to(dtype)
    dout = torch.randn(shape, generator=g, device=gdev).to(dtype) if backward else None
    a = torch.randn((H, P), generator=g, device=gdev) * ar_std
    r = torch.randn((H, P), generator=g, device=gdev) * ar_std
    out = LayerInputs(q, k, v, dout, a.float(), r.float(), list(replaced))
    if device != "cpu":
        for name in ("q", "k", "v", "dout", "a", "r"):
            t = getattr(out, name)
            if t is not None:
                setattr(out, name, t.to(device))
    return out


def score_range_inputs(T, d, dtype, trend, seed=SEED0 + 300, device="cpu"):
    """One batch entry, two heads (head 0 ordinary, head 1 replaced) whose ordinary scores span a
    wide range with a set shape along the keys.  Every query is 8u plus small noise and key j is
    c_j u plus small noise, for one random unit vector u, so that with the 1/sqrt(d) scale of
    d = 64 the score of key j is about c_j:
      rising:  c_j = 150 j / (T-1)   (the row maximum moves with almost every 32 keys)
      falling: c_j = 150 (T-1-j) / (T-1)   (the first key dominates every row)
      spiky:   c_j = 120 at j = 5, 42, 79, ... (j % 37 == 5), else 0   (isolated jumps of about
               173 in log2 units, past the fp32 exponent range)
    V, dO ~ N(0, 1); a, r ~ N(0, 0.25)."""
    g = torch.Generator().manual_seed(seed)
    u = torch.randn(d, generator=g, dtype=torch.float64)
    u /= u.norm()
    j = torch.arange(T, dtype=torch.float64)
    if trend == "rising":
        c = 150.0 * j / max(T - 1, 1)
    elif trend == "falling":
        c = 150.0 * (T - 1 - j) / max(T - 1, 1)
    elif trend == "spiky":
        c = torch.where(j % 37 == 5, torch.full_like(j, 120.0), torch.zeros_like(j))
    else:
        raise ValueError(trend)
    shape = (1, 2, T, d)
    q = 8.0 * u.expand(shape).clone() + 0.05 * torch.randn(shape, generator=g, dtype=torch.float64)
    k = c[None, None, :, None] * u + 0.05 * torch.randn(shape, generator=g, dtype=torch.float64)
    v = torch.randn(shape, generator=g)
    dout = torch.randn(shape, generator=g)
    a = torch.randn((2, T), generator=g) * 0.5
    r = torch.randn((2, T), generator=g) * 0.5
    out = LayerInputs(q.to(dtype), k.to(dtype), v.to(dtype), dout.to(dtype), a.float(), r.float(),
                      [False, True])
    if device != "cpu":
        for name in ("q", "k", "v", "dout", "a", "r"):
            setattr(out, name, getattr(out, name).to(device))
    return out


def workload_inputs(w: Workload, placement="interleaved", device="cpu"):
    return layer_inputs(w.B, w.H, w.T, w.d, w.torch_dtype, w.replaced(placement), w.ar_std,
                        SEED0 + w.index, w.backward, device=device, Hkv=w.Hkv or None)


def calib_inputs(N, H, T, d, dtype, seed=SEED0 + 100, device="cpu"):
    """Queries and keys of N synthetic calibration sequences, [N, H, T, d], N(0,1)."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((N, H, T, d), generator=g).to(dtype)
    k = torch.randn((N, H, T, d), generator=g).to(dtype)
    return q.to(device), k.to(device)
