"""Seeded synthetic inputs for exact attention (shared by tests and bench).

This module holds no attention arithmetic: it only draws Q, K, V and dO,
and names the workload shapes.  Both the GPU path and the CPU oracle are
fed from it.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws
``torch.randn(B, H, N, d, float32)`` for Q, K, V and then dO, in that
order (dO is skipped for forward-only workloads); the values are cast to
the workload's dtype with round-to-nearest-even.  The oracle receives the
exact float64 up-cast of the same rounded values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str = "bf16"
    causal: bool = False
    dropout_p: float = 0.0
    backward: bool = False
    seed: int = 0
    dropout_seed: int = 0
    scale: float = field(default=None)  # None -> 1/sqrt(d)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    def flops_fwd(self) -> float:
        """4 B H N^2 d, halved when causal (exp and masking not counted)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def flops_bwd(self) -> float:
        """Five products of the forward's size (the recompute included)."""
        return 2.5 * self.flops_fwd()


def draw(w: Workload, with_dout: bool | None = None, seed: int | None = None):
    """(q, k, v, dout-or-None) on the CPU in the workload dtype, [B,H,N,d]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    q = torch.randn(shape, dtype=torch.float32, generator=g)
    k = torch.randn(shape, dtype=torch.float32, generator=g)
    v = torch.randn(shape, dtype=torch.float32, generator=g)
    if with_dout is None:
        with_dout = w.backward
    do = torch.randn(shape, dtype=torch.float32, generator=g) if with_dout else None
    cast = lambda t: None if t is None else t.to(w.torch_dtype)
    return cast(q), cast(k), cast(v), cast(do)


def draw_cross(w: Workload, Nk: int, with_dout: bool = False):
    """q [B,H,N,d] and k, v [B,H,Nk,d] (and dO [B,H,N,d]) for attention over
    Nk keys: N(0,1) draws in the order q, k, v, dO from a CPU generator
    seeded with ``w.seed``, cast to the workload's type with
    round-to-nearest-even."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    q = torch.randn((w.B, w.H, w.N, w.d), dtype=torch.float32, generator=g)
    k = torch.randn((w.B, w.H, Nk, w.d), dtype=torch.float32, generator=g)
    v = torch.randn((w.B, w.H, Nk, w.d), dtype=torch.float32, generator=g)
    out = [q.to(w.torch_dtype), k.to(w.torch_dtype), v.to(w.torch_dtype)]
    if with_dout:
        out.append(torch.randn((w.B, w.H, w.N, w.d), dtype=torch.float32, generator=g)
                   .to(w.torch_dtype))
    return tuple(out)


E4M3_MAX = 448.0   # largest finite OCP e4m3 value


def quantize_e4m3(x: torch.Tensor):
    """Per-(b, h) e4m3 quantization of an fp32 [B,H,N,d] draw: descale =
    max|x| / 448 over the head (float32), x8 = RNE(x / descale) in e4m3.
    Returns (x8 torch.float8_e4m3fn, descale float32 [B,H]); the attention
    inputs are x8 * descale."""
    amax = x.abs().amax(dim=(2, 3)).to(torch.float32)
    descale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    x8 = (x / descale[:, :, None, None]).to(torch.float8_e4m3fn)
    return x8, descale


def draw_fp8(w: Workload, Nk: int | None = None):
    """q8, k8, v8 (torch.float8_e4m3fn) and their float32 [B,H] descale
    factors: N(0,1) draws in the order q, k, v from a CPU generator seeded
    with ``w.seed`` (k and v with Nk rows when given), each head quantized
    with quantize_e4m3."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    nk = w.N if Nk is None else Nk
    q = torch.randn((w.B, w.H, w.N, w.d), dtype=torch.float32, generator=g)
    k = torch.randn((w.B, w.H, nk, w.d), dtype=torch.float32, generator=g)
    v = torch.randn((w.B, w.H, nk, w.d), dtype=torch.float32, generator=g)
    (q8, dq), (k8, dk), (v8, dv) = quantize_e4m3(q), quantize_e4m3(k), quantize_e4m3(v)
    return q8, k8, v8, dq, dk, dv


def dequantize(x8: torch.Tensor, descale: torch.Tensor) -> torch.Tensor:
    """float64 values of an e4m3 tensor times its per-(b, h) descale (exact:
    a 4-bit significand times a 24-bit one fits in float64)."""
    return x8.to(torch.float64) * descale.to(torch.float64)[:, :, None, None]


DROPOUT_SEED = 0x5EED000000000005

# The five workloads the targets are stated on (shapes, dtypes, modes).
WORKLOADS = {
    "single_head_f32": Workload("single_head_f32", 1, 1, 128, 64, "f32", causal=False,
                                backward=True, seed=1),
    "small_fwd_bf16": Workload("small_fwd_bf16", 2, 8, 1024, 64, "bf16", causal=False,
                               seed=2),
    "small_fwd_bf16_causal": Workload("small_fwd_bf16_causal", 2, 8, 1024, 64, "bf16",
                                      causal=True, seed=2),
    "mid_fwdbwd_causal": Workload("mid_fwdbwd_causal", 8, 16, 2048, 128, "bf16",
                                  causal=True, backward=True, seed=3),
    "long_causal_4k": Workload("long_causal_4k", 1, 32, 4096, 128, "bf16", causal=True,
                               seed=4),
    "long_causal_16k": Workload("long_causal_16k", 1, 32, 16384, 128, "bf16", causal=True,
                                seed=4),
    "long_causal_64k": Workload("long_causal_64k", 1, 32, 65536, 128, "bf16", causal=True,
                                seed=4),
    "train_dropout": Workload("train_dropout", 4, 32, 4096, 128, "bf16", causal=True,
                              dropout_p=0.1, backward=True, seed=5,
                              dropout_seed=DROPOUT_SEED),
}

# The training shape at the other supported head dimensions (measured beside
# the five; same inputs recipe, seed 5).
for _d in (32, 64, 96, 256):
    WORKLOADS["train_d%d" % _d] = Workload("train_d%d" % _d, 4, 32, 4096, _d, "bf16", causal=True,
                                           dropout_p=0.1, backward=True, seed=5,
                                           dropout_seed=DROPOUT_SEED)


def score_matrix_bytes(N: int, heads: int = 1, elem_bytes: int = 2) -> int:
    """HBM bytes of the N x N score (or probability) matrices that standard
    attention materialises, for ``heads`` heads."""
    return N * N * elem_bytes * heads


def fwd_output_bytes(w: Workload, out_bytes: int | None = None) -> int:
    """Bytes the fused forward writes: O [B,H,N,d] plus LSE [B,H,N] fp32."""
    ob = out_bytes if out_bytes is not None else torch.empty((), dtype=w.torch_dtype).element_size()
    return w.B * w.H * w.N * w.d * ob + w.B * w.H * w.N * 4
