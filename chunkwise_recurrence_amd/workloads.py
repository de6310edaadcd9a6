"""Seeded synthetic inputs for the five workloads (and for ad-hoc test cases).

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the HIP path's tests and the CPU oracle can take
their inputs from it.  Every tensor is drawn on the CPU with a
`torch.Generator`, so the same seed gives the same values on any machine.

Workloads (the pages' demos draw i.i.d. Gaussian q, k, v; CS336 lecture 4
code 1 `demo_two_forms` draws q, k, v = randn(300, 16) three times after
seeding 0 and splits the sequence into chunks of 64):

  small_fp32   B=1 H=1  L=300   d=16  fp32, no feature map, no decay, C=64
  elu_bf16     B=4 H=16 L=4096  d=64  bf16, phi = elu+1, no decay, C=64
  retnet_bf16  B=2 H=32 L=16384 d=128 bf16, q,k,v / sqrt(128), gamma_h =
               linspace(0.9, 0.999, 32), C=64
  gated_bf16   B=1 H=16 L=65536 d=128 bf16, q,k,v / sqrt(128), g ~ N(0,1)
               per token per head, a_t = exp(-softplus(g_t)), C=64
  decode_bf16  N=256 H=32 d=128, fp32 state ~ 0.01 N(0,1), bf16 q,k,v /
               sqrt(128) per step, 1000 steps
  delta_bf16   the delta rule (Gated DeltaNet) on the retnet_bf16 shapes:
               q, v / sqrt(128); keys uniform on the unit sphere (a Gaussian
               row divided by its length -- the pages normalise keys before the
               delta rule); beta ~ U(0, 1) per token and head; the gated
               workload's gate g ~ N(0,1); C = 64 (the pages print no workload
               for it)
  gla_bf16     the retnet_bf16 shapes with a per-channel gate (GLA's
               diagonal decay): log a[b,h,t,d] = -Exp(mean 0.8), i.i.d. per
               token, head and key channel (the pages print no workload for
               this variant; 0.8 is close to the mean of softplus(N(0,1)),
               the gated workload's per-token decay)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

PHI_IDENTITY = 0
PHI_ELU1 = 1
DECAY_NONE = 0
DECAY_HEAD = 1
DECAY_LOG = 2
DECAY_GATE = 3
DECAY_CHANNEL = 4


@dataclass
class ChunkWorkload:
    name: str
    B: int
    H: int
    L: int
    dk: int
    dv: int
    C: int
    dtype: torch.dtype
    phi: int
    decay_kind: int
    seed: int
    scale: float = 1.0
    gate_shift: float = 0.0
    channel_mean: float = 0.8
    note: str = ""


@dataclass
class DecodeWorkload:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    steps: int
    dtype: torch.dtype
    seed: int
    state_std: float = 0.01
    scale: float = 1.0 / math.sqrt(128.0)
    phi: int = PHI_IDENTITY
    decay_kind: int = DECAY_NONE
    note: str = ""


WORKLOADS = {
    "small_fp32": ChunkWorkload("small_fp32", 1, 1, 300, 16, 16, 64, torch.float32, PHI_IDENTITY,
                                DECAY_NONE, seed=0,
                                note="chunks of 64,64,64,64,44; q,k,v drawn as in demo_two_forms"),
    "elu_bf16": ChunkWorkload("elu_bf16", 4, 16, 4096, 64, 64, 64, torch.bfloat16, PHI_ELU1,
                              DECAY_NONE, seed=2),
    "retnet_bf16": ChunkWorkload("retnet_bf16", 2, 32, 16384, 128, 128, 64, torch.bfloat16,
                                 PHI_IDENTITY, DECAY_HEAD, seed=3, scale=1.0 / math.sqrt(128.0)),
    "gated_bf16": ChunkWorkload("gated_bf16", 1, 16, 65536, 128, 128, 64, torch.bfloat16,
                                PHI_IDENTITY, DECAY_GATE, seed=4, scale=1.0 / math.sqrt(128.0)),
    "gla_bf16": ChunkWorkload("gla_bf16", 2, 32, 16384, 128, 128, 64, torch.bfloat16,
                              PHI_IDENTITY, DECAY_CHANNEL, seed=6, scale=1.0 / math.sqrt(128.0),
                              channel_mean=0.8),
}

DELTA = ChunkWorkload("delta_bf16", 2, 32, 16384, 128, 128, 64, torch.bfloat16, PHI_IDENTITY,
                      DECAY_GATE, seed=7, scale=1.0 / math.sqrt(128.0))

DECODE = DecodeWorkload("decode_bf16", 256, 32, 128, 128, 1000, torch.bfloat16, seed=5)


def retnet_gammas(H: int) -> torch.Tensor:
    """Per-head decay constants, evenly spaced in [0.9, 0.999] (fp32)."""
    return torch.linspace(0.9, 0.999, H, dtype=torch.float64).to(torch.float32)


def chunk_inputs(w: ChunkWorkload, heads: slice | None = None):
    """Draw (q, k, v, decay) for workload `w` on the CPU.

    Draw order: q, k, v, then the gate g (gated workload only), each as one
    fp32 `randn` over the full [B,H,L,d] shape, multiplied by `scale` in fp32
    and rounded to the workload dtype (round-to-nearest-even); the
    per-channel log decay is one fp32 `exponential_` draw over [B,H,L,dk].
    `heads` (a slice over the flattened B*H axis) trims what is returned but
    not what is drawn, so a subset is bit-identical to the full tensors.
    """
    g = torch.Generator().manual_seed(w.seed)
    shp_k = (w.B, w.H, w.L, w.dk)
    shp_v = (w.B, w.H, w.L, w.dv)

    def draw(shape):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if w.scale != 1.0:
            x = x * torch.tensor(w.scale, dtype=torch.float32)
        return x.to(w.dtype)

    q = draw(shp_k)
    k = draw(shp_k)
    v = draw(shp_v)
    if w.decay_kind == DECAY_HEAD:
        decay = retnet_gammas(w.H)
    elif w.decay_kind in (DECAY_GATE, DECAY_LOG):
        decay = torch.randn((w.B, w.H, w.L), generator=g, dtype=torch.float32)
        if w.gate_shift:
            decay = decay + torch.tensor(w.gate_shift, dtype=torch.float32)
    elif w.decay_kind == DECAY_CHANNEL:
        decay = -torch.empty(shp_k, dtype=torch.float32).exponential_(1.0 / w.channel_mean,
                                                                      generator=g)
    else:
        decay = None
    if heads is not None:
        def sel(x):
            return x.reshape(w.B * w.H, *x.shape[2:])[heads].contiguous()
        q, k, v = sel(q), sel(k), sel(v)
        if decay is not None and decay.dim() >= 3:
            decay = sel(decay)
    return q, k, v, decay


def unit_rows(x: torch.Tensor) -> torch.Tensor:
    """Rows of a Gaussian draw scaled to length 1 (uniform on the unit sphere)."""
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def delta_inputs(w: ChunkWorkload = DELTA, heads: slice | None = None):
    """Draw (q, k, v, beta, decay) for a delta-rule workload on the CPU.

    Draw order: q, k, v as one fp32 `randn` each over [B,H,L,d] (q and v
    times `scale`; k rows scaled to unit length in fp32), then beta as one
    fp32 `rand` over [B,H,L], then the gate g (gate kinds) as one `randn`;
    q, k, v are rounded to the workload dtype.
    """
    g = torch.Generator().manual_seed(w.seed)
    shp_k = (w.B, w.H, w.L, w.dk)
    sc = torch.tensor(w.scale, dtype=torch.float32)
    q = (torch.randn(shp_k, generator=g) * sc).to(w.dtype)
    k = unit_rows(torch.randn(shp_k, generator=g)).to(w.dtype)
    v = (torch.randn((w.B, w.H, w.L, w.dv), generator=g) * sc).to(w.dtype)
    beta = torch.rand((w.B, w.H, w.L), generator=g)
    if w.decay_kind in (DECAY_GATE, DECAY_LOG):
        decay = torch.randn((w.B, w.H, w.L), generator=g)
    elif w.decay_kind == DECAY_HEAD:
        decay = retnet_gammas(w.H)
    else:
        decay = None
    if heads is not None:
        def sel(x):
            return x.reshape(w.B * w.H, *x.shape[2:])[heads].contiguous()
        q, k, v, beta = sel(q), sel(k), sel(v), sel(beta)
        if decay is not None and decay.dim() >= 3:
            decay = sel(decay)
    return q, k, v, beta, decay


def random_delta_inputs(c: "RandomCase"):
    """random_inputs with unit-length keys and beta ~ U(0.05, 1) drawn after them."""
    q, k, v, decay, state = random_inputs(c)
    g = torch.Generator().manual_seed(c.seed + 1)
    k = unit_rows(k.float()).to(c.dtype)
    beta = 0.05 + 0.95 * torch.rand((c.B, c.H, c.L), generator=g)
    return q, k, v, beta, decay, state


def small_fp32_inputs():
    """The 300 x 16 fp32 demo: global seed 0, then q, k, v = randn(300, 16) in that order."""
    g = torch.Generator().manual_seed(0)
    q = torch.randn(300, 16, generator=g)
    k = torch.randn(300, 16, generator=g)
    v = torch.randn(300, 16, generator=g)
    return q[None, None], k[None, None], v[None, None]


class DecodeStream:
    """Seeded inputs of the decode workload: S_0 first, then q, k, v per step."""

    def __init__(self, w: DecodeWorkload = DECODE, N: int | None = None):
        self.w = w
        self.N = w.N if N is None else N
        self.g = torch.Generator().manual_seed(w.seed)

    def initial_state(self) -> torch.Tensor:
        w = self.w
        s = torch.randn((self.N, w.H, w.dk, w.dv), generator=self.g, dtype=torch.float32)
        return s * torch.tensor(w.state_std, dtype=torch.float32)

    def step(self):
        w = self.w
        sc = torch.tensor(w.scale, dtype=torch.float32)
        q = (torch.randn((self.N, w.H, w.dk), generator=self.g) * sc).to(w.dtype)
        k = (torch.randn((self.N, w.H, w.dk), generator=self.g) * sc).to(w.dtype)
        v = (torch.randn((self.N, w.H, w.dv), generator=self.g) * sc).to(w.dtype)
        return q, k, v


@dataclass
class RandomCase:
    B: int
    H: int
    L: int
    dk: int
    dv: int
    dtype: torch.dtype = torch.float32
    phi: int = PHI_IDENTITY
    decay_kind: int = DECAY_NONE
    seed: int = 0
    scale: float = 1.0
    gate_shift: float = 0.0
    channel_mean: float = 0.5
    with_state: bool = False
    extra: dict = field(default_factory=dict)


def random_inputs(c: RandomCase):
    """Seeded q, k, v, decay data and (optionally) an initial state for a test case.

    Decay data: gamma[H] in [0.8, 1.0] for per-head decay, g ~ N(0,1) + shift
    for the gate, log a = -|N(0, 0.1)| for the log-decay kind, log a[b,h,t,d]
    = -Exp(mean channel_mean) for the per-channel kind.
    """
    g = torch.Generator().manual_seed(c.seed)
    sc = torch.tensor(c.scale, dtype=torch.float32)
    q = (torch.randn((c.B, c.H, c.L, c.dk), generator=g) * sc).to(c.dtype)
    k = (torch.randn((c.B, c.H, c.L, c.dk), generator=g) * sc).to(c.dtype)
    v = (torch.randn((c.B, c.H, c.L, c.dv), generator=g) * sc).to(c.dtype)
    if c.decay_kind == DECAY_HEAD:
        decay = 0.8 + 0.2 * torch.rand((c.H,), generator=g)
    elif c.decay_kind == DECAY_GATE:
        decay = torch.randn((c.B, c.H, c.L), generator=g) + c.gate_shift
    elif c.decay_kind == DECAY_LOG:
        decay = -(0.1 * torch.randn((c.B, c.H, c.L), generator=g)).abs()
    elif c.decay_kind == DECAY_CHANNEL:
        decay = -torch.empty((c.B, c.H, c.L, c.dk)).exponential_(1.0 / c.channel_mean, generator=g)
    else:
        decay = None
    state = None
    if c.with_state:
        state = torch.randn((c.B, c.H, c.dk, c.dv), generator=g) * 0.1
    return q, k, v, decay, state
