"""Seeded synthetic inputs for the data-parallel sync path.

This module is shared by the GPU path's tests/bench and by the oracle's
tests. It holds no arithmetic of the synchronisation method itself: it only
turns (seed, tensor id, rank, element index) into numbers.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), with the output finaliser of Vigna's
public-domain splitmix64.c. It is used counter-based: element i of stream
(seed, tensor, rank) is the finaliser applied to key + (i + 1) * GAMMA,
where key is itself a SplitMix64 output of the stream identifiers. Every
output therefore depends only on its coordinates, so any sub-range can be
generated on its own, on the host or on the GPU, with identical bits.

Distributions:
  uniform_pm1  top 24 bits u of the output, x = (u - 2^23) * 2^-23, which lies
               in [-1, 1 - 2^-23] and is exactly representable in fp32.
  normal       Box-Muller in fp64 from two 53-bit uniforms drawn at counters
               2i and 2i+1, then scaled and rounded to fp32.
  int copy     round-half-even(1000 * x) of the uniform above, in [-1000, 1000].

All integer arithmetic is done in torch int64 with wrap-around multiplication
(two's complement), and logical right shifts are emulated with masks.
"""
from __future__ import annotations

import math

import torch

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1


def _s64(v: int) -> int:
    """Reinterpret an unsigned 64-bit constant as a signed int64."""
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


_GAMMA_S = _s64(GAMMA)
_MIX1_S = _s64(MIX1)
_MIX2_S = _s64(MIX2)


def _srl(z: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 lanes."""
    return (z >> k) & ((1 << (64 - k)) - 1)


def _finalise(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _srl(z, 30)) * _MIX1_S
    z = (z ^ _srl(z, 27)) * _MIX2_S
    return z ^ _srl(z, 31)


def _finalise_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def splitmix64_sequence(seed: int, count: int) -> list[int]:
    """The plain sequential generator: state += GAMMA, output finalise(state).

    Pinned in the tests against the published reference outputs.
    """
    out, s = [], seed & MASK64
    for _ in range(count):
        s = (s + GAMMA) & MASK64
        out.append(_finalise_int(s))
    return out


def stream_key(seed: int, tensor: int, rank: int) -> int:
    """64-bit key of stream (seed, tensor id, rank), as an unsigned int."""
    k = _finalise_int(seed * GAMMA + 1)
    k = _finalise_int(k ^ ((tensor + 1) * MIX1))
    k = _finalise_int(k ^ ((rank + 1) * MIX2))
    return k


def raw_u64(seed: int, tensor: int, rank: int, start: int, count: int,
            device="cpu") -> torch.Tensor:
    """Outputs at counters start .. start+count-1, as int64 bit patterns."""
    key = _s64(stream_key(seed, tensor, rank))
    i = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    return _finalise(i * _GAMMA_S + key)


def uniform_pm1(seed, tensor, rank, count, start=0, device="cpu") -> torch.Tensor:
    """fp32 values (u - 2^23) * 2^-23 with u the top 24 bits: [-1, 1 - 2^-23]."""
    u = _srl(raw_u64(seed, tensor, rank, start, count, device), 40)
    return (u - (1 << 23)).to(torch.float32) * (2.0 ** -23)


def int_copy(x: torch.Tensor) -> torch.Tensor:
    """round-half-even(1000 * x) as int32 (x in [-1, 1] gives [-1000, 1000])."""
    return torch.round(x.to(torch.float64) * 1000.0).to(torch.int32)


def normal(seed, tensor, rank, count, std=1.0, mean=0.0, start=0,
           device="cpu") -> torch.Tensor:
    """fp32 N(mean, std^2) by Box-Muller in fp64 (one draw per pair of counters)."""
    z = raw_u64(seed, tensor, rank, 2 * start, 2 * count, device).view(count, 2)
    scale = 2.0 ** -53
    u1 = (_srl(z[:, 0], 11) + 1).to(torch.float64) * scale   # (0, 1]
    u2 = _srl(z[:, 1], 11).to(torch.float64) * scale         # [0, 1)
    g = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)
    return (g * std + mean).to(torch.float32)


# --------------------------------------------------------------------------
# Workload recipes. Tensor ids are fixed per workload so every consumer draws
# the same values.
# --------------------------------------------------------------------------

def ring_uniform_inputs(seed: int, k: int, n: int, device="cpu") -> list[torch.Tensor]:
    """K per-rank fp32 gradients, uniform in [-1, 1), tensor id 0."""
    return [uniform_pm1(seed, 0, r, n, device=device) for r in range(k)]


def token_counts(seed: int, k: int, docs_per_rank: int = 2, mu: float = 7.0,
                 sigma: float = 1.0) -> list[int]:
    """Per-rank token counts: sum over docs of max(1, rne(exp(mu + sigma*Z)))."""
    out = []
    for r in range(k):
        z = normal(seed, 9, r, docs_per_rank).to(torch.float64)
        lens = torch.clamp(torch.round(torch.exp(mu + sigma * z)), min=1.0)
        out.append(int(lens.sum().item()))
    return out


def bf16_normal(seed, tensor, rank, count, std, start=0, device="cpu") -> torch.Tensor:
    """bf16 gradient values: fp32 N(0, std^2) rounded to nearest-even bf16."""
    return normal(seed, tensor, rank, count, std=std, start=start,
                  device=device).to(torch.bfloat16)


# One transformer layer of a GQA + SwiGLU model, hidden 4096 (q/o 4096x4096,
# k/v 4096x1024, gate/up/down 4096x14336), flattened in reverse registration
# order the way DDP assigns gradients to buckets.
LAYER_MATRICES = [
    ("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
    ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096),
]
LAYER_PARAMS = sum(a * b for _, a, b in LAYER_MATRICES)   # 218,103,808
BUCKET_ELEMS = 25_000_000


def layer_grads_bf16(seed: int, k: int, device="cpu", total: int = LAYER_PARAMS,
                     std: float = 1e-3) -> list[torch.Tensor]:
    """K flat bf16 gradient vectors of one layer, N(0, std^2), tensor id 3."""
    return [bf16_normal(seed, 3, r, total, std, device=device) for r in range(k)]


def fsdp_fixture(seed: int = 2, k: int = 8, m: int = 1024, d: int = 512, f: int = 512,
                 device="cpu") -> dict:
    """Global x[m,d] ~ N(0,1), w[d,f] ~ N(0,0.02^2), dy[m,f] ~ N(0,1), fp32."""
    x = normal(seed, 20, 0, m * d, device=device).view(m, d)
    w = normal(seed, 21, 0, d * f, std=0.02, device=device).view(d, f)
    dy = normal(seed, 22, 0, m * f, device=device).view(m, f)
    return {"x": x, "w": w, "dy": dy}


def gemm_bf16_inputs(seed: int, m: int, n: int, kk: int, device="cpu", b_layout: str = "kn"):
    """A[m,kk] and B, bf16 from N(0,1): B[kk,n] for C = A B (b_layout "kn"), or
    B[n,kk] for C = A B^T ("nk", the k-contiguous weight layout). The same
    draws fill B in both layouts: element (k, j) of the product's B is draw
    j*kk + k, so the "kn" tensor is the transpose of the "nk" one."""
    a = bf16_normal(seed, 30, 0, m * kk, 1.0, device=device).view(m, kk)
    b = bf16_normal(seed, 31, 0, n * kk, 1.0, device=device).view(n, kk)
    if b_layout == "kn":
        b = b.t().contiguous()
    elif b_layout != "nk":
        raise ValueError("b_layout must be 'kn' or 'nk'")
    return a, b


# Variable-length minibatch of an SFT step: each rank's documents are packed
# into microbatches of at most MICROBATCH_TOKENS tokens, so ranks run uneven
# microbatch counts.
MICROBATCH_TOKENS = 2048


def microbatch_counts(seed: int, k: int, tokens_per_microbatch: int = MICROBATCH_TOKENS,
                      docs_per_rank: int = 2) -> list[int]:
    """Per-rank microbatch counts max(1, ceil(t_r / tokens_per_microbatch)) for
    the token counts of token_counts(seed, k, docs_per_rank)."""
    t = token_counts(seed, k, docs_per_rank)
    return [max(1, -(-x // tokens_per_microbatch)) for x in t]


def microbatch_grad(seed: int, rank: int, m: int, n: int, dtype=torch.bfloat16,
                    std: float = 1e-3, device="cpu") -> torch.Tensor:
    """Rank `rank`'s gradient from its m-th microbatch: N(0, std^2) in fp32,
    rounded to nearest-even `dtype` (tensor id 40 + m)."""
    return normal(seed, 40 + m, rank, n, std=std, device=device).to(dtype)


def layer_backward_pieces() -> list[tuple[int, int, int]]:
    """(offset, m, n) of the layer's weight gradients in the flat per-rank
    vector, in backward order (down, up, gate, o, v, k, q: the reverse of
    registration order, as DDP assigns buckets)."""
    out, off = [], 0
    for _, a, b in reversed(LAYER_MATRICES):
        out.append((off, a, b))
        off += a * b
    return out


def backward_operands(seed: int, k: int, pieces, t: int, device="cpu", dy_std: float = 1e-3):
    """Per (piece g, rank r), index g*k + r: dy [m, t] ~ N(0, dy_std^2) and
    x [n, t] ~ N(0, 1), bf16, token-contiguous (tensor ids 70 + g and 90 + g)."""
    dy, x = [], []
    for g, (_, m, n) in enumerate(pieces):
        for r in range(k):
            dy.append(bf16_normal(seed, 70 + g, r, m * t, dy_std, device=device).view(m, t))
            x.append(bf16_normal(seed, 90 + g, r, n * t, 1.0, device=device).view(n, t))
    return dy, x
