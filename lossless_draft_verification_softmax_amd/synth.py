"""Seeded synthetic inputs shaped like the AngelSpec pages' workloads.

This module only draws random inputs (logits, draft tokens, confidences,
temperatures); it holds none of the verification or budget arithmetic.  Both
the HIP path and the CPU oracle are fed from it.

Workloads (the pages report MTP depth 3, block drafting, concurrency 4-64 and
Qwen3/Hy3-class vocabularies; the token distributions of their benchmarks are
not given, so Gaussian logits stand in for them):

  c1  tiny exhaustive: B=2, D=3, V=32, fp32; P ~ N(0, 2^2), Q = P + N(0, 1).
  c2  MTP chat: B=16, D=3, V=128000, bf16; P ~ N(0, 3^2), 1% of target rows
      get +8 on one uniform token (before draft noise, so the draft inherits
      it); Q_k = P_k + N(0, s_k^2), s = 0.5, 1.0, 1.5.  T = 1.
  c3  block: B=32, D=16, V=151936, bf16; P ~ N(0, 3^2),
      Q_i = P_i + N(0, (0.3 + 0.1 i)^2).  T = 0 or 1.
  c4  budget: as c3 with B=64; confidences Beta(8, 2) for requests 0-31
      (code-like), Beta(3, 3) for 32-63 (chat-like); top-K with K=256.  T = 1.
  c4full  the same 64 x 16 x 151936 bf16 batch with K = 1024 (every position).
  c5  mixed T: B=64, D=16, V=262144, fp32; P ~ N(0, 4^2), Q = 0.8 P + N(0, 1);
      T_r uniform over {0, 0.6, 1.0}; confidences as c4; K = 512.

Draft tokens are drawn from softmax(Q / T) by the Gumbel-max trick (argmax of
Q / T plus Gumbel noise), and are argmax Q when T = 0.  Generation runs on the
requested torch device with seeded torch.Generator objects (data seed
1000 + i for logits, 2000 + i for tokens, 3000 + i for confidences and
temperatures).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    D: int
    V: int
    dtype: torch.dtype
    target: torch.Tensor          # (B, D + 1, V): every row a drafter + target pass could produce
    draft: torch.Tensor           # (B, D, V)
    draft_tokens: torch.Tensor    # (B, D) int32
    temperature: torch.Tensor     # (B,) float32
    conf: torch.Tensor | None     # (B, D) float32 drafter confidences, or None (full depth)
    K: int | None                 # budget (draft positions kept), None = full depth


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    B: int
    D: int
    V: int
    dtype: torch.dtype
    index: int          # seeds: 1000 + index, 2000 + index, 3000 + index
    T: float | None     # None = mixed temperatures {0, 0.6, 1.0}
    K: int | None
    kind: str           # logit recipe


SPECS = {
    "c1": Spec("c1", 2, 3, 32, torch.float32, 0, 1.0, None, "c1"),
    "c1_t0": Spec("c1_t0", 2, 3, 32, torch.float32, 0, 0.0, None, "c1"),
    "c2": Spec("c2", 16, 3, 128000, torch.bfloat16, 1, 1.0, None, "c2"),
    "c3": Spec("c3", 32, 16, 151936, torch.bfloat16, 2, 1.0, None, "c3"),
    "c3_t0": Spec("c3_t0", 32, 16, 151936, torch.bfloat16, 2, 0.0, None, "c3"),
    "c4": Spec("c4", 64, 16, 151936, torch.bfloat16, 3, 1.0, 256, "c3"),
    "c4full": Spec("c4full", 64, 16, 151936, torch.bfloat16, 3, 1.0, 1024, "c3"),
    "c5": Spec("c5", 64, 16, 262144, torch.float32, 4, None, 512, "c5"),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, g, device) -> torch.Tensor:
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def make_logits(kind: str, B: int, D: int, V: int, dtype: torch.dtype, seed: int, device):
    """Target (B, D+1, V) and draft (B, D, V) logits for one recipe."""
    g = _gen(device, seed)
    if kind == "c1":
        P = 2.0 * _randn((B, D + 1, V), g, device)
        Q = P[:, :D] + _randn((B, D, V), g, device)
    elif kind == "c2":
        P = 3.0 * _randn((B, D + 1, V), g, device)
        rows = B * (D + 1)
        spike = torch.rand((rows,), generator=g, device=device) < 0.01
        tok = torch.randint(0, V, (rows,), generator=g, device=device)
        flat = P.view(rows, V)
        idx = torch.nonzero(spike).flatten()
        flat[idx, tok[idx]] += 8.0
        sig = torch.tensor([0.5, 1.0, 1.5], device=device)[:D].view(1, D, 1)
        Q = P[:, :D] + sig * _randn((B, D, V), g, device)
    elif kind == "c3":
        P = 3.0 * _randn((B, D + 1, V), g, device)
        sig = (0.3 + 0.1 * torch.arange(D, device=device, dtype=torch.float32)).view(1, D, 1)
        Q = torch.empty((B, D, V), device=device, dtype=torch.float32)
        for k in range(D):  # row by row keeps peak memory to one extra (B, V) slice
            Q[:, k] = P[:, k] + sig[0, k, 0] * _randn((B, V), g, device)
    elif kind == "c5":
        P = 4.0 * _randn((B, D + 1, V), g, device)
        Q = torch.empty((B, D, V), device=device, dtype=torch.float32)
        for k in range(D):
            Q[:, k] = 0.8 * P[:, k] + _randn((B, V), g, device)
    else:
        raise ValueError(kind)
    return P.to(dtype).contiguous(), Q.to(dtype).contiguous()


def draw_draft_tokens(draft: torch.Tensor, temperature: torch.Tensor, seed: int) -> torch.Tensor:
    """A fake drafter: Gumbel-max sample of softmax(Q / T) per row, argmax at T = 0."""
    B, D, V = draft.shape
    device = draft.device
    g = _gen(device, seed)
    out = torch.empty((B, D), dtype=torch.int32, device=device)
    for r in range(B):
        q = draft[r].float()
        T = float(temperature[r])
        if T == 0.0:
            out[r] = torch.argmax(q, dim=-1).to(torch.int32)
        else:
            u = torch.rand((D, V), generator=g, device=device, dtype=torch.float64)
            u = u.clamp_min(1e-300)
            gumbel = -torch.log(-torch.log(u))
            out[r] = torch.argmax(q.double() / T + gumbel, dim=-1).to(torch.int32)
    return out


def draw_confidences(B: int, D: int, seed: int) -> torch.Tensor:
    """Beta(8, 2) for the code-like first half, Beta(3, 3) for the chat-like rest."""
    rng = np.random.default_rng(seed)
    half = B // 2
    c = np.empty((B, D), dtype=np.float32)
    c[:half] = rng.beta(8.0, 2.0, size=(half, D))
    c[half:] = rng.beta(3.0, 3.0, size=(B - half, D))
    return torch.from_numpy(c)


def draw_temperatures(B: int, T: float | None, seed: int) -> torch.Tensor:
    if T is not None:
        return torch.full((B,), float(T), dtype=torch.float32)
    rng = np.random.default_rng(seed)
    choice = np.array([0.0, 0.6, 1.0], dtype=np.float32)
    return torch.from_numpy(choice[rng.integers(0, 3, size=B)])


def make(name: str, device="cpu", B: int | None = None, V: int | None = None) -> Workload:
    """Build a named workload on `device` (optionally with a smaller B or V)."""
    s = SPECS[name]
    B = s.B if B is None else B
    V = s.V if V is None else V
    P, Q = make_logits(s.kind, B, s.D, V, s.dtype, 1000 + s.index, device)
    temp = draw_temperatures(B, s.T, 3000 + s.index)
    tokens = draw_draft_tokens(Q, temp, 2000 + s.index)
    conf = draw_confidences(B, s.D, 3000 + s.index) if s.K is not None else None
    K = None if s.K is None else int(min(s.K, B * s.D) if B == s.B else math.ceil(s.K * B / s.B))
    return Workload(name, B, s.D, V, s.dtype, P, Q, tokens, temp.to(device), conf, K)


def random_rows(shape, scale: float, seed: int, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """Plain Gaussian logits for property tests."""
    g = _gen(device, seed)
    return (scale * _randn(shape, g, device)).to(dtype)
