"""Seeded synthetic workloads for the IceCache hot path.

This module only draws inputs (keys, values, queries). It holds none of the
method's arithmetic: no lift, no promotion, no distances, no selection. The
same tensors feed the GPU library and the fp64 oracle, so both sides always see
bit-identical inputs.

Workload shapes follow the method pages: keys of one attention head cluster by
meaning (papernotes.org "IceCache: Memory-Efficient KV-cache Management for
Long-Sequence LLMs", key design 1: semantically similar tokens should share a
page), so keys are drawn from a Gaussian mixture whose components are picked
independently per token. Related tokens are therefore scattered in position,
which is the case the notes' "motivation" section says sequential pages handle
badly.

Recipe (every draw comes from one ``torch.Generator`` seeded by the caller):

* centres ``c_m ~ N(0, I_d)``, ``m < C`` per head;
* key ``k_t = c_{m_t} + sigma * N(0, I_d)`` with ``m_t`` uniform, ``sigma = 0.3``;
* value ``v_t ~ N(0, I_d)``;
* decode query ``q = c_m + sigma * N(0, I_d)``, ``m`` uniform per query head;
* optional per-head random rotation ``R_h`` (QR of a Gaussian matrix, signs of
  ``diag(R)`` made positive) applied to centres, keys and queries;
* bf16 inputs are the fp32 draws rounded to nearest-even by ``Tensor.to``.

Generation can run on the CPU (tests) or on the GPU (large benchmark shapes);
the two devices give different streams for the same seed, so a test that needs
the oracle copies the very tensors it fed to the GPU back to the host.
"""
from __future__ import annotations

import dataclasses
import math

import torch

SIGMA = 0.3


@dataclasses.dataclass
class Mixture:
    """Per-head Gaussian-mixture key distribution."""

    centres: torch.Tensor          # [H, C, d] float32
    rot: torch.Tensor | None       # [H, d, d] float32 or None

    @property
    def n_heads(self) -> int:
        return self.centres.shape[0]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def random_rotations(n_heads: int, d: int, gen: torch.Generator, device) -> torch.Tensor:
    """Haar-distributed orthogonal matrices: QR of a Gaussian, sign-fixed."""
    a = torch.randn(n_heads, d, d, generator=gen, device=device, dtype=torch.float32)
    # QR in float64 on the host keeps the factorisation device independent.
    q, r = torch.linalg.qr(a.double().cpu())
    s = torch.sign(torch.diagonal(r, dim1=-2, dim2=-1))
    s[s == 0] = 1.0
    q = q * s.unsqueeze(-2)
    return q.float().to(device)


def make_mixture(n_heads: int, n_centres: int, d: int, gen: torch.Generator, device,
                 rotate: bool = False) -> Mixture:
    centres = torch.randn(n_heads, n_centres, d, generator=gen, device=device, dtype=torch.float32)
    rot = random_rotations(n_heads, d, gen, device) if rotate else None
    return Mixture(centres=centres, rot=rot)


def _apply_rot(x: torch.Tensor, mix: Mixture) -> torch.Tensor:
    if mix.rot is None:
        return x
    # x: [H, n, d]; rotate row vectors of head h by R_h.
    return torch.bmm(x, mix.rot.transpose(1, 2).contiguous())


def draw_keys(mix: Mixture, n_tokens: int, gen: torch.Generator, device,
              sigma: float = SIGMA, chunk: int = 1 << 22) -> torch.Tensor:
    """Keys [H, N, d] float32 from the mixture (component uniform per token)."""
    h, c, d = mix.centres.shape
    out = torch.empty(h, n_tokens, d, device=device, dtype=torch.float32)
    rows = max(1, chunk // max(1, h * d))
    for s in range(0, n_tokens, rows):
        e = min(n_tokens, s + rows)
        m = torch.randint(0, c, (h, e - s), generator=gen, device=device)
        noise = torch.randn(h, e - s, d, generator=gen, device=device, dtype=torch.float32)
        k = torch.gather(mix.centres, 1, m.unsqueeze(-1).expand(h, e - s, d)) + sigma * noise
        out[:, s:e] = _apply_rot(k, mix)
    return out


def draw_values(n_heads: int, n_tokens: int, d: int, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn(n_heads, n_tokens, d, generator=gen, device=device, dtype=torch.float32)


def draw_queries(mix: Mixture, group: int, gen: torch.Generator, device,
                 sigma: float = SIGMA) -> torch.Tensor:
    """One decode query per query head: [H, G, d] float32, centre + noise."""
    h, c, d = mix.centres.shape
    m = torch.randint(0, c, (h, group), generator=gen, device=device)
    noise = torch.randn(h, group, d, generator=gen, device=device, dtype=torch.float32)
    q = torch.gather(mix.centres, 1, m.unsqueeze(-1).expand(h, group, d)) + sigma * noise
    return _apply_rot(q, mix)


def to_dtype(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """'f32' keeps float32; 'bf16' rounds to nearest-even bfloat16."""
    if dtype == "f32":
        return x.float().contiguous()
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


@dataclasses.dataclass
class Workload:
    K: torch.Tensor      # [H, N, d] in the workload dtype
    V: torch.Tensor      # [H, N, d]
    mix: Mixture
    dtype: str


def clustered_kv(n_heads: int, n_tokens: int, d: int, n_centres: int, dtype: str, seed: int,
                 device="cpu", rotate: bool = False) -> tuple[Workload, torch.Generator]:
    """Keys from a per-head Gaussian mixture and N(0,1) values, seeded.

    Returns the workload and the generator, so the caller can keep drawing
    decode queries / new tokens from the same stream.
    """
    gen = _gen(seed, device)
    mix = make_mixture(n_heads, n_centres, d, gen, device, rotate=rotate)
    K = draw_keys(mix, n_tokens, gen, device)
    V = draw_values(n_heads, n_tokens, d, gen, device)
    return Workload(K=to_dtype(K, dtype), V=to_dtype(V, dtype), mix=mix, dtype=dtype), gen


def decode_queries(w: Workload, group: int, gen: torch.Generator, device="cpu") -> torch.Tensor:
    return to_dtype(draw_queries(w.mix, group, gen, device), w.dtype)


def new_tokens(w: Workload, gen: torch.Generator, device="cpu") -> tuple[torch.Tensor, torch.Tensor]:
    """One fresh (k, v) per head from the same mixture: [H, 1, d] each."""
    h, c, d = w.mix.centres.shape
    k = draw_keys(w.mix, 1, gen, device)
    v = draw_values(h, 1, d, gen, device)
    return to_dtype(k, w.dtype), to_dtype(v, w.dtype)


def resident_tokens(w: Workload, n: int, gen: torch.Generator, device="cpu") -> tuple[torch.Tensor, torch.Tensor]:
    """n (k, v) per head from the same mixture, [H, n, d] each: stand-ins for
    the sink and window tokens kept beside the index."""
    h, c, d = w.mix.centres.shape
    k = draw_keys(w.mix, n, gen, device)
    v = draw_values(h, n, d, gen, device)
    return to_dtype(k, w.dtype), to_dtype(v, w.dtype)


def projection_dirs(rows: int, d: int, seed: int, device="cpu") -> torch.Tensor:
    """``rows`` random unit directions over lifted keys [k, e] (d + 1 wide),
    float32 [rows, d + 1], seeded: the projections of P-DCI's simple indices."""
    gen = torch.Generator().manual_seed(seed)
    u = torch.randn(rows, d + 1, generator=gen, dtype=torch.float64)
    return (u / u.norm(dim=1, keepdim=True)).float().to(device)


def needle_workload(n_heads: int, group: int, n_tokens: int, d: int, n_centres: int, depth: float,
                    seed: int, dtype: str = "bf16", device="cpu", span: int = 16,
                    cosine: float = 0.9):
    """Background mixture keys plus one planted span aligned with a fresh query.

    For query head 0 of every KV head the final query is ``q ~ N(0, 1.09 I)``
    (a direction that is no mixture centre). The span's keys are
    ``k_j = r_j (cos * q_hat + sqrt(1 - cos^2) * w_j)`` with ``w_j`` a unit
    vector orthogonal to ``q_hat`` and ``r_j`` the norm of a random background
    key, so every needle key has exactly the requested cosine with ``q``.
    The span starts at ``round(depth * (N - span))``. Other query heads get
    centre queries. Returns (workload, Q [H,G,d], start).
    """
    w, gen = clustered_kv(n_heads, n_tokens, d, n_centres, "f32", seed, device)
    K = w.K.clone()
    start = int(round(depth * (n_tokens - span)))
    q = draw_queries(w.mix, group, gen, device)
    q0 = math.sqrt(1.09) * torch.randn(n_heads, d, generator=gen, device=device, dtype=torch.float32)
    q[:, 0] = q0
    qh = q0 / q0.norm(dim=-1, keepdim=True)
    g = torch.randn(n_heads, span, d, generator=gen, device=device, dtype=torch.float32)
    g = g - (g * qh.unsqueeze(1)).sum(-1, keepdim=True) * qh.unsqueeze(1)
    wdir = g / g.norm(dim=-1, keepdim=True)
    pick = torch.randint(0, n_tokens, (n_heads, span), generator=gen, device=device)
    r = torch.gather(K.norm(dim=-1), 1, pick)
    sin = math.sqrt(1.0 - cosine * cosine)
    K[:, start:start + span] = r.unsqueeze(-1) * (cosine * qh.unsqueeze(1) + sin * wdir)
    wl = Workload(K=to_dtype(K, dtype), V=to_dtype(w.V, dtype), mix=w.mix, dtype=dtype)
    return wl, to_dtype(q, dtype), start


class QueryWalk:
    """Queries that drift between mixture centres along a seeded walk.

    Query head g of KV head h visits centres a_0, a_1, ... ; for step t with
    j = t // seg: ``w_t = c_{a_j} + ((t - seg*j)/seg) (c_{a_{j+1}} - c_{a_j})`` and
    ``q_t = w_t + sigma N(0, I)``. The new key of KV head h at step t is the walk
    point of its query head 0 plus fresh noise; its value is N(0, I).
    """

    def __init__(self, w: Workload, group: int, gen: torch.Generator, device="cpu", seg: int = 64):
        self.w, self.group, self.gen, self.device, self.seg = w, group, gen, device, seg
        h, c, d = w.mix.centres.shape
        self.a_prev = torch.randint(0, c, (h, group), generator=gen, device=device)
        self.a_next = torch.randint(0, c, (h, group), generator=gen, device=device)
        self.t = 0

    def _centre(self, a):
        h, c, d = self.w.mix.centres.shape
        return torch.gather(self.w.mix.centres, 1, a.unsqueeze(-1).expand(h, self.group, d))

    def step(self):
        """Returns (Q [H,G,d], k_new [H,1,d], v_new [H,1,d]) for the current step."""
        h, c, d = self.w.mix.centres.shape
        j, r = divmod(self.t, self.seg)
        if r == 0 and self.t > 0:
            self.a_prev = self.a_next
            self.a_next = torch.randint(0, c, (h, self.group), generator=self.gen, device=self.device)
        frac = r / self.seg
        wpt = self._centre(self.a_prev) + frac * (self._centre(self.a_next) - self._centre(self.a_prev))
        wpt = _apply_rot(wpt, self.w.mix)
        q = wpt + SIGMA * torch.randn(h, self.group, d, generator=self.gen, device=self.device)
        k = wpt[:, :1] + SIGMA * torch.randn(h, 1, d, generator=self.gen, device=self.device)
        v = torch.randn(h, 1, d, generator=self.gen, device=self.device)
        self.t += 1
        return to_dtype(q, self.w.dtype), to_dtype(k, self.w.dtype), to_dtype(v, self.w.dtype)
