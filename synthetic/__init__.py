"""Seeded synthetic inputs for the speculative-decoding verification step.

This module only makes inputs.  It holds no part of the verification rule (no
acceptance test, no residual, no normalised distribution, no argmax of target
logits) and is the one piece of code that both the GPU path's callers and the
CPU oracle's callers share.

Workloads (the pages measure on HumanEval/MBPP/GSM8K/... decoding with real
target and draft models; these synthetic rows stand in for those logits, with
the vocabulary sizes of the model families involved):

  id  B    k   V       dtype  target logits              draft logits         T    modes
  1   1    4   32000   fp32   N(0, var 2)                target + N(0, var 1)   1.0  greedy, sample
  2   64   5   32000   fp16   N(0, var 3)                target + N(0, var 1.5) 1.0  sample
  3   256  8   128256  bf16   N(0, var 2) + 8 spike      target + N(0, var 2)   0.7  greedy, sample
  4   32   8x8 152064  bf16   N(0, var 3) + 8 spike      (candidates, see below) -   greedy candidates
  5   512  16  128256  bf16   N(0, var 3) + 8 spike      target + N(0, var 3)   1.0  sample (+ greedy)

The second parameter of N(., .) is read as a variance.  "Spike": +8 added to
one uniformly chosen index per target row; the draft rows inherit it through
"draft = target + noise".  Draft tokens are sampled from softmax(draft / T) of
the dtype-rounded draft logits (Gumbel-max: the index of the largest
draft/T + Gumbel noise), and the same tokens serve greedy mode; for greedy
drafting, greedy_drafts() gives the draft's own argmax at each position.  Uniforms are
24-bit floats k / 2^24 in [0, 1 - 2^-24]: one per draft position plus one for
the round's single sampling step.

Workload 4 (multi-candidate phrase drafts): per sequence C = 8 candidates of
L = 8 tokens sharing a 2-token prefix, R = 8 target rows per candidate.  Row
(c, i) scores candidate token (c, i), so rows (c, 0..2) see the same context
for every c and are generated once and repeated.  Each candidate token is the
spike index of its row with probability 0.8, else a uniform other index.

Every draw comes from a torch.Generator seeded with 1000 + workload id
(+ 7919 * set index for rotated input sets), in a fixed order per chunk of
sequences: target normals, spike indices, draft noise, Gumbel uniforms,
verification uniforms (workload 4: shared rows, distinct rows, spikes,
candidate choices).  Generation runs on the device the tensors live on; the
oracle reads the very same bytes after a copy to the host.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    B: int
    k: int
    V: int
    dtype: str
    var_target: float
    var_noise: float
    spike: float
    T: float
    modes: tuple
    C: int = 0          # candidates (workload 4 only)
    L: int = 0
    R: int = 0
    shared_rows: int = 0
    p_match: float = 0.0

    @property
    def rows_per_seq(self) -> int:
        if self.C:
            return self.C * self.R
        return self.k + 1


WORKLOADS = {
    1: Config(1, B=1, k=4, V=32000, dtype="fp32", var_target=2.0, var_noise=1.0, spike=0.0,
              T=1.0, modes=("greedy", "sample")),
    2: Config(2, B=64, k=5, V=32000, dtype="fp16", var_target=3.0, var_noise=1.5, spike=0.0,
              T=1.0, modes=("sample",)),
    3: Config(3, B=256, k=8, V=128256, dtype="bf16", var_target=2.0, var_noise=2.0, spike=8.0,
              T=0.7, modes=("greedy", "sample")),
    4: Config(4, B=32, k=8, V=152064, dtype="bf16", var_target=3.0, var_noise=0.0, spike=8.0,
              T=1.0, modes=("candidates",), C=8, L=8, R=8, shared_rows=3, p_match=0.8),
    5: Config(5, B=512, k=16, V=128256, dtype="bf16", var_target=3.0, var_noise=3.0, spike=8.0,
              T=1.0, modes=("sample", "greedy")),
}


def make_generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def uniforms24(shape, gen: torch.Generator, device) -> torch.Tensor:
    """float32 uniforms m / 2^24, m uniform in [0, 2^24): never 1.0."""
    m = torch.randint(0, 1 << 24, shape, generator=gen, device=device, dtype=torch.int32)
    return m.to(torch.float32) * (1.0 / (1 << 24))


def gumbel_max_sample(logits: torch.Tensor, T: float, gen: torch.Generator,
                      chunk_rows: int = 1024) -> torch.Tensor:
    """One draw per row from softmax(logits / T) by the Gumbel-max construction.

    logits: [N, V] (any float dtype).  Returns int32 [N].  This plays the
    proposer's part (the draft model sampling its own tokens)."""
    N, V = logits.shape
    out = torch.empty(N, dtype=torch.int32, device=logits.device)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        m = torch.randint(1, 1 << 24, (r1 - r0, V), generator=gen, device=logits.device,
                          dtype=torch.int32)
        uu = m.to(torch.float32) * (1.0 / (1 << 24))
        g = -torch.log(-torch.log(uu))
        out[r0:r1] = torch.argmax(logits[r0:r1].to(torch.float32) / T + g, dim=1).to(torch.int32)
    return out


def greedy_drafts(draft: torch.Tensor, chunk_rows: int = 1024) -> torch.Tensor:
    """Greedy drafting (a draft model decoding at temperature 0): at every
    position the draft's own most likely token, the argmax of its logits.
    draft: [B, k, V]; returns int32 [B, k].  This plays the proposer's part."""
    B, k, V = draft.shape
    flat = draft.reshape(B * k, V)
    out = torch.empty(B * k, dtype=torch.int32, device=draft.device)
    for r0 in range(0, B * k, chunk_rows):
        r1 = min(B * k, r0 + chunk_rows)
        out[r0:r1] = torch.argmax(flat[r0:r1].to(torch.float32), dim=1).to(torch.int32)
    return out.reshape(B, k)


@dataclasses.dataclass
class Workload:
    cfg: Config
    target: torch.Tensor                 # [B, k+1, V] or [B, C, R, V] (cfg dtype)
    draft: Optional[torch.Tensor]        # [B, k, V] or None
    tokens: torch.Tensor                 # [B, k] int32, or candidates [B, C, L]
    uniforms: Optional[torch.Tensor]     # [B, k+1] float32 or None
    T: float

    @property
    def B(self):
        return self.target.shape[0]


def generate(cid: int, device="cpu", set_index: int = 0, B: Optional[int] = None,
             V: Optional[int] = None, k: Optional[int] = None, seed: Optional[int] = None,
             chunk_seqs: Optional[int] = None) -> Workload:
    """Materialise workload `cid` (optionally with B, V or k overridden for
    reduced-size cases) on `device`."""
    cfg = WORKLOADS[cid]
    if B is not None or V is not None or k is not None:
        cfg = dataclasses.replace(cfg, B=B or cfg.B, V=V or cfg.V, k=k or cfg.k)
    if seed is None:
        seed = 1000 + cid + 7919 * set_index
    gen = make_generator(seed, device)
    if cfg.C:
        return _generate_candidates(cfg, gen, device, chunk_seqs)
    return _generate_chain(cfg, gen, device, chunk_seqs)


def _rows_per_chunk(cfg: Config, chunk_seqs):
    if chunk_seqs:
        return chunk_seqs
    # bound the float32 temporaries to ~1 GiB
    per_seq = (2 * cfg.k + 1) * cfg.V * 4
    return max(1, min(cfg.B, (1 << 30) // max(1, per_seq)))


def _generate_chain(cfg: Config, gen, device, chunk_seqs) -> Workload:
    B, k, V = cfg.B, cfg.k, cfg.V
    dt = DTYPES[cfg.dtype]
    target = torch.empty((B, k + 1, V), dtype=dt, device=device)
    draft = torch.empty((B, k, V), dtype=dt, device=device)
    tokens = torch.empty((B, k), dtype=torch.int32, device=device)
    unif = torch.empty((B, k + 1), dtype=torch.float32, device=device)
    sd_t = math.sqrt(cfg.var_target)
    sd_n = math.sqrt(cfg.var_noise)
    step = _rows_per_chunk(cfg, chunk_seqs)
    for b0 in range(0, B, step):
        b1 = min(B, b0 + step)
        nb = b1 - b0
        z = torch.randn((nb, k + 1, V), generator=gen, device=device, dtype=torch.float32) * sd_t
        if cfg.spike:
            idx = torch.randint(0, V, (nb, k + 1, 1), generator=gen, device=device)
            z.scatter_add_(2, idx, torch.full((nb, k + 1, 1), cfg.spike, device=device))
        y = z[:, :k, :] + torch.randn((nb, k, V), generator=gen, device=device,
                                      dtype=torch.float32) * sd_n
        target[b0:b1] = z.to(dt)
        draft[b0:b1] = y.to(dt)
        del z, y
        tokens[b0:b1] = gumbel_max_sample(draft[b0:b1].reshape(nb * k, V), cfg.T, gen).reshape(nb, k)
        unif[b0:b1] = uniforms24((nb, k + 1), gen, device)
    return Workload(cfg, target, draft, tokens, unif, cfg.T)


def _generate_candidates(cfg: Config, gen, device, chunk_seqs) -> Workload:
    B, C, L, R, V = cfg.B, cfg.C, cfg.L, cfg.R, cfg.V
    S = cfg.shared_rows
    dt = DTYPES[cfg.dtype]
    sd_t = math.sqrt(cfg.var_target)
    target = torch.empty((B, C, R, V), dtype=dt, device=device)
    cand = torch.empty((B, C, L), dtype=torch.int32, device=device)
    step = chunk_seqs or max(1, min(B, (1 << 30) // (C * R * V * 4)))
    for b0 in range(0, B, step):
        b1 = min(B, b0 + step)
        nb = b1 - b0
        shared = torch.randn((nb, 1, S, V), generator=gen, device=device) * sd_t
        distinct = torch.randn((nb, C, R - S, V), generator=gen, device=device) * sd_t
        sp_shared = torch.randint(0, V, (nb, 1, S, 1), generator=gen, device=device)
        sp_distinct = torch.randint(0, V, (nb, C, R - S, 1), generator=gen, device=device)
        shared.scatter_add_(3, sp_shared, torch.full((nb, 1, S, 1), cfg.spike, device=device))
        distinct.scatter_add_(3, sp_distinct, torch.full((nb, C, R - S, 1), cfg.spike, device=device))
        z = torch.cat([shared.expand(nb, C, S, V), distinct], dim=2)
        target[b0:b1] = z.to(dt)
        del z, shared, distinct
        spikes = torch.cat([sp_shared.expand(nb, C, S, 1), sp_distinct], dim=2)[..., 0]  # [nb,C,R]
        # token (c, i) for i < L: spike of row (c, i) w.p. p_match, else another index;
        # the 2-token prefix (positions < S - 1) is one draw shared by every candidate
        P = S - 1
        hit = uniforms24((nb, C, L), gen, device) < cfg.p_match
        other = torch.randint(1, V, (nb, C, L), generator=gen, device=device)
        tok = torch.where(hit, spikes[:, :, :L], (spikes[:, :, :L] + other) % V)
        tok[:, :, :P] = tok[:, :1, :P]
        cand[b0:b1] = tok.to(torch.int32)
    return Workload(cfg, target, None, cand, None, 1.0)


def chain(B: int, k: int, V: int, dtype: str = "bf16", var_target: float = 2.0,
          var_noise: float = 1.0, spike: float = 0.0, T: float = 1.0, seed: int = 0,
          device="cpu") -> Workload:
    """A chain-draft workload of any shape (test cases beyond the five workloads)."""
    cfg = Config(0, B=B, k=k, V=V, dtype=dtype, var_target=var_target, var_noise=var_noise,
                 spike=spike, T=T, modes=("greedy", "sample"))
    return _generate_chain(cfg, make_generator(seed, device), device, None)


def candidates(B: int, C: int, L: int, R: int, V: int, dtype: str = "bf16",
               var_target: float = 3.0, spike: float = 8.0, p_match: float = 0.8,
               shared_rows: int = 3, seed: int = 0, device="cpu") -> Workload:
    """A multi-candidate workload of any shape."""
    cfg = Config(0, B=B, k=L, V=V, dtype=dtype, var_target=var_target, var_noise=0.0,
                 spike=spike, T=1.0, modes=("candidates",), C=C, L=L, R=R,
                 shared_rows=min(shared_rows, L), p_match=p_match)
    return _generate_candidates(cfg, make_generator(seed, device), device, None)


def as_tree(w: Workload):
    """The token-tree form of a candidate workload: rows that every candidate
    shares (its first `shared_rows` rows) are stored once, then each
    candidate's own rows.  Returns (nodes [B, N, V], cand_rows [B, C, R]) with
    nodes[b, cand_rows[b, c, i]] == w.target[b, c, i]."""
    cfg = w.cfg
    B, C, R, V = w.target.shape
    S = cfg.shared_rows
    own = R - S
    nodes = torch.cat([w.target[:, 0, :S], w.target[:, :, S:].reshape(B, C * own, V)], dim=1)
    rows = torch.empty((C, R), dtype=torch.int32)
    for c in range(C):
        rows[c, :S] = torch.arange(S)
        rows[c, S:] = S + c * own + torch.arange(own)
    return nodes.contiguous(), rows.to(w.target.device).expand(B, C, R).contiguous()
