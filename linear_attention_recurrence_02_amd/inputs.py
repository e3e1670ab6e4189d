"""Seeded synthetic workloads shared by the GPU tests, the oracle tests and the
benchmark.

This module draws random numbers and shapes them into inputs; it holds none of
the gated delta rule's arithmetic.  Both the GPU path and the CPU oracle are
fed from here, and neither computes its inputs itself.

Recipe (the same for every workload):
  * sequence lengths (packed batches only) come from a CPU ``torch.Generator``
    seeded with ``seed``; the tensors come from a ``torch.Generator`` on the
    target device seeded with ``seed`` (float32 ``randn`` in the fixed order q,
    k, v, g_raw, beta_raw, S0).  Drawing on the device keeps the multi-GB
    workloads quick to make; a workload is reproducible for a given device
    type and torch build;
  * q and k are divided by their L2 norm over the head dimension (in fp32),
    then cast to the io dtype; v is cast as drawn;
  * g = -softplus(g_raw) (a log-decay <= 0), beta = sigmoid(beta_raw), both fp32;
  * S0 = 0.1 * randn, fp32.
The pages run these recurrences inside whole models on prompts and images; no
public dataset is involved, and these draws stand in for the projected q/k/v
and gate activations of such a model (unit-norm keys and queries, a decay that
forgets within a few tokens, a write strength in (0, 1)).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch
import torch.nn.functional as F

DK = 128
DV = 128


@dataclass
class Workload:
    """Host-side tensors for one call of the prompt form or of decode steps."""
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    S0: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor] = None   # int32 [N+1] or None
    chunk: int = 64
    meta: dict = field(default_factory=dict)

    @property
    def io_dtype(self) -> torch.dtype:
        return self.q.dtype

    def to(self, device) -> "Workload":
        mv = lambda t: None if t is None else t.to(device)
        return Workload(self.name, mv(self.q), mv(self.k), mv(self.v), mv(self.g),
                        mv(self.beta), mv(self.S0), mv(self.cu_seqlens), self.chunk,
                        dict(self.meta))


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def _generator(seed: int, device) -> torch.Generator:
    return torch.Generator(device=torch.device(device)).manual_seed(seed)


def _draw(gen, lead, dk, dv, io_dtype, n_states, s0: bool):
    """Draw q, k, v, g, beta, S0 in the fixed order for token shape ``lead``."""
    dev = gen.device
    rn = lambda *shape: torch.randn(*shape, generator=gen, device=dev)
    q = _unit(rn(*lead, dk)).to(io_dtype)
    k = _unit(rn(*lead, dk)).to(io_dtype)
    v = rn(*lead, dv).to(io_dtype)
    g = -F.softplus(rn(*lead))
    beta = torch.sigmoid(rn(*lead))
    S0 = 0.1 * rn(*n_states, dk, dv) if s0 else None
    return q, k, v, g, beta, S0


def prefill_workload(B: int, T: int, H: int, *, chunk: int = 64,
                     io_dtype=torch.bfloat16, s0: bool = True, seed: int = 0,
                     dk: int = DK, dv: int = DV, name: str = "prefill",
                     device="cpu") -> Workload:
    """B sequences of T tokens each, q/k/v laid out [B, T, H, d]."""
    gen = _generator(seed, device)
    q, k, v, g, beta, S0 = _draw(gen, (B, T, H), dk, dv, io_dtype, (B, H), s0)
    return Workload(name, q, k, v, g, beta, S0, None, chunk,
                    dict(B=B, T=T, H=H, seed=seed, tokens=B * T))


def varlen_workload(lengths=None, *, n_seqs: int = 32, lo: int = 17, hi: int = 8192,
                    H: int = 16, chunk: int = 64, io_dtype=torch.bfloat16,
                    s0: bool = True, seed: int = 0, dk: int = DK, dv: int = DV,
                    name: str = "varlen", device="cpu") -> Workload:
    """A packed batch: sequence lengths drawn uniformly from [lo, hi] (integers,
    both ends inclusive) unless given, laid out [1, sum(L), H, d] with
    cu_seqlens offsets and one S0 slice per sequence."""
    if lengths is None:
        lengths = torch.randint(lo, hi + 1, (n_seqs,), generator=_generator(seed, "cpu"))
    gen = _generator(seed, device)
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    cu = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    total = int(cu[-1])
    q, k, v, g, beta, S0 = _draw(gen, (1, total, H), dk, dv, io_dtype,
                                 (lengths.numel(), H), s0)
    return Workload(name, q, k, v, g, beta, S0, cu.to(torch.int32).to(device), chunk,
                    dict(N=lengths.numel(), T=total, H=H, seed=seed, tokens=total,
                         lengths=lengths.tolist()))


def verify_workload(n_seqs: int = 256, block: int = 16, H: int = 16, *, chunk: int = 64,
                    io_dtype=torch.bfloat16, seed: int = 0, device="cpu") -> Workload:
    """Speculative-verify blocks: ``n_seqs`` sequences of ``block`` tokens each,
    packed with cu_seqlens, each starting from its own snapshotted state."""
    return varlen_workload([block] * n_seqs, H=H, chunk=chunk, io_dtype=io_dtype,
                           s0=True, seed=seed, name="verify", device=device)


def decode_workload(steps: int, B: int, H: int, *, io_dtype=torch.bfloat16,
                    seed: int = 0, dk: int = DK, dv: int = DV, device="cpu") -> Workload:
    """``steps`` consecutive single-token steps for a batch of B x H states:
    q/k/v are [steps, B, H, d], g/beta [steps, B, H], S0 the [B, H, dk, dv]
    state the first step starts from."""
    gen = _generator(seed, device)
    q, k, v, g, beta, S0 = _draw(gen, (steps, B, H), dk, dv, io_dtype, (B, H), True)
    return Workload("decode", q, k, v, g, beta, S0, None, 1,
                    dict(steps=steps, B=B, H=H, seed=seed))


# The five workloads, named by what they are.
def tiny_prefill(seed=0, device="cpu"):
    """B=1, H=2, T=256, chunk 16, fp32 inputs, nonzero S0."""
    return prefill_workload(1, 256, 2, chunk=16, io_dtype=torch.float32, s0=True,
                            seed=seed, name="tiny_prefill", device=device)


def long_prefill(seed=0, device="cpu"):
    """B=1, H=16, T=4096, chunk 64, bf16 inputs, nonzero S0."""
    return prefill_workload(1, 4096, 16, chunk=64, s0=True, seed=seed,
                            name="long_prefill", device=device)


def large_prefill(seed=0, device="cpu"):
    """B=8, H=32, T=16384, chunk 64, bf16 inputs, zero S0."""
    return prefill_workload(8, 16384, 32, chunk=64, s0=False, seed=seed,
                            name="large_prefill", device=device)


def batched_decode(seed=0, steps=1000, device="cpu"):
    """B=64 sequences x H=16 heads, one bf16 token each per step."""
    return decode_workload(steps, 64, 16, seed=seed, device=device)


def varlen_prefill(seed=0, device="cpu"):
    """32 sequences, lengths uniform in [17, 8192], H=16, chunk 64, bf16,
    per-sequence nonzero S0."""
    return varlen_workload(n_seqs=32, lo=17, hi=8192, H=16, seed=seed, device=device)


def verify_blocks(seed=0, device="cpu"):
    """256 sequences x 16-token verify blocks, H=16, from snapshotted states."""
    return verify_workload(256, 16, 16, seed=seed, device=device)


def norm_gate(w: Workload, seed: int = 0, eps: float = 1e-6):
    """Inputs of the gated RMS norm on the output of workload ``w``: the gate z
    ~ N(0, 1) with v's shape and io dtype, and weights ~ U(0.5, 1.5) fp32 [dv],
    both from a generator on v's device seeded with ``seed + 7919`` (so that they
    do not repeat the workload's own draws); eps as given (1e-6 by default, the
    usual RMS-norm epsilon).  Returns (z, norm_w, eps)."""
    gen = _generator(seed + 7919, w.v.device)
    z = torch.randn(*w.v.shape, generator=gen, device=w.v.device).to(w.v.dtype)
    norm_w = 0.5 + torch.rand(w.v.shape[-1], generator=gen, device=w.v.device)
    return z, norm_w, eps


@dataclass
class PreopInputs:
    """Inputs of the block's pre-operations for one call."""
    xq: torch.Tensor
    xk: torch.Tensor
    xv: torch.Tensor
    a: torch.Tensor
    b: torch.Tensor
    conv_w: torch.Tensor
    state: torch.Tensor
    cu_seqlens: Optional[torch.Tensor] = None


def preop_inputs(B: int, T: int, H: int, *, lengths=None, io_dtype=torch.bfloat16,
                 seed: int = 0, device="cpu") -> PreopInputs:
    """Raw projections and gate inputs for B sequences of T tokens (or a packed
    batch of ``lengths``), drawn from a generator on ``device`` seeded with
    ``seed`` in the order xq, xk, xv, a, b, conv_w, state: projections, gate
    inputs and FIFO state ~ N(0, 1) (projections and state in the io dtype),
    conv weights ~ N(0, 0.5^2) fp32.  No trained weights are involved; the
    draws stand in for a model's projections and its conv parameters."""
    gen = _generator(seed, device)
    rn = lambda *shape: torch.randn(*shape, generator=gen, device=gen.device)
    cu = None
    if lengths is not None:
        lengths = torch.as_tensor(lengths, dtype=torch.int64)
        c = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
        c[1:] = torch.cumsum(lengths, 0)
        cu = c.to(torch.int32).to(device)
        B, T, N = 1, int(c[-1]), lengths.numel()
    else:
        N = B
    xq, xk, xv = (rn(B, T, H, DK).to(io_dtype) for _ in range(3))
    a, b = rn(B, T, H), rn(B, T, H)
    conv_w = 0.5 * rn(3, H, DK, 4)
    state = rn(N, 3, H, 3, DK).to(io_dtype)
    return PreopInputs(xq, xk, xv, a, b, conv_w, state, cu)


# --- inputs at the edges of the method's numerics ------------------------------
#
# The Qwen3.5-9B-npu model page ("How it works" -> "Gated DeltaNet on the NPU"
# and "fp16 precision of the DeltaNet output") names two hazards for reduced
# precision: real keys are highly correlated, and some heads carry outputs far
# smaller than others.  These draws reproduce both, plus the special cases of
# the recurrence (no write, a full read-back, full decay), at any size.

KEYS = ("iid", "corr", "exact")
DECAYS = ("normal", "slow", "none", "full", "reset")
WRITES = ("sigmoid", "one", "zero")


def edge_workload(B: int, T: int, H: int, *, keys: str = "iid", sigma: float = 0.1,
                  decay: str = "normal", write: str = "sigmoid", value_scale: float = 1.0,
                  q_is_k: bool = False, lengths=None, chunk: int = 64,
                  io_dtype=torch.bfloat16, s0: bool = True, seed: int = 0,
                  device="cpu") -> Workload:
    """A prompt-form workload at an edge of the numerics.

    keys: "iid" draws unit keys as the other workloads do; "corr" draws
      k = normalize(b + sigma n / sqrt(dk)) around one unit direction b per
      (sequence, head), n ~ N(0, I), so that neighbouring keys have cosine
      about 1 / sqrt(1 + sigma^2) (0.958, 0.995, 0.9996 at sigma 0.3, 0.1, 0.03);
      "exact" draws keys whose norm is exactly 1 in bf16: +-1/8 on 64 of the
      128 coordinates (random signs and coordinates), zero elsewhere.
    decay: "normal" g = -softplus(x), "slow" 0.02 times that, "none" g = 0,
      "full" g = -1e4 (exp(g) underflows to zero in fp32), "reset" the normal
      draws with g = -1e4 at every 97th token (a token that clears the state,
      at varying positions within 64- and 16-token chunks).
    write: "sigmoid" beta = sigmoid(x), "one" beta = 1, "zero" beta = 0.
    value_scale: v and S0 are multiplied by it (the page's small heads have an
      output RMS of 1e-3..2e-2).
    q_is_k: queries equal to the keys.
    lengths: a packed batch of these lengths (B must then be 1 and T their sum).
    Draw order from one generator seeded with ``seed`` on ``device``: q, k (or
    the key directions and the spread), v, g_raw, beta_raw, S0.
    """
    if keys not in KEYS or decay not in DECAYS or write not in WRITES:
        raise ValueError("unknown edge workload option")
    gen = _generator(seed, device)
    dev = gen.device
    rn = lambda *shape: torch.randn(*shape, generator=gen, device=dev)
    cu = None
    n_states = B
    if lengths is not None:
        lengths = torch.as_tensor(lengths, dtype=torch.int64)
        c = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
        c[1:] = torch.cumsum(lengths, 0)
        if B != 1 or int(c[-1]) != T:
            raise ValueError("a packed batch needs B == 1 and T == sum(lengths)")
        cu = c.to(torch.int32).to(device)
        n_states = lengths.numel()
    lead = (B, T, H)
    q = _unit(rn(*lead, DK))
    if keys == "corr":
        base = _unit(rn(B, 1, H, DK))
        k = _unit(base + sigma * rn(*lead, DK) / DK ** 0.5)
    elif keys == "exact":
        x = rn(*lead, DK)
        rank = x.abs().argsort(dim=-1).argsort(dim=-1)      # a random half of the coordinates
        k = torch.where(rank >= DK // 2, torch.sign(x) / 8, torch.zeros_like(x))
    else:
        k = _unit(rn(*lead, DK))
    if q_is_k:
        q = k
    v = rn(*lead, DV) * value_scale
    g = -F.softplus(rn(*lead))
    if decay == "slow":
        g = 0.02 * g
    elif decay == "none":
        g = torch.zeros_like(g)
    elif decay == "full":
        g = torch.full_like(g, -1e4)
    elif decay == "reset":
        g[:, 96::97] = -1e4
    beta = torch.sigmoid(rn(*lead))
    if write == "one":
        beta = torch.ones_like(beta)
    elif write == "zero":
        beta = torch.zeros_like(beta)
    S0 = 0.1 * value_scale * rn(n_states, H, DK, DV) if s0 else None
    name = f"edge[{keys}{'' if keys == 'iid' else f' s={sigma}'} g={decay} b={write} x{value_scale:g}]"
    meta = dict(B=B, T=T, H=H, seed=seed, tokens=T if lengths is not None else B * T)
    if lengths is not None:
        meta.update(N=n_states, lengths=lengths.tolist())
    return Workload(name, q.to(io_dtype), k.to(io_dtype), v.to(io_dtype), g, beta, S0,
                    cu, chunk, meta)
