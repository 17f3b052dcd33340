"""Seeded synthetic inputs for every workload (shared by the tests, the bench and the oracle legs).

This module holds no attention arithmetic: it only draws tensors.  All draws use a CPU
``torch.Generator`` and ``torch.randn`` in float32; bf16 tensors are the float32 draws rounded to
nearest-even by ``.to(torch.bfloat16)``.  The oracle receives these exact bf16 values upcast to
float64, the HIP path receives the same bits on the device.

Shapes follow the pages: the d20 model has 1280 channels in 10 heads of dimension 128 and each GPU
processes 32 rows of 2048 tokens per step (walkthrough on followin.io, section "Pretraining").
The pages name FineWeb-EDU rows and SmolTalk chats as the real inputs; those datasets are not used
here, and N(0,1) tensors of the same shapes stand in for the activations.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class AttnCase:
    """One training-attention workload (forward, optionally backward)."""

    name: str
    B: int
    T: int
    H: int
    D: int
    window: int | None  # None = full causal
    dtype: torch.dtype
    seed: int
    qkv_scale: float = 1.0
    unit_rms_qk: bool = False
    backward: bool = True


TINY_F32 = AttnCase("tiny-fp32 B1 H2 T128 D64 full", 1, 128, 2, 64, 128, torch.float32, 0,
                    backward=False)
SMALL_W128 = AttnCase("small-bf16 B2 H4 T512 D128 w128", 2, 512, 4, 128, 128, torch.bfloat16, 1,
                      qkv_scale=0.5)
D20_LAYER = AttnCase("d20-layer B32 T2048 H10 D128 full", 32, 2048, 10, 128, None,
                     torch.bfloat16, 2, unit_rms_qk=True)
D26_WINDOWS = (512, None, 512, None)
D26_B, D26_T, D26_H, D26_D, D26_SEED = 16, 2048, 13, 128, 3


# Packed documents in the d20 rows: each of the 32 rows of 2048 tokens holds consecutive
# documents, which the beginning-of-sequence token separates (walkthrough, section "Midtraining");
# a document that runs past the end of a row is cut there and continues as the next row's first
# document, so every row boundary is a document boundary.  The pages give no document-length
# distribution (FineWeb-EDU is not used here): lengths are seeded log-normal draws, median 600
# tokens, log-sigma 1.0, rounded and clipped to [16, 8192].
D20_PACKED_SEED = 5


def d20_packed_cu(B: int = 32, T: int = 2048, seed: int = D20_PACKED_SEED, median: float = 600.0,
                  sigma: float = 1.0) -> torch.Tensor:
    """Sequence offsets (int32 [nseq + 1]) of the packed documents over B rows of T tokens."""
    g = torch.Generator("cpu").manual_seed(seed)
    cu, carry = [0], 0
    for b in range(B):
        pos = 0
        while pos < T:
            if carry == 0:
                z = float(torch.randn((), generator=g, dtype=torch.float64))
                carry = int(min(max(round(median * float(torch.tensor(sigma * z).exp())), 16), 8192))
            take = min(carry, T - pos)
            pos += take
            carry -= take
            cu.append(b * T + pos)
    return torch.tensor(cu, dtype=torch.int32)


def _unit_rms(x: torch.Tensor) -> torch.Tensor:
    # per-(b, t, h) rescaling of the raw draw to unit root-mean-square over D (input shaping only)
    return x / x.pow(2).mean(dim=-1, keepdim=True).sqrt()


def attn_inputs(case: AttnCase):
    """Draw q, k, v, dO for ``case`` in that order, shape [B, T, H, D]."""
    g = torch.Generator("cpu").manual_seed(case.seed)
    shape = (case.B, case.T, case.H, case.D)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    if case.unit_rms_qk:
        q = _unit_rms(q)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    if case.unit_rms_qk:
        k = _unit_rms(k)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if case.qkv_scale != 1.0:
        q, k, v = q * case.qkv_scale, k * case.qkv_scale, v * case.qkv_scale
    out = [q.to(case.dtype), k.to(case.dtype), v.to(case.dtype)]
    if case.backward:
        out.append(torch.randn(shape, generator=g, dtype=torch.float32).to(case.dtype))
    return tuple(out)


def d26_layer_inputs(layer: int, B=D26_B, T=D26_T, H=D26_H, D=D26_D, seed=D26_SEED):
    """Four-layer alternating stack: one generator, layers drawn in order, q, k, v, dO each."""
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (B, T, H, D)
    for l in range(layer + 1):
        tens = [torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(4)]
    return tuple(t.to(torch.bfloat16) for t in tens)


def random_attn(B, T, H, D, seed, dtype=torch.bfloat16, scale=1.0, with_do=True):
    """Generic seeded q, k, v (, dO) of shape [B, T, H, D] for edge sweeps."""
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (B, T, H, D)
    n = 4 if with_do else 3
    out = []
    for i in range(n):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if i < 3:
            x = x * scale
        out.append(x.to(dtype))
    return tuple(out)


# ------------------------------------------------------------------------------------------------
# KV-cache Engine workload (d30-style: 30 layers, 15 heads of 128; windows 1024 on odd layers).
# Each (purpose, layer, step) has its own generator so that any layer or step can be drawn alone:
#   lens                 seed S
#   prefill layer l      seed S*100000 + 1 + l            (packed q, k, v [sum L_b, H, D])
#   decode step s, l     seed S*100000 + 1000 + s*64 + l  (q, k_new, v_new [B, H, D])
# ------------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class EngineCase:
    name: str = "d30-engine B64 H15 D128 Lcap2048 prompts U[32,1024] 64 steps"
    n_layer: int = 30
    B: int = 64
    H: int = 15
    D: int = 128
    Lcap: int = 2048
    len_lo: int = 32
    len_hi: int = 1024
    steps: int = 64
    seed: int = 4

    def window(self, layer: int):
        return 1024 if layer % 2 == 1 else None


D30_ENGINE = EngineCase()


def engine_lens(case: EngineCase = D30_ENGINE) -> torch.Tensor:
    g = torch.Generator("cpu").manual_seed(case.seed)
    return torch.randint(case.len_lo, case.len_hi + 1, (case.B,), generator=g, dtype=torch.int64).to(
        torch.int32)


def engine_prefill_packed(layer: int, lens: torch.Tensor, case: EngineCase = D30_ENGINE):
    """Packed prompt q, k, v [sum(lens), H, D] bf16 for one layer."""
    g = torch.Generator("cpu").manual_seed(case.seed * 100000 + 1 + layer)
    n = int(lens.sum())
    shape = (n, case.H, case.D)
    return tuple(torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)
                 for _ in range(3))


def engine_decode_step(step: int, layer: int, case: EngineCase = D30_ENGINE):
    """q, k_new, v_new [B, H, D] bf16 for one decode step of one layer."""
    g = torch.Generator("cpu").manual_seed(case.seed * 100000 + 1000 + step * 64 + layer)
    shape = (case.B, case.H, case.D)
    return tuple(torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)
                 for _ in range(3))


def pad_prompts(packed: torch.Tensor, lens: torch.Tensor, rows: int) -> torch.Tensor:
    """Scatter packed [sum L, H, D] into zero-padded [B, rows, H, D] (pure data movement)."""
    B = lens.numel()
    out = torch.zeros((B, rows) + tuple(packed.shape[1:]), dtype=packed.dtype)
    off = 0
    for b in range(B):
        L = int(lens[b])
        out[b, :L] = packed[off : off + L]
        off += L
    return out
