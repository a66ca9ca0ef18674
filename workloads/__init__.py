"""Seeded synthetic inputs shaped like the pages' workloads.

Shared by the GPU parity tests, the oracle pins, ``__graft_entry__.smoke()`` and ``bench.py``.
This module holds none of the method's arithmetic: it draws Gaussian tensors with torch's
CPU generator and stores them in the dtype the kernels read (BF16, or FP32 for a
zero-centred training weight).  Nothing here normalises, adds residuals or quantises.

The pages' workloads are LLM / DiT activations; Gaussians of the stated mean and spread
stand in for them (there is no public dataset behind the pages' figures).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

BF16 = torch.bfloat16
F32 = torch.float32


def _gen(seed: int, tensor_id: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1000003 + tensor_id)
    return g


def normal(shape, seed: int, tensor_id: int, mean: float = 0.0, std: float = 1.0,
           dtype=BF16) -> torch.Tensor:
    """N(mean, std^2) drawn in FP32 from a generator keyed by (seed, tensor_id), then stored
    in ``dtype`` (round to nearest even for BF16)."""
    t = torch.randn(tuple(shape), generator=_gen(seed, tensor_id), dtype=F32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def with_outliers(t: torch.Tensor, seed: int, tensor_id: int, frac: float = 0.01,
                  factor: float = 50.0) -> torch.Tensor:
    """Scale an independent Bernoulli(frac) subset of the elements by ``factor``
    (activation outliers), re-stored in the tensor's dtype."""
    u = torch.rand(tuple(t.shape), generator=_gen(seed, tensor_id))
    scaled = (t.float() * factor).to(t.dtype)
    return torch.where(u < frac, scaled, t)


@dataclass
class Workload:
    name: str
    tensors: dict = field(default_factory=dict)
    params: dict = field(default_factory=dict)


# --- the five workloads ------------------------------------------------------------------
# Each takes optional row overrides so tests can draw the same distributions at smaller
# sizes (the oracle then finishes in seconds).

def rmsnorm_fwd(rows: int = 32, hidden: int = 4096, seed: int = 1) -> Workload:
    """rmsnorm forward: x ~ N(0,1), w ~ N(0,1), eps 1e-6 (the norm guide's §2.1 example)."""
    return Workload("rmsnorm", {
        "x": normal((rows, hidden), seed, 0),
        "w": normal((hidden,), seed, 1),
    }, {"eps": 1e-6, "rows": rows, "hidden": hidden})


def fused_add_quant(rows: int = 8192, hidden: int = 4096, seed: int = 2,
                    heads: int | None = None) -> Workload:
    """fused add + RMSNorm + static FP8: x, residual ~ N(0,1); w ~ N(1, 0.1); scale 0.04.
    With ``heads`` the activations are [rows, heads, hidden] (per-head rows)."""
    shape = (rows, hidden) if heads is None else (rows, heads, hidden)
    return Workload("fused_add_rmsnorm_quant", {
        "x": normal(shape, seed, 0),
        "residual": normal(shape, seed, 1),
        "w": normal((hidden,), seed, 2, mean=1.0, std=0.1),
    }, {"eps": 1e-6, "scale": 0.04, "rows": rows, "hidden": hidden, "heads": heads})


def block_quant(rows: int = 16384, hidden: int = 7168, seed: int = 3) -> Workload:
    """fused add + RMSNorm + 1x128 FP8 blocks: x, residual ~ N(0,1) with 1 % of the elements
    scaled by 50; w ~ N(1, 0.1)."""
    return Workload("fused_add_rmsnorm_fp8_block_quant", {
        "x": with_outliers(normal((rows, hidden), seed, 0), seed, 10),
        "residual": with_outliers(normal((rows, hidden), seed, 1), seed, 11),
        "w": normal((hidden,), seed, 2, mean=1.0, std=0.1),
    }, {"eps": 1e-6, "rows": rows, "hidden": hidden})


def train(rows: int = 16384, hidden: int = 8192, seed: int = 4) -> Workload:
    """training forward + backward with residual: h, residual, g ~ N(0,1); FP32 w ~
    N(0, 0.02) used as the effective weight 1 + w."""
    return Workload("train", {
        "h": normal((rows, hidden), seed, 0),
        "residual": normal((rows, hidden), seed, 1),
        "w": normal((hidden,), seed, 2, std=0.02, dtype=F32),
        "g": normal((rows, hidden), seed, 3),
    }, {"eps": 1e-6, "w_bias": 1.0, "rows": rows, "hidden": hidden})


def ada(rows: int = 2520, dim: int = 3072, seed: int = 5, broadcast: bool = False) -> Workload:
    """AdaRMSNorm gated residual + static FP8: x, residual, gate ~ N(0,1); weight ones;
    style ~ N(0,1) of (rows, 3*dim), or (1, 3*dim) when broadcast; scale 0.04."""
    style_rows = 1 if broadcast else rows
    return Workload("ada", {
        "x": normal((rows, dim), seed, 0),
        "residual": normal((rows, dim), seed, 1),
        "gate": normal((rows, dim), seed, 2),
        "w": torch.ones((dim,), dtype=BF16),
        "style": normal((style_rows, 3 * dim), seed, 3 + (100 if broadcast else 0)),
    }, {"eps": 1e-6, "scale": 0.04, "rows": rows, "dim": dim, "broadcast": broadcast})


# --- the LayerNorm family ---------------------------------------------------------------

def layernorm(rows: int = 8192, hidden: int = 4096, seed: int = 6, mean: float = 0.5) -> Workload:
    """LayerNorm (+ static FP8): x ~ N(mean, 1) (a non-zero mean exercises the centring);
    FP32 gamma ~ N(1, 0.1) and beta ~ N(0, 0.1); scale 0.04."""
    return Workload("layernorm", {
        "x": normal((rows, hidden), seed, 0, mean=mean),
        "gamma": normal((hidden,), seed, 1, mean=1.0, std=0.1, dtype=F32),
        "beta": normal((hidden,), seed, 2, std=0.1, dtype=F32),
    }, {"eps": 1e-6, "scale": 0.04, "rows": rows, "hidden": hidden})


DIT_CHUNKS = ("shift", "scale", "gate", "shift_mlp", "scale_mlp", "gate_mlp")


def dit(rows: int = 2520, hidden: int = 3072, seed: int = 7) -> Workload:
    """DiT gate/residual + LayerNorm: x, residual ~ N(0,1); a per-token modulation tensor
    temb [rows, 6*hidden] ~ N(0, 0.5) whose six chunks (shift, scale, gate, and the MLP's
    three) are views with row stride 6*hidden; FP32 gamma ~ N(1, 0.1), beta ~ N(0, 0.1);
    scalar biases gate 0.25, scale 0.125, shift -0.0625."""
    temb = normal((rows, 6 * hidden), seed, 2, std=0.5)
    t = {
        "x": normal((rows, hidden), seed, 0),
        "residual": normal((rows, hidden), seed, 1),
        "temb": temb,
        "gamma": normal((hidden,), seed, 3, mean=1.0, std=0.1, dtype=F32),
        "beta": normal((hidden,), seed, 4, std=0.1, dtype=F32),
    }
    for k, name in enumerate(DIT_CHUNKS):
        t[name] = temb[:, k * hidden:(k + 1) * hidden]
    return Workload("dit", t, {"eps": 1e-6, "rows": rows, "hidden": hidden, "gate_bias": 0.25,
                               "scale_bias": 0.125, "shift_bias": -0.0625})


def qk_rope(ppf: int = 16, pph: int = 24, ppw: int = 32, batch: int = 1, nq: int = 24,
            nk: int = 24, nv: int = 24, head_dim: int = 128, channels=(44, 42, 42),
            seed: int = 8) -> Workload:
    """Fused QK RMSNorm + 3-D RoPE: qkv BF16 [batch*ppf*pph*ppw, (nq+nk+nv)*head_dim]
    ~ N(0,1); q_weight, k_weight BF16 ~ N(1, 0.1).  The default head layout (24 heads of
    128 channels; 44 frame, 42 height and 42 width channels) is that of a 3072-wide
    video DiT; the patch grid 16 x 24 x 32 is a stand-in video latent."""
    tokens = batch * ppf * pph * ppw
    return Workload("qk_rope", {
        "qkv": normal((tokens, (nq + nk + nv) * head_dim), seed, 0),
        "q_weight": normal((nq * head_dim,), seed, 1, mean=1.0, std=0.1),
        "k_weight": normal((nk * head_dim,), seed, 2, mean=1.0, std=0.1),
    }, {"eps": 1e-6, "tokens": tokens, "nq": nq, "nk": nk, "nv": nv, "head_dim": head_dim,
        "channels": tuple(channels), "ppf": ppf, "pph": pph, "ppw": ppw, "base": 10000.0,
        "output_scale": 0.05, "v_scale": 0.02})


def rmsnorm_silu(tokens: int = 99840, hidden: int = 512, seed: int = 9) -> Workload:
    """Fused RMSNorm + SiLU: x BF16 [tokens, hidden] ~ N(0,1), w BF16 ~ N(1, 0.1); FP8 scale
    0.02.  The pages tune this op for a video VAE decoder over hidden sizes 64 ... 1024 and
    1560 ... 399360 tokens."""
    return Workload("rmsnorm_silu", {
        "x": normal((tokens, hidden), seed, 0),
        "w": normal((hidden,), seed, 1, mean=1.0, std=0.1),
    }, {"eps": 1e-6, "tokens": tokens, "hidden": hidden, "scale": 0.02})


SILU_HIDDEN = (64, 128, 160, 256, 320, 512, 640, 1024)
SILU_TOKENS = (1560, 6240, 24960, 99840, 399360)


def sigmoid_gate(tokens: int = 16384, heads: int = 64, head_dim: int = 64,
                 seed: int = 10) -> Workload:
    """Per-head RMSNorm + sigmoid gate: x, gate BF16 [tokens, heads*head_dim] ~ N(0,1) and
    N(0, 2); w BF16 [head_dim] ~ N(1, 0.1).  Head dim 64 is the pages' width; 64 heads of
    64 make a 4096-wide attention output."""
    return Workload("sigmoid_gate", {
        "x": normal((tokens, heads * head_dim), seed, 0),
        "gate": normal((tokens, heads * head_dim), seed, 1, std=2.0),
        "w": normal((head_dim,), seed, 2, mean=1.0, std=0.1),
    }, {"eps": 1e-6, "tokens": tokens, "heads": heads, "head_dim": head_dim})


def gated_residual(rows: int = 16384, hidden: int = 8192, seed: int = 11,
                   per_token_gate: bool = True) -> Workload:
    """Gated-residual RMSNorm (+ next RMSNorm): branch, residual BF16 [rows, hidden] ~ N(0,1);
    gate BF16 ~ N(0, 0.5) per token ([rows, hidden]) or one shared row ([1, hidden]);
    w, w_next BF16 ~ N(1, 0.1).  Hidden 8192 is the pages' width."""
    return Workload("gated_residual", {
        "branch": normal((rows, hidden), seed, 0),
        "residual": normal((rows, hidden), seed, 1),
        "gate": normal((rows if per_token_gate else 1, hidden), seed,
                       2 if per_token_gate else 3, std=0.5),
        "w": normal((hidden,), seed, 4, mean=1.0, std=0.1),
        "w_next": normal((hidden,), seed, 5, mean=1.0, std=0.1),
    }, {"eps": 1e-6, "rows": rows, "hidden": hidden})
