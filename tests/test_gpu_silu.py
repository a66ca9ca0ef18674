"""GPU parity of the fused RMSNorm + SiLU against the FP64 oracle: BF16 within one ulp
(the cancellation-aware gate with SiLU's error amplification 1 + |y|), FP8 codes equal
except at flagged ties."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import silu as S
from tests.conftest import values
from tests.parity import assert_bf16, assert_fp8, rows_of, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def dev(t):
    return t.to("cuda")


@pytest.mark.parametrize("hidden", W.SILU_HIDDEN)
@pytest.mark.parametrize("tokens", [37, 1560])
def test_rmsnorm_silu_bf16(dn, tokens, hidden):
    wl = W.rmsnorm_silu(tokens, hidden)
    t = wl.tensors
    out = dn.dn_fused_rmsnorm_silu(dev(t["x"]), dev(t["w"]), 1e-6)
    r = S.fused_rmsnorm_silu(values(t["x"]), values(t["w"]), 1e-6)
    assert_bf16(out, r.s_exact, f"silu [{tokens},{hidden}]", mag=r.mag)


@pytest.mark.parametrize("hidden", W.SILU_HIDDEN)
def test_rmsnorm_silu_fp8(dn, hidden):
    wl = W.rmsnorm_silu(1560, hidden)
    t = wl.tensors
    q = dn.dn_fused_rmsnorm_silu(dev(t["x"]), dev(t["w"]), 1e-6, output_fp8=True,
                                 scale=wl.params["scale"])
    r, ref = S.fused_rmsnorm_silu_fp8(values(t["x"]), values(t["w"]), wl.params["scale"], 1e-6)
    assert q.dtype == torch.float8_e4m3fn
    assert_fp8(q, ref.q, ref.tie, f"silu e4m3 [{hidden}]")


@pytest.mark.parametrize("case", ["spiked rows", "tiny scale", "unit scale"])
def test_rmsnorm_silu_fp8_saturation(dn, case):
    """e4m3 outputs beyond +-448 saturate.  At scale 0.02, rows 0..39 carry a spike that
    normalises to ~21, past 448 after the scale, and the other rows stay inside (both
    sides of the kernel's in-range vote); at scale 5e-4 SiLU's negative lobe (down to
    -0.28 / scale) saturates on its own; at scale 1 every output is in range."""
    x = W.normal((96, 512), 71, 0)
    w = W.normal((512,), 71, 1, mean=1.0, std=0.1)
    scale = {"spiked rows": 0.02, "tiny scale": 5e-4, "unit scale": 1.0}[case]
    if case == "spiked rows":
        x[:40, 7] = 50.0
    q = dn.dn_fused_rmsnorm_silu(dev(x), dev(w), 1e-6, output_fp8=True, scale=scale)
    r, ref = S.fused_rmsnorm_silu_fp8(values(x), values(w), scale, 1e-6)
    sat = (ref.q.astype(np.int64) & 0x7F) == 0x7E
    if case == "spiked rows":
        assert sat[:40].any(axis=1).all() and not sat[40:].any()
    elif case == "tiny scale":
        assert (ref.q == 0xFE).any()
    else:
        assert not sat.any()
    assert_fp8(q, ref.q, ref.tie, f"silu e4m3 saturation ({case})")


def test_rmsnorm_silu_wide_range_and_fp32_weight(dn):
    """Weights of spread 40 push y to +-100 and beyond: the exponential of -|y| never
    overflows, tiny negative outputs round like the exact ones; FP32 weight with bias 1."""
    x = W.normal((64, 320), 70, 0)
    w = W.normal((320,), 70, 1, std=40.0)
    out = dn.dn_fused_rmsnorm_silu(dev(x), dev(w), 1e-6)
    r = S.fused_rmsnorm_silu(values(x), values(w), 1e-6)
    assert np.abs(r.y_exact).max() > 90
    assert_bf16(out, r.s_exact, "wide range", mag=r.mag)
    w32 = W.normal((320,), 70, 2, std=0.2, dtype=torch.float32)
    out = dn.dn_fused_rmsnorm_silu(dev(x), dev(w32), 1e-6, w_bias=1.0)
    r = S.fused_rmsnorm_silu(values(x), values(w32), 1e-6, bias=1.0)
    assert_bf16(out, r.s_exact, "FP32 weight + 1", mag=r.mag)


@pytest.mark.parametrize("tokens,hidden", [(399360, 128), (99840, 512), (24960, 1024)])
def test_rmsnorm_silu_full_size_sampled(dn, tokens, hidden):
    wl = W.rmsnorm_silu(tokens, hidden)
    t = wl.tensors
    out = dn.dn_fused_rmsnorm_silu(dev(t["x"]), dev(t["w"]), 1e-6)
    rows = sample_rows(tokens, 96, seed=hidden)
    r = S.fused_rmsnorm_silu(values(t["x"][torch.as_tensor(rows)]), values(t["w"]), 1e-6)
    assert_bf16(rows_of(out, rows), r.s_exact, f"silu [{tokens},{hidden}] sampled", mag=r.mag)


def test_rmsnorm_silu_empty(dn):
    out = dn.dn_fused_rmsnorm_silu(dev(torch.empty((0, 256), dtype=torch.bfloat16)),
                                   dev(torch.ones(256, dtype=torch.bfloat16)))
    assert out.shape == (0, 256)
