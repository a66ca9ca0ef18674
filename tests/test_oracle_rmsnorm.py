"""Pins of the oracle's RMSNorm family against things other than the oracle itself: torch CPU
float64 library routines (rms_norm, autograd), closed forms, invariants, central finite
differences, exactly rounded sums (math.fsum), and reductions of one operation to another."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import rmsnorm as O
from tests.parity import block_quant_ok

RNG = np.random.default_rng(7)


def bf16_values(shape, std=1.0, mean=0.0):
    return F.bf16_round(RNG.normal(mean, std, shape))


def torch_rms_norm64(x, w_eff, eps):
    """torch CPU float64 RMSNorm with the same FP32 eps (library routine)."""
    eps32 = float(np.float32(eps))
    t = torch.from_numpy(np.ascontiguousarray(x))
    return torch.nn.functional.rms_norm(t, (x.shape[-1],), weight=torch.from_numpy(w_eff),
                                        eps=eps32).numpy()


# ----------------------------------------------------------------------------- forward

@pytest.mark.parametrize("hidden", [8, 128, 3072, 4096])
@pytest.mark.parametrize("bias", [0.0, 1.0])
def test_rmsnorm_matches_torch_rms_norm(hidden, bias):
    x = bf16_values((33, hidden))
    w = bf16_values((hidden,), std=0.3, mean=0.2)
    n = O.rmsnorm(x, w, bias, 1e-6)
    ref = torch_rms_norm64(x, F.f32_round(w + bias), 1e-6)
    np.testing.assert_allclose(n.y_exact, ref, rtol=1e-13, atol=0)
    # rstd is the FP32 rounding of the reciprocal RMS torch would use.
    r = 1 / np.sqrt(np.mean(x * x, axis=1) + float(np.float32(1e-6)))
    np.testing.assert_allclose(n.r64, r, rtol=1e-14)
    assert (n.rstd == r.astype(np.float32).astype(np.float64)).all()


def test_constant_row_closed_form():
    # x_j = c, eps = 0: r = 1/|c| exactly and y_j = sign(c) * w_j exactly.
    for c in [1.0, -2.0, 0.25, 2.0 ** -20, -(2.0 ** 40)]:
        x = np.full((1, 256), c)
        w = bf16_values((256,))
        n = O.rmsnorm(x, w, 0.0, 0.0)
        assert n.rstd[0] == 1 / abs(c)
        assert (n.y == np.sign(c) * w).all()


def test_zero_row_gives_rstd_of_eps_and_zero_output():
    # Zero input (the pages' test grid): r = 1/sqrt(FP32(1e-6)) which rounds to 1000.0 in FP32.
    n = O.rmsnorm(np.zeros((3, 64)), bf16_values((64,)), 0.0, 1e-6)
    assert (n.rstd == 1000.0).all()
    assert (n.y == 0).all()


@pytest.mark.parametrize("k", [-30, -7, 1, 13, 40])
def test_power_of_two_scale_invariance_is_exact(k):
    # With eps = 0, y(2^k x) is bit-identical to y(x) and rstd scales by exactly 2^-k.
    x = bf16_values((16, 512))
    w = bf16_values((512,))
    a = O.rmsnorm(x, w, 0.0, 0.0)
    b = O.rmsnorm(x * 2.0 ** k, w, 0.0, 0.0)
    assert (a.y == b.y).all()
    assert (b.rstd == a.rstd * 2.0 ** -k).all()


@pytest.mark.parametrize("k", [-10, 10])
def test_scale_invariance_with_eps_scaled_alongside(k):
    # The pages test inputs scaled by about 1e-3 and 1e3 (norm guide §6.5).  Exactly:
    # y(2^k x, 4^k eps) is bit-identical to y(x, eps), and rstd scales by 2^-k.
    x = bf16_values((64, 1024))
    w = bf16_values((1024,))
    a = O.rmsnorm(x, w, 0.0, 1e-6)
    b = O.rmsnorm(x * 2.0 ** k, w, 0.0, float(np.float32(1e-6)) * 4.0 ** k)
    assert (a.y == b.y).all()
    assert (b.rstd == a.rstd * 2.0 ** -k).all()


def test_hidden_one_brute_force_over_every_bf16_value():
    # H = 1, eps = 0: x / sqrt(x^2) = sign(x), so y = sign(x) * w for every finite nonzero x.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = F.bf16_bits_to_f64(bits)
    x = x[np.isfinite(x) & (x != 0)].reshape(-1, 1)
    w = np.array([0.75])
    n = O.rmsnorm(x, w, 0.0, 0.0)
    assert (n.y[:, 0] == np.sign(x[:, 0]) * 0.75).all()


def test_gemma_bias_is_weight_plus_one():
    # gemma_rmsnorm = rmsnorm with (w + 1) (norm guide §2.2): checked against torch with the
    # weight w+1, and equal bitwise to the plain form given FP32(w + 1) as the weight.
    x = bf16_values((20, 768))
    w = bf16_values((768,), std=0.1)
    g = O.rmsnorm(x, w, 1.0, 1e-6)
    np.testing.assert_allclose(g.y_exact, torch_rms_norm64(x, w + 1.0, 1e-6), rtol=1e-13)
    p = O.rmsnorm(x, F.f32_round(w + 1.0), 0.0, 1e-6)
    assert (g.y == p.y).all() and (g.rstd == p.rstd).all()


def test_residual_add_matches_torch_bf16_add_and_add_then_norm():
    xt = torch.randn(64, 1024).to(torch.bfloat16)
    rt = (torch.randn(64, 1024) * 3).to(torch.bfloat16)
    xt[0, :8] = torch.tensor([1e-30, -1e30, 3.0, 0.0, -0.0, 2.0 ** -8, 1.0, 65504.0])
    rt[0, :8] = torch.tensor([1.0, 1e30, -3.0, -0.0, -0.0, 1.0, 2.0 ** -9, 1.0])
    x = xt.double().numpy()
    r = rt.double().numpy()
    w = bf16_values((1024,), mean=1.0, std=0.1)
    fa = O.fused_add_rmsnorm(x, r, w, 0.0, 1e-6)
    ref = (xt + rt).double().numpy()  # torch CPU BF16 add: FP32 sum rounded once to BF16
    assert (fa.h_new == ref).all()
    # "add, then rmsnorm": the fused result equals rmsnorm of the BF16 sum.
    assert (fa.norm.y == O.rmsnorm(ref, w, 0.0, 1e-6).y).all()


def test_static_fp8_known_codes():
    # Constant positive row, eps = 0: y_j = w_j exactly, scale 1 -> code = e4m3(w_j).
    w = np.array([1.0625, 432.0, 500.0, -1.1875, 0.5, 2.0 ** -10, 3 * 2.0 ** -10, 448.0])
    x = np.full((2, w.size), 3.0)
    n, q = O.rmsnorm_quant(x, w, 1.0, 0.0, 0.0)
    assert list(q.q[0]) == [0x38, 0x7E, 0x7E, 0xBA, 0x30, 0x00, 0x02, 0x7E]
    assert q.tie[0].tolist() == [True, True, False, True, False, True, True, False]
    # Division by the scale: scale 2 halves every value before rounding.
    _, q2 = O.rmsnorm_quant(x, w * 2, 2.0, 0.0, 0.0)
    assert (q2.q == q.q).all()


def test_static_fp8_against_torch_cast_in_range():
    x = bf16_values((32, 512))
    w = bf16_values((512,), mean=1.0, std=0.1)
    fa, q = O.fused_add_rmsnorm_quant(x, bf16_values((32, 512)), w, 0.04, 0.0, 1e-6)
    v32 = (fa.norm.y_exact / float(np.float32(0.04)))
    assert np.abs(v32).max() < 448
    ref = torch.from_numpy(v32.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    agree = F.codes_equal_e4m3(q.q, ref)
    assert (agree | q.tie).all()


# ----------------------------------------------------------------------------- 1x128 blocks

def test_block_quant_properties():
    x = bf16_values((24, 1024))
    r = bf16_values((24, 1024))
    x[3, :128] = 5.0                     # a block of one repeated value
    r[3, :128] = 0.0
    w = bf16_values((1024,), mean=1.0, std=0.1)
    w[:128] = 1.0
    b = O.fused_add_rmsnorm_fp8_block_quant(x, r, w, 0.0, 1e-6)
    vals = F.e4m3_code_to_f64(b.q)
    assert np.abs(vals).max() <= 448
    blocks = np.abs(b.normed.reshape(24, 8, 128))
    amax = blocks.max(axis=2)
    # The amax element maps to exactly +-448.
    qa = np.abs(vals.reshape(24, 8, 128))
    at_max = blocks == amax[:, :, None]
    assert (qa[at_max] == 448).all()
    assert (qa[3, 0] == 448).all()
    # The scale is the FP32 rounding of amax/448, checked with exact rationals.
    from fractions import Fraction
    for a, s in zip(amax.ravel()[:64], b.scale.ravel()[:64]):
        exact = Fraction(float(a)) / 448
        lo = np.float32(float(exact))
        cands = [np.nextafter(lo, np.float32(-1)), lo, np.nextafter(lo, np.float32(1e30))]
        best = min(cands, key=lambda c: abs(Fraction(float(c)) - exact))
        assert s == float(best)
    # Dequantised codes reproduce the BF16 normed values to FP8 precision (3 fraction bits).
    deq = O.dequantize_blocks(b.q, b.scale)
    big = np.abs(b.normed) > amax.repeat(128, axis=1) * 2.0 ** -6
    rel = np.abs(deq - b.normed)[big] / np.abs(b.normed)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-12


def test_block_quant_zero_block():
    x = np.zeros((2, 256))
    b = O.fused_add_rmsnorm_fp8_block_quant(x, np.zeros((2, 256)), np.ones(256), 0.0, 1e-6)
    assert (b.scale == 0).all() and (b.q == 0).all()


def test_block_quant_nan_elements():
    """IEEE maxNum reading: a NaN element neither sets nor hides its block's scale and is
    coded NaN.  Row 0 holds +inf (rstd 0: that element is 0 * inf = NaN, the rest 0, so
    its blocks have scale 0 and zero codes around the NaN); row 1 holds a NaN (NaN
    throughout: scale 0, NaN codes); row 2 is finite and equals its own run alone."""
    x = bf16_values((3, 256))
    x[0, 5] = np.inf
    x[1, 200] = np.nan
    w = bf16_values((256,), mean=1.0, std=0.1)
    with np.errstate(invalid="ignore", over="ignore"):
        b = O.fused_add_rmsnorm_fp8_block_quant(x, np.zeros((3, 256)), w, 0.0, 1e-6)
    nan_code = (b.q & 0x7F) == 0x7F
    assert (b.scale[:2] == 0).all()
    assert nan_code[0, 5] and not nan_code[0, np.arange(256) != 5].any()
    assert (b.q[0, np.arange(256) != 5] == 0).all()
    assert nan_code[1].all()
    alone = O.fused_add_rmsnorm_fp8_block_quant(x[2:], np.zeros((1, 256)), w, 0.0, 1e-6)
    assert (b.scale[2] == alone.scale[0]).all() and (b.q[2] == alone.q[0]).all()
    # A NaN weight column puts one NaN among numbers in every row's first block: the scale
    # is the one the same rows get with that weight set to 0 (a zero element never sets a
    # block's maximum unless every element is zero), every other code is unchanged, and
    # the NaN element is coded NaN.
    x = bf16_values((4, 256))
    w0 = w.copy()
    w0[9] = 0.0
    wn = w.copy()
    wn[9] = np.nan
    ref = O.fused_add_rmsnorm_fp8_block_quant(x, np.zeros((4, 256)), w0, 0.0, 1e-6)
    with np.errstate(invalid="ignore"):
        got = O.fused_add_rmsnorm_fp8_block_quant(x, np.zeros((4, 256)), wn, 0.0, 1e-6)
    assert (got.scale == ref.scale).all()
    others = np.arange(256) != 9
    assert (got.q[:, others] == ref.q[:, others]).all()
    assert ((got.q[:, 9] & 0x7F) == 0x7F).all()


# The gate of the block quantiser where results are not unique.  Rows of ones with eps = 0
# have rstd exactly 1, so the normalised value is exactly the FP32 weight; weights that
# sit on BF16 midpoints (1 + odd * 2^-8) make elements whose BF16 rounding an FP32 kernel
# may take either way.  Every choice of those roundings is enumerated and its result is
# computed from the definition with exact rationals (block maximum, FP32 scale by nearest
# search, e4m3 codes by nearest search over the decoded code table), independently of the
# oracle; the gate must admit each of them and nothing further than one code step.

def _e4m3_table():
    """(code, exact value) of every finite e4m3fn code, from the format definition."""
    from fractions import Fraction
    out = []
    for c in range(256):
        e, m = (c >> 3) & 0xF, c & 7
        if e == 0xF and m == 7:
            continue                                  # NaN
        mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else \
            (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        out.append((c, -mag if c & 0x80 else mag))
    return out


E4M3_TABLE = _e4m3_table()


def _e4m3_codes_exact(v):
    """Nearest e4m3fn code of an exact rational (ties to the even code, saturating at 448),
    and the codes an evaluation within 2^-21 relative of v may produce."""
    from fractions import Fraction
    v = max(min(v, Fraction(448)), Fraction(-448))
    dist = sorted((abs(val - v), c & 1, c) for c, val in E4M3_TABLE
                  if (val >= 0) == (v >= 0) or val == 0)
    best = dist[0][2]
    reach = {best}
    for lo, hi in ((v * (1 - Fraction(1, 2 ** 21)), v * (1 + Fraction(1, 2 ** 21))),):
        for w in (lo, hi):
            w = max(min(w, Fraction(448)), Fraction(-448))
            reach.add(sorted((abs(val - w), c & 1, c) for c, val in E4M3_TABLE
                             if (val >= 0) == (w >= 0) or val == 0)[0][2])
    return best, reach


def _f32_nearest(q):
    """FP32 nearest-even rounding of an exact rational, by search around float()."""
    from fractions import Fraction
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(np.array(c).view(np.uint32)) & 1))


def _enumerate_block(w_block):
    """Every (scale, codes, reachable codes) an evaluation may produce for one block of
    normalised values w_block (exact FP32 numbers), over all roundings of its BF16 ties."""
    from fractions import Fraction
    import itertools
    exact = [Fraction(float(v)) for v in w_block]
    nominal = F.bf16_round(np.asarray(w_block, dtype=np.float64))
    tied = [j for j, v in enumerate(exact) if Fraction(float(nominal[j])) != v]
    results = []
    for choice in itertools.product((0, 1), repeat=len(tied)):
        n = [Fraction(float(v)) for v in nominal]
        for j, up in zip(tied, choice):
            lo = Fraction(float(F.bf16_round(np.float64(float(exact[j]) * (1 - 2 ** -12)))))
            hi = Fraction(float(F.bf16_round(np.float64(float(exact[j]) * (1 + 2 ** -12)))))
            n[j] = hi if up else lo
        amax = max(abs(v) for v in n)
        s = _f32_nearest(amax / 448)
        codes, reach = [], []
        for v in n:
            best, r = _e4m3_codes_exact(v / Fraction(float(s))) if s > 0 else (0, {0})
            codes.append(best)
            reach.append(r)
        results.append((float(s), np.array(codes, dtype=np.uint8), reach))
    return results


def _tie_rows():
    """Rows of FP32 weights (the normalised values at x = 1, eps = 0) built on BF16
    midpoints; two blocks of 128 per row."""
    base = np.array([0.5 * (1 + (j % 96) * 2.0 ** -7) for j in range(256)])  # exact BF16
    rows = []
    def row(**at):
        r = base.copy()
        for j, v in at.items():
            r[int(j[1:])] = v
        return r
    m = lambda k: 1.0 + k * 2.0 ** -8            # k odd: a BF16 midpoint
    rows.append(row(c0=m(1), c1=1.0))            # amax 1 (nominal) or 1 + 2^-7
    rows.append(row(c0=m(3), c1=1.0))            # nominal up to 1 + 2^-6, or 1 + 2^-7
    rows.append(row(c0=m(3), c1=m(5)))           # two ties moving in opposite directions
    # a tie whose upper value equals the untied amax cannot move it: not flagged
    rows.append(row(c0=m(1), c1=1.0 + 2.0 ** -7, c130=-m(1), c131=-(1.0 + 2.0 ** -7)))
    rows.append(row(c0=-m(3), c1=m(5), c2=-m(5), c129=m(7), c130=-m(9)))
    # ties below an untied amax (block 0); a tie just below 1 above the rest (block 1)
    rows.append(row(c0=2.0, c5=m(1), c7=-m(3), c200=m(255) / 2))
    return np.array(rows)


TIE_ROW_FLAGS = [[1, 0], [1, 0], [1, 0], [0, 0], [1, 1], [0, 1]]


def _tie_refs():
    """The oracle's block-quant results of each tie row (x = 1, residual 0, eps = 0, the
    row's FP32 weights), one row per call (the weight is shared by a call's rows)."""
    w = _tie_rows()
    refs = []
    for t in range(w.shape[0]):
        x = np.ones((1, w.shape[1]))
        refs.append(O.fused_add_rmsnorm_fp8_block_quant(x, np.zeros_like(x), w[t], 0.0, 0.0))
        assert (refs[-1].normed_exact[0] == w[t]).all(), "rstd must be exactly 1 here"
    return w, refs


def test_block_quant_tie_gate_admits_every_reachable_result():
    w, refs = _tie_refs()
    rows, hidden = w.shape
    flagged = 0
    for t in range(rows):
        ref = refs[t]
        per_block = [_enumerate_block(w[t, b * 128:(b + 1) * 128]) for b in range(2)]
        scales_seen = [sorted({r[0] for r in res}) for res in per_block]
        for b in range(2):
            # The oracle flags exactly the blocks with two reachable scales and names both.
            want = {float(ref.scale[0, b]), float(ref.scale_alt[0, b])}
            assert set(scales_seen[b]) == want, (t, b, scales_seen[b], want)
            assert bool(ref.block_flag[0, b]) == (len(scales_seen[b]) == 2), (t, b)
            flagged += int(ref.block_flag[0, b])
        import itertools
        for r0, r1 in itertools.product(*per_block):
            s = np.array([[r0[0], r1[0]]])
            q = np.concatenate([r0[1], r1[1]])[None, :]
            sub = ref
            scale_ok, codes_ok = block_quant_ok(s, q, sub)
            assert scale_ok.all() and codes_ok.all(), (t, s)
            # every code an evaluation may reach, one element at a time
            for j, reach in enumerate(r0[2] + r1[2]):
                for c in reach:
                    q2 = q.copy()
                    q2[0, j] = c
                    assert block_quant_ok(s, q2, sub)[1][0, j], (t, j, c)
    assert flagged == sum(map(sum, TIE_ROW_FLAGS))
    assert [[int(f) for f in r.block_flag[0]] for r in refs] == TIE_ROW_FLAGS


def test_block_quant_tie_gate_rejects_the_rest():
    w, refs = _tie_refs()
    rows, hidden = w.shape
    # Two code steps anywhere, or one step where no reachable result has it, fail.
    for t in range(rows):
        ref = sub = refs[t]
        nominal = ref.scale
        reach = [set() for _ in range(hidden)]
        for b in range(2):
            for s_b, codes, rc in _enumerate_block(w[t, b * 128:(b + 1) * 128]):
                if s_b != nominal[0, b]:
                    continue                  # codes under the other scale: checked above
                for j in range(128):
                    reach[b * 128 + j] |= rc[j]
        for j in range(0, hidden, 5):
            ordinal = lambda c: -(c & 0x7F) if c & 0x80 else (c & 0x7F)
            code = int(ref.q[0, j])
            for step in (-2, -1, 1, 2):
                o = ordinal(code) + step
                if abs(o) > 0x7E:
                    continue
                c2 = (0x80 | -o) if o < 0 else o
                reached = c2 in reach[j]
                # the gate's e4m3 band (2^-16) is wider than what an evaluation reaches
                band = ref.fp8_tie[0, j] or (ref.bf_tie[0, j] and ref.nb_tie[0, j])
                q2 = ref.q.copy()
                q2[0, j] = c2
                ok = block_quant_ok(nominal, q2, sub)[1][0, j]
                if abs(step) == 2:
                    assert not ok, (t, j, step)
                elif not reached and not band:
                    assert not ok, (t, j, step)
                if reached:
                    assert ok, (t, j, step)
        # A scale that no rounding reaches fails, flagged block or not.
        for b in range(2):
            bad = nominal.copy()
            bad[0, b] = float(np.nextafter(np.float32(nominal[0, b]), np.float32(1e30)))
            if bad[0, b] != ref.scale_alt[0, b]:
                assert not block_quant_ok(bad, ref.q, sub)[0][0, b], (t, b)
    # Codes must follow the scale the block took: nominal codes under the other scale fail
    # where an untied element's code differs between the two.
    ref, b = refs[0], 0
    assert ref.block_flag[0, b]
    diff = (ref.q_alt[0, :128] != ref.q[0, :128]) & ~ref.fp8_tie_alt[0, :128] & \
        ~ref.fp8_tie[0, :128] & ~ref.bf_tie[0, :128]
    assert diff.any(), "the case needs an element whose code follows the scale"
    s = ref.scale.copy()
    s[0, b] = ref.scale_alt[0, b]
    assert block_quant_ok(s, ref.q_alt, ref)[1].all()
    assert not block_quant_ok(s, ref.q, ref)[1].all()


# ----------------------------------------------------------------------------- AdaRMSNorm

def test_ada_matches_torch_float64():
    rows, dim = 12, 384
    x = bf16_values((rows, dim))
    w = bf16_values((dim,), mean=1.0, std=0.1)
    style = bf16_values((rows, 3 * dim))
    a, out = O.ada_rms_norm(x, w, style, 1e-6)
    n = torch_rms_norm64(x, w, 1e-6)
    ref = n * (1 + style[:, :dim]) + style[:, dim:2 * dim]
    np.testing.assert_allclose(a.o_exact, ref, rtol=1e-12, atol=1e-14)
    assert (a.gate_out == style[:, 2 * dim:]).all()
    assert (out == F.bf16_round(a.o_exact)).all()


def test_ada_reduces_to_fused_add_quant():
    # style scale = shift = 0 and gate = 1: the gated path is fused_add_rmsnorm_quant.
    rows, dim = 16, 512
    x, r = bf16_values((rows, dim)), bf16_values((rows, dim))
    w = bf16_values((dim,), mean=1.0, std=0.1)
    style = np.zeros((rows, 3 * dim))
    style[:, 2 * dim:] = bf16_values((rows, dim))
    a, q = O.gate_residual_ada_norm_fp8(r, x, np.ones((rows, dim)), w, style, 0.04, 1e-6)
    fa, qf = O.fused_add_rmsnorm_quant(x, r, w, 0.04, 0.0, 1e-6)
    assert (a.h == fa.h_new).all()
    assert (q.q == qf.q).all()


def test_ada_broadcast_equals_repeated_style():
    rows, dim = 9, 256
    x, r, g = bf16_values((rows, dim)), bf16_values((rows, dim)), bf16_values((rows, dim))
    w = bf16_values((dim,))
    s1 = bf16_values((1, 3 * dim))
    a1, q1 = O.gate_residual_ada_norm_fp8(r, x, g, w, s1, 0.04, 1e-6)
    a2, q2 = O.gate_residual_ada_norm_fp8(r, x, g, w, np.repeat(s1, rows, 0), 0.04, 1e-6)
    assert (q1.q == q2.q).all() and (a1.gate_out == a2.gate_out).all()


def test_gated_residual_matches_torch_fp32_fma():
    # residual + x*gate: the BF16*BF16 product is exact in FP32, so torch's FP32
    # r + x*g has one rounding, like an FMA; then BF16.
    xt, gt, rt = (torch.randn(50000) * 4).to(torch.bfloat16), torch.randn(50000).to(torch.bfloat16), \
        torch.randn(50000).to(torch.bfloat16)
    ref = (rt.float() + xt.float() * gt.float()).to(torch.bfloat16).double().numpy()
    got = O.gated_residual(rt.double().numpy(), xt.double().numpy(), gt.double().numpy())
    assert (got == ref).all()


# ----------------------------------------------------------------------------- training

def _autograd64(x, w_eff, g, eps):
    xt = torch.from_numpy(x.copy()).requires_grad_(True)
    wt = torch.from_numpy(w_eff.copy()).requires_grad_(True)
    eps32 = float(np.float32(eps))
    y = xt * torch.rsqrt((xt * xt).mean(dim=1, keepdim=True) + eps32) * wt
    y.backward(torch.from_numpy(g))
    return xt.grad.numpy(), wt.grad.numpy()


@pytest.mark.parametrize("bias", [0.0, 1.0])
def test_backward_matches_torch_autograd(bias):
    rows, hidden = 40, 640
    x, g = bf16_values((rows, hidden)), bf16_values((rows, hidden))
    w = bf16_values((hidden,), std=0.02) if bias else bf16_values((hidden,), mean=1.0, std=0.1)
    w_eff = F.f32_round(w + bias)
    fwd = O.train_forward(x, w, bias, 1e-6)
    # With the unrounded r the oracle's formulas must equal autograd's gradients.
    b = O.train_backward(g, x, w, fwd.r64, bias)
    dx_ref, dw_ref = _autograd64(x, w_eff, g, 1e-6)
    np.testing.assert_allclose(b.dx_exact, dx_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b.dw_exact, dw_ref, rtol=1e-10, atol=1e-12)


def test_backward_orthogonality_invariant():
    # sum_j x_j dx_j = r * sum_j g_j w_j x_j * eps / (ms + eps): zero at eps = 0.
    x, g = bf16_values((8, 256)), bf16_values((8, 256))
    w = bf16_values((256,), mean=1.0, std=0.1)
    for eps in [0.0, 0.5]:
        eps32 = float(np.float32(eps))
        r = O.rms_reciprocal(x, eps)
        b = O.train_backward(g, x, w, r)
        lhs = np.sum(x * b.dx_exact, axis=1)
        ms = np.mean(x * x, axis=1)
        rhs = r * np.sum(g * w * x, axis=1) * eps32 / (ms + eps32)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-9)


def test_backward_central_finite_differences():
    # Brute force on tiny rows: d/dx_k of sum_j g_j y_j and d/dw_k, in FP64.
    rng = np.random.default_rng(3)
    x = rng.normal(size=(3, 6))
    w = rng.normal(size=6)
    g = rng.normal(size=(3, 6))
    eps = 0.25

    def loss(xx, ww):
        r = 1 / np.sqrt(np.mean(xx * xx, axis=1) + eps)
        return np.sum(g * xx * r[:, None] * ww[None, :])

    r = O.rms_reciprocal(x, eps)
    b = O.train_backward(g, x, w, r)
    h = 1e-6
    for t in range(3):
        for k in range(6):
            e = np.zeros_like(x)
            e[t, k] = h
            fd = (loss(x + e, w) - loss(x - e, w)) / (2 * h)
            assert abs(fd - b.dx_exact[t, k]) < 1e-7
    for k in range(6):
        e = np.zeros(6)
        e[k] = h
        fd = (loss(x, w + e) - loss(x, w - e)) / (2 * h)
        assert abs(fd - b.dw_exact[k]) < 1e-7


def test_dw_is_the_exactly_rounded_column_sum():
    rows, hidden = 200, 64
    x, g = bf16_values((rows, hidden)), bf16_values((rows, hidden))
    rstd = F.f32_round(O.rms_reciprocal(x, 1e-6))
    b = O.train_backward(g, x, np.ones(hidden), rstd)
    for j in range(hidden):
        s = math.fsum(float(g[t, j]) * float(x[t, j]) * float(rstd[t]) for t in range(rows))
        assert b.dw[j] == float(np.float32(s))


def test_backward_g_residual_adds_before_rounding():
    x, g, gr = bf16_values((5, 128)), bf16_values((5, 128)), bf16_values((5, 128))
    r = F.f32_round(O.rms_reciprocal(x, 1e-6))
    a = O.train_backward(g, x, np.ones(128), r)
    b = O.train_backward(g, x, np.ones(128), r, 0.0, gr)
    assert np.allclose(b.dx_exact, a.dx_exact + gr, rtol=0, atol=1e-12)
    assert (b.dw == a.dw).all()


def test_train_forward_residual_route_is_fused_add():
    h, u = bf16_values((10, 256)), bf16_values((10, 256))
    w = RNG.normal(0, 0.02, 256).astype(np.float32).astype(np.float64)
    t = O.train_forward(h, w, 1.0, 1e-6, residual=u)
    ref = torch_rms_norm64(F.bf16_round(h + u), F.f32_round(1.0 + w), 1e-6)
    np.testing.assert_allclose(t.y_exact, ref, rtol=1e-13)
    assert (t.h_new == F.bf16_round(h + u)).all()


def _dx_fp32_model(g, x, w_eff, r, coef_error: float = 0.0, r_cubed: bool = False):
    """dx as an FP32 kernel evaluates it (lane partials of g*w*x over 32 terms, the row sum
    in FP64, k = FP32(r^2*c), dx = FP32(FMA(-x, k, g*w) * r)), rounded to BF16; coef_error
    perturbs the coupled coefficient.  r_cubed evaluates the other order, coef = FP32(r^3*c)
    and dx = FMA(-x, coef, (g*w)*r), whose coefficient leaves FP32's range for rows whose
    scale is far from 1."""
    f32 = np.float32
    H = x.shape[1]
    gw = (g.astype(f32) * w_eff.astype(f32)).astype(f32)
    out = np.empty_like(x)
    for t in range(x.shape[0]):
        lanes = [f32(0)] * (H // 32)
        for k in range(32):
            for ln in range(H // 32):
                j = ln + k * (H // 32)
                lanes[ln] = f32(float(gw[t, j]) * float(x[t, j]) + float(lanes[ln]))
        c = sum(float(v) for v in lanes) / H
        with np.errstate(over="ignore", under="ignore", invalid="ignore"):
            if r_cubed:
                coef = f32(float(r[t]) ** 3 * c * (1.0 + coef_error))
                first = f32(gw[t] * f32(r[t]))
                out[t] = (-x[t] * float(coef) + first.astype(np.float64)).astype(f32)
            else:
                k2 = f32(float(r[t]) ** 2 * c * (1.0 + coef_error))
                inner = (-x[t] * float(k2) + gw[t].astype(np.float64)).astype(f32)
                out[t] = (inner * f32(r[t])).astype(f32)
    return F.bf16_round(out)


def test_dx_gate_admits_fp32_evaluation_and_rejects_a_wrong_coefficient():
    """The per-element dx gate of the GPU tests: an FP32 evaluation of the formula passes;
    the same evaluation with the coupled term's coefficient off by 0.1 % does not."""
    from tests.parity import assert_dx
    g = bf16_values((6, 1024))
    x = bf16_values((6, 1024))
    w = bf16_values((1024,), mean=1.0, std=0.1)
    r = F.f32_round(1.0 / np.sqrt(np.mean(x * x, axis=1) + 1e-6))
    ref = O.train_backward(g, x, w, r, 0.0)
    to_t = lambda v: torch.from_numpy(F.f64_to_bf16_bits(v).view(np.int16)).view(torch.bfloat16)
    assert_dx(to_t(_dx_fp32_model(g, x, w, r)), ref, "fp32 model")
    with pytest.raises(AssertionError, match="per-element"):
        assert_dx(to_t(_dx_fp32_model(g, x, w, r, 1e-3)), ref, "perturbed model")


def test_dx_gate_sees_the_coupled_coefficient_leave_fp32():
    """Rows of RMS ~1e17 with gradients ~1e-13 (and the mirror case, RMS ~1e-17 with
    gradients ~1e12): dx is an ordinary FP32 number, but r^3*c underflows (overflows) FP32.
    The kernel's order, r*(g*w - x*(r^2*c)), passes the dx gate; the r^3 order fails it."""
    from tests.parity import assert_dx
    to_t = lambda v: torch.from_numpy(F.f64_to_bf16_bits(v).view(np.int16)).view(torch.bfloat16)
    w = bf16_values((1024,), mean=1.0, std=0.1)
    for sx, sg in ((1e17, 1e-13), (1e-17, 1e12)):
        x = F.bf16_round(bf16_values((4, 1024)) * sx)
        g = F.bf16_round(bf16_values((4, 1024)) * sg)
        r = F.f32_round(1.0 / np.sqrt(np.mean(x * x, axis=1)))
        ref = O.train_backward(g, x, w, r, 0.0)
        assert np.isfinite(ref.dx_exact).all() and (np.abs(ref.dx_exact) > 1e-37).mean() > 0.9
        assert_dx(to_t(_dx_fp32_model(g, x, w, r)), ref, f"kernel order at {sx:g}")
        with pytest.raises(AssertionError):
            assert_dx(to_t(_dx_fp32_model(g, x, w, r, r_cubed=True)), ref, f"r^3 order at {sx:g}")
