"""Host logic of bench.py (no GPU): the algorithmic byte counts of the measured workloads,
the one-GPU rule, and the counter summary that turns rocprofv3 FETCH_SIZE / WRITE_SIZE
rows into per-call HBM bytes."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_step_bytes_are_each_tensor_once():
    ab = bench.alg_bytes()
    t2, h2 = bench.C2
    t4, h4 = bench.C4
    # fused add: x, residual in; y, h_new out (BF16) + the BF16 weight
    assert ab["fused_add_rmsnorm"] == 4 * 2 * t2 * h2 + 2 * h2 == 268_443_648
    # + static FP8: e4m3 out instead of y, and the FP32 scale
    assert ab["fused_add_rmsnorm_quant"] == 7 * t2 * h2 + 2 * h2 + 4 == 234_889_220
    assert ab["train_forward"] == 8 * t4 * h4 + 4 * t4 + 4 * h4 == 1_073_840_128
    # backward: g, x (h_new) in, dx out (BF16); rstd, FP32 weight; FP32 dw out
    assert ab["train_backward"] == 6 * t4 * h4 + 4 * t4 + 4 * h4 + 4 * h4 == 805_437_440
    assert set(ab) == set(bench.STEP_KERNELS)
    assert set(bench.PAIR_KERNELS) == {"fused_add_rmsnorm", "train_backward"}
    # the counter summary maps dispatches: the backward's two launches share its bytes
    db = bench.step_dispatch_bytes()
    assert list(db) == bench.STEP_DISPATCHES
    assert db["train_backward_partials"] + db["train_backward_reduce"] == ab["train_backward"]
    assert db["train_backward_reduce"] == 4 * h4


def test_family_tables_cover_every_family():
    assert set(bench.FAMILY_BYTES) == {"rmsnorm", "configs", "layernorm", "qk_rope", "silu",
                                       "fixed_width"}
    cf = bench.configs_alg_bytes()
    assert cf["block_quant_16384x7168"] == 825_767_936            # 7 B/elem + scales + w
    assert cf["block_quant_normed_out_16384x7168"] == 825_767_936 + 2 * 16384 * 7168
    assert cf["ada_gated_fp8_2520x3072"] == 17 * 2520 * 3072 + 2 * 3072 + 4
    assert cf["ada_gated_fp8_broadcast_2520x3072"] == 11 * 2520 * 3072 + 8 * 3072 + 4
    qk = bench.qk_alg_bytes()
    e = 12288 * 72 * 128
    assert qk["qk_rope_neox_bf16"] == 4 * e + 2 * 48 * 128
    assert qk["qk_rope_interleaved_fp8"] == 3 * e + 2 * 48 * 128 + 8
    silu = bench.silu_alg_bytes()
    assert len(silu) == 2 * len(bench.SILU_SHAPES)
    assert silu["silu_bf16_99840x512"] == 4 * 99840 * 512 + 2 * 512
    fw = bench.fixed_alg_bytes()
    assert fw["gated_residual_next_token_gate"] == 10 * 16384 * 8192 + 4 * 8192
    ln = bench.ln_alg_bytes()
    assert ln["dit_gate_residual_layernorm_scale_shift"] == 14 * 16384 * 3072


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr


FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_counter_csv(path, counter, rounds, copy_kib, per_call):
    """Two 1 GiB copies, then `rounds` rounds of the calls (name, symbol, KiB)."""
    rows, d = [], 0
    for _ in range(2):
        d += 1
        rows.append({"Dispatch_Id": d, "Kernel_Name": "__amd_rocclr_copyBuffer",
                     "Counter_Name": counter, "Counter_Value": copy_kib})
    for r in range(rounds):
        for sym, kib in per_call:
            d += 1
            rows.append({"Dispatch_Id": d, "Kernel_Name": sym, "Counter_Name": counter,
                         "Counter_Value": kib + r})
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        w.writerows(rows[::-1])          # dispatch ids, not file order, fix the rounds


def test_counter_summary_maps_dispatches_by_round_position(tmp_path):
    """Two calls of the fixed-width family share a kernel symbol: the k-th library dispatch
    still goes to the k-th call of its round.  FETCH_SIZE here reads half the copy's bytes,
    WRITE_SIZE all of them, and the scales follow."""
    ab = bench.fixed_alg_bytes()
    names = list(ab)
    syms = ["void dn::gres_kernel<false>(x)", "void dn::gres_kernel<false>(x)",
            "void dn::gres_kernel<true>(x)", "void dn::fwd_kernel<0, 10>(x)"]
    gib_kib = float(1 << 20)
    fetch = [(s, 1000.0 * (k + 1)) for k, s in enumerate(syms)]
    write = [(s, 500.0 * (k + 1)) for k, s in enumerate(syms)]
    f, w, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _write_counter_csv(f, "FETCH_SIZE", 3, gib_kib / 2, fetch)
    _write_counter_csv(w, "WRITE_SIZE", 3, gib_kib, write)
    assert bench.summarize_counters(str(f), str(w), "fixed_width", str(out)) == 0
    d = json.loads(out.read_text())
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    for k, n in enumerate(names):
        kern = d["kernels"][n]
        assert kern["symbol"] == syms[k]
        # rounds add 0, 1, 2 KiB: the mean adds 1
        assert kern["fetch_kib"] == pytest.approx(1000.0 * (k + 1) + 1)
        assert kern["read_bytes"] == int((1000.0 * (k + 1) + 1) * 1024 * 2.0)
        assert kern["write_bytes"] == int((500.0 * (k + 1) + 1) * 1024)
        assert kern["algorithmic_bytes"] == ab[n]
    assert d["source_sha256"] == bench.kernel_source_sha256()


def test_counter_summary_rejects_partial_rounds(tmp_path):
    syms = [("void dn::a(x)", 1.0)] * 3
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_counter_csv(f, "FETCH_SIZE", 1, float(1 << 19), syms)
    _write_counter_csv(w, "WRITE_SIZE", 1, float(1 << 20), syms)
    with pytest.raises(SystemExit, match="whole rounds"):
        bench.summarize_counters(str(f), str(w), "fixed_width", str(tmp_path / "t.json"))


def test_traffic_is_withheld_once_the_sources_change(tmp_path, monkeypatch):
    path = tmp_path / "t.json"
    path.write_text(json.dumps({"source_sha256": "0" * 64,
                                "kernels": {"k": {"traffic_bytes": 5}}}))
    monkeypatch.setattr(bench, "traffic_path", lambda family="rmsnorm": str(path))
    assert bench.measured_traffic("k") is None
    path.write_text(json.dumps({"source_sha256": bench.kernel_source_sha256(),
                                "kernels": {"k": {"traffic_bytes": 5}}}))
    assert bench.measured_traffic("k") == 5


def test_kernel_resources_of_the_hot_path():
    """Registers and scratch of the library's kernels, read from the gfx950 code objects: the
    kernels of the benchmark step and of the other hot-path configurations keep their rows
    in registers without spilling to scratch memory, and every kernel declares wave64."""
    res = {r["name"]: r for r in bench.kernel_resources()}
    assert len(res) > 100
    hot = ["dn::fwd_kernel<1, 0, 128, 4, 1, 256>",      # fused_add_rmsnorm [8192,4096]
           "dn::fwd_kernel<1, 0, 256, 4, 1, 256>",      # train_forward [16384,8192]
           "dn::fwd_kernel<1, 1, 128, 4, 1, 256>",      # fused add + static FP8 [8192,4096]
           "dn::fwd_kernel<1, 1, 16, 1, 4, 256>",       # ... per head [8192,32,128]
           "dn::fwd_kernel<1, 2, 448, 2, 1, 448>",      # block FP8 [16384,7168]
           "dn::fwd_kernel<2, 4, 128, 3, 1, 256>",      # gated Ada + FP8 [2520,3072]
           "dn::fwd_kernel<0, 0, 128, 4, 1, 256>",      # rmsnorm [32,4096]
           "dn::bwd_partials_kernel<256, 4, 1, 512, false>",   # backward [16384,8192]
           "dn::bwd_reduce_kernel<256>"]
    for k in hot:
        r = res[k]
        assert r["scratch"] == 0 and r["vgpr_spill"] == 0 and r["sgpr_spill"] == 0, r
        assert r["agpr"] == 0, r


def test_committed_counters_belong_to_the_committed_sources():
    """Every committed HBM-counter summary was taken from the kernel sources in the tree (its
    fingerprint matches), so bench.py reports the measured traffic rather than withholding
    it; a kernel change without new counters fails here."""
    want = bench.kernel_source_sha256()
    families = ["rmsnorm", "configs", "layernorm", "qk_rope", "silu", "fixed_width"]
    for fam in families:
        with open(bench.traffic_path(fam)) as fh:
            d = json.load(fh)
        assert d.get("source_sha256") == want, f"{bench.traffic_path(fam)} is stale"
    assert bench.measured_traffic("train_backward") is not None
    assert bench.measured_traffic("fused_add_rmsnorm") is not None
