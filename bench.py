#!/usr/bin/env python3
"""Throughput of the RMSNorm family's hot path on one MI355X, as achieved HBM GB/s.

The metric is the pair the target names: the fused_add_rmsnorm forward and the training
backward.  One timed round is
  1. fused_add_rmsnorm forward, in place, x/residual BF16 [8192, 4096]      (plain BF16 y)
  2. training backward, BF16 [16384, 8192]: dx and the deterministic FP32 dw, in one call
     (two launches: the producers, then the fixed-order reduction), on the h_new and rstd
     of a training forward with residual (FP32 w = 1 + w0) run once before anything is
     timed
and `value` = algorithmic bytes of a round / wall time of a round (K rounds between device
synchronisations; inputs resident in HBM).  The two shapes alternate, so each kernel's
inputs have been pushed out of the 256 MB Infinity Cache by the other's traffic.  K is 200
by default: the first round after a synchronisation waits ~0.1 ms for the queue to start,
which K = 20 would spread as ~5 us over every round (measured: 194.0, 188.2 and 185.3 us
per round at K = 20, 100 and 400, without events).

`whole_step` times the whole hot-path step the same way: the pair plus the training
forward with residual [16384, 8192] and the fused add + static FP8 forward [8192, 4096]
(scale 0.04), in the order fused add, training forward, fused add + FP8, backward.

Algorithmic bytes count each tensor the definition reads or writes once; the backward's
FP64 chunk rows in the workspace are not counted.  Inside the timed region only the
dominant kernel (the backward, the roofline's kernel) is bracketed by HIP events (created
without the system-scope fence, see HipTimingEvent) on the kernels' stream, in every fourth
round (50 of the default 200 launches are timed live); the per-kernel
tables come from K more rounds with an event between every two kernels (each record still
costs the stream about a microsecond, which the tables' durations include).
`cpu_baseline` times the FP64 numpy oracle on a bounded sample of the same workload on
this host's cores.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-cpu-baseline]

Profiler runs pass --step-only (no copy ceiling, no shard shape), so that every library
dispatch belongs to the step.  Profiler summaries (host only, no GPU):
    python bench.py --summarize-counters FETCH.csv WRITE.csv   # rocprofv3 --pmc outputs of a
        bench run with --copy-calibration: writes profiles/hbm_traffic.json, prints a table
    python bench.py --summarize-trace STATS.csv                # rocprofv3 --stats output

`--family layernorm` times the LayerNorm family instead (one line, per-kernel GB/s):
layernorm and layernorm_quant on BF16 [8192, 4096], and the three DiT gate/residual +
LayerNorm modes on BF16 [16384, 3072] with gate/scale/shift read as row-stride-6*hidden
chunks of one per-token modulation tensor.  `--family qk_rope` times the fused QK
RMSNorm + 3-D RoPE + V copy on qkv BF16 [12288, 9216] (both pairings, BF16 and e4m3fn);
`--family silu` the fused RMSNorm + SiLU at three video-VAE shapes; `--family fixed_width`
the gated-residual RMSNorm (+ next) at hidden 8192 and the per-head sigmoid-gate norm.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s and % of peak, fused_add_rmsnorm fwd + train bwd"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak (8 TB/s)
C2 = (8192, 4096)
C4 = (16384, 8192)


def alg_bytes():
    """Algorithmic HBM bytes per launch (each tensor of the definition once)."""
    t2, h2 = C2
    t4, h4 = C4
    e2, e4 = t2 * h2, t4 * h4
    return {
        # read x, residual; write h_new (into residual) and y (into x); bf16 weight
        "fused_add_rmsnorm": 8 * e2 + 2 * h2,
        # read x, residual; write h_new and FP8 out; bf16 weight; scale
        "fused_add_rmsnorm_quant": 7 * e2 + 2 * h2 + 4,
        # read h, residual; write y, h_new; FP32 rstd out; FP32 weight
        "train_forward": 8 * e4 + 4 * t4 + 4 * h4,
        # read g, x (h_new), rstd, FP32 weight; write dx and FP32 dw (the FP64 chunk rows it
        # passes through the workspace are not algorithmic)
        "train_backward": 6 * e4 + 4 * t4 + 4 * h4 + 4 * h4,
    }


def kernel_source_sha256() -> str:
    """Fingerprint of the library's kernel sources (every file of dit_normalization_amd/csrc)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "dit_normalization_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_path(family: str = "rmsnorm") -> str:
    """The committed counter summary of a bench family (the step's is hbm_traffic.json)."""
    name = "hbm_traffic.json" if family == "rmsnorm" else f"{family}_family_hbm_traffic.json"
    return os.path.join(ROOT, "profiles", name)


def measured_traffic(kernel: str, family: str = "rmsnorm"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE / WRITE_SIZE scaled by a plain copy), or None when the kernel sources have
    changed since the counters were taken."""
    path = traffic_path(family)
    try:
        with open(path) as fh:
            d = json.load(fh)
    except OSError:
        return None
    if d.get("source_sha256") != kernel_source_sha256():
        return None
    ks = d.get("kernels", {})
    if kernel not in ks and kernel == "train_backward":
        parts = [ks.get(n) for n in ("train_backward_partials", "train_backward_reduce")]
        return None if None in parts else sum(k["traffic_bytes"] for k in parts)
    k = ks.get(kernel)
    return None if k is None else k["traffic_bytes"]


# The roofline kernel's live events bracket its launch in every LIVE_EVERY-th timed round.
LIVE_EVERY = 4

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence (hip_runtime_api.h)
_EVENT_KIND = {"kind": None}


class HipTimingEvent:
    """A HIP event created with hipEventDisableSystemFence, recorded on a torch stream.

    torch.cuda.Event records with a system-scope fence, whose cache write-back costs the
    stream ~3 us per record (measured on MI355X: a bench step with an event between every
    two kernels takes 430 us with torch's events, 418 us with these, 410 us with none).
    Without that fence the record only timestamps the stream, which is all a timing event
    needs.  The runtime is the one torch loaded (same soname), so torch's streams are valid
    handles for it."""
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self, torch):
        import ctypes
        self._torch = torch
        self._ev = ctypes.c_void_p()
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(self._ev),
                                                     HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream=None):
        import ctypes
        st = stream if stream is not None else self._torch.cuda.current_stream()
        rc = self._hip.hipEventRecord(self._ev, ctypes.c_void_p(st.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def synchronize(self):
        rc = self._hip.hipEventSynchronize(self._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({rc})")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        import ctypes
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        try:
            if self._ev:
                self._hip.hipEventDestroy(self._ev)
        except Exception:
            pass


def timing_event(torch):
    """A timing event on torch's streams: HipTimingEvent, or torch.cuda.Event where the HIP
    runtime cannot be reached through ctypes (the kind used is reported in the JSON line)."""
    if _EVENT_KIND["kind"] != "torch":
        try:
            ev = HipTimingEvent(torch)
            _EVENT_KIND["kind"] = "hipEventDisableSystemFence"
            return ev
        except (OSError, AttributeError, RuntimeError):
            _EVENT_KIND["kind"] = "torch"
    return torch.cuda.Event(enable_timing=True)


STEP_KERNELS = ["fused_add_rmsnorm", "train_forward", "fused_add_rmsnorm_quant",
                "train_backward"]
# The library dispatches of a step: the backward is two launches (dx and the FP64 chunk
# rows, then the fixed-order dw reduction).
STEP_DISPATCHES = ["fused_add_rmsnorm", "train_forward", "fused_add_rmsnorm_quant",
                   "train_backward_partials", "train_backward_reduce"]


def step_dispatch_bytes():
    """Algorithmic bytes per library dispatch of a step (the backward split into its two
    launches: the reduction's algorithmic bytes are dw's; the chunk rows it reads are
    workspace traffic)."""
    ab = alg_bytes()
    dw = 4 * C4[1]
    out = {n: ab[n] for n in STEP_DISPATCHES[:3]}
    out["train_backward_partials"] = ab["train_backward"] - dw
    out["train_backward_reduce"] = dw
    return out
# The metric's pair: the fused add forward and the training backward.
PAIR_KERNELS = ["fused_add_rmsnorm", "train_backward"]
GIB_KIB = float(1 << 20)


def _read_csv(path):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _library_dispatches(rows, names):
    """Map every library dispatch of a counter run to a call name.  A bench round launches
    the calls in `names` order, so the k-th library dispatch (by dispatch id) belongs to
    names[k % len(names)]; each name must always dispatch the same kernel symbol.  Returns
    {name: (symbol, [rows])}."""
    lib = [r for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
           if r["Kernel_Name"].startswith("void dn::")]
    if not lib or len(lib) % len(names):
        raise SystemExit(f"{len(lib)} library dispatches are not whole rounds of {names}")
    out = {}
    for k, r in enumerate(lib):
        n = names[k % len(names)]
        sym, rs = out.setdefault(n, (r["Kernel_Name"], []))
        if sym != r["Kernel_Name"]:
            raise SystemExit(f"{n} dispatched both {sym} and {r['Kernel_Name']}")
        rs.append(r)
    return out


def _counter(rows, name, names):
    """Per-call mean of one counter (KiB per dispatch), the symbol of each call, and the
    copy calibration scale: bytes per KiB reported, from the 1 GiB device copies (the
    copy dispatches above a quarter of a GiB)."""
    rows = [r for r in rows if r["Counter_Name"] == name]
    copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]
              and float(r["Counter_Value"]) > GIB_KIB / 4]
    if not copies:
        raise SystemExit(f"no 1 GiB calibration copy in the {name} run (use --copy-calibration)")
    scale = GIB_KIB / (sum(copies) / len(copies))
    per = _library_dispatches(rows, names)
    mean = {n: sum(float(r["Counter_Value"]) for r in rs) / len(rs) for n, (_, rs) in per.items()}
    return mean, {n: sym for n, (sym, _) in per.items()}, scale, len(copies)


def summarize_counters(fetch_csv: str, write_csv: str, family: str = "rmsnorm",
                       out_path: str | None = None) -> int:
    """Per-kernel HBM traffic from the two counter runs of one bench family; the result also
    goes to `out_path` (default: the family's file under profiles/, traffic_path), which
    bench.py reads for `traffic`."""
    fr, wr = _read_csv(fetch_csv), _read_csv(write_csv)
    ab = step_dispatch_bytes() if family == "rmsnorm" else FAMILY_BYTES[family]()
    names = list(ab)   # dispatch order
    fetch, sym, fscale, nf = _counter(fr, "FETCH_SIZE", names)
    write, wsym, wscale, nw = _counter(wr, "WRITE_SIZE", names)
    if wsym != sym:
        raise SystemExit("the two counter runs dispatched different kernels")
    out = {"source_sha256": kernel_source_sha256(), "fetch_scale": fscale, "write_scale": wscale,
           "calibration": f"{nf} and {nw} device copies of 1 GiB", "kernels": {}}
    print("| kernel | symbol | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled traffic MiB | "
          "algorithmic MiB | ratio |")
    print("|---|---|---|---|---|---|---|")
    for k in names:
        s_ = sym[k]
        rb = fetch[k] * 1024 * fscale
        wb = write[k] * 1024 * wscale
        t = rb + wb
        out["kernels"][k] = {"symbol": s_, "fetch_kib": round(fetch[k], 1),
                             "write_kib": round(write[k], 1), "read_bytes": int(rb),
                             "write_bytes": int(wb), "traffic_bytes": int(t),
                             "algorithmic_bytes": ab[k],
                             "traffic_over_algorithmic": round(t / ab[k], 4)}
        short = s_.replace("void ", "").split("(")[0]
        ratio = f"{t / ab[k]:.3f}" if ab[k] > 1 << 20 else "(workspace)"
        print(f"| {k} | `{short}` | {fetch[k]:,.1f} | {write[k]:,.1f} | {t / 2**20:,.1f} | "
              f"{ab[k] / 2**20:,.1f} | {ratio} |")
    print(f"\nscales: FETCH_SIZE x{fscale:.4f}, WRITE_SIZE x{wscale:.4f}")
    path = out_path or traffic_path(family)
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(f"wrote {path}")
    return 0


def kernel_resources(lib_path: str | None = None):
    """Register, scratch and LDS figures of every kernel in libdnorm.so, from the AMDGPU
    metadata notes of its gfx950 code objects (one per compile unit in the .hip_fatbin
    section; extracted with the ROCm LLVM tools).  Returns a list of dicts with the
    demangled name and: vgpr, agpr, sgpr, scratch bytes per lane (private segment),
    vgpr/sgpr spill counts, static LDS bytes, the largest block size, and the waves one
    SIMD can hold by registers (512 VGPRs per lane, allocated in groups of 8, at most 8)."""
    import re
    import shutil
    import subprocess
    import tempfile

    import yaml
    llvm = "/opt/rocm/llvm/bin"
    so = lib_path or os.path.join(ROOT, "dit_normalization_amd", "libdnorm.so")
    kernels = []
    with tempfile.TemporaryDirectory() as d:
        fb = os.path.join(d, "fatbin")
        subprocess.run([f"{llvm}/llvm-objcopy", "--dump-section", f".hip_fatbin={fb}", so,
                        os.path.join(d, "stripped")], check=True, capture_output=True)
        data = open(fb, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(b"__CLANG_OFFLOAD_BUNDLE__"), data)]
        for i, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
            part, co = os.path.join(d, f"{i}.bundle"), os.path.join(d, f"{i}.co")
            with open(part, "wb") as fh:
                fh.write(data[a:b])
            subprocess.run([f"{llvm}/clang-offload-bundler", "--unbundle", "--type=o",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={part}",
                            f"--output={co}"], check=True, capture_output=True)
            notes = subprocess.run([f"{llvm}/llvm-readelf", "--notes", co], check=True,
                                   capture_output=True, text=True).stdout
            doc = notes[notes.index("---"):]
            doc = doc[:doc.index("\n...")] if "\n..." in doc else doc
            kernels += yaml.safe_load(doc)["amdhsa.kernels"]
    names = [k[".name"] for k in kernels]
    if shutil.which("c++filt"):
        names = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True,
                               text=True, check=True).stdout.split("\n")[:len(kernels)]
    out = []
    for n, k in zip(names, kernels):
        regs = k[".vgpr_count"] + k.get(".agpr_count", 0)
        alloc = max(8, (regs + 7) // 8 * 8)
        out.append({"name": n.replace("void ", "").split("(")[0], "vgpr": k[".vgpr_count"],
                    "agpr": k.get(".agpr_count", 0), "sgpr": k[".sgpr_count"],
                    "scratch": k[".private_segment_fixed_size"],
                    "vgpr_spill": k.get(".vgpr_spill_count", 0),
                    "sgpr_spill": k.get(".sgpr_spill_count", 0),
                    "lds_static": k[".group_segment_fixed_size"],
                    "max_block": k[".max_flat_workgroup_size"],
                    "waves_per_simd": min(8, 512 // alloc)})
    return out


def print_kernel_resources(match: str = "") -> int:
    rows = [r for r in kernel_resources() if match in r["name"]]
    print("| kernel | VGPR | AGPR | SGPR | scratch B/lane | spills (V/S) | static LDS B | "
          "block | waves/SIMD by registers |")
    print("|---|---|---|---|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: r["name"]):
        print(f"| `{r['name']}` | {r['vgpr']} | {r['agpr']} | {r['sgpr']} | {r['scratch']} | "
              f"{r['vgpr_spill']}/{r['sgpr_spill']} | {r['lds_static']} | {r['max_block']} | "
              f"{r['waves_per_simd']} |")
    return 0


def summarize_sq(lds_csv: str, occ_csv: str, family: str = "rmsnorm", cus: int = 256,
                 xcds: int = 8) -> int:
    """Per-call LDS and occupancy figures from two rocprofv3 --pmc runs of one bench family
    (SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE, SQ_INSTS_LDS, GRBM_GUI_ACTIVE; SQ_WAVE_CYCLES,
    SQ_WAVES, SQ_BUSY_CYCLES, GRBM_GUI_ACTIVE), next to the registers of each kernel from the
    code objects.  Bank conflicts per LDS access = conflict cycles / (active cycles -
    conflict cycles) (rocprofv3's LdsBankConflict); mean waves per CU = 4 * SQ_WAVE_CYCLES /
    (GRBM_GUI_ACTIVE / xcds * cus) (rocprofv3's OccupancyPercent * 32 / 100; the CSV sums
    GRBM_GUI_ACTIVE over the XCDs)."""
    names = STEP_DISPATCHES if family == "rmsnorm" else list(FAMILY_BYTES[family]())

    def per_call(path):
        rows = _read_csv(path)
        counters = sorted({r["Counter_Name"] for r in rows})
        out, sym = {}, {}
        for c in counters:
            per = _library_dispatches([r for r in rows if r["Counter_Name"] == c], names)
            for n, (sy, rs) in per.items():
                out.setdefault(n, {})[c] = sum(float(r["Counter_Value"]) for r in rs) / len(rs)
                sym[n] = sy
        return out, sym

    lds, sym = per_call(lds_csv)
    occ, sym2 = per_call(occ_csv)
    if sym != sym2:
        raise SystemExit("the two counter runs dispatched different kernels")
    res = {r["name"]: r for r in kernel_resources()}
    print("| call | kernel | VGPR | SGPR | scratch B | waves/SIMD by registers | mean waves "
          "per CU | LDS instructions | LDS bank conflicts per access | LDS busy |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for n in names:
        short = sym[n].replace("void ", "").split("(")[0]
        r = res.get(short, {})
        lm, om = lds[n], occ[n]
        grbm = lm["GRBM_GUI_ACTIVE"] / xcds
        act, conf = lm["SQ_LDS_IDX_ACTIVE"], lm["SQ_LDS_BANK_CONFLICT"]
        ratio = conf / (act - conf) if act > conf else 0.0
        waves = 4 * om["SQ_WAVE_CYCLES"] / (om["GRBM_GUI_ACTIVE"] / xcds * cus)
        print(f"| {n} | `{short}` | {r.get('vgpr', '?')} | {r.get('sgpr', '?')} | "
              f"{r.get('scratch', '?')} | {r.get('waves_per_simd', '?')} | {waves:.2f} | "
              f"{lm['SQ_INSTS_LDS']:,.0f} | {ratio:.4f} | {act / (grbm * cus):.2%} |")
    return 0


def summarize_trace(stats_csv: str) -> int:
    rows = _read_csv(stats_csv)
    print("| kernel | calls | average ns | min ns | max ns | share |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        name = r["Name"].replace("void ", "").split("(")[0]
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']):,.0f} | "
              f"{int(float(r['MinNs'])):,} | {int(float(r['MaxNs'])):,} | "
              f"{float(r['Percentage']):.2f} % |")
    return 0


def host_cores() -> int:
    """Host threads the CPU baseline uses: the CPUs this process may run on, at most 16 (one
    GPU's share of an 8-GPU node's host cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _oracle_rate(run, bytes_per_pass: int, seconds: float, what: str):
    """Time the oracle: `run` (one pass over a bounded sample of `bytes_per_pass` algorithmic
    bytes) repeated for about `seconds` on every host core (one thread per core, each
    looping the same pass; the oracle's numpy arithmetic releases the interpreter lock),
    after a quarter as long on one core.  The cpu_baseline object of a bench line."""
    from concurrent.futures import ThreadPoolExecutor

    def loop(sec):
        done, t0 = 0, time.perf_counter()
        while True:
            run()
            done += 1
            if time.perf_counter() - t0 >= sec:
                return done

    t0 = time.perf_counter()
    one = loop(seconds / 4)
    single = bytes_per_pass * one / (time.perf_counter() - t0) / 1e9
    cores = host_cores()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        done = sum(ex.map(loop, [seconds] * cores))
    el = time.perf_counter() - t0
    return {"value": round(bytes_per_pass * done / el / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "single_core_value": round(single, 4),
            "sample": f"{done} passes of {what} on {cores} threads in {el:.1f} s (numpy FP64; "
                      f"{one} passes on one thread first)"}


def cpu_baseline(seconds: float = 10.0):
    """The oracle, as it stands, on a bounded sample of the same workload as `value`: row
    blocks of the fused-add forward [*, 4096] and of the training backward [*, 8192] (on
    the h_new and rstd of the oracle's training forward, computed once before the timing,
    as the GPU pair's backward reads a forward run once before its timing), repeated for
    about `seconds` on every host core."""
    import workloads as W
    from oracle import rmsnorm as O

    fa = W.fused_add_quant(rows=256)
    tr = W.train(rows=128)
    x, r, w = (_vals(fa.tensors[k]) for k in ("x", "residual", "w"))
    h, u, w4, g = (_vals(tr.tensors[k]) for k in ("h", "residual", "w", "g"))
    tf = O.train_forward(h, w4, 1.0, 1e-6, residual=u)
    b2 = 256 * C2[1]
    b4 = 128 * C4[1]
    per_pass = (8 * b2 + 2 * C2[1]) + (6 * b4 + 4 * 128 + 8 * C4[1])

    def run():
        O.fused_add_rmsnorm(x, r, w, 0.0, 1e-6)
        O.train_backward(g, tf.h_new, w4, tf.rstd, 1.0)

    return _oracle_rate(run, per_pass, seconds,
                        "fused add + RMSNorm on 256 rows x 4096 and the training backward on "
                        "128 rows x 8192")


LN = (8192, 4096)
DIT = (16384, 3072)


def ln_alg_bytes():
    """Algorithmic HBM bytes per launch of the LayerNorm family, in dispatch order (the
    [8192,4096] and [16384,3072] shapes alternate, so no kernel finds its inputs in the
    Infinity Cache)."""
    tl, hl = LN
    td, hd = DIT
    el, ed = tl * hl, td * hd
    return {
        # read x; write y; FP32 gamma and beta
        "layernorm": 4 * el + 8 * hl,
        # read x, residual, gate; write residual_out, norm_out; gamma, beta
        "dit_gate_residual_layernorm_gamma_beta": 10 * ed + 8 * hd,
        # read x; write FP8 out; gamma, beta, scale
        "layernorm_quant": 3 * el + 8 * hl + 4,
        # read x, residual, gate, scale, shift; write residual_out, norm_out
        "dit_gate_residual_layernorm_scale_shift": 14 * ed,
        # read x, residual, scale, shift; write residual_out, norm_out
        "dit_residual_layernorm_scale_shift": 12 * ed,
    }


# Fused QK RMSNorm + 3-D RoPE: a 16 x 24 x 32 patch grid, 24 + 24 + 24 heads of 128.
QK = {"tokens": 16 * 24 * 32, "nq": 24, "nk": 24, "nv": 24, "head_dim": 128}
SILU_SHAPES = ((399360, 128), (99840, 512), (24960, 1024))
GRES = (16384, 8192)
SIGMOID = (16384, 64, 64)     # tokens, heads, head dim


def qk_alg_bytes():
    """Per launch, in dispatch order: read qkv; write q, k, v (BF16, or e4m3fn plus the two
    scales); the two BF16 norm weights."""
    e = QK["tokens"] * (QK["nq"] + QK["nk"] + QK["nv"]) * QK["head_dim"]
    wb = 2 * (QK["nq"] + QK["nk"]) * QK["head_dim"]
    return {"qk_rope_interleaved_bf16": 4 * e + wb, "qk_rope_neox_bf16": 4 * e + wb,
            "qk_rope_interleaved_fp8": 3 * e + wb + 8, "qk_rope_neox_fp8": 3 * e + wb + 8}


def silu_alg_bytes():
    """Per launch, in dispatch order: read x; write y (BF16) or q (e4m3fn, plus the scale);
    the BF16 weight."""
    ab = {}
    for T, H in SILU_SHAPES:
        ab[f"silu_bf16_{T}x{H}"] = 4 * T * H + 2 * H
        ab[f"silu_fp8_{T}x{H}"] = 3 * T * H + 2 * H + 4
    return ab


def fixed_alg_bytes():
    """Per launch, in dispatch order.  Gated residual: read branch, residual and the gate
    (per token, or one shared row), write residual; + next: also write the next norm's
    output and read its weight.  Sigmoid gate: read x and gate, write x."""
    T, H = GRES
    e = T * H
    es = SIGMOID[0] * SIGMOID[1] * SIGMOID[2]
    return {"gated_residual_token_gate": 8 * e + 2 * H,
            "gated_residual_shared_gate": 6 * e + 4 * H,
            "gated_residual_next_token_gate": 10 * e + 4 * H,
            "rmsnorm_sigmoid_gate": 6 * es + 2 * SIGMOID[2]}


C3 = (16384, 7168)
C5 = (2520, 3072)


def configs_alg_bytes():
    """Algorithmic HBM bytes per launch of the other hot-path configurations, in dispatch
    order (large and small shapes alternate, so no launch finds its inputs in the Infinity
    Cache)."""
    t3, h3 = C3
    t5, d5 = C5
    t2, h2 = C2
    e3, e5, e2 = t3 * h3, t5 * d5, t2 * h2
    bq = 7 * e3 + 4 * t3 * (h3 // 128) + 2 * h3
    # read x, residual, gate and the style rows' three chunks; write residual, e4m3 out and
    # gate_out (each tensor of the definition once)
    ada = (2 + 2 + 2 + 2 + 1 + 2) * e5 + 2 * d5 + 4
    return {
        # read x, residual; write h_new, e4m3 out, FP32 scales (MN-major); BF16 weight
        "block_quant_16384x7168": bq,
        "ada_gated_fp8_2520x3072": ada + 6 * e5,
        # ... and normed_out
        "block_quant_normed_out_16384x7168": bq + 2 * e3,
        "ada_gated_fp8_broadcast_2520x3072": ada + 6 * d5,
        # read x, residual; write h_new, e4m3 out; weight [128]
        "fused_add_quant_per_head_8192x32x128": 7 * e2 + 2 * 128 + 4,
        "fused_add_quant_gemma_8192x4096": 7 * e2 + 2 * h2 + 4,
    }


def run_configs_family(a) -> int:
    """The other configurations of the hot path, back to back: 1x128 block FP8
    [16384,7168] (with and without normed_out), the gated AdaRMSNorm + FP8 [2520,3072] with
    per-row and broadcast style, and the fused add + static FP8 per head [8192,32,128] and
    with the Gemma offset [8192,4096]."""
    import torch

    import workloads as W
    from dit_normalization_amd import dnorm as dn
    from oracle import rmsnorm as O

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] generating the configurations' inputs", file=sys.stderr, flush=True)
    scale = torch.tensor([0.04], dtype=torch.float32, device=dev)
    c3 = W.block_quant()
    x3, r3, w3 = (c3.tensors[k].to(dev) for k in ("x", "residual", "w"))
    t3, h3 = C3
    q3 = torch.empty(C3, dtype=torch.float8_e4m3fn, device=dev)
    s3 = torch.empty((h3 // 128, (t3 + 3) // 4 * 4), dtype=torch.float32, device=dev)
    n3 = torch.empty_like(x3)
    ada = {}
    for bc in (False, True):
        c5 = W.ada(broadcast=bc)
        t = {k: c5.tensors[k].to(dev) for k in ("x", "residual", "gate", "w", "style")}
        t["q"] = torch.empty(C5, dtype=torch.float8_e4m3fn, device=dev)
        t["go"] = torch.empty(C5, dtype=torch.bfloat16, device=dev)
        ada[bc] = t
    c2h = W.fused_add_quant(8192, 128, heads=32)
    x2h, r2h, w2h = (c2h.tensors[k].to(dev) for k in ("x", "residual", "w"))
    q2h = torch.empty(x2h.shape, dtype=torch.float8_e4m3fn, device=dev)
    c2 = W.fused_add_quant()
    x2, r2 = c2.tensors["x"].to(dev), c2.tensors["residual"].to(dev)
    wg = W.normal((C2[1],), 2, 7, std=0.1).to(dev)
    q2 = torch.empty(C2, dtype=torch.float8_e4m3fn, device=dev)

    def ada_call(bc):
        t = ada[bc]
        return lambda: dn.dn_gate_residual_ada_norm_fp8(t["residual"], t["x"], t["gate"], t["w"],
                                                        t["style"], scale, 1e-6, out=t["q"],
                                                        gate_out=t["go"])

    calls = {
        "block_quant_16384x7168": lambda: dn.dn_fused_add_rmsnorm_fp8_block_quant(
            x3, r3, w3, 1e-6, out=q3, block_scale=s3),
        "ada_gated_fp8_2520x3072": ada_call(False),
        "block_quant_normed_out_16384x7168": lambda: dn.dn_fused_add_rmsnorm_fp8_block_quant(
            x3, r3, w3, 1e-6, out=q3, block_scale=s3, normed_out=n3),
        "ada_gated_fp8_broadcast_2520x3072": ada_call(True),
        "fused_add_quant_per_head_8192x32x128": lambda: dn.dn_fused_add_rmsnorm_quant(
            x2h, r2h, w2h, scale, 1e-6, out=q2h),
        "fused_add_quant_gemma_8192x4096": lambda: dn.dn_fused_add_rmsnorm_quant(
            x2, r2, wg, scale, 1e-6, w_bias=1.0, out=q2),
    }

    def cpu():
        b = W.block_quant(rows=64)
        xb, rb, wb = (_vals(b.tensors[k]) for k in ("x", "residual", "w"))
        c5 = W.ada(rows=64)
        d = {k: _vals(c5.tensors[k]) for k in ("x", "residual", "gate", "w", "style")}
        per = 7 * 64 * h3 + 17 * 64 * C5[1]

        def run():
            O.fused_add_rmsnorm_fp8_block_quant(xb, rb, wb, 0.0, 1e-6)
            O.gate_residual_ada_norm_fp8(d["residual"], d["x"], d["gate"], d["w"], d["style"],
                                         0.04, 1e-6)
        return _oracle_rate(run, per, a.cpu_seconds / 2,
                            "block FP8 on 64 rows x 7168 and the gated AdaRMSNorm + FP8 on 64 "
                            "rows x 3072")

    return time_family(a, torch, dev, calls, "achieved HBM GB/s, the other hot-path "
                       "configurations", "block FP8 [16384,7168] (+normed_out), gated "
                       "AdaRMSNorm + FP8 [2520,3072] per-row and broadcast style, fused add + "
                       "static FP8 per head [8192,32,128] and Gemma [8192,4096]", cpu)


FAMILY_BYTES = {"rmsnorm": alg_bytes, "configs": configs_alg_bytes, "layernorm": ln_alg_bytes,
                "qk_rope": qk_alg_bytes, "silu": silu_alg_bytes, "fixed_width": fixed_alg_bytes}


def _stats(ts):
    """Average, median, p10 and p90 of a list of durations in seconds, as microseconds."""
    v = sorted(ts)
    q = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]
    return {"us": round(sum(v) / len(v) * 1e6, 2), "median_us": round(q(0.5) * 1e6, 2),
            "p10_us": round(q(0.1) * 1e6, 2), "p90_us": round(q(0.9) * 1e6, 2)}


def device_copy_ceiling(torch, dev, reps: int = 5) -> float:
    """Measured copy ceiling: a 1 GiB device-to-device copy (reads 1 GiB, writes 1 GiB),
    median of `reps`, in GB/s of bytes moved."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    ts = []
    for _ in range(reps):
        e0, e1 = timing_event(torch), timing_event(torch)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del src, dst
    return round(2 * (1 << 30) / sorted(ts)[len(ts) // 2] / 1e9, 1)


PROBE_SRC = os.path.join(ROOT, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(ROOT, "probe", "libdnprobe.so")


def probe_library(rebuild: bool = False) -> str:
    """Path of the stream-ceiling probe library (probe/stream_probe.hip, a measurement aid
    outside the norm library), compiled with hipcc for gfx950 when it is missing or older
    than its sources (the probe shares the norm kernels' memory helpers, dn_device.h)."""
    srcs = [PROBE_SRC, os.path.join(ROOT, "dit_normalization_amd", "csrc", "dn_device.h")]
    stale = not os.path.exists(PROBE_LIB) or \
        os.path.getmtime(PROBE_LIB) < max(os.path.getmtime(s) for s in srcs)
    if rebuild or stale:
        import subprocess

        from dit_normalization_amd import build as B
        obj = B._compile(PROBE_SRC, False, objdir=os.path.dirname(PROBE_LIB))
        tmp = PROBE_LIB + ".tmp"
        r = subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", tmp,
                            obj], capture_output=True, text=True)
        os.remove(obj)
        if r.returncode != 0:
            raise RuntimeError(f"probe link failed:\n{r.stdout}{r.stderr}")
        os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


PROBE_MODES = {0: "grid-stride", 1: "contiguous chunk per block", 2: "XCD partition",
               3: "LDS pipeline (loads straight into LDS)", 4: "block read/write phases"}


def stream_ceilings(torch, dev, reps: int = 5):
    """Measured HBM stream ceilings (probe/stream_probe.hip): plain kernels with the norm
    kernels' 16-byte non-temporal buffer loads and stores at their read:write mixes, 256 MiB
    per stream, caches flushed before every launch, under five access strategies (PROBE_MODES)
    at 1 and 2 blocks of 256 threads per CU.  Returns the best median GB/s (bytes moved) per
    mix over every strategy, the best per strategy under `strategies`, and 2R:2W at 64 MiB and
    2R:1W at 32 MiB per stream (the fused add's and the backward shard's own sizes)."""
    import ctypes
    lib = ctypes.CDLL(probe_library())
    f = lib.dn_probe_stream
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] + [ctypes.c_int] * 4 + [ctypes.c_void_p]
    f.restype = ctypes.c_int
    n = 256 << 20
    bufs = [torch.empty(n, dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(5)]
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    st = torch.cuda.current_stream(dev).cuda_stream
    out, strategies = {}, {}
    for reads, writes in ((1, 1), (2, 2), (2, 1), (3, 1)):
        mix = f"{reads}r{writes}w"
        best = 0.0
        for mode in PROBE_MODES:
            mbest = 0.0
            for blocks in (cus, 2 * cus):
                ts = []
                for _ in range(reps):
                    flush.fill_(1.0)
                    e0 = timing_event(torch)
                    e1 = timing_event(torch)
                    e0.record()
                    rc = f(*(b.data_ptr() for b in bufs), n, reads, writes, blocks, mode, st)
                    e1.record()
                    e1.synchronize()
                    if rc != 0:
                        raise RuntimeError(f"stream probe failed ({rc})")
                    ts.append(e0.elapsed_time(e1) * 1e-3)
                gbs = (reads + writes) * n / sorted(ts)[len(ts) // 2] / 1e9
                mbest = max(mbest, gbs)
            strategies.setdefault(PROBE_MODES[mode], {})[mix] = round(mbest, 1)
            best = max(best, mbest)
        out[f"stream_{mix}_GB/s"] = round(best, 1)
    out["strategies"] = strategies
    # The same mixes at the per-stream sizes of the shorter launches (fused add [8192,4096]:
    # 64 MiB per stream; the backward at [2048,8192]: 32 MiB), where the ramp and the last
    # partial round weigh as they do on the kernel; the two launch shapes that win above.
    for reads, writes, mib in ((2, 2, 64), (2, 1, 32)):
        m = mib << 20
        best = 0.0
        for mode in (0, 1):
            for blocks in (cus, 2 * cus):
                ts = []
                for _ in range(reps):
                    flush.fill_(1.0)
                    e0 = timing_event(torch)
                    e1 = timing_event(torch)
                    e0.record()
                    rc = f(*(b.data_ptr() for b in bufs), m, reads, writes, blocks, mode, st)
                    e1.record()
                    e1.synchronize()
                    if rc != 0:
                        raise RuntimeError(f"stream probe failed ({rc})")
                    ts.append(e0.elapsed_time(e1) * 1e-3)
                best = max(best, (reads + writes) * m / sorted(ts)[len(ts) // 2] / 1e9)
        out[f"stream_{reads}r{writes}w_{mib}MiB_GB/s"] = round(best, 1)
    del bufs, flush
    return out


SHARD = (2048, 8192)


def shard_measurement(torch, dev, dn, W, reps: int = 50):
    """The training forward + backward at one GPU's share of an 8-way data-parallel C4
    batch ([2048, 8192]); a 1 GiB buffer is overwritten before every launch so that the
    32 MiB tensors come from HBM, not from the Infinity Cache."""
    T, H = SHARD
    wl = W.train(rows=T, hidden=H)
    h, u, w, g = (wl.tensors[k].to(dev) for k in ("h", "residual", "w", "g"))
    y, hn, dx = torch.empty_like(h), torch.empty_like(h), torch.empty_like(h)
    rs = torch.empty(T, dtype=torch.float32, device=dev)
    dw = torch.empty(H, dtype=torch.float32, device=dev)
    ws = dn.train_backward_workspace(H, dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    e = T * H
    calls = {
        "train_forward": (8 * e + 4 * T + 4 * H, lambda: dn.dn_train_forward(
            h, w, 1e-6, w_bias=1.0, residual=u, out=y, rstd=rs, residual_out=hn)),
        "train_backward": (6 * e + 4 * T + 8 * H, lambda: dn.dn_train_backward(
            g, hn, w, rs, w_bias=1.0, workspace=ws, dx=dx, dw=dw)),
    }
    out = {}
    for name, (nbytes, fn) in calls.items():
        fn()
        ts = []
        for _ in range(reps):
            flush.fill_(1.0)
            e0, e1 = timing_event(torch), timing_event(torch)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        st = _stats(ts)
        gbs = nbytes / (st["median_us"] * 1e-6) / 1e9
        out[name] = dict(st, bytes=nbytes, **{"GB/s": round(gbs, 1)},
                         frac=round(gbs / HBM_PEAK_GBS, 4))
    del flush
    return {"shape": list(SHARD), "note": "one GPU's rows of C4 split 8 ways; median of "
                                          f"{reps} cold launches", "kernels": out}


def isolated(torch, fn, nbytes: int, flush, reps: int = 50):
    """Median/p10/p90 of `reps` launches of `fn`, each after a 1 GiB write that evicts L2 and
    the 256 MB Infinity Cache, so every launch streams its inputs from HBM."""
    fn()
    ts = []
    for _ in range(reps):
        flush.fill_(1.0)
        e0, e1 = timing_event(torch), timing_event(torch)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    st = _stats(ts)
    gbs = nbytes / (st["median_us"] * 1e-6) / 1e9
    return dict(st, bytes=nbytes, **{"GB/s": round(gbs, 1)}, frac=round(gbs / HBM_PEAK_GBS, 4))


def config_measurements(torch, dev, dn, W, reps: int = 50):
    """The other configurations of the hot path, each launch isolated (caches evicted):
    rmsnorm [32,4096] (launch-bound), fused add + static FP8 per head [8192,32,128] and with
    the Gemma weight offset, 1x128 block FP8 [16384,7168] (with and without normed_out), and
    the gated AdaRMSNorm + FP8 [2520,3072] with per-row and broadcast style."""
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    scale = torch.tensor([0.04], dtype=torch.float32, device=dev)
    out = {}

    c1 = W.rmsnorm_fwd()
    x1, w1 = c1.tensors["x"].to(dev), c1.tensors["w"].to(dev)
    y1 = torch.empty_like(x1)
    r1 = torch.empty(x1.shape[0], dtype=torch.float32, device=dev)
    t1, h1 = x1.shape
    out["rmsnorm_32x4096"] = isolated(torch, lambda: dn.dn_rmsnorm(
        x1, w1, 1e-6, out=y1, rstd=r1, return_rstd=True), 4 * t1 * h1 + 2 * h1 + 4 * t1, flush,
        reps)

    c2 = W.fused_add_quant(8192, 128, heads=32)
    x2, r2, w2 = (c2.tensors[k].to(dev) for k in ("x", "residual", "w"))
    q2 = torch.empty(x2.shape, dtype=torch.float8_e4m3fn, device=dev)
    out["fused_add_quant_per_head_8192x32x128"] = isolated(torch, lambda: (
        dn.dn_fused_add_rmsnorm_quant(x2, r2, w2, scale, 1e-6, out=q2)),
        7 * x2.numel() + 2 * 128 + 4, flush, reps)
    del x2, r2, q2

    c2 = W.fused_add_quant()
    x2, r2, w2 = (c2.tensors[k].to(dev) for k in ("x", "residual", "w"))
    q2 = torch.empty(x2.shape, dtype=torch.float8_e4m3fn, device=dev)
    out["fused_add_quant_gemma_8192x4096"] = isolated(torch, lambda: (
        dn.dn_fused_add_rmsnorm_quant(x2, r2, w2, scale, 1e-6, w_bias=1.0, out=q2)),
        7 * x2.numel() + 2 * 4096 + 4, flush, reps)
    del x2, r2, q2

    c3 = W.block_quant()
    x3, r3, w3 = (c3.tensors[k].to(dev) for k in ("x", "residual", "w"))
    t3, h3 = x3.shape
    q3 = torch.empty(x3.shape, dtype=torch.float8_e4m3fn, device=dev)
    s3 = torch.empty((h3 // 128, (t3 + 3) // 4 * 4), dtype=torch.float32, device=dev)
    n3 = torch.empty_like(x3)
    b3 = 7 * t3 * h3 + 4 * t3 * (h3 // 128) + 2 * h3
    out["block_quant_16384x7168"] = isolated(torch, lambda: (
        dn.dn_fused_add_rmsnorm_fp8_block_quant(x3, r3, w3, 1e-6, out=q3, block_scale=s3)),
        b3, flush, reps)
    out["block_quant_normed_out_16384x7168"] = isolated(torch, lambda: (
        dn.dn_fused_add_rmsnorm_fp8_block_quant(x3, r3, w3, 1e-6, out=q3, block_scale=s3,
                                                normed_out=n3)), b3 + 2 * t3 * h3, flush, reps)
    del x3, r3, q3, s3, n3

    for bc in (False, True):
        c5 = W.ada(broadcast=bc)
        x5, r5, g5, w5, st5 = (c5.tensors[k].to(dev) for k in ("x", "residual", "gate", "w",
                                                                 "style"))
        t5, d5 = x5.shape
        q5 = torch.empty(x5.shape, dtype=torch.float8_e4m3fn, device=dev)
        go5 = torch.empty_like(x5)
        # read x, residual, gate and the style rows (scale, shift, gate chunks); write
        # residual, FP8 out and gate_out
        per_row = 2 * 3 * d5 * (t5 if not bc else 1)
        b5 = (2 + 2 + 2 + 2 + 1 + 2) * t5 * d5 + per_row + 2 * d5 + 4
        name = "ada_gated_fp8_" + ("broadcast_" if bc else "") + f"{t5}x{d5}"
        out[name] = isolated(torch, lambda: dn.dn_gate_residual_ada_norm_fp8(
            r5, x5, g5, w5, st5, scale, 1e-6, out=q5, gate_out=go5), b5, flush, reps)
        del x5, r5, g5, st5, q5, go5
    del flush
    return out


def run_layernorm_family(a) -> int:
    import torch

    import workloads as W
    from dit_normalization_amd import dnorm as dn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] generating LayerNorm inputs", file=sys.stderr, flush=True)
    lw = W.layernorm(*LN)
    x, gam, bet = (lw.tensors[k].to(dev) for k in ("x", "gamma", "beta"))
    y = torch.empty_like(x)
    q = torch.empty(LN, dtype=torch.float8_e4m3fn, device=dev)
    scale = torch.tensor([0.04], dtype=torch.float32, device=dev)
    dw = W.dit(*DIT)
    p = dw.params
    td, hd = DIT
    dx, dr = dw.tensors["x"].to(dev), dw.tensors["residual"].to(dev)
    temb = dw.tensors["temb"].to(dev)
    chunk = {n: temb[:, k * hd:(k + 1) * hd] for k, n in enumerate(W.DIT_CHUNKS)}
    dg, db = dw.tensors["gamma"].to(dev), dw.tensors["beta"].to(dev)
    ro, no = torch.empty_like(dx), torch.empty_like(dx)

    calls = {
        "layernorm": lambda: dn.dn_layernorm(x, gam, bet, 1e-6, out=y),
        "dit_gate_residual_layernorm_gamma_beta": lambda: (
            dn.dn_fused_dit_gate_residual_layernorm_gamma_beta(
                dx, dr, chunk["gate"], dg, db, 1e-6, gate_bias=p["gate_bias"], residual_out=ro,
                norm_out=no)),
        "layernorm_quant": lambda: dn.dn_layernorm_quant(x, gam, bet, scale, 1e-6, out=q),
        "dit_gate_residual_layernorm_scale_shift": lambda: (
            dn.dn_fused_dit_gate_residual_layernorm_scale_shift(
                dx, dr, chunk["gate"], chunk["scale"], chunk["shift"], 1e-6,
                gate_bias=p["gate_bias"], scale_bias=p["scale_bias"],
                shift_bias=p["shift_bias"], residual_out=ro, norm_out=no)),
        "dit_residual_layernorm_scale_shift": lambda: (
            dn.dn_fused_dit_residual_layernorm_scale_shift(
                dx, chunk["scale"], chunk["shift"], dr, 1e-6, scale_bias=p["scale_bias"],
                shift_bias=p["shift_bias"], residual_out=ro, norm_out=no)),
    }
    def cpu():
        from oracle import layernorm as L
        xs, gs, bs = _vals(lw.tensors["x"][:128]), _vals(lw.tensors["gamma"]), _vals(lw.tensors["beta"])
        d = {k: _vals(dw.tensors[k][:128]) for k in ("x", "residual", "gate", "scale", "shift")}
        dg_, db_ = _vals(dw.tensors["gamma"]), _vals(dw.tensors["beta"])
        tl, hl = 128, LN[1]
        hd = DIT[1]
        per = (4 + 3) * tl * hl + (10 + 14 + 12) * 128 * hd

        def run():
            L.layernorm_quant(xs, gs, bs, 0.04, 1e-6)
            L.layernorm(xs, gs, bs, 1e-6)
            L.dit_gate_residual_layernorm_gamma_beta(d["residual"], d["x"], d["gate"], dg_, db_,
                                                     p["gate_bias"], 1e-6)
            L.dit_gate_residual_layernorm_scale_shift(d["residual"], d["x"], d["gate"], d["scale"],
                                                      d["shift"], p["gate_bias"], p["scale_bias"],
                                                      p["shift_bias"], 1e-6)
            L.dit_residual_layernorm_scale_shift(d["x"], d["scale"], d["shift"], d["residual"],
                                                 p["scale_bias"], p["shift_bias"], 1e-6)
        return _oracle_rate(run, per, a.cpu_seconds / 2,
                            "the five LayerNorm-family calls on 128 rows each")

    return time_family(a, torch, dev, calls, "achieved HBM GB/s, LayerNorm family",
                       "layernorm + layernorm_quant BF16 [8192,4096]; DiT gate/residual "
                       "+ LayerNorm (gamma/beta, scale/shift) and residual + LayerNorm "
                       "scale/shift BF16 [16384,3072], modulation chunks of a "
                       "[16384,18432] tensor", cpu)


def _vals(t):
    """Host float64 values of a BF16 / FP32 torch CPU tensor (the oracle's BF16 decoder)."""
    import numpy as np
    import torch

    from oracle import formats as F
    if t.dtype == torch.bfloat16:
        return F.bf16_bits_to_f64(t.contiguous().view(torch.int16).numpy().view(np.uint16))
    return t.double().numpy()


def time_family(a, torch, dev, calls, metric, workload, cpu=None) -> int:
    """Warm up, then time `a.steps` rounds of every call in `calls` (one event between every
    two calls on the calls' stream) and print one JSON line with per-call GB/s, a roofline
    object for the call that takes the most time (with its counter-measured traffic while
    the kernel sources match the family's committed summary), and (unless
    --no-cpu-baseline) the oracle's rate from `cpu()`."""
    ab = FAMILY_BYTES[a.family]()
    names = list(calls)
    if names != list(ab):
        raise RuntimeError(f"{a.family}: calls {names} differ from the byte table {list(ab)}")
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(a.warmup):
        for n in names:
            calls[n]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    evs = [[timing_event(torch) for _ in range(len(names) + 1)]
           for _ in range(a.steps)]
    print(f"[bench] timing {a.steps} rounds", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        for j, n in enumerate(names):
            e[j].record(stream)
            calls[n]()
        e[-1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernels = {}
    for j, n in enumerate(names):
        st = _stats([e[j].elapsed_time(e[j + 1]) * 1e-3 for e in evs])
        gbs = ab[n] / (st["us"] * 1e-6) / 1e9
        kernels[n] = dict(st, bytes=ab[n], **{"GB/s": round(gbs, 1)},
                          frac=round(gbs / HBM_PEAK_GBS, 4))
    step_bytes = sum(ab.values())
    value = step_bytes / (wall / a.steps) / 1e9
    dom = max(names, key=lambda n: kernels[n]["us"])
    roofline = {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["GB/s"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kernels[dom]["frac"],
                "traffic": measured_traffic(dom, a.family), "algorithmic_bytes": ab[dom]}
    cpu_line = None
    if cpu is not None and not a.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        cpu_line = cpu()
    line = {
        "metric": metric, "value": round(value, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(wall / a.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": workload,
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4), "step_bytes": step_bytes,
                   "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu_line, "kernels": kernels,
        "timing_events": _EVENT_KIND["kind"],
    }
    print(json.dumps(line), flush=True)
    return 0


def run_qk_rope_family(a) -> int:
    """fused_qk_rmsnorm_rope on the stand-in video latent (12288 tokens, 24+24+24 heads of
    128 channels, 44/42/42 frame/height/width channels): interleaved and NeoX pairing, BF16
    and e4m3fn outputs."""
    import torch

    import workloads as W
    from dit_normalization_amd import dnorm as dn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] generating QK RoPE inputs", file=sys.stderr, flush=True)
    wl = W.qk_rope()
    t, p = wl.tensors, wl.params
    qkv, wq, wk = (t[k].to(dev) for k in ("qkv", "q_weight", "k_weight"))
    T, width = qkv.shape
    qs = torch.tensor([p["output_scale"]], dtype=torch.float32, device=dev)
    vs = torch.tensor([p["v_scale"]], dtype=torch.float32, device=dev)
    outs = {}
    for fp8 in (False, True):
        dt = torch.float8_e4m3fn if fp8 else torch.bfloat16
        outs[fp8] = [torch.empty((T, n * p["head_dim"]), dtype=dt, device=dev)
                     for n in (p["nq"], p["nk"], p["nv"])]

    def call(interleave, fp8):
        q, k, v = outs[fp8]
        return lambda: dn.dn_fused_qk_rmsnorm_rope(
            qkv, wq, wk, p["nq"], p["nk"], p["nv"], p["head_dim"], p["ppf"], p["pph"], p["ppw"],
            p["channels"], p["eps"], interleave=interleave, output_fp8=fp8,
            output_quant_scale=qs, v_quant_scale=vs, q_out=q, k_out=k, v_out=v)

    calls = {"qk_rope_interleaved_bf16": call(True, False), "qk_rope_neox_bf16": call(False, False),
             "qk_rope_interleaved_fp8": call(True, True), "qk_rope_neox_fp8": call(False, True)}
    if any(p[k] != QK[k] for k in QK):
        raise RuntimeError(f"the QK RoPE workload {p} is not the byte table's {QK}")
    def cpu():
        from oracle import qk_rope as Q
        n = 64
        x = _vals(t["qkv"][:n])
        wq_, wk_ = _vals(t["q_weight"]), _vals(t["k_weight"])
        ids = list(range(n))

        def run():
            for il in (True, False):
                Q.qk_rmsnorm_rope(x, wq_, wk_, p["nq"], p["nk"], p["nv"], p["head_dim"],
                                  p["channels"], p["ppf"], p["pph"], p["ppw"], p["eps"],
                                  p["base"], il, token_ids=ids)
        return _oracle_rate(run, 2 * 4 * n * width, a.cpu_seconds / 2,
                            f"both pairings on {n} tokens x {width}")

    return time_family(a, torch, dev, calls, "achieved HBM GB/s, fused QK RMSNorm + 3-D RoPE",
                       f"fused_qk_rmsnorm_rope qkv BF16 [{T},{width}] (24+24+24 heads x 128, "
                       f"patches {p['ppf']}x{p['pph']}x{p['ppw']}), BF16 or e4m3fn q/k/v out", cpu)


def run_silu_family(a) -> int:
    """fused_rmsnorm_silu at three of the pages' video-VAE shapes, BF16 and e4m3fn out."""
    import torch

    import workloads as W
    from dit_normalization_amd import dnorm as dn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] generating RMSNorm + SiLU inputs", file=sys.stderr, flush=True)
    calls = {}
    scale = torch.tensor([0.02], dtype=torch.float32, device=dev)
    for T, H in SILU_SHAPES:
        wl = W.rmsnorm_silu(T, H)
        x, w = wl.tensors["x"].to(dev), wl.tensors["w"].to(dev)
        ob = torch.empty_like(x)
        o8 = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=dev)
        calls[f"silu_bf16_{T}x{H}"] = (lambda x=x, w=w, ob=ob: dn.dn_fused_rmsnorm_silu(
            x, w, 1e-6, out=ob))
        calls[f"silu_fp8_{T}x{H}"] = (lambda x=x, w=w, o8=o8: dn.dn_fused_rmsnorm_silu(
            x, w, 1e-6, out=o8, scale=scale))
    def cpu():
        from oracle import silu as S
        wl = W.rmsnorm_silu(1024, 512)
        xs, ws = _vals(wl.tensors["x"]), _vals(wl.tensors["w"])
        return _oracle_rate(lambda: S.fused_rmsnorm_silu(xs, ws, 1e-6), 4 * 1024 * 512,
                            a.cpu_seconds / 2, "BF16 out on 1024 rows x 512")

    return time_family(a, torch, dev, calls, "achieved HBM GB/s, fused RMSNorm + SiLU",
                       "fused_rmsnorm_silu BF16 [399360,128], [99840,512], [24960,1024]; "
                       "BF16 or e4m3fn out", cpu)


def run_fixed_width_family(a) -> int:
    """The fixed-width norms at the pages' widths: gated-residual RMSNorm (+ next RMSNorm) at
    hidden 8192, per-token and shared gate; per-head RMSNorm + sigmoid gate at head dim 64."""
    import torch

    import workloads as W
    from dit_normalization_amd import dnorm as dn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] generating fixed-width norm inputs", file=sys.stderr, flush=True)
    gw = W.gated_residual(*GRES)
    b, r, g, w, w2 = (gw.tensors[k].to(dev) for k in ("branch", "residual", "gate", "w", "w_next"))
    g1 = g[0].contiguous()
    y = torch.empty_like(b)
    T, H = b.shape
    sw = W.sigmoid_gate(*SIGMOID)
    sp = sw.params
    x = sw.tensors["x"].to(dev).reshape(sp["tokens"], sp["heads"], sp["head_dim"])
    sg = sw.tensors["gate"].to(dev).reshape(sp["tokens"], sp["heads"], sp["head_dim"])
    sww = sw.tensors["w"].to(dev)
    calls = {
        "gated_residual_token_gate": lambda: dn.dn_gated_residual_rmsnorm(b, r, g, w, 1e-6),
        "gated_residual_shared_gate": lambda: dn.dn_gated_residual_rmsnorm(b, r, g1, w, 1e-6),
        "gated_residual_next_token_gate": lambda: dn.dn_gated_residual_next_rmsnorm(
            b, r, g, w, w2, 1e-6, out=y),
        "rmsnorm_sigmoid_gate": lambda: dn.dn_rmsnorm_sigmoid_gate(x, sg, 1e-6, weight=sww),
    }
    def cpu():
        from oracle import gated as Gd
        from oracle import silu as S
        n = 64
        bb, rr_, gg = (_vals(gw.tensors[k][:n]) for k in ("branch", "residual", "gate"))
        w1, w2_ = _vals(gw.tensors["w"]), _vals(gw.tensors["w_next"])
        xs = _vals(sw.tensors["x"][:n]).reshape(-1, sp["head_dim"])
        gs = _vals(sw.tensors["gate"][:n]).reshape(-1, sp["head_dim"])
        sw_ = _vals(sw.tensors["w"])

        def run():
            Gd.gated_residual_rmsnorm(bb, rr_, gg, w1, 1e-6, next_w=w2_)
            S.rmsnorm_sigmoid_gate(xs, gs, sw_, 1e-6)
        return _oracle_rate(run, 10 * n * H + 6 * xs.size, a.cpu_seconds / 2,
                            f"gated residual + next on {n} rows x {H} and the sigmoid gate on "
                            f"{n} tokens")

    return time_family(a, torch, dev, calls, "achieved HBM GB/s, fixed-width fused norms",
                       f"gated-residual RMSNorm (+ next) BF16 [{T},{H}]; per-head RMSNorm + "
                       f"sigmoid gate BF16 [{sp['tokens']},{sp['heads']}x{sp['head_dim']}]", cpu)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="skip the copy ceiling and the shard shape (profiler runs: every "
                         "library dispatch is then a bench-step kernel)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-trace", metavar="STATS_CSV")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("LDS_CSV", "OCC_CSV"),
                    help="LDS bank conflicts and occupancy per call from two rocprofv3 --pmc "
                         "runs (see summarize_sq)")
    ap.add_argument("--kernel-resources", nargs="?", const="", metavar="MATCH",
                    help="print the registers, scratch and LDS of the library's kernels "
                         "(those whose name contains MATCH) from the code objects; no GPU")
    ap.add_argument("--family", choices=("rmsnorm", "configs", "layernorm", "qk_rope", "silu",
                                         "fixed_width"),
                    default="rmsnorm",
                    help="rmsnorm: the hot-path step (default); layernorm: the LayerNorm "
                         "family; qk_rope: the fused QK RMSNorm + 3-D RoPE; silu: the fused "
                         "RMSNorm + SiLU; fixed_width: gated-residual and sigmoid-gate norms")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reads 1 GiB, writes 1 GiB) five "
                         "times, to scale profiler byte counters")
    a = ap.parse_args(argv)
    if a.summarize_counters:
        return summarize_counters(*a.summarize_counters, family=a.family)
    if a.summarize_trace:
        return summarize_trace(a.summarize_trace)
    if a.summarize_sq:
        return summarize_sq(*a.summarize_sq, family=a.family)
    if a.kernel_resources is not None:
        return print_kernel_resources(a.kernel_resources)
    if a.gpus != 1:
        print(f"bench.py measures one GPU: the RMSNorm path here is built and timed on a single "
              f"MI355X (rows shard across GPUs with no communication except dw); --gpus {a.gpus} "
              f"is not supported.", file=sys.stderr)
        return 2

    import torch

    import workloads as W
    from dit_normalization_amd import dnorm as dn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.family == "configs":
        return run_configs_family(a)
    if a.family == "layernorm":
        return run_layernorm_family(a)
    if a.family == "qk_rope":
        return run_qk_rope_family(a)
    if a.family == "silu":
        return run_silu_family(a)
    if a.family == "fixed_width":
        return run_fixed_width_family(a)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating inputs", file=sys.stderr, flush=True)
    c2 = W.fused_add_quant()
    x2, r2, w2 = (c2.tensors[k].to(dev) for k in ("x", "residual", "w"))
    x2q, r2q = c2.tensors["x"].to(dev), c2.tensors["residual"].to(dev)
    c4 = W.train()
    h4, u4, w4, g4 = (c4.tensors[k].to(dev) for k in ("h", "residual", "w", "g"))
    T4, H4 = C4
    y4 = torch.empty_like(h4)
    hn4 = torch.empty_like(h4)
    rs4 = torch.empty(T4, dtype=torch.float32, device=dev)
    dx4 = torch.empty_like(h4)
    dw4 = torch.empty(H4, dtype=torch.float32, device=dev)
    q2 = torch.empty(C2, dtype=torch.float8_e4m3fn, device=dev)
    scale = torch.tensor([0.04], dtype=torch.float32, device=dev)
    ws = dn.train_backward_workspace(H4, dev)

    calls = {
        "fused_add_rmsnorm": lambda: dn.dn_fused_add_rmsnorm(x2, r2, w2, 1e-6),
        "train_forward": lambda: dn.dn_train_forward(h4, w4, 1e-6, w_bias=1.0, residual=u4,
                                                     out=y4, rstd=rs4, residual_out=hn4),
        "fused_add_rmsnorm_quant": lambda: dn.dn_fused_add_rmsnorm_quant(x2q, r2q, w2, scale,
                                                                         1e-6, out=q2),
        "train_backward": lambda: dn.dn_train_backward(g4, hn4, w4, rs4, w_bias=1.0,
                                                       workspace=ws, dx=dx4, dw=dw4),
    }

    def run(names, events=None, only=None):
        """One round of `names`; events[j] is recorded before names[j] (and events[-1] after
        the last) when j is in `only` (every j when only is None)."""
        def mark(j):
            if events is not None and (only is None or j in only):
                events[j].record()
        for j, n in enumerate(names):
            mark(j)
            calls[n]()
        mark(len(names))

    def rounds(names, k, events_per_round=False, only=None, every=1):
        """K rounds between synchronisations; with events_per_round, every `every`-th round
        carries events (the others none).  Returns the wall time and the sampled rounds'
        events."""
        evs = [[timing_event(torch) for _ in range(len(names) + 1)]
               if events_per_round and i % every == 0 else None for i in range(k)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e in evs:
            run(names, e, only)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, [e for e in evs if e is not None]

    def durations(names, evs):
        return {n: [e[j].elapsed_time(e[j + 1]) * 1e-3 for e in evs] for j, n in enumerate(names)}

    ab = alg_bytes()
    pair_bytes = sum(ab[n] for n in PAIR_KERNELS)
    step_bytes = sum(ab[n] for n in STEP_KERNELS)
    # The backward reads the training forward's h_new and rstd: one forward before anything
    # is timed (inputs resident in HBM).  Profiler runs leave it out, so that their library
    # dispatches are whole steps (the first warm-up step's forward precedes its backward).
    if not a.step_only:
        calls["train_forward"]()
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] warmup {a.warmup}", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        run(STEP_KERNELS)
    torch.cuda.synchronize()

    dom = "train_backward"
    if not a.step_only:
        # Timed region: K rounds of the metric's pair between synchronisations (wall clock);
        # only the dominant kernel (the backward) is bracketed by events, in every fourth
        # round, since even a fence-free event record costs the stream about a microsecond.
        print(f"[bench] timing {a.steps} rounds of the pair", file=sys.stderr, flush=True)
        di = PAIR_KERNELS.index(dom)
        wall, evs = rounds(PAIR_KERNELS, a.steps, True, only=(di, di + 1), every=LIVE_EVERY)
        dom_live = [e[di].elapsed_time(e[di + 1]) * 1e-3 for e in evs]
        # The pair's per-kernel breakdown: K more rounds with an event between the kernels.
        _, evs = rounds(PAIR_KERNELS, a.steps, True)
        pair_per = durations(PAIR_KERNELS, evs)
    # The whole hot-path step (all four kernels), K rounds: wall clock, then per kernel.
    print(f"[bench] timing {a.steps} whole steps", file=sys.stderr, flush=True)
    step_wall, _ = rounds(STEP_KERNELS, a.steps)
    _, evs = rounds(STEP_KERNELS, a.steps, True)
    per = durations(STEP_KERNELS, evs)
    if a.step_only:
        # profiler runs time whole steps only: the pair's figures come from their events
        pair_per = {n: per[n] for n in PAIR_KERNELS}
        dom_live = per[dom]
        wall = sum(sum(pair_per[n]) for n in PAIR_KERNELS)
    ms_per_step = wall / a.steps * 1e3
    value = pair_bytes / (wall / a.steps) / 1e9

    kernels = {}
    for n in STEP_KERNELS:
        st = _stats(per[n])
        gbs = ab[n] / (st["us"] * 1e-6) / 1e9
        kernels[n] = dict(st, bytes=ab[n], **{"GB/s": round(gbs, 1)},
                          frac=round(gbs / HBM_PEAK_GBS, 4))
    fa_s = sum(pair_per["fused_add_rmsnorm"]) / a.steps
    bwd_s = sum(pair_per["train_backward"]) / a.steps
    headline = {
        "fused_add_rmsnorm_fwd_GB/s": round(ab["fused_add_rmsnorm"] / fa_s / 1e9, 1),
        "train_bwd_GB/s": round(ab["train_backward"] / bwd_s / 1e9, 1),
        "fused_add_fwd_plus_train_bwd_GB/s": round(pair_bytes / (fa_s + bwd_s) / 1e9, 1),
    }
    whole_step = {"GB/s": round(step_bytes / (step_wall / a.steps) / 1e9, 1),
                  "ms_per_step": round(step_wall / a.steps * 1e3, 4), "bytes": step_bytes,
                  "frac": round(step_bytes / (step_wall / a.steps) / 1e9 / HBM_PEAK_GBS, 4),
                  "kernels": STEP_KERNELS}
    dom_avg = sum(dom_live) / len(dom_live)
    achieved = ab[dom] / dom_avg / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom), "algorithmic_bytes": ab[dom]}

    ceiling = shard = configs = None
    if not a.step_only:
        print("[bench] copy ceiling and one GPU's shard of the training shape", file=sys.stderr,
              flush=True)
        ceiling = {"device_copy_1GiB_GB/s": device_copy_ceiling(torch, dev)}
        ceiling.update(stream_ceilings(torch, dev))
        mix = {"fused_add_rmsnorm": "stream_2r2w_GB/s", "train_forward": "stream_2r2w_GB/s",
               "train_backward": "stream_2r1w_GB/s"}
        for k, m in mix.items():
            kernels[k]["of_stream_ceiling"] = round(kernels[k]["GB/s"] / ceiling[m], 4)
        # against a stream of the kernel's own size (256 MiB per stream is the training
        # shapes' own: [16384,8192] BF16)
        matched = dict(mix, fused_add_rmsnorm="stream_2r2w_64MiB_GB/s")
        for k, m in matched.items():
            kernels[k]["of_size_matched_ceiling"] = round(kernels[k]["GB/s"] / ceiling[m], 4)
        shard = shard_measurement(torch, dev, dn, W)
        sb = shard["kernels"]["train_backward"]
        sb["of_size_matched_ceiling"] = round(sb["GB/s"] / ceiling["stream_2r1w_32MiB_GB/s"], 4)
        print("[bench] the other configurations, isolated", file=sys.stderr, flush=True)
        configs = config_measurements(torch, dev, dn, W)

    cpu = None
    if not a.no_cpu_baseline:
        print(f"[bench] cpu baseline ({a.cpu_seconds:.0f} s of oracle work)", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(a.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "fused_add_rmsnorm fwd BF16 [8192,4096] in place + training "
                               "RMSNorm bwd BF16 [16384,8192] (dx and deterministic FP32 dw of "
                               "the residual-route forward, FP32 weight 1+w)",
                   "storage": "bf16 activations, fp32 statistics/weights/dw",
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
                   "step_bytes": pair_bytes, "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels, "headline": headline,
        "whole_step": whole_step,
        "ceilings": ceiling, "shard_2048x8192": shard, "isolated_configs": configs,
        "timing_events": _EVENT_KIND["kind"],
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
