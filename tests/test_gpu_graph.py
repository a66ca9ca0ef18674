"""The library allocates nothing and never synchronises, so its calls can be captured into a
HIP graph.  A captured training step (forward with residual, backward into a reused
workspace, static-FP8 norm) is replayed several times with new inputs copied in between,
eager work and synchronisations between the replays, and every replay is compared bit for
bit with the same calls made eagerly."""
from __future__ import annotations

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

T, H = 96, 2048


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def fresh_inputs(seed):
    wl = W.train(rows=T, hidden=H, seed=seed)
    t = wl.tensors
    return {k: t[k].to("cuda") for k in ("h", "residual", "g")}


def bits(t):
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t.view(torch.int16) \
        if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_captured_training_step_replays_match_eager(dn):
    w = W.train(rows=T, hidden=H).tensors["w"].to("cuda")
    wq = W.normal((H,), 60, 0, mean=1.0, std=0.1).to("cuda")
    scale = torch.tensor([0.04], dtype=torch.float32, device="cuda")
    inp = {k: torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
           for k in ("h", "residual", "g")}
    out = {"y": torch.empty(T, H, dtype=torch.bfloat16, device="cuda"),
           "h_new": torch.empty(T, H, dtype=torch.bfloat16, device="cuda"),
           "rstd": torch.empty(T, dtype=torch.float32, device="cuda"),
           "dx": torch.empty(T, H, dtype=torch.bfloat16, device="cuda"),
           "dw": torch.empty(H, dtype=torch.float32, device="cuda"),
           "q": torch.empty(T, H, dtype=torch.float8_e4m3fn, device="cuda")}
    ws = dn.train_backward_workspace(H, "cuda")

    def step():
        dn.dn_train_forward(inp["h"], w, 1e-6, w_bias=1.0, residual=inp["residual"],
                            out=out["y"], rstd=out["rstd"], residual_out=out["h_new"])
        dn.dn_train_backward(inp["g"], out["h_new"], w, out["rstd"], w_bias=1.0, workspace=ws,
                             dx=out["dx"], dw=out["dw"])
        dn.dn_rmsnorm_quant(out["h_new"], wq, scale, 1e-6, out=out["q"])

    def eager(seed):
        for k, v in fresh_inputs(seed).items():
            inp[k].copy_(v)
        step()
        torch.cuda.synchronize()
        return {k: v.clone() for k, v in out.items()}

    eager(0)                                   # warm-up: launch caches filled outside capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for seed in (1, 2, 3, 1):
        want = eager(seed)                     # eager work between the replays
        for k in out:
            out[k].zero_()
        for k, v in fresh_inputs(seed).items():
            inp[k].copy_(v)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(bits(out[k]), bits(want[k])), f"replay with seed {seed}: {k}"
