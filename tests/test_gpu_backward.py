"""GPU parity of the layer backward (hstu_layer_backward) against the
oracle's chain-rule gradients: dx, dW1, dW2 and drab of one layer on small
and longer jagged batches with candidates, and a two-layer chain."""
import numpy as np
import pytest
import torch

import oracle
from generative_recommender_sequence_amd import runtime
from generative_recommender_sequence_amd.workloads import generate, round_bf16, small_config
from gpu_checks import rel, say, to64

pytestmark = pytest.mark.gpu

# bf16 operands (activations, their gradients and the weights), fp32 sums:
# the forward's bf16 rounding of U, V, Q, K and of dO, dA propagates into every
# gradient; the same 2e-2 as the forward's per-tensor bound
TOL_BWD = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    runtime.require_gpu()


def _case(hist, T, layers=1, seed=0, H=2):
    cfg = small_config(dtype="bf16", num_heads=H, head_dim=128, num_layers=layers, n_targets=T, cache="none")
    w = generate(cfg, seed, batch=len(hist), hist_override=list(hist))
    for lw in w.layers:
        lw.w1 *= 4.0
        lw.w2 *= 4.0
    return w


def _run(w, seed):
    scn = runtime.Scenario(w)
    req, x = scn.make_request()
    y, saved = runtime.forward_for_backward(scn.model, req, x)
    rng = np.random.default_rng(seed)
    dy_np = round_bf16(rng.standard_normal(tuple(y.shape)).astype(np.float32))
    dy = torch.from_numpy(dy_np).cuda().to(torch.bfloat16)
    dx, grads = runtime.backward(scn.model, req, saved, dy)
    torch.cuda.synchronize()
    return scn, req, x, dy_np, saved, dx, grads


def _oracle_layer(scn, req, li, x64, dy64):
    lw = scn.w.layers[li]
    cfg = scn.cfg
    return oracle.layer_backward(x64, lw.w1, lw.w2, lw.rab, req.new_len, req.n_targets, req.norm_n, dy64,
                                 cfg.num_heads, cfg.head_dim, cfg.eps)


@pytest.mark.parametrize("hist,T", [([70, 129, 200], 8), ([1, 31, 64, 257], 0), ([700, 1000], 64)])
def test_layer_backward_vs_oracle(hist, T):
    say(f"backward hist={hist} T={T}")
    w = _case(hist, T, seed=len(hist))
    scn, req, x, dy_np, saved, dx, grads = _run(w, seed=5)
    ref = _oracle_layer(scn, req, 0, to64(x), dy_np.astype(np.float64))
    g = grads[0]
    got = {"x": to64(dx), "w1": to64(g["dw1"]).T, "w2": to64(g["dw2"]).T, "rab": to64(g["drab"])}
    errs = {k: rel(got[k], ref[k]) for k in got}
    say("  " + " ".join(f"d{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v < TOL_BWD}
    assert not bad, bad
    req.close()


def test_two_layer_chain():
    """Layer 1's dx is layer 0's dy: each layer's gradients against the
    oracle fed that layer's GPU input and the GPU's dL/dY of that layer."""
    say("backward two-layer chain")
    w = _case([90, 300], 16, layers=2, seed=9)
    scn = runtime.Scenario(w)
    req, x = scn.make_request()
    y, saved = runtime.forward_for_backward(scn.model, req, x)
    rng = np.random.default_rng(1)
    dy_np = round_bf16(rng.standard_normal(tuple(y.shape)).astype(np.float32))
    dy = torch.from_numpy(dy_np).cuda().to(torch.bfloat16)
    dy0, _ = runtime.backward(scn.model, req, saved, dy, stop_at=1)   # dL/dY of layer 0
    dx, grads = runtime.backward(scn.model, req, saved, dy)
    torch.cuda.synchronize()
    for li, up in ((1, dy_np.astype(np.float64)), (0, to64(dy0))):
        ref = _oracle_layer(scn, req, li, to64(saved[li]["x"]), up)
        got = {"w1": to64(grads[li]["dw1"]).T, "w2": to64(grads[li]["dw2"]).T, "rab": to64(grads[li]["drab"])}
        if li == 0:
            got["x"] = to64(dx)
        errs = {k: rel(got[k], ref[k]) for k in got}
        say(f"  layer {li}: " + " ".join(f"d{k}={v:.2e}" for k, v in errs.items()))
        bad = {k: v for k, v in errs.items() if not v < TOL_BWD}
        assert not bad, (li, bad)
    req.close()


def test_backward_is_deterministic():
    """Every gradient, drab included, is bit-identical across repeated runs
    in one process: the rab gradient is summed per item in a fixed order and
    the items' partials in item order (no float atomics); users longer than
    the 256-distance window exercise the far-distance path too."""
    say("backward determinism")
    w = _case([700, 1000, 33], 64, seed=4)
    scn = runtime.Scenario(w)
    req, x = scn.make_request()
    y, saved = runtime.forward_for_backward(scn.model, req, x)
    dy = torch.from_numpy(round_bf16(np.random.default_rng(8).standard_normal(tuple(y.shape)).astype(
        np.float32))).cuda().to(torch.bfloat16)
    runs = []
    for _ in range(3):
        dx, grads = runtime.backward(scn.model, req, saved, dy)
        torch.cuda.synchronize()
        runs.append((dx.clone(), {k: v.clone() for k, v in grads[0].items()}))
    for dx, g in runs[1:]:
        assert torch.equal(dx, runs[0][0])
        for k in ("dw1", "dw2", "drab"):
            assert torch.equal(g[k], runs[0][1][k]), k
    req.close()
