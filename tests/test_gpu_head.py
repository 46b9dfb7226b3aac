"""GPU parity of the multitask ranking head (hstu_head_forward) against the
oracle: small ragged row lists, the BM = 128 launch at a full candidate count
(sampled rows), repeated and out-of-range row indices, and the head on the
stack's output at the candidate rows."""
import numpy as np
import pytest
import torch

import oracle
from generative_recommender_sequence_amd import runtime
from generative_recommender_sequence_amd.hstu import HSTU_BF16
from generative_recommender_sequence_amd.workloads import head_weights, round_bf16
from gpu_checks import rel, say, to64

pytestmark = pytest.mark.gpu

TOL_HEAD = 1e-4   # bf16-exact inputs, fp32 accumulation: rounding of the sums only


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    runtime.require_gpu()


def _y(rng, n, d):
    y = round_bf16(rng.standard_normal((n, d)).astype(np.float32))
    return y, torch.from_numpy(y).cuda().to(torch.bfloat16)


def _run(hw, y_dev, rows):
    head = runtime.Head(hw, HSTU_BF16)
    r = torch.from_numpy(np.asarray(rows, np.int32)).cuda()
    out = head(y_dev, r)
    torch.cuda.synchronize()
    return to64(out)


@pytest.mark.parametrize("n_y,n_rows,tasks,hidden", [(300, 277, 3, 256), (64, 1, 1, 128), (130, 129, 5, 384)])
def test_head_vs_oracle(n_y, n_rows, tasks, hidden):
    say(f"head n_y={n_y} rows={n_rows} tasks={tasks} hidden={hidden}")
    rng = np.random.default_rng(n_rows)
    hw = head_weights(512, tasks, hidden, seed=n_y)
    y, y_dev = _y(rng, n_y, 512)
    rows = rng.integers(0, n_y, size=n_rows)
    rows[0] = n_y - 1
    got = _run(hw, y_dev, rows)
    want = oracle.head(y, rows, hw.a, hw.b, hw.w, hw.c)
    err = rel(got, want)
    say(f"  rel err {err:.2e}")
    assert got.shape == (n_rows, tasks) and err < TOL_HEAD


def test_head_full_candidate_count_sampled():
    """32768 candidate rows (128 users x 256 candidates), 4 tasks x 256: the
    launch shape the benchmark's large workload uses; 384 rows checked."""
    rng = np.random.default_rng(5)
    n = 128 * 256
    hw = head_weights(512, seed=1)
    y, y_dev = _y(rng, n + 1000, 512)
    rows = rng.permutation(n + 1000)[:n]
    got = _run(hw, y_dev, rows)
    pick = np.concatenate([[0, n - 1], rng.choice(n, 382, replace=False)])
    want = oracle.head(y, rows[pick], hw.a, hw.b, hw.w, hw.c)
    err = rel(got[pick], want)
    say(f"head full count: rel err {err:.2e} on {len(pick)} rows")
    assert err < TOL_HEAD


def test_head_row_indices_are_clamped():
    rng = np.random.default_rng(9)
    hw = head_weights(512, 2, 128, seed=2)
    y, y_dev = _y(rng, 40, 512)
    rows = np.array([-5, 0, 39, 43, 7], np.int32)
    got = _run(hw, y_dev, rows)
    want = oracle.head(y, np.clip(rows, 0, 39), hw.a, hw.b, hw.w, hw.c)
    assert rel(got, want) < TOL_HEAD


def test_head_on_stack_candidates():
    """The stack's output scored at each user's candidate rows."""
    from generative_recommender_sequence_amd.workloads import generate, small_config
    cfg = small_config(dtype="bf16", num_heads=2, head_dim=128, num_layers=2, n_targets=16, cache="none")
    w = generate(cfg, 4, batch=3, hist_override=[100, 7, 260])
    scn = runtime.Scenario(w)
    req, x = scn.make_request()
    y = runtime.forward(scn.model, req, x, None)
    rows = runtime.candidate_row_list(req.new_len, req.n_targets)
    hw = head_weights(cfg.d_model, seed=3)
    got = _run(hw, y, rows)
    want = oracle.head(to64(y), oracle.candidate_rows(req.new_len, req.n_targets), hw.a, hw.b, hw.w, hw.c)
    err = rel(got, want)
    say(f"head on stack candidates: {len(rows)} rows, rel err {err:.2e}")
    assert got.shape == (48, 4) and err < TOL_HEAD
    req.close()
