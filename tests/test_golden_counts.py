"""Numbers the pages print, checked against the workloads and the oracle."""
import json
import os

import numpy as np

import wa_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_active_context_is_four_pages_of_eight_frames():
    g = _load("worldattention_hkv_counts.json")
    wl = W.WORKLOADS["wan_kp4"]
    assert wl.page_frames == g["frames_per_page"] and wl.frame_tokens == g["tokens_per_frame"]
    assert wl.k_p == g["k_p"]
    assert wl.n_ctx == g["active_tokens"] == g["k_p"] * g["frames_per_page"] * g["tokens_per_frame"]
    for name in ("prompt_page", "long_horizon"):
        assert W.WORKLOADS[name].n_ctx == g["active_tokens"]


def test_work_figures_of_the_worked_example():
    g = _load("worldattention_hkv_counts.json")
    L, d, r = g["example_L"], g["example_d_k"], g["example_r"]
    assert abs(L * r * d / g["linear_branch_work_approx"] - 1) < 0.01
    assert abs(L * L * d / g["full_qk_work_approx"] - 1) < 0.01
    assert round(L / r, -1) == g["ratio_L_over_r_approx"]


def test_score_shape_of_the_einsum_example(oracle_lib):
    """The oracle's attention consumes [tokens, H, d]; the pages' einsum example
    (b, h, q, d) x (b, h, k, d) -> (b, h, q, k) fixes which axes contract."""
    g = _load("einsum_scores_shape.json")
    rng = np.random.default_rng(0)
    q = rng.standard_normal(tuple(g["q_shape"]))
    k = rng.standard_normal(tuple(g["k_shape"]))
    assert np.einsum("bhqd,bhkd->bhqk", q, k).shape == tuple(g["scores_shape"])
    # the oracle, fed batch 0 as [tokens, H, d], gives one lse per (head, query)
    qt = np.ascontiguousarray(q[0].transpose(1, 0, 2)).astype(np.float32)
    kt = np.ascontiguousarray(k[0].transpose(1, 0, 2)).astype(np.float32)
    _, lse = oracle_lib.attention(qt, None, None, kt, kt, 1.0)
    assert lse.shape == (g["q_shape"][1], g["q_shape"][2])
    s = np.einsum("bhqd,bhkd->bhqk", q.astype(np.float32).astype(np.float64),
                  k.astype(np.float32).astype(np.float64))[0]
    assert np.abs(np.log(np.exp(s).sum(-1)) - lse).max() < 1e-12
