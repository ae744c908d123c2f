"""Sliding window plus selective fetch (wa_select_window) against the oracle,
and the attention over the pages it returns.

The window's ids come first, in the caller's order, then the top K_p of the
candidates outside the window; indices must be int-equal to the oracle's,
scores within fp64 rounding, and the attention over the returned pages (read
in place with wa_paged_attention) within the attention tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_page_amd as wa
import wa_workloads as W
from tests.pipeline import PoolRun, attention_tolerance, rows_sample, say, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wa.load_library()


SMALL = W.scaled(W.WORKLOADS["wan_kp4"], n_heads=2, frame_tokens=64, page_frames=2, n_pages=8,
                 chunk_frames=3, k_p=3)


def _pool(wl):
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    return run


def _window(run, q, recent, k_p, cand=None):
    wl = run.wl
    rd = torch.tensor(recent, dtype=torch.int32, device="cuda") if len(recent) else None
    cd = torch.tensor(cand, dtype=torch.int32, device="cuda") if cand is not None else None
    n_cand = len(cand) if cand is not None else wl.max_pages
    scores = torch.empty(n_cand, dtype=torch.float64, device="cuda")
    say("select window", recent, "k_p", k_p, "cand", cand)
    idx = wa.wa_select_window(run.L, to_device(q), run.means, rd, k_p, cand=cd,
                              out_scores=scores)
    ref = oracle.select_window(q, run.oracle_means(range(wl.n_pages)), k_p, recent,
                               cand=None if cand is None else np.array(cand, np.int32))
    assert idx.cpu().numpy().tolist() == ref["idx"].tolist()
    serr = np.abs(scores.cpu().numpy() - ref["alpha"]).max()
    assert serr <= 1e-12 * max(1.0, np.abs(ref["alpha"]).max())
    return idx, ref["idx"]


def test_window_selection_matches_the_oracle():
    run = _pool(SMALL)
    q = W.chunk_qkv(SMALL, 0, 0)[0]
    _window(run, q, [7, 6], 3)
    _window(run, q, [7], 0)                                  # window only
    _window(run, q, [], 4)                                   # no window: the page stage
    _window(run, q, [3, 1, 4], 2)                            # window out of page order
    _window(run, q, list(range(8)), 2)                       # window holds every candidate
    _window(run, q, [5, 2], 3, cand=[2, 0, 5, 6, 1])         # explicit candidates
    _window(run, q, [0], 2, cand=[4, 4, 0, 3])               # repeated candidate


def test_window_then_attention_in_place():
    wl = SMALL
    run = _pool(wl)
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    idx_d, idx = _window(run, q, [7, 6], 3)
    n = len(idx)
    say("paged attention over window + fetch", idx.tolist())
    out = wa.wa_paged_attention(run.L, to_device(q), run.k_pool, run.v_pool, idx_d, n,
                                to_device(ko), to_device(vo), wl.softmax_scale,
                                out_dtype=wa.WA_F32)
    torch.cuda.synchronize()
    k_ctx = np.concatenate([run.host_k[s] for s in idx])
    v_ctx = np.concatenate([run.host_v[s] for s in idx])
    ref, _ = oracle.attention(q, k_ctx, v_ctx, ko, vo, wl.softmax_scale)
    assert np.abs(to_f64(out) - ref).max() <= attention_tolerance(wl)


def test_window_full_size():
    """wan_kp4 at full size: the two most recent slots as the window plus the
    top 4 of the other 14 pages, then attention over the 6 pages in place
    (74,880 + 4,680 keys), sampled rows against the oracle."""
    wl = W.WORKLOADS["wan_kp4"]
    run = _pool(wl)
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    idx_d, idx = _window(run, q, [15, 14], 4)
    rows = rows_sample(wl.n_q, 10)
    say("paged attention, full size window", idx.tolist())
    out = wa.wa_paged_attention(run.L, to_device(q), run.k_pool, run.v_pool, idx_d, len(idx),
                                to_device(ko), to_device(vo), wl.softmax_scale,
                                out_dtype=wa.WA_BF16)
    torch.cuda.synchronize()
    k_ctx = np.concatenate([run.host_k[s] for s in idx])
    v_ctx = np.concatenate([run.host_v[s] for s in idx])
    ref, _ = oracle.attention(q, k_ctx, v_ctx, ko, vo, wl.softmax_scale, rows=rows)
    assert np.abs(to_f64(out)[rows] - ref).max() <= attention_tolerance(wl)
