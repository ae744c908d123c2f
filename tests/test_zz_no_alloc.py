"""wa_select_pages_noalloc -- the page selection with the library's fixed
per-device workspace, for callers that cannot allocate -- against
wa_select_pages with a caller-owned workspace, through the C ABI: calls in a
row, each with a smaller input than the one before (100 listed candidates,
which take the two-level one-launch path; all 12 pages; fewer queries and 6
listed candidates with a repeated id), then the prompt stage.  The two entry
points run the same kernels in the same order, so ids and scores must be
bit for bit equal.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_page_amd as wa
import wa_workloads as W
from tests.pipeline import PoolRun, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wa.load_library()


def _same(a, b):
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())


def test_noalloc_selection_equals_the_workspace_call():
    wl = W.scaled(W.WORKLOADS["wan_kp4"], name="noalloc", n_heads=4, frame_tokens=200,
                  n_pages=12, chunk_frames=6, k_p=4)       # 1,600-token pages, 1,200 queries
    run = PoolRun(wl, keep_host_pages=False)
    for j in range(wl.n_pages):
        run.append(j)
    q, _, _ = W.chunk_qkv(wl, 0, 0)
    qd = to_device(q)
    small = torch.tensor([7, 2, 9, 2, 11, 0], dtype=torch.int32, device="cuda")
    many = torch.from_numpy(np.random.default_rng(3).integers(0, wl.n_pages, 100)
                            .astype(np.int32)).cuda()
    cases = [("100 listed candidates (ids repeated), 1,200 queries", qd, many, 100, 5),
             ("all 12 pages, 1,200 queries", qd, None, wl.n_pages, 4),
             ("6 listed candidates, 300 queries", qd[:300].contiguous(), small, 6, 3)]
    for name, qq, cand, n_cand, k_p in cases:
        say("select noalloc:", name)
        ref_s = torch.empty(n_cand, dtype=torch.float64, device="cuda")
        got_s = torch.full((n_cand,), float("nan"), dtype=torch.float64, device="cuda")
        got_i = torch.full((k_p,), -7, dtype=torch.int32, device="cuda")
        ref_i = wa.wa_select_pages(run.L, qq, run.means, k_p, cand=cand, n_cand=n_cand,
                                   out_scores=ref_s)
        wa.wa_select_pages_noalloc(run.L, qq, run.means, k_p, cand=cand, n_cand=n_cand,
                                   out_idx=got_i, out_scores=got_s)
        _same(got_i, ref_i)
        _same(got_s.view(torch.int64), ref_s.view(torch.int64))

    # the prompt stage (its workspace also holds the chunk cosines)
    pw = W.scaled(W.WORKLOADS["prompt_page"], name="noalloc_prompt", n_heads=2, frame_tokens=10)
    prun = PoolRun(pw, keep_host_pages=False)
    for j in range(pw.n_pages):
        prun.append(j)
    pq, _, _ = W.chunk_qkv(pw, 0, 0)
    prompt = dict(chunk_prompts=torch.from_numpy(W.chunk_prompts(pw)).cuda(),
                  cur_prompt=torch.from_numpy(W.current_prompt(pw)).cuda(),
                  chunk_pages=torch.from_numpy(W.chunk_page_map(pw)).cuda(),
                  n_keep=pw.n_cand_groups)
    say("select noalloc: prompt stage")
    ref_i = wa.wa_select_pages(prun.L, to_device(pq), prun.means, pw.k_p, prompt=prompt)
    got_i = wa.wa_select_pages_noalloc(prun.L, to_device(pq), prun.means, pw.k_p, prompt=prompt)
    _same(got_i, ref_i)
