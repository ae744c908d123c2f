"""Paged attention (pages read in place from the pool through idx) against the
gathered path and the oracle.

With the same pages in the same order, the paged call does the same
arithmetic on the same keys as wa_gather followed by wa_block_attention, so
the two must agree bit for bit; the oracle (attention over the gathered
pages, as the pages define it) bounds both.  Cases cover the whole-tile fast
path (page_tokens a multiple of 64), the per-row path (page_tokens not a
multiple of 64, context ending inside a tile), repeated ids, the launch that
splits few items over all CUs, fp32, and the full-size workload.
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


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def _pool(wl):
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    return run


def _compare(wl, run, idx, chunk=0, rows=None, out_dtypes=None):
    """Paged vs gathered (bitwise, out and lse) vs oracle (tolerance)."""
    k_p = len(idx)
    idx_d = torch.tensor(idx, dtype=torch.int32, device="cuda")
    q, ko, vo = W.chunk_qkv(wl, chunk, 0)
    qd, kod, vod = to_device(q), to_device(ko), to_device(vo)
    say("gather for paged comparison", wl.name, "idx", idx)
    k_ctx, v_ctx = wa.wa_gather(run.L, run.k_pool, run.v_pool, idx_d, k_p)
    k_ctx_h = np.concatenate([run.host_k[s] for s in idx])
    v_ctx_h = np.concatenate([run.host_v[s] for s in idx])
    ref, ref_lse = oracle.attention(q, k_ctx_h, v_ctx_h, ko, vo, wl.softmax_scale, rows=rows)
    tol = attention_tolerance(wl)
    if out_dtypes is None:
        out_dtypes = [wa.WA_F32] if wl.dtype == W.F32 else [wa.WA_F32, wa.WA_BF16]
    for odt in out_dtypes:
        lse_p = torch.empty(wl.n_heads, q.shape[0], dtype=torch.float32, device="cuda")
        lse_g = torch.empty_like(lse_p)
        say("paged attention", wl.name, "out_dtype", odt, "k_p", k_p, "page_tokens",
            wl.page_tokens, "n_q", q.shape[0])
        out_p = wa.wa_paged_attention(run.L, qd, run.k_pool, run.v_pool, idx_d, k_p, kod, vod,
                                      wl.softmax_scale, out_dtype=odt, lse=lse_p)
        say("gathered attention", wl.name, "out_dtype", odt)
        out_g = wa.wa_block_attention(run.L, qd, k_ctx, v_ctx, kod, vod, wl.softmax_scale,
                                      out_dtype=odt, lse=lse_g)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out_p), _bits(out_g)), "paged and gathered outputs differ"
        assert np.array_equal(_bits(lse_p), _bits(lse_g)), "paged and gathered lse differ"
        got = to_f64(out_p)
        got_lse = lse_p.cpu().double().numpy()
        if rows is not None:
            got, got_lse = got[rows], got_lse[:, rows]
        err = np.abs(got - ref).max()
        assert err <= tol, "paged attention max |err| %g > %g" % (err, tol)
        lerr = np.abs(got_lse - ref_lse).max()
        assert lerr <= tol, "paged lse max |err| %g" % lerr


def test_paged_whole_tile_pages_permuted_ids():
    """128-token pages (two 64-key tiles each), ids out of order."""
    wl = W.scaled(W.WORKLOADS["wan_kp4"], n_heads=2, frame_tokens=64, page_frames=2, n_pages=8,
                  chunk_frames=3, k_p=3)
    run = _pool(wl)
    _compare(wl, run, [5, 0, 3])


def test_paged_pages_not_a_multiple_of_the_tile():
    """100-token pages: the context ends inside a tile and tiles straddle pages
    (the per-row copy path)."""
    wl = W.scaled(W.WORKLOADS["wan_kp4"], n_heads=2, frame_tokens=50, page_frames=2, n_pages=6,
                  chunk_frames=3, k_p=3)
    run = _pool(wl)
    _compare(wl, run, [4, 1, 2])


def test_paged_repeated_ids_and_single_page():
    wl = W.scaled(W.WORKLOADS["wan_kp4"], n_heads=2, frame_tokens=64, page_frames=2, n_pages=4,
                  chunk_frames=2, k_p=3)
    run = _pool(wl)
    _compare(wl, run, [1, 1, 0])
    _compare(wl, run, [2])


def test_paged_split_launch_three_heads():
    """3 heads x 257 queries = 6 items over 37,697 keys: the launch splits the
    items' key tiles over all CUs and merges the pieces."""
    wl = W.scaled(W.WORKLOADS["wan_kp4"], n_heads=3, n_pages=4, k_p=3)
    run = _pool(wl)
    L = run.L
    assert wa.wa_attention_workspace_bytes(L, 257, 3 * wl.page_tokens, 257) > 0
    # 257 queries and own keys: the chunk's first rows
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    q, ko, vo = q[:257], ko[:257], vo[:257]
    idx = [2, 0, 3]
    idx_d = torch.tensor(idx, dtype=torch.int32, device="cuda")
    qd, kod, vod = to_device(q), to_device(ko), to_device(vo)
    k_ctx, v_ctx = wa.wa_gather(L, run.k_pool, run.v_pool, idx_d, 3)
    for odt in (wa.WA_F32, wa.WA_BF16):
        say("paged split", odt)
        out_p = wa.wa_paged_attention(L, qd, run.k_pool, run.v_pool, idx_d, 3, kod, vod,
                                      wl.softmax_scale, out_dtype=odt)
        out_g = wa.wa_block_attention(L, qd, k_ctx, v_ctx, kod, vod, wl.softmax_scale,
                                      out_dtype=odt)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out_p), _bits(out_g))
    rows = rows_sample(257, 24)
    k_ctx_h = np.concatenate([run.host_k[s] for s in idx])
    v_ctx_h = np.concatenate([run.host_v[s] for s in idx])
    ref, _ = oracle.attention(q, k_ctx_h, v_ctx_h, ko, vo, wl.softmax_scale, rows=rows)
    assert np.abs(to_f64(out_p)[rows] - ref).max() <= attention_tolerance(wl)


def test_paged_tiny_f32():
    wl = W.WORKLOADS["tiny_f32"]
    run = _pool(wl)
    _compare(wl, run, [6, 2])
    _compare(wl, run, [3, 3])


def test_paged_full_size_workload():
    """wan_kp4 at full size: 16 pages of 12,480 tokens, K_p 4, 4,680 queries;
    bitwise equal to the gathered path, sampled rows against the oracle."""
    wl = W.WORKLOADS["wan_kp4"]
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    _compare(wl, run, [11, 3, 14, 7], rows=rows_sample(wl.n_q, 12), out_dtypes=[wa.WA_BF16])


def test_paged_ids_outside_the_pool_stay_inside_it():
    """An id outside [0, max_pages) is clamped into the pool before any
    address is formed (the ABI leaves the result unspecified): the call
    completes and the output is finite, on both copy paths."""
    for ft in (64, 50):   # 128-token pages (whole tiles) and 100-token pages (per row)
        wl = W.scaled(W.WORKLOADS["wan_kp4"], n_heads=2, frame_tokens=ft, page_frames=2,
                      n_pages=4, chunk_frames=2, k_p=2)
        run = _pool(wl)
        q, ko, vo = W.chunk_qkv(wl, 0, 0)
        idx_d = torch.tensor([-1, 99], dtype=torch.int32, device="cuda")
        say("paged attention, ids outside the pool", wl.page_tokens)
        out = wa.wa_paged_attention(run.L, to_device(q), run.k_pool, run.v_pool, idx_d, 2,
                                    to_device(ko), to_device(vo), wl.softmax_scale,
                                    out_dtype=wa.WA_F32)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all())
