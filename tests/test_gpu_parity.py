"""HIP path vs the fp64 oracle, element by element, on the same seeded inputs.

Bars: page indices and candidate lists int-equal (order included); gathered
buffers bit-equal; attention max |err| <= 1e-5 (fp32 inputs) or <= 1e-2
(bf16 inputs, fp32 accumulation), on fp32 and bf16 outputs; lse within the
same bound.  Page means and scores are fp64 on both sides and must agree to
1e-12 (relative); the margin between the K_p-th and (K_p+1)-th score is
checked to be far above that, so index parity is meaningful.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_page_amd as wa
import wa_workloads as W
from tests.pipeline import (PoolRun, attention_tolerance, rows_sample, say, to_bits, to_device,
                            to_f64, wa_layout)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wa.load_library()


def check_means(run: PoolRun, slots):
    got = run.means[list(slots)].cpu().numpy()
    want = run.oracle_means(slots)
    err = np.abs(got - want).max()
    assert err <= 1e-12 * max(1.0, np.abs(want).max()), "page means differ by %g" % err


def check_select(run: PoolRun, q_host, q_dev, k_p, cand=None, prompt_dev=None, prompt_host=None):
    wl = run.wl
    n_cand = (len(cand) if cand is not None else
              (prompt_host["n_keep"] * prompt_host["chunk_pages"].shape[1] if prompt_host
               else wl.max_pages))
    scores = torch.empty(n_cand, dtype=torch.float64, device="cuda")
    cand_dev = torch.from_numpy(np.asarray(cand, np.int32)).cuda() if cand is not None else None
    say("select", wl.name, "k_p", k_p, "n_cand", n_cand)
    idx = wa.wa_select_pages(run.L, q_dev, run.means, k_p, cand=cand_dev, n_cand=n_cand,
                             prompt=prompt_dev, out_scores=scores)
    torch.cuda.synchronize()
    host_means = np.full((wl.max_pages, wl.n_heads, wl.head_dim), np.nan)
    for s in run.host_k:
        host_means[s] = oracle.page_mean(run.host_k[s])
    ref = oracle.select_pages(q_host, host_means, k_p, cand=cand, prompt=prompt_host)
    got_idx = idx.cpu().numpy()
    assert got_idx.tolist() == ref["idx"].tolist(), (got_idx, ref["idx"])
    got_scores = scores.cpu().numpy()
    serr = np.abs(got_scores - ref["alpha"]).max()
    assert serr <= 1e-12 * max(1.0, np.abs(ref["alpha"]).max()), "scores differ by %g" % serr
    margin = oracle.boundary_margin(ref["alpha"], k_p)
    assert margin > 1e-9 * np.abs(ref["alpha"]).max(), "selection margin too small: %g" % margin
    return idx, ref


def check_gather(run: PoolRun, idx_dev, k_p):
    say("gather", run.wl.name, "k_p", k_p)
    k_ctx, v_ctx = wa.wa_gather(run.L, run.k_pool, run.v_pool, idx_dev, k_p)
    torch.cuda.synchronize()
    idx = idx_dev.cpu().numpy()
    pool_k = np.stack([run.host_k[s] for s in sorted(run.host_k)])
    pool_v = np.stack([run.host_v[s] for s in sorted(run.host_v)])
    assert sorted(run.host_k) == list(range(len(run.host_k)))
    want_k = oracle.gather(pool_k, idx)
    want_v = oracle.gather(pool_v, idx)
    assert to_bits(k_ctx).tobytes() == want_k.tobytes()
    assert to_bits(v_ctx).tobytes() == want_v.tobytes()
    return k_ctx, v_ctx, want_k, want_v


def check_attention(wl, q, k_ctx_h, v_ctx_h, ko, vo, k_ctx_d, v_ctx_d, rows=None,
                    out_dtypes=None):
    L = wa_layout(wl)
    tol = attention_tolerance(wl)
    ref, ref_lse = oracle.attention(q, k_ctx_h, v_ctx_h, ko, vo, wl.softmax_scale, rows=rows)
    sel = slice(None) if rows is None else torch.from_numpy(rows)
    if out_dtypes is None:
        out_dtypes = [wa.WA_F32] if wl.dtype == W.F32 else [wa.WA_F32, wa.WA_BF16]
    qd, kod, vod = to_device(q), to_device(ko), to_device(vo)
    for odt in out_dtypes:
        lse = torch.empty(wl.n_heads, q.shape[0], dtype=torch.float32, device="cuda")
        say("attention", wl.name, "out_dtype", odt, "n_q", q.shape[0], "n_ctx",
            0 if k_ctx_d is None else k_ctx_d.shape[0], "n_own", ko.shape[0])
        out = wa.wa_block_attention(L, qd, k_ctx_d, v_ctx_d, kod, vod, wl.softmax_scale,
                                    out_dtype=odt, lse=lse)
        torch.cuda.synchronize()
        got = to_f64(out)[sel] if rows is not None else to_f64(out)
        err = np.abs(got - ref).max()
        assert err <= tol, "attention max |err| %g > %g (out dtype %d)" % (err, tol, odt)
        got_lse = lse.cpu().double().numpy()[:, sel] if rows is not None else lse.cpu().double().numpy()
        lerr = np.abs(got_lse - ref_lse).max()
        assert lerr <= tol, "lse max |err| %g" % lerr
    return ref


# ---------------------------------------------------------------------------

def test_tiny_f32_pipeline():
    """1 head, d 64, 32-token pages, 8 pages, 48 queries, K_p 2, fp32."""
    wl = W.WORKLOADS["tiny_f32"]
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    check_means(run, range(wl.n_pages))
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    idx, ref = check_select(run, q, to_device(q), wl.k_p)
    k_ctx, v_ctx, hk, hv = check_gather(run, idx, wl.k_p)
    check_attention(wl, q, hk, hv, ko, vo, k_ctx, v_ctx)


SMALL_BF16 = W.scaled(W.WORKLOADS["wan_kp4"], name="small_bf16", n_heads=2, frame_tokens=25,
                      n_pages=6, chunk_frames=12, k_p=3)   # P_t 200, N_q 300, N_k 900


def test_small_bf16_pipeline():
    """2 heads, d 128, 200-token pages; several key tiles, ragged key and query tails."""
    wl = SMALL_BF16
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    check_means(run, range(wl.n_pages))
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    idx, _ = check_select(run, q, to_device(q), wl.k_p)
    k_ctx, v_ctx, hk, hv = check_gather(run, idx, wl.k_p)
    check_attention(wl, q, hk, hv, ko, vo, k_ctx, v_ctx)


def test_wan_kp4_full_size_sampled_rows():
    """Wan2.1-1.3B-shaped layer: 12 heads, 12,480-token pages, 16 pages, K_p 4,
    4,680 queries, 49,920 + 4,680 keys, in the launch configuration the bench
    times.  Attention (fp32 and bf16 outputs, lse) checked on every row of one
    whole 256-query block and of the ragged last block (72 rows), for every
    head, plus 40 rows spread over the rest."""
    wl = W.WORKLOADS["wan_kp4"]
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    check_means(run, range(wl.n_pages))
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    idx, _ = check_select(run, q, to_device(q), wl.k_p)
    k_ctx, v_ctx, hk, hv = check_gather(run, idx, wl.k_p)
    block = np.arange(9 * 256, 10 * 256, dtype=np.int64)           # a whole interior block
    tail = np.arange((wl.n_q // 256) * 256, wl.n_q, dtype=np.int64)  # the ragged last block
    assert tail.size == 72
    rows = np.unique(np.concatenate([rows_sample(wl.n_q, 40), block, tail]))
    check_attention(wl, q, hk, hv, ko, vo, k_ctx, v_ctx, rows=rows)


@pytest.mark.parametrize("n_chunks", [16, 20])
def test_prompt_stage_pipeline(n_chunks):
    """Prompt stage over 16 (or 20) chunks of 4 pages (4,096-dim prompts), then
    the page stage over the 4 kept chunks' 16 pages; small pages keep the
    oracle fast.  64 pages in all take the one-launch selection, 80 the
    three-launch one."""
    wl = W.scaled(W.WORKLOADS["prompt_page"], name="prompt_small_%d" % n_chunks, n_heads=2,
                  frame_tokens=10, n_chunk_groups=n_chunks, n_pages=4 * n_chunks)
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    cp, cur = W.chunk_prompts(wl), W.current_prompt(wl)
    pages = W.chunk_page_map(wl)
    out_chunks = torch.empty(wl.n_cand_groups, dtype=torch.int32, device="cuda")
    out_cand = torch.empty(wl.n_cand_groups * wl.pages_per_group, dtype=torch.int32,
                           device="cuda")
    prompt_dev = dict(chunk_prompts=torch.from_numpy(cp).cuda(),
                      cur_prompt=torch.from_numpy(cur).cuda(),
                      chunk_pages=torch.from_numpy(pages).cuda(), n_keep=wl.n_cand_groups,
                      out_chunks=out_chunks, out_cand=out_cand)
    prompt_host = dict(chunk_prompts=cp, cur_prompt=cur, chunk_pages=pages,
                       n_keep=wl.n_cand_groups)
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    idx, ref = check_select(run, q, to_device(q), wl.k_p, prompt_dev=prompt_dev,
                            prompt_host=prompt_host)
    assert out_chunks.cpu().numpy().tolist() == ref["chunks"].tolist()
    assert out_cand.cpu().numpy().tolist() == ref["cand"].tolist()
    cos = ref["cos"]
    s = np.sort(cos)[::-1]
    assert s[wl.n_cand_groups - 1] - s[wl.n_cand_groups] > 1e-9
    k_ctx, v_ctx, hk, hv = check_gather(run, idx, wl.k_p)
    check_attention(wl, q, hk, hv, ko, vo, k_ctx, v_ctx)


def test_full_history_steps():
    """K_p = all pages (6 of 6), 4 denoising steps with fresh queries and own K/V
    over the same gathered pages; full-size shapes, sampled rows.  Also checks
    that all pages selected equals attention over the temporal history."""
    wl = W.WORKLOADS["full_history"]
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    q0, _, _ = W.chunk_qkv(wl, 0, 0)
    idx, ref = check_select(run, q0, to_device(q0), wl.k_p)
    assert sorted(ref["idx"].tolist()) == list(range(wl.n_pages))
    k_ctx, v_ctx, hk, hv = check_gather(run, idx, wl.k_p)
    hist_k = np.concatenate([run.host_k[j] for j in range(wl.n_pages)])
    hist_v = np.concatenate([run.host_v[j] for j in range(wl.n_pages)])
    rows = rows_sample(wl.n_q, 12)
    for step in range(wl.steps):
        q, ko, vo = W.chunk_qkv(wl, 0, step)
        got = check_attention(wl, q, hk, hv, ko, vo, k_ctx, v_ctx, rows=rows,
                              out_dtypes=[wa.WA_BF16, wa.WA_F32])
        if step == 0:
            hist, _ = oracle.attention(q, hist_k, hist_v, ko, vo, wl.softmax_scale, rows=rows)
            assert np.abs(hist - got).max() < 1e-12


def test_long_horizon_chunks():
    """128 resident pages (9.8 GB of bf16 K/V), then 8 chunks in sequence: the
    page stage over every page in the pool, gather, 4 denoising steps with
    fresh queries and own K/V, then one new page appended.  Full-size shapes;
    attention on sampled rows.  No host copy of the pool is kept: the oracle's
    page means are taken as pages are drawn, and the selected pages are drawn
    again from their seeds for the gather and attention checks."""
    wl = W.WORKLOADS["long_horizon"]
    run = PoolRun(wl, keep_host_pages=False)
    host_means = np.full((wl.max_pages, wl.n_heads, wl.head_dim), np.nan)

    def append(page):
        k, _ = run.append(page)
        host_means[page] = oracle.page_mean(k)

    for j in range(wl.n_pages):
        append(j)
    rows = rows_sample(wl.n_q, 6)
    tol = attention_tolerance(wl)
    for c in range(wl.chunks):
        n_live = wl.n_pages + c * wl.appended_per_chunk
        got_means = run.means[:n_live].cpu().numpy()
        merr = np.abs(got_means - host_means[:n_live]).max()
        assert merr <= 1e-12 * max(1.0, np.abs(host_means[:n_live]).max())
        q0, _, _ = W.chunk_qkv(wl, c, 0)
        scores = torch.empty(n_live, dtype=torch.float64, device="cuda")
        say("long horizon chunk", c, "select over", n_live, "pages")
        idx = wa.wa_select_pages(run.L, to_device(q0), run.means, wl.k_p, n_cand=n_live,
                                 out_scores=scores)
        ref = oracle.select_pages(q0, host_means[:n_live], wl.k_p)
        assert idx.cpu().numpy().tolist() == ref["idx"].tolist()
        assert oracle.boundary_margin(ref["alpha"], wl.k_p) > 1e-9 * np.abs(ref["alpha"]).max()
        say("long horizon chunk", c, "gather", ref["idx"].tolist())
        k_ctx, v_ctx = wa.wa_gather(run.L, run.k_pool, run.v_pool, idx, wl.k_p)
        drawn = [W.page_kv(wl, int(j)) for j in ref["idx"]]
        hk = np.concatenate([d[0] for d in drawn])
        hv = np.concatenate([d[1] for d in drawn])
        del drawn
        assert to_bits(k_ctx).tobytes() == hk.tobytes()
        assert to_bits(v_ctx).tobytes() == hv.tobytes()
        for step in range(wl.steps):
            q, ko, vo = W.chunk_qkv(wl, c, step)
            ref_out, ref_lse = oracle.attention(q, hk, hv, ko, vo, wl.softmax_scale, rows=rows)
            # bf16 outputs every step, fp32 outputs and lse on the chunk's first step
            for odt in ([wa.WA_BF16, wa.WA_F32] if step == 0 else [wa.WA_BF16]):
                say("long horizon chunk", c, "step", step, "attention, out dtype", odt)
                lse = torch.empty(wl.n_heads, wl.n_q, dtype=torch.float32, device="cuda")
                out = wa.wa_block_attention(run.L, to_device(q), k_ctx, v_ctx, to_device(ko),
                                            to_device(vo), wl.softmax_scale, out_dtype=odt,
                                            lse=lse)
                err = np.abs(to_f64(out)[rows] - ref_out).max()
                assert err <= tol, "chunk %d step %d: attention max |err| %g" % (c, step, err)
                lerr = np.abs(lse.cpu().double().numpy()[:, rows] - ref_lse).max()
                assert lerr <= tol, "chunk %d step %d: lse max |err| %g" % (c, step, lerr)
        del k_ctx, v_ctx, hk, hv
        append(wl.n_pages + c)
    got_means = run.means.cpu().numpy()
    assert np.abs(got_means - host_means).max() <= 1e-12 * max(1.0, np.abs(host_means).max())


def test_prompt_page_full_size():
    """Prompt stage at full size: 64 pages of 12,480 tokens in 16 chunks of 4,
    4,096-dim prompts, the top 4 chunks' 16 pages scored, K_p 4, then gather
    and attention on sampled rows.  The selected pages are drawn again from
    their seeds for the oracle."""
    wl = W.WORKLOADS["prompt_page"]
    run = PoolRun(wl, keep_host_pages=False)
    host_means = np.full((wl.max_pages, wl.n_heads, wl.head_dim), np.nan)
    for j in range(wl.n_pages):
        k, _ = run.append(j)
        host_means[j] = oracle.page_mean(k)
    cp, cur = W.chunk_prompts(wl), W.current_prompt(wl)
    pages = W.chunk_page_map(wl)
    n_cand = wl.n_cand_groups * wl.pages_per_group
    out_chunks = torch.empty(wl.n_cand_groups, dtype=torch.int32, device="cuda")
    out_cand = torch.empty(n_cand, dtype=torch.int32, device="cuda")
    prompt_dev = dict(chunk_prompts=torch.from_numpy(cp).cuda(),
                      cur_prompt=torch.from_numpy(cur).cuda(),
                      chunk_pages=torch.from_numpy(pages).cuda(), n_keep=wl.n_cand_groups,
                      out_chunks=out_chunks, out_cand=out_cand)
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    scores = torch.empty(n_cand, dtype=torch.float64, device="cuda")
    say("prompt stage full size: select")
    idx = wa.wa_select_pages(run.L, to_device(q), run.means, wl.k_p, prompt=prompt_dev,
                             out_scores=scores)
    ref = oracle.select_pages(q, host_means, wl.k_p,
                              prompt=dict(chunk_prompts=cp, cur_prompt=cur, chunk_pages=pages,
                                          n_keep=wl.n_cand_groups))
    assert out_chunks.cpu().numpy().tolist() == ref["chunks"].tolist()
    assert out_cand.cpu().numpy().tolist() == ref["cand"].tolist()
    assert idx.cpu().numpy().tolist() == ref["idx"].tolist()
    serr = np.abs(scores.cpu().numpy() - ref["alpha"]).max()
    assert serr <= 1e-12 * max(1.0, np.abs(ref["alpha"]).max())
    say("prompt stage full size: gather", ref["idx"].tolist())
    k_ctx, v_ctx = wa.wa_gather(run.L, run.k_pool, run.v_pool, idx, wl.k_p)
    drawn = [W.page_kv(wl, int(j)) for j in ref["idx"]]
    hk = np.concatenate([d[0] for d in drawn])
    hv = np.concatenate([d[1] for d in drawn])
    assert to_bits(k_ctx).tobytes() == hk.tobytes()
    assert to_bits(v_ctx).tobytes() == hv.tobytes()
    rows = rows_sample(wl.n_q, 8)
    check_attention(wl, q, hk, hv, ko, vo, k_ctx, v_ctx, rows=rows,
                    out_dtypes=[wa.WA_BF16, wa.WA_F32])
