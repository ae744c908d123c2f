"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test checks one step against a closed form, an invariant of the
definition, brute force on tiny inputs, or a textbook library routine, so
that a dropped term, a wrong sign, a wrong index or a transposed operand in
``oracle/wa_oracle.c`` fails at least one of them (``test_oracle_mutations``
plants such mistakes and checks that).
"""
import itertools
import math

import numpy as np
import pytest
import torch

import wa_workloads as W

RNG = np.random.default_rng(20261202)


def f32(*shape):
    return RNG.standard_normal(shape).astype(np.float32)


# ----------------------------------------------------------------------------
# page mean key / chunk mean query (WorldAttention review, "HKV")

def test_mean_of_constant_page_is_exact(oracle_lib):
    x = np.full((37, 3, 8), 0.7578125, dtype=np.float32)   # exact in fp32 and bf16
    assert np.array_equal(oracle_lib.column_mean(x), np.full((3, 8), 0.7578125))
    xb = W.f32_to_bf16_bits(x)
    assert np.array_equal(oracle_lib.column_mean(xb), np.full((3, 8), 0.7578125))


def test_mean_matches_exactly_rounded_sum(oracle_lib):
    x = f32(29, 2, 16)
    got = oracle_lib.column_mean(x)
    for h in range(2):
        for c in range(16):
            exact = math.fsum(float(t) for t in x[:, h, c]) / 29
            assert abs(got[h, c] - exact) <= 1e-15 * max(1.0, abs(exact))


def test_mean_is_linear_in_the_page_offset(oracle_lib):
    wl = W.WORKLOADS["tiny_f32"]
    raw = f32(32, 1, 64).astype(np.float64)
    u = W.offset_direction(wl).astype(np.float64)
    c = 3.5
    shifted = (raw + c * u).astype(np.float32)
    got = oracle_lib.column_mean(shifted)
    want = raw.mean(axis=0) + c * u
    assert np.abs(got - want).max() < 1e-6       # float32 rounding of the shifted page


def test_mean_reads_bf16_patterns_exactly(oracle_lib):
    # 1.0, -2.0, 0.5, 3.0 as bf16
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x4040], dtype=np.uint16).reshape(4, 1, 1)
    assert oracle_lib.column_mean(bits)[0, 0] == (1.0 - 2.0 + 0.5 + 3.0) / 4


# ----------------------------------------------------------------------------
# page-stage score

def test_score_is_mean_of_all_pairwise_dots(oracle_lib):
    """Bilinearity: qbar . kbar_j / sqrt(d) = (1/(N_q P_t sqrt(d))) sum_i sum_t q_i . k_t."""
    H, d, nq, pt, npages = 3, 16, 7, 5, 4
    q = f32(nq, H, d)
    pages = f32(npages, pt, H, d)
    qbar = oracle_lib.mean_query(q)
    means = np.stack([oracle_lib.page_mean(pages[j]) for j in range(npages)])
    cand = np.array([2, 0, 3], dtype=np.int32)
    alpha = oracle_lib.page_scores(qbar, means, cand)
    for n, j in enumerate(cand):
        brute = 0.0
        for i in range(nq):
            for t in range(pt):
                brute += float(np.dot(q[i].astype(np.float64).ravel(),
                                      pages[j, t].astype(np.float64).ravel()))
        brute /= nq * pt * math.sqrt(d)
        assert abs(alpha[n] - brute) < 1e-12 * max(1.0, abs(brute))


def test_score_closed_form_for_constant_pages(oracle_lib):
    """Pages whose keys all equal c_j u and queries all equal u: alpha_j = c_j H / sqrt(d)."""
    H, d = 2, 16
    u = np.zeros(d, dtype=np.float32)
    u[3] = 1.0
    q = np.broadcast_to(u, (5, H, d)).copy()
    cs = [0.5, -1.5, 2.0]
    means = np.stack([oracle_lib.page_mean(np.broadcast_to(np.float32(c) * u, (4, H, d)).copy())
                      for c in cs])
    alpha = oracle_lib.page_scores(oracle_lib.mean_query(q), means, np.arange(3, dtype=np.int32))
    np.testing.assert_allclose(alpha, [c * H / 4.0 for c in cs], rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------
# top-K_p

@pytest.mark.parametrize("n,k", [(8, 2), (6, 3), (10, 4), (5, 5), (7, 1)])
def test_top_k_is_the_best_subset_by_brute_force(oracle_lib, n, k):
    for trial in range(5):
        score = RNG.standard_normal(n)
        ids = RNG.permutation(100)[:n].astype(np.int32)
        got = oracle_lib.top_k(score, ids, k)
        best = max(itertools.combinations(range(n), k), key=lambda s: sum(score[j] for j in s))
        assert set(got.tolist()) == {int(ids[j]) for j in best}
        # rank order: scores strictly descending along the output
        pos = {int(i): j for j, i in enumerate(ids)}
        s_out = [score[pos[int(i)]] for i in got]
        assert all(a > b for a, b in zip(s_out, s_out[1:]))


def test_top_k_tie_goes_to_lower_id(oracle_lib):
    score = np.array([1.0, 2.0, 2.0, 0.5, 2.0])
    ids = np.array([9, 7, 3, 1, 5], dtype=np.int32)
    assert oracle_lib.top_k(score, ids, 3).tolist() == [3, 5, 7]
    assert oracle_lib.top_k(score, ids, 5).tolist() == [3, 5, 7, 9, 1]


def test_top_k_all_returns_every_id(oracle_lib):
    score = RNG.standard_normal(9)
    ids = np.arange(9, dtype=np.int32)
    got = oracle_lib.top_k(score, ids, 9)
    assert sorted(got.tolist()) == list(range(9))
    assert got.tolist() == sorted(range(9), key=lambda j: (-score[j], j))


# ----------------------------------------------------------------------------
# sliding window plus selective fetch (Inferix summary, "Dual access patterns")

def _constant_pool(values, H=2, d=8):
    """Page j's keys all equal values[j]: its mean is values[j] everywhere."""
    return np.stack([np.full((H, d), v, dtype=np.float64) for v in values])


def test_window_closed_form_on_constant_pages(oracle_lib):
    """With q = 1 everywhere, alpha_j = values[j] * H * d / sqrt(d), so the
    ranking is the order of values: 5, 1, 3, 7, 4, 0, 6, 2.  The window keeps
    its own order, its best page (5) is not fetched again, and the fetched
    pages are the next best outside the window."""
    values = [0.3, 2.0, -1.0, 1.5, 0.7, 2.5, 0.1, 1.2]
    means = _constant_pool(values)
    q = np.ones((4, 2, 8), dtype=np.float32)
    got = oracle_lib.select_window(q, means, 3, [6, 5])
    assert got["idx"].tolist() == [6, 5, 1, 3, 7]
    assert np.allclose(got["alpha"], np.array(values) * 2 * 8 / math.sqrt(8))
    assert oracle_lib.select_window(q, means, 0, [2, 0])["idx"].tolist() == [2, 0]
    assert oracle_lib.select_window(q, means, 2, [])["idx"].tolist() == [5, 1]


def test_window_empty_is_the_page_stage(oracle_lib):
    means = RNG.standard_normal((9, 2, 8))
    q = f32(5, 2, 8)
    for k in (1, 4, 9):
        assert (oracle_lib.select_window(q, means, k, [])["idx"].tolist()
                == oracle_lib.select_pages(q, means, k)["idx"].tolist())


@pytest.mark.parametrize("n,w,k", [(7, 2, 3), (8, 3, 2), (6, 1, 5), (9, 4, 1)])
def test_window_fetch_is_the_best_subset_outside_the_window(oracle_lib, n, w, k):
    for trial in range(4):
        means = RNG.standard_normal((n, 2, 8))
        q = f32(3, 2, 8)
        window = RNG.permutation(n)[:w].astype(np.int32)
        res = oracle_lib.select_window(q, means, k, window)
        idx, alpha = res["idx"], res["alpha"]
        assert idx[:w].tolist() == window.tolist()
        rest = [j for j in range(n) if j not in set(window.tolist())]
        kk = min(k, len(rest))
        best = max(itertools.combinations(rest, kk), key=lambda s: sum(alpha[j] for j in s))
        assert set(idx[w:w + kk].tolist()) == set(best)
        assert idx[w + kk:].tolist() == [-1] * (k - kk)
        s_out = [alpha[j] for j in idx[w:w + kk]]
        assert all(a > b for a, b in zip(s_out, s_out[1:]))


def test_window_covering_every_candidate_fetches_nothing(oracle_lib):
    means = RNG.standard_normal((4, 2, 8))
    q = f32(3, 2, 8)
    got = oracle_lib.select_window(q, means, 2, [3, 1, 0, 2])
    assert got["idx"].tolist() == [3, 1, 0, 2, -1, -1]


def test_window_order_only_moves_the_window(oracle_lib):
    means = RNG.standard_normal((10, 2, 8))
    q = f32(3, 2, 8)
    a = oracle_lib.select_window(q, means, 3, [7, 2, 9])["idx"]
    b = oracle_lib.select_window(q, means, 3, [9, 7, 2])["idx"]
    assert b[:3].tolist() == [9, 7, 2] and a[3:].tolist() == b[3:].tolist()


# ----------------------------------------------------------------------------
# prompt stage

def test_cosine_closed_forms(oracle_lib):
    a = f32(64)
    b = f32(64)
    e0 = np.zeros(64, np.float32); e0[0] = 1
    e1 = np.zeros(64, np.float32); e1[1] = 1
    cp = np.stack([a, 3.0 * a, -a, b, e1])
    cos = oracle_lib.prompt_cosine(cp, a)
    assert abs(cos[0] - 1) < 1e-15 and abs(cos[1] - 1) < 1e-15 and abs(cos[2] + 1) < 1e-15
    want_b = float(np.dot(a.astype(np.float64), b)) / (np.linalg.norm(a.astype(np.float64))
                                                       * np.linalg.norm(b.astype(np.float64)))
    assert abs(cos[3] - want_b) < 1e-14
    assert oracle_lib.prompt_cosine(np.stack([e1]), e0)[0] == 0.0


def test_zero_norm_prompt_ranks_last(oracle_lib):
    """Reading: a prompt embedding of zero norm has no direction, so its
    cosine is -inf.  A zero chunk prompt ranks after every other chunk (two
    such chunks in id order); a zero current prompt leaves every chunk at -inf,
    so the kept chunks are the lowest ids."""
    a, b, c = f32(32), f32(32), f32(32)
    z = np.zeros(32, np.float32)
    cp = np.stack([z, a, z, b, c])
    cos = oracle_lib.prompt_cosine(cp, a)
    assert np.isneginf(cos[0]) and np.isneginf(cos[2]) and np.isfinite(cos[[1, 3, 4]]).all()
    pages = np.arange(10, dtype=np.int32).reshape(5, 2)
    chunks, cand = oracle_lib.prompt_candidates(cos, pages, 5)
    assert chunks.tolist()[:3] == sorted([1, 3, 4], key=lambda m: (-cos[m], m))
    assert chunks.tolist()[3:] == [0, 2]
    assert cand.tolist() == [p for m in chunks for p in (2 * m, 2 * m + 1)]
    cos0 = oracle_lib.prompt_cosine(cp, z)
    assert np.isneginf(cos0).all()
    assert oracle_lib.prompt_candidates(cos0, pages, 3)[0].tolist() == [0, 1, 2]


def test_prompt_stage_recalls_the_matching_chunk(oracle_lib):
    """A current prompt equal to past chunk m0's prompt ranks m0 first."""
    wl = W.scaled(W.WORKLOADS["prompt_page"], emb_dim=256)
    cp = W.chunk_prompts(wl)
    m0 = 11
    cos = oracle_lib.prompt_cosine(cp, cp[m0])
    chunks, cand = oracle_lib.prompt_candidates(cos, W.chunk_page_map(wl), 4)
    assert chunks[0] == m0
    assert cand[:4].tolist() == [44, 45, 46, 47]
    # the rest follow by descending cosine (brute-force sort of the same cosines)
    assert chunks.tolist() == sorted(range(16), key=lambda m: (-cos[m], m))[:4]
    assert cand.tolist() == [p for m in chunks for p in range(4 * m, 4 * m + 4)]


# ----------------------------------------------------------------------------
# gather

def test_gather_identity_reproduces_the_pool(oracle_lib):
    pool = W.f32_to_bf16_bits(f32(5, 6, 2, 8))
    out = oracle_lib.gather(pool, np.arange(5, dtype=np.int32))
    assert out.tobytes() == pool.tobytes()


def test_gather_matches_fancy_indexing(oracle_lib):
    pool = f32(7, 4, 3, 8)
    idx = np.array([6, 2, 2, 0], dtype=np.int32)
    out = oracle_lib.gather(pool, idx)
    assert out.tobytes() == pool[idx].reshape(16, 3, 8).tobytes()


# ----------------------------------------------------------------------------
# block attention (Inferix, section 3.4, Step 3)

def _sdpa(q, k, v, scale):
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2)
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], scale=scale)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("scale", [1.0 / 8.0, 0.37])
def test_attention_matches_textbook_sdpa(oracle_lib, scale):
    H, d = 2, 32
    q, kc, vc, ko, vo = f32(9, H, d), f32(13, H, d), f32(13, H, d), f32(9, H, d), f32(9, H, d)
    out, _ = oracle_lib.attention(q, kc, vc, ko, vo, scale)
    ref = _sdpa(q, np.concatenate([kc, ko]), np.concatenate([vc, vo]), scale)
    assert np.abs(out - ref).max() < 1e-13


def test_attention_bf16_matches_sdpa_on_widened_values(oracle_lib):
    H, d = 3, 16
    xs = [W.f32_to_bf16_bits(f32(n, H, d)) for n in (6, 10, 10, 6, 6)]
    q, kc, vc, ko, vo = xs
    out, _ = oracle_lib.attention(q, kc, vc, ko, vo, 0.25)
    w = [W.bf16_bits_to_f32(x) for x in xs]
    ref = _sdpa(w[0], np.concatenate([w[1], w[3]]), np.concatenate([w[2], w[4]]), 0.25)
    assert np.abs(out - ref).max() < 1e-13


def test_attention_unit_values_give_unit_output(oracle_lib):
    H, d = 2, 16
    q, kc, ko = f32(5, H, d), f32(11, H, d), f32(5, H, d)
    ones_c, ones_o = np.ones((11, H, d), np.float32), np.ones((5, H, d), np.float32)
    out, _ = oracle_lib.attention(q, kc, ones_c, ko, ones_o, 0.3)
    assert np.abs(out - 1.0).max() < 1e-14


def test_attention_zero_query_averages_all_values(oracle_lib):
    H, d = 2, 16
    q = np.zeros((4, H, d), np.float32)
    kc, vc, ko, vo = f32(7, H, d), f32(7, H, d), f32(4, H, d), f32(4, H, d)
    out, lse = oracle_lib.attention(q, kc, vc, ko, vo, 0.5)
    want = np.concatenate([vc, vo]).astype(np.float64).mean(axis=0)
    assert np.abs(out - want[None]).max() < 1e-14
    assert np.abs(lse - math.log(11)).max() < 1e-14


def test_attention_single_key_returns_its_value(oracle_lib):
    H, d = 2, 8
    q, k, v = f32(3, H, d), f32(1, H, d), f32(1, H, d)
    out, lse = oracle_lib.attention(q, None, None, k, v, 0.5)
    assert np.array_equal(out, np.broadcast_to(v.astype(np.float64), out.shape))
    s = 0.5 * np.einsum("qhd,hd->hq", q.astype(np.float64), k[0].astype(np.float64))
    assert np.abs(lse - s).max() < 1e-14


def test_attention_lse_normalises_the_scores(oracle_lib):
    H, d = 2, 16
    q, kc, vc, ko, vo = f32(6, H, d), f32(9, H, d), f32(9, H, d), f32(6, H, d), f32(6, H, d)
    _, lse = oracle_lib.attention(q, kc, vc, ko, vo, 0.25)
    k = np.concatenate([kc, ko]).astype(np.float64)
    s = 0.25 * np.einsum("qhd,khd->hqk", q.astype(np.float64), k)
    assert np.abs(np.exp(s - lse[:, :, None]).sum(-1) - 1).max() < 1e-13


def test_attention_invariant_to_page_order_and_split(oracle_lib):
    H, d, pt = 2, 16, 6
    pages = [f32(pt, H, d) for _ in range(4)]
    vals = [f32(pt, H, d) for _ in range(4)]
    q, ko, vo = f32(5, H, d), f32(5, H, d), f32(5, H, d)
    base, _ = oracle_lib.attention(q, np.concatenate(pages), np.concatenate(vals), ko, vo, 0.25)
    order = [2, 0, 3, 1]
    perm, _ = oracle_lib.attention(q, np.concatenate([pages[i] for i in order]),
                                   np.concatenate([vals[i] for i in order]), ko, vo, 0.25)
    assert np.abs(base - perm).max() < 1e-13
    # moving the ctx/own boundary does not change the concatenated sequence
    allk = np.concatenate(pages + [ko])
    allv = np.concatenate(vals + [vo])
    for cut in (0, 7, 24, allk.shape[0]):
        o, _ = oracle_lib.attention(q, allk[:cut], allv[:cut], allk[cut:], allv[cut:], 0.25)
        assert np.abs(o - base).max() < 1e-13


def test_attention_row_subset_equals_full_rows(oracle_lib):
    H, d = 1, 8
    q, kc, vc, ko, vo = f32(10, H, d), f32(5, H, d), f32(5, H, d), f32(10, H, d), f32(10, H, d)
    full, lse_full = oracle_lib.attention(q, kc, vc, ko, vo, 0.4)
    rows = np.array([9, 0, 4])
    sub, lse_sub = oracle_lib.attention(q, kc, vc, ko, vo, 0.4, rows=rows)
    assert np.array_equal(sub, full[rows]) and np.array_equal(lse_sub, lse_full[:, rows])


def test_full_history_equals_all_pages_selected(oracle_lib):
    """K_p = all pages reproduces attention over the whole temporal history."""
    wl = W.scaled(W.WORKLOADS["tiny_f32"], n_pages=4, k_p=4)
    pages = [W.page_kv(wl, j) for j in range(4)]
    pool_k = np.stack([p[0] for p in pages])
    pool_v = np.stack([p[1] for p in pages])
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    means = np.stack([oracle_lib.page_mean(pool_k[j]) for j in range(4)])
    sel = oracle_lib.select_pages(q, means, 4)
    assert sorted(sel["idx"].tolist()) == [0, 1, 2, 3]
    kc, vc = oracle_lib.gather(pool_k, sel["idx"]), oracle_lib.gather(pool_v, sel["idx"])
    got, _ = oracle_lib.attention(q, kc, vc, ko, vo, wl.softmax_scale)
    hist_k = np.concatenate([pool_k.reshape(-1, 1, 64), ko])
    hist_v = np.concatenate([pool_v.reshape(-1, 1, 64), vo])
    ref = _sdpa(q, hist_k, hist_v, wl.softmax_scale)
    assert np.abs(got - ref).max() < 1e-13


# ----------------------------------------------------------------------------
# whole chunk on the small workload: margins hold far above fp64 rounding

def test_tiny_workload_selection_has_a_clear_margin(oracle_lib):
    wl = W.WORKLOADS["tiny_f32"]
    pool_k = np.stack([W.page_kv(wl, j)[0] for j in range(wl.n_pages)])
    means = np.stack([oracle_lib.page_mean(pool_k[j]) for j in range(wl.n_pages)])
    q, _, _ = W.chunk_qkv(wl, 0, 0)
    sel = oracle_lib.select_pages(q, means, wl.k_p)
    margin = oracle_lib.boundary_margin(sel["alpha"], wl.k_p)
    assert margin > 1e-6 * np.abs(sel["alpha"]).max()


# ----------------------------------------------------------------------------
# HSA sparse branch (WorldAttention review, "HSA: Dual Branches of Linear +
# Sparse"): key blocks, pooled map, Gini coefficient, cumulative-mass
# selection, attention over the selected blocks

def test_gini_closed_forms(oracle_lib):
    assert oracle_lib.gini(np.full(6, 0.25)) == 0.0
    assert abs(oracle_lib.gini([0, 0, 1.0, 0, 0]) - 4 / 5) < 1e-15      # one-hot: (n-1)/n
    assert abs(oracle_lib.gini([1.0, 3.0]) - 0.25) < 1e-15               # |1-3|*2 / (2*2*4)
    p = RNG.random(9)
    assert abs(oracle_lib.gini(p) - oracle_lib.gini(7.5 * p)) < 1e-14    # scale invariant


@pytest.mark.parametrize("n", [5, 7, 8])
def test_select_blocks_is_the_fewest_by_brute_force(oracle_lib, n):
    for trial in range(6):
        mass = RNG.random(n)
        mass /= mass.sum()
        tau = float(RNG.uniform(0.05, 0.95))
        got = oracle_lib.select_blocks(mass, tau)
        m = len(got)
        reach = [k for k in range(1, n + 1)
                 if any(sum(mass[j] for j in s) >= tau for s in itertools.combinations(range(n), k))]
        assert m == min(reach)
        best = max(itertools.combinations(range(n), m), key=lambda s: sum(mass[j] for j in s))
        assert got == sorted(best)
    mass = np.array([0.1, 0.5, 0.2, 0.2])
    assert oracle_lib.select_blocks(mass, 0.3) == [1]                    # the largest alone
    assert oracle_lib.select_blocks(mass, 2.0) == [0, 1, 2, 3]            # unreachable: all
    assert oracle_lib.select_blocks(mass, 0.0) == [1]                    # at least one block
    assert oracle_lib.select_blocks(mass, -1.0) == [1]
    assert oracle_lib.select_blocks(mass, 0.7) == [1, 2]                  # tie 0.2/0.2 -> lower index


def test_key_blocks_cover_every_key_once(oracle_lib):
    got = oracle_lib.hsa_key_blocks(300, 130)
    assert got == [(0, 128), (128, 256), (256, 300), (300, 364), (364, 428), (428, 430)]
    assert oracle_lib.hsa_key_blocks(0, 64) == [(0, 64)]


def test_pooled_map_closed_form(oracle_lib):
    """Keys of block j all equal c_j e, queries all equal a e: the block means
    are c_j e and a e, so the map row is softmax_j(a c_j |e|^2 scale)."""
    d, H = 8, 2
    e = np.arange(1, d + 1, dtype=np.float32) / 8
    c = [0.5, -1.0, 2.0, 0.25]
    blocks = oracle_lib.hsa_key_blocks(3 * 16, 16, b_inter=16, b_intra=16)
    k = np.concatenate([np.tile(cj * e, (16, H, 1)) for cj in c]).astype(np.float32)
    q = np.tile(0.75 * e, (5, H, 1)).astype(np.float32)
    got = oracle_lib.hsa_pooled_map(q, k, blocks, 0.3)
    s = np.array([0.75 * cj * float(e @ e) * 0.3 for cj in c])
    want = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    assert np.allclose(got, np.tile(want, (H, 1)), rtol=1e-12, atol=0)


def _hsa_inputs(n_q=300, n_ctx=384, n_own=140, H=2, d=16):
    return f32(n_q, H, d), f32(n_ctx, H, d), f32(n_ctx, H, d), f32(n_own, H, d), f32(n_own, H, d)


def test_hsa_every_block_is_dense_attention(oracle_lib):
    q, kc, vc, ko, vo = _hsa_inputs()
    r = oracle_lib.hsa_sparse(q, kc, vc, ko, vo, 0.25, [2.0, 2.0])
    dense, lse = oracle_lib.attention(q, kc, vc, ko, vo, 0.25)
    assert all(len(v) == len(r["blocks"]) for v in r["sel"].values())
    assert np.array_equal(r["out"], dense) and np.array_equal(r["lse"], lse)


def test_hsa_one_block_is_softmax_over_its_keys(oracle_lib):
    """tau below every mass keeps one block: the map's argmax; each row is then
    the textbook softmax over that block's keys (numpy, fp64)."""
    q, kc, vc, ko, vo = _hsa_inputs()
    scale = 0.25
    rows = np.array([0, 17, 255, 256, 299])
    r = oracle_lib.hsa_sparse(q, kc, vc, ko, vo, scale, [1e-12, 1e-12], rows=rows)
    k_all = np.concatenate([kc, ko]).astype(np.float64)
    v_all = np.concatenate([vc, vo]).astype(np.float64)
    for i, row in enumerate(rows):
        b = row // 256
        for h in range(2):
            (j,) = r["sel"][(h, b)]
            pmap = oracle_lib.hsa_pooled_map(q[b * 256:(b + 1) * 256], np.concatenate([kc, ko]),
                                             r["blocks"], scale)
            assert j == int(np.argmax(pmap[h]))
            a, z = r["blocks"][j]
            s = k_all[a:z, h] @ q[row, h].astype(np.float64) * scale
            p = np.exp(s - s.max())
            want = (p[:, None] * v_all[a:z, h]).sum(axis=0) / p.sum()
            assert np.abs(r["out"][i, h] - want).max() < 1e-12
            assert abs(r["lse"][h, i] - (s.max() + np.log(p.sum()))) < 1e-12


def test_hsa_threshold_is_per_head(oracle_lib):
    """tau = [tiny, above 1]: head 0 keeps exactly the argmax block of its own
    map, head 1 keeps every block, in every query block."""
    q, kc, vc, ko, vo = _hsa_inputs()
    r = oracle_lib.hsa_sparse(q, kc, vc, ko, vo, 0.25, [1e-12, 2.0])
    nb = len(r["blocks"])
    for (h, b), chosen in r["sel"].items():
        pmap = r["maps"][b][h]
        if h == 0:
            assert chosen == [int(np.argmax(pmap))]
        else:
            assert chosen == list(range(nb))


@pytest.mark.parametrize("cut", [1, 37, 64, 90])
def test_merge_of_two_key_sets_is_attention_over_their_union(oracle_lib, cut):
    """Attention over keys [0, cut) merged with attention over [cut, n) equals
    the attention over all n keys (computed in one piece by the C oracle)."""
    rng = np.random.default_rng(11)
    n, H, d, nq = 100, 2, 16, 9
    q = rng.standard_normal((nq, H, d)).astype(np.float32)
    k = (2.0 * rng.standard_normal((n, H, d))).astype(np.float32)
    v = rng.standard_normal((n, H, d)).astype(np.float32)
    full, lse = oracle_lib.attention(q, k, v, None, None, 0.3)
    oa, la = oracle_lib.attention(q, k[:cut], v[:cut], None, None, 0.3)
    ob, lb = oracle_lib.attention(q, k[cut:], v[cut:], None, None, 0.3)
    out, l = oracle_lib.merge_attention(oa, la, ob, lb)
    assert np.abs(out - full).max() < 1e-12 and np.abs(l - lse).max() < 1e-12
    out2, l2 = oracle_lib.merge_attention(ob, lb, oa, la)        # order of the parts
    assert np.abs(out2 - full).max() < 1e-12 and np.abs(l2 - lse).max() < 1e-12


def test_merge_with_an_empty_part_is_the_other_part(oracle_lib):
    rng = np.random.default_rng(12)
    oa = rng.standard_normal((5, 2, 8))
    la = rng.standard_normal((2, 5)) + 40.0        # large lse: no overflow
    ob = rng.standard_normal((5, 2, 8))
    lb = np.full((2, 5), -np.inf)
    out, l = oracle_lib.merge_attention(oa, la, ob, lb)
    assert np.array_equal(out, oa) and np.array_equal(l, la)
