"""Edge and degenerate cases of the HIP path, against the oracle or against
properties that hold exactly (bitwise reruns, page-order invariance, device
handling of out-of-range ids)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_page_amd as wa
import wa_workloads as W
from tests.pipeline import PoolRun, say, to_bits, to_device, to_f64, wa_layout

pytestmark = pytest.mark.gpu

BF = W.scaled(W.WORKLOADS["wan_kp4"], name="edge_bf16", n_heads=3, frame_tokens=16,
              page_frames=4, n_pages=5, chunk_frames=5, k_p=2)    # P_t 64, N_q 80


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wa.load_library()


def rand_rows(wl, n, seed):
    rng = np.random.default_rng([wl.wid, 99, seed])
    x = rng.standard_normal((n, wl.n_heads, wl.head_dim), dtype=np.float32)
    return W.encode(wl, x)


def attend(wl, q, kc, vc, ko, vo, odt=None, lse=False):
    L = wa_layout(wl)
    dev = [to_device(x) if x is not None and x.shape[0] > 0 else None for x in (q, kc, vc, ko, vo)]
    lse_t = torch.empty(wl.n_heads, q.shape[0], dtype=torch.float32, device="cuda") if lse else None
    out = wa.wa_block_attention(L, *dev, wl.softmax_scale, out_dtype=odt, lse=lse_t)
    torch.cuda.synchronize()
    return (out, lse_t) if lse else out


@pytest.mark.parametrize("wl", [BF, W.WORKLOADS["tiny_f32"]], ids=["bf16", "f32"])
@pytest.mark.parametrize("n_q,n_ctx,n_own", [
    (1, 0, 1),        # a single key
    (1, 64, 0),       # context only, one query
    (80, 0, 80),      # own keys only
    (257, 128, 65),   # one query past a 256-query block, keys ragged by one
    (33, 1, 63),      # ctx/own boundary inside the first key tile
    (64, 191, 2),     # boundary near a tile edge
])
def test_attention_shapes(wl, n_q, n_ctx, n_own):
    q = rand_rows(wl, n_q, 1)
    kc, vc = rand_rows(wl, n_ctx, 2), rand_rows(wl, n_ctx, 3)
    ko, vo = rand_rows(wl, n_own, 4), rand_rows(wl, n_own, 5)
    say("attention shape", wl.name, n_q, n_ctx, n_own)
    out, lse = attend(wl, q, kc, vc, ko, vo, odt=wa.WA_F32, lse=True)
    ref, ref_lse = oracle.attention(q, kc if n_ctx else None, vc if n_ctx else None,
                                    ko if n_own else None, vo if n_own else None,
                                    wl.softmax_scale)
    tol = 1e-5 if wl.dtype == W.F32 else 1e-2
    assert np.abs(to_f64(out) - ref).max() <= tol
    assert np.abs(lse.cpu().double().numpy() - ref_lse).max() <= tol


@pytest.mark.parametrize("n_q,n_ctx,n_own", [(300, 200, 70), (40, 3000, 40)],
                         ids=["one_block_per_item", "split_launch"])
def test_attention_widest_row(n_q, n_ctx, n_own):
    """The widest row the library takes (WA_MAX_ROW_ELEMS = 32 heads x 128, an
    8 KB token stride), bf16, against the oracle on both output dtypes and the
    lse; the second shape has few items and many keys, so the launch splits."""
    wl = W.scaled(BF, name="edge_wide_row_attn", n_heads=32)
    assert wl.n_heads * wl.head_dim == 4096
    q = rand_rows(wl, n_q, 21)
    kc, vc = rand_rows(wl, n_ctx, 22), rand_rows(wl, n_ctx, 23)
    ko, vo = rand_rows(wl, n_own, 24), rand_rows(wl, n_own, 25)
    ref, ref_lse = oracle.attention(q, kc, vc, ko, vo, wl.softmax_scale)
    for odt in (wa.WA_F32, wa.WA_BF16):
        say("attention widest row", n_q, n_ctx, n_own, "out dtype", odt)
        out, lse = attend(wl, q, kc, vc, ko, vo, odt=odt, lse=True)
        assert np.abs(to_f64(out) - ref).max() <= 1e-2
        assert np.abs(lse.cpu().double().numpy() - ref_lse).max() <= 1e-2


@pytest.mark.parametrize("odt", [wa.WA_F32, wa.WA_BF16], ids=["f32_out", "bf16_out"])
def test_attention_split_over_cus(odt):
    """Few (query block, head) items and many keys: the launch splits each
    item's 630 key tiles into up to 36 pieces over 192 blocks and merges them.
    Sampled rows of both query blocks against the oracle, lse included."""
    wl = BF
    n_q, n_ctx, n_own = 257, 40000, 257
    L = wa_layout(wl)
    assert wa.wa_attention_workspace_bytes(L, n_q, n_ctx, n_own) > 0, "expected a split launch"
    q = rand_rows(wl, n_q, 11)
    kc, vc = rand_rows(wl, n_ctx, 12), rand_rows(wl, n_ctx, 13)
    ko, vo = rand_rows(wl, n_own, 14), rand_rows(wl, n_own, 15)
    say("attention split", n_q, n_ctx, n_own, odt)
    out, lse = attend(wl, q, kc, vc, ko, vo, odt=odt, lse=True)
    rows = np.array([0, 1, 31, 32, 100, 200, 254, 255, 256], dtype=np.int64)
    ref, ref_lse = oracle.attention(q, kc, vc, ko, vo, wl.softmax_scale, rows=rows)
    got = to_f64(out)[rows]
    assert np.abs(got - ref).max() <= 1e-2
    assert np.abs(lse.cpu().double().numpy()[:, rows] - ref_lse).max() <= 1e-2


@pytest.mark.parametrize("wl", [BF, W.WORKLOADS["tiny_f32"]], ids=["bf16", "f32"])
def test_attention_scores_growing_along_the_keys(wl):
    """Scores that climb steadily along the keys (each key adds a multiple of
    one direction that every query shares): the running maximum grows many
    times over, so the output is rescaled repeatedly.  Against the oracle."""
    n_q, n_ctx, n_own = 70, 700, 90
    rng = np.random.default_rng([wl.wid, 7])
    u = np.ones(wl.head_dim, np.float32) / np.sqrt(wl.head_dim)
    def rows(n, ramp):
        x = 0.25 * rng.standard_normal((n, wl.n_heads, wl.head_dim), dtype=np.float32)
        if ramp is not None:
            x += (ramp[:, None, None] * u[None, None, :]).astype(np.float32)
        return W.encode(wl, x)
    keys = np.arange(n_ctx + n_own, dtype=np.float32)
    q = rows(n_q, np.full(n_q, 4.0, np.float32))
    kc, ko = rows(n_ctx, 0.06 * keys[:n_ctx]), rows(n_own, 0.06 * keys[n_ctx:])
    vc, vo = rows(n_ctx, None), rows(n_own, None)
    say("attention growing scores", wl.name)
    out, lse = attend(wl, q, kc, vc, ko, vo, odt=wa.WA_F32, lse=True)
    ref, ref_lse = oracle.attention(q, kc, vc, ko, vo, wl.softmax_scale)
    tol = 1e-5 if wl.dtype == W.F32 else 1e-2
    assert np.abs(to_f64(out) - ref).max() <= tol
    assert np.abs(lse.cpu().double().numpy() - ref_lse).max() <= tol


def test_attention_unit_values_and_reruns_are_bitwise_equal():
    wl = BF
    q, kc, ko = rand_rows(wl, 200, 1), rand_rows(wl, 300, 2), rand_rows(wl, 70, 4)
    ones_c = W.encode(wl, np.ones((300, wl.n_heads, wl.head_dim), np.float32))
    ones_o = W.encode(wl, np.ones((70, wl.n_heads, wl.head_dim), np.float32))
    say("attention unit values")
    out = attend(wl, q, kc, ones_c, ko, ones_o, odt=wa.WA_F32)
    # probabilities are rounded to bf16 before the value product: |O - 1| <= 2^-8
    assert np.abs(to_f64(out) - 1.0).max() <= 2.0 ** -8
    vc, vo = rand_rows(wl, 300, 3), rand_rows(wl, 70, 5)
    a = attend(wl, q, kc, vc, ko, vo, odt=wa.WA_BF16)
    b = attend(wl, q, kc, vc, ko, vo, odt=wa.WA_BF16)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_attention_invariant_to_page_order():
    """Permuting the pages of the gathered context changes nothing beyond
    rounding (one softmax over the whole set)."""
    wl = BF
    pages_k = [rand_rows(wl, 64, 10 + j) for j in range(4)]
    pages_v = [rand_rows(wl, 64, 20 + j) for j in range(4)]
    q, ko, vo = rand_rows(wl, 80, 1), rand_rows(wl, 80, 2), rand_rows(wl, 80, 3)
    a = attend(wl, q, np.concatenate(pages_k), np.concatenate(pages_v), ko, vo, odt=wa.WA_F32)
    order = [3, 1, 0, 2]
    b = attend(wl, q, np.concatenate([pages_k[i] for i in order]),
               np.concatenate([pages_v[i] for i in order]), ko, vo, odt=wa.WA_F32)
    assert np.abs(to_f64(a) - to_f64(b)).max() <= 1e-2


def test_append_mean_only_and_rerun():
    wl = BF
    run = PoolRun(wl)
    k, v = W.page_kv(wl, 2)
    # producer wrote the page in place: k_src is the slot itself
    run.k_pool[1].copy_(to_device(k))
    say("append mean-only")
    wa.wa_append_page(run.L, run.k_pool[1], None, run.k_pool, None, 1, run.means,
                      workspace=run.ws)
    torch.cuda.synchronize()
    want = oracle.page_mean(k)
    got = run.means[1].cpu().numpy()
    assert np.abs(got - want).max() <= 1e-12
    # the V slot was not touched, the K slot still holds the page
    assert torch.count_nonzero(run.v_pool[1]).item() == 0
    assert to_bits(run.k_pool[1]).tobytes() == k.tobytes()
    first = run.means[1].clone()
    wa.wa_append_page(run.L, run.k_pool[1], None, run.k_pool, None, 1, run.means,
                      workspace=run.ws)
    torch.cuda.synchronize()
    assert torch.equal(first, run.means[1])


def _pool_with_pages(wl, n):
    run = PoolRun(wl)
    for j in range(n):
        run.append(j)
    return run


def test_select_with_explicit_candidates_and_all_pages():
    wl = BF
    run = _pool_with_pages(wl, wl.n_pages)
    q = W.chunk_qkv(wl, 0, 0)[0]
    qd = to_device(q)
    host_means = run.oracle_means(range(wl.n_pages))
    for cand, k_p in (([4, 1, 3], 2), ([2, 0, 4, 1, 3], 5), ([3], 1)):
        cd = torch.tensor(cand, dtype=torch.int32, device="cuda")
        say("select cand", cand, k_p)
        idx = wa.wa_select_pages(run.L, qd, run.means, k_p, cand=cd)
        ref = oracle.select_pages(q, host_means, k_p, cand=np.array(cand, np.int32))
        assert idx.cpu().numpy().tolist() == ref["idx"].tolist()


def test_select_skips_out_of_range_candidates():
    wl = BF
    run = _pool_with_pages(wl, wl.n_pages)
    q = W.chunk_qkv(wl, 0, 0)[0]
    cand = [2, 99, -4, 0, 3]
    cd = torch.tensor(cand, dtype=torch.int32, device="cuda")
    scores = torch.empty(5, dtype=torch.float64, device="cuda")
    say("select invalid cand")
    idx = wa.wa_select_pages(run.L, to_device(q), run.means, 5, cand=cd, out_scores=scores)
    got = idx.cpu().numpy().tolist()
    ref = oracle.select_pages(q, run.oracle_means(range(wl.n_pages)), 3,
                              cand=np.array([2, 0, 3], np.int32))
    assert got[:3] == ref["idx"].tolist() and got[3:] == [-1, -1]
    s = scores.cpu().numpy()
    assert np.isneginf(s[1]) and np.isneginf(s[2])


@pytest.mark.parametrize("n_cand,k_p", [(1024, 7), (1025, 7), (3000, 40), (11, 3)])
def test_select_long_candidate_lists_with_repeats(n_cand, k_p):
    """Both top-K paths (one thread per candidate up to 1,024 candidates, an
    argmax per rank beyond): a repeated page id is selected once per
    occurrence, and ids outside the pool are never selected."""
    wl = BF
    run = _pool_with_pages(wl, wl.n_pages)
    q = W.chunk_qkv(wl, 0, 0)[0]
    rng = np.random.default_rng([n_cand, k_p])
    cand = rng.integers(0, wl.n_pages, n_cand).astype(np.int32)
    cand[rng.choice(n_cand, n_cand // 7, replace=False)] = 99     # outside the pool
    say("select long cand", n_cand, k_p)
    idx = wa.wa_select_pages(run.L, to_device(q), run.means, k_p,
                             cand=torch.from_numpy(cand).cuda())
    valid = cand[cand < wl.n_pages]
    ref = oracle.select_pages(q, run.oracle_means(range(wl.n_pages)), min(k_p, valid.size),
                              cand=valid)["idx"].tolist()
    assert idx.cpu().numpy().tolist() == ref + [-1] * (k_p - len(ref))


def test_select_exact_ties_between_pages():
    """Byte-identical pages in several slots have identical mean keys, so their
    scores tie exactly: the order is then by page id, and a repeated id by
    list position.  Every rank is checked against the oracle, on the
    one-launch path (12 candidates), the three-launch path (70 candidates
    with repeats) and with a window holding one member of a tie group."""
    wl = W.scaled(BF, name="edge_ties", n_pages=12)
    run = PoolRun(wl)
    twins = {6: 3, 9: 3, 10: 1, 11: 7}          # slot -> the page stored there again
    for s_ in range(wl.n_pages):
        run.append(twins.get(s_, s_), slot=s_)
    q = W.chunk_qkv(wl, 0, 0)[0]
    qd = to_device(q)
    host_means = run.oracle_means(range(wl.n_pages))
    means = run.means.cpu().numpy()
    assert np.array_equal(means[6], means[3]) and np.array_equal(means[10], means[1])
    rng = np.random.default_rng(5)
    cases = [("all 12 slots", np.arange(12, dtype=np.int32), 12),
             ("70 listed", rng.permutation(np.tile(np.arange(12, dtype=np.int32), 6)[:70]).astype(np.int32), 20)]
    for name, cand, k_p in cases:
        say("select exact ties:", name)
        scores = torch.empty(cand.size, dtype=torch.float64, device="cuda")
        idx = wa.wa_select_pages(run.L, qd, run.means, k_p, cand=torch.from_numpy(cand).cuda(),
                                 out_scores=scores)
        ref = oracle.select_pages(q, host_means, k_p, cand=cand)
        assert idx.cpu().numpy().tolist() == ref["idx"].tolist()
        got = scores.cpu().numpy()
        assert got[cand == 6][0] == got[cand == 3][0] == got[cand == 9][0]
        assert np.abs(got - ref["alpha"]).max() <= 1e-12 * max(1.0, np.abs(ref["alpha"]).max())
    say("select exact ties: window [9]")
    recent = np.array([9], dtype=np.int32)
    idx = wa.wa_select_window(run.L, qd, run.means, torch.from_numpy(recent).cuda(), 8)
    ref = oracle.select_window(q, host_means, 8, recent)
    assert idx.cpu().numpy().tolist() == ref["idx"].tolist()


def test_select_at_the_limits():
    """Selections at the library's limits, against the oracle: the widest row
    (WA_MAX_ROW_ELEMS = 32 heads x 128) with 16 candidates (one launch, 32
    column groups), 100 candidates (64 column groups of 8 vectors: more than
    the two-level path's counters hold, so three launches) and 300 candidates
    (three launches), and WA_MAX_CANDIDATES listed candidates (ids repeated);
    then the gather of the last selection at that width, byte for byte."""
    wl = W.scaled(W.WORKLOADS["wan_kp4"], name="edge_wide_row", n_heads=32, frame_tokens=8,
                  page_frames=2, n_pages=20, chunk_frames=30, k_p=5)   # 16-token pages, 240 queries
    assert wl.n_heads * wl.head_dim == 4096
    run = _pool_with_pages(wl, wl.n_pages)
    q = W.chunk_qkv(wl, 0, 0)[0]
    qd = to_device(q)
    host_means = run.oracle_means(range(wl.n_pages))
    rng = np.random.default_rng(11)
    for n_cand in (16, 100, 300, 4096):
        cand = (rng.permutation(wl.n_pages)[:n_cand] if n_cand <= wl.n_pages else
                rng.integers(0, wl.n_pages, n_cand)).astype(np.int32)
        say("select at the limits:", n_cand, "candidates, row of", wl.n_heads * wl.head_dim)
        scores = torch.empty(n_cand, dtype=torch.float64, device="cuda")
        idx = wa.wa_select_pages(run.L, qd, run.means, wl.k_p, cand=torch.from_numpy(cand).cuda(),
                                 out_scores=scores)
        ref = oracle.select_pages(q, host_means, wl.k_p, cand=cand)
        assert idx.cpu().numpy().tolist() == ref["idx"].tolist()
        got = scores.cpu().numpy()
        assert np.abs(got - ref["alpha"]).max() <= 1e-12 * max(1.0, np.abs(ref["alpha"]).max())
    # the pages appended at this width gather byte for byte
    k_ctx, v_ctx = wa.wa_gather(run.L, run.k_pool, run.v_pool, idx, wl.k_p)
    torch.cuda.synchronize()
    sel = idx.cpu().numpy()
    assert to_bits(k_ctx).tobytes() == oracle.gather(np.stack([run.host_k[i] for i in range(wl.n_pages)]), sel).tobytes()
    assert to_bits(v_ctx).tobytes() == oracle.gather(np.stack([run.host_v[i] for i in range(wl.n_pages)]), sel).tobytes()


@pytest.mark.parametrize("n_cand", [11, 1031])
def test_select_fewer_valid_candidates_than_k_p(n_cand):
    wl = BF
    run = _pool_with_pages(wl, wl.n_pages)
    q = W.chunk_qkv(wl, 0, 0)[0]
    cand = np.full(n_cand, 99, np.int32)
    cand[n_cand // 2] = 2
    say("select sparse cand", n_cand)
    idx = wa.wa_select_pages(run.L, to_device(q), run.means, 3, cand=torch.from_numpy(cand).cuda())
    assert idx.cpu().numpy().tolist() == [2, -1, -1]


def test_gather_skips_out_of_range_index():
    wl = BF
    run = _pool_with_pages(wl, wl.n_pages)
    idx = torch.tensor([3, 7, -1, 0], dtype=torch.int32, device="cuda")
    shape = (4 * wl.page_tokens, wl.n_heads, wl.head_dim)
    k_ctx = torch.full(shape, 5.0, dtype=torch.bfloat16, device="cuda")
    v_ctx = torch.full(shape, 5.0, dtype=torch.bfloat16, device="cuda")
    say("gather invalid idx")
    wa.wa_gather(run.L, run.k_pool, run.v_pool, idx, 4, k_ctx, v_ctx)
    torch.cuda.synchronize()
    pt = wl.page_tokens
    assert to_bits(k_ctx[:pt]).tobytes() == run.host_k[3].tobytes()
    assert to_bits(v_ctx[3 * pt:]).tobytes() == run.host_v[0].tobytes()
    assert bool((k_ctx[pt:3 * pt] == 5.0).all()) and bool((v_ctx[pt:3 * pt] == 5.0).all())


def test_selection_follows_pool_slots_under_permutation():
    """Pages stored in permuted slots: the selected slots map back to the same
    pages, and the gathered buffers are identical."""
    wl = BF
    perm = [3, 0, 4, 1, 2]            # page j lives in slot perm[j]
    a = PoolRun(wl)
    b = PoolRun(wl)
    for j in range(wl.n_pages):
        a.append(j)
        b.append(j, slot=perm[j])
    qd = to_device(W.chunk_qkv(wl, 0, 0)[0])
    ia = wa.wa_select_pages(a.L, qd, a.means, wl.k_p).cpu().numpy()
    ib = wa.wa_select_pages(b.L, qd, b.means, wl.k_p).cpu().numpy()
    inv = {s: j for j, s in enumerate(perm)}
    # ties impossible here (distinct offsets); same pages in the same rank order
    assert [inv[s] for s in ib.tolist()] == ia.tolist()
    ka, va = wa.wa_gather(a.L, a.k_pool, a.v_pool, torch.from_numpy(ia).cuda(), wl.k_p)
    kb, vb = wa.wa_gather(b.L, b.k_pool, b.v_pool, torch.from_numpy(ib).cuda(), wl.k_p)
    assert torch.equal(ka.view(torch.int16), kb.view(torch.int16))
    assert torch.equal(va.view(torch.int16), vb.view(torch.int16))


@pytest.mark.parametrize("n_chunks", [16, 20])
def test_prompt_stage_with_window(n_chunks):
    """wa_select_window with a prompt stage: the window's ids first, then the
    top K_p of the kept chunks' pages outside the window, against the oracle;
    the window holds one page of the best-ranked chunk and one page no kept
    chunk holds.  16 chunks of 4 pages take the one-launch selection, 20 the
    three-launch one."""
    wl = W.scaled(W.WORKLOADS["prompt_page"], name="prompt_window_%d" % n_chunks, n_heads=2,
                  frame_tokens=10, n_chunk_groups=n_chunks, n_pages=4 * n_chunks)
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    cp, cur, pages = W.chunk_prompts(wl), W.current_prompt(wl), W.chunk_page_map(wl)
    host_prompt = dict(chunk_prompts=cp, cur_prompt=cur, chunk_pages=pages,
                       n_keep=wl.n_cand_groups)
    q, _, _ = W.chunk_qkv(wl, 0, 0)
    host_means = run.oracle_means(range(wl.n_pages))
    plain = oracle.select_pages(q, host_means, wl.k_p, prompt=host_prompt)
    best = int(plain["chunks"][0])
    outside = [m for m in range(n_chunks) if m not in plain["chunks"].tolist()][0]
    recent = np.array([pages[best][1], pages[outside][0]], dtype=np.int32)
    dev_prompt = dict(chunk_prompts=torch.from_numpy(cp).cuda(),
                      cur_prompt=torch.from_numpy(cur).cuda(),
                      chunk_pages=torch.from_numpy(pages).cuda(), n_keep=wl.n_cand_groups)
    say("prompt stage with a window:", n_chunks, "chunks, recent", recent.tolist())
    scores = torch.empty(wl.n_cand_groups * wl.pages_per_group, dtype=torch.float64,
                         device="cuda")
    idx = wa.wa_select_window(run.L, to_device(q), run.means, torch.from_numpy(recent).cuda(),
                              wl.k_p, prompt=dev_prompt, out_scores=scores)
    ref = oracle.select_window(q, host_means, wl.k_p, recent, prompt=host_prompt)
    assert idx.cpu().numpy().tolist() == ref["idx"].tolist()
    got = scores.cpu().numpy()
    assert np.abs(got - ref["alpha"]).max() <= 1e-12 * max(1.0, np.abs(ref["alpha"]).max())


@pytest.mark.parametrize("zero", ["chunk_prompts", "cur_prompt"])
def test_prompt_stage_with_zero_norm_prompts(zero):
    """A prompt embedding of zero norm has no direction: its cosine is -inf on
    both sides, so zeroed chunk prompts rank last (in chunk id order) and a
    zero current prompt keeps the lowest chunk ids.  Kept chunks, candidate
    pages and idx int-equal to the oracle."""
    wl = W.scaled(W.WORKLOADS["prompt_page"], name="prompt_zero", n_heads=2, frame_tokens=10)
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    cp, cur = W.chunk_prompts(wl).copy(), W.current_prompt(wl).copy()
    if zero == "chunk_prompts":
        # zero the chunks that would rank first and third
        order = np.argsort(-oracle.prompt_cosine(cp, cur), kind="stable")
        cp[order[0]] = 0.0
        cp[order[2]] = 0.0
    else:
        cur[:] = 0.0
    pages = W.chunk_page_map(wl)
    out_chunks = torch.empty(wl.n_cand_groups, dtype=torch.int32, device="cuda")
    out_cand = torch.empty(wl.n_cand_groups * wl.pages_per_group, dtype=torch.int32,
                           device="cuda")
    prompt_dev = dict(chunk_prompts=torch.from_numpy(cp).cuda(),
                      cur_prompt=torch.from_numpy(cur).cuda(),
                      chunk_pages=torch.from_numpy(pages).cuda(), n_keep=wl.n_cand_groups,
                      out_chunks=out_chunks, out_cand=out_cand)
    q, _, _ = W.chunk_qkv(wl, 0, 0)
    say("prompt stage with zero-norm prompts:", zero)
    idx = wa.wa_select_pages(run.L, to_device(q), run.means, wl.k_p, prompt=prompt_dev)
    torch.cuda.synchronize()
    host_means = np.stack([oracle.page_mean(run.host_k[s]) for s in range(wl.n_pages)])
    ref = oracle.select_pages(q, host_means, wl.k_p,
                              prompt=dict(chunk_prompts=cp, cur_prompt=cur, chunk_pages=pages,
                                          n_keep=wl.n_cand_groups))
    if zero == "cur_prompt":
        assert ref["chunks"].tolist() == list(range(wl.n_cand_groups))
    else:
        assert not set(ref["chunks"].tolist()) & {int(order[0]), int(order[2])}
    assert out_chunks.cpu().numpy().tolist() == ref["chunks"].tolist()
    assert out_cand.cpu().numpy().tolist() == ref["cand"].tolist()
    assert idx.cpu().numpy().tolist() == ref["idx"].tolist()


def test_select_one_workspace_across_both_paths():
    """One zero-filled workspace serves a run of selections ordered on one
    stream: the one-launch path (no prompt stage, at most 64 candidates,
    whose last block clears the completion counter), the two-level
    one-launch path (65 to 256 candidates, which also clears one counter per
    column group) and the three-launch path (300 candidates, ids repeated)
    in turn, with and without a window, each against the oracle; afterwards
    the counters are zero again."""
    wl = W.scaled(W.WORKLOADS["wan_kp4"], name="edge_ws", n_heads=2, frame_tokens=16,
                  page_frames=2, n_pages=70, chunk_frames=9, k_p=3)   # 32-token pages, 144 queries
    run = _pool_with_pages(wl, wl.n_pages)
    q = W.chunk_qkv(wl, 0, 0)[0]
    qd = to_device(q)
    host_means = run.oracle_means(range(wl.n_pages))
    rng = np.random.default_rng(5)
    cases = [(16, None), (64, None), (65, None), (5, [3, 7]), (70, [1]), (64, [0, 2, 4]),
             (300, None), (1, None), (256, [5]), (64, None)]
    nbytes = max(wa.wa_select_workspace_bytes(run.L, q.shape[0], n) for n, _ in cases)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for n_cand, recent in cases:
        cand = (rng.permutation(wl.n_pages)[:n_cand] if n_cand <= wl.n_pages else
                rng.integers(0, wl.n_pages, n_cand)).astype(np.int32)
        cd = torch.from_numpy(cand).cuda()
        k_p = min(wl.k_p, n_cand - (len(recent) if recent else 0))
        say("select one workspace", n_cand, recent)
        if recent is None:
            idx = wa.wa_select_pages(run.L, qd, run.means, k_p, cand=cd, workspace=ws)
            ref = oracle.select_pages(q, host_means, k_p, cand=cand)["idx"]
        else:
            rd = torch.tensor(recent, dtype=torch.int32, device="cuda")
            idx = wa.wa_select_window(run.L, qd, run.means, rd, k_p, cand=cd, workspace=ws)
            ref = oracle.select_window(q, host_means, k_p, np.array(recent, np.int32),
                                       cand=cand)["idx"]
        assert idx.cpu().numpy().tolist() == np.asarray(ref).tolist()
    torch.cuda.synchronize()
    assert not bool(ws[:256].any())


@pytest.mark.parametrize("dtype,n_heads,head_dim,n_q,n_pages", [
    (W.F32, 2, 64, 700, 10),      # fp32: 32 column vectors, one group, 6 row blocks
    (W.F32, 3, 128, 1500, 9),     # fp32: 96 vectors, two groups (64 + 32)
    (W.BF16, 3, 64, 1100, 12),    # bf16: 24 vectors, a group narrower than 64
    (W.BF16, 5, 128, 2000, 40),   # bf16: 80 vectors, two groups (64 + 16); 40 candidates
    (W.F32, 3, 128, 1500, 100),   # fp32, 100 candidates: the two-level path, 8-vector groups
    (W.BF16, 3, 64, 1100, 90),    # bf16, 90 candidates: 24 vectors in 3 groups of 8
], ids=["f32_h2_d64", "f32_h3_d128", "bf16_h3_d64", "bf16_h5_d128_40cand", "f32_h3_d128_100cand",
        "bf16_h3_d64_90cand"])
def test_select_layouts_and_shapes(dtype, n_heads, head_dim, n_q, n_pages):
    """The one-launch selection (and past 64 candidates the two-level one)
    over layouts whose column groups are narrower than their width or ragged,
    with several row blocks, against the oracle (ids, scores to 1e-12)."""
    base = W.WORKLOADS["tiny_f32"] if dtype == W.F32 else W.WORKLOADS["wan_kp4"]
    wl = W.scaled(base, name="sel_%s_%d_%d" % (dtype, n_heads, head_dim), dtype=dtype,
                  n_heads=n_heads, head_dim=head_dim, frame_tokens=16, page_frames=2,
                  n_pages=n_pages, chunk_frames=1, k_p=3, scale=head_dim ** -0.5)
    run = _pool_with_pages(wl, wl.n_pages)
    rng = np.random.default_rng([n_q, n_pages])
    q = W.encode(wl, rng.standard_normal((n_q, n_heads, head_dim), dtype=np.float32))
    scores = torch.empty(n_pages, dtype=torch.float64, device="cuda")
    say("select layout", dtype, n_heads, head_dim, n_q, n_pages)
    idx = wa.wa_select_pages(run.L, to_device(q), run.means, wl.k_p, out_scores=scores)
    ref = oracle.select_pages(q, run.oracle_means(range(n_pages)), wl.k_p)
    assert idx.cpu().numpy().tolist() == ref["idx"].tolist()
    got = scores.cpu().numpy()
    assert np.abs(got - ref["alpha"]).max() <= 1e-12 * max(1.0, np.abs(ref["alpha"]).max())
