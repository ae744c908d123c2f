"""Sparse branch (wa_hsa_select + wa_sparse_attention) against the oracle.

Selection: the tile lists must be int-equal to the tiles of the oracle's
selected blocks (every case first checks that the oracle's cut is clear: no
near tie at the cut and the running sum not within rounding of tau, so that
one answer is right), the Gini coefficient within fp64 rounding.  Attention
over the selected tiles: within the attention tolerance of the oracle, and
bit for bit equal to wa_block_attention where the two do the same arithmetic
(the full list; one item over a gathered copy of its selected keys).  Uneven
lists at full size are cut into runs over all CUs and merged (the split);
those cases are held to the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_page_amd as wa
import wa_workloads as W
from tests.pipeline import attention_tolerance, say, to_device, to_f64, wa_layout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wa.load_library()


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


# 3 heads, 128-token pages, 576 queries (query blocks of 256, 256, 64); the
# context is 4.5 pages (576 keys: its last block holds 64 keys), the own
# segment 560 keys (its last block and tile hold 48).
SMALL = W.scaled(W.WORKLOADS["wan_kp4"], n_heads=3, frame_tokens=64, page_frames=2, n_pages=8,
                 chunk_frames=9)


def _inputs(wl, pages, n_ctx, n_own, gain):
    q = W.aligned_queries(wl, 0, 0, gain)
    _, ko, vo = W.chunk_qkv(wl, 0, 0)
    if pages:
        kv = [W.page_kv(wl, p) for p in pages]
        kc = np.concatenate([k for k, _ in kv])[:n_ctx]
        vc = np.concatenate([v for _, v in kv])[:n_ctx]
    else:
        kc = vc = None
    return q, kc, vc, ko[:n_own], vo[:n_own]


def _dev(x):
    return None if x is None or x.shape[0] == 0 else to_device(x)


def _clear_cut(pm_row, tau, eps=1e-9):
    """The oracle's selection is the only right one: no near tie between the
    last block in and the first block out, and tau not within eps of the
    running sums that decide the count."""
    order = sorted(range(pm_row.size), key=lambda j: (-pm_row[j], j))
    srt = pm_row[order]
    cum = np.cumsum(srt)
    m = len(oracle.select_blocks(pm_row, tau))
    if m < pm_row.size:
        assert srt[m - 1] - srt[m] > eps, "near tie at the cut"
        assert cum[m - 1] >= tau + eps, "running sum within eps of tau"
    if m >= 2:
        assert cum[m - 2] <= tau - eps, "running sum within eps of tau"


def _tiles_of(blocks, chosen):
    """Ascending 64-key tiles covering the chosen key blocks."""
    ts = set()
    for j in chosen:
        a, b = blocks[j]
        ts.update(range(a // 64, (b + 63) // 64))
    return sorted(ts)


def _check_selection(L, wl, q, kc, ko, tau, scale):
    n_q, n_ctx, n_own = q.shape[0], (0 if kc is None else kc.shape[0]), ko.shape[0]
    say("hsa select", wl.name, "n_q", n_q, "n_ctx", n_ctx, "n_own", n_own, "tau", tau)
    tau_d = torch.tensor(tau, dtype=torch.float64, device="cuda")
    tiles, count, gini = wa.wa_hsa_select(L, to_device(q), _dev(kc), _dev(ko), tau_d, scale=scale)
    torch.cuda.synchronize()
    tiles, count, gini = tiles.cpu().numpy(), count.cpu().numpy(), gini.cpu().numpy()
    q_blocks, items, n_tiles = wa.hsa_shape(L, n_q, n_ctx, n_own)
    assert tiles.shape == (items, n_tiles)
    blocks = oracle.hsa_key_blocks(n_ctx, n_own)
    k_all = ko if kc is None else np.concatenate([kc, ko])
    for b in range(q_blocks):
        pm = oracle.hsa_pooled_map(q[256 * b:256 * (b + 1)], k_all, blocks, scale)
        for h in range(L.n_heads):
            item = h * q_blocks + b
            _clear_cut(pm[h], tau[h])
            want = _tiles_of(blocks, oracle.select_blocks(pm[h], tau[h]))
            got = tiles[item, :count[item]].tolist()
            assert got == want, "item %d (head %d, query block %d): %s != %s" % (item, h, b, got,
                                                                               want)
            assert abs(gini[item] - oracle.gini(pm[h])) <= 1e-12
    return tiles, count


def test_selection_matches_the_oracle():
    wl = SMALL
    L = wa_layout(wl)
    q, kc, _, ko, _ = _inputs(wl, [5, 0, 3, 7, 2], 576, 560, gain=8.0)
    for tau in ([0.5, 0.8, 0.95], [0.3, 0.6, 0.9], [0.0, 1.5, 0.7]):
        _check_selection(L, wl, q, kc, ko, tau, wl.softmax_scale)


@pytest.mark.parametrize("dtype,head_dim", [(W.F32, 64), (W.F32, 128), (W.BF16, 64)],
                         ids=["f32_d64", "f32_d128", "bf16_d64"])
def test_selection_other_layouts(dtype, head_dim):
    """The selection over fp32 inputs and head_dim 64 (the attention over the
    lists is bf16 at head_dim 128 only; the selection takes any layout up to
    head_dim 128)."""
    wl = W.scaled(SMALL, name="hsa_%s_d%d" % (dtype, head_dim), dtype=dtype, head_dim=head_dim)
    L = wa_layout(wl)
    q, kc, _, ko, _ = _inputs(wl, [5, 0, 3, 7, 2], 576, 560, gain=8.0)
    _check_selection(L, wl, q, kc, ko, [0.5, 0.8, 0.95], wl.softmax_scale)


def test_selection_one_segment_only():
    """Context only (n_own = 0) and own keys only (n_ctx = 0)."""
    wl = SMALL
    L = wa_layout(wl)
    q, kc, _, ko, _ = _inputs(wl, [1, 4, 6], 384, 0, gain=8.0)
    _check_selection(L, wl, q, kc, ko, [0.6, 0.85, 0.4], wl.softmax_scale)
    q, _, _, ko, _ = _inputs(wl, [], 0, 576, gain=8.0)
    _check_selection(L, wl, q, None, ko, [0.6, 0.85, 0.4], wl.softmax_scale)


def test_selection_reusing_the_context_sums():
    """Two denoising steps of one chunk: the context keys stay, the queries and
    own keys are drawn anew.  The second call takes the context block sums the
    first left in the workspace (ctx_sums_ready) and must equal, bit for bit,
    a call that pools every block, which is held to the oracle."""
    wl = SMALL
    L = wa_layout(wl)
    n_ctx, n_own = 576, 560
    q1, kc, _, ko1, _ = _inputs(wl, [5, 0, 3, 7, 2], n_ctx, n_own, gain=8.0)
    q2 = W.aligned_queries(wl, 0, 1, 6.0)
    _, ko2, _ = W.chunk_qkv(wl, 0, 1)
    ko2 = ko2[:n_own]
    tau = [0.5, 0.8, 0.95]
    tau_d = torch.tensor(tau, dtype=torch.float64, device="cuda")
    kcd = to_device(kc)
    ws = torch.empty(wa.wa_hsa_workspace_bytes(L, q1.shape[0], n_ctx, n_own), dtype=torch.uint8,
                     device="cuda")
    say("hsa select, step 1 pools everything")
    wa.wa_hsa_select(L, to_device(q1), kcd, to_device(ko1), tau_d, scale=wl.softmax_scale,
                     workspace=ws)
    say("hsa select, step 2 reuses the context sums")
    reused = wa.wa_hsa_select(L, to_device(q2), kcd, to_device(ko2), tau_d,
                              scale=wl.softmax_scale, workspace=ws, ctx_sums_ready=True)
    torch.cuda.synchronize()
    reused = [x.cpu().numpy() for x in reused]
    full_tiles, full_count = _check_selection(L, wl, q2, kc, ko2, tau, wl.softmax_scale)
    fresh = wa.wa_hsa_select(L, to_device(q2), kcd, to_device(ko2), tau_d,
                             scale=wl.softmax_scale)
    torch.cuda.synchronize()
    fresh = [x.cpu().numpy() for x in fresh]
    # counts and Gini coefficients bit for bit; each list up to its count (the
    # entries after it are not written)
    assert np.array_equal(reused[1], fresh[1]) and np.array_equal(reused[1], full_count)
    assert np.array_equal(reused[2].view(np.int64), fresh[2].view(np.int64))
    for item in range(reused[1].size):
        c = reused[1][item]
        assert np.array_equal(reused[0][item, :c], fresh[0][item, :c])
        assert np.array_equal(reused[0][item, :c], full_tiles[item, :c])
    with pytest.raises(ValueError):
        wa.wa_hsa_select(L, to_device(q2), kcd, to_device(ko2), tau_d, ctx_sums_ready=True)
    # no context keys: the flag has nothing to reuse and is ignored
    say("hsa select, own keys only, flag set")
    own_only = wa.wa_hsa_select(L, to_device(q2), None, to_device(ko2), tau_d,
                                scale=wl.softmax_scale, workspace=ws, ctx_sums_ready=True)
    plain = wa.wa_hsa_select(L, to_device(q2), None, to_device(ko2), tau_d, scale=wl.softmax_scale)
    torch.cuda.synchronize()
    a_t, a_c, a_g = [x.cpu().numpy() for x in own_only]
    b_t, b_c, b_g = [x.cpu().numpy() for x in plain]
    assert np.array_equal(a_c, b_c) and np.array_equal(a_g.view(np.int64), b_g.view(np.int64))
    for item in range(a_c.size):
        assert np.array_equal(a_t[item, :a_c[item]], b_t[item, :b_c[item]])


def _sparse_vs_oracle(wl, q, kc, vc, ko, vo, tau, rows=None, out_dtypes=(wa.WA_F32, wa.WA_BF16)):
    L = wa_layout(wl)
    tiles, count = _check_selection(L, wl, q, kc, ko, tau, wl.softmax_scale)
    ref = oracle.hsa_sparse(q, kc, vc, ko, vo, wl.softmax_scale, tau, rows=rows)
    tiles_d = torch.from_numpy(tiles).cuda()
    count_d = torch.from_numpy(count).cuda()
    tol = attention_tolerance(wl)
    outs = {}
    for odt in out_dtypes:
        lse = torch.empty(wl.n_heads, q.shape[0], dtype=torch.float32, device="cuda")
        say("sparse attention", wl.name, "out_dtype", odt)
        out = wa.wa_sparse_attention(L, to_device(q), _dev(kc), _dev(vc), _dev(ko), _dev(vo),
                                     tiles_d, count_d, wl.softmax_scale, out_dtype=odt, lse=lse)
        torch.cuda.synchronize()
        got, got_lse = to_f64(out), lse.cpu().double().numpy()
        if rows is not None:
            got, got_lse = got[rows], got_lse[:, rows]
        err = np.abs(got - ref["out"]).max()
        assert err <= tol, "sparse attention max |err| %g > %g" % (err, tol)
        lerr = np.abs(got_lse - ref["lse"]).max()
        assert lerr <= tol, "sparse lse max |err| %g" % lerr
        outs[odt] = out
    return tiles, count, outs


def test_sparse_attention_matches_the_oracle():
    wl = SMALL
    q, kc, vc, ko, vo = _inputs(wl, [5, 0, 3, 7, 2], 576, 560, gain=8.0)
    _sparse_vs_oracle(wl, q, kc, vc, ko, vo, [0.5, 0.8, 0.95])


def test_sparse_attention_moderate_map_and_ctx_only():
    wl = SMALL
    q, kc, vc, ko, vo = _inputs(wl, [2, 6, 1, 4], 512, 560, gain=4.0)
    _sparse_vs_oracle(wl, q, kc, vc, ko, vo, [0.3, 0.6, 0.9])
    q, kc, vc, ko, vo = _inputs(wl, [1, 4, 6], 384, 0, gain=8.0)
    _sparse_vs_oracle(wl, q, kc, vc, ko, vo, [0.6, 0.85, 0.4])   # ko, vo: 0 rows


def test_full_list_equals_dense_bitwise():
    """tau above 1 keeps every block: the sparse call is then the dense one,
    tile for tile (the dense launch does not split at this size)."""
    wl = SMALL
    L = wa_layout(wl)
    q, kc, vc, ko, vo = _inputs(wl, [5, 0, 3, 7, 2], 576, 560, gain=8.0)
    n_tiles = wa.hsa_shape(L, q.shape[0], 576, 560)[2]
    assert wa.wa_attention_workspace_bytes(L, q.shape[0], 576, 560) == 0   # no split
    tau = torch.full((wl.n_heads,), 2.0, dtype=torch.float64, device="cuda")
    qd, kcd, vcd, kod, vod = (to_device(x) for x in (q, kc, vc, ko, vo))
    say("hsa select, keep all")
    tiles, count, _ = wa.wa_hsa_select(L, qd, kcd, kod, tau, scale=wl.softmax_scale)
    torch.cuda.synchronize()
    assert (count.cpu().numpy() == n_tiles).all()
    assert (tiles.cpu().numpy() == np.arange(n_tiles)[None, :]).all()
    for odt in (wa.WA_F32, wa.WA_BF16):
        ls = torch.empty(wl.n_heads, q.shape[0], dtype=torch.float32, device="cuda")
        ld = torch.empty_like(ls)
        say("sparse vs dense", odt)
        o_s = wa.wa_sparse_attention(L, qd, kcd, vcd, kod, vod, tiles, count, wl.softmax_scale,
                                     out_dtype=odt, lse=ls)
        o_d = wa.wa_block_attention(L, qd, kcd, vcd, kod, vod, wl.softmax_scale, out_dtype=odt,
                                    lse=ld)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(o_s), _bits(o_d))
        assert np.array_equal(_bits(ls), _bits(ld))


def test_one_item_equals_dense_over_its_gathered_keys():
    """Each (head, query block) item equals dense attention (one head) over a
    gathered copy of its selected keys, bit for bit: the selected tiles, laid
    end to end, are the dense call's tiles."""
    wl = SMALL
    L = wa_layout(wl)
    q, kc, vc, ko, vo = _inputs(wl, [5, 0, 3, 7, 2], 576, 560, gain=8.0)
    tau = [0.5, 0.8, 0.95]
    tiles, count = _check_selection(L, wl, q, kc, ko, tau, wl.softmax_scale)
    say("sparse attention for the gathered comparison")
    out = wa.wa_sparse_attention(L, to_device(q), to_device(kc), to_device(vc), to_device(ko),
                                 to_device(vo), torch.from_numpy(tiles).cuda(),
                                 torch.from_numpy(count).cuda(), wl.softmax_scale,
                                 out_dtype=wa.WA_F32)
    torch.cuda.synchronize()
    out = out.cpu()
    k_all, v_all = np.concatenate([kc, ko]), np.concatenate([vc, vo])
    n_keys = k_all.shape[0]
    q_blocks = wa.hsa_shape(L, q.shape[0], 576, 560)[0]
    L1 = wa.layout(L.dtype, 1, wl.head_dim)
    for h in range(wl.n_heads):
        for b in range(q_blocks):
            item = h * q_blocks + b
            keys = np.concatenate([np.arange(64 * t, min(64 * t + 64, n_keys))
                                   for t in tiles[item, :count[item]]])
            rows = slice(256 * b, min(256 * (b + 1), q.shape[0]))
            qh = np.ascontiguousarray(q[rows, h:h + 1])
            kh = np.ascontiguousarray(k_all[keys, h:h + 1])
            vh = np.ascontiguousarray(v_all[keys, h:h + 1])
            say("dense over gathered keys, head", h, "block", b, "keys", keys.size)
            o_d = wa.wa_block_attention(L1, to_device(qh), to_device(kh), to_device(vh), None,
                                        None, wl.softmax_scale, out_dtype=wa.WA_F32)
            torch.cuda.synchronize()
            assert np.array_equal(_bits(out[rows, h:h + 1].contiguous()), _bits(o_d))


def test_hand_written_lists():
    """Lists not made by the selection: a single tile (the ragged last one, and
    the first), every other tile, and the ragged tile after a gap."""
    wl = SMALL
    L = wa_layout(wl)
    q, kc, vc, ko, vo = _inputs(wl, [5, 0, 3, 7, 2], 576, 560, gain=8.0)
    q_blocks, items, n_tiles = wa.hsa_shape(L, q.shape[0], 576, 560)
    k_all, v_all = np.concatenate([kc, ko]), np.concatenate([vc, vo])
    n_keys = k_all.shape[0]
    lists = [[n_tiles - 1], [0], list(range(0, n_tiles, 2)), [1, 4, n_tiles - 1]]
    qd, kcd, vcd, kod, vod = (to_device(x) for x in (q, kc, vc, ko, vo))
    for lst in lists:
        tiles = np.zeros((items, n_tiles), np.int32)
        count = np.zeros(items, np.int32)
        for i in range(items):   # rotate the lists over the items
            li = lists[(lists.index(lst) + i) % len(lists)]
            tiles[i, :len(li)] = li
            count[i] = len(li)
        say("sparse attention, hand-written lists", lst)
        out = wa.wa_sparse_attention(L, qd, kcd, vcd, kod, vod, torch.from_numpy(tiles).cuda(),
                                     torch.from_numpy(count).cuda(), wl.softmax_scale,
                                     out_dtype=wa.WA_F32)
        torch.cuda.synchronize()
        got = to_f64(out)
        for h in range(wl.n_heads):
            for b in range(q_blocks):
                item = h * q_blocks + b
                keys = np.concatenate([np.arange(64 * t, min(64 * t + 64, n_keys))
                                       for t in tiles[item, :count[item]]])
                rows = np.arange(256 * b, min(256 * (b + 1), q.shape[0]))[::37]
                ref, _ = oracle.attention(np.ascontiguousarray(q[:, h:h + 1]),
                                          np.ascontiguousarray(k_all[keys, h:h + 1]),
                                          np.ascontiguousarray(v_all[keys, h:h + 1]), None, None,
                                          wl.softmax_scale, rows=rows)
                assert np.abs(got[rows, h:h + 1] - ref).max() <= attention_tolerance(wl)


def test_sparse_full_size():
    """wan_kp4 at full size: 4 gathered pages (49,920 keys) + 4,680 own keys,
    12 heads, 4,680 queries (19 query blocks, 464 key blocks); the selection
    of three query blocks, and every row of query block 9 and of the ragged
    last block (72 rows) plus sampled rows of block 0, in both output dtypes,
    against the oracle."""
    wl = W.WORKLOADS["wan_kp4"]
    q, kc, vc, ko, vo = _inputs(wl, [11, 3, 14, 7], 49920, 4680, gain=8.0)
    tau = [0.5 + 0.04 * h for h in range(wl.n_heads)]
    L = wa_layout(wl)
    tau_d = torch.tensor(tau, dtype=torch.float64, device="cuda")
    say("hsa select, full size")
    tiles, count, gini = wa.wa_hsa_select(L, to_device(q), to_device(kc), to_device(ko), tau_d,
                                          scale=wl.softmax_scale)
    torch.cuda.synchronize()
    tiles, count, gini = tiles.cpu().numpy(), count.cpu().numpy(), gini.cpu().numpy()
    q_blocks = wa.hsa_shape(L, q.shape[0], 49920, 4680)[0]
    rows = np.concatenate([np.arange(0, 256, 51), np.arange(256 * 9, 256 * 10),
                           np.arange(256 * 18, q.shape[0])])
    ref = oracle.hsa_sparse(q, kc, vc, ko, vo, wl.softmax_scale, tau, rows=rows)
    blocks = ref["blocks"]
    for (h, b), chosen in ref["sel"].items():
        item = h * q_blocks + b
        _clear_cut(ref["maps"][b][h], tau[h])
        assert tiles[item, :count[item]].tolist() == _tiles_of(blocks, chosen)
        assert abs(gini[item] - ref["gini"][(h, b)]) <= 1e-12
    for odt in (wa.WA_BF16, wa.WA_F32):
        say("sparse attention, full size", odt)
        out = wa.wa_sparse_attention(L, to_device(q), to_device(kc), to_device(vc),
                                     to_device(ko), to_device(vo), torch.from_numpy(tiles).cuda(),
                                     torch.from_numpy(count).cuda(), wl.softmax_scale,
                                     out_dtype=odt)
        torch.cuda.synchronize()
        assert np.abs(to_f64(out)[rows] - ref["out"]).max() <= attention_tolerance(wl)


def test_full_size_full_list_does_not_split_and_equals_dense():
    """Every tile of every item at full size (228 items of 854 tiles): even
    lists, so the launch keeps one workgroup per item, and the output is bit
    for bit the dense call's."""
    wl = W.WORKLOADS["wan_kp4"]
    L = wa_layout(wl)
    q, kc, vc, ko, vo = _inputs(wl, [11, 3, 14, 7], 49920, 4680, gain=8.0)
    qd, kcd, vcd, kod, vod = (to_device(x) for x in (q, kc, vc, ko, vo))
    assert wa.wa_attention_workspace_bytes(L, q.shape[0], 49920, 4680) == 0   # dense: no split
    tau = torch.full((wl.n_heads,), 2.0, dtype=torch.float64, device="cuda")
    say("hsa select, full size, keep all")
    tiles, count, _ = wa.wa_hsa_select(L, qd, kcd, kod, tau, scale=wl.softmax_scale)
    say("sparse and dense attention, full size, every tile")
    o_s = wa.wa_sparse_attention(L, qd, kcd, vcd, kod, vod, tiles, count, wl.softmax_scale,
                                 out_dtype=wa.WA_BF16)
    o_d = wa.wa_block_attention(L, qd, kcd, vcd, kod, vod, wl.softmax_scale, out_dtype=wa.WA_BF16)
    torch.cuda.synchronize()
    assert (count.cpu().numpy() == wa.hsa_shape(L, q.shape[0], 49920, 4680)[2]).all()
    assert np.array_equal(_bits(o_s), _bits(o_d))


def test_split_one_long_list_over_many_blocks():
    """One head, 320 queries (two items) over 76,800 + 320 keys (1,205 tiles):
    item 0 lists every tile, item 1 every 30th and the last (ragged) one.  The
    lists are uneven, so the launch splits them over 64 blocks (19-tile runs)
    and item 0 is merged from about 64 pieces; sampled rows against the
    oracle, fp32 and bf16 outputs, with lse."""
    wl = W.scaled(W.WORKLOADS["wan_kp4"], n_heads=1, frame_tokens=64, page_frames=200,
                  n_pages=6, chunk_frames=5)
    L = wa_layout(wl)
    q, kc, vc, ko, vo = _inputs(wl, list(range(6)), 6 * 12800, 320, gain=0.0)
    q_blocks, items, n_tiles = wa.hsa_shape(L, q.shape[0], kc.shape[0], ko.shape[0])
    assert (q_blocks, items, n_tiles) == (2, 2, 1205)
    lists = [list(range(n_tiles)), sorted(set(range(0, n_tiles, 30)) | {n_tiles - 1})]
    tiles = np.zeros((items, n_tiles), np.int32)
    count = np.zeros(items, np.int32)
    for i, li in enumerate(lists):
        tiles[i, :len(li)] = li
        count[i] = len(li)
    k_all, v_all = np.concatenate([kc, ko]), np.concatenate([vc, vo])
    n_keys = k_all.shape[0]
    qd = to_device(q)
    for odt in (wa.WA_F32, wa.WA_BF16):
        lse = torch.empty(1, q.shape[0], dtype=torch.float32, device="cuda")
        say("sparse attention, split over many blocks", odt)
        out = wa.wa_sparse_attention(L, qd, to_device(kc), to_device(vc), to_device(ko),
                                     to_device(vo), torch.from_numpy(tiles).cuda(),
                                     torch.from_numpy(count).cuda(), wl.softmax_scale,
                                     out_dtype=odt, lse=lse)
        torch.cuda.synchronize()
        got, got_lse = to_f64(out), lse.cpu().double().numpy()
        for i in range(items):
            keys = np.concatenate([np.arange(64 * t, min(64 * t + 64, n_keys)) for t in lists[i]])
            rows = np.arange(256 * i, min(256 * (i + 1), q.shape[0]))[::23]
            ref, ref_lse = oracle.attention(q, np.ascontiguousarray(k_all[keys]),
                                            np.ascontiguousarray(v_all[keys]), None, None,
                                            wl.softmax_scale, rows=rows)
            assert np.abs(got[rows] - ref).max() <= attention_tolerance(wl)
            assert np.abs(got_lse[:, rows] - ref_lse).max() <= attention_tolerance(wl)


def test_more_items_than_compute_units():
    """12 heads x 24 query blocks = 288 items (more than the 256 CUs: the
    launch plans in rounds) over 4 pages of 1,024 keys plus 6,144 own keys,
    thresholds that differ by head; selection of three query blocks and
    sampled rows of the output against the oracle."""
    wl = W.scaled(W.WORKLOADS["wan_kp4"], frame_tokens=128, page_frames=8, n_pages=4,
                  chunk_frames=48)
    L = wa_layout(wl)
    q, kc, vc, ko, vo = _inputs(wl, [3, 0, 2, 1], 4096, wl.n_q, gain=8.0)
    q_blocks, items, n_tiles = wa.hsa_shape(L, q.shape[0], 4096, wl.n_q)
    assert (q_blocks, items) == (24, 288)
    tau = [0.3 + 0.06 * h for h in range(wl.n_heads)]
    tau_d = torch.tensor(tau, dtype=torch.float64, device="cuda")
    say("hsa select, 288 items")
    tiles, count, gini = wa.wa_hsa_select(L, to_device(q), to_device(kc), to_device(ko), tau_d,
                                          scale=wl.softmax_scale)
    say("sparse attention, 288 items")
    out = wa.wa_sparse_attention(L, to_device(q), to_device(kc), to_device(vc), to_device(ko),
                                 to_device(vo), tiles, count, wl.softmax_scale,
                                 out_dtype=wa.WA_F32)
    torch.cuda.synchronize()
    tiles, count, gini = tiles.cpu().numpy(), count.cpu().numpy(), gini.cpu().numpy()
    rows = np.concatenate([np.arange(0, 256, 37), np.arange(256 * 11, 256 * 12, 37),
                           np.arange(256 * 23, q.shape[0], 37), [q.shape[0] - 1]])
    ref = oracle.hsa_sparse(q, kc, vc, ko, vo, wl.softmax_scale, tau, rows=rows)
    for (h, b), chosen in ref["sel"].items():
        item = h * q_blocks + b
        _clear_cut(ref["maps"][b][h], tau[h])
        assert tiles[item, :count[item]].tolist() == _tiles_of(ref["blocks"], chosen)
        assert abs(gini[item] - ref["gini"][(h, b)]) <= 1e-12
    assert np.abs(to_f64(out)[rows] - ref["out"]).max() <= attention_tolerance(wl)
