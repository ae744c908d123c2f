"""The attention kernel's LDS ring under the debug build libwa_poison.so
(WA_DEBUG_POISON): the whole K/V ring holds NaN when a block starts, and every
stage is filled with NaN again after the barrier that ends its last reads and
before the copies that refill it.  A read of a stage whose tile has not landed
(a missing wait), of a stage nothing was copied into, or of a stage's previous
tile would carry NaN into the products.  The regular kernel issues the last
tile again into a stage nobody reads and computes the (discarded) products of
the tile after the last; here every output stays finite, bit for bit equal to
the regular build's, and within the oracle's tolerance, in the contiguous,
paged (whole-tile and per-row pages), split and tile-list modes.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_page_amd as wa
import wa_workloads as W
from tests.pipeline import attention_tolerance, rows_sample, say, to_device, to_f64

pytestmark = pytest.mark.gpu

POISON = os.path.join(os.path.dirname(os.path.abspath(wa.__file__)), "libwa_poison.so")
WL = W.scaled(W.WORKLOADS["wan_kp4"], name="poison_bf16", n_heads=3, frame_tokens=64,
              page_frames=2, n_pages=8, chunk_frames=5)      # 128-token pages, 320 queries


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(POISON):
        raise RuntimeError("libwa_poison.so is not built; run __graft_entry__.build()")
    wa.load_library()


def _rows(n, seed):
    rng = np.random.default_rng([WL.wid, 77, seed])
    return W.encode(WL, rng.standard_normal((n, WL.n_heads, WL.head_dim), dtype=np.float32))


def _both(call):
    """call() with the regular library, then with the poison build."""
    torch.cuda.synchronize()
    reg = call()
    torch.cuda.synchronize()
    prev = wa.use_library(POISON)
    try:
        poi = call()
        torch.cuda.synchronize()
    finally:
        wa.use_library(prev)
    return reg, poi


def _same(reg, poi):
    for a, b in zip(reg, poi):
        assert torch.isfinite(b).all(), "a poisoned stage reached an output"
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


def _attn(L, q, kc, vc, ko, vo, odt):
    lse = torch.empty(WL.n_heads, q.shape[0], dtype=torch.float32, device="cuda")
    out = wa.wa_block_attention(L, q, kc, vc, ko, vo, WL.softmax_scale, out_dtype=odt, lse=lse)
    return out, lse


@pytest.mark.parametrize("n_q,n_ctx,n_own", [(300, 600, 300), (64, 0, 65), (257, 128, 1)])
def test_contiguous(n_q, n_ctx, n_own):
    L = wa.layout(wa.WA_BF16, WL.n_heads, WL.head_dim)
    q, kc, vc, ko, vo = (_rows(n_q, 1), _rows(n_ctx, 2), _rows(n_ctx, 3), _rows(n_own, 4),
                         _rows(n_own, 5))
    dev = [to_device(x) if x.shape[0] else None for x in (q, kc, vc, ko, vo)]
    say("poison: contiguous", n_q, n_ctx, n_own)
    reg, poi = _both(lambda: _attn(L, *dev, wa.WA_F32))
    _same(reg, poi)
    ref, ref_lse = oracle.attention(q, kc if n_ctx else None, vc if n_ctx else None, ko, vo,
                                    WL.softmax_scale)
    assert np.abs(to_f64(poi[0]) - ref).max() <= attention_tolerance(WL)
    assert np.abs(poi[1].cpu().double().numpy() - ref_lse).max() <= attention_tolerance(WL)


@pytest.mark.parametrize("odt", [wa.WA_F32, wa.WA_BF16], ids=["f32_out", "bf16_out"])
def test_split_launch(odt):
    """3 heads x 257 queries over 40,000 + 257 keys: the launch splits each
    item's key tiles over all CUs (a block then runs several pieces, its
    ring carried from one piece to the next) and merges the pieces."""
    n_q, n_ctx, n_own = 257, 40000, 257
    L = wa.layout(wa.WA_BF16, WL.n_heads, WL.head_dim)
    assert wa.wa_attention_workspace_bytes(L, n_q, n_ctx, n_own) > 0, "expected a split launch"
    q, kc, vc, ko, vo = (_rows(n_q, 11), _rows(n_ctx, 12), _rows(n_ctx, 13), _rows(n_own, 14),
                         _rows(n_own, 15))
    dev = [to_device(x) for x in (q, kc, vc, ko, vo)]
    say("poison: split", n_q, n_ctx, n_own, odt)
    reg, poi = _both(lambda: _attn(L, *dev, odt))
    _same(reg, poi)
    rows = np.array([0, 31, 32, 200, 255, 256], dtype=np.int64)
    ref, _ = oracle.attention(q, kc, vc, ko, vo, WL.softmax_scale, rows=rows)
    assert np.abs(to_f64(poi[0])[rows] - ref).max() <= attention_tolerance(WL)


@pytest.mark.parametrize("page_tokens", [128, 100], ids=["whole_tiles", "per_row"])
def test_paged(page_tokens):
    """Pages read in place through idx, out of order, then 90 own keys."""
    n_pages, k_p, n_q, n_own = 6, 4, 200, 90
    L = wa.layout(wa.WA_BF16, WL.n_heads, WL.head_dim, page_tokens, n_pages)
    kp = _rows(n_pages * page_tokens, 21).reshape(n_pages, page_tokens, WL.n_heads, WL.head_dim)
    vp = _rows(n_pages * page_tokens, 22).reshape(n_pages, page_tokens, WL.n_heads, WL.head_dim)
    q, ko, vo = _rows(n_q, 23), _rows(n_own, 24), _rows(n_own, 25)
    idx = np.array([4, 1, 5, 2], np.int32)
    kpd, vpd = to_device(kp), to_device(vp)
    qd, kod, vod = to_device(q), to_device(ko), to_device(vo)
    idxd = torch.from_numpy(idx).cuda()

    def call():
        lse = torch.empty(WL.n_heads, n_q, dtype=torch.float32, device="cuda")
        out = wa.wa_paged_attention(L, qd, kpd, vpd, idxd, k_p, kod, vod, WL.softmax_scale,
                                    out_dtype=wa.WA_F32, lse=lse)
        return out, lse
    say("poison: paged", page_tokens)
    reg, poi = _both(call)
    _same(reg, poi)
    kc = np.concatenate([kp[i] for i in idx])
    vc = np.concatenate([vp[i] for i in idx])
    ref, _ = oracle.attention(q, kc, vc, ko, vo, WL.softmax_scale)
    assert np.abs(to_f64(poi[0]) - ref).max() <= attention_tolerance(WL)


def _lists(items, n_tiles, lists):
    tiles = np.zeros((items, n_tiles), np.int32)
    count = np.zeros(items, np.int32)
    for i, lst in enumerate(lists):
        tiles[i, :len(lst)] = lst
        count[i] = len(lst)
    return torch.from_numpy(tiles).cuda(), torch.from_numpy(count).cuda()


@pytest.mark.parametrize("case", ["one_ragged_tile", "every_other", "uneven_split"])
def test_tile_lists(case):
    """wa_sparse_attention over hand-written tile lists: a single ragged last
    tile, every other tile, and lists uneven enough that the plan cuts them
    into runs over all CUs (one item holds every tile of 100,032 + 300 keys,
    the others every other tile)."""
    n_q = 300 if case != "uneven_split" else 512
    n_ctx = 640 if case != "uneven_split" else 100032
    n_own = 300
    L = wa.layout(wa.WA_BF16, WL.n_heads, WL.head_dim)
    q, kc, vc, ko, vo = (_rows(n_q, 31), _rows(n_ctx, 32), _rows(n_ctx, 33), _rows(n_own, 34),
                         _rows(n_own, 35))
    q_blocks, items, n_tiles = wa.hsa_shape(L, n_q, n_ctx, n_own)
    if case == "one_ragged_tile":
        lists = [[n_tiles - 1]] * items
    elif case == "every_other":
        lists = [list(range(i % 2, n_tiles, 2)) for i in range(items)]
    else:
        lists = [list(range(n_tiles)) if i == 0 else list(range(i % 2, n_tiles, 2))
                 for i in range(items)]
    tiles, count = _lists(items, n_tiles, lists)
    dev = [to_device(x) for x in (q, kc, vc, ko, vo)]

    def call():
        lse = torch.empty(WL.n_heads, n_q, dtype=torch.float32, device="cuda")
        out = wa.wa_sparse_attention(L, *dev, tiles, count, WL.softmax_scale,
                                     out_dtype=wa.WA_F32, lse=lse)
        return out, lse
    say("poison: tile lists", case)
    reg, poi = _both(call)
    _same(reg, poi)
    n_keys = n_ctx + n_own
    kall, vall = np.concatenate([kc, ko]), np.concatenate([vc, vo])
    for item in (0, items - 1):
        h, b = item // q_blocks, item % q_blocks
        keys = np.concatenate([np.arange(64 * t, min(64 * t + 64, n_keys)) for t in lists[item]])
        rows = rows_sample(min(256, n_q - 256 * b), 5) + 256 * b
        sub = lambda x: x[:, h:h + 1]
        ref, _ = oracle.attention(sub(q[rows]), sub(kall[keys]), sub(vall[keys]), None, None,
                                  WL.softmax_scale)
        got = to_f64(poi[0])[rows][:, h:h + 1]
        assert np.abs(got - ref).max() <= attention_tolerance(WL)
