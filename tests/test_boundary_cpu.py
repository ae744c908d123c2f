"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments on the host before anything is launched.

Pointers here are fake aligned addresses: every call below fails validation,
which runs before any HIP call, so nothing touches a device.
"""
import ctypes
import os
import re

import pytest

import paged_kv_attention_page_amd as wa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wa.h")

A = ctypes.c_void_p(0x10000)        # a 16-byte aligned stand-in pointer
B = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)      # misaligned
NULL = None


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(wa.library_path()):
        pytest.skip("libwa.so not built (run __graft_entry__.build())")
    return wa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("wa_append_page", "wa_select_pages", "wa_gather", "wa_block_attention"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), "libwa.so does not export %s" % n


def test_status_strings(lib):
    assert wa.wa_status_string(wa.WA_OK) == "ok"
    for s in (wa.WA_ERR_INVALID_ARG, wa.WA_ERR_UNSUPPORTED, wa.WA_ERR_HIP):
        assert wa.wa_status_string(s) not in ("ok", "unknown status")
    assert wa.wa_status_string(-99) == "unknown status"


def L(dtype=wa.WA_BF16, H=12, d=128, pt=12480, pages=16):
    return ctypes.byref(wa.layout(dtype, H, d, pt, pages))


# ---------------------------------------------------------------------------
# append

def test_append_workspace_size(lib):
    n = lib.wa_append_workspace_bytes(L())
    assert n > 0 and n % 8 == 0
    assert lib.wa_append_workspace_bytes(None) == 0
    assert lib.wa_append_workspace_bytes(L(H=0)) == 0


@pytest.mark.parametrize("case,expect", [
    ("null_layout", wa.WA_ERR_INVALID_ARG),
    ("null_k_src", wa.WA_ERR_INVALID_ARG),
    ("null_pool", wa.WA_ERR_INVALID_ARG),
    ("null_means", wa.WA_ERR_INVALID_ARG),
    ("null_ws", wa.WA_ERR_INVALID_ARG),
    ("slot_neg", wa.WA_ERR_INVALID_ARG),
    ("slot_big", wa.WA_ERR_INVALID_ARG),
    ("small_ws", wa.WA_ERR_INVALID_ARG),
    ("misaligned", wa.WA_ERR_INVALID_ARG),
    ("v_without_pool", wa.WA_ERR_INVALID_ARG),
    ("bad_dtype", wa.WA_ERR_UNSUPPORTED),
    ("row_too_wide", wa.WA_ERR_UNSUPPORTED),
    ("row_not_16B", wa.WA_ERR_UNSUPPORTED),
])
def test_append_rejects(lib, case, expect):
    lay = L()
    big = 1 << 40
    args = dict(layout=lay, k_src=A, v_src=B, k_pool=A, v_pool=B, slot=3, means=A, ws=A, wsb=big)
    if case == "null_layout":
        args["layout"] = None
    elif case == "null_k_src":
        args["k_src"] = NULL
    elif case == "null_pool":
        args["k_pool"] = NULL
    elif case == "null_means":
        args["means"] = NULL
    elif case == "null_ws":
        args["ws"] = NULL
    elif case == "slot_neg":
        args["slot"] = -1
    elif case == "slot_big":
        args["slot"] = 16
    elif case == "small_ws":
        args["wsb"] = 8
    elif case == "misaligned":
        args["k_src"] = MIS
    elif case == "v_without_pool":
        args["v_pool"] = NULL
    elif case == "bad_dtype":
        args["layout"] = L(dtype=7)
    elif case == "row_too_wide":
        args["layout"] = L(H=64, d=128)
    elif case == "row_not_16B":
        args["layout"] = L(dtype=wa.WA_BF16, H=1, d=4)
    st = lib.wa_append_page(args["layout"], args["k_src"], args["v_src"], args["k_pool"],
                            args["v_pool"], args["slot"], args["means"], args["ws"],
                            args["wsb"], None)
    assert st == expect


# ---------------------------------------------------------------------------
# select

def test_select_workspace_size(lib):
    assert lib.wa_select_workspace_bytes(L(), 4680, 16, None) > 0
    assert lib.wa_select_workspace_bytes(L(), 0, 16, None) == 0
    assert lib.wa_select_workspace_bytes(L(), 4680, 0, None) == 0
    assert lib.wa_select_workspace_bytes(L(), 4680, 5000, None) == 0


def _select(lib, lay=None, q=A, n_q=100, means=A, cand=NULL, n_cand=16, prompt=None, k_p=4,
            out=A, ws=A, wsb=1 << 40):
    return lib.wa_select_pages(lay if lay is not None else L(), q, n_q, means, cand, n_cand,
                               prompt, k_p, out, None, ws, wsb, None)


def test_select_rejects(lib):
    E, U = wa.WA_ERR_INVALID_ARG, wa.WA_ERR_UNSUPPORTED
    assert _select(lib, q=NULL) == E
    assert _select(lib, means=NULL) == E
    assert _select(lib, out=NULL) == E
    assert _select(lib, ws=NULL) == E
    assert _select(lib, n_q=0) == E
    assert _select(lib, n_cand=0) == E
    assert _select(lib, k_p=0) == E
    assert _select(lib, k_p=-2) == E
    assert _select(lib, k_p=17) == E
    assert _select(lib, n_cand=5000, k_p=4) == U
    assert _select(lib, wsb=16) == E
    assert _select(lib, q=MIS) == E
    assert _select(lib, lay=L(pages=0)) == E


def _select_noalloc(lib, lay=None, q=A, n_q=100, means=A, cand=NULL, n_cand=16, prompt=None,
                    k_p=4, out=A):
    return lib.wa_select_pages_noalloc(lay if lay is not None else L(), q, n_q, means, cand,
                                       n_cand, prompt, k_p, out, None, None)


def test_select_noalloc_rejects_before_touching_the_gpu(lib):
    """wa_select_pages_noalloc: the same argument rules as wa_select_pages, and
    a selection whose workspace would exceed the library's fixed per-device
    array (WA_SELECT_NOALLOC_MAX_WORKSPACE) is refused; all of it before any
    HIP call."""
    E, U = wa.WA_ERR_INVALID_ARG, wa.WA_ERR_UNSUPPORTED
    assert _select_noalloc(lib, q=NULL) == E
    assert _select_noalloc(lib, means=NULL) == E
    assert _select_noalloc(lib, out=NULL) == E
    assert _select_noalloc(lib, n_q=0) == E
    assert _select_noalloc(lib, k_p=0) == E
    assert _select_noalloc(lib, k_p=17) == E
    assert _select_noalloc(lib, n_cand=5000, k_p=4) == U
    assert _select_noalloc(lib, q=MIS) == E
    assert _select_noalloc(lib, lay=L(pages=0)) == E
    # workspace of 12 x 128 bf16 rows: fits up to a few hundred thousand queries
    limit = 8 << 20
    assert lib.wa_select_workspace_bytes(L(), 4680, 16, None) <= limit
    big = 1 << 22
    assert lib.wa_select_workspace_bytes(L(), big, 16, None) > limit
    assert _select_noalloc(lib, n_q=big) == U


def _window(lib, lay=None, q=A, n_q=100, means=A, cand=NULL, n_cand=16, recent=B, n_recent=2,
            k_p=4, out=A, ws=A, wsb=1 << 40):
    return lib.wa_select_window(lay if lay is not None else L(), q, n_q, means, cand, n_cand,
                                None, recent, n_recent, k_p, out, None, ws, wsb, None)


def test_select_window_rejects(lib):
    """The window's own rules, one bad argument per call (the rest of the
    page-stage rules are shared with wa_select_pages)."""
    E, U = wa.WA_ERR_INVALID_ARG, wa.WA_ERR_UNSUPPORTED
    assert _window(lib, recent=NULL) == E                    # n_recent > 0 needs the ids
    assert _window(lib, n_recent=-1) == E
    assert _window(lib, n_recent=0, k_p=0) == E              # nothing to select
    assert _window(lib, k_p=-1) == E
    assert _window(lib, k_p=17) == E                         # more than the candidates
    assert _window(lib, recent=ctypes.c_void_p(0x20002)) == E
    assert _window(lib, n_recent=65) == U                    # over WA_MAX_WINDOW
    assert _window(lib, q=NULL) == E
    assert _window(lib, ws=NULL) == E
    assert _window(lib, wsb=16) == E
    assert _window(lib, lay=L(pages=0)) == E


def _prompt(n_chunks=16, emb=4096, ppc=4, keep=4):
    return wa.PromptStage(0x30000, 0x40000, 0x50000, n_chunks, emb, ppc, keep, None, None)


def test_select_workspace_size_with_prompt_stage(lib):
    """With a prompt stage the workspace depends on the prompt's shape: an
    inconsistent one gets 0 (as the selection itself rejects it), and the
    one-launch layout holds a partial score for every page of every chunk, so
    fewer chunks need less room."""
    ws = lambda n_cand, p: lib.wa_select_workspace_bytes(L(), 4680, n_cand, ctypes.byref(p))
    full = ws(16, _prompt())                          # 16 chunks x 4 pages: one launch
    assert full > 0
    assert ws(16, _prompt(n_chunks=8)) < full         # 32 pages scored instead of 64
    assert ws(12, _prompt()) == 0                     # n_cand != n_keep * pages_per_chunk
    assert ws(16, _prompt(keep=17)) == 0              # n_keep > n_chunks
    assert ws(16, _prompt(ppc=0, keep=4)) == 0
    assert ws(16, _prompt(keep=0)) == 0
    assert ws(16, _prompt(n_chunks=17)) > 0           # 68 pages: three launches


def test_select_rejects_bad_prompt_stage(lib):
    E, U = wa.WA_ERR_INVALID_ARG, wa.WA_ERR_UNSUPPORTED
    ok = _prompt()
    # candidates given as well as a prompt stage
    assert _select(lib, cand=B, prompt=ctypes.byref(ok)) == E
    # n_cand must equal n_keep * pages_per_chunk
    assert _select(lib, n_cand=12, prompt=ctypes.byref(ok)) == E
    assert _select(lib, prompt=ctypes.byref(_prompt(keep=17))) == E
    assert _select(lib, prompt=ctypes.byref(_prompt(keep=0))) == E
    assert _select(lib, prompt=ctypes.byref(_prompt(emb=0))) == E
    assert _select(lib, n_cand=4, k_p=4, prompt=ctypes.byref(_prompt(n_chunks=5000, ppc=1, keep=4))) == U
    bad = _prompt()
    bad.chunk_prompts = None
    assert _select(lib, prompt=ctypes.byref(bad)) == E


# ---------------------------------------------------------------------------
# gather

def test_gather_rejects(lib):
    E, U = wa.WA_ERR_INVALID_ARG, wa.WA_ERR_UNSUPPORTED
    g = lib.wa_gather
    assert g(None, A, B, A, 4, A, B, None) == E
    assert g(L(), NULL, B, A, 4, A, B, None) == E
    assert g(L(), A, B, NULL, 4, A, B, None) == E
    assert g(L(), A, B, A, 4, NULL, B, None) == E
    assert g(L(), A, NULL, A, 4, A, B, None) == E        # only one of v_pool / v_ctx
    assert g(L(), A, B, A, 0, A, B, None) == E
    assert g(L(), A, B, A, 70000, A, B, None) == U
    assert g(L(), MIS, B, A, 4, A, B, None) == E
    assert g(L(pt=0), A, B, A, 4, A, B, None) == E


# ---------------------------------------------------------------------------
# attention

def _attn(lib, lay=None, q=A, n_q=64, kc=A, vc=B, n_ctx=64, ko=A, vo=B, n_own=64, scale=0.1,
          odt=wa.WA_F32, out=B, lse=NULL, ws=NULL, ws_bytes=0):
    return lib.wa_block_attention(lay if lay is not None else L(), q, n_q, kc, vc, n_ctx, ko, vo,
                                  n_own, scale, odt, out, lse, ws, ws_bytes, None)


def test_attention_workspace_size(lib):
    """A launch splits its items' key tiles over the CUs (256 on MI355X, and
    when no device can be queried) only when one block per (query block, head)
    item would leave more than a quarter of them idle.  The workspace then
    holds one slot per piece an item was cut into: 256 x 128 fp32 outputs plus
    a max and a row sum per query row.  4 query blocks x 12 heads x 318 tiles
    on 256 blocks: 59 head tiles per item (at most 2 pieces), a 259-tile tail
    (at most ceil(259 / 59) + 1 = 6 pieces)."""
    assert lib.wa_attention_workspace_bytes(L(), 4680, 49920, 4680) == 0   # 228 items: no split
    n = lib.wa_attention_workspace_bytes(L(), 1024, 20000, 300)
    assert n == 48 * 8 * 256 * (128 + 2) * 4
    assert lib.wa_attention_workspace_bytes(L(), 64, 64, 64) == 0          # too few tiles
    assert lib.wa_attention_workspace_bytes(L(dtype=wa.WA_F32, d=64), 1024, 20000, 300) == 0
    assert lib.wa_attention_workspace_bytes(L(), 0, 64, 64) == 0           # rejected arguments
    assert lib.wa_attention_workspace_bytes(None, 64, 64, 64) == 0


def test_attention_rejects(lib):
    E, U = wa.WA_ERR_INVALID_ARG, wa.WA_ERR_UNSUPPORTED
    assert _attn(lib, q=NULL) == E
    assert _attn(lib, out=NULL) == E
    assert _attn(lib, n_q=0) == E
    assert _attn(lib, n_ctx=-1) == E
    assert _attn(lib, n_own=-1) == E
    assert _attn(lib, n_ctx=0, n_own=0) == E
    assert _attn(lib, kc=NULL) == E
    assert _attn(lib, vo=NULL) == E
    assert _attn(lib, scale=float("nan")) == E
    assert _attn(lib, scale=float("inf")) == E
    assert _attn(lib, scale=0.0) == E
    assert _attn(lib, scale=-0.5) == E
    assert _attn(lib, q=MIS) == E
    assert _attn(lib, lse=ctypes.c_void_p(0x10002)) == E
    assert _attn(lib, lay=L(d=64)) == U                       # bf16 needs head_dim 128
    assert _attn(lib, lay=L(dtype=wa.WA_F32, d=96)) == U       # fp32: 64 or 128
    assert _attn(lib, lay=L(dtype=wa.WA_F32, d=64), odt=wa.WA_BF16) == U
    assert _attn(lib, odt=5) == U
    big = dict(n_q=1024, n_ctx=20000, n_own=300, odt=wa.WA_BF16)
    assert _attn(lib, **big) == E                                         # workspace missing
    assert _attn(lib, ws=A, ws_bytes=1024, **big) == E                    # too small
    assert _attn(lib, ws=MIS, ws_bytes=1 << 30, **big) == E               # misaligned


def _pattn(lib, lay=None, q=A, n_q=64, kp=A, vp=B, idx=A, k_p=2, ko=A, vo=B, n_own=64,
           scale=0.1, odt=wa.WA_F32, out=B, lse=NULL, ws=NULL, ws_bytes=0):
    return lib.wa_paged_attention(lay if lay is not None else L(), q, n_q, kp, vp, idx, k_p, ko,
                                  vo, n_own, scale, odt, out, lse, ws, ws_bytes, None)


def test_paged_attention_rejects(lib):
    """Every argument rule of wa_paged_attention, one bad argument per call."""
    E, U = wa.WA_ERR_INVALID_ARG, wa.WA_ERR_UNSUPPORTED
    assert lib.wa_paged_attention(None, A, 64, A, B, A, 2, A, B, 64, 0.1, wa.WA_F32, B, NULL,
                                  NULL, 0, None) == E
    assert _pattn(lib, kp=NULL) == E
    assert _pattn(lib, vp=NULL) == E
    assert _pattn(lib, idx=NULL) == E
    assert _pattn(lib, idx=ctypes.c_void_p(0x10002)) == E     # int32 alignment
    assert _pattn(lib, k_p=0) == E
    assert _pattn(lib, k_p=-3) == E
    assert _pattn(lib, lay=L(pt=0)) == E
    assert _pattn(lib, lay=L(pages=0)) == E
    assert _pattn(lib, k_p=200000) == U                       # k_p * page_tokens overflows
    assert _pattn(lib, q=NULL) == E
    assert _pattn(lib, out=NULL) == E
    assert _pattn(lib, n_q=0) == E
    assert _pattn(lib, n_own=-1) == E
    assert _pattn(lib, ko=NULL) == E
    assert _pattn(lib, kp=MIS) == E
    assert _pattn(lib, scale=float("nan")) == E
    assert _pattn(lib, lay=L(d=64)) == U
    assert _pattn(lib, odt=5) == U
    big = dict(n_q=1024, k_p=2, n_own=300, odt=wa.WA_BF16)
    assert lib.wa_attention_workspace_bytes(L(), 1024, 2 * 12480, 300) > 0
    assert _pattn(lib, **big) == E                           # workspace missing
    assert _pattn(lib, ws=A, ws_bytes=1024, **big) == E      # too small


# ---------------------------------------------------------------------------
# sparse branch (every case below is rejected on the host: nothing launches)

def test_hsa_workspace_size(lib):
    """fp64 key-block sums [390 context + 74 own blocks][1536], query-block
    sums [19][1536] (each 256-byte aligned), then block scores [19 x 12
    items][464], for 49,920 + 4,680 keys and 4,680 queries of 12 x 128."""
    kb = (390 + 74) * 1536 * 8
    qb = 19 * 1536 * 8
    assert lib.wa_hsa_workspace_bytes(L(), 4680, 49920, 4680) == \
        (kb + 255) // 256 * 256 + (qb + 255) // 256 * 256 + 19 * 12 * 464 * 8
    assert lib.wa_hsa_workspace_bytes(L(), 4680, 49900, 4680) == 0      # n_ctx % 64
    assert lib.wa_hsa_workspace_bytes(L(), 0, 64, 64) == 0
    assert lib.wa_hsa_workspace_bytes(L(), 64, 0, 0) == 0
    assert lib.wa_hsa_workspace_bytes(L(), 64, 128 * 2048, 64) == 0     # 2,049 key blocks
    assert lib.wa_hsa_workspace_bytes(L(H=2, d=512), 64, 64, 64) == 0   # head_dim > 128
    assert lib.wa_hsa_workspace_bytes(L(H=2, d=256), 64, 64, 64) == 0   # head_dim > 128
    assert lib.wa_hsa_workspace_bytes(None, 64, 64, 64) == 0


def _hsel(lib, lay=None, q=A, n_q=300, kc=A, n_ctx=640, ko=B, n_own=100, scale=0.1, tau=A,
          tiles=B, count=A, gini=NULL, ws=A, ws_bytes=1 << 20):
    return lib.wa_hsa_select(lay if lay is not None else L(), q, n_q, kc, n_ctx, ko, n_own, scale,
                             tau, tiles, count, gini, 0, ws, ws_bytes, None)


def test_hsa_select_rejects(lib):
    """Every argument rule of wa_hsa_select, one bad argument per call."""
    E, U = wa.WA_ERR_INVALID_ARG, wa.WA_ERR_UNSUPPORTED
    assert lib.wa_hsa_select(None, A, 300, A, 640, B, 100, 0.1, A, B, A, NULL, 0, A, 1 << 20,
                             None) == E
    for bad in ("q", "tau", "tiles", "count", "ws"):
        assert _hsel(lib, **{bad: NULL}) == E, bad
    assert _hsel(lib, n_q=0) == E
    assert _hsel(lib, n_ctx=-64) == E
    assert _hsel(lib, n_own=-1) == E
    assert _hsel(lib, n_ctx=0, n_own=0) == E
    assert _hsel(lib, kc=NULL) == E
    assert _hsel(lib, ko=NULL) == E
    for s in (float("nan"), float("inf"), 0.0, -1.0):
        assert _hsel(lib, scale=s) == E
    assert _hsel(lib, q=MIS) == E
    assert _hsel(lib, ws=MIS) == E
    assert _hsel(lib, kc=MIS) == E
    assert _hsel(lib, tau=ctypes.c_void_p(0x10004)) == E     # double alignment
    assert _hsel(lib, gini=ctypes.c_void_p(0x10004)) == E
    assert _hsel(lib, tiles=ctypes.c_void_p(0x10002)) == E   # int32 alignment
    assert _hsel(lib, count=ctypes.c_void_p(0x10002)) == E
    assert _hsel(lib, ws_bytes=1024) == E                    # workspace too small
    assert _hsel(lib, n_ctx=100) == U                        # context not whole tiles
    assert _hsel(lib, lay=L(H=2, d=512)) == U                # head_dim > 128
    assert _hsel(lib, lay=L(H=2, d=256)) == U                # head_dim > 128
    assert _hsel(lib, n_ctx=128 * 2048, n_own=64) == U       # 2,049 key blocks
    assert _hsel(lib, lay=L(dtype=7)) == U


def test_sparse_workspace_size(lib):
    """Plan (256 bytes), list offsets [items + 1] (256-byte aligned), then
    partial results (256 rows x (128 outputs + max + sum) fp32) for items +
    CUs slots: 19 query blocks x 12 heads = 228 items, 256 CUs when no device
    can be queried."""
    items = 19 * 12
    assert lib.wa_sparse_workspace_bytes(L(), 4680, 49920, 4680) == \
        256 + (4 * (items + 1) + 255) // 256 * 256 + (items + 256) * 256 * 130 * 4
    assert lib.wa_sparse_workspace_bytes(L(dtype=wa.WA_F32), 4680, 49920, 4680) == 0
    assert lib.wa_sparse_workspace_bytes(L(), 0, 64, 64) == 0
    assert lib.wa_sparse_workspace_bytes(L(), 64, 64 * 4096, 64) == 0   # 4,097 tiles


def _sattn(lib, lay=None, q=A, n_q=64, kc=A, vc=B, n_ctx=64, ko=A, vo=B, n_own=64, scale=0.1,
           tiles=A, count=B, odt=wa.WA_F32, out=B, lse=NULL, ws=A, ws_bytes=1 << 30):
    return lib.wa_sparse_attention(lay if lay is not None else L(), q, n_q, kc, vc, n_ctx, ko, vo,
                                   n_own, scale, tiles, count, odt, out, lse, ws, ws_bytes, None)


def test_sparse_attention_rejects(lib):
    """Every argument rule of wa_sparse_attention, one bad argument per call."""
    E, U = wa.WA_ERR_INVALID_ARG, wa.WA_ERR_UNSUPPORTED
    assert lib.wa_sparse_attention(None, A, 64, A, B, 64, A, B, 64, 0.1, A, B, wa.WA_F32, B, NULL,
                                   A, 1 << 30, None) == E
    assert _sattn(lib, tiles=NULL) == E
    assert _sattn(lib, count=NULL) == E
    assert _sattn(lib, tiles=ctypes.c_void_p(0x10002)) == E
    assert _sattn(lib, count=ctypes.c_void_p(0x10002)) == E
    assert _sattn(lib, q=NULL) == E
    assert _sattn(lib, out=NULL) == E
    assert _sattn(lib, n_q=0) == E
    assert _sattn(lib, n_ctx=-1) == E
    assert _sattn(lib, n_ctx=0, n_own=0) == E
    assert _sattn(lib, kc=NULL) == E
    assert _sattn(lib, vo=NULL) == E
    assert _sattn(lib, scale=float("nan")) == E
    assert _sattn(lib, q=MIS) == E
    assert _sattn(lib, lay=L(dtype=wa.WA_F32)) == U           # bf16 only
    assert _sattn(lib, lay=L(d=64)) == U                      # head_dim 128
    assert _sattn(lib, odt=5) == U
    assert _sattn(lib, n_ctx=64 * 4096, n_own=64) == U        # 4,097 tiles
    assert _sattn(lib, ws=NULL) == E                          # workspace missing
    assert _sattn(lib, ws=MIS) == E
    assert _sattn(lib, ws_bytes=1024) == E                    # too small


# ---------------------------------------------------------------------------
# host-memory page tier and the merge (rejected on the host: nothing runs)

def _pin(lib, fn="wa_page_in", lay=None, hk=A, hv=B, host_pages=4, host_slot=1, kp=A, vp=B,
         slot=2, row0=100, n_rows=3000):
    f = getattr(lib, fn)
    lay = None if lay == "null" else (lay if lay is not None else L())
    if fn == "wa_page_in":
        return f(lay, hk, hv, host_pages, host_slot, kp, vp, slot, None)
    if fn == "wa_page_in_rows":
        return f(lay, hk, hv, host_pages, host_slot, kp, vp, slot, row0, n_rows, None)
    return f(lay, kp, vp, slot, hk, hv, host_pages, host_slot, None)


@pytest.mark.parametrize("fn", ["wa_page_in", "wa_page_out", "wa_page_in_rows"])
def test_page_copy_rejects(lib, fn):
    """Every argument rule of wa_page_in / wa_page_out / wa_page_in_rows, one
    bad argument per call; the last case passes every other check with a host
    pointer that is not pinned host memory (a stand-in address), so nothing is
    copied."""
    E = wa.WA_ERR_INVALID_ARG
    assert _pin(lib, fn, lay="null") == E
    assert _pin(lib, fn, hk=NULL) == E
    assert _pin(lib, fn, kp=NULL) == E
    assert _pin(lib, fn, hv=NULL) == E                      # one of host_v / v_pool
    assert _pin(lib, fn, vp=NULL) == E
    assert _pin(lib, fn, host_pages=0) == E
    assert _pin(lib, fn, host_slot=-1) == E
    assert _pin(lib, fn, host_slot=4) == E
    assert _pin(lib, fn, slot=-1) == E
    assert _pin(lib, fn, slot=16) == E
    assert _pin(lib, fn, lay=L(pt=0)) == E
    assert _pin(lib, fn, hk=MIS) == E
    assert _pin(lib, fn, vp=MIS) == E
    if fn == "wa_page_in_rows":                             # the row range (page of 12,480)
        assert _pin(lib, fn, row0=-1) == E
        assert _pin(lib, fn, n_rows=0) == E
        assert _pin(lib, fn, row0=12000, n_rows=481) == E
        assert _pin(lib, fn, row0=0, n_rows=12481) == E
        assert _pin(lib, fn, row0=12479, n_rows=1) == E     # in range: fails only on pinning
    assert _pin(lib, fn) == E                               # not pinned host memory


def _merge(lib, lay=None, n_q=64, oa=A, la=B, ob=A, lb=B, odt=wa.WA_F32, out=B, lse=NULL):
    return lib.wa_merge_attention(lay if lay is not None else L(), n_q, oa, la, ob, lb, odt, out,
                                  lse, None)


def test_merge_attention_rejects(lib):
    E, U = wa.WA_ERR_INVALID_ARG, wa.WA_ERR_UNSUPPORTED
    assert lib.wa_merge_attention(None, 64, A, B, A, B, wa.WA_F32, B, NULL, None) == E
    for bad in ("oa", "la", "ob", "lb", "out"):
        assert _merge(lib, **{bad: NULL}) == E, bad
    assert _merge(lib, n_q=0) == E
    assert _merge(lib, oa=MIS) == E
    assert _merge(lib, out=MIS) == E
    assert _merge(lib, la=ctypes.c_void_p(0x10002)) == E
    assert _merge(lib, lse=ctypes.c_void_p(0x10002)) == E
    assert _merge(lib, odt=7) == U
    assert _merge(lib, lay=L(d=30)) == U                     # head_dim % 4
