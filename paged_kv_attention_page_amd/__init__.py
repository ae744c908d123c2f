"""Python binding of libwa.so, the gfx950 paged-KV retrieval attention library.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in ``include/wa.h``; torch provides device memory and the
stream.  The functions carry the C names:

  wa_append_page      copy one page into the pool, record its fp64 mean key
  wa_select_pages     mean query -> page scores -> top-K_p (optional prompt stage)
  wa_gather           copy the selected pages into one contiguous K/V buffer
  wa_block_attention  unmasked softmax attention over [gathered ++ own] K/V

and the rest of ``wa.h`` under the same names: wa_select_window,
wa_select_pages_noalloc, wa_paged_attention, wa_hsa_select,
wa_sparse_attention, wa_page_in, wa_page_in_rows, wa_page_out, wa_merge_attention and the
workspace-size queries.

Host-side shape checks here only make sure every pointer handed to the
library covers the extent the call will touch.  If ``libwa.so`` has not been
built, loading fails loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["WA_OK", "WA_ERR_INVALID_ARG", "WA_ERR_UNSUPPORTED", "WA_ERR_HIP", "WA_F32", "WA_BF16",
           "Layout", "PromptStage", "WaError", "load_library", "library_path", "layout",
           "wa_append_workspace_bytes", "wa_append_page", "wa_select_workspace_bytes",
           "wa_select_pages", "wa_select_window", "wa_gather", "wa_attention_workspace_bytes",
           "wa_block_attention", "wa_paged_attention", "hsa_shape", "wa_hsa_workspace_bytes",
           "wa_hsa_select", "wa_sparse_workspace_bytes", "wa_sparse_attention",
           "wa_page_in", "wa_page_in_rows", "wa_page_out", "wa_merge_attention", "wa_status_string",
           "use_library", "wa_select_pages_noalloc"]

WA_OK, WA_ERR_INVALID_ARG, WA_ERR_UNSUPPORTED, WA_ERR_HIP = 0, -1, -2, -3
WA_F32, WA_BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libwa.so")
_lib = None

_TORCH_DTYPE = {WA_F32: torch.float32, WA_BF16: torch.bfloat16}


class Layout(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_tokens", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]

    @property
    def row_elems(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]


class PromptStage(ctypes.Structure):
    _fields_ = [("chunk_prompts", ctypes.c_void_p), ("cur_prompt", ctypes.c_void_p),
                ("chunk_pages", ctypes.c_void_p), ("n_chunks", ctypes.c_int32),
                ("emb_dim", ctypes.c_int32), ("pages_per_chunk", ctypes.c_int32),
                ("n_keep", ctypes.c_int32), ("out_chunks", ctypes.c_void_p),
                ("out_cand", ctypes.c_void_p)]


class WaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, wa_status_string(status), status))


def library_path() -> str:
    return _LIB_PATH


def use_library(path: str | None = None) -> str:
    """Point the binding at another build of the library (e.g. the debug copy
    libwa_poison.so); None goes back to libwa.so.  Returns the previous path."""
    global _LIB_PATH, _lib
    prev = _LIB_PATH
    _LIB_PATH = path if path is not None else os.path.join(_HERE, "libwa.so")
    _lib = None
    return prev


def kernel_source(name: str) -> bytes:
    """Bytes of one kernel source file (csrc/<name>), e.g. to tie a stored
    profile to the kernel it was taken on."""
    with open(os.path.join(_HERE, "csrc", name), "rb") as f:
        return f.read()


def load_library():
    """Load libwa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libwa.so is not built (%s); run __graft_entry__.build()" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    p, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    L = ctypes.POINTER(Layout)
    P = ctypes.POINTER(PromptStage)
    lib.wa_append_workspace_bytes.argtypes = [L]
    lib.wa_append_workspace_bytes.restype = sz
    lib.wa_append_page.argtypes = [L, p, p, p, p, i32, p, p, sz, p]
    lib.wa_append_page.restype = i32
    lib.wa_select_workspace_bytes.argtypes = [L, i32, i32, P]
    lib.wa_select_workspace_bytes.restype = sz
    lib.wa_select_pages.argtypes = [L, p, i32, p, p, i32, P, i32, p, p, p, sz, p]
    lib.wa_select_pages.restype = i32
    lib.wa_select_pages_noalloc.argtypes = [L, p, i32, p, p, i32, P, i32, p, p, p]
    lib.wa_select_pages_noalloc.restype = i32
    lib.wa_select_window.argtypes = [L, p, i32, p, p, i32, P, p, i32, i32, p, p, p, sz, p]
    lib.wa_select_window.restype = i32
    lib.wa_gather.argtypes = [L, p, p, p, i32, p, p, p]
    lib.wa_gather.restype = i32
    lib.wa_attention_workspace_bytes.argtypes = [L, i32, i32, i32]
    lib.wa_attention_workspace_bytes.restype = sz
    lib.wa_block_attention.argtypes = [L, p, i32, p, p, i32, p, p, i32, f32, i32, p, p, p, sz, p]
    lib.wa_block_attention.restype = i32
    lib.wa_paged_attention.argtypes = [L, p, i32, p, p, p, i32, p, p, i32, f32, i32, p, p, p, sz,
                                       p]
    lib.wa_paged_attention.restype = i32
    lib.wa_hsa_workspace_bytes.argtypes = [L, i32, i32, i32]
    lib.wa_hsa_workspace_bytes.restype = sz
    lib.wa_hsa_select.argtypes = [L, p, i32, p, i32, p, i32, ctypes.c_double, p, p, p, p, i32, p,
                                  sz, p]
    lib.wa_hsa_select.restype = i32
    lib.wa_sparse_attention.argtypes = [L, p, i32, p, p, i32, p, p, i32, f32, p, p, i32, p, p, p,
                                        sz, p]
    lib.wa_page_in.argtypes = [L, p, p, i32, i32, p, p, i32, p]
    lib.wa_page_in.restype = i32
    lib.wa_page_in_rows.argtypes = [L, p, p, i32, i32, p, p, i32, i32, i32, p]
    lib.wa_page_in_rows.restype = i32
    lib.wa_page_out.argtypes = [L, p, p, i32, p, p, i32, i32, p]
    lib.wa_page_out.restype = i32
    lib.wa_merge_attention.argtypes = [L, i32, p, p, p, p, i32, p, p, p]
    lib.wa_merge_attention.restype = i32
    lib.wa_sparse_workspace_bytes.argtypes = [L, i32, i32, i32]
    lib.wa_sparse_workspace_bytes.restype = sz
    lib.wa_sparse_attention.restype = i32
    lib.wa_status_string.argtypes = [i32]
    lib.wa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def wa_status_string(status: int) -> str:
    return load_library().wa_status_string(int(status)).decode()


def layout(dtype: int, n_heads: int, head_dim: int, page_tokens: int = 1,
           max_pages: int = 1) -> Layout:
    return Layout(n_heads, head_dim, page_tokens, max_pages, dtype)


# ----------------------------------------------------------------------------
# marshalling helpers

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status: int, where: str):
    if status != WA_OK:
        raise WaError(status, where)


def _need(t, name, dtype=None, min_elems=None, device=True):
    if t is None:
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if device and not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if min_elems is not None and t.numel() < min_elems:
        raise ValueError("%s holds %d elements, the call needs %d" % (name, t.numel(), min_elems))
    return t


def _rows(t, name, dt, row):
    """Token rows of an optional [T][H][d] segment (0 when absent)."""
    if t is None:
        return 0
    _need(t, name, dt)
    if t.numel() % row:
        raise ValueError("%s is not a whole number of token rows" % name)
    return t.numel() // row


def _workspace(nbytes, ws, like):
    if ws is None:
        return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=like.device)
    _need(ws, "workspace", torch.uint8, nbytes)
    return ws


# ----------------------------------------------------------------------------
# entry points

def wa_append_workspace_bytes(L: Layout) -> int:
    return int(load_library().wa_append_workspace_bytes(ctypes.byref(L)))


def wa_append_page(L: Layout, k_src, v_src, k_pool, v_pool, slot: int, page_means,
                   workspace=None, stream=None):
    """Copy a page into pool slot `slot` and write page_means[slot] (fp64)."""
    lib = load_library()
    page = L.page_tokens * L.row_elems
    dt = L.torch_dtype
    _need(k_src, "k_src", dt, page)
    _need(k_pool, "k_pool", dt, L.max_pages * page)
    if v_src is not None:
        _need(v_src, "v_src", dt, page)
        _need(v_pool, "v_pool", dt, L.max_pages * page)
    _need(page_means, "page_means", torch.float64, L.max_pages * L.row_elems)
    nbytes = wa_append_workspace_bytes(L)
    ws = _workspace(nbytes, workspace, k_pool)
    st = lib.wa_append_page(ctypes.byref(L), _ptr(k_src), _ptr(v_src), _ptr(k_pool),
                            _ptr(v_pool), int(slot), _ptr(page_means), _ptr(ws), ws.numel(),
                            _stream(stream))
    _check(st, "wa_append_page")


def _prompt_struct(prompt):
    if prompt is None:
        return None
    cp = _need(prompt["chunk_prompts"], "chunk_prompts", torch.float32)
    cur = _need(prompt["cur_prompt"], "cur_prompt", torch.float32)
    pages = _need(prompt["chunk_pages"], "chunk_pages", torch.int32)
    n_chunks, emb = cp.shape
    ppc = pages.shape[1]
    if cur.numel() < emb or pages.shape[0] != n_chunks:
        raise ValueError("prompt stage shapes disagree")
    n_keep = int(prompt["n_keep"])
    oc = prompt.get("out_chunks")
    ocand = prompt.get("out_cand")
    if oc is not None:
        _need(oc, "out_chunks", torch.int32, n_keep)
    if ocand is not None:
        _need(ocand, "out_cand", torch.int32, n_keep * ppc)
    return PromptStage(cp.data_ptr(), cur.data_ptr(), pages.data_ptr(), n_chunks, emb, ppc,
                       n_keep, oc.data_ptr() if oc is not None else None,
                       ocand.data_ptr() if ocand is not None else None)


def wa_select_workspace_bytes(L: Layout, n_q: int, n_cand: int, prompt=None) -> int:
    ps = _prompt_struct(prompt)
    return int(load_library().wa_select_workspace_bytes(
        ctypes.byref(L), int(n_q), int(n_cand), ctypes.byref(ps) if ps is not None else None))


def _select(L, q, page_means, k_p, cand, n_cand, prompt, recent, out_idx, out_scores, workspace,
            stream, where):
    lib = load_library()
    _need(q, "q", L.torch_dtype)
    n_q = q.numel() // L.row_elems
    if q.numel() != n_q * L.row_elems:
        raise ValueError("q is not a whole number of token rows")
    _need(page_means, "page_means", torch.float64, L.max_pages * L.row_elems)
    ps = _prompt_struct(prompt)
    if ps is not None:
        n_cand = ps.n_keep * ps.pages_per_chunk
    elif cand is not None:
        _need(cand, "cand", torch.int32)
        n_cand = cand.numel() if n_cand is None else n_cand
        _need(cand, "cand", torch.int32, n_cand)
    elif n_cand is None:
        n_cand = L.max_pages
    n_recent = 0
    if recent is not None:
        _need(recent, "recent", torch.int32)
        n_recent = recent.numel()
    n_out = n_recent + int(k_p)
    if out_idx is None:
        out_idx = torch.empty(max(n_out, 1), dtype=torch.int32, device=q.device)
    _need(out_idx, "out_idx", torch.int32, n_out)
    if out_scores is not None:
        _need(out_scores, "out_scores", torch.float64, n_cand)
    pst = ctypes.byref(ps) if ps is not None else None
    if where == "wa_select_pages_noalloc":
        # the library's own fixed workspace: nothing allocated here or there
        st = lib.wa_select_pages_noalloc(ctypes.byref(L), _ptr(q), int(n_q), _ptr(page_means),
                                         _ptr(cand), int(n_cand), pst, int(k_p), _ptr(out_idx),
                                         _ptr(out_scores), _stream(stream))
        _check(st, where)
        return out_idx
    nbytes = lib.wa_select_workspace_bytes(ctypes.byref(L), int(n_q), int(n_cand),
                                           ctypes.byref(ps) if ps is not None else None)
    if workspace is None:
        # zero-filled before its first use; every call leaves it so again
        workspace = torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=q.device)
    ws = _workspace(nbytes, workspace, q)
    if where == "wa_select_pages":
        st = lib.wa_select_pages(ctypes.byref(L), _ptr(q), int(n_q), _ptr(page_means), _ptr(cand),
                                 int(n_cand), pst, int(k_p), _ptr(out_idx), _ptr(out_scores),
                                 _ptr(ws), ws.numel(), _stream(stream))
    else:
        st = lib.wa_select_window(ctypes.byref(L), _ptr(q), int(n_q), _ptr(page_means),
                                  _ptr(cand), int(n_cand), pst, _ptr(recent), int(n_recent),
                                  int(k_p), _ptr(out_idx), _ptr(out_scores), _ptr(ws),
                                  ws.numel(), _stream(stream))
    _check(st, where)
    return out_idx


def wa_select_pages(L: Layout, q, page_means, k_p: int, cand=None, n_cand=None, prompt=None,
                    out_idx=None, out_scores=None, workspace=None, stream=None):
    """Top-K_p page ids (device int32 [k_p]) for the chunk's queries q [n_q, H, d]."""
    return _select(L, q, page_means, k_p, cand, n_cand, prompt, None, out_idx, out_scores,
                   workspace, stream, "wa_select_pages")


def wa_select_pages_noalloc(L: Layout, q, page_means, k_p: int, cand=None, n_cand=None,
                            prompt=None, out_idx=None, out_scores=None, stream=None):
    """wa_select_pages with the library's fixed per-device workspace (no
    allocation when out_idx is given)."""
    return _select(L, q, page_means, k_p, cand, n_cand, prompt, None, out_idx, out_scores,
                   None, stream, "wa_select_pages_noalloc")


def wa_select_window(L: Layout, q, page_means, recent, k_p: int, cand=None, n_cand=None,
                     prompt=None, out_idx=None, out_scores=None, workspace=None, stream=None):
    """The pages of `recent` (device int32, the sliding window) followed by the
    top-K_p of the other candidates: device int32 [len(recent) + k_p]."""
    return _select(L, q, page_means, k_p, cand, n_cand, prompt, recent, out_idx, out_scores,
                   workspace, stream, "wa_select_window")


def wa_gather(L: Layout, k_pool, v_pool, idx, k_p: int, k_ctx=None, v_ctx=None, stream=None):
    """Contiguous [k_p * page_tokens, H, d] copies of the pages idx[0..k_p)."""
    lib = load_library()
    page = L.page_tokens * L.row_elems
    dt = L.torch_dtype
    _need(k_pool, "k_pool", dt, L.max_pages * page)
    _need(idx, "idx", torch.int32, k_p)
    shape = (k_p * L.page_tokens, L.n_heads, L.head_dim)
    if k_ctx is None:
        k_ctx = torch.empty(shape, dtype=dt, device=k_pool.device)
    _need(k_ctx, "k_ctx", dt, k_p * page)
    if v_pool is not None:
        _need(v_pool, "v_pool", dt, L.max_pages * page)
        if v_ctx is None:
            v_ctx = torch.empty(shape, dtype=dt, device=v_pool.device)
        _need(v_ctx, "v_ctx", dt, k_p * page)
    st = lib.wa_gather(ctypes.byref(L), _ptr(k_pool), _ptr(v_pool), _ptr(idx), int(k_p),
                       _ptr(k_ctx), _ptr(v_ctx) if v_pool is not None else None, _stream(stream))
    _check(st, "wa_gather")
    return k_ctx, v_ctx


def wa_attention_workspace_bytes(L: Layout, n_q: int, n_ctx: int, n_own: int) -> int:
    return int(load_library().wa_attention_workspace_bytes(ctypes.byref(L), int(n_q), int(n_ctx),
                                                           int(n_own)))


def wa_block_attention(L: Layout, q, k_ctx, v_ctx, k_own, v_own, softmax_scale=None,
                       out_dtype=None, out=None, lse=None, workspace=None, stream=None):
    """Unmasked attention of q over [k_ctx ++ k_own]; returns out [n_q, H, d]."""
    lib = load_library()
    dt = L.torch_dtype
    row = L.row_elems
    _need(q, "q", dt)
    n_q = q.numel() // row

    def rows(t, name):
        if t is None:
            return 0
        _need(t, name, dt)
        if t.numel() % row:
            raise ValueError("%s is not a whole number of token rows" % name)
        return t.numel() // row

    n_ctx, n_ctx_v = rows(k_ctx, "k_ctx"), rows(v_ctx, "v_ctx")
    n_own, n_own_v = rows(k_own, "k_own"), rows(v_own, "v_own")
    if n_ctx != n_ctx_v or n_own != n_own_v:
        raise ValueError("K and V segments differ in length")
    if softmax_scale is None:
        softmax_scale = 1.0 / (L.head_dim ** 0.5)
    if out_dtype is None:
        out_dtype = L.dtype
    odt = _TORCH_DTYPE[out_dtype]
    if out is None:
        out = torch.empty((n_q, L.n_heads, L.head_dim), dtype=odt, device=q.device)
    _need(out, "out", odt, n_q * row)
    if lse is not None:
        _need(lse, "lse", torch.float32, n_q * L.n_heads)
    nbytes = lib.wa_attention_workspace_bytes(ctypes.byref(L), int(n_q), int(n_ctx), int(n_own))
    ws = _workspace(nbytes, workspace, q)
    st = lib.wa_block_attention(ctypes.byref(L), _ptr(q), int(n_q), _ptr(k_ctx), _ptr(v_ctx),
                                int(n_ctx), _ptr(k_own), _ptr(v_own), int(n_own),
                                float(softmax_scale), int(out_dtype), _ptr(out), _ptr(lse),
                                _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "wa_block_attention")
    return out


def wa_paged_attention(L: Layout, q, k_pool, v_pool, idx, k_p, k_own, v_own, softmax_scale=None,
                       out_dtype=None, out=None, lse=None, workspace=None, stream=None):
    """Attention of q over [pages idx[0..k_p) of the pools ++ k_own], read in
    place; the same result as wa_gather followed by wa_block_attention."""
    lib = load_library()
    dt = L.torch_dtype
    row = L.row_elems
    _need(q, "q", dt)
    n_q = q.numel() // row
    pool_elems = L.max_pages * L.page_tokens * row
    _need(k_pool, "k_pool", dt, pool_elems)
    _need(v_pool, "v_pool", dt, pool_elems)
    _need(idx, "idx", torch.int32, int(k_p))
    n_own = 0
    if k_own is not None or v_own is not None:
        _need(k_own, "k_own", dt)
        _need(v_own, "v_own", dt)
        n_own = k_own.numel() // row
        if k_own.numel() % row or v_own.numel() != k_own.numel():
            raise ValueError("k_own / v_own are not matching whole token rows")
    if softmax_scale is None:
        softmax_scale = 1.0 / (L.head_dim ** 0.5)
    if out_dtype is None:
        out_dtype = L.dtype
    odt = _TORCH_DTYPE[out_dtype]
    if out is None:
        out = torch.empty((n_q, L.n_heads, L.head_dim), dtype=odt, device=q.device)
    _need(out, "out", odt, n_q * row)
    if lse is not None:
        _need(lse, "lse", torch.float32, n_q * L.n_heads)
    n_ctx = int(k_p) * L.page_tokens
    nbytes = lib.wa_attention_workspace_bytes(ctypes.byref(L), int(n_q), int(n_ctx), int(n_own))
    ws = _workspace(nbytes, workspace, q)
    st = lib.wa_paged_attention(ctypes.byref(L), _ptr(q), int(n_q), _ptr(k_pool), _ptr(v_pool),
                                _ptr(idx), int(k_p), _ptr(k_own), _ptr(v_own), int(n_own),
                                float(softmax_scale), int(out_dtype), _ptr(out), _ptr(lse),
                                _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "wa_paged_attention")
    return out


# ----------------------------------------------------------------------------
# sparse branch

HSA_CTX_BLOCK, HSA_OWN_BLOCK, HSA_Q_BLOCK = 128, 64, 256


def hsa_shape(L: Layout, n_q: int, n_ctx: int, n_own: int):
    """(q_blocks, items, n_tiles) of a sparse-branch call: the selection
    writes sel_tiles [items][n_tiles] and sel_count [items], item =
    head * q_blocks + query block."""
    q_blocks = -(-int(n_q) // HSA_Q_BLOCK)
    return q_blocks, q_blocks * L.n_heads, -(-(int(n_ctx) + int(n_own)) // 64)


def wa_hsa_workspace_bytes(L: Layout, n_q: int, n_ctx: int, n_own: int) -> int:
    return int(load_library().wa_hsa_workspace_bytes(ctypes.byref(L), int(n_q), int(n_ctx),
                                                      int(n_own)))


def wa_hsa_select(L: Layout, q, k_ctx, k_own, tau, scale=None, sel_tiles=None, sel_count=None,
                  gini=None, want_gini=True, workspace=None, ctx_sums_ready=False, stream=None):
    """Block selection of the sparse branch; returns (sel_tiles [items,
    n_tiles] int32, sel_count [items] int32, gini [items] float64 or None).
    tau: device float64 [H].  ctx_sums_ready: reuse the context block sums an
    earlier call left in `workspace` (same layout, n_ctx and k_ctx contents);
    it needs that workspace passed in."""
    if ctx_sums_ready and workspace is None:
        raise ValueError("wa_hsa_select: ctx_sums_ready needs the workspace of the earlier call")
    lib = load_library()
    dt, row = L.torch_dtype, L.row_elems
    _need(q, "q", dt)
    n_q = q.numel() // row
    n_ctx, n_own = _rows(k_ctx, "k_ctx", dt, row), _rows(k_own, "k_own", dt, row)
    _need(tau, "tau", torch.float64, L.n_heads)
    if scale is None:
        scale = 1.0 / (L.head_dim ** 0.5)
    _, items, n_tiles = hsa_shape(L, n_q, n_ctx, n_own)
    if sel_tiles is None:
        sel_tiles = torch.empty((items, n_tiles), dtype=torch.int32, device=q.device)
    if sel_count is None:
        sel_count = torch.empty(items, dtype=torch.int32, device=q.device)
    if gini is None and want_gini:
        gini = torch.empty(items, dtype=torch.float64, device=q.device)
    _need(sel_tiles, "sel_tiles", torch.int32, items * n_tiles)
    _need(sel_count, "sel_count", torch.int32, items)
    if gini is not None:
        _need(gini, "gini", torch.float64, items)
    nbytes = lib.wa_hsa_workspace_bytes(ctypes.byref(L), int(n_q), int(n_ctx), int(n_own))
    ws = _workspace(nbytes, workspace, q)
    st = lib.wa_hsa_select(ctypes.byref(L), _ptr(q), int(n_q), _ptr(k_ctx), int(n_ctx),
                           _ptr(k_own), int(n_own), float(scale), _ptr(tau), _ptr(sel_tiles),
                           _ptr(sel_count), _ptr(gini), 1 if ctx_sums_ready else 0, _ptr(ws),
                           ws.numel(), _stream(stream))
    _check(st, "wa_hsa_select")
    return sel_tiles, sel_count, gini


def wa_sparse_workspace_bytes(L: Layout, n_q: int, n_ctx: int, n_own: int) -> int:
    return int(load_library().wa_sparse_workspace_bytes(ctypes.byref(L), int(n_q), int(n_ctx),
                                                         int(n_own)))


def wa_sparse_attention(L: Layout, q, k_ctx, v_ctx, k_own, v_own, sel_tiles, sel_count,
                        softmax_scale=None, out_dtype=None, out=None, lse=None, workspace=None,
                        stream=None):
    """Attention of each (query block, head) over its listed 64-key tiles of
    [k_ctx ++ k_own]; returns out [n_q, H, d]."""
    lib = load_library()
    dt, row = L.torch_dtype, L.row_elems
    _need(q, "q", dt)
    n_q = q.numel() // row
    n_ctx, n_ctx_v = _rows(k_ctx, "k_ctx", dt, row), _rows(v_ctx, "v_ctx", dt, row)
    n_own, n_own_v = _rows(k_own, "k_own", dt, row), _rows(v_own, "v_own", dt, row)
    if n_ctx != n_ctx_v or n_own != n_own_v:
        raise ValueError("K and V segments differ in length")
    _, items, n_tiles = hsa_shape(L, n_q, n_ctx, n_own)
    _need(sel_tiles, "sel_tiles", torch.int32, items * n_tiles)
    _need(sel_count, "sel_count", torch.int32, items)
    if softmax_scale is None:
        softmax_scale = 1.0 / (L.head_dim ** 0.5)
    if out_dtype is None:
        out_dtype = L.dtype
    odt = _TORCH_DTYPE[out_dtype]
    if out is None:
        out = torch.empty((n_q, L.n_heads, L.head_dim), dtype=odt, device=q.device)
    _need(out, "out", odt, n_q * row)
    if lse is not None:
        _need(lse, "lse", torch.float32, n_q * L.n_heads)
    nbytes = lib.wa_sparse_workspace_bytes(ctypes.byref(L), int(n_q), int(n_ctx), int(n_own))
    ws = _workspace(nbytes, workspace, q)
    st = lib.wa_sparse_attention(ctypes.byref(L), _ptr(q), int(n_q), _ptr(k_ctx), _ptr(v_ctx),
                                 int(n_ctx), _ptr(k_own), _ptr(v_own), int(n_own),
                                 float(softmax_scale), _ptr(sel_tiles), _ptr(sel_count),
                                 int(out_dtype), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                 _stream(stream))
    _check(st, "wa_sparse_attention")
    return out


# ----------------------------------------------------------------------------
# host-memory page tier

def _host_pool(t, name, L):
    if t is None:
        return 0
    _need(t, name, L.torch_dtype, device=False)
    if not t.is_pinned():
        raise ValueError("%s must be pinned host memory (pin_memory=True)" % name)
    page = L.page_tokens * L.row_elems
    if t.numel() % page:
        raise ValueError("%s is not a whole number of pages" % name)
    return t.numel() // page


def _dev_pool(k_pool, v_pool, L, slot):
    """The HBM pools hold slot `slot` (the library checks slot < max_pages)."""
    need = (int(slot) + 1) * L.page_tokens * L.row_elems if slot >= 0 else None
    _need(k_pool, "k_pool", L.torch_dtype, need)
    if v_pool is not None:
        _need(v_pool, "v_pool", L.torch_dtype, need)


def wa_page_in(L: Layout, host_k, host_v, host_slot: int, k_pool, v_pool, slot: int,
               stream=None):
    """k_pool[slot] = host_k[host_slot] (and V), queued on the copy engines."""
    lib = load_library()
    _dev_pool(k_pool, v_pool, L, slot)
    n = _host_pool(host_k, "host_k", L)
    if host_v is not None and _host_pool(host_v, "host_v", L) != n:
        raise ValueError("host_k and host_v hold different page counts")
    st = lib.wa_page_in(ctypes.byref(L), _ptr(host_k), _ptr(host_v), int(n), int(host_slot),
                        _ptr(k_pool), _ptr(v_pool), int(slot), _stream(stream))
    _check(st, "wa_page_in")


def wa_page_in_rows(L: Layout, host_k, host_v, host_slot: int, k_pool, v_pool, slot: int,
                    row0: int, n_rows: int, stream=None):
    """Token rows [row0, row0 + n_rows) of k_pool[slot] = the same rows of
    host_k[host_slot] (and V), queued on the copy engines."""
    lib = load_library()
    _dev_pool(k_pool, v_pool, L, slot)
    n = _host_pool(host_k, "host_k", L)
    if host_v is not None and _host_pool(host_v, "host_v", L) != n:
        raise ValueError("host_k and host_v hold different page counts")
    st = lib.wa_page_in_rows(ctypes.byref(L), _ptr(host_k), _ptr(host_v), int(n), int(host_slot),
                             _ptr(k_pool), _ptr(v_pool), int(slot), int(row0), int(n_rows),
                             _stream(stream))
    _check(st, "wa_page_in_rows")


def wa_page_out(L: Layout, k_pool, v_pool, slot: int, host_k, host_v, host_slot: int,
                stream=None):
    """host_k[host_slot] = k_pool[slot] (and V), queued on the copy engines."""
    lib = load_library()
    _dev_pool(k_pool, v_pool, L, slot)
    n = _host_pool(host_k, "host_k", L)
    if host_v is not None and _host_pool(host_v, "host_v", L) != n:
        raise ValueError("host_k and host_v hold different page counts")
    st = lib.wa_page_out(ctypes.byref(L), _ptr(k_pool), _ptr(v_pool), int(slot), _ptr(host_k),
                         _ptr(host_v), int(n), int(host_slot), _stream(stream))
    _check(st, "wa_page_out")


def wa_merge_attention(L: Layout, out_a, lse_a, out_b, lse_b, out_dtype=WA_F32, out=None,
                       lse=None, stream=None):
    """Attention over A u B from the attentions over A and over B (fp32
    outputs with their lse); returns out [n_q, H, d]."""
    lib = load_library()
    row = L.row_elems
    _need(out_a, "out_a", torch.float32)
    n_q = out_a.numel() // row
    _need(out_b, "out_b", torch.float32, n_q * row)
    _need(lse_a, "lse_a", torch.float32, n_q * L.n_heads)
    _need(lse_b, "lse_b", torch.float32, n_q * L.n_heads)
    odt = _TORCH_DTYPE[out_dtype]
    if out is None:
        out = torch.empty((n_q, L.n_heads, L.head_dim), dtype=odt, device=out_a.device)
    _need(out, "out", odt, n_q * row)
    if lse is not None:
        _need(lse, "lse", torch.float32, n_q * L.n_heads)
    st = lib.wa_merge_attention(ctypes.byref(L), int(n_q), _ptr(out_a), _ptr(lse_a), _ptr(out_b),
                                _ptr(lse_b), int(out_dtype), _ptr(out), _ptr(lse),
                                _stream(stream))
    _check(st, "wa_merge_attention")
    return out
