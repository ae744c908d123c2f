"""fp64 CPU oracle of the paged-KV block-attention path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never do; the two implementations share no code.  Inputs come from
``wa_workloads`` (element arrays: float32, or bf16 bit patterns as uint16).

The arithmetic lives in ``wa_oracle.c`` (plain loops in double precision);
this module marshals numpy arrays into it and strings its steps together in
the order the pages give them:

* page mean key and chunk mean query, page-stage score, top-K_p, and the
  prompt stage -- WorldAttention review (jaehun.me), "HKV: Page-Level
  Multi-Tier Memory";
* gather into one contiguous buffer -- same page, "Core Idea", item 3;
* attention over [cached ++ own] K/V with one softmax and no mask -- Inferix
  summary, section 3.4, "The Block-Diffusion Generation Pipeline", Step 3;
  softmax and value weighting after the score contraction -- the einsum post,
  "Where the mental model stops";
* the merge of two attentions over disjoint key sets -- Inferix summary,
  "Ring Attention" (partial attention over one chunk of keys at a time,
  accumulated), used for the host-memory page tier;
* the sparse branch (key blocks, pooled attention map, Gini coefficient,
  cumulative-mass block selection, attention over the selected blocks) --
  WorldAttention review, "HSA: Dual Branches of Linear + Sparse"; these
  compose the C attention with numpy, and their pins are planted with
  mistakes in ``tests/test_oracle_mutations_py.py``.

Parity status of each function: pinned by ``tests/test_oracle_pins.py``
(closed forms, invariants, brute force, and a textbook library routine).
The page-stage and prompt-stage readings are listed in ``wa_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wa_oracle.c")
_LIB = os.path.join(_HERE, "libwa_oracle.so")
_LIB_NATIVE = os.path.join(_HERE, "libwa_oracle_native.so")

F32, BF16 = 0, 1

_lib = None


def build(force: bool = True, native: bool = False) -> str:
    """Compile the oracle with gcc -O3 (fp64, OpenMP over rows and heads).

    native=True builds a copy tuned for the host it runs on (-march=native,
    for the CPU-baseline timing; built where it runs, never shipped between
    machines); the tests use the portable build."""
    lib = _LIB_NATIVE if native else _LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + ".tmp%d" % os.getpid()
        arch = ["-march=native"] if native else []
        subprocess.check_call(["gcc", "-O3"] + arch + ["-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, lib)
    return lib


def use_native() -> None:
    """Build the host-tuned copy here and make every later call use it."""
    global _lib
    _lib = configure(ctypes.CDLL(build(force=True, native=True)))


def configure(lib):
    """Declare the C signatures on a loaded oracle library and return it."""
    p, i64, i32, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.wao_column_mean.argtypes = [p, i32, i64, i64, p]
    lib.wao_page_scores.argtypes = [p, p, i64, i32, p, i32, p]
    lib.wao_top_k.argtypes = [p, p, i32, i32, p]
    lib.wao_prompt_cosine.argtypes = [p, p, i32, i32, p]
    lib.wao_prompt_candidates.argtypes = [p, i32, p, i32, i32, p, p]
    lib.wao_gather.argtypes = [p, i64, p, i32, p]
    lib.wao_attention.argtypes = [p, p, p, i64, p, p, i64, i32, i32, i32, d, p, i64,
                                  p, p, i32]
    for f in (lib.wao_column_mean, lib.wao_page_scores, lib.wao_top_k,
              lib.wao_prompt_cosine, lib.wao_prompt_candidates, lib.wao_gather,
              lib.wao_attention):
        f.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or bf16 bit patterns (uint16), got %s" % x.dtype)


def n_threads() -> int:
    """Threads for the attention loop: every core this process may run on,
    at most 16 (the CPU share of one GPU on the measurement boxes)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------
# steps

def column_mean(x: np.ndarray) -> np.ndarray:
    """[rows, H, d] -> [H, d] fp64 mean over rows (page mean key, chunk mean query)."""
    x = np.ascontiguousarray(x)
    rows = x.shape[0]
    hd = int(np.prod(x.shape[1:]))
    out = np.empty(x.shape[1:], dtype=np.float64)
    _load().wao_column_mean(_ptr(x), _dtype_code(x), rows, hd, _ptr(out))
    return out


page_mean = column_mean
mean_query = column_mean


def page_scores(qbar: np.ndarray, page_means: np.ndarray, cand: np.ndarray) -> np.ndarray:
    """alpha_j = sum_h qbar[h] . kbar_{cand[j]}[h] / sqrt(d), fp64."""
    qbar = np.ascontiguousarray(qbar, dtype=np.float64)
    page_means = np.ascontiguousarray(page_means, dtype=np.float64)
    cand = np.ascontiguousarray(cand, dtype=np.int32)
    head_dim = qbar.shape[-1]
    hd = qbar.size
    assert page_means.shape[1:] == qbar.shape
    assert cand.size == 0 or (cand.min() >= 0 and cand.max() < page_means.shape[0])
    alpha = np.empty(cand.size, dtype=np.float64)
    _load().wao_page_scores(_ptr(qbar), _ptr(page_means), hd, head_dim, _ptr(cand),
                            cand.size, _ptr(alpha))
    return alpha


def top_k(score: np.ndarray, ids: np.ndarray, k: int) -> np.ndarray:
    """The k ids ranked first by (score desc, id asc), in rank order."""
    score = np.ascontiguousarray(score, dtype=np.float64)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    assert 0 <= k <= ids.size == score.size
    out = np.empty(k, dtype=np.int32)
    _load().wao_top_k(_ptr(score), _ptr(ids), ids.size, k, _ptr(out))
    return out


def prompt_cosine(chunk_prompts: np.ndarray, cur: np.ndarray) -> np.ndarray:
    cp = np.ascontiguousarray(chunk_prompts, dtype=np.float32)
    cur = np.ascontiguousarray(cur, dtype=np.float32)
    out = np.empty(cp.shape[0], dtype=np.float64)
    _load().wao_prompt_cosine(_ptr(cp), _ptr(cur), cp.shape[0], cp.shape[1], _ptr(out))
    return out


def prompt_candidates(cos_m: np.ndarray, chunk_pages: np.ndarray, n_keep: int):
    """(kept chunk ids in rank order, their pages laid end to end)."""
    cos_m = np.ascontiguousarray(cos_m, dtype=np.float64)
    chunk_pages = np.ascontiguousarray(chunk_pages, dtype=np.int32)
    n_chunks, ppc = chunk_pages.shape
    assert cos_m.size == n_chunks and 0 < n_keep <= n_chunks
    chunks = np.empty(n_keep, dtype=np.int32)
    cand = np.empty(n_keep * ppc, dtype=np.int32)
    _load().wao_prompt_candidates(_ptr(cos_m), n_chunks, _ptr(chunk_pages), ppc, n_keep,
                                  _ptr(chunks), _ptr(cand))
    return chunks, cand


def gather(pool: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """pool [pages, P_t, H, d] -> [k_p * P_t, H, d], page idx[r] at rank r."""
    pool = np.ascontiguousarray(pool)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    assert idx.size == 0 or (idx.min() >= 0 and idx.max() < pool.shape[0])
    page_bytes = pool[0].nbytes
    out = np.empty((idx.size * pool.shape[1],) + pool.shape[2:], dtype=pool.dtype)
    _load().wao_gather(_ptr(pool), page_bytes, _ptr(idx), idx.size, _ptr(out))
    return out


def attention(q, k_ctx, v_ctx, k_own, v_own, scale: float, rows=None, threads=None):
    """Block attention over [ctx ++ own] for the given query rows.

    Returns (out [n_rows, H, d] fp64, lse [H, n_rows] fp64).
    """
    q = np.ascontiguousarray(q)
    dt = _dtype_code(q)
    n_heads, head_dim = q.shape[1], q.shape[2]

    def prep(x):
        if x is None:
            return np.zeros((0, n_heads, head_dim), dtype=q.dtype)
        x = np.ascontiguousarray(x)
        assert x.dtype == q.dtype and x.shape[1:] == q.shape[1:]
        return x

    k_ctx, v_ctx, k_own, v_own = (prep(x) for x in (k_ctx, v_ctx, k_own, v_own))
    assert k_ctx.shape == v_ctx.shape and k_own.shape == v_own.shape
    if rows is None:
        rows = np.arange(q.shape[0], dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < q.shape[0])
    out = np.empty((rows.size, n_heads, head_dim), dtype=np.float64)
    lse = np.empty((n_heads, rows.size), dtype=np.float64)
    _load().wao_attention(_ptr(q), _ptr(k_ctx), _ptr(v_ctx), k_ctx.shape[0], _ptr(k_own),
                          _ptr(v_own), k_own.shape[0], n_heads, head_dim, dt, float(scale),
                          _ptr(rows), rows.size, _ptr(out), _ptr(lse),
                          threads or n_threads())
    return out, lse


# ----------------------------------------------------------------------------
# the steps strung together (one chunk)

def select_pages(q, page_means, k_p, cand=None, prompt=None):
    """Page stage (and optional prompt stage) for one chunk.

    prompt: None or dict(chunk_prompts, cur_prompt, chunk_pages, n_keep).
    Returns dict(idx, alpha, cand, qbar, chunks, cos).
    """
    res = {}
    if prompt is not None:
        cos_m = prompt_cosine(prompt["chunk_prompts"], prompt["cur_prompt"])
        chunks, cand = prompt_candidates(cos_m, prompt["chunk_pages"], prompt["n_keep"])
        res["cos"], res["chunks"] = cos_m, chunks
    elif cand is None:
        cand = np.arange(page_means.shape[0], dtype=np.int32)
    cand = np.ascontiguousarray(cand, dtype=np.int32)
    qbar = mean_query(q)
    alpha = page_scores(qbar, page_means, cand)
    res.update(idx=top_k(alpha, cand, k_p), alpha=alpha, cand=cand, qbar=qbar)
    return res


def select_window(q, page_means, k_p, recent, cand=None, prompt=None):
    """Sliding window plus selective fetch -- Inferix summary, "Dual access
    patterns" (range access to the most recent blocks, index-based fetch of
    distant ones).  The page stage of ``select_pages`` run over the candidates
    whose id is not in the window; the window's ids come first, in the given
    order, then the top k_p of the rest; ranks with no candidate left are -1.
    Returns dict(idx, alpha, cand) with alpha for every candidate."""
    recent = np.ascontiguousarray(recent, dtype=np.int32)
    res = select_pages(q, page_means, 0, cand=cand, prompt=prompt)
    keep = ~np.isin(res["cand"], recent)
    rest_alpha, rest_ids = res["alpha"][keep], res["cand"][keep]
    kk = min(int(k_p), rest_ids.size)
    sel = top_k(rest_alpha, rest_ids, kk)
    idx = np.concatenate([recent, sel, np.full(int(k_p) - kk, -1, np.int32)]).astype(np.int32)
    return dict(idx=idx, alpha=res["alpha"], cand=res["cand"])


# ----------------------------------------------------------------------------
# HSA sparse branch (WorldAttention review, "HSA: Dual Branches of Linear +
# Sparse"): block-level selection with a pooled attention map, a per-head
# cumulative-mass threshold, attention over the selected blocks only.  The
# readings taken where the page is silent (query pooling per 256-query block,
# an unweighted softmax over block means, tau_h given per head because the
# Gini-to-threshold formula did not survive extraction) are listed with the
# build's design notes.

def _widen(x) -> np.ndarray:
    """Input encoding (float32, or bf16 patterns as uint16) -> float64, exactly."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def hsa_key_blocks(n_ctx: int, n_own: int, b_inter: int = 128, b_intra: int = 64):
    """[start, end) of every key block in [ctx ++ own] key order: the context
    (past pages) in blocks of b_inter keys, the chunk's own keys in blocks of
    b_intra; a last block may be shorter."""
    blocks = [(s, min(s + b_inter, n_ctx)) for s in range(0, n_ctx, b_inter)]
    blocks += [(n_ctx + s, n_ctx + min(s + b_intra, n_own)) for s in range(0, n_own, b_intra)]
    return blocks


def gini(p) -> float:
    """Gini coefficient sum_i sum_j |p_i - p_j| / (2 n sum_i p_i) of a
    non-negative distribution."""
    p = np.asarray(p, dtype=np.float64)
    return float(np.abs(p[:, None] - p[None, :]).sum() / (2.0 * p.size * p.sum()))


def select_blocks(mass, tau: float):
    """The fewest blocks whose mass reaches tau: blocks taken in decreasing mass
    (ties to the lower index) until the running sum is >= tau, at least one;
    returned in ascending (key) order."""
    order = sorted(range(len(mass)), key=lambda j: (-float(mass[j]), j))
    total, chosen = 0.0, []
    for j in order:
        chosen.append(j)
        total += float(mass[j])
        if total >= tau:
            break
    return sorted(chosen)


def hsa_pooled_map(q_rows, k_all, blocks, scale: float) -> np.ndarray:
    """Pooled attention map of one query block for every head: softmax over key
    blocks of (mean query . mean key of the block) * scale.  q_rows
    [n, H, d], k_all [n_keys, H, d] (input encoding); returns [H, n_blocks]."""
    qbar = _widen(q_rows).mean(axis=0)                          # [H, d]
    k = _widen(k_all)
    kbar = np.stack([k[a:b].mean(axis=0) for a, b in blocks])  # [nb, H, d]
    s = np.einsum("hd,jhd->hj", qbar, kbar) * scale
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def hsa_sparse(q, k_ctx, v_ctx, k_own, v_own, scale: float, tau, q_block: int = 256,
               b_inter: int = 128, b_intra: int = 64, rows=None):
    """Sparse branch: for each head h and query block b (q_block queries), the
    key blocks chosen by select_blocks(pooled map row, tau[h]); each query of
    the block attends (one softmax, no mask) over the keys of those blocks in
    key order.  Returns dict(out [n_rows, H, d], lse [H, n_rows], sel
    {(h, b): block list}, gini {(h, b): G}, maps {b: pooled map [H, nb]},
    blocks)."""
    q = np.ascontiguousarray(q)
    n_heads = q.shape[1]
    n_ctx = 0 if k_ctx is None else k_ctx.shape[0]
    n_own = 0 if k_own is None else k_own.shape[0]
    parts_k = [x for x in (k_ctx, k_own) if x is not None and x.shape[0]]
    parts_v = [x for x in (v_ctx, v_own) if x is not None and x.shape[0]]
    k_all, v_all = np.concatenate(parts_k), np.concatenate(parts_v)
    blocks = hsa_key_blocks(n_ctx, n_own, b_inter, b_intra)
    if rows is None:
        rows = np.arange(q.shape[0], dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, n_heads, q.shape[2]), dtype=np.float64)
    lse = np.empty((n_heads, rows.size), dtype=np.float64)
    sel, gin, maps = {}, {}, {}
    for b in sorted(set((rows // q_block).tolist())):
        lo, hi = b * q_block, min((b + 1) * q_block, q.shape[0])
        pmap = hsa_pooled_map(q[lo:hi], k_all, blocks, scale)
        maps[b] = pmap
        mine = np.nonzero(rows // q_block == b)[0]
        for h in range(n_heads):
            chosen = select_blocks(pmap[h], float(tau[h]))
            sel[(h, b)], gin[(h, b)] = chosen, gini(pmap[h])
            keys = np.concatenate([np.arange(blocks[j][0], blocks[j][1]) for j in chosen])
            kh = np.ascontiguousarray(k_all[keys][:, h:h + 1])
            vh = np.ascontiguousarray(v_all[keys][:, h:h + 1])
            o, l = attention(np.ascontiguousarray(q[:, h:h + 1]), kh, vh, None, None, scale,
                             rows=rows[mine])
            out[mine, h] = o[:, 0]
            lse[h, mine] = l[0]
    return dict(out=out, lse=lse, sel=sel, gini=gin, maps=maps, blocks=blocks)


def merge_attention(out_a, lse_a, out_b, lse_b):
    """Attention over A u B from attentions over disjoint key sets A and B
    (outputs [n, H, d], lse [H, n], natural log): the softmax over the union
    weights each part by its share of the total, exp(lse_X - lse), with
    lse = log(exp(lse_A) + exp(lse_B)); taken against the larger lse."""
    oa, ob = np.asarray(out_a, np.float64), np.asarray(out_b, np.float64)
    la, lb = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    m = np.maximum(la, lb)
    wa, wb = np.exp(la - m), np.exp(lb - m)
    tot = wa + wb
    out = (wa / tot).T[:, :, None] * oa + (wb / tot).T[:, :, None] * ob
    return out, m + np.log(tot)


def boundary_margin(alpha: np.ndarray, k_p: int) -> float:
    """Gap between the k_p-th and (k_p+1)-th best score (inf if none)."""
    s = np.sort(np.asarray(alpha, dtype=np.float64))[::-1]
    if k_p >= s.size:
        return float("inf")
    return float(s[k_p - 1] - s[k_p])
