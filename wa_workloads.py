"""Seeded synthetic inputs for the paged-KV block-attention path.

This module only *draws* inputs: it holds none of the method's arithmetic
(no means, scores, selection, gathering or attention).  Both the CPU oracle
(``oracle/``) and the HIP path (``paged_kv_attention_page_amd``) take their
inputs from here, and from nowhere else.

Workload shapes follow the WorldAttention review (jaehun.me, "HKV:
Page-Level Multi-Tier Memory"): a page holds 8 latent frames of 1,560 tokens
(12,480 tokens), the page stage keeps K_p = 4 pages, so the active context is
4 x 8 x 1,560 = 49,920 tokens.  The current chunk is 3 latent frames (4,680
query tokens plus 4,680 own K/V tokens).  The Wan2.1-1.3B-shaped layer has 12
heads of dimension 128.

Value recipe (the pages fix none; stated so both sides can reproduce it):

* every array is i.i.d. N(0,1) drawn with ``numpy.random.default_rng`` in
  float32, one generator per (workload, tensor tag, page or chunk, step,
  frame) so that large pages can be drawn by several threads;
* bf16 workloads round each float32 value to bfloat16 (round to nearest,
  ties to even) and carry the 16-bit patterns as ``uint16`` arrays;
* the keys of page ``j`` are shifted by ``c_j * u`` before rounding, where
  ``u`` is one seeded unit vector of length ``head_dim`` shared by all heads
  and ``c_j = 0.5 * (1 + pi(j))`` for a seeded permutation ``pi`` over every
  page the workload ever holds.  Offsets are therefore 0.5 apart and their
  order differs from page order, so page scores do not tie.  Values carry no
  offset;
* for the sparse branch, ``aligned_queries`` shifts the chunk's queries by
  ``gain * u`` (the same noise as ``chunk_qkv``'s queries): the pooled
  attention map then favours the blocks of the pages with large ``c_j``, as a
  head that attends to a few places would, instead of the near-uniform map
  that i.i.d. queries give.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

# Tag ids keep the generator streams of different tensors apart.
TAG_Q, TAG_K, TAG_V, TAG_KOWN, TAG_VOWN = 1, 2, 3, 4, 5
TAG_U, TAG_PERM, TAG_PROMPT, TAG_CURPROMPT = 6, 7, 8, 9

F32, BF16 = "f32", "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype and cadence."""

    name: str
    wid: int                 # seed component identifying the workload
    dtype: str               # "f32" or "bf16"
    n_heads: int
    head_dim: int
    frame_tokens: int        # tokens per latent frame
    page_frames: int         # frames per page
    n_pages: int             # pages resident before the first chunk
    chunk_frames: int        # frames per chunk (queries = own K/V tokens)
    k_p: int                 # pages kept by the page stage
    steps: int = 1           # denoising steps per chunk
    chunks: int = 1          # chunks processed in sequence
    appended_per_chunk: int = 0   # pages appended after each chunk
    n_chunk_groups: int = 0  # prompt stage: past chunks holding the pages
    pages_per_group: int = 0
    emb_dim: int = 0         # prompt embedding width
    n_cand_groups: int = 0   # prompt stage: chunks kept as candidates
    scale: float | None = None

    @property
    def page_tokens(self) -> int:
        return self.frame_tokens * self.page_frames

    @property
    def n_q(self) -> int:
        return self.frame_tokens * self.chunk_frames

    @property
    def n_ctx(self) -> int:
        return self.k_p * self.page_tokens

    @property
    def max_pages(self) -> int:
        return self.n_pages + self.chunks * self.appended_per_chunk

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / np.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == F32 else np.uint16

    @property
    def has_prompt_stage(self) -> bool:
        return self.n_chunk_groups > 0


WORKLOADS = {
    # 1 head, d 64, 16-token frames, 2-frame pages, 8 pages, 3-frame chunk.
    "tiny_f32": Workload("tiny_f32", 1, F32, 1, 64, 16, 2, 8, 3, 2,
                         scale=1.0 / 8.0),
    # Wan2.1-1.3B-shaped layer, K_p = 4 of 16 pages, one denoising step.
    "wan_kp4": Workload("wan_kp4", 2, BF16, 12, 128, 1560, 8, 16, 3, 4),
    # Full history: all 6 pages attended, 4 denoising steps.
    "full_history": Workload("full_history", 3, BF16, 12, 128, 1560, 8, 6, 3, 6,
                             steps=4),
    # Prompt stage over 16 chunks of 4 pages, then page stage over 4 chunks.
    "prompt_page": Workload("prompt_page", 4, BF16, 12, 128, 1560, 8, 64, 3, 4,
                            n_chunk_groups=16, pages_per_group=4, emb_dim=4096,
                            n_cand_groups=4),
    # 128 resident pages, 8 chunks x 4 steps, one page appended per chunk.
    "long_horizon": Workload("long_horizon", 5, BF16, 12, 128, 1560, 8, 128, 3, 4,
                             steps=4, chunks=8, appended_per_chunk=1),
}


def scaled(wl: Workload, **changes) -> Workload:
    """A copy of ``wl`` with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(wl, **changes)


# ----------------------------------------------------------------------------
# encoding helpers (input encoding only)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; return uint16 patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 patterns to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def encode(wl: Workload, x: np.ndarray) -> np.ndarray:
    """Cast float32 values to the workload's element encoding."""
    return x.astype(np.float32) if wl.dtype == F32 else f32_to_bf16_bits(x)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _draw_rows(wl: Workload, tag: int, a: int, b: int, rows: int,
               shift: np.ndarray | None = None) -> np.ndarray:
    """[rows, H, d] of N(0,1), drawn one latent frame of rows per generator.

    ``shift`` (length head_dim, float32) is added to every (row, head)
    before the dtype encoding.
    """
    hd = wl.n_heads * wl.head_dim
    out = np.empty((rows, wl.n_heads, wl.head_dim), dtype=wl.np_dtype)
    ft = wl.frame_tokens
    n_frames = (rows + ft - 1) // ft

    def one(f: int) -> None:
        r0, r1 = f * ft, min(rows, (f + 1) * ft)
        rng = np.random.default_rng([wl.wid, tag, a, b, f])
        x = rng.standard_normal((r1 - r0) * hd, dtype=np.float32)
        x = x.reshape(r1 - r0, wl.n_heads, wl.head_dim)
        if shift is not None:
            x += shift
        out[r0:r1] = encode(wl, x)

    if n_frames > 1 and rows * hd > (1 << 20):
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(n_frames)))
    else:
        for f in range(n_frames):
            one(f)
    return out


# ----------------------------------------------------------------------------
# the workload's arrays

def offset_direction(wl: Workload) -> np.ndarray:
    """Unit vector u (float32, length head_dim) shared by all heads."""
    rng = np.random.default_rng([wl.wid, TAG_U])
    u = rng.standard_normal(wl.head_dim)
    return (u / np.linalg.norm(u)).astype(np.float32)


def offset_coefficients(wl: Workload) -> np.ndarray:
    """c_j = 0.5 * (1 + pi(j)) for every page the workload ever holds."""
    rng = np.random.default_rng([wl.wid, TAG_PERM])
    perm = rng.permutation(wl.max_pages)
    return 0.5 * (1.0 + perm.astype(np.float64))


def page_kv(wl: Workload, page: int) -> tuple[np.ndarray, np.ndarray]:
    """Keys and values of page ``page``: two [page_tokens, H, d] arrays."""
    shift = (np.float32(offset_coefficients(wl)[page]) * offset_direction(wl)).astype(np.float32)
    k = _draw_rows(wl, TAG_K, page, 0, wl.page_tokens, shift)
    v = _draw_rows(wl, TAG_V, page, 0, wl.page_tokens)
    return k, v


def chunk_qkv(wl: Workload, chunk: int, step: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Queries, own keys and own values of ``chunk`` at denoising ``step``."""
    q = _draw_rows(wl, TAG_Q, chunk, step, wl.n_q)
    k = _draw_rows(wl, TAG_KOWN, chunk, step, wl.n_q)
    v = _draw_rows(wl, TAG_VOWN, chunk, step, wl.n_q)
    return q, k, v


def aligned_queries(wl: Workload, chunk: int, step: int, gain: float) -> np.ndarray:
    """The queries of ``chunk_qkv`` shifted by ``gain * u`` before rounding."""
    shift = (np.float32(gain) * offset_direction(wl)).astype(np.float32)
    return _draw_rows(wl, TAG_Q, chunk, step, wl.n_q, shift)


def chunk_prompts(wl: Workload) -> np.ndarray:
    """[n_chunk_groups, emb_dim] float32 prompt embeddings of past chunks."""
    rng = np.random.default_rng([wl.wid, TAG_PROMPT])
    return rng.standard_normal((wl.n_chunk_groups, wl.emb_dim), dtype=np.float32)


def current_prompt(wl: Workload, chunk: int = 0) -> np.ndarray:
    """[emb_dim] float32 prompt embedding of the current chunk."""
    rng = np.random.default_rng([wl.wid, TAG_CURPROMPT, chunk])
    return rng.standard_normal(wl.emb_dim, dtype=np.float32)


def chunk_page_map(wl: Workload) -> np.ndarray:
    """[n_chunk_groups, pages_per_group] int32: past chunk m holds pages
    m*pages_per_group ... m*pages_per_group + pages_per_group - 1."""
    return np.arange(wl.n_chunk_groups * wl.pages_per_group,
                     dtype=np.int32).reshape(wl.n_chunk_groups, wl.pages_per_group)
