"""Run one workload through the HIP path and through the oracle, side by side.

Both sides take their inputs from ``wa_workloads`` only.  The HIP side goes
through the C ABI (via the thin binding); the oracle side through
``oracle``.  Comparisons live in the tests.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_kv_attention_page_amd as wa
import wa_workloads as W


def say(*args):
    """Name the GPU step about to run, flushed, so a failed run shows where it was."""
    print("[gpu-step]", *args, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, dev="cuda") -> torch.Tensor:
    """numpy float32 / bf16 bit pattern (uint16) array -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(dev)


def to_bits(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy array with the same encoding as the inputs."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.uint16).numpy()
    return t.numpy()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def wa_layout(wl: W.Workload):
    dt = wa.WA_F32 if wl.dtype == W.F32 else wa.WA_BF16
    return wa.layout(dt, wl.n_heads, wl.head_dim, wl.page_tokens, wl.max_pages)


class PoolRun:
    """Pool of a workload on the device (filled through wa_append_page) plus the
    host copies the oracle needs."""

    def __init__(self, wl: W.Workload, keep_host_pages: bool = True):
        self.wl = wl
        self.L = wa_layout(wl)
        dt = self.L.torch_dtype
        shape = (wl.max_pages, wl.page_tokens, wl.n_heads, wl.head_dim)
        say("alloc pool", wl.name, shape)
        self.k_pool = torch.zeros(shape, dtype=dt, device="cuda")
        self.v_pool = torch.zeros(shape, dtype=dt, device="cuda")
        self.means = torch.full((wl.max_pages, wl.n_heads, wl.head_dim), float("nan"),
                                dtype=torch.float64, device="cuda")
        self.ws = torch.empty(wa.wa_append_workspace_bytes(self.L), dtype=torch.uint8,
                              device="cuda")
        self.host_k = {}
        self.host_v = {}
        self.keep = keep_host_pages

    def append(self, page: int, slot: int | None = None):
        slot = page if slot is None else slot
        k, v = W.page_kv(self.wl, page)
        if self.keep:
            self.host_k[slot], self.host_v[slot] = k, v
        kd, vd = to_device(k), to_device(v)
        say("append page", page, "slot", slot)
        wa.wa_append_page(self.L, kd, vd, self.k_pool, self.v_pool, slot, self.means,
                          workspace=self.ws)
        return k, v

    def oracle_means(self, slots) -> np.ndarray:
        return np.stack([oracle.page_mean(self.host_k[s]) for s in slots])


def rows_sample(n_q: int, n: int) -> np.ndarray:
    """Deterministic spread of query rows, always including the first and last."""
    if n >= n_q:
        return np.arange(n_q, dtype=np.int64)
    r = np.unique(np.linspace(0, n_q - 1, n).round().astype(np.int64))
    return r


def attention_tolerance(wl: W.Workload) -> float:
    """Max abs error allowed on attention outputs: 1e-5 for fp32 inputs, 1e-2 for
    bf16 inputs with fp32 accumulation."""
    return 1e-5 if wl.dtype == W.F32 else 1e-2
