"""Benchmark of the paged-KV block-attention path on one MI355X.

Workload: the Wan2.1-1.3B-shaped layer -- 12 heads of dimension 128, pages of
8 frames x 1,560 tokens (12,480 tokens), 16 resident pages, a 3-frame chunk
(4,680 queries and 4,680 own K/V tokens), K_p = 4, so 49,920 gathered + 4,680
own keys per head; bf16 inputs, one denoising step per chunk.

One step = one pass of the whole path over the chunk, on one stream:
  append the chunk's page (copy into a spare pool slot + fp64 mean key),
  select (mean query -> scores over the 16 pages -> top-4),
  gather the 4 pages into one contiguous K/V buffer,
  block attention of the 4,680 queries over 54,600 keys.
Inputs are resident in HBM before the timed region.

Output: one JSON line.  `value` is block-attention TFLOP/s over the whole
step (attention FLOPs / step time).  Kernel-level figures (attention TFLOP/s
and its fraction of the bf16 matrix-core peak, select + gather GB/s and its
fraction of HBM peak) are measured with HIP events on the launch stream
(timing-only events, recorded without a system-scope fence).
The CPU baseline is the fp64 oracle timed on a bounded row sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E


class TimingEvent:
    """A HIP event used for timing only, created with hipEventDisableSystemFence.

    A default event performs a system-scope release when it is recorded (a
    cache write-back and invalidate), which delays the next kernel on the
    stream by microseconds and so shows up inside the intervals being
    measured; an event created with this flag skips that fence and records the
    same end-of-pipe timestamp (HIP runtime API, hipEventCreateWithFlags).
    Recorded on the stream the kernels are launched on; read after a device
    synchronisation."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            for name in ("libamdhip64.so.7", "libamdhip64.so"):
                try:   # the runtime torch and libwa.so already share
                    lib = ctypes.CDLL(name, mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
                    break
                except OSError:
                    continue
            else:
                raise RuntimeError("the HIP runtime is not loaded in this process")
            vp = ctypes.c_void_p
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [vp, vp]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            lib.hipEventDestroy.argtypes = [vp]
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        self._c = ctypes
        self.hip = self._runtime()
        self.ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(self.ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)

    def record(self, stream):
        rc = self.hip.hipEventRecord(self.ev, self._c.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = self._c.c_float()
        rc = self.hip.hipEventElapsedTime(self._c.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value

    def __del__(self):
        if getattr(self, "ev", None) and self.hip is not None:
            self.hip.hipEventDestroy(self.ev)


def cold_entry(ms, nbytes):
    """An HBM kernel's figures after a 1 GiB overwrite (L2s and MALL evicted)."""
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GB/s": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
            "note": "median of 10 reps, each after a 1 GiB overwrite (L2 and MALL evicted)"}


def attention_flops(n_q, n_k, head_dim, n_heads):
    """2 FLOP per multiply-add, two contractions (Q K^T and P V); softmax excluded."""
    return 4.0 * n_q * n_k * head_dim * n_heads


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--config", default="2", choices=["2", "3", "4", "5", "share"],
                    help="2: the Wan-shaped K_p=4 step (the headline line); 3: full history "
                         "(6 pages, all attended, 4 denoising steps per chunk); 4: prompt + page "
                         "selection (64 pages in 16 chunks, the prompt stage keeps 4 chunks); "
                         "5: long horizon "
                         "(128 -> 136 resident pages, 8 chunks x 4 steps, one page appended per "
                         "chunk); share: config 2 at 3 heads, one GPU's share of a 4-way "
                         "head-sharded layer")
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first; the clock takes ~20 launches to ramp from idle")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle sample for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles",
                                                      "k_attn_bf16_wan_kp4_hbm_traffic.txt"),
                    help="HBM traffic summary from rocprofv3 counters (optional)")
    return ap.parse_args()


class ClockSampler:
    """GFX clock and socket power of the GPU (amdsmi GPU metrics, every 10 ms:
    the firmware's averaged GFX clock, the current clock of each XCD, the
    memory clock) while the timed steps run.  Everything happens on a daemon thread, so a monitoring library
    that is missing or refuses never stalls or fails the bench; the summary
    then names the reason instead of the clocks."""

    def __init__(self, pci_bus_id):
        import threading
        self.bus = pci_bus_id
        self.gfx, self.xcd, self.mem, self.power = [], [], [], []
        self.error = None
        self.stop_flag = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if len(handles) > 1 and self.bus is not None:
                handles = [h for h in handles
                           if int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == self.bus]
            if len(handles) != 1:
                raise RuntimeError("%d matching GPUs" % len(handles))
            h = handles[0]
            num = lambda x: isinstance(x, (int, float))
            while not self.stop_flag.is_set():
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                self.gfx.append(m.get("average_gfxclk_frequency"))
                xcd = [x for x in (m.get("current_gfxclks") or []) if num(x) and x > 0]
                if xcd:
                    self.xcd.append(float(np.mean(xcd)))
                mem = m.get("average_uclk_frequency", m.get("current_uclk"))
                if not num(mem):
                    mem = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.MEM)["clk"]
                self.mem.append(mem)
                self.power.append(m.get("average_socket_power", m.get("current_socket_power")))
                self.stop_flag.wait(0.01)
        except Exception as e:          # report, never fail the bench
            self.error = "%s: %s" % (type(e).__name__, e)

    def start(self):
        self.thread.start()

    def stop(self):
        self.stop_flag.set()
        self.thread.join(timeout=2.0)
        def stats(v):
            v = [x for x in v if isinstance(x, (int, float))]
            if not v:
                return None
            return {"median": float(np.median(v)), "min": float(min(v)), "max": float(max(v))}
        if self.error or not self.gfx:
            return {"note": "not sampled (%s)" % (self.error or "no samples")}
        return {"unit": "MHz (power: W)", "samples": len(self.gfx),
                "gfx_average": stats(self.gfx), "gfx_current_xcd_mean": stats(self.xcd),
                "mem": stats(self.mem), "socket_power": stats(self.power),
                "note": "amdsmi GPU metrics every 10 ms over the timed steps"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the path is built and measured on one GPU's "
              "share of the work; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.config in ("3", "4", "5"):
        print(json.dumps(bench_chunks(args)), flush=True)
        return

    import torch

    import paged_kv_attention_page_amd as wa
    import wa_workloads as W

    wl = W.WORKLOADS["wan_kp4"]
    if args.config == "share":
        wl = W.scaled(wl, name="wan_kp4_share3", n_heads=3)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    L = wa.layout(wa.WA_BF16, wl.n_heads, wl.head_dim, wl.page_tokens, wl.n_pages + 1)
    spare = wl.n_pages                     # slot the per-step append writes

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).view(torch.bfloat16).to(dev)

    # ---- inputs, resident in HBM before timing
    shape = (L.max_pages, wl.page_tokens, wl.n_heads, wl.head_dim)
    k_pool = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    v_pool = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    means = torch.zeros(L.max_pages, wl.n_heads, wl.head_dim, dtype=torch.float64, device=dev)
    ws_append = torch.empty(wa.wa_append_workspace_bytes(L), dtype=torch.uint8, device=dev)
    for j in range(wl.n_pages):
        k, v = W.page_kv(wl, j)
        k_pool[j].copy_(up(k))
        v_pool[j].copy_(up(v))
    for j in range(wl.n_pages):
        wa.wa_append_page(L, k_pool[j], v_pool[j], k_pool, v_pool, j, means, workspace=ws_append)
    k_new, v_new = W.page_kv(W.scaled(wl, n_pages=wl.n_pages + 1), wl.n_pages)
    k_new, v_new = up(k_new), up(v_new)
    q_h, ko_h, vo_h = W.chunk_qkv(wl, 0, 0)
    q, k_own, v_own = up(q_h), up(ko_h), up(vo_h)
    cand = torch.arange(wl.n_pages, dtype=torch.int32, device=dev)
    idx = torch.empty(wl.k_p, dtype=torch.int32, device=dev)
    ws_sel = torch.zeros(wa.wa_select_workspace_bytes(L, wl.n_q, wl.n_pages), dtype=torch.uint8,
                         device=dev)
    ws_attn = torch.empty(max(16, wa.wa_attention_workspace_bytes(L, wl.n_q, wl.n_ctx, wl.n_q)),
                          dtype=torch.uint8, device=dev)
    ctx_shape = (wl.n_ctx, wl.n_heads, wl.head_dim)
    k_ctx = torch.empty(ctx_shape, dtype=torch.bfloat16, device=dev)
    v_ctx = torch.empty(ctx_shape, dtype=torch.bfloat16, device=dev)
    out = torch.empty((wl.n_q, wl.n_heads, wl.head_dim), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    n_k = wl.n_ctx + wl.n_q
    flops = attention_flops(wl.n_q, n_k, wl.head_dim, wl.n_heads)
    page_bytes = wl.page_tokens * wl.n_heads * wl.head_dim * 2
    row_means = wl.n_heads * wl.head_dim * 8
    bytes_append = 2 * 2 * page_bytes + row_means
    bytes_select = wl.n_q * wl.n_heads * wl.head_dim * 2 + wl.n_pages * row_means + 4 * wl.k_p
    bytes_gather = 2 * 2 * wl.k_p * page_bytes
    # Each event recorded between two calls costs the stream a few microseconds
    # (a marker packet between the kernels), so the timed steps record only the
    # boundaries the reported figures need: append | select + gather | attention.
    # select and gather alone come from a short pass after the timed region.
    def step(timed=None, split=None):
        if timed is not None:
            timed[0].record(stream)
        wa.wa_append_page(L, k_new, v_new, k_pool, v_pool, spare, means, workspace=ws_append,
                          stream=stream)
        if timed is not None:
            timed[1].record(stream)
        if split is not None:
            split[0].record(stream)
        wa.wa_select_pages(L, q, means, wl.k_p, cand=cand, out_idx=idx, workspace=ws_sel,
                           stream=stream)
        if split is not None:
            split[1].record(stream)
        wa.wa_gather(L, k_pool, v_pool, idx, wl.k_p, k_ctx, v_ctx, stream=stream)
        if timed is not None:
            timed[2].record(stream)
        if split is not None:
            split[2].record(stream)
        wa.wa_block_attention(L, q, k_ctx, v_ctx, k_own, v_own, wl.softmax_scale,
                              out_dtype=wa.WA_BF16, out=out, workspace=ws_attn, stream=stream)
        if timed is not None:
            timed[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # K timed steps between two synchronisations; HIP events recorded on the
    # launch stream inside the same region give the per-kernel durations
    evs = [[TimingEvent() for _ in range(4)] for _ in range(args.steps)]
    clocks = ClockSampler(getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None))
    clocks.start()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    clock_summary = clocks.stop()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    names = ("append", "select_gather", "attention")
    per = {n: [e[i].elapsed_time(e[i + 1]) for e in evs] for i, n in enumerate(names)}
    avg = {k: float(np.mean(v)) for k, v in per.items()}
    med = {k: float(np.median(v)) for k, v in per.items()}

    # split pass (untimed for the step figure): select and gather separately
    n_split = min(args.steps, 10)
    sev = [[TimingEvent() for _ in range(3)] for _ in range(n_split)]
    for k in range(n_split):
        step(split=sev[k])
    torch.cuda.synchronize()
    split = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in sev]))
             for i, n in enumerate(("select", "gather"))}

    # cold pass (after the timed region): a 1 GiB overwrite before each rep
    # evicts the L2s and the 256 MB MALL, so the HBM kernels start from HBM;
    # the in-step figures above run with the step's other kernels in between
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = {"append": [], "select_gather": []}
    for k in range(10):
        for name in ("append", "select_gather"):
            flush.fill_(k & 0xff)
            e0, e1 = TimingEvent(), TimingEvent()
            e0.record(stream)
            if name == "append":
                wa.wa_append_page(L, k_new, v_new, k_pool, v_pool, spare, means,
                                  workspace=ws_append, stream=stream)
            else:
                wa.wa_select_pages(L, q, means, wl.k_p, cand=cand, out_idx=idx, workspace=ws_sel,
                                   stream=stream)
                wa.wa_gather(L, k_pool, v_pool, idx, wl.k_p, k_ctx, v_ctx, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            cold[name].append(e0.elapsed_time(e1))
    del flush
    cold_ms = {n: float(np.median(v)) for n, v in cold.items()}

    # paged pass (after the timed region; not part of the step figure): the
    # same step with the attention reading the selected pages in place from
    # the pool (wa_paged_attention) instead of gather + attention over the copy
    def step_paged(ev=None):
        wa.wa_append_page(L, k_new, v_new, k_pool, v_pool, spare, means, workspace=ws_append,
                          stream=stream)
        wa.wa_select_pages(L, q, means, wl.k_p, cand=cand, out_idx=idx, workspace=ws_sel,
                           stream=stream)
        if ev is not None:
            ev[0].record(stream)
        wa.wa_paged_attention(L, q, k_pool, v_pool, idx, wl.k_p, k_own, v_own, wl.softmax_scale,
                              out_dtype=wa.WA_BF16, out=out, workspace=ws_attn, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    n_paged = args.steps
    for _ in range(5):
        step_paged()
    pev = [[TimingEvent() for _ in range(2)] for _ in range(n_paged)]
    torch.cuda.synchronize()
    tp0 = time.perf_counter()
    for k in range(n_paged):
        step_paged(pev[k])
    torch.cuda.synchronize()
    tp1 = time.perf_counter()
    paged_ms_step = (tp1 - tp0) * 1e3 / n_paged
    paged_attn_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in pev]))

    # sparse pass (after the timed region; not part of the step figure): the
    # sparse branch over the same gathered context and own keys -- key-block
    # selection (wa_hsa_select), then attention over the selected 64-key
    # tiles only (wa_sparse_attention).  Its queries are the chunk's queries
    # shifted along the page-offset direction (a concentrated pooled map; the
    # plain queries give a near-uniform one), with per-head thresholds
    # 0.50, 0.54, ..., 0.94.
    share = args.config == "share"
    sparse = None if share else sparse_pass(wa, W, wl, L, up, k_ctx, v_ctx, k_own, v_own, out,
                                            stream, args.steps, avg["attention"], torch)

    # host-tier pass (after the sparse pass; not part of the step figure): the
    # first selected page lives in pinned host memory and is copied into the
    # spare slot while the attention over the other selected pages runs
    tier = None if share else tier_pass(wa, wl, L, k_pool, v_pool, q, k_own, v_own, idx, spare,
                                        stream, min(args.steps, 20), paged_attn_ms, torch)

    attn_tflops = flops / (avg["attention"] * 1e-3) / 1e12
    sg_gbps = (bytes_select + bytes_gather) / (avg["select_gather"] * 1e-3) / 1e9
    value = flops / (ms_per_step * 1e-3) / 1e12
    # the committed counter summary covers the 12-head launch only
    traffic = None if share else load_traffic(args.traffic, wa.kernel_source("k_attn_bf16.hip"))

    result = {
        "metric": "block-attn TFLOP/s (MFMA %) + select/gather HBM GB/s at Kp=4, 49,920-tok KV",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("wan_kp4: Wan2.1-1.3B-shaped layer, 12 heads x 128, 12,480-token pages, "
                         "16 resident pages, K_p=4, 4,680-query chunk, 49,920+4,680 keys, "
                         "1 denoising step") if not share else
                        ("wan_kp4_share3: one GPU's share of the Wan2.1-1.3B-shaped layer "
                         "head-sharded over 4 GPUs: 3 heads x 128, 12,480-token pages, 16 "
                         "resident pages, K_p=4, 4,680-query chunk, 49,920+4,680 keys, 1 "
                         "denoising step (57 query-block x head items: the split launch)"),
            "n_heads": wl.n_heads, "head_dim": wl.head_dim, "page_tokens": wl.page_tokens,
            "pages": wl.n_pages, "k_p": wl.k_p, "n_q": wl.n_q, "n_ctx": wl.n_ctx,
            "n_keys": n_k,
            "parallelism": "single GPU" if not share else "1 GPU's share of 4-way head sharding",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "k_attn_bf16",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
        "kernels_ms": {k: round(v, 4) for k, v in avg.items()},
        "kernels_ms_median": {k: round(v, 4) for k, v in med.items()},
        "kernels_ms_min": {k: round(float(np.min(v)), 4) for k, v in per.items()},
        "select_gather": {
            "bytes": bytes_select + bytes_gather,
            "GB/s": round(sg_gbps, 1),
            "hbm_frac": round(sg_gbps / PEAK_HBM_GBPS, 4),
            "split_pass_ms": {k: round(v, 4) for k, v in split.items()},
            "gather_GB/s": round(bytes_gather / (split["gather"] * 1e-3) / 1e9, 1),
            "select_GB/s": round(bytes_select / (split["select"] * 1e-3) / 1e9, 1),
            "cold": cold_entry(cold_ms["select_gather"], bytes_select + bytes_gather),
        },
        "append": {
            "bytes": bytes_append,
            "GB/s": round(bytes_append / (avg["append"] * 1e-3) / 1e9, 1),
            "cold": cold_entry(cold_ms["append"], bytes_append),
        },
        "clocks": clock_summary,
        "paged": {
            "note": "append + select + wa_paged_attention (pages read in place, no gather), "
                    "same inputs, timed after the step figure",
            "ms_per_step": round(paged_ms_step, 4),
            "attention_ms": round(paged_attn_ms, 4),
            "attention_TFLOP/s": round(flops / (paged_attn_ms * 1e-3) / 1e12, 2),
            "step_speedup_vs_gathered": round(ms_per_step / paged_ms_step, 4),
        },
        "sparse": sparse,
        "tier": tier,
        "flops_per_step": flops,
        "attention_split_launch": bool(wa.wa_attention_workspace_bytes(L, wl.n_q, wl.n_ctx,
                                                                        wl.n_q) > 0),
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, q_h, k_pool, v_pool, idx, ko_h, vo_h, means,
                                              args.cpu_seconds, torch)
    print(json.dumps(result), flush=True)


def roofline_mfma(flops, ms, traffic=None):
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": "k_attn_bf16", "achieved": round(tf, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic}


def bench_chunks(args):
    """Configs 3, 4 and 5: whole chunks of the block-diffusion cadence (Inferix
    summary, section 3.4, Steps 3 and 4): per chunk, select + gather once, then
    T denoising steps of attention (4 in configs 3 and 5, 1 in config 4), each
    with fresh queries and own K/V over the same gathered pages; config 5 then
    appends one new page (the pool grows from 128 to 136 pages over 8 chunks).
    Config 4 selects in two stages (WorldAttention review, "HKV: Page-Level
    Multi-Tier Memory"): the prompt stage keeps the 4 of 16 past chunks whose
    4,096-dim prompt embeddings are closest in cosine to the current one, and
    the page stage the top 4 of their 16 pages.  One timed step = one chunk;
    `value` = attention FLOPs of the chunk / chunk time."""
    import torch

    import paged_kv_attention_page_amd as wa
    import wa_workloads as W

    long_h = args.config == "5"
    two_stage = args.config == "4"
    name = {"3": "full_history", "4": "prompt_page", "5": "long_horizon"}[args.config]
    wl = W.WORKLOADS[name]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    L = wa.layout(wa.WA_BF16, wl.n_heads, wl.head_dim, wl.page_tokens, wl.max_pages)
    T = wl.steps
    n_chunks = wl.chunks

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).view(torch.bfloat16).to(dev)

    shape = (L.max_pages, wl.page_tokens, wl.n_heads, wl.head_dim)
    k_pool = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    v_pool = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    means = torch.zeros(L.max_pages, wl.n_heads, wl.head_dim, dtype=torch.float64, device=dev)
    ws_append = torch.empty(wa.wa_append_workspace_bytes(L), dtype=torch.uint8, device=dev)
    for j in range(wl.max_pages):
        k, v = W.page_kv(wl, j)
        k_pool[j].copy_(up(k))
        v_pool[j].copy_(up(v))
    for j in range(wl.n_pages):
        wa.wa_append_page(L, k_pool[j], v_pool[j], k_pool, v_pool, j, means, workspace=ws_append)
    # pages appended after chunk c (config 5): page n_pages + c, from a staging copy
    new_pages = [(k_pool[wl.n_pages + c].clone(), v_pool[wl.n_pages + c].clone())
                 for c in range(n_chunks * wl.appended_per_chunk)]
    qkv = [[tuple(up(x) for x in W.chunk_qkv(wl, c, t)) for t in range(T)]
           for c in range(n_chunks)]
    idx = torch.empty(wl.k_p, dtype=torch.int32, device=dev)
    prompt = prompt_h = None
    if two_stage:
        prompt_h = dict(chunk_prompts=W.chunk_prompts(wl), cur_prompt=W.current_prompt(wl),
                        chunk_pages=W.chunk_page_map(wl), n_keep=wl.n_cand_groups)
        prompt = {k: (torch.from_numpy(v).to(dev) if isinstance(v, np.ndarray) else v)
                  for k, v in prompt_h.items()}
        max_cand = wl.n_cand_groups * wl.pages_per_group
    else:
        max_cand = wl.n_pages + (n_chunks - 1) * wl.appended_per_chunk
    ws_sel = torch.zeros(wa.wa_select_workspace_bytes(L, wl.n_q, max_cand, prompt),
                         dtype=torch.uint8, device=dev)
    ws_attn = torch.empty(max(16, wa.wa_attention_workspace_bytes(L, wl.n_q, wl.n_ctx, wl.n_q)),
                          dtype=torch.uint8, device=dev)
    ctx_shape = (wl.n_ctx, wl.n_heads, wl.head_dim)
    k_ctx = torch.empty(ctx_shape, dtype=torch.bfloat16, device=dev)
    v_ctx = torch.empty(ctx_shape, dtype=torch.bfloat16, device=dev)
    out = torch.empty((wl.n_q, wl.n_heads, wl.head_dim), dtype=torch.bfloat16, device=dev)
    cands = [None if two_stage else
             torch.arange(wl.n_pages + c * wl.appended_per_chunk, dtype=torch.int32, device=dev)
             for c in range(n_chunks)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    n_k = wl.n_ctx + wl.n_q
    flops_step = attention_flops(wl.n_q, n_k, wl.head_dim, wl.n_heads)
    page_bytes = wl.page_tokens * wl.n_heads * wl.head_dim * 2
    row_means = wl.n_heads * wl.head_dim * 8

    def chunk(c, ev=None):
        """ev: T + 3 events (select+gather start, attention boundaries, append end)."""
        cand = cands[c]
        if ev is not None:
            ev[0].record(stream)
        wa.wa_select_pages(L, qkv[c][0][0], means, wl.k_p, cand=cand, prompt=prompt,
                           out_idx=idx, workspace=ws_sel, stream=stream)
        wa.wa_gather(L, k_pool, v_pool, idx, wl.k_p, k_ctx, v_ctx, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        for t in range(T):
            q, ko, vo = qkv[c][t]
            wa.wa_block_attention(L, q, k_ctx, v_ctx, ko, vo, wl.softmax_scale,
                                  out_dtype=wa.WA_BF16, out=out, workspace=ws_attn, stream=stream)
            if ev is not None:
                ev[2 + t].record(stream)
        for a in range(wl.appended_per_chunk):
            slot = wl.n_pages + c * wl.appended_per_chunk + a
            kn, vn = new_pages[c * wl.appended_per_chunk + a]
            wa.wa_append_page(L, kn, vn, k_pool, v_pool, slot, means, workspace=ws_append,
                              stream=stream)
        if ev is not None:
            ev[2 + T].record(stream)

    for w in range(args.warmup):
        chunk(w % n_chunks)
    torch.cuda.synchronize()
    evs = [[TimingEvent() for _ in range(T + 3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        chunk(k % n_chunks, evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_chunk = (t1 - t0) * 1e3 / args.steps
    sg = [e[0].elapsed_time(e[1]) for e in evs]
    att = [e[1 + t].elapsed_time(e[2 + t]) for e in evs for t in range(T)]
    app = [e[1 + T].elapsed_time(e[2 + T]) for e in evs] if wl.appended_per_chunk else []
    att_ms = float(np.mean(att))
    # Q once, the candidates' page means, the top-K_p ids; config 4 also reads
    # the prompt embeddings and the chunk-to-page map
    prompt_bytes = (4 * wl.emb_dim * (wl.n_chunk_groups + 1)
                    + 4 * wl.n_chunk_groups * wl.pages_per_group) if two_stage else 0
    sel_bytes = [wl.n_q * wl.n_heads * wl.head_dim * 2 + max_cand * row_means + prompt_bytes
                 + 4 * wl.k_p if two_stage else
                 wl.n_q * wl.n_heads * wl.head_dim * 2 + cands[k % n_chunks].numel() * row_means
                 + 4 * wl.k_p for k in range(args.steps)]
    sg_bytes = float(np.mean(sel_bytes)) + 2 * 2 * wl.k_p * page_bytes
    sg_ms = float(np.mean(sg))
    value = T * flops_step / (ms_chunk * 1e-3) / 1e12
    desc = {"long_horizon":
            "long_horizon: Wan2.1-1.3B-shaped layer, 12 heads x 128, 12,480-token pages, 128 "
            "resident pages growing to 136 (one appended per chunk), K_p=4 selected over every "
            "resident page, 4,680-query chunks, 49,920+4,680 keys, 8 chunks x 4 denoising steps",
            "full_history":
            "full_history: Wan2.1-1.3B-shaped layer, 12 heads x 128, 12,480-token pages, 6 "
            "resident pages all attended (K_p=6), 4,680-query chunk, 74,880+4,680 keys, 4 "
            "denoising steps with fresh queries and own K/V",
            "prompt_page":
            "prompt_page: Wan2.1-1.3B-shaped layer, 12 heads x 128, 12,480-token pages, 64 "
            "resident pages in 16 past chunks of 4, N(0,1) 4,096-dim prompt embeddings; the "
            "prompt stage keeps 4 chunks by cosine to the current prompt, the page stage the "
            "top K_p=4 of their 16 pages; 4,680-query chunk, 49,920+4,680 keys, 1 denoising "
            "step"}[name]
    result = {
        "metric": "block-attn TFLOP/s (MFMA %) + select/gather HBM GB/s, " + name,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_chunk, 4),
        "step": "one chunk: select + gather, %d attention step%s%s" % (
            T, "s" if T > 1 else "", ", append of one page" if wl.appended_per_chunk else ""),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "n_heads": wl.n_heads, "head_dim": wl.head_dim,
                   "page_tokens": wl.page_tokens, "pages": wl.n_pages,
                   "pages_max": wl.max_pages, "k_p": wl.k_p, "n_q": wl.n_q, "n_ctx": wl.n_ctx,
                   "n_keys": n_k, "steps_per_chunk": T, "chunks": n_chunks,
                   "parallelism": "single GPU"},
        "roofline": roofline_mfma(flops_step, att_ms),
        "attention_ms_per_step": {"mean": round(att_ms, 4),
                                  "median": round(float(np.median(att)), 4),
                                  "min": round(float(np.min(att)), 4)},
        "attention_target_ms": round(flops_step / (0.6 * PEAK_BF16_TFLOPS * 1e12) * 1e3, 4),
        "select_gather": {"bytes": int(sg_bytes), "ms": round(sg_ms, 4),
                          "GB/s": round(sg_bytes / (sg_ms * 1e-3) / 1e9, 1),
                          "hbm_frac": round(sg_bytes / (sg_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
        "flops_per_attention_step": flops_step,
        "cpu_baseline": None,
    }
    if app:
        app_ms = float(np.mean(app))
        app_bytes = 2 * 2 * page_bytes + row_means
        result["append"] = {"bytes": app_bytes, "ms": round(app_ms, 4),
                            "GB/s": round(app_bytes / (app_ms * 1e-3) / 1e9, 1)}
        result["pool_bytes"] = {"first_chunk": 2 * wl.n_pages * page_bytes,
                                "after_last_chunk": 2 * wl.max_pages * page_bytes}
    if not args.no_cpu_baseline:
        c_last = (args.steps - 1) % n_chunks
        q_h, ko_h, vo_h = W.chunk_qkv(wl, c_last, T - 1)
        result["cpu_baseline"] = cpu_baseline(wl, q_h, k_pool, v_pool, idx, ko_h, vo_h, means,
                                              args.cpu_seconds, torch,
                                              n_resident=wl.n_pages if two_stage else
                                              cands[c_last].numel(), prompt_h=prompt_h)
    return result


def sparse_pass(wa, W, wl, L, up, k_ctx, v_ctx, k_own, v_own, out, stream, steps, dense_ms,
                torch):
    dev = k_ctx.device
    n_ctx, n_own, n_q = wl.n_ctx, wl.n_q, wl.n_q
    q_sp = up(W.aligned_queries(wl, 0, 0, 8.0))
    tau = torch.tensor([0.5 + 0.04 * h for h in range(wl.n_heads)], dtype=torch.float64,
                       device=dev)
    q_blocks, items, n_tiles = wa.hsa_shape(L, n_q, n_ctx, n_own)
    tiles = torch.empty((items, n_tiles), dtype=torch.int32, device=dev)
    count = torch.empty(items, dtype=torch.int32, device=dev)
    ws = torch.empty(max(16, wa.wa_hsa_workspace_bytes(L, n_q, n_ctx, n_own)), dtype=torch.uint8,
                     device=dev)
    ws_att = torch.empty(max(16, wa.wa_sparse_workspace_bytes(L, n_q, n_ctx, n_own)),
                         dtype=torch.uint8, device=dev)

    def one(ev=None):
        if ev is not None:
            ev[0].record(stream)
        wa.wa_hsa_select(L, q_sp, k_ctx, k_own, tau, scale=wl.softmax_scale, sel_tiles=tiles,
                         sel_count=count, want_gini=False, workspace=ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        wa.wa_sparse_attention(L, q_sp, k_ctx, v_ctx, k_own, v_own, tiles, count,
                               wl.softmax_scale, out_dtype=wa.WA_BF16, out=out, workspace=ws_att,
                               stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(5):
        one()
    evs = [[TimingEvent() for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        one(evs[k])
    torch.cuda.synchronize()
    sel_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    att_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    # a chunk's later denoising steps: same context, so the selection takes
    # the context block sums the calls above left in ws
    rev = [[TimingEvent() for _ in range(2)] for _ in range(steps)]
    for k in range(steps):
        rev[k][0].record(stream)
        wa.wa_hsa_select(L, q_sp, k_ctx, k_own, tau, scale=wl.softmax_scale, sel_tiles=tiles,
                         sel_count=count, want_gini=False, workspace=ws, ctx_sums_ready=True,
                         stream=stream)
        rev[k][1].record(stream)
    torch.cuda.synchronize()
    sel_reuse_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in rev]))
    # flops over the keys actually attended: per item, its query rows times
    # the keys of its listed tiles (the last tile of [ctx ++ own] is short)
    t_h, c_h = tiles.cpu().numpy(), count.cpu().numpy()
    n_keys = n_ctx + n_own
    kept_flops, kept_keys = 0, 0
    for item in range(items):
        b = item % q_blocks
        rows = min(256, n_q - 256 * b)
        lst = t_h[item, :c_h[item]]
        keys = 64 * lst.size - (64 * n_tiles - n_keys if (lst == n_tiles - 1).any() else 0)
        kept_keys += keys
        kept_flops += 4 * rows * keys * wl.head_dim
    tflops = kept_flops / (att_ms * 1e-3) / 1e12
    return {
        "note": "wa_hsa_select + wa_sparse_attention over the gathered 49,920 + own 4,680 keys; "
                "queries aligned with the page offsets (gain 8), tau_h = 0.50 + 0.04 h",
        "select_ms": round(sel_ms, 4),
        "attention_ms": round(att_ms, 4),
        "kept_key_fraction": round(kept_keys / (items * n_keys), 4),
        "attention_TFLOP/s_on_kept_keys": round(tflops, 2),
        "attention_frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "speedup_vs_dense_attention": round(dense_ms / (sel_ms + att_ms), 3),
        "select_ms_context_sums_reused": round(sel_reuse_ms, 4),
        "speedup_vs_dense_attention_later_steps": round(dense_ms / (sel_reuse_ms + att_ms), 3),
    }


def tier_pass(wa, wl, L, k_pool, v_pool, q, k_own, v_own, idx, spare, stream, reps,
              resident_ms, torch):
    dev = k_pool.device
    sel = idx.cpu().numpy().tolist()           # once per chunk in a tiered step
    page_shape = (1, wl.page_tokens, wl.n_heads, wl.head_dim)
    hk = torch.empty(page_shape, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty(page_shape, dtype=torch.bfloat16, pin_memory=True)
    wa.wa_page_out(L, k_pool, v_pool, sel[0], hk, hv, 0, stream=stream)
    torch.cuda.synchronize()
    rest = torch.tensor(sel[1:], dtype=torch.int32, device=dev)
    one = torch.tensor([spare], dtype=torch.int32, device=dev)
    four = torch.tensor([spare] + sel[1:], dtype=torch.int32, device=dev)
    n_q = wl.n_q
    oa = torch.empty((n_q, wl.n_heads, wl.head_dim), dtype=torch.float32, device=dev)
    ob = torch.empty_like(oa)
    la = torch.empty((wl.n_heads, n_q), dtype=torch.float32, device=dev)
    lb = torch.empty_like(la)
    oc = torch.empty_like(oa)
    lc = torch.empty_like(la)
    out = torch.empty((n_q, wl.n_heads, wl.head_dim), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(16, wa.wa_attention_workspace_bytes(L, n_q, wl.n_ctx, n_q)),
                     dtype=torch.uint8, device=dev)
    copy = torch.cuda.Stream()                 # default priority
    parts = 4
    bounds = [wl.page_tokens * i // parts for i in range(parts + 1)]

    def page_in(st):
        wa.wa_page_in(L, hk, hv, 0, k_pool, v_pool, spare, stream=st)

    def serial():
        page_in(stream)
        wa.wa_paged_attention(L, q, k_pool, v_pool, four, 4, k_own, v_own, wl.softmax_scale,
                              out_dtype=wa.WA_BF16, out=out, workspace=ws, stream=stream)

    def overlapped():
        copy.wait_stream(stream)               # the previous step is done with the slot
        page_in(copy)
        done = torch.cuda.Event()
        done.record(copy)
        wa.wa_paged_attention(L, q, k_pool, v_pool, rest, 3, k_own, v_own, wl.softmax_scale,
                              out_dtype=wa.WA_F32, out=oa, lse=la, workspace=ws, stream=stream)
        stream.wait_event(done)
        wa.wa_paged_attention(L, q, k_pool, v_pool, one, 1, None, None, wl.softmax_scale,
                              out_dtype=wa.WA_F32, out=ob, lse=lb, workspace=ws, stream=stream)
        wa.wa_merge_attention(L, oa, la, ob, lb, wa.WA_BF16, out=out, stream=stream)

    def in_parts():
        # the page copied in row ranges, each attended as soon as it has
        # landed and merged into the running result
        copy.wait_stream(stream)
        landed = []
        for r0, r1 in zip(bounds[:-1], bounds[1:]):
            wa.wa_page_in_rows(L, hk, hv, 0, k_pool, v_pool, spare, r0, r1 - r0, stream=copy)
            ev = torch.cuda.Event()
            ev.record(copy)
            landed.append(ev)
        wa.wa_paged_attention(L, q, k_pool, v_pool, rest, 3, k_own, v_own, wl.softmax_scale,
                              out_dtype=wa.WA_F32, out=oa, lse=la, workspace=ws, stream=stream)
        cur = (oa, la)
        for i, (r0, r1) in enumerate(zip(bounds[:-1], bounds[1:])):
            stream.wait_event(landed[i])
            wa.wa_block_attention(L, q, k_pool[spare, r0:r1], v_pool[spare, r0:r1], None, None,
                                  wl.softmax_scale, out_dtype=wa.WA_F32, out=ob, lse=lb,
                                  workspace=ws, stream=stream)
            if i == parts - 1:
                wa.wa_merge_attention(L, cur[0], cur[1], ob, lb, wa.WA_BF16, out=out,
                                      stream=stream)
            else:
                nxt = (oc, lc) if cur[0] is oa else (oa, la)
                wa.wa_merge_attention(L, cur[0], cur[1], ob, lb, wa.WA_F32, out=nxt[0],
                                      lse=nxt[1], stream=stream)
                cur = nxt

    def timed(fn, st, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record(st)
        for _ in range(n):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # blocks of a few steps per variant, the variants interleaved, median
    # block: a transient slowdown of the copy engines or the clock then moves
    # one block, not one variant's whole figure
    variants = {"copy": (lambda: page_in(copy), copy), "serial": (serial, stream),
                "overlapped": (overlapped, stream), "in_parts": (in_parts, stream)}
    blocks = {k: [] for k in variants}
    per_block = max(1, reps // 5)
    for _ in range(5):
        for k, (fn, st) in variants.items():
            blocks[k].append(timed(fn, st, per_block))
    copy_ms, serial_ms, over_ms, parts_ms = (float(np.median(blocks[k])) for k in variants)
    page_bytes = 2 * wl.page_tokens * wl.n_heads * wl.head_dim * 2
    # the page is back in HBM where it was (slot sel[0] was never changed)
    return {
        "note": "1 of the K_p=4 selected pages in pinned host memory; page-in (K and V, copy "
                "engines) on a second stream during the attention over the other 3 pages and "
                "the own keys, then attention over the copied page and the log-sum-exp merge",
        "page_in_ms": round(copy_ms, 4),
        "page_in_GB/s": round(page_bytes / (copy_ms * 1e-3) / 1e9, 1),
        "serial_ms": round(serial_ms, 4),
        "overlapped_ms": round(over_ms, 4),
        "all_resident_ms": round(resident_ms, 4),
        "copy_hidden_fraction": round((serial_ms - over_ms) / copy_ms, 3),
        "in_parts": {
            "note": "the host page copied in %d row ranges (wa_page_in_rows), each attended "
                    "(wa_block_attention on those rows of the slot) as soon as it has landed "
                    "and merged into the running result" % parts,
            "overlapped_ms": round(parts_ms, 4),
            "copy_hidden_fraction": round((serial_ms - parts_ms) / copy_ms, 3),
        },
    }


def load_traffic(path, kernel_src):
    """HBM bytes per attention launch from the rocprofv3 counter summary, or
    None when there is none or it was taken on a different kernel source."""
    if not path or not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    import hashlib
    if fields.get("kernel_source_sha256") != hashlib.sha256(kernel_src).hexdigest():
        return None
    return int(fields["bytes_per_launch"])


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, q_h, k_pool, v_pool, idx, ko_h, vo_h, means, seconds, torch,
                 n_resident=None, prompt_h=None):
    """The fp64 oracle's attention on a bounded sample of query rows (all heads),
    on the host cores, in the metric's unit (TFLOP/s); the other stages of the
    step (one page mean, the selection, the gather) timed once each beside it."""
    import oracle
    oracle.use_native()          # gcc -O3 -march=native, built on this host
    sel = idx.cpu().numpy()
    k_ctx = np.ascontiguousarray(k_pool[torch.from_numpy(sel).long()].view(torch.uint16).cpu()
                                 .numpy().reshape(-1, wl.n_heads, wl.head_dim))
    v_ctx = np.ascontiguousarray(v_pool[torch.from_numpy(sel).long()].view(torch.uint16).cpu()
                                 .numpy().reshape(-1, wl.n_heads, wl.head_dim))
    n_k = k_ctx.shape[0] + ko_h.shape[0]
    threads = oracle.n_threads()
    rows = np.arange(0, wl.n_q, wl.n_q // 8, dtype=np.int64)[:8]
    t0 = time.perf_counter()
    oracle.attention(q_h, k_ctx, v_ctx, ko_h, vo_h, wl.softmax_scale, rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    n_rows = int(min(wl.n_q, max(8, round(8 * seconds / max(dt, 1e-3)))))
    if n_rows > 8:
        rows = np.unique(np.linspace(0, wl.n_q - 1, n_rows).round().astype(np.int64))
        t0 = time.perf_counter()
        oracle.attention(q_h, k_ctx, v_ctx, ko_h, vo_h, wl.softmax_scale, rows=rows,
                         threads=threads)
        dt = time.perf_counter() - t0
    fl = attention_flops(len(rows), n_k, wl.head_dim, wl.n_heads)
    stages = {}
    t0 = time.perf_counter()
    oracle.page_mean(k_ctx[:wl.page_tokens])
    stages["append_page_mean"] = time.perf_counter() - t0
    n_resident = wl.n_pages if n_resident is None else n_resident
    pm = np.ascontiguousarray(means[:n_resident].cpu().numpy())
    t0 = time.perf_counter()
    oracle.select_pages(q_h, pm, wl.k_p, prompt=prompt_h)
    stages["select"] = time.perf_counter() - t0
    pages = np.ascontiguousarray(k_ctx.reshape(wl.k_p, wl.page_tokens, wl.n_heads, wl.head_dim))
    pages_v = np.ascontiguousarray(v_ctx.reshape(wl.k_p, wl.page_tokens, wl.n_heads, wl.head_dim))
    order = np.arange(wl.k_p, dtype=np.int32)
    t0 = time.perf_counter()
    oracle.gather(pages, order)
    oracle.gather(pages_v, order)
    stages["gather"] = time.perf_counter() - t0
    return {
        "value": round(fl / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "build": "gcc -O3 -march=native -fopenmp (fp64, OpenMP over rows and heads)",
        "sample": "block attention of %d of %d query rows x %d heads over %d keys (fp64, "
                  "%.1f s)" % (len(rows), wl.n_q, wl.n_heads, n_k, dt),
        "stages_s": {k: round(v, 4) for k, v in stages.items()},
        "stages_note": "the oracle once each: the mean key of one page, the selection over "
                       "the %d resident pages (%smean query, scores, top-%d), the gather of the "
                       "K and V of %d pages (single-threaded; attention uses the cores above)"
                       % (n_resident, "prompt stage, " if prompt_h is not None else "", wl.k_p,
                          wl.k_p),
        "nproc": os.cpu_count(),
        "cpu_model": cpu_model(),
    }


if __name__ == "__main__":
    main()
