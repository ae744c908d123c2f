"""One whole step -- append a page, select with the library's fixed workspace
(wa_select_pages_noalloc), gather, bf16 block attention -- captured in one
HIP graph and replayed, against the same calls made eagerly on the same
inputs.  Between replays the inputs change (another page into the appended
slot, queries and own K/V of another denoising step), the outputs are
overwritten with junk, and an eager selection over 100 listed candidates
(the two-level path, whose completion counters share the fixed workspace)
runs outside the graph.  The graph holds kernels only (the library issues no
memset or copy on these calls), and the kernels are the eager ones, so every
replay must equal the eager step bit for bit.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_page_amd as wa
import wa_workloads as W
from tests.pipeline import PoolRun, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wa.load_library()


def _fill(dst: torch.Tensor, x: np.ndarray):
    src = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        src = src.view(torch.bfloat16)
    dst.copy_(src.view(dst.shape))


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float64:
        return t.view(torch.int64).numpy()
    if t.dtype in (torch.bfloat16, torch.float32):
        return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()
    return t.numpy()


def test_graph_replays_of_a_step_equal_the_eager_step():
    wl = W.scaled(W.WORKLOADS["wan_kp4"], name="graph_step", n_heads=4, frame_tokens=200,
                  n_pages=12, chunk_frames=6, k_p=4)     # 1,600-token pages, 1,200 queries
    run = PoolRun(wl, keep_host_pages=False)
    for j in range(wl.n_pages - 1):
        run.append(j)
    L, dt, kp = run.L, run.L.torch_dtype, wl.k_p
    slot = wl.n_pages - 1
    row = (wl.n_heads, wl.head_dim)
    dev = "cuda"
    kin = torch.empty((wl.page_tokens,) + row, dtype=dt, device=dev)
    vin = torch.empty_like(kin)
    q = torch.empty((wl.n_q,) + row, dtype=dt, device=dev)
    kown, vown = torch.empty_like(q), torch.empty_like(q)
    cand = torch.arange(wl.n_pages, dtype=torch.int32, device=dev)
    idx = torch.empty(kp, dtype=torch.int32, device=dev)
    scores = torch.empty(wl.n_pages, dtype=torch.float64, device=dev)
    k_ctx = torch.empty((kp * wl.page_tokens,) + row, dtype=dt, device=dev)
    v_ctx = torch.empty_like(k_ctx)
    out = torch.empty_like(q)
    lse = torch.empty(wl.n_q * wl.n_heads, dtype=torch.float32, device=dev)
    attn_ws = torch.empty(wa.wa_attention_workspace_bytes(L, wl.n_q, kp * wl.page_tokens, wl.n_q),
                          dtype=torch.uint8, device=dev)
    outputs = (idx, scores, k_ctx, v_ctx, out, lse, run.means[slot])

    def step():
        wa.wa_append_page(L, kin, vin, run.k_pool, run.v_pool, slot, run.means,
                          workspace=run.ws)
        wa.wa_select_pages_noalloc(L, q, run.means, kp, cand=cand, out_idx=idx,
                                   out_scores=scores)
        wa.wa_gather(L, run.k_pool, run.v_pool, idx, kp, k_ctx=k_ctx, v_ctx=v_ctx)
        wa.wa_block_attention(L, q, k_ctx, v_ctx, kown, vown, out=out, lse=lse,
                              workspace=attn_ws)

    def load(r):
        k, v = W.page_kv(wl, (slot, 3, 7)[r])
        qq, ko, vo = W.chunk_qkv(wl, 0, r)
        for t, x in ((kin, k), (vin, v), (q, qq), (kown, ko), (vown, vo)):
            _fill(t, x)

    def junk():
        idx.fill_(-5)
        for t in outputs[1:]:
            t.fill_(float("nan"))

    load(0)
    say("graph: eager warm-up step")
    step()
    torch.cuda.synchronize()

    say("graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    many = torch.from_numpy(np.random.default_rng(5).integers(0, wl.n_pages, 100)
                            .astype(np.int32)).to(dev)
    other_idx = torch.empty(5, dtype=torch.int32, device=dev)
    first_out = None
    for r in range(3):
        load(r)
        junk()
        say("graph: replay", r)
        g.replay()
        torch.cuda.synchronize()
        got = [_bits(t) for t in outputs]

        say("graph: eager selection over 100 listed candidates after replay", r)
        wa.wa_select_pages_noalloc(L, q, run.means, 5, cand=many, n_cand=100, out_idx=other_idx)
        torch.cuda.synchronize()

        junk()
        say("graph: eager step", r)
        step()
        torch.cuda.synchronize()
        ref = [_bits(t) for t in outputs]
        for name, a, b in zip(("idx", "scores", "k_ctx", "v_ctx", "out", "lse", "mean"), got, ref):
            assert np.array_equal(a, b), "replay %d: %s differs from the eager step" % (r, name)
        assert np.all(got[0] >= 0) and np.all(got[0] < wl.n_pages)
        assert not torch.isnan(out).any().item()
        if first_out is None:
            first_out = got[4]
        else:   # the replay read this step's inputs, not the captured ones
            assert not np.array_equal(first_out, got[4])


def test_graph_replays_of_the_sparse_branch_equal_the_eager_calls():
    """wa_hsa_select then wa_sparse_attention (plan, tile-list attention,
    merge) captured in one HIP graph, replayed with new queries, against the
    eager calls: tile lists, counts, output and lse bit for bit.  The shape
    (12 items of up to 1,005 tiles on all CUs) takes the split launch."""
    H, d, n_q, n_ctx, n_own = 4, 128, 700, 64 * 1000, 300
    L = wa.layout(wa.WA_BF16, H, d)
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(11)
    q = torch.empty((n_q, H, d), dtype=torch.bfloat16, device=dev)
    k_ctx = torch.randn((n_ctx, H, d), device=dev, generator=g).to(torch.bfloat16)
    v_ctx = torch.randn((n_ctx, H, d), device=dev, generator=g).to(torch.bfloat16)
    k_own = torch.randn((n_own, H, d), device=dev, generator=g).to(torch.bfloat16)
    v_own = torch.randn((n_own, H, d), device=dev, generator=g).to(torch.bfloat16)
    tau = torch.tensor([0.5, 0.7, 0.9, 0.95], dtype=torch.float64, device=dev)
    _, items, n_tiles = wa.hsa_shape(L, n_q, n_ctx, n_own)
    tiles = torch.empty((items, n_tiles), dtype=torch.int32, device=dev)
    count = torch.empty(items, dtype=torch.int32, device=dev)
    ws_sel = torch.empty(max(16, wa.wa_hsa_workspace_bytes(L, n_q, n_ctx, n_own)),
                         dtype=torch.uint8, device=dev)
    ws_att = torch.empty(max(16, wa.wa_sparse_workspace_bytes(L, n_q, n_ctx, n_own)),
                         dtype=torch.uint8, device=dev)
    out = torch.empty((n_q, H, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((H, n_q), dtype=torch.float32, device=dev)
    outputs = (tiles, count, out, lse)

    def branch():
        wa.wa_hsa_select(L, q, k_ctx, k_own, tau, sel_tiles=tiles, sel_count=count,
                         want_gini=False, workspace=ws_sel)
        wa.wa_sparse_attention(L, q, k_ctx, v_ctx, k_own, v_own, tiles, count,
                               out_dtype=wa.WA_BF16, out=out, lse=lse, workspace=ws_att)

    def load(r):
        # queries with a shared direction, so the pooled map is concentrated
        # and the heads keep different numbers of blocks
        gr = torch.Generator(device=dev).manual_seed(100 + r)
        x = torch.randn((n_q, H, d), device=dev, generator=gr)
        q.copy_((x + 2.0 * k_ctx[:1].float()).to(torch.bfloat16))

    def junk():
        tiles.fill_(-9)
        count.fill_(-9)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))

    load(0)
    say("graph: eager sparse branch")
    branch()
    torch.cuda.synchronize()
    assert int(ws_att[:4].view(torch.int32)[0]) == 1, "the shape should take the split launch"
    say("graph: capture of the sparse branch")
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        branch()
    torch.cuda.synchronize()
    first = None
    for r in range(3):
        load(r)
        junk()
        say("graph: sparse replay", r)
        gr.replay()
        torch.cuda.synchronize()
        got = [_bits(t) for t in outputs]
        junk()
        say("graph: eager sparse branch", r)
        branch()
        torch.cuda.synchronize()
        ref = [_bits(t) for t in outputs]
        for name, a, b in zip(("tiles", "count", "out", "lse"), got, ref):
            assert np.array_equal(a, b), "replay %d: %s differs from the eager calls" % (r, name)
        assert np.all(got[1] >= 1) and np.all(got[1] <= n_tiles)
        assert not torch.isnan(out).any().item()
        if first is None:
            first = got[2]
        else:
            assert not np.array_equal(first, got[2])
