"""Host-memory page tier: wa_page_out / wa_page_in / wa_page_in_rows between a
pinned host pool and the HBM pool (bit-exact byte copies), wa_merge_attention against the
oracle's merge and its attention over the union of the keys, and the tiered
step: the selected pages that live in host memory are copied in on a second
stream while the attention over the resident pages runs, then the attention
over the copied pages and the merge -- held to the oracle's attention over
all the selected pages; also with the host page copied in row ranges, each
attended as soon as it has landed.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_page_amd as wa
import wa_workloads as W
from tests.pipeline import PoolRun, attention_tolerance, rows_sample, say, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wa.load_library()


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


SMALL = W.scaled(W.WORKLOADS["wan_kp4"], n_heads=2, frame_tokens=64, page_frames=2, n_pages=8,
                 chunk_frames=3, k_p=3)


def _host_pool(wl, pages):
    shape = (pages, wl.page_tokens, wl.n_heads, wl.head_dim)
    dt = torch.bfloat16 if wl.dtype == W.BF16 else torch.float32
    return (torch.zeros(shape, dtype=dt, pin_memory=True),
            torch.zeros(shape, dtype=dt, pin_memory=True))


def test_page_out_then_in_is_a_byte_copy():
    wl = SMALL
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    hk, hv = _host_pool(wl, 3)
    say("page out slot 5 -> host 2, slot 1 -> host 0 (K only)")
    wa.wa_page_out(run.L, run.k_pool, run.v_pool, 5, hk, hv, 2)
    wa.wa_page_out(run.L, run.k_pool, None, 1, hk, None, 0)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(hk[2]), _bits(run.k_pool[5])) and np.array_equal(
        _bits(hv[2]), _bits(run.v_pool[5]))
    assert np.array_equal(_bits(hk[0]), _bits(run.k_pool[1]))
    say("page in host 2 -> slot 7")
    wa.wa_page_in(run.L, hk, hv, 2, run.k_pool, run.v_pool, 7)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(run.k_pool[7]), run.host_k[5].view(np.int16))
    assert np.array_equal(_bits(run.v_pool[7]), run.host_v[5].view(np.int16))
    # pageable host memory is refused by the binding and by the library
    pageable = torch.zeros_like(hk, pin_memory=False)
    with pytest.raises(ValueError):
        wa.wa_page_in(run.L, pageable, None, 0, run.k_pool, None, 0)
    lib = wa.load_library()
    st = lib.wa_page_in(ctypes.byref(run.L), ctypes.c_void_p(pageable.data_ptr()), None, 3, 0,
                        ctypes.c_void_p(run.k_pool.data_ptr()), None, 0, None)
    assert st == wa.WA_ERR_INVALID_ARG


def test_page_in_rows_copies_those_rows_only():
    """wa_page_in_rows in three uneven parts (and a K-only part): after each
    part the copied rows are byte copies of the host page and the rest of
    the slot is untouched."""
    wl = SMALL                                     # 128-token pages
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    hk, hv = _host_pool(wl, 2)
    wa.wa_page_out(run.L, run.k_pool, run.v_pool, 5, hk, hv, 1)
    torch.cuda.synchronize()
    slot, P_t = 7, wl.page_tokens
    run.k_pool[slot].fill_(-3.0)
    run.v_pool[slot].fill_(-3.0)
    before_k, before_v = _bits(run.k_pool[slot]).copy(), _bits(run.v_pool[slot]).copy()
    done = 0
    for r0, n in ((0, 37), (37, 63), (100, P_t - 100)):
        say("page in rows", r0, "..", r0 + n, "of host page 1 -> slot", slot)
        wa.wa_page_in_rows(run.L, hk, hv, 1, run.k_pool, run.v_pool, slot, r0, n)
        torch.cuda.synchronize()
        done = r0 + n
        gk, gv = _bits(run.k_pool[slot]), _bits(run.v_pool[slot])
        assert np.array_equal(gk[:done], run.host_k[5][:done].view(np.int16))
        assert np.array_equal(gv[:done], run.host_v[5][:done].view(np.int16))
        assert np.array_equal(gk[done:], before_k[done:])
        assert np.array_equal(gv[done:], before_v[done:])
    # K only, one row in the middle of slot 6
    k6, v6 = _bits(run.k_pool[6]).copy(), _bits(run.v_pool[6]).copy()
    say("page in row 64 of host page 1 (K only) -> slot 6")
    wa.wa_page_in_rows(run.L, hk, None, 1, run.k_pool, None, 6, 64, 1)
    torch.cuda.synchronize()
    gk = _bits(run.k_pool[6])
    assert np.array_equal(gk[64], run.host_k[5][64].view(np.int16))
    assert np.array_equal(np.delete(gk, 64, axis=0), np.delete(k6, 64, axis=0))
    assert np.array_equal(_bits(run.v_pool[6]), v6)
    with pytest.raises(wa.WaError):
        wa.wa_page_in_rows(run.L, hk, hv, 1, run.k_pool, run.v_pool, slot, 100, P_t - 99)


def test_merge_matches_the_oracle():
    """Attention over the first 300 context keys and over the rest (with the
    own keys), merged, against the oracle's attention over all of them."""
    wl = W.scaled(SMALL, n_pages=6)
    kv = [W.page_kv(wl, p) for p in range(4)]
    kc = np.concatenate([k for k, _ in kv])
    vc = np.concatenate([v for _, v in kv])
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    L = wa.layout(wa.WA_BF16, wl.n_heads, wl.head_dim)
    cut = 300
    lse_a = torch.empty(wl.n_heads, wl.n_q, dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    say("attention over two key sets, then merge")
    out_a = wa.wa_block_attention(L, to_device(q), to_device(kc[:cut]), to_device(vc[:cut]), None,
                                  None, wl.softmax_scale, out_dtype=wa.WA_F32, lse=lse_a)
    out_b = wa.wa_block_attention(L, to_device(q), to_device(kc[cut:]), to_device(vc[cut:]),
                                  to_device(ko), to_device(vo), wl.softmax_scale,
                                  out_dtype=wa.WA_F32, lse=lse_b)
    lse = torch.empty_like(lse_a)
    out = wa.wa_merge_attention(L, out_a, lse_a, out_b, lse_b, wa.WA_F32, lse=lse)
    out16 = wa.wa_merge_attention(L, out_a, lse_a, out_b, lse_b, wa.WA_BF16)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, kc, vc, ko, vo, wl.softmax_scale)
    tol = attention_tolerance(wl)
    assert np.abs(to_f64(out) - ref).max() <= tol
    assert np.abs(to_f64(out16) - ref).max() <= tol
    assert np.abs(lse.cpu().double().numpy() - ref_lse).max() <= tol
    # against the oracle's own merge of the GPU parts: fp32 rounding only
    m, ml = oracle.merge_attention(to_f64(out_a), lse_a.cpu().double().numpy(), to_f64(out_b),
                                   lse_b.cpu().double().numpy())
    assert np.abs(to_f64(out) - m).max() <= 1e-5
    assert np.abs(lse.cpu().double().numpy() - ml).max() <= 1e-5


def _tiered_step(run, q, ko, vo, idx, on_host, hk, hv, spare):
    """Attention over pages idx: the pages in on_host (logical page -> host
    slot) are copied into spare HBM slots on a second stream while the
    attention over the resident ones (with the own keys) runs; then the
    attention over the copied pages and the merge."""
    wl, L = run.wl, run.L
    resident = [p for p in idx if p not in on_host]
    missing = [p for p in idx if p in on_host]
    copy = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    copy.wait_stream(main)
    slots = spare[:len(missing)]
    with torch.cuda.stream(copy):
        for p, s in zip(missing, slots):
            wa.wa_page_in(L, hk, hv, on_host[p], run.k_pool, run.v_pool, s, stream=copy)
    done = torch.cuda.Event()
    done.record(copy)
    qd, kod, vod = to_device(q), to_device(ko), to_device(vo)
    lse_a = torch.empty(wl.n_heads, q.shape[0], dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    res = torch.tensor(resident, dtype=torch.int32, device="cuda")
    say("tiered step: resident", resident, "copied in", missing, "into", slots)
    out_a = wa.wa_paged_attention(L, qd, run.k_pool, run.v_pool, res, len(resident), kod, vod,
                                  wl.softmax_scale, out_dtype=wa.WA_F32, lse=lse_a)
    main.wait_event(done)
    mis = torch.tensor(slots, dtype=torch.int32, device="cuda")
    out_b = wa.wa_paged_attention(L, qd, run.k_pool, run.v_pool, mis, len(slots), None, None,
                                  wl.softmax_scale, out_dtype=wa.WA_F32, lse=lse_b)
    return wa.wa_merge_attention(L, out_a, lse_a, out_b, lse_b, wa.WA_BF16)


def _tiered_step_in_parts(run, q, ko, vo, idx, page, host_slot, hk, hv, spare, parts):
    """Attention over pages idx, of which `page` lives in host memory: it is
    copied into slot `spare` in `parts` row ranges on a second stream, each
    followed by an event; the attention over the resident pages (with the own
    keys) runs first, then the attention over each range as soon as it has
    landed (wa_block_attention on those rows of the slot), each merged into
    the running result."""
    wl, L = run.wl, run.L
    resident = [p for p in idx if p != page]
    copy = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    copy.wait_stream(main)
    bounds = [wl.page_tokens * i // parts for i in range(parts + 1)]
    landed = []
    with torch.cuda.stream(copy):
        for r0, r1 in zip(bounds[:-1], bounds[1:]):
            wa.wa_page_in_rows(L, hk, hv, host_slot, run.k_pool, run.v_pool, spare, r0, r1 - r0,
                               stream=copy)
            ev = torch.cuda.Event()
            ev.record(copy)
            landed.append(ev)
    qd, kod, vod = to_device(q), to_device(ko), to_device(vo)
    lse = torch.empty(wl.n_heads, q.shape[0], dtype=torch.float32, device="cuda")
    res = torch.tensor(resident, dtype=torch.int32, device="cuda")
    say("tiered step in", parts, "parts: resident", resident, "page", page, "into slot", spare)
    out = wa.wa_paged_attention(L, qd, run.k_pool, run.v_pool, res, len(resident), kod, vod,
                                wl.softmax_scale, out_dtype=wa.WA_F32, lse=lse)
    for i, (r0, r1) in enumerate(zip(bounds[:-1], bounds[1:])):
        main.wait_event(landed[i])
        lse_b = torch.empty_like(lse)
        out_b = wa.wa_block_attention(L, qd, run.k_pool[spare, r0:r1], run.v_pool[spare, r0:r1],
                                      None, None, wl.softmax_scale, out_dtype=wa.WA_F32,
                                      lse=lse_b)
        if i == parts - 1:
            return wa.wa_merge_attention(L, out, lse, out_b, lse_b, wa.WA_BF16)
        lse_m = torch.empty_like(lse)
        out = wa.wa_merge_attention(L, out, lse, out_b, lse_b, wa.WA_F32, lse=lse_m)
        lse = lse_m


@pytest.mark.parametrize("parts", [1, 3, 4])
def test_tiered_step_in_parts_matches_the_oracle(parts):
    wl = SMALL
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    idx = wa.wa_select_pages(run.L, to_device(q), run.means, wl.k_p).cpu().numpy().tolist()
    hk, hv = _host_pool(wl, 1)
    wa.wa_page_out(run.L, run.k_pool, run.v_pool, idx[1], hk, hv, 0)
    torch.cuda.synchronize()
    run.k_pool[idx[1]].zero_()
    run.v_pool[idx[1]].zero_()
    spare = [p for p in range(wl.max_pages) if p not in idx][0]
    out = _tiered_step_in_parts(run, q, ko, vo, idx, idx[1], 0, hk, hv, spare, parts)
    torch.cuda.synchronize()
    k_ctx = np.concatenate([run.host_k[p] for p in idx])
    v_ctx = np.concatenate([run.host_v[p] for p in idx])
    ref, _ = oracle.attention(q, k_ctx, v_ctx, ko, vo, wl.softmax_scale)
    assert np.abs(to_f64(out) - ref).max() <= attention_tolerance(wl)


def test_tiered_step_in_parts_full_size():
    """wan_kp4 at full size, the first selected page copied in 4 parts during
    the attention; sampled rows against the oracle."""
    wl = W.WORKLOADS["wan_kp4"]
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    idx = wa.wa_select_pages(run.L, to_device(q), run.means, wl.k_p).cpu().numpy().tolist()
    hk, hv = _host_pool(wl, 1)
    wa.wa_page_out(run.L, run.k_pool, run.v_pool, idx[0], hk, hv, 0)
    torch.cuda.synchronize()
    run.k_pool[idx[0]].zero_()
    run.v_pool[idx[0]].zero_()
    spare = [p for p in range(wl.max_pages) if p not in idx][0]
    out = _tiered_step_in_parts(run, q, ko, vo, idx, idx[0], 0, hk, hv, spare, 4)
    torch.cuda.synchronize()
    rows = rows_sample(wl.n_q, 10)
    k_ctx = np.concatenate([run.host_k[p] for p in idx])
    v_ctx = np.concatenate([run.host_v[p] for p in idx])
    ref, _ = oracle.attention(q, k_ctx, v_ctx, ko, vo, wl.softmax_scale, rows=rows)
    assert np.abs(to_f64(out)[rows] - ref).max() <= attention_tolerance(wl)


def test_tiered_step_matches_the_oracle():
    wl = SMALL
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    idx = wa.wa_select_pages(run.L, to_device(q), run.means, wl.k_p).cpu().numpy().tolist()
    # two of the selected pages live in host memory (moved out, slots reused)
    hk, hv = _host_pool(wl, 2)
    on_host = {idx[0]: 1, idx[2]: 0}
    for p, h in on_host.items():
        wa.wa_page_out(run.L, run.k_pool, run.v_pool, p, hk, hv, h)
    torch.cuda.synchronize()
    for p in on_host:                      # the HBM slots are overwritten
        run.k_pool[p].zero_()
        run.v_pool[p].zero_()
    spare = [p for p in range(wl.max_pages) if p not in idx][:2]
    out = _tiered_step(run, q, ko, vo, idx, on_host, hk, hv, spare)
    torch.cuda.synchronize()
    k_ctx = np.concatenate([run.host_k[p] for p in idx])
    v_ctx = np.concatenate([run.host_v[p] for p in idx])
    ref, _ = oracle.attention(q, k_ctx, v_ctx, ko, vo, wl.softmax_scale)
    assert np.abs(to_f64(out) - ref).max() <= attention_tolerance(wl)


def test_tiered_step_full_size():
    """wan_kp4 at full size: of the 4 selected 12,480-token pages, the first
    lives in host memory (copied in during the attention over the other 3 and
    the own keys); sampled rows against the oracle."""
    wl = W.WORKLOADS["wan_kp4"]
    run = PoolRun(wl)
    for j in range(wl.n_pages):
        run.append(j)
    q, ko, vo = W.chunk_qkv(wl, 0, 0)
    idx = wa.wa_select_pages(run.L, to_device(q), run.means, wl.k_p).cpu().numpy().tolist()
    hk, hv = _host_pool(wl, 1)
    on_host = {idx[0]: 0}
    wa.wa_page_out(run.L, run.k_pool, run.v_pool, idx[0], hk, hv, 0)
    torch.cuda.synchronize()
    run.k_pool[idx[0]].zero_()
    run.v_pool[idx[0]].zero_()
    spare = [p for p in range(wl.max_pages) if p not in idx][:1]
    out = _tiered_step(run, q, ko, vo, idx, on_host, hk, hv, spare)
    torch.cuda.synchronize()
    rows = rows_sample(wl.n_q, 10)
    k_ctx = np.concatenate([run.host_k[p] for p in idx])
    v_ctx = np.concatenate([run.host_v[p] for p in idx])
    ref, _ = oracle.attention(q, k_ctx, v_ctx, ko, vo, wl.softmax_scale, rows=rows)
    assert np.abs(to_f64(out)[rows] - ref).max() <= attention_tolerance(wl)


def test_tiered_step_on_growing_scores():
    """The tiered step on scores far from unit variance: keys climb along one
    direction that every query shares, so the scores rise to about 16 over the
    768 context keys.  The merge weights each part by exp(lse_part - lse), so
    this holds the parts' log-sum-exps, through the merged output and lse, to
    the same bar as the outputs (one softmax over all the selected pages,
    Inferix summary, section 3.4, Step 3; partial results accumulated as in
    its "Ring Attention" paragraph)."""
    wl = W.scaled(SMALL, name="tier_growing")     # 8 slots of 128 tokens; 6 hold data
    L = wa.layout(wa.WA_BF16, wl.n_heads, wl.head_dim, wl.page_tokens, wl.max_pages)
    P_t, n_own, n_q = wl.page_tokens, 90, 70
    rng = np.random.default_rng([wl.wid, 31])
    u = np.ones(wl.head_dim, np.float32) / np.sqrt(wl.head_dim)

    def rows(n, ramp):
        x = 0.25 * rng.standard_normal((n, wl.n_heads, wl.head_dim), dtype=np.float32)
        if ramp is not None:
            x += (ramp[:, None, None] * u[None, None, :]).astype(np.float32)
        return W.encode(wl, x)

    n_sel = 6
    n_ctx = n_sel * P_t
    ramp = 0.06 * np.arange(n_ctx + n_own, dtype=np.float32)
    q = rows(n_q, np.full(n_q, 4.0, np.float32))
    kc, ko = rows(n_ctx, ramp[:n_ctx]), rows(n_own, ramp[n_ctx:])
    vc, vo = rows(n_ctx, None), rows(n_own, None)
    shape = (wl.max_pages, P_t, wl.n_heads, wl.head_dim)
    k_pool = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    v_pool = torch.zeros_like(k_pool)
    for j in range(n_sel):
        k_pool[j].copy_(to_device(kc[j * P_t:(j + 1) * P_t]))
        v_pool[j].copy_(to_device(vc[j * P_t:(j + 1) * P_t]))
    # selected pages in a non-temporal order; pages 5 and 1 live in host memory
    idx = [3, 5, 0, 1, 4, 2]
    on_host = {5: 0, 1: 1}
    hk, hv = _host_pool(wl, 2)
    for p, h in on_host.items():
        wa.wa_page_out(L, k_pool, v_pool, p, hk, hv, h)
    torch.cuda.synchronize()
    for p in on_host:
        k_pool[p].zero_()
        v_pool[p].zero_()
    spare = [6, 7]
    resident = [p for p in idx if p not in on_host]
    missing = [p for p in idx if p in on_host]
    copy = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    copy.wait_stream(main)
    with torch.cuda.stream(copy):
        for p, s in zip(missing, spare):
            wa.wa_page_in(L, hk, hv, on_host[p], k_pool, v_pool, s, stream=copy)
    done = torch.cuda.Event()
    done.record(copy)
    qd, kod, vod = to_device(q), to_device(ko), to_device(vo)
    lse_a = torch.empty(wl.n_heads, n_q, dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    say("tiered step on growing scores: resident", resident, "copied in", missing)
    out_a = wa.wa_paged_attention(L, qd, k_pool, v_pool,
                                  torch.tensor(resident, dtype=torch.int32, device="cuda"),
                                  len(resident), kod, vod, wl.softmax_scale, out_dtype=wa.WA_F32,
                                  lse=lse_a)
    main.wait_event(done)
    out_b = wa.wa_paged_attention(L, qd, k_pool, v_pool,
                                  torch.tensor(spare, dtype=torch.int32, device="cuda"),
                                  len(spare), None, None, wl.softmax_scale, out_dtype=wa.WA_F32,
                                  lse=lse_b)
    lse = torch.empty_like(lse_a)
    out = wa.wa_merge_attention(L, out_a, lse_a, out_b, lse_b, wa.WA_F32, lse=lse)
    out16 = wa.wa_merge_attention(L, out_a, lse_a, out_b, lse_b, wa.WA_BF16)
    torch.cuda.synchronize()
    order = [p for p in idx]                       # keys in the order attended: any order
    k_sel = np.concatenate([kc[p * P_t:(p + 1) * P_t] for p in order])
    v_sel = np.concatenate([vc[p * P_t:(p + 1) * P_t] for p in order])
    ref, ref_lse = oracle.attention(q, k_sel, v_sel, ko, vo, wl.softmax_scale)
    assert ref_lse.max() > 14.0, "scores should climb far beyond unit variance"
    tol = attention_tolerance(wl)
    assert np.abs(to_f64(out) - ref).max() <= tol
    assert np.abs(to_f64(out16) - ref).max() <= tol
    assert np.abs(lse.cpu().double().numpy() - ref_lse).max() <= tol
