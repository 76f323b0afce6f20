"""Graph capture and replay of a step's path: append + extend attention (+ the
split combine) captured once into a HIP graph, with the metadata built before
capture and reused by every replay (the way a step's plan serves every layer).
Each replay runs after eager work and a synchronization of its own and must
reproduce the eager result exactly (same kernels, same inputs), which in turn
meets the oracle bound. The library's launches record kernels only: no memset,
allocation or synchronization is captured."""
import numpy as np
import pytest
import torch

import workloads as wl
from pkv_testlib import assert_parity, oracle_out, oracle_pools

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_chunked_prefill_amd as pkv
    from gpu_harness import DeviceCache, shape_of, upload_q, values_of


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    assert pkv.device_supported(torch.cuda.current_device()), "not a gfx950 device"


def _workload(name):
    if name == "ragged_splits":
        return wl.config2()            # 96 tiles < 256 slots: long tiles are split, the combine runs
    if name == "decode_splits":
        w = wl.config5(decode_only=True)
        return w.subset(list(range(8)))  # 8 one-token rows, 8 KV splits each
    return wl.config4(mid_page=True)   # window, no splits


def _pool_rows(cache, w, dev):
    """The cache's page table as rows of a larger request pool in a shuffled
    order, with req_pool_indices pointing each request at its row."""
    rows = 3 * w.batch + 5
    perm = np.random.default_rng(17).permutation(rows)[:w.batch].astype(np.int32)
    big = np.full((rows, w.page_table.shape[1]), -1, np.int32)
    big[perm] = w.page_table
    pkv.check_req_pool_indices(perm, rows, w.batch)
    cache.page_table = torch.from_numpy(big).to(dev)
    return torch.from_numpy(perm).to(dev)


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused_append"])
@pytest.mark.parametrize("name,pool_rows", [("ragged_splits", False), ("decode_splits", False), ("window", False),
                                            ("ragged_splits", True), ("decode_splits", True)])
def test_graph_replay_matches_eager(name, pool_rows, fused):
    w = _workload(name)
    dev = torch.device("cuda", torch.cuda.current_device())
    print(f"[graph] {name} fused={fused} req_pool_indices={pool_rows}: P={list(w.prefix_lens)[:4]} "
          f"L={list(w.chunk_lens)[:4]} batch={w.batch}", flush=True)
    cache = DeviceCache(w, dev)
    cache.fill_prefix(w)
    rpi = _pool_rows(cache, w, dev) if pool_rows else None
    plan = pkv.build_extend_metadata(w.prefix_lens, w.chunk_lens, shape_of(w), w.window, w.decode_splits, device=dev)
    kn, vn = cache._gather_new_kv(w)
    q = upload_q(w, dev)
    out = torch.empty_like(q)
    ws = plan.workspace()   # allocated before capture

    def path():
        if fused:   # paged_extend_attn_append: one launch for these plans where it fuses
            pkv.paged_extend_attn_append(q, kn, vn, cache.k_pool, cache.v_pool, cache.page_table, plan, out=out,
                                         workspace=ws, req_pool_indices=rpi)
            return
        pkv.pkv_append(kn, vn, cache.k_pool, cache.v_pool, cache.page_table, plan, req_pool_indices=rpi)
        pkv.paged_extend_attn(q, cache.k_pool, cache.v_pool, cache.page_table, plan, out=out, workspace=ws,
                              req_pool_indices=rpi)

    path()                  # eager: the reference result (appending again later writes the same bytes)
    torch.cuda.synchronize()
    eager = out.clone()
    assert pkv.read_status(plan) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()              # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    scratch = torch.randn(1 << 20, device=dev)
    for r in range(4):
        out.fill_(float("nan"))                 # eager work between replays
        scratch.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager result"
    assert pkv.read_status(plan) == 0
    if name == "ragged_splits":   # small enough for the whole oracle
        ref = oracle_out(w, oracle_pools(w), dtype=np.float32)
        rep = assert_parity(values_of(out), ref, w.dtype, f"graph {name}")
        print(f"[parity] graph {name}: max_abs={rep['max_abs']:.3e} max_rel={rep['max_rel']:.3e}", flush=True)


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused_append"])
def test_whole_prompt_graph_matches_eager_and_oracle(fused):
    """A whole chunked prefill in one graph: the 4097-token prompt's nine chunks
    of at most 512 tokens (each chunk's append, then its attention over the
    prefix the earlier chunks appended), planned before capture and captured in
    order into one graph. Every replay equals the eager pass bit for bit, and
    the outputs match the oracle's full prefill."""
    w = wl.config3(4097)
    dev = torch.device("cuda", torch.cuda.current_device())
    steps = wl.chunked_steps(w, wl.chunk_partition(4097, 512))
    cache = DeviceCache(w, dev)
    batches = []
    for st in steps:
        plan = pkv.build_extend_metadata(st.prefix_lens, st.chunk_lens, shape_of(st), 0, 0, device=dev)
        kn, vn = cache._gather_new_kv(st)
        q = upload_q(st, dev)
        batches.append((plan, kn, vn, q, torch.empty_like(q), plan.workspace()))
    print(f"[graph] whole prompt, {len(batches)} chunks, fused={fused}", flush=True)

    def path():
        for plan, kn, vn, q, out, ws in batches:
            if fused:
                pkv.paged_extend_attn_append(q, kn, vn, cache.k_pool, cache.v_pool, cache.page_table, plan, out=out,
                                             workspace=ws)
            else:
                pkv.pkv_append(kn, vn, cache.k_pool, cache.v_pool, cache.page_table, plan)
                pkv.paged_extend_attn(q, cache.k_pool, cache.v_pool, cache.page_table, plan, out=out, workspace=ws)

    path()
    torch.cuda.synchronize()
    eager = torch.cat([b[4] for b in batches]).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    scratch = torch.randn(1 << 20, device=dev)
    for r in range(3):
        for b in batches:
            b[4].fill_(float("nan"))
        scratch.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = torch.cat([b[4] for b in batches])
        assert torch.equal(got, eager), f"replay {r} differs from the eager result"
    assert all(pkv.read_status(b[0]) == 0 for b in batches)
    ref = oracle_out(w, oracle_pools(w), dtype=np.float32)
    rep = assert_parity(values_of(eager), ref, "bf16", "whole-prompt graph")
    print(f"[parity] whole-prompt graph fused={fused}: max_abs={rep['max_abs']:.3e}", flush=True)
