"""paged_extend_attn_append (append + attention in one call; one launch for
bf16) against the two-call path (pkv_append, then paged_extend_attn) on the
same plan and inputs, and against the CPU oracle.

The fused gather reads the chunk's own key rows from k_new / v_new instead of
the pool slots the same launch fills, so it sees the very bytes the two-call
path reads back from the pool: outputs must agree bit for bit, and so must
every pool byte (NaN canaries in unwritten slots included). The outputs are
also held to the oracle's bar (bf16 2e-2 + 1e-2 |ref|, fp32 1e-5 + 1e-5 |ref|).
"""
import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import workloads as wl
from pkv_testlib import assert_parity, oracle_out, oracle_pools

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_chunked_prefill_amd as pkv
    from gpu_harness import DeviceCache, from_dev, shape_of, spare_page_pools, upload_q, values_of


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    assert pkv.device_supported(torch.cuda.current_device()), "not a gfx950 device"


def _bits(t: torch.Tensor) -> np.ndarray:
    a = from_dev(t)
    return a.view(np.uint16 if a.dtype == np.uint16 else np.uint32)


def fused_and_two_call(w: wl.Workload, splits: int = 0, causal: bool = True, caches=None, page_table=None):
    """One step of `w` both ways on twin caches; asserts bitwise agreement of
    outputs and pools and a clean status. Returns (fused output, caches, plan)."""
    if caches is None:
        caches = (DeviceCache(w, page_table=page_table), DeviceCache(w, page_table=page_table))
        for c in caches:
            c.fill_prefix(w)
    two, fused = caches
    plan = pkv.build_extend_metadata(w.prefix_lens, w.chunk_lens, shape_of(w), w.window, splits, device="cuda",
                                     causal=causal)
    q = upload_q(w)
    kn, vn = two._gather_new_kv(w)
    pkv.pkv_append(kn, vn, two.k_pool, two.v_pool, two.page_table, plan)
    out2 = pkv.paged_extend_attn(q, two.k_pool, two.v_pool, two.page_table, plan)
    outf = pkv.paged_extend_attn_append(q, kn, vn, fused.k_pool, fused.v_pool, fused.page_table, plan)
    torch.cuda.synchronize()
    assert pkv.read_status(plan) == 0
    assert np.array_equal(_bits(outf), _bits(out2)), "fused output differs from append + attention"
    for a, b, name in ((fused.k_pool, two.k_pool, "K"), (fused.v_pool, two.v_pool, "V")):
        x, y = _bits(a), _bits(b)
        assert np.array_equal(x, y), f"{name} pool bytes differ at {np.argwhere(x != y)[:5].tolist()}"
    return outf, caches, plan


def check_oracle(name, out, w, causal=True):
    got = values_of(out)
    assert not np.isnan(got).any(), f"{name}: NaN in output"
    rep = assert_parity(got, oracle_out(w, oracle_pools(w), causal=causal), w.dtype, name)
    print(f"[fused] {name}: max_abs={rep['max_abs']:.3e} max_rel={rep['max_rel']:.3e}", flush=True)


def small(dtype, P, L, hq, hkv, D, ps, window=0, seed=3, splits=0):
    P, L = np.array(P, np.int32), np.array(L, np.int32)
    pages = int(sum((int(n) + ps - 1) // ps for n in P + L)) + 3
    return wl.Workload("fused", 47, dtype, hq, hkv, D, ps, pages, window, P, L,
                       wl.shuffled_page_table(seed, pages, P + L, ps), decode_splits=splits)


@pytest.mark.parametrize("dtype,P,L,hq,hkv,D,ps,window,splits", [
    ("bf16", [0, 100, 513, 1025], [1, 64, 128, 512], 32, 8, 128, 16, 0, 0),   # ragged; prefixes end mid copy
    ("bf16", [3, 70], [200, 61], 4, 4, 128, 16, 0, 0),    # G=1: 256-token tiles, owned rows past the prologue's
    ("bf16", [5], [250], 8, 4, 64, 64, 0, 0),             # G=2 at D=64: exactly the prologue's share
    ("bf16", [37, 0], [90, 33], 16, 4, 128, 3, 0, 0),      # page size 3 (per-lane page ids)
    ("bf16", [9, 130], [77, 5], 16, 4, 128, 2, 0, 0),      # page size 2 < rows per copy
    ("bf16", [0, 6001], [300, 700], 32, 8, 128, 16, 256, 0),   # window
    ("bf16", [2047, 3000, 17], [1, 1, 1], 64, 8, 128, 16, 0, 8),   # one-token rows, 8 splits
    ("bf16", [800, 5, 0], [1, 0, 129], 16, 4, 128, 64, 0, 0),      # an empty chunk between rows
    ("fp32", [20, 47], [45, 33], 4, 2, 64, 16, 0, 0),     # fp32: the append kernel then the attention
    # every prefix a multiple of 8: no 4- or 8-row gather copy straddles P_b
    ("bf16", [0, 512, 1024], [64, 128, 512], 32, 8, 128, 16, 0, 0),
    ("bf16", [64, 8, 0], [100, 1, 77], 8, 2, 64, 64, 0, 3),
    ("bf16", [4096, 16], [300, 40], 16, 4, 128, 16, 1000, 0),
    ("bf16", [0], [700], 4, 4, 128, 64, 0, 0),            # aligned, G=1: owned rows past the prologue's
])
def test_fused_matches_two_calls_and_oracle(dtype, P, L, hq, hkv, D, ps, window, splits):
    w = small(dtype, P, L, hq, hkv, D, ps, window, splits=splits)
    out, _, _ = fused_and_two_call(w, splits)
    check_oracle(f"{dtype} P={P} L={L} {hq}/{hkv} D={D} ps={ps} W={window} S={splits}", out, w)


@pytest.mark.parametrize("P,L,hq,hkv,D,ps,window", [
    ([0], [512], 16, 4, 128, 64, 0),          # the 4097-token prompt's first 512-token chunk
    ([1024], [512], 16, 4, 128, 64, 0),       # padding items between real ones
    ([2048], [128], 16, 4, 128, 64, 0),       # 17 pieces per tile
    ([0], [512], 8, 2, 64, 16, 0),            # D = 64
    ([3000], [1000], 32, 4, 128, 16, 0),      # G = 8, runs of two pieces, padding
    ([1500, 0], [300, 200], 16, 2, 64, 16, 0),   # two requests in one stream
    ([0], [1536], 32, 8, 128, 16, 0),         # 8 KV heads (one XCD each), runs of several pieces
    ([0], [512], 16, 4, 128, 16, 128),        # sliding window: pieces start inside the window, padding
    ([500], [300], 16, 4, 128, 16, 1000),     # window reaching into the prefix, padding
    ([0], [1024], 16, 2, 64, 16, 256),        # window at D = 64
])
def test_stream_plans(P, L, hq, hkv, D, ps, window):
    """Plans whose work list is cut end to end per KV head (stream plans, with
    runs of several pieces and padding items): fused and two-call paths agree
    bit for bit and match the oracle; the automatic plan is a stream plan, i.e.
    differs from the equal cuts that an explicit split count selects."""
    w = small("bf16", P, L, hq, hkv, D, ps, window)
    Pa, La, s = np.array(P, np.int32), np.array(L, np.int32), shape_of(w)
    auto = pkv.build_extend_metadata(Pa, La, s, window, 0, num_cus=256).host_sections()["items"]
    equal = pkv.build_extend_metadata(Pa, La, s, window, 1, num_cus=256).host_sections()["items"]
    assert len(auto) != len(equal) or not np.array_equal(auto, equal), "expected a stream plan"
    out, _, _ = fused_and_two_call(w)
    check_oracle(f"stream plan P={P} L={L} {hq}/{hkv} D={D} ps={ps} W={window}", out, w)


@pytest.mark.parametrize("P,L,hq,hkv,D", [([100, 37, 0], [64, 200, 1], 16, 4, 128), ([0], [300], 8, 8, 64)])
def test_fused_non_causal(P, L, hq, hkv, D):
    w = small("bf16", P, L, hq, hkv, D, 16, seed=7)
    out, _, _ = fused_and_two_call(w, causal=False)
    check_oracle(f"non-causal P={P} L={L}", out, w, causal=False)


@pytest.mark.parametrize("budget,first", [(512, None), (2048, 2047), (128, 127)])
def test_fused_chunked_prompt(budget, first):
    """The 4097-token prompt prefilled chunk by chunk with the fused call, the
    pool filled by the fused launches only (first chunk of budget-1 tokens:
    every later chunk starts mid-page and mid-copy)."""
    w = wl.config3(4097)
    caches = (DeviceCache(w), DeviceCache(w))
    for step in wl.chunked_steps(w, wl.chunk_partition(4097, budget, first)):
        fused_and_two_call(step, caches=caches)
    kp, vp = oracle_pools(w)
    for dev, ref in zip((caches[1].k_pool, caches[1].v_pool), (kp, vp)):
        x = _bits(dev)
        y = ref.view(x.dtype)
        assert np.array_equal(x, y), "pool after the fused prefill differs from the oracle's append"


@settings(max_examples=25, deadline=None, derandomize=True, database=None)
@given(st.data())
def test_fused_random(data):
    """Random small batches (a fixed, derandomized set) both ways."""
    dtype = data.draw(st.sampled_from(["bf16", "bf16", "bf16", "fp32"]))
    D = data.draw(st.sampled_from([64, 128]))
    B = data.draw(st.integers(1, 4))
    P = data.draw(st.lists(st.integers(0, 700), min_size=B, max_size=B))
    if data.draw(st.booleans()):
        P = [8 * (x // 8) for x in P]     # aligned prefixes: no gather copy straddles P_b
    L = data.draw(st.lists(st.sampled_from([0, 1, 1, 3, 16, 33, 64, 100, 257]), min_size=B, max_size=B))
    if sum(L) == 0:
        L[0] = 1
    hkv = data.draw(st.sampled_from([1, 2, 4]))
    hq = hkv * data.draw(st.sampled_from([1, 2, 4, 8]))
    ps = data.draw(st.sampled_from([1, 3, 4, 16, 64]))
    window = data.draw(st.sampled_from([0, 0, 1, 50]))
    splits = data.draw(st.sampled_from([0, 0, 2, 7]))
    seed = data.draw(st.integers(0, 1000))
    w = small(dtype, P, L, hq, hkv, D, ps, window, seed=seed, splits=splits)
    out, _, _ = fused_and_two_call(w, splits)
    check_oracle(f"random {dtype} D={D} {hq}/{hkv} ps={ps} W={window} S={splits} P={P} L={L}", out, w)


def test_long_launch_takes_the_append_kernel():
    """A plan whose busiest slot streams more than 128 key blocks (16 requests
    of 8000 cached + 256 new tokens: 512 items of about 130 blocks): the call
    runs the append kernel and the plain attention, with the same bits as the
    two calls."""
    w = small("bf16", [8000] * 16, [256] * 16, 32, 8, 128, 64, seed=11)
    plan = pkv.build_extend_metadata(w.prefix_lens, w.chunk_lens, shape_of(w), 0, 0, device="cuda")
    assert plan.plan.slot_blocks > 128
    fused_and_two_call(w)


def test_fused_bad_page_is_flagged_and_not_written():
    """A new position whose page id lies just past the pool (inside a spare,
    sentinel-filled allocation): the status word says so and no pool byte is
    written for it (the two-call path skips it too); the spare pages keep their
    sentinels, so a failed guard would show as changed bytes, not a fault."""
    P, L = np.array([32], np.int32), np.array([32], np.int32)
    w = wl.Workload("bad", 45, "bf16", 8, 2, 128, 16, 16, 0, P, L, wl.shuffled_page_table(45, 16, P + L, 16))
    bad = w.page_table.copy()
    bad[0, 3] = 20                            # positions 48..63: past the declared 16 pages
    pools = []
    for _ in range(2):
        c = DeviceCache(w)
        c.fill_prefix(w)
        c.page_table = torch.from_numpy(np.ascontiguousarray(bad, np.int32)).cuda()
        (kbig, kp), (vbig, vp) = spare_page_pools(c)
        c.k_pool, c.v_pool = kp, vp
        pools.append((c, kbig, vbig))
    (two, two_kbig, two_vbig), (fused, fused_kbig, fused_vbig) = pools
    plan = pkv.build_extend_metadata(P, L, shape_of(w), 0, 0, device="cuda")
    q = upload_q(w)
    kn, vn = two._gather_new_kv(w)
    pkv.pkv_append(kn, vn, two.k_pool, two.v_pool, two.page_table, plan)
    torch.cuda.synchronize()
    assert pkv.read_status(plan) == pkv.PKV_STATUS_BAD_PAGE
    plan2 = pkv.build_extend_metadata(P, L, shape_of(w), 0, 0, device="cuda")
    out = pkv.paged_extend_attn_append(q, kn, vn, fused.k_pool, fused.v_pool, fused.page_table, plan2)
    torch.cuda.synchronize()
    assert pkv.read_status(plan2) == pkv.PKV_STATUS_BAD_PAGE
    assert not torch.isnan(out.float()).any()
    for a, b in ((fused_kbig, two_kbig), (fused_vbig, two_vbig)):
        assert np.array_equal(_bits(a), _bits(b))
    for kbig, vbig in ((two_kbig, two_vbig), (fused_kbig, fused_vbig)):
        assert bool((kbig[16:] == 1.0).all()) and bool((vbig[16:] == 16384.0).all()), "a spare page was written"


def test_fused_rejects_overlap_and_null():
    w = small("bf16", [4], [8], 8, 2, 128, 16)
    c = DeviceCache(w)
    plan = pkv.build_extend_metadata(w.prefix_lens, w.chunk_lens, shape_of(w), 0, 0, device="cuda")
    q = upload_q(w)
    kn = c.k_pool.view(-1)[: w.total_q * 2 * 128].view(w.total_q, 2, 128)   # inside the K pool
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_extend_attn_append(q, kn, kn, c.k_pool, c.v_pool, c.page_table, plan)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARGUMENT
