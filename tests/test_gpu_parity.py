"""Parity of the HIP path (called through the C ABI via the Python binding)
with the CPU oracle, on the seeded workloads: element by element at sizes the
oracle finishes in seconds, on sampled rows at full size.

Bar: bf16 |gpu - ref| <= 2e-2 + 1e-2 |ref|, fp32 <= 1e-5 + 1e-5 |ref|, against
the fp32 oracle; page-table and indptr handling bit-exact (append compared
bytewise, NaN canaries included)."""
import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
import workloads as wl
from pkv_testlib import assert_parity, oracle_out, oracle_pools

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_chunked_prefill_amd as pkv
    from gpu_harness import (DeviceCache, chunked_prefill, from_dev, prefill_and_attend, run_attention, shape_of,
                             spare_page_pools, upload_q, values_of)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    assert pkv.device_supported(torch.cuda.current_device()), "not a gfx950 device"


def report(name, rep):
    print(f"[parity] {name}: max_abs={rep['max_abs']:.3e} max_rel={rep['max_rel']:.3e}", flush=True)


def check(name, out, ref, dtype):
    got = values_of(out) if isinstance(out, torch.Tensor) else out
    assert not np.isnan(got).any(), f"{name}: NaN in output"
    report(name, assert_parity(got, ref, dtype, name))


def oracle_request_rows(w: wl.Workload, b: int, rows, dtype=np.float32):
    """Oracle output of chunk rows `rows` (0-based within request b's chunk) of
    one request, from a compact pool holding only that request's pages."""
    P, L = int(w.prefix_lens[b]), int(w.chunk_lens[b])
    n = P + L
    npg = (n + w.page_size - 1) // w.page_size
    one = wl.Workload(w.name, w.config_id, w.dtype, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, npg,
                      w.window, np.array([P], np.int32), np.array([L], np.int32),
                      np.arange(npg, dtype=np.int32)[None], request_ids=np.array([w.rid(b)]),
                      data_scale=w.data_scale, zero_q=w.zero_q, ramp_v=w.ramp_v, ramp_v_step=w.ramp_v_step)
    k, v = w.kv_seq(b, storage=True)
    kp, vp = one.empty_pool(), one.empty_pool()
    kp, vp = oracle.append_kv(kp, vp, k, v, one.page_table, [0], [n])
    return oracle_out(one, (kp, vp), dtype=dtype, rows=list(rows))[list(rows)]


# ---------------------------------------------------------------------------
# append (bit-exact)
# ---------------------------------------------------------------------------

def pools_equal_bytes(cache, pools):
    for dev, ref in zip((cache.k_pool, cache.v_pool), pools):
        got = from_dev(dev)
        a = got.view(np.uint16 if got.dtype == np.uint16 else np.uint32)
        b = ref.view(np.uint16 if ref.dtype == np.uint16 else np.uint32)
        assert np.array_equal(a, b), f"pool bytes differ at {np.argwhere(a != b)[:5].tolist()}"


def test_canary_bits_match():
    t = torch.full((4,), float("nan"), dtype=torch.bfloat16, device="cuda")
    assert (from_dev(t) == wl.nan_fill("bf16")).all()


def test_append_bitexact_ragged():
    w = wl.config2()
    cache = DeviceCache(w)
    cache.fill_prefix(w)
    cache.append_step(w)
    torch.cuda.synchronize()
    pools_equal_bytes(cache, oracle_pools(w))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_append_bitexact_mid_page(dtype):
    P = np.array([6001 + 2 * b for b in range(8)], np.int32)
    L = np.array([3, 17, 1, 0, 33, 16, 2, 64], np.int32)
    pt = wl.shuffled_page_table(40, 4096, P + L, 16)
    w = wl.Workload("mid-page", 40, dtype, 8, 2, 64, 16, 4096, 0, P, L, pt)
    cache = DeviceCache(w)
    cache.fill_prefix(w)
    cache.append_step(w)
    torch.cuda.synchronize()
    pools_equal_bytes(cache, oracle_pools(w))


# ---------------------------------------------------------------------------
# config 1 (fp32): parity at 1e-5, zero-score closed form, partitions
# ---------------------------------------------------------------------------

def test_config1_fp32():
    w = wl.config1()
    out, cache, plan = prefill_and_attend(w)
    check("config1", out, oracle_out(w, oracle_pools(w)), "fp32")


@pytest.mark.parametrize("chunks", [[64], [48, 16], [16, 16, 16, 16], [1] * 64, [15, 33, 16]])
def test_config1_zero_score_exact(chunks):
    w = wl.config1(zero_score=True).with_lengths([0], [64])
    out, _ = chunked_prefill(w, chunks)
    t = np.arange(64, dtype=np.float32)
    want = np.broadcast_to(((t + 2) / 2)[:, None, None], (64, 2, 64))
    assert np.array_equal(values_of(out), want)


@pytest.mark.parametrize("chunks", [[16, 16, 16, 16], [1] * 64, [48, 16]])
def test_config1_partitions_match_full_prefill(chunks):
    w = wl.config1().with_lengths([0], [64])
    full, _ = chunked_prefill(w, [64])
    part, _ = chunked_prefill(w, chunks)
    ref = oracle_out(w, oracle_pools(w))
    check(f"config1 full", full, ref, "fp32")
    check(f"config1 {chunks[:3]}..", part, ref, "fp32")
    bitwise = torch.equal(full, part)
    print(f"[parity] config1 partition {len(chunks)} chunks bitwise-equal to full prefill: {bitwise}")


def test_zero_score_page_literal_bf16():
    """The PR's regression numbers on the bf16 path: [1,2,3,4] across two chunks of two."""
    w = wl.Workload("literal", 41, "bf16", 8, 8, 128, 2, 8, 0, np.array([0], np.int32), np.array([4], np.int32),
                    np.array([[5, 2, 7, 0]], np.int32), zero_q=True, ramp_v=True, ramp_v_step=2.0)
    out, _ = chunked_prefill(w, [2, 2])
    assert np.array_equal(values_of(out)[:, 0, 0], np.array([1, 2, 3, 4], np.float32))
    assert np.array_equal(values_of(out), np.broadcast_to(np.array([1, 2, 3, 4], np.float32)[:, None, None],
                                                          (4, 8, 128)))


# ---------------------------------------------------------------------------
# config 2 (ragged bf16, NaN canaries)
# ---------------------------------------------------------------------------

def test_config2_ragged():
    w = wl.config2()
    out, cache, plan = prefill_and_attend(w)
    check("config2", out, oracle_out(w, oracle_pools(w)), "bf16")
    assert pkv.read_status(plan) == 0


def test_page_permutation_invariance_bitwise():
    w = wl.config2()
    out1, _, _ = prefill_and_attend(w)
    pt2 = wl.shuffled_page_table(999, w.num_pages, w.kv_lens, w.page_size)
    w2 = wl.Workload(**{**w.__dict__, "page_table": pt2})
    out2, _, _ = prefill_and_attend(w2)
    assert torch.equal(out1, out2)


# ---------------------------------------------------------------------------
# config 3 (long prompt, chunk budgets)
# ---------------------------------------------------------------------------

_REF3 = {}


def ref3(prompt):
    if prompt not in _REF3:
        w = wl.config3(prompt)
        _REF3[prompt] = oracle_out(w, oracle_pools(w))
    return _REF3[prompt]


@pytest.mark.parametrize("prompt", [4097, 8193])
@pytest.mark.parametrize("budget,first", [(2048, None), (512, None), (128, None), (512, 511), (None, None)])
def test_config3_chunked_matches_full(prompt, budget, first):
    w = wl.config3(prompt)
    chunks = [prompt] if budget is None else wl.chunk_partition(prompt, budget, first)
    out, _ = chunked_prefill(w, chunks)
    check(f"config3 {prompt} budget={budget} first={first}", out, ref3(prompt), "bf16")


@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_split_partials_precision(q_scale):
    """Split items keep their unnormalised partial outputs in bf16 (fp32 max and
    sum). The 4097-token prompt under 512-token chunks, planned for 256 compute
    units (every chunk's tiles split up to 8 ways) and for 1 (nothing split),
    both held to the bar against the oracle; with q scaled by 8 the softmax is
    far more peaked (scores of tens of units: each row is dominated by a few
    keys). Prints max |split - unsplit|."""
    w = wl.config3(4097)
    chunks = wl.chunk_partition(4097, 512)
    qv = wl.values(w.q_all(), "bf16") * np.float32(q_scale)
    q_bits = wl.to_storage(qv, "bf16")
    q_full = torch.from_numpy(q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    split, _ = chunked_prefill(w, chunks, num_cus=256, q_full=q_full)
    whole, _ = chunked_prefill(w, chunks, num_cus=1, q_full=q_full)
    kp, vp = oracle_pools(w)
    ref = oracle.extend_attention(wl.values(q_bits, "bf16"), wl.values(kp, "bf16"), wl.values(vp, "bf16"),
                                  w.page_table, w.prefix_lens, w.chunk_lens)
    check(f"prompt 4097/512 q x{q_scale:g} split partials", split, ref, "bf16")
    check(f"prompt 4097/512 q x{q_scale:g} unsplit", whole, ref, "bf16")
    d = (split.float() - whole.float()).abs()
    print(f"[parity] prompt 4097/512 q x{q_scale:g}: max |split - unsplit| = {float(d.max()):.3e} "
          f"(mean {float(d.mean()):.3e})", flush=True)


@pytest.mark.parametrize("case,window,spike,q_scale", [
    ("keys x40 at 1000..1015", 0, (1000, 1016, 40.0), 1.0),
    ("keys x40 inside a window", 600, (1900, 1916, 40.0), 1.0),
    ("q x8, window", 300, None, 8.0),
])
def test_reference_raised_on_large_scores(case, window, spike, q_scale):
    """Scores that jump far past a row's reference after its first tiles: a
    block of 16 keys scaled by 40 (their weights against the old reference
    overflow to inf before the tile is caught), or q scaled by 8 under a
    sliding window (a row's first tile holds few of its keys, so its reference
    starts low and later tiles' weights sum past the catch limit). A 2048 + 512
    request, split over the GPU; the plain launch (append kernel first) and the
    fused one against the oracle, and bitwise equal to each other."""
    P, L = np.array([2048], np.int32), np.array([512], np.int32)
    pages = 200
    w = wl.Workload("large scores", 47, "bf16", 16, 4, 128, 64, pages, window, P, L,
                    wl.shuffled_page_table(47, pages, P + L, 64))
    kp, vp = oracle_pools(w)
    slots = []
    if spike is not None:
        lo, hi, factor = spike
        for pos in range(lo, hi):   # prefix positions: written by fill_prefix
            page, slot = int(w.page_table[0][pos // 64]), pos % 64
            kp[page, slot] = wl.to_storage(wl.values(kp[page, slot], "bf16") * np.float32(factor), "bf16")
            slots.append((page, slot))
    qv = wl.values(w.q_all(), "bf16") * np.float32(q_scale)
    q_bits = wl.to_storage(qv, "bf16")
    ref = oracle.extend_attention(wl.values(q_bits, "bf16"), wl.values(kp, "bf16"), wl.values(vp, "bf16"),
                                  w.page_table, w.prefix_lens, w.chunk_lens, window=window)

    def cache_with_spike():
        c = DeviceCache(w)
        c.fill_prefix(w)
        for page, slot in slots:
            c.k_pool[page, slot] = torch.from_numpy(kp[page, slot].view(np.int16).copy()).cuda().view(torch.bfloat16)
        return c

    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    c1 = cache_with_spike()
    plan = c1.append_step(w)
    assert plan.plan.n_split_rows > 0, "expected split items"
    plain = pkv.paged_extend_attn(q, c1.k_pool, c1.v_pool, c1.page_table, plan)
    c2 = cache_with_spike()
    fplan = pkv.build_extend_metadata(P, L, shape_of(w), window, 0, device="cuda")
    kn, vn = c2._gather_new_kv(w)
    fused = pkv.paged_extend_attn_append(q, kn, vn, c2.k_pool, c2.v_pool, c2.page_table, fplan)
    torch.cuda.synchronize()
    assert fplan.plan.slot_blocks <= 128, "expected the fused launch"
    check(f"large scores, {case}: plain", plain, ref, "bf16")
    check(f"large scores, {case}: fused", fused, ref, "bf16")
    assert torch.equal(plain.view(torch.int16), fused.view(torch.int16)), "plain and fused launches differ"


# configs 4 and 5 at full size: every row, in test_gpu_full_size.py


def test_budget_steps_decode_rows_and_chunks():
    """A prompt prefilled under a step budget shared with ongoing decodes: every
    step's one-token rows and prompt chunk against the oracle at that step's
    lengths (the pools hold all positions; each row reads only its visible ones)."""
    w, steps = wl.budget_steps(prompt=700, budget=160, n_decode=8)
    pools = oracle_pools(w)
    cache = DeviceCache(w)
    cache.fill_prefix(w)
    for s_, st in enumerate(steps):
        out, plan = run_attention(cache, st, decode_splits=0)
        ref = oracle_out(st, pools)
        check(f"budget step {s_} ({int(st.chunk_lens[-1])}-token chunk at {int(st.prefix_lens[-1])})",
              out, ref, "bf16")


@pytest.mark.parametrize("dtype,P,L,hq,hkv,D", [
    ("bf16", [0, 0], [256, 128], 32, 4, 128),          # the pages' non-causal case: q_len = kv_len
    ("bf16", [100, 37, 0], [64, 200, 1], 16, 4, 128),  # extend: rows also see the chunk rows after them
    ("bf16", [0], [300], 8, 8, 64),
    ("fp32", [20, 0], [45, 33], 4, 2, 64)])
def test_non_causal(dtype, P, L, hq, hkv, D):
    P, L = np.array(P, np.int32), np.array(L, np.int32)
    ps = 16
    pages = int(sum((int(n) + ps - 1) // ps for n in P + L)) + 4
    pt = wl.shuffled_page_table(7, pages, P + L, ps)
    w = wl.Workload("noncausal", 7, dtype, hq, hkv, D, ps, pages, 0, P, L, pt)
    cache = DeviceCache(w)
    cache.fill_prefix(w)
    plan = pkv.build_extend_metadata(P, L, shape_of(w), 0, 0, device="cuda", causal=False)
    kn, vn = cache._gather_new_kv(w)
    pkv.pkv_append(kn, vn, cache.k_pool, cache.v_pool, cache.page_table, plan)
    out = pkv.paged_extend_attn(upload_q(w), cache.k_pool, cache.v_pool, cache.page_table, plan)
    check(f"non-causal {dtype} D={D} P={P.tolist()} L={L.tolist()}", out, oracle_out(w, oracle_pools(w), causal=False),
          dtype)


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 8, 12, 0])
def test_decode_splits_agree(splits):
    w = wl.config5(decode_only=True).subset(range(6))
    out, _, plan = prefill_and_attend(w, decode_splits=splits)
    got = values_of(out)
    for b in range(6):
        check(f"decode splits={splits} req {b}", got[[b]], oracle_request_rows(w, b, [0]), "bf16")


def test_split_zero_score_exact():
    P = np.array([999, 2047, 77], np.int32)
    L = np.ones(3, np.int32)
    w = wl.Workload("zs-split", 42, "fp32", 4, 2, 64, 16, 512, 0, P, L,
                    wl.shuffled_page_table(42, 512, P + L, 16), zero_q=True, ramp_v=True, decode_splits=8)
    out, _, plan = prefill_and_attend(w)
    assert plan.plan.n_split_rows == 3
    want = (P.astype(np.float32) + 2) / 2          # mean of 1..N
    assert np.array_equal(values_of(out)[:, 0, 0], want)


# ---------------------------------------------------------------------------
# edge cases and variants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,D,hq,hkv,ps,window", [
    ("bf16", 64, 4, 4, 1, 0), ("bf16", 128, 6, 2, 3, 0), ("bf16", 64, 12, 4, 7, 33), ("fp32", 128, 4, 1, 16, 0),
    ("fp32", 64, 3, 3, 5, 10), ("bf16", 128, 16, 1, 64, 100), ("bf16", 128, 8, 8, 128, 0),
    ("bf16", 128, 32, 2, 256, 57), ("bf16", 64, 128, 1, 16, 0), ("bf16", 128, 6, 3, 2, 0)])
def test_variants(dtype, D, hq, hkv, ps, window):
    P = np.array([0, 37, 0, 130, 64], np.int32)
    L = np.array([70, 0, 1, 45, 129], np.int32)
    pages = int(sum((int(n) + ps - 1) // ps for n in P + L)) + 5
    w = wl.Workload(f"variant", 43, dtype, hq, hkv, D, ps, pages, window, P, L,
                    wl.shuffled_page_table(43, pages, P + L, ps))
    out, _, _ = prefill_and_attend(w)
    check(f"variant {dtype} D={D} {hq}/{hkv} ps={ps} W={window}", out, oracle_out(w, oracle_pools(w)), dtype)


@pytest.mark.parametrize("D,hq,hkv,ps", [(128, 6, 2, 16), (64, 12, 4, 7), (128, 40, 8, 16)])
def test_split_partials_odd_group(D, hq, hkv, ps):
    """Split items whose GQA group does not divide the 4-row pieces of the
    output store (G = 3 and 5): the partial rows (token x query head) of every
    split land where the combine reads them."""
    P = np.array([1500, 700, 0], np.int32)
    L = np.array([40, 90, 33], np.int32)
    pages = int(sum((int(n) + ps - 1) // ps for n in P + L)) + 5
    w = wl.Workload("odd-group splits", 44, "bf16", hq, hkv, D, ps, pages, 0, P, L,
                    wl.shuffled_page_table(44, pages, P + L, ps))
    out, _, plan = prefill_and_attend(w)
    assert plan.plan.n_split_rows > 0 and plan.plan.max_splits > 1, "expected split rows"
    check(f"odd-group splits D={D} {hq}/{hkv} ps={ps}", out, oracle_out(w, oracle_pools(w)), "bf16")


# Short chunks and one-token rows whose rows all fit one 16-row block
# (max_q_len * G <= 16), with splits, windows and small pages.
@pytest.mark.parametrize("hq,hkv,ps,P,L,window,splits", [
    (8, 2, 16, [0, 37, 500, 130, 64], [1, 1, 1, 4, 2], 0, 0),
    (4, 4, 64, [0, 100, 999, 63], [16, 3, 1, 16], 0, 0),
    (16, 2, 4, [77, 0, 300], [2, 1, 2], 50, 0),
    (16, 1, 16, [1000, 5], [1, 1], 0, 5),
    (4, 2, 32, [0, 129, 64, 7], [8, 5, 1, 0], 0, 3),
    (8, 2, 64, [4095, 1, 2000], [1, 4, 3], 130, 12),
    (4, 1, 8, [0, 0], [4, 1], 0, 0),
])
def test_one_block_items(hq, hkv, ps, P, L, window, splits):
    P, L = np.array(P, np.int32), np.array(L, np.int32)
    assert int(L.max()) * (hq // hkv) <= 16
    pages = int(sum((int(n) + ps - 1) // ps for n in P + L)) + 3
    w = wl.Workload("one-block", 44, "bf16", hq, hkv, 128, ps, pages, window, P, L,
                    wl.shuffled_page_table(44, pages, P + L, ps), decode_splits=splits)
    out, _, plan = prefill_and_attend(w)
    assert pkv.read_status(plan) == 0
    check(f"one-block G={hq // hkv} ps={ps} L={L.tolist()} W={window} splits={splits}", out,
          oracle_out(w, oracle_pools(w)), "bf16")


def test_one_block_zero_score_exact():
    """Zero scores on one-token rows with splits: every output is the mean of the values 1..N."""
    P = np.array([999, 2047, 77, 0], np.int32)
    L = np.array([1, 1, 1, 1], np.int32)
    w = wl.Workload("zs-one-block", 45, "bf16", 8, 2, 128, 16, 512, 0, P, L,
                    wl.shuffled_page_table(45, 512, P + L, 16), zero_q=True, ramp_v=True, decode_splits=4)
    out, _, plan = prefill_and_attend(w)
    want = (P.astype(np.float64) + 2) / 2          # mean of 1..N
    got = values_of(out)[:, :, :]
    ref = np.broadcast_to(want[:, None, None], got.shape)
    check("one-block zero scores", out, ref.astype(np.float32), "bf16")


@settings(max_examples=40, deadline=None, derandomize=True, database=None)
@given(st.data())
def test_random_batches(data):
    """Random small batches (a fixed, derandomized set): ragged prefixes and
    chunks (empty chunks and one-token rows among them), bf16 or fp32, D 64 or
    128, GQA groups, page sizes, windows and split counts, against the oracle."""
    dtype = data.draw(st.sampled_from(["bf16", "bf16", "fp32"]))
    D = data.draw(st.sampled_from([64, 128]))
    B = data.draw(st.integers(1, 4))
    P = np.array(data.draw(st.lists(st.integers(0, 700), min_size=B, max_size=B)), np.int32)
    L = np.array(data.draw(st.lists(st.sampled_from([0, 1, 1, 3, 16, 33, 64, 100]), min_size=B, max_size=B)),
                 np.int32)
    if int(L.sum()) == 0:
        L[0] = 1
    hkv = data.draw(st.sampled_from([1, 2, 4]))
    hq = hkv * data.draw(st.sampled_from([1, 2, 4, 8]))
    ps = data.draw(st.sampled_from([1, 4, 16, 64]))
    window = data.draw(st.sampled_from([0, 0, 1, 50]))
    splits = data.draw(st.sampled_from([0, 0, 2, 7]))
    seed = data.draw(st.integers(0, 1000))
    pages = int(sum((int(n) + ps - 1) // ps for n in P + L)) + 2
    w = wl.Workload("random", 46, dtype, hq, hkv, D, ps, pages, window, P, L,
                    wl.shuffled_page_table(seed, pages, P + L, ps), decode_splits=splits)
    out, _, plan = prefill_and_attend(w)
    assert pkv.read_status(plan) == 0
    check(f"random {dtype} D={D} {hq}/{hkv} ps={ps} W={window} splits={splits} P={P.tolist()} L={L.tolist()}",
          out, oracle_out(w, oracle_pools(w)), dtype)


def test_one_row_longest_range_most_splits():
    """One token after 131071 cached keys, split the most ways the ABI allows
    (32), next to a short row: sampled against the oracle row by row."""
    P = np.array([131071, 9], np.int32)
    L = np.ones(2, np.int32)
    pages = int(sum((int(n) + 15) // 16 for n in P + L))
    w = wl.Workload("long1", 47, "bf16", 8, 2, 128, 16, pages, 0, P, L,
                    wl.shuffled_page_table(47, pages, P + L, 16), decode_splits=pkv.PKV_MAX_SPLITS)
    out, _, plan = prefill_and_attend(w)
    assert plan.plan.max_splits == pkv.PKV_MAX_SPLITS
    got = values_of(out)
    for b in range(2):
        check(f"long row N={int(P[b]) + 1} splits=32 req {b}", got[[b]], oracle_request_rows(w, b, [0]), "bf16")


def test_window_with_split_tiles():
    """A window and KV splits together (few long tiles: the planner cuts them)."""
    P, L = np.array([3000], np.int32), np.array([300], np.int32)
    pages = (3300 + 15) // 16
    w = wl.Workload("wsplit", 48, "bf16", 16, 4, 128, 16, pages, 700, P, L,
                    wl.shuffled_page_table(48, pages, P + L, 16))
    out, _, plan = prefill_and_attend(w)
    assert plan.plan.n_split_rows > 0
    check("window 700 + splits", out, oracle_out(w, oracle_pools(w)), "bf16")


def test_many_requests_more_items_than_slots():
    """1000 one-token requests of assorted lengths: more work items than the
    GPU has workgroup slots, each item's request resolved from its record."""
    rng = np.random.default_rng(49)
    P = rng.integers(0, 700, 1000).astype(np.int32)
    L = np.ones(1000, np.int32)
    pages = int(sum((int(n) + 15) // 16 for n in P + L))
    w = wl.Workload("many", 49, "bf16", 8, 4, 64, 16, pages, 0, P, L, wl.shuffled_page_table(49, pages, P + L, 16))
    out, _, plan = prefill_and_attend(w)
    assert plan.plan.n_items > 256
    got = values_of(out)
    for b in (0, 1, 499, 998, 999):
        check(f"many req {b}", got[[b]], oracle_request_rows(w, b, [0]), "bf16")


def test_req_pool_indices_and_scale():
    w = wl.config2()
    out_ref, cache, plan = prefill_and_attend(w, decode_splits=0)
    # the same requests stored in permuted page-table rows
    perm = np.array([2, 0, 3, 1], np.int32)
    pt_rows = np.full((4, w.page_table.shape[1]), -1, np.int32)
    pt_rows[perm] = w.page_table
    rpi = torch.from_numpy(perm).cuda()
    table = torch.from_numpy(pt_rows).cuda()
    q = upload_q(w)
    out = pkv.paged_extend_attn(q, cache.k_pool, cache.v_pool, table, plan, req_pool_indices=rpi)
    assert torch.equal(out, out_ref)
    out_s = pkv.paged_extend_attn(q, cache.k_pool, cache.v_pool, cache.page_table, plan, sm_scale=0.3)
    check("config2 sm_scale=0.3", out_s, oracle_out(w, oracle_pools(w), sm_scale=0.3), "bf16")


def test_window_one_is_own_value_bitwise():
    P, L = np.array([40], np.int32), np.array([24], np.int32)
    w = wl.Workload("w1", 44, "bf16", 8, 2, 128, 16, 8, 1, P, L, wl.shuffled_page_table(44, 8, P + L, 16))
    out, _, _ = prefill_and_attend(w)
    v = w.kv_seq(0, storage=True)[1][40:64]
    assert np.array_equal(from_dev(out), np.repeat(v, 4, axis=1))


def test_bad_page_id_is_flagged_not_read():
    """A page id just past the pool (inside a spare, sentinel-filled allocation):
    flagged, never read. Were it read, its V rows of 16384 would dominate the
    output."""
    P, L = np.array([32], np.int32), np.array([32], np.int32)
    w = wl.Workload("bad", 45, "bf16", 8, 2, 128, 16, 16, 0, P, L, wl.shuffled_page_table(45, 16, P + L, 16))
    cache = DeviceCache(w)
    cache.fill_prefix(w)
    plan = cache.append_step(w)
    torch.cuda.synchronize()
    assert pkv.read_status(plan) == 0
    (kbig, kp), (vbig, vp) = spare_page_pools(cache)
    bad = w.page_table.copy()
    bad[0, 1] = 20                            # past the declared 16 pages: must never be dereferenced
    table = torch.from_numpy(bad).cuda()
    out = pkv.paged_extend_attn(upload_q(w), kp, vp, table, plan)
    torch.cuda.synchronize()
    assert pkv.read_status(plan) == pkv.PKV_STATUS_BAD_PAGE
    o = out.float()
    assert not torch.isnan(o).any()
    assert float(o.abs().max()) < 100.0, "a sentinel V row reached the output"
    assert bool((kbig[16:] == 1.0).all()) and bool((vbig[16:] == 16384.0).all())


def test_empty_chunks_only():
    P, L = np.array([5, 9], np.int32), np.array([0, 0], np.int32)
    w = wl.Workload("empty", 46, "bf16", 4, 2, 64, 16, 4, 0, P, L, wl.shuffled_page_table(46, 4, P + L, 16))
    cache = DeviceCache(w)
    plan = cache.append_step(w)
    q = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    out = pkv.paged_extend_attn(q, cache.k_pool, cache.v_pool, cache.page_table, plan)
    torch.cuda.synchronize()
    assert out.shape == (0, 4, 64)


# ---------------------------------------------------------------------------
# explicit keep-mask (paged_extend_attn_masked)
# ---------------------------------------------------------------------------

def _masked_case(dtype, P, L, hq, hkv, D, ps, mh, mr, causal, seed, p_keep=0.6, splits=0, empty_row=None):
    P, L = np.array(P, np.int32), np.array(L, np.int32)
    pages = int(sum((int(n) + ps - 1) // ps for n in P + L)) + 4
    pt = wl.shuffled_page_table(seed, pages, P + L, ps)
    w = wl.Workload("masked", 8, dtype, hq, hkv, D, ps, pages, 0, P, L, pt)
    ks = int(((P + L).max() + 3) // 4 * 4) + 4
    rows = 1 if mr == 1 else int(L.max())
    rng = np.random.default_rng(seed)
    m = (rng.random((len(L), mh, rows, ks)) < p_keep).astype(np.uint8)
    if empty_row is not None:
        b, h, i = empty_row
        m[b, h, i] = 0
    cache = DeviceCache(w)
    cache.fill_prefix(w)
    plan = pkv.build_extend_metadata(P, L, shape_of(w), 0, splits, device="cuda", causal=causal)
    kn, vn = cache._gather_new_kv(w)
    pkv.pkv_append(kn, vn, cache.k_pool, cache.v_pool, cache.page_table, plan)
    md = torch.from_numpy(m).to("cuda")
    out = pkv.paged_extend_attn_masked(upload_q(w), cache.k_pool, cache.v_pool, cache.page_table, plan, md)
    torch.cuda.synchronize()
    assert pkv.read_status(plan) == 0
    return values_of(out), oracle_out(w, oracle_pools(w), causal=causal, mask=m), m


@pytest.mark.parametrize("dtype,P,L,hq,hkv,D,ps,mh,mr,causal", [
    ("bf16", [0, 100, 513], [64, 128, 1], 16, 4, 128, 16, 16, 128, True),    # per head and row, ragged + 1-token row
    ("bf16", [0, 0], [256, 128], 32, 4, 128, 64, 1, 256, False),             # the pages' [batch, 1, q_len, kv_len]
    ("bf16", [37, 5], [90, 200], 8, 2, 64, 16, 1, 1, True),                   # 2-D [batch, kv_len]
    ("bf16", [20, 7], [45, 60], 6, 3, 128, 3, 6, 60, True),                   # pages of 3 tokens (general gather)
    ("fp32", [10, 0], [40, 33], 4, 2, 64, 16, 4, 40, True),
    ("fp32", [0], [70], 2, 1, 128, 5, 1, 70, False),
])
def test_masked(dtype, P, L, hq, hkv, D, ps, mh, mr, causal):
    got, ref, _ = _masked_case(dtype, P, L, hq, hkv, D, ps, mh, mr, causal, seed=11)
    assert not np.isnan(got).any()
    check(f"masked {dtype} D={D} ps={ps} mask[{mh},{mr}] causal={causal}", got, ref, dtype)


@settings(max_examples=30, deadline=None, derandomize=True, database=None)
@given(st.data())
def test_masked_random(data):
    """Random keep-masks (a fixed, derandomized set) over random small batches:
    dtype, head dim, GQA, page sizes (general gather included), mask head and
    row axes shared or not, causal or not, keep rates from almost none to all,
    split counts."""
    dtype = data.draw(st.sampled_from(["bf16", "bf16", "fp32"]))
    D = data.draw(st.sampled_from([64, 128]))
    B = data.draw(st.integers(1, 3))
    P = data.draw(st.lists(st.integers(0, 400), min_size=B, max_size=B))
    L = data.draw(st.lists(st.sampled_from([1, 2, 17, 64, 90]), min_size=B, max_size=B))
    hkv = data.draw(st.sampled_from([1, 2]))
    hq = hkv * data.draw(st.sampled_from([1, 4]))
    ps = data.draw(st.sampled_from([3, 16, 64]))
    mh = data.draw(st.sampled_from([1, hq]))
    mr = data.draw(st.sampled_from([1, 2]))   # 1: shared row axis; else one row per chunk row
    causal = data.draw(st.booleans())
    p_keep = data.draw(st.sampled_from([0.05, 0.5, 0.95, 1.0]))
    splits = data.draw(st.sampled_from([0, 3]))
    seed = data.draw(st.integers(0, 1000))
    got, ref, _ = _masked_case(dtype, P, L, hq, hkv, D, ps, mh, mr, causal, seed=seed, p_keep=p_keep, splits=splits)
    assert not np.isnan(got).any()
    check(f"masked random {dtype} D={D} {hq}/{hkv} ps={ps} mask[{mh},{mr}] causal={causal} keep={p_keep} "
          f"splits={splits} P={P} L={L}", got, ref, dtype)


def test_masked_split_rows_and_an_empty_row():
    # one-token rows split 8 ways over long ranges; head 3 of row 0 of request 1 keeps nothing -> 0
    got, ref, _ = _masked_case("bf16", [3000, 1500, 0], [1, 1, 64], 16, 4, 128, 16, 16, 64, True, seed=12,
                               splits=8, empty_row=(1, 3, 0))
    check("masked split rows", got, ref, "bf16")
    assert np.array_equal(got[1, 3], np.zeros(128, np.float32))


def test_causal_mask_written_out_equals_the_causal_plan():
    """The causal mask given explicitly to a non-causal plan gives the causal
    result (the pages' 4-D causal-mask regression)."""
    P, L = np.array([0, 64], np.int32), np.array([200, 130], np.int32)
    ps, hq, hkv, D = 16, 8, 2, 128
    pages = int(sum((int(n) + ps - 1) // ps for n in P + L)) + 4
    w = wl.Workload("causalmask", 9, "bf16", hq, hkv, D, ps, pages, 0, P, L, wl.shuffled_page_table(9, pages, P + L, ps))
    ks = 272                     # >= the longest request (264), a multiple of 4
    m = np.zeros((2, 1, 200, ks), np.uint8)
    for b in range(2):
        for i in range(int(L[b])):
            m[b, 0, i, :int(P[b]) + i + 1] = 1
    out_c, cache, plan_c = prefill_and_attend(w)
    plan_n = pkv.build_extend_metadata(P, L, shape_of(w), 0, 0, device="cuda", causal=False)
    out_m = pkv.paged_extend_attn_masked(upload_q(w), cache.k_pool, cache.v_pool, cache.page_table, plan_n,
                                         torch.from_numpy(m).to("cuda"))
    check("causal mask on a non-causal plan", out_m, values_of(out_c), "bf16")
