"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- the numbers printed on the pages, closed forms, a library routine
for special cases, or exact identities -- chosen so that a plausible mistake
(a dropped prefix, a top-left causal mask, a wrong head mapping, an
off-by-one window edge, a wrong page slot) fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.paged_attention as oracle_mod
import workloads as wl
from pkv_testlib import oracle_out, oracle_pools

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(P, L, hq=2, hkv=1, d=8, ps=4, window=0, dtype="fp32", zero_q=False, ramp_v=False, step=1.0,
         config_id=101, pool_pages=None):
    n = P + L
    need = (n + ps - 1) // ps
    pages = pool_pages or need + 5
    pt = wl.shuffled_page_table(config_id, pages, [n], ps)
    return wl.Workload(f"tiny{P}+{L}", config_id, dtype, hq, hkv, d, ps, pages, window,
                       np.array([P], np.int32), np.array([L], np.int32), pt,
                       zero_q=zero_q, ramp_v=ramp_v, ramp_v_step=step)


def run_chunks(w_full, chunks, dtype=np.float32):
    """Prefill the request chunk by chunk through the oracle; return all rows."""
    kp, vp = w_full.empty_pool(), w_full.empty_pool()
    outs, p = [], 0
    for c in chunks:
        step = w_full.with_lengths([p], [c])
        kn, vn = step.new_kv_all()
        kp, vp = oracle.append_kv(kp, vp, kn, vn, step.page_table, step.prefix_lens, step.chunk_lens)
        outs.append(oracle_out(step, (kp, vp), dtype=dtype))
        p += c
    return np.concatenate(outs, 0)


# ---------------------------------------------------------------------------
# the page's own numbers
# ---------------------------------------------------------------------------

def test_zero_score_page_literal():
    g = json.load(open(os.path.join(GOLDEN, "zero_score_chunks.json")))
    v = g["v"]
    step = v[1] - v[0]
    w = tiny(0, len(v), hq=1, hkv=1, d=4, ps=2, zero_q=True, ramp_v=True, step=step)
    assert np.array_equal(w.kv_seq(0)[1][:, 0, 0], np.array(v, np.float32))
    out = run_chunks(w, g["chunks"])
    assert np.array_equal(out[:, 0, :], np.repeat(np.array(g["expected"], np.float32)[:, None], 4, 1))
    # the bug the PR fixes: the second chunk attends to its own tokens only
    c0 = g["chunks"][0]
    k, vv = w.kv_seq(0)
    q = np.zeros((len(v) - c0, 1, 4), np.float32)
    pt = np.arange(4, dtype=np.int32)[None]
    pool_k = np.full((4, 2, 1, 4), np.nan, np.float32)
    pool_v = pool_k.copy()
    lone = [len(v) - c0]
    pool_k, pool_v = oracle.append_kv(pool_k, pool_v, k[c0:], vv[c0:], pt, [0], lone)
    dropped = oracle.extend_attention(q, pool_k, pool_v, pt, [0], lone)
    assert np.array_equal(np.concatenate([out[:c0, 0, 0], dropped[:, 0, 0]]),
                          np.array(g["prefix_dropped"], np.float32))


@pytest.mark.parametrize("chunks", [[64], [16, 16, 16, 16], [1] * 64, [48, 16], [15, 33, 16]])
def test_zero_score_closed_form_config1(chunks):
    """q = 0, v[t] = t + 1: row t sees 0..t, so its output is (t + 2) / 2 exactly."""
    w = wl.config1(zero_score=True).with_lengths([0], [64])
    out = run_chunks(w, chunks)
    t = np.arange(64, dtype=np.float32)
    want = (t + 2) / 2
    assert np.array_equal(out, np.broadcast_to(want[:, None, None], out.shape))
    # the prefix-dropping form (s + t + 2)/2 for a chunk starting at s > 0 must not match
    s = 0
    for c in chunks:
        if s > 0:
            dropped = (s + t[s:s + c] + 2) / 2
            assert not np.array_equal(out[s:s + c, 0, 0], dropped)
        s += c


@pytest.mark.parametrize("window", [1, 2, 5, 16, 63])
def test_zero_score_window_closed_form(window):
    """With a window the visible set is p-W+1..p: mean of (j+1) over it."""
    w = tiny(0, 64, hq=2, hkv=1, d=4, ps=16, window=window, zero_q=True, ramp_v=True)
    out = run_chunks(w, [20, 20, 24])
    p = np.arange(64, dtype=np.float64)
    lo = np.maximum(0, p - window + 1)
    want = (lo + p + 2) / 2
    assert np.allclose(out[:, 0, 0], want, rtol=0, atol=1e-5)
    assert np.array_equal(out[:, 1, :], out[:, 0, :])
    assert np.array_equal(out[:, 0, :], np.repeat(out[:, 0, :1], 4, 1))


# ---------------------------------------------------------------------------
# library routine on the full sequence (chunked prefill == full prefill)
# ---------------------------------------------------------------------------

def sdpa_full(w, window=0):
    """torch SDPA in float64 over the contiguous full sequence 0..N-1 (no pages),
    with the textbook causal mask (or band mask for a window); rows P..N-1."""
    P, N = int(w.prefix_lens[0]), int(w.kv_lens[0])
    k, v = w.kv_seq(0)
    q = w.q_rows(0, 0, N)
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2)[None]
    if window <= 0:
        o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True)
    else:
        i = torch.arange(N)[:, None]
        j = torch.arange(N)[None, :]
        band = (j <= i) & (j > i - window)
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=band, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()[P:N]


@pytest.mark.parametrize("P,L,hq,hkv,d,ps", [
    (0, 37, 2, 1, 8, 4), (30, 7, 4, 2, 16, 3), (45, 19, 4, 4, 8, 16), (63, 1, 6, 2, 4, 1),
    (100, 28, 8, 2, 64, 16), (17, 47, 3, 3, 4, 5)])
def test_matches_sdpa_on_full_sequence(P, L, hq, hkv, d, ps):
    w = tiny(P, L, hq=hq, hkv=hkv, d=d, ps=ps, config_id=200 + P)
    pools = oracle_pools(w)
    got = oracle_out(w, pools, dtype=np.float64)
    want = sdpa_full(w)
    assert np.abs(got - want).max() < 1e-12
    got32 = oracle_out(w, pools, dtype=np.float32)
    assert np.abs(got32 - want).max() < 1e-5


@pytest.mark.parametrize("window,P,L", [(1, 20, 9), (5, 40, 24), (17, 3, 50), (64, 70, 10), (3, 0, 12)])
def test_window_matches_sdpa_band_mask(window, P, L):
    w = tiny(P, L, hq=4, hkv=2, d=16, ps=8, window=window, config_id=300 + window)
    got = oracle_out(w, oracle_pools(w), dtype=np.float64)
    assert np.abs(got - sdpa_full(w, window)).max() < 1e-12


@pytest.mark.parametrize("P,L,hq,hkv,d,ps", [(0, 37, 2, 1, 8, 4), (30, 7, 4, 2, 16, 3), (17, 47, 3, 3, 4, 5)])
def test_non_causal_matches_sdpa_without_mask(P, L, hq, hkv, d, ps):
    """Non-causal: each chunk row attends to all N keys of its request, later
    chunk rows included -- torch SDPA with no mask over the full sequence."""
    w = tiny(P, L, hq=hq, hkv=hkv, d=d, ps=ps, config_id=250 + P)
    got = oracle_out(w, oracle_pools(w), dtype=np.float64, causal=False)
    N = P + L
    k, v = w.kv_seq(0)
    q = w.q_rows(0, P, N)
    t = lambda a: torch.from_numpy(a.astype(np.float64)).permute(1, 0, 2)[None]  # noqa: E731
    want = F.scaled_dot_product_attention(t(q), t(k), t(v), enable_gqa=True)[0].permute(1, 0, 2).numpy()
    assert np.abs(got - want).max() < 1e-12
    # and it differs from the causal result wherever a row has later keys
    causal = oracle_out(w, oracle_pools(w), dtype=np.float64)
    assert np.abs(got[:-1] - causal[:-1]).max() > 1e-3 and np.abs(got[-1] - causal[-1]).max() < 1e-12


def test_non_causal_zero_score_is_the_mean_of_all_values():
    w = tiny(5, 11, hq=2, hkv=1, d=4, ps=4, zero_q=True, ramp_v=True, config_id=251)
    got = oracle_out(w, oracle_pools(w), dtype=np.float64, causal=False)
    assert np.array_equal(got, np.full_like(got, (16 + 1) / 2))   # v[t] = t + 1, t < 16


def rand_mask(rng, B, hm, qm, ks, p=0.7):
    m = (rng.random((B, hm, qm, ks)) < p).astype(np.uint8)
    return m


def test_mask_all_true_and_causal_mask_reproduce_the_unmasked_results():
    w = tiny(9, 23, hq=4, hkv=2, d=16, ps=4, config_id=260)
    pools = oracle_pools(w)
    N = 9 + 23
    ones = np.ones((1, 1, 1, N + 3), np.uint8)
    # (the masked path evaluates head by head, the unmasked one a GQA group at once: same sums,
    # another rounding order, so the comparison is in float64)
    ref = oracle_out(w, pools, dtype=np.float64)
    assert np.abs(oracle_out(w, pools, dtype=np.float64, causal=True, mask=ones) - ref).max() < 1e-12
    # the causal mask written out, applied without the causal flag
    cm = np.zeros((1, 1, 23, N), np.uint8)
    for i in range(23):
        cm[0, 0, i, :9 + i + 1] = 1
    assert np.abs(oracle_out(w, pools, dtype=np.float64, causal=False, mask=cm) - ref).max() < 1e-12


def test_mask_matches_sdpa_with_bool_mask():
    """Random per-head, per-row mask (non-causal): torch SDPA with the same bool
    attn_mask over the contiguous sequence, fp64 (every row keeps >= 1 key)."""
    P, L, hq, hkv, d = 6, 21, 4, 2, 8
    w = tiny(P, L, hq=hq, hkv=hkv, d=d, ps=4, config_id=261)
    N = P + L
    rng = np.random.default_rng(3)
    m = rand_mask(rng, 1, hq, L, N + 5)
    m[..., P] = 1                                   # every row keeps key P
    got = oracle_out(w, oracle_pools(w), dtype=np.float64, causal=False, mask=m)
    k, v = w.kv_seq(0)
    q = w.q_rows(0, P, N)
    t = lambda a: torch.from_numpy(a.astype(np.float64)).permute(1, 0, 2)[None]  # noqa: E731
    am = torch.from_numpy(m[0, :, :, :N].astype(bool))[None]                      # [1, Hq, L, N]
    want = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=am, enable_gqa=True)[0].permute(1, 0, 2)
    assert np.abs(got - want.numpy()).max() < 1e-12


def test_mask_broadcast_axes_and_empty_rows():
    w = tiny(4, 10, hq=4, hkv=1, d=8, ps=4, config_id=262)
    pools = oracle_pools(w)
    rng = np.random.default_rng(4)
    m2 = rand_mask(rng, 1, 1, 1, 16)                 # 2-D: one key mask for every head and row
    full = np.broadcast_to(m2, (1, 4, 10, 16)).copy()
    assert np.array_equal(oracle_out(w, pools, mask=m2), oracle_out(w, pools, mask=full))
    m = np.ones((1, 4, 10, 16), np.uint8)
    m[0, 2, 3, :] = 0                                # head 2 of row 3 keeps nothing -> 0
    out = oracle_out(w, pools, mask=m, causal=False)
    assert np.array_equal(out[3, 2], np.zeros(8, np.float32)) and np.abs(out[3, 1]).max() > 0


def test_one_token_row_sees_every_key():
    """A one-token chunk after P cached tokens is plain softmax attention over all P+1 keys."""
    w = tiny(57, 1, hq=4, hkv=1, d=16, ps=8, config_id=401)
    got = oracle_out(w, oracle_pools(w), dtype=np.float64)[0]
    k, v = w.kv_seq(0)
    q = w.q_chunk(0)[0].astype(np.float64)                       # [Hq, D]
    qt = torch.from_numpy(q)[:, None, :]                           # [Hq, 1, D]
    kt = torch.from_numpy(k[:, 0].astype(np.float64))[None].expand(4, -1, -1)
    vt = torch.from_numpy(v[:, 0].astype(np.float64))[None].expand(4, -1, -1)
    want = F.scaled_dot_product_attention(qt, kt, vt)[:, 0].numpy()
    assert np.abs(got - want).max() < 1e-12


def test_window_one_returns_own_value():
    w = tiny(13, 11, hq=2, hkv=1, d=8, ps=4, window=1, config_id=402)
    got = oracle_out(w, oracle_pools(w))
    v = w.kv_seq(0)[1][13:24]
    assert np.array_equal(got, np.repeat(v, 2, axis=1))


def test_first_token_sees_only_itself():
    w = tiny(0, 5, hq=2, hkv=2, d=8, ps=4, config_id=403)
    got = oracle_out(w, oracle_pools(w))
    assert np.array_equal(got[0], w.kv_seq(0)[1][0])


def test_gqa_head_mapping():
    """V constant per KV head: query head h must return the constant of KV head h // G."""
    hq, hkv, d, n = 8, 2, 4, 12
    pt = np.arange(3, dtype=np.int32)[None]
    kp = np.zeros((3, 4, hkv, d), np.float32)
    vp = np.zeros((3, 4, hkv, d), np.float32)
    vp[:, :, 0], vp[:, :, 1] = 10.0, 20.0
    q = np.random.default_rng(0).standard_normal((n, hq, d)).astype(np.float32)
    out = oracle.extend_attention(q, kp, vp, pt, [0], [n])
    assert np.array_equal(out[:, :4], np.full((n, 4, d), 10.0, np.float32))
    assert np.array_equal(out[:, 4:], np.full((n, 4, d), 20.0, np.float32))


def test_scale_default_and_explicit():
    w = tiny(9, 6, hq=2, hkv=1, d=16, ps=4, config_id=404)
    pools = oracle_pools(w)
    a = oracle_out(w, pools, dtype=np.float64)
    b = oracle_out(w, pools, dtype=np.float64, sm_scale=1.0 / math.sqrt(16))
    assert np.array_equal(a, b)
    c = oracle_out(w, pools, dtype=np.float64, sm_scale=0.5)
    assert np.abs(a - c).max() > 1e-3


# ---------------------------------------------------------------------------
# partitions, pages, metadata
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("window", [0, 50])
def test_partition_invariance_bitwise(window):
    """A row's visible set depends only on its absolute position, so the oracle
    gives the same bits for every chunk partition of a prompt."""
    w = tiny(0, 300, hq=4, hkv=2, d=16, ps=8, window=window, config_id=500)
    ref = run_chunks(w, [300])
    for chunks in ([128, 128, 44], [63, 64, 64, 64, 45], [100, 1, 1, 1, 197], [1] * 20 + [280]):
        assert np.array_equal(run_chunks(w, chunks), ref)


def test_page_permutation_invariance_bitwise():
    w1 = tiny(40, 24, hq=4, hkv=2, d=16, ps=4, config_id=501, pool_pages=40)
    pt2 = wl.shuffled_page_table(777, 40, [64], 4)
    w2 = wl.Workload(**{**w1.__dict__, "page_table": pt2})
    assert not np.array_equal(w1.page_table, w2.page_table)
    assert np.array_equal(oracle_out(w1, oracle_pools(w1)), oracle_out(w2, oracle_pools(w2)))


def test_append_round_trip_and_canaries():
    """Chunk-by-chunk appends (starting mid-page) then a gather through the page
    table give back the contiguous sequence; every other slot keeps its canary."""
    ps, n = 16, 77
    w = tiny(0, n, hq=2, hkv=2, d=8, ps=ps, dtype="bf16", config_id=502, pool_pages=12)
    kp, vp = w.empty_pool(), w.empty_pool()
    p = 0
    for c in [5, 11, 17, 1, 43]:                       # starts 0, 5, 16, 33, 34: mid-page
        step = w.with_lengths([p], [c])
        kn, vn = step.new_kv_all()
        kp, vp = oracle.append_kv(kp, vp, kn, vn, step.page_table, step.prefix_lens, step.chunk_lens)
        p += c
    k, v = w.kv_seq(0)
    pages = w.page_table[0]
    assert np.array_equal(oracle.gather_kv(kp, pages, n), wl.to_storage(k, "bf16"))
    assert np.array_equal(oracle.gather_kv(vp, pages, n), wl.to_storage(v, "bf16"))
    written = np.zeros(kp.shape[:2], bool)
    for j in range(n):
        written[pages[j // ps], j % ps] = True
    assert written.sum() == n
    canary = wl.nan_fill("bf16")
    assert (kp[~written] == canary).all() and (vp[~written] == canary).all()


def test_metadata_closed_form():
    """The ragged batch P={0,100,513,1025}, L={1,64,128,512}: total_q = 705,
    N = {1,164,641,1537}."""
    qo, kv = oracle.extend_metadata([0, 100, 513, 1025], [1, 64, 128, 512])
    assert qo.tolist() == [0, 1, 65, 193, 705]
    assert kv.tolist() == [0, 1, 165, 806, 2343]
    qo, kv = oracle.extend_metadata([5, 0, 7], [0, 0, 3])
    assert qo.tolist() == [0, 0, 0, 3] and kv.tolist() == [0, 5, 5, 15]


def test_empty_and_zero_length_requests():
    hq, hkv, d, ps = 2, 1, 4, 4
    pt = np.arange(8, dtype=np.int32).reshape(2, 4)
    kp = np.random.default_rng(1).standard_normal((8, ps, hkv, d)).astype(np.float32)
    vp = np.random.default_rng(2).standard_normal((8, ps, hkv, d)).astype(np.float32)
    q = np.random.default_rng(3).standard_normal((3, hq, d)).astype(np.float32)
    both = oracle.extend_attention(q, kp, vp, pt, [4, 9], [0, 3])
    alone = oracle.extend_attention(q, kp, vp, pt[1:], [9], [3])
    assert np.array_equal(both, alone)
    empty = oracle.extend_attention(np.zeros((0, hq, d), np.float32), kp, vp, pt, [4, 9], [0, 0])
    assert empty.shape == (0, hq, d)


# ---------------------------------------------------------------------------
# planted mistakes: the pins above must catch them
# ---------------------------------------------------------------------------

def test_pins_catch_planted_mistakes(monkeypatch):
    real = oracle_mod.visible_range
    w = tiny(0, 64, hq=2, hkv=1, d=4, ps=16, window=5, zero_q=True, ramp_v=True)
    p = np.arange(64, dtype=np.float64)
    want = (np.maximum(0, p - 5 + 1) + p + 2) / 2

    def off_by_one_window(pos, window):
        lo, hi = real(pos, window)
        return max(0, lo - 1), hi
    monkeypatch.setattr(oracle_mod, "visible_range", off_by_one_window)
    assert not np.allclose(run_chunks(w, [20, 44])[:, 0, 0], want)

    def excludes_self(pos, window):
        lo, hi = real(pos, window)
        return lo, hi - 1
    monkeypatch.setattr(oracle_mod, "visible_range", excludes_self)
    assert not np.allclose(run_chunks(w, [64])[:, 0, 0], want)

    monkeypatch.setattr(oracle_mod, "visible_range", real)
    assert np.allclose(run_chunks(w, [20, 44])[:, 0, 0], want)
