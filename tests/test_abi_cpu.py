"""CPU-only checks of the C ABI library: it loads, exports every function that
include/pkv.h declares, plans steps bit-exactly on the host, and rejects bad
arguments with the documented status codes before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
import paged_chunked_prefill_amd as pkv
import workloads as wl
from paged_chunked_prefill_amd import _abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(_abi.EXPORTS), names
    lib = ctypes.CDLL(_abi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_sizes_match_header_layout(tmp_path):
    """The ctypes mirrors against the header itself: a C program built with
    gcc from include/pkv.h prints every field's offset and each struct's size."""
    import subprocess
    structs = {"pkv_shape": pkv.PkvShape, "pkv_plan": pkv.PkvPlan}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "pkv.h"', 'int main(void) {']
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'  printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-std=c11", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], check=True, capture_output=True, text=True)
               .stdout.splitlines())
    for cname, cls in structs.items():
        assert int(got[cname]) == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert int(got[f"{cname}.{fname}"]) == getattr(cls, fname).offset, f"{cname}.{fname}"


def shape(hq=32, hkv=8, d=128, ps=16, pages=4096, dtype="bf16"):
    return pkv.make_shape(hq, hkv, d, ps, pages, dtype)


def test_indptrs_bit_exact():
    w = wl.config2()
    p = pkv.build_extend_metadata(w.prefix_lens, w.chunk_lens, shape())
    h = p.host_sections()
    qo, kv = oracle.extend_metadata(w.prefix_lens, w.chunk_lens)
    assert np.array_equal(h["qo_indptr"], qo) and np.array_equal(h["kv_indptr"], kv)
    assert np.array_equal(h["prefix_lens"], w.prefix_lens)
    assert p.plan.total_q == 705 and p.plan.max_q_len == 512 and p.plan.max_kv_len == 1537
    assert h["status"][0] == 0
    # every work item carries its tile's offsets (the attention reads nothing else to start)
    it = h["items"]
    r = it["req"]
    assert np.array_equal(it["tok0"], qo[r] + it["q_begin"])
    assert np.array_equal(it["pos0"], w.prefix_lens[r] + it["q_begin"])
    assert np.all(it["q_begin"] + it["q_count"] <= w.chunk_lens[r]) and np.all(it["kv_end"] <= kv[r + 1] - kv[r])
    # bf16 items hold 256 query-head rows = 64 tokens x 4 heads: (1 + 1 + 2 + 8) tiles x 8 KV heads
    # = 96 < 256 resident slots, so the long tiles are split over KV
    tiles = {(int(i["req"]), int(i["kv_head"]), int(i["q_begin"])) for i in h["items"]}
    assert len(tiles) == 96 and p.plan.n_items > 96 and p.plan.n_split_rows > 0


def coverage(p, P, L, hq, hkv, window):
    """Every (token, query head) row is covered by exactly one tile item, or by
    S split items whose key ranges partition the row's visible range."""
    h = p.host_sections()
    items = h["items"]
    G = hq // hkv
    qo, _ = oracle.extend_metadata(P, L)
    seen = {}
    for it in items:
        b, hk = int(it["req"]), int(it["kv_head"])
        for t in range(int(it["q_begin"]), int(it["q_begin"]) + int(it["q_count"])):
            for g in range(G):
                seen.setdefault((int(qo[b]) + t, hk * G + g), []).append(it)
    split_tok = {int(r[0]): int(r[1]) for r in h["split_rows"]}
    assert len(seen) == int(np.sum(L)) * hq
    for (tok, head), its in seen.items():
        b = int(np.searchsorted(qo, tok, side="right") - 1)
        i = tok - int(qo[b])
        pos = int(P[b]) + i
        lo, hi = oracle.visible_range(pos, window)
        if len(its) == 1:
            assert its[0]["part_row"] == -1
            assert its[0]["kv_begin"] <= lo and its[0]["kv_end"] >= hi
        else:
            assert split_tok[tok] == len(its)
            rng = sorted((int(x["kv_begin"]), int(x["kv_end"])) for x in its)
            assert sorted(int(x["split"]) for x in its) == list(range(len(its)))
            assert rng[0][0] <= lo and rng[-1][1] >= hi
            for a, c in zip(rng, rng[1:]):
                assert a[1] == c[0]          # contiguous, disjoint
            assert all(a < c for a, c in rng)  # no empty split


@pytest.mark.parametrize("cfg", ["config2", "config5", "config4", "mixed"])
def test_work_list_covers_every_row_once(cfg):
    if cfg == "config2":
        w, s, splits = wl.config2(), shape(), 0
    elif cfg == "config5":
        w = wl.config5()
        s, splits = shape(64, 8, 128, 16, w.num_pages), 8
    elif cfg == "config4":
        w = wl.config4(mid_page=True)
        s, splits = shape(32, 8, 128, 16, w.num_pages), 0
    else:
        P = np.array([0, 5000, 17, 1, 0, 3], np.int32)
        L = np.array([300, 1, 1, 0, 1, 64], np.int32)
        w = wl.Workload("mixed", 7, "bf16", 12, 4, 64, 16, 1024, 0, P, L, wl.shuffled_page_table(7, 1024, P + L, 16))
        s, splits = shape(12, 4, 64, 16, 1024), 0
    p = pkv.build_extend_metadata(w.prefix_lens, w.chunk_lens, s, w.window, splits)
    coverage(p, w.prefix_lens, w.chunk_lens, s.num_q_heads, s.num_kv_heads, w.window)


@settings(max_examples=80, deadline=None, derandomize=True, database=None)
@given(st.data())
def test_work_list_coverage_random(data):
    """Random batches (ragged prefixes and chunks, empty chunks, one-token rows,
    GQA groups, windows, page sizes, explicit split counts): the coverage
    invariants above hold for every plan."""
    B = data.draw(st.integers(1, 6))
    P = np.array(data.draw(st.lists(st.integers(0, 3000), min_size=B, max_size=B)), np.int32)
    L = np.array(data.draw(st.lists(st.sampled_from([0, 1, 1, 2, 5, 17, 64, 65, 255, 300]),
                                    min_size=B, max_size=B)), np.int32)
    if int(L.sum()) == 0:
        L[0] = 1
    hkv = data.draw(st.sampled_from([1, 2, 4, 8]))
    hq = hkv * data.draw(st.sampled_from([1, 2, 3, 4, 8, 16]))
    window = data.draw(st.sampled_from([0, 0, 1, 7, 64, 500]))
    splits = data.draw(st.sampled_from([0, 0, 1, 3, 8, pkv.PKV_MAX_SPLITS]))
    ps = data.draw(st.sampled_from([1, 3, 16, 64]))
    pages = int(sum((int(n) + ps - 1) // ps for n in P + L)) + 1
    s = shape(hq, hkv, 128, ps, pages)
    p = pkv.build_extend_metadata(P, L, s, window, splits)
    coverage(p, P, L, hq, hkv, window)


@settings(max_examples=60, deadline=None, derandomize=True, database=None)
@given(st.data())
def test_non_causal_plan_random(data):
    """Random non-causal batches: every (request, query tile, KV head) key range,
    merged over its splits, is exactly the request's [0, N_b), contiguous and
    disjoint, and every chunk row of every head is covered."""
    B = data.draw(st.integers(1, 5))
    P = np.array(data.draw(st.lists(st.integers(0, 2000), min_size=B, max_size=B)), np.int32)
    L = np.array(data.draw(st.lists(st.sampled_from([0, 1, 3, 64, 100, 257]), min_size=B, max_size=B)), np.int32)
    if int(L.sum()) == 0:
        L[-1] = 3
    hkv = data.draw(st.sampled_from([1, 2, 4]))
    hq = hkv * data.draw(st.sampled_from([1, 4, 8]))
    splits = data.draw(st.sampled_from([0, 2, 8]))
    ps = data.draw(st.sampled_from([1, 16, 64]))
    pages = int(sum((int(n) + ps - 1) // ps for n in P + L)) + 1
    p = pkv.build_extend_metadata(P, L, shape(hq, hkv, 128, ps, pages), 0, splits, causal=False)
    it = p.host_sections()["items"]
    assert (it["pos0"] == 1 << 30).all()
    ranges, rows = {}, set()
    for x in it:
        b = int(x["req"])
        ranges.setdefault((b, int(x["q_begin"]), int(x["kv_head"])), []).append((int(x["kv_begin"]), int(x["kv_end"])))
        for t in range(int(x["q_begin"]), int(x["q_begin"]) + int(x["q_count"])):
            rows.add((b, t, int(x["kv_head"])))
    for (b, _, _), rs in ranges.items():
        rs.sort()
        assert rs[0][0] == 0 and rs[-1][1] == P[b] + L[b], rs
        assert all(a[1] == c[0] and a[0] < a[1] for a, c in zip(rs, rs[1:])), rs
    assert rows == {(b, t, h) for b in range(B) for t in range(int(L[b])) for h in range(hkv)}


def test_config5_split_plan():
    w = wl.config5()
    p = pkv.build_extend_metadata(w.prefix_lens, w.chunk_lens, shape(64, 8, 128, 16, w.num_pages), 0, 8)
    assert p.plan.n_items == 64 * 8 * 8 + 2 * 8 * (2048 // 32)      # 8 splits; 32-token tiles (G=8)
    assert p.plan.n_split_rows == 64 and p.plan.max_splits == 8
    # bf16 partial outputs (D x 2 bytes) plus fp32 (max, sum) per row, head and split
    assert p.plan.workspace_bytes >= 64 * 64 * 8 * (128 * 2 + 2 * 4)
    mb, wb = pkv.extend_metadata_size(w.prefix_lens, w.chunk_lens, shape(64, 8, 128, 16, w.num_pages), 0, 8)
    assert wb == p.plan.workspace_bytes and mb == p.meta_host.size


def test_window_ranges_are_tight():
    """The key ranges of a tile's items (one item, or its splits) together span
    exactly [first row's window start, last row's position + 1)."""
    P, L = np.array([6000], np.int32), np.array([1000], np.int32)
    p = pkv.build_extend_metadata(P, L, shape(32, 8, 128, 16, 1000), 4096, 0)
    span = {}
    for it in p.host_sections()["items"]:
        key = (int(it["kv_head"]), int(it["q_begin"]), int(it["q_count"]))
        lo, hi = span.get(key, (1 << 30, -1))
        span[key] = (min(lo, int(it["kv_begin"])), max(hi, int(it["kv_end"])))
    for (_, q0, n), (lo, hi) in span.items():
        first = 6000 + q0
        assert lo == first - 4096 + 1 and hi == first + n


def status_of(fn):
    try:
        fn()
    except pkv.PkvError as e:
        return e.status
    return 0


@pytest.mark.parametrize("kw,status", [
    (dict(P=[-1], L=[4]), pkv.PKV_ERR_INVALID_ARGUMENT),
    (dict(P=[0], L=[-4]), pkv.PKV_ERR_INVALID_ARGUMENT),
    (dict(P=[2**31 - 2], L=[4]), pkv.PKV_ERR_INVALID_ARGUMENT),
    (dict(P=[2**30, 2**30], L=[4, 4]), pkv.PKV_ERR_INVALID_ARGUMENT),
    (dict(s=dict(hq=30, hkv=8)), pkv.PKV_ERR_INVALID_ARGUMENT),
    (dict(s=dict(hkv=0)), pkv.PKV_ERR_INVALID_ARGUMENT),
    (dict(s=dict(ps=0)), pkv.PKV_ERR_INVALID_ARGUMENT),
    (dict(s=dict(pages=0)), pkv.PKV_ERR_INVALID_ARGUMENT),
    (dict(s=dict(d=96)), pkv.PKV_ERR_UNSUPPORTED),
    (dict(s=dict(d=256)), pkv.PKV_ERR_UNSUPPORTED),
    (dict(s=dict(dtype=7)), pkv.PKV_ERR_UNSUPPORTED),
    (dict(s=dict(hq=256, hkv=1)), pkv.PKV_ERR_UNSUPPORTED),
    (dict(s=dict(hq=32768, hkv=32768, d=64, dtype="fp32")), pkv.PKV_ERR_UNSUPPORTED),   # KV head field of an item
    (dict(splits=33), pkv.PKV_ERR_INVALID_ARGUMENT),
    (dict(splits=-1), pkv.PKV_ERR_INVALID_ARGUMENT),
])
def test_invalid_arguments_rejected(kw, status):
    P = kw.get("P", [3, 5])
    L = kw.get("L", [1, 2])
    s = shape(**kw.get("s", {}))
    assert status_of(lambda: pkv.build_extend_metadata(P, L, s, 0, kw.get("splits", 0))) == status
    assert pkv.lib().pkv_last_error().decode()


def test_batch_zero_and_small_buffers_rejected():
    lib = pkv.lib()
    s = shape()
    plan = pkv.PkvPlan()
    P = np.array([1], np.int32)
    L = np.array([1], np.int32)
    buf = np.zeros(16, np.uint8)
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    assert lib.build_extend_metadata(0, vp(P), vp(L), ctypes.byref(s), 0, 0, vp(buf), 16, None, 0,
                                     ctypes.byref(plan), None) == pkv.PKV_ERR_INVALID_ARGUMENT
    assert lib.build_extend_metadata(1, vp(P), vp(L), ctypes.byref(s), 0, 0, vp(buf), 16, None, 0,
                                     ctypes.byref(plan), None) == pkv.PKV_ERR_WORKSPACE
    assert lib.build_extend_metadata(1, None, vp(L), ctypes.byref(s), 0, 0, vp(buf), 16, None, 0,
                                     ctypes.byref(plan), None) == pkv.PKV_ERR_INVALID_ARGUMENT


def test_host_only_plan_cannot_launch():
    """A host-only plan has no device metadata: the launches refuse it before any HIP call."""
    lib = pkv.lib()
    s = shape()
    p = pkv.build_extend_metadata([3], [2], s)
    dummy = ctypes.c_void_p(0x1000)
    st = lib.pkv_append(dummy, dummy, dummy, dummy, dummy, 4, None, ctypes.byref(p.plan), ctypes.byref(s), None)
    assert st == pkv.PKV_ERR_INVALID_ARGUMENT
    st = lib.paged_extend_attn(dummy, dummy, dummy, dummy, 4, None, None, None, None, 0, 0.0, ctypes.byref(p.plan),
                               ctypes.byref(s), dummy, None, 0, None)
    assert st == pkv.PKV_ERR_INVALID_ARGUMENT
    assert "device metadata" in lib.pkv_last_error().decode()
    st = lib.pkv_rope_append(dummy, dummy, dummy, dummy, dummy, 64, dummy, dummy, dummy, 4, None,
                             ctypes.byref(p.plan), ctypes.byref(s), None)
    assert st == pkv.PKV_ERR_INVALID_ARGUMENT
    assert "device metadata" in lib.pkv_last_error().decode()


def test_auto_splits_follow_the_cu_heuristic():
    # 4 one-token rows with long KV and 8 KV heads: 32 base items -> ceil(512/32) = 16 splits
    P = np.full(4, 20000, np.int32)
    L = np.ones(4, np.int32)
    p = pkv.build_extend_metadata(P, L, shape(32, 8, 128, 16, 8000), 0, 0)
    assert p.plan.max_splits == 16 and p.plan.n_items == 4 * 8 * 16
    # one-token rows with very short KV are not split below 2 blocks of 64 keys per split
    p = pkv.build_extend_metadata([100], [1], shape(32, 8, 128, 16, 8000), 0, 0)
    assert p.plan.max_splits == 1


def test_slot_blocks_estimate():
    """plan.slot_blocks (the fused-append choice): the 64-key blocks of the
    longest item, or of the average slot when items outnumber the 256 slots."""
    cases = [([3584], [512], shape(16, 4, 128, 64, 1000)),
             ([16384, 16384], [2048, 2048], shape(64, 8, 128, 16, 5000)),
             ([100, 0, 7], [1, 300, 65], shape(32, 8, 128, 16, 100)),
             ([6000] * 8, [1000] * 8, shape(32, 8, 128, 16, 4000))]
    for P, L, s in cases:
        p = pkv.build_extend_metadata(P, L, s, 4096 if P[0] == 6000 else 0)
        blocks = [-(-int(x["kv_end"]) // 64) - int(x["kv_begin"]) // 64 if x["kv_end"] > x["kv_begin"] else 0
                  for x in p.host_sections()["items"]]
        assert p.plan.slot_blocks == max(max(blocks), -(-sum(blocks) // 256)), (P, L)
    # the headline chunk is fused, the long prefills are not
    assert pkv.build_extend_metadata([3584], [512], cases[0][2]).plan.slot_blocks <= 128
    assert pkv.build_extend_metadata([16384] * 2, [2048] * 2, cases[1][2]).plan.slot_blocks > 128


def test_prefill_tiles_split_only_when_few():
    """A launch with fewer items than 2 per compute unit cuts its longest tiles
    over KV (whole 64-key blocks, >= 2 per split); a full launch is not cut."""
    s16 = shape(16, 4, 128, 64, 1000)
    few = pkv.build_extend_metadata([3584], [512], s16)          # 8 tiles x 4 heads = 32 items
    h = few.host_sections()
    assert few.plan.n_items > 32 and few.plan.max_splits <= 16
    for it in h["items"]:
        if it["part_row"] >= 0:
            assert it["kv_end"] - it["kv_begin"] >= 64
    many = pkv.build_extend_metadata([16384, 16384], [2048, 2048], shape(64, 8, 128, 16, 5000))
    assert many.plan.n_items == 2 * 8 * 64 and many.plan.n_split_rows == 0


def test_non_causal_plan_covers_whole_requests():
    """PKV_FLAG_NON_CAUSAL: every tile's key range, merged over its splits, is its
    request's whole [0, N_b); pos0 sits past every key."""
    s = shape()
    P, L = [0, 37, 500, 3000], [256, 64, 1, 300]
    p = pkv.build_extend_metadata(P, L, s, causal=False)
    assert p.plan.flags == pkv.PKV_FLAG_NON_CAUSAL
    it = p.host_sections()["items"]
    assert (it["pos0"] == 1 << 30).all()
    ranges = {}
    for x in it:
        ranges.setdefault((int(x["req"]), int(x["q_begin"]), int(x["kv_head"])), []).append(
            (int(x["kv_begin"]), int(x["kv_end"])))
    for (b, _, _), rs in ranges.items():
        rs.sort()
        assert rs[0][0] == 0 and rs[-1][1] == P[b] + L[b]
        assert all(a[1] == c[0] for a, c in zip(rs, rs[1:])), rs
    # the causal plan of the same batch bounds each tile by its last row
    pc = pkv.build_extend_metadata(P, L, s)
    assert pc.plan.flags == 0
    assert max(int(x["kv_end"]) for x in pc.host_sections()["items"] if x["req"] == 0 and x["q_begin"] == 0) == 64


def test_non_causal_flag_errors():
    lib = pkv.lib()
    s = shape()
    P, L = np.array([3], np.int32), np.array([2], np.int32)
    mb, wb = ctypes.c_size_t(), ctypes.c_size_t()
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    assert lib.pkv_extend_metadata_size_ex(1, vp(P), vp(L), ctypes.byref(s), 0, 2, 0, 0, ctypes.byref(mb),
                                           ctypes.byref(wb)) == pkv.PKV_ERR_INVALID_ARGUMENT
    assert "flags" in lib.pkv_last_error().decode()
    assert lib.pkv_extend_metadata_size_ex(1, vp(P), vp(L), ctypes.byref(s), 5, pkv.PKV_FLAG_NON_CAUSAL, 0, 0,
                                           ctypes.byref(mb), ctypes.byref(wb)) == pkv.PKV_ERR_INVALID_ARGUMENT
    assert "window" in lib.pkv_last_error().decode()
    assert lib.pkv_extend_metadata_size_ex(1, vp(P), vp(L), ctypes.byref(s), 0, pkv.PKV_FLAG_NON_CAUSAL, 0, 0,
                                           ctypes.byref(mb), ctypes.byref(wb)) == pkv.PKV_OK


def test_kv_head_limit_is_the_item_field():
    """The largest KV head count the work items encode is accepted and decodes
    back; one more is refused (the field would reach the sign bit)."""
    ok = pkv.make_shape(32767, 32767, 64, 1, 64, "fp32")
    p = pkv.build_extend_metadata([0], [1], ok)
    it = p.host_sections()["items"]
    assert sorted(it["kv_head"].tolist()) == list(range(32767)) and (it["head_split"] > 0).all()
    bad = pkv.make_shape(32768, 32768, 64, 1, 64, "fp32")
    assert status_of(lambda: pkv.build_extend_metadata([0], [1], bad)) == pkv.PKV_ERR_UNSUPPORTED


@pytest.mark.parametrize("P,L,splits,any_split", [([3584], [512], 0, True), ([100, 0, 7, 5000], [1, 300, 65, 1], 0, True),
                                                  ([20000] * 3, [1] * 3, 8, True), ([6000] * 8, [1000] * 8, 0, False)])
def test_split_count_field_matches_item_count(P, L, splits, any_split):
    """Each item's split count field S equals the number of items of its tile
    (request, KV head, first token), and its split index runs over 0..S-1."""
    p = pkv.build_extend_metadata(P, L, shape(32, 8, 128, 16, 8000), 4096 if P[0] == 6000 else 0, splits)
    it = p.host_sections()["items"]
    S = (it["head_split"] >> pkv.SPLIT_BITS) & ((1 << pkv.SPLIT_BITS) - 1)
    tiles = {}
    for x, s_ in zip(it, S):
        tiles.setdefault((int(x["req"]), int(x["kv_head"]), int(x["q_begin"])), []).append((int(x["split"]), int(s_)))
    assert any(len(v) > 1 for v in tiles.values()) == any_split
    for v in tiles.values():
        assert all(s_ == len(v) for _, s_ in v)
        assert sorted(k for k, _ in v) == list(range(len(v)))


def test_plan_sized_for_the_given_compute_units():
    """The work list follows the compute-unit count: a 32-unit device gets the
    headline chunk's 32 tiles unsplit (one item per unit), 256 units split them;
    one-token rows get ceil(2 * CUs / base items) splits."""
    s16 = shape(16, 4, 128, 64, 1000)
    small = pkv.build_extend_metadata([3584], [512], s16, num_cus=32)
    assert small.plan.num_cus == 32
    assert small.plan.n_items == 32 and small.plan.n_split_rows == 0 and small.plan.workspace_bytes == 0
    big = pkv.build_extend_metadata([3584], [512], s16, num_cus=256)
    assert big.plan.num_cus == 256 and 32 < big.plan.n_items <= 256 and big.plan.n_split_rows == 512
    # 80 units: 32 tiles cut 2 or 3 ways leave the units uneven; the stream plan
    # (runs of equal predicted time, some of two pieces) takes over
    mid = pkv.build_extend_metadata([3584], [512], s16, num_cus=80)
    real = mid.host_sections()["items"]
    assert 32 < len(real) <= 2 * 80 and mid.plan.n_items >= len(real)
    coverage(mid, np.array([3584], np.int32), np.array([512], np.int32), 16, 4, 0)
    P, L = np.full(4, 20000, np.int32), np.ones(4, np.int32)
    for cus, want in ((32, 2), (64, 4), (256, 16), (1024, 32)):
        p = pkv.build_extend_metadata(P, L, shape(32, 8, 128, 16, 8000), num_cus=cus)
        assert p.plan.max_splits == want, (cus, p.plan.max_splits)
    # the size query plans the same list
    for cus in (32, 80, 256):
        mb, wb = pkv.extend_metadata_size([3584], [512], s16, num_cus=cus)
        p = pkv.build_extend_metadata([3584], [512], s16, num_cus=cus)
        assert mb == p.meta_host.size and wb == p.plan.workspace_bytes


@pytest.mark.parametrize("P,L,cus,window", [(6144, 2048, 256, 0), (2048, 2048, 256, 0), (0, 512, 256, 0),
                                            (1024, 128, 256, 0), (3584, 512, 80, 0), (100, 300, 256, 0),
                                            (0, 512, 256, 128), (500, 300, 256, 1000)])
def test_stream_plan_structure(P, L, cus, window):
    """Plans whose equal cuts would leave the compute units uneven (a causal
    chunk's later tiles see more keys) cut each KV head's work end to end into
    runs of nearly equal predicted time. Every row stays covered once, each
    tile keeps one split count for all KV heads (the combine reads one per
    token), padding items are empty and come only after the last real item of
    their XCD and shader-engine class, and the predicted load per XCD is even."""
    s = shape(16, 4, 128, 64, 1000)
    p = pkv.build_extend_metadata([P], [L], s, window, num_cus=cus)
    h = p.host_sections()
    coverage(p, np.array([P], np.int32), np.array([L], np.int32), 16, 4, window)
    equal = pkv.build_extend_metadata([P], [L], s, window, 1, num_cus=cus).host_sections()["items"]
    assert len(h["items"]) != len(equal) or len(h["padding"]) or not np.array_equal(h["items"], equal), \
        "expected a stream plan"
    items, pad = h["items"], h["padding"]
    counts = {}
    for it in items:
        counts.setdefault(int(it["q_begin"]), set()).add((int(it["head_split"]) >> 8) & 0xFF)
    assert all(len(v) == 1 for v in counts.values())
    assert (pad["q_count"] == 0).all() and (pad["kv_begin"] == pad["kv_end"]).all() and (pad["part_row"] == -1).all()
    # workgroup q runs on XCD q % 8, shader-engine class (q // 8) % 4 (in order per XCD):
    # padding sits only after the last real item of its (XCD, class)
    real_pos = set(int(x) for x in items["position"])
    group = lambda q: (q % 8, (q // 8) % 4)  # noqa: E731
    last_real = {}
    for q in real_pos:
        last_real[group(q)] = max(last_real.get(group(q), -1), q)
    for q in range(p.plan.n_items):
        if q not in real_pos:
            assert q > last_real.get(group(q), -1), "padding before a real item of its engine class"
    # predicted time per XCD (2.8 us per item, 1.39 + 0.067 w us per 64-key block) within 10 % of the mean
    load = np.zeros(8)
    for it in items:
        blocks = -(-int(it["kv_end"]) // 64) - int(it["kv_begin"]) // 64
        waves = min(8, -(-int(it["q_count"]) * 4 // 32))
        load[int(it["position"]) % 8] += 2.8 + blocks * (1.39 + 0.067 * waves)
    used = load[load > 0]
    assert used.max() <= 1.1 * used.mean() + 3.0, load
    mb, wb = pkv.extend_metadata_size([P], [L], s, window, num_cus=cus)
    assert mb == p.meta_host.size and wb == p.plan.workspace_bytes


def test_plan_without_device_uses_nominal_cus():
    """With no HIP device to query (this host), num_cus = 0 sizes the list for
    an MI355X's 256 compute units."""
    p = pkv.build_extend_metadata([3584], [512], shape(16, 4, 128, 64, 1000))
    assert p.plan.num_cus == 256


@pytest.mark.parametrize("cus", [-1, 65537])
def test_num_cus_out_of_range_rejected(cus):
    assert status_of(lambda: pkv.build_extend_metadata([3], [2], shape(), num_cus=cus)) == \
        pkv.PKV_ERR_INVALID_ARGUMENT
    assert status_of(lambda: pkv.extend_metadata_size([3], [2], shape(), num_cus=cus)) == \
        pkv.PKV_ERR_INVALID_ARGUMENT


def test_batch_arrays_must_be_the_plans_own():
    """paged_extend_attn(_masked) takes qo_indptr / kv_indptr / prefix_lens only
    as NULL or the plan's own device arrays; any other pointer is refused before
    any HIP call. (The plan's device pointers are stand-ins here: nothing runs.)"""
    lib = pkv.lib()
    s = shape()
    p = pkv.build_extend_metadata([3], [2], s)
    assert p.plan.workspace_bytes == 0
    fake = p.plan
    fake.qo_indptr, fake.kv_indptr, fake.prefix_lens = 0x10000, 0x20000, 0x30000
    fake.items, fake.status = 0x40000, 0x50000
    d = ctypes.c_void_p(0x1000)
    other = ctypes.c_void_p(0x60000)

    def attn(qo, kv, pre):
        return lib.paged_extend_attn(d, d, d, d, 4, None, qo, kv, pre, 0, 0.0, ctypes.byref(fake), ctypes.byref(s), d,
                                     None, 0, None)

    def masked(qo, kv, pre):
        return lib.paged_extend_attn_masked(d, d, d, d, 4, None, qo, kv, pre, 0, 0.0, d, 1, 1, 8,
                                            ctypes.byref(fake), ctypes.byref(s), d, None, 0, None)

    own = [ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000)]
    for fn in (attn, masked):
        for i in range(3):
            args = [None, None, None]
            args[i] = other
            assert fn(*args) == pkv.PKV_ERR_INVALID_ARGUMENT
            assert "plan's own device array" in lib.pkv_last_error().decode()
        # swapped arrays are refused too
        assert fn(own[1], own[0], None) == pkv.PKV_ERR_INVALID_ARGUMENT
        # NULL or the plan's own pass this check; the call then stops at the device check (no GPU here)
        for args in ([None, None, None], own):
            assert fn(*args) == pkv.PKV_ERR_HIP, lib.pkv_last_error().decode()
            assert "device" in lib.pkv_last_error().decode()


def test_misaligned_tensors_are_refused():
    """Every kernel moves 16-byte vectors: a q, pool, out, workspace or new-K/V
    pointer that is not 16-byte aligned is refused before any HIP call.
    (Stand-in device pointers: nothing runs.)"""
    lib = pkv.lib()
    s = shape()
    p = pkv.build_extend_metadata([3], [2], s)
    fake = p.plan
    fake.qo_indptr, fake.kv_indptr, fake.prefix_lens, fake.items, fake.status = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
    d, bad = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1008)

    def attn(q=d, k=d, v=d, out=d):
        return lib.paged_extend_attn(q, k, v, d, 4, None, None, None, None, 0, 0.0, ctypes.byref(fake),
                                     ctypes.byref(s), out, None, 0, None)

    for kw in ({"q": bad}, {"k": bad}, {"v": bad}, {"out": bad}):
        assert attn(**kw) == pkv.PKV_ERR_INVALID_ARGUMENT
        assert "16-byte aligned" in lib.pkv_last_error().decode()
    assert attn() == pkv.PKV_ERR_HIP   # aligned: stops at the device check (no GPU here)
    kn, vn, kp, vp_ = (ctypes.c_void_p(a) for a in (0x100008, 0x200000, 0x1000000, 0x2000000))
    st = lib.paged_extend_attn_append(d, kn, vn, kp, vp_, d, 4, None, 0, 0.0, ctypes.byref(fake), ctypes.byref(s),
                                      d, None, 0, None)
    assert st == pkv.PKV_ERR_INVALID_ARGUMENT and "16-byte aligned" in lib.pkv_last_error().decode()
    for args in ((bad, d, d, d), (d, d, d, bad)):
        assert lib.pkv_append(*args, d, 4, None, ctypes.byref(fake), ctypes.byref(s), None) == pkv.PKV_ERR_INVALID_ARGUMENT
        assert "16-byte aligned" in lib.pkv_last_error().decode()
    st = lib.pkv_rope_append(d, bad, d, d, d, 64, d, d, d, 4, None, ctypes.byref(fake), ctypes.byref(s), None)
    assert st == pkv.PKV_ERR_INVALID_ARGUMENT and "16-byte aligned" in lib.pkv_last_error().decode()


def test_noalloc_refuses_plans_beyond_its_scratch():
    """paged_extend_attn_noalloc: a plan whose split partials exceed the static
    scratch is refused with PKV_ERR_WORKSPACE before any HIP call; a NULL plan
    with PKV_ERR_INVALID_ARGUMENT. (Stand-in device pointers: nothing runs.)"""
    lib = pkv.lib()
    s = shape(64, 8, 128, 16, 1 << 20)
    P, L = np.full(1000, 20000, np.int32), np.ones(1000, np.int32)
    p = pkv.build_extend_metadata(P, L, s, 0, 8)
    assert p.plan.workspace_bytes > pkv.PKV_NOALLOC_SCRATCH_BYTES
    fake = p.plan
    fake.qo_indptr, fake.kv_indptr, fake.prefix_lens, fake.items, fake.status = 0x1000, 0x2000, 0x3000, 0x4000, 0x5000
    d = ctypes.c_void_p(0x1000)
    st = lib.paged_extend_attn_noalloc(d, d, d, d, 2048, None, None, None, None, 0, 0.0, ctypes.byref(fake),
                                       ctypes.byref(s), d, None)
    assert st == pkv.PKV_ERR_WORKSPACE and "static scratch" in lib.pkv_last_error().decode()
    assert lib.paged_extend_attn_noalloc(d, d, d, d, 2048, None, None, None, None, 0, 0.0, None, ctypes.byref(s), d,
                                         None) == pkv.PKV_ERR_INVALID_ARGUMENT


def test_unfused_append_path_checks_attention_arguments_first():
    """paged_extend_attn_append on a plan it does not fuse (slot_blocks > 128:
    the append kernel runs first, then the attention) refuses a wrong window
    or a short workspace before the append is launched: the status is the
    argument error, not the device check the append would reach first (no GPU
    here). Stand-in device pointers: nothing runs."""
    lib = pkv.lib()
    s = shape(64, 8, 128, 16, 5000)
    p = pkv.build_extend_metadata([16384, 16384], [2048, 2048], s)
    assert p.plan.slot_blocks > 128 and p.plan.workspace_bytes == 0
    fake = p.plan
    fake.qo_indptr, fake.kv_indptr, fake.prefix_lens, fake.items, fake.status = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
    d = ctypes.c_void_p(0x1000)
    kn, vn, kp, vp_ = (ctypes.c_void_p(a) for a in (0x100000, 0x8000000, 0x10000000, 0x80000000))

    def call(window):
        return lib.paged_extend_attn_append(d, kn, vn, kp, vp_, d, 2048, None, window, 0.0, ctypes.byref(fake),
                                            ctypes.byref(s), d, None, 0, None)

    assert call(7) == pkv.PKV_ERR_INVALID_ARGUMENT
    assert "differs from the plan" in lib.pkv_last_error().decode()
    assert call(0) == pkv.PKV_ERR_HIP   # every argument fine: stops at the device check
    # a split plan on the unfused path with too little workspace
    ps = pkv.build_extend_metadata([100000], [300], s)
    assert ps.plan.slot_blocks > 128 and ps.plan.workspace_bytes > 0
    fs = ps.plan
    fs.qo_indptr, fs.kv_indptr, fs.prefix_lens, fs.items, fs.status = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
    st = lib.paged_extend_attn_append(d, kn, vn, kp, vp_, d, 8192, None, 0, 0.0, ctypes.byref(fs), ctypes.byref(s),
                                      d, d, 16, None)
    assert st == pkv.PKV_ERR_WORKSPACE, lib.pkv_last_error().decode()
