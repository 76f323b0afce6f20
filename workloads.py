"""Seeded synthetic inputs for paged extend attention.

This module only *makes inputs*: lengths, page tables and the q/k/v values of
each request. It holds none of the attention arithmetic, no page-slot
addressing and no metadata cumsums, so that the CPU oracle (``oracle/``) and the
HIP library can both be fed from it without sharing any part of the method.

Every random draw comes from ``numpy.random.Generator(PCG64(SeedSequence(
[config_id, stream, request, block])))``: q/k/v rows are drawn in blocks of 256
positions, so any position range of any request can be regenerated on its own
(the full-size GPU checks recompute only the requests they sample).
Streams: 0 = q, 1 = k, 2 = v, 3 = page permutation, 4 = lengths.

Values are stored either as float32 or as bfloat16 bit patterns (uint16,
round-to-nearest-even from the float32 sample). ``values()`` gives the float32
numbers that the stored bits represent exactly, which is what the oracle reads.

Workload shapes follow the pages: the AReno PR #642 performance and
long-prompt-logprob tables (4097/8193-token prompts under 2048/512/128 chunk
budgets, an ongoing decode mixed with an incoming long prompt) and the
coverage list of its tests (one-token chunks, GQA, page boundaries, sliding
windows, mixed prefix lengths).
"""
from __future__ import annotations

import dataclasses
import math
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

Q_STREAM, K_STREAM, V_STREAM, PAGE_STREAM, LEN_STREAM = 0, 1, 2, 3, 4
ROW_BLOCK = 256


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def rng(config_id: int, stream: int, request: int = 0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([int(config_id), int(stream), int(request)])))


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the float32 numbers they represent (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def values(stored: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_values(stored)
    if dtype == "fp32":
        return np.asarray(stored, dtype=np.float32)
    raise ValueError(dtype)


def nan_fill(dtype: str):
    """The canary pattern for unused pool slots (a quiet NaN in either format)."""
    return np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)


def storage_np_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


# ---------------------------------------------------------------------------
# workload description
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    """One batch of requests for one step: each request b has a cached prefix of
    ``prefix_lens[b]`` tokens and ``chunk_lens[b]`` new tokens this step."""
    name: str
    config_id: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    window: int
    prefix_lens: np.ndarray          # int32 [B]
    chunk_lens: np.ndarray           # int32 [B]
    page_table: np.ndarray           # int32 [B, stride]; -1 past each request's pages
    decode_splits: int = 0           # 0 = let the planner choose
    data_scale: float = 1.0          # applied to the N(0,1) samples before rounding
    zero_q: bool = False             # zero-score variant: q = 0 ...
    ramp_v: bool = False             # ... and v[t] = t + 1 on every channel
    ramp_v_step: float = 1.0         # v[t] = ramp_v_step * t + 1
    request_ids: Optional[np.ndarray] = None   # generator stream id per request

    @property
    def batch(self) -> int:
        return int(self.prefix_lens.shape[0])

    @property
    def kv_lens(self) -> np.ndarray:
        return (self.prefix_lens.astype(np.int64) + self.chunk_lens).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(self.chunk_lens.sum())

    def rid(self, b: int) -> int:
        return int(self.request_ids[b]) if self.request_ids is not None else b

    # -- per-request values (float32, exactly representable in the storage dtype)
    def _normal_rows(self, stream: int, b: int, lo: int, hi: int, heads: int, storage: bool) -> np.ndarray:
        """N(0,1) x data_scale rows lo..hi-1 of one request, rounded to the storage
        dtype; returned as storage (bf16 bits / float32) or as the float32 values
        those bits hold. Rows are drawn in blocks of ``ROW_BLOCK`` positions, each
        block from its own seeded stream, so any range can be regenerated without
        drawing the rows before it (and blocks can be drawn on several threads
        with the same result)."""
        out_dt = storage_np_dtype(self.dtype) if storage else np.float32
        out = np.empty((max(0, hi - lo), heads, self.head_dim), out_dt)
        rid = self.rid(b)
        scale = np.float32(self.data_scale)

        def fill(blk):
            b0 = blk * ROW_BLOCK
            g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
                [int(self.config_id), int(stream), rid, blk])))
            s, e = max(lo, b0), min(hi, b0 + ROW_BLOCK)
            rows = g.standard_normal((ROW_BLOCK, heads, self.head_dim), dtype=np.float32)[s - b0:e - b0]
            if self.data_scale != 1.0:
                rows = rows * scale
            st = to_storage(rows, self.dtype)
            out[s - lo:e - lo] = st if storage else values(st, self.dtype)

        blocks = range(lo // ROW_BLOCK, (hi + ROW_BLOCK - 1) // ROW_BLOCK)
        if len(blocks) > 4:
            list(_pool().map(fill, blocks))
        else:
            for blk in blocks:
                fill(blk)
        return out

    def kv_seq(self, b: int, upto: Optional[int] = None, start: int = 0,
               storage: bool = False) -> Tuple[np.ndarray, np.ndarray]:
        """K/V of request b for positions start..upto-1 (default 0..N_b-1), as
        float32 values (default) or in storage format."""
        n = int(self.kv_lens[b]) if upto is None else int(upto)
        k = self._normal_rows(K_STREAM, b, start, n, self.num_kv_heads, storage)
        if self.ramp_v:
            t = np.arange(start, n, dtype=np.float32) * np.float32(self.ramp_v_step) + np.float32(1)
            v = np.broadcast_to(t[:, None, None], k.shape).astype(np.float32)
            v = to_storage(v, self.dtype) if storage else values(to_storage(v, self.dtype), self.dtype)
        else:
            v = self._normal_rows(V_STREAM, b, start, n, self.num_kv_heads, storage)
        return k, v

    def q_rows(self, b: int, lo: int, hi: int, storage: bool = False) -> np.ndarray:
        """Queries of request b at positions lo..hi-1. A position's query does not
        depend on how the prompt was partitioned into chunks."""
        if self.zero_q:
            z = np.zeros((max(0, hi - lo), self.num_q_heads, self.head_dim), np.float32)
            return to_storage(z, self.dtype) if storage else z
        return self._normal_rows(Q_STREAM, b, lo, hi, self.num_q_heads, storage)

    def q_chunk(self, b: int, storage: bool = False) -> np.ndarray:
        return self.q_rows(b, int(self.prefix_lens[b]), int(self.kv_lens[b]), storage)

    def chunk_kv(self, b: int, storage: bool = False) -> Tuple[np.ndarray, np.ndarray]:
        return self.kv_seq(b, start=int(self.prefix_lens[b]), storage=storage)

    # -- whole-batch arrays, in storage format, for handing to either side
    def _cat(self, parts, heads):
        if parts:
            return np.concatenate(parts, 0)
        return np.zeros((0, heads, self.head_dim), storage_np_dtype(self.dtype))

    def q_all(self) -> np.ndarray:
        return self._cat([self.q_chunk(b, storage=True) for b in range(self.batch)], self.num_q_heads)

    def new_kv_all(self) -> Tuple[np.ndarray, np.ndarray]:
        kv = [self.chunk_kv(b, storage=True) for b in range(self.batch)]
        return (self._cat([k for k, _ in kv], self.num_kv_heads), self._cat([v for _, v in kv], self.num_kv_heads))

    def prefix_kv_all(self) -> Tuple[np.ndarray, np.ndarray]:
        """K/V of every request's cached prefix, concatenated in request order
        (what an earlier step would have appended)."""
        kv = [self.kv_seq(b, upto=int(self.prefix_lens[b]), storage=True) for b in range(self.batch)]
        return (self._cat([k for k, _ in kv], self.num_kv_heads), self._cat([v for _, v in kv], self.num_kv_heads))

    def empty_pool(self) -> np.ndarray:
        shape = (self.num_pages, self.page_size, self.num_kv_heads, self.head_dim)
        return np.full(shape, nan_fill(self.dtype), dtype=storage_np_dtype(self.dtype))

    def with_lengths(self, prefix_lens: Sequence[int], chunk_lens: Sequence[int], name: str = None) -> "Workload":
        """Same requests, pages and values; another step (other P and L)."""
        return dataclasses.replace(self, name=name or self.name,
                                   prefix_lens=np.asarray(prefix_lens, np.int32),
                                   chunk_lens=np.asarray(chunk_lens, np.int32))

    def prefix_step(self) -> "Workload":
        """The step that writes every request's cached prefix (P'=0, L'=P)."""
        return self.with_lengths(np.zeros(self.batch, np.int32), self.prefix_lens, self.name + "/prefix")

    def subset(self, reqs: Sequence[int]) -> "Workload":
        reqs = list(reqs)
        ids = np.array([self.rid(b) for b in reqs], np.int64)
        return dataclasses.replace(self, prefix_lens=self.prefix_lens[reqs].copy(),
                                   chunk_lens=self.chunk_lens[reqs].copy(),
                                   page_table=self.page_table[reqs].copy(), request_ids=ids)


def rope_table(table_len: int, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """Rotary-embedding table: (cos, sin) of p * base**(-2j/D) for positions
    p < table_len and pairs j, float32 [table_len, D/2, 2] (the pages' freqs_cis
    layout, one row per position). An input: the method takes any table."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    ang = np.arange(table_len, dtype=np.float64)[:, None] * base ** (-2.0 * j / head_dim)[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def shuffled_page_table(config_id: int, num_pages: int, kv_lens: Sequence[int], page_size: int,
                        stride: Optional[int] = None, pad: int = -1) -> np.ndarray:
    """Request b gets the next ceil(N_b/ps) ids of a seeded permutation of the pool;
    entries past a request's pages hold ``pad`` (never to be read)."""
    need = [(int(n) + page_size - 1) // page_size for n in kv_lens]
    stride = stride or max(1, max(need) if need else 1)
    perm = rng(config_id, PAGE_STREAM).permutation(num_pages).astype(np.int32)
    if sum(need) > num_pages:
        raise ValueError("pool too small")
    pt = np.full((len(need), stride), pad, np.int32)
    off = 0
    for b, c in enumerate(need):
        pt[b, :c] = perm[off:off + c]
        off += c
    return pt


# ---------------------------------------------------------------------------
# the five configurations
# ---------------------------------------------------------------------------

def config1(zero_score: bool = False, prefix: int = 48, chunk: int = 16) -> Workload:
    """1 request, fp32, 48 cached + 16 new, 2 query heads / 1 KV head, D=64, ps=16,
    pages from a seeded permutation of a 16-page pool."""
    ps, pages = 16, 16
    n = prefix + chunk
    pt = shuffled_page_table(1, pages, [64], ps)          # covers all 64 positions
    return Workload("config1" + ("/zero-score" if zero_score else ""), 1, "fp32",
                    2, 1, 64, ps, pages, 0,
                    np.array([prefix], np.int32), np.array([chunk], np.int32), pt,
                    zero_q=zero_score, ramp_v=zero_score)


def config2() -> Workload:
    """Ragged batch: P={0,100,513,1025}, L={1,64,128,512}; Hq=32, Hkv=8, D=128,
    ps=16; 4096-page shuffled pool whose unused slots hold NaN; data x 1/sqrt(128)."""
    P = np.array([0, 100, 513, 1025], np.int32)
    L = np.array([1, 64, 128, 512], np.int32)
    pt = shuffled_page_table(2, 4096, P + L, 16)
    return Workload("config2", 2, "bf16", 32, 8, 128, 16, 4096, 0, P, L, pt,
                    data_scale=1.0 / math.sqrt(128.0))


def config3(prompt: int = 4097, pool_pages: Optional[int] = None) -> Workload:
    """Single long prompt, Hq=16, Hkv=4, D=128, ps=64; the page table covers the
    whole prompt (use ``chunked_steps`` for the per-chunk batches)."""
    ps = 64
    need = (prompt + ps - 1) // ps
    pages = pool_pages or 2 * need
    pt = shuffled_page_table(3, pages, [prompt], ps)
    return Workload(f"config3/{prompt}", 3, "bf16", 16, 4, 128, ps, pages, 0,
                    np.array([0], np.int32), np.array([prompt], np.int32), pt)


def chunk_partition(total: int, budget: int, first: Optional[int] = None) -> List[int]:
    """Chunk lengths of a prompt run to completion under a token budget: full
    budgets and a final remainder; ``first`` shortens the first chunk so the
    later chunk starts fall mid-page."""
    out, done = [], 0
    if first is not None and total > 0:
        out.append(min(first, total))
        done = out[0]
    while done < total:
        c = min(budget, total - done)
        out.append(c)
        done += c
    return out


def chunked_steps(w: Workload, chunks: Sequence[int]) -> List[Workload]:
    """One single-request step per chunk (prefix = tokens already cached)."""
    steps, p = [], 0
    for c in chunks:
        steps.append(w.with_lengths([p], [c], f"{w.name}/chunk@{p}+{c}"))
        p += c
    return steps


def budget_steps(prompt: int = 4097, budget: int = 512, n_decode: int = 32,
                 config_id: int = 6) -> Tuple[Workload, List[Workload]]:
    """Chunked prefill under a per-step token budget shared with ongoing decodes
    (AReno PR #642, "Performance": an ongoing request keeps decoding while an
    incoming prompt is prefilled in budget-sized chunks). Every step holds the
    n_decode one-token rows (cached lengths uniform in 1024..8192, one more per
    step) first, then the prompt's next chunk of budget - n_decode tokens.
    16 query / 4 KV heads, D=128, 64-token pages, bf16. Returns the workload at
    its final lengths (its page table covers every step) and the steps."""
    chunk = budget - n_decode
    if chunk < 1:
        raise ValueError("budget must leave room for the prompt")
    chunks = chunk_partition(prompt, chunk)
    n_steps = len(chunks)
    dec0 = rng(config_id, LEN_STREAM).integers(1024, 8192, size=n_decode, endpoint=True).astype(np.int32)
    P_fin = np.concatenate([dec0 + n_steps - 1, [0]]).astype(np.int32)
    L_fin = np.concatenate([np.ones(n_decode, np.int32), [prompt]]).astype(np.int32)
    ps = 64
    need = int(sum((int(n) + ps - 1) // ps for n in P_fin + L_fin))
    pt = shuffled_page_table(config_id, need + 8, P_fin + L_fin, ps)
    w = Workload(f"budget{budget}_decode{n_decode}", config_id, "bf16", 16, 4, 128, ps, need + 8, 0,
                 P_fin, L_fin, pt)
    steps, p = [], 0
    for s_, c in enumerate(chunks):
        P = np.concatenate([dec0 + s_, [p]]).astype(np.int32)
        L = np.concatenate([np.ones(n_decode, np.int32), [c]]).astype(np.int32)
        steps.append(w.with_lengths(P, L, f"{w.name}/step{s_}"))
        p += c
    return w, steps


def config4(mid_page: bool = False) -> Workload:
    """8 requests, 6000 cached + 1000 new, window 4096, Hq=32, Hkv=8, D=128, ps=16.
    ``mid_page`` uses prefixes 6001+2b so every append starts inside a page."""
    B = 8
    P = (np.array([6001 + 2 * b for b in range(B)], np.int32) if mid_page
         else np.full(B, 6000, np.int32))
    L = np.full(B, 1000, np.int32)
    need = int(sum((int(n) + 15) // 16 for n in P + L))
    pages = need + 64
    pt = shuffled_page_table(4, pages, P + L, 16)
    return Workload("config4" + ("/mid-page" if mid_page else ""), 4, "bf16", 32, 8, 128, 16,
                    pages, 4096, P, L, pt)


def config5_lengths() -> Tuple[np.ndarray, np.ndarray]:
    g = rng(5, LEN_STREAM)
    dec_n = g.integers(2048, 32768, size=64, endpoint=True).astype(np.int32)
    P = np.concatenate([dec_n - 1, np.full(2, 16384, np.int32)]).astype(np.int32)
    L = np.concatenate([np.ones(64, np.int32), np.full(2, 2048, np.int32)]).astype(np.int32)
    return P, L


def config5(decode_only: bool = False, prefill_only: bool = False) -> Workload:
    """64 one-token rows (N uniform in 2048..32768) then 2 prefill rows (16384 + 2048);
    Hq=64, Hkv=8, D=128, ps=16; one-token rows are split 8 ways."""
    P, L = config5_lengths()
    need = int(sum((int(n) + 15) // 16 for n in P + L))
    pt = shuffled_page_table(5, need + 64, P + L, 16)
    w = Workload("config5", 5, "bf16", 64, 8, 128, 16, need + 64, 0, P, L, pt, decode_splits=8)
    if decode_only:
        w = w.subset(range(64))
        w.name = "config5/decode"
    elif prefill_only:
        w = w.subset([64, 65])
        w.name = "config5/prefill"
    return w
