"""Parity of pkv_rope_append (rotary embedding of the chunk's q and k rows at
their absolute positions, fused with the KV append) with the CPU oracle, called
through the C ABI via the Python binding.

Bar: V rows bit-exact; rotated q and K rows within one unit in the last place
of the storage type of the oracle's value plus 2^-20 (|a| + |b|) of the input
pair (a, b) (the GPU rotates in fp32 and rounds once, the oracle in fp64; the
fp32 products' error shows when they cancel), with at least 99.9 % of bf16
elements bitwise equal; every pool byte outside the written slots keeps its
NaN canary;
a chunked prefill equal bit for bit to one full call; rope + attention within
the attention bar (bf16 2e-2 + 1e-2|ref|, fp32 1e-5 + 1e-5|ref|)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from pkv_testlib import assert_parity

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_chunked_prefill_amd as pkv
    from gpu_harness import from_dev, to_dev


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    assert pkv.device_supported(torch.cuda.current_device()), "not a gfx950 device"


def check_rotated(got: np.ndarray, ref: np.ndarray, x_in: np.ndarray, dtype: str, what: str):
    """got/ref/x_in: rotated rows (GPU, oracle) and the input rows, same shape
    [..., D], storage form. The GPU's fp32 products carry an error of order
    2^-24 (|a| + |b|) for the pair (a, b) -- large next to the result's own ulp
    when the two products cancel -- so the bound is one ulp of the reference
    plus 2^-20 (|a| + |b|)."""
    g, r, x = wl.values(got, dtype).astype(np.float64), wl.values(ref, dtype).astype(np.float64), \
        wl.values(x_in, dtype).astype(np.float64)
    m = np.abs(x[..., 0::2]) + np.abs(x[..., 1::2])
    m = np.repeat(m, 2, axis=-1)
    ulp = np.spacing(np.abs(r).astype(np.float32)).astype(np.float64) * (65536.0 if dtype == "bf16" else 1.0)
    err = np.abs(g - r)
    bound = ulp + 2.0 ** -20 * m
    same = float((got.view(np.uint8).reshape(got.shape + (-1,)) == ref.view(np.uint8).reshape(ref.shape + (-1,)))
                 .all(axis=-1).mean())
    print(f"[rope] {what}: max err/bound {float((err / bound).max()):.3f}, bitwise equal {same:.5f}", flush=True)
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} elements beyond the bound"
    if dtype == "bf16":
        assert same >= 0.999, f"{what}: only {same:.4f} bitwise equal"


class RopeCase:
    def __init__(self, P, L, dtype="bf16", hq=8, hkv=2, D=128, ps=16, seed=31, extra_pages=4):
        self.P, self.L = np.array(P, np.int32), np.array(L, np.int32)
        self.dtype, self.hq, self.hkv, self.D, self.ps = dtype, hq, hkv, D, ps
        n = self.P + self.L
        need = int(sum((x + ps - 1) // ps for x in n))
        self.pages = need + extra_pages
        self.pt = wl.shuffled_page_table(seed, self.pages, n, ps)
        rng = np.random.default_rng(seed)
        tq = int(self.L.sum())
        mk = lambda *s: wl.to_storage(rng.standard_normal(s).astype(np.float32), dtype)  # noqa: E731
        self.q, self.k, self.v = mk(tq, hq, D), mk(tq, hkv, D), mk(tq, hkv, D)
        self.table = wl.rope_table(int(n.max()) + 3, D)
        self.shape = pkv.make_shape(hq, hkv, D, ps, self.pages, dtype)
        canary = wl.nan_fill(dtype)
        self.pool0 = np.full((self.pages, ps, hkv, D), canary, wl.storage_np_dtype(dtype))

    def oracle(self):
        return oracle.rope_append(self.q, self.k, self.v, self.table, self.pool0, self.pool0.copy(), self.pt,
                                  self.P, self.L, self.dtype)

    def gpu(self, in_place=False, chunks=None):
        dev = "cuda"
        kp, vp = to_dev(self.pool0, self.dtype, dev), to_dev(self.pool0, self.dtype, dev)
        pt = torch.from_numpy(np.ascontiguousarray(self.pt, np.int32)).to(dev)
        table = torch.from_numpy(self.table).to(dev)
        q = to_dev(self.q, self.dtype, dev)
        k, v = to_dev(self.k, self.dtype, dev), to_dev(self.v, self.dtype, dev)
        if chunks is None:
            plan = pkv.build_extend_metadata(self.P, self.L, self.shape, 0, 0, device=dev)
            q_out = pkv.pkv_rope_append(q, k, v, table, kp, vp, pt, plan, q_out=q if in_place else None)
        else:   # one request, fed in chunks at growing prefixes
            assert len(self.L) == 1
            outs, t, P = [], 0, int(self.P[0])
            for n in chunks:
                plan = pkv.build_extend_metadata([P], [n], self.shape, 0, 0, device=dev)
                outs.append(pkv.pkv_rope_append(q[t:t + n].contiguous(), k[t:t + n].contiguous(),
                                                v[t:t + n].contiguous(), table, kp, vp, pt, plan))
                t, P = t + n, P + n
            q_out = torch.cat(outs)
        torch.cuda.synchronize()
        assert pkv.read_status(plan) == 0
        return from_dev(q_out), from_dev(kp), from_dev(vp), (q_out, kp, vp, pt)


@pytest.mark.parametrize("dtype,D,hq,hkv,ps", [("bf16", 128, 8, 2, 16), ("bf16", 64, 12, 4, 3),
                                               ("fp32", 128, 4, 4, 16), ("fp32", 64, 6, 2, 5)])
def test_rope_append_matches_oracle(dtype, D, hq, hkv, ps):
    c = RopeCase([0, 5, 63, 130], [7, 1, 40, 33], dtype, hq, hkv, D, ps)
    q_ref, k_ref, v_ref = c.oracle()
    q_got, k_got, v_got, _ = c.gpu()
    assert np.array_equal(v_got.view(np.uint8), v_ref.view(np.uint8)), "V rows are a bit copy"
    written = np.zeros(c.pool0.shape[:2], bool)
    slots = []   # (page, offset) of every new token, in token order
    for b in range(len(c.L)):
        for p in range(int(c.P[b]), int(c.P[b] + c.L[b])):
            written[c.pt[b][p // ps], p % ps] = True
            slots.append((c.pt[b][p // ps], p % ps))
    assert np.array_equal(k_got[~written].view(np.uint8), c.pool0[~written].view(np.uint8)), "canaries"
    assert np.array_equal(v_got[~written].view(np.uint8), c.pool0[~written].view(np.uint8)), "canaries"
    pg, off = np.array(slots).T
    check_rotated(k_got[pg, off], k_ref[pg, off], c.k, dtype, f"K {dtype} D={D}")
    check_rotated(q_got, q_ref, c.q, dtype, f"q {dtype} D={D}")


def test_rope_in_place_equals_out_of_place():
    c = RopeCase([3, 0], [20, 9])
    a = c.gpu()
    b = c.gpu(in_place=True)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_rope_chunked_equals_full_bitwise():
    c = RopeCase([17], [97], seed=5)
    full = c.gpu()
    chunked = c.gpu(chunks=[31, 1, 50, 15])
    for x, y in zip(full[:3], chunked[:3]):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rope_then_attention_matches_oracle(dtype):
    c = RopeCase([0, 40, 129], [64, 33, 1], dtype, hq=8, hkv=2, D=128 if dtype == "bf16" else 64, ps=16)
    # prefix K/V: the oracle's rotated rows of positions 0..P-1 (any cached values do)
    q_ref, k_ref, v_ref = c.oracle()
    q_got, k_got, v_got, (q_dev, kp, vp, pt) = c.gpu()
    # the prefix slots hold canaries: give both sides the same prefix keys
    rng = np.random.default_rng(9)
    for b in range(len(c.L)):
        for p in range(int(c.P[b])):
            page, off = c.pt[b][p // c.ps], p % c.ps
            kv = wl.to_storage(rng.standard_normal((2, c.hkv, c.D)).astype(np.float32), dtype)
            k_ref[page, off], v_ref[page, off] = kv[0], kv[1]
    kp.copy_(to_dev(k_ref, dtype, "cuda"))
    vp.copy_(to_dev(v_ref, dtype, "cuda"))
    # K rows of the chunk differ by at most one ulp between the sides: use the GPU's in both
    k_ref = from_dev(kp)
    plan = pkv.build_extend_metadata(c.P, c.L, c.shape, 0, 0, device="cuda")
    out = pkv.paged_extend_attn(q_dev, kp, vp, pt, plan)
    ref = oracle.extend_attention(wl.values(q_got, dtype), wl.values(k_ref, dtype), wl.values(v_ref, dtype), c.pt,
                                  c.P, c.L)
    assert_parity(out.float().cpu().numpy(), ref, dtype, f"rope + attention {dtype}")
    check_rotated(q_got, q_ref, c.q, dtype, "q before attention")
