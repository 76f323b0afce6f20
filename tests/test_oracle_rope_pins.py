"""Pins for the rotary-embedding oracle (oracle/rope.py): exact turns, the
hand-worked adjacent-pair example, complex multiplication, norm preservation,
angle composition, the relative-position identity that rotary embedding exists
for, the bf16 rounding, and the fused append's slots and chunk invariance.
Each catches a plausible mistake: a swapped pair layout (j, j + D/2), a wrong
sign, cos and sin exchanged, a position taken relative to the chunk, a wrong
slot, V rotated."""
import numpy as np
import pytest

import oracle
import workloads as wl


def f64(bits):   # bf16 bit patterns -> float64 (test-side decoding)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_quarter_half_and_identity_turns_exact():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 2, 8)).astype(np.float32)
    bits = wl.bf16_bits(x)
    ident = np.zeros((1, 4, 2), np.float32); ident[..., 0] = 1
    quarter = np.zeros((1, 4, 2), np.float32); quarter[..., 1] = 1
    half = np.zeros((1, 4, 2), np.float32); half[..., 0] = -1
    pos = [0, 0, 0]
    assert np.array_equal(oracle.rope_rows(bits, pos, ident, "bf16"), bits)
    assert np.array_equal(oracle.rope_rows(x, pos, ident, "fp32"), x)
    q = oracle.rope_rows(x, pos, quarter, "fp32")              # (a, b) -> (-b, a)
    assert np.array_equal(q[..., 0::2], -x[..., 1::2]) and np.array_equal(q[..., 1::2], x[..., 0::2])
    h = oracle.rope_rows(bits, pos, half, "bf16")              # (a, b) -> (-a, -b): sign bits flip
    assert np.array_equal(h, bits ^ np.uint16(0x8000))


def test_hand_worked_adjacent_pairs():
    # D = 4, x = [1, 2, 3, 4]; pair 0 unrotated, pair 1 a quarter turn:
    # adjacent pairs give [1, 2, -4, 3]; the (j, j+D/2) layout would give [1, -4, 3, 2]
    x = np.array([[[1, 2, 3, 4]]], np.float32)
    table = np.array([[[1, 0], [0, 1]]], np.float32)
    assert np.array_equal(oracle.rope_rows(x, [0], table, "fp32"), np.array([[[1, 2, -4, 3]]], np.float32))
    # pair 1 by 60 degrees: (3, 4) -> (3/2 - 2 sqrt3, 3 sqrt3/2 + 2)
    c, s = 0.5, np.sqrt(3) / 2
    table = np.array([[[1, 0], [c, s]]], np.float64)
    got = oracle.rotate_pairs(x.astype(np.float64), table[[0]][:, None])
    assert np.allclose(got[0, 0], [1, 2, 1.5 - 2 * np.sqrt(3), 1.5 * np.sqrt(3) + 2], rtol=0, atol=1e-15)


def test_matches_complex_multiplication():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 3, 16))
    cs = rng.standard_normal((5, 1, 8, 2))
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * (cs[..., 0] + 1j * cs[..., 1])
    got = oracle.rotate_pairs(x, cs)
    assert np.allclose(got[..., 0::2], z.real, rtol=0, atol=1e-13)
    assert np.allclose(got[..., 1::2], z.imag, rtol=0, atol=1e-13)


def test_norm_composition_and_relative_position():
    D, n = 64, 300
    # float64 angles here (the float32 input table keeps cos^2 + sin^2 = 1 only to ~1e-7)
    ang = np.arange(n)[:, None] * 10000.0 ** (-2.0 * np.arange(D // 2) / D)[None, :]
    table = np.stack([np.cos(ang), np.sin(ang)], axis=-1)
    rng = np.random.default_rng(11)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    rot = lambda v, p: oracle.rotate_pairs(v, table[p])
    # rotation: pair norms kept
    r = rot(q, 123)
    assert np.allclose(r[0::2] ** 2 + r[1::2] ** 2, q[0::2] ** 2 + q[1::2] ** 2, rtol=1e-12)
    # composition: turning by m then by n equals turning by m + n (same frequencies)
    assert np.allclose(rot(rot(q, 40), 77), rot(q, 117), rtol=0, atol=1e-9)
    # the dot product of rotated rows depends only on the position difference
    for m, n_ in [(5, 2), (250, 247), (17, 17), (3, 200)]:
        lhs = rot(q, m) @ rot(k, n_)
        rhs = rot(q, m - n_) @ k if m >= n_ else q @ rot(k, n_ - m)
        assert abs(lhs - rhs) < 1e-9


def test_bf16_rounding_agrees_with_float32_rne():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2 ** -130, -(2 ** -133) * 1.5]])
    x32 = x.astype(np.float32).astype(np.float64)          # values exact in float32: no double rounding
    assert np.array_equal(oracle.round_to_bf16_bits(x32), wl.bf16_bits(x32.astype(np.float32)))
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert oracle.round_to_bf16_bits(np.array([1.0 + 2 ** -8]))[0] == 0x3F80
    assert oracle.round_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8]))[0] == 0x3F82


def _rope_workload(P, L, dtype="bf16", hq=4, hkv=2, D=16, ps=4, seed=21):
    n = P + L
    need = (n + ps - 1) // ps
    pages = need + 3
    pt = wl.shuffled_page_table(seed, pages, [n], ps)
    rng = np.random.default_rng(seed)
    mk = lambda *s: wl.to_storage(rng.standard_normal(s).astype(np.float32), dtype)
    return dict(q=mk(L, hq, D), k=mk(L, hkv, D), v=mk(L, hkv, D), pt=pt, pages=pages, ps=ps, D=D, hkv=hkv)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rope_append_slots_and_v_untouched(dtype):
    P, L = 5, 7
    w = _rope_workload(P, L, dtype)
    table = wl.rope_table(64, w["D"])
    canary = wl.nan_fill(dtype)
    kp = np.full((w["pages"], w["ps"], w["hkv"], w["D"]), canary, wl.storage_np_dtype(dtype))
    vp = kp.copy()
    q_rot, k2, v2 = oracle.rope_append(w["q"], w["k"], w["v"], table, kp, vp, w["pt"], [P], [L], dtype)
    k_rot = oracle.rope_rows(w["k"], np.arange(P, P + L), table, dtype)
    for i in range(L):
        p = P + i
        page, off = w["pt"][0][p // w["ps"]], p % w["ps"]
        assert np.array_equal(v2[page, off].view(np.uint8), w["v"][i].view(np.uint8))   # V: bit copy
        assert np.array_equal(k2[page, off].view(np.uint8), k_rot[i].view(np.uint8))
    written = np.zeros(kp.shape[:2], bool)
    for p in range(P, P + L):
        written[w["pt"][0][p // w["ps"]], p % w["ps"]] = True
    assert np.array_equal(k2[~written].view(np.uint8), kp[~written].view(np.uint8))   # canaries kept
    # q rows rotated at absolute positions P.., not chunk positions 0..
    assert np.array_equal(q_rot, oracle.rope_rows(w["q"], np.arange(P, P + L), table, dtype))
    assert not np.array_equal(q_rot, oracle.rope_rows(w["q"], np.arange(L), table, dtype))


def test_rope_append_chunks_equal_one_full_call():
    P0, parts = 3, [5, 1, 9, 4]
    L = sum(parts)
    w = _rope_workload(P0, L)
    table = wl.rope_table(64, w["D"])
    kp = np.zeros((w["pages"], w["ps"], w["hkv"], w["D"]), np.uint16)
    q_full, k_full, v_full = oracle.rope_append(w["q"], w["k"], w["v"], table, kp, kp.copy(), w["pt"], [P0], [L], "bf16")
    k_c, v_c, qs, t, P = kp.copy(), kp.copy(), [], 0, P0
    for n in parts:
        qr, k_c, v_c = oracle.rope_append(w["q"][t:t + n], w["k"][t:t + n], w["v"][t:t + n], table, k_c, v_c,
                                          w["pt"], [P], [n], "bf16")
        qs.append(qr)
        t, P = t + n, P + n
    assert np.array_equal(np.concatenate(qs), q_full)
    assert np.array_equal(k_c, k_full) and np.array_equal(v_c, v_full)
