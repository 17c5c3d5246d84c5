"""Pins of the paged-KV oracle (CPU only).

The page gather is held to an element-by-element loop over the page table
and to the contiguous cache it was cut from (pages stored in a shuffled
order, then found again through the table); the attention on top of it is
``oracle.attention`` (pinned elsewhere), held here to the dense oracle on
the contiguous keys and to its special cases (no token, one token).
"""

import numpy as np
import pytest

import oracle
from oracle import paged as PG


def _cut(k_dense, page_size, rng, extra_pages=3):
    """Cut contiguous [B, H, L, d] rows into a shuffled paged cache; returns
    (cache [num_pages, page_size, H, d], block_table [B, max_pages])."""
    B, H, L, d = k_dense.shape
    max_pages = -(-L // page_size)
    n = B * max_pages + extra_pages
    perm = rng.permutation(n)
    cache = rng.standard_normal((n, page_size, H, d))  # unused pages hold noise
    table = np.zeros((B, max_pages), dtype=np.int32)
    for b in range(B):
        for j in range(max_pages):
            pg = perm[b * max_pages + j]
            table[b, j] = pg
            rows = k_dense[b, :, j * page_size:(j + 1) * page_size, :]  # [H, r, d]
            cache[pg, :rows.shape[1]] = np.transpose(rows, (1, 0, 2))
    return cache, table


def gather_loops(cache, table, seqlens, b):
    P, H, d = cache.shape[1:]
    n = int(seqlens[b])
    out = np.zeros((H, n, d))
    for h in range(H):
        for t in range(n):
            for c in range(d):
                out[h, t, c] = cache[table[b, t // P], t % P, h, c]
    return out


def pin_gather(mod):
    rng = np.random.default_rng(1)
    k = rng.standard_normal((3, 2, 23, 4))
    cache, table = _cut(k, 8, rng)
    seqlens = np.array([23, 9, 0])
    for b in range(3):
        g = mod.gather(cache, table, seqlens, b)
        assert g.shape == (2, int(seqlens[b]), 4)
        np.testing.assert_array_equal(g, gather_loops(cache, table, seqlens, b))
        np.testing.assert_array_equal(g, k[b, :, :seqlens[b], :])


def pin_equals_dense(mod):
    rng = np.random.default_rng(2)
    B, H, L, d, P = 2, 3, 40, 8, 16
    q = rng.standard_normal((B, H, 5, d))
    k = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    kc, table = _cut(k, P, np.random.default_rng(7))
    vc, table_v = _cut(v, P, np.random.default_rng(7))
    assert np.array_equal(table, table_v)
    seqlens = np.array([40, 17])
    o, lse = mod.attention_paged(q, kc, vc, table, seqlens, 0.3)
    for b in range(B):
        ro, rl = oracle.attention(q[b], k[b, :, :seqlens[b]], v[b, :, :seqlens[b]], 0.3, False)
        np.testing.assert_allclose(o[b], ro, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b], rl, rtol=0, atol=1e-14)


def pin_special_cases(mod):
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 1, 3, 4))
    k = rng.standard_normal((2, 1, 8, 4))
    v = rng.standard_normal((2, 1, 8, 4))
    kc, table = _cut(k, 4, np.random.default_rng(5))
    vc, _ = _cut(v, 4, np.random.default_rng(5))
    o, lse = mod.attention_paged(q, kc, vc, table, np.array([0, 1]), 1.0)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))  # no token
    np.testing.assert_allclose(o[1, 0], np.repeat(v[1, 0, :1], 3, axis=0), rtol=0, atol=1e-15)  # one token
    np.testing.assert_allclose(lse[1, 0], q[1, 0] @ k[1, 0, 0], rtol=1e-14)


PINS = [pin_gather, pin_equals_dense, pin_special_cases]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(PG)


class _Mutant:
    def __init__(self, gather):
        self.gather = gather

    def attention_paged(self, q, kc, vc, table, seqlens, scale):
        o = np.zeros(q.shape)
        lse = np.full(q.shape[:3], -np.inf)
        for b in range(q.shape[0]):
            o[b], lse[b] = oracle.attention(q[b], self.gather(kc, table, seqlens, b),
                                            self.gather(vc, table, seqlens, b), scale, False)
        return o, lse


def _gather_page_major(cache, table, seqlens, b):  # rows read as [H, page_size] instead of [page_size, H]
    n = int(seqlens[b])
    P, H, d = cache.shape[1:]
    pages = [cache[int(table[b, j])].reshape(H, P, d) for j in range(-(-n // P))]
    return np.concatenate(pages, axis=1)[:, :n] if n else np.zeros((H, 0, d))


def _gather_no_table(cache, table, seqlens, b):  # pages taken in storage order
    n = int(seqlens[b])
    P = cache.shape[1]
    rows = np.concatenate([cache[b * table.shape[1] + j] for j in range(-(-n // P))], axis=0)[:n] if n else \
        np.zeros((0,) + cache.shape[2:])
    return np.transpose(rows, (1, 0, 2))


def _gather_full_pages(cache, table, seqlens, b):  # ignores seqlens inside the last page
    P = cache.shape[1]
    n = -(-int(seqlens[b]) // P) * P
    return PG.gather(cache, table, np.array([n if i == b else 0 for i in range(len(seqlens))]), b)


@pytest.mark.parametrize("name,fn", [("page-major rows", _gather_page_major), ("no page table", _gather_no_table),
                                     ("whole last page", _gather_full_pages)])
def test_mutations(name, fn):
    caught = 0
    for pin in PINS:
        try:
            pin(_Mutant(fn))
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin catches: {name}"


# ---------------------------------------------------------------- 8-bit caches

def test_dequantize_int8_and_e4m3():
    codes = np.array([[[[0x00, 0x01, 0x7f, 0x80, 0x81, 0xff, 0x38, 0xb8]]]], dtype=np.uint8)
    sc = np.array([[[0.5]]])
    # int8: two's complement
    np.testing.assert_array_equal(PG.dequantize(codes, sc, "int8")[0, 0, 0],
                                  0.5 * np.array([0, 1, 127, -128, -127, -1, 56, -72]))
    # e4m3: 0x38 = 1.0, 0xb8 = -1.0, 0x01 = 2^-9 (smallest subnormal), 0x7f is NaN in e4m3fn
    e = PG.dequantize(codes, sc, "e4m3")[0, 0, 0]
    assert e[0] == 0.0 and e[1] == 0.5 * 2.0 ** -9 and e[6] == 0.5 and e[7] == -0.5
    assert np.isnan(e[2])


def test_quantized_cache_per_token_scales():
    """A per-(token, head) scale multiplies that key row (or value row); with
    codes and scales built from a dense cache the result is the dense one."""
    rng = np.random.default_rng(8)
    B, H, L, d, P = 2, 2, 20, 4, 8
    q = rng.standard_normal((B, H, 3, d))
    kint = rng.integers(-100, 100, size=(B, H, L, d))
    vint = rng.integers(-100, 100, size=(B, H, L, d))
    ks = rng.uniform(0.01, 0.03, size=(B, H, L))
    vs = rng.uniform(0.01, 0.03, size=(B, H, L))
    kc, table = _cut(kint.astype(np.float64), P, np.random.default_rng(4))
    vc, _ = _cut(vint.astype(np.float64), P, np.random.default_rng(4))
    ksc, _ = _cut(ks[..., None], P, np.random.default_rng(4))
    vsc, _ = _cut(vs[..., None], P, np.random.default_rng(4))
    codes_k = kc.astype(np.int64).astype(np.int8).view(np.uint8)
    codes_v = vc.astype(np.int64).astype(np.int8).view(np.uint8)
    seqlens = np.array([20, 11])
    o, lse = PG.attention_paged_quant(q, codes_k, codes_v, ksc[..., 0], vsc[..., 0], table, seqlens, 0.7, "int8")
    for b in range(B):
        n = seqlens[b]
        kd = ks[b, :, :n, None] * kint[b, :, :n]
        vd = vs[b, :, :n, None] * vint[b, :, :n]
        ro, rl = oracle.attention(q[b], kd, vd, 0.7, False)
        np.testing.assert_allclose(o[b], ro, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b], rl, rtol=0, atol=1e-13)
