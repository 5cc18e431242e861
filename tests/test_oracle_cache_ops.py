"""The cache-write and block-copy oracles against the pages' slot numbering
and against decode round trips."""
import ctypes

import numpy as np
import pytest

import oracle
from tests import oracle_pins as P
from workloads import v_slab


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("bs", [1, 4, 16, 32])
def test_write_single_head_is_flat_slot_array(orc, bs):
    """Hkv = 1 and D = 4 (one 16-byte fp32 K piece): physical block b covers
    the flat slots b*BS ... (b+1)*BS-1, so the K pool read as [slot][D] rows,
    and the V pool once its slabs are turned back into rows, are indexed by
    the slot itself."""
    nb, D = 6, 4
    vs = v_slab(bs)
    rng = np.random.default_rng(bs)
    slots = rng.permutation(nb * bs)[: nb * bs - 3].astype(np.int64)
    T = len(slots)
    k = rng.standard_normal((T, 1, D)).astype(np.float32)
    v = rng.standard_normal((T, 1, D)).astype(np.float32)
    kc = np.full(nb * bs * D, np.nan, dtype=np.float32)
    vc = np.full(nb * bs * D, np.nan, dtype=np.float32)
    orc.reshape_and_cache(k, v, kc, vc, slots, 1, D, bs, "f32")
    k_rows = kc.reshape(nb * bs, D)
    v_rows = vc.reshape(nb * bs // vs, D, vs).transpose(0, 2, 1).reshape(nb * bs, D)
    want_k = np.full((nb * bs, D), np.nan, dtype=np.float32)
    want_v = np.full((nb * bs, D), np.nan, dtype=np.float32)
    want_k[slots] = k[:, 0]
    want_v[slots] = v[:, 0]
    assert np.array_equal(k_rows, want_k, equal_nan=True)
    assert np.array_equal(v_rows, want_v, equal_nan=True)


@pytest.mark.parametrize("bs", [2, 4, 16, 32])
def test_write_then_decode_is_dense_attention(orc, bs):
    """Writing every token of each sequence into its slot, then decoding,
    reproduces numpy dense attention over the sequences."""
    rng = np.random.default_rng(20 + bs)
    lens = [1, 7, 16, 35]
    hq, hkv, D = 4, 2, 8
    Ks = [rng.standard_normal((L, hkv, D)).astype(np.float32) for L in lens]
    Vs = [rng.standard_normal((L, hkv, D)).astype(np.float32) for L in lens]
    q = rng.standard_normal((len(lens), hq, D)).astype(np.float32)
    t, nb = P.random_tables(lens, bs, rng)
    kc = np.full((nb, hkv, D // 4, bs, 4), np.nan, dtype=np.float32)
    vc = np.full((nb, hkv, bs // v_slab(bs), D, v_slab(bs)), np.nan, dtype=np.float32)
    slots = [int(t[i, u // bs]) * bs + u % bs for i, L in enumerate(lens) for u in range(L)]
    k = np.concatenate(Ks)
    v = np.concatenate(Vs)
    order = rng.permutation(len(slots))  # write order must not matter
    orc.reshape_and_cache(np.ascontiguousarray(k[order]), np.ascontiguousarray(v[order]), kc, vc,
                          np.array(slots)[order], hkv, D, bs, "f32")
    out = orc.decode(q, kc, vc, t, lens, 0.3, bs, hkv, "f32")
    assert np.abs(out - P.dense_attention(q, Ks, Vs, 0.3, 2)).max() < 1e-12


def test_write_skips_negative_slots_and_leaves_rest(orc):
    rng = np.random.default_rng(30)
    nb, hkv, bs, D = 5, 2, 4, 8
    kc = rng.standard_normal((nb, hkv, D // 4, bs, 4)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, 1, D, bs)).astype(np.float32)
    k0, v0 = kc.copy(), vc.copy()
    k = rng.standard_normal((3, hkv, D)).astype(np.float32)
    v = rng.standard_normal((3, hkv, D)).astype(np.float32)
    orc.reshape_and_cache(k, v, kc, vc, np.array([-1, 9, -5]), hkv, D, bs, "f32")
    # only slot 9 = block 2, offset 1 changed
    k0[2, :, :, 1, :] = k[1].reshape(hkv, D // 4, 4)
    v0[2, :, 0, :, 1] = v[1]
    assert np.array_equal(kc, k0) and np.array_equal(vc, v0)


def test_write_strided_token_rows(orc):
    """Token rows may be views with a larger stride (e.g. a fused QKV buffer)."""
    rng = np.random.default_rng(31)
    nb, hkv, bs, D = 4, 2, 16, 8
    qkv = rng.standard_normal((5, 3, hkv, D)).astype(np.float32)
    vs = v_slab(bs)
    kc = np.zeros((nb, hkv, D // 4, bs, 4), dtype=np.float32)
    vc = np.zeros((nb, hkv, bs // vs, D, vs), dtype=np.float32)
    slots = np.array([0, 17, 33, 50, 63])
    flat = np.ascontiguousarray(qkv.reshape(5, -1))
    base = flat.ctypes.data  # k rows start hkv*D elements in, v rows 2*hkv*D
    rc = orc.lib.oracle_reshape_and_cache(
        ctypes.c_void_p(base + 4 * hkv * D), ctypes.c_void_p(base + 8 * hkv * D),
        kc.ctypes.data_as(ctypes.c_void_p), vc.ctypes.data_as(ctypes.c_void_p),
        slots.astype(np.int64).ctypes.data_as(ctypes.c_void_p), 5, 3 * hkv * D, 3 * hkv * D,
        hkv, D, bs, nb, 0)
    assert rc == 0
    for t, s in enumerate(slots):
        assert np.array_equal(kc[s // bs, :, :, s % bs, :], qkv[t, 1].reshape(hkv, D // 4, 4))
        assert np.array_equal(vc[s // bs, :, (s % bs) // vs, :, s % vs], qkv[t, 2])


def test_copy_blocks_bytes_and_decode(orc):
    rng = np.random.default_rng(40)
    lens = [10, 6]
    q, Ks, Vs, t, nb, kp, vp = P.random_case(rng, lens, bs=4)
    free = sorted(set(range(nb)) - set(t[t >= 0].tolist()))
    src = int(t[0, 2])  # seq 0's partial tail block
    dst = free[0]
    k0, v0 = kp.copy(), vp.copy()
    orc.copy_blocks(kp, vp, [[src, dst]], 2, 8, 4, "f32")
    assert np.array_equal(kp[dst], k0[src], equal_nan=True)
    assert np.array_equal(vp[dst], v0[src], equal_nan=True)
    mask = np.ones(nb, bool)
    mask[dst] = False
    assert np.array_equal(kp[mask], k0[mask], equal_nan=True)
    assert np.array_equal(vp[mask], v0[mask], equal_nan=True)
    t2 = t.copy()
    t2[0, 2] = dst
    a = orc.decode(q, kp, vp, t, lens, 0.3, 4, 2, "f32")
    b = orc.decode(q, kp, vp, t2, lens, 0.3, 4, 2, "f32")
    assert np.array_equal(a, b)


def test_copy_blocks_rejects_out_of_range(orc):
    kp = np.zeros((3, 1, 1, 4, 4), np.float32)
    vp = np.zeros((3, 1, 1, 4, 4), np.float32)
    with pytest.raises(ValueError):
        orc.copy_blocks(kp, vp, [[0, 3]], 1, 4, 4, "f32")


def test_swap_blocks_bytes_and_round_trip(orc):
    """Swap oracle: every moved block arrives bit for bit, the rest of the
    destination is untouched, and swapping out then back in at new ids
    restores the original blocks."""
    rng = np.random.default_rng(21)
    hkv, D, bs, dt = 2, 16, 4, "f16"
    x = 8
    ns, nh = 9, 5
    src_k = rng.integers(0, 65535, size=(ns, hkv, D // x, bs, x), dtype=np.uint16)
    src_v = rng.integers(0, 65535, size=(ns, hkv, 1, D, bs), dtype=np.uint16)
    host_k = np.full((nh, hkv, D // x, bs, x), 0x7E01, dtype=np.uint16)
    host_v = np.full((nh, hkv, 1, D, bs), 0x7E01, dtype=np.uint16)
    out_pairs = np.array([[7, 0], [2, 3], [4, 1]], dtype=np.int64)
    orc.swap_blocks(src_k, src_v, host_k, host_v, out_pairs, hkv, D, bs, dt)
    for s, d in out_pairs:
        assert np.array_equal(host_k[d], src_k[s]) and np.array_equal(host_v[d], src_v[s])
    for d in set(range(nh)) - set(out_pairs[:, 1].tolist()):
        assert (host_k[d] == 0x7E01).all() and (host_v[d] == 0x7E01).all()
    back_k = np.zeros_like(src_k)
    back_v = np.zeros_like(src_v)
    in_pairs = np.array([[0, 5], [3, 8], [1, 0]], dtype=np.int64)
    orc.swap_blocks(host_k, host_v, back_k, back_v, in_pairs, hkv, D, bs, dt)
    for (s, _), (_, d) in zip(out_pairs, in_pairs):
        assert np.array_equal(back_k[d], src_k[s]) and np.array_equal(back_v[d], src_v[s])
    with pytest.raises(ValueError):
        orc.swap_blocks(src_k, src_v, host_k, host_v, np.array([[0, nh]]), hkv, D, bs, dt)
