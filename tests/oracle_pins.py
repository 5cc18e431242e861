"""Pins for the decode oracle: values fixed by the pages and by mathematics.

Each pin takes an oracle build and returns None when it holds, or a short
failure message.  ``test_oracle_decode.py`` runs them on the real oracle (all
must hold) and on builds with one planted mistake (each must break one).

The pool is filled here with numpy shaped indexing -- K as
[blocks][Hkv][D/X][BS][X] (X dims per 16-byte piece: 4 for fp32, 8 for 16-bit
types), V as [blocks][Hkv][BS/VS][D][VS] -- independently of the oracle's
pointer arithmetic.
"""
from __future__ import annotations

import math

import numpy as np

from workloads import v_slab


def place(seqs_k, seqs_v, tables, bs, num_blocks, fill=np.nan, x=4):
    """Pool arrays holding each sequence's logical K/V rows ([L][Hkv][D]);
    x = dims per 16-byte K piece of the storage dtype the pools will be cast to."""
    hkv, D = seqs_k[0].shape[1], seqs_k[0].shape[2]
    vs = v_slab(bs)
    kp = np.full((num_blocks, hkv, D // x, bs, x), fill, dtype=np.float32)
    vp = np.full((num_blocks, hkv, bs // vs, D, vs), fill, dtype=np.float32)
    for i, (K, V) in enumerate(zip(seqs_k, seqs_v)):
        for u in range(K.shape[0]):
            blk, off = int(tables[i, u // bs]), u % bs
            kp[blk, :, :, off, :] = K[u].reshape(hkv, D // x, x)
            vp[blk, :, off // vs, :, off % vs] = V[u]
    return kp, vp


def random_tables(lens, bs, rng, extra_blocks=3, max_blocks=None):
    need = [-(-int(L) // bs) for L in lens]
    nb = sum(need) + extra_blocks
    perm = rng.permutation(nb)
    mb = max_blocks or max(max(need), 1)
    t = np.full((len(lens), mb), -1, dtype=np.int32)
    c = 0
    for i, n in enumerate(need):
        t[i, :n] = perm[c:c + n]
        c += n
    return t, nb


def dense_attention(q, Ks, Vs, scale, group):
    """numpy fp64 softmax(q K^T * scale) V per (seq, q-head) on contiguous K/V."""
    B, hq, D = q.shape
    out = np.zeros((B, hq, D))
    for b in range(B):
        K = Ks[b].astype(np.float64)
        V = Vs[b].astype(np.float64)
        if K.shape[0] == 0:
            continue
        for h in range(hq):
            s = K[:, h // group, :] @ q[b, h].astype(np.float64) * scale
            w = np.exp(s - s.max())
            out[b, h] = (w / w.sum()) @ V[:, h // group, :]
    return out


def random_case(rng, lens, hq=4, hkv=2, D=8, bs=4, max_blocks=None, x=4):
    Ks = [rng.standard_normal((L, hkv, D)).astype(np.float32) for L in lens]
    Vs = [rng.standard_normal((L, hkv, D)).astype(np.float32) for L in lens]
    q = rng.standard_normal((len(lens), hq, D)).astype(np.float32)
    t, nb = random_tables(lens, bs, rng, max_blocks=max_blocks)
    kp, vp = place(Ks, Vs, t, bs, nb, x=x)
    return q, Ks, Vs, t, nb, kp, vp


def _run(orc, q, kp, vp, t, lens, scale, bs, hkv):
    return orc.decode(q, kp, vp, t, lens, scale, bs, hkv, "f32")


# ----------------------------------------------------------------- pins --
def pin_single_key(orc):
    """L = 1: the only weight is exp(0) / exp(0) = 1, so o = v_0 exactly."""
    rng = np.random.default_rng(1)
    lens = [1, 1, 1]
    q, Ks, Vs, t, nb, kp, vp = random_case(rng, lens, bs=4)
    out = _run(orc, q, kp, vp, t, lens, 0.3, 4, 2)
    for b in range(3):
        for h in range(4):
            if not np.array_equal(out[b, h], Vs[b][0, h // 2].astype(np.float64)):
                return f"single key: seq {b} head {h} != v_0"
    return None


def pin_constant_v(orc):
    """Every valid V row equal to c: the weights sum to one, so o = c."""
    rng = np.random.default_rng(2)
    lens = [7, 13, 2]
    q, Ks, Vs, t, nb, _, _ = random_case(rng, lens, bs=4)
    c = rng.standard_normal((2, 8)).astype(np.float32)
    Vs = [np.broadcast_to(c, (L, 2, 8)).copy() for L in lens]
    kp, vp = place(Ks, Vs, t, 4, nb)
    out = _run(orc, q, kp, vp, t, lens, 0.5, 4, 2)
    for b in range(3):
        for h in range(4):
            if not np.allclose(out[b, h], c[h // 2], rtol=0, atol=1e-12):
                return f"constant V: seq {b} head {h}"
    return None


def pin_zero_k(orc):
    """K = 0: every score is 0, the weights are uniform, o = mean of V rows."""
    rng = np.random.default_rng(3)
    lens = [5, 11]
    q, _, Vs, t, nb, _, _ = random_case(rng, lens, bs=4)
    Ks = [np.zeros((L, 2, 8), dtype=np.float32) for L in lens]
    kp, vp = place(Ks, Vs, t, 4, nb)
    out = _run(orc, q, kp, vp, t, lens, 0.7, 4, 2)
    for b in range(2):
        for h in range(4):
            if not np.allclose(out[b, h], Vs[b][:, h // 2].astype(np.float64).mean(0), rtol=0,
                               atol=1e-12):
                return f"zero K: seq {b} head {h}"
    return None


def pin_weights_1_2_4(orc):
    """Scores 0, ln2, 2 ln2 over three keys in two shuffled blocks of two:
    the global weights are 1 : 2 : 4, o = (v0 + 2 v1 + 4 v2) / 7."""
    # head_dim 4 (one fp32 K piece): the last two dims are zero padding
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]], dtype=np.float32)
    K = np.array([[[0.0, 7.0, 0, 0]], [[1.0, -3.0, 0, 0]], [[2.0, 5.0, 0, 0]]], dtype=np.float32)
    V = np.array([[[1.0, -2.0, 0, 0]], [[3.0, 0.5, 0, 0]], [[-4.0, 8.0, 0, 0]]], dtype=np.float32)
    t = np.array([[2, 0]], dtype=np.int32)
    kp, vp = place([K], [V], t, 2, 3)
    out = orc.decode(q, kp, vp, t, [3], math.log(2.0), 2, 1, "f32")
    want = (V[0, 0] + 2 * V[1, 0] + 4 * V[2, 0]).astype(np.float64) / 7.0
    if not np.allclose(out[0, 0], want, rtol=0, atol=1e-14):
        return f"1:2:4 weights: got {out[0, 0]}, want {want}"
    return None


def pin_dense_library(orc):
    """Gathering through random tables then softmax attention == numpy dense
    attention on the contiguous sequences (GQA group 2, ragged lengths)."""
    rng = np.random.default_rng(4)
    lens = [1, 4, 9, 17, 30]
    for bs in (4, 32):
        q, Ks, Vs, t, nb, kp, vp = random_case(rng, lens, bs=bs)
        out = _run(orc, q, kp, vp, t, lens, 0.35, bs, 2)
        want = dense_attention(q, Ks, Vs, 0.35, 2)
        err = np.abs(out - want).max()
        if not err < 1e-12:
            return f"dense attention mismatch bs={bs}: {err}"
    return None


def pin_permutation_invariance(orc):
    """Physical placement does not change the result (same logical data)."""
    rng = np.random.default_rng(5)
    lens = [6, 19, 3]
    q, Ks, Vs, t1, nb, kp1, vp1 = random_case(rng, lens, bs=4)
    t2, nb2 = random_tables(lens, 4, rng, extra_blocks=9)
    kp2, vp2 = place(Ks, Vs, t2, 4, nb2)
    a = _run(orc, q, kp1, vp1, t1, lens, 0.4, 4, 2)
    b = _run(orc, q, kp2, vp2, t2, lens, 0.4, 4, 2)
    return None if np.array_equal(a, b) else "physical permutation changed the output"


def pin_block_size_invariance(orc):
    rng = np.random.default_rng(6)
    lens = [21, 40, 5]
    q, Ks, Vs, _, _, _, _ = random_case(rng, lens, bs=4)
    ref = None
    for bs in (1, 2, 4, 8, 16, 32, 64):
        t, nb = random_tables(lens, bs, rng)
        kp, vp = place(Ks, Vs, t, bs, nb)
        o = _run(orc, q, kp, vp, t, lens, 0.4, bs, 2)
        if ref is None:
            ref = o
        elif not np.abs(o - ref).max() < 1e-12:
            return f"block size {bs} changed the output"
    return None


def pin_masked_nan(orc):
    """Unfilled tail slots and unused blocks hold NaN; the output is finite and
    equals the run with zeros there."""
    rng = np.random.default_rng(7)
    lens = [5, 10, 3]
    q, Ks, Vs, t, nb, kp, vp = random_case(rng, lens, bs=8)
    kz, vz = place(Ks, Vs, t, 8, nb, fill=0.0)
    a = _run(orc, q, kp, vp, t, lens, 0.4, 8, 2)
    b = _run(orc, q, kz, vz, t, lens, 0.4, 8, 2)
    if not np.isfinite(a).all():
        return "NaN from masked slots leaked into the output"
    return None if np.array_equal(a, b) else "masked slots changed the output"


def pin_gqa_is_repeated_mha(orc):
    """Hq = 8 over Hkv = 2 equals Hq = 8 over Hkv = 8 with each kv head
    repeated for its group of 4 consecutive q heads."""
    rng = np.random.default_rng(8)
    lens = [9, 14]
    q, Ks, Vs, t, nb, kp, vp = random_case(rng, lens, hq=8, hkv=2, bs=4)
    a = _run(orc, q, kp, vp, t, lens, 0.4, 4, 2)
    Kr = [np.repeat(K, 4, axis=1) for K in Ks]
    Vr = [np.repeat(V, 4, axis=1) for V in Vs]
    kr, vr = place(Kr, Vr, t, 4, nb)
    b = _run(orc, q, kr, vr, t, lens, 0.4, 4, 8)
    return None if np.array_equal(a, b) else "GQA differs from repeated-head MHA"


def pin_zero_length(orc):
    rng = np.random.default_rng(9)
    lens = [0, 3]
    q, Ks, Vs, t, nb, kp, vp = random_case(rng, lens, bs=4)
    out = _run(orc, q, kp, vp, t, lens, 0.4, 4, 2)
    if not (out[0] == 0).all():
        return "L = 0 must give a zero row"
    want = dense_attention(q[1:], Ks[1:], Vs[1:], 0.4, 2)
    return None if np.abs(out[1:] - want).max() < 1e-12 else "L = 0 disturbed its neighbour"


ALL_PINS = [pin_single_key, pin_constant_v, pin_zero_k, pin_weights_1_2_4, pin_dense_library,
            pin_permutation_invariance, pin_block_size_invariance, pin_masked_nan,
            pin_gqa_is_repeated_mha, pin_zero_length]


def failures(orc):
    out = []
    for p in ALL_PINS:
        try:
            msg = p(orc)
        except Exception as e:  # a mutant may also crash a pin
            msg = f"raised {type(e).__name__}: {e}"
        if msg:
            out.append(f"{p.__name__}: {msg}")
    return out
