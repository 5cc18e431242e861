"""Pins for the chunked-prefill oracle: values fixed by the pages' definition
(zhy-blog.vercel.app vLLM post, section 4.2: a chunk's attention mask follows
its position in the whole prompt) and by mathematics.

Each pin takes an oracle build and returns None when it holds, or a short
failure message.  ``test_oracle_prefill.py`` runs them on the real oracle (all
must hold) and on builds with one planted mistake (each must break one).
Pools are filled with the decode pins' numpy placement, independently of the
oracle's pointer arithmetic.
"""
from __future__ import annotations

import numpy as np

from tests.oracle_pins import place, random_tables


def _case(rng, ctx, qlens, hq=4, hkv=2, D=8, bs=4):
    """Sequences with contexts ctx[i]; the last qlens[i] tokens are queries."""
    Ks = [rng.standard_normal((L, hkv, D)).astype(np.float32) for L in ctx]
    Vs = [rng.standard_normal((L, hkv, D)).astype(np.float32) for L in ctx]
    T = int(sum(qlens))
    q = rng.standard_normal((T, hq, D)).astype(np.float32)
    t, nb = random_tables(ctx, bs, rng)
    kp, vp = place(Ks, Vs, t, bs, nb)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return q, Ks, Vs, t, nb, kp, vp, qs


def _prefill(orc, q, kp, vp, t, ctx, qs, scale, bs, hkv):
    return orc.prefill(q, kp, vp, t, ctx, qs, scale, bs, hkv, "f32")


def dense_causal(q, K, V, scale, group):
    """numpy fp64 softmax(Q K^T * scale + causal mask) V for one whole prompt:
    q [T][Hq][D], K / V [T][Hkv][D]; row t sees keys 0 .. t."""
    T, hq, D = q.shape
    out = np.zeros((T, hq, D))
    mask = np.triu(np.full((T, T), -np.inf), k=1)
    for h in range(hq):
        Kh = K[:, h // group, :].astype(np.float64)
        Vh = V[:, h // group, :].astype(np.float64)
        s = q[:, h, :].astype(np.float64) @ Kh.T * scale + mask
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (w / w.sum(axis=1, keepdims=True)) @ Vh
    return out


def pin_one_token_chunk_is_decode(orc):
    """A chunk of one token at the end of its context is a decode step: the
    prefill and decode oracles sum the same terms in the same order."""
    rng = np.random.default_rng(11)
    ctx = [5, 9, 16, 1]
    q, Ks, Vs, t, nb, kp, vp, qs = _case(rng, ctx, [1, 1, 1, 1])
    a = _prefill(orc, q, kp, vp, t, ctx, qs, 0.35, 4, 2)
    b = orc.decode(q, kp, vp, t, ctx, 0.35, 4, 2, "f32")
    return None if np.array_equal(a, b) else "one-token chunk differs from decode"


def pin_first_token_sees_itself(orc):
    """The first token of a prompt (context = chunk) attends only to position 0,
    so its output is v_0 exactly."""
    rng = np.random.default_rng(12)
    ctx = [6, 3]
    q, Ks, Vs, t, nb, kp, vp, qs = _case(rng, ctx, ctx)
    out = _prefill(orc, q, kp, vp, t, ctx, qs, 0.5, 4, 2)
    for i in range(2):
        for h in range(4):
            if not np.array_equal(out[qs[i], h], Vs[i][0, h // 2].astype(np.float64)):
                return f"first token of seq {i} head {h} != v_0"
    return None


def pin_whole_prompt_is_dense_causal(orc):
    """A chunk covering the whole context is ordinary causal attention (numpy
    fp64 matrix products with an upper-triangular -inf mask)."""
    rng = np.random.default_rng(13)
    ctx = [11, 7, 17]
    q, Ks, Vs, t, nb, kp, vp, qs = _case(rng, ctx, ctx)
    out = _prefill(orc, q, kp, vp, t, ctx, qs, 0.45, 4, 2)
    for i in range(3):
        want = dense_causal(q[qs[i]:qs[i + 1]], Ks[i], Vs[i], 0.45, 2)
        if np.abs(out[qs[i]:qs[i + 1]] - want).max() > 1e-12:
            return f"seq {i} differs from dense causal attention"
    return None


def pin_chunking_invariance(orc):
    """The last tokens of a prompt give the same output whether the chunk is
    the whole prompt or only its tail (its keys and positions are the same)."""
    rng = np.random.default_rng(14)
    ctx = [13]
    q, Ks, Vs, t, nb, kp, vp, qs = _case(rng, ctx, ctx)
    whole = _prefill(orc, q, kp, vp, t, ctx, qs, 0.4, 4, 2)
    for tail in (1, 5, 12):
        qs2 = np.array([0, tail], dtype=np.int32)
        part = _prefill(orc, np.ascontiguousarray(q[13 - tail:]), kp, vp, t, ctx, qs2, 0.4, 4, 2)
        if not np.array_equal(part, whole[13 - tail:]):
            return f"tail chunk of {tail} tokens differs from the whole-prompt result"
    return None


def pin_gqa_is_repeated_mha(orc):
    rng = np.random.default_rng(15)
    ctx = [10, 6]
    qlens = [4, 6]
    q, Ks, Vs, t, nb, kp, vp, qs = _case(rng, ctx, qlens, hq=8, hkv=2)
    a = _prefill(orc, q, kp, vp, t, ctx, qs, 0.4, 4, 2)
    Kr = [np.repeat(K, 4, axis=1) for K in Ks]
    Vr = [np.repeat(V, 4, axis=1) for V in Vs]
    kr, vr = place(Kr, Vr, t, 4, nb)
    b = _prefill(orc, q, kr, vr, t, ctx, qs, 0.4, 4, 8)
    return None if np.array_equal(a, b) else "GQA prefill differs from repeated-head MHA"


ALL_PINS = [pin_one_token_chunk_is_decode, pin_first_token_sees_itself,
            pin_whole_prompt_is_dense_causal, pin_chunking_invariance, pin_gqa_is_repeated_mha]


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
