"""Seeded random shapes against the fp64 oracle, beyond the enumerated
cases of the other GPU tests: dtype, kv heads and group size (1-16), head
dim, block size, ragged and edge lengths (empty, one token, block and
step boundaries), split mode (token-balanced, none, 256/512-token
partitions), for pa_decode, pa_decode_write (pools bit-exact) and
pa_prefill.  A shape a call does not support must be refused with
PA_ENOTSUP, never computed wrongly."""
import numpy as np
import pytest

import paged_kv_cache_118_amd as pa
import workloads as W
from tests import test_gpu_decode_write as TW
from tests import test_gpu_prefill as TP
from tests.gpu_util import DEV, TOL, gpu_decode, log, max_err, oracle_decode, to_dev

pytestmark = pytest.mark.gpu

EDGES = [0, 1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 512, 513,
         1023, 1024, 1025]


def _shape(rng, dtypes, dims, sizes):
    dt = str(rng.choice(dtypes))
    D = int(rng.choice(dims))
    hkv = int(rng.integers(1, 5))
    G = min(int(rng.choice([1, 1, 2, 3, 4, 8, 16])), max(1, 32 // hkv))
    bs = int(rng.choice(sizes))
    return dt, D, hkv, G, bs


def _lens(rng, B, hi):
    kind = int(rng.integers(0, 3))
    if kind == 0:
        lens = rng.integers(0, hi + 1, size=B)
    elif kind == 1:
        lens = np.minimum(rng.choice(EDGES, size=B), hi)
    else:
        lens = np.full(B, int(rng.integers(1, hi + 1)))
    return lens.astype(np.int32)


def _spec(rng, dt, D, hkv, G, bs, lens):
    return W.Spec("random", dt, hkv * G, hkv, D, bs, len(lens),
                  ("fixed", tuple(int(x) for x in lens)), seed=int(rng.integers(1, 1 << 30)))


@pytest.mark.parametrize("seed", [0, 1])
def test_random_decode_shapes(seed):
    rng = np.random.default_rng(1180 + seed)
    for i in range(40):
        dt, D, hkv, G, bs = _shape(rng, ["f32", "f16", "bf16"], [16, 32, 64, 128, 256],
                                   [1, 2, 4, 8, 16, 32, 64, 128])
        lens = _lens(rng, int(rng.integers(1, 13)), int(rng.choice([40, 300, 1100, 2100])))
        part = int(rng.choice([0, 0, -1, 256, 512]))
        spec = _spec(rng, dt, D, hkv, G, bs, lens)
        tag = f"{dt} Hq {hkv * G} Hkv {hkv} D {D} BS {bs} partition {part} lens {lens.tolist()}"
        log(f"[random decode {seed}.{i}] {tag}")
        case = to_dev(W.make_decode_case(spec, device=DEV, poison=True, lens=lens))
        err = max_err(gpu_decode(case, partition_size=part), oracle_decode(case))
        assert err <= TOL[dt], f"{tag}: max abs err {err}"


@pytest.mark.parametrize("seed", [0, 1])
def test_random_decode_write_shapes(seed):
    rng = np.random.default_rng(2180 + seed)
    for i in range(30):
        dt, D, hkv, G, bs = _shape(rng, ["f32", "f16", "bf16"], [16, 32, 64, 128, 256],
                                   [1, 2, 4, 8, 16, 32, 64, 128])
        lens = _lens(rng, int(rng.integers(1, 13)), int(rng.choice([40, 300, 1100])))
        part = int(rng.choice([0, 0, -1, 256, 512]))
        spec = _spec(rng, dt, D, hkv, G, bs, lens)
        tag = f"{dt} Hq {hkv * G} Hkv {hkv} D {D} BS {bs} partition {part} lens {lens.tolist()}"
        log(f"[random decode write {seed}.{i}] {tag}")
        case = to_dev(W.make_decode_case(spec, device=DEV, poison=True, lens=lens))
        kn, vn = TW._new_rows(spec, len(lens), spec.seed + 7, strided=bool(rng.integers(0, 2)))
        TW._check(case, kn, vn, part, tag)


def test_random_prefill_shapes():
    rng = np.random.default_rng(3180)
    for i in range(12):
        dt, D, hkv, G, bs = _shape(rng, ["f16", "bf16"], [64, 128], [8, 16, 32, 64, 128])
        ctx = [max(1, int(x)) for x in _lens(rng, int(rng.integers(1, 6)), 600)]
        ql = [int(rng.integers(1, c + 1)) for c in ctx]
        spec = _spec(rng, dt, D, hkv, G, bs, ctx)
        tag = f"{dt} Hq {hkv * G} Hkv {hkv} D {D} BS {bs} contexts {ctx} chunks {ql}"
        log(f"[random prefill {i}] {tag}")
        case, q, qs = TP.make_prefill_case(spec, ctx, ql)
        err = max_err(TP.run_prefill(case, q, qs), TP.oracle_prefill(case, q, qs))
        assert err <= TOL[dt], f"{tag}: max abs err {err}"


def test_unsupported_shapes_are_refused():
    """fp32 and head dims other than 64 / 128 have no prefill kernel: the
    call returns PA_ENOTSUP before anything runs."""
    rng = np.random.default_rng(4180)
    for dt, D in (("f32", 64), ("f16", 32), ("bf16", 256)):
        spec = _spec(rng, dt, D, 2, 1, 16, [8])
        case, q, qs = TP.make_prefill_case(spec, [8], [8])
        with pytest.raises(pa.PAError) as e:
            TP.run_prefill(case, q, qs)
        assert e.value.status == -2


def test_random_shared_prefix_groups():
    """pa_decode_shared on seeded random group structures: 1-6 groups of up
    to the members a 16-row prefix tile holds, prefixes of 0-40 blocks, tails
    of 0-600 tokens (empty sequences included), every dtype and tail path;
    against the oracle, and within 2 x TOL of the plain decode of the same
    batch."""
    from tests.test_gpu_shared import run_shared
    rng = np.random.default_rng(5180)
    for i in range(12):
        dt, D, hkv, G, bs = _shape(rng, ["f32", "f16", "bf16"], [64, 128, 128, 256],
                                   [8, 16, 32, 64])
        G = min(G, 8)
        mm = 16 // G
        sizes = [int(rng.integers(1, mm + 1)) for _ in range(int(rng.integers(1, 7)))]
        pblocks = [int(rng.choice([0, 1, int(rng.integers(2, 41))])) for _ in sizes]
        tails = [0 if rng.random() < 0.1 else int(rng.integers(1, 601)) for _ in range(sum(sizes))]
        spec = W.Spec("random", dt, hkv * G, hkv, D, bs, sum(sizes), ("fixed", ()),
                      seed=int(rng.integers(1, 1 << 30)))
        tag = (f"{dt} Hq {hkv * G} Hkv {hkv} D {D} BS {bs} groups {sizes} prefix blocks "
               f"{pblocks} tails {tails}")
        log(f"[random shared {i}] {tag}")
        case = to_dev(W.make_shared_case(spec, sizes, pblocks, tails, device=DEV, poison=True))
        out = run_shared(case)
        err = max_err(out, oracle_decode(case))
        plain = (out.double() - gpu_decode(case).double()).abs().max().item()
        assert err <= TOL[dt], f"{tag}: max abs err {err}"
        assert plain <= 2 * TOL[dt], f"{tag}: against pa_decode {plain}"
