"""The decode oracle against values fixed by the pages and by mathematics."""
import numpy as np
import pytest
import torch

import oracle
from tests import oracle_pins as P


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda p: p.__name__)
def test_pin_holds(orc, pin):
    assert pin(orc) is None


# Each planted mistake must break at least one pin.
MUTANTS = {
    1: "per-block softmax, then sum (the rejected counter-example)",
    2: "tail of the last block not masked",
    3: "q-head -> kv-head map h % Hkv",
    4: "K and V swapped",
    5: "scale dropped",
    6: "off-by-one logical block",
    7: "V read as plain token-major rows",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m])
def test_mutant_is_caught(mutant):
    fails = P.failures(oracle.build_mutant(mutant))
    assert fails, f"mutant {mutant} ({MUTANTS[mutant]}) passed every pin"


def test_half_widening_exact(orc):
    bits = np.arange(65536, dtype=np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.lib.oracle_half_to_double(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_bf16_widening_exact(orc):
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([orc.lib.oracle_bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_16bit_inputs_match_dense(orc, dtype):
    """16-bit storage: oracle == numpy dense attention on the widened values."""
    rng = np.random.default_rng(11)
    lens = [3, 16, 33]
    q, Ks, Vs, t, nb, kp, vp = P.random_case(rng, lens, bs=16, D=16, x=8)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(tdt).view(torch.int16).numpy().view(
            np.uint16)

    def widened(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(tdt).double().numpy()

    out = orc.decode(bits(q), bits(kp), bits(vp), t, lens, 0.25, 16, 2, dtype)
    want = P.dense_attention(widened(q), [widened(K) for K in Ks], [widened(V) for V in Vs],
                             0.25, 2)
    assert np.abs(out - want).max() < 1e-12


def test_threads_do_not_change_result(orc):
    rng = np.random.default_rng(12)
    lens = list(rng.integers(1, 60, size=13))
    q, Ks, Vs, t, nb, kp, vp = P.random_case(rng, lens, bs=8)
    a = orc.decode(q, kp, vp, t, lens, 0.3, 8, 2, "f32", nthreads=1)
    b = orc.decode(q, kp, vp, t, lens, 0.3, 8, 2, "f32", nthreads=5)
    assert np.array_equal(a, b)


def test_rejects_bad_table(orc):
    rng = np.random.default_rng(13)
    q, Ks, Vs, t, nb, kp, vp = P.random_case(rng, [5], bs=4)
    t[0, 1] = nb + 4
    with pytest.raises(ValueError):
        orc.decode(q, kp, vp, t, [5], 0.3, 4, 2, "f32")
