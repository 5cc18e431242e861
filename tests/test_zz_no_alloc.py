"""pa_decode_noalloc (the split's scratch in libpa's static per-device array)
against pa_decode with a caller workspace, through the C ABI: two calls in a
row, the second with a smaller input, on the vector-ALU and matrix-core
paths and every split mode; outputs bitwise equal to pa_decode's (the same
kernels and split) and within the dtype tolerance of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_118_amd as pa
import workloads as W
from tests.gpu_util import DEV, TOL, gpu_decode, log, max_err, oracle_decode, to_dev

pytestmark = pytest.mark.gpu

SPECS = {
    "mha_f16": W.OPT13B.with_(num_seqs=12, num_q_heads=8, num_kv_heads=8),
    "gqa_bf16": W.GQA_LONG.with_(num_seqs=3, num_q_heads=16, num_kv_heads=2,
                                 lengths=("uniform", 700, 3000)),
    "mha_bf16_bs8": W.OPT13B.with_(dtype="bf16", num_seqs=8, num_q_heads=4, num_kv_heads=4,
                                   block_size=8),
}


def _noalloc(case, part):
    sp = case.spec
    out = torch.full_like(case.q, float("nan"))
    pa.pa_decode_noalloc(out, case.q, case.k_cache, case.v_cache,
                         torch.from_numpy(case.tables).to(DEV),
                         torch.from_numpy(case.lens).to(DEV), sp.scale, sp.block_size,
                         sp.num_kv_heads, case.max_context_len, partition_size=part)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", sorted(SPECS))
@pytest.mark.parametrize("part", [0, 512, -1])
def test_noalloc_equals_pa_decode_twice(name, part):
    spec = SPECS[name]
    big = to_dev(W.make_decode_case(spec, device=DEV, poison=True))
    small_lens = [max(1, int(x) // 3) for x in big.lens[: max(1, len(big.lens) // 2)]]
    small = to_dev(W.make_decode_case(spec.with_(seed=spec.seed + 1), device=DEV, poison=True,
                                      lens=small_lens))
    for tag, case in (("first", big), ("second, smaller", small)):
        log(f"[noalloc] {name} partition={part} {tag} call")
        got = _noalloc(case, part)
        want = gpu_decode(case, partition_size=part)
        assert torch.equal(got, want), f"{tag}: differs from pa_decode"
        err = max_err(got, oracle_decode(case))
        log(f"  max abs err vs oracle {err:.3e}")
        assert err <= TOL[spec.dtype]


def test_noalloc_full_size_opt13b():
    spec = W.OPT13B
    case = to_dev(W.make_decode_case(spec, device=DEV, poison=False))
    log("[noalloc] full-size OPT-13B-shaped batch")
    assert torch.equal(_noalloc(case, 0), gpu_decode(case, partition_size=0))


def test_noalloc_rejects_oversize_before_launch():
    """A call needing more than the static scratch returns PA_ESCRATCH (-7)
    before touching any pointer (null pointers here)."""
    cap = pa.pa_decode_noalloc_scratch_bytes()
    need = pa.pa_decode_workspace_bytes(8192, 64, 64, 256, 16, 8192, 0, torch.float16)
    assert need > cap
    rc = pa.lib().pa_decode_noalloc(None, None, None, None, None, None, ctypes.c_float(0.1), 16,
                                    64, 8192, 64, 256, 512, 8192, 1 << 20, 1, 0, None)
    assert rc == -7
    assert "static" in pa.pa_strerror(-7)
