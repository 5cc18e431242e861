"""pa_decode_shared on the GPU against the fp64 oracle: groups of consecutive
sequences whose tables share leading blocks, read once per group by the
prefix pass (matrix cores, members x q heads per kv head as rows) and joined
with each sequence's own tail.  Every tail path (vector ALUs, matrix cores),
block sizes 8 / 16 / 32, mixed groups (singletons, prefix 0, empty tails,
empty sequences), the fallback to a plain decode, determinism, PA_VALIDATE,
and the full LLaMA-13B-shaped sharing batch."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_118_amd as pa
import workloads as W
from tests.gpu_util import DEV, TOL, gpu_decode, log, max_err, oracle_decode, to_dev

pytestmark = pytest.mark.gpu

BASE = W.LLAMA13B_SHARE
SPECS = {  # (spec, members per group at most)
    "mha_bf16_bs16": (BASE.with_(num_q_heads=8, num_kv_heads=8), 16),
    "mha_f16_bs8": (BASE.with_(dtype="f16", num_q_heads=4, num_kv_heads=4, block_size=8), 16),
    "mha_bf16_bs32": (BASE.with_(num_q_heads=4, num_kv_heads=4, block_size=32), 16),
    "gqa_g2_f16_mfma_tail": (BASE.with_(dtype="f16", num_q_heads=8, num_kv_heads=4), 8),
    "gqa_g8_bf16_mfma_tail": (BASE.with_(num_q_heads=16, num_kv_heads=2, block_size=32), 2),
    "gqa_g4_bf16_d64": (BASE.with_(num_q_heads=8, num_kv_heads=2, head_dim=64), 4),
    "mha_f32_fallback": (BASE.with_(dtype="f32", num_q_heads=4, num_kv_heads=4), 16),
}


def layout(max_members, rng):
    """Group sizes, prefix blocks and tails: full groups with long and short
    prefixes, a singleton, a group sharing nothing, empty tails."""
    sizes = [max_members, 1, min(3, max_members), max_members, min(2, max_members), 2]
    pblocks = [20, 0, 7, 1, 33, 0]
    tails = []
    for g, m in enumerate(sizes):
        for i in range(m):
            tails.append(0 if (g == 2 and i == 1) else int(rng.integers(1, 300)))
    return sizes, pblocks, tails


def run_shared(case, ws=None):
    sp = case.spec
    out = torch.full_like(case.q, float("nan"))
    pa.pa_decode_shared(out, case.q, case.k_cache, case.v_cache,
                        torch.from_numpy(case.tables).to(DEV), torch.from_numpy(case.lens).to(DEV),
                        torch.from_numpy(case.extra["group_start"]).to(DEV),
                        torch.from_numpy(case.extra["group_prefix_len"]).to(DEV), sp.scale,
                        sp.block_size, sp.num_kv_heads, case.max_context_len, workspace=ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", sorted(SPECS))
def test_shared_parity(name):
    spec, mm = SPECS[name]
    rng = np.random.default_rng(118_500)
    sizes, pblocks, tails = layout(mm, rng)
    if spec.block_size == 32:
        pblocks = [p // 2 for p in pblocks]
    case = to_dev(W.make_shared_case(spec, sizes, pblocks, tails, device=DEV, poison=True))
    log(f"[shared] {name}: {len(case.lens)} seqs, groups {sizes}")
    out = run_shared(case)
    err = max_err(out, oracle_decode(case))
    plain = (out.double() - gpu_decode(case).double()).abs().max().item()
    log(f"  max abs err {err:.3e}, vs pa_decode {plain:.3e} (tol {TOL[spec.dtype]})")
    assert err <= TOL[spec.dtype]
    assert plain <= 2 * TOL[spec.dtype]


def test_shared_edge_lengths():
    """Members whose whole context is the prefix (empty tail), a group with
    one-block prefix and one-token tails, and an empty sequence alone."""
    spec, mm = SPECS["mha_bf16_bs16"]
    sizes = [4, 3, 1, 2]
    pblocks = [3, 1, 0, 64]
    tails = [0, 0, 1, 15, 1, 16, 17, 0, 4100, 1]
    case = to_dev(W.make_shared_case(spec, sizes, pblocks, tails, device=DEV, poison=True))
    assert case.lens[7] == 0
    out = run_shared(case)
    assert (out[7] == 0).all(), "L = 0 must give a zero row"
    err = max_err(out, oracle_decode(case))
    log(f"[shared edges] max abs err {err:.3e}")
    assert err <= TOL[spec.dtype]


def test_shared_deterministic_and_workspace_reuse():
    spec, mm = SPECS["gqa_g2_f16_mfma_tail"]
    sizes, pblocks, tails = layout(mm, np.random.default_rng(3))
    case = to_dev(W.make_shared_case(spec, sizes, pblocks, tails, device=DEV))
    need = pa.pa_decode_shared_workspace_bytes(len(case.lens), len(sizes), spec.num_q_heads,
                                               spec.num_kv_heads, spec.head_dim, spec.block_size,
                                               case.max_context_len, W.TORCH_DTYPE[spec.dtype])
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device=DEV)
    first = run_shared(case, ws)
    for _ in range(3):
        assert torch.equal(run_shared(case, ws), first)


def test_shared_validate_rejects_bad_groups():
    """PA_VALIDATE=1 (read once per process: a child process) refuses a group
    whose members do not share the claimed prefix blocks."""
    code = r'''
import numpy as np, torch
import paged_kv_cache_118_amd as pa, workloads as W
from tests.test_gpu_shared import SPECS, run_shared
spec, mm = SPECS["mha_bf16_bs16"]
case = W.make_shared_case(spec, [3], [4], [5, 6, 7], device="cuda:0")
case.tables[1, 2] = case.tables[2, 3]
try:
    run_shared(case)
    print("accepted")
except pa.PAError as e:
    print("status", e.status)
'''
    env = dict(os.environ, PA_VALIDATE="1")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=root, timeout=300)
    assert r.stdout.strip().endswith("status -5"), r.stdout + r.stderr[-2000:]


def test_shared_full_size_llama13b():
    """The whole LLaMA-13B-shaped sharing batch (32 groups of 8 sharing 512
    tokens, tails U[1, 512], 40 heads, bf16): every sequence against the
    oracle."""
    spec = W.LLAMA13B_SHARE
    _, gsize, plen, lo, hi = spec.lengths
    rng = np.random.default_rng(spec.seed)
    groups = spec.num_seqs // gsize
    tails = rng.integers(lo, hi + 1, size=spec.num_seqs)
    case = to_dev(W.make_shared_case(spec, [gsize] * groups, [plen // spec.block_size] * groups,
                                     tails, device=DEV, poison=False))
    log("[shared full size] 256 sequences")
    out = run_shared(case)
    err = max_err(out, oracle_decode(case))
    log(f"  max abs err {err:.3e}")
    assert err <= TOL[spec.dtype]
