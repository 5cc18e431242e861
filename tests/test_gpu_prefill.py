"""pa_prefill (chunked-prefill attention over the paged cache) on the GPU
against the fp64 oracle: ragged chunks and contexts, whole prompts, one-token
chunks, several 64-row tiles with a ragged tail, every supported block size,
MHA and grouped heads, NaN in every slot a chunk must not read."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_118_amd as pa
import workloads as W
from tests.gpu_util import DEV, TOL, log, max_err

pytestmark = pytest.mark.gpu


def make_prefill_case(spec, ctx, qlens, seed=0):
    """Pools holding every sequence's context (NaN elsewhere), and the query
    rows of each sequence's chunk (its last qlens[i] tokens)."""
    case = W.make_decode_case(spec.with_(num_seqs=len(ctx)), device=DEV, poison=True,
                              lens=ctx, seed=spec.seed + seed)
    T = int(sum(qlens))
    gen = W.make_generator(spec.seed + 7 + seed, DEV)
    q = W.randn((max(T, 1), spec.num_q_heads, spec.head_dim), spec.dtype, gen, DEV)[:T]
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return case, q.contiguous(), qs


def run_prefill(case, q, qs, max_context_len=None):
    sp = case.spec
    out = torch.full_like(q, float("nan"))
    pa.pa_prefill(out, q, case.k_cache, case.v_cache, torch.from_numpy(case.tables).to(DEV),
                  torch.from_numpy(case.lens).to(DEV), torch.from_numpy(qs).to(DEV), sp.scale,
                  sp.block_size, sp.num_kv_heads, int(np.diff(qs).max(initial=0)),
                  case.max_context_len if max_context_len is None else max_context_len)
    torch.cuda.synchronize()
    return out


def oracle_prefill(case, q, qs):
    sp = case.spec
    return oracle.get().prefill(W.to_numpy_bits(q), W.to_numpy_bits(case.k_cache),
                                W.to_numpy_bits(case.v_cache), case.tables, case.lens, qs,
                                sp.scale, sp.block_size, sp.num_kv_heads, sp.dtype)


SPECS = {
    "mha_f16_bs16": W.OPT66B_SWEEP.with_(num_q_heads=4, num_kv_heads=4),
    "mha_f16_bs8": W.OPT66B_SWEEP.with_(num_q_heads=2, num_kv_heads=2, block_size=8),
    "mha_bf16_bs32": W.OPT66B_SWEEP.with_(dtype="bf16", num_q_heads=2, num_kv_heads=2,
                                          block_size=32),
    "mha_f16_bs128_d64": W.OPT66B_SWEEP.with_(num_q_heads=4, num_kv_heads=4, block_size=128,
                                              head_dim=64),
    "gqa_bf16_g8_bs32": W.GQA_LONG.with_(num_q_heads=16, num_kv_heads=2),
    "gqa_f16_g4_bs16_d64": W.GQA_LONG.with_(dtype="f16", num_q_heads=8, num_kv_heads=2,
                                            block_size=16, head_dim=64),
}
# (context, chunk) pairs: whole prompts, one-token chunks, chunks of 1..4
# 64-row tiles with ragged tails, chunks starting mid-block
CASES = [(1, 1), (17, 17), (64, 64), (100, 37), (300, 1), (517, 256), (700, 129), (1030, 300)]


@pytest.mark.parametrize("name", sorted(SPECS))
def test_prefill_parity(name):
    spec = SPECS[name]
    ctx = [c for c, _ in CASES]
    ql = [q for _, q in CASES]
    log(f"[prefill parity] {name}")
    case, q, qs = make_prefill_case(spec, ctx, ql)
    out = run_prefill(case, q, qs)
    err = max_err(out, oracle_prefill(case, q, qs))
    log(f"  max abs err {err:.3e} (tol {TOL[spec.dtype]})")
    assert err <= TOL[spec.dtype]


def test_prefill_one_token_chunks_match_decode():
    """Chunks of one token are decode steps: pa_prefill and pa_decode agree
    within the tolerance (different kernels, same definition)."""
    spec = SPECS["mha_f16_bs16"]
    ctx = [5, 33, 250, 1000]
    case, q, qs = make_prefill_case(spec, ctx, [1] * len(ctx))
    out = run_prefill(case, q, qs)
    dec = torch.empty_like(q)
    pa.pa_decode(dec, q, case.k_cache, case.v_cache, torch.from_numpy(case.tables).to(DEV),
                 torch.from_numpy(case.lens).to(DEV), spec.scale, spec.block_size,
                 spec.num_kv_heads, case.max_context_len)
    torch.cuda.synchronize()
    assert (out.double() - dec.double()).abs().max().item() <= TOL[spec.dtype]


def test_prefill_chunking_consistent():
    """A prompt's last 200 tokens: as the tail of a whole-prompt chunk or as a
    chunk of their own, the outputs agree (same keys, same positions)."""
    spec = SPECS["gqa_bf16_g8_bs32"]
    ctx = [777]
    case, q, qs = make_prefill_case(spec, ctx, [777])
    whole = run_prefill(case, q, qs)
    tail = run_prefill(case, q[577:].contiguous(), np.array([0, 200], dtype=np.int32))
    assert (whole[577:].double() - tail.double()).abs().max().item() <= TOL[spec.dtype]


def test_prefill_rejects_unsupported():
    """head_dim 256 has no prefill kernel: PA_ENOTSUP before anything runs."""
    spec = SPECS["mha_f16_bs16"].with_(head_dim=256)
    case, q, qs = make_prefill_case(spec, [8], [8])
    with pytest.raises(pa.PAError) as e:
        run_prefill(case, q, qs)
    assert e.value.status == -2


@pytest.mark.parametrize("rows,waves,dma", [(16, 2, 0), (16, 4, 0), (32, 2, 0), (32, 4, 0),
                                             (32, 2, 1), (32, 4, 1)])
def test_prefill_every_workgroup_shape(rows, waves, dma, monkeypatch):
    """Each workgroup shape the library can launch (rows per wavefront x
    wavefronts x register-staged or direct LDS loads, forced through the
    tuning overrides) on ragged chunks, MHA and grouped heads, against the
    oracle."""
    monkeypatch.setenv("PA_PREFILL_ROWS", str(rows))
    monkeypatch.setenv("PA_PREFILL_WAVES", str(waves))
    monkeypatch.setenv("PA_PREFILL_DMA", str(dma))
    for name in ("mha_f16_bs16", "gqa_bf16_g8_bs32", "mha_f16_bs8", "gqa_f16_g4_bs16_d64"):
        spec = SPECS[name]
        log(f"[prefill shape] {rows}x{waves} dma={dma} {name}")
        case, q, qs = make_prefill_case(spec, [c for c, _ in CASES], [q for _, q in CASES],
                                        seed=rows + waves)
        err = max_err(run_prefill(case, q, qs), oracle_prefill(case, q, qs))
        log(f"  max abs err {err:.3e}")
        assert err <= TOL[spec.dtype]


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.01, 1.5])
@pytest.mark.parametrize("rows", [16, 32])
def test_prefill_any_scale(scale, rows, monkeypatch):
    """Scales other than 1/sqrt(D): zero (every visible key weighs the same,
    and the masked keys' -inf scores must not turn into NaN), negative (the
    kernel flips q's sign bits and keeps a positive factor), small (flat
    weights) and large (sharp weights), on both wavefront shapes, against the
    oracle at the same scale."""
    monkeypatch.setenv("PA_PREFILL_ROWS", str(rows))
    for name in ("mha_f16_bs16", "gqa_bf16_g8_bs32"):
        spec = SPECS[name]
        log(f"[prefill scale] {scale} rows {rows} {name}")
        case, q, qs = make_prefill_case(spec, [17, 300, 700], [17, 1, 129], seed=3)
        out = torch.full_like(q, float("nan"))
        pa.pa_prefill(out, q, case.k_cache, case.v_cache, torch.from_numpy(case.tables).to(DEV),
                      torch.from_numpy(case.lens).to(DEV), torch.from_numpy(qs).to(DEV), scale,
                      spec.block_size, spec.num_kv_heads, int(np.diff(qs).max()),
                      case.max_context_len)
        torch.cuda.synchronize()
        want = oracle.get().prefill(W.to_numpy_bits(q), W.to_numpy_bits(case.k_cache),
                                    W.to_numpy_bits(case.v_cache), case.tables, case.lens, qs,
                                    scale, spec.block_size, spec.num_kv_heads, spec.dtype)
        err = max_err(out, want)
        # a large scale makes the rows near single V values (|v| up to ~4.5), whose
        # storage rounding alone reaches the absolute tolerance: relative bound
        bound = TOL[spec.dtype] * max(1.0, float(np.abs(want).max()))
        log(f"  max abs err {err:.3e} (bound {bound:.3e})")
        assert err <= bound


@pytest.mark.parametrize("name,ctx", [("mha_f16_bs16", [16500, 300, 1]),
                                      ("mha_bf16_bs32", [33000, 700])])
def test_prefill_rows_longer_than_the_staged_table(name, ctx):
    """Rows of more than 1,024 blocks take their block ids through the table
    window, shorter ones from the row staged in LDS; one launch mixing both,
    against the oracle."""
    spec = SPECS[name]
    ql = [40, 30, 1][:len(ctx)]
    log(f"[prefill long rows] {name} contexts {ctx}")
    case, q, qs = make_prefill_case(spec, ctx, ql, seed=5)
    assert -(-max(ctx) // spec.block_size) > 1024
    err = max_err(run_prefill(case, q, qs), oracle_prefill(case, q, qs))
    log(f"  max abs err {err:.3e}")
    assert err <= TOL[spec.dtype]
