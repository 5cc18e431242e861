"""pa_decode on the GPU against the fp64 oracle: every kernel path (MHA on the
vector ALUs, GQA on MFMA, the generic kernel, split + reduce), ragged lengths,
block sizes, dtypes, and the closed forms / invariants of the definition."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_118_amd as pa
import workloads as W
from tests.gpu_util import DEV, TOL, gpu_decode, log, max_err, oracle_decode, to_dev

pytestmark = pytest.mark.gpu

# Reduced-size versions of the workload families: several partitions and
# 16/32-token steps per sequence, with a ragged tail.
SMALL = {
    "tiny": W.TINY,
    "opt13b_f16_bs16": W.OPT13B.with_(num_seqs=12, num_q_heads=8, num_kv_heads=8),
    "opt13b_f16_bs8": W.OPT13B.with_(num_seqs=8, num_q_heads=4, num_kv_heads=4, block_size=8),
    "opt13b_f16_bs32": W.OPT13B.with_(num_seqs=8, num_q_heads=4, num_kv_heads=4, block_size=32),
    "opt13b_f16_bs128": W.OPT13B.with_(num_seqs=8, num_q_heads=4, num_kv_heads=4,
                                       block_size=128),
    "llama_bf16_bs16": W.OPT13B.with_(dtype="bf16", num_seqs=8, num_q_heads=6, num_kv_heads=6),
    "mha_f32_d128": W.OPT13B.with_(dtype="f32", num_seqs=6, num_q_heads=4, num_kv_heads=4),
    "mha_f16_d64": W.OPT13B.with_(num_seqs=6, num_q_heads=4, num_kv_heads=4, head_dim=64),
    "mha_bf16_d256": W.OPT13B.with_(dtype="bf16", num_seqs=5, num_q_heads=2, num_kv_heads=2,
                                    head_dim=256),
    "gqa_bf16_g8_bs32": W.GQA_LONG.with_(num_seqs=3, num_q_heads=16, num_kv_heads=2,
                                         lengths=("uniform", 700, 3000)),
    "gqa_f16_g4_bs16": W.GQA_LONG.with_(dtype="f16", num_seqs=4, num_q_heads=8, num_kv_heads=2,
                                        block_size=16, lengths=("uniform", 1, 2500)),
    "gqa_bf16_g8_bs8": W.GQA_LONG.with_(num_seqs=3, num_q_heads=8, num_kv_heads=1, block_size=8,
                                        lengths=("uniform", 1, 1500)),
    "gqa_bf16_g16_d64": W.GQA_LONG.with_(num_seqs=3, num_q_heads=32, num_kv_heads=2, head_dim=64,
                                         block_size=128, lengths=("uniform", 1, 2000)),
    "gqa_f16_g16_d128_bs32": W.GQA_LONG.with_(dtype="f16", num_seqs=3, num_q_heads=32,
                                              num_kv_heads=2, lengths=("uniform", 1, 3000)),
    "gqa_f32_g4_generic_path": W.GQA_LONG.with_(dtype="f32", num_seqs=3, num_q_heads=8,
                                                num_kv_heads=2, lengths=("uniform", 1, 700)),
    "mha_f16_d32_bs4_generic": W.OPT13B.with_(num_seqs=4, num_q_heads=2, num_kv_heads=2,
                                              head_dim=32, block_size=4,
                                              lengths=("uniform", 1, 300)),
    "gqa_g2_f16": W.GQA_LONG.with_(dtype="f16", num_seqs=3, num_q_heads=4, num_kv_heads=2,
                                   block_size=16, lengths=("uniform", 1, 1200)),
    "gqa_g3_bf16": W.GQA_LONG.with_(num_seqs=3, num_q_heads=6, num_kv_heads=2,
                                    lengths=("uniform", 1, 1500)),
    # D 256 has no MFMA kernel: a GQA group on the VALU path
    "gqa_g2_bf16_d256_valu": W.OPT13B.with_(dtype="bf16", num_seqs=4, num_q_heads=4,
                                            num_kv_heads=2, head_dim=256,
                                            lengths=("uniform", 1, 900)),
}


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("part", [0, -1, 256])
def test_decode_parity(name, part):
    spec = SMALL[name]
    log(f"[decode parity] {name} partition={part}")
    case = to_dev(W.make_decode_case(spec, device=DEV, poison=True))
    out = gpu_decode(case, partition_size=part)
    err = max_err(out, oracle_decode(case))
    log(f"  max abs err {err:.3e} (tol {TOL[spec.dtype]})")
    assert err <= TOL[spec.dtype]


EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025,
             4100]


@pytest.mark.parametrize("spec_name", ["opt13b_f16_bs16", "opt13b_f16_bs8", "gqa_bf16_g8_bs32",
                                       "gqa_bf16_g8_bs8", "opt13b_f16_bs128"])
@pytest.mark.parametrize("part", [0, -1, 512])
def test_decode_edge_lengths(spec_name, part):
    """Empty sequence, one token, block / step / partition boundaries +-1, and a
    sequence long enough to reload the block-table window (> 64 blocks)."""
    spec = SMALL[spec_name].with_(num_seqs=len(EDGE_LENS))
    log(f"[edge lengths] {spec_name} partition={part}")
    case = to_dev(W.make_decode_case(spec, device=DEV, poison=True, lens=EDGE_LENS))
    out = gpu_decode(case, partition_size=part)
    assert (out[0] == 0).all(), "L = 0 must give a zero row"
    err = max_err(out, oracle_decode(case))
    log(f"  max abs err {err:.3e}")
    assert err <= TOL[spec.dtype]


def test_max_context_len_larger_than_needed():
    spec = SMALL["gqa_bf16_g8_bs32"]
    case = to_dev(W.make_decode_case(spec, device=DEV))
    out = gpu_decode(case, partition_size=512, max_context_len=case.max_context_len + 5000)
    assert max_err(out, oracle_decode(case)) <= TOL[spec.dtype]


@pytest.mark.parametrize("spec_name", ["opt13b_f16_bs16", "gqa_bf16_g8_bs32", "mha_f32_d128",
                                       "tiny"])
def test_single_key_returns_v0_exactly(spec_name):
    """L = 1: the weight is exp2(0) / exp2(0) = 1, so the output is v_0 rounded
    to the output dtype -- here v_0 itself, bit for bit."""
    spec = SMALL[spec_name]
    B = spec.num_seqs
    case = to_dev(W.make_decode_case(spec, device=DEV, lens=[1] * B))
    out = gpu_decode(case)
    bs, vs = spec.block_size, W.v_slab(spec.block_size)
    G = spec.num_q_heads // spec.num_kv_heads
    for b in range(B):
        blk = int(case.tables[b, 0])
        v0 = case.v_cache[blk, :, 0, :, 0]  # [Hkv][D] of offset 0
        want = v0.repeat_interleave(G, dim=0)
        assert torch.equal(out[b], want), f"seq {b}"


@pytest.mark.parametrize("spec_name", ["opt13b_f16_bs16", "gqa_bf16_g8_bs32"])
def test_constant_v_returns_constant(spec_name):
    spec = SMALL[spec_name]
    case = to_dev(W.make_decode_case(spec, device=DEV, poison=False))
    c = W.randn((spec.num_kv_heads, spec.head_dim), spec.dtype, W.make_generator(5, DEV), DEV)
    vs = W.v_slab(spec.block_size)
    # every slot of every block holds c for its head: [nb][Hkv][BS/VS][D][VS]
    case.v_cache[:] = c[None, :, None, :, None]
    out = gpu_decode(case, partition_size=256)
    G = spec.num_q_heads // spec.num_kv_heads
    want = c.repeat_interleave(G, dim=0).double()
    err = (out.double() - want[None]).abs().max().item()
    assert err <= TOL[spec.dtype]


@pytest.mark.parametrize("spec_name", ["opt13b_f16_bs16", "gqa_bf16_g8_bs32", "opt13b_f16_bs8"])
def test_physical_permutation_bitwise_invariant(spec_name):
    """Same logical K/V at different physical blocks: the kernels' reduction
    order depends only on logical position, so the output is bit-identical."""
    spec = SMALL[spec_name]
    a = to_dev(W.make_decode_case(spec, device=DEV, poison=True))
    rng = np.random.default_rng(99)
    nb = a.num_blocks + 17
    perm = rng.permutation(nb)[: a.num_blocks]  # old block i -> new block perm[i]
    k2 = torch.full((nb,) + tuple(a.k_cache.shape[1:]), float("nan"), dtype=a.k_cache.dtype,
                    device=DEV)
    v2 = torch.full((nb,) + tuple(a.v_cache.shape[1:]), float("nan"), dtype=a.v_cache.dtype,
                    device=DEV)
    pidx = torch.from_numpy(perm).to(DEV)
    k2[pidx] = a.k_cache
    v2[pidx] = a.v_cache
    t2 = np.where(a.tables >= 0, perm[np.maximum(a.tables, 0)], -1).astype(np.int32)
    b = W.DecodeCase(spec, a.lens, t2, nb, a.q, k2, v2)
    for part in (0, -1):
        assert torch.equal(gpu_decode(a, part), gpu_decode(b, part))


@pytest.mark.parametrize("bs", [8, 16, 32, 128])
def test_contiguous_layout_matches_shuffled(bs):
    """The paged-vs-contiguous sweep's two layouts: every sequence one
    contiguous run of the pool, or the same logical blocks at shuffled ids.
    Outputs are bitwise identical, and equal to the oracle within tolerance."""
    spec = SMALL["opt13b_f16_bs16"].with_(block_size=bs, num_seqs=5)
    lens = [1, bs - 1, 3 * bs + 5, 700, 1500]
    ct, nb = W.contiguous_tables(lens, bs)
    gen = W.make_generator(1181, DEV)
    H, D = spec.num_kv_heads, spec.head_dim
    k = W.randn(W.k_pool_shape(nb, H, bs, D, spec.dtype), spec.dtype, gen, DEV)
    v = W.randn(W.v_pool_shape(nb, H, bs, D), spec.dtype, gen, DEV)
    q = W.randn((len(lens), spec.num_q_heads, D), spec.dtype, gen, DEV)
    a = W.DecodeCase(spec, np.asarray(lens, dtype=np.int32), ct, nb, q, k, v)
    perm = np.random.default_rng(bs).permutation(nb).astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(nb, dtype=np.int32)
    idx = torch.from_numpy(inv.astype(np.int64)).to(DEV)
    st = np.where(ct >= 0, perm[np.maximum(ct, 0)], -1).astype(np.int32)
    b = W.DecodeCase(spec, a.lens, st, nb, q, k.index_select(0, idx), v.index_select(0, idx))
    log(f"[contiguous vs shuffled] bs={bs}")
    for part in (0, -1):
        oa = gpu_decode(a, part)
        assert torch.equal(oa, gpu_decode(b, part))
        assert max_err(oa, oracle_decode(a)) <= TOL[spec.dtype]


def test_nan_in_masked_slots_does_not_leak():
    spec = SMALL["opt13b_f16_bs16"]
    a = to_dev(W.make_decode_case(spec, device=DEV, poison=True))
    b = to_dev(W.make_decode_case(spec, device=DEV, poison=False))
    # same valid data: copy b's values, then re-poison
    oa, ob = gpu_decode(a), gpu_decode(b)
    assert torch.isfinite(oa).all()
    assert torch.equal(oa, ob)


@pytest.mark.parametrize("spec_name", ["opt13b_f16_bs16", "gqa_bf16_g8_bs32", "llama_bf16_bs16"])
def test_split_and_unsplit_agree(spec_name):
    spec = SMALL[spec_name]
    case = to_dev(W.make_decode_case(spec, device=DEV))
    a = gpu_decode(case, partition_size=-1).double()
    b = gpu_decode(case, partition_size=256).double()
    assert (a - b).abs().max().item() <= TOL[spec.dtype]


def test_gqa_equals_repeated_mha():
    """Hq = 8 over Hkv = 1 (MFMA path) equals Hq = Hkv = 8 with the kv head
    repeated (vector-ALU path), within the dtype tolerance."""
    g = SMALL["gqa_bf16_g8_bs32"].with_(num_q_heads=8, num_kv_heads=1)
    case = to_dev(W.make_decode_case(g, device=DEV))
    m = g.with_(num_kv_heads=8)
    rep = W.DecodeCase(m, case.lens, case.tables, case.num_blocks, case.q,
                       case.k_cache.repeat_interleave(8, dim=1).contiguous(),
                       case.v_cache.repeat_interleave(8, dim=1).contiguous())
    a = gpu_decode(case).double()
    b = gpu_decode(rep).double()
    assert (a - b).abs().max().item() <= TOL["bf16"]


def test_run_to_run_deterministic():
    spec = SMALL["gqa_bf16_g8_bs32"]
    case = to_dev(W.make_decode_case(spec, device=DEV))
    x = gpu_decode(case, 256)
    for _ in range(3):
        assert torch.equal(x, gpu_decode(case, 256))


def test_per_block_softmax_mutant_is_rejected():
    """Negative control: the per-block-softmax reading (rejected by the pages)
    differs from the kernel by far more than the tolerance."""
    spec = SMALL["opt13b_f16_bs16"]
    case = to_dev(W.make_decode_case(spec, device=DEV))
    out = gpu_decode(case)
    mutant = oracle.build_mutant(1)
    err = max_err(out, oracle_decode(case, orc=mutant))
    assert err > 50 * TOL[spec.dtype]


def test_bad_table_ids_do_not_fault():
    """Out-of-range block ids are clamped inside the kernels (no fault); the
    rows of the other sequences are unaffected."""
    spec = SMALL["opt13b_f16_bs16"]
    case = to_dev(W.make_decode_case(spec, device=DEV))
    good = gpu_decode(case)
    t = case.tables.copy()
    t[0, 0] = 10**9
    t[1, 0] = -7
    bad = W.DecodeCase(spec, case.lens, t, case.num_blocks, case.q, case.k_cache, case.v_cache)
    out = gpu_decode(bad)
    assert torch.equal(out[2:], good[2:])


def test_stream_argument_is_honoured():
    spec = SMALL["gqa_bf16_g8_bs32"]
    case = to_dev(W.make_decode_case(spec, device=DEV))
    ref = gpu_decode(case)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = gpu_decode(case, stream=s)
    assert torch.equal(out, ref)


def test_host_workspace_and_foreign_stream_refused():
    """A workspace in host memory, or a stream of another device than the
    tensors', is refused before anything runs (the kernels would dereference
    the workspace on the device); the output is left untouched."""
    import paged_kv_cache_118_amd as pa
    spec = SMALL["opt13b_f16_bs16"]
    case = to_dev(W.make_decode_case(spec, device=DEV))
    sp = case.spec
    nbytes = pa.pa_decode_workspace_bytes(len(case.lens), sp.num_q_heads, sp.num_kv_heads,
                                          sp.head_dim, sp.block_size, case.max_context_len, 0,
                                          case.q.dtype)
    assert nbytes > 0
    out = torch.full_like(case.q, 7.0)
    args = (out, case.q, case.k_cache, case.v_cache, torch.from_numpy(case.tables).to(DEV),
            torch.from_numpy(case.lens).to(DEV), sp.scale, sp.block_size, sp.num_kv_heads,
            case.max_context_len)
    with pytest.raises(ValueError):
        pa.pa_decode(*args, workspace=torch.empty(nbytes, dtype=torch.uint8))

    class OtherDeviceStream(torch.cuda.Stream):
        @property
        def device(self):
            return torch.device("cuda", 1)
    with pytest.raises(ValueError):
        pa.pa_decode(*args, stream=OtherDeviceStream())
    torch.cuda.synchronize()
    assert (out == 7.0).all()


def _decode_ws(case, part, ws):
    c = case
    sp = c.spec
    out = torch.empty_like(c.q)
    import paged_kv_cache_118_amd as pa
    pa.pa_decode(out, c.q, c.k_cache, c.v_cache, torch.from_numpy(c.tables).to(DEV),
                 torch.from_numpy(c.lens).to(DEV), sp.scale, sp.block_size, sp.num_kv_heads,
                 c.max_context_len, partition_size=part, workspace=ws)
    torch.cuda.synchronize()
    return out


def test_workspace_reused_across_shapes():
    """One workspace (starting as garbage) serves a sequence of calls with
    other shapes and split modes in between: every call equals the same call
    on a fresh workspace, bit for bit (nothing a call leaves behind is read by
    the next)."""
    import paged_kv_cache_118_amd as pa
    names = ["opt13b_f16_bs16", "gqa_bf16_g8_bs32", "llama_bf16_bs16", "gqa_f16_g4_bs16"]
    cases = {n: to_dev(W.make_decode_case(SMALL[n], device=DEV)) for n in names}
    need = 0
    for n, c in cases.items():
        sp = c.spec
        for part in (0, 256):
            need = max(need, pa.pa_decode_workspace_bytes(
                len(c.lens), sp.num_q_heads, sp.num_kv_heads, sp.head_dim, sp.block_size,
                c.max_context_len, part, W.TORCH_DTYPE[sp.dtype]))
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device=DEV)  # garbage, not zeros
    fresh = {(n, p): gpu_decode(c, partition_size=p) for n, c in cases.items() for p in (0, 256)}
    order = [(n, p) for _ in range(3) for n in names for p in (0, 256)]
    for n, p in order:
        log(f"[ws reuse] {n} partition={p}")
        assert torch.equal(_decode_ws(cases[n], p, ws), fresh[(n, p)])


@pytest.mark.parametrize("spec_name", ["opt13b_f16_bs16", "gqa_bf16_g8_bs32"])
def test_item_shared_by_many_workers(spec_name):
    """A 32k-token sequence with 256-token partitions: each item is shared by
    128 wavefronts, whose partials the merge combines."""
    spec = SMALL[spec_name].with_(num_seqs=2)
    log(f"[many workers] {spec_name}")
    case = to_dev(W.make_decode_case(spec, device=DEV, lens=[32768, 300]))
    out = gpu_decode(case, partition_size=256)
    err = max_err(out, oracle_decode(case))
    log(f"  max abs err {err:.3e}")
    assert err <= TOL[spec.dtype]


@pytest.mark.parametrize("spec_name,part", [("opt13b_f16_bs16", 0), ("opt13b_f16_bs16", 512),
                                            ("gqa_bf16_g8_bs32", 0), ("gqa_bf16_g8_bs32", 256),
                                            ("gqa_f16_g4_bs16", 512)])
def test_workspace_same_layout_many_calls(spec_name, part):
    """Calls with one layout reuse one workspace (starting as garbage).
    Lengths change every call, so the slots an item's pieces use move, and
    slots left over from the previous call sit between them; every call must
    equal the same call on a fresh workspace, bit for bit, and the oracle
    within tolerance."""
    import paged_kv_cache_118_amd as pa
    spec = SMALL[spec_name]
    cap = 3000
    rng = np.random.default_rng(1180 + part)
    need = pa.pa_decode_workspace_bytes(spec.num_seqs, spec.num_q_heads, spec.num_kv_heads,
                                        spec.head_dim, spec.block_size, cap, part,
                                        W.TORCH_DTYPE[spec.dtype])
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device=DEV)
    for call in range(6):
        lens = rng.integers(1, cap + 1, size=spec.num_seqs)
        if call == 3:
            lens[::2] = rng.integers(1, 40, size=len(lens[::2]))  # many short items
        case = to_dev(W.make_decode_case(spec.with_(seed=spec.seed + call), device=DEV,
                                         lens=list(lens)))
        log(f"[ws same layout] {spec_name} partition={part} call {call}")
        out = torch.empty_like(case.q)
        pa.pa_decode(out, case.q, case.k_cache, case.v_cache,
                     torch.from_numpy(case.tables).to(DEV), torch.from_numpy(case.lens).to(DEV),
                     spec.scale, spec.block_size, spec.num_kv_heads, cap, partition_size=part,
                     workspace=ws)
        fresh = gpu_decode(case, partition_size=part, max_context_len=cap)
        assert torch.equal(out, fresh)
        assert max_err(out, oracle_decode(case)) <= TOL[spec.dtype]


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.01, 1.5])
@pytest.mark.parametrize("spec_name", ["opt13b_f16_bs16", "gqa_bf16_g8_bs32",
                                       "mha_f16_d32_bs4_generic"])
@pytest.mark.parametrize("part", [0, 512])
def test_decode_any_scale(scale, spec_name, part, orc):
    """Scales other than 1/sqrt(D) -- zero (the mean of V), negative, small
    (flat weights), large (sharp weights) -- on the VALU, MFMA and generic
    kernels, split and partitioned, against the oracle at the same scale."""
    spec = SMALL[spec_name]
    log(f"[decode scale] {scale} {spec_name} partition={part}")
    c = to_dev(W.make_decode_case(spec, device=DEV, poison=True))
    out = torch.empty_like(c.q)
    pa.pa_decode(out, c.q, c.k_cache, c.v_cache, torch.from_numpy(c.tables).to(DEV),
                 torch.from_numpy(c.lens).to(DEV), scale, spec.block_size, spec.num_kv_heads,
                 c.max_context_len, partition_size=part)
    torch.cuda.synchronize()
    from tests.gpu_util import subset_for_oracle
    qb, kb, vb, t, lens = subset_for_oracle(c, range(len(c.lens)))
    want = orc.decode(qb, kb, vb, t, lens, scale, spec.block_size, spec.num_kv_heads, spec.dtype)
    err = max_err(out, want)
    # a large scale makes the rows near single V values (|v| up to ~4.5), whose
    # storage rounding alone reaches the absolute tolerance: relative bound
    bound = TOL[spec.dtype] * max(1.0, float(np.abs(want).max()))
    log(f"  max abs err {err:.3e} (bound {bound:.3e})")
    assert err <= bound
