"""Seeded synthetic inputs for the paged decode path.

This module is shared by the test suite, the benchmark and the smoke check.
It draws random numbers and builds input *structure* (sequence lengths,
shuffled physical block ids, block tables, slot lists for given positions,
pool contents); it holds none of the attention or block-manager arithmetic.

Workloads are shaped after the setups on the pages (OPT-13B / 66B and
LLaMA-13B models, request lengths drawn from a distribution rather than a
dataset); no dataset item is reproduced.  Values are N(0, 1) drawn in fp32 and
rounded to the storage dtype (round-to-nearest-even).

Pool layout (shapes only; the index formula is documented in include/pa.h):
  K: [num_blocks][Hkv][D/X][BS][X],  X = 16 / element size (16-byte pieces)
  V: [num_blocks][Hkv][BS/VS][D][VS],  VS = min(BS, 8)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def v_slab(block_size: int) -> int:
    return block_size if block_size < 8 else 8


ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def k_piece(dtype: str) -> int:
    """Dims per 16-byte K piece."""
    return 16 // ELEM_BYTES[dtype]


def k_pool_shape(num_blocks, num_kv_heads, block_size, head_dim, dtype):
    x = k_piece(dtype)
    return (num_blocks, num_kv_heads, head_dim // x, block_size, x)


def v_pool_shape(num_blocks, num_kv_heads, block_size, head_dim):
    vs = v_slab(block_size)
    return (num_blocks, num_kv_heads, block_size // vs, head_dim, vs)


@dataclass(frozen=True)
class Spec:
    """One workload family.  ``lengths`` is (kind, *params)."""
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_seqs: int
    lengths: tuple
    pool_factor: float = 1.25
    pool_blocks: int | None = None  # fixed pool size overrides pool_factor
    partition_size: int = 0         # 0 = library default
    seed: int = 118_000

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "Spec":
        d = dict(self.__dict__)
        d.update(kw)
        return Spec(**d)


# The five workload families (the first is the tiny worked example).
TINY = Spec("tiny", "f32", 2, 2, 16, 4, 2, ("fixed", (5, 9)), pool_blocks=8, seed=118_000)
OPT13B = Spec("opt13b_decode", "f16", 40, 40, 128, 16, 64, ("lognormal", 350.0, 1.0, 16, 2048),
              seed=118_001)
LLAMA13B_SHARE = Spec("llama13b_prefix_share", "bf16", 40, 40, 128, 16, 256,
                      ("share", 8, 512, 1, 512), seed=118_002)
GQA_LONG = Spec("gqa_long", "bf16", 64, 8, 128, 32, 32, ("uniform", 16384, 32768),
                partition_size=512, seed=118_003)
OPT66B_SWEEP = Spec("opt66b_sweep", "f16", 72, 72, 128, 16, 128, ("uniform", 1, 8192),
                    seed=118_004)
SPECS = {s.name: s for s in (TINY, OPT13B, LLAMA13B_SHARE, GQA_LONG, OPT66B_SWEEP)}


def draw_lengths(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    kind = spec.lengths[0]
    if kind == "fixed":
        lens = np.array(spec.lengths[1], dtype=np.int64)
    elif kind == "lognormal":  # median m, sigma s, clipped to [lo, hi]
        _, m, s, lo, hi = spec.lengths
        z = rng.standard_normal(spec.num_seqs)
        lens = np.clip(np.rint(np.exp(math.log(m) + s * z)), lo, hi).astype(np.int64)
    elif kind == "uniform":  # inclusive integer range
        _, lo, hi = spec.lengths
        lens = rng.integers(lo, hi + 1, size=spec.num_seqs)
    else:
        raise ValueError(kind)
    return lens.astype(np.int32)


def blocks_needed(length: int, block_size: int) -> int:
    return -(-int(length) // block_size)


def shuffled_tables(lens, block_size, rng, pool_factor=1.25, num_blocks=None, max_blocks=None):
    """Random block tables: each sequence gets ceil(L / BS) distinct physical
    ids drawn from a shuffled pool of ``num_blocks`` (default pool_factor x the
    blocks required).  Unused entries are -1."""
    need = [blocks_needed(L, block_size) for L in lens]
    total = int(sum(need))
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(pool_factor * total)))
    if total > num_blocks:
        raise ValueError("pool too small")
    if max_blocks is None:
        max_blocks = max(1, max(need) if need else 1)
    perm = rng.permutation(num_blocks)
    tables = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    cursor = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[cursor:cursor + n]
        cursor += n
    return tables, int(num_blocks)


def contiguous_tables(lens, block_size, max_blocks=None):
    """Identity-like tables: sequence i's logical blocks are the consecutive
    physical ids starting after sequence i-1's, so every sequence is one
    contiguous run of the pool (the layout a non-paged cache would have).
    Returns (tables, num_blocks)."""
    need = [blocks_needed(L, block_size) for L in lens]
    if max_blocks is None:
        max_blocks = max(1, max(need) if need else 1)
    tables = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    cursor = 0
    for i, n in enumerate(need):
        tables[i, :n] = np.arange(cursor, cursor + n, dtype=np.int32)
        cursor += n
    return tables, max(1, cursor)


def shared_prefix_tables(group_sizes, prefix_blocks, tail_lens, block_size, rng,
                         pool_factor=1.25):
    """Tables of consecutive groups of sequences that share leading blocks:
    group g's members (group_sizes[g] of them, in order) all start with the
    same prefix_blocks[g] physical blocks (full), then each has its own
    blocks for its tail_lens[i] further positions.  Physical ids come from a
    seeded shuffle of a pool of pool_factor x the distinct blocks needed.
    Returns (tables int32 [B][max_blocks] -1 padded, lens int32 [B],
    num_blocks, group_start int32 [G+1], group_prefix_len int32 [G])."""
    group_sizes = [int(x) for x in group_sizes]
    B = sum(group_sizes)
    tail_lens = [int(x) for x in tail_lens]
    assert len(tail_lens) == B and len(prefix_blocks) == len(group_sizes)
    need = sum(int(p) for p in prefix_blocks) + sum(blocks_needed(t, block_size) for t in tail_lens)
    num_blocks = max(1, int(math.ceil(pool_factor * need)))
    perm = list(rng.permutation(num_blocks))
    lens = np.zeros(B, dtype=np.int32)
    rows = []
    b = 0
    starts = [0]
    for g, m in enumerate(group_sizes):
        pre = [int(perm.pop()) for _ in range(int(prefix_blocks[g]))]
        for _ in range(m):
            own = [int(perm.pop()) for _ in range(blocks_needed(tail_lens[b], block_size))]
            rows.append(pre + own)
            lens[b] = int(prefix_blocks[g]) * block_size + tail_lens[b]
            b += 1
        starts.append(b)
    maxb = max(1, max(len(r) for r in rows))
    tables = np.full((B, maxb), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = r
    return (tables, lens, num_blocks, np.array(starts, dtype=np.int32),
            np.array([int(p) * block_size for p in prefix_blocks], dtype=np.int32))


def make_shared_case(spec: Spec, group_sizes, prefix_blocks, tail_lens, device="cpu",
                     poison=True, seed=None):
    """A decode case on shared_prefix_tables: q, K, V ~ N(0, 1) drawn as in
    make_decode_case.  The groups travel in extra["group_start"] and
    extra["group_prefix_len"]."""
    seed = spec.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    tables, lens, nb, gs, gp = shared_prefix_tables(group_sizes, prefix_blocks, tail_lens,
                                                    spec.block_size, rng, spec.pool_factor)
    gen = make_generator(seed, device)
    hq, hkv, D, bs = spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    q = randn((len(lens), hq, D), spec.dtype, gen, device)
    k = randn(k_pool_shape(nb, hkv, bs, D, spec.dtype), spec.dtype, gen, device)
    v = randn(v_pool_shape(nb, hkv, bs, D), spec.dtype, gen, device)
    if poison:
        poison_unused(k, v, tables, lens, bs)
    return DecodeCase(spec, lens, tables, nb, q, k, v,
                      {"group_start": gs, "group_prefix_len": gp})


def slots_for_positions(tables: np.ndarray, seq_pos, block_size: int) -> np.ndarray:
    """Slot of each (seq, position) pair: physical block * BS + offset."""
    out = np.empty(len(seq_pos), dtype=np.int64)
    for i, (s, p) in enumerate(seq_pos):
        out[i] = int(tables[s, p // block_size]) * block_size + p % block_size
    return out


def randn(shape, dtype: str, gen: torch.Generator, device) -> torch.Tensor:
    """N(0, 1) in fp32, rounded to ``dtype``; filled in chunks to bound memory."""
    out = torch.empty(shape, dtype=TORCH_DTYPE[dtype], device=device)
    flat = out.view(-1)
    chunk = 1 << 26
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
    return out


def make_generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def poison_unused(k_cache, v_cache, tables, lens, block_size):
    """Set every pool position that holds no valid token to NaN: blocks no
    table references and the unfilled tail of each sequence's last block."""
    nb = k_cache.shape[0]
    used = np.zeros(nb, dtype=bool)
    vs = v_slab(block_size)
    for i, L in enumerate(lens):
        n = blocks_needed(L, block_size)
        used[tables[i, :n]] = True
    unused = torch.from_numpy(np.nonzero(~used)[0]).to(k_cache.device)
    if unused.numel():
        k_cache[unused] = float("nan")
        v_cache[unused] = float("nan")
    for i, L in enumerate(lens):
        n = blocks_needed(L, block_size)
        if n == 0:
            continue
        blk = int(tables[i, n - 1])
        for off in range(int(L) - (n - 1) * block_size, block_size):
            k_cache[blk, :, :, off, :] = float("nan")
            v_cache[blk, :, off // vs, :, off % vs] = float("nan")


@dataclass
class DecodeCase:
    spec: Spec
    lens: np.ndarray            # int32 [B]
    tables: np.ndarray          # int32 [B][max_blocks], -1 padded
    num_blocks: int
    q: torch.Tensor             # [B][Hq][D]
    k_cache: torch.Tensor       # K pool shape
    v_cache: torch.Tensor       # V pool shape
    extra: dict = field(default_factory=dict)

    @property
    def max_context_len(self) -> int:
        return int(self.lens.max()) if len(self.lens) else 0


def make_decode_case(spec: Spec, device="cpu", poison=True, lens=None, seed=None,
                     num_blocks=None) -> DecodeCase:
    """Pool pre-filled with N(0, 1) K/V, random shuffled tables, random q."""
    seed = spec.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = draw_lengths(spec, rng)
    lens = np.asarray(lens, dtype=np.int32)
    if num_blocks is None:
        num_blocks = spec.pool_blocks
    tables, nb = shuffled_tables(lens, spec.block_size, rng, spec.pool_factor, num_blocks)
    gen = make_generator(seed, device)
    B, hq, hkv, D, bs = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, \
        spec.block_size
    B = len(lens)
    q = randn((B, hq, D), spec.dtype, gen, device)
    k = randn(k_pool_shape(nb, hkv, bs, D, spec.dtype), spec.dtype, gen, device)
    v = randn(v_pool_shape(nb, hkv, bs, D), spec.dtype, gen, device)
    if poison:
        poison_unused(k, v, tables, lens, bs)
    return DecodeCase(spec, lens, tables, nb, q, k, v)


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy for the oracle: fp32 as float32, 16-bit types as uint16 bits."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def new_token_rows(num_tokens, num_kv_heads, head_dim, dtype, gen, device):
    """K and V rows [T][Hkv][D] for tokens about to be written."""
    k = randn((num_tokens, num_kv_heads, head_dim), dtype, gen, device)
    v = randn((num_tokens, num_kv_heads, head_dim), dtype, gen, device)
    return k, v


def share_prompts(spec: Spec, rng: np.random.Generator, vocab: int = 32000):
    """Prompts of a prefix-sharing workload, lengths ("share", group, prefix,
    lo, hi): num_seqs / group groups, each with its own random prefix of
    ``prefix`` token ids, and every member with its own random tail of
    U[lo, hi] ids; returned in a random arrival order as (list of int32
    arrays, group of each prompt, tail length of each prompt)."""
    _, group, plen, lo, hi = spec.lengths
    G = spec.num_seqs // group
    prefixes = [rng.integers(0, vocab, size=plen).astype(np.int32) for _ in range(G)]
    groups = np.repeat(np.arange(G), group)
    tails = rng.integers(lo, hi + 1, size=len(groups)).astype(np.int32)
    order = rng.permutation(len(groups))
    groups, tails = groups[order], tails[order]
    prompts = [np.concatenate([prefixes[g], rng.integers(0, vocab, size=t).astype(np.int32)])
               for g, t in zip(groups, tails)]
    return prompts, groups.astype(np.int32), tails


class ShareKV:
    """K / V rows of the prefix-sharing prompts: row (prompt i, position p) is
    the group's prefix row p for p < prefix, else prompt i's own tail row.
    Every prompt of a group thus has the same K / V over the shared prefix,
    as a model would compute for equal tokens, and its own afterwards."""

    def __init__(self, spec: Spec, groups, tails, gen, device, plen: int):
        hkv, D, dt = spec.num_kv_heads, spec.head_dim, spec.dtype
        G = int(groups.max()) + 1 if len(groups) else 0
        self.plen, self.groups = plen, torch.from_numpy(np.asarray(groups, np.int64)).to(device)
        mt = max(1, int(np.max(tails)) if len(tails) else 1)
        self.pk = randn((G, plen, hkv, D), dt, gen, device)
        self.pv = randn((G, plen, hkv, D), dt, gen, device)
        self.tk = randn((len(groups), mt + 1, hkv, D), dt, gen, device)
        self.tv = randn((len(groups), mt + 1, hkv, D), dt, gen, device)

    def rows(self, prompt_idx, positions):
        """(K, V) rows [T][Hkv][D] for the given prompt indices and positions
        (int64 device tensors)."""
        pre = positions < self.plen
        g = self.groups[prompt_idx]
        pp = positions.clamp(max=self.plen - 1)
        tp = (positions - self.plen).clamp(min=0)
        m = pre[:, None, None]
        k = torch.where(m, self.pk[g, pp], self.tk[prompt_idx, tp])
        v = torch.where(m, self.pv[g, pp], self.tv[prompt_idx, tp])
        return k.contiguous(), v.contiguous()
