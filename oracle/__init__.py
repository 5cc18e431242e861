"""Reference oracle for the paged decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it: ``pa_oracle.c`` re-implements the pool layout from its
written definition, and ``alloc_ref.py`` re-implements the block manager from
the pages' description.

What each function follows (web pages on PagedAttention):

* ``decode`` -- the Z / o equations in section 二 ("分块以后，注意力仍需对整个
  历史归一化") of wq-win.github.io "079 | vLLM 与 PagedAttention": one softmax
  denominator over every valid position of every block, the unfilled tail of
  the last block excluded; gathering through the block table as in section 3
  of gitcode.csdn.net "vLLM 推理引擎：PagedAttention 与 KVCache 管理".
  Pinned by: closed forms (single key, constant V, zero K, a 3-token example
  with weights 1:2:4), numpy dense attention on identity tables, invariants
  (physical permutation, block size, NaN in masked slots, GQA == repeated MHA)
  and mutation tests.
* ``prefill`` -- chunked prefill, section 4.2 ("Chunked Prefill的解决方案") of
  the zhy-blog.vercel.app vLLM post: a chunk's query tokens are the last ones
  of their sequence's context and attend causally (mask by position in the
  whole prompt) through the block table.  Pinned by: one-token chunks equal
  the decode oracle bit for bit; the first prompt token returns v_0; a whole
  prompt equals numpy dense causal attention; a prompt's last tokens do not
  depend on how the earlier part was chunked; mutation tests (no causal mask,
  mask off by one).
* ``reshape_and_cache`` -- slot = physical block * block_size + offset, the
  flat slot numbering of the kernel pseudocode on vkads.cloudxian.cn "vLLM
  PagedAttention源码：KV Cache".  Pinned by the one-head, one-piece special
  case (head_dim 4 in fp32: the K pool, and the V pool with its slabs turned
  back into rows, are [slot][D] tables) and by write-then-decode round trips
  against numpy dense attention.
* ``copy_blocks`` -- copy-on-write of whole blocks, section 二 "共享与写时复制"
  of the wq-win page.  Pinned by byte identity of the copied block, untouched
  bytes elsewhere, and decode through the copy.
* ``swap_blocks`` -- whole-block copies between two pools (device and host),
  the "Swap 机制" part of deepinsea.top "PagedAttention 内存管理深度解析".
  Pinned by byte identity of every moved block, untouched bytes elsewhere in
  the destination, and a swap-out / swap-in round trip that restores the
  original pool's blocks at new ids.
* ``alloc_ref.BlockPool`` -- ref-counted pool per section 三 of the wq-win page
  and the BlockManager of deepinsea.top "PagedAttention 内存管理深度解析".
  Pinned by the two worked allocation examples of the wq-win page (stored in
  ``tests/golden/``) and by the tail-waste bound of its section 二.
* ``alloc_ref.PrefixCachingPool`` -- automatic prefix caching, section 2.2 (5)
  of the zhy-blog.vercel.app vLLM post (blocks keyed by their tokens and all
  tokens before them, reused by later requests) and question 2 of the wq-win
  page's self-test (reuse only for the same prefix).  Pinned by
  ``tests/prefix_cache_pins.py``: a caller simulation that checks every
  sequence reads the K/V of its own tokens through its table after each of
  hundreds of random requests, appends, forks and releases with constant
  eviction; maximal reuse against a brute-force search of the history; tiny
  hand-derived eviction scenarios; and mutation tests (key without the
  prefix, salt ignored, newest-first or evict-before-free, forward release,
  no revive, no retention, partial blocks cached, no reuse).

No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
LIB_PATH = os.path.join(_HERE, "libpa_oracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}


SAN_LIB_PATH = os.path.join(_HERE, "san", "libpa_oracle_san.so")


def build(mutant: int = 0, out_path: str | None = None, sanitize: bool = False) -> str:
    """Compile the oracle with gcc.  ``mutant > 0`` plants one known mistake
    (mutation tests only) and must go to a separate ``out_path``.
    ``sanitize`` builds under AddressSanitizer and UndefinedBehaviorSanitizer
    (to SAN_LIB_PATH; load it with PA_ORACLE_LIB and gcc's libasan preloaded)."""
    if out_path is None:
        if mutant:
            raise ValueError("a mutant build needs its own output path")
        out_path = SAN_LIB_PATH if sanitize else LIB_PATH
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    tmp = out_path + f".tmp{os.getpid()}"
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=all", "-g"] if sanitize else []
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", *san,
           f"-DORACLE_MUTANT={int(mutant)}", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


class Oracle:
    """ctypes view of one build of ``pa_oracle.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_decode.restype = i32
        lib.oracle_decode.argtypes = [vp, vp, vp, vp, vp, vp, f64, i32, i32, i32, i32, i32,
                                      i32, i64, i32, i32]
        lib.oracle_prefill.restype = i32
        lib.oracle_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, f64, i32, i32, i32, i32, i32,
                                       i32, i64, i32]
        lib.oracle_reshape_and_cache.restype = i32
        lib.oracle_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i32, i32,
                                                 i32, i64, i32]
        lib.oracle_copy_blocks.restype = i32
        lib.oracle_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i64, i32]
        lib.oracle_swap_blocks.restype = i32
        lib.oracle_swap_blocks.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, i32]
        lib.oracle_half_to_double.restype = f64
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = f64
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        self.lib = lib

    # -- helpers ---------------------------------------------------------
    @staticmethod
    def _c(a: np.ndarray) -> np.ndarray:
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("oracle inputs must be C-contiguous")
        return a

    @staticmethod
    def _ptr(a: np.ndarray):
        return a.ctypes.data_as(ctypes.c_void_p)

    # -- decode ----------------------------------------------------------
    def decode(self, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
               num_kv_heads, dtype, num_blocks=None, nthreads=None):
        """fp64 output [num_seqs][num_q_heads][head_dim].

        ``q`` is [B][Hq][D]; f16 / bf16 data are uint16 bit arrays, f32 data
        float32.  Pools are flat or shaped arrays in the documented layout."""
        q = self._c(q)
        k_cache, v_cache = self._c(k_cache), self._c(v_cache)
        bt = self._c(np.asarray(block_tables, dtype=np.int32))
        cl = self._c(np.asarray(context_lens, dtype=np.int32))
        B, hq, D = q.shape
        if num_blocks is None:
            num_blocks = k_cache.size // (num_kv_heads * block_size * D)
        out = np.zeros((B, hq, D), dtype=np.float64)
        if nthreads is None:
            nthreads = min(os.cpu_count() or 1, 64)
        maxb = bt.shape[1] if bt.ndim == 2 else 0
        rc = self.lib.oracle_decode(self._ptr(out), self._ptr(q), self._ptr(k_cache),
                                    self._ptr(v_cache), self._ptr(bt), self._ptr(cl),
                                    float(scale), int(block_size), int(num_kv_heads), int(B),
                                    int(hq), int(D), int(maxb), int(num_blocks),
                                    DTYPE_CODE[dtype], int(nthreads))
        if rc != 0:
            raise ValueError(f"oracle_decode rejected its inputs (rc={rc})")
        return out

    # -- chunked prefill -------------------------------------------------
    def prefill(self, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                block_size, num_kv_heads, dtype, num_blocks=None):
        """fp64 output [num_tokens][num_q_heads][head_dim]: sequence i's query
        tokens query_start[i] .. query_start[i+1]-1 are the last ones of its
        context and attend causally (see pa_oracle.c)."""
        q = self._c(q)
        k_cache, v_cache = self._c(k_cache), self._c(v_cache)
        bt = self._c(np.asarray(block_tables, dtype=np.int32))
        cl = self._c(np.asarray(context_lens, dtype=np.int32))
        qs = self._c(np.asarray(query_start, dtype=np.int32))
        T, hq, D = q.shape
        if num_blocks is None:
            num_blocks = k_cache.size // (num_kv_heads * block_size * D)
        out = np.zeros((T, hq, D), dtype=np.float64)
        maxb = bt.shape[1] if bt.ndim == 2 else 0
        rc = self.lib.oracle_prefill(self._ptr(out), self._ptr(q), self._ptr(k_cache),
                                     self._ptr(v_cache), self._ptr(bt), self._ptr(cl),
                                     self._ptr(qs), float(scale), int(block_size),
                                     int(num_kv_heads), int(len(cl)), int(hq), int(D), int(maxb),
                                     int(num_blocks), DTYPE_CODE[dtype])
        if rc != 0:
            raise ValueError(f"oracle_prefill rejected its inputs (rc={rc})")
        return out

    # -- cache ops -------------------------------------------------------
    def reshape_and_cache(self, k, v, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim,
                          block_size, dtype, k_token_stride=None, v_token_stride=None):
        """Writes into ``k_cache`` / ``v_cache`` in place (numpy arrays)."""
        sm = self._c(np.asarray(slot_mapping, dtype=np.int64))
        T = sm.shape[0]
        if k_token_stride is None:
            k_token_stride = num_kv_heads * head_dim
        if v_token_stride is None:
            v_token_stride = num_kv_heads * head_dim
        num_blocks = k_cache.size // (num_kv_heads * block_size * head_dim)
        rc = self.lib.oracle_reshape_and_cache(
            self._ptr(self._c(k)), self._ptr(self._c(v)), self._ptr(self._c(k_cache)),
            self._ptr(self._c(v_cache)), self._ptr(sm), int(T), int(k_token_stride),
            int(v_token_stride), int(num_kv_heads), int(head_dim), int(block_size),
            int(num_blocks), DTYPE_CODE[dtype])
        if rc != 0:
            raise ValueError(f"oracle_reshape_and_cache rejected its inputs (rc={rc})")

    def copy_blocks(self, k_cache, v_cache, pairs, num_kv_heads, head_dim, block_size, dtype):
        p = self._c(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
        num_blocks = k_cache.size // (num_kv_heads * block_size * head_dim)
        rc = self.lib.oracle_copy_blocks(self._ptr(self._c(k_cache)), self._ptr(self._c(v_cache)),
                                         self._ptr(p), int(p.shape[0]), int(num_kv_heads),
                                         int(head_dim), int(block_size), int(num_blocks),
                                         DTYPE_CODE[dtype])
        if rc != 0:
            raise ValueError(f"oracle_copy_blocks rejected its inputs (rc={rc})")


    def swap_blocks(self, src_k, src_v, dst_k, dst_v, pairs, num_kv_heads, head_dim, block_size,
                    dtype):
        """Writes into ``dst_k`` / ``dst_v`` in place (numpy arrays)."""
        p = self._c(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
        per = num_kv_heads * block_size * head_dim
        rc = self.lib.oracle_swap_blocks(self._ptr(self._c(src_k)), self._ptr(self._c(src_v)),
                                         self._ptr(self._c(dst_k)), self._ptr(self._c(dst_v)),
                                         self._ptr(p), int(p.shape[0]), int(src_k.size // per),
                                         int(dst_k.size // per), int(num_kv_heads), int(head_dim),
                                         int(block_size), DTYPE_CODE[dtype])
        if rc != 0:
            raise ValueError(f"oracle_swap_blocks rejected its inputs (rc={rc})")


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle build (PA_ORACLE_LIB, e.g. the sanitizer build, if set);
    compiled with gcc if nothing is built yet."""
    global _default
    if _default is None:
        path = os.environ.get("PA_ORACLE_LIB") or LIB_PATH
        if path == LIB_PATH and not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(path)
    return _default


def build_mutant(mutant: int) -> Oracle:
    """A separately compiled oracle with one planted mistake (CPU tests only)."""
    d = tempfile.mkdtemp(prefix="pa_oracle_mut")
    return Oracle(build(mutant, os.path.join(d, f"libpa_oracle_m{mutant}.so")))
