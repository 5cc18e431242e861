"""A decode step (cache write, then pa_decode with its merge) captured in a
HIP graph through torch and replayed: every replay, with eager work and
synchronisations between replays, equals the eager step bit for bit.  The
library records no memset and allocates nothing inside the calls, so the
step can be captured as is."""
import numpy as np
import pytest
import torch

import paged_kv_cache_118_amd as pa
import workloads as W
from tests.gpu_util import DEV, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("spec", [W.OPT13B.with_(num_seqs=24),
                                  W.GQA_LONG.with_(num_seqs=4, lengths=("uniform", 3000, 9000))],
                         ids=["mha_f16", "gqa_bf16"])
def test_step_graph_replays_match_eager(spec):
    log(f"[graph] {spec.name}")
    case = W.make_decode_case(spec, device=DEV, poison=False)
    B = len(case.lens)
    gen = W.make_generator(spec.seed + 3, DEV)
    k_new, v_new = W.new_token_rows(B, spec.num_kv_heads, spec.head_dim, spec.dtype, gen, DEV)
    pos = case.lens - 1  # rewrite each sequence's last token
    slots = torch.from_numpy(W.slots_for_positions(case.tables, list(enumerate(pos)),
                                                   spec.block_size)).to(DEV)
    tables = torch.from_numpy(case.tables).to(DEV)
    lens = torch.from_numpy(case.lens).to(DEV)
    ws = torch.empty(max(1, pa.pa_decode_workspace_bytes(
        B, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.block_size,
        case.max_context_len, spec.partition_size, W.TORCH_DTYPE[spec.dtype])),
        dtype=torch.uint8, device=DEV)
    out = torch.empty_like(case.q)

    def step():
        pa.pa_reshape_and_cache(k_new, v_new, case.k_cache, case.v_cache, slots, spec.block_size)
        pa.pa_decode(out, case.q, case.k_cache, case.v_cache, tables, lens, spec.scale,
                     spec.block_size, spec.num_kv_heads, case.max_context_len,
                     partition_size=spec.partition_size, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.fill_(float("nan"))
        ws.fill_(0x7f)  # eager work between replays; the workspace needs no clearing
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager step"
