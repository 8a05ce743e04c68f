"""Two layers with different key-list splits in one process, on two streams.

The split count is an argument of every call and the workspace layout, and
per-kernel timing is kept per stream, so nothing one layer does can change
another's result or its timing records. Each layer's output here must be bit
for bit what the same layer gives when it runs alone, and each stream's timing
must count only its own launches.
"""
import pytest
import torch

import workloads
from tests import parity
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]

WL = workloads.custom("stateless", seed=41, heads=3, head_dim=128, hidden=128,
                      prefix_segments=(70, 9), grid=(4, 12, 20), tile=(4, 4, 4), keep_k=7)


def _layer(tsv, split):
    return tsv.TileSparseAttention(WL.prefix_segments, WL.grid, WL.tile, WL.heads, WL.head_dim,
                                   keep_k=WL.keep_k, device="cuda", split_chunks=split)


def test_two_splits_interleaved_on_two_streams():
    import tile_sparse_video_amd as tsv
    print("[gpu] two layers, splits 3 and 8, two streams", flush=True)
    inp = parity.make_inputs(WL)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    g = torch.randn((WL.tokens, WL.heads * WL.head_dim),
                    generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).cuda()

    # Alone: each layer on its own, before the other exists.
    alone = {}
    for split in (3, 8):
        att = _layer(tsv, split)
        alone[split] = att(q, k, v, g).clone()
        torch.cuda.synchronize()
        del att

    a, b = _layer(tsv, 3), _layer(tsv, 8)
    assert (a.split_chunks, b.split_chunks) == (3, 8)
    assert a.layout.total_bytes < b.layout.total_bytes  # 8 chunk partials need more room
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    out_a, out_b = torch.empty_like(q), torch.empty_like(q)
    torch.cuda.synchronize()
    tsv.vsa_timing_enable(True, s1)
    tsv.vsa_timing_enable(True, s2)
    # Interleaved: a's coarse stage, b's whole layer, then a's fine pass, each on its stream.
    with torch.cuda.stream(s1):
        a.coarse(q, k, v, stream=s1)
    with torch.cuda.stream(s2):
        b(q, k, v, g, out_b, stream=s2)
        b.fine(q, g, out_b, stream=s2)
    with torch.cuda.stream(s1):
        a.fine(q, g, out_a, stream=s1)
    torch.cuda.synchronize()
    n1, _ = tsv.vsa_timing_read("fine_attn", s1)
    n2, _ = tsv.vsa_timing_read("fine_attn", s2)
    m1, _ = tsv.vsa_timing_read("merge", s1)
    m2, _ = tsv.vsa_timing_read("merge", s2)
    tsv.vsa_timing_enable(False, s1)
    tsv.vsa_timing_enable(False, s2)
    assert (n1, n2) == (1, 2), (n1, n2)
    assert (m1, m2) == (1, 2), (m1, m2)
    assert torch.equal(out_a.view(torch.int16), alone[3].view(torch.int16))
    assert torch.equal(out_b.view(torch.int16), alone[8].view(torch.int16))
    # The two splits give the same layer within the output bar (different summation order).
    for h in range(WL.heads):
        parity.check_output(out_a[:, h, :].float().cpu().numpy(), out_b[:, h, :].float().cpu().numpy(),
                            f"split 3 vs 8, head {h}")
