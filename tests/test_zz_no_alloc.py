"""vsa_layer_fwd_static (the layer with the library's static workspace, for
callers that cannot allocate) against the existing entry points it varies:
vsa_coarse_topk + vsa_sparse_attn_fwd with the key lists unsplit. Same kernels
on the same inputs, so keep lists, O_coarse and the output must be identical
bit for bit; two calls in a row, the second on a smaller layer, so the second
must not depend on what the first left in the shared array.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import parity
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]


def _existing(inp, g):
    """The existing entry points (through the C ABI), unsplit key lists."""
    run = parity.run_gpu(inp, gate=g, split_chunks=1)
    return run.out, run.att


def _static(inp, att, g):
    import tile_sparse_video_amd as tsv
    wl = inp.wl
    dev = "cuda"
    qd, kd, vd = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    out = torch.full_like(qd, float("nan"))
    keep = torch.full_like(att.keep_idx, -7)
    oc = torch.full_like(att.o_coarse, float("nan"))
    tsv.vsa_layer_fwd_static(att.plan.info, att.row_src, att.block_len, wl.heads, wl.head_dim,
                             qd, kd, vd, g.to(dev), keep if keep.numel() else None, oc, out,
                             sparsity=wl.sparsity, keep_k=wl.keep_k)
    torch.cuda.synchronize()
    return out, keep, oc


def test_static_workspace_matches_existing_entry_points():
    import tile_sparse_video_amd as tsv
    cases = [workloads.WORKLOADS["mid"], workloads.WORKLOADS["tiny"]]   # second call smaller
    for wl in cases:
        print(f"[gpu] static workspace: {wl.name}", flush=True)
        lay = tsv.vsa_workspace_layout(tsv.cached_plan(wl.prefix_segments, wl.grid, wl.tile).info,
                                       wl.heads, wl.head_dim, 1)
        assert lay.total_bytes <= tsv.STATIC_WORKSPACE_BYTES
        inp = parity.make_inputs(wl)
        gen = torch.Generator().manual_seed(3)
        g = torch.randn(wl.tokens, wl.heads * wl.head_dim, generator=gen).to(torch.bfloat16)
        want_out, att = _existing(inp, g)
        got_out, got_keep, got_oc = _static(inp, att, g)
        assert torch.equal(got_keep, att.keep_idx), wl.name
        assert torch.equal(got_oc.view(torch.int32), att.o_coarse.view(torch.int32)), wl.name
        assert torch.equal(got_out.view(torch.int16), want_out.view(torch.int16)), wl.name
        assert torch.isfinite(got_out.float()).all()
        del att, want_out
        torch.cuda.empty_cache()


def test_static_workspace_rejects_a_large_layer():
    import tile_sparse_video_amd as tsv
    wl = workloads.WORKLOADS["page5"]      # 2 heads x 43,904 padded rows: about 56 MB + scores
    pl = tsv.cached_plan(wl.prefix_segments, wl.grid, wl.tile)
    need = tsv.vsa_workspace_layout(pl.info, wl.heads, wl.head_dim, 1).total_bytes
    heads = wl.heads if need > tsv.STATIC_WORKSPACE_BYTES else 4
    dev = "cuda"
    z = torch.zeros((wl.tokens, heads, wl.head_dim), dtype=torch.bfloat16, device=dev)
    rs = torch.from_numpy(pl.row_src).to(dev)
    bl = torch.from_numpy(pl.block_len).to(dev)
    keep = torch.empty((heads, pl.n_v, 1), dtype=torch.int32, device=dev)
    oc = torch.empty((heads, pl.n_t, wl.head_dim), dtype=torch.float32, device=dev)
    with pytest.raises(tsv.VsaError) as e:
        tsv.vsa_layer_fwd_static(pl.info, rs, bl, heads, wl.head_dim, z, z, z,
                                 z.view(wl.tokens, -1), keep, oc, z.clone(), keep_k=1)
    assert e.value.status == tsv.VSA_ERR_ARG
