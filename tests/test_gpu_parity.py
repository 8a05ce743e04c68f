"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Bit-exact: the plan arrays, k, the pooled tile means, the coarse scores, the
keep-sets, and the tiled K/V copies. Within tolerance: O_coarse (fp32 vs fp64)
and the layer output (max-abs 2e-2 and relative L2 1e-2 against the oracle's
bf16 result), plus O_fine on its own (gate = 0 run). Small cases are checked
on every token and head; the full-size layers on sampled heads and tokens, in
the same launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]


def _u32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check_layer(inp, run, heads, tokens, score_rows=None, tol_fine=True):
    wl = inp.wl
    att = run.att
    pl = parity.oracle_plan(wl)
    k = parity.oracle_k(wl, pl)
    H, D, n_t, n_v = wl.heads, wl.head_dim, pl.n_t, pl.n_v
    scale = D ** -0.5
    # plan and k: bit-exact
    assert np.array_equal(att.plan.untile, pl.untile)
    assert np.array_equal(att.plan.row_src, pl.row_src)
    assert np.array_equal(att.plan.block_len, pl.block_len)
    assert att.k == k
    qm = att.workspace_view("q_mean", torch.float32, (H, n_t, D))
    km = att.workspace_view("k_mean", torch.float32, (H, n_t, D))
    vm = att.workspace_view("v_mean", torch.float32, (H, n_t, D))
    sc = att.workspace_view("scores", torch.float32, (H, n_v, n_v))
    keep = att.keep_idx.cpu().numpy()
    oc = att.o_coarse.cpu().numpy()
    Qb, Kb, Vb = inp.qb, inp.kb, inp.vb
    toks = np.asarray(tokens, dtype=np.int64)
    g_or = oracle.gate_proj(parity.bits(inp.x), parity.bits(inp.w), toks)
    out_gpu = run.out[torch.from_numpy(toks).cuda()].cpu()
    worst = {}
    for h in heads:
        hr = oracle.head(Qb, Kb, Vb, h, pl, k, scale, score_rows)
        assert np.array_equal(_u32(qm[h].cpu().numpy()), _u32(hr.qm)), f"q means, head {h}"
        assert np.array_equal(_u32(km[h].cpu().numpy()), _u32(hr.km)), f"k means, head {h}"
        assert np.array_equal(_u32(vm[h].cpu().numpy()), _u32(hr.vm)), f"v means, head {h}"
        rows = hr.score_rows
        got_sc = sc[h].cpu().numpy()[rows]
        assert np.array_equal(_u32(got_sc), _u32(hr.scores)), f"scores, head {h}"
        assert np.array_equal(keep[h][rows], hr.keep), f"keep-sets, head {h}"
        assert parity.rel_l2(oc[h], hr.o_coarse) < 1e-4, f"O_coarse, head {h}"
        if score_rows is not None:
            # full keep lists are needed for the fine pass of the sampled tokens
            hr = oracle.head(Qb, Kb, Vb, h, pl, k, scale)
        ref_bits, _ = oracle.layer_tokens(Qb, Kb, Vb, g_or, h, pl, hr, k, scale, toks,
                                          g_is_rows=True)
        ref = oracle.bf16_value(ref_bits)
        got = out_gpu[:, h, :].float().numpy().astype(np.float64)
        mx = float(np.abs(got - ref).max())
        rl = parity.rel_l2(got, ref)
        worst[h] = (mx, rl)
        parity.check_output(got, ref, f"head {h}")
    print(f"[{wl.name}] worst max-abs {max(v[0] for v in worst.values()):.3e} "
          f"rel-L2 {max(v[1] for v in worst.values()):.3e}", flush=True)
    return worst


def check_tiled_kv(inp, run, heads):
    """The workspace K/V are exact copies of the inputs in tile order, padding zero."""
    wl, att = inp.wl, run.att
    pl = parity.oracle_plan(wl)
    D, SUB = wl.head_dim, pl.B // 64
    kt = att.workspace_view("k_tiled", torch.int16, (wl.heads, pl.n_t, SUB, D // 8, 64, 8))
    vt = att.workspace_view("v_tiled", torch.int16, (wl.heads, pl.n_t, SUB, D // 8, 64, 8))
    Kb, Vb = inp.kb, inp.vb
    for h in heads:
        kh = kt[h].cpu().numpy().view(np.uint16)
        vh = vt[h].cpu().numpy().view(np.uint16)
        for t in range(pl.n_t):
            for s in range(SUB):
                rows = pl.row_src[t * pl.B + 64 * s: t * pl.B + 64 * s + 64]
                want_k = np.where(rows[:, None] >= 0, Kb[np.maximum(rows, 0), h, :], 0)
                want_v = np.where(rows[:, None] >= 0, Vb[np.maximum(rows, 0), h, :], 0)
                assert np.array_equal(parity.unswizzle_k(kh[t, s], D), want_k), (h, t, s)
                assert np.array_equal(parity.unswizzle_v(vh[t, s], D), want_v), (h, t, s)


# ----------------------------------------------------------- small cases --

CUSTOM = {
    # partial tiles in every dimension, a one-token prefix segment, B = 64
    "ragged64": workloads.custom("ragged64", seed=11, heads=3, head_dim=128, hidden=128,
                                 prefix_segments=(5, 70, 1), grid=(5, 6, 9), tile=(4, 4, 4), keep_k=3),
    # B = 128 tiles with partial edges; a prefix tile of 2 rows (second 64-row half empty)
    "ragged128": workloads.custom("ragged128", seed=12, heads=2, head_dim=128, hidden=128,
                                  prefix_segments=(130, 7), grid=(5, 10, 6), tile=(4, 8, 4),
                                  sparsity=0.5),
    "d64": workloads.custom("d64", seed=13, heads=2, head_dim=64, hidden=128, prefix_segments=(3,),
                            grid=(3, 5, 7), tile=(4, 4, 4), keep_k=1),
    "d64_b128": workloads.custom("d64_b128", seed=14, heads=2, head_dim=64, hidden=64,
                                 prefix_segments=(40,), grid=(4, 9, 8), tile=(4, 8, 4), keep_k=2),
    # no prefix: video queries see only their kept tiles
    "no_prefix": workloads.custom("no_prefix", seed=15, heads=2, head_dim=128, hidden=256,
                                  prefix_segments=(), grid=(4, 8, 8), tile=(4, 4, 4), keep_k=2),
    # k = 0: video queries see only the prefix
    "k0": workloads.custom("k0", seed=16, heads=2, head_dim=128, hidden=128,
                           prefix_segments=(64, 20), grid=(4, 8, 8), tile=(4, 4, 4), keep_k=0),
    # sparsity 0: every tile kept (dense)
    "dense": workloads.custom("dense", seed=17, heads=2, head_dim=128, hidden=128,
                              prefix_segments=(33,), grid=(4, 8, 12), tile=(4, 4, 4), sparsity=0.0),
    # a single video tile
    "one_tile": workloads.custom("one_tile", seed=18, heads=1, head_dim=128, hidden=128,
                                 prefix_segments=(10,), grid=(2, 3, 3), tile=(4, 4, 4), keep_k=1),
}


@pytest.mark.parametrize("name", sorted(CUSTOM))
def test_small_case_every_token(name):
    wl = CUSTOM[name]
    print(f"[gpu] small case {name}", flush=True)
    inp = parity.make_inputs(wl)
    run = parity.run_gpu(inp)
    check_layer(inp, run, range(wl.heads), np.arange(wl.tokens))
    check_tiled_kv(inp, run, range(wl.heads))


def test_tiny_every_token():
    wl = workloads.WORKLOADS["tiny"]
    print("[gpu] tiny", flush=True)
    inp = parity.make_inputs(wl)
    run = parity.run_gpu(inp)
    check_layer(inp, run, range(wl.heads), np.arange(wl.tokens))
    check_tiled_kv(inp, run, range(wl.heads))


def test_mid_all_heads_sampled_tokens():
    wl = workloads.WORKLOADS["mid"]
    print("[gpu] mid", flush=True)
    inp = parity.make_inputs(wl)
    run = parity.run_gpu(inp)
    pl = parity.oracle_plan(wl)
    check_layer(inp, run, range(wl.heads), parity.sample_tokens(pl, 400, 2))
    check_tiled_kv(inp, run, [0, wl.heads - 1])


def test_page5_geometry_partial_tiles():
    wl = workloads.WORKLOADS["page5"]
    print("[gpu] page5", flush=True)
    inp = parity.make_inputs(wl)
    run = parity.run_gpu(inp)
    pl = parity.oracle_plan(wl)
    check_layer(inp, run, range(wl.heads), parity.sample_tokens(pl, 500, 3))


def check_gate_components(wl, heads, tokens, split_chunks=0):
    """The layer run with g = 0 and with g = 1, per head and token:
    - g = 0: the output is bf16(O_fine), against the oracle's O_fine rounded once;
    - g = 1: the output is bf16(O_fine + O_coarse), against the oracle's layer with g = 1;
    - the difference of the two runs is O_coarse up to the two bf16 roundings, element
      by element: |(out1 - out0) - O_coarse| <= 2^-8 (|out1| + |out0|) (1 + 2^-7), plus
      1e-4 max |O_coarse| (the O_coarse bar of the other tests) for the fp32 coarse
      attention against the fp64 oracle.
    The fine part does not depend on g, so it cancels in the difference."""
    inp = parity.make_inputs(wl)
    S, HD, D = wl.tokens, wl.heads * wl.head_dim, wl.head_dim
    r0 = parity.run_gpu(inp, gate=torch.zeros((S, HD), dtype=torch.bfloat16), split_chunks=split_chunks)
    out0 = r0.out[torch.from_numpy(tokens).cuda()].float().cpu().numpy().astype(np.float64)
    del r0
    r1 = parity.run_gpu(inp, gate=torch.ones((S, HD), dtype=torch.bfloat16), split_chunks=split_chunks)
    out1 = r1.out[torch.from_numpy(tokens).cuda()].float().cpu().numpy().astype(np.float64)
    del r1
    pl = parity.oracle_plan(wl)
    k = parity.oracle_k(wl, pl)
    scale = D ** -0.5
    n = len(tokens)
    g0 = np.zeros((n, HD), dtype=np.uint16)
    g1 = np.full((n, HD), 0x3F80, dtype=np.uint16)  # bf16 1.0
    tiles = pl.untile[tokens] // pl.B
    for h in heads:
        hr = oracle.head(inp.qb, inp.kb, inp.vb, h, pl, k, scale)
        want0 = oracle.bf16_value(oracle.layer_tokens(inp.qb, inp.kb, inp.vb, g0, h, pl, hr, k, scale,
                                                      tokens, g_is_rows=True)[0])
        want1 = oracle.bf16_value(oracle.layer_tokens(inp.qb, inp.kb, inp.vb, g1, h, pl, hr, k, scale,
                                                      tokens, g_is_rows=True)[0])
        a0, a1 = out0[:, h, :], out1[:, h, :]
        parity.check_output(a0, want0, f"g = 0, head {h}")
        parity.check_output(a1, want1, f"g = 1, head {h}")
        oc = hr.o_coarse[tiles]
        bound = 2.0 ** -8 * (np.abs(a1) + np.abs(a0)) * (1 + 2.0 ** -7) + 1e-4 * np.abs(oc).max()
        err = np.abs((a1 - a0) - oc)
        assert (err <= bound).all(), f"coarse term, head {h}: worst excess {float((err - bound).max()):.3e}"
    print(f"[{wl.name}] gate 0 / 1 components of {n} tokens x {len(heads)} heads ok", flush=True)


def test_gate_components_every_token():
    wl = CUSTOM["ragged64"]
    print("[gpu] gate components ragged64", flush=True)
    check_gate_components(wl, range(wl.heads), np.arange(wl.tokens))


@pytest.mark.parametrize("chunks", [3, 8])
def test_gate_components_split(chunks):
    wl = CUSTOM["ragged128"]
    print(f"[gpu] gate components ragged128 chunks={chunks}", flush=True)
    check_gate_components(wl, range(wl.heads), np.arange(wl.tokens), split_chunks=chunks)


@pytest.mark.timeout(600)
def test_gate_components_full_size_h3():
    """The g = 0 / g = 1 decomposition at the H3-shaped layer, in the benchmark's
    launch configuration (16 key chunks + merge), on 4 heads x 128 sampled tokens."""
    wl = workloads.WORKLOADS["h3"]
    print("[gpu] gate components h3", flush=True)
    pl = parity.oracle_plan(wl)
    check_gate_components(wl, [0, 13, 28, 41], np.asarray(parity.sample_tokens(pl, 128, 9), dtype=np.int64))
    torch.cuda.empty_cache()


def test_deterministic_repeat():
    wl = CUSTOM["ragged128"]
    print("[gpu] determinism", flush=True)
    inp = parity.make_inputs(wl)
    a = parity.run_gpu(inp)
    out_a, keep_a = a.out.clone(), a.att.keep_idx.clone()
    b = parity.run_gpu(inp)
    assert torch.equal(out_a.view(torch.int16), b.out.view(torch.int16))
    assert torch.equal(keep_a, b.att.keep_idx)


def assert_gate_close(got_bits, want_bits, x_bits, w_bits):
    """GPU gate (fp32 accumulation, one bf16 rounding) vs the oracle's correctly
    rounded fp64 result: |got - want| <= two bf16 roundings (2^-8 |v| each) plus
    the fp32 accumulation bound K * 2^-23 * sum_c |x_c w_c|, for any summation order."""
    got, want = oracle.bf16_value(got_bits), oracle.bf16_value(want_bits)
    K = x_bits.shape[1]
    absdot = np.abs(oracle.bf16_value(x_bits)) @ np.abs(oracle.bf16_value(w_bits)).T
    bound = 2.0 ** -8 * (np.abs(want) + np.abs(got)) + K * 2.0 ** -23 * absdot + 1e-30
    assert (np.abs(got - want) <= bound).all()
    assert (got_bits == want_bits).mean() > 0.97


def test_gate_proj_matches_oracle():
    wl = workloads.WORKLOADS["mid"]
    print("[gpu] gate projection", flush=True)
    inp = parity.make_inputs(wl)
    g = torch.empty((wl.tokens, wl.heads * wl.head_dim), dtype=torch.bfloat16, device="cuda")
    import tile_sparse_video_amd as tsv
    tsv.vsa_gate_proj(inp.x.cuda(), inp.w.cuda(), g)
    torch.cuda.synchronize()
    toks = parity.sample_tokens(parity.oracle_plan(wl), 300, 5)
    xb, wb = parity.bits(inp.x), parity.bits(inp.w)
    want = oracle.gate_proj(xb, wb, toks)
    got = parity.bits(g.cpu())[toks]
    assert_gate_close(got, want, xb[toks], wb)


def test_gate_proj_ragged_rows():
    """Row counts that are not multiples of the 128-row block."""
    import tile_sparse_video_amd as tsv
    for rows, hidden, out_f in ((1, 64, 64), (130, 192, 320), (257, 64, 128)):
        gen = torch.Generator().manual_seed(rows)
        x = torch.randn(rows, hidden, generator=gen).to(torch.bfloat16)
        w = (torch.randn(out_f, hidden, generator=gen) * 0.05).to(torch.bfloat16)
        g = torch.empty((rows, out_f), dtype=torch.bfloat16, device="cuda")
        tsv.vsa_gate_proj(x.cuda(), w.cuda(), g)
        torch.cuda.synchronize()
        xb, wb = parity.bits(x), parity.bits(w)
        assert_gate_close(parity.bits(g.cpu()), oracle.gate_proj(xb, wb), xb, wb)


def test_device_call_rejects_small_workspace():
    import tile_sparse_video_amd as tsv
    wl = CUSTOM["one_tile"]
    att = tsv.TileSparseAttention(wl.prefix_segments, wl.grid, wl.tile, wl.heads, wl.head_dim,
                                  keep_k=1)
    q = torch.zeros((wl.tokens, 1, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tsv.VsaError) as e:
        tsv.vsa_coarse_topk(att.plan.info, att.row_src, att.block_len, 1, wl.head_dim, q, q, q,
                            att.workspace[:1024], att.keep_idx, att.o_coarse, keep_k=1)
    assert e.value.status == tsv.VSA_ERR_ARG


# -------------------------------------------------- full-size layers --

def check_coarse_every_head(inp, run, oc_rows=None):
    """Every head of a full-size layer: tile means, every coarse score and every
    keep-set bit-exact against the oracle (scores pulled one head at a time),
    O_coarse within rel-L2 1e-4 (on oc_rows, or every tile). Returns the oracle's
    per-head results (means and keep lists) for the output check."""
    wl, att = inp.wl, run.att
    pl = parity.oracle_plan(wl)
    k = parity.oracle_k(wl, pl)
    H, D, n_t, n_v = wl.heads, wl.head_dim, pl.n_t, pl.n_v
    scale = D ** -0.5
    assert np.array_equal(att.plan.row_src, pl.row_src) and att.k == k
    qm = att.workspace_view("q_mean", torch.float32, (H, n_t, D))
    km = att.workspace_view("k_mean", torch.float32, (H, n_t, D))
    vm = att.workspace_view("v_mean", torch.float32, (H, n_t, D))
    sc = att.workspace_view("scores", torch.float32, (H, n_v, n_v))
    rows = np.arange(n_t, dtype=np.int32) if oc_rows is None else np.asarray(oc_rows, dtype=np.int32)
    Qb, Kb, Vb = inp.qb, inp.kb, inp.vb
    results = {}
    for h in range(H):
        m = [oracle.tile_means(X, h, pl) for X in (Qb, Kb, Vb)]
        for name, got, want in zip("qkv", (qm, km, vm), m):
            assert np.array_equal(_u32(got[h].cpu().numpy()), _u32(want)), f"{name} means, head {h}"
        scores = oracle.video_scores(m[0], m[1], pl.P, n_v)
        assert np.array_equal(_u32(sc[h].cpu().numpy()), _u32(scores)), f"scores, head {h}"
        keep = oracle.topk_rows(scores, k, pl.P)
        assert np.array_equal(att.keep_idx[h].cpu().numpy(), keep), f"keep-sets, head {h}"
        oc = oracle.coarse_attn(*m, scale, rows)
        assert parity.rel_l2(att.o_coarse[h].cpu().numpy()[rows], oc) < 1e-4, f"O_coarse, head {h}"
        results[h] = (m, keep)
        print(f"[{wl.name}] head {h}: means, {n_v} x {n_v} scores and keep-sets bit-exact", flush=True)
    return results


def check_outputs_sampled(inp, run, results, heads, tokens):
    """Layer outputs of sampled tokens on the given heads, against the oracle's
    fp64 result rounded once to bf16 (max-abs 2e-2, rel-L2 1e-2)."""
    wl = inp.wl
    pl = parity.oracle_plan(wl)
    k = parity.oracle_k(wl, pl)
    scale = wl.head_dim ** -0.5
    toks = np.asarray(tokens, dtype=np.int64)
    g_or = oracle.gate_proj(parity.bits(inp.x), parity.bits(inp.w), toks)
    out_gpu = run.out[torch.from_numpy(toks).cuda()].cpu()
    worst = (0.0, 0.0)
    for h in heads:
        m, keep = results[h]
        hr = oracle.HeadResult(*m, None, None, keep, oracle.coarse_attn(*m, scale))
        ref_bits, _ = oracle.layer_tokens(inp.qb, inp.kb, inp.vb, g_or, h, pl, hr, k, scale, toks,
                                          g_is_rows=True)
        ref = oracle.bf16_value(ref_bits)
        got = out_gpu[:, h, :].float().numpy().astype(np.float64)
        mx, rl = float(np.abs(got - ref).max()), parity.rel_l2(got, ref)
        worst = (max(worst[0], mx), max(worst[1], rl))
        parity.check_output(got, ref, f"head {h}")
    print(f"[{wl.name}] outputs of {len(toks)} tokens x {len(heads)} heads: worst max-abs "
          f"{worst[0]:.3e} rel-L2 {worst[1]:.3e}", flush=True)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["h3", "veda", "long"])
def test_full_size_every_head(name):
    """Full-size layers in the benchmark's launch configuration: means, scores and
    keep-sets of all heads bit-exact; outputs of 256 sampled tokens on 8 heads."""
    wl = workloads.WORKLOADS[name]
    print(f"[gpu] full size {name}: generating inputs", flush=True)
    inp = parity.make_inputs(wl)
    print(f"[gpu] full size {name}: running the HIP path", flush=True)
    run = parity.run_gpu(inp)
    pl = parity.oracle_plan(wl)
    # Long: O_coarse on 512 sampled tiles per head (the oracle's fp64 tile softmax
    # over 5,570 tiles takes seconds per head); every tile elsewhere
    oc_rows = (np.sort(np.random.default_rng(1).choice(pl.n_t, 512, replace=False))
               if name == "long" else None)
    results = check_coarse_every_head(inp, run, oc_rows)
    heads = sorted({int(h) for h in np.linspace(0, wl.heads - 1, 8).round()})
    check_outputs_sampled(inp, run, results, heads, parity.sample_tokens(pl, 256, 7))
    del run
    torch.cuda.empty_cache()


# ------------------------------------------------ split fine pass --

@pytest.mark.parametrize("chunks", [3, 8, 16])
@pytest.mark.parametrize("name", ["ragged64", "ragged128", "d64", "no_prefix", "k0", "one_tile"])
def test_split_key_lists_every_token(name, chunks):
    """The fine pass split into chunks (partials + merge) gives the same layer."""
    import tile_sparse_video_amd as tsv
    wl = CUSTOM[name]
    print(f"[gpu] split {name} chunks={chunks}", flush=True)
    inp = parity.make_inputs(wl)
    run = parity.run_gpu(inp, split_chunks=chunks)
    assert run.att.split_chunks == chunks
    check_layer(inp, run, range(wl.heads), np.arange(wl.tokens))


# ------------------------------------------------ workspace canary --

@pytest.mark.parametrize("name,chunks,ref", [("ragged64", 0, None), ("ragged128", 8, None),
                                             ("no_prefix", 3, None), ("ragged64", 8, (0.5, None))])
def test_nan_canary_every_output_written(name, chunks, ref):
    """Workspace, outputs, keep lists and O_coarse filled with NaN / -1 before the
    layer: every output and keep entry is written, finite and in range, and the
    result is bit-identical to a run on fresh buffers (no stage reads a region
    it did not write first)."""
    wl = CUSTOM[name]
    print(f"[gpu] canary {name} chunks={chunks} ref={ref}", flush=True)
    inp = parity.make_inputs(wl)
    clean = (parity.run_gpu(inp, split_chunks=chunks) if ref is None
             else parity.run_gpu_ref(inp, *ref, split_chunks=chunks))
    att = clean.att
    att.workspace.fill_(0xFF)                       # NaN as fp32 and as bf16
    att.keep_idx.fill_(-1)
    att.o_coarse.fill_(float("nan"))
    qd, kd, vd = (t.cuda() for t in (inp.q, inp.k, inp.v))
    out = torch.full_like(qd, float("nan"))
    att(qd, kd, vd, clean.g, out)
    torch.cuda.synchronize()
    pl = parity.oracle_plan(wl)
    keep = att.keep_idx.cpu().numpy()
    assert torch.isfinite(out.float()).all(), "an output element was not written"
    assert torch.isfinite(att.o_coarse).all(), "an O_coarse element was not written"
    if ref is None:
        assert ((keep >= pl.P) & (keep < pl.n_t)).all()
        assert (np.diff(keep, axis=-1) > 0).all()
    else:
        k_ref = att.k_ref
        assert ((keep[..., :k_ref] >= 0) & (keep[..., :k_ref] < pl.P)).all()
        assert ((keep[..., k_ref:] >= pl.P) & (keep[..., k_ref:] < pl.n_t)).all()
    assert torch.equal(out.view(torch.int16), clean.out.view(torch.int16))
