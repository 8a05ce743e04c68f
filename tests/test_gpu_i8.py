"""INT8 fine pass: HIP path vs the CPU oracle, through the C ABI.

[Veda] "How Veda works" and its performance table: the tile-skip kernel does
its attention arithmetic in INT8. Reading: symmetric INT8 codes for Q and K
with one fp32 scale per 64-row block of the tiled layout; only the score
product uses the codes (softmax, P.V and the gated combine as the bf16 path).

Bit-exact: the K codes and block scales the library writes to its workspace
(both sides decide each code in fp32 with the same operations). Within
tolerance: the layer output against the oracle's INT8 result (max-abs 2e-2,
relative L2 1e-2, the bf16 path's bar: the oracle applies the same codes, so
what remains is the bf16 rounding of P, fp32 accumulation and the fp32 product
of the two block scales). The distance to the unquantised layer is reported
and kept under 5e-2 relative L2 (an accuracy check of the scheme, not parity).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity
from tests.conftest import gpu_available
from tests.test_gpu_parity import CUSTOM

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]

EXACT_REL_L2 = 5e-2


def run_gpu_i8(inp, ref_sparsity=None, ref_keep_k=None, dev="cuda", split_chunks=0):
    import tile_sparse_video_amd as tsv
    wl = inp.wl
    att = tsv.TileSparseAttention(wl.prefix_segments, wl.grid, wl.tile, wl.heads, wl.head_dim,
                                  sparsity=wl.sparsity, keep_k=wl.keep_k, device=dev,
                                  reference_sparsity=ref_sparsity, ref_keep_k=ref_keep_k, int8=True,
                                  split_chunks=split_chunks)
    qd, kd, vd = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    xd, wd = inp.x.to(dev), inp.w.to(dev)
    g = torch.empty((wl.tokens, wl.heads * wl.head_dim), dtype=torch.bfloat16, device=dev)
    tsv.vsa_gate_proj(xd, wd, g)
    out = att(qd, kd, vd, g)
    torch.cuda.synchronize()
    return parity.GpuRun(att, out, g)


def expected_k_frags(codes, D):
    """Oracle codes [S_pad][D] -> the library's fragment order
    [blocks][2 (kb)][D/32 (c)][64 lanes][16]: lane l, byte e = row 32kb + l%32,
    d = 32c + 16(l/32) + e."""
    nb = codes.shape[0] // 64
    x = codes.reshape(nb, 2, 32, D // 32, 2, 16)          # [b][kb][l32][c][hh][e]
    return x.transpose(0, 1, 3, 4, 2, 5).reshape(nb, 2, D // 32, 64, 16)


def check_k_codes(inp, run, heads):
    wl, att = inp.wl, run.att
    pl = parity.oracle_plan(wl)
    D, SUB = wl.head_dim, pl.B // 64
    k8 = att.workspace_view("k_i8", torch.int8, (wl.heads, pl.n_t * SUB, 2, D // 32, 64, 16))
    ks = att.workspace_view("k_scale", torch.float32, (wl.heads, pl.n_t * SUB))
    for h in heads:
        codes, scales = oracle.quant_blocks_i8(inp.kb, h, pl)
        assert np.array_equal(k8[h].cpu().numpy(), expected_k_frags(codes, D)), f"K codes, head {h}"
        got = ks[h].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), scales.view(np.uint32)), f"K scales, head {h}"


def check_layer_i8(inp, run, heads, tokens, ref_mode=False, ref_sparsity=None, ref_keep_k=None):
    wl, att = inp.wl, run.att
    pl = parity.oracle_plan(wl)
    H, D = wl.heads, wl.head_dim
    scale = D ** -0.5
    Qb, Kb, Vb = inp.qb, inp.kb, inp.vb
    toks = np.asarray(tokens, dtype=np.int64)
    tiles = pl.untile[toks] // pl.B
    g_or = oracle.gate_proj(parity.bits(inp.x), parity.bits(inp.w), toks)
    out_gpu = run.out[torch.from_numpy(toks).cuda()].cpu()
    keep_gpu = att.keep_idx.cpu().numpy()
    worst, dist = [], []
    for h in heads:
        if ref_mode:
            k_ref, k_gen = oracle.ref_keep_counts(pl, ref_sparsity, ref_keep_k, wl.sparsity, wl.keep_k)
            hr = oracle.head_ref(Qb, Kb, Vb, h, pl, k_ref, k_gen, scale)
            csr = oracle.key_lists_explicit(hr.keep)
            exact = oracle.fine_tokens_lists(Qb, Kb, Vb, h, pl, hr.keep, scale, toks)
        else:
            k = parity.oracle_k(wl, pl)
            hr = oracle.head(Qb, Kb, Vb, h, pl, k, scale)
            csr = oracle.key_lists_default(pl, hr.keep)
            exact = oracle.fine_tokens(Qb, Kb, Vb, h, pl, hr.keep, k, scale, toks)
        assert np.array_equal(keep_gpu[h], hr.keep), f"keep lists, head {h}"
        o_fine = oracle.fine_tokens_i8(Qb, Kb, Vb, h, pl, csr, scale, toks)
        g_rows = np.ascontiguousarray(g_or[:, h * D:(h + 1) * D])
        ref = oracle.bf16_value(oracle.combine(o_fine, g_rows, hr.o_coarse[tiles]))
        ref_exact = oracle.bf16_value(oracle.combine(exact, g_rows, hr.o_coarse[tiles]))
        got = out_gpu[:, h, :].float().numpy().astype(np.float64)
        mx, rl = float(np.abs(got - ref).max()), parity.rel_l2(got, ref)
        worst.append((mx, rl))
        dist.append(parity.rel_l2(got, ref_exact))
        parity.check_output(got, ref, f"head {h}")
        assert dist[-1] <= EXACT_REL_L2, f"head {h}: {dist[-1]} from the unquantised layer"
    print(f"[{wl.name} int8] worst max-abs {max(w[0] for w in worst):.3e} rel-L2 "
          f"{max(w[1] for w in worst):.3e}; vs unquantised rel-L2 {max(dist):.3e}", flush=True)


SMALL = ["ragged64", "ragged128", "d64", "d64_b128", "no_prefix", "k0", "dense", "one_tile"]


@pytest.mark.parametrize("chunks", [0, 8])
@pytest.mark.parametrize("name", SMALL)
def test_i8_small_every_token(name, chunks):
    import tile_sparse_video_amd as tsv
    wl = CUSTOM[name]
    print(f"[gpu] int8 {name} chunks={chunks}", flush=True)
    inp = parity.make_inputs(wl)
    run = run_gpu_i8(inp, split_chunks=chunks)
    check_k_codes(inp, run, range(wl.heads))
    check_layer_i8(inp, run, range(wl.heads), np.arange(wl.tokens))


@pytest.mark.parametrize("name,rs,rk", [("ragged64", None, 1), ("ragged128", 0.5, None),
                                        ("d64", None, 1), ("no_prefix", 0.9, None)])
def test_i8_reference_sparsity_every_token(name, rs, rk):
    wl = CUSTOM[name]
    print(f"[gpu] int8 ref {name}", flush=True)
    inp = parity.make_inputs(wl)
    run = run_gpu_i8(inp, rs, rk)
    check_layer_i8(inp, run, range(wl.heads), np.arange(wl.tokens), True, rs, rk)


def test_i8_zero_and_tiny_blocks():
    """An all-zero query tile and key tile (scale 0, codes 0: their scores are exactly 0),
    and a tile scaled by 2^-100 (scales far below 1, codes unchanged)."""
    wl = CUSTOM["ragged64"]
    print("[gpu] int8 zero and tiny blocks", flush=True)
    inp = parity.make_inputs(wl)
    pl = parity.oracle_plan(wl)
    zq = pl.row_src[(pl.P + 1) * pl.B:(pl.P + 2) * pl.B]
    zk = pl.row_src[(pl.P + 2) * pl.B:(pl.P + 3) * pl.B]
    tiny = pl.row_src[0:pl.B]
    q, k = inp.q.clone(), inp.k.clone()
    q[torch.from_numpy(zq[zq >= 0]).long()] = 0
    k[torch.from_numpy(zk[zk >= 0]).long()] = 0
    q[torch.from_numpy(tiny[tiny >= 0]).long()] *= 2.0 ** -100
    inp = parity.Inputs(wl, q, k, inp.v, inp.x, inp.w)
    run = run_gpu_i8(inp)
    check_k_codes(inp, run, range(wl.heads))
    check_layer_i8(inp, run, range(wl.heads), np.arange(wl.tokens))


def test_i8_tiny_and_mid():
    for name in ("tiny", "mid"):
        wl = workloads.WORKLOADS[name]
        print(f"[gpu] int8 {name}", flush=True)
        inp = parity.make_inputs(wl)
        run = run_gpu_i8(inp)
        pl = parity.oracle_plan(wl)
        toks = np.arange(wl.tokens) if name == "tiny" else parity.sample_tokens(pl, 300, 5)
        check_k_codes(inp, run, [0, wl.heads - 1])
        check_layer_i8(inp, run, range(wl.heads), toks)


@pytest.mark.parametrize("name", ["h3", "veda"])
def test_i8_full_size_sampled(name):
    wl = workloads.WORKLOADS[name]
    print(f"[gpu] int8 full size {name}: generating inputs", flush=True)
    inp = parity.make_inputs(wl)
    print(f"[gpu] int8 full size {name}: running the HIP path", flush=True)
    run = run_gpu_i8(inp)
    pl = parity.oracle_plan(wl)
    heads = sorted({0, wl.heads - 1})
    toks = parity.sample_tokens(pl, 32, 3)
    print(f"[gpu] int8 full size {name}: oracle on heads {heads}, {len(toks)} tokens", flush=True)
    check_k_codes(inp, run, heads)
    check_layer_i8(inp, run, heads, toks)
    del run
    torch.cuda.empty_cache()
