"""Backward pass: HIP path vs the CPU oracle, through the C ABI.

Gradients of the layer with the keep sets held fixed, for q, k, v and the gate.
Both sides use the same bf16 inputs and gate g; the oracle works in fp64, the
GPU rounds P and dS to bf16 for the matrix products (relative error 2^-9 each,
P also inside the recomputed O_fine that gives the softmax row term D_t). Each
gradient is a sum of such terms with independent signs, so its
relative error is a small multiple of 2^-9 (about 2e-3, as measured); the
bound leaves a factor of 5: relative L2 <= GRAD_REL_L2 and max-abs <=
GRAD_MAX_REL times the largest reference magnitude, per head and tensor.
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

GRAD_REL_L2 = 1e-2
GRAD_MAX_REL = 2e-2


def make_dout(wl, seed=99):
    gen = torch.Generator().manual_seed(seed)
    return torch.randn(wl.tokens, wl.heads, wl.head_dim, generator=gen).to(torch.bfloat16)


def run_case(wl, ref=None, heads=None, train=False, split_chunks=0):
    """ref: None (default mode) or (ref_sparsity, ref_keep_k). train: rerun the fine
    pass as the training forward (its output must be bit-identical) so that the
    backward uses the statistics it saved."""
    inp = parity.make_inputs(wl)
    pl = parity.oracle_plan(wl)
    g_bits = oracle.gate_proj(parity.bits(inp.x), parity.bits(inp.w))
    g = torch.from_numpy(g_bits.view(np.int16)).view(torch.bfloat16)
    if ref is None:
        run = parity.run_gpu(inp, gate=g, split_chunks=split_chunks)
    else:
        run = parity.run_gpu_ref(inp, ref[0], ref[1], gate=g, split_chunks=split_chunks)
    dout = make_dout(wl)
    dev = run.out.device
    qd, kd, vd = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    if train:
        out2 = torch.empty_like(run.out)
        run.att.fine_train(qd, run.g, out2)
        torch.cuda.synchronize()
        assert torch.equal(out2.view(torch.int16), run.out.view(torch.int16)), "training forward output"
    dq, dk, dv, dg = run.att.backward(qd, kd, vd, run.g, dout.to(dev))
    torch.cuda.synchronize()
    got = {"dq": dq.cpu().numpy(), "dk": dk.cpu().numpy(), "dv": dv.cpu().numpy(),
           "dg": dg.cpu().numpy().reshape(wl.tokens, wl.heads, wl.head_dim)}
    scale = wl.head_dim ** -0.5
    Qb, Kb, Vb, dOb = inp.qb, inp.kb, inp.vb, parity.bits(dout)
    worst = {}
    for h in (range(wl.heads) if heads is None else heads):
        if ref is None:
            k = parity.oracle_k(wl, pl)
            hr = oracle.head(Qb, Kb, Vb, h, pl, k, scale)
            csr = oracle.key_lists_default(pl, hr.keep)
        else:
            k_ref, k_gen = oracle.ref_keep_counts(pl, ref[0], ref[1], wl.sparsity, wl.keep_k)
            hr = oracle.head_ref(Qb, Kb, Vb, h, pl, k_ref, k_gen, scale)
            csr = oracle.key_lists_explicit(hr.keep)
        want = oracle.layer_bwd(Qb, Kb, Vb, g_bits, dOb, h, pl, csr, scale)
        for name in ("dq", "dk", "dv", "dg"):
            a, b = got[name][:, h, :].astype(np.float64), want[name]
            rl = parity.rel_l2(a, b)
            mx = float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))
            worst[name] = max(worst.get(name, (0, 0)), (rl, mx))
            assert rl <= GRAD_REL_L2 and mx <= GRAD_MAX_REL, f"{name} head {h}: rel-L2 {rl:.3e} max {mx:.3e}"
    print(f"[{wl.name} bwd] " + " ".join(f"{n} rel-L2 {v[0]:.2e} max {v[1]:.2e}"
                                          for n, v in worst.items()), flush=True)


@pytest.mark.parametrize("name", sorted(CUSTOM))
def test_bwd_small_every_token(name):
    print(f"[gpu] bwd {name}", flush=True)
    run_case(CUSTOM[name])


@pytest.mark.parametrize("name,rs,rk", [("ragged64", None, 1), ("ragged128", 0.5, None),
                                        ("no_prefix", 0.9, None), ("dense", 0.0, None)])
def test_bwd_reference_sparsity(name, rs, rk):
    print(f"[gpu] bwd ref {name}", flush=True)
    run_case(CUSTOM[name], ref=(rs, rk))


@pytest.mark.parametrize("name", ["ragged64", "ragged128", "d64", "no_prefix", "k0"])
def test_bwd_saved_stats_every_token(name):
    """Key lists split into 8 chunks; the training forward saves lse and O_fine and the
    backward uses them instead of recomputing the fine forward."""
    print(f"[gpu] bwd saved stats {name}", flush=True)
    run_case(CUSTOM[name], train=True, split_chunks=8)


def test_bwd_saved_stats_reference_sparsity():
    print("[gpu] bwd saved stats ref", flush=True)
    run_case(CUSTOM["ragged128"], ref=(0.5, None), train=True, split_chunks=8)


def test_bwd_tiny():
    print("[gpu] bwd tiny", flush=True)
    run_case(workloads.WORKLOADS["tiny"])


def test_bwd_mid_two_heads():
    print("[gpu] bwd mid", flush=True)
    wl = workloads.WORKLOADS["mid"]
    run_case(wl, heads=[0, wl.heads - 1])


def host_gate(wl, seed=77):
    """A seeded bf16 gate drawn on the host, fed as the same bytes to both sides."""
    gen = torch.Generator().manual_seed(seed)
    return (torch.randn(wl.tokens, wl.heads * wl.head_dim, generator=gen) * 0.5).to(torch.bfloat16)


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("name,train,all_heads", [("h3", False, False), ("veda", False, True),
                                                  ("h3", True, True)])
def test_bwd_full_size(name, train, all_heads):
    """Full-size layers, both sides fed the same host-drawn gate: dk and dv of one
    sampled key tile per head element by element against the oracle (every head,
    or 8 spread heads), dq of 128 sampled tokens on 8 heads, dg = dout * O_coarse
    on every token, and the identities sum(dv) = sum(dout * (1 + g)), sum(dk) = 0."""
    wl = workloads.WORKLOADS[name]
    print(f"[gpu] bwd full size {name}: inputs", flush=True)
    inp = parity.make_inputs(wl)
    pl = parity.oracle_plan(wl)
    dev = "cuda"
    g_host = host_gate(wl)
    run = parity.run_gpu(inp, gate=g_host)
    dout = make_dout(wl).to(dev)
    qd, kd, vd = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    if train:
        out2 = torch.empty_like(run.out)
        run.att.fine_train(qd, run.g, out2)
        torch.cuda.synchronize()
        assert torch.equal(out2.view(torch.int16), run.out.view(torch.int16)), "training forward output"
        del out2
    print(f"[gpu] bwd full size {name}: backward (saved stats: {train})", flush=True)
    dq, dk, dv, dg = run.att.backward(qd, kd, vd, run.g, dout)
    torch.cuda.synchronize()
    oc = run.att.o_coarse                                           # [H][n_t][D]
    tile_of = torch.from_numpy((pl.untile // pl.B).astype(np.int64)).to(dev)
    do32, g32 = dout.float(), run.g.float().view(wl.tokens, wl.heads, wl.head_dim)
    want_dg = do32 * oc.permute(1, 0, 2)[tile_of]
    assert torch.allclose(dg.view_as(want_dg), want_dg, rtol=1e-5, atol=1e-6)
    sdv = dv.double().sum(0)
    want_sdv = (do32.double() * (1.0 + g32.double())).sum(0)
    assert parity.rel_l2(sdv.cpu().numpy(), want_sdv.cpu().numpy()) < 1e-3
    sdk = dk.double().sum(0).abs()
    assert (sdk <= 1e-2 * dk.double().abs().sum(0) + 1e-6).all()
    keep_gpu = run.att.keep_idx.cpu().numpy()
    scale = wl.head_dim ** -0.5
    k = parity.oracle_k(wl, pl)
    H = wl.heads
    spread = sorted({int(h) for h in np.linspace(0, H - 1, 8).round()})
    dk_heads = list(range(H)) if all_heads else spread
    # one key tile per head: a video tile, and a prefix tile (kept by every query
    # tile) on the first and last head
    rng = np.random.default_rng(13)
    tiles = {h: (int(rng.integers(pl.P)) if h in (dk_heads[0], dk_heads[-1]) and pl.P
                 else pl.P + int(rng.integers(pl.n_v))) for h in dk_heads}
    dkdv_host = {}
    for h, t in tiles.items():
        rows = torch.from_numpy(np.maximum(pl.row_src[t * pl.B:(t + 1) * pl.B], 0).astype(np.int64)).to(dev)
        dkdv_host[h] = (dk[rows, h].cpu().numpy(), dv[rows, h].cpu().numpy())
    toks = parity.sample_tokens(pl, 128, 11)
    dq_host = dq[torch.from_numpy(toks).to(dev)].cpu().numpy()
    del run, dq, dk, dv, dg
    torch.cuda.empty_cache()
    g_bits, d_bits = parity.bits(g_host), parity.bits(dout.cpu())
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for h in dk_heads:
        hr = oracle.head(inp.qb, inp.kb, inp.vb, h, pl, k, scale)
        assert np.array_equal(keep_gpu[h], hr.keep), f"keep-sets, head {h}"
        csr = oracle.key_lists_default(pl, hr.keep)
        means = (hr.qm, hr.km, hr.vm)
        t = tiles[h]
        real = pl.row_src[t * pl.B:(t + 1) * pl.B] >= 0
        want_k, want_v = oracle.dkdv_tile(inp.qb, inp.kb, inp.vb, g_bits, d_bits, h, pl, csr, scale,
                                          t, means=means)
        for nm, got, want in (("dk", dkdv_host[h][0], want_k), ("dv", dkdv_host[h][1], want_v)):
            got, want = got[real].astype(np.float64), want[real]
            rl = parity.rel_l2(got, want)
            mx = float(np.abs(got - want).max() / np.abs(want).max())
            worst[nm] = max(worst[nm], rl)
            assert rl <= GRAD_REL_L2 and mx <= GRAD_MAX_REL, f"{nm} head {h} tile {t}: {rl} {mx}"
        if h in spread:
            want = oracle.dq_tokens(inp.qb, inp.kb, inp.vb, g_bits, d_bits, h, pl, csr, scale, toks,
                                    means=means)
            got = dq_host[:, h, :].astype(np.float64)
            rl = parity.rel_l2(got, want)
            mx = float(np.abs(got - want).max() / np.abs(want).max())
            worst["dq"] = max(worst["dq"], rl)
            assert rl <= GRAD_REL_L2 and mx <= GRAD_MAX_REL, f"dq head {h}: {rl} {mx}"
        print(f"[{name} bwd] head {h}: dk/dv of tile {t} "
              f"({'prefix' if t < pl.P else 'video'}) ok", flush=True)
    print(f"[{name} bwd] worst rel-L2 {worst}", flush=True)
