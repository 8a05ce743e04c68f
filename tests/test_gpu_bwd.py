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


@pytest.mark.parametrize("name,train", [("h3", False), ("veda", False), ("h3", True)])
def test_bwd_full_size_sampled(name, train):
    """Full-size layers: dq on sampled tokens against the oracle, dg = dout * O_coarse
    on every token, and the identities sum(dv) = sum(dout * (1 + g)), sum(dk) = 0."""
    wl = workloads.WORKLOADS[name]
    print(f"[gpu] bwd full size {name}: inputs", flush=True)
    inp = parity.make_inputs(wl)
    pl = parity.oracle_plan(wl)
    dev = "cuda"
    import tile_sparse_video_amd as tsv
    xd, wd = inp.x.to(dev), inp.w.to(dev)
    g = torch.empty((wl.tokens, wl.heads * wl.head_dim), dtype=torch.bfloat16, device=dev)
    tsv.vsa_gate_proj(xd, wd, g)
    del xd, wd
    run = parity.run_gpu(inp, gate=g)
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
    scale = wl.head_dim ** -0.5
    k = parity.oracle_k(wl, pl)
    toks = parity.sample_tokens(pl, 48, 11)
    g_bits = parity.bits(run.g.cpu())
    dq_host = dq[torch.from_numpy(toks).to(dev)].cpu().numpy()
    del run, dq, dk, dv, dg
    torch.cuda.empty_cache()
    for h in sorted({0, wl.heads - 1}):
        print(f"[gpu] bwd full size {name}: oracle head {h}", flush=True)
        hr = oracle.head(inp.qb, inp.kb, inp.vb, h, pl, k, scale)
        csr = oracle.key_lists_default(pl, hr.keep)
        want = oracle.dq_tokens(inp.qb, inp.kb, inp.vb, g_bits, parity.bits(dout.cpu()), h, pl, csr,
                                scale, toks, means=(hr.qm, hr.km, hr.vm))
        got = dq_host[:, h, :].astype(np.float64)
        rl = parity.rel_l2(got, want)
        mx = float(np.abs(got - want).max() / np.abs(want).max())
        print(f"[{name} bwd] head {h} dq rel-L2 {rl:.2e} max {mx:.2e}", flush=True)
        assert rl <= GRAD_REL_L2 and mx <= GRAD_MAX_REL
