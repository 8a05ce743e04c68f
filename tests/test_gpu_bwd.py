"""Backward pass: HIP path vs the CPU oracle, through the C ABI.

Gradients of the layer with the keep sets held fixed, for q, k, v and the gate.
Both sides use the same bf16 inputs and gate g; the oracle works in fp64, the
GPU rounds P and dS to bf16 for the matrix products (relative error 2^-9 each)
and takes the softmax row term D_t from the bf16 output (another 2^-9 on
O_fine). Each gradient is a sum of such terms with independent signs, so its
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


def run_case(wl, ref=None, heads=None):
    """ref: None (default mode) or (ref_sparsity, ref_keep_k)."""
    inp = parity.make_inputs(wl)
    pl = parity.oracle_plan(wl)
    g_bits = oracle.gate_proj(parity.bits(inp.x), parity.bits(inp.w))
    g = torch.from_numpy(g_bits.view(np.int16)).view(torch.bfloat16)
    if ref is None:
        run = parity.run_gpu(inp, gate=g)
    else:
        run = parity.run_gpu_ref(inp, ref[0], ref[1], gate=g)
    dout = make_dout(wl)
    dev = run.out.device
    qd, kd, vd = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    dq, dk, dv, dg = run.att.backward(qd, kd, vd, run.g, run.out, dout.to(dev))
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


def test_bwd_tiny():
    print("[gpu] bwd tiny", flush=True)
    run_case(workloads.WORKLOADS["tiny"])


def test_bwd_mid_two_heads():
    print("[gpu] bwd mid", flush=True)
    wl = workloads.WORKLOADS["mid"]
    run_case(wl, heads=[0, wl.heads - 1])
