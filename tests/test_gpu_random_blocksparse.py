"""A seeded sweep of random shapes through the block-sparse attention on top of the token selection.

Each draw picks the storage type, head dimension, KV heads and group size, a length from 1 to ~2500
(a single partial block to ~20 blocks of 128 rows; mostly several blocks), q, tau and gamma.  On the
compressed tensors the HIP stages produce:
- pooled block means bit-exact against the oracle's pool of the same stored rows;
- kept-block lists equal to the oracle's rule on those means (a float64 near-tie of the cumulative
  weight with gamma, within 1e-12, is the only allowed difference);
- every compressed row of the block-sparse attention within 2e-2 + 1e-2 |ref| (bf16) or
  1e-4 + 1e-4 |ref| (fp32) of the oracle on the HIP's lists;
- the fused block-sparse layer bitwise equal to its stages (select, attention, scatter + residual).
"""

import numpy as np
import pytest
import torch

import oracle
from token_sparse_attention_amd import binding
from token_sparse_attention_amd.configs import Workload
from test_gpu_blocksparse import Comp, kept_lists

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
B = oracle.BLOCK
SEEDS = range(24)


def draw(seed):
    r = np.random.default_rng(5000 + seed)
    dtype = "bf16" if r.random() < 0.7 else "f32"
    d = int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2]))
    G = int(r.choice([1, 2, 4]))
    L = int(np.exp(r.uniform(0, np.log(2500)))) if r.random() < 0.3 else int(r.integers(129, 2500))
    q = int(r.integers(1, min(L, 32) + 1))
    tau = float(r.choice([0.0, r.uniform(0.001, 0.3), r.uniform(0.5, 0.9)]))
    gamma = float(r.choice([0.0, 1.0, r.uniform(0.05, 0.99), r.uniform(0.05, 0.99)]))
    cfg = Workload(f"rbs{seed}", L=L, Hq=Hkv * G, Hkv=Hkv, d=d, q=q, tau=tau, dtype=dtype,
                   salient_frac=float(r.uniform(0.0, 0.1)), shared_frac=float(r.uniform(0, 1)),
                   sink=int(r.choice([0, 4])), seed=6000 + seed)
    return cfg, gamma


def f64(t):
    return t.double().cpu().numpy()


@pytest.mark.timeout(120)
@pytest.mark.parametrize("seed", SEEDS)
def test_random_block_sparse(gpu, seed):
    cfg, gamma = draw(seed)
    print(f"\n[{cfg.name}] {cfg.dtype} d={cfg.d} Hq={cfg.Hq} Hkv={cfg.Hkv} L={cfg.L} q={cfg.q} "
          f"tau={cfg.tau:.3f} gamma={gamma:.3f}", flush=True)
    comp = Comp(cfg, gpu)
    Lp, nb = comp.Lp, -(-comp.Lp // B)
    g = float(np.float32(gamma))
    blist, bcnt, lists, counts, qbar, kbar = comp.select(gamma)
    for h in range(cfg.Hq):
        assert np.array_equal(qbar[h, :nb], oracle.block_pool(f64(comp.Qh[h]), Lp)), h
        assert np.array_equal(kbar[h, :nb], oracle.block_pool(f64(comp.Kh[h]), Lp)), h
        assert (counts[h, nb:] == 0).all()
        want = oracle.block_select(qbar[h, :nb], kbar[h, :nb], g)
        got = kept_lists(lists, counts, h, nb)
        for I in range(nb):
            if np.array_equal(got[I], want[I]):
                continue
            z = (kbar[h, : I + 1] @ qbar[h, I]) / np.sqrt(cfg.d)
            a = np.exp(z - z.max())
            a /= a.sum()
            cum = np.cumsum(a[np.lexsort((np.arange(I + 1), -a))])
            assert np.min(np.abs(cum - g)) <= 1e-12, (h, I, got[I], want[I])
    Oh = comp.attend(blist, bcnt)
    atol, rtol = TOL[cfg.dtype]
    for h in range(cfg.Hq):
        if Lp == 0:
            break
        keep = kept_lists(lists, counts, h, nb)
        Qh, Kh = f64(comp.Qh[h, :Lp]), f64(comp.Kh[h, :Lp])
        Vh = f64(comp.Vht[h, :, :Lp]).T.copy()
        want = oracle.block_sparse_attention_rows(Qh, Kh, Vh, keep)
        got = f64(Oh[h, :Lp])
        bad = np.abs(got - want) > atol + rtol * np.abs(want)
        assert not bad.any(), (h, int(bad.sum()), float(np.abs(got - want).max()))
    ws = binding.workspace(binding.layer_block_sparse_workspace_bytes(comp.s), gpu)
    kl = torch.zeros(2, dtype=torch.int32, device=gpu)
    Y = torch.empty_like(comp.d["X"])
    binding.layer_block_sparse(comp.s, gamma, comp.d["Q"], comp.d["K"], comp.d["V"], comp.d["X"], Y, kl, ws)
    assert kl.tolist() == comp.kl.tolist()
    Y2 = torch.empty_like(comp.d["X"])
    binding.scatter_residual(comp.s, Oh, comp.idx, comp.inv, comp.kl[1:2], comp.d["X"], Y2)
    assert torch.equal(Y, Y2)
    print(f"[{cfg.name}] L'={Lp}, {nb} blocks, kept {int(counts[:, :nb].sum())} of "
          f"{cfg.Hq * nb * (nb + 1) // 2} block pairs ok", flush=True)
