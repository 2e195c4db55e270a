"""A seeded sweep of random varlen batches against per-sample runs and the oracle.

Each draw picks the storage type, head dimension, KV heads and group size, q, tau and a sink, then a
batch of 1-12 samples (one draw in four: 33-40 samples, past the attention's 32-sequence segment
table) with lengths from q to ~1200, log-uniform.  For every batch:
- the fused varlen layer's keep counts and output rows equal each sample run alone through
  tsa_layer, bit for bit;
- every sample's keep count is exact for its own float32 s_l and inside the oracle's band; rows
  outside a head's selection equal X bit for bit; selected rows are within 2e-2 + 1e-2 |ref| (bf16)
  or 1e-4 + 1e-4 |ref| (fp32) of the oracle's attention on the GPU's selection plus X.
"""

import numpy as np
import pytest
import torch

import oracle
from token_sparse_attention_amd import binding
from token_sparse_attention_amd.configs import Workload
from token_sparse_attention_amd.inputs import make_batch

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
SEEDS = range(24)


def draw(seed):
    r = np.random.default_rng(3000 + seed)
    dtype = "bf16" if r.random() < 0.7 else "f32"
    d = int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4]))
    q = int(np.exp(r.uniform(0, np.log(64))))
    tau = float(r.choice([0.0, r.uniform(0.001, 0.3), r.uniform(0.5, 0.95)]))
    sink = int(r.choice([0, 4]))
    B = int(r.integers(33, 41)) if seed % 4 == 3 else int(r.integers(1, 13))
    hi = 300 if B > 32 else 1200
    lens = [int(np.exp(r.uniform(np.log(q), np.log(hi)))) for _ in range(B)]
    cfg = Workload(f"rvar{seed}", L=1, Hq=Hkv * G, Hkv=Hkv, d=d, q=q, tau=tau, dtype=dtype,
                   salient_frac=float(r.uniform(0.0, 0.1)), shared_frac=float(r.uniform(0, 1)),
                   sink=sink, seed=4000 + seed)
    return cfg, lens


def f64(t):
    return t.double().cpu().numpy()


def shape_for(cfg, L):
    return binding.shape(L, cfg.Hq, cfg.Hkv, cfg.d, cfg.q, cfg.tau, cfg.dtype)


@pytest.mark.timeout(120)
@pytest.mark.parametrize("seed", SEEDS)
def test_random_varlen_batch(gpu, seed):
    cfg, lens = draw(seed)
    print(f"\n[{cfg.name}] {cfg.dtype} d={cfg.d} Hq={cfg.Hq} Hkv={cfg.Hkv} q={cfg.q} tau={cfg.tau:.3f} "
          f"B={len(lens)} lengths={lens}", flush=True)
    b = make_batch(cfg, lens)
    cu = [int(v) for v in b["cu_seqlens"]]
    host = {n: b[n] for n in ("Q", "K", "V", "X")}
    dv = {n: t.to(gpu) for n, t in host.items()}
    s = shape_for(cfg, cu[-1])
    ws = binding.workspace(binding.layer_varlen_workspace_bytes(s, cu), gpu)
    kLp = torch.full((len(lens), 2), -1, dtype=torch.int32, device=gpu)
    Y = torch.empty_like(dv["X"])
    binding.layer_varlen(s, cu, dv["Q"], dv["K"], dv["V"], dv["X"], Y, kLp, ws)
    kl_all = kLp.tolist()
    Yc = f64(Y)
    tau = float(np.float32(cfg.tau))
    G = cfg.Hq // cfg.Hkv
    atol, rtol = TOL[cfg.dtype]
    for i, L in enumerate(lens):
        r = slice(cu[i], cu[i + 1])
        smp = {n: t[r].contiguous() for n, t in dv.items()}
        sb = shape_for(cfg, L)
        # the sample alone: the same keep count and the same bits
        kl = torch.zeros(2, dtype=torch.int32, device=gpu)
        Yb = torch.empty_like(smp["X"])
        binding.layer(sb, smp["Q"], smp["K"], smp["V"], smp["X"], Yb, kl, binding.workspace(
            binding.layer_workspace_bytes(sb), gpu))
        assert kl.tolist() == kl_all[i], (i, kl.tolist(), kl_all[i])
        assert torch.equal(Y[r], Yb), i
        # the sample's stages alone, for its float32 scores and its selection
        sws = binding.workspace(binding.stage_workspace_bytes(sb), gpu)
        s_h = torch.empty(cfg.Hq, L, dtype=torch.float32, device=gpu)
        s_l = torch.empty(L, dtype=torch.float32, device=gpu)
        binding.score(sb, smp["Q"], smp["K"], s_h, s_l, sws)
        k2 = torch.zeros(2, dtype=torch.int32, device=gpu)
        binding.budget(sb, s_l, k2[0:1], k2[1:2], sws)
        k, Lp = kl_all[i]
        assert k2.tolist() == [k, Lp], i
        idx_t = torch.empty(cfg.Hq, L, dtype=torch.int32, device=gpu)
        binding.select(sb, s_h, k2[1:2], idx_t, None, sws)
        idx = idx_t[:, :Lp].cpu().numpy().astype(np.int64)
        assert (idx == oracle.select(f64(s_h), Lp)).all(), i
        # against the oracle
        h = {n: f64(host[n][r]) for n in ("Q", "K", "V", "X")}
        ref_sl = oracle.layer_score(oracle.head_scores(h["Q"], h["K"], cfg.q))
        rk, _ = oracle.budget(ref_sl, tau)
        if k != rk:
            C = np.concatenate([[0.0], np.cumsum(np.sort(ref_sl))])
            assert C[k] >= tau * (1 - 1e-5) and (k == 0 or C[k - 1] < tau * (1 + 1e-5)), (i, k, rk)
        got = Yc[r]
        for hh in range(cfg.Hq):
            un = np.setdiff1d(np.arange(L), idx[hh])
            assert (got[un, hh] == h["X"][un, hh]).all(), (i, hh)
            if Lp == 0:
                continue
            pos = idx[hh]
            O = oracle.attention_rows(h["Q"][pos, hh], h["K"][pos, hh // G], h["V"][pos, hh // G], pos)
            want = h["X"][pos, hh] + O
            bad = np.abs(got[pos, hh] - want) > atol + rtol * np.abs(want)
            assert not bad.any(), (i, hh, int(bad.sum()), float(np.abs(got[pos, hh] - want).max()))
    print(f"[{cfg.name}] keep counts {[v[1] for v in kl_all]} ok", flush=True)
