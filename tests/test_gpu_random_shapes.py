"""A seeded sweep of random shapes through the whole layer, against the oracle.

Each draw picks the storage type, the head dimension, the KV heads and the group size, a length
from 1 to ~2500 (log-uniform, so most lengths leave a ragged last tile), the recent-query count, tau
(zero, small or large), a sink and the planted salient fractions.  For every draw:
- s_h and s_l within the score tolerance of the oracle (1e-6 relative bf16, 2e-7 fp32);
- k exact for the GPU's float32 s_l (exact integer arithmetic), and inside the oracle's band;
- the selection exactly the oracle's on the GPU's scores, and tie-band equal to the oracle's own;
- the fused layer's keep counts equal the stage calls'; rows outside a head's selection equal X
  bit for bit; every selected row within 2e-2 + 1e-2 |ref| (bf16) or 1e-4 + 1e-4 |ref| (fp32) of
  the oracle's attention on the GPU's selection plus X.
Every third draw also runs the fixed-ratio layer at a random sparsity.
"""

import numpy as np
import pytest
import torch

import oracle
from token_sparse_attention_amd import binding
from token_sparse_attention_amd.configs import Workload
from token_sparse_attention_amd.inputs import make_layer

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
SCORE_RTOL = {"bf16": 1e-6, "f32": 2e-7}
SEEDS = range(96)


def draw(seed):
    r = np.random.default_rng(1000 + seed)
    dtype = "bf16" if r.random() < 0.7 else "f32"
    d = int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 8]))
    L = int(np.exp(r.uniform(0, np.log(2500))))
    q = int(r.integers(1, min(L, 64) + 1))
    tau = float(r.choice([0.0, r.uniform(0.001, 0.3), r.uniform(0.5, 0.95)]))
    sink = int(r.choice([0, 0, 4, 64]))
    return Workload(f"rand{seed}", L=L, Hq=Hkv * G, Hkv=Hkv, d=d, q=q, tau=tau, dtype=dtype,
                    salient_frac=float(r.uniform(0.0, 0.1)), shared_frac=float(r.uniform(0, 1)),
                    sink=min(sink, L), seed=2000 + seed)


def f64(t):
    return t.double().cpu().numpy()


def exact_budget(vals32, tau):
    """min k with (sum of the k smallest float32 values) >= tau, in integers (float32 x 2^149)."""
    v = sorted(int(x * 2.0 ** 149) for x in vals32.astype(np.float64))
    target = int(np.float64(tau) * 2.0 ** 149)
    if target <= 0:
        return 0
    acc = 0
    for j, iv in enumerate(v):
        acc += iv
        if acc >= target:
            return j + 1
    return len(v)


@pytest.mark.timeout(120)
@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_layer(gpu, seed):
    cfg = draw(seed)
    print(f"\n[{cfg.name}] {cfg}", flush=True)
    L, Hq, Hkv, d = cfg.L, cfg.Hq, cfg.Hkv, cfg.d
    inp = make_layer(cfg)
    Q, K, V, X = (inp[n].to(gpu) for n in ("Q", "K", "V", "X"))
    h = {n: f64(inp[n]) for n in ("Q", "K", "V", "X")}
    s = binding.shape_of(cfg)
    tau = float(np.float32(cfg.tau))

    sws = binding.workspace(binding.stage_workspace_bytes(s), gpu)
    s_h = torch.empty(Hq, L, dtype=torch.float32, device=gpu)
    s_l = torch.empty(L, dtype=torch.float32, device=gpu)
    binding.score(s, Q, K, s_h, s_l, sws)
    ref_sh = oracle.head_scores(h["Q"], h["K"], cfg.q)
    ref_sl = oracle.layer_score(ref_sh)
    rtol = SCORE_RTOL[cfg.dtype]
    np.testing.assert_allclose(f64(s_h), ref_sh, rtol=rtol, atol=1e-30)
    np.testing.assert_allclose(f64(s_l), ref_sl, rtol=rtol, atol=1e-30)

    kl = torch.zeros(2, dtype=torch.int32, device=gpu)
    binding.budget(s, s_l, kl[0:1], kl[1:2], sws)
    k, Lp = kl.tolist()
    assert k + Lp == L and k == exact_budget(s_l.cpu().numpy(), tau)
    rk, _ = oracle.budget(ref_sl, tau)
    if k != rk:
        C = np.concatenate([[0.0], np.cumsum(np.sort(ref_sl))])
        assert C[k] >= tau * (1 - 1e-5) and (k == 0 or C[k - 1] < tau * (1 + 1e-5)), (k, rk)

    idx_t = torch.full((Hq, L), -7, dtype=torch.int32, device=gpu)
    binding.select(s, s_h, kl[1:2], idx_t, None, sws)
    idx = idx_t[:, :Lp].cpu().numpy().astype(np.int64)
    assert (idx == oracle.select(f64(s_h), Lp)).all()
    want_idx = oracle.select(ref_sh, Lp)
    for hh in range(Hq):
        diff = np.setxor1d(idx[hh], want_idx[hh])
        if len(diff):
            b = np.sort(ref_sh[hh])[::-1][Lp - 1]
            assert (np.abs(ref_sh[hh][diff] - b) <= 1e-6 * b).all(), (hh, diff)

    lws = binding.workspace(binding.layer_workspace_bytes(s), gpu)
    kl2 = torch.zeros(2, dtype=torch.int32, device=gpu)
    Y = torch.empty_like(X)
    binding.layer(s, Q, K, V, X, Y, kl2, lws)
    assert kl2.tolist() == [k, Lp]
    got = f64(Y)
    G = Hq // Hkv
    atol, rtol = TOL[cfg.dtype]
    for hh in range(Hq):
        un = np.setdiff1d(np.arange(L), idx[hh])
        assert (got[un, hh] == h["X"][un, hh]).all(), hh
        if Lp == 0:
            continue
        pos = idx[hh]
        O = oracle.attention_rows(h["Q"][pos, hh], h["K"][pos, hh // G], h["V"][pos, hh // G], pos)
        want = h["X"][pos, hh] + O
        bad = np.abs(got[pos, hh] - want) > atol + rtol * np.abs(want)
        assert not bad.any(), (hh, int(bad.sum()), float(np.abs(got[pos, hh] - want).max()))
    print(f"[{cfg.name}] k={k} L'={Lp} ok", flush=True)


@pytest.mark.timeout(120)
@pytest.mark.parametrize("seed", range(0, 96, 3))
def test_random_shape_layer_fixed_ratio(gpu, seed):
    """The fixed-ratio layer on every third draw, at a random sparsity in [0, 1): k exactly the
    oracle's integer rule, the selection exactly the oracle's on the GPU's scores, unselected rows
    equal to X bit for bit, selected rows within the tolerance of the oracle's attention plus X."""
    cfg = draw(seed)
    sparsity = float(np.random.default_rng(7000 + seed).uniform(0.0, 1.0))
    print(f"\n[{cfg.name}] {cfg} sparsity={sparsity:.4f}", flush=True)
    L, Hq, Hkv = cfg.L, cfg.Hq, cfg.Hkv
    inp = make_layer(cfg)
    Q, K, V, X = (inp[n].to(gpu) for n in ("Q", "K", "V", "X"))
    h = {n: f64(inp[n]) for n in ("Q", "K", "V", "X")}
    s = binding.shape_of(cfg)
    lws = binding.workspace(binding.layer_workspace_bytes(s), gpu)
    kl = torch.zeros(2, dtype=torch.int32, device=gpu)
    Y = torch.empty_like(X)
    binding.layer_ratio(s, sparsity, Q, K, V, X, Y, kl, lws)
    k, Lp = kl.tolist()
    assert (k, Lp) == oracle.budget_fixed_ratio(L, sparsity)
    sws = binding.workspace(binding.stage_workspace_bytes(s), gpu)
    s_h = torch.empty(Hq, L, dtype=torch.float32, device=gpu)
    s_l = torch.empty(L, dtype=torch.float32, device=gpu)
    binding.score(s, Q, K, s_h, s_l, sws)
    idx_t = torch.empty(Hq, L, dtype=torch.int32, device=gpu)
    binding.select(s, s_h, kl[1:2], idx_t, None, sws)
    idx = idx_t[:, :Lp].cpu().numpy().astype(np.int64)
    assert (idx == oracle.select(f64(s_h), Lp)).all()
    got = f64(Y)
    G = Hq // Hkv
    atol, rtol = TOL[cfg.dtype]
    for hh in range(Hq):
        un = np.setdiff1d(np.arange(L), idx[hh])
        assert (got[un, hh] == h["X"][un, hh]).all(), hh
        if Lp == 0:
            continue
        pos = idx[hh]
        O = oracle.attention_rows(h["Q"][pos, hh], h["K"][pos, hh // G], h["V"][pos, hh // G], pos)
        want = h["X"][pos, hh] + O
        bad = np.abs(got[pos, hh] - want) > atol + rtol * np.abs(want)
        assert not bad.any(), (hh, int(bad.sum()), float(np.abs(got[pos, hh] - want).max()))
