"""The attention's two workgroup shapes: 4 waves (128 query rows) when every sequence of a launch
has at most 49152 rows, 8 waves (256 rows) otherwise.  A row's keys are walked in the same 64-key
tiles in either shape, so a short sequence must give the same bits both ways.

A varlen batch of one long (50001) and one short (3000) sample launches its attention with 8-wave
workgroups for both samples; the short sample alone takes 4-wave workgroups.  Checked for d = 64 and
d = 128, for the fused layer and for the dense baseline:
- the batch's rows of each sample equal that sample run alone, bit for bit (and the keep counts);
- the long sample's layer output is within 2e-2 + 1e-2 |ref| of the oracle on sampled rows, on the
  GPU's own selection.
"""

import numpy as np
import pytest
import torch

import oracle
from token_sparse_attention_amd import binding
from token_sparse_attention_amd.configs import Workload
from token_sparse_attention_amd.inputs import make_batch

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2


@pytest.mark.timeout(300)
@pytest.mark.parametrize("d", [64, 128])
def test_short_sample_same_bits_in_both_shapes(gpu, d):
    cfg = Workload(f"waves_d{d}", L=1, Hq=8, Hkv=2, d=d, q=16, tau=0.02, dtype="bf16",
                   salient_frac=0.01, shared_frac=0.5, seed=80 + d)
    lengths = [50001, 3000]
    b = make_batch(cfg, lengths)
    cu = [int(v) for v in b["cu_seqlens"]]
    Q, K, V, X = (b[n].to(gpu) for n in ("Q", "K", "V", "X"))
    s = binding.shape(cu[-1], cfg.Hq, cfg.Hkv, d, cfg.q, cfg.tau, "bf16")
    ws = binding.workspace(binding.layer_varlen_workspace_bytes(s, cu), gpu)
    kl = torch.zeros(len(lengths), 2, dtype=torch.int32, device=gpu)
    Y = torch.empty_like(X)
    binding.layer_varlen(s, cu, Q, K, V, X, Y, kl, ws)
    dws = binding.workspace(binding.dense_varlen_workspace_bytes(s, cu), gpu)
    Yd = torch.empty_like(X)
    binding.dense_attn_causal_varlen(s, cu, Q, K, V, X, Yd, dws)
    torch.cuda.synchronize()
    for i, n in enumerate(lengths):
        a, e = cu[i], cu[i + 1]
        si = binding.shape(n, cfg.Hq, cfg.Hkv, d, cfg.q, cfg.tau, "bf16")
        lws = binding.workspace(binding.layer_workspace_bytes(si), gpu)
        kli = torch.zeros(2, dtype=torch.int32, device=gpu)
        Yi = torch.empty_like(X[a:e])
        binding.layer(si, Q[a:e], K[a:e], V[a:e], X[a:e], Yi, kli, lws)
        Ydi = torch.empty_like(X[a:e])
        binding.dense_attn_causal(si, Q[a:e], K[a:e], V[a:e], X[a:e], Ydi,
                                  binding.workspace(binding.dense_workspace_bytes(si), gpu))
        torch.cuda.synchronize()
        assert kli.tolist() == kl[i].tolist(), (n, kli.tolist(), kl[i].tolist())
        assert torch.equal(Yi, Y[a:e]), n
        assert torch.equal(Ydi, Yd[a:e]), n

    # the long sample against the oracle, on the GPU's own selection
    n = lengths[0]
    si = binding.shape(n, cfg.Hq, cfg.Hkv, d, cfg.q, cfg.tau, "bf16")
    sws = binding.workspace(binding.stage_workspace_bytes(si), gpu)
    s_h = torch.empty(cfg.Hq, n, dtype=torch.float32, device=gpu)
    s_l = torch.empty(n, dtype=torch.float32, device=gpu)
    k2 = torch.zeros(2, dtype=torch.int32, device=gpu)
    idx = torch.empty(cfg.Hq, n, dtype=torch.int32, device=gpu)
    binding.score(si, Q[:n], K[:n], s_h, s_l, sws)
    binding.budget(si, s_l, k2[0:1], k2[1:2], sws)
    binding.select(si, s_h, k2[1:2], idx, None, sws)
    Lp = int(k2[1].item())
    assert k2.tolist() == kl[0].tolist()
    G = cfg.Hq // cfg.Hkv
    f64 = lambda t: t.double().cpu().numpy()
    rng = np.random.default_rng(d)
    for h in (0, 3, 6):
        sel = idx[h, :Lp].cpu().numpy().astype(np.int64)
        rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, Lp // 2, Lp - 1], rng.integers(0, Lp, 8)]))
        t = torch.from_numpy(sel).to(gpu)
        want = oracle.attention_rows(f64(Q[t, h]), f64(K[t, h // G]), f64(V[t, h // G]), sel, rows)
        tok = torch.from_numpy(sel[rows]).to(gpu)
        ref = f64(X[tok, h]) + want
        got = f64(Y[tok, h])
        bad = np.abs(got - ref) > ATOL + RTOL * np.abs(ref)
        assert not bad.any(), (d, h, int(bad.sum()), float(np.abs(got - ref).max()))
