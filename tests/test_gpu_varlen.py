"""Varlen batches (samples of different lengths, each with its own keep count L'_b) through the C ABI.

Every sample of a batch must come out bitwise identical to the same sample run on its own through
the single-sequence entry points (the same kernels on the same data); the oracle then checks the
numbers: scores, budget and selection of each sample as in the single-sequence parity tests, and
the layer output on the HIP's own selection within 2e-2 + 1e-2 |ref| (bf16) / 1e-4 + 1e-4 |ref|
(fp32).
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

BATCHES = {
    "bf16_d128_gqa": (Workload("varlen_bf16", L=1, Hq=4, Hkv=2, d=128, q=5, tau=0.05, dtype="bf16",
                               salient_frac=0.02, shared_frac=0.5, seed=31),
                      [1000, 37, 300, 129, 5, 256, 777]),
    "bf16_d64_heads8": (Workload("varlen_d64", L=1, Hq=8, Hkv=8, d=64, q=16, tau=0.02, dtype="bf16",
                                 salient_frac=0.03, shared_frac=0.5, sink=4, seed=32),
                        [513, 16, 2048, 700]),
    "f32_d128": (Workload("varlen_f32", L=1, Hq=2, Hkv=2, d=128, q=3, tau=0.02, dtype="f32",
                          salient_frac=0.05, shared_frac=1.0, seed=33),
                 [300, 17, 64]),
    "many_tiny_40": (Workload("varlen_many", L=1, Hq=8, Hkv=2, d=128, q=4, tau=0.1, dtype="bf16",
                              salient_frac=0.05, shared_frac=0.5, seed=34),
                     np.random.default_rng(34).integers(4, 200, size=40).tolist()),
}


def f64(t):
    return t.double().cpu().numpy()


def shape_for(cfg, L, tau=None):
    return binding.shape(L, cfg.Hq, cfg.Hkv, cfg.d, cfg.q, cfg.tau if tau is None else tau, cfg.dtype)


class Batch:
    def __init__(self, name, dev):
        self.cfg, self.lens = BATCHES[name]
        b = make_batch(self.cfg, self.lens)
        self.cu = [int(v) for v in b["cu_seqlens"]]
        self.host = {n: b[n] for n in ("Q", "K", "V", "X")}
        self.d = {n: b[n].to(dev) for n in ("Q", "K", "V", "X")}
        self.dev = dev
        self.s = shape_for(self.cfg, self.cu[-1])
        self.B = len(self.lens)

    def rows(self, b):
        return slice(self.cu[b], self.cu[b + 1])

    def sample(self, b):
        return {n: t[self.rows(b)].contiguous() for n, t in self.d.items()}


@pytest.fixture(scope="module", params=list(BATCHES))
def batch(request, gpu):
    return Batch(request.param, gpu)


def assert_close(got, want, dtype, what):
    atol, rtol = TOL[dtype]
    bad = np.abs(got - want) > atol + rtol * np.abs(want)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside {atol}+{rtol}|ref|, "
                           f"max |diff| {np.abs(got - want).max():.3e}")


def test_layer_varlen_equals_each_sample_alone(batch):
    cfg, dev = batch.cfg, batch.dev
    ws = binding.workspace(binding.layer_varlen_workspace_bytes(batch.s, batch.cu), dev)
    kLp = torch.full((batch.B, 2), -1, dtype=torch.int32, device=dev)
    Y = torch.empty_like(batch.d["X"])
    binding.layer_varlen(batch.s, batch.cu, batch.d["Q"], batch.d["K"], batch.d["V"], batch.d["X"], Y, kLp, ws)
    kl_all = kLp.tolist()
    for b in range(batch.B):
        sb = shape_for(cfg, batch.lens[b])
        smp = batch.sample(b)
        wsb = binding.workspace(binding.layer_workspace_bytes(sb), dev)
        kl = torch.zeros(2, dtype=torch.int32, device=dev)
        Yb = torch.empty_like(smp["X"])
        binding.layer(sb, smp["Q"], smp["K"], smp["V"], smp["X"], Yb, kl, wsb)
        assert kl_all[b] == kl.tolist(), b
        assert torch.equal(Y[batch.rows(b)], Yb), b
    # the keep counts really are ragged
    assert len({tuple(v) for v in kl_all}) > 1
    # deterministic, and in place (Y aliases X) gives the same result
    Xc = batch.d["X"].clone()
    binding.layer_varlen(batch.s, batch.cu, batch.d["Q"], batch.d["K"], batch.d["V"], Xc, Xc, None, ws)
    assert torch.equal(Xc, Y)


def test_layer_varlen_against_oracle(batch):
    """Each sample (up to 4, the shortest ones skipped only for the 40-sample batch) against the
    oracle: budget exact or inside the band, selection inside the tie band, Y on the HIP's sets."""
    cfg, dev = batch.cfg, batch.dev
    ws = binding.workspace(binding.layer_varlen_workspace_bytes(batch.s, batch.cu), dev)
    kLp = torch.zeros((batch.B, 2), dtype=torch.int32, device=dev)
    Y = torch.empty_like(batch.d["X"])
    binding.layer_varlen(batch.s, batch.cu, batch.d["Q"], batch.d["K"], batch.d["V"], batch.d["X"], Y, kLp, ws)
    Yc = f64(Y)
    tau = float(np.float32(cfg.tau))
    for b in range(min(batch.B, 4)):
        L = batch.lens[b]
        h = {n: f64(batch.host[n][batch.rows(b)]) for n in ("Q", "K", "V", "X")}
        s_h = oracle.head_scores(h["Q"], h["K"], cfg.q)
        k, Lp = kLp[b].tolist()
        rk, _ = oracle.budget(oracle.layer_score(s_h), tau)
        if k != rk:
            C = np.concatenate([[0.0], np.cumsum(np.sort(oracle.layer_score(s_h)))])
            assert C[k] >= tau * (1 - 1e-5) and (k == 0 or C[k - 1] < tau * (1 + 1e-5)), (b, k, rk)
        # the HIP's own selection for this sample (stage calls on the sample alone)
        sb = shape_for(cfg, L)
        smp = batch.sample(b)
        sws = binding.workspace(binding.stage_workspace_bytes(sb), dev)
        gs_h = torch.empty(cfg.Hq, L, dtype=torch.float32, device=dev)
        binding.score(sb, smp["Q"], smp["K"], gs_h, None, sws)
        idx = torch.empty(cfg.Hq, L, dtype=torch.int32, device=dev)
        binding.select(sb, gs_h, kLp[b, 1:2], idx, None, sws)
        idx = idx[:, :Lp].cpu().numpy().astype(np.int64)
        want_sets = oracle.select(s_h, Lp)
        for hh in range(cfg.Hq):
            diff = np.setxor1d(idx[hh], want_sets[hh])
            if len(diff):
                bnd = np.sort(s_h[hh])[::-1][Lp - 1]
                assert (np.abs(s_h[hh][diff] - bnd) <= 1e-6 * bnd).all(), (b, hh, diff)
        oq, ok, ov = oracle.gather(h["Q"], h["K"], h["V"], idx)
        Oh = oracle.compressed_attention(oq, ok, ov, idx)
        want = oracle.residual(h["X"], oracle.decompress(Oh, idx, L))
        assert_close(Yc[batch.rows(b)], want, cfg.dtype, f"sample {b} (L={L}, L'={Lp})")


def test_attn_varlen_equals_each_sample_alone(batch):
    """The compressed attention alone on gathered random selections, keep counts from 0 to L_b."""
    cfg, dev = batch.cfg, batch.dev
    dt = batch.d["Q"].dtype
    P = binding.varlen_capacity(batch.cu)
    caps = [binding.capacity(L) for L in batch.lens]
    off = np.concatenate([[0], np.cumsum(caps)]).astype(np.int64)
    Hq, d = cfg.Hq, cfg.d
    Qh = torch.zeros(Hq * P * d, dtype=dt, device=dev)
    Kh, Vht, Oh = torch.zeros_like(Qh), torch.zeros_like(Qh), torch.zeros_like(Qh)
    rng = np.random.default_rng(7)
    Lps, sets = [], []
    for b in range(batch.B):
        L, C = batch.lens[b], caps[b]
        Lp = [0, L, int(rng.integers(0, L + 1))][b % 3]
        sel = np.stack([np.sort(rng.choice(L, Lp, replace=False)) for _ in range(Hq)]).astype(np.int32)
        it = torch.full((Hq, L), -1, dtype=torch.int32)
        it[:, :Lp] = torch.from_numpy(sel)
        reg = slice(Hq * d * off[b], Hq * d * off[b + 1])
        smp = batch.sample(b)
        binding.gather(shape_for(cfg, L), smp["Q"], smp["K"], smp["V"], it.to(dev),
                       torch.tensor([Lp], dtype=torch.int32, device=dev),
                       Qh[reg].view(Hq, C, d), Kh[reg].view(Hq, C, d), Vht[reg].view(Hq, d, C))
        Lps.append(Lp)
        sets.append(sel.astype(np.int64))
    Lp_dev = torch.tensor(Lps, dtype=torch.int32, device=dev)
    binding.attn_causal_varlen(batch.s, batch.cu, Qh, Kh, Vht, Lp_dev, Oh)
    checked = 0
    for b in range(batch.B):
        L, C, Lp = batch.lens[b], caps[b], Lps[b]
        reg = slice(Hq * d * off[b], Hq * d * off[b + 1])
        O1 = torch.zeros(Hq, C, d, dtype=dt, device=dev)
        binding.attn_causal(shape_for(cfg, L), Qh[reg].view(Hq, C, d), Kh[reg].view(Hq, C, d),
                            Vht[reg].view(Hq, d, C), Lp_dev[b:b + 1], O1)
        Ov = Oh[reg].view(Hq, C, d)
        assert torch.equal(Ov[:, :Lp], O1[:, :Lp]), b
        if checked < 3 and Lp > 0:
            checked += 1
            h = {n: f64(batch.host[n][batch.rows(b)]) for n in ("Q", "K", "V")}
            oq, ok, ov = oracle.gather(h["Q"], h["K"], h["V"], sets[b])
            want = oracle.compressed_attention(oq, ok, ov, sets[b])
            assert_close(f64(Ov[:, :Lp]), want, cfg.dtype, f"attention sample {b}")


def test_dense_varlen_equals_each_sample_alone(batch):
    cfg, dev = batch.cfg, batch.dev
    ws = binding.workspace(binding.dense_varlen_workspace_bytes(batch.s, batch.cu), dev)
    Y = torch.empty_like(batch.d["X"])
    binding.dense_attn_causal_varlen(batch.s, batch.cu, batch.d["Q"], batch.d["K"], batch.d["V"], batch.d["X"], Y, ws)
    for b in range(batch.B):
        sb = shape_for(cfg, batch.lens[b])
        smp = batch.sample(b)
        wsb = binding.workspace(binding.dense_workspace_bytes(sb), dev)
        Yb = torch.empty_like(smp["X"])
        binding.dense_attn_causal(sb, smp["Q"], smp["K"], smp["V"], smp["X"], Yb, wsb)
        assert torch.equal(Y[batch.rows(b)], Yb), b
    b = int(np.argmax(batch.lens))
    h = {n: f64(batch.host[n][batch.rows(b)]) for n in ("Q", "K", "V", "X")}
    assert_close(f64(Y[batch.rows(b)]), oracle.dense_layer(h["Q"], h["K"], h["V"], h["X"]), cfg.dtype,
                 f"dense sample {b}")
