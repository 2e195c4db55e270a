"""Block sparsity inside the compressed space (token filter first, then block-sparse attention) through
the C ABI, against the oracle.

Acceptance: pooled means bit-exact (float64 sums of the stored values, one division, one rounding
to float32 on both sides); kept-block lists identical to the oracle's rule applied to those means
(a difference is allowed only where the cumulative weight meets gamma within 1e-12, i.e. a float64
near-tie); attention on the HIP's lists within 2e-2 + 1e-2 |ref| (bf16) / 1e-4 + 1e-4 |ref|
(fp32); with every block kept, bit-identical to the plain compressed attention.
"""

import numpy as np
import pytest
import torch

import oracle
from token_sparse_attention_amd import binding
from token_sparse_attention_amd.configs import WORKLOADS, Workload, scaled
from token_sparse_attention_amd.inputs import make_layer

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
B = oracle.BLOCK

CASES = {
    "bf16_gqa_L1000": Workload("bs_gqa", L=1000, Hq=4, Hkv=2, d=128, q=5, tau=0.05, dtype="bf16",
                               salient_frac=0.02, shared_frac=0.5, seed=41),
    "bf16_d64_L777": Workload("bs_d64", L=777, Hq=2, Hkv=1, d=64, q=16, tau=0.01, dtype="bf16",
                              salient_frac=0.03, shared_frac=0.5, sink=8, seed=42),
    "f32_d128_L300": Workload("bs_f32", L=300, Hq=2, Hkv=2, d=128, q=3, tau=0.02, dtype="f32",
                              salient_frac=0.05, shared_frac=1.0, seed=43),
    "bf16_L4096_h8": scaled(WORKLOADS[2], 4096, Hq=8, Hkv=2, seed=44),
}


def f64(t):
    return t.double().cpu().numpy()


class Comp:
    """A layer's compressed tensors produced by the HIP stages (score, budget, select, gather)."""

    def __init__(self, cfg, dev):
        self.cfg, self.dev = cfg, dev
        inp = make_layer(cfg)
        self.d = {n: inp[n].to(dev) for n in ("Q", "K", "V", "X")}
        self.s = binding.shape_of(cfg)
        self.C = binding.capacity(cfg.L)
        self.NB = binding.block_count(cfg.L)
        L, Hq, d = cfg.L, cfg.Hq, cfg.d
        sws = binding.workspace(binding.stage_workspace_bytes(self.s), dev)
        s_h = torch.empty(Hq, L, dtype=torch.float32, device=dev)
        s_l = torch.empty(L, dtype=torch.float32, device=dev)
        binding.score(self.s, self.d["Q"], self.d["K"], s_h, s_l, sws)
        self.kl = torch.zeros(2, dtype=torch.int32, device=dev)
        binding.budget(self.s, s_l, self.kl[0:1], self.kl[1:2], sws)
        self.idx = torch.empty(Hq, L, dtype=torch.int32, device=dev)
        self.inv = torch.empty(Hq, L, dtype=torch.int32, device=dev)
        binding.select(self.s, s_h, self.kl[1:2], self.idx, self.inv, sws)
        dt = self.d["Q"].dtype
        self.Qh = torch.empty(Hq, self.C, d, dtype=dt, device=dev)
        self.Kh = torch.empty_like(self.Qh)
        self.Vht = torch.empty(Hq, d, self.C, dtype=dt, device=dev)
        binding.gather(self.s, self.d["Q"], self.d["K"], self.d["V"], self.idx, self.kl[1:2], self.Qh, self.Kh,
                       self.Vht)
        self.Lp = int(self.kl[1])

    def select(self, gamma, Lp_dev=None):
        Hq, NB = self.cfg.Hq, self.NB
        blist = torch.full((Hq, NB, NB), -1, dtype=torch.int16, device=self.dev)
        bcnt = torch.full((Hq, NB), -1, dtype=torch.int32, device=self.dev)
        ws = binding.workspace(binding.block_select_workspace_bytes(self.s), self.dev)
        binding.block_select(self.s, gamma, self.Qh, self.Kh, self.kl[1:2] if Lp_dev is None else Lp_dev,
                             blist, bcnt, ws)
        nbytes = Hq * NB * self.cfg.d * 4
        off = (nbytes + 255) // 256 * 256
        qbar = ws[:nbytes].view(torch.float32).view(Hq, NB, self.cfg.d)
        kbar = ws[off:off + nbytes].view(torch.float32).view(Hq, NB, self.cfg.d)
        lists = blist.cpu().numpy().view(np.uint16)
        counts = bcnt.cpu().numpy()
        return blist, bcnt, lists, counts, f64(qbar), f64(kbar)

    def attend(self, blist, bcnt):
        Oh = torch.zeros_like(self.Qh)
        binding.attn_block_sparse(self.s, self.Qh, self.Kh, self.Vht, self.kl[1:2], blist, bcnt, Oh)
        return Oh


@pytest.fixture(scope="module", params=list(CASES))
def comp(request, gpu):
    return Comp(CASES[request.param], gpu)


def assert_close(got, want, dtype, what):
    atol, rtol = TOL[dtype]
    bad = np.abs(got - want) > atol + rtol * np.abs(want)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside {atol}+{rtol}|ref|, "
                           f"max |diff| {np.abs(got - want).max():.3e}")


def kept_lists(lists, counts, h, nb):
    return [lists[h, I, :counts[h, I]].astype(np.int64) for I in range(nb)]


def test_pool_bit_exact(comp):
    _, _, _, _, qbar, kbar = comp.select(0.9)
    Lp, nb = comp.Lp, -(-comp.Lp // B)
    for h in range(comp.cfg.Hq):
        assert np.array_equal(qbar[h, :nb], oracle.block_pool(f64(comp.Qh[h]), Lp)), h
        assert np.array_equal(kbar[h, :nb], oracle.block_pool(f64(comp.Kh[h]), Lp)), h


@pytest.mark.parametrize("gamma", [0.0, 0.3, 0.9, 1.0])
def test_select_against_oracle(comp, gamma):
    _, _, lists, counts, qbar, kbar = comp.select(gamma)
    g = float(np.float32(gamma))
    nb = -(-comp.Lp // B)
    for h in range(comp.cfg.Hq):
        assert (counts[h, nb:] == 0).all()
        want = oracle.block_select(qbar[h, :nb], kbar[h, :nb], g)
        got = kept_lists(lists, counts, h, nb)
        for I in range(nb):
            if np.array_equal(got[I], want[I]):
                continue
            # only a float64 near-tie of the cumulative weight with gamma may differ
            z = (kbar[h, : I + 1] @ qbar[h, I]) / np.sqrt(comp.cfg.d)
            a = np.exp(z - z.max())
            a /= a.sum()
            cum = np.cumsum(a[np.lexsort((np.arange(I + 1), -a))])
            assert np.min(np.abs(cum - g)) <= 1e-12, (h, I, got[I], want[I])
        if gamma >= 1.0:
            assert all(len(k) == I + 1 for I, k in enumerate(got))
    if gamma == 0.3 and nb >= 8:               # the rule really drops blocks here
        assert counts[:, :nb].sum() < comp.cfg.Hq * nb * (nb + 1) // 2


@pytest.mark.parametrize("gamma", [0.3, 0.9])
def test_attention_against_oracle(comp, gamma):
    blist, bcnt, lists, counts, _, _ = comp.select(gamma)
    Oh = comp.attend(blist, bcnt)
    Lp, nb = comp.Lp, -(-comp.Lp // B)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(min(Lp, 8)), np.arange(max(0, Lp - 8), Lp),
                                     rng.integers(0, max(Lp, 1), size=64),
                                     [r for k in range(B, Lp, B) for r in (k - 1, k, k + 1)]]))
    rows = rows[(rows >= 0) & (rows < Lp)]
    for h in range(comp.cfg.Hq):
        keep = kept_lists(lists, counts, h, nb)
        Qh, Kh = f64(comp.Qh[h, :Lp]), f64(comp.Kh[h, :Lp])
        Vh = f64(comp.Vht[h, :, :Lp]).T.copy()
        want = oracle.block_sparse_attention_rows(Qh, Kh, Vh, keep, rows=rows)
        assert_close(f64(Oh[h, rows]), want, comp.cfg.dtype, f"head {h} gamma {gamma}")
    assert sum(int(c) for c in counts[:, :nb].ravel()) >= 2 * nb - 1


def test_full_coverage_is_the_plain_attention_bitwise(comp):
    blist, bcnt, _, counts, _, _ = comp.select(1.0)
    Oh = comp.attend(blist, bcnt)
    O1 = torch.zeros_like(comp.Qh)
    binding.attn_causal(comp.s, comp.Qh, comp.Kh, comp.Vht, comp.kl[1:2], O1)
    Lp = comp.Lp
    assert torch.equal(Oh[:, :Lp], O1[:, :Lp])


def test_layer_block_sparse_equals_its_stages(comp):
    cfg, dev = comp.cfg, comp.dev
    gamma = 0.5
    ws = binding.workspace(binding.layer_block_sparse_workspace_bytes(comp.s), dev)
    kl = torch.zeros(2, dtype=torch.int32, device=dev)
    Y = torch.empty_like(comp.d["X"])
    binding.layer_block_sparse(comp.s, gamma, comp.d["Q"], comp.d["K"], comp.d["V"], comp.d["X"], Y, kl, ws)
    assert kl.tolist() == comp.kl.tolist()
    blist, bcnt, _, _, _, _ = comp.select(gamma)
    Oh = comp.attend(blist, bcnt)
    Y2 = torch.empty_like(comp.d["X"])
    binding.scatter_residual(comp.s, Oh, comp.idx, comp.inv, comp.kl[1:2], comp.d["X"], Y2)
    assert torch.equal(Y, Y2)
    # a smaller gamma keeps fewer blocks than a larger one
    _, _, _, c_lo, _, _ = comp.select(0.2)
    _, _, _, c_hi, _, _ = comp.select(0.95)
    assert c_lo.sum() <= c_hi.sum()


def test_empty_keep_set(gpu):
    c = Comp(CASES["bf16_gqa_L1000"], gpu)
    zero = torch.zeros(1, dtype=torch.int32, device=gpu)
    blist, bcnt, _, counts, _, _ = c.select(0.9, Lp_dev=zero)
    assert (counts == 0).all()
    Oh = torch.full_like(c.Qh, 3.0)
    binding.attn_block_sparse(c.s, c.Qh, c.Kh, c.Vht, zero, blist, bcnt, Oh)
    assert (Oh == 3.0).all()
