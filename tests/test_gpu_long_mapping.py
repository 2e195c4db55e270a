"""Long compressed sequences (at least 163840 rows) run the bf16 attention with 4 heads in flight
instead of 8, and sequences of at most 16384 rows spread each XCD's query blocks over all its heads:
two different blockIdx -> (head, query block) maps.  These tests check, through the C ABI,
that the map covers every query row of every head exactly once and nothing past the keep count:
the output starts as NaN, every row below L' must be finite afterwards and every row from L' on
must still be NaN.  Sampled rows are compared with the oracle's attention, computed one by one
(2e-2 + 1e-2 |ref|), and a varlen launch that mixes a long sequence (4 heads in flight) with short
ones (8) must match each sequence launched alone bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
from token_sparse_attention_amd import binding

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2


def rand_compressed(Hq, C, d, dev, seed):
    g = torch.Generator(device=dev).manual_seed(seed)
    Qh = torch.randn(Hq, C, d, device=dev, generator=g).to(torch.bfloat16)
    Kh = torch.randn(Hq, C, d, device=dev, generator=g).to(torch.bfloat16)
    Vht = torch.randn(Hq, d, C, device=dev, generator=g).to(torch.bfloat16)
    return Qh, Kh, Vht


def check_rows(Qh, Kh, Vht, Oh, h, Lp, rows, atol=ATOL, rtol=RTOL):
    q = Qh[h, :Lp].double().cpu().numpy()
    k = Kh[h, :Lp].double().cpu().numpy()
    v = Vht[h, :, :Lp].double().cpu().numpy().T.copy()
    want = oracle.attention_rows(q, k, v, np.arange(Lp), rows)
    got = Oh[h, rows].double().cpu().numpy()
    err = np.abs(got - want)
    assert (err <= atol + rtol * np.abs(want)).all(), (h, float(err.max()))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("L,cut", [(196608, 77), (163840, 0)])
def test_long_compressed_attention_covers_every_row(gpu, L, cut):
    Hq, d = 8, 128
    s = binding.shape(L, Hq, Hq, d, 16, 0.005, "bf16")
    C = binding.capacity(L)
    Lp = L - cut
    Qh, Kh, Vht = rand_compressed(Hq, C, d, gpu, seed=L)
    Oh = torch.full_like(Qh, float("nan"))
    binding.attn_causal(s, Qh, Kh, Vht, torch.tensor([Lp], dtype=torch.int32, device=gpu), Oh)
    torch.cuda.synchronize()
    assert not torch.isnan(Oh[:, :Lp]).any(), "a query row below L' was never written"
    assert torch.isnan(Oh[:, Lp:]).all(), "a row at or past L' was written"
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, Lp - 257, Lp - 256, Lp - 1],
                                     rng.integers(0, Lp, size=9)]))
    for h in (0, Hq - 1):
        check_rows(Qh, Kh, Vht, Oh, h, Lp, rows)


@pytest.mark.timeout(300)
def test_varlen_mixing_four_and_eight_heads_in_flight(gpu):
    Hq, d = 8, 128
    lens = [163840, 4096, 1000]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    caps = [binding.capacity(L) for L in lens]
    off = np.concatenate([[0], np.cumsum(caps)]).astype(np.int64)
    s = binding.shape(cu[-1], Hq, Hq, d, 16, 0.005, "bf16")
    P = binding.varlen_capacity(cu)
    Qh, Kh, Vht = (t.reshape(-1) for t in rand_compressed(Hq, P, d, gpu, seed=11))
    Lps = [lens[0] - 300, lens[1], 999]
    Lp_dev = torch.tensor(Lps, dtype=torch.int32, device=gpu)
    Oh = torch.full_like(Qh, float("nan"))
    binding.attn_causal_varlen(s, cu, Qh, Kh, Vht, Lp_dev, Oh)
    for b, (L, C, Lp) in enumerate(zip(lens, caps, Lps)):
        reg = slice(Hq * d * int(off[b]), Hq * d * int(off[b + 1]))
        q, k, v = Qh[reg].view(Hq, C, d), Kh[reg].view(Hq, C, d), Vht[reg].view(Hq, d, C)
        O1 = torch.full((Hq, C, d), float("nan"), dtype=torch.bfloat16, device=gpu)
        binding.attn_causal(binding.shape(L, Hq, Hq, d, 16, 0.005, "bf16"), q, k, v, Lp_dev[b:b + 1], O1)
        Ov = Oh[reg].view(Hq, C, d)
        assert not torch.isnan(Ov[:, :Lp]).any(), b
        assert torch.isnan(Ov[:, Lp:]).all(), b
        assert torch.equal(Ov[:, :Lp], O1[:, :Lp]), b
    q = Qh[: Hq * d * caps[0]].view(Hq, caps[0], d)
    k = Kh[: Hq * d * caps[0]].view(Hq, caps[0], d)
    v = Vht[: Hq * d * caps[0]].view(Hq, d, caps[0])
    check_rows(q, k, v, Oh[: Hq * d * caps[0]].view(Hq, caps[0], d), 3, Lps[0],
               np.array([0, 4097, Lps[0] // 2, Lps[0] - 1]))


# Sequences of at most 16384 rows take the other map: each XCD walks the heaviest query blocks of
# all its heads first.  Both sides of that limit, with 1, 2 and 3 heads per XCD, bf16 and fp32
# (64-row blocks), must cover every row below L' once and leave the rest untouched.
@pytest.mark.timeout(300)
@pytest.mark.parametrize("L,Hq,d,dtype,cut", [(16384, 24, 128, "bf16", 5), (16385, 24, 128, "bf16", 0),
                                              (16384, 8, 64, "bf16", 0), (16384, 16, 128, "bf16", 1),
                                              (16384, 8, 64, "f32", 3), (16385, 8, 64, "f32", 0)])
def test_all_heads_order_covers_every_row(gpu, L, Hq, d, dtype, cut):
    s = binding.shape(L, Hq, Hq, d, 16, 0.005, dtype)
    C = binding.capacity(L)
    Lp = L - cut
    Qh, Kh, Vht = rand_compressed(Hq, C, d, gpu, seed=L + Hq)
    if dtype == "f32":
        Qh, Kh, Vht = Qh.float(), Kh.float(), Vht.float()
    Oh = torch.full_like(Qh, float("nan"))
    binding.attn_causal(s, Qh, Kh, Vht, torch.tensor([Lp], dtype=torch.int32, device=gpu), Oh)
    torch.cuda.synchronize()
    assert not torch.isnan(Oh[:, :Lp]).any(), "a query row below L' was never written"
    assert torch.isnan(Oh[:, Lp:]).all(), "a row at or past L' was written"
    rng = np.random.default_rng(L + Hq)
    rows = np.unique(np.concatenate([[0, 63, 64, 127, 128, Lp - 129, Lp - 128, Lp - 1],
                                     rng.integers(0, Lp, size=6)]))
    tol = (ATOL, RTOL) if dtype == "bf16" else (1e-4, 1e-4)
    for h in (0, 9 % Hq, Hq - 1):
        check_rows(Qh, Kh, Vht, Oh, h, Lp, rows, *tol)


@pytest.mark.timeout(300)
def test_varlen_mixing_all_heads_and_one_head_per_xcd(gpu):
    Hq, d = 16, 128
    lens = [20000, 16384, 3001]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    caps = [binding.capacity(L) for L in lens]
    off = np.concatenate([[0], np.cumsum(caps)]).astype(np.int64)
    s = binding.shape(cu[-1], Hq, Hq, d, 16, 0.005, "bf16")
    P = binding.varlen_capacity(cu)
    Qh, Kh, Vht = (t.reshape(-1) for t in rand_compressed(Hq, P, d, gpu, seed=12))
    Lps = [lens[0] - 17, lens[1] - 2, 2900]
    Lp_dev = torch.tensor(Lps, dtype=torch.int32, device=gpu)
    Oh = torch.full_like(Qh, float("nan"))
    binding.attn_causal_varlen(s, cu, Qh, Kh, Vht, Lp_dev, Oh)
    for b, (L, C, Lp) in enumerate(zip(lens, caps, Lps)):
        reg = slice(Hq * d * int(off[b]), Hq * d * int(off[b + 1]))
        q, k, v = Qh[reg].view(Hq, C, d), Kh[reg].view(Hq, C, d), Vht[reg].view(Hq, d, C)
        O1 = torch.full((Hq, C, d), float("nan"), dtype=torch.bfloat16, device=gpu)
        binding.attn_causal(binding.shape(L, Hq, Hq, d, 16, 0.005, "bf16"), q, k, v, Lp_dev[b:b + 1], O1)
        Ov = Oh[reg].view(Hq, C, d)
        assert not torch.isnan(Ov[:, :Lp]).any(), b
        assert torch.isnan(Ov[:, Lp:]).all(), b
        assert torch.equal(Ov[:, :Lp], O1[:, :Lp]), b
