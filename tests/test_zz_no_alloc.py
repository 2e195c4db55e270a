"""The allocation-free layer (tsa_layer_noalloc) against tsa_layer with a caller workspace.

Both run the same kernels, so Y and {k, L'} must be bitwise equal.  The calls run one after another
on one stream, each smaller than the one before it, so every call finds the scratch holding the
previous call's intermediates: a stale histogram, count or score left there would show up as a
difference.  The first shape is longer than the one-workgroup selection limit (its multi-block radix
histograms live in the scratch and must be cleared on every call)."""

import pytest
import torch

from token_sparse_attention_amd import binding
from token_sparse_attention_amd.configs import Workload
from token_sparse_attention_amd.inputs import make_layer

pytestmark = pytest.mark.gpu

SHAPES = [
    Workload("noalloc_multiblock", L=40000, Hq=4, Hkv=1, d=128, q=16, tau=0.3, dtype="bf16",
             salient_frac=0.01, shared_frac=0.5, sink=16, seed=81),
    Workload("noalloc_gqa", L=3000, Hq=8, Hkv=2, d=128, q=16, tau=0.2, dtype="bf16",
             salient_frac=0.02, shared_frac=0.5, seed=82),
    Workload("noalloc_d64", L=1000, Hq=4, Hkv=4, d=64, q=8, tau=0.05, dtype="bf16",
             salient_frac=0.03, shared_frac=1.0, seed=83),
    Workload("noalloc_f32", L=700, Hq=2, Hkv=1, d=64, q=16, tau=0.1, dtype="f32",
             salient_frac=0.03, shared_frac=1.0, seed=84),
]


@pytest.mark.timeout(300)
def test_noalloc_layer_equals_layer(gpu):
    for cfg in SHAPES:
        print(f"\n[noalloc] {cfg.name}: L={cfg.L} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d} {cfg.dtype}", flush=True)
        s = binding.shape_of(cfg)
        assert binding.layer_workspace_bytes(s) <= binding.NOALLOC_SCRATCH_BYTES
        inp = make_layer(cfg)
        Q, K, V, X = (inp[n].to(gpu) for n in ("Q", "K", "V", "X"))
        ws = binding.workspace(binding.layer_workspace_bytes(s), gpu)
        kl_ref = torch.zeros(2, dtype=torch.int32, device=gpu)
        Y_ref = torch.full_like(X, float("nan"))
        binding.layer(s, Q, K, V, X, Y_ref, kl_ref, ws)
        del ws
        kl = torch.full((2,), -7, dtype=torch.int32, device=gpu)
        Y = torch.full_like(X, float("nan"))
        binding.layer_noalloc(s, Q, K, V, X, Y, kl)
        torch.cuda.synchronize()
        assert kl.tolist() == kl_ref.tolist(), cfg.name
        assert 0 < kl_ref.tolist()[1] < cfg.L, cfg.name
        assert torch.equal(Y, Y_ref), cfg.name
        # in place (Y aliases X), and without a residual
        Xc = X.clone()
        binding.layer_noalloc(s, Q, K, V, Xc, Xc, None)
        assert torch.equal(Xc, Y_ref), cfg.name
        Y0_ref = torch.empty_like(X)
        ws = binding.workspace(binding.layer_workspace_bytes(s), gpu)
        binding.layer(s, Q, K, V, None, Y0_ref, None, ws)
        Y0 = torch.empty_like(X)
        binding.layer_noalloc(s, Q, K, V, None, Y0, None)
        assert torch.equal(Y0, Y0_ref), cfg.name
        del ws


@pytest.mark.timeout(120)
def test_noalloc_refuses_oversized_problems_before_launch(gpu):
    big = binding.shape(131072, 32, 8, 128, 16, 0.005, "bf16")
    assert binding.layer_workspace_bytes(big) > binding.NOALLOC_SCRATCH_BYTES
    Q = torch.zeros(16, dtype=torch.bfloat16, device=gpu)        # never read: the call is refused first
    with pytest.raises(binding.TsaError) as e:
        binding.layer_noalloc(big, _Raw(Q), _Raw(Q), _Raw(Q), None, _Raw(Q))
    assert e.value.status == 8


class _Raw:
    """A raw device address (not a tensor), so only the library's own size rule applies."""

    def __init__(self, t):
        self.t = t

    def data_ptr(self):
        return self.t.data_ptr()
