"""Guard bands around every buffer the library touches.

Each input, output, device scalar and workspace is a view into a larger device allocation whose
margins (4 KiB on each side) hold seeded random bytes.  After every entry point (each stage call,
the layer and its fixed-ratio and block-sparse variants, the varlen batch, the stage-4b varlen
attention and the dense baselines) the margins must be unchanged: no kernel writes outside the
buffers it was given, whatever the tile raggedness.  Shapes are ragged (no length is a multiple of a
tile), one case keeps almost nothing (tau near 1), and a varlen batch mixes samples on both sides of
the one-workgroup selection limit.
"""

import math

import pytest
import torch

from token_sparse_attention_amd import binding
from token_sparse_attention_amd.configs import Workload
from token_sparse_attention_amd.inputs import make_batch, make_layer

pytestmark = pytest.mark.gpu

G = 4096   # guard bytes on each side: a multiple of the 256-byte workspace alignment

CASES = {
    "bf16_gqa_L1000": Workload("guard_gqa", L=1000, Hq=4, Hkv=2, d=128, q=5, tau=0.05, dtype="bf16",
                               salient_frac=0.02, shared_frac=0.5, seed=71),
    "bf16_d64_L777": Workload("guard_d64", L=777, Hq=2, Hkv=1, d=64, q=16, tau=0.01, dtype="bf16",
                              salient_frac=0.03, shared_frac=0.5, sink=8, seed=72),
    "f32_L300": Workload("guard_f32", L=300, Hq=2, Hkv=2, d=128, q=3, tau=0.02, dtype="f32",
                         salient_frac=0.05, shared_frac=1.0, seed=73),
    "bf16_keep_few_L530": Workload("guard_few", L=530, Hq=8, Hkv=2, d=128, q=4, tau=0.99999, dtype="bf16",
                                   salient_frac=0.02, shared_frac=0.5, seed=74),
}


class Arena:
    """Device buffers with guarded margins."""

    def __init__(self, dev, seed):
        self.dev, self.bufs = dev, []
        self.gen = torch.Generator().manual_seed(seed)

    def alloc(self, shape, dtype):
        n = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
        pat = torch.randint(0, 256, (n + 2 * G,), generator=self.gen, dtype=torch.uint8)
        raw = pat.to(self.dev)
        self.bufs.append((raw, n, pat[:G].clone(), pat[G + n:].clone()))
        return raw[G:G + n].view(dtype).view(shape)

    def copy_of(self, t):
        v = self.alloc(tuple(t.shape), t.dtype)
        v.copy_(t.to(self.dev))
        return v

    def check(self, what):
        torch.cuda.synchronize()
        for i, (raw, n, lo, hi) in enumerate(self.bufs):
            assert torch.equal(raw[:G].cpu(), lo), f"{what}: bytes written before buffer {i}"
            assert torch.equal(raw[G + n:].cpu(), hi), f"{what}: bytes written after buffer {i}"


@pytest.mark.parametrize("name", list(CASES))
def test_no_write_outside_buffers(gpu, name):
    cfg = CASES[name]
    L, Hq, Hkv, d = cfg.L, cfg.Hq, cfg.Hkv, cfg.d
    A = Arena(gpu, cfg.seed)
    inp = make_layer(cfg)
    Q, K, V, X = (A.copy_of(inp[n]) for n in ("Q", "K", "V", "X"))
    dt = Q.dtype
    s = binding.shape_of(cfg)
    C = binding.capacity(L)
    i32 = torch.int32

    # stages
    ws = A.alloc((binding.stage_workspace_bytes(s),), torch.uint8)
    s_h, s_l = A.alloc((Hq, L), torch.float32), A.alloc((L,), torch.float32)
    binding.score(s, Q, K, s_h, s_l, ws)
    A.check("score")
    k_dev, Lp_dev = A.alloc((1,), i32), A.alloc((1,), i32)
    binding.budget(s, s_l, k_dev, Lp_dev, ws)
    A.check("budget")
    Lp = int(Lp_dev.item())
    idx, inv = A.alloc((Hq, L), i32), A.alloc((Hq, L), i32)
    binding.select(s, s_h, Lp_dev, idx, inv, ws)
    A.check("select")
    Qh, Kh, Vht = A.alloc((Hq, C, d), dt), A.alloc((Hq, C, d), dt), A.alloc((Hq, d, C), dt)
    binding.gather(s, Q, K, V, idx, Lp_dev, Qh, Kh, Vht)
    A.check("gather")
    Oh = A.alloc((Hq, C, d), dt)
    binding.attn_causal(s, Qh, Kh, Vht, Lp_dev, Oh)
    A.check("attn_causal")
    Y = A.alloc((L, Hq, d), dt)
    binding.scatter_residual(s, Oh, idx, inv, Lp_dev, X, Y)
    A.check("scatter_residual")
    k2, Lp2 = A.alloc((1,), i32), A.alloc((1,), i32)
    binding.budget_ratio(s, 0.3, k2, Lp2)
    A.check("budget_ratio")

    # the layer and its variants
    lws = A.alloc((binding.layer_workspace_bytes(s),), torch.uint8)
    kl = A.alloc((2,), i32)
    Y1 = A.alloc((L, Hq, d), dt)
    binding.layer(s, Q, K, V, X, Y1, kl, lws)
    A.check("layer")
    assert kl.tolist() == [int(k_dev.item()), Lp]
    binding.layer(s, Q, K, V, None, Y1, kl, lws)
    A.check("layer without X")
    Y2 = A.alloc((L, Hq, d), dt)
    binding.layer_ratio(s, 0.5, Q, K, V, X, Y2, kl, lws)
    A.check("layer_ratio")
    bws = A.alloc((binding.layer_block_sparse_workspace_bytes(s),), torch.uint8)
    Y3 = A.alloc((L, Hq, d), dt)
    binding.layer_block_sparse(s, 0.5, Q, K, V, X, Y3, kl, bws)
    A.check("layer_block_sparse")
    NB = binding.block_count(L)
    blist, bcnt = A.alloc((Hq, NB, NB), torch.uint16), A.alloc((Hq, NB), i32)
    sws = A.alloc((binding.block_select_workspace_bytes(s),), torch.uint8)
    binding.block_select(s, 0.5, Qh, Kh, Lp_dev, blist, bcnt, sws)
    A.check("block_select")
    Oh2 = A.alloc((Hq, C, d), dt)
    binding.attn_block_sparse(s, Qh, Kh, Vht, Lp_dev, blist, bcnt, Oh2)
    A.check("attn_block_sparse")
    dws = A.alloc((binding.dense_workspace_bytes(s),), torch.uint8)
    Y4 = A.alloc((L, Hq, d), dt)
    binding.dense_attn_causal(s, Q, K, V, X, Y4, dws)
    A.check("dense_attn_causal")


def test_varlen_no_write_outside_buffers(gpu):
    cfg = Workload("guard_varlen", L=1, Hq=8, Hkv=2, d=128, q=4, tau=0.05, dtype="bf16",
                   salient_frac=0.05, shared_frac=0.5, seed=75)
    lengths = [700, 37, 33001, 1500]        # 33001: past the one-workgroup selection limit
    b = make_batch(cfg, lengths)
    cu = [int(v) for v in b["cu_seqlens"]]
    A = Arena(gpu, 75)
    Q, K, V, X = (A.copy_of(b[n]) for n in ("Q", "K", "V", "X"))
    s = binding.shape(cu[-1], cfg.Hq, cfg.Hkv, cfg.d, cfg.q, cfg.tau, cfg.dtype)
    B = len(lengths)
    ws = A.alloc((binding.layer_varlen_workspace_bytes(s, cu),), torch.uint8)
    kl = A.alloc((B, 2), torch.int32)
    Y = A.alloc(tuple(X.shape), X.dtype)
    binding.layer_varlen(s, cu, Q, K, V, X, Y, kl, ws)
    A.check("layer_varlen")
    dws = A.alloc((binding.dense_varlen_workspace_bytes(s, cu),), torch.uint8)
    Yd = A.alloc(tuple(X.shape), X.dtype)
    binding.dense_attn_causal_varlen(s, cu, Q, K, V, X, Yd, dws)
    A.check("dense_attn_causal_varlen")
    # stage 4b over the batch, on compressed tensors laid out per sample at the capacity offsets
    P = binding.varlen_capacity(cu)
    Hq, d = cfg.Hq, cfg.d
    Qh, Kh, Oh = (A.alloc((Hq * P * d,), Q.dtype) for _ in range(3))
    Vht = A.alloc((Hq * P * d,), Q.dtype)
    for t in (Qh, Kh, Vht):
        t.copy_(torch.randn(t.shape, device=gpu).to(t.dtype))
    lp = A.copy_of(torch.tensor([max(1, n // 3) for n in lengths], dtype=torch.int32))
    binding.attn_causal_varlen(s, cu, Qh, Kh, Vht, lp, Oh)
    A.check("attn_causal_varlen")
