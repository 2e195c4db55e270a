"""The fused layer captured in a HIP graph.  The library allocates nothing, clears its workspace
with a kernel (no memset nodes) and never synchronises with the host, so a call can be captured
once and replayed.  Every replay must equal the eager result bit for bit, with other eager work
and synchronisations between the replays."""

import numpy as np
import pytest
import torch

from token_sparse_attention_amd import binding
from token_sparse_attention_amd.configs import WORKLOADS, Workload, scaled
from token_sparse_attention_amd.inputs import make_batch, make_layer

pytestmark = pytest.mark.gpu


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up outside the capture, as torch requires
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("cfg", [scaled(WORKLOADS[2], 2048, Hq=8, Hkv=2, seed=61),
                                 # past 32768 rows: the multi-block radix budget and selection, whose
                                 # histograms the captured call clears with a kernel on every replay
                                 scaled(WORKLOADS[2], 40001, Hq=4, Hkv=2, seed=64),
                                 Workload("graph_f32", L=300, Hq=2, Hkv=2, d=128, q=3, tau=0.02, dtype="f32",
                                          salient_frac=0.05, shared_frac=1.0, seed=62)],
                         ids=["bf16_L2048", "bf16_L40001_multiblock", "f32_L300"])
def test_layer_replays_bitwise(gpu, cfg):
    inp = make_layer(cfg)
    Q, K, V, X = (inp[n].to(gpu) for n in ("Q", "K", "V", "X"))
    s = binding.shape_of(cfg)
    ws = binding.workspace(binding.layer_workspace_bytes(s), gpu)
    kl_e = torch.zeros(2, dtype=torch.int32, device=gpu)
    Ye = torch.empty_like(X)
    binding.layer(s, Q, K, V, X, Ye, kl_e, ws)
    torch.cuda.synchronize()

    Yg = torch.empty_like(X)
    kl_g = torch.zeros(2, dtype=torch.int32, device=gpu)
    g = capture(lambda: binding.layer(s, Q, K, V, X, Yg, kl_g, ws))
    other_ws = binding.workspace(binding.layer_workspace_bytes(s), gpu)
    for i in range(4):
        Yg.fill_(float(i + 3))
        kl_g.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Yg, Ye), i
        assert kl_g.tolist() == kl_e.tolist(), i
        # unrelated eager work between replays, on the same inputs and another workspace
        Y2 = torch.empty_like(X)
        binding.layer(s, Q, K, V, X, Y2, None, other_ws)
        torch.cuda.synchronize()
        assert torch.equal(Y2, Ye), i


@pytest.mark.parametrize("lengths", [[700, 37, 1500, 256], [40001, 300, 33000]],
                         ids=["short", "multiblock_and_one_workgroup"])
def test_varlen_layer_replays_bitwise(gpu, lengths):
    """Samples past 32768 rows take the multi-block radix kernels (histograms cleared by a kernel
    inside the captured call), the others the one-workgroup kernels."""
    cfg = Workload("graph_varlen", L=1, Hq=8, Hkv=2, d=128, q=4, tau=0.05, dtype="bf16",
                   salient_frac=0.05, shared_frac=0.5, seed=63)
    b = make_batch(cfg, lengths)
    cu = [int(v) for v in b["cu_seqlens"]]
    Q, K, V, X = (b[n].to(gpu) for n in ("Q", "K", "V", "X"))
    s = binding.shape(cu[-1], cfg.Hq, cfg.Hkv, cfg.d, cfg.q, cfg.tau, cfg.dtype)
    ws = binding.workspace(binding.layer_varlen_workspace_bytes(s, cu), gpu)
    kl_e = torch.zeros(len(cu) - 1, 2, dtype=torch.int32, device=gpu)
    Ye = torch.empty_like(X)
    binding.layer_varlen(s, cu, Q, K, V, X, Ye, kl_e, ws)
    torch.cuda.synchronize()
    Yg = torch.empty_like(X)
    kl_g = torch.zeros_like(kl_e)
    g = capture(lambda: binding.layer_varlen(s, cu, Q, K, V, X, Yg, kl_g, ws))
    for i in range(3):
        Yg.fill_(-float(i + 1))
        kl_g.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Yg, Ye), i
        assert np.array_equal(kl_g.cpu().numpy(), kl_e.cpu().numpy()), i
