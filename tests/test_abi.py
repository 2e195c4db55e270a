"""Host-side checks of the C ABI: the library loads, exports every function include/tsa.h declares,
and rejects bad arguments before launching anything (so these run without a GPU)."""

import ctypes
import math
import os
import re

import pytest

from token_sparse_attention_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tsa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(tsa_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_binding_surface():
    assert set(declared_functions()) == set(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def good():
    return binding.shape(4096, 32, 8, 128, 16, 0.005, "bf16")


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 7, 3), ("tau", -0.1, 1), ("tau", 1.0, 1), ("tau", math.nan, 1),
    ("L", 0, 2), ("L", 1 << 31, 2), ("L", (1 << 24) + 1, 2), ("Hq", 0, 2), ("Hkv", 3, 2), ("Hkv", 64, 2), ("q", 0, 2),
    ("q", 4097, 2), ("q", 2000, 2), ("d", 96, 7), ("d", 256, 7),
])
def test_check_args_rejects(field, value, status):
    s = good()
    setattr(s, field, value)
    assert binding.check_args(s) == status


def test_check_args_length_limit():
    s = good()
    s.L = 1 << 24                         # the largest length the 32-bit buffer offsets allow
    assert binding.check_args(s) == 0


def test_check_args_accepts_the_workloads():
    from token_sparse_attention_amd.configs import WORKLOADS
    for cfg in WORKLOADS.values():
        assert binding.check_args(binding.shape_of(cfg)) == 0
    s = good()
    s.q = s.L = 7
    assert binding.check_args(s) == 0


def test_status_strings():
    L = binding.lib()
    for code in range(9):
        assert L.tsa_status_string(code).decode() == binding._STATUS[code]
    assert L.tsa_status_string(99).decode() == "unknown status"


def test_capacity_and_workspace_sizes():
    assert [binding.capacity(n) for n in (1, 256, 257, 1000)] == [256, 256, 512, 1024]
    small, big = good(), good()
    big.L = 131072
    for fn in (binding.stage_workspace_bytes, binding.layer_workspace_bytes, binding.dense_workspace_bytes):
        assert 0 < fn(small) < fn(big)
        assert fn(small) % 256 == 0
    bad = good()
    bad.d = 96
    assert binding.layer_workspace_bytes(bad) == 0
    # the bf16 layer reads its query and key rows through the selection and writes Y from the
    # attention, so its workspace holds V_hat^T at capacity but no Q_hat, K_hat or O_hat; the fp32
    # layer and the block-sparse layer materialise all four
    s = good()
    comp = 32 * binding.capacity(4096) * 128 * 2
    assert comp <= binding.layer_workspace_bytes(s) < 2 * comp
    assert binding.layer_block_sparse_workspace_bytes(s) >= 4 * comp
    f = good()
    f.dtype = binding.F32
    assert binding.layer_workspace_bytes(f) >= 4 * 2 * comp


class FakePtr:
    """Stands in for a tensor: only its address is used, and nothing is launched on these paths."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def test_entry_points_validate_before_launch():
    s = good()
    p = FakePtr(1 << 20)           # aligned, never dereferenced: every call below fails validation
    mis = FakePtr((1 << 20) + 2)
    with pytest.raises(binding.TsaError) as e:
        binding.score(s, None, p, p, ws=None, stream=0)
    assert e.value.status == 1
    with pytest.raises(binding.TsaError) as e:
        binding.score(s, mis, p, p, stream=0)
    assert e.value.status == 4
    with pytest.raises(binding.TsaError) as e:           # missing workspace
        binding.score(s, p, p, p, stream=0)
    assert e.value.status == 5
    with pytest.raises(binding.TsaError) as e:
        binding.layer(s, p, p, p, None, None, stream=0)
    assert e.value.status == 1
    bad = good()
    bad.tau = 2.0
    with pytest.raises(binding.TsaError) as e:
        binding.attn_causal(bad, p, p, p, p, p, stream=0)
    assert e.value.status == 1
    with pytest.raises(binding.TsaError) as e:
        binding.select(s, p, None, p, stream=0)
    assert e.value.status == 1
    with pytest.raises(binding.TsaError) as e:
        binding.scatter_residual(s, p, None, None, p, None, p, stream=0)    # no inv and no idx
    assert e.value.status == 1
    for sp in (-0.25, 1.5, float("nan")):                 # fixed ratio outside [0, 1]
        with pytest.raises(binding.TsaError) as e:
            binding.budget_ratio(s, sp, p, p, stream=0)
        assert e.value.status == 1
        with pytest.raises(binding.TsaError) as e:
            binding.layer_ratio(s, sp, p, p, p, None, p, stream=0)
        assert e.value.status == 1
    with pytest.raises(binding.TsaError) as e:
        binding.budget_ratio(s, 0.3, mis, p, stream=0)
    assert e.value.status == 4
    with pytest.raises(binding.TsaError) as e:           # layer_ratio still needs its workspace
        binding.layer_ratio(s, 0.3, p, p, p, None, p, stream=0)
    assert e.value.status == 5


def test_select_sparse_layers_rule():
    from token_sparse_attention_amd.configs import WORKLOADS
    from token_sparse_attention_amd.inputs import chain_drift_values
    from token_sparse_attention_amd.runtime import select_sparse_layers
    cfg = WORKLOADS[5]
    assert select_sparse_layers(chain_drift_values(cfg)) == list(cfg.sparse_layers)
    assert select_sparse_layers([0.3, 0.1, 0.2, 0.1]) == [2, 4]


def test_every_kernel_has_its_host_launch_stub():
    """A kernel whose host-side stub the compiler dropped would fail to load at run time; catch it
    on the CPU: the library may not leave any __device_stub__ symbol undefined."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", binding._LIB_PATH], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    assert "__device_stub__" not in out.stdout


def test_varlen_capacity_and_validation():
    """Host-side rules of the varlen batch entry points (nothing is launched on these paths)."""
    assert binding.varlen_capacity([0, 1, 300, 1000]) == 256 + 512 + 768
    assert binding.varlen_capacity([0, 4096]) == 4096
    assert binding.varlen_capacity([0, 5, 5]) == -1 and binding.varlen_capacity([1, 5]) == -1
    s = binding.shape(1000, 4, 2, 128, 5, 0.05, "bf16")
    cu = [0, 37, 700, 1000]
    comp = 4 * 128 * 2 * binding.varlen_capacity(cu)        # one compressed tensor of the batch
    assert comp <= binding.layer_varlen_workspace_bytes(s, cu) < 2 * comp
    assert binding.dense_varlen_workspace_bytes(s, cu) >= 2 * 128 * 2 * binding.varlen_capacity(cu)
    for bad, status in (([0, 37, 700, 999], 1), ([0, 700, 37, 1000], 1), ([1, 37, 700, 1000], 1),
                        ([0, 3, 700, 1000], 2)):              # last: a sample shorter than q = 5
        assert binding.layer_varlen_workspace_bytes(s, bad) == 0
        p = FakePtr(1 << 20)
        with pytest.raises(binding.TsaError) as e:
            binding.layer_varlen(s, bad, p, p, p, None, p, stream=0)
        assert e.value.status == status, bad
        with pytest.raises(binding.TsaError) as e:
            binding.attn_causal_varlen(s, bad, p, p, p, p, p, stream=0)
        assert e.value.status == status, bad
    p = FakePtr(1 << 20)
    with pytest.raises(binding.TsaError) as e:                # valid batch, no workspace
        binding.layer_varlen(s, cu, p, p, p, None, p, stream=0)
    assert e.value.status == 5


def test_block_sparse_host_rules():
    assert binding.block_count(1) == 2 and binding.block_count(131072) == 1024
    s = good()
    assert binding.block_select_workspace_bytes(s) >= 2 * 32 * binding.block_count(4096) * 128 * 4
    assert binding.layer_block_sparse_workspace_bytes(s) > binding.layer_workspace_bytes(s)
    p = FakePtr(1 << 20)
    for g in (-0.5, float("nan")):
        with pytest.raises(binding.TsaError) as e:
            binding.block_select(s, g, p, p, p, p, p, stream=0)
        assert e.value.status == 1
        with pytest.raises(binding.TsaError) as e:
            binding.layer_block_sparse(s, g, p, p, p, None, p, stream=0)
        assert e.value.status == 1
    big = binding.shape(524289, 8, 8, 128, 16, 0.005, "bf16")       # more than 4096 key blocks
    with pytest.raises(binding.TsaError) as e:
        binding.attn_block_sparse(big, p, p, p, p, p, p, p, stream=0)
    assert e.value.status == 7
    with pytest.raises(binding.TsaError) as e:                       # no workspace
        binding.block_select(s, 0.9, p, p, p, p, p, stream=0)
    assert e.value.status == 5


def test_binding_validates_tensors_before_the_library():
    """The binding refuses a tensor that would make a kernel read or write outside its buffer (wrong
    element type, too few elements, a non-contiguous view, host memory) before libtsa sees its
    address; these raise on the CPU, so nothing is launched."""
    import torch
    s = binding.shape(300, 4, 2, 64, 8, 0.05, "bf16")
    L, Hq, Hkv, d = 300, 4, 2, 64
    bf = lambda *sh: torch.zeros(*sh, dtype=torch.bfloat16)
    Q, K, V, X, Y = bf(L, Hq, d), bf(L, Hkv, d), bf(L, Hkv, d), bf(L, Hq, d), bf(L, Hq, d)
    kl = torch.zeros(2, dtype=torch.int32)
    ws = torch.zeros(256, dtype=torch.uint8)

    def status(fn, *a):
        with pytest.raises(binding.TsaError) as e:
            fn(*a)
        return e.value.status, str(e.value)

    st, msg = status(binding.layer, s, Q.float(), K, V, X, Y, kl, ws)            # fp32 under a bf16 shape
    assert st == 3 and "Q" in msg
    st, msg = status(binding.layer, s, Q, K[:-1], V, X, Y, kl, ws)               # one row short
    assert st == 1 and "K holds" in msg
    st, msg = status(binding.layer, s, Q, K, V, X.transpose(0, 1), Y, kl, ws)    # a strided view
    assert st == 1 and "contiguous" in msg
    st, msg = status(binding.layer, s, Q, K, V, X, Y, kl[:1], ws)                # {k, L'} needs two words
    assert st == 1 and "kLp_dev" in msg
    st, msg = status(binding.layer, s, Q, K, V, X, Y, kl, ws)                    # all well formed, on the host
    assert st == 1 and "not a device tensor" in msg
    s_h = torch.zeros(Hq, L)
    st, msg = status(binding.select, s, s_h, kl[1:2], torch.zeros(Hq, L, dtype=torch.int64), None, ws)
    assert st == 3 and "idx" in msg
    C = binding.capacity(L)
    Qh, Kh, Oh = bf(Hq, C, d), bf(Hq, C, d), bf(Hq, C, d)
    st, msg = status(binding.attn_causal, s, Qh, Kh, bf(Hq, d, C - 1), kl[1:2], Oh)   # V_hat^T below capacity
    assert st == 1 and "Vht" in msg
    nb = binding.block_count(L)
    st, msg = status(binding.attn_block_sparse, s, Qh, Kh, bf(Hq, d, C), kl[1:2],
                     torch.zeros(Hq, nb, nb, dtype=torch.int32), torch.zeros(Hq, nb, dtype=torch.int32), Oh)
    assert st == 3 and "blist" in msg
    st, msg = status(binding.layer_varlen, s, [0, 100, 300], Q, K, V, X, Y, kl, ws)    # {k_b, L'_b} per sample
    assert st == 1 and "kLp_dev" in msg


def test_noalloc_entry_point_host_rules():
    """The allocation-free layer validates like tsa_layer and refuses a problem whose intermediates
    exceed its fixed scratch, both before any GPU call (these run without a GPU)."""
    import re
    src = open(HEADER).read()
    m = re.search(r"#define TSA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.NOALLOC_SCRATCH_BYTES
    p = FakePtr(1 << 20)
    s = good()
    assert binding.layer_workspace_bytes(s) <= binding.NOALLOC_SCRATCH_BYTES
    with pytest.raises(binding.TsaError) as e:
        binding.layer_noalloc(s, None, p, p, None, p, stream=0)
    assert e.value.status == 1
    with pytest.raises(binding.TsaError) as e:
        binding.layer_noalloc(s, FakePtr((1 << 20) + 4), p, p, None, p, stream=0)
    assert e.value.status == 4
    big = binding.shape(131072, 32, 8, 128, 16, 0.005, "bf16")
    assert binding.layer_workspace_bytes(big) > binding.NOALLOC_SCRATCH_BYTES
    with pytest.raises(binding.TsaError) as e:
        binding.layer_noalloc(big, p, p, p, None, p, stream=0)
    assert e.value.status == 8
