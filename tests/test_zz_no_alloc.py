"""The allocation-free entry point (sparse_attn_forward_noalloc) against
sparse_attn_forward on the same plan and inputs, through the C ABI: the same
kernels on the library's per-device scratch array instead of a caller
workspace, so the outputs must be bit-identical.  Several calls in a row on
the one array, each later one smaller, check that nothing left there by an
earlier call leaks into a later one."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_sparse_video_fp32_amd import binding, inputs

pytestmark = pytest.mark.gpu

CASES = [
    # (B, N, H, D, plan kwargs), each smaller than the one before
    (1, 4096, 8, 128, dict(tau=1.0, reweight=True)),
    (1, 1000, 2, 64, dict(topk_ratio=0.2, prefix_len=70)),
    (2, 700, 2, 128, dict(tau=0.5, prefix_len=30, reblock=True, int8_qk=True)),
]


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def test_noalloc_matches_forward_on_consecutive_calls():
    dev = _dev()
    for i, (B, N, H, D, kw) in enumerate(CASES):
        q, k, v = inputs.clustered_soft(B, N, H, D, seed=60 + i)
        tq, tk, tv = (inputs.to_torch_bf16(x, dev) for x in (q, k, v))
        plan = binding.SparseAttnPlan(B, N, H, D, **kw)
        assert plan.workspace_bytes <= binding.SA_NOALLOC_SCRATCH_BYTES
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
        ref = plan.forward(tq, tk, tv, ws=ws)
        got = torch.full_like(tq, float("nan"))
        plan.forward_noalloc(tq, tk, tv, out=got)
        torch.cuda.synchronize()
        print(f"  call {i}: B={B} N={N} H={H} D={D} {kw}: workspace {plan.workspace_bytes} bytes", flush=True)
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"call {i} differs from sparse_attn_forward"


def test_noalloc_refuses_plans_beyond_the_scratch():
    dev = _dev()
    plan = binding.SparseAttnPlan(1, 131072, 8, 128, tau=1.0)
    assert plan.workspace_bytes > binding.SA_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((1, 64, 1, 64), dtype=torch.bfloat16, device=dev)  # never reached
    lib = binding.load_library()
    rc = lib.sparse_attn_forward_noalloc(plan._h, x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(), None)
    assert rc == -4  # SA_EWORKSPACE, before any launch
    assert "allocation-free scratch" in lib.sparse_attn_last_error().decode()
