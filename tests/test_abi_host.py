"""Host-side checks of the C-ABI library (no GPU needed, nothing launched):
the library loads, exports every function include/sparse_attn.h declares,
validates parameters with the documented error codes and sizes the
workspace as documented."""

import ctypes
import math
import os
import re

import pytest

from block_sparse_video_fp32_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

SA_EINVAL, SA_EUNSUPPORTED_SHAPE, SA_EALIGN, SA_EWORKSPACE = -1, -2, -5, -4


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(sparse_attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("sparse_attn_plan_create", "sparse_attn_forward", "sparse_attn_pool",
                 "sparse_attn_select", "sparse_attn_attend", "sparse_attn_workspace_layout"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.sparse_attn_abi_version() == 6
    # the binding's expected version is the header's
    assert f"#define SA_ABI_VERSION {binding.SA_ABI_VERSION}" in open(HEADER).read()


def _params(**kw):
    p = binding._Params()
    p.B, p.N, p.H, p.D = 1, 1024, 2, 64
    p.route, p.tau, p.prefix_len, p.flags = 0, 1.0, 0, 3
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _create(lib, p):
    h = ctypes.c_void_p()
    rc = lib.sparse_attn_plan_create(ctypes.byref(p), ctypes.byref(h))
    if rc == 0:
        lib.sparse_attn_plan_destroy(h)
    else:
        assert not h.value
    return rc


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(), 0),
        (dict(D=128), 0),
        (dict(D=96), SA_EUNSUPPORTED_SHAPE),
        (dict(D=256), SA_EUNSUPPORTED_SHAPE),
        (dict(N=0), SA_EINVAL),
        (dict(B=0), SA_EINVAL),
        (dict(H=-1), SA_EINVAL),
        (dict(N=131072), 0),
        (dict(N=131073), SA_EUNSUPPORTED_SHAPE),
        (dict(tau=float("nan")), SA_EINVAL),
        (dict(tau=float("inf")), 0),
        (dict(tau=float("-inf")), 0),
        (dict(route=1, topk_ratio=0.0), SA_EINVAL),
        (dict(route=1, topk_ratio=1.5), SA_EINVAL),
        (dict(route=1, topk_ratio=float("nan")), SA_EINVAL),
        (dict(route=1, topk_ratio=1.0), 0),
        (dict(route=2), SA_EINVAL),
        (dict(prefix_len=-1), SA_EINVAL),
        (dict(prefix_len=1025), SA_EINVAL),
        (dict(prefix_len=1024), 0),
        (dict(sm_scale=float("inf")), SA_EINVAL),
        (dict(flags=64), SA_EINVAL),
        (dict(in_stride_b=3 * 1024 * 128, in_stride_t=3 * 128, in_stride_h=64), 0),
        (dict(in_stride_b=1024 * 128, in_stride_t=130, in_stride_h=64), SA_EALIGN),
        (dict(in_stride_b=0, in_stride_t=128, in_stride_h=64), SA_EINVAL),
        (dict(out_stride_b=8, out_stride_t=-8, out_stride_h=8), SA_EINVAL),
    ],
)
def test_plan_validation(lib, kw, code):
    assert _create(lib, _params(**kw)) == code
    if code:
        assert lib.sparse_attn_last_error().decode() != ""
        assert lib.sparse_attn_strerror(code).decode() not in ("", "unknown error")


def test_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.sparse_attn_plan_create(None, ctypes.byref(h)) == SA_EINVAL
    p = _params()
    assert lib.sparse_attn_plan_create(ctypes.byref(p), None) == SA_EINVAL
    lay = binding._Layout()
    assert lib.sparse_attn_workspace_layout(None, ctypes.byref(lay)) == SA_EINVAL
    lib.sparse_attn_plan_destroy(None)


@pytest.mark.parametrize("int8_qk", [False, True])
def test_workspace_layout_matches_documented_sizes(int8_qk):
    plan = binding.SparseAttnPlan(2, 1000, 3, 128, tau=1.0, prefix_len=70, int8_qk=int8_qk)
    L = plan.layout
    nb = 16
    assert L["n_blocks"] == nb and L["n_blocks_padded"] == 64
    assert L["tail_rows"] == 1000 - 64 * 15 and L["prefix_blocks"] == 2 and L["dense"] == 0
    names = ("qbar", "kbar", "vbar", "k_packed", "v_packed", "kbar_packed", "vbar_packed", "counts", "lists",
             "anchor", "cbias", "k_int8", "kbase", "rb_gram", "rb_metric", "rb_units", "rb_munits", "rb_order",
             "rb_keys", "rb_qkv", "rb_out")
    offs = sorted((L[n], n) for n in names)
    sizes = dict(qbar=2 * 3 * nb * 128 * 4, kbar=2 * 3 * nb * 128 * 4, vbar=2 * 3 * nb * 128 * 4,
                 k_packed=2 * 3 * nb * 64 * 128 * 2, v_packed=2 * 3 * nb * 64 * 128 * 2,
                 kbar_packed=2 * 3 * 64 * 128 * 2, vbar_packed=2 * 3 * 64 * 128 * 2,
                 counts=2 * 3 * nb * 4, lists=2 * 3 * nb * nb * 4, anchor=2 * 3 * 128 * 4, cbias=2 * 3 * 64 * 4,
                 k_int8=2 * 3 * nb * 64 * 128 if int8_qk else 0,
                 kbase=2 * 3 * nb * (128 + 8) * 2 if int8_qk else 0,
                 rb_gram=0, rb_metric=0, rb_units=0, rb_munits=0, rb_order=0, rb_keys=0, rb_qkv=0, rb_out=0)
    for (o, n), (o2, _) in zip(offs, offs[1:] + [(L["total_bytes"], "end")]):
        assert o % 256 == 0
        assert o2 - o >= sizes[n]
    if not int8_qk:
        assert L["kbase"] == L["k_int8"]  # empty sections


@pytest.mark.parametrize("ratio,nb,k", [(0.1, 598, 60), (0.1, 640, 64), (0.2, 512, 103), (1.0, 17, 17), (1e-9, 100, 1)])
def test_topk_count(ratio, nb, k):
    plan = binding.SparseAttnPlan(1, nb * 64, 1, 64, topk_ratio=ratio)
    assert plan.layout["topk"] == k
    from oracle import sol_oracle as O  # independent definition on the oracle side
    assert O.topk_count(ratio, nb) == k


def test_dense_flag():
    assert binding.SparseAttnPlan(1, 128, 1, 64, tau=-math.inf).dense
    assert not binding.SparseAttnPlan(1, 128, 1, 64, tau=math.inf).dense


def test_call_validation_before_launch(lib):
    """Errors that need no device: NULL tensors, misalignment, short workspace."""
    plan = binding.SparseAttnPlan(1, 1024, 2, 64)
    h = plan._h
    need = plan.workspace_bytes
    fake = 1 << 20  # never dereferenced: validation fails first
    f = lib.sparse_attn_forward
    lib.sparse_attn_attend.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]
    assert f(h, None, fake, fake, fake, fake, need, None) == SA_EINVAL
    assert f(h, fake + 2, fake, fake, fake, fake, need, None) == SA_EALIGN
    assert f(h, fake, fake, fake, fake, fake + 16, need, None) == SA_EALIGN
    assert f(h, fake, fake, fake, fake, fake, need - 1, None) == SA_EWORKSPACE
    assert "plan needs" in lib.sparse_attn_last_error().decode()
    assert f(None, fake, fake, fake, fake, fake, need, None) == SA_EINVAL
    assert lib.sparse_attn_select(h, None, need, None) == SA_EINVAL
    assert lib.sparse_attn_pool(h, fake, fake, fake, fake, need - 256, None) == SA_EWORKSPACE
    assert lib.sparse_attn_attend(h, fake, None, fake, need, None) == SA_EINVAL
    assert lib.sparse_attn_attend(h, fake, fake, fake, need - 1, None) == SA_EWORKSPACE


def test_device_mismatch_names_required_and_detected_arch(lib, monkeypatch):
    """An architecture mismatch is refused before any launch with
    SA_EUNSUPPORTED_DEVICE and a message naming the required and the
    detected architecture (Star7 README, 环境与分发), forced here by the
    library's test hook, which never queries a device."""
    SA_EUNSUPPORTED_DEVICE = -3
    plan = binding.SparseAttnPlan(1, 1024, 2, 64)
    h, need, fake = plan._h, plan.workspace_bytes, 1 << 20  # never dereferenced
    lib.sparse_attn_attend.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]
    monkeypatch.setenv("SPARSE_ATTN_ARCH_OVERRIDE", "gfx942")
    calls = [
        ("forward", lambda: lib.sparse_attn_forward(h, fake, fake, fake, fake, fake, need, None)),
        ("pool", lambda: lib.sparse_attn_pool(h, fake, fake, fake, fake, need, None)),
        ("select", lambda: lib.sparse_attn_select(h, fake, need, None)),
        ("route", lambda: lib.sparse_attn_route(h, fake, fake, fake, fake, need, None)),
        ("attend", lambda: lib.sparse_attn_attend(h, fake, fake, fake, need, None)),
    ]
    for name, call in calls:
        assert call() == SA_EUNSUPPORTED_DEVICE, name
        msg = lib.sparse_attn_last_error().decode()
        assert "requires gfx950" in msg and "gfx942" in msg, msg
    assert "gfx950" in lib.sparse_attn_strerror(SA_EUNSUPPORTED_DEVICE).decode()
    # argument errors still come first (nothing reaches the device check)
    assert lib.sparse_attn_forward(h, fake, fake, fake, fake, fake, need - 1, None) == SA_EWORKSPACE
    # the binding surfaces it as an exception carrying the code and message
    with pytest.raises(binding.SparseAttnError) as e:
        binding._check(lib.sparse_attn_select(h, fake, need, None), "sparse_attn_select")
    assert e.value.code == SA_EUNSUPPORTED_DEVICE and "gfx942" in str(e.value)


def test_plan_log_line(tmp_path):
    """SPARSE_ATTN_LOG=1 prints one summary line per plan on stderr."""
    import subprocess
    import sys

    code = ("import sys; sys.path.insert(0, %r); from block_sparse_video_fp32_amd import binding; "
            "binding.SparseAttnPlan(1, 38247, 4, 128, topk_ratio=0.1, prefix_len=1024, reweight=True)" % ROOT)
    env = dict(os.environ, SPARSE_ATTN_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [x for x in r.stderr.splitlines() if x.startswith("sparse_attn: plan")]
    assert len(lines) == 1, r.stderr
    for part in ("N=38247", "n_b=598", "tail=39", "topk 0.1 (k=60)", "prefix 1024 rows (16 blocks",
                 "reweight 1", "workspace"):
        assert part in lines[0], (part, lines[0])
    env.pop("SPARSE_ATTN_LOG")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert "sparse_attn: plan" not in r.stderr


def test_binding_rejects_bad_tensors():
    import torch

    plan = binding.SparseAttnPlan(1, 128, 1, 64)
    x = torch.zeros(1, 128, 1, 64, dtype=torch.float32)
    with pytest.raises(TypeError):
        plan.forward(x, x, x)
    y = torch.zeros(1, 128, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        plan.forward(y, y, y)  # CPU tensors


def test_binding_checks_strides_against_the_plan():
    """A tensor whose strides differ from the plan's is refused before any
    call (the library would address it with the plan's strides): a fused-QKV
    view given to a contiguous plan, a non-contiguous output, a
    batch-expanded (stride 0) input.  Strides of size-1 dimensions are never
    used and are not compared."""
    import torch

    B, N, H, D = 2, 128, 3, 64
    plan = binding.SparseAttnPlan(B, N, H, D)
    assert plan.strides("in") == plan.strides("out") == (N * H * D, H * D, D)
    fused = torch.zeros(B, N, 3, H, D, dtype=torch.bfloat16)
    q = fused[:, :, 0]
    with pytest.raises(ValueError, match="input strides"):
        plan._check_io(ins=(q,))
    big = torch.zeros(B, N, 2, H, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="output strides"):
        plan._check_io(outs=(big[:, :, 1],))
    one = torch.zeros(1, N, H, D, dtype=torch.bfloat16).expand(B, N, H, D)
    assert one.stride(0) == 0
    with pytest.raises(ValueError, match="input strides"):
        plan._check_io(ins=(one,))
    # matching strides pass the stride check and stop at the device check
    c = torch.zeros(B, N, H, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        plan._check_io(ins=(c, c, c), outs=(c,))
    fplan = binding.SparseAttnPlan(B, N, H, D, in_strides=q.stride()[:3], out_strides=big[:, :, 1].stride()[:3])
    with pytest.raises(ValueError, match="HIP device"):
        fplan._check_io(ins=(q, fused[:, :, 1], fused[:, :, 2]), outs=(big[:, :, 1],))
    with pytest.raises(ValueError, match="input strides"):
        fplan._check_io(ins=(c,))
    # B = 1: the batch stride is never used
    p1 = binding.SparseAttnPlan(1, N, H, D)
    odd = torch.zeros(1, N, 2, H, D, dtype=torch.bfloat16)[:, :, 0]
    with pytest.raises(ValueError, match="input strides"):  # t and h strides still differ
        p1._check_io(ins=(odd,))
    with pytest.raises(ValueError, match="HIP device"):
        p1._check_io(ins=(torch.zeros(2, N, H, D, dtype=torch.bfloat16)[1:],))


def test_plan_error_raises():
    with pytest.raises(binding.SparseAttnError) as e:
        binding.SparseAttnPlan(1, 128, 1, 96)
    assert e.value.code == SA_EUNSUPPORTED_SHAPE and "64 or 128" in str(e.value)


def test_exact_kv_flag_is_accepted(lib):
    from block_sparse_video_fp32_amd.binding import SA_FLAG_EXACT_KV_ONLY
    assert SA_FLAG_EXACT_KV_ONLY == 4
    assert _create(lib, _params(flags=3 | SA_FLAG_EXACT_KV_ONLY, prefix_len=100)) == 0
    plan = binding.SparseAttnPlan(1, 1024, 2, 64, prefix_len=100, exact_kv_only=True)
    assert plan.params.flags == 3 | SA_FLAG_EXACT_KV_ONLY


def test_reweight_flag_needs_centroids(lib):
    from block_sparse_video_fp32_amd.binding import SA_FLAG_REWEIGHT
    assert SA_FLAG_REWEIGHT == 8
    assert _create(lib, _params(flags=3 | SA_FLAG_REWEIGHT)) == 0
    assert _create(lib, _params(flags=2 | SA_FLAG_REWEIGHT)) == SA_EINVAL  # centroids off
    assert "SA_FLAG_CENTROID" in lib.sparse_attn_last_error().decode()


def test_int8_flag_is_accepted(lib):
    from block_sparse_video_fp32_amd.binding import SA_FLAG_INT8_QK
    assert SA_FLAG_INT8_QK == 16
    for f in (3, 0, 3 | 8, 3 | 4):
        assert _create(lib, _params(flags=f | SA_FLAG_INT8_QK)) == 0
    assert _create(lib, _params(flags=128)) == SA_EINVAL


@pytest.mark.parametrize("layout", ["q_reuse_k", "separate"])
def test_reblock_layout_and_stage_calls(lib, layout):
    """SA_FLAG_REBLOCK adds the partition sections (sizes as documented: one
    problem per (b, h) in the shared q_reuse_k layout, two with
    SA_FLAG_REBLOCK_KV_OWN; the copy sections rb_qkv and rb_out are empty)
    and runs through sparse_attn_forward only: the stage calls refuse the
    plan before touching any device."""
    from block_sparse_video_fp32_amd.binding import SA_FLAG_REBLOCK, SA_FLAG_REBLOCK_KV_OWN
    assert SA_FLAG_REBLOCK == 32 and SA_FLAG_REBLOCK_KV_OWN == 64
    B, N, H, D, pre = 2, 1000, 3, 128, 70
    plan = binding.SparseAttnPlan(B, N, H, D, tau=1.0, prefix_len=pre, reblock=True, reblock_layout=layout)
    assert bool(plan.params.flags & SA_FLAG_REBLOCK_KV_OWN) == (layout == "separate")
    L = plan.layout
    nv, P = N - 128, (2 if layout == "separate" else 1) * B * H
    assert L["reblock_levels"] == 4  # ceil(872 / 64) = 14 blocks
    sizes = dict(rb_gram=P * 1 * D * D * 4, rb_metric=P * D * D * 4, rb_units=P * nv * D * 2,
                 rb_munits=P * nv * D * 2, rb_order=2 * P * nv * 4, rb_keys=P * nv * 4, rb_qkv=0, rb_out=0)
    names = sorted(sizes, key=lambda n: L[n])
    ends = [L[n] for n in names[1:]] + [L["total_bytes"]]
    for n, e in zip(names, ends):
        assert e - L[n] >= sizes[n], n
    # sections sized for P problems, not more (the shared layout halves them)
    assert L["rb_munits"] - L["rb_units"] < sizes["rb_units"] + 256
    # no reordered copies: the path reads its rows through the orders
    assert L["rb_qkv"] == L["rb_out"] and L["rb_out"] >= L["rb_keys"] + sizes["rb_keys"]
    dense = binding.SparseAttnPlan(B, N, H, D, tau=-math.inf, reblock=True)
    assert dense.layout["reblock_levels"] == 0  # no effect on the dense path
    buf = ctypes.create_string_buffer(1 << 12)
    addr = (ctypes.addressof(buf) + 255) // 256 * 256
    for fn, args in ((lib.sparse_attn_pool, (addr, addr, addr, addr, 1 << 40, None)),
                     (lib.sparse_attn_select, (addr, 1 << 40, None)),
                     (lib.sparse_attn_attend, (addr, addr, addr, 1 << 40, None))):
        assert fn(plan._h, *args) == SA_EINVAL
        assert "sparse_attn_forward" in lib.sparse_attn_last_error().decode()
    # the separate layout is an option of SA_FLAG_REBLOCK only
    assert _create(lib, _params(flags=3 | SA_FLAG_REBLOCK_KV_OWN)) == SA_EINVAL
    assert "needs SA_FLAG_REBLOCK" in lib.sparse_attn_last_error().decode()
    with pytest.raises(ValueError):
        binding.SparseAttnPlan(B, N, H, D, reblock=True, reblock_layout="k_reuse_q")


def test_workspace_bytes_and_route_entry_points(lib):
    """sparse_attn_workspace_bytes reports the layout's total; the route
    call validates like the pool call (refused before any launch)."""
    plan = binding.SparseAttnPlan(1, 1000, 2, 64, tau=1.0)
    assert plan.workspace_bytes == plan.layout["total_bytes"] > 0
    n = ctypes.c_size_t()
    assert lib.sparse_attn_workspace_bytes(None, ctypes.byref(n)) == SA_EINVAL
    assert lib.sparse_attn_route(plan._h, None, None, None, None, 0, None) == SA_EINVAL


def test_launch_grid_limits(lib):
    """Shapes whose launch grids would exceed 65535 in y or z are refused at
    plan time with SA_EUNSUPPORTED_SHAPE (never at launch)."""
    assert _create(lib, _params(B=1, N=64, H=70000)) == SA_EUNSUPPORTED_SHAPE
    assert _create(lib, _params(B=70000, N=64, H=8)) == SA_EUNSUPPORTED_SHAPE
    assert _create(lib, _params(B=1, N=64, H=40000)) == 0
    assert _create(lib, _params(B=1, N=64, H=40000, flags=3 | 32)) == 0  # B*H problems
    assert _create(lib, _params(B=2, N=64, H=40000, flags=3 | 32)) == SA_EUNSUPPORTED_SHAPE
    assert "REBLOCK" in lib.sparse_attn_last_error().decode()
    assert _create(lib, _params(B=1, N=64, H=40000, flags=3 | 32 | 64)) == SA_EUNSUPPORTED_SHAPE
    assert "2*B*H" in lib.sparse_attn_last_error().decode()


def test_missing_library_fails_loudly(tmp_path):
    """Without the built library every entry point raises: there is no
    other implementation to fall back to (checked in a fresh process)."""
    code = (
        "import torch\n"
        "from block_sparse_video_fp32_amd import binding\n"
        "for f in (binding.load_library,\n"
        "          lambda: binding.SparseAttnPlan(1, 128, 1, 64, tau=1.0),\n"
        "          lambda: binding.sparse_attn(*(torch.zeros(1, 128, 1, 64, dtype=torch.bfloat16) for _ in range(3)))):\n"
        "    try:\n"
        "        f()\n"
        "    except ImportError as e:\n"
        "        assert 'not found' in str(e), e\n"
        "    else:\n"
        "        raise SystemExit('no error')\n"
        "print('ok')\n"
    )
    import subprocess
    import sys

    env = dict(os.environ, SPARSE_ATTN_LIB=str(tmp_path / "absent.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]
