"""The C ABI without a GPU: the library loads, exports what include/elb.h declares, and
rejects bad arguments with the documented status before queueing anything."""

import ctypes
import os
import re
import subprocess

import pytest

from expert_load_balancing_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "elb.h")

OK, NULL, SHAPE, UNSUPPORTED, ALIGN, WORKSPACE = 0, 1, 2, 3, 4, 5
FAKE = 0x10000  # a non-NULL, 64 KiB-aligned address that is never dereferenced


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(elb_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def test_exports_every_declared_function(lib):
    declared = header_functions()
    assert declared == sorted(_lib.SIGNATURES), declared
    for name in declared:
        assert getattr(lib, name) is not None


def test_flag_constants_match_header():
    """The binding's flag and enum constants are the header's values."""
    text = open(HEADER).read()
    found = {}
    for name, val in re.findall(r"\b(ELB_[A-Z0-9_]+)\s*=\s*([0-9]+u?\s*<<\s*[0-9]+|[0-9]+)", text):
        found[name] = eval(val.replace("u", ""))  # "1u << 3" or "5": plain integer arithmetic
    for name in ("ELB_GATES_RAW", "ELB_ACCUMULATE_COUNTS", "ELB_FORCE_GENERIC", "ELB_CLEAR_COUNTS", "ELB_DX_BF16",
                 "ELB_F32", "ELB_BF16", "ELB_MODE_SMEBU", "ELB_MODE_SIGN", "ELB_MODE_LINEAR"):
        assert getattr(_lib, name) == found[name], name


def test_version_matches_header(lib):
    m = re.search(r"#define ELB_VERSION (\d+)", open(HEADER).read())
    assert lib.elb_version() == int(m.group(1))


def test_status_strings(lib):
    for code in range(7):
        assert lib.elb_status_str(code)
    assert lib.elb_status_str(99) == b"unknown status"


def fwd(lib, x=FAKE, dtype=1, T=1024, d=256, w=FAKE, bias=FAKE, n=256, k=4, flags=0, idx=FAKE, gates=FAKE,
        counts=FAKE, logits=None, lse=None):
    return lib.elb_router_forward(x, dtype, T, d, w, bias, n, k, flags, idx, gates, counts, logits, lse, None)


@pytest.mark.parametrize("kw,want", [
    (dict(w=None), NULL), (dict(bias=None), NULL), (dict(counts=None), NULL), (dict(x=None), NULL),
    (dict(idx=None), NULL), (dict(gates=None), NULL),
    (dict(dtype=2), UNSUPPORTED), (dict(flags=1 << 7), UNSUPPORTED),
    (dict(T=-1), SHAPE), (dict(d=0), SHAPE), (dict(n=0), SHAPE), (dict(n=257), SHAPE),
    (dict(k=0), SHAPE), (dict(k=9), SHAPE), (dict(n=2, k=3), SHAPE), (dict(T=1 << 29, k=4), SHAPE),
    (dict(d=100), ALIGN), (dict(dtype=0, d=98), ALIGN), (dict(x=FAKE + 8), ALIGN), (dict(w=FAKE + 2), ALIGN),
    (dict(idx=FAKE + 4), ALIGN), (dict(bias=FAKE + 2), ALIGN),
])
def test_router_forward_rejects(lib, kw, want):
    assert fwd(lib, **kw) == want


def test_empty_batch_may_pass_null_token_buffers(lib):
    # With T = 0 only counts is written; a NULL x / idx / gates is then not an error, but
    # the call does launch the counter reset, so only the argument check is exercised here.
    assert fwd(lib, T=0, x=None, idx=None, gates=None, dtype=7) == UNSUPPORTED


def test_dispatch_workspace_size(lib):
    # Tiles of 256 tokens: a [n_experts][n_tiles rounded up to 4] table of tile loads, then
    # the n_experts totals.
    assert lib.elb_dispatch_workspace_bytes(65536, 4, 256) == (256 * 256 + 256) * 4
    assert lib.elb_dispatch_workspace_bytes(262144, 4, 256) == (1024 * 256 + 256) * 4
    assert lib.elb_dispatch_workspace_bytes(262144, 1, 256) == (1024 * 256 + 256) * 4
    assert lib.elb_dispatch_workspace_bytes(10, 2, 16) == (4 * 16 + 16) * 4
    assert lib.elb_dispatch_workspace_bytes(1300, 8, 64) == (8 * 64 + 64) * 4
    assert lib.elb_dispatch_workspace_bytes(0, 4, 256) == 0
    assert lib.elb_dispatch_workspace_bytes(-1, 4, 256) == 0
    assert lib.elb_dispatch_workspace_bytes(16, 4, 300) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(offsets=None), NULL), (dict(idx=None), NULL), (dict(perm=None), NULL), (dict(ws=None), NULL),
    (dict(n=0), SHAPE), (dict(n=257), SHAPE), (dict(k=0), SHAPE), (dict(T=-5), SHAPE),
    (dict(ws_bytes=16), WORKSPACE), (dict(ws=FAKE + 4), ALIGN), (dict(perm=FAKE + 2), ALIGN),
    (dict(T=(1 << 31) // 8, k=8, ws_bytes=1 << 31), SHAPE),  # T * k = 2^31: past the int32 positions
])
def test_router_dispatch_rejects(lib, kw, want):
    a = dict(idx=FAKE, T=4096, k=4, n=256, ws=FAKE, ws_bytes=1 << 20, offsets=FAKE, perm=FAKE, inv=None)
    a.update(kw)
    st = lib.elb_router_dispatch(a["idx"], a["T"], a["k"], a["n"], a["ws"], a["ws_bytes"], a["offsets"],
                                 a["perm"], a["inv"], None)
    assert st == want


@pytest.mark.parametrize("kw,want", [
    (dict(mode=3), UNSUPPORTED), (dict(mode=-1), UNSUPPORTED), (dict(counts=None), NULL), (dict(bias=None), NULL),
    (dict(momentum=None), NULL), (dict(momentum=None, mode=2), NULL), (dict(n=0), SHAPE), (dict(n=1025), SHAPE),
    (dict(bias=FAKE + 1), ALIGN), (dict(flags=2), UNSUPPORTED), (dict(flags=1 << 31), UNSUPPORTED),
])
def test_smebu_update_rejects(lib, kw, want):
    a = dict(counts=FAKE, n=256, mode=0, bias=FAKE, momentum=FAKE, delta=None, mv=None, flags=0)
    a.update(kw)
    p = _lib.BalanceParams(a["mode"], 5e-4, 0.5, 2.0, 1e-3, a["flags"])
    assert lib.elb_smebu_update(a["counts"], a["n"], p, a["bias"], a["momentum"], a["delta"], a["mv"], None) == want


def test_maxvio_rejects(lib):
    assert lib.elb_maxvio(None, 256, FAKE, None) == NULL
    assert lib.elb_maxvio(FAKE, 256, None, None) == NULL
    assert lib.elb_maxvio(FAKE, 0, FAKE, None) == SHAPE
    assert lib.elb_maxvio(FAKE, 2000, FAKE, None) == SHAPE


def test_stream_xor_rejects(lib):
    assert lib.elb_stream_xor(None, 64, FAKE, None) == NULL
    assert lib.elb_stream_xor(FAKE, 64, None, None) == NULL
    assert lib.elb_stream_xor(FAKE, 24, FAKE, None) == SHAPE
    assert lib.elb_stream_xor(FAKE + 8, 64, FAKE, None) == ALIGN
    assert lib.elb_stream_xor(FAKE, 64, FAKE + 2, None) == ALIGN


def step_args(**kw):
    a = _lib.StepArgs()
    base = dict(x=FAKE, dtype=1, T=4096, d=256, w=FAKE, bias=FAKE, n_experts=256, k=4, flags=2, topk_idx=FAKE,
                gates=FAKE, counts=FAKE, logits=None, lse=None, workspace=FAKE, workspace_bytes=1 << 20,
                offsets=FAKE, perm=FAKE, inv_perm=None, update=1, momentum=FAKE, delta_b=None, maxvio=None,
                timing=None)
    params = dict(mode=0, lambda_=5e-4, beta=0.5, kappa=2.0, gamma=1e-3, flags=1)
    for key, val in kw.items():
        (params if key.startswith("p_") else base)[key[2:] if key.startswith("p_") else key] = val
    for key, val in base.items():
        setattr(a, key, val)
    a.params = _lib.BalanceParams(**params)
    return a


@pytest.mark.parametrize("kw,want", [
    # forward checks
    (dict(w=None), NULL), (dict(x=None), NULL), (dict(counts=None), NULL), (dict(dtype=5), UNSUPPORTED),
    (dict(flags=1 << 9), UNSUPPORTED), (dict(k=9), SHAPE), (dict(n_experts=300), SHAPE), (dict(d=100), ALIGN),
    # dispatch checks
    (dict(offsets=None), NULL), (dict(perm=None), NULL), (dict(workspace=None), NULL),
    (dict(workspace_bytes=64), WORKSPACE), (dict(workspace=FAKE + 4), ALIGN),
    # update checks, only when the update is asked for
    (dict(p_mode=7), UNSUPPORTED), (dict(p_flags=4), UNSUPPORTED), (dict(momentum=None), NULL),
    (dict(momentum=None, p_mode=1, p_flags=0, update=1, bias=FAKE + 1), ALIGN),
    # no dispatch (offsets, perm, inv_perm all NULL): the forward and update checks still apply
    (dict(offsets=None, perm=None, workspace=None, k=9), SHAPE),
    (dict(offsets=None, perm=None, workspace=None, momentum=None), NULL),
    (dict(offsets=None, perm=None, workspace=None, x=FAKE + 8), ALIGN),
])
def test_route_step_rejects(lib, kw, want):
    assert lib.elb_route_step(ctypes.byref(step_args(**kw)), None) == want


def test_route_step_null_args(lib):
    assert lib.elb_route_step(None, None) == NULL


def _c_layout(struct: str, fields: list[str], tmp_path) -> dict:
    """offsetof/sizeof of a struct of include/elb.h as the host C compiler lays it out."""
    src = tmp_path / "layout.c"
    lines = [f'printf("{f} %zu\\n", offsetof({struct}, {f}));' for f in fields]
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"elb.h\"\nint main(void) {\n" +
                   "\n".join(lines) + f'\nprintf("sizeof %zu\\n", sizeof({struct}));\nreturn 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    return {ln.split()[0]: int(ln.split()[1]) for ln in out.splitlines()}


@pytest.mark.parametrize("cls,cname", [(_lib.BalanceParams, "elb_balance_params"), (_lib.StepArgs, "elb_step_args")])
def test_struct_layout_matches_header(cls, cname, tmp_path):
    names = [f for f, _ in cls._fields_]
    c_names = ["lambda" if f == "lambda_" else f for f in names]
    got = _c_layout(cname, c_names, tmp_path)
    for f, cf in zip(names, c_names):
        assert getattr(cls, f).offset == got[cf], (cname, cf)
    assert ctypes.sizeof(cls) == got["sizeof"]


@pytest.mark.parametrize("kw,want", [
    (dict(counts=None), NULL), (dict(bias=None), NULL), (dict(momentum=None), NULL), (dict(L=0), SHAPE),
    (dict(L=-3), SHAPE), (dict(n=0), SHAPE), (dict(n=1025), SHAPE), (dict(L=1 << 22, n=1024), SHAPE),
    (dict(mode=9), UNSUPPORTED), (dict(flags=8), UNSUPPORTED), (dict(mv=FAKE + 2), ALIGN),
])
def test_smebu_update_layers_rejects(lib, kw, want):
    a = dict(counts=FAKE, L=60, n=256, mode=0, bias=FAKE, momentum=FAKE, delta=None, mv=None, flags=0)
    a.update(kw)
    p = _lib.BalanceParams(a["mode"], 5e-4, 0.5, 2.0, 1e-3, a["flags"])
    st = lib.elb_smebu_update_layers(a["counts"], a["L"], a["n"], p, a["bias"], a["momentum"], a["delta"], a["mv"],
                                     None)
    assert st == want


def test_zloss_rejects(lib):
    assert lib.elb_zloss(FAKE, 100, None, None) == NULL
    assert lib.elb_zloss(None, 100, FAKE, None) == NULL
    assert lib.elb_zloss(FAKE, -1, FAKE, None) == SHAPE
    assert lib.elb_zloss(FAKE + 2, 100, FAKE, None) == ALIGN


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(inv=None), NULL), (dict(xp=None), NULL), (dict(dtype=3), UNSUPPORTED),
    (dict(T=-1), SHAPE), (dict(d=0), SHAPE), (dict(k=0), SHAPE), (dict(k=9), SHAPE), (dict(T=1 << 29, k=4), SHAPE),
    (dict(d=100), ALIGN), (dict(dtype=0, d=98), ALIGN), (dict(x=FAKE + 8), ALIGN), (dict(xp=FAKE + 4), ALIGN),
])
def test_permute_rows_rejects(lib, kw, want):
    a = dict(x=FAKE, dtype=1, T=1000, d=256, k=4, inv=FAKE, xp=FAKE)
    a.update(kw)
    assert lib.elb_permute_rows(a["x"], a["dtype"], a["T"], a["d"], a["k"], a["inv"], a["xp"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(eo=None), NULL), (dict(inv=None), NULL), (dict(g=None), NULL), (dict(y=None), NULL),
    (dict(dtype=2), UNSUPPORTED), (dict(ydt=5), UNSUPPORTED), (dict(T=-2), SHAPE), (dict(k=9), SHAPE),
    (dict(d=100), ALIGN), (dict(dtype=0, d=102), ALIGN), (dict(y=FAKE + 8), ALIGN), (dict(g=FAKE + 1), ALIGN),
])
def test_unpermute_combine_rejects(lib, kw, want):
    a = dict(eo=FAKE, dtype=1, T=1000, d=256, k=4, inv=FAKE, g=FAKE, y=FAKE, ydt=0)
    a.update(kw)
    st = lib.elb_unpermute_combine(a["eo"], a["dtype"], a["T"], a["d"], a["k"], a["inv"], a["g"], a["y"], a["ydt"],
                                   None)
    assert st == want


def test_route_step_zloss_needs_lse(lib):
    a = step_args(zloss=FAKE, lse=None)
    assert lib.elb_route_step(ctypes.byref(a), None) == NULL


def test_backward_workspace_size(lib):
    # dZ token-major (T x 256 bf16), then the dW partials (splits x 256 x d fp32), each rounded
    # up to 256 bytes.  splits = 256 // ceil(d / 256) token ranges (one workgroup per CU), at
    # most ceil(T / 64).  d = 3072: 12 column tiles -> 21 ranges.
    assert lib.elb_backward_workspace_bytes(65536, 3072, 256) == 65536 * 512 + 21 * 256 * 3072 * 4
    # 2100 tokens, d = 192: 1 column tile -> 256 ranges wanted, 33 stages of 64 tokens -> 33.
    assert lib.elb_backward_workspace_bytes(2100, 192, 64) == 2100 * 512 + 33 * 256 * 192 * 4
    # 1 token: one range; the dZ row rounds up to 512 bytes.
    assert lib.elb_backward_workspace_bytes(1, 64, 8) == 512 + 256 * 64 * 4
    # No tokens: a minimal workspace (nothing of it is read).
    assert lib.elb_backward_workspace_bytes(0, 64, 8) == 256
    assert lib.elb_backward_workspace_bytes(-1, 64, 8) == 0
    assert lib.elb_backward_workspace_bytes(100, 100, 8) == 0
    assert lib.elb_backward_workspace_bytes(100, 64, 300) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(w=None), NULL), (dict(ws=None), NULL), (dict(x=None), NULL), (dict(idx=None), NULL), (dict(g=None), NULL),
    (dict(dtype=0), UNSUPPORTED), (dict(flags=2), UNSUPPORTED), (dict(flags=8 | 4), UNSUPPORTED),
    (dict(d=96), UNSUPPORTED),
    (dict(T=-1), SHAPE), (dict(T=(1 << 22) + 1), SHAPE), (dict(n=0), SHAPE), (dict(n=257), SHAPE), (dict(k=9), SHAPE),
    (dict(n=4, k=5), SHAPE), (dict(zc=float("nan")), SHAPE), (dict(zc=float("inf")), SHAPE),
    (dict(x=FAKE + 8), ALIGN), (dict(dw=FAKE + 4), ALIGN), (dict(dx=FAKE + 8), ALIGN), (dict(ws=FAKE + 64), ALIGN),
    (dict(ws_bytes=1024), WORKSPACE),
])
def test_router_backward_rejects(lib, kw, want):
    a = dict(x=FAKE, dtype=1, T=4096, d=256, w=FAKE, n=256, k=4, flags=0, idx=FAKE, g=FAKE, zc=0.0, dx=FAKE, dw=FAKE,
             ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    st = lib.elb_router_backward(a["x"], a["dtype"], a["T"], a["d"], a["w"], a["n"], a["k"], a["flags"], a["idx"],
                                 a["g"], a["zc"], a["dx"], a["dw"], a["ws"], a["ws_bytes"], None)
    assert st == want


def test_binding_checks_buffer_sizes_before_the_device():
    """The Python binding refuses caller buffers of the wrong size before anything else (a
    buffer too small would be written past its end on the device); these checks need no GPU."""
    import torch

    import expert_load_balancing_amd as elb

    x = torch.zeros(10, 64, dtype=torch.bfloat16)
    w = torch.zeros(256, 64, dtype=torch.bfloat16)
    b = torch.zeros(256)
    i32 = torch.int32
    with pytest.raises(ValueError, match="T\\*k = 40"):
        elb.router_forward(x, w, b, 4, out=(torch.zeros(10, 3, dtype=i32), torch.zeros(10, 4)))
    with pytest.raises(ValueError, match="T\\*k = 40"):
        elb.router_forward(x, w, b, 4, out=(torch.zeros(10, 4, dtype=i32), torch.zeros(39)))
    with pytest.raises(ValueError, match="N_r = 256"):
        elb.router_forward(x, w, b, 4, counts=torch.zeros(255, dtype=i32))
    with pytest.raises(ValueError, match="shapes do not match"):
        elb.router_forward(x, w[:, :32], b, 4)
    with pytest.raises(ValueError, match=r"\[T, k\]"):
        elb.router_dispatch(torch.zeros(40, dtype=i32), 256)
    # Right sizes: the next refusal is the device.
    with pytest.raises(ValueError, match="GPU"):
        elb.router_forward(x, w, b, 4, out=(torch.zeros(10, 4, dtype=i32), torch.zeros(10, 4)),
                           counts=torch.zeros(256, dtype=i32))


@pytest.mark.parametrize("kw,want", [
    (dict(offsets=None), NULL), (dict(idx=None), NULL), (dict(perm=None), NULL),
    (dict(n=0), SHAPE), (dict(n=257), SHAPE), (dict(k=0), SHAPE), (dict(k=9), SHAPE), (dict(T=-5), SHAPE),
    (dict(T=(1 << 31) // 8, k=8), SHAPE),  # T * k = 2^31: past the int32 positions
    (dict(T=2_096_129), WORKSPACE),  # one token past what the 8 MiB static workspace holds at 256 experts
    (dict(T=8_388_608, n=64, k=1), WORKSPACE),
    (dict(offsets=FAKE + 2), ALIGN), (dict(inv=FAKE + 1), ALIGN),
])
def test_router_dispatch_noalloc_rejects(lib, kw, want):
    """The allocation-free dispatch refuses what elb_router_dispatch refuses, and sizes past its
    static workspace, before touching any device."""
    a = dict(idx=FAKE, T=4096, k=4, n=256, offsets=FAKE, perm=FAKE, inv=None)
    a.update(kw)
    st = lib.elb_router_dispatch_noalloc(a["idx"], a["T"], a["k"], a["n"], a["offsets"], a["perm"], a["inv"], None)
    assert st == want


def test_noalloc_limit_matches_the_workspace_size(lib):
    """The largest batch the static workspace holds at 256 experts: 2,096,128 tokens (8188 tiles)."""
    assert lib.elb_dispatch_workspace_bytes(2_096_128, 4, 256) <= 8 << 20
    assert lib.elb_dispatch_workspace_bytes(2_096_129, 4, 256) > 8 << 20
