"""C-ABI checks that need no GPU: the library loads, exports what include/fa.h declares,
validates arguments before touching the device, and links no vendor math library."""

import os
import re
import subprocess

import pytest

import attention_forward_fwd_amd as fa
from attention_forward_fwd_amd import fa as fab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _lib():
    if not os.path.exists(fa.lib_path()):
        pytest.skip("libfa.so not built (run __graft_entry__.build())")
    return fa.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_entry_points():
    assert _declared_functions() == sorted(fab.EXPORTS)


def test_library_exports_every_declared_symbol():
    _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", fa.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, f"{name} declared in fa.h but not exported"


def test_no_vendor_math_library_linked():
    _lib()
    out = subprocess.run(["readelf", "-d", fa.lib_path()], capture_output=True, text=True,
                         check=True).stdout
    needed = re.findall(r"\(NEEDED\).*\[(.+?)\]", out)
    banned = ("rocblas", "hipblas", "miopen", "composable", "ck_", "rocwmma", "triton", "torch")
    assert not [n for n in needed if any(b in n.lower() for b in banned)], needed
    undef = subprocess.run(["nm", "-D", "--undefined-only", fa.lib_path()], capture_output=True,
                           text=True, check=True).stdout.lower()
    assert not any(b in undef for b in ("rocblas", "hipblas", "miopen")), "vendor GEMM symbols"


def test_abi_version_and_status_strings():
    lib = _lib()
    assert lib.fa_abi_version() == 9
    header = open(HEADER).read()
    assert re.search(r"#define FA_ABI_VERSION 9\b", header)
    # the first five failure codes in the boundary's order; extensions after them
    for name, code in (("FA_OK", 0), ("FA_ERR_NULL_PTR", 1), ("FA_ERR_BAD_SHAPE", 2),
                       ("FA_ERR_UNSUPPORTED", 3), ("FA_ERR_BAD_MASK_MODE", 4), ("FA_ERR_HIP", 5),
                       ("FA_ERR_BAD_SCALE", 6), ("FA_ERR_WORKSPACE", 7),
                       ("FA_ERR_SCRATCH_LIMIT", 8)):
        assert re.search(rf"\b{name} = {code}\b", header), name
        assert fab.STATUS[code] == name
    assert "fa_status_string(fa_status status)" in header
    for code, name in fab.STATUS.items():
        s = fa.fa_status_string(code)
        assert s and isinstance(s, str)
    assert fa.fa_status_string(12345) == "unknown status"


def test_kernel_events_hook_arguments():
    # Setting or clearing the hook makes no HIP call; exactly one NULL event is refused.  A pair
    # set before a call that fails validation is consumed by that call (it records nothing: the
    # fake handles below are never passed to HIP).
    lib = _lib()
    assert lib.fa_set_kernel_events(None, None) == 0
    assert lib.fa_set_kernel_events(0x1000, None) == 1
    assert lib.fa_set_kernel_events(None, 0x1000) == 1
    assert lib.fa_set_kernel_events(0x1000, 0x2000) == 0
    assert fa.fa_fwd_raw(1, 0, 1, 1, 1, 64, 128, 1.0, 0, 0x10000, 0x10000, 0, 0x10000, 0) == 1
    assert lib.fa_set_kernel_events(None, None) == 0
    with pytest.raises(ValueError):
        fa.set_kernel_events(object(), None)


# Arguments that must be rejected synchronously, before any HIP call (no GPU is touched, so
# these run on a CPU-only machine).  Fake but 16-byte-aligned pointers are never dereferenced.
P = 0x10000


def _call(**kw):
    a = dict(dtype=1, mode=0, B=1, Hq=2, Hkv=1, S=8, D=128, scale=0.1, q=P, k=P, v=P, mask=0,
             o=P, stream=0)
    a.update(kw)
    return fa.fa_fwd_raw(a["dtype"], a["mode"], a["B"], a["Hq"], a["Hkv"], a["S"], a["D"],
                         a["scale"], a["q"], a["k"], a["v"], a["mask"], a["o"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(o=0), 1),
    (dict(B=0), 2), (dict(S=0), 2), (dict(S=-5), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2),
    (dict(Hq=6, Hkv=4), 2), (dict(S=1 << 20, Hq=128, Hkv=1), 2),
    (dict(D=96), 3), (dict(D=256), 3), (dict(dtype=7), 3), (dict(q=P + 8), 3), (dict(o=P + 2), 3),
    (dict(mode=3), 4), (dict(mode=-1), 4), (dict(mode=2, mask=0), 4), (dict(mode=2, mask=P + 2), 4),
    (dict(scale=float("nan")), 6), (dict(scale=float("inf")), 6), (dict(scale=float("-inf")), 6),
])
def test_invalid_arguments_rejected_before_launch(kw, status):
    _lib()
    assert _call(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(o=0), 1), (dict(D=96), 3), (dict(mode=2, mask=0), 4),
    (dict(scale=float("nan")), 6), (dict(S=0), 2),
])
def test_lse_entry_invalid_arguments_rejected(kw, status):
    # fa_fwd_lse validates like fa_fwd, given a valid lse pointer
    _lib()
    a = dict(dtype=1, mode=0, B=1, Hq=2, Hkv=1, S=8, D=128, scale=0.1, q=P, k=P, v=P, mask=0, o=P)
    a.update(kw)
    assert fa.fa_fwd_lse_raw(a["dtype"], a["mode"], a["B"], a["Hq"], a["Hkv"], a["S"], a["D"],
                             a["scale"], a["q"], a["k"], a["v"], a["mask"], a["o"], P, 0) == status


@pytest.mark.parametrize("kw,status", [
    (dict(tiles=P), 4), (dict(mode=1, tiles=P), 4), (dict(mode=2, mask=P, tiles=P + 2), 3),
    (dict(mode=2, mask=P, tiles=P, S=131073, D=64, Hq=1), 3), (dict(mode=2, mask=P, lse=P + 1), 3),
    (dict(q=0), 1), (dict(mode=2, mask=0, tiles=P), 4),
    (dict(splits=-1), 3), (dict(splits=17), 3), (dict(mode=2, mask=P, tiles=P, splits=2), 3),
])
def test_ex_entry_validates(kw, status):
    assert _ex(**kw) == status


def _ex(**kw):
    _lib()
    a = dict(dtype=1, mode=0, B=1, Hq=2, Hkv=1, S=8, D=128, scale=0.1, q=P, k=P, v=P, mask=0,
             tiles=0, splits=1, o=P, lse=0, ws=0, ws_bytes=0)
    a.update(kw)
    return fa.fa_fwd_ex_raw(a["dtype"], a["mode"], a["B"], a["Hq"], a["Hkv"], a["S"], a["D"],
                            a["scale"], a["q"], a["k"], a["v"], a["mask"], a["tiles"],
                            a["splits"], a["o"], a["lse"], a["ws"], a["ws_bytes"], 0)


WS_CASE = dict(B=4, Hq=16, Hkv=16, S=8192)   # packed V: the plan needs a workspace


@pytest.mark.parametrize("kw", [
    dict(ws=P, ws_bytes=1),                           # far too small
    dict(ws=P, ws_bytes=-1 + 4 * 16 * 128 * 64 * 128 * 2),  # one byte short of the plan
    dict(ws=P + 16, ws_bytes=1 << 30),                # large enough but not 256-byte aligned
    dict(ws=P, ws_bytes=0),                           # a pointer with no size
])
def test_caller_workspace_checked_before_launch(kw):
    # Rejected synchronously (FA_ERR_WORKSPACE), before any HIP call: these run without a GPU.
    need = _plan()["workspace_bytes"]
    assert need == 4 * 16 * 128 * 64 * 128 * 2
    assert _ex(**WS_CASE, **kw) == 7


def test_plan_workspace_layout_with_split_and_packed_v():
    # packed V^T first, then the split-KV partials at the next 256-byte boundary
    p = _plan(B=1, Hq=16, Hkv=16, S=8200, splits=2)
    vt = 16 * 129 * 64 * 128 * 2
    part = 2 * 8200 * 16 * (128 + 2) * 4
    assert p["packed_v"] == 1 and p["kv_splits"] == 2
    assert p["workspace_bytes"] == ((vt + 255) // 256) * 256 + part


@pytest.mark.parametrize("lse,status", [(0, 1), (P + 2, 3)])
def test_lse_pointer_checked(lse, status):
    _lib()
    assert fa.fa_fwd_lse_raw(1, 0, 1, 2, 1, 8, 128, 0.1, P, P, P, 0, P, lse, 0) == status


@pytest.mark.parametrize("fn", ["fa_pack_mask_raw", "fa_mask_tiles_raw"])
@pytest.mark.parametrize("args,status", [
    ((1, 1, 8, 0, P, 0), 1), ((1, 1, 8, P, 0, 0), 1), ((0, 1, 8, P, P, 0), 2),
    ((1, 0, 8, P, P, 0), 2), ((1, 1, 0, P, P, 0), 2), ((1, 1, -3, P, P, 0), 2),
    ((1, 1, 8, P, P + 2, 0), 3), ((1 << 20, 64, 1 << 14, P, P, 0), 2),
])
def test_mask_entries_validate(fn, args, status):
    _lib()
    assert getattr(fa, fn)(*args) == status


def test_python_binding_refuses_cpu_tensors():
    import torch
    _lib()
    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa.fa_fwd(q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        fa.fa_fwd_lse(q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        fa.pack_mask(torch.zeros(1, 1, 8, 8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU"):
        fa.mask_tiles(torch.zeros(1, 1, 8, 1, dtype=torch.int32))


def test_python_binding_checks_every_tensor_device():
    # Only q can be checked for "is a GPU tensor" without a GPU here; the same helper checks k,
    # v, mask, tiles, out and workspace against q's device (a CPU out would hand a host pointer
    # to a kernel that writes through it).
    import torch
    _lib()
    t = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    for name in ("out", "k", "v", "mask", "tiles", "workspace"):
        with pytest.raises(ValueError, match=f"{name} must be a GPU tensor"):
            fab._same_gpu(name, t, torch.device("cuda:0"))


def test_kernel_launch_stubs_defined():
    """Every kernel the library launches is defined in it: an undefined kernel symbol makes the
    library fail to load on a GPU machine even though lazy binding lets it load here."""
    _lib()
    undef = subprocess.run(["nm", "-D", "--undefined-only", fa.lib_path()], capture_output=True,
                           text=True, check=True).stdout
    assert "fa_fwd_kernel" not in undef, [l for l in undef.splitlines() if "fa_fwd_kernel" in l]


# ---------------------------------------------------------------- launch plan (host logic, no GPU)
NONE, CAUSAL, BITMASK, BF16, F16 = 0, 1, 2, 1, 0


def _plan(**kw):
    a = dict(dtype=BF16, mode=NONE, B=4, Hq=16, Hkv=16, S=8192, D=128, tiles=False, splits=1)
    a.update(kw)
    _lib()
    return fa.fa_fwd_plan(a["dtype"], a["mode"], a["B"], a["Hq"], a["Hkv"], a["S"], a["D"],
                          a["tiles"], a["splits"])


def test_plan_prefill_uses_256_row_workgroups_and_packed_v():
    p = _plan()
    n_kt = 8192 // 64
    assert p["rows_per_workgroup"] == 256 and p["packed_v"] == 1 and p["kv_splits"] == 1
    assert p["workgroups"] == 4 * 16 * 8192 // 256 and p["kernels"] == 2
    assert p["workspace_bytes"] == 4 * 16 * n_kt * 64 * 128 * 2      # packed V^T: about V's size


def test_plan_row_thresholds():
    # 256-row workgroups from these rows per KV head (S x G): 512 at head_dim 128 and 2048 at
    # head_dim 64 (none, bitmask); causal 2048 at head_dim 128 and 8192 at head_dim 64
    assert _plan(B=8, S=4096)["rows_per_workgroup"] == 256
    assert _plan(B=16, S=2048)["rows_per_workgroup"] == 256
    assert _plan(B=16, S=512)["rows_per_workgroup"] == 256
    assert _plan(B=16, S=511)["rows_per_workgroup"] == 128
    assert _plan(B=16, S=511, mode=BITMASK)["rows_per_workgroup"] == 128
    assert _plan(B=16, S=512, mode=BITMASK)["rows_per_workgroup"] == 256
    assert _plan(B=16, S=2047, D=64, dtype=F16)["rows_per_workgroup"] == 128
    assert _plan(B=16, S=2048, D=64, dtype=F16)["rows_per_workgroup"] == 256
    assert _plan(B=16, S=1000, D=64, dtype=F16, mode=BITMASK)["rows_per_workgroup"] == 128
    assert _plan(B=8, S=4096, mode=CAUSAL)["rows_per_workgroup"] == 256
    assert _plan(B=8, S=2048, mode=CAUSAL)["rows_per_workgroup"] == 256
    assert _plan(B=8, S=2047, mode=CAUSAL)["rows_per_workgroup"] == 128
    assert _plan(B=2, S=4096, mode=CAUSAL, D=64, dtype=F16)["rows_per_workgroup"] == 128
    assert _plan(B=2, S=8192, mode=CAUSAL, D=64, dtype=F16)["rows_per_workgroup"] == 256
    assert _plan(B=4, S=8192, mode=CAUSAL)["rows_per_workgroup"] == 256
    assert _plan(B=16, S=256, Hq=32, Hkv=8)["rows_per_workgroup"] == 256   # 256 x 4 rows


def test_plan_short_masked():
    # S = 512 and 1000: four and eight 128-row tiles per head, V's rows read by each workgroup,
    # nothing allocated
    p = _plan(dtype=F16, mode=BITMASK, B=16, S=512, D=64)
    assert p == {"rows_per_workgroup": 128, "packed_v": 0, "kv_splits": 1, "kernels": 1,
                 "workgroups": 16 * 16 * 4, "workspace_bytes": 0}
    p = _plan(dtype=F16, mode=BITMASK, B=16, S=1000, D=64)
    assert p["packed_v"] == 0 and p["workspace_bytes"] == 0 and p["kernels"] == 1


@pytest.mark.parametrize("mode,rows,nw_rows,packed", [
    (NONE, 2047, 128, 0), (NONE, 2048, 256, 0), (NONE, 4096, 256, 0), (NONE, 7936, 256, 0),
    (NONE, 7937, 256, 1), (BITMASK, 2047, 128, 0), (BITMASK, 4095, 256, 0), (BITMASK, 7937, 256, 1),
    (CAUSAL, 3968, 128, 0), (CAUSAL, 3969, 128, 1), (CAUSAL, 8191, 128, 1), (CAUSAL, 8192, 256, 1),
])
def test_plan_packs_v_from_32_row_tiles(mode, rows, nw_rows, packed):
    # V is packed once per call when a KV head's rows make 32 or more row tiles; otherwise each
    # workgroup reads V's rows (no workspace).  One head: rows per KV head = S.
    p = _plan(mode=mode, dtype=F16, D=64, B=1, Hq=1, Hkv=1, S=rows)
    assert p["rows_per_workgroup"] == nw_rows and p["packed_v"] == packed
    assert (p["workspace_bytes"] > 0) == bool(packed) and p["kernels"] == 1 + packed


def test_plan_causal_d128_packs_v_from_64_row_tiles():
    # causal at head_dim 128 does half the work per row tile: V is packed from 64 row tiles
    for rows, packed in ((8192, 0), (16128, 0), (16129, 1)):
        p = _plan(mode=CAUSAL, B=1, Hq=1, Hkv=1, S=rows)
        assert p["rows_per_workgroup"] == 256 and p["packed_v"] == packed, (rows, p)
    assert _plan(mode=NONE, B=1, Hq=1, Hkv=1, S=8192)["packed_v"] == 1


def test_plan_split_kv():
    # explicit shares are capped at the key tiles; the partials are n x B x S x Hq x (d + 2) x 4 B
    p = _plan(B=1, Hq=1, Hkv=1, S=130, splits=16)
    assert p["kv_splits"] == 3 and p["kernels"] == 2
    assert p["workspace_bytes"] == 3 * 130 * (128 + 2) * 4
    # automatic: a small grid (one head, S = 4096: 32 row tiles of 128 rows) is split to fill
    # the chip, at least 8 key tiles per share
    p = _plan(B=1, Hq=1, Hkv=1, S=4096, splits=0)
    assert p["rows_per_workgroup"] == 256 and p["kv_splits"] == 8 and p["workgroups"] == 16 * 8
    # automatic on a full grid, or with a tile summary: no split
    assert _plan(splits=0)["kv_splits"] == 1
    assert _plan(mode=BITMASK, B=1, Hq=1, Hkv=1, S=4096, tiles=True, splits=0)["kv_splits"] == 1


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=9), 3), (dict(mode=5), 4), (dict(S=0), 2), (dict(Hq=6, Hkv=4), 2), (dict(D=96), 3),
    (dict(tiles=True), 4), (dict(splits=17), 3), (dict(mode=BITMASK, tiles=True, splits=2), 3),
    (dict(mode=BITMASK, tiles=True, S=131073, Hq=1, Hkv=1, D=64), 3),
])
def test_plan_rejects_what_the_call_rejects(kw, status):
    with pytest.raises(fab.FaError) as ei:
        _plan(**kw)
    assert ei.value.status == status


# ---------------------------------------------------------------- fa_fwd_noalloc (validation only)
def _noalloc(**kw):
    _lib()
    a = dict(dtype=1, mode=0, B=1, Hq=2, Hkv=1, S=8, D=128, scale=0.1, q=P, k=P, v=P, mask=0,
             tiles=0, splits=1, o=P, lse=0)
    a.update(kw)
    return fa.fa_fwd_noalloc_raw(a["dtype"], a["mode"], a["B"], a["Hq"], a["Hkv"], a["S"],
                                 a["D"], a["scale"], a["q"], a["k"], a["v"], a["mask"],
                                 a["tiles"], a["splits"], a["o"], a["lse"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(S=0), 2), (dict(D=96), 3), (dict(mode=2, mask=0), 4),
    (dict(scale=float("nan")), 6), (dict(splits=17), 3), (dict(tiles=P), 4),
])
def test_noalloc_validates_like_ex(kw, status):
    assert _noalloc(**kw) == status


def test_noalloc_rejects_more_scratch_than_its_array():
    # packed V^T is about V's size: B8 S8192 H16 d128 fills the 256 MiB array exactly, B9 is
    # over it -> status 8, before any HIP call; B4 S8192 (128 MiB) fits.
    limit = 256 << 20
    assert re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \(256u << 20\)", open(HEADER).read())
    assert _plan(B=4)["workspace_bytes"] <= limit
    assert _plan(B=8, S=8192)["workspace_bytes"] == limit
    assert _plan(B=9, S=8192)["workspace_bytes"] > limit
    assert _noalloc(B=9, Hq=16, Hkv=16, S=8192) == 8
    # split-KV partials of two long heads in 16 shares: 16 x 32768 x 2 x 130 x 4 B > 256 MiB
    assert _plan(B=1, Hq=2, Hkv=2, S=32768, splits=16)["workspace_bytes"] > limit
    assert _noalloc(B=1, Hq=2, Hkv=2, S=32768, splits=16) == 8
