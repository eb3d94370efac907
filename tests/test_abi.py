"""The C ABI without a GPU: the library loads, exports every function that
include/*.h declares, and rejects every bad argument with its status code
before touching the HIP runtime.  CPU only (no compute calls)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from exact_attention_forward_02_amd import _binding, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CODES = {
    "ATTN_OK": 0, "ATTN_ERR_NULL_PTR": 1, "ATTN_ERR_BAD_SHAPE": 2, "ATTN_ERR_GQA_RATIO": 3,
    "ATTN_ERR_UNSUPPORTED_HEAD_DIM": 4, "ATTN_ERR_BAD_SCALE": 5, "ATTN_ERR_MISALIGNED": 6,
    "ATTN_ERR_TOO_LARGE": 7, "ATTN_ERR_NO_DEVICE": 8, "ATTN_ERR_UNSUPPORTED_ARCH": 9,
    "ATTN_ERR_HIP": 10, "ATTN_ERR_BAD_ARGUMENT": 11, "ATTN_ERR_BAD_STRIDE": 12,
    "ATTN_ERR_SCRATCH": 13,
}


def _declared_functions():
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(",
                             text, flags=re.M):
            names.add(m.group(1))
    return names


def _exported_symbols(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], check=True,
                         capture_output=True, text=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


def test_header_declares_the_entry_points():
    assert {"attn_fwd", "attn_fwd_dbg", "attn_fwd_ex", "attn_bwd", "attn_bwd_ex", "attn_bwd_noalloc",
            "attn_split_keys", "attn_fwd_split",
            "attn_merge", "attn_varlen_plan", "attn_fwd_varlen", "attn_fwd_decode",
            "attn_status_string",
            "attn_abi_version"} <= _declared_functions()


def test_status_codes_match_header():
    text = open(os.path.join(ROOT, "include", "attn_fwd.h"), encoding="utf-8").read()
    for name, value in CODES.items():
        assert re.search(rf"\b{name}\s*=\s*{value}\b", text), name


def test_library_exports_every_declared_function():
    lib = _binding.library()
    assert lib is not None
    exported = _exported_symbols(build.LIBRARY)
    missing = _declared_functions() - exported
    assert not missing, f"declared but not exported: {sorted(missing)}"


def test_abi_version_and_status_strings():
    lib = _binding.library()
    assert lib.attn_abi_version() == 8
    for code in CODES.values():
        s = _binding.status_string(code)
        assert s and s != "unknown attn status"
    assert _binding.status_string(999) == "unknown attn status"


# fake device addresses: never dereferenced, validation happens first
A = 0x10000
GOOD = dict(q=A, k=A * 2, v=A * 3, o=A * 4, lse=A * 5, B=1, Hq=4, Hkv=2, Lq=64, Lk=64,
            d_qk=128, d_v=128, causal=0, scale=0.088, stream=None)
ORDER = ["q", "k", "v", "o", "lse", "B", "Hq", "Hkv", "Lq", "Lk", "d_qk", "d_v", "causal",
         "scale", "stream"]


def _call(**over):
    args = dict(GOOD)
    args.update(over)
    return _binding.library().attn_fwd(*[args[n] for n in ORDER])


def _call_dbg(threshold, exp_mode=0, **over):
    args = dict(GOOD)
    args.update(over)
    return _binding.library().attn_fwd_dbg(*[args[n] for n in ORDER], threshold, exp_mode, None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), "ATTN_ERR_NULL_PTR"),
    (dict(k=None), "ATTN_ERR_NULL_PTR"),
    (dict(v=None), "ATTN_ERR_NULL_PTR"),
    (dict(o=None), "ATTN_ERR_NULL_PTR"),
    (dict(lse=None), "ATTN_ERR_NULL_PTR"),
    (dict(B=0), "ATTN_ERR_BAD_SHAPE"),
    (dict(Hq=0), "ATTN_ERR_BAD_SHAPE"),
    (dict(Hkv=-1), "ATTN_ERR_BAD_SHAPE"),
    (dict(Lq=0), "ATTN_ERR_BAD_SHAPE"),
    (dict(Lk=0), "ATTN_ERR_BAD_SHAPE"),
    (dict(Hq=6, Hkv=4), "ATTN_ERR_GQA_RATIO"),
    (dict(d_qk=96, d_v=96), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(d_qk=128, d_v=64), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(d_qk=192, d_v=192), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(scale=0.0), "ATTN_ERR_BAD_SCALE"),
    (dict(scale=-1.0), "ATTN_ERR_BAD_SCALE"),
    (dict(scale=float("inf")), "ATTN_ERR_BAD_SCALE"),
    (dict(scale=float("nan")), "ATTN_ERR_BAD_SCALE"),
    (dict(q=A + 8), "ATTN_ERR_MISALIGNED"),
    (dict(o=A * 4 + 2), "ATTN_ERR_MISALIGNED"),
    (dict(lse=A * 5 + 2), "ATTN_ERR_MISALIGNED"),
    (dict(B=2 ** 16, Hq=2 ** 8, Hkv=2 ** 8, Lq=2 ** 8), "ATTN_ERR_TOO_LARGE"),
])
def test_argument_errors_come_before_any_device_call(over, code):
    assert _call(**over) == CODES[code]


def test_debug_threshold_is_validated():
    assert _call_dbg(-1.0) == CODES["ATTN_ERR_BAD_ARGUMENT"]
    assert _call_dbg(float("nan")) == CODES["ATTN_ERR_BAD_ARGUMENT"]
    assert _call_dbg(float("inf")) == CODES["ATTN_ERR_BAD_ARGUMENT"]


def test_debug_exp_mode_is_validated():
    # only the hardware exponential (mode 0) is built; every other mode is refused
    for mode in (1, 2, -1, 7):
        assert _call_dbg(8.0, exp_mode=mode) == CODES["ATTN_ERR_BAD_ARGUMENT"]


def test_valid_call_without_a_gpu_reports_no_device():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call() == CODES["ATTN_ERR_NO_DEVICE"]
    assert _call_dbg(8.0) == CODES["ATTN_ERR_NO_DEVICE"]


def test_python_binding_rejects_bad_tensors():
    import torch

    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        _binding.attn_fwd(q, q, q)  # CPU tensors are refused before any call
    with pytest.raises(TypeError):
        _binding.attn_fwd(q.float(), q, q)


def test_binding_refuses_outputs_off_the_input_device():
    """Caller-supplied outputs on another device than the inputs are refused
    before any library call (the kernels would write through a host or foreign
    address).  Without a GPU the rule is checked on the binding's output
    helper, with inputs on the meta device standing in for a GPU."""
    import torch

    q = torch.empty((1, 2, 8, 64), dtype=torch.bfloat16, device="meta")
    good_o = torch.empty((1, 2, 8, 64), dtype=torch.bfloat16, device="meta")
    good_l = torch.empty((1, 2, 8), dtype=torch.float32, device="meta")
    out, lse = _binding._outputs(q, 64, good_o, good_l)
    assert out is good_o and lse is good_l
    with pytest.raises(ValueError, match="out must be on"):
        _binding._outputs(q, 64, torch.empty((1, 2, 8, 64), dtype=torch.bfloat16), good_l)
    with pytest.raises(ValueError, match="lse must be on"):
        _binding._outputs(q, 64, good_o, torch.empty((1, 2, 8), dtype=torch.float32))
    with pytest.raises(TypeError):
        _binding._require_device(None, q.device, "out")
    # merge takes its device from o_part, which must be a GPU tensor
    o_part = torch.zeros((2, 4, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        _binding.attn_merge(o_part, torch.zeros((2, 4), dtype=torch.float32))


def test_noalloc_backward_row_limit_comes_before_any_device_call():
    """attn_bwd_noalloc refuses problems whose D rows exceed its static scratch
    (ATTN_BWD_NOALLOC_MAX_ROWS) before touching a device; a problem at the limit
    passes validation and, without a GPU, stops at the device check."""
    import torch

    lib = _binding.library()
    mx = _binding.BWD_NOALLOC_MAX_ROWS
    header = open(os.path.join(ROOT, "include", "attn_fwd.h"), encoding="utf-8").read()
    assert "#define ATTN_BWD_NOALLOC_MAX_ROWS (4LL << 20)" in header and mx == 4 << 20

    def call(Hq, Lq, lse=A * 5):
        return lib.attn_bwd_noalloc(A, A * 2, A * 3, A * 4, A * 6, lse, A * 7, A * 8, A * 9,
                                    1, Hq, 1, Lq, 64, 128, 128, 0, 0.088, None)

    assert call(64, mx // 64 + 1) == CODES["ATTN_ERR_SCRATCH"]
    assert call(64, mx // 64, lse=None) == CODES["ATTN_ERR_NULL_PTR"]
    if not torch.cuda.is_available():
        assert call(64, mx // 64) == CODES["ATTN_ERR_NO_DEVICE"]


def test_split_keys_arithmetic():
    """W = 64 * ceil(ceil(Lk / 64) / n_split) (host arithmetic, no GPU)."""
    for Lk, n, want in ((2048, 1, 2048), (2048, 4, 512), (2048, 3, 704), (100, 2, 64),
                        (100, 8, 64), (1, 1, 64), (32768, 32, 1024), (5000, 7, 768)):
        assert _binding.split_keys(Lk, n) == want, (Lk, n)
        # the splits cover every key exactly once
        assert n * want >= Lk and (n - 1) * want < Lk or want == 64
    lib = _binding.library()
    assert lib.attn_split_keys(0, 4) == -CODES["ATTN_ERR_BAD_SHAPE"]
    assert lib.attn_split_keys(100, 0) == -CODES["ATTN_ERR_BAD_ARGUMENT"]
    assert lib.attn_split_keys(100, 4097) == -CODES["ATTN_ERR_BAD_ARGUMENT"]


def _call_split(n_split, **over):
    args = dict(GOOD)
    args.update(over)
    a = [args[n] for n in ORDER]
    return _binding.library().attn_fwd_split(*a[:14], n_split, a[14])


def _call_merge(o_part=A, lse_part=A * 2, o=A * 3, lse=A * 4, n_split=4, rows=100, d_v=128):
    return _binding.library().attn_merge(o_part, lse_part, o, lse, n_split, rows, d_v, None)


def test_split_and_merge_arguments_are_validated_first():
    assert _call_split(0) == CODES["ATTN_ERR_BAD_ARGUMENT"]
    assert _call_split(4097) == CODES["ATTN_ERR_BAD_ARGUMENT"]
    assert _call_split(4, q=None) == CODES["ATTN_ERR_NULL_PTR"]
    assert _call_split(4, o=A * 4 + 4) == CODES["ATTN_ERR_MISALIGNED"]
    assert _call_split(4, Hq=6, Hkv=4) == CODES["ATTN_ERR_GQA_RATIO"]
    # split count times rows beyond the 32-bit row range
    assert _call_split(4096, B=2 ** 10, Hq=2 ** 8, Hkv=2 ** 8, Lq=2) == CODES["ATTN_ERR_TOO_LARGE"]
    assert _call_merge(o_part=None) == CODES["ATTN_ERR_NULL_PTR"]
    assert _call_merge(lse=None) == CODES["ATTN_ERR_NULL_PTR"]
    assert _call_merge(n_split=0) == CODES["ATTN_ERR_BAD_ARGUMENT"]
    assert _call_merge(rows=-1) == CODES["ATTN_ERR_BAD_ARGUMENT"]
    assert _call_merge(d_v=96) == CODES["ATTN_ERR_UNSUPPORTED_HEAD_DIM"]
    assert _call_merge(o=A * 3 + 8) == CODES["ATTN_ERR_MISALIGNED"]


def test_valid_split_and_merge_without_a_gpu_report_no_device():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call_split(4) == CODES["ATTN_ERR_NO_DEVICE"]
    assert _call_merge() == CODES["ATTN_ERR_NO_DEVICE"]


# attn_fwd_ex: [B, S, H, d] strides of the GOOD shape (B1 Hq4 Hkv2 L64 d128)
def _bshd(H, L, d):
    return _binding.Strides(L * H * d, d, H * d)


def _call_ex(dtype=0, qs=None, ks=None, vs=None, os_=None, **over):
    args = dict(GOOD)
    args.update(over)
    a = [args[n] for n in ORDER]
    qs = qs or _bshd(args["Hq"], args["Lq"], args["d_qk"])
    ks = ks or _bshd(args["Hkv"], args["Lk"], args["d_qk"])
    vs = vs or _bshd(args["Hkv"], args["Lk"], args["d_v"])
    os_ = os_ or _bshd(args["Hq"], args["Lq"], args["d_v"])
    return _binding.library().attn_fwd_ex(*a[:12], qs, ks, vs, os_, dtype, a[12], a[13], a[14])


def test_strided_entry_point_is_validated_first():
    S = _binding.Strides
    assert _call_ex(dtype=2) == CODES["ATTN_ERR_BAD_ARGUMENT"]
    assert _call_ex(dtype=-1) == CODES["ATTN_ERR_BAD_ARGUMENT"]
    assert _call_ex(q=None) == CODES["ATTN_ERR_NULL_PTR"]
    assert _call_ex(o=A * 4 + 2) == CODES["ATTN_ERR_MISALIGNED"]
    # negative, not a multiple of 8 elements, rows closer than the head dim
    assert _call_ex(qs=S(-4 * 64 * 128, 128, 4 * 128)) == CODES["ATTN_ERR_BAD_STRIDE"]
    assert _call_ex(ks=S(2 * 64 * 128, 132, 2 * 128)) == CODES["ATTN_ERR_BAD_STRIDE"]
    assert _call_ex(vs=S(2 * 64 * 128, 128, 120)) == CODES["ATTN_ERR_BAD_STRIDE"]
    assert _call_ex(os_=S(4 * 64 * 128, 128, 4 * 128 + 4)) == CODES["ATTN_ERR_BAD_STRIDE"]
    # one K head spanning 2^31 bytes or more
    assert _call_ex(ks=S(0, 0, 2 ** 25)) == CODES["ATTN_ERR_TOO_LARGE"]
    # the contiguous [B, H, L, d] strides are accepted like attn_fwd's
    import torch

    if not torch.cuda.is_available():
        bhsd = dict(qs=S(4 * 64 * 128, 64 * 128, 128), ks=S(2 * 64 * 128, 64 * 128, 128),
                    vs=S(2 * 64 * 128, 64 * 128, 128), os_=S(4 * 64 * 128, 64 * 128, 128))
        assert _call_ex(**bhsd) == CODES["ATTN_ERR_NO_DEVICE"]
        assert _call_ex(dtype=1) == CODES["ATTN_ERR_NO_DEVICE"]


def test_python_strided_binding_rejects_bad_tensors():
    import torch

    q = torch.zeros((1, 8, 2, 64), dtype=torch.float16).transpose(1, 2)
    with pytest.raises((ValueError, TypeError)):
        _binding.attn_fwd_ex(q, q, q)  # CPU tensors are refused before any call
    with pytest.raises(TypeError):
        _binding.attn_fwd_ex(q.float(), q, q)


BWD_ORDER = ["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "delta", "B", "Hq", "Hkv",
             "Lq", "Lk", "d_qk", "d_v", "causal", "scale", "stream"]


def _call_bwd(**over):
    args = dict(GOOD, dout=A * 6, dq=A * 7, dk=A * 8, dv=A * 9, delta=A * 10)
    args.update(over)
    return _binding.library().attn_bwd(*[args[n] for n in BWD_ORDER])


@pytest.mark.parametrize("over,code", [
    (dict(dout=None), "ATTN_ERR_NULL_PTR"),
    (dict(dq=None), "ATTN_ERR_NULL_PTR"),
    (dict(dk=None), "ATTN_ERR_NULL_PTR"),
    (dict(dv=None), "ATTN_ERR_NULL_PTR"),
    (dict(delta=None), "ATTN_ERR_NULL_PTR"),
    (dict(q=None), "ATTN_ERR_NULL_PTR"),
    (dict(lse=None), "ATTN_ERR_NULL_PTR"),
    (dict(Lq=0), "ATTN_ERR_BAD_SHAPE"),
    (dict(Hq=6, Hkv=4), "ATTN_ERR_GQA_RATIO"),
    (dict(d_qk=192, d_v=192), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(d_qk=128, d_v=64), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(d_qk=96, d_v=96), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(scale=float("nan")), "ATTN_ERR_BAD_SCALE"),
    (dict(dout=A * 6 + 2), "ATTN_ERR_MISALIGNED"),
    (dict(dq=A * 7 + 8), "ATTN_ERR_MISALIGNED"),
    (dict(delta=A * 10 + 2), "ATTN_ERR_MISALIGNED"),
    (dict(B=2 ** 16, Hq=2 ** 8, Hkv=2 ** 8, Lq=2 ** 8), "ATTN_ERR_TOO_LARGE"),
])
def test_backward_arguments_are_validated_first(over, code):
    assert _call_bwd(**over) == CODES[code]


def test_valid_backward_call_without_a_gpu_reports_no_device():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call_bwd() == CODES["ATTN_ERR_NO_DEVICE"]
    assert _call_bwd(d_qk=64, d_v=64, causal=1) == CODES["ATTN_ERR_NO_DEVICE"]


# --------------------------------------------------------------------------
# Packed variable-length batches: the host planner and the entry point's checks
# --------------------------------------------------------------------------

def _plan_cost(rec, causal, bm_pos):
    q0, lq, k0, lk, unit, m = rec[:6]
    if lq == 0:
        return None  # padding
    kend = lk
    if causal:
        kend = min(lk, min(lq, (m + 1) * bm_pos) - 1 + lk - lq + 1)
    return (max(kend, 0) + 63) // 64 + 2


@pytest.mark.parametrize("lens_q,lens_k,Hq,Hkv,causal", [
    ([7267, 4408, 2434, 1720, 3470, 527, 3413, 5988, 3541], None, 16, 16, True),
    ([5, 0, 300, 1, 1000], [700, 4, 0, 1, 999], 32, 8, True),
    ([129, 257, 64], None, 6, 3, False),
    ([1], [1], 1, 1, False),
])
def test_varlen_plan_covers_every_tile_once(lens_q, lens_k, Hq, Hkv, causal):
    import numpy as np
    lens_k = lens_k or lens_q
    cq = np.concatenate([[0], np.cumsum(lens_q)])
    ck = np.concatenate([[0], np.cumsum(lens_k)])
    plan = _binding.varlen_plan(cq, ck, Hq, Hkv, causal)
    assert plan.shape[1] == 8 and plan.shape[0] % 8 == 0
    G = Hq // Hkv
    Gp = 8 if G % 8 == 0 else 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
    bm_pos = 256 // Gp
    units = Hkv * (G // Gp)
    want = {(int(cq[s]), lq, int(ck[s]), lk, u, m)
            for s, (lq, lk) in enumerate(zip(lens_q, lens_k)) if lq > 0
            for u in range(units) for m in range(-(-lq // bm_pos))}
    got = [tuple(int(x) for x in r[:6]) for r in plan if r[1] > 0]
    assert len(got) == len(set(got)) == len(want) and set(got) == want
    assert all(not r.any() for r in plan if r[1] == 0), "padding records must be all zero"
    # Replay the kernel's order (32 workgroups per XCD; XCD x owns records
    # x, x + 8, ...; round r gives slot s local tile 32 r + s, or 32 r + 31 - s
    # in odd rounds).  Each tile went to the least loaded slot of its XCD, so
    # no slot ends later than the XCD's mean load plus its largest tile.
    loads = []
    for x in range(8):
        recs = plan[x::8]
        assert len(recs) % 32 == 0
        slot = np.zeros(32)
        for r in range(len(recs) // 32):
            for s in range(32):
                c = _plan_cost(recs[32 * r + (31 - s if r & 1 else s)], causal, bm_pos)
                slot[s] += c or 0
        costs = [c for c in (_plan_cost(rec, causal, bm_pos) for rec in recs) if c]
        if costs:
            assert slot.max() <= slot.mean() + max(costs) + 1e-9
        loads.append(slot.sum())
    # and the XCDs' loads are balanced to within one unit of work
    unit_cost = max(sum(_plan_cost((0, lq, 0, lk, 0, m), causal, bm_pos)
                        for m in range(-(-lq // bm_pos))) for lq, lk in zip(lens_q, lens_k) if lq)
    assert max(loads) - min(loads) <= unit_cost


def test_varlen_plan_rejects_bad_offsets():
    lib = _binding.library()
    i32p = ctypes.POINTER(ctypes.c_int)
    n = ctypes.c_int(-1)

    def plan(cq, ck, n_seq, Hq=4, Hkv=2, cap=0, out=None):
        aq = (ctypes.c_int * len(cq))(*cq)
        ak = (ctypes.c_int * len(ck))(*ck)
        return lib.attn_varlen_plan(ctypes.cast(aq, i32p), ctypes.cast(ak, i32p), n_seq, Hq, Hkv,
                                    1, out, cap, ctypes.byref(n))

    assert plan([0, 5], [0, 5], 1) == 0 and n.value == 256  # one round of 8 x 32
    assert plan([1, 5], [0, 5], 1) == CODES["ATTN_ERR_BAD_SHAPE"]     # must start at 0
    assert plan([0, 5, 3], [0, 5, 6], 2) == CODES["ATTN_ERR_BAD_SHAPE"]  # decreasing
    assert plan([0, 5], [0, 5], 0) == CODES["ATTN_ERR_BAD_SHAPE"]
    assert plan([0, 5], [0, 5], 1, Hq=3, Hkv=2) == CODES["ATTN_ERR_GQA_RATIO"]
    small = (ctypes.c_int * 8)()
    assert plan([0, 5], [0, 5], 1, cap=1, out=ctypes.cast(small, i32p)) == \
        CODES["ATTN_ERR_BAD_ARGUMENT"]
    assert lib.attn_varlen_plan(None, None, 1, 1, 1, 0, None, 0, ctypes.byref(n)) == \
        CODES["ATTN_ERR_NULL_PTR"]


VGOOD = dict(q=A, k=A * 2, v=A * 3, o=A * 4, lse=A * 5, plan=A * 6, n_records=8, total_q=100,
             total_k=100, Hq=4, Hkv=2, d_qk=128, d_v=128, causal=1, scale=0.088, stream=None)
VORDER = ["q", "k", "v", "o", "lse", "plan", "n_records", "total_q", "total_k", "Hq", "Hkv",
          "d_qk", "d_v", "causal", "scale", "stream"]


@pytest.mark.parametrize("over,code", [
    ({"plan": None}, "ATTN_ERR_NULL_PTR"),
    ({"q": None}, "ATTN_ERR_NULL_PTR"),
    ({"total_q": 0}, "ATTN_ERR_BAD_SHAPE"),
    ({"total_k": -1}, "ATTN_ERR_BAD_SHAPE"),
    ({"n_records": 12}, "ATTN_ERR_BAD_ARGUMENT"),
    ({"Hq": 3}, "ATTN_ERR_GQA_RATIO"),
    ({"d_qk": 96}, "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    ({"scale": 0.0}, "ATTN_ERR_BAD_SCALE"),
    ({"plan": A * 6 + 4}, "ATTN_ERR_MISALIGNED"),
    ({"total_k": 1 << 22}, "ATTN_ERR_TOO_LARGE"),
])
def test_varlen_arguments_are_validated_first(over, code):
    args = dict(VGOOD)
    args.update(over)
    assert _binding.library().attn_fwd_varlen(*[args[n] for n in VORDER]) == CODES[code]


def test_valid_varlen_call_without_a_gpu_reports_no_device():
    args = [VGOOD[n] for n in VORDER]
    assert _binding.library().attn_fwd_varlen(*args) in (CODES["ATTN_ERR_NO_DEVICE"],
                                                          CODES["ATTN_ERR_UNSUPPORTED_ARCH"])


def test_largest_head_is_accepted_and_one_more_key_is_not():
    """d = 128: a head of 8388607 keys spans 2^31 - 256 bytes, the last size the
    kernel's 32-bit buffer offsets address; 8388608 keys are rejected."""
    ok = _call(B=1, Hq=1, Hkv=1, Lq=64, Lk=(2 ** 31 - 1) // 256)
    assert ok in (CODES["ATTN_ERR_NO_DEVICE"], CODES["ATTN_ERR_UNSUPPORTED_ARCH"])
    assert _call(B=1, Hq=1, Hkv=1, Lq=64, Lk=2 ** 23) == CODES["ATTN_ERR_TOO_LARGE"]


def _call_decode(**over):
    args = dict(GOOD, B=2, Hq=8, Hkv=2, Lq=1, Lk=1000, n_split=4)
    args.update(over)
    order = ["q", "k", "v", "o", "lse", "B", "Hq", "Hkv", "Lq", "Lk", "d_qk", "d_v", "causal",
             "scale", "n_split", "stream"]
    return _binding.library().attn_fwd_decode(*[args[n] for n in order])


@pytest.mark.parametrize("over,code", [
    ({"q": None}, "ATTN_ERR_NULL_PTR"),
    ({"Lq": 0}, "ATTN_ERR_BAD_SHAPE"),
    ({"Hq": 6, "Hkv": 4}, "ATTN_ERR_GQA_RATIO"),
    ({"d_qk": 192, "d_v": 192}, "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    ({"Lq": 5}, "ATTN_ERR_BAD_ARGUMENT"),          # 5 x 4 = 20 rows per K/V head
    ({"Hq": 34, "Hkv": 2}, "ATTN_ERR_BAD_ARGUMENT"),  # 17 rows
    ({"n_split": 0}, "ATTN_ERR_BAD_ARGUMENT"),
    ({"scale": float("nan")}, "ATTN_ERR_BAD_SCALE"),
    ({"Lk": 2 ** 23}, "ATTN_ERR_TOO_LARGE"),
])
def test_decode_arguments_are_validated_first(over, code):
    assert _call_decode(**over) == CODES[code]


def test_valid_decode_call_without_a_gpu_reports_no_device():
    assert _call_decode() in (CODES["ATTN_ERR_NO_DEVICE"], CODES["ATTN_ERR_UNSUPPORTED_ARCH"])
    assert _call_decode(Lq=4) in (CODES["ATTN_ERR_NO_DEVICE"], CODES["ATTN_ERR_UNSUPPORTED_ARCH"])
    assert _call_decode(d_qk=192, d_v=128) in (CODES["ATTN_ERR_NO_DEVICE"],
                                                CODES["ATTN_ERR_UNSUPPORTED_ARCH"])
