"""libflce's C ABI on the host: exported symbols, argument validation, planner.

None of these make a device call: validation happens before any HIP call,
so fake (never dereferenced) pointers are enough.
"""
import ctypes
import os
import re
import subprocess

import pytest

import linear_cross_entropy_04_amd as fl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flce.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fl.lib_path()):
        from linear_cross_entropy_04_amd import build_lib
        build_lib.build()
    return fl._load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flce_\w+)\s*\(", text)))


def test_header_declares_abi():
    names = _declared()
    for n in ("flce_fwd_bwd", "flce_fwd", "flce_plan", "flce_workspace_bytes",
              "flce_status_string", "flce_scale_inplace", "flce_last_error"):
        assert n in names


def test_exports_match_header(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fl.lib_path()], stdout=subprocess.PIPE,
                         text=True, check=True).stdout
    exported = sorted(set(re.findall(r"\bT (flce_\w+)", out)))
    assert exported == _declared()
    for n in _declared():
        assert hasattr(lib, n)


FAKE = ctypes.c_void_p(0x100000)        # 256-aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x100008)


def _fwd_bwd(lib, X=FAKE, W=FAKE, labels=FAKE, N=16, H=64, V=100, dt=fl.FLCE_BF16, chunk=0,
             loss=True, dX=FAKE, dW=FAKE, ws=FAKE, ws_bytes=1 << 40):
    lv = ctypes.c_float(0)
    return lib.flce_fwd_bwd(X, W, labels, N, H, V, dt, -100, chunk,
                            ctypes.byref(lv) if loss else None, dX, dW, None, None, ws,
                            ws_bytes, None)


def test_validation_codes(lib):
    assert _fwd_bwd(lib, dt=7) == fl.FLCE_EINVAL
    assert _fwd_bwd(lib, N=-1) == fl.FLCE_EINVAL
    assert _fwd_bwd(lib, H=0) == fl.FLCE_EINVAL
    assert _fwd_bwd(lib, V=0) == fl.FLCE_EINVAL
    assert _fwd_bwd(lib, loss=False) == fl.FLCE_EINVAL
    assert _fwd_bwd(lib, X=None) == fl.FLCE_EINVAL
    assert _fwd_bwd(lib, W=None) == fl.FLCE_EINVAL
    assert _fwd_bwd(lib, labels=None) == fl.FLCE_EINVAL
    assert _fwd_bwd(lib, dX=None) == fl.FLCE_EINVAL
    assert _fwd_bwd(lib, dW=None) == fl.FLCE_EINVAL
    assert _fwd_bwd(lib, ws=None) == fl.FLCE_EINVAL
    assert _fwd_bwd(lib, ws=FAKE_ODD) == fl.FLCE_EINVAL
    assert _fwd_bwd(lib, H=12) == fl.FLCE_EUNSUPPORTED            # bf16 needs H % 8 == 0
    assert _fwd_bwd(lib, X=FAKE_ODD) == fl.FLCE_EUNSUPPORTED      # bf16 needs 16-byte rows
    assert _fwd_bwd(lib, V=9_000_000) == fl.FLCE_EUNSUPPORTED
    need = fl.flce_workspace_bytes(16, 64, 100, fl.FLCE_BF16, 0)
    assert _fwd_bwd(lib, ws_bytes=need - 1) == fl.FLCE_EWORKSPACE
    # fp32 accepts any H
    need32 = fl.flce_workspace_bytes(16, 12, 100, fl.FLCE_F32, 0)
    assert need32 > 0
    assert _fwd_bwd(lib, H=12, dt=fl.FLCE_F32, ws_bytes=need32 - 1) == fl.FLCE_EWORKSPACE


def test_fwd_validation(lib):
    lv = ctypes.c_float(0)
    st = lib.flce_fwd(FAKE, FAKE, FAKE, 16, 64, 100, fl.FLCE_BF16, -100, 0, ctypes.byref(lv),
                      None, None, FAKE, 10, None)
    assert st == fl.FLCE_EWORKSPACE
    st = lib.flce_fwd(FAKE, FAKE, FAKE, 16, 64, 100, 3, -100, 0, ctypes.byref(lv), None, None,
                      FAKE, 1 << 40, None)
    assert st == fl.FLCE_EINVAL


def _orpo(lib, X=FAKE, W=FAKE, labels=FAKE, B=2, T=8, H=64, V=100, dt=fl.FLCE_BF16,
          chunk_pairs=1, loss=True, dX=FAKE, dW=FAKE, ws=FAKE, ws_bytes=1 << 40):
    lv = ctypes.c_float(0)
    return lib.flce_orpo_fwd_bwd(X, W, labels, B, T, H, V, dt, -100, 0.1, chunk_pairs,
                                 ctypes.byref(lv) if loss else None, None, dX, dW, None, None,
                                 None, ws, ws_bytes, None)


def test_orpo_validation(lib):
    assert _orpo(lib, B=0) == fl.FLCE_EINVAL
    assert _orpo(lib, T=0) == fl.FLCE_EINVAL
    assert _orpo(lib, dt=5) == fl.FLCE_EINVAL
    assert _orpo(lib, loss=False) == fl.FLCE_EINVAL
    assert _orpo(lib, X=None) == fl.FLCE_EINVAL
    assert _orpo(lib, dX=None) == fl.FLCE_EINVAL
    assert _orpo(lib, ws=FAKE_ODD) == fl.FLCE_EINVAL
    assert _orpo(lib, H=12) == fl.FLCE_EUNSUPPORTED              # bf16 needs H % 8 == 0
    assert _orpo(lib, X=FAKE_ODD) == fl.FLCE_EUNSUPPORTED
    need = fl.flce_orpo_workspace_bytes(2, 8, 64, 100, fl.FLCE_BF16, 1)
    assert need > 0
    assert _orpo(lib, ws_bytes=need - 1) == fl.FLCE_EWORKSPACE
    assert fl.flce_orpo_workspace_bytes(0, 8, 64, 100, fl.FLCE_BF16, 1) == 0
    # a chunk holds whole pairs: more pairs per chunk, more scratch; auto stops at 4096 rows
    sizes = [fl.flce_orpo_workspace_bytes(8, 512, 4096, 128256, fl.FLCE_BF16, k)
             for k in (1, 2, 4)]
    assert sizes[0] < sizes[1] < sizes[2]
    assert fl.flce_orpo_workspace_bytes(8, 512, 4096, 128256, fl.FLCE_BF16, 0) == sizes[2]


def test_pair_validation(lib):
    lv, nv = ctypes.c_float(0), ctypes.c_float(0)

    def call(kind, ref=FAKE):
        return lib.flce_pair_fwd_bwd(kind, FAKE, FAKE, FAKE, 2, 8, 64, 100, fl.FLCE_BF16, -100,
                                     0.1, 0.0, 0.0, ref, ref, 1, ctypes.byref(lv),
                                     ctypes.byref(nv), FAKE, FAKE, None, None, None, FAKE, 10,
                                     None)
    assert call(4) == fl.FLCE_EINVAL                       # unknown kind
    assert call(-1) == fl.FLCE_EINVAL
    assert call(fl.PAIR_KINDS["dpo"], ref=None) == fl.FLCE_EINVAL     # DPO needs references
    for k in ("orpo", "simpo", "cpo", "dpo"):              # valid: stops at the small workspace
        assert call(fl.PAIR_KINDS[k]) == fl.FLCE_EWORKSPACE
    assert fl.flce_pair_workspace_bytes(2, 8, 64, 100, fl.FLCE_BF16, 1) == \
        fl.flce_orpo_workspace_bytes(2, 8, 64, 100, fl.FLCE_BF16, 1)


def test_scale_validation(lib):
    assert lib.flce_scale_inplace(FAKE, 10, 5, FAKE, None) == fl.FLCE_EINVAL
    assert lib.flce_scale_inplace(FAKE, -1, 0, FAKE, None) == fl.FLCE_EINVAL
    assert lib.flce_scale_inplace(FAKE, 10, 0, None, None) == fl.FLCE_EINVAL


def test_kernel_classes_match_the_header(lib):
    # the binding's count of kernel classes is the header's FLCE_K_COUNT
    names = [lib.flce_kernel_name(k).decode() for k in range(fl.KERNEL_CLASSES)]
    assert all(names) and len(set(names)) == len(names)
    assert lib.flce_kernel_name(fl.KERNEL_CLASSES).decode() == ""


def test_profile_select(lib):
    # host only: the class mask is stored; the binding maps names to bits
    assert lib.flce_profile_select(ctypes.c_uint32(1 << 6)) == fl.FLCE_OK
    fl.flce_profile_select(["dw_gemm", "fwd_tile"])
    fl.flce_profile_select([0, 11])
    with pytest.raises(KeyError):
        fl.flce_profile_select(["no such kernel"])
    with pytest.raises(ValueError):
        fl.flce_profile_select([fl.KERNEL_CLASSES])
    fl.flce_profile_select(None)                      # every class again


def test_status_strings(lib):
    for s in range(6):
        assert fl.flce_status_string(s) and fl.flce_status_string(s) != "unknown status"
    assert fl.flce_status_string(99) == "unknown status"
    assert fl.flce_last_error() == ""


def test_workspace_bounded_by_chunk_not_N():
    # Llama-3-8B head, long context: scratch grows with the chunk, not with N.
    H, V = 4096, 128256
    a = fl.flce_workspace_bytes(16384, H, V, fl.FLCE_BF16, 1024)
    b = fl.flce_workspace_bytes(16384 * 4, H, V, fl.FLCE_BF16, 1024)
    assert b - a == pytest.approx(16384 * 3 * 4, abs=512)     # only the per-token loss array grows
    sizes = [fl.flce_workspace_bytes(16384, H, V, fl.FLCE_BF16, c) for c in (512, 1024, 4096)]
    assert sizes[0] < sizes[1] < sizes[2]
    for c, s in zip((512, 1024, 4096), sizes):
        assert s >= c * V * 2                       # the bf16 logits chunk (W is read in place)
        # plus the packed X chunk, log-sum-exp partials (3 fp32 per token and
        # 128 vocabulary ids) and at most 32 fp32 split-K partial sums of dX
        assert s < c * V * 2 + c * V // 128 * 12 + c * H * (2 + 4 * 32) + 16384 * 4 + (1 << 20)
    # at chunk 1024 the whole workspace is below the bf16 logits of the batch
    assert fl.flce_workspace_bytes(8192, H, V, fl.FLCE_BF16, 1024) < 8192 * V * 2


def _largest_fitting_chunk(N, H, V, budget):
    """The rule flce_plan states: the largest power-of-two multiple of 256
    tokens (at most N) whose whole workspace fits the budget."""
    best, c = None, 256
    while True:
        cc = min(c, N)
        if fl.flce_workspace_bytes(N, H, V, fl.FLCE_BF16, cc) > budget:
            return best
        best = cc
        if c >= N:
            return best
        c *= 2


def test_plan_default_budget_keeps_scratch_below_the_logits():
    # chunk 0 on the Llama-3-8B head: several chunks, and less scratch than N x V bf16 logits
    N, H, V = 8192, 4096, 128256
    st, c, peak = fl.flce_plan(N, H, V, fl.FLCE_BF16)
    assert st == fl.FLCE_OK and c < N and peak < N * V * 2
    # the default budget is W's bytes (at least 256 MiB); the plan is its largest fit
    assert c == _largest_fitting_chunk(N, H, V, H * V * 2)
    assert peak == fl.flce_workspace_bytes(N, H, V, fl.FLCE_BF16, 0) <= H * V * 2
    # a tiny head gets the floor
    st, c, peak = fl.flce_plan(100000, 64, 1000, fl.FLCE_BF16)
    assert st == fl.FLCE_OK and peak <= 256 << 20
    assert c == _largest_fitting_chunk(100000, 64, 1000, 256 << 20)


def test_plan_auto_and_explicit():
    st, c, peak = fl.flce_plan(8192, 2304, 256000, fl.FLCE_BF16)      # large-vocabulary head
    assert st == fl.FLCE_OK and c == _largest_fitting_chunk(8192, 2304, 256000, 2304 * 256000 * 2)
    assert peak == fl.flce_workspace_bytes(8192, 2304, 256000, fl.FLCE_BF16, 0)
    st, c, peak = fl.flce_plan(8192, 4096, 128256, fl.FLCE_BF16, chunk_tokens=1024)
    assert st == fl.FLCE_OK and c == 1024
    assert peak == fl.flce_workspace_bytes(8192, 4096, 128256, fl.FLCE_BF16, 1024)
    st, c, _ = fl.flce_plan(100, 64, 1000, fl.FLCE_BF16, chunk_tokens=5000)
    assert st == fl.FLCE_OK and c == 100                                  # clamped to N
    st, c, _ = fl.flce_plan(100, 64, 1000, fl.FLCE_BF16)
    assert st == fl.FLCE_OK and c == 100
    # the budget bounds the whole workspace: 256 tokens of bf16 logits alone exceed 64 MiB here
    st, c, peak = fl.flce_plan(8192, 4096, 128256, fl.FLCE_BF16, scratch_budget_bytes=64 << 20)
    assert st == fl.FLCE_EWORKSPACE and c == 256 and peak > 64 << 20   # smallest chunk reported
    for budget in (200 << 20, 300 << 20, 700 << 20, 1200 << 20, 3000 << 20):
        st, c, peak = fl.flce_plan(8192, 4096, 128256, fl.FLCE_BF16, scratch_budget_bytes=budget)
        assert st == fl.FLCE_OK and c == _largest_fitting_chunk(8192, 4096, 128256, budget)
        assert peak <= budget
        if c < 8192:       # the next chunk up does not fit
            assert fl.flce_workspace_bytes(8192, 4096, 128256, fl.FLCE_BF16, 2 * c) > budget
    # an explicit chunk beyond an explicit budget is reported, not changed
    st, c, peak = fl.flce_plan(8192, 4096, 128256, fl.FLCE_BF16, chunk_tokens=4096,
                               scratch_budget_bytes=1000 << 20)
    assert st == fl.FLCE_EWORKSPACE and c == 4096 and peak > 1000 << 20
    st, c, peak = fl.flce_plan(0, 64, 100, fl.FLCE_BF16)
    assert st == fl.FLCE_OK and c == 0 and peak > 0
    # chunks stop at 2^23 tokens
    st, c, _ = fl.flce_plan((1 << 31) - 1, 8, 1, fl.FLCE_BF16, chunk_tokens=1 << 30)
    assert st == fl.FLCE_OK and c == 1 << 23
    st, c, _ = fl.flce_plan((1 << 31) - 1, 8, 1, fl.FLCE_BF16, scratch_budget_bytes=1 << 50)
    assert st == fl.FLCE_OK and c == 1 << 23


def test_limits_refused_one_past():
    # N_valid is counted in 32 bits
    assert fl.flce_plan((1 << 31) - 1, 8, 1, fl.FLCE_BF16, chunk_tokens=1024)[0] == fl.FLCE_OK
    assert fl.flce_plan(1 << 31, 8, 1, fl.FLCE_BF16, chunk_tokens=1024)[0] == fl.FLCE_EUNSUPPORTED
    assert fl.flce_workspace_bytes(1 << 31, 8, 1, fl.FLCE_BF16, 1024) == 0
    # V and H each within their limits, but dW's grid (V/256 x H/128 workgroups of 256)
    # would pass 2^32 work-items: refused by the planner and by the call
    st, c, _ = fl.flce_plan(1024, 1 << 20, 8000000, fl.FLCE_BF16, chunk_tokens=1024)
    assert st == fl.FLCE_EUNSUPPORTED
    assert fl.flce_plan(1024, 1 << 20, 4096, fl.FLCE_BF16, chunk_tokens=1024)[0] == fl.FLCE_OK
    assert fl.flce_plan(1024, 4096, 8000000, fl.FLCE_BF16, chunk_tokens=1024)[0] == fl.FLCE_OK


def test_fwd_bwd_refuses_oversized_grids(lib):
    assert _fwd_bwd(lib, N=1024, H=1 << 20, V=8000000, chunk=1024) == fl.FLCE_EUNSUPPORTED


def test_ce_row_limit(lib):
    lv = ctypes.c_float(0)
    max_rows = ((1 << 32) - 1) // 1024          # one workgroup of 1024 work-items per row
    for n, want in ((max_rows, fl.FLCE_EWORKSPACE), (max_rows + 1, fl.FLCE_EUNSUPPORTED)):
        st = lib.flce_ce_fwd_bwd(FAKE, FAKE, n, 8, fl.FLCE_BF16, -100, 0, None,
                                 ctypes.byref(lv), None, None, None, FAKE, 10, None)
        assert st == want


def test_kto_reference_point_validation(lib):
    z = ctypes.c_float(-1.0)

    def call(ref=FAKE, ws_bytes=10, n_seq=2, T=8):
        return lib.flce_kto_reference_point(FAKE, FAKE, FAKE, n_seq, T, 64, 100, fl.FLCE_BF16, -100,
                                            ref, 1, ctypes.byref(z), None, None, FAKE, ws_bytes,
                                            None)
    assert call(ref=None) == fl.FLCE_EINVAL              # the reference sums are required
    assert call(n_seq=0) == fl.FLCE_EINVAL
    assert call() == fl.FLCE_EWORKSPACE                   # valid: stops at the small workspace
    assert z.value == -1.0                                # untouched
    ws = fl.flce_kto_workspace_bytes(2, 8, 64, 100, fl.FLCE_BF16, 1)
    assert ws > 0 and call(ws_bytes=ws - 1) == fl.FLCE_EWORKSPACE


def test_binding_has_no_cpu_fallback():
    import torch
    X = torch.zeros(4, 8, dtype=torch.bfloat16)
    W = torch.zeros(16, 8, dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError):
        fl.flce_fwd(X, W, y, -100, 0, torch.zeros(1024, dtype=torch.uint8))
