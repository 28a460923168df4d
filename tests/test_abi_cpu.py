"""The C-ABI library without a GPU: it loads, exports every declared symbol,
its pure host functions agree bit for bit with the oracle, and invalid
arguments are rejected with the documented status before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

from long_context_causal_amd import build as cbuild
from long_context_causal_amd import cpattn as C
from oracle import cp as ocp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built_library():
    cbuild.ensure_built()
    yield


def _declared_functions():
    text = ""
    for name in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if name.endswith(".h"):
            with open(os.path.join(ROOT, "include", name)) as f:
                text += f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cpattn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 8
    lib = ctypes.CDLL(C.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    for st in range(7):
        assert C.cpattn_status_str(st).startswith("CPATTN_")
    assert "UNKNOWN" in C.cpattn_status_str(99)


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8, 16])
def test_step_mode_matches_oracle(cp):
    for r in range(cp):
        for i in range(cp):
            assert C.cpattn_step_mode(i, r, cp) == ocp.step_schedule(i, r, cp)


def test_step_mode_rejects():
    for args in [(0, 0, 0), (2, 0, 2), (0, 2, 2), (-1, 0, 2)]:
        with pytest.raises(C.CpattnError) as e:
            C.cpattn_step_mode(*args)
        assert e.value.status == C.CPATTN_EINVAL
    assert C.lib().cpattn_step_mode(0, 0, 1, None, None) == C.CPATTN_EINVAL


@pytest.mark.parametrize("s,cp", [(8, 2), (16, 4), (512, 2), (32768, 8), (131072, 16),
                                  (96, 6)])
def test_positions_bit_exact_vs_oracle(s, cp):
    for r in range(cp):
        got = C.cpattn_partition_positions(s, cp, r)
        assert got.dtype == np.int32
        assert np.array_equal(got, ocp.zigzag_positions(s, cp, r))


def test_positions_rejects():
    buf = (ctypes.c_int32 * 16)()
    L = C.lib()
    assert L.cpattn_partition_positions(10, 3, 0, buf) == C.CPATTN_ESHAPE
    assert L.cpattn_partition_positions(8, 2, 2, buf) == C.CPATTN_EINVAL
    assert L.cpattn_partition_positions(8, 2, 0, None) == C.CPATTN_EINVAL


def _dims(**kw):
    base = dict(b=1, s=512, hq=4, hkv=4, d=64, cp=2)
    base.update(kw)
    return C.make_dims(**base)


ALIGNED = 1 << 20          # never dereferenced: validation fails first


def _step(dims, dtype=C.CPATTN_F32, mode=C.CPATTN_CAUSAL, ptrs=None, scale=0.0):
    p = ptrs or [ALIGNED] * 5
    return C.lib().cpattn_step_fwd(ctypes.byref(dims), dtype, scale, mode, *p, 0)


def test_step_fwd_validation_before_launch():
    assert _step(_dims(s=510)) == C.CPATTN_ESHAPE                 # s % 2cp
    assert _step(_dims(hq=6, hkv=4)) == C.CPATTN_ESHAPE           # hq % hkv
    assert _step(_dims(d=96)) == C.CPATTN_ESHAPE                  # head dim
    assert _step(_dims(b=0)) == C.CPATTN_ESHAPE
    assert _step(_dims(), dtype=7) == C.CPATTN_EDTYPE
    assert _step(_dims(), mode=3) == C.CPATTN_EINVAL
    assert _step(_dims(), ptrs=[0, ALIGNED, ALIGNED, ALIGNED, ALIGNED]) == C.CPATTN_EINVAL
    assert _step(_dims(), ptrs=[ALIGNED + 2] + [ALIGNED] * 4) == C.CPATTN_EALIGN
    assert _step(_dims(), scale=float("nan")) == C.CPATTN_EINVAL
    assert C.lib().cpattn_step_fwd(None, 0, 0.0, 0, *([ALIGNED] * 5), 0) == C.CPATTN_EINVAL


def test_partition_validation_before_launch():
    L = C.lib()
    d = _dims()
    rope_bad = C.cpattn_rope(0.0)
    assert L.cpattn_partition(ctypes.byref(_dims(s=510)), 0, 4, ALIGNED, ALIGNED, None, None,
                              0) == C.CPATTN_ESHAPE
    assert L.cpattn_partition(ctypes.byref(d), 5, 4, ALIGNED, ALIGNED, None, None,
                              0) == C.CPATTN_EDTYPE
    assert L.cpattn_partition(ctypes.byref(d), 0, 4, None, ALIGNED, None, None,
                              0) == C.CPATTN_EINVAL
    assert L.cpattn_partition(ctypes.byref(d), 0, 4, ALIGNED + 8, ALIGNED, None, None,
                              0) == C.CPATTN_EALIGN
    assert L.cpattn_partition(ctypes.byref(d), 0, 0, ALIGNED, ALIGNED, None, None,
                              0) == C.CPATTN_ESHAPE
    assert L.cpattn_partition(ctypes.byref(d), 0, 4, ALIGNED, ALIGNED, None,
                              ctypes.byref(rope_bad), 0) == C.CPATTN_EINVAL


def test_merge_validation_before_launch():
    L = C.lib()
    d = _dims()
    two_c = 512 // 2
    good = (C.cpattn_partial * 2)(C.cpattn_partial(ALIGNED, ALIGNED, 0, two_c),
                                  C.cpattn_partial(ALIGNED, ALIGNED, 128, 128))
    bad_rows = (C.cpattn_partial * 1)(C.cpattn_partial(ALIGNED, ALIGNED, 200, 100))
    assert L.cpattn_merge(ctypes.byref(d), 0, good, 0, ALIGNED, None, 0) == C.CPATTN_ESHAPE
    many = (C.cpattn_partial * 65)(*([C.cpattn_partial(ALIGNED, ALIGNED, 0, two_c)] * 65))
    # more than one pass: the running result needs an fp32 O and an L
    assert L.cpattn_merge(ctypes.byref(d), 65, many, 0, ALIGNED, None, 0) == C.CPATTN_ESHAPE
    assert L.cpattn_merge(ctypes.byref(d), 65, many, 1, ALIGNED, ALIGNED, 0) == C.CPATTN_ESHAPE
    assert L.cpattn_merge(ctypes.byref(d), 1, bad_rows, 0, ALIGNED, None, 0) == C.CPATTN_ESHAPE
    assert L.cpattn_merge(ctypes.byref(d), 2, good, 9, ALIGNED, None, 0) == C.CPATTN_EDTYPE
    assert L.cpattn_merge(ctypes.byref(d), 2, good, 0, None, None, 0) == C.CPATTN_EINVAL
    assert L.cpattn_merge(ctypes.byref(d), 2, good, 0, ALIGNED + 4, None, 0) == C.CPATTN_EALIGN
    assert L.cpattn_merge(ctypes.byref(d), 65, many, 0, ALIGNED, ALIGNED + 2, 0) == C.CPATTN_EALIGN


def test_forward_workspace_and_validation():
    L = C.lib()
    d = _dims(b=1, s=32768, hq=64, hkv=8, d=128, cp=8)
    ws = C.cpattn_forward_workspace(d, 3)
    c = 32768 // 16
    # 4 steps of 2c rows (causal + 3 kv_first_half) and 4 of c rows
    want = 4 * (2 * c * 64 * 128 * 4 + 64 * 2 * c * 4) + 4 * (c * 64 * 128 * 4 + 64 * c * 4)
    assert ws == want
    assert C.cpattn_forward_workspace(d, 8) == 0
    args = [ctypes.byref(d), C.CPATTN_BF16, ctypes.c_float(0.0), 3, ALIGNED, ALIGNED, ALIGNED,
            ALIGNED, ws - 1, C.CPATTN_F32, ALIGNED, None, 0]
    assert L.cpattn_forward(*args) == C.CPATTN_ENOSPACE
    args[8] = ws
    args[7] = ALIGNED + 16                         # workspace must be 256-aligned
    assert L.cpattn_forward(*args) == C.CPATTN_EALIGN
    args[7] = ALIGNED
    args[3] = 8
    assert L.cpattn_forward(*args) == C.CPATTN_EINVAL


@pytest.mark.parametrize("cp,rank", [(8, 3), (8, 0), (1, 0), (128, 77), (256, 255)])
def test_forward_partials_layout(cp, rank):
    """cpattn_forward_partials: step order, O then L per step, 256-byte
    regions, the rows of each step's mode; for cp above one merge pass the
    workspace also holds the running fp32 O and L of the 2c rows."""
    b, s, hq, hkv, d = 1, 32768, 4, 2, 128
    dims = _dims(b=b, s=s, hq=hq, hkv=hkv, d=d, cp=cp)
    c = s // (2 * cp)
    ws_bytes = C.cpattn_forward_workspace(dims, rank)
    parts = C.cpattn_forward_partials(dims, rank, ALIGNED, ws_bytes)
    assert len(parts) == cp
    r256 = lambda x: (x + 255) // 256 * 256
    off = 0
    for i, (o, lse, row0, rows) in enumerate(parts):
        mode, _ = ocp.step_schedule(i, rank, cp)
        want_rows = c if mode == ocp.Q_SECOND_HALF else 2 * c
        assert (row0, rows) == ((c, c) if mode == ocp.Q_SECOND_HALF else (0, 2 * c))
        assert rows == want_rows
        assert o == ALIGNED + off
        off += r256(b * rows * hq * d * 4)
        assert lse == ALIGNED + off
        off += r256(b * hq * rows * 4)
    running = r256(b * 2 * c * hq * d * 4) + r256(b * hq * 2 * c * 4) if cp > 64 else 0
    assert ws_bytes == off + running
    with pytest.raises(C.CpattnError) as e:
        C.cpattn_forward_partials(dims, rank, ALIGNED, ws_bytes - 1)
    assert e.value.status == C.CPATTN_ENOSPACE
    with pytest.raises(C.CpattnError) as e:
        C.cpattn_forward_partials(dims, rank, ALIGNED + 16, ws_bytes)
    assert e.value.status == C.CPATTN_EALIGN
    with pytest.raises(C.CpattnError) as e:
        C.cpattn_forward_partials(dims, cp, ALIGNED, ws_bytes)
    assert e.value.status == C.CPATTN_EINVAL


def test_backward_grids_past_32_bits_rejected():
    """A share whose backward would need more than 2^31-1 workgroups is
    refused before any launch (here 2^23 query tiles x 512 heads)."""
    L = C.lib()
    d = _dims(b=1, s=1 << 30, hq=512, hkv=512, d=128, cp=1)
    args = [ctypes.byref(d), C.CPATTN_BF16, ctypes.c_float(0.0), 0] + [ALIGNED] * 11 + [0]
    assert L.cpattn_backward(*args) == C.CPATTN_ESHAPE
    sargs = [ctypes.byref(d), C.CPATTN_BF16, ctypes.c_float(0.0), C.CPATTN_CAUSAL] + \
        [ALIGNED] * 10 + [0]
    assert L.cpattn_step_bwd(*sargs) == C.CPATTN_ESHAPE
    d2 = _dims(b=1, s=1 << 30, hq=8192, hkv=8, d=128, cp=1)
    assert L.cpattn_bwd_delta(ctypes.byref(d2), ALIGNED, ALIGNED, ALIGNED, 0) == C.CPATTN_ESHAPE


def test_backward_head_dims():
    """The bf16 backward entry points take d = 64 and 128 (here: validation
    passes the shape and stops at a NULL pointer) and refuse other d."""
    L = C.lib()
    for d_ok, want in ((64, C.CPATTN_EINVAL), (96, C.CPATTN_ESHAPE)):
        d = _dims(b=1, s=4096, hq=8, hkv=2, d=d_ok, cp=4)
        args = [ctypes.byref(d), C.CPATTN_BF16, ctypes.c_float(0.0), 0, None] + \
            [ALIGNED] * 9 + [0]
        assert L.cpattn_backward(*args) == want
        sargs = [ctypes.byref(d), C.CPATTN_BF16, ctypes.c_float(0.0), C.CPATTN_CAUSAL, None] + \
            [ALIGNED] * 8 + [0]
        assert L.cpattn_step_bwd(*sargs) == want
        assert L.cpattn_bwd_delta(ctypes.byref(d), None, ALIGNED, ALIGNED, 0) == want


def test_forward_steps_validation():
    L = C.lib()
    d = _dims(b=1, s=32768, hq=64, hkv=8, d=128, cp=8)
    ws = C.cpattn_forward_workspace(d, 3)
    args = [ctypes.byref(d), C.CPATTN_BF16, ctypes.c_float(0.0), 3, ALIGNED, ALIGNED, ALIGNED,
            ALIGNED, ws - 1, 0]
    assert L.cpattn_forward_steps(*args) == C.CPATTN_ENOSPACE
    args[8] = ws
    args[7] = ALIGNED + 16
    assert L.cpattn_forward_steps(*args) == C.CPATTN_EALIGN
    args[7] = ALIGNED
    args[4] = ALIGNED + 8                          # Q block not 16-byte aligned
    assert L.cpattn_forward_steps(*args) == C.CPATTN_EALIGN
    args[4] = ALIGNED
    args[3] = -1
    assert L.cpattn_forward_steps(*args) == C.CPATTN_EINVAL
    args[3] = 3
    args[2] = ctypes.c_float(float("nan"))
    assert L.cpattn_forward_steps(*args) == C.CPATTN_EINVAL
    args[2] = ctypes.c_float(0.0)
    args[1] = 7
    assert L.cpattn_forward_steps(*args) == C.CPATTN_EDTYPE
    args[1] = C.CPATTN_BF16
    args[6] = None
    assert L.cpattn_forward_steps(*args) == C.CPATTN_EINVAL


def test_binding_names_match_header():
    for name in _declared_functions():
        assert hasattr(C, name), name


def test_forward_fused_validation_before_launch():
    L = C.lib()
    d = _dims(b=1, s=32768, hq=64, hkv=8, d=128, cp=8)
    args = [ctypes.byref(d), C.CPATTN_BF16, ctypes.c_float(0.0), 3, ALIGNED, ALIGNED, ALIGNED,
            C.CPATTN_F32, ALIGNED, None, 0]
    bad_dtype = list(args)
    bad_dtype[1] = C.CPATTN_F32                    # the fused form is bf16 only
    assert L.cpattn_forward_fused(*bad_dtype) == C.CPATTN_EDTYPE
    bad_out = list(args)
    bad_out[7] = 9
    assert L.cpattn_forward_fused(*bad_out) == C.CPATTN_EDTYPE
    bad_rank = list(args)
    bad_rank[3] = 8
    assert L.cpattn_forward_fused(*bad_rank) == C.CPATTN_EINVAL
    bad_align = list(args)
    bad_align[8] = ALIGNED + 8
    assert L.cpattn_forward_fused(*bad_align) == C.CPATTN_EALIGN
    null_q = list(args)
    null_q[4] = None
    assert L.cpattn_forward_fused(*null_q) == C.CPATTN_EINVAL
    d96 = _dims(b=1, s=32768, hq=64, hkv=8, d=96, cp=8)
    bad_d = list(args)
    bad_d[0] = ctypes.byref(d96)
    assert L.cpattn_forward_fused(*bad_d) == C.CPATTN_ESHAPE
    bad_s = _dims(b=1, s=1000, hq=64, hkv=8, d=128, cp=8)   # s % 2cp != 0
    bad_shape = list(args)
    bad_shape[0] = ctypes.byref(bad_s)
    assert L.cpattn_forward_fused(*bad_shape) == C.CPATTN_ESHAPE


# --- packed variable-length samples ---------------------------------------

from oracle import varlen as ovl  # noqa: E402


@pytest.mark.parametrize("cu,cp", [([0, 8, 24, 32], 2), ([0, 6, 12, 30], 3),
                                   ([0, 16, 32, 48, 64, 128], 8), ([0, 32768], 8),
                                   ([0, 4096, 6144, 32768], 8)])
def test_positions_varlen_bit_exact_vs_oracle(cu, cp):
    s = cu[-1]
    for r in range(cp):
        got = C.cpattn_partition_positions_varlen(s, cp, r, cu)
        assert got.dtype == np.int32
        assert np.array_equal(got, ovl.local_positions(cu, cp, r))
    # no offsets: the unpacked positions
    out = np.empty(s // cp, dtype=np.int32)
    assert C.lib().cpattn_partition_positions_varlen(
        s, cp, 0, None, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))) == C.CPATTN_OK
    assert np.array_equal(out, ocp.zigzag_positions(s, cp, 0))


def _vl_status(cu, s=32, cp=2, nseq=None):
    vl, keep = C.make_varlen(cu)
    if nseq is not None:
        vl.nseq = nseq
    out = np.empty(s // cp, dtype=np.int32)
    st = C.lib().cpattn_partition_positions_varlen(
        s, cp, 0, ctypes.byref(vl), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    del keep
    return st


def test_varlen_offsets_rejected():
    assert _vl_status([0, 8, 32]) == C.CPATTN_OK
    assert _vl_status([0, 6, 32]) == C.CPATTN_ESHAPE        # 6 % 2cp
    assert _vl_status([0, 8, 8, 32]) == C.CPATTN_ESHAPE     # empty sample
    assert _vl_status([4, 8, 32]) == C.CPATTN_ESHAPE        # not from 0
    assert _vl_status([0, 8, 28]) == C.CPATTN_ESHAPE        # not to s
    assert _vl_status([0, 8, 32], nseq=0) == C.CPATTN_ESHAPE
    many = list(range(0, 4 * 130, 4))
    assert _vl_status(many, s=many[-1], nseq=129) == C.CPATTN_ESHAPE   # > CPATTN_MAX_SEQS
    null_cu = C.cpattn_varlen(2, None)
    out = np.empty(16, dtype=np.int32)
    assert C.lib().cpattn_partition_positions_varlen(
        32, 2, 0, ctypes.byref(null_cu),
        out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))) == C.CPATTN_EINVAL


def test_varlen_device_calls_validate_before_launch():
    L = C.lib()
    d = _dims(b=1, s=4096, hq=8, hkv=2, d=128, cp=4)
    bad, keep = C.make_varlen([0, 100, 4096])                # 100 % 8 != 0
    good, keep2 = C.make_varlen([0, 1024, 4096])
    assert L.cpattn_partition_varlen(ctypes.byref(d), 1, 8, ctypes.byref(bad), ALIGNED,
                                     ALIGNED, None, None, 0) == C.CPATTN_ESHAPE
    assert L.cpattn_partition_varlen(ctypes.byref(d), 1, 8, ctypes.byref(good), ALIGNED + 8,
                                     ALIGNED, None, None, 0) == C.CPATTN_EALIGN
    args = [ctypes.byref(d), C.CPATTN_BF16, ctypes.c_float(0.0), 1, ctypes.byref(bad), ALIGNED,
            ALIGNED, ALIGNED, C.CPATTN_F32, ALIGNED, None, 0]
    assert L.cpattn_forward_fused_varlen(*args) == C.CPATTN_ESHAPE
    args[4] = ctypes.byref(good)
    args[1] = C.CPATTN_F32
    assert L.cpattn_forward_fused_varlen(*args) == C.CPATTN_EDTYPE
    args[1] = C.CPATTN_BF16
    args[3] = 4                                               # rank out of range
    assert L.cpattn_forward_fused_varlen(*args) == C.CPATTN_EINVAL
    del keep, keep2


def test_backward_varlen_validates_before_launch():
    L = C.lib()
    d = _dims(b=1, s=4096, hq=8, hkv=2, d=128, cp=4)
    bad, keep = C.make_varlen([0, 100, 4096])
    good, keep2 = C.make_varlen([0, 1024, 4096])
    args = [ctypes.byref(d), C.CPATTN_BF16, ctypes.c_float(0.0), 1, ctypes.byref(bad)] + \
        [ALIGNED] * 10 + [0]
    assert L.cpattn_backward_varlen(*args) == C.CPATTN_ESHAPE
    args[4] = ctypes.byref(good)
    args[3] = 4                                               # rank out of range
    assert L.cpattn_backward_varlen(*args) == C.CPATTN_EINVAL
    args[3] = 1
    args[2] = ctypes.c_float(float("nan"))
    assert L.cpattn_backward_varlen(*args) == C.CPATTN_EINVAL
    args[2] = ctypes.c_float(0.0)
    args[1] = C.CPATTN_F32
    assert L.cpattn_backward_varlen(*args) == C.CPATTN_EDTYPE
    args[1] = C.CPATTN_BF16
    args[5] = ALIGNED + 8
    assert L.cpattn_backward_varlen(*args) == C.CPATTN_EALIGN
    del keep, keep2


def test_probe_validation_before_launch():
    L = C.lib()
    assert L.cpattn_probe_mfma(None, ALIGNED, 1, 1, None) == 1
    assert L.cpattn_probe_mfma(ALIGNED + 8, ALIGNED, 1, 1, None) == 1   # 16-byte alignment
    assert L.cpattn_probe_mfma(ALIGNED, ALIGNED, 0, 1, None) == 1
    assert L.cpattn_probe_mfma(ALIGNED, ALIGNED, 1, 0, None) == 1
    assert L.cpattn_device_info(None, None) == 1
    assert L.cpattn_probe_fill_lds(0, 0, None) == 1    # no workgroups
    assert L.cpattn_probe_fill_lds(0, -4, None) == 1
