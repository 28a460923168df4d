"""ctypes binding of ``libcpattn.so`` (declared in ``include/cpattn.h``).

Argument marshalling only: every function forwards to the C entry point of
the same name.  Device buffers are torch tensors (their ``data_ptr()``) or
raw integer addresses; ``stream`` is a ``torch.cuda.Stream``, a raw
``hipStream_t`` integer, or None for torch's current stream.  A nonzero
status raises :class:`CpattnError`.  There is no fallback: if the library
is not built, every call raises.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcpattn.so")

CPATTN_F32 = 0
CPATTN_BF16 = 1
CPATTN_CAUSAL = 0
CPATTN_KV_FIRST_HALF = 1
CPATTN_Q_SECOND_HALF = 2
CPATTN_OK, CPATTN_EINVAL, CPATTN_ESHAPE, CPATTN_EDTYPE, CPATTN_EALIGN, \
    CPATTN_ENOSPACE, CPATTN_EHIP = range(7)
CPATTN_MERGE_PASS = 64
CPATTN_NOALLOC_SCRATCH_BYTES = 256 << 20
CPATTN_MAX_SEQS = 128


class cpattn_dims(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("s", ctypes.c_int64), ("hq", ctypes.c_int32),
                ("hkv", ctypes.c_int32), ("d", ctypes.c_int32), ("cp", ctypes.c_int32)]


class cpattn_rope(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_double)]


class cpattn_partial(ctypes.Structure):
    _fields_ = [("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("row0", ctypes.c_int64), ("rows", ctypes.c_int64)]


class cpattn_varlen(ctypes.Structure):
    _fields_ = [("nseq", ctypes.c_int32), ("cu_seqlens", ctypes.POINTER(ctypes.c_int64))]


def make_varlen(cu_seqlens):
    """A cpattn_varlen over a host copy of the offsets; keep the returned
    pair alive for the call (the struct points into the array)."""
    arr = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    vl = cpattn_varlen(arr.size - 1, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    return vl, arr


class CpattnError(RuntimeError):
    def __init__(self, status, func):
        self.status = status
        super().__init__(f"{func}: {cpattn_status_str(status)}")


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m long_context_causal_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.POINTER(cpattn_dims)
        L.cpattn_step_mode.argtypes = [I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)]
        L.cpattn_partition_positions.argtypes = [ctypes.c_int64, I, I,
                                                 ctypes.POINTER(ctypes.c_int32)]
        L.cpattn_partition.argtypes = [D, I, I, P, P, P, ctypes.POINTER(cpattn_rope), P]
        L.cpattn_step_fwd.argtypes = [D, I, ctypes.c_float, I, P, P, P, P, P, P]
        L.cpattn_merge.argtypes = [D, I, ctypes.POINTER(cpattn_partial), I, P, P, P]
        L.cpattn_forward_workspace.argtypes = [D, I]
        L.cpattn_forward_workspace.restype = ctypes.c_size_t
        L.cpattn_forward_partials.argtypes = [D, I, P, ctypes.c_size_t,
                                              ctypes.POINTER(cpattn_partial)]
        L.cpattn_forward_steps.argtypes = [D, I, ctypes.c_float, I, P, P, P, P,
                                           ctypes.c_size_t, P]
        L.cpattn_forward.argtypes = [D, I, ctypes.c_float, I, P, P, P, P, ctypes.c_size_t,
                                     I, P, P, P]
        L.cpattn_forward_fused.argtypes = [D, I, ctypes.c_float, I, P, P, P, I, P, P, P]
        L.cpattn_forward_noalloc.argtypes = [D, I, ctypes.c_float, I, P, P, P, I, P, P, P]
        V = ctypes.POINTER(cpattn_varlen)
        L.cpattn_partition_positions_varlen.argtypes = [ctypes.c_int64, I, I, V,
                                                        ctypes.POINTER(ctypes.c_int32)]
        L.cpattn_partition_varlen.argtypes = [D, I, I, V, P, P, P, ctypes.POINTER(cpattn_rope), P]
        L.cpattn_forward_fused_varlen.argtypes = [D, I, ctypes.c_float, I, V, P, P, P, I, P, P,
                                                  P]
        L.cpattn_backward_varlen.argtypes = [D, I, ctypes.c_float, I, V, P, P, P, P, P, P, P, P,
                                             P, P, P]
        L.cpattn_bwd_delta.argtypes = [D, P, P, P, P]
        L.cpattn_step_bwd.argtypes = [D, I, ctypes.c_float, I, P, P, P, P, P, P, P, P, P, P]
        L.cpattn_backward.argtypes = [D, I, ctypes.c_float, I, P, P, P, P, P, P, P, P, P, P, P]
        L.cpattn_probe_mfma.argtypes = [P, P, I, I, P]
        L.cpattn_device_info.argtypes = [ctypes.POINTER(I), ctypes.POINTER(I)]
        L.cpattn_probe_fill_lds.argtypes = [ctypes.c_uint, I, P]
        L.cpattn_status_str.argtypes = [I]
        L.cpattn_status_str.restype = ctypes.c_char_p
        for name in ("cpattn_step_mode", "cpattn_partition_positions", "cpattn_partition",
                     "cpattn_step_fwd", "cpattn_merge", "cpattn_forward_partials",
                     "cpattn_forward_steps", "cpattn_forward",
                     "cpattn_forward_fused", "cpattn_forward_noalloc", "cpattn_bwd_delta", "cpattn_step_bwd",
                     "cpattn_backward", "cpattn_partition_positions_varlen",
                     "cpattn_partition_varlen", "cpattn_forward_fused_varlen",
                     "cpattn_backward_varlen", "cpattn_probe_mfma", "cpattn_device_info",
                     "cpattn_probe_fill_lds"):
            getattr(L, name).restype = I
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, func):
    if status != CPATTN_OK:
        raise CpattnError(status, func)


def make_dims(b, s, hq, hkv, d, cp):
    return cpattn_dims(b, s, hq, hkv, d, cp)


def cpattn_status_str(status):
    return lib().cpattn_status_str(int(status)).decode()


def cpattn_step_mode(step, rank, cp):
    mode, src = ctypes.c_int(), ctypes.c_int()
    _check(lib().cpattn_step_mode(step, rank, cp, ctypes.byref(mode), ctypes.byref(src)),
           "cpattn_step_mode")
    return mode.value, src.value


def cpattn_partition_positions(s, cp, rank):
    if s % (2 * cp) != 0:
        raise CpattnError(CPATTN_ESHAPE, "cpattn_partition_positions")
    out = np.empty(s // cp, dtype=np.int32)
    _check(lib().cpattn_partition_positions(
        s, cp, rank, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
        "cpattn_partition_positions")
    return out


def cpattn_partition(dims, dtype, h, x, xz, pos=None, rope_theta=None, stream=None):
    rope = ctypes.byref(cpattn_rope(rope_theta)) if rope_theta is not None else None
    _check(lib().cpattn_partition(ctypes.byref(dims), dtype, h, _ptr(x), _ptr(xz), _ptr(pos),
                                  rope, _stream(stream)), "cpattn_partition")


def cpattn_step_fwd(dims, dtype, scale, mode, q_r, k_src, v_src, o, lse, stream=None):
    _check(lib().cpattn_step_fwd(ctypes.byref(dims), dtype, float(scale), mode, _ptr(q_r),
                                 _ptr(k_src), _ptr(v_src), _ptr(o), _ptr(lse),
                                 _stream(stream)), "cpattn_step_fwd")


def cpattn_merge(dims, partials, out_dtype, o_out, lse_out=None, stream=None):
    """partials: sequence of (o, lse, row0, rows)."""
    arr = (cpattn_partial * max(1, len(partials)))()
    for i, (o, lse, row0, rows) in enumerate(partials):
        arr[i] = cpattn_partial(_ptr(o), _ptr(lse), row0, rows)
    _check(lib().cpattn_merge(ctypes.byref(dims), len(partials), arr, out_dtype, _ptr(o_out),
                              _ptr(lse_out), _stream(stream)), "cpattn_merge")


def cpattn_forward_workspace(dims, rank):
    return int(lib().cpattn_forward_workspace(ctypes.byref(dims), rank))


def cpattn_forward_partials(dims, rank, ws, ws_bytes):
    """The step partials inside a workspace: a list of (o address, lse
    address, row0, rows), one per step."""
    arr = (cpattn_partial * dims.cp)()
    _check(lib().cpattn_forward_partials(ctypes.byref(dims), rank, _ptr(ws), int(ws_bytes), arr),
           "cpattn_forward_partials")
    return [(p.o, p.lse, p.row0, p.rows) for p in arr]


def cpattn_forward_steps(dims, dtype, scale, rank, qz, kz, vz, ws, ws_bytes, stream=None):
    _check(lib().cpattn_forward_steps(ctypes.byref(dims), dtype, float(scale), rank, _ptr(qz),
                                      _ptr(kz), _ptr(vz), _ptr(ws), int(ws_bytes),
                                      _stream(stream)),
           "cpattn_forward_steps")


def cpattn_forward(dims, dtype, scale, rank, qz, kz, vz, ws, ws_bytes, out_dtype, o_out,
                   lse_out=None, stream=None):
    _check(lib().cpattn_forward(ctypes.byref(dims), dtype, float(scale), rank, _ptr(qz),
                                _ptr(kz), _ptr(vz), _ptr(ws), int(ws_bytes), out_dtype,
                                _ptr(o_out), _ptr(lse_out), _stream(stream)),
           "cpattn_forward")


def cpattn_forward_noalloc(dims, dtype, scale, rank, qz, kz, vz, out_dtype, o_out, lse_out=None,
                           stream=None):
    _check(lib().cpattn_forward_noalloc(ctypes.byref(dims), dtype, float(scale), rank, _ptr(qz),
                                        _ptr(kz), _ptr(vz), out_dtype, _ptr(o_out),
                                        _ptr(lse_out), _stream(stream)),
           "cpattn_forward_noalloc")


def cpattn_forward_fused(dims, dtype, scale, rank, qz, kz, vz, out_dtype, o_out, lse_out=None,
                         stream=None):
    _check(lib().cpattn_forward_fused(ctypes.byref(dims), dtype, float(scale), rank, _ptr(qz),
                                      _ptr(kz), _ptr(vz), out_dtype, _ptr(o_out), _ptr(lse_out),
                                      _stream(stream)),
           "cpattn_forward_fused")


def cpattn_bwd_delta(dims, o_r, do_r, delta_r, stream=None):
    _check(lib().cpattn_bwd_delta(ctypes.byref(dims), _ptr(o_r), _ptr(do_r), _ptr(delta_r),
                                  _stream(stream)), "cpattn_bwd_delta")


def cpattn_step_bwd(dims, dtype, scale, mode, q_r, k_src, v_src, do_r, lse_r, delta_r, dq_r,
                    dk_src, dv_src, stream=None):
    _check(lib().cpattn_step_bwd(ctypes.byref(dims), dtype, float(scale), mode, _ptr(q_r),
                                 _ptr(k_src), _ptr(v_src), _ptr(do_r), _ptr(lse_r),
                                 _ptr(delta_r), _ptr(dq_r), _ptr(dk_src), _ptr(dv_src),
                                 _stream(stream)), "cpattn_step_bwd")


def cpattn_backward(dims, dtype, scale, rank, qz, kz, vz, o_r, do_r, lse_r, delta_ws, dq_r, dkz,
                    dvz, stream=None):
    _check(lib().cpattn_backward(ctypes.byref(dims), dtype, float(scale), rank, _ptr(qz),
                                 _ptr(kz), _ptr(vz), _ptr(o_r), _ptr(do_r), _ptr(lse_r),
                                 _ptr(delta_ws), _ptr(dq_r), _ptr(dkz), _ptr(dvz),
                                 _stream(stream)), "cpattn_backward")


def cpattn_partition_positions_varlen(s, cp, rank, cu_seqlens):
    if s % cp != 0:
        raise CpattnError(CPATTN_ESHAPE, "cpattn_partition_positions_varlen")
    vl, keep = make_varlen(cu_seqlens)
    out = np.empty(s // cp, dtype=np.int32)
    _check(lib().cpattn_partition_positions_varlen(
        s, cp, rank, ctypes.byref(vl), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
        "cpattn_partition_positions_varlen")
    del keep
    return out


def cpattn_partition_varlen(dims, dtype, h, cu_seqlens, x, xz, pos=None, rope_theta=None,
                            stream=None):
    vl, keep = make_varlen(cu_seqlens)
    rope = ctypes.byref(cpattn_rope(rope_theta)) if rope_theta is not None else None
    _check(lib().cpattn_partition_varlen(ctypes.byref(dims), dtype, h, ctypes.byref(vl),
                                         _ptr(x), _ptr(xz), _ptr(pos), rope, _stream(stream)),
           "cpattn_partition_varlen")
    del keep


def cpattn_forward_fused_varlen(dims, dtype, scale, rank, cu_seqlens, qz, kz, vz, out_dtype,
                                o_out, lse_out=None, stream=None):
    vl, keep = make_varlen(cu_seqlens)
    _check(lib().cpattn_forward_fused_varlen(ctypes.byref(dims), dtype, float(scale), rank,
                                             ctypes.byref(vl), _ptr(qz), _ptr(kz), _ptr(vz),
                                             out_dtype, _ptr(o_out), _ptr(lse_out),
                                             _stream(stream)),
           "cpattn_forward_fused_varlen")
    del keep


def cpattn_backward_varlen(dims, dtype, scale, rank, cu_seqlens, qz, kz, vz, o_r, do_r, lse_r,
                           delta_ws, dq_r, dkz, dvz, stream=None):
    vl, keep = make_varlen(cu_seqlens)
    _check(lib().cpattn_backward_varlen(ctypes.byref(dims), dtype, float(scale), rank,
                                        ctypes.byref(vl), _ptr(qz), _ptr(kz), _ptr(vz),
                                        _ptr(o_r), _ptr(do_r), _ptr(lse_r), _ptr(delta_ws),
                                        _ptr(dq_r), _ptr(dkz), _ptr(dvz), _stream(stream)),
           "cpattn_backward_varlen")
    del keep


# --- measurement helpers (include/cpattn_probe.h) -------------------------------

def cpattn_probe_mfma(operands, out, blocks, iters, stream=None):
    """Pure-MFMA rate probe: blocks * 8 * iters * 16 * 32768 FLOP."""
    if lib().cpattn_probe_mfma(_ptr(operands), _ptr(out), int(blocks), int(iters),
                               _stream(stream)) != 0:
        raise RuntimeError("cpattn_probe_mfma failed")


def cpattn_device_info():
    """(compute units, maximum engine clock in kHz) of the current device."""
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    if lib().cpattn_device_info(ctypes.byref(cus), ctypes.byref(khz)) != 0:
        raise RuntimeError("cpattn_device_info failed")
    return cus.value, khz.value


def cpattn_probe_fill_lds(pattern, blocks, stream=None):
    """Every 32-bit word of the LDS of 'blocks' full-LDS workgroups set to
    'pattern' (tests: LDS a later launch must not read unwritten)."""
    if lib().cpattn_probe_fill_lds(int(pattern) & 0xFFFFFFFF, int(blocks),
                                   _stream(stream)) != 0:
        raise RuntimeError("cpattn_probe_fill_lds failed")
