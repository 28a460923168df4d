"""GPU step attention (cpattn_step_fwd) vs the oracle's step attention, for
every mode, both dtypes, GQA and ragged tails."""
import numpy as np
import pytest

from gpu_helpers import (BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, C, as_f32, assert_close,
                         ocp, say, to_device, torch)
from long_context_causal_amd.inputs import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

MODES = [C.CPATTN_CAUSAL, C.CPATTN_KV_FIRST_HALF, C.CPATTN_Q_SECOND_HALF]


def _blocks(seed, b, two_c, hq, hkv, d, dtype, qk_scale=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((b, two_c, hq, d), dtype=np.float32) * np.float32(qk_scale)
    k = rng.standard_normal((b, two_c, hkv, d), dtype=np.float32) * np.float32(qk_scale)
    v = rng.standard_normal((b, two_c, hkv, d), dtype=np.float32)
    if dtype == "bf16":
        return tuple(f32_to_bf16_bits(x) for x in (q, k, v))
    return q, k, v


def _run_step(dtype, mode, b, c, hq, hkv, d, seed, qk_scale=1.0, scale=0.0):
    two_c = 2 * c
    say(f"step dtype={dtype} mode={ocp.MODE_NAMES[mode]} b={b} c={c} hq={hq} hkv={hkv} d={d} "
        f"seed={seed}")
    q, k, v = _blocks(seed, b, two_c, hq, hkv, d, dtype, qk_scale)
    dims = C.make_dims(b, two_c * 3, hq, hkv, d, 3)      # c = s / (2 cp)
    rows = c if mode == C.CPATTN_Q_SECOND_HALF else two_c
    o = torch.empty((b, rows, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((b, hq, rows), dtype=torch.float32, device="cuda")
    C.cpattn_step_fwd(dims, C.CPATTN_BF16 if dtype == "bf16" else C.CPATTN_F32, scale, mode,
                      to_device(q), to_device(k), to_device(v), o, lse)
    torch.cuda.synchronize()
    qf, kf, vf = (as_f32(x).astype(np.float64) for x in (q, k, v))
    o_ref, l_ref, row0 = ocp.step_attention(qf, kf, vf, mode,
                                            scale=None if scale == 0.0 else scale)
    assert row0 == (c if mode == C.CPATTN_Q_SECOND_HALF else 0)
    return o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("b,c,hq,hkv,d", [(1, 128, 4, 4, 64), (2, 37, 4, 2, 128),
                                          (1, 200, 2, 1, 64)])
def test_step_f32(mode, b, c, hq, hkv, d):
    o, l, o_ref, l_ref = _run_step("f32", mode, b, c, hq, hkv, d, seed=c + mode)
    assert_close("O", o, o_ref, F32_MAX_ABS)
    assert_close("L", l, l_ref, F32_MAX_ABS)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("b,c,hq,hkv,qk", [(1, 256, 8, 2, 0.5),    # whole tiles
                                           (2, 100, 4, 4, 1.0),    # ragged query and key tiles
                                           (1, 37, 8, 1, 1.0),     # tiny, MQA
                                           (1, 300, 2, 2, 2.24)])  # logits ~ +-30
def test_step_bf16(mode, b, c, hq, hkv, qk):
    o, l, o_ref, l_ref = _run_step("bf16", mode, b, c, hq, hkv, 128, seed=7 * c + mode,
                                   qk_scale=qk)
    assert_close("O", o, o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    assert_close("L", l, l_ref, 1e-3)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("b,c,hq,hkv,qk", [(1, 256, 8, 2, 0.5),    # whole tiles
                                           (2, 100, 4, 4, 1.0),    # ragged query and key tiles
                                           (1, 37, 8, 1, 1.0),     # tiny, MQA
                                           (1, 300, 2, 2, 2.24)])  # logits ~ +-30
def test_step_bf16_head_dim_64(mode, b, c, hq, hkv, qk):
    """The bf16 kernel built for 64-wide heads (128-byte LDS rows, eight rows
    per copy, its own swizzles, four matrix steps per phase)."""
    o, l, o_ref, l_ref = _run_step("bf16", mode, b, c, hq, hkv, 64, seed=11 * c + mode,
                                   qk_scale=qk)
    assert_close("O", o, o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    assert_close("L", l, l_ref, 1e-3)


def test_step_explicit_scale():
    o, l, o_ref, l_ref = _run_step("bf16", C.CPATTN_CAUSAL, 1, 64, 2, 2, 128, seed=3,
                                   scale=0.02)
    assert_close("O", o, o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    assert_close("L", l, l_ref, 1e-3)
    o, l, o_ref, l_ref = _run_step("f32", C.CPATTN_KV_FIRST_HALF, 1, 64, 2, 2, 64, seed=4,
                                   scale=0.3)
    assert_close("O", o, o_ref, F32_MAX_ABS)
    assert_close("L", l, l_ref, F32_MAX_ABS)


def test_step_closed_form_zero_query():
    """Q = 0, V[j] = j: causal row i gets O = i/2 and L = ln(i+1)."""
    b, c, hq, d = 1, 96, 2, 128
    two_c = 2 * c
    q = np.zeros((b, two_c, hq, d), np.float32)
    k = np.random.default_rng(0).standard_normal((b, two_c, 1, d)).astype(np.float32)
    v = np.broadcast_to(np.arange(two_c, dtype=np.float32)[None, :, None, None],
                        (b, two_c, 1, d)).copy()
    dims = C.make_dims(b, two_c * 2, hq, 1, d, 2)
    for dtype, tdt in ((C.CPATTN_BF16, "bf16"), (C.CPATTN_F32, "f32")):
        say(f"closed form dtype={tdt}")
        qq, kk, vv = ((f32_to_bf16_bits(x) if tdt == "bf16" else x) for x in (q, k, v))
        o = torch.empty((b, two_c, hq, d), dtype=torch.float32, device="cuda")
        lse = torch.empty((b, hq, two_c), dtype=torch.float32, device="cuda")
        C.cpattn_step_fwd(dims, dtype, 0.0, C.CPATTN_CAUSAL, to_device(qq), to_device(kk),
                          to_device(vv), o, lse)
        torch.cuda.synchronize()
        want = np.arange(two_c) / 2.0
        # bf16 P: the uniform weight 1 is exact, V = j is exact in bf16 up to 256
        assert_close("O", o.cpu().numpy()[0, :, :, :],
                     np.broadcast_to(want[:, None, None], (two_c, hq, d)), 1e-4)
        assert_close("L", lse.cpu().numpy()[0], np.log(np.arange(1, two_c + 1))[None, :], 1e-5)
