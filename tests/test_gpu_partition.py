"""GPU zigzag partition vs the oracle's split: bit-exact bytes and indices;
RoPE rows against the oracle's fp64 rotation at global positions."""
import dataclasses

import numpy as np
import pytest

from gpu_helpers import (C, CPProblem, as_f32, assert_close, host_f32, make_inputs, ocp, say,
                         small, torch)
from long_context_causal_amd.inputs import WORKLOADS
from long_context_causal_amd.runner import bf16_bits

pytestmark = pytest.mark.gpu


def _bits(t):
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.cpu().numpy().view(np.uint32)


def _host_bits(x):
    return x if x.dtype == np.uint16 else x.view(np.uint32)


CASES = [
    ("fp32_mha_s512_cp2", None),             # full size
    ("bf16_gqa_s8k_cp4", 8 * 100),           # c = 100: ragged against every tile
    ("bf16_mha_s16k_cp4_widelogits", 8 * 37),
    ("bf16_gqa_s32k_cp8", 16 * 3),           # c = 3
    ("bf16_gqa_s8k_cp4", None),              # full size
]


@pytest.mark.parametrize("name,s", CASES)
def test_partition_bit_exact(name, s):
    w = WORKLOADS[name]
    w = small(w, s) if s else w
    w = dataclasses.replace(w, rope_theta=None)
    say(f"partition {name} s={w.s} cp={w.cp} b={w.b}")
    q, k, v = make_inputs(w)
    P = CPProblem(w, q, k, v)
    P.partition()
    torch.cuda.synchronize()
    for host, dev in ((q, P.qz), (k, P.kz), (v, P.vz)):
        want = ocp.partition(_host_bits(host), w.cp)
        assert np.array_equal(_bits(dev), want)
    pos = P.pos.cpu().numpy()
    for r in range(w.cp):
        assert np.array_equal(pos[r], ocp.zigzag_positions(w.s, w.cp, r))


def test_partition_headline_full_size():
    w = WORKLOADS["bf16_gqa_s32k_cp8"]
    say(f"partition full {w.name}")
    q, k, v = make_inputs(w)
    P = CPProblem(w, q, k, v)
    P.partition()
    torch.cuda.synchronize()
    for host, dev in ((k, P.kz), (v, P.vz), (q, P.qz)):
        assert np.array_equal(_bits(dev), ocp.partition(host, w.cp))


@pytest.mark.parametrize("dtype,s,cp", [("bf16", 1024, 4), ("f32", 640, 5), ("bf16", 131072, 16)])
def test_partition_rope_global_positions(dtype, s, cp):
    base = WORKLOADS["bf16_gqa_s128k_cp16_rope"]
    w = dataclasses.replace(base, s=s, cp=cp, dtype=dtype,
                            hq=8 if s > 100000 else base.hq)
    say(f"partition+rope {dtype} s={s} cp={cp} hq={w.hq}")
    q, k, v = make_inputs(w)
    P = CPProblem(w, q, k, v)
    P.partition()
    torch.cuda.synchronize()
    qz, kz = host_f32(P.qz), host_f32(P.kz)
    ranks = range(cp) if s < 100000 else [0, 7, cp - 1]
    for r in ranks:
        pos = ocp.zigzag_positions(s, cp, r)
        for name, host, dev in (("q", q, qz), ("k", k, kz)):
            want = ocp.rope(as_f32(host[:, pos]).astype(np.float64), pos, w.rope_theta)
            if dtype == "bf16":
                # one bf16 rounding of the fp32 rotation: half an ulp, 2^-9 relative
                err = np.abs(dev[r] - want)
                bound = np.abs(want) * 2.0 ** -8 + 1e-6
                say(f"  rank {r} {name}: max err/bound {float((err / bound).max()):.3f}")
                assert np.all(err <= bound)
            else:
                assert_close(f"rank {r} {name}", dev[r], want, 1e-5)
    # V is never rotated
    assert np.array_equal(_bits(P.vz), ocp.partition(_host_bits(v), cp))
