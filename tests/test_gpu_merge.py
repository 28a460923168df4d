"""GPU LSE merge (cpattn_merge) vs the oracle's per-step L correction and
final O merge, on synthetic partials with uncovered rows, empty partials
and large LSE gaps."""
import numpy as np
import pytest

from gpu_helpers import C, assert_close, host_f32, ocp, say, torch

pytestmark = pytest.mark.gpu


def _partials(seed, b, two_c, hq, d, spans, gap=0.0):
    rng = np.random.default_rng(seed)
    parts = []
    for i, (row0, rows) in enumerate(spans):
        o = rng.standard_normal((b, rows, hq, d)).astype(np.float32)
        l = (rng.standard_normal((b, hq, rows)) * 3 + (gap if i % 2 else -gap)).astype(np.float32)
        parts.append((o, l, row0))
    return parts


def _gpu_merge(parts, b, two_c, hq, d, out_dtype):
    dims = C.make_dims(b, two_c * 4, hq, hq, d, 4)
    dev = [(torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda(), row0, o.shape[1])
           for o, l, row0 in parts]
    o_out = torch.empty((b, two_c, hq, d), device="cuda",
                        dtype=torch.bfloat16 if out_dtype == C.CPATTN_BF16 else torch.float32)
    l_out = torch.empty((b, hq, two_c), device="cuda", dtype=torch.float32)
    C.cpattn_merge(dims, dev, out_dtype, o_out, l_out)
    torch.cuda.synchronize()
    return host_f32(o_out), l_out.cpu().numpy()


@pytest.mark.parametrize("gap", [0.0, 30.0])
@pytest.mark.parametrize("n_parts", [2, 8, 16])
def test_merge_cp_like_spans(n_parts, gap):
    b, c, hq, d = 2, 50, 8, 128
    two_c = 2 * c
    spans = [(0, two_c)] + [((0, two_c) if i % 3 else (c, c)) for i in range(1, n_parts)]
    say(f"merge n={n_parts} gap={gap}")
    parts = _partials(n_parts, b, two_c, hq, d, spans, gap)
    o, l = _gpu_merge(parts, b, two_c, hq, d, C.CPATTN_F32)
    o_ref, l_ref = ocp.merge_outputs([(p[0].astype(np.float64), p[1].astype(np.float64), p[2])
                                      for p in parts], two_c)
    assert_close("O", o, o_ref, 1e-5)
    assert_close("L", l, l_ref, 1e-5)


def test_merge_uncovered_rows_and_empty_partial():
    b, two_c, hq, d = 1, 64, 4, 64
    parts = _partials(1, b, two_c, hq, d, [(0, 20), (40, 24), (10, 30)])
    # the third partial says "no keys" on every row: L = -inf, O = 0
    parts[2] = (np.zeros_like(parts[2][0]), np.full_like(parts[2][1], -np.inf), 10)
    say("merge uncovered rows")
    o, l = _gpu_merge(parts, b, two_c, hq, d, C.CPATTN_F32)
    o_ref, l_ref = ocp.merge_outputs([(p[0].astype(np.float64), p[1].astype(np.float64), p[2])
                                      for p in parts], two_c)
    # rows 20..39 are covered only by the empty partial: L = -inf, O = 0
    assert np.all(l[:, :, 20:40] == -np.inf) and np.all(o[:, 20:40] == 0)
    fin = np.isfinite(l_ref)
    assert np.array_equal(fin, np.isfinite(l))
    assert_close("L", l[fin], l_ref[fin], 1e-5)
    assert_close("O", o, o_ref, 1e-5)


def test_merge_bf16_output_rounding():
    b, c, hq, d = 1, 64, 4, 128
    two_c = 2 * c
    parts = _partials(5, b, two_c, hq, d, [(0, two_c), (0, two_c), (c, c)])
    say("merge bf16 out")
    o, l = _gpu_merge(parts, b, two_c, hq, d, C.CPATTN_BF16)
    o_ref, l_ref = ocp.merge_outputs([(p[0].astype(np.float64), p[1].astype(np.float64), p[2])
                                      for p in parts], two_c)
    err = np.abs(o - o_ref)
    assert np.all(err <= np.abs(o_ref) * 2.0 ** -8 + 1e-5)
    assert_close("L", l, l_ref, 1e-5)


def test_merge_heads_in_several_runs():
    """More (head, partial) weights than the kernel's LDS holds at once: the
    heads are merged in runs (208 heads x 40 covering partials)."""
    b, c, hq, d = 1, 16, 208, 64
    two_c = 2 * c
    spans = [(0, two_c) if i % 4 else (c, c) for i in range(40)]
    say("merge 208 heads x 40 partials")
    parts = _partials(7, b, two_c, hq, d, spans, 5.0)
    o, l = _gpu_merge(parts, b, two_c, hq, d, C.CPATTN_F32)
    o_ref, l_ref = ocp.merge_outputs([(p[0].astype(np.float64), p[1].astype(np.float64), p[2])
                                      for p in parts], two_c)
    assert_close("O", o, o_ref, 1e-5)
    assert_close("L", l, l_ref, 1e-5)
