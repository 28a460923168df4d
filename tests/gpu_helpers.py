"""Shared helpers of the GPU parity tests (not collected by pytest)."""
import dataclasses

import numpy as np
import torch

from long_context_causal_amd import cpattn as C
from long_context_causal_amd.inputs import Workload, as_f32, make_inputs
from long_context_causal_amd.runner import CPProblem, bf16_bits, to_device
from oracle import attention_rows, causal_attention
from oracle import cp as ocp

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5
# backward bound (bf16 rounding of P and dS in the products, 2^-9 relative
# per term; gradients are sums with cancellation, so the error is measured
# against the gradient's own scale), per gradient
GRAD_MAX_REL, GRAD_MEAN_REL = 1e-2, 5e-3


def say(msg):
    print(msg, flush=True)


def host_f32(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        from long_context_causal_amd.inputs import bf16_bits_to_f32
        return bf16_bits_to_f32(bf16_bits(t))
    return t.detach().float().cpu().numpy()


def errors(got, want):
    diff = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    return float(diff.max()), float(diff.mean())


def assert_close(name, got, want, max_abs, mean_abs=None):
    mx, mn = errors(got, want)
    say(f"  [{name}] max_abs={mx:.3e} mean_abs={mn:.3e} (bounds {max_abs:g}"
        f"{'' if mean_abs is None else f', mean {mean_abs:g}'})")
    assert np.isfinite(np.asarray(got)).all(), f"{name}: non-finite output"
    assert mx <= max_abs, f"{name}: max abs {mx} > {max_abs}"
    if mean_abs is not None:
        assert mn <= mean_abs, f"{name}: mean abs {mn} > {mean_abs}"


def assert_grad(name, got, ref):
    """max |err| <= GRAD_MAX_REL max |ref| and mean |err| <= GRAD_MEAN_REL
    mean |ref|."""
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    mx, mn = err.max(), err.mean()
    rmx, rmn = np.abs(ref).max(), np.abs(ref).mean()
    say(f"  [{name}] max_err={mx:.3e} ({mx / rmx:.2e} of max|ref|) "
        f"mean_err={mn:.3e} ({mn / rmn:.2e} of mean|ref|)")
    assert mx <= GRAD_MAX_REL * rmx, f"{name}: max error {mx} > {GRAD_MAX_REL} * {rmx}"
    assert mn <= GRAD_MEAN_REL * rmn, f"{name}: mean error {mn} > {GRAD_MEAN_REL} * {rmn}"


def seeded_dout(w: Workload, seed=99):
    """dO of a workload: seeded standard normal, rounded to bf16 bits."""
    from long_context_causal_amd.inputs import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((w.b, w.s, w.hq, w.d)).astype(np.float32))


def small(w: Workload, s: int, b=None) -> Workload:
    """The same workload (heads, d, cp, dtype, distribution) at length s."""
    return dataclasses.replace(w, s=s, b=w.b if b is None else b)


def oracle_full(w: Workload, q, k, v):
    """Non-CP oracle (O [b, s, hq, d], L [b, hq, s]) in fp64, RoPE applied."""
    qf, kf, vf = (as_f32(x).astype(np.float64) for x in (q, k, v))
    if w.rope_theta is not None:
        ar = np.arange(qf.shape[1])
        qf, kf = ocp.rope(qf, ar, w.rope_theta), ocp.rope(kf, ar, w.rope_theta)
    return causal_attention(qf, kf, vf)


def run_rank(P: CPProblem, rank, out_dtype=C.CPATTN_F32):
    buf = P.alloc_rank(rank, out_dtype)
    P.forward(buf)
    torch.cuda.synchronize()
    return host_f32(buf["o"]), buf["lse"].cpu().numpy()


__all__ = ["C", "CPProblem", "Workload", "make_inputs", "to_device", "torch", "np", "ocp",
           "attention_rows", "causal_attention", "as_f32"]
