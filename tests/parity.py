"""Comparison rules between the HIP path and the fp64 oracle.

Official bar (per element, max-abs, absolute): O, dQ, dK, dV within 2e-2 for
bf16 inputs and 1e-4 for fp32 inputs; selected pages identical except inside
the near-tie band (K-th and (K+1)-th oracle scores closer than 1e-4 relative).

Internal bars, named separately from the official one, so that a localised bug
cannot hide under an absolute bound close to the outputs' own RMS:
rms(err) / rms(ref) <= 1e-2 (bf16) or 1e-5 (fp32), and |LSE err| <= 2e-4
(bf16) or 1e-5 (fp32).  The bf16 bound follows from the arithmetic: S and dP
are exact products of bf16 inputs summed in fp32; P and dS are rounded once to
bf16 (8 significant bits: relative error at most 2^-8 ~ 3.9e-3, about 2^-8/sqrt(3)
rms) before their MFMAs, so relative RMS errors of a few 1e-3 are expected.
The rms bar applies where the reference is not zero: a reference whose RMS is
below ZERO_REF (an exact zero up to fp64 rounding, as dQ and dK are when every
value vector of a head is the same) is held to the absolute bar alone.
"""
from __future__ import annotations

import numpy as np

MAX_ABS = {"bf16": 2e-2, "f32": 1e-4}
RMS_REL = {"bf16": 1e-2, "f32": 1e-5}
LSE_ABS = {"bf16": 2e-4, "f32": 1e-5}
TIE_REL = 1e-4
ZERO_REF = 1e-12


def compare(name, got, want, dtype, report=None, max_abs=None):
    """Official max-abs bar, plus the internal rms bar.  `max_abs` replaces the
    official bar only for a documented known limit (see
    test_gpu_parity.test_bf16_large_scale_known_limit)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if got.size == 0:
        return
    err = np.abs(got - want)
    max_err = float(err.max())
    rms_ref = float(np.sqrt(np.mean(want ** 2)))
    rms_rel = float(np.sqrt(np.mean(err ** 2))) / max(rms_ref, 1e-30)
    if report is not None:
        report[name] = dict(max_abs=max_err, rms_rel=rms_rel, rms_ref=rms_ref)
    if max_abs is None:
        max_abs = MAX_ABS[dtype]
    assert max_err <= max_abs, f"{name}: max |err| {max_err:.3e} > {max_abs:.2e}"
    if rms_ref > ZERO_REF:
        assert rms_rel <= RMS_REL[dtype], f"{name}: rms rel err {rms_rel:.3e} > {RMS_REL[dtype]:.0e}"


def compare_lse(got, want, dtype, report=None):
    err = float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64)))) if np.size(want) else 0.0
    if report is not None:
        report["lse"] = dict(max_abs=err)
    assert err <= LSE_ABS[dtype], f"lse: max |err| {err:.3e} > {LSE_ABS[dtype]:.0e}"


def check_selection(gpu_sel, scores, keff):
    """Accept the GPU's pages for every kv-head.  Returns True when identical to
    the oracle's choice, False when they differ only inside the near-tie band.
    Band rule: with s_K, s_K+1 the K-th and (K+1)-th best oracle scores, if
    |s_K - s_K+1| < 1e-4 * max(|s_K|, |s_K+1|) the GPU set must hold every page
    scoring above the band {n : |s_n - s_K| <= 1e-4 |s_K|}, its other pages must
    lie in the band, and it must have K_eff distinct pages."""
    scores = np.asarray(scores, dtype=np.float64)
    gpu_sel = np.asarray(gpu_sel)
    hkv, n = scores.shape
    assert gpu_sel.shape == (hkv, keff), (gpu_sel.shape, (hkv, keff))
    exact = True
    for h in range(hkv):
        got = [int(v) for v in gpu_sel[h]]
        assert got == sorted(set(got)), f"head {h}: selection not ascending/distinct"
        assert all(0 <= v < n for v in got), f"head {h}: page out of range"
        order = sorted(range(n), key=lambda m: (-scores[h, m], m))
        want = sorted(order[:keff])
        if got == want:
            continue
        assert 0 < keff < n, f"head {h}: K_eff in (0, N) required for a tie"
        sK, sK1 = scores[h, order[keff - 1]], scores[h, order[keff]]
        assert abs(sK - sK1) < TIE_REL * max(abs(sK), abs(sK1)), f"head {h}: selection differs outside a tie"
        band = {m for m in range(n) if abs(scores[h, m] - sK) <= TIE_REL * abs(sK)}
        above = {m for m in range(n) if scores[h, m] > sK and m not in band}
        assert above <= set(got), f"head {h}: a page above the tie band is missing"
        assert set(got) - above <= band, f"head {h}: a page outside the tie band was taken"
        exact = False
    return exact
