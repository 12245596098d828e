"""Parity rule between the GPU output and the oracle (test helper).

Several results are correct: the pages fix an fp32 accumulator and the bf16
rounding points, not the order of the fp32 sum. Two correct orders can land
on opposite sides of a bf16 rounding boundary (one ulp), and near zero — or
after a bias or residual cancels most of the conv value — one ulp of the
larger intermediate is many ulps of the small result. The rule therefore
measures the allowed error in bf16 ulps of the largest magnitude the error
can have been made at:

  ulp(s) = 2^(floor(log2 s) - 7)                       (bf16: 8 significant bits)
  raw:    |y - r| <= 2 ulp(max(|r|, |conv|, 2^-8 RMS(r)))
          (the saved residual sum value = B(B(conv + bias) + residual) is
          measured at max(|r|, |conv|, |main|, 2^-8 RMS(r)))
  fused:  |y - r| <= 4 ulp(max(|r|, |affine|, k*max(|conv|,|main|,|value|), 2^-8 RMS(r)))
          with k = sqrt(C) |gamma_c| / den, which carries a pre-norm error to
          the output's scale.

2 and 4 ulps are the bounds stated for the raw and the fused path. The
2^-8 RMS floor covers results within 1/256 of the layer's RMS of zero,
where a correct fp32 sum of tens of thousands of terms has an absolute
error comparable to the value itself.
"""
from __future__ import annotations

import numpy as np


def b2f(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def ulp_bf16(s: np.ndarray) -> np.ndarray:
    s = np.maximum(np.abs(s).astype(np.float64), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(s)) - 7)


def rms_of(bits) -> float:
    """Root mean square of a bf16 tensor given as bit patterns."""
    r = b2f(bits).astype(np.float64)
    return float(np.sqrt(np.mean(r * r))) if r.size else 0.0


def check(y_bits, ref, *, fused=False, gamma_bits=None, cout=None, what="", rms=None,
          through=("conv",)):
    """Assert the rule; return diagnostics. ref: oracle dict (intermediates=True).
    rms: the RMS of the whole reference output when y / ref are one chunk of
    it (the floor is a property of the layer, not of the chunk).
    through: the oracle intermediates the raw result was rounded through;
    the error is measured in ulps of the largest of them. A raw conv output
    passes through `conv` alone; the saved residual sum `value` =
    B(main + residual) with main = B(conv + bias) passes through conv and
    main, so one ulp of a correct conv can move it by one ulp of main."""
    y = b2f(y_bits).astype(np.float64)
    r = b2f(ref["y"]).astype(np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    if rms is None:
        rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    floor = 2.0 ** -8 * rms
    conv = np.abs(b2f(ref["conv"]).astype(np.float64))
    if fused:
        C = cout if cout is not None else r.shape[-1]
        g = np.abs(b2f(gamma_bits).astype(np.float64))
        den = ref["den"].astype(np.float64).reshape(r.shape[:-1] + (1,))
        k = np.sqrt(C) * g / den
        pre = np.maximum(np.maximum(conv, np.abs(b2f(ref["main"]))), np.abs(b2f(ref["value"])))
        scale = np.maximum.reduce([np.abs(r), np.abs(b2f(ref["affine"]).astype(np.float64)),
                                   k * pre, np.full_like(r, floor)])
        nulp = 4.0
    else:
        terms = [np.abs(r), np.full_like(r, floor)]
        terms += [np.abs(b2f(ref[k]).astype(np.float64)) for k in through]
        scale = np.maximum.reduce(terms)
        nulp = 2.0
    err = np.abs(y - r)
    allowed = nulp * ulp_bf16(scale)
    bad = err > allowed
    # diagnostics in ulps of |r| (floored, so exact zeros do not divide by ~0)
    at = ulp_bf16(np.maximum(np.abs(r), floor))
    diag = {
        "n": int(r.size),
        "bit_identical": float(np.mean(y_bits == ref["y"])) if r.size else 1.0,
        "max_ulp_rule": float(np.max(err / ulp_bf16(scale))) if r.size else 0.0,
        "max_ulp_at_r": float(np.max(err / at)) if r.size else 0.0,
        "mean_signed_ulp": float(np.mean((y - r) / at)) if r.size else 0.0,
    }
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(int(v) for v in i), float(y[tuple(i)]), float(r[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {r.size} outside the rule; "
                             f"first {detail}; diag {diag}")
    return diag


def check_group_norm(y_bits, ref, *, what="", rms=None):
    """GroupNorm (+ SiLU) rule. The GPU forms the affine as an fp32 fma on
    fp32 statistics (mean and 1/sqrt(var + eps) from fp32 per-thread sums
    combined in fp64), the oracle in fp64; either side's value can land on
    the other side of a bf16 rounding boundary, which moves a by one ulp, and
    the SiLU (slope below 1.1) carries that ulp plus its own rounding:

      |y - r| <= 2 ulp(max(|r|, |a|, 2^-8 RMS(r)))

    with a the oracle's rounded norm output. The RMS floor covers outputs
    within 1/256 of the tensor's RMS of zero (and the SiLU's far negative
    tail, where the exact value is below fp32's normal range)."""
    y = b2f(y_bits).astype(np.float64)
    r = b2f(ref["y"]).astype(np.float64)
    a = b2f(ref["a"]).astype(np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    if rms is None:
        rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    scale = np.maximum.reduce([np.abs(r), np.abs(a), np.full_like(r, 2.0 ** -8 * rms)])
    err = np.abs(y - r)
    allowed = 2.0 * ulp_bf16(scale)
    diag = {
        "n": int(r.size),
        "bit_identical": float(np.mean(y_bits == ref["y"])) if r.size else 1.0,
        "max_ulp_rule": float(np.max(err / ulp_bf16(scale))) if r.size else 0.0,
    }
    bad = err > allowed
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(int(v) for v in i), float(y[tuple(i)]), float(r[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {r.size} outside the rule; "
                             f"first {detail}; diag {diag}")
    return diag


def check_fp8(y_bits, ref, sum_abs, *, what="", rms=None):
    """e4m3 operands: the raw rule plus an accumulation term. The gfx950 fp8
    MFMA (32x32x64) does not sum its 64 products exactly: measured on N(0,1)
    operands its error stays below 2^-18.9 of the sum of the products'
    magnitudes (it behaves like aligning a group to its largest product and
    keeping about 20 bits), while bf16 products are summed exactly. So

      |y - r| <= 2 ulp(max(|r|, |conv|, 2^-8 RMS(r))) + 2^-16 * sum_k |x_k w_k|

    (8x the largest measured ratio); sum_abs is that sum per output."""
    y = b2f(y_bits).astype(np.float64)
    r = b2f(ref["y"]).astype(np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    if rms is None:
        rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    conv = np.abs(b2f(ref["conv"]).astype(np.float64))
    scale = np.maximum.reduce([np.abs(r), conv, np.full_like(r, 2.0 ** -8 * rms)])
    allowed = 2.0 * ulp_bf16(scale) + 2.0 ** -16 * np.asarray(sum_abs, dtype=np.float64)
    err = np.abs(y - r)
    diag = {"n": int(r.size), "bit_identical": float(np.mean(y_bits == ref["y"])),
            "max_err_over_sum_abs": float(np.max(err / np.maximum(sum_abs, 1e-30)))}
    bad = err > allowed
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(int(v) for v in i), float(y[tuple(i)]), float(r[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {r.size} outside the rule; "
                             f"first {detail}; diag {diag}")
    return diag


# ------------------------------------------------------------ whole layers

RULE_KEYS = ("y", "conv", "main", "value", "affine", "den")


def oracle_every_pixel(run, M: int, chunk: int, what: str = ""):
    """The oracle over all M output pixels, chunk pixels per call: run(pixels)
    returns the oracle's dict for those pixels; the pieces the parity rules
    read are concatenated ([M, C] bit patterns, den [M])."""
    parts = {k: [] for k in RULE_KEYS}
    for p0 in range(0, M, chunk):
        ref = run(np.arange(p0, min(M, p0 + chunk)))
        for k in RULE_KEYS:
            if k in ref:
                parts[k].append(ref[k])
        if what and (p0 // chunk) % 8 == 0:
            print(f"  oracle {what}: {min(M, p0 + chunk)} of {M} pixels", flush=True)
    return {k: np.concatenate(v) for k, v in parts.items() if v}


def check_every_element(y_bits, ref, *, chunk: int, what: str = "", **kw):
    """The rule of check() on every element of [M, C] outputs, in chunks of
    pixels with the whole layer's RMS floor; returns merged diagnostics."""
    M = ref["y"].shape[0]
    rms = rms_of(ref["y"])
    n = 0
    same = 0.0
    diag = {"max_ulp_rule": 0.0, "max_ulp_at_r": 0.0}
    signed = 0.0
    for p0 in range(0, M, chunk):
        sl = slice(p0, min(M, p0 + chunk))
        part = {k: v[sl] for k, v in ref.items()}
        d = check(y_bits[sl], part, what=f"{what} pixels {sl.start}..{sl.stop - 1}", rms=rms,
                  **kw)
        n += d["n"]
        same += d["bit_identical"] * d["n"]
        signed += d["mean_signed_ulp"] * d["n"]
        diag["max_ulp_rule"] = max(diag["max_ulp_rule"], d["max_ulp_rule"])
        diag["max_ulp_at_r"] = max(diag["max_ulp_at_r"], d["max_ulp_at_r"])
    diag.update(n=n, bit_identical=same / max(n, 1), mean_signed_ulp=signed / max(n, 1))
    return diag
