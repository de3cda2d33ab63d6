"""Error measures the parity tolerances are stated in.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix no tolerance.  The bars are "max relative error 1e-4" for fp32
inputs and "2e-2 normwise" for bf16 inputs, read as follows.

* fp32 inputs: componentwise relative error against the magnitude of the
  terms that are summed into each output,
      max_i |g_i - o_i| / a_i  <=  1e-4,
  where a = the oracle evaluated on |x|, |B|, |C|, |D|, |initial_state| (same
  dt and A, so every decay factor is the same positive number).  a_i is then
  exactly the sum of the absolute values of all products that make up o_i,
  the quantity rounding errors of any summation order scale with.  Plain
  fp32 evaluation of the recurrence scores ~1e-7 here; rounding any operand
  to bf16 scores ~1e-3; a dropped or misplaced term scores O(1).
  (A relative error floored at 1e-3 * max|o| was tried first and rejected:
  the textbook fp32 serial recurrence itself scores 1.25e-4 under it for
  headdim 128, dstate 256, so that reading would fail correct fp32 code.)
  Because a_i can be tens of times |o_i|, the fp32 checks also bound the
  floored relative error below (``fp32_floored_bar``): no worse than twice
  what the textbook fp32 recurrence scores on the same inputs, and never
  above the 1e-4 bar where that recurrence meets it.  A change of 1e-3 |o|
  on typical outputs passes the componentwise measure alone but fails the
  pair.
* bf16 inputs: normwise relative error in fp64
      ||g - o||_2 / ||o||_2  <=  2e-2
  applied to y and to the final state separately, and to y also over every
  32-token block of every slice (``block_normwise_err``).
"""
from __future__ import annotations

import numpy as np

FP32_MAX_REL = 1e-4
BF16_NORMWISE = 2e-2


def componentwise_err(got, ref, ref_abs) -> float:
    """max_i |got_i - ref_i| / ref_abs_i (entries with ref_abs_i == 0 must be
    exact; any error there counts as infinite)."""
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    a = np.asarray(ref_abs, dtype=np.float64)
    if o.size == 0:
        return 0.0
    d = np.abs(g - o)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(a > 0, d / np.where(a > 0, a, 1.0), np.where(d > 0, np.inf, 0.0))
    return float(np.max(r))


def max_rel_err(got, ref, floor: float = 1e-3) -> float:
    """Relative error floored at ``floor`` * max|ref| (informational only)."""
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    if o.size == 0:
        return 0.0
    scale = np.maximum(np.abs(o), floor * np.max(np.abs(o)))
    scale = np.where(scale == 0.0, 1.0, scale)
    return float(np.max(np.abs(g - o) / scale))


def fp32_floored_bar(textbook_err: float) -> float:
    """Bar on ``max_rel_err`` for an fp32 result, given the score of the
    textbook fp32 recurrence (``forms.serial_fp32``) on the same inputs:
    1e-4 where that recurrence meets 1e-4, else twice its score."""
    return max(FP32_MAX_REL, 2.0 * textbook_err)


def normwise_err(got, ref) -> float:
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(o.ravel())
    num = np.linalg.norm((g - o).ravel())
    if den == 0.0:
        return float(num)
    return float(num / den)


BLOCK = 32


def block_normwise_err(got, ref, tok_axis: int, block: int = BLOCK):
    """Largest normwise error over blocks of ``block`` tokens of every slice,
    and where it occurs.  The token axis is cut into blocks (the last one
    ragged); every other axis except the last (the feature axis) indexes a
    slice.  With every block under the bar, so is every slice and the whole
    array (squared norms add), but one wrong token row cannot hide in the
    norm of a long sequence."""
    worst, where = 0.0, None
    g_all = np.moveaxis(np.asarray(got), tok_axis, -2)
    o_all = np.moveaxis(np.asarray(ref), tok_axis, -2)
    # one leading index at a time keeps the float64 temporaries small
    lead = g_all.shape[0] if g_all.ndim > 2 else 1
    for i in range(lead):
        g = np.asarray(g_all[i] if g_all.ndim > 2 else g_all, dtype=np.float64)
        o = np.asarray(o_all[i] if o_all.ndim > 2 else o_all, dtype=np.float64)
        L, F = g.shape[-2], g.shape[-1]
        pad = (-L) % block
        if pad:
            widths = [(0, 0)] * (g.ndim - 2) + [(0, pad), (0, 0)]
            g, o = np.pad(g, widths), np.pad(o, widths)
        shp = g.shape[:-2] + ((L + pad) // block, block, F)
        d2 = ((g - o) ** 2).reshape(shp).sum(axis=(-2, -1))
        o2 = (o ** 2).reshape(shp).sum(axis=(-2, -1))
        r = np.sqrt(np.where(o2 > 0, d2 / np.where(o2 > 0, o2, 1.0), d2))
        k = int(np.argmax(r))
        if r.ravel()[k] > worst or where is None:
            worst = float(r.ravel()[k])
            where = ((i,) if g_all.ndim > 2 else ()) + tuple(int(v) for v in np.unravel_index(k, r.shape))
    return worst, where


def parity_error(got, ref, io_dtype: str, ref_abs=None) -> float:
    """Error in the measure that applies to ``io_dtype`` ('f32' or 'bf16').
    fp32 needs ``ref_abs`` (the oracle on absolute-valued inputs)."""
    if io_dtype == "f32":
        if ref_abs is None:
            raise ValueError("the fp32 measure needs the magnitude reference")
        return componentwise_err(got, ref, ref_abs)
    return normwise_err(got, ref)


def tolerance(io_dtype: str) -> float:
    return FP32_MAX_REL if io_dtype == "f32" else BF16_NORMWISE


def abs_inputs(inp: dict) -> dict:
    """Inputs whose oracle result is the magnitude reference of ``inp``."""
    out = dict(inp)
    for k in ("x", "B", "C", "D", "initial_state"):
        if out.get(k) is not None:
            out[k] = np.abs(out[k])
    return out
