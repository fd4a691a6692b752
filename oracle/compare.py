"""The parity bar between a device result and the oracle (test infrastructure).

  fp64 (parameters, m, v):       bit-exact.
  fp32 (master / parameter, m, v): |got - ref| <= 1e-6 * max(1, |ref|); the
                                   number of bit-identical elements and the
                                   largest distance in ulps are reported too.
  bf16 / fp16 (gathered parameters): at most 1 ulp from the oracle's rounded
                                   value (distance between the ordered bit
                                   patterns).
NaN on both sides counts as equal.
"""
import numpy as np

F32_REL = 1e-6


def _ordered(bits, width):
    """Map IEEE bit patterns to integers that are monotonic in the value."""
    b = bits.astype(np.int64)
    sign = np.int64(1) << (width - 1)
    return np.where(b & sign, -(b & (sign - 1)), b)


def ulp_distance(got, ref):
    if got.dtype == np.float64:
        w, gi, ri = 64, got.view(np.uint64), ref.view(np.uint64)
    elif got.dtype == np.float32:
        w, gi, ri = 32, got.view(np.uint32), ref.view(np.uint32)
    elif got.dtype == np.uint16:
        w, gi, ri = 16, got, ref
    else:
        raise TypeError(got.dtype)
    if w == 64:
        # int64 arithmetic cannot hold every fp64 distance; clip
        g = np.where(gi >> 63, -(gi & 0x7FFFFFFFFFFFFFFF).astype(np.float64),
                     gi.astype(np.float64))
        r = np.where(ri >> 63, -(ri & 0x7FFFFFFFFFFFFFFF).astype(np.float64),
                     ri.astype(np.float64))
        return np.abs(g - r)
    return np.abs(_ordered(gi, w) - _ordered(ri, w))


def compare(name, got, ref, kind):
    """kind: 'exact', 'f32', 'bf16' or 'fp16'. Returns a stats dict; raises
    AssertionError when the bar is not met."""
    got = np.ascontiguousarray(got)
    ref = np.ascontiguousarray(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    n = got.size
    if kind in ("bf16", "fp16"):
        assert got.dtype == np.uint16 and ref.dtype == np.uint16
        inf_bits = 0x7F80 if kind == "bf16" else 0x7C00
        nan_g = (got & 0x7FFF) > inf_bits
        nan_r = (ref & 0x7FFF) > inf_bits
        d = ulp_distance(got, ref)
        d = np.where(nan_g & nan_r, 0, d)
        bad = np.flatnonzero((d > 1) | (nan_g != nan_r))
        stats = dict(name=name, n=n, bitexact=int(np.sum(d == 0)), max_ulp=int(d.max(initial=0)))
        assert bad.size == 0, (f"{name}: {bad.size} of {n} {kind} elements beyond 1 ulp; "
                               f"first at {bad[:5]}: got {got[bad[:5]]} ref {ref[bad[:5]]}")
        return stats
    gv = got.view(np.uint8).reshape(n, -1) if n else got
    same = np.all(gv == ref.view(np.uint8).reshape(n, -1), axis=1) if n else np.zeros(0, bool)
    both_nan = np.isnan(got) & np.isnan(ref)
    same = same | both_nan
    stats = dict(name=name, n=n, bitexact=int(same.sum()))
    if kind == "exact":
        bad = np.flatnonzero(~same)
        if bad.size:
            i = bad[:5]
            raise AssertionError(f"{name}: {bad.size} of {n} elements not bit-exact; first at {i}:"
                                 f" got {got[i]!r} ref {ref[i]!r}")
        stats["max_ulp"] = 0
        return stats
    assert kind == "f32", kind
    with np.errstate(invalid="ignore", over="ignore"):  # inf - inf where both are inf
        diff = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        lim = F32_REL * np.maximum(1.0, np.abs(ref.astype(np.float64)))
    bad = np.flatnonzero(~(same | (diff <= lim)))
    stats["max_abs"] = float(np.nanmax(diff, initial=0.0)) if n else 0.0
    stats["max_ulp"] = int(np.max(np.where(same, 0, ulp_distance(got, ref)), initial=0))
    if bad.size:
        i = bad[:5]
        raise AssertionError(f"{name}: {bad.size} of {n} beyond 1e-6*max(1,|ref|); first at {i}:"
                             f" got {got[i]!r} ref {ref[i]!r}")
    return stats
