"""Borderline certificates for accepted meshes that differ in binary32.

The binary32 solves (the neural field, HIRES with Rosenbrock23) cannot be
bitwise: the matrix cores' summation order and the kernel's tanh differ from
any CPU code in the last bits.  So the GPU's accepted mesh is compared with
the oracle's binary32 instantiation step by step, and wherever the two part,
the oracle's own attempt trace must show a decision that rounding can flip:

* the oracle's msq at one of the attempts that decided the diverging step
  (from the attempt that accepted the previous step through the one that
  accepted this step) is within its rounding uncertainty of 1 (the accept
  test), or
* the controller factor 0.9 msq^(-1/q) at one of those attempts is within
  its rounding uncertainty of a boundary of what the solve does with it: a
  point of the 8-bit truncation grid, or the clamps 0.2, 10 and 1.

The rounding uncertainty of msq is derived from the trace's floor, the mean
square of s kabs_c / sc_c (kabs_c: the sizes of the terms the embedded
error combination cancels): an estimate computed from stages that are each
off by C units of roundoff can be off by C u kabs_c per component, so with
F = (C u)^2 floor the relative uncertainty of msq is 2 sqrt(F / msq) + F / msq.
C = 16 (u = 2^-24): the GPU's stages differ from the oracle's by a few units
of roundoff (matrix-core summation order, the tanh rule, states carried over
from earlier steps).  The factor's relative uncertainty is that of msq over q.
A divergence without such a borderline decision is a real mesh difference
and fails the test.
"""
import numpy as np

U32 = 2.0 ** -24
C_ROUND = 16.0


def _grid_distance(x):
    """Relative distance from x > 0 to the nearest point of the binary32
    8-explicit-bit truncation grid (m 2^(e - 8), m integer)."""
    m, e = np.frexp(x)  # x = m 2^e, m in [1/2, 1)
    scaled = m * 512.0  # 9 significant bits: 256 <= scaled < 512
    return min(scaled - np.floor(scaled), np.ceil(scaled) - scaled) / scaled


def attempt_is_borderline(msq, fac, floor_, q, prev_rejected):
    if not (np.isfinite(msq) and msq > 0):
        return True
    F = (C_ROUND * U32) ** 2 * floor_
    rel = 2.0 * np.sqrt(F / msq) + F / msq  # relative uncertainty of msq
    if abs(msq - 1.0) <= rel * msq:
        return True
    rf = rel / q  # relative uncertainty of the factor
    bounds = [0.2, 10.0] + ([1.0] if prev_rejected else [])
    if any(abs(fac - b) <= rf * b for b in bounds):
        return True
    return _grid_distance(fac) <= rf


def first_divergence(h_gpu, h_orc):
    """Index of the first accepted step whose size differs (bitwise), or None."""
    m = min(len(h_gpu), len(h_orc))
    for i in range(m):
        if h_gpu[i] != h_orc[i]:
            return i
    return None if len(h_gpu) == len(h_orc) else m


def certify(trace, h_gpu, q):
    """(ok, info) for one trajectory: the GPU's accepted steps h_gpu against the
    oracle's trace (oracle.trace); ok if the meshes agree or part at a
    borderline decision of the oracle."""
    acc = trace["acc"]
    h_orc = trace["h"][acc].astype(np.float32)
    i = first_divergence(np.asarray(h_gpu, np.float32), h_orc)
    if i is None:
        return True, "same mesh"
    acc_idx = np.flatnonzero(acc)
    lo = acc_idx[i - 1] if i >= 1 else 0
    hi = acc_idx[i] if i < len(acc_idx) else len(acc) - 1
    prev_rej = False
    for a in range(len(acc)):
        if lo <= a <= hi and attempt_is_borderline(trace["msq"][a], trace["fac"][a],
                                                   trace["floor"][a], q, prev_rej):
            return True, f"step {i}: attempt {a} borderline (msq {trace['msq'][a]:.3e})"
        prev_rej = not acc[a]
    return False, (f"step {i}: no borderline decision in attempts {lo}..{hi} "
                   f"(msq {trace['msq'][lo:hi + 1]}, floor {trace['floor'][lo:hi + 1]})")
