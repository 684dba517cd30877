"""Oracle comparison of 16-bit casts over a run of consecutive fp32 bit patterns (used by the
exhaustive GPU cast test; pinned on the CPU by planted mistakes)."""

import numpy as np

import oracle as O


def check_cast_slice(lo, got, got_p):
    """Check one slice of consecutive fp32 patterns starting at ``lo``: ``got`` maps "bf16" and
    "f16" to the device's 16-bit outputs, ``got_p`` is the master copy after the step. Returns None
    when every non-NaN cast equals the oracle's and every NaN stays a NaN, else a message."""
    pats = np.arange(lo, lo + got_p.size, dtype=np.uint64).astype(np.uint32)
    x = pats.view(np.float32)
    nan = (pats & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    for dt, cast, e, mant in (("bf16", O.cast_bf16_rne, 0x7F80, 0x007F),
                              ("f16", O.cast_fp16_rne, 0x7C00, 0x03FF)):
        g, want = got[dt], cast(x)
        ok = nan | (g == want)
        if not ok.all():
            i = int(np.argmin(ok))
            return f"{dt}: pattern {pats[i]:#010x} casts to {g[i]:#06x}, want {want[i]:#06x}"
        gn = g[nan]
        if not (((gn & e) == e).all() and ((gn & mant) != 0).all()):
            return f"{dt}: a NaN lost its NaN-ness"
    if not (nan | (got_p == pats)).all():
        return "non-NaN master changed"
    return None
