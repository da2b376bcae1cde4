"""Logit decode and per-row token distributions (float64).

Test infrastructure only (see ``oracle/__init__``).

The pages describe the exits L_d, L_i, L_f of one early-exit model as producing
token distributions at every drafted position (HiSpec summary, section 2
"Kernmechanismus"); a distribution is the softmax of that exit's logits at the
sequence's temperature.  Temperature 0 is greedy decoding: the distribution is
the one-hot of the lowest-index maximum (reading of the pages' remark that the
method holds across sampling temperatures, SSD summary section 4
"Robustheit").
"""

import numpy as np

DTYPE_F32 = 0
DTYPE_BF16 = 1


def decode_bf16(bits):
    """bf16 bit patterns (uint16) -> float64: the bf16 value is the float32 whose
    upper 16 bits are the pattern and whose lower 16 bits are zero."""
    bits = np.asarray(bits, dtype=np.uint16)
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(invalid="ignore"):
        return f32.astype(np.float64)


def decode(raw):
    """Raw logits (uint16 holding bf16 bits, float32, or float64 logits that an
    LM head produced in float64) -> float64."""
    raw = np.asarray(raw)
    if raw.dtype == np.uint16:
        return decode_bf16(raw)
    if raw.dtype in (np.float32, np.float64):
        return raw.astype(np.float64)
    raise TypeError(f"unsupported logit storage {raw.dtype}")


def row_distribution(logits, tau):
    """Token distribution of one logit row at temperature ``tau`` (float64).

    tau > 0: P_v = exp((l_v - m)/tau) / sum_w exp((l_w - m)/tau), m = max l.
    tau = 0: one-hot at the lowest index attaining max l.
    """
    l = np.asarray(logits, dtype=np.float64)
    tau = float(tau)
    if tau == 0.0:
        P = np.zeros_like(l)
        P[int(np.argmax(l))] = 1.0          # argmax returns the first maximum
        return P
    if not tau > 0.0:
        raise ValueError("temperature must be >= 0")
    m = np.max(l)
    w = np.exp((l - m) / tau)
    return w / np.sum(w)
