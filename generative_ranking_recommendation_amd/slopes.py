"""ALiBi slope schedule ("一、 GenRank [2025]", section 1.4.2: m_h = 2^(-8(h+1)/H); for
H = 8 the slopes are 1/2 .. 1/256).  The time slopes are the position slopes times a
caller-chosen ratio."""
import numpy as np


def alibi_slopes(H: int, time_ratio: float = 0.25):
    sp = np.exp2(-8.0 * (np.arange(H, dtype=np.float64) + 1.0) / H)
    return sp.astype(np.float32), (sp * time_ratio).astype(np.float32)
