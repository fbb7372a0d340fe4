"""Gate parametrisation of the KDA decode step, fp64 (TEST INFRASTRUCTURE ONLY: imported by
tests, the smoke check and the benchmark's CPU-baseline leg, never by the GPU library).

[LA-Infra] "KDA实现逻辑概述": the forget gate of key channel c of head h is produced from the
token's gate projection forget_b[c], a per-(head, channel) bias dt_bias[h, c] and a per-head
scalar A_log[h]:
    x = forget_b + dt_bias;   z = e^{A_log} x;   forget_log = lower_bound * sigmoid(z),
so forget_log lies in (lower_bound, 0) and the per-step decay alpha = e^{forget_log} in
(e^{lower_bound}, 1). The write gate is beta = sigmoid(write_logit), one per head.
"""
import numpy as np


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def kda_forget_log(forget_b, dt_bias, A_log, lower_bound):
    """forget_b [..., H, dk]; dt_bias [H, dk]; A_log [H]; returns forget_log [..., H, dk]."""
    fb = np.asarray(forget_b, dtype=np.float64)
    x = fb + np.asarray(dt_bias, dtype=np.float64)
    z = np.exp(np.asarray(A_log, dtype=np.float64))[:, None] * x
    return float(lower_bound) * sigmoid(z)
