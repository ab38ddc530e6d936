"""Plain CPU oracle of the expert-bias controller (fp64, numpy).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the GPU library.

The pages (LongCat-Flash article, itouyu.top / kqgmpj.cn / dhxrcw.cn, section
"Zero-computation experts", bias paragraph) say that each expert's selection bias follows
the expert's recent usage, stays decoupled from the training objective, and is adjusted
in real time by a PID controller, which keeps the parameters activated per token within a
band.  They give neither the error signal nor the gains.  Reading taken here: the
controlled quantity is each expert's share of the step's T*K picks, the set point is a
per-expert target share chosen by the caller, and the textbook discrete PID law acts on
the bias:

  e_i       = target_i - load_i / (T*K)
  I_i      <- I_i + e_i
  b_i      <- b_i + kp*e_i + ki*I_i + kd*(e_i - e_prev_i)
  e_prev_i <- e_i

An expert picked less often than its target share gets a larger bias and is picked more
often on the next step.  Targets on the zero-computation experts set the zero share of the
picks and so the mean number of FFN experts per token.
"""
from __future__ import annotations

import numpy as np


def pid_step(bias, integral, prev_err, load, target, T, K, kp, ki, kd):
    """One controller update (bias paragraph of "Zero-computation experts"); returns the
    new (bias, integral, prev_err) as fp64 arrays."""
    bias = np.asarray(bias, np.float64)
    integral = np.asarray(integral, np.float64)
    prev_err = np.asarray(prev_err, np.float64)
    share = np.asarray(load, np.float64) / float(T * K)
    e = np.asarray(target, np.float64) - share
    integral = integral + e
    bias = bias + (kp * e + ki * integral + kd * (e - prev_err))
    return bias, integral, e


def share_targets(N, Z, zero_share):
    """Per-expert target shares: the FFN experts split 1 - zero_share evenly and the Z
    zero-computation experts split zero_share evenly (all zero if Z = 0)."""
    t = np.empty(N + Z, np.float64)
    t[:N] = (1.0 - (zero_share if Z else 0.0)) / N
    if Z:
        t[N:] = zero_share / Z
    return t
