"""The seeded workloads of gdn_inputs with their final gates, for the tests.

gdn_inputs draws the raw gate projections a, b ~ N(0, 1) and the per-head
decay rate; the workloads define the operator's gates from them as
beta = sigmoid(b) and g = ssm_a * softplus(a + ssm_dt) (ssm_dt = 0 unless a
case asks for a gate bias).  The tests evaluate those with the fp64 oracle's
gate activations and round them once to fp32; the GPU and the oracle then
consume the same fp32 values.  Everything else is re-exported unchanged.
"""
from __future__ import annotations

import functools

import numpy as np

import oracle
from gdn_inputs import *  # noqa: F401,F403
import gdn_inputs as _gi


def final_gates(a, b, ssm_a, ssm_dt):
    """(g, beta) in fp32 from the raw projections, via oracle.gates (fp64)."""
    g, beta = oracle.gates(a, b, ssm_a, ssm_dt)
    return g.astype(np.float32), beta.astype(np.float32)


make_case = functools.partial(_gi.make_case, final_gates=final_gates)
make_decode = functools.partial(_gi.make_decode, final_gates=final_gates)
config0 = functools.partial(_gi.config0, final_gates=final_gates)
config1 = functools.partial(_gi.config1, final_gates=final_gates)
config2 = functools.partial(_gi.config2, final_gates=final_gates)
config3 = functools.partial(_gi.config3, final_gates=final_gates)
config4 = functools.partial(_gi.config4, final_gates=final_gates)
