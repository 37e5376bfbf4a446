"""Helpers shared by the tests: oracle-side views of the synthetic inputs."""
import numpy as np

from synth import inputs as si


def oracle_arrays(w, li=None):
    """(q_rows, K, V, P, xs, xo) in fp64 for the oracle from the seeded inputs."""
    if li is None:
        li = si.make_layer_inputs(w)
    Qf = si.bf16_to_f64(li.Q) if li.Q is not None else None

    def q_rows(r0, r1):
        if Qf is not None:
            return Qf[r0:r1]
        return si.bf16_to_f64(si.gen_q(w, r0, r1))

    K = si.bf16_to_f64(li.K)
    V = si.bf16_to_f64(li.V)
    P = None if li.P is None else li.P.astype(np.float64)
    xs = None if li.xa_scale is None else li.xa_scale.astype(np.float64)
    xo = None if li.xa_offset is None else li.xa_offset.astype(np.float64)
    return q_rows, K, V, P, xs, xo
