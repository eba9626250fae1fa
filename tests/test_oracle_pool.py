"""The multi-process oracle runner gives exactly the single-process oracle's result."""
import numpy as np

import synth
from oracle.pool import OraclePool


def test_pool_equals_single_process(O):
    w16 = synth.half_bits(synth.student_t_weights(48, 1024, 21)).reshape(-1)
    for nbits, g in ((4, 64), (2, 16), (3, 32)):
        ref = O.solve_groups(w16, g, nbits)
        with OraclePool(procs=2) as P:
            got = P.solve_groups(w16, g, nbits, parts=7)       # ragged ranges
            got_b = P.solve_groups(w16, g, nbits, beta=1e4)    # live shrink, reused workers
        for k in ref:
            assert np.array_equal(got[k], ref[k]), k
        ref_b = O.solve_groups(w16, g, nbits, beta=1e4)
        for k in ref_b:
            assert np.array_equal(got_b[k], ref_b[k]), k
