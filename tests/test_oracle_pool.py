"""The process pool that the full-size GPU parity tests use for the oracle
gives what the oracle gives in-process (CPU)."""
import numpy as np

import oracle_pool
from oracle import formats as fm
from oracle import moe
from decode_moe_mul_amd import synth


def test_pool_expert_job_equals_in_process_oracle():
    H, F = 256, 64
    cols = np.array([0, 5, 17, 100, 255])
    jobs, want = [], []
    for e, (fgu, fd) in enumerate([("q4_k", "q4_0"), ("q6_k", "q8_0"), ("mxfp4", "mxfp4")]):
        wg = synth.normal((F, H), 0.02, 0, synth.GATE, e)
        wu = synth.normal((F, H), 0.02, 0, synth.UP, e)
        wd = synth.normal((H, F), 0.02, 0, synth.DOWN, e)
        X = synth.normal((3 + e, H), 1.0, 0, synth.ACT, e)
        jobs.append((fgu, wg, wu, fd, np.ascontiguousarray(wd[cols]), X))
        r = moe.expert_ffn((fgu, fm.quantize(fgu, wg), fm.quantize(fgu, wu), fd,
                            fm.quantize(fd, wd)), H, F, X)
        want.append((r["o"][:, cols], r["bound_o"][:, cols]))
    got = oracle_pool.run(oracle_pool.expert_job, iter(jobs), inflight=2)
    assert len(got) == len(want)
    for (o, b), (wo, wb) in zip(got, want):
        # (a BLAS product over a row subset may sum in another order)
        assert np.allclose(o, wo, rtol=1e-12, atol=1e-15) and np.allclose(b, wb, rtol=1e-12)
