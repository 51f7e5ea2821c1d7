"""The library's kernel-timing switch on the GPU: every launch of a profiled step is
recorded in launch order with its class, the timed step gives the same outputs as an
untimed one, and launches past the requested count run untimed."""
import numpy as np
import pytest

from verifier_block_forward_amd import configs
from tests.gpu_harness import Prepared, torch

pytestmark = pytest.mark.gpu


def test_profile_records_every_launch():
    from verifier_block_forward_amd import dbf
    t = torch()
    cfg = configs.C0
    prep = Prepared(cfg)
    plain = prep.run()
    print("\n[profile] c0 block, profiled", flush=True)
    dbf.profile_start(4096)
    timed = prep.run()
    recs = dbf.profile_stop(4096)
    assert np.array_equal(plain["h_final"], timed["h_final"])
    classes = {c for c, _, _ in recs}
    assert {"projections", "attention", "row_kernels"} <= classes, classes
    assert all(np.isfinite(us) and 0.0 < us < 1e5 for _, _, us in recs), recs
    names = [n for _, n, _ in recs]
    assert names.count("k_attn") == cfg.n_layers
    # a cap below the launch count times only the first launches
    dbf.profile_start(3)
    prep.run()
    assert len(dbf.profile_stop(4096)) == 3
    # profiling off: nothing recorded
    prep.run()
    t.cuda.synchronize()
    dbf.profile_start(8)
    assert dbf.profile_stop() == []
