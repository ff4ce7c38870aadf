"""The noise contract's coefficient table as the GPU library compiles it
(sparsity_masks_weights_amd/csrc/maskgs_gumbel_table.inc) against the oracle's
own table: the two sides build it independently (a Python generator next to
the kernels, the C oracle at load time) from the same closed forms, and must
agree bit for bit, or the kernels' noise would not be the oracle's."""
import os
import re
import sys

import numpy as np

from conftest import REPO

CSRC = os.path.join(REPO, "sparsity_masks_weights_amd", "csrc")
INC = os.path.join(CSRC, "maskgs_gumbel_table.inc")


def _parse_inc():
    rows = []
    with open(INC) as f:
        for line in f:
            m = re.match(r"\{(.*)\},", line.strip())
            if m:
                rows.append([float.fromhex(t.strip().rstrip("f")) for t in m.group(1).split(",")])
    return np.array(rows, dtype=np.float64)


def test_compiled_table_equals_the_oracle_table(orc):
    inc = _parse_inc()
    assert inc.shape == (2 * 24 * 32, 4)
    # every literal is an fp32 value written exactly
    assert np.array_equal(inc.astype(np.float32).astype(np.float64), inc)
    ref = orc.gumbel_coef().reshape(-1, 4)
    assert np.array_equal(inc.astype(np.float32).view(np.uint32), ref.view(np.uint32))


def test_generator_reproduces_the_committed_table():
    sys.path.insert(0, CSRC)
    try:
        import gen_gumbel_table
    finally:
        sys.path.remove(CSRC)
    with open(INC) as f:
        assert f.read() == gen_gumbel_table.render()
