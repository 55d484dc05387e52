"""The chained form of split calls and its workspace's epoch word, on the GPU.

A chained split call tags the words it publishes with the previous call's tag
plus one (never 0), held in the workspace's first word, and its last
workgroup stores that tag there for the next call.  The tests start from
fresh workspaces filled with one 32-bit pattern and check the tag sequence
and that repeated calls on one workspace give the same results, which match
the oracle.
"""
import numpy as np
import pytest
import torch

import reverse_linear_recurrence_amd as rl
from gpu_common import (DEFAULT_PARAMS, TOL, assert_close, params32, random_inputs, run_oracle,
                        to_device)
from test_gpu_split import assert_split, plain_by_window

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def chained():
    prev = rl.rlca_set_chained(True)
    yield
    rl.rlca_set_chained(prev)


@pytest.mark.parametrize("N,T", [(2, 65536), (130, 32768)])
@pytest.mark.parametrize("fill", [0x00000000, 0x7FC00000, 0xFFFFFFFF, 0x3F800000])
def test_chained_calls_advance_the_epoch_from_any_fill(fill, N, T):
    # A fresh workspace filled with one 32-bit pattern (zeros, NaN, all ones,
    # 1.0f): the first chained call's tag is the pattern plus one (0 skipped),
    # each later call's the previous plus one, and every call on the same
    # workspace gives the same results.  130 rows: the last workgroup waits
    # on the rows in chunks of 64 (two whole, one of 2).
    p = params32(DEFAULT_PARAMS)
    host = random_inputs("gae", N, T, 811, "f32", p_term=0.001, p_trunc=0.001, bootstrap=False)
    dev = to_device(host)
    ref = run_oracle("gae", host, p)
    ws = rl.split_workspace(N, T)
    ws.view(torch.int32).fill_(np.array(fill, dtype=np.uint32).view(np.int32).item())
    expect = fill
    first = None
    for i in range(3):
        expect = expect + 1 if expect + 1 < (1 << 32) else 1
        got = plain_by_window("gae", dev, p, ws)
        assert_split(ws, N, T, "f32", "gae")
        epoch = ws[:2].view(torch.int32).cpu().numpy().view(np.uint32)
        assert epoch[0] == expect and epoch[1] == 0, (i, hex(epoch[0]), hex(expect))
        if first is None:
            first = got
            assert_close(got, ref, TOL["f32"], "gae/chained fill %#x" % fill)
        else:
            for k in first:
                assert np.array_equal(got[k], first[k]), (i, k)
