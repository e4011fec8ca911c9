"""The tap machinery used by the full-size GPU checks, exercised on the CPU
with the oracle's own run standing in for the GPU's buffers."""

import numpy as np

import oracle
from persistent_fusion_amd import workloads
from taps import add_taps, check_taps


def _tapped(n_ops=600, sample=(0, 7, 63, 64, 300, 599)):
    wl = workloads.gen_dynamic_dag(seed=5, n_ops=n_ops, n_max=1 << 14, pool_len=1 << 14,
                                   group=100)
    return wl, add_taps(wl, sample)


def test_taps_keep_order_and_deps():
    wl, (twl, taps) = _tapped()
    assert len(twl.ops) == len(wl.ops) + sum(len(t["ins"]) + 1 for t in taps)
    for i, op in enumerate(twl.ops):
        assert all(d < i for d in op.deps)
    # groups still cover the stream contiguously
    assert twl.groups[0][0] == 0 and twl.groups[-1][1] == len(twl.ops)
    for (a0, a1), (b0, b1) in zip(twl.groups, twl.groups[1:]):
        assert a1 == b0
    # the untapped ops appear in their original order
    orig = [op for op in twl.ops if not op.out.buf.startswith("tap_")]
    assert [op.kind for op in orig] == [op.kind for op in wl.ops]


def test_taps_agree_with_the_oracle_run():
    wl, (twl, taps) = _tapped()
    with np.errstate(all="ignore"):
        got = oracle.run(twl)
        assert check_taps(twl, taps, got) == []


def test_taps_catch_a_wrong_output():
    wl, (twl, taps) = _tapped()
    with np.errstate(all="ignore"):
        got = oracle.run(twl)
        t = next(t for t in taps if t["op"].kind in ("add", "mul", "relu"))
        y = got[t["out"]]
        k = int(np.flatnonzero(np.isfinite(y))[0])
        y[k] = np.nextafter(y[k], np.float32(np.inf))
        bad = check_taps(twl, taps, got)
    assert [b[0] for b in bad] == [t["index"]]
