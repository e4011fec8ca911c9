"""Pins of the oracle's checkers: the per-op local check, the end-to-end
comparison and the GEMV weight cache.

A checker that accepts everything would make every parity test pass, so each
one is shown here to reject plausible mistakes: a result off by one unit in
the last place of an exact op, a transposed weight matrix, a dropped scale
factor, a dropped gain, a flipped sign in the rotation, a softmax row shifted
by one position.  The mistakes are planted on the CPU, into a copy of the
oracle's own outputs, which stand in for a correct device result.
"""

from dataclasses import replace

import numpy as np

import oracle
from oracle.interpreter import f32_to_bf16, bf16_to_f32, out_positions
from persistent_fusion_amd import workloads


def small_decode():
    # two layers, three tokens, every activation in its own buffer
    return workloads.gen_decode(seed=3, layers=2, hidden=128, heads=2, head_dim=64, ffn=256,
                                kv_len=16, tokens=3, distinct=True)


def first_index(wl, kind, skip=0):
    idx = [i for i, op in enumerate(wl.ops) if op.kind == kind]
    return idx[skip]


def state_before(wl, final, i):
    """The buffers as op i sees them: initial contents plus the outputs of
    ops 0..i-1 (write-once workload)."""
    st = {k: v.copy() for k, v in wl.buffers.items()}
    for op in wl.ops[:i]:
        if oracle.out_len(op):
            pos = out_positions(op)
            st[op.out.buf][pos] = final[op.out.buf][pos]
    return st


def plant(wl, final, i, values):
    """A device result that is right except for op i, which wrote `values`:
    ops after i run (in the oracle) on what op i wrote, as they would on the
    device."""
    got = state_before(wl, final, i)
    op = wl.ops[i]
    got[op.out.buf][out_positions(op)] = values
    for later in wl.ops[i + 1:]:
        oracle.apply_op(later, got, wl.dtypes)
    return got


def bad_ops(wl, got):
    return sorted({b[0] for b in oracle.local_check(wl, got, oracle.compare)})


def test_local_check_accepts_the_oracle_itself():
    wl = small_decode()
    final = oracle.run(wl)
    assert bad_ops(wl, final) == []


def test_local_check_rejects_one_ulp_in_an_exact_op():
    wl = small_decode()
    final = oracle.run(wl)
    i = first_index(wl, "add")
    op = wl.ops[i]
    vals = final[op.out.buf][out_positions(op)].copy()
    vals[5] = vals[5] + 1  # next bf16 bit pattern
    assert bad_ops(wl, plant(wl, final, i, vals)) == [i]


def test_local_check_rejects_a_transposed_weight_matrix():
    wl = small_decode()
    final = oracle.run(wl)
    i = first_index(wl, "gemv", skip=1)  # the square output projection
    op = wl.ops[i]
    M, K = op.dims
    assert M == K
    st = state_before(wl, final, i)
    W = bf16_to_f32(st[op.aux.buf][op.aux.off:op.aux.off + M * K]).astype(np.float64).reshape(M, K)
    x = bf16_to_f32(st[op.ins[0].buf][op.ins[0].off:op.ins[0].off + K]).astype(np.float64)
    wrong = f32_to_bf16((W.T @ x).astype(np.float32))
    assert bad_ops(wl, plant(wl, final, i, wrong)) == [i]


def _wrong_by(wl, final, i, **changes):
    """Output of op i computed by the oracle with some fields changed."""
    st = state_before(wl, final, i)
    op = replace(wl.ops[i], **changes)
    oracle.apply_op(op, st, wl.dtypes)
    return st[op.out.buf][out_positions(op)].copy()


def test_local_check_rejects_a_dropped_score_scale():
    wl = small_decode()
    final = oracle.run(wl)
    i = first_index(wl, "attn_score", skip=2)
    assert bad_ops(wl, plant(wl, final, i, _wrong_by(wl, final, i, alpha=1.0))) == [i]


def test_local_check_rejects_a_dropped_gain():
    wl = small_decode()
    final = oracle.run(wl)
    i = first_index(wl, "rmsnorm", skip=1)
    # the gain buffer replaced by the input row itself: a different vector
    op = wl.ops[i]
    assert bad_ops(wl, plant(wl, final, i, _wrong_by(wl, final, i, aux=op.ins[0]))) == [i]


def test_local_check_rejects_a_flipped_rotation():
    wl = small_decode()
    final = oracle.run(wl)
    i = first_index(wl, "rope", skip=3)
    op = wl.ops[i]
    st = state_before(wl, final, i)
    n, h = op.n, op.row_len
    x = bf16_to_f32(st[op.ins[0].buf][op.ins[0].off:op.ins[0].off + n]).reshape(-1, h)
    tab = st[op.aux.buf][op.aux.off:op.aux.off + h]
    c, s = tab[:h // 2], tab[h // 2:]
    x1, x2 = x[:, :h // 2], x[:, h // 2:]
    y = np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=1).astype(np.float32)  # angle -p
    assert bad_ops(wl, plant(wl, final, i, f32_to_bf16(y.reshape(-1)))) == [i]


def test_local_check_rejects_a_shifted_softmax_row():
    wl = small_decode()
    final = oracle.run(wl)
    i = first_index(wl, "row_softmax", skip=1)
    op = wl.ops[i]
    vals = final[op.out.buf][out_positions(op)].copy().reshape(op.rows, op.row_len)
    vals[1] = np.roll(vals[1], 1)
    assert bad_ops(wl, plant(wl, final, i, vals.reshape(-1))) == [i]


def test_local_check_rejects_a_relative_error_above_1e_5_in_fp32():
    # a fp32 tolerance-class op: exp on a dynamic-DAG queue
    wl = workloads.gen_dynamic_dag(seed=5, n_ops=60, n_min=256, n_max=2048, distinct_outputs=True)
    final = oracle.run(wl)
    assert bad_ops(wl, final) == []
    i = next(k for k, op in enumerate(wl.ops) if op.kind == "exp")
    op = wl.ops[i]
    vals = final[op.out.buf][out_positions(op)].copy()
    j = int(np.argmax(np.abs(vals)))
    vals[j] = np.float32(vals[j] * (1 + 3e-5))
    assert bad_ops(wl, plant(wl, final, i, vals)) == [i]
    # within the bound: 3 units in the last place of fp32 (about 1.8e-7)
    vals = final[op.out.buf][out_positions(op)].copy()
    vals[j] = np.nextafter(np.nextafter(np.nextafter(vals[j], np.float32(np.inf)),
                                        np.float32(np.inf)), np.float32(np.inf))
    assert bad_ops(wl, plant(wl, final, i, vals)) == []


def test_weight_cache_gives_the_same_run():
    wl = small_decode()
    with_cache = oracle.run(wl)
    # a run without the cache: every op applied on its own
    bufs = {k: v.copy() for k, v in wl.buffers.items()}
    for op in wl.ops:
        oracle.apply_op(op, bufs, wl.dtypes)
    for name in wl.buffers:
        assert np.array_equal(with_cache[name].view(np.uint8), bufs[name].view(np.uint8)), name


def test_weight_cache_skips_written_buffers():
    wl = small_decode()
    c = oracle.WeightCache.for_workload(wl)
    written = {op.out.buf for op in wl.ops}
    assert not (c.frozen & written)
    assert {name for name in wl.buffers if name.startswith("W")} <= c.frozen
    assert {name for name in wl.buffers if name.startswith(("K", "V"))} <= written


def test_end_to_end_counts():
    rng = np.random.default_rng(0)
    o = rng.standard_normal(1000).astype(np.float32)
    r = oracle.end_to_end(o, o.copy(), "f32")
    assert r.count == 0 and r.bit_equal == 1000 and r.rel_l2 == 0.0
    g = o.copy()
    g[7] = np.float32(g[7] * 1.02)           # 2% off: outside 1e-5
    g[8] = np.nextafter(g[8], np.float32(np.inf))  # one ulp: inside
    r = oracle.end_to_end(g, o, "f32")
    assert r.count == 1 and r.bit_equal == 998
    assert abs(r.max_rel - 0.02) < 1e-6
    # classes must match; NaN matches NaN
    g = o.copy()
    w = o.copy()
    g[0], w[0] = np.nan, np.nan
    g[1] = np.inf
    r = oracle.end_to_end(g, w, "f32")
    assert r.count == 1 and r.bit_equal == 999
    # bf16: 1e-2 relative
    ob = f32_to_bf16(o)
    gb = ob.copy()
    gb[3] = gb[3] + 1  # one bf16 ulp, at most 2^-7 relative: inside
    assert oracle.end_to_end(gb, ob, "bf16").count == 0
    gb[4] = f32_to_bf16(np.array([bf16_to_f32(ob[4:5])[0] * 1.05], np.float32))[0]
    assert oracle.end_to_end(gb, ob, "bf16").count == 1
