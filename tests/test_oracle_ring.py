"""Pins for the oracle's delayed-scaling amax-history ring.

The pages give the ring's storage ([hist | scale | counter], AstrAI ops.cu
``pack_quantize_params``), its job (fold this step's amax into hist[idx],
reduce the window, publish the next scale: the same file's commit message) and
the non-finite rule (hip-quant README, "Training-path numerical guards"). The
closed-form sequences below follow from those statements with a max-reduced
window and next scale = max * 2^margin / fmax.
"""
import numpy as np
import pytest

from oracle import fp8, quantize as Q


def _run(samples, length=16, margin=0, fmt=fp8.E4M3):
    st = Q.ring_new(length)
    flag = 0
    scales = []
    for t, a in enumerate(samples):
        nonfinite = not np.isfinite(a)
        st, flag = Q.ring_update(st, t % length, margin, np.float32(a) if np.isfinite(a) else 0.0,
                                 nonfinite, fmt, flag)
        scales.append(float(st[length]))
        assert st[length + 1] == 0.0
    return st, flag, scales


def test_initial_state():
    st = Q.ring_new(16)
    assert st.dtype == np.float32 and st.size == 18
    assert np.all(st[:16] == 0) and st[16] == 1.0 and st[17] == 0.0


def test_constant_amax_gives_closed_form_scale():
    for margin in (0, 1, -2, 5):
        _, flag, scales = _run([3.5] * 20, margin=margin)
        assert flag == 0
        want = np.float32(np.float32(3.5 * 2.0 ** margin) / np.float32(448.0))
        assert all(s == want for s in scales)


def test_spike_forgotten_exactly_len_steps_later():
    length = 16
    samples = [1.0] * 3 + [100.0] + [1.0] * 40
    _, _, scales = _run(samples, length=length)
    hi = np.float32(np.float32(100.0) / np.float32(448.0))
    lo = np.float32(np.float32(1.0) / np.float32(448.0))
    spike = 3
    for t, s in enumerate(scales):
        if spike <= t < spike + length:
            assert s == hi, t
        elif t >= spike + length:
            assert s == lo, t


def test_nonfinite_sample_leaves_state_and_sets_flag():
    st = Q.ring_new(4)
    st, flag = Q.ring_update(st, 0, 0, 2.0, False, fp8.E4M3, 0)
    before = st.copy()
    st2, flag2 = Q.ring_update(st, 1, 0, 0.0, True, fp8.E4M3, 0)
    assert flag2 == 1 and np.array_equal(st2, before)
    st3, flag3 = Q.ring_update(st2, 1, 0, np.float32(np.nan), False, fp8.E4M3, flag2)
    assert flag3 == 1 and np.array_equal(st3, before)
    # sticky: a later good sample updates the ring but does not clear the flag
    st4, flag4 = Q.ring_update(st3, 1, 0, 4.0, False, fp8.E4M3, flag3)
    assert flag4 == 1 and st4[1] == 4.0 and st4[4] == np.float32(4.0) / np.float32(448.0)


def test_all_zero_window_keeps_scale():
    st = Q.ring_new(2)
    st[2] = 0.125
    st2, flag = Q.ring_update(st, 0, 0, 0.0, False, fp8.E4M3, 0)
    assert st2[2] == np.float32(0.125) and flag == 0


def test_overflowing_candidate_keeps_scale_and_flags():
    st = Q.ring_new(2)
    st2, flag = Q.ring_update(st, 0, 10, 3.0e38, False, fp8.E4M3, 0)
    assert st2[2] == 1.0 and flag == 1 and st2[0] == np.float32(3.0e38)


def test_tiny_candidate_is_floored():
    st = Q.ring_new(2)
    st2, _ = Q.ring_update(st, 0, -20, 1e-37, False, fp8.E5M2, 0)
    assert st2[2] == np.float32(2.0 ** -126)


def test_counter_slot_reset():
    st = Q.ring_new(3)
    st[4] = 7.0
    st2, _ = Q.ring_update(st, 2, 0, 1.0, False, fp8.E4M3, 0)
    assert st2[4] == 0.0


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_delayed_quantize_uses_scale_at_call(fmt):
    rng = np.random.default_rng(21)
    st = Q.ring_new(16)
    st[16] = np.float32(0.01)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    q, s_used, amax, st2, flag = Q.quantize_delayed(x, Q.F32, fmt, st, 0, 0, 0)
    assert s_used[0] == np.float32(0.01)
    r = np.float32(1.0) / np.float32(0.01)
    assert np.array_equal(q, fp8.encode((x * r).astype(np.float32), fmt))
    assert amax[0] == np.abs(x).max()
    assert st2[0] == amax[0]
    assert st2[16] == np.float32(amax[0] / np.float32(fp8.fmax(fmt)))
    assert flag == 0


def test_delayed_quantize_with_nonfinite_element():
    st = Q.ring_new(4)
    x = np.ones((2, 16), dtype=np.float32)
    x[1, 3] = np.inf
    q, s_used, amax, st2, flag = Q.quantize_delayed(x, Q.F32, fp8.E4M3, st, 2, 0, 0)
    assert flag == 1 and np.array_equal(st2, st)
    assert amax[0] == 1.0 and q[1, 3] == 0x7E
