"""The seeded input generator: counter-based slicing, row redraws, Zipf
offsets, encoding ranges."""
import numpy as np

import synth


def test_slices_are_independent():
    full = synth.normal_bf16(4, synth.T_GATE, 1001, 0.02, nthreads=3)
    part = synth.normal_bf16(4, synth.T_GATE, 500, 0.02, start=333, nthreads=1)
    assert np.array_equal(full[333:833], part)


def test_row_redraw_touches_one_row():
    a = synth.x_rows(1, 5, 64)
    rd = np.array([0, 0, 2, 0, 0], dtype=np.uint32)
    b = synth.x_rows(1, 5, 64, redraw=rd)
    assert np.array_equal(a[[0, 1, 3, 4]], b[[0, 1, 3, 4]]) and not np.array_equal(a[2], b[2])


def test_normal_moments():
    z = synth.normal_f32(0, 1, 1 << 20, 1.0)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3


def test_zipf_offsets_closed_form():
    """exp(bias/c) = rank^-s / H_s, a probability distribution over ranks."""
    for s in (1.0, 1.5):
        b = synth.zipf_bias(3, 256, s, 1.2)
        p = np.exp(b.astype(np.float64) / 1.2)
        assert abs(p.sum() - 1) < 1e-5
        ranks = np.sort(p)[::-1] * sum(r ** -s for r in range(1, 257))
        assert np.allclose(ranks, np.arange(1, 257) ** -s, rtol=1e-5)


def test_q4_encoding_ranges():
    qw, sc, bi = synth.q4_matrix(2, synth.T_UP, 2, 8, 128, 64, 0.02)
    assert qw.shape == (2, 8, 16) and sc.shape == (2, 8, 2)
    assert np.all(synth.bf16_to_f32(sc) >= 0)
    w = synth.normal_f32(2, synth.T_UP, 2 * 8 * 128, 0.02).reshape(2, 8, 2, 64)
    mn = w.min(axis=3)
    assert np.allclose(synth.bf16_to_f32(bi), mn, rtol=8e-3, atol=0)
