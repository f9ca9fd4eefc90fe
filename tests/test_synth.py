"""The seeded input generators are deterministic and range-independent."""
import numpy as np

import synth


def test_rows_do_not_depend_on_requested_range():
    a = synth.gaussian_rows(9, synth.TAG_MAIN_KV, 0, 1, 0, 3 * synth.CHUNK_ROWS // 2 + 5, 16)
    b = synth.gaussian_rows(9, synth.TAG_MAIN_KV, 0, 1, synth.CHUNK_ROWS - 7, 20, 16)
    c = synth.gaussian_rows(9, synth.TAG_MAIN_KV, 0, 1, 123, 1, 16)
    assert np.array_equal(a[synth.CHUNK_ROWS - 7:synth.CHUNK_ROWS + 13], b)
    assert np.array_equal(a[123:124], c)


def test_seeds_separate_tensors():
    a = synth.main_kv_rows(0, 0, 0, 4, 16)
    b = synth.main_kv_rows(0, 1, 0, 4, 16)
    c = synth.swa_rows(0, 0, 0, 4, 16)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
    assert np.array_equal(a, synth.main_kv_rows(0, 0, 0, 4, 16))


def test_bf16_rounding_helper():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e-39], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(b)
    assert back[0] == 1.0 and back[1] == 1.0          # tie to even
    assert back[2] == 1.0078125 and back[3] == -2.5
    q = synth.q_idx(1, 0, 2, 8, 128)
    assert q.dtype == np.uint16 and q.shape == (2, 8, 128)


def test_c3_lengths():
    wl = synth.workload(3)
    lens = np.array(wl.seq_lens)
    assert len(lens) == 32 and lens.min() >= 32768 and lens.max() < 262144
