"""The seeded input generator: Philox known answers, determinism, shapes and
the distributions each workload asks for."""
import numpy as np

import synth


def test_philox_known_answers():
    # known-answer vectors published with the Random123 reference implementation
    # of Philox4x32-10 (Salmon et al., SC'11)
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        assert list(synth.philox_block(ctr, key)) == want


def test_streams_are_slices():
    a = synth.normal_f32(5, 3, 1000)
    b = synth.normal_f32(5, 3, 600, offset=400)
    assert np.array_equal(a[400:], b)
    assert not np.array_equal(a, synth.normal_f32(5, 4, 1000))
    assert not np.array_equal(a, synth.normal_f32(6, 3, 1000))


def test_normal_moments():
    z = synth.normal_f32(9, 1, 400000, 1.0, 0.1)
    assert abs(z.mean() - 1.0) < 1e-3 and abs(z.std() - 0.1) < 1e-3
    assert abs(np.mean((z - 1) ** 4) / 0.1 ** 4 - 3.0) < 0.05  # Gaussian kurtosis


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-40, np.inf], np.float32)
    bits = synth.round_bf16(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert list(back[:4]) == [1.0, 1.0, 1.0 + 2 ** -6, -2.5]  # ties to even
    assert back[5] == np.inf
    f = synth.normal_f32(2, 2, 1000, 0, 0.02)
    nb = synth.normal_bf16(2, 2, 1000, 0, 0.02)
    assert np.array_equal(synth.round_bf16(f), nb)


def test_uniform_range():
    u = synth.uniform_f32(1, 7, 100000)
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.01
    assert np.array_equal(u.astype(np.float64) * 2 ** 24, np.floor(u.astype(np.float64) * 2 ** 24))


def test_tiny_and_params():
    c0 = synth.make_config(0)
    assert c0.hidden.shape == (1, 256) and c0.w_t.shape == (256, 4096) and c0.k == 16
    assert c0.params[0].tolist() == [[8.0, np.float32(0.9), np.float32(0.7), 0.5]]
    p = synth.random_params(4, 256, greedy_rows=64)
    assert (p[:, 2] == 0).sum() == 64
    assert p[:, 0].min() >= 1 and p[:, 0].max() <= 256 and np.all(p[:, 0] == np.floor(p[:, 0]))
    assert p[:, 1].min() >= 0.5 and p[:, 1].max() <= 1.0
    t = p[p[:, 2] > 0, 2]
    assert t.min() >= 0.3 and t.max() <= 1.5
    assert p[:, 3].min() >= 0 and p[:, 3].max() < 1


def test_pad_lanes():
    lanes = synth.pad_lanes(3072, 2880)
    assert lanes.size == 192 and np.all(lanes % 16 == 15)
