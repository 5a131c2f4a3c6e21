"""The seeded input generator (host side): published known-answer vectors of
Philox4x32-10, index addressability, and the moments of the deviates.  The
generator's bits are inputs, not results; its distribution is checked
statistically only (parity of the optimizer never depends on it)."""
import numpy as np

import synth


def test_philox_known_answers():
    # Known-answer vectors distributed with the Random123 library for
    # philox4x32 with 10 rounds (Salmon et al., SC'11).
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        assert synth.philox4x32_10(ctr, key) == want


def test_index_addressable_and_bf16_is_truncation():
    kw = dict(stream=3, block=7, purpose=synth.PURPOSE_GRAD, step=5, sigma=1e-3)
    full = synth.normal_f32(10000, **kw)
    part = synth.normal_f32(100, start=4321, **kw)
    assert np.array_equal(full[4321:4421], part)
    idx = np.array([0, 9999, 17, 5000], np.uint64)
    assert np.array_equal(synth.normal_f32_at(idx, **kw), full[idx.astype(np.int64)])
    b = synth.normal_bf16(10000, **kw)
    assert np.array_equal(b, (full.view(np.uint32) >> 16).astype(np.uint16))
    assert np.array_equal(synth.normal_bf16_at(idx, **kw), b[idx.astype(np.int64)])


def test_streams_blocks_steps_are_independent_draws():
    base = dict(stream=1, block=0, purpose=2, step=1, sigma=1.0)
    a = synth.normal_f32(4096, **base)
    for k, val in (("stream", 2), ("block", 1), ("purpose", 0), ("step", 2)):
        b = synth.normal_f32(4096, **dict(base, **{k: val}))
        assert abs(np.corrcoef(a, b)[0, 1]) < 0.06, k
        assert not np.array_equal(a, b)


def test_moments():
    x = synth.normal_f32(1 << 20, stream=0, block=0, purpose=0, step=0, sigma=0.02).astype(np.float64)
    assert abs(x.mean()) < 0.01 * 0.02
    assert abs(x.std() / 0.02 - 1) < 0.01
    # Irwin-Hall(8): excess kurtosis -1.2/8 = -0.15, support +-sqrt(24) sigma
    k = np.mean((x / x.std()) ** 4) - 3
    assert abs(k + 0.15) < 0.02
    assert np.max(np.abs(x)) <= np.sqrt(24.0) * 0.02 * 1.0001


def test_raw_words_follow_the_same_counter():
    """philox_words(n) is Philox4x32-10 at counter (index lo, index hi,
    block, purpose << 24 | step), key (seed, stream), element by element."""
    w = synth.philox_words(5, stream=7, block=3, purpose=synth.PURPOSE_EDGE, step=9, start=(1 << 32) - 2)
    for k in range(5):
        i = (1 << 32) - 2 + k
        want = synth.philox4x32_10([i & 0xFFFFFFFF, i >> 32, 3, (synth.PURPOSE_EDGE << 24) | 9], [synth.SEED, 7])
        assert list(w[k]) == want
