"""Seeded generators: determinism and the workload shapes (CPU only)."""
import numpy as np

import synth


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 3.140625], dtype=np.float32)
    b = synth.bf16_bits(x)
    assert list(b) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x4049]
    assert np.array_equal(synth.bf16_to_f32(b)[[0, 3, 4]], x[[0, 3, 4]])


def test_generators_are_deterministic():
    a, b = synth.cfg1(), synth.cfg1()
    assert np.array_equal(a.lens, b.lens) and np.array_equal(a.k, b.k)
    assert np.array_equal(a.q, b.q) and a.pool_seed == b.pool_seed


def test_cfg_shapes_and_ranges():
    c1 = synth.cfg1()
    assert c1.B == 4 and c1.q.shape == (4, 8, 64) and c1.k.dtype == np.float32
    assert np.all((c1.lens >= 2) & (c1.lens <= 257)) and c1.pool_blocks == 128
    c2 = synth.cfg2(B=4)
    full = synth.cfg2.__wrapped__ if hasattr(synth.cfg2, "__wrapped__") else None
    assert c2.q.shape == (4, 64, 128) and c2.k.dtype == np.uint16
    assert np.all((c2.lens >= 512) & (c2.lens <= 4096))
    assert c2.k.shape == (int(c2.lens.sum()), 8, 128)
    c4 = synth.cfg4(B=3)
    assert np.all(c4.lens >= 2048 + 64) and np.all(c4.lens <= 2048 + 512)
    st = c4.seq_start()
    # The duplicated logical rows repeat the same prefix for every sequence.
    assert np.array_equal(c4.k[st[0]:st[0] + 2048], c4.k[st[1]:st[1] + 2048])
    pre, dec = synth.cfg5(S=2, n_decode=3)
    assert list(pre.chunk) == [512, 512] and np.all(pre.prior <= 7680)
    assert pre.q.shape == (1024, 64, 128) and dec.B == 3


def test_cfg3_lengths_and_churn():
    c3 = synth.cfg3_initial(B=256)
    pre = c3.lens - 1
    assert pre.min() >= 16 and pre.max() <= 8192
    assert 700 < np.median(pre) < 1400
    ev = synth.cfg3_churn(1, 256, c3.shape)
    assert len(ev.finished) == 26 and len(set(ev.finished.tolist())) == 26
    assert np.all((ev.new_lens >= 16) & (ev.new_lens <= 128))
    assert ev.new_k[0].shape == (int(ev.new_lens[0]), 8, 128)
