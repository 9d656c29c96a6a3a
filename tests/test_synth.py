"""The seeded input generators hold what they claim (checked through the
oracle's own field decoders): the edge-case weights reach the ends of the
ranges the formats allow."""
import numpy as np

import oracle
import synth


def test_q6k_full_range_scales():
    N, K = 40, 1024
    w = synth.q6k_rows_full_range(N, K, 1, "cover").view(-1, 210)
    scs = np.stack([oracle.q6k_fields(w[i].numpy())[1] for i in range(w.shape[0])]).reshape(N, 4, 16)
    assert scs.min() == -128 and scs.max() == 127
    assert np.all(scs[:, 0] == np.array([-128, 127] * 8))
    assert np.all(scs[:, 1] >= 64) and np.all(scs[:, 2] <= -65)
    assert scs[:, 3].min() < -100 and scs[:, 3].max() > 100


def test_q4k_log_uniform_scales_reach_f16_subnormals():
    w = synth.q4k_rows(40, 1024, 1, "cover", d_range=(1e-7, 1e-1), dmin_range=(1e-7, 1e-1), log=True).view(-1, 144)
    f = [oracle.q4k_fields(w[i].numpy()) for i in range(w.shape[0])]
    for v in (np.array([x[0] for x in f]), np.array([x[1] for x in f])):
        assert v.min() < 1e-6 and v.max() > 1e-2
        assert 0.3 < np.mean(v < 2.0 ** -14) < 0.7  # f16 subnormals
        assert np.all(v > 0)
    # the log-uniform draw: roughly equal counts per decade
    d = np.array([x[0] for x in f])
    counts = np.histogram(np.log10(d), bins=6, range=(-7, -1))[0]
    assert counts.min() > 0.5 * counts.mean()


def test_default_generators_unchanged_ranges():
    w = synth.q6k_rows(10, 512, 2, "plain").view(-1, 210)
    scs = np.stack([oracle.q6k_fields(w[i].numpy())[1] for i in range(w.shape[0])])
    assert scs.min() >= -64 and scs.max() <= 63
    w4 = synth.q4k_rows(10, 512, 2, "plain").view(-1, 144)
    d = np.array([oracle.q4k_fields(w4[i].numpy())[0] for i in range(w4.shape[0])])
    assert d.min() >= 1e-3 * (1 - 2 ** -10) and d.max() <= 1e-2 * (1 + 2 ** -10)
