"""The seeded input generator (CPU only): determinism, distributions, and the
MXFP4 / int8 encoders checked against the pinned decode of the golden E2M1
table."""
import math

import numpy as np

import synth
from oracle_pins import decode_mxfp4_table, golden_e2m1


def test_counter_based_and_deterministic():
    a = synth.normal_f32(0, 5, 0, 1001)
    b = synth.normal_f32(0, 5, 0, 1001)
    assert np.array_equal(a, b)
    one = np.array([synth.lib().synth_normal_at(0, 5, 0, i) for i in range(1001)], np.float32)
    assert np.array_equal(a, one)  # element i is a pure function of its index
    assert not np.array_equal(a, synth.normal_f32(0, 5, 1, 1001))
    assert not np.array_equal(a, synth.normal_f32(1, 5, 0, 1001))
    # chunked generation (offsets not multiples of the pair size) agrees
    tok = synth.normal_bf16(0, 8, 3, 40000)
    assert np.array_equal(tok, synth.f32_to_bf16(synth.normal_f32(0, 8, 3, 40000)))


def test_gaussian_moments():
    z = synth.normal_f32(7, 1, 0, 1 << 20).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    assert abs((np.abs(z) > 2).mean() - 0.0455) < 2e-3


def _mx_step(mag_over_scale):
    a = np.abs(mag_over_scale)
    return np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))


def test_mxfp4_encoder_error_bound():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[3, :32] = 0.0                       # an all-zero group
    w[5, 32:64] *= 1e-30                  # tiny magnitudes
    codes, scales = synth.quant_mxfp4(w)
    dq = decode_mxfp4_table(codes, scales)
    wg = w.astype(np.float64).reshape(64, 8, 32)
    amax = np.abs(wg).max(-1)
    for r in range(64):
        for g in range(8):
            if amax[r, g] == 0:
                assert np.all(dq[r, g * 32:(g + 1) * 32] == 0)
                continue
            X = math.frexp(amax[r, g])[1] - 1 - 2
            assert scales[r, g] == X + 127
            v = wg[r, g] / 2.0 ** X
            d = dq[r, g * 32:(g + 1) * 32] / 2.0 ** X
            sat = np.abs(v) > 6
            assert np.all(np.abs(d[sat]) == 6) and np.all(np.sign(d[sat]) == np.sign(v[sat]))
            ok = np.abs(d - v) <= _mx_step(v) / 2 + 1e-12
            assert np.all(ok[~sat]), (r, g)


def test_mxfp4_round_trip():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(16, 64), dtype=np.uint8)
    # force a magnitude code >= 6 (value 4 or 6) in every group so the scale is recoverable
    codes[:, ::16] = (codes[:, ::16] & 0xF0) | 0x07
    scales = rng.integers(100, 150, size=(16, 4), dtype=np.uint8)
    w = decode_mxfp4_table(codes, scales).astype(np.float32)
    c2, s2 = synth.quant_mxfp4(w)
    assert np.array_equal(s2, scales)
    # -0.0 and +0.0 both decode to zero; compare decoded values and signs of nonzeros
    assert np.array_equal(decode_mxfp4_table(c2, s2), decode_mxfp4_table(codes, scales))


def test_mxfp4_ties_to_even():
    tab = golden_e2m1()
    vals = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -2.5, 0.0, 7.0, 0.5, 3.0, 6.0, -6.0]
    want = [4.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, -0.0, -2.0, 0.0, 6.0, 0.5, 3.0, 6.0, -6.0]
    w = np.array(vals + [0.0] * 16, np.float32)[None, :]
    codes, scales = synth.quant_mxfp4(w)
    assert scales[0, 0] == 127  # max 7.0 -> floor(log2 7) - 2 = 0
    got = decode_mxfp4_table(codes, scales)[0, :16]
    assert np.array_equal(got, np.array(want))
    assert math.copysign(1, got[8]) == -1.0  # the sign of a rounded-away negative is kept
    assert set(np.unique(codes & 15)) <= set(range(16)) and tab.shape == (16,)


def test_int8_encoder():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((33, 100)) * 0.02).astype(np.float32)
    w[4] = 0.0
    q, s = synth.quant_int8(w)
    assert q.dtype == np.int8 and np.all(np.abs(q.astype(int)) <= 127)
    nz = np.arange(33) != 4
    assert np.all(np.abs(q[nz].astype(int)).max(1) == 127)
    assert s[4] == 1.0 and np.all(q[4] == 0)
    err = np.abs(q.astype(np.float64) * s.astype(np.float64)[:, None] - w)
    assert np.all(err <= s.astype(np.float64)[:, None] / 2 * (1 + 1e-6))


def test_zipf_ids():
    V, n, s = 129280, 200000, 1.1
    ids = synth.zipf_ids(0, 9, 0, n, V, s)
    assert ids.min() >= 0 and ids.max() < V
    Hn = (np.arange(1, V + 1, dtype=np.float64) ** -s).sum()
    for r in (1, 2, 10):
        p = r ** -s / Hn
        f = (ids == r - 1).mean()
        assert abs(f - p) < 5 * math.sqrt(p * (1 - p) / n), (r, f, p)


def test_tid2eid_rows_distinct():
    t = synth.tid2eid(0, 10, 0, 5000, 256, 6)
    assert t.shape == (5000, 6) and t.min() >= 0 and t.max() < 256
    assert all(len(set(r)) == 6 for r in t)
    counts = np.bincount(t.ravel(), minlength=256)
    assert counts.min() > 0.7 * counts.mean() and counts.max() < 1.3 * counts.mean()


def test_workload_shapes_tiny():
    L = synth.make_layer(synth.WORKLOADS["tiny"])
    wl = L.wl
    assert L.w13_codes.shape == (16, 256, 128) and L.w13_scales.shape == (16, 256, 8)
    assert L.w2_codes.shape == (16, 256, 64) and L.w2_scales.shape == (16, 256, 4)
    assert L.sh_w13.shape == (256, 256) and L.sh_w2.shape == (256, 128)
    routed = L.w13_codes.nbytes + L.w13_scales.nbytes + L.w2_codes.nbytes + L.w2_scales.nbytes
    assert routed == 835_584
    assert synth.make_tokens(wl).shape == (16, 256)
