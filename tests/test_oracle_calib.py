"""Pins for the oracle's filter rules (Q-Filters page, "Calibrated — the paper's
actual mechanism", "Key-SVD fallback", "Evidence").

Closed forms (rank-1 activations), the planted-geometry thresholds the pages
state (signed cosine > 0.99 with sign tracking; the no-centring contrast; the
key-SVD fallback losing a pure drift direction, cosine < 0.3), and GQA averaging
(identity, unit norm, contiguous grouping)."""
import numpy as np
import pytest

from oracle import calib

D = 128


def _unit(x):
    return x / np.linalg.norm(x)


def test_rank_one_closed_form():
    rng = np.random.default_rng(0)
    for _ in range(5):
        a = rng.standard_normal(300)
        b = rng.standard_normal(D)
        f = calib.qfilter_one_head(np.outer(a, b))
        want = np.sign(a.sum()) * _unit(b)
        assert np.allclose(f, want, atol=1e-12)


@pytest.mark.parametrize("orient", [1.0, -1.0])
def test_planted_query_drift_recovered_with_sign(orient):
    rng = np.random.default_rng(1)
    H, N = 4, 3000
    mus = np.stack([_unit(rng.standard_normal(D)) for _ in range(H)])
    drift = rng.uniform(0.5, 2.0, (H, N, 1))
    acts = orient * drift * mus[:, None, :] + 0.5 * rng.standard_normal((H, N, D))
    f = calib.compute_qfilters(acts)
    for h in range(H):
        cos = float(f[h] @ (orient * mus[h]))
        assert cos > 0.99, cos
        assert abs(np.linalg.norm(f[h]) - 1) < 1e-12


def test_no_mean_centering_returns_drift_axis_not_variance_axis():
    rng = np.random.default_rng(2)
    N = 4000
    e1, e2 = np.eye(D)[0], np.eye(D)[1]
    q = 3.0 * e1 + 2.0 * rng.standard_normal((N, 1)) * e2 + 0.1 * rng.standard_normal((N, D))
    f = calib.qfilter_one_head(q)
    assert f @ e1 > 0.99                          # the paper's estimator: drift axis, right sign
    centred = calib.estimate_filter_dir(q)        # a centring estimator on the same data
    assert abs(centred @ e2) > 0.99 and abs(centred @ e1) < 0.1


def test_key_svd_loses_pure_drift_direction():
    rng = np.random.default_rng(3)
    N = 2000
    mu = _unit(rng.standard_normal(D))
    keys = 1.5 * mu + 0.3 * rng.standard_normal((N, D))      # pure drift, isotropic spread
    assert abs(calib.estimate_filter_dir(keys) @ mu) < 0.3
    assert calib.qfilter_one_head(keys) @ mu > 0.99


def test_key_svd_recovers_planted_dominant_direction_and_sign_rule():
    rng = np.random.default_rng(4)
    N = 1000
    mu = _unit(rng.standard_normal(D))
    keys = 5.0 * rng.standard_normal((N, 1)) * mu + rng.standard_normal((N, D)) + 0.7
    f = calib.estimate_filter_dir(keys)
    assert abs(f @ mu) > 0.99
    i = np.argmax(np.abs(f))
    assert f[i] > 0 and abs(np.linalg.norm(f) - 1) < 1e-12
    # the sign rule is a property of the direction only
    assert np.array_equal(calib.estimate_filter_dir(-keys), f)


def test_gqa_average_identity_unit_norm_and_contiguous_groups():
    rng = np.random.default_rng(5)
    f = np.stack([_unit(rng.standard_normal(D)) for _ in range(8)])
    assert np.allclose(calib.average_gqa_filters(f, 8), f, atol=1e-15)
    out = calib.average_gqa_filters(np.stack([_unit(rng.standard_normal(D)) for _ in range(24)]), 8)
    assert np.allclose(np.linalg.norm(out, axis=1), 1.0)
    # query heads 3j..3j+2 belong to KV head j
    eye = np.eye(D)
    grouped = np.stack([eye[j] for j in range(8) for _ in range(3)])
    assert np.allclose(calib.average_gqa_filters(grouped, 8), eye[:8])
    # two opposite filters in one group have no mean direction
    with pytest.raises(calib.CalibError):
        calib.average_gqa_filters(np.stack([eye[0], -eye[0]]), 1)
    with pytest.raises(calib.CalibError):
        calib.average_gqa_filters(f, 3)


def test_degenerate_inputs_raise():
    with pytest.raises(calib.CalibError):
        calib.qfilter_one_head(np.eye(D))                 # sigma1 == sigma2
    with pytest.raises(calib.CalibError):
        calib.qfilter_one_head(np.zeros((10, D)))
    with pytest.raises(calib.CalibError):
        calib.estimate_filter_dir(np.ones((10, D)))       # nothing left after centring


def test_query_calibration_recovers_planted_directions():
    """The page's claim for compute_qfilters on planted query drift: each
    head's filter has signed cosine > 0.99 to its planted direction; GQA
    averaging then points along the normalised mean of the group's directions."""
    from kv_cache_token_amd import synth
    L, Hq, Hkv, N = 2, 6, 2, 3000
    q = synth.query_acts(L, Hq, Hkv, N, seed=3, dtype="f32")
    mu = synth.query_head_mu(L, Hq, Hkv, seed=3)
    for l in range(L):
        f = calib.compute_qfilters(q[l].astype(np.float64))
        assert np.all(np.sum(f * mu[l], axis=1) > 0.99)
        avg = calib.average_gqa_filters(f, Hkv)
        m = mu[l].reshape(Hkv, Hq // Hkv, -1).mean(axis=1)
        m /= np.linalg.norm(m, axis=1, keepdims=True)
        assert np.all(np.sum(avg * m, axis=1) > 0.99)
