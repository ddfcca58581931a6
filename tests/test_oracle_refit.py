"""Pins of the oracle's output-aware centroid refit (the AI Radio episode on CodeQuant:
centroids fine-tuned to minimise the layer's output error; CodeQuant2 Figure 1 right)
against results fixed by other means: cluster means, a library least-squares solver, and
the least-squares property itself."""
import numpy as np

import datagen
import oracle


def _bf16(a):
    return datagen.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _case(seed, R=5, K=128, bits=3):
    w = datagen.weights_bf16(seed, datagen.TAG_W_FULL, 0, R, K)
    idx, cb, _ = oracle.kmeans_codebooks(w, bits, 50)
    return w, idx, cb


def test_identity_calibration_gives_cluster_means():
    # X = I: the output error is the weight error, minimised by each cluster's mean
    w, idx, cb = _case(1)
    K = w.shape[1]
    new = oracle.refit_codebooks(w, idx, cb, _bf16(np.eye(K)))
    wf = oracle.bf16_bits_to_f64(w)
    for r in range(w.shape[0]):
        for j in range(cb.shape[1]):
            m = idx[r] == j
            want = oracle.round_f64_to_f16_bits(np.array([wf[r, m].mean()]))[0] if m.any() else cb[r, j]
            assert new[r, j] == want, (r, j)


def test_matches_library_least_squares():
    w, idx, cb = _case(2, R=6, K=160)
    X = datagen.random_tokens(21, 48, 160)
    new = oracle.refit_codebooks(w, idx, cb, X)
    Xf, wf = oracle.bf16_bits_to_f64(X), oracle.bf16_bits_to_f64(w)
    for r in range(w.shape[0]):
        act = [j for j in range(cb.shape[1]) if (idx[r] == j).any()]
        S = np.zeros((160, len(act)))
        for q, j in enumerate(act):
            S[idx[r] == j, q] = 1.0
        sol = np.linalg.lstsq(Xf @ S, Xf @ wf[r], rcond=None)[0]
        got = oracle.f16_bits_to_f64(new[r, act])
        ulp = np.abs(sol) * 2.0 ** -10 + 2.0 ** -24
        assert np.all(np.abs(got - sol) <= ulp), r


def test_refit_lowers_the_calibration_error_and_helps_held_out_data():
    w, idx, cb = _case(3, R=8, K=256)
    X = datagen.random_tokens(31, 96, 256)
    Xt = datagen.random_tokens(32, 96, 256)
    new = oracle.refit_codebooks(w, idx, cb, X)
    assert oracle.output_error(w, idx, new, X) < oracle.output_error(w, idx, cb, X)
    assert oracle.output_error(w, idx, new, Xt) < oracle.output_error(w, idx, cb, Xt)


def test_empty_and_dependent_clusters_keep_their_centroids():
    K = 64
    wf = np.linspace(-1, 1, K)
    w = _bf16(wf[None, :])
    idx = (np.arange(K) % 3)[None, :]                      # clusters 3..7 empty
    cb = oracle.round_f64_to_f16_bits(np.array([[0.1, 0.2, 0.3, 0.4, 0.5, 0.6, 0.7, 0.8]]))
    X = np.zeros((1, K), np.float32)
    X[0, :] = 1.0                                          # one calibration row: rank 1
    new = oracle.refit_codebooks(w, idx, cb, _bf16(X))
    assert np.array_equal(new[0, 3:], cb[0, 3:])           # empty clusters untouched
    # rank 1: cluster 0 absorbs the output, clusters 1 and 2 are left out and keep theirs
    assert np.array_equal(new[0, 1:3], cb[0, 1:3])
    c = oracle.f16_bits_to_f64(new[0])
    counts = np.bincount(idx[0], minlength=8)
    want0 = (wf.sum() - counts[1] * c[1] - counts[2] * c[2]) / counts[0]
    assert new[0, 0] == oracle.round_f64_to_f16_bits(np.array([want0]))[0]


def test_power_of_two_calibration_scale_changes_nothing():
    w, idx, cb = _case(4, R=4, K=96)
    X = datagen.random_tokens(41, 32, 96)
    a = oracle.refit_codebooks(w, idx, cb, X)
    X4 = _bf16(datagen.bf16_bits_to_f32(X) * 4.0)
    assert np.array_equal(a, oracle.refit_codebooks(w, idx, cb, X4))


def _clustered(R=4, K=64, bits=2, seed=7):
    w = datagen.weights_bf16(seed, datagen.TAG_W_FULL, 0, R, K)
    idx, cb, _ = oracle.kmeans_codebooks(w, bits, 20)
    return w, idx, cb


def test_output_error_identity_calibration_is_the_weight_error():
    # X = I: ||X (W - W_hat)^T||_F / ||X W^T||_F = ||W - W_hat||_F / ||W||_F, a sum of
    # squares over the weights written out with plain loops
    w, idx, cb = _clustered()
    R, K = w.shape
    wf = oracle.bf16_bits_to_f64(w)
    cf = oracle.f16_bits_to_f64(cb)
    num = den = 0.0
    for r in range(R):
        for k in range(K):
            d = wf[r, k] - cf[r, idx[r, k]]
            num += d * d
            den += wf[r, k] * wf[r, k]
    want = (num / den) ** 0.5
    got = oracle.output_error(w, idx, cb, _bf16(np.eye(K)))
    assert abs(got - want) <= 1e-12 * want


def test_output_error_one_hot_token_selects_a_column():
    # one calibration token e_j: the error of column j of W alone (Euclidean norm over rows)
    w, idx, cb = _clustered(seed=8)
    R, K = w.shape
    wf = oracle.bf16_bits_to_f64(w)
    cf = oracle.f16_bits_to_f64(cb)
    for j in (0, 5, K - 1):
        x = np.zeros((1, K))
        x[0, j] = 1.0
        col = wf[:, j]
        err = np.array([wf[r, j] - cf[r, idx[r, j]] for r in range(R)])
        want = np.sqrt((err ** 2).sum()) / np.sqrt((col ** 2).sum())
        got = oracle.output_error(w, idx, cb, _bf16(x))
        assert abs(got - want) <= 1e-12 * want, j


def test_output_error_hand_example():
    # W = [[1, 2]], centroids (1, 1.5), assignments (0, 1): W_hat = [[1, 1.5]].
    # X = [[1, 1], [2, 0]]: X W^T = (3, 2), X (W - W_hat)^T = (0.5, 0):
    # error = 0.5 / sqrt(13).  A Frobenius norm of W - W_hat alone would give 0.5/sqrt(5).
    w = _bf16([[1.0, 2.0]])
    cb = oracle.round_f64_to_f16_bits(np.array([[1.0, 1.5]]))
    idx = np.array([[0, 1]])
    X = _bf16([[1.0, 1.0], [2.0, 0.0]])
    assert oracle.output_error(w, idx, cb, X) == 0.5 / np.sqrt(13.0)
    # zero error when every weight sits on its centroid
    assert oracle.output_error(w, idx, oracle.round_f64_to_f16_bits(np.array([[1.0, 2.0]])), X) == 0.0
