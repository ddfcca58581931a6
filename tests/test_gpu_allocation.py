"""GPU test of the cluster-allocation inputs (CodeQuant2, Figure 3 left: importance and
kernel latency guide how many clusters each weight matrix gets).

The pipeline takes its importance from the library's routing (cbq_moe_route_gather)
and its clustering errors from the library's per-row K-means (cbq_kmeans_codebooks),
decoded by the allocation module.  Both inputs are checked here against the oracle
run on the same seeded inputs (its routing, its K-means, its bit unpacking), and the
allocation drawn from them against the one drawn from the oracle's inputs."""
import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.gpu

cbq = pytest.importorskip("codebook_bit_quantized_amd")
from codebook_bit_quantized_amd.allocation import (allocate_bits, clustering_errors,  # noqa: E402
                                                   route_share)
from gpu_util import DEV, to_dev  # noqa: E402

E, S, TOPK, T, ROWS, K = 8, 1, 2, 96, 16, 256
CHOICES = (2, 3, 4)
ITERS = 30


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cbq.load_library()


def _oracle_errors(w_bits, groups):
    out = np.zeros((groups, len(CHOICES)))
    wf = oracle.bf16_bits_to_f64(w_bits)
    for c, bits in enumerate(CHOICES):
        idx, cb, _ = oracle.kmeans_codebooks(w_bits, bits, ITERS)
        W_hat = oracle.dequantize(idx, cb)
        sq = ((wf - W_hat) ** 2).sum(axis=1)
        out[:, c] = sq.reshape(groups, -1).sum(axis=1)
    return out


def test_allocation_inputs_match_the_oracle():
    lg = datagen.random_logits(41, T, E)
    share = route_share(cbq, to_dev(lg), TOPK, S)
    rt = oracle.route(lg, TOPK, True, S)
    want_share = np.concatenate([rt["counts"] / float(T), np.ones(S)])
    assert np.array_equal(share, want_share)
    print(f"importance (token share per expert): {np.round(share, 4).tolist()}")

    groups = E + S
    w_bits = np.concatenate([datagen.weights_bf16(4100, datagen.TAG_W_FULL, e, ROWS, K)
                             for e in range(groups)])
    assert all(oracle.kmeans_precondition(r) for r in w_bits)   # sums exact: bit-exact K-means
    got = clustering_errors(cbq, torch, w_bits, groups, CHOICES, ITERS, DEV)
    want = _oracle_errors(w_bits, groups)
    rel = np.abs(got - want) / want
    print(f"clustering error per expert and width, worst relative gap {rel.max():.2e}")
    assert np.all(rel <= 1e-12)
    assert np.all(np.diff(got, axis=1) < 0)      # more centroids: less error

    # the allocation drawn from the library's inputs is the oracle-input allocation
    lat = np.array([[1.0, 1.3, 1.7]] * groups) * (1.0 + 0.1 * np.arange(groups))[:, None]
    budget = float(lat[:, 1].sum())
    mine = allocate_bits(lat, share[:, None] * got, budget)
    ref = allocate_bits(lat, want_share[:, None] * want, budget)
    assert np.array_equal(mine, ref)
    assert lat[np.arange(groups), mine - 2].sum() <= budget
