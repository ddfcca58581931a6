"""GPU test of cbq_moe_route_gather_noalloc, the routing entry point for callers that
cannot allocate: called through the C ABI, its outputs must equal, bit for bit,
those of cbq_moe_route_gather with a caller-provided workspace, on two calls in a row
(the second smaller, so stale counts of the first call sit in the shared scratch)."""
import numpy as np
import pytest
import torch

import datagen

pytestmark = pytest.mark.gpu

cbq = pytest.importorskip("codebook_bit_quantized_amd")
from gpu_util import DEV, to_dev  # noqa: E402

KEYS = ("ids", "weights", "offsets", "sorted_tokens", "slot_of")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cbq.load_library()


def _both(lg, k, S, renorm=True):
    want = cbq.moe_route_gather(lg, k, renorm, S)
    got = cbq.moe_route_gather_noalloc(lg, k, renorm, S)
    torch.cuda.synchronize()
    for key in KEYS:
        a, b = got[key].cpu(), want[key].cpu()
        assert a.shape == b.shape, key
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), key
    return got


@pytest.mark.parametrize("T1,T2,E,k,S", [(65536, 4096, 256, 8, 2), (4096, 32, 64, 6, 2),
                                          (20000, 7, 128, 8, 0)])
def test_noalloc_route_matches_workspace_route(T1, T2, E, k, S):
    for T, seed in ((T1, 1), (T2, 2)):            # second call smaller than the first
        lg = to_dev(datagen.random_logits(700 + seed + E, T, E))
        got = _both(lg, k, S)
        offs = got["offsets"].cpu().numpy()
        assert offs[-1] == T * k + S * T and np.all(np.diff(offs) >= 0)


def test_noalloc_route_after_other_work_and_zero_tokens():
    lg = to_dev(datagen.random_logits(711, 3000, 32))
    _both(lg, 4, 1, renorm=False)
    r = cbq.moe_route_gather_noalloc(torch.empty((0, 32), dtype=torch.float32, device=DEV), 4, True, 1)
    torch.cuda.synchronize()
    assert r["offsets"].cpu().tolist() == [0] * 34
    _both(to_dev(datagen.random_logits(712, 100, 32)), 4, 1)
