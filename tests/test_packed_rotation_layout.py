"""Host check of the packed rotate_quantize kernel's data movement (CPU, no GPU).

The kernel (rotate_quantize_packed_kernel<g>, blocks of b = 32 << g channels) places a
block's 1 << g lanes 64 >> g lanes apart, loads each lane's 32 channels in an order chosen
for the half-swap lane stages (v_permlane16_swap / v_permlane32_swap), runs five in-thread
butterfly stages, the DPP stages below lane distance 16 (with the sign folded into the
quantiser), then the half-swaps.  This test replays those moves in numpy, with the swap
semantics measured on the device (the even 16-lane row keeps its first operand and receives
the odd row's first operand in its second; the odd row receives the even row's second
operand in its first), and checks that every lane ends up holding the block transform of
32 consecutive channels, 32 * jj onwards, that every load and store stays inside the token,
and that each channel is stored once.
"""
import numpy as np
import pytest


def _hadamard(b):
    i = np.arange(b)
    return np.where(np.bitwise_count(i[:, None] & i[None, :]) & 1, -1.0, 1.0) \
        if hasattr(np, "bitwise_count") else \
        np.array([[(-1.0) ** bin(r & c).count("1") for c in range(b)] for r in range(b)])


def _emulate(K, g, T, ldx, seed):
    b, rows = 32 << g, 64 >> g
    bpt, tpb = K >> (5 + g), (512 >> g) // (K >> (5 + g))
    x = np.random.default_rng(seed).integers(-50, 50, size=(T, ldx)).astype(np.float64)
    out = np.full((T, K), np.nan)
    for it in range(-(-T // tpb)):
        V = np.zeros((512, 32))
        info = {}
        for tid in range(512):
            lane, wave = tid & 63, tid >> 6
            r, jj = lane & (rows - 1), (0 if g == 0 else lane >> (6 - g))
            lt, bt = divmod(wave * rows + r, bpt)
            c0 = 0 if g == 0 else 16 * jj if g == 1 else 8 * (jj >> (g - 2)) + 32 * (jj & ((1 << (g - 2)) - 1))
            c0 += bt * b
            t = it * tpb + lt
            if lt < tpb and t < T:
                info[tid] = (t, bt, jj)
                for h in range(4):
                    ch = 8 * h if g == 0 else (8 * (h & 1) + 32 * (h >> 1) if g == 1 else (b // 4) * h)
                    assert 0 <= c0 + ch and c0 + ch + 8 <= K
                    V[tid, 8 * h:8 * h + 8] = x[t, c0 + ch:c0 + ch + 8]
        hs = 1
        while hs < 32:                                   # in-thread stages
            for i in range(32):
                if not i & hs:
                    a_, c_ = V[:, i].copy(), V[:, i + hs].copy()
                    V[:, i], V[:, i + hs] = a_ + c_, a_ - c_
            hs <<= 1
        for M in [m for m, gmin in ((1, 6), (2, 5), (4, 4), (8, 3)) if g >= gmin]:   # DPP stages
            P = V[np.array([(t - (t & 63)) + ((t & 63) ^ M) for t in range(512)])]
            sgn = np.array([-1.0 if (t & 63) & M else 1.0 for t in range(512)])[:, None]
            V = P * sgn + V
        for D, pairs in ((16, [(i, i + 8) for i in range(32) if not i & 8] if g >= 2 else []),
                         (32, [(i, i + 16) for i in range(16)] if g >= 1 else [])):
            for ia, ib in pairs:                         # half-swap, then the butterfly
                for t in range(512):
                    if not (t & 63) & D:
                        V[t, ib], V[t + D, ia] = V[t + D, ia], V[t, ib]
                A, B = V[:, ia].copy(), V[:, ib].copy()
                V[:, ia], V[:, ib] = A + B, A - B
        for tid, (t, bt, jj) in info.items():
            neg = g >= 3 and bin(jj & ((1 << (g - 2)) - 1)).count("1") & 1
            cpos = bt * b + 32 * jj
            assert cpos + 32 <= K and np.isnan(out[t, cpos:cpos + 32]).all()
            out[t, cpos:cpos + 32] = -V[tid] if neg else V[tid]
    assert not np.isnan(out).any()
    H = _hadamard(b)
    want = np.concatenate([x[:, i * b:(i + 1) * b] @ H.T for i in range(K // b)], axis=1)
    assert np.array_equal(out, want)


@pytest.mark.parametrize("K,g", [(1408, 2), (1408, 0), (1088, 1), (1280, 3), (1536, 4),
                                 (2048, 6), (2048, 5), (768, 3), (2560, 4)])
def test_packed_layout_gives_the_block_transform(K, g):
    _emulate(K, g, T=13, ldx=K + 8, seed=K + g)
