"""Pins of the oracle's inference pieces around the backbone (CPU only):
2D -> 3D inflation (§3.4), the classification head and the multi-view score
average (readings D23-D25).

Each pin compares the oracle with something it does not compute itself: a 2D
convolution of one frame (torch), the 2D relative-position table looked up
directly, brute-force loops on tiny inputs, and scipy's softmax.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import vswin as ov


@pytest.mark.parametrize("pt", [2, 3, 4])
def test_inflated_patch_embed_on_a_static_video_is_the_2d_embedding(pt):
    """§3.4: with the kernel repeated over the pt temporal slots and divided by
    pt, a video whose frames are all equal embeds, in every temporal patch, as
    the single frame does through the 2D patch convolution."""
    rng = np.random.default_rng(pt)
    C, Cin, ph, pw = 8, 3, 4, 4
    w2 = rng.standard_normal((C, Cin, ph, pw))
    b = rng.standard_normal(C)
    frame = rng.standard_normal((2, Cin, 8, 12))
    video = np.repeat(frame[:, :, None], 2 * pt, axis=2)            # 2 temporal patches
    y3 = ov.patch_embed(video, ov.inflate_patch_embed(w2, pt), b)   # (2, 2, 2, 3, C)
    y2 = F.conv2d(torch.from_numpy(frame), torch.from_numpy(w2), torch.from_numpy(b), stride=(ph, pw))
    y2 = y2.numpy().transpose(0, 2, 3, 1)                           # (2, 2, 3, C)
    assert y3.shape == (2, 2, 2, 3, C)
    for t in range(2):
        np.testing.assert_allclose(y3[:, t], y2, rtol=0, atol=1e-12)


def test_inflated_patch_embed_values():
    w2 = np.arange(2 * 1 * 2 * 2, dtype=np.float64).reshape(2, 1, 2, 2)
    w3 = ov.inflate_patch_embed(w2, 2)
    assert w3.shape == (2, 1, 2, 2, 2)
    assert np.array_equal(w3[:, :, 0], w2 / 2) and np.array_equal(w3[:, :, 1], w2 / 2)


@pytest.mark.parametrize("P,M", [(4, 7), (2, 3)])
def test_inflated_table_gives_every_frame_pair_the_2d_bias(P, M):
    """§3.4: the table repeated over the 2P - 1 temporal offsets makes the
    bias of any query / key pair of a (P, M, M) window the 2D bias of their
    spatial offset, whatever their temporal offset (brute force over pairs)."""
    heads = 3
    t2 = np.random.default_rng(M).standard_normal(((2 * M - 1) ** 2, heads))
    t3 = ov.inflate_bias_table(t2, P)
    assert t3.shape == (ov.table_rows((P, M, M)), heads)
    rel3 = ov.relative_index((P, M, M))
    n2 = M * M
    for i in range(P * n2):
        hi, wi = divmod(i % n2, M)
        for j in range(P * n2):
            hj, wj = divmod(j % n2, M)
            row2 = (hi - hj + M - 1) * (2 * M - 1) + (wi - wj + M - 1)
            assert np.array_equal(t3[rel3[i, j]], t2[row2])


def test_head_pools_over_every_token():
    rng = np.random.default_rng(1)
    B, T, H, W, C, K = 2, 2, 3, 2, 5, 4
    x = rng.standard_normal((B, T, H, W, C))
    w = rng.standard_normal((K, C))
    b = rng.standard_normal(K)
    got = ov.head(x, w, b)
    # brute force: explicit sums over the tokens and channels
    for bb in range(B):
        for k in range(K):
            acc = 0.0
            for c in range(C):
                tot = 0.0
                for t in range(T):
                    for h in range(H):
                        for ww in range(W):
                            tot += x[bb, t, h, ww, c]
                acc += w[k, c] * tot / (T * H * W)
            assert math.isclose(got[bb, k], acc + b[k], rel_tol=1e-12, abs_tol=1e-12)
    # identical tokens pool to that token; the token order does not matter
    v = rng.standard_normal(C)
    same = np.broadcast_to(v, (1, T, H, W, C))
    np.testing.assert_allclose(ov.head(same, w, None)[0], w @ v, rtol=1e-12)
    perm = rng.permutation(T * H * W)
    xs = x.reshape(B, -1, C)[:, perm].reshape(x.shape)
    np.testing.assert_allclose(ov.head(xs, w, b), got, rtol=1e-12)


def test_multiview_average():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((3, 4, 6)) * 3
    got = ov.multiview_average(z)
    # brute force on the tiny input
    for bb in range(3):
        for k in range(6):
            acc = 0.0
            for v in range(4):
                den = sum(math.exp(z[bb, v, j]) for j in range(6))
                acc += math.exp(z[bb, v, k]) / den
            assert math.isclose(got[bb, k], acc / 4, rel_tol=1e-12)
    # identical views reduce to one softmax; rows sum to one; a constant
    # added to one view's logits changes nothing
    same = np.repeat(z[:, :1], 5, axis=1)
    np.testing.assert_allclose(ov.multiview_average(same), scipy.special.softmax(z[:, 0], axis=-1), rtol=1e-12)
    np.testing.assert_allclose(got.sum(axis=-1), 1.0, rtol=1e-12)
    shifted = z + rng.standard_normal((3, 4, 1)) * 50
    np.testing.assert_allclose(ov.multiview_average(shifted), got, rtol=1e-10)
