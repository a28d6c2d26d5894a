"""Host logic of the Python binding, on the CPU: the token stride it derives for
q, k, v given as views of one [B, T, s] buffer.  Strides of dimensions of size
one never move an address, so they are ignored (torch reports arbitrary values
there); uneven token spacing and q, k, v with different spacings are rejected
before anything reaches the library."""
import pytest
import torch

import linear_attention_gated_amd as gdn

CPU = torch.device("cpu")


def views(B, T, H, D, pad):
    w = H * D
    buf = torch.zeros(B, T, 3 * w + pad)
    return [buf[..., i * w:(i + 1) * w].view(B, T, H, D) for i in range(3)]


def stride_of(ts):
    return gdn._qkv_stride(ts, ("q", "k", "v"), torch.float32, CPU)


def test_token_stride_of_slices_of_one_buffer():
    assert stride_of(views(2, 5, 2, 64, 8)) == 3 * 128 + 8
    assert stride_of(views(1, 7, 3, 64, 0)) == 3 * 192


def test_one_token_per_sequence_takes_the_batch_stride():
    # T = 1: torch may report any token stride; the tokens are a batch stride apart
    q, k, v = views(2, 1, 1, 64, 64)
    assert stride_of((q, k, v)) == 3 * 64 + 64
    odd = [t.as_strided(t.shape, (t.stride(0), 7, t.stride(2), 1), t.storage_offset()) for t in (q, k, v)]
    assert stride_of(odd) == 3 * 64 + 64


def test_a_single_token_has_no_spacing():
    q, k, v = views(1, 1, 2, 64, 64)
    odd = [t.as_strided(t.shape, (999, 123, 64, 1), t.storage_offset()) for t in (q, k, v)]
    assert stride_of(odd) == 0


def test_one_head_ignores_the_head_stride():
    q, k, v = views(2, 3, 1, 64, 16)
    odd = [t.as_strided(t.shape, (t.stride(0), t.stride(1), 4321, 1), t.storage_offset()) for t in (q, k, v)]
    assert stride_of(odd) == 3 * 64 + 16


def test_uneven_spacing_and_mixed_strides_are_rejected():
    q, k, v = views(2, 3, 2, 64, 0)
    uneven = q.as_strided(q.shape, (q.stride(0) + 8, q.stride(1), 64, 1), q.storage_offset())
    with pytest.raises(ValueError):
        stride_of((uneven, k, v))
    k2 = k.as_strided(k.shape, (2 * (k.stride(1) + 8), k.stride(1) + 8, 64, 1), k.storage_offset())
    with pytest.raises(ValueError):
        stride_of((q, k2, v))
    rows = q.as_strided(q.shape, (q.stride(0), q.stride(1), 80, 1), q.storage_offset())
    with pytest.raises(ValueError):
        stride_of((rows, k, v))
