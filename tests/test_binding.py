"""The Python binding rejects output tensors of the wrong shape before anything is launched
(an undersized buffer would otherwise be written past its end by the kernels). These calls
use CPU tensors: the structural checks run first, the device check last."""
import pytest
import torch

import io_aware_exact_21_amd as fa

bf, f32 = torch.bfloat16, torch.float32


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def test_fwd_rejects_wrong_output_shapes():
    q, k = z(2, 5, 4, 64), z(2, 7, 2, 64)
    with pytest.raises(ValueError, match="out has shape"):
        fa.fwd(q, k, k, out=z(2, 5, 4, 32))
    with pytest.raises(ValueError, match="out has shape"):
        fa.fwd(q, k, k, out=z(1, 5, 4, 64, dtype=f32), out_f32=True)
    with pytest.raises(ValueError, match="lse has shape"):
        fa.fwd(q, k, k, lse=z(2, 4, 4, dtype=f32))
    with pytest.raises(ValueError, match="no CPU path"):          # shapes right: the device check fires
        fa.fwd(q, k, k, out=z(2, 5, 4, 64), lse=z(2, 4, 5, dtype=f32))


def test_decode_rejects_wrong_output_shapes():
    q, kc = z(3, 8, 128), z(3, 100, 2, 128)
    with pytest.raises(ValueError, match="out has shape"):
        fa.decode(q, kc, kc, num_splits=2, out=z(3, 4, 128))
    with pytest.raises(ValueError, match="lse has shape"):
        fa.decode(q, kc, kc, num_splits=2, lse=z(3, 9, dtype=f32))
    with pytest.raises(ValueError, match="no CPU path"):
        fa.decode(q, kc, kc, num_splits=2)


def test_decode_paged_rejects_wrong_output_shapes():
    q, pages = z(2, 8, 64), z(10, 16, 2, 64)
    bt, sl = torch.zeros((2, 4), dtype=torch.int32), torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="out has shape"):
        fa.decode_paged(q, pages, pages, bt, sl, num_splits=2, out=z(2, 8, 32))
    with pytest.raises(ValueError, match="lse has shape"):
        fa.decode_paged(q, pages, pages, bt, sl, num_splits=2, lse=z(8, 2, dtype=f32))


def test_fwd_fp8_rejects_wrong_output_shapes():
    u8 = torch.uint8
    q8, k8, vt8 = z(1, 6, 4, 64, dtype=u8), z(1, 9, 2, 64, dtype=u8), z(1, 2, 64, 16, dtype=u8)
    qs, ks = z(1, 4, dtype=f32), z(1, 2, dtype=f32)
    with pytest.raises(ValueError, match="out has shape"):
        fa.fwd_fp8(q8, k8, vt8, qs, ks, ks, out=z(1, 6, 4, 128))
    with pytest.raises(ValueError, match="lse has shape"):
        fa.fwd_fp8(q8, k8, vt8, qs, ks, ks, lse=z(1, 6, 4, dtype=f32))


def test_bpt_layer_rejects_wrong_output_shape():
    q, k = z(1, 8, 2, 64), z(1, 8, 1, 64)
    w1, b1, w2, b2 = z(512, 128), z(512), z(128, 512), z(128)
    with pytest.raises(ValueError, match="out has shape"):
        fa.bpt_layer(q, k, k, w1, b1, w2, b2, out=z(1, 8, 64))
