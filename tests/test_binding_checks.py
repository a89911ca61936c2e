"""The Python binding refuses mismatched tensors before any pointer reaches
the library (CPU only: every case raises before the C call, so no handle
and no GPU are needed; the handle is a registered stand-in that the library
never sees)."""
import ctypes

import pytest
import torch

from decode_step_token_amd import _binding as b

FAKE = ctypes.c_void_p(0x1000)


@pytest.fixture(autouse=True)
def _fake_handle():
    b._HANDLES[FAKE.value] = ("f32", 1000, 8)
    yield
    b._HANDLES.pop(FAKE.value, None)


def _call(logits, **kw):
    b.sample_batch(FAKE, logits, **kw)


def test_wrong_logits_dtype():
    with pytest.raises(TypeError, match="reads f32 rows"):
        _call(torch.zeros((4, 1000), dtype=torch.bfloat16))


def test_rows_shorter_than_vocab():
    with pytest.raises(ValueError, match="vocab_size"):
        _call(torch.zeros((4, 999)))


def test_more_rows_than_the_tensor_or_the_handle():
    with pytest.raises(ValueError, match="outside"):
        _call(torch.zeros((4, 1000)), B=5)
    with pytest.raises(ValueError, match="max_batch"):
        _call(torch.zeros((9, 1000)))


def test_row_stride_past_the_tensor():
    with pytest.raises(ValueError, match="row_stride"):
        _call(torch.zeros((4, 1000)), row_stride=999)
    with pytest.raises(ValueError, match="reaches past"):
        _call(torch.zeros((4, 1000)), row_stride=1200)


def test_short_outputs():
    x = torch.zeros((4, 1000))
    with pytest.raises(ValueError, match="tokens_out"):
        _call(x, tokens_out=torch.zeros(3, dtype=torch.int32))
    for field, dt, n in (("probs_out", torch.float32, 4 * 1000 - 1), ("kept_out", torch.int32, 3),
                         ("topk_idx_out", torch.int32, 4 * 64 - 1), ("rand_out", torch.int64, 3)):
        with pytest.raises(ValueError, match=field):
            _call(x, debug={field: torch.zeros(n, dtype=dt)})


def test_bf16_handle_accepts_bit_patterns_only_of_two_bytes():
    b._HANDLES[FAKE.value] = ("bf16", 1000, 8)
    with pytest.raises(TypeError, match="reads bf16 rows"):
        _call(torch.zeros((4, 1000), dtype=torch.float32))


def test_static_entry_checks_dtype_and_width():
    with pytest.raises(TypeError):
        b.sample_batch_static(torch.zeros((2, 100), dtype=torch.float32), 100, "bf16", 1)
    with pytest.raises(ValueError, match="vocab_size"):
        b.sample_batch_static(torch.zeros((2, 100)), 101, "f32", 1)
