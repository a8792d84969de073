"""emb_stream_copy (the bandwidth reference the benchmark reports against):
an exact copy for sizes that fill whole chunks, end in a partial one, or are
smaller than one; bad sizes and alignments are refused before any launch."""
import pytest
import torch

import embedding_columns_amd as E

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [1, 255, 1024, 1024 * 37 + 5, 1 << 22])
def test_copy_is_exact(words):
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(words)
    src = torch.randint(-2**31, 2**31 - 1, (words * 4 + 4,), dtype=torch.int32, device=dev,
                        generator=g)
    dst = torch.full_like(src, -1)
    E.emb_stream_copy(dst, src, words * 16)
    torch.cuda.synchronize()
    assert torch.equal(dst[:words * 4], src[:words * 4])
    assert torch.all(dst[words * 4:] == -1), "wrote past the end"


def test_copy_refuses_bad_sizes():
    dev = torch.device("cuda")
    a = torch.zeros(64, dtype=torch.int32, device=dev)
    b = torch.zeros(64, dtype=torch.int32, device=dev)
    with pytest.raises(E.EmbError):
        E.emb_stream_copy(a, b, 17)
    with pytest.raises(E.EmbError):
        E.emb_stream_copy(a[1:], b, 16)
