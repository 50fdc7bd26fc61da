"""The binding checks every caller-given buffer before a launch: the C ABI
takes plain pointers and cannot, so a short, misplaced or mistyped output
buffer is refused in Python and no kernel runs."""
import pytest

torch = pytest.importorskip("torch")

import allreduce_compatible_gradient_amd as gq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.lib()


def test_short_or_mistyped_buffers_are_refused():
    n, d, s, W = 3, 1000, 7, 6
    x = torch.randn(n, d, device=DEV)
    norm = gq.gq_global_norm(x)
    short_mean = torch.empty(d - 1, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        gq.gq_compress_mean(x, s, 2.0, 2.0, "L", 1, mean=short_mean)
    with pytest.raises(TypeError):
        gq.gq_compress_mean(x, s, 2.0, 2.0, "L", 1, mean=torch.empty(d, dtype=torch.float64,
                                                                     device=DEV))
    with pytest.raises(ValueError):
        gq.gq_quantize(x, s, "L", norm, 1, W,
                       codes=torch.empty((n, 8), dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        gq.gq_quantize_words(x, s, "L", norm, 1, W,
                             words=torch.empty((n - 1, gq.gq_word_row_bytes(d, W) // 4),
                                               dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        gq.gq_dequantize(torch.empty(4, dtype=torch.uint8, device=DEV), n, d, s, "L", W, norm)
    with pytest.raises(ValueError):  # norm on the host
        gq.gq_quantize(x, s, "L", norm.cpu(), 1, W)
    with pytest.raises(ValueError):  # a strided output
        gq.gq_compress_mean(x, s, 2.0, 2.0, "L", 1,
                            mean=torch.empty((d, 2), dtype=torch.float32, device=DEV)[:, 0])
    with pytest.raises(ValueError):
        gq.gq_e8_tree(torch.empty((2, 16), dtype=torch.uint8, device=DEV), 4, 16, 1)
    torch.cuda.synchronize()
    # buffers of exactly the needed size are taken
    mean, _, _ = gq.gq_compress_mean(x, s, 2.0, 2.0, "L", 1,
                                     mean=torch.empty(d, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert mean.shape == (d,)
