"""gpt_op_newton_schulz_noalloc (Newton-Schulz with its scratch in the
library's fixed device array) against gpt_op_newton_schulz (caller-provided
scratch), through the C ABI. Both run the same kernels, so the results must
agree bit for bit. Two calls in a row, the second on a smaller input, check
that nothing left in the shared array by the first call leaks into the
second; a request beyond the array is refused on the host."""
import numpy as np
import pytest

from gpu_util import dev, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpt_pretraining_step_bf16_amd import binding, synthetic as syn  # noqa: E402


def _with_scratch(X, count, rows, cols):
    Xd = dev(torch, X)
    scratch = torch.empty(binding.ns_scratch_bytes(count, rows, cols), dtype=torch.uint8, device="cuda")
    binding.op_newton_schulz(Xd, count, rows, cols, syn.NS_COEFFS, scratch)
    torch.cuda.synchronize()
    return Xd.cpu().numpy()


def _no_alloc(X, count, rows, cols):
    Xd = dev(torch, X)
    binding.op_newton_schulz_noalloc(Xd, count, rows, cols, syn.NS_COEFFS)
    torch.cuda.synchronize()
    return Xd.cpu().numpy()


def test_no_alloc_newton_schulz_matches_the_scratch_entry_point():
    # Larger first (two 1280 x 1280 matrices), then a smaller, ragged batch
    # (three 384 x 128) that reuses the same array.
    for (count, rows, cols), seed in (((2, 1280, 1280), 1), ((3, 384, 128), 2)):
        log(f"no-alloc newton-schulz count={count} rows={rows} cols={cols}")
        assert binding.ns_scratch_bytes(count, rows, cols) <= binding.NS_STATIC_SCRATCH_BYTES
        X = np.random.default_rng(seed).standard_normal((count, rows, cols)).astype(np.float32)
        want = _with_scratch(X, count, rows, cols)
        got = _no_alloc(X, count, rows, cols)
        assert np.isfinite(got).all()
        np.testing.assert_array_equal(got, want)


def test_no_alloc_newton_schulz_refuses_sizes_beyond_its_array():
    count, rows, cols = 6, 1280, 1280
    assert binding.ns_scratch_bytes(count, rows, cols) > binding.NS_STATIC_SCRATCH_BYTES
    X = torch.zeros((count, rows, cols), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.GptError) as e:
        binding.op_newton_schulz_noalloc(X, count, rows, cols, syn.NS_COEFFS)
    assert e.value.status == binding.GPT_EWORKSPACE
    assert torch.count_nonzero(X).item() == 0
