"""moe_permute_noalloc (the permute with its scratch in a static device array,
for callers that cannot allocate) against moe_permute, through the C ABI:
bit-identical results on consecutive calls of different sizes, indices-only
calls, the largest histogram the scratch holds, and the size check."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host, say
from mixture_experts_layer_free_amd import _lib as L

pytestmark = pytest.mark.gpu


def _choice(T, E, k, seed):
    """k distinct experts per token: a random first expert and the k-1 after it
    (mod E), in a random slot order."""
    rng = np.random.default_rng(seed)
    idx = (rng.integers(0, E, (T, 1)) + np.arange(k)[None, :]) % E
    return np.take_along_axis(idx, np.argsort(rng.random((T, k)), axis=1), 1).astype(np.int32)


def _both(idx, x, E, copy=True):
    t_idx = dev(idx)
    ref = L.moe_permute(t_idx, x, E, copy=copy)
    got = L.moe_permute_noalloc(t_idx, x, E, copy=copy)
    torch.cuda.synchronize()
    for name, a, b in zip(("counts", "offsets", "row_of", "token_of", "x_perm"), got, ref):
        if a is None and b is None:
            continue
        assert np.array_equal(host(a), host(b)), name
    return got


def test_noalloc_matches_permute_on_consecutive_calls():
    """A larger call, then a smaller one on the same scratch, then the first
    size again: each bit-identical to moe_permute's results."""
    for T, E, k, d, seed in ((6000, 64, 8, 256, 1), (700, 24, 3, 64, 2), (6000, 64, 8, 256, 3)):
        say(f"[noalloc permute T={T} E={E} k={k} d={d}]")
        x = dev(np.random.default_rng(seed).standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
        _both(_choice(T, E, k, seed), x, E)


def test_noalloc_indices_only_and_skewed():
    """x_perm NULL (indices only), with every token on the same few experts."""
    T, E, k = 5000, 128, 4
    idx = np.tile(np.array([7, 0, 99, 3], np.int32), (T, 1))
    x = torch.zeros((T, 64), dtype=torch.bfloat16, device="cuda")
    say(f"[noalloc permute indices only T={T} E={E} k={k}]")
    got = _both(idx, x, E, copy=False)
    assert got[4] is None


def test_noalloc_largest_histogram_and_size_check():
    """ceil(T*k/256) * E * 4 bytes equal to the scratch size runs; one more
    chunk is refused with ENOTSUP before anything is launched."""
    E, k = 256, 8
    T = L.PERMUTE_NOALLOC_SCRATCH // (E * 4) * 256 // k          # exactly the scratch
    say(f"[noalloc permute at the scratch limit T={T} E={E} k={k}]")
    x = torch.zeros((T, 8), dtype=torch.bfloat16, device="cuda")
    _both(_choice(T, E, k, 5), x, E, copy=False)
    T2 = T + 256 // k                                              # one more 256-assignment chunk
    idx2 = torch.zeros((T2, k), dtype=torch.int32, device="cuda")
    x2 = torch.zeros((T2, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.MoEError) as e:
        L.moe_permute_noalloc(idx2, x2, E, copy=False)
    assert e.value.status == L.MOE_ENOTSUP
