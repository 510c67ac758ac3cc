"""The allocation-free GEMM entry point (s1k_gemm_noalloc) against the
allocating one (s1k_gemm) on the same operands: the same kernels and the same
fixed-order split-K reduction, so the outputs must be bitwise equal; two
calls in a row, the second smaller (its partial sums reuse the scratch the
first left behind), and a size beyond the scratch rejected on the host."""
import numpy as np
import pytest

from s1_workloads import f32_to_bf16_bits
from tests.gpu_util import dev_bits, log, require_gpu, stream_ptr

pytestmark = pytest.mark.gpu


def _case(B, torch, rng, M, N, K, split):
    A = f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    W = f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    dA, dW = dev_bits(A), dev_bits(W)
    ref = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    B.gemm(B.S1_BF16, dA.data_ptr(), dW.data_ptr(), ref.data_ptr(), M, N, K, split, stream_ptr())
    B.gemm_noalloc(B.S1_BF16, dA.data_ptr(), dW.data_ptr(), got.data_ptr(), M, N, K, split, stream_ptr())
    torch.cuda.synchronize()
    r, g = ref.cpu().numpy(), got.cpu().numpy()
    diff = int((r.view(np.uint32) != g.view(np.uint32)).sum())
    log(f"noalloc GEMM M={M} N={N} K={K} split={split}: {diff} elements differ from s1k_gemm")
    assert not np.isnan(g).any() and diff == 0


def test_noalloc_gemm_matches_the_allocating_entry():
    torch = require_gpu()
    from prefill_only_decision_amd import binding as B
    rng = np.random.default_rng(99)
    _case(B, torch, rng, 512, 2560, 9728, 4)     # the down projection at 512 rows, four-way split
    _case(B, torch, rng, 200, 640, 2048, 3)      # smaller, ragged rows: reuses the scratch
    _case(B, torch, rng, 77, 256, 512, 1)        # no split: no scratch at all


def test_noalloc_gemm_rejects_sizes_beyond_its_scratch():
    require_gpu()
    from prefill_only_decision_amd import binding as B
    import prefill_only_decision_amd as s1
    M, N, split = 4096, 2560, 2                   # 80 MiB of partial sums
    assert split * M * N * 4 > B_SCRATCH
    with pytest.raises(s1.S1Error) as e:
        B.gemm_noalloc(B.S1_BF16, 1, 1, 1, M, N, 2560, split, stream_ptr())
    assert e.value.code == -1 and "scratch" in str(e.value)


B_SCRATCH = 32 << 20
