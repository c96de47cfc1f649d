"""fa_bwd_noalloc (the backward for callers that cannot allocate) against
fa_bwd, through the C ABI: same kernels, so the gradients must agree bit for
bit. Two calls in a row, the second on a smaller problem, so the static
scratch array's leftover contents from the first call must not leak into the
second; a problem too large for the array is refused on the host."""
import math

import pytest
import torch

from exact_attention_117_amd import inputs
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_117_amd import fa as fa_mod
    return fa_mod


def _case(fa, shape, causal, seed, dtype=torch.bfloat16, window=None):
    B, N, H, d = shape
    say("noalloc bwd", shape, "causal", causal, "window", window, dtype)
    _, (qb, kb, vb, dob) = inputs.qkv(shape, seed=seed, n=4, dtype=dtype)
    q, k, v, do = dev(qb), dev(kb), dev(vb), dev(dob)
    o, lse = fa.fa_fwd(q, k, v, causal=causal, window=window)
    ref = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, window=window)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    fa.fa_bwd_noalloc(q, k, v, o, do, lse, *got, causal=causal, window=window)
    torch.cuda.synchronize()
    for n, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(g, r), n


def test_two_calls_second_smaller(fa):
    # first call fills most of the 16 MiB array (B*H*N = 1.5M rows -> 12 MiB)
    _case(fa, (2, 8192, 96, 64), True, 9100)
    _case(fa, (1, 777, 3, 128), False, 9101)


def test_fp16_and_window(fa):
    _case(fa, (2, 1000, 4, 128), True, 9102, dtype=torch.float16)
    _case(fa, (1, 2000, 2, 256), True, 9103, window=(300, -1))


def test_too_large_is_refused_before_any_launch(fa):
    B, N, H, d = 1, 65536, 40, 64  # 2.6M rows: 21 MB of scratch
    q = torch.zeros((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
    dq = torch.full_like(q, 3.0)
    with pytest.raises(fa.FaError) as e:
        fa.fa_bwd_noalloc(q, q, q, q, q, lse, dq, dq, dq, causal=True)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert (dq == 3.0).all()
