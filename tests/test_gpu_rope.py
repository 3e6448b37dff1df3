"""attn_rope_apply on the GPU against the oracle's explicit fp64 rotation."""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, normal
from gpu_util import require_gpu, say, dev, dev_bf16, host_bf16, bits_to_f32

pytestmark = pytest.mark.gpu

NTK = WORKLOADS["gqa_prefill_s131072"].theta


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("shape,theta,far", [((2, 300, 8, 128), 10000.0, False), ((1, 97, 4, 64), NTK, True),
                                             ((3, 5, 2, 6), 10000.0, True), ((1, 33, 3, 24), 500.0, False)])
def test_rope_matches_oracle(dtype, interleaved, shape, theta, far):
    ta = require_gpu()
    say(f"rope dtype={dtype} interleaved={interleaved} shape={shape} theta={theta} far={far}")
    b, s, h, d = shape
    x = normal(1, "test.rope", shape, dtype)
    if far:   # large positions exercise the fp64 angle path (up to 131071)
        pos = np.random.default_rng(2).integers(0, 131072, size=b * s).astype(np.int32)
    else:
        pos = np.tile(np.arange(s, dtype=np.int32), b)
    xf = bits_to_f32(x) if dtype == "bf16" else x
    ref = oracle.rope(xf.reshape(b * s, h, d), pos, theta, interleaved)
    xd = dev_bf16(x) if dtype == "bf16" else dev(x)
    ta.attn_rope_apply(xd.view(b * s, h, d), dev(pos), theta, interleaved)
    torch.cuda.synchronize()
    got = bits_to_f32(host_bf16(xd)) if dtype == "bf16" else xd.cpu().numpy()
    got = got.reshape(b * s, h, d).astype(np.float64)
    err = np.abs(got - ref)
    if dtype == "bf16":
        # result is the fp32 rotation rounded to bf16: within one bf16 half-ulp (2^-9 relative) plus fp32 noise
        bound = np.abs(ref) * 2.0 ** -8 + 1e-6
    else:
        bound = 1e-5
    say(f"  max abs err {err.max():.3e}, mean {err.mean():.3e}")
    assert np.all(err <= bound)


def test_rope_position_zero_is_exact():
    ta = require_gpu()
    x = normal(3, "test.rope0", (16, 4, 128), "bf16")
    xd = dev_bf16(x)
    ta.attn_rope_apply(xd, dev(np.zeros(16, np.int32)), 10000.0)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(xd), x)
