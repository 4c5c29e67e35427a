"""The seeded input generator: determinism, shapes and the logit scale."""
import math

import numpy as np
import torch

import synth_inputs as si


def test_generator_is_deterministic_and_shaped():
    wl = si.WORKLOADS[0]
    a = si.make_inputs(wl)
    b = si.make_inputs(wl)
    for x, y in zip(a, b):
        assert x.shape == (1, 256, 2, 64) and x.dtype == torch.float32
        assert torch.equal(x, y)
    sub = si.make_inputs(wl, heads=[1])
    assert torch.equal(sub[0][:, :, 0], a[0][:, :, 1])


def test_logit_scale_and_temperatures():
    wl = si.WORKLOADS[0]
    q, k, _ = si.head_tensors(0, 0, wl.grid, wl.head_dim, 1.0)
    lg = (q.astype(np.float64) @ k.astype(np.float64).T) / math.sqrt(wl.head_dim)
    assert abs(lg.std() - 2.0) < 1e-3        # all pairs used when N <= 4096
    t1 = si.temperatures(1, 40, "u13")
    t3 = si.temperatures(3, 40, "loguniform")
    assert (t1 >= 1).all() and (t1 <= 3).all()
    assert (t3 >= 0.3).all() and (t3 <= 6).all() and t3.max() / t3.min() > 5


def test_bf16_cast_is_round_to_nearest_even():
    wl = si.WORKLOADS[1]
    q = si.head_tensors(1, 0, (2, 8, 8), 128, 1.0)[0]
    qb = torch.from_numpy(q).to(torch.bfloat16).float().numpy()
    # bf16 keeps 8 significant bits: relative error at most 2^-8
    rel = np.abs(qb - q) / np.maximum(np.abs(q), 1e-30)
    assert rel.max() <= 2.0 ** -8
    # bit-level round-to-nearest-even on the float32 pattern
    bits = q.view(np.uint32).astype(np.uint64)
    rne = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    np.testing.assert_array_equal(rne.astype(np.uint32).view(np.float32), qb)
    assert wl.dtype == "bf16"
