"""The seeded synthetic inputs: the five configurations' shapes and kinds, the
outlier-key recipe of the long causal configuration, reproducibility, and the
FLOP and byte counts the measurements divide by.  CPU only, small sizes where
the recipe is size-independent."""

import math

import numpy as np
import torch

import workloads


def test_the_five_configurations():
    w = workloads.WORKLOADS
    shape = {i: (w[i].B, w[i].Hq, w[i].Hkv, w[i].Nq, w[i].Nkv, w[i].D, w[i].dtype, w[i].causal)
             for i in range(1, 6)}
    assert shape[1] == (1, 1, 1, 256, 256, 64, "f32", False)
    assert shape[2] == (4, 16, 16, 1024, 1024, 64, "bf16", False)
    assert shape[3] == (2, 32, 32, 8192, 8192, 128, "bf16", False)
    assert shape[4] == (1, 28, 4, 4096, 4096, 128, "bf16", True)
    assert shape[5] == (1, 28, 4, 32768, 32768, 128, "bf16", True)
    assert (w[5].sigma, w[5].outlier_frac, w[5].outlier_mult) == (0.5, 0.01, 8.0)
    for i in range(1, 5):
        assert (w[i].sigma, w[i].outlier_frac) == (1.0, 0.0)


def test_flops_and_compulsory_bytes():
    w3, w4 = workloads.WORKLOADS[3], workloads.WORKLOADS[4]
    assert w3.flops() == 4.0 * 2 * 32 * 8192 * 8192 * 128 == 2.199023255552e12
    assert w4.flops() == 4.0 * 28 * 4096 * 4096 * 128 / 2
    # Q, K, V read once and O written once in bf16, lse in fp32
    assert w3.io_bytes() == 2 * (3 * 2 * 32 * 8192 * 128) + 2 * 2 * 32 * 8192 * 128 \
        + 4 * 2 * 32 * 8192
    assert abs(w3.io_bytes() / 2**20 - 514.0) < 0.5


def test_same_seed_same_inputs_and_different_seed_differs():
    a = workloads.make_inputs(1, 4, 2, 100, 130, 64, "bf16", seed=3)
    b = workloads.make_inputs(1, 4, 2, 100, 130, 64, "bf16", seed=3)
    c = workloads.make_inputs(1, 4, 2, 100, 130, 64, "bf16", seed=4)
    for x, y in zip(a, b):
        assert torch.equal(x, y) and x.is_contiguous()
    assert not torch.equal(a[0], c[0])
    q, k, v = a
    assert q.shape == (1, 4, 100, 64) and k.shape == v.shape == (1, 2, 130, 64)
    assert q.dtype == k.dtype == v.dtype == torch.bfloat16


def test_outlier_keys_are_one_percent_of_rows_scaled_by_eight():
    """Per (b, kv head), round(0.01 * N_kv) distinct K rows are multiplied by 8 after the
    draw (a power of two, so it commutes with the rounding to bf16); the other rows, Q
    and V keep sigma = 0.5.  Drawn at N_kv = 4096 (41 rows per head) with the recipe of
    the N = 32768 configuration (328 rows per head)."""
    B, Hq, Hkv, N, D = 1, 28, 4, 4096, 128
    q, k, v = workloads.make_inputs(B, Hq, Hkv, N, N, D, "bf16", seed=11, sigma=0.5,
                                    outlier_frac=0.01, outlier_mult=8.0)
    n_out = int(round(0.01 * N))
    rms = k.float().pow(2).mean(-1).sqrt()             # [B, Hkv, N]
    for g in range(Hkv):
        big = torch.nonzero(rms[0, g] > 2.0).flatten()  # 8 x 0.5 = 4 against 0.5
        assert big.numel() == n_out, (g, big.numel())
        assert rms[0, g, big].min() > 3.0 and rms[0, g].max() < 5.0
    normal = rms[rms < 2.0]
    assert abs(normal.mean().item() - 0.5) < 0.01
    assert abs(q.float().std().item() - 0.5) < 0.01 and abs(v.float().std().item() - 0.5) < 0.01
    assert int(round(0.01 * 32768)) == 328


def test_outlier_rows_are_exact_multiples():
    """The same draw without the outlier step gives K rows whose bf16 values times 8 are
    exactly the outlier rows (q is drawn first, so it is identical)."""
    kw = dict(seed=5, sigma=0.5)
    q0, k0, _ = workloads.make_inputs(1, 2, 1, 64, 500, 64, "bf16", **kw)
    q1, k1, _ = workloads.make_inputs(1, 2, 1, 64, 500, 64, "bf16", outlier_frac=0.01,
                                      outlier_mult=8.0, **kw)
    assert torch.equal(q0, q1)
    ratio = k1.float() / k0.float()
    rows = torch.nonzero((ratio[0, 0] == 8.0).all(-1)).flatten()
    same = torch.nonzero((ratio[0, 0] == 1.0).all(-1)).flatten()
    assert rows.numel() == 5 and same.numel() == 495


def test_default_scale_is_the_fp32_inverse_square_root():
    for d in (64, 128):
        assert workloads.default_scale(d) == float(np.float32(1.0 / math.sqrt(d)))
