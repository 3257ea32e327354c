"""The shared seeded input generator: deterministic, subset-consistent, dtype-exact."""

import numpy as np
import torch

import workloads as wl


def test_rows_are_subset_consistent_and_deterministic():
    full = wl.token_range(7, "k", 0, 1000, 2, 8)
    rows = np.array([999, 3, 512, 0, 257, 256, 255])
    part = wl.token_rows(7, "k", rows, 2, 8)
    assert torch.equal(part, full[torch.as_tensor(rows)])
    assert torch.equal(full, wl.token_range(7, "k", 0, 1000, 2, 8))
    assert not torch.equal(full, wl.token_range(8, "k", 0, 1000, 2, 8))
    assert not torch.equal(full, wl.token_range(7, "v", 0, 1000, 2, 8))


def test_distributions_and_rounding():
    u = wl.token_range(1, "v", 0, 4096, 1, 16, dist="uniform")
    assert float(u.min()) >= -1.0 and float(u.max()) <= 1.0
    n = wl.token_range(1, "q", 0, 4096, 1, 16)
    assert abs(float(n.mean())) < 0.02 and abs(float(n.std()) - 1.0) < 0.02
    b16 = wl.token_range(1, "q", 0, 64, 1, 16, dtype=torch.bfloat16)
    assert torch.equal(b16, n[:64].to(torch.bfloat16))
    k2 = wl.token_range(1, "k", 0, 64, 1, 16, scale=2.0, dtype=torch.bfloat16)
    assert torch.equal(k2.float(), 2.0 * wl.token_range(1, "k", 0, 64, 1, 16, dtype=torch.bfloat16).float())


def test_workload_presets():
    for w in wl.WORKLOADS.values():
        assert w.N % w.P == 0 and w.Hq % w.Hkv == 0
        assert all(0 <= u < w.P for u in w.ranks)


def test_sample_local_rows():
    s = wl.sample_local_rows(1000, 64, 5, 2)
    assert s.size == 64 and s[0] == 0 and s[1] == 1 and s[-1] == 999
    assert np.all(np.diff(s) > 0)
    assert np.array_equal(s, wl.sample_local_rows(1000, 64, 5, 2))
    assert np.array_equal(wl.sample_local_rows(10, 64, 5, 0), np.arange(10))


def test_threaded_oracle_rows_equal_plain_oracle_rows():
    """The thread-pool evaluation used for large parity samples gives the plain
    oracle's values (it only splits the rows)."""
    import numpy as np

    import parity_util as pu

    w = wl.Workload("thr", N=2048, P=4, ranks=(3,), layout="striped", causal=True, Hq=4, Hkv=2, d=64,
                    dtype="bf16", seed=5)
    k_glob, v_glob = wl.global_kv(w)
    rows = wl.sample_local_rows(w.b, 300, 5, 0)
    o1, l1 = pu.oracle_rows(w, 3, rows, k_glob, v_glob)
    o2, l2 = pu.oracle_rows_threaded(w, 3, rows, k_glob, v_glob, threads=3)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)
