"""The seeded input generators: published splitmix64 values, determinism, and the
structure of the given block indices."""
import numpy as np
import torch

import gen
from gen import workloads as W


def test_splitmix64_published_first_output():
    # splitmix64 seeded with 0 produces 0xE220A8397B1DCDAF first (Steele et al.;
    # the reference value quoted by every public port of the generator).
    assert gen._mix_int(gen._GAMMA) == 0xE220A8397B1DCDAF
    assert gen._mix_int(2 * gen._GAMMA) == 0x6E789E6AA1B965F4


def test_tensor_path_matches_python_ints():
    idx = torch.arange(0, 257, dtype=torch.int64)
    t = gen.u64_at(7, 3, idx)
    for i in (0, 1, 100, 256):
        want = gen.u64_py(7, 3, i)
        got = int(t[i]) & ((1 << 64) - 1)
        assert got == want


def test_normal_moments_and_determinism():
    a = gen.normal(11, 1, (1 << 16,))
    b = gen.normal(11, 1, (1 << 16,))
    assert torch.equal(a, b)
    assert abs(float(a.mean())) < 0.02
    assert abs(float(a.std()) - 1.0) < 0.02
    c = gen.normal(11, 2, (1 << 16,))
    assert not torch.equal(a, c)
    s = gen.sigmoid_normal(11, 4, (4096,))
    assert float(s.min()) > 0.0 and float(s.max()) < 1.0


def test_bf16_rounding_is_rne_of_fp32():
    x = gen.normal(3, 1, (4096,))
    y = gen.normal(3, 1, (4096,), dtype=torch.bfloat16)
    assert torch.equal(x.to(torch.bfloat16), y)


def test_uniform_lengths_in_range():
    w = W.nosa1b_decode()
    assert len(w.lengths) == 8
    assert all(8192 <= L <= 32768 for L in w.lengths)


def test_given_block_indices_structure():
    w = W.scaled(W.selected_prefill(), [300, 3000])
    idx = W.given_block_indices(w).numpy()
    pos = np.concatenate([np.arange(L) for L in w.lengths])
    for r in range(idx.shape[0]):
        t = pos[r]
        n_avail = t // 64 + 1
        for g in range(w.kv_heads):
            row = idx[r, g]
            valid = row[row >= 0]
            assert len(valid) == min(16, n_avail)
            assert np.all(valid <= t // 64)
            assert np.all(np.diff(valid) > 0)
            assert np.all(row[len(valid):] == -1)
    # the draw is not the same set for every row
    assert len({tuple(idx[r, 0]) for r in range(idx.shape[0] - 200, idx.shape[0])}) > 100
