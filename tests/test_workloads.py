"""The shared input generator: bf16 rounding, determinism, subsets, masks (CPU)."""

import numpy as np
import torch

from workloads import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_block_keep, make_workload, random_f16


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.normal(size=100000).astype(np.float32),
                        (rng.normal(size=1000) * 1e-39).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(x), ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                                  .float().numpy())


def test_f16_inputs_round_like_torch():
    x = random_f16(5, (3, 200, 64), "block_offset")
    assert x.dtype == np.float16
    rng = np.random.default_rng(np.random.SeedSequence([5, 0]))
    raw = rng.standard_normal((3, 200, 64), dtype=np.float32)
    # the offsets move values, the rounding must still be torch's float -> half
    np.testing.assert_array_equal(random_f16(5, (3, 200, 64), "normal"),
                                  torch.from_numpy(raw).half().numpy())
    assert 0.9 < float(np.std(x.astype(np.float64))) < 1.3
    np.testing.assert_array_equal(x, random_f16(5, (3, 200, 64), "block_offset"))


def test_deterministic_and_head_subsets():
    a = make_workload("c2_dense_8k", S=512, N=4)
    b = make_workload("c2_dense_8k", S=512, N=4)
    np.testing.assert_array_equal(a.q, b.q)
    sub = make_workload("c2_dense_8k", S=512, N=4, heads=[2])
    np.testing.assert_array_equal(sub.q[:, 0], a.q[:, 2])
    np.testing.assert_array_equal(sub.k[:, 0], a.k[:, 2])


def test_recipes_statistics():
    w = make_workload("c4_blocksparse_64k", S=4096, N=2)
    q = bf16_bits_to_f32(w.q)
    blk_means = q[0, 0].reshape(32, 128, -1).mean(axis=1)
    assert 0.3 < blk_means.std() < 0.7               # per-block offsets N(0, 0.5^2)
    assert w.keep.shape == (1, 2, 32, 32)
    assert np.all(np.diagonal(w.keep, axis1=2, axis2=3) == 1)
    c5 = make_workload("c5_qbsa_60k", S=2048, N=1)
    v = bf16_bits_to_f32(c5.v)[0, 0]
    chan = np.abs(v).mean(axis=0)
    assert chan.max() / chan.min() > 3                # log-normal channel magnitudes


def test_keep_rate():
    keep = make_block_keep(1004, 1, 4, 512, 512, 0.1)
    frac = keep.mean()
    assert abs(frac - (0.1 + 0.9 / 512)) < 0.005


def test_varlen_config():
    w = make_workload("c3_varlen_gqa_causal")
    lens = np.diff(w.cu_seqlens_q)
    assert len(lens) == 8 and lens.min() >= 512 and lens.max() <= 4096
    assert w.q.shape == (w.Sq, 32, 128) and w.k.shape == (w.Sq, 8, 128)
    assert w.sparse_mode == 3


def test_config_table_complete():
    assert set(CONFIGS) == {"c1_dense_small", "c2_dense_8k", "c3_varlen_gqa_causal", "c4_blocksparse_64k",
                            "c5_qbsa_60k"}
