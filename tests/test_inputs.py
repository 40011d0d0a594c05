"""Seeded synthetic inputs: determinism, the bf16 encoder and the distributions.  CPU only."""
import numpy as np
import torch

import mha_inputs as mi


def test_bf16_encoder_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38, 1e-40],
                                 dtype=np.float32)])
    # exact ties: 1 + 2^-8 rounds to 1 (even), 1 + 3*2^-8 rounds up to 1 + 2^-6
    ours = mi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert ours[-5] == 0x3F80 and ours[-4] == 0x3F82


def test_f16_encoder_matches_torch_rne():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00048828125, 1.00146484375, 65504.0, 6.0e-8, 7.0e4],
                                 dtype=np.float32)])
    # exact ties: 1 + 2^-11 rounds to 1 (even), 1 + 3*2^-11 rounds up to 1 + 2^-9;
    # 7e4 overflows to inf
    ours = mi.f32_to_f16_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert ours[-6] == 0x3C00 and ours[-5] == 0x3C00 and ours[-4] == 0x3C02 and ours[-1] == 0x7C00


def test_draw_is_deterministic_and_seed_dependent():
    a = mi.draw((1, 2, 8, 4), "bf16", 3)
    b = mi.draw((1, 2, 8, 4), "bf16", 3)
    c = mi.draw((1, 2, 8, 4), "bf16", 4)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[0], c[0])
    assert not np.array_equal(a[0], a[1])  # Q and K come from different streams


def test_distributions():
    w = mi.Workload("t", 2, 4, 4096, 64, "bf16", False, seed=9,
                    qk_dist=mi.Dist("normal", 3.0), v_dist=mi.Dist("uniform", -1.0, 1.0))
    q, k, v = mi.draw_qkv(w)
    dec = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    qf, vf = dec(q), dec(v)
    assert abs(qf.std() - 3.0) < 0.02 and abs(qf.mean()) < 0.02
    assert vf.min() >= -1.0 and vf.max() <= 1.0 and abs(vf.std() - 1 / np.sqrt(3)) < 0.01
    f = mi.draw((1, 1, 64, 64), "f32", 1)[0]
    assert f.dtype == np.float32 and f.shape == (1, 1, 64, 64)


def test_named_workloads():
    w = mi.WORKLOADS["bf16_B4_H32_N4096_d128_causal"]
    assert (w.B, w.H, w.N, w.d, w.causal, w.dtype) == (4, 32, 4096, 128, True, "bf16")
    assert w.credited_flops() == 4 * 4 * 32 * 4096 * 4096 * 128 / 2
    assert abs(w.scale - 1 / np.sqrt(128)) < 1e-15


def test_pages_sweep_table():
    # 32k tokens, sequence 1k..32k, hidden 2048 = H * d with d in {64, 128}, both masks
    assert len(mi.SWEEP) == 24
    for w in mi.SWEEP.values():
        assert w.B * w.N == 32768 and w.H * w.d == 2048 and w.dtype == "f16"
        assert w.N in (1024, 2048, 4096, 8192, 16384, 32768) and w.d in (64, 128)
    assert len({w.seed for w in mi.SWEEP.values()}) == 24
    q = mi.draw((1, 1, 8, 8), "f16", 3)[0]
    assert q.dtype == np.uint16


def test_decode_table_and_kv_shapes():
    for w in mi.DECODE.values():
        assert w.Nk > w.N and not w.causal and w.kv_shape == (w.B, w.H, w.Nk, w.d)
        assert w.credited_flops() == 4.0 * w.B * w.H * w.N * w.Nk * w.d
    assert len({w.seed for w in mi.DECODE.values()}) == len(mi.DECODE)
    q, k, v = mi.draw((1, 2, 3, 8), "bf16", 5, kv_shape=(1, 2, 40, 8))
    assert q.shape == (1, 2, 3, 8) and k.shape == v.shape == (1, 2, 40, 8)


def test_draw_paged_scatters_each_block_once():
    lens = [0, 1, 16, 17, 100]
    q, kp, vp, table, sl = mi.draw_paged(5, 3, 2, 64, "bf16", 16, lens, seed=11, spare=4)
    per = [-(-L // 16) for L in lens]
    assert q.shape == (5, 3, 2, 64) and kp.shape == vp.shape == (sum(per) + 4, 3, 16, 64)
    assert table.dtype == np.int32 and sl.dtype == np.int32 and list(sl) == lens
    assert table.shape == (5, max(per))
    used = np.concatenate([table[b, :c] for b, c in enumerate(per)])
    assert len(set(used.tolist())) == len(used) and used.min() >= 0 and used.max() < kp.shape[0]
    for b, c in enumerate(per):
        assert np.all(table[b, c:] == -1)
    again = mi.draw_paged(5, 3, 2, 64, "bf16", 16, lens, seed=11, spare=4)
    for x, y in zip((q, kp, vp, table, sl), again):
        np.testing.assert_array_equal(x, y)


def test_paged_workloads():
    for name, w in mi.PAGED.items():
        lens = mi.paged_lengths(w)
        assert lens.shape == (w.B,) and lens.min() >= w.len_lo and lens.max() <= w.len_hi, name
        assert w.block_size & (w.block_size - 1) == 0 and w.block_size >= 16, name
        assert name.startswith(w.dtype) and f"_bs{w.block_size}_" in name, name


def test_draw_gemm_and_workloads():
    a, b = mi.draw_gemm(5, 7, 9, "bf16", seed=3)
    assert a.shape == (5, 9) and b.shape == (9, 7) and a.dtype == np.uint16
    a2, b2 = mi.draw_gemm(5, 7, 9, "bf16", seed=3)
    np.testing.assert_array_equal(a, a2)
    np.testing.assert_array_equal(b, b2)
    assert not np.array_equal(mi.draw_gemm(5, 7, 9, "bf16", seed=4)[0], a)
    assert len(mi.GEMM) == 15 and len(mi.GEMM_MEMBOUND) == 3
    for name, w in list(mi.GEMM.items()) + list(mi.GEMM_MEMBOUND.items()):
        assert name == f"bf16_gemm_M{w.M}_N{w.N}_K{w.K}" and w.flops() == 2.0 * w.M * w.N * w.K
