"""The seeded input generators: determinism and bf16 rounding (CPU only)."""
import numpy as np
import torch

from workloads import bf16_bits, bf16_to_f32, centres, head_kv_numpy, workload, rng


def test_bf16_rounding_matches_torch_cast():
    x = rng(400).standard_normal(100000).astype(np.float32) * np.float32(3.7)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 65504.0]   # ties to even
    ours = bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_deterministic_and_shaped():
    w = workload(2, T=300)
    mu, qb, _ = centres(w)
    assert mu.shape == (1, 8, 128) and qb.dtype == np.float32
    K1, V1 = head_kv_numpy(w, 0, 0, mu)
    K2, V2 = head_kv_numpy(w, 0, 0, mu)
    assert K1.dtype == np.uint16 and np.array_equal(K1, K2) and np.array_equal(V1, V2)


def test_workload_shapes():
    w3 = workload(3)
    assert w3.entries == 36 * 8 * 8 * 32768
    w5 = workload(5)
    assert np.all(w5.seq_len >= 4096) and np.all(w5.seq_len <= 32768)
    assert np.all(w5.prompt_len >= 128) and np.all(w5.prompt_len <= 4096)
    w4 = workload(4)
    assert w4.t_cap == 2176 and np.all((w4.prompt_len >= 256) & (w4.prompt_len <= 2048))
