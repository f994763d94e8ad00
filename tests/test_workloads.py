"""Host-side checks of the seeded input recipe (no attention arithmetic)."""
import numpy as np
import torch

from exact_attention_flashattention_amd import workloads as wl
from oracle import attention_oracle as ao


def test_bf16_cast_is_round_to_nearest_even():
    x = torch.tensor([1.00390625, 1.01171875, -1.00390625, 3.0e38], dtype=torch.float32)
    y = x.to(torch.bfloat16).float()
    assert y[0].item() == 1.0          # halfway, ties to even (mantissa 0)
    assert y[1].item() == 1.015625     # halfway, ties to even (mantissa 2)
    assert y[2].item() == -1.0


def test_prefill_recipe_is_deterministic_and_shaped():
    a = wl.prefill_inputs(2, 33, 4, 2, 64, seed=7)
    b = wl.prefill_inputs(2, 33, 4, 2, 64, seed=7)
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    assert a.q.shape == (2, 33, 4, 64) and a.k.shape == (2, 33, 2, 64)
    assert a.q.dtype == torch.bfloat16
    h = wl.prefill_inputs(2, 33, 4, 2, 64, seed=7, layout="BHND", dtype=torch.float32)
    assert h.q.shape == (2, 4, 33, 64) and h.q.dtype == torch.float32
    # bf16 draws are the float32 draws rounded once
    f = wl.prefill_inputs(2, 33, 4, 2, 64, seed=7, dtype=torch.float32)
    assert torch.equal(f.q.to(torch.bfloat16), a.q)


def test_workload_1_matches_its_description():
    w = wl.workload_1()
    assert (w.B, w.N, w.Hq, w.Hkv, w.d, w.layout) == (1, 128, 4, 2, 64, "BHND")
    assert w.q.dtype == torch.float32 and w.scale == 0.125


def test_paged_recipe_table_is_a_permutation_of_the_pool():
    x = wl.paged_decode_inputs(3, 8, 2, 64, [37, 16, 1], seed=5, page_size=16)
    n = [ao.pages_needed(L, 16) for L in (37, 16, 1)]
    assert x.num_pages == sum(n) == 5
    used = []
    for b in range(3):
        row = x.block_table[b].tolist()
        used += row[:n[b]]
        assert all(e == -1 for e in row[n[b]:])
    assert sorted(used) == list(range(5))
    y = wl.paged_decode_inputs(3, 8, 2, 64, [37, 16, 1], seed=5, page_size=16, permute=False)
    assert y.block_table[0, :3].tolist() == [0, 1, 2] and y.block_table[2, 0].item() == 4


def test_identity_table_pool_is_a_contiguous_cache():
    x = wl.paged_decode_inputs(2, 4, 2, 8, [32, 32], seed=9, page_size=16, permute=False)
    flat = x.k_pages.reshape(2, 32, 2, 8)
    for b in range(2):
        g = ao.gather_kv_ref(x.k_pages.float().numpy(), x.block_table[b].numpy(), 32, 16)
        assert np.array_equal(g, flat[b].float().numpy())


def test_pool_size_follows_cache_size_formula():
    lens = [1000, 17, 4096]
    x = wl.paged_decode_inputs(3, 8, 4, 128, lens, seed=1, page_size=16)
    pool_bytes = 2 * x.k_pages.numel() * 2  # K and V, bf16
    exact = ao.kv_cache_bytes(1, 4, sum(lens), 128, 2)
    waste = pool_bytes - exact
    assert 0 <= waste < 3 * 16 * ao.kv_cache_bytes(1, 4, 1, 128, 2)


def test_poison_marks_only_unused_slots():
    x = wl.paged_decode_inputs(2, 4, 2, 8, [5, 16], seed=2, page_size=4)
    before = x.k_pages.clone()
    wl.poison_unused_slots(x)
    for b, L in enumerate((5, 16)):
        g = ao.gather_kv_ref(x.k_pages.float().numpy(), x.block_table[b].numpy(), L, 4)
        ref = ao.gather_kv_ref(before.float().numpy(), x.block_table[b].numpy(), L, 4)
        assert np.array_equal(g, ref)
    last = int(x.block_table[0, 1])
    assert torch.isnan(x.k_pages[last, 1:].float()).all()


def test_random_lengths_are_in_range():
    x = wl.paged_decode_inputs(4, 8, 2, 16, (100, 140), seed=11, page_size=16)
    assert all(100 <= L <= 140 for L in x.seq_lens.tolist())
