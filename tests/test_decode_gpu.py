"""Paged decode parity on the GPU: the split-K kernel plus LSE merge (through
the C ABI) against the CPU float64 oracle, with NaN-poisoned unused slots,
ragged lengths, empty sequences, several split counts, and the bit-exact
requirements (gather indices; permuted table == identity table).

Tolerance against the fp64 oracle: bf16 inputs, fp32 accumulation,
max-abs <= 2e-2 and mean-abs <= 5e-3.
"""
import sys

import numpy as np
import pytest
import torch

from exact_attention_flashattention_amd import binding as bd
from exact_attention_flashattention_amd import workloads as wl
from oracle import attention_oracle as ao

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 5e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_gpu(x: wl.DecodeInputs):
    return [t.cuda() for t in (x.q, x.k_pages, x.v_pages, x.block_table, x.seq_lens)]


def run(x: wl.DecodeInputs, num_splits=0):
    q, kp, vp, bt, sl = to_gpu(x)
    o = bd.attn_decode(q, kp, vp, bt, sl, scale=x.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.cpu()


def oracle(x: wl.DecodeInputs):
    return ao.decode_ref(x.q, x.k_pages, x.v_pages, x.block_table, x.seq_lens, x.scale)


def check(got, ref, what=""):
    e = np.abs(got.double().numpy() - ref)
    log(f"  {what} max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
    assert e.max() <= BF16_MAX and e.mean() <= BF16_MEAN


LENS = [1, 15, 16, 17, 100, 257, 1000]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 8), (8, 1), (64, 8), (32, 1)])
def test_small_poisoned(d, Hq, Hkv):
    x = wl.paged_decode_inputs(len(LENS), Hq, Hkv, d, LENS, seed=d + Hq + Hkv)
    wl.poison_unused_slots(x)
    log(f"case: decode Hq={Hq} Hkv={Hkv} d={d} lens={LENS}")
    got = run(x)
    assert bool(torch.isfinite(got.float()).all())
    check(got, oracle(x))


@pytest.mark.parametrize("splits", [1, 2, 7, 0, 100])
def test_split_counts(splits):
    x = wl.paged_decode_inputs(3, 16, 4, 128, [500, 33, 1600], seed=21)
    wl.poison_unused_slots(x)
    ref = oracle(x)
    got = run(x, num_splits=splits)
    check(got, ref, f"splits={splits}")


def test_empty_sequence_gives_zero():
    x = wl.paged_decode_inputs(3, 8, 2, 128, [40, 0, 5], seed=22)
    wl.poison_unused_slots(x)
    got = run(x)
    assert torch.equal(got[1], torch.zeros_like(got[1]))
    check(got, oracle(x))


def test_permuted_table_is_bit_identical_to_identity():
    lens = [700, 31, 1234, 16]
    a = wl.paged_decode_inputs(4, 32, 8, 128, lens, seed=23, permute=False)
    n = a.num_pages
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(5))
    b = wl.DecodeInputs(a.q, torch.empty_like(a.k_pages), torch.empty_like(a.v_pages),
                        a.block_table.clone(), a.seq_lens, a.B, a.Hq, a.Hkv, a.d, a.page_size,
                        a.max_pages_per_seq, a.scale)
    b.k_pages[perm] = a.k_pages
    b.v_pages[perm] = a.v_pages
    used = a.block_table >= 0
    b.block_table[used] = perm[a.block_table[used].long()].to(torch.int32)
    for splits in (0, 3):
        oa, ob = run(a, splits), run(b, splits)
        assert torch.equal(oa, ob)


def test_gather_is_bit_exact():
    x = wl.paged_decode_inputs(3, 8, 4, 64, [50, 16, 129], seed=24)
    wl.poison_unused_slots(x)
    _, kp, _, bt, sl = to_gpu(x)
    out = bd.attn_gather_pages(kp, bt, sl, max_len=129)
    torch.cuda.synchronize()
    bits = out.cpu().view(torch.int16)
    pool_bits = x.k_pages.view(torch.int16).numpy()  # compare raw bit patterns
    for b, L in enumerate([50, 16, 129]):
        ref = ao.gather_kv_ref(pool_bits, x.block_table[b].numpy(), L, 16)
        assert np.array_equal(bits[b, :L].numpy(), ref)
        assert not bits[b, L:].any()


def test_decode_equals_prefill_row():
    # the decode of token t equals row t of the causal prefill (both against the oracle)
    N, Hq, Hkv, d = 300, 8, 2, 128
    x = wl.prefill_inputs(1, N, Hq, Hkv, d, seed=25)
    for t in (0, 16, 17, 299):
        L = t + 1
        pages = (L + 15) // 16
        kp = torch.zeros(pages * 16, Hkv, d, dtype=torch.bfloat16)
        vp = torch.zeros_like(kp)
        kp[:L], vp[:L] = x.k[0, :L], x.v[0, :L]
        dx = wl.DecodeInputs(x.q[:, t].contiguous(), kp.view(pages, 16, Hkv, d), vp.view(pages, 16, Hkv, d),
                             torch.arange(pages, dtype=torch.int32)[None], torch.tensor([L], dtype=torch.int32),
                             1, Hq, Hkv, d, 16, pages, x.scale)
        got = run(dx)
        ref = ao.prefill_rows_ref(x.q, x.k, x.v, x.scale, [(0, t, h) for h in range(Hq)])
        check(got[0], ref, f"t={t}")


def full_size(x: wl.DecodeInputs, batches=None):
    log(f"case: {x.name} num_pages={x.num_pages}")
    o = run(x)
    assert bool(torch.isfinite(o.float()).all())
    sel = range(x.B) if batches is None else batches
    sub = wl.DecodeInputs(x.q[list(sel)], x.k_pages, x.v_pages, x.block_table[list(sel)],
                          x.seq_lens[list(sel)], len(sel), x.Hq, x.Hkv, x.d, x.page_size,
                          x.max_pages_per_seq, x.scale)
    check(o[list(sel)], oracle(sub), f"{len(sel)} sequences")


def test_workload_4_full_size():
    full_size(wl.workload_4())


def test_workload_5_full_size():
    full_size(wl.workload_5())


def test_launch_stream_other_than_the_current_one():
    """The binding's own workspace belongs to the launch stream: after the call
    returns, the next allocations on that stream are stream-ordered behind the
    kernels. Here the decode runs on a side stream with no workspace passed,
    and the side stream at once allocates and fills memory of the same size
    many times; the output must still match the oracle."""
    x = wl.paged_decode_inputs(3, 32, 8, 128, [4000, 17, 2500], seed=31)
    q, kp, vp, bt, sl = to_gpu(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o = torch.empty_like(q)
    bd.attn_decode(q, kp, vp, bt, sl, o, scale=x.scale, num_splits=7, stream=side)
    need = bd.attn_decode_workspace_size(x.B, x.Hq, x.Hkv, x.d, x.max_pages_per_seq, 7)
    with torch.cuda.stream(side):
        junk = [torch.full((need // 4 + 4,), float("nan"), device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    del junk
    check(o.cpu(), oracle(x), "side stream")
