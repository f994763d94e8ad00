"""Absorbed-MLA decode on the GPU (through the C ABI) against the CPU float64
oracle: ragged lengths, an empty sequence, several split counts, head counts
that leave waves idle, NaN-poisoned unused slots, a permuted table against the
identity table (bit-exact), and the whole output of the full-size workload.

Tolerance against the fp64 oracle: bf16 inputs, fp32 accumulation,
max-abs <= 2e-2 and mean-abs <= 5e-3 (the outputs are convex combinations of
N(0, 1) latent values, as in the GQA decode).
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


def run(x: wl.MlaDecodeInputs, splits=0):
    o = bd.attn_decode_mla(x.q.cuda(), x.kv_pages.cuda(), x.block_table.cuda(), x.seq_lens.cuda(),
                           scale=x.scale, num_splits=splits)
    torch.cuda.synchronize()
    return o.cpu()


CASES = [
    # B, Hq, seq_lens, splits
    (2, 16, [1, 17], 0),
    (3, 32, [100, 33, 511], 0),
    (2, 128, [1000, 2049], 3),
    (1, 144, [700], 0),              # a second head chunk with one live wave
    (4, 64, [0, 16, 31, 64], 0),     # an empty sequence
    (2, 128, [4097, 3000], 1),       # one split: every page in one work-group
    (2, 48, [5000, 1], 40),          # more splits than some sequences have pages
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_mla_small_poisoned(case):
    B, Hq, lens, splits = case
    x = wl.mla_decode_inputs(B, Hq, 512, 64, lens, seed=900 + sum(lens))
    wl.poison_unused_mla_slots(x)
    log(f"case: B={B} Hq={Hq} lens={lens} splits={splits}")
    got = run(x, splits)
    ref = ao.mla_decode_ref(x.q, x.kv_pages, x.block_table, x.seq_lens, x.scale, 512)
    e = np.abs(got.double().numpy() - ref)
    log(f"  max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
    assert e.max() <= BF16_MAX and e.mean() <= BF16_MEAN
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.count_nonzero(got[b]) == 0


def test_mla_permuted_table_is_bit_identical_to_identity():
    a = wl.mla_decode_inputs(2, 64, 512, 64, [777, 1500], seed=950, permute=False)
    b = wl.mla_decode_inputs(2, 64, 512, 64, [777, 1500], seed=950, permute=True)
    # same rows, placed through a different table: move b's pool so that the
    # logical cache equals a's
    for s in range(2):
        for pg in range(-(-int(a.seq_lens[s]) // 16)):
            b.kv_pages[int(b.block_table[s, pg])] = a.kv_pages[int(a.block_table[s, pg])]
    ga, gb = run(a), run(b)
    assert torch.equal(ga.view(torch.int16), gb.view(torch.int16))


def test_workload_7_full_size():
    """Every head of every sequence of the full-size workload against the oracle."""
    x = wl.workload_7()
    log(f"case: {x.name}, seq_lens={x.seq_lens.tolist()}")
    got = run(x)
    assert bool(torch.isfinite(got.float()).all())
    ref = ao.mla_decode_ref(x.q, x.kv_pages, x.block_table, x.seq_lens, x.scale, x.d_c)
    e = np.abs(got.double().numpy() - ref)
    log(f"  whole output: max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
    assert e.max() <= BF16_MAX and e.mean() <= BF16_MEAN


def test_mla_on_a_stream_other_than_the_current_one():
    """The MLA call's own scratch (split partials) belongs to the launch
    stream: the decode runs on a side stream with no workspace passed, and
    the side stream at once allocates and fills NaN blocks of the
    workspace's size; the output must still match the oracle."""
    x = wl.mla_decode_inputs(3, 128, 512, 64, [3000, 17, 1200], seed=960)
    q, kv, bt, sl = x.q.cuda(), x.kv_pages.cuda(), x.block_table.cuda(), x.seq_lens.cuda()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o = torch.empty((x.B, x.Hq, 512), dtype=torch.bfloat16, device="cuda")
    log("case: MLA B=3 Hq=128 lens=[3000, 17, 1200] splits=5 on a side stream")
    bd.attn_decode_mla(q, kv, bt, sl, o, scale=x.scale, num_splits=5, stream=side)
    need = bd.attn_decode_mla_workspace_size(x.B, x.Hq, x.block_table.shape[1], 5)
    with torch.cuda.stream(side):
        junk = [torch.full((need // 4 + 4,), float("nan"), device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    del junk
    ref = ao.mla_decode_ref(x.q, x.kv_pages, x.block_table, x.seq_lens, x.scale, 512)
    e = np.abs(o.cpu().double().numpy() - ref)
    log(f"  max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
    assert e.max() <= BF16_MAX and e.mean() <= BF16_MEAN
