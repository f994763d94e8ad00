"""attn_decode_noalloc on the GPU: the decode whose split partials live in
the library's fixed per-GPU scratch array instead of a caller workspace,
for callers that cannot allocate device memory. Called through the C ABI
and compared with attn_decode on the same arguments (same kernels and split
count, so bit-identical) and with the CPU float64 oracle (bf16 bar:
max-abs <= 2e-2, mean-abs <= 5e-3), on two calls in a row, the second with a
smaller input (fewer sequences, heads and pages), so a stale partial left by
the first call would show up in the second."""
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


def both(x, splits):
    q, kp, vp, bt, sl = [t.cuda() for t in (x.q, x.k_pages, x.v_pages, x.block_table, x.seq_lens)]
    o_ws = bd.attn_decode(q, kp, vp, bt, sl, scale=x.scale, num_splits=splits)
    o_na = torch.full_like(q, float("nan"))
    bd.attn_decode_noalloc(q, kp, vp, bt, sl, o_na, scale=x.scale, num_splits=splits)
    torch.cuda.synchronize()
    return o_ws.cpu(), o_na.cpu()


def check(x, splits, what):
    log(f"case: {what} B={x.B} Hq={x.Hq} Hkv={x.Hkv} d={x.d} lens={x.seq_lens.tolist()} splits={splits}")
    o_ws, o_na = both(x, splits)
    assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16))
    ref = ao.decode_ref(x.q, x.k_pages, x.v_pages, x.block_table, x.seq_lens, x.scale)
    e = np.abs(o_na.double().numpy() - ref)
    log(f"  bit-identical to attn_decode; vs oracle max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
    assert e.max() <= BF16_MAX and e.mean() <= BF16_MEAN


@pytest.mark.parametrize("splits", [0, 5])
def test_two_calls_second_smaller(splits):
    big = wl.paged_decode_inputs(4, 32, 8, 128, [5000, 33, 1700, 2999], seed=1201)
    wl.poison_unused_slots(big)
    check(big, splits, "first (larger)")
    small = wl.paged_decode_inputs(2, 8, 2, 64, [300, 0], seed=1202)
    wl.poison_unused_slots(small)
    check(small, splits, "second (smaller, one empty sequence)")


def test_long_context_workload():
    """The long-context decode the benchmark times (its automatic split count
    needs 8.5 MB of the 16 MiB scratch)."""
    x = wl.workload_5()
    log(f"case: {x.name}")
    q, kp, vp, bt, sl = [t.cuda() for t in (x.q, x.k_pages, x.v_pages, x.block_table, x.seq_lens)]
    o_ws = bd.attn_decode(q, kp, vp, bt, sl, scale=x.scale)
    o_na = torch.empty_like(q)
    bd.attn_decode_noalloc(q, kp, vp, bt, sl, o_na, scale=x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_na.cpu().view(torch.int16), o_ws.cpu().view(torch.int16))


def test_oversized_call_is_refused():
    # 8 sequences x 64 heads x 1024 splits x (128 + 2) floats = 272 MB of
    # partials, far past the 16 MiB scratch: refused on the host, nothing runs
    x = wl.paged_decode_inputs(8, 64, 8, 128, [16] * 8, seed=1203, max_pages_per_seq=1024)
    q, kp, vp, bt, sl = [t.cuda() for t in (x.q, x.k_pages, x.v_pages, x.block_table, x.seq_lens)]
    o = torch.zeros_like(q)
    with pytest.raises(bd.AttnError) as ei:
        bd.attn_decode_noalloc(q, kp, vp, bt, sl, o, scale=x.scale, num_splits=1024)
    assert ei.value.status == -11
    torch.cuda.synchronize()
    assert torch.count_nonzero(o.cpu()) == 0      # no output written
