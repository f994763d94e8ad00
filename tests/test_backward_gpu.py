"""Backward of the prefill on the GPU (through the C ABI) against the CPU
float64 oracle: dq, dk and dv element by element on small and ragged shapes
(both layouts, causal and not, MHA / GQA / MQA, d = 64 and 128), whole head
groups of the full-size workloads, and run-to-run bit identity.

The GPU backward takes the GPU forward's o and lse (the product path); the
oracle computes the exact gradients from q, k, v and dout alone.

Tolerance against the fp64 oracle (bf16 inputs and outputs, fp32
accumulation): every element within 2e-2 + 2^-8 |ref|, and mean-abs <= 5e-3.
The absolute part is the forward's bar. The relative part is needed because
the gradients of a KV head sum over its g query heads and reach |dv| ~ 12
for g = 8, where storing in bf16 alone costs up to half an ulp = 2^-8 |x|
(0.03 at |x| in [8, 16)); P and dS are also rounded to bf16 (2^-9 relative)
before the dV, dK, dQ products, and D = rowsum(dO * O) uses the bf16 forward
output, errors that stay well inside the absolute part at these shapes.
"""
import sys

import numpy as np
import pytest
import torch

from exact_attention_flashattention_amd import binding as bd
from exact_attention_flashattention_amd import workloads as wl
from oracle import attention_oracle as ao

pytestmark = pytest.mark.gpu

BF16_ABS, BF16_REL, BF16_MEAN = 2e-2, 2.0 ** -8, 5e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bits(t):
    return t.view(torch.int16)


def gpu_grads(x: wl.PrefillInputs, dout):
    q, k, v, do = x.q.cuda(), x.k.cuda(), x.v.cuda(), dout.cuda()
    B, Hq, N = x.B, x.Hq, x.N
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    o = bd.attn_prefill_ex(q, k, v, causal=x.causal, scale=x.scale, layout=x.layout, lse=lse)
    dq, dk, dv = bd.attn_backward(q, k, v, o, do, lse, causal=x.causal, scale=x.scale, layout=x.layout)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check(name, got, ref):
    e = np.abs(got.double().numpy() - ref)
    excess = (e - (BF16_ABS + BF16_REL * np.abs(ref))).max()
    log(f"  {name}: max-abs {e.max():.3e} mean-abs {e.mean():.3e} (max |ref| {np.abs(ref).max():.2f}, "
        f"worst margin {excess:.3e})")
    assert excess <= 0 and e.mean() <= BF16_MEAN, name


CASES = [
    # B, N, Hq, Hkv, d, causal, layout
    (1, 1, 2, 1, 64, True, "BNHD"),       # one token
    (2, 77, 4, 2, 128, True, "BNHD"),     # shorter than a tile
    (1, 200, 8, 2, 64, False, "BNHD"),    # full attention, ragged
    (2, 300, 4, 4, 128, True, "BHND"),    # MHA, head-major layout
    (1, 513, 8, 1, 128, True, "BNHD"),    # MQA, several key blocks and query tiles
    (1, 129, 6, 3, 64, True, "BHND"),
    (1, 256, 4, 2, 128, False, "BHND"),   # tile-aligned, full attention
    (1, 640, 16, 1, 128, True, "BNHD"),   # g = 16, an odd number of 128-key blocks (one runs alone)
    (2, 384, 8, 2, 64, False, "BHND"),    # three key blocks, full attention
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_backward_small(case):
    B, N, Hq, Hkv, d, causal, layout = case
    x = wl.prefill_inputs(B, N, Hq, Hkv, d, seed=800 + N, layout=layout, causal=causal)
    dout = wl.output_gradient(x, seed=801 + N)
    log(f"case: B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} causal={causal} layout={layout}")
    dq, dk, dv = gpu_grads(x, dout)
    rq, rk, rv = ao.sdpa_backward_ref(ao.to_bhnd(x.q, layout), ao.to_bhnd(x.k, layout), ao.to_bhnd(x.v, layout),
                                      ao.to_bhnd(dout, layout), x.scale, causal)
    check("dq", dq, ao.from_bhnd(rq, layout))
    check("dk", dk, ao.from_bhnd(rk, layout))
    check("dv", dv, ao.from_bhnd(rv, layout))


def test_backward_is_deterministic():
    x = wl.prefill_inputs(2, 333, 8, 2, 128, seed=820)
    dout = wl.output_gradient(x, seed=821)
    a = gpu_grads(x, dout)
    b = gpu_grads(x, dout)
    for u, w in zip(a, b):
        assert torch.equal(bits(u), bits(w))


def group_check(x: wl.PrefillInputs, dout, b: int, kvh: int):
    """Compare one (batch entry, KV head) group — the KV head and its g query
    heads, a self-contained sub-problem — against the oracle."""
    dq, dk, dv = gpu_grads(x, dout)
    g = x.Hq // x.Hkv
    heads = list(range(kvh * g, (kvh + 1) * g))
    t = lambda a, hs: ao.as_f64(a[b:b + 1][:, :, hs]).transpose(0, 2, 1, 3)  # BNHD -> [1, H, N, d]
    rq, rk, rv = ao.sdpa_backward_ref(t(x.q, heads), t(x.k, [kvh]), t(x.v, [kvh]), t(dout, heads), x.scale,
                                      x.causal)
    check("dq", dq[b][:, heads], rq[0].transpose(1, 0, 2))
    check("dk", dk[b][:, [kvh]], rk[0].transpose(1, 0, 2))
    check("dv", dv[b][:, [kvh]], rv[0].transpose(1, 0, 2))


def test_workload_2_shape_full_head_group():
    x = wl.workload_2()
    dout = wl.output_gradient(x, seed=144)
    log(f"case: {x.name}, head group (b=3, kv head 5)")
    group_check(x, dout, 3, 5)


@pytest.mark.parametrize("hkv", [16, 1])
def test_workload_3_shape_full_head_group(hkv):
    x = wl.workload_3(hkv)
    dout = wl.output_gradient(x, seed=145)
    log(f"case: {x.name}, head group (b=6, kv head {hkv - 1})")
    group_check(x, dout, 6, hkv - 1)


def test_backward_on_a_stream_other_than_the_current_one():
    """With no workspace passed, the binding allocates the backward's scratch
    on the launch stream, so later allocations on that stream are ordered
    behind the kernels. The backward runs on a side stream, which at once
    allocates and fills NaN blocks of the workspace's size; the gradients
    must still match the oracle."""
    x = wl.prefill_inputs(1, 300, 8, 2, 128, seed=840)
    dout = wl.output_gradient(x, seed=841)
    q, k, v, do = x.q.cuda(), x.k.cuda(), x.v.cuda(), dout.cuda()
    lse = torch.empty((x.B, x.Hq, x.N), dtype=torch.float32, device="cuda")
    o = bd.attn_prefill_ex(q, k, v, causal=True, scale=x.scale, lse=lse)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    log("case: backward B=1 N=300 Hq=8 Hkv=2 d=128 on a side stream")
    dq, dk, dv = bd.attn_backward(q, k, v, o, do, lse, causal=True, scale=x.scale, stream=side)
    need = bd.attn_backward_workspace_size(x.B, x.N, x.Hq)
    with torch.cuda.stream(side):
        junk = [torch.full((need // 4 + 4,), float("nan"), device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    del junk
    rq, rk, rv = ao.sdpa_backward_ref(ao.to_bhnd(x.q, "BNHD"), ao.to_bhnd(x.k, "BNHD"), ao.to_bhnd(x.v, "BNHD"),
                                      ao.to_bhnd(dout, "BNHD"), x.scale, True)
    check("dq", dq.cpu(), ao.from_bhnd(rq, "BNHD"))
    check("dk", dk.cpu(), ao.from_bhnd(rk, "BNHD"))
    check("dv", dv.cpu(), ao.from_bhnd(rv, "BNHD"))
