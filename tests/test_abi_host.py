"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host with the documented
status codes before any launch (so no kernel runs in these tests)."""
import ctypes
import os
import re

import pytest

from exact_attention_flashattention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def header_enum(name):
    text = open(HEADER).read()
    m = re.search(rf"\b{name}\s*=\s*(-?\d+)", text)
    return int(m.group(1))


@pytest.fixture(scope="module")
def L():
    return binding.lib()


def test_every_declared_symbol_is_exported(L):
    names = header_functions()
    assert len(names) == 17
    for n in names:
        assert hasattr(L, n), n
    assert sorted(n for n, _, _ in binding.SIGNATURES) == names


def test_status_strings_and_version(L):
    for code in range(0, -12, -1):
        s = binding.status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in binding.status_string(-99)
    assert L.attn_version() >= 10000


# Host buffers stand in for device pointers: every call below fails validation
# before anything touches the GPU.
BUF = (ctypes.c_uint8 * 4096)()
A = (ctypes.addressof(BUF) + 15) & ~15
ERR = {n: header_enum(n) for n in ("ATTN_ERR_NULL", "ATTN_ERR_SHAPE", "ATTN_ERR_GQA", "ATTN_ERR_HEAD_DIM",
                                  "ATTN_ERR_DTYPE", "ATTN_ERR_LAYOUT", "ATTN_ERR_WORKSPACE",
                                  "ATTN_ERR_ALIGN", "ATTN_ERR_PAGE", "ATTN_ERR_SCRATCH")}


def prefill(L, **kw):
    a = dict(q=A, k=A, v=A, o=A, lse=None, B=1, N=8, Hq=4, Hkv=2, d=64, scale=0.125, causal=1,
             dtype=1, layout=0, var=None)
    a.update(kw)
    return L.attn_prefill_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["N"], a["Hq"], a["Hkv"],
                             a["d"], a["scale"], a["causal"], a["dtype"], a["layout"], a["var"], None)


def var(window=0, n_sink=0, sinks=None):
    return ctypes.pointer(binding.AttnVariant(window, n_sink, sinks))


@pytest.mark.parametrize("kw,err", [
    (dict(q=None), "ATTN_ERR_NULL"), (dict(o=None), "ATTN_ERR_NULL"),
    (dict(B=0), "ATTN_ERR_SHAPE"), (dict(N=-1), "ATTN_ERR_SHAPE"), (dict(Hkv=0), "ATTN_ERR_SHAPE"),
    (dict(Hq=6, Hkv=4), "ATTN_ERR_GQA"), (dict(d=96), "ATTN_ERR_HEAD_DIM"), (dict(d=256), "ATTN_ERR_HEAD_DIM"),
    (dict(dtype=7), "ATTN_ERR_DTYPE"), (dict(layout=3), "ATTN_ERR_LAYOUT"),
    (dict(scale=float("nan")), "ATTN_ERR_SHAPE"), (dict(scale=float("inf")), "ATTN_ERR_SHAPE"),
    (dict(q=A + 2), "ATTN_ERR_ALIGN"), (dict(v=A + 8), "ATTN_ERR_ALIGN"), (dict(lse=A + 1), "ATTN_ERR_ALIGN"),
    (dict(B=1 << 20, N=1 << 20, Hq=64, Hkv=8), "ATTN_ERR_SHAPE"),
    (dict(var=var(window=-1)), "ATTN_ERR_SHAPE"), (dict(var=var(n_sink=4)), "ATTN_ERR_SHAPE"),
    (dict(var=var(window=8), causal=0), "ATTN_ERR_SHAPE"), (dict(var=var(window=8), dtype=0), "ATTN_ERR_DTYPE"),
    (dict(var=var(sinks=A + 2)), "ATTN_ERR_ALIGN"),
])
def test_prefill_rejects(L, kw, err):
    assert prefill(L, **kw) == ERR[err]


def test_prefill_plain_entry_validates(L):
    assert L.attn_prefill(A, A, A, A, 1, 8, 4, 3, 64, 0.125, 1, None) == ERR["ATTN_ERR_GQA"]
    assert L.attn_prefill(A, None, A, A, 1, 8, 4, 2, 64, 0.125, 1, None) == ERR["ATTN_ERR_NULL"]


def decode(L, **kw):
    a = dict(q=A, k=A, v=A, table=A, lens=A, o=A, B=2, Hq=8, Hkv=2, d=128, page_size=16, mpps=4,
             num_pages=8, scale=0.1, splits=0, dtype=1, ws=A, ws_bytes=1 << 30, var=None)
    a.update(kw)
    args = (a["q"], a["k"], a["v"], a["table"], a["lens"], a["o"], a["B"], a["Hq"], a["Hkv"],
            a["d"], a["page_size"], a["mpps"], a["num_pages"], a["scale"], a["splits"], a["dtype"])
    if a["var"] is None:
        return L.attn_decode(*args, a["ws"], a["ws_bytes"], None)
    return L.attn_decode_ex(*args, a["var"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,err", [
    (dict(q=None), "ATTN_ERR_NULL"), (dict(table=None), "ATTN_ERR_NULL"), (dict(lens=None), "ATTN_ERR_NULL"),
    (dict(B=0), "ATTN_ERR_SHAPE"), (dict(mpps=0), "ATTN_ERR_SHAPE"), (dict(num_pages=0), "ATTN_ERR_SHAPE"),
    (dict(splits=-1), "ATTN_ERR_SHAPE"), (dict(Hq=8, Hkv=3), "ATTN_ERR_GQA"), (dict(d=32), "ATTN_ERR_HEAD_DIM"),
    (dict(page_size=8), "ATTN_ERR_PAGE"), (dict(scale=float("nan")), "ATTN_ERR_SHAPE"),
    # the workspace is needed for every split count: NULL is ERR_NULL, too small ERR_WORKSPACE
    (dict(ws=None), "ATTN_ERR_NULL"), (dict(ws=None, splits=1), "ATTN_ERR_NULL"),
    (dict(ws_bytes=16), "ATTN_ERR_WORKSPACE"),
    # bf16 is the one element type of the decode
    (dict(dtype=0), "ATTN_ERR_DTYPE"), (dict(dtype=2), "ATTN_ERR_DTYPE"),
    (dict(dtype=0, var=var(window=5)), "ATTN_ERR_DTYPE"),
    (dict(k=A + 4), "ATTN_ERR_ALIGN"), (dict(table=A + 2), "ATTN_ERR_ALIGN"),
    (dict(mpps=1 << 28), "ATTN_ERR_SHAPE"),
    (dict(var=var(window=-3)), "ATTN_ERR_SHAPE"), (dict(var=var(n_sink=2)), "ATTN_ERR_SHAPE"),
    (dict(var=var(window=5, n_sink=-1)), "ATTN_ERR_SHAPE"), (dict(var=var(sinks=A + 1)), "ATTN_ERR_ALIGN"),
    (dict(q=None, var=var(window=5)), "ATTN_ERR_NULL"),
])
def test_decode_rejects(L, kw, err):
    assert decode(L, **kw) == ERR[err]


def test_decode_accepts_bf16(L):
    # ATTN_BF16 passes the dtype check: the call goes on to fail a later one
    # (no kernel is launched in these host tests)
    assert decode(L, dtype=1, ws_bytes=16) == ERR["ATTN_ERR_WORKSPACE"]
    assert decode(L, dtype=1, var=var(window=5), k=A + 4) == ERR["ATTN_ERR_ALIGN"]


def noalloc(L, **kw):
    a = dict(q=A, k=A, v=A, table=A, lens=A, o=A, B=2, Hq=8, Hkv=2, d=128, page_size=16, mpps=4,
             num_pages=8, scale=0.1, splits=0, dtype=1)
    a.update(kw)
    return L.attn_decode_noalloc(a["q"], a["k"], a["v"], a["table"], a["lens"], a["o"], a["B"], a["Hq"],
                                 a["Hkv"], a["d"], a["page_size"], a["mpps"], a["num_pages"], a["scale"],
                                 a["splits"], a["dtype"], None)


@pytest.mark.parametrize("kw,err", [
    (dict(q=None), "ATTN_ERR_NULL"), (dict(o=None), "ATTN_ERR_NULL"), (dict(dtype=0), "ATTN_ERR_DTYPE"),
    (dict(B=0), "ATTN_ERR_SHAPE"), (dict(Hq=8, Hkv=3), "ATTN_ERR_GQA"), (dict(d=32), "ATTN_ERR_HEAD_DIM"),
    (dict(page_size=8), "ATTN_ERR_PAGE"), (dict(k=A + 4), "ATTN_ERR_ALIGN"),
    # 64 * 64 * 100 splits * 130 floats is 213 MB, past the 16 MiB scratch
    (dict(B=64, Hq=64, Hkv=8, mpps=1000, splits=100), "ATTN_ERR_SCRATCH"),
])
def test_decode_noalloc_rejects(L, kw, err):
    # every refusal happens on the host, before the scratch address is taken
    assert noalloc(L, **kw) == ERR[err]


def test_noalloc_scratch_limit_matches_the_workspace_rule(L):
    limit = 16 << 20
    assert binding.ATTN_NOALLOC_SCRATCH_BYTES == limit
    # the benchmark's long-context and batched decode shapes fit
    assert L.attn_decode_workspace_size(4, 64, 8, 128, 8192, 0) <= limit
    assert L.attn_decode_workspace_size(64, 32, 8, 128, 512, 0) <= limit
    # the first split count past the limit is refused; the largest one that
    # fits passes the size check and fails the alignment check after it
    B, Hq, Hkv, d, mpps = 8, 64, 8, 128, 4096
    per_split = B * Hq * (d + 2) * 4
    s_max = limit // per_split
    assert noalloc(L, B=B, Hq=Hq, Hkv=Hkv, d=d, mpps=mpps, splits=s_max + 1) == ERR["ATTN_ERR_SCRATCH"]
    assert noalloc(L, B=B, Hq=Hq, Hkv=Hkv, d=d, mpps=mpps, splits=s_max, k=A + 4) == ERR["ATTN_ERR_ALIGN"]


def test_split_count_and_workspace_size(L):
    # explicit counts are clamped to the page count; 0 picks a device-independent value
    assert L.attn_decode_num_splits(4, 8, 100, 7) == 7
    assert L.attn_decode_num_splits(4, 8, 5, 7) == 5
    auto = L.attn_decode_num_splits(4, 8, 8192, 0)
    assert 1 <= auto <= 8192 // 16
    assert L.attn_decode_num_splits(64, 8, 512, 0) >= 1
    assert L.attn_decode_num_splits(0, 8, 512, 0) == ERR["ATTN_ERR_SHAPE"]
    assert L.attn_decode_workspace_size(4, 64, 8, 128, 8192, 0) == 4 * 64 * auto * 130 * 4
    assert L.attn_decode_workspace_size(4, 64, 8, 128, 8192, 3) == 4 * 64 * 3 * 130 * 4
    assert L.attn_decode_workspace_size(4, 64, 7, 128, 8192, 3) == 0
    assert L.attn_decode_workspace_size(4, 64, 8, 96, 8192, 3) == 0


def test_gather_rejects(L):
    g = L.attn_gather_pages
    assert g(None, A, A, A, 1, 2, 64, 16, 4, 8, 10, 2, None) == ERR["ATTN_ERR_NULL"]
    assert g(A, A, A, A, 1, 2, 64, 8, 4, 8, 10, 2, None) == ERR["ATTN_ERR_PAGE"]
    assert g(A, A, A, A, 1, 2, 64, 16, 4, 8, 10, 3, None) == ERR["ATTN_ERR_DTYPE"]
    assert g(A, A, A, A, 0, 2, 64, 16, 4, 8, 10, 2, None) == ERR["ATTN_ERR_SHAPE"]
    assert g(A + 4, A, A, A, 1, 2, 64, 16, 4, 8, 10, 2, None) == ERR["ATTN_ERR_ALIGN"]


def append(L, **kw):
    a = dict(kn=A, vn=A, kp=A, vp=A, table=A, cu=A, start=A, B=2, Hkv=2, d=64, page_size=16, mpps=4,
             num_pages=8, total=10, max_new=5)
    a.update(kw)
    return L.attn_kv_append(a["kn"], a["vn"], a["kp"], a["vp"], a["table"], a["cu"], a["start"], a["B"],
                            a["Hkv"], a["d"], a["page_size"], a["mpps"], a["num_pages"], a["total"],
                            a["max_new"], None)


@pytest.mark.parametrize("kw,err", [
    (dict(kn=None), "ATTN_ERR_NULL"), (dict(cu=None), "ATTN_ERR_NULL"), (dict(start=None), "ATTN_ERR_NULL"),
    (dict(B=0), "ATTN_ERR_SHAPE"), (dict(B=70000), "ATTN_ERR_SHAPE"), (dict(total=-1), "ATTN_ERR_SHAPE"),
    (dict(max_new=-1), "ATTN_ERR_SHAPE"), (dict(d=96), "ATTN_ERR_HEAD_DIM"), (dict(page_size=32), "ATTN_ERR_PAGE"),
    (dict(kp=A + 8), "ATTN_ERR_ALIGN"), (dict(cu=A + 2), "ATTN_ERR_ALIGN"),
])
def test_kv_append_rejects(L, kw, err):
    assert append(L, **kw) == ERR[err]


def test_kv_append_with_nothing_to_write_is_a_no_op(L):
    # returns before any launch, so host pointers are fine here
    assert append(L, total=0) == 0
    assert append(L, max_new=0) == 0


def paged(L, **kw):
    a = dict(q=A, kp=A, vp=A, table=A, cu=A, lens=A, o=A, lse=None, B=2, Hq=8, Hkv=2, d=128,
             page_size=16, mpps=4, num_pages=8, total=10, max_q=5, scale=0.1)
    a.update(kw)
    return L.attn_prefill_paged(a["q"], a["kp"], a["vp"], a["table"], a["cu"], a["lens"], a["o"], a["lse"],
                                a["B"], a["Hq"], a["Hkv"], a["d"], a["page_size"], a["mpps"],
                                a["num_pages"], a["total"], a["max_q"], a["scale"], a.get("var"), None)


@pytest.mark.parametrize("kw,err", [
    (dict(q=None), "ATTN_ERR_NULL"), (dict(cu=None), "ATTN_ERR_NULL"), (dict(lens=None), "ATTN_ERR_NULL"),
    (dict(B=0), "ATTN_ERR_SHAPE"), (dict(mpps=0), "ATTN_ERR_SHAPE"), (dict(total=-2), "ATTN_ERR_SHAPE"),
    (dict(Hq=6, Hkv=4), "ATTN_ERR_GQA"), (dict(d=32), "ATTN_ERR_HEAD_DIM"), (dict(page_size=8), "ATTN_ERR_PAGE"),
    (dict(scale=float("inf")), "ATTN_ERR_SHAPE"), (dict(o=A + 4), "ATTN_ERR_ALIGN"),
    (dict(lse=A + 2), "ATTN_ERR_ALIGN"), (dict(lens=A + 1), "ATTN_ERR_ALIGN"),
    (dict(var=var(n_sink=1)), "ATTN_ERR_SHAPE"), (dict(var=var(window=-2)), "ATTN_ERR_SHAPE"),
])
def test_prefill_paged_rejects(L, kw, err):
    assert paged(L, **kw) == ERR[err]


def test_prefill_paged_with_no_rows_is_a_no_op(L):
    assert paged(L, total=0) == 0
    assert paged(L, max_q=0) == 0


def backward(L, **kw):
    a = dict(q=A, k=A, v=A, o=A, do=A, lse=A, dq=A, dk=A, dv=A, B=1, N=8, Hq=4, Hkv=2, d=64, scale=0.125,
             causal=1, layout=0, ws=A, ws_bytes=1 << 20)
    a.update(kw)
    return L.attn_backward(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"],
                           a["N"], a["Hq"], a["Hkv"], a["d"], a["scale"], a["causal"], a["layout"], a["ws"],
                           a["ws_bytes"], None)


@pytest.mark.parametrize("kw,err", [
    (dict(do=None), "ATTN_ERR_NULL"), (dict(lse=None), "ATTN_ERR_NULL"), (dict(dv=None), "ATTN_ERR_NULL"),
    (dict(B=0), "ATTN_ERR_SHAPE"), (dict(N=0), "ATTN_ERR_SHAPE"), (dict(Hq=4, Hkv=3), "ATTN_ERR_GQA"),
    (dict(d=80), "ATTN_ERR_HEAD_DIM"), (dict(layout=5), "ATTN_ERR_LAYOUT"), (dict(scale=float("nan")), "ATTN_ERR_SHAPE"),
    (dict(ws=None), "ATTN_ERR_NULL"), (dict(ws_bytes=8), "ATTN_ERR_WORKSPACE"), (dict(dk=A + 8), "ATTN_ERR_ALIGN"),
    (dict(lse=A + 2), "ATTN_ERR_ALIGN"),
])
def test_backward_rejects(L, kw, err):
    assert backward(L, **kw) == ERR[err]


def test_backward_workspace_size(L):
    assert L.attn_backward_workspace_size(2, 100, 8) == 2 * 2 * 8 * 128 * 4
    assert L.attn_backward_workspace_size(1, 64, 1) == 2 * 64 * 4
    assert L.attn_backward_workspace_size(0, 64, 1) == 0


def mla(L, **kw):
    a = dict(q=A, kv=A, table=A, lens=A, o=A, B=2, Hq=32, d_c=512, d_r=64, page_size=16, mpps=8, num_pages=16,
             scale=0.07, splits=0, ws=A, ws_bytes=1 << 30)
    a.update(kw)
    return L.attn_decode_mla(a["q"], a["kv"], a["table"], a["lens"], a["o"], a["B"], a["Hq"], a["d_c"], a["d_r"],
                             a["page_size"], a["mpps"], a["num_pages"], a["scale"], a["splits"], a["ws"],
                             a["ws_bytes"], None)


@pytest.mark.parametrize("kw,err", [
    (dict(kv=None), "ATTN_ERR_NULL"), (dict(table=None), "ATTN_ERR_NULL"), (dict(B=0), "ATTN_ERR_SHAPE"),
    (dict(ws=None), "ATTN_ERR_NULL"), (dict(Hq=24), "ATTN_ERR_SHAPE"), (dict(d_c=256), "ATTN_ERR_HEAD_DIM"), (dict(d_r=32), "ATTN_ERR_HEAD_DIM"),
    (dict(page_size=64), "ATTN_ERR_PAGE"), (dict(scale=float("inf")), "ATTN_ERR_SHAPE"),
    (dict(ws_bytes=100), "ATTN_ERR_WORKSPACE"), (dict(o=A + 2), "ATTN_ERR_ALIGN"), (dict(splits=-1), "ATTN_ERR_SHAPE"),
])
def test_decode_mla_rejects(L, kw, err):
    assert mla(L, **kw) == ERR[err]


def test_decode_mla_sizes(L):
    assert L.attn_decode_mla_num_splits(4, 128, 100, 7) == 7
    assert L.attn_decode_mla_num_splits(4, 128, 5, 7) == 5
    auto = L.attn_decode_mla_num_splits(16, 128, 1024, 0)
    assert auto == 16  # one round of 256 work-groups (16 sequences x 16 splits)
    assert L.attn_decode_mla_num_splits(1, 128, 1024, 0) == 1024 // 48  # at least 48 pages per split
    assert L.attn_decode_mla_workspace_size(16, 128, 1024, 0) == 16 * 128 * auto * 514 * 4
    assert L.attn_decode_mla_workspace_size(16, 120, 1024, 0) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.attn_prefill(x, x, x, o=torch.empty_like(x))
