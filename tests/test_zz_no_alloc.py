"""The decode call that allocates nothing (pkv_paged_attention_decode_noalloc)
against the balanced decode + reduce with a caller's workspace: two calls in
a row, the second with a smaller batch, each equal to the existing entry
points bit for bit and within the tolerance of the oracle.  Also the
rejection of a call that needs more than the fixed array."""
import numpy as np
import pytest
import torch

import paged_kv_cache_361_amd as pkv
import workloads
from gpu_case import DevCase, assert_within, bound, from_dev, oracle_run

pytestmark = pytest.mark.gpu

BAL = pkv.PARTITION_BALANCED


def _noalloc(d: DevCase):
    c = d.c
    d.out.fill_(float("nan"))
    pkv.paged_attention_decode_noalloc(d.out, d.query, d.k_cache, d.v_cache, d.tables, d.lens,
                                       scale=c.scale, max_seq_len=c.max_seq_len,
                                       k_scale=c.k_scale, v_scale=c.v_scale)
    torch.cuda.synchronize()
    return d.out.clone()


def _with_workspace(d: DevCase):
    d.out.fill_(float("nan"))
    d.decode("mfma", BAL)
    torch.cuda.synchronize()
    return d.out.clone()


def _case(name, seed, S, dtype="bf16", cache=None, G=4, bs=16):
    return workloads.make_case(name, seed, lambda r: workloads.llama3_8b_gqa_lens(r, S),
                               8 * G, 8, 128, bs, q_dtype=dtype, cache_dtype=cache or dtype,
                               src_dtype=dtype if cache == "fp8" else None, max_seq_len=4096,
                               append_last=cache != "fp8")


@pytest.mark.parametrize("dtype,cache,G,bs", [("bf16", None, 4, 16), ("f16", "fp8", 8, 32)])
def test_noalloc_equals_workspace_call_twice_shrinking(dtype, cache, G, bs):
    big = _case("noalloc-big", 201, 96, dtype, cache, G, bs)
    small = _case("noalloc-small", 202, 9, dtype, cache, G, bs)
    for c in (big, small):                     # the second call is the smaller one
        d = DevCase(c)
        d.write()
        got = _noalloc(d)
        ref_dev = _with_workspace(d)
        assert torch.equal(got.view(torch.uint8), ref_dev.view(torch.uint8)), c.name
        out = from_dev(got)
        assert_within(out, oracle_run(c), bound(oracle_run(c), c.cache_dtype, c.q_dtype))


def test_noalloc_rejects_a_call_beyond_the_array():
    """16 query heads per KV head at head_dim 128 need about 85 MB of partials
    on a grid of one wave per SIMD: more than the 64 MiB array."""
    c = workloads.make_case("noalloc-too-big", 203, [40, 70], 32, 2, 128, 16,
                            q_dtype="bf16", cache_dtype="bf16")
    d = DevCase(c)
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_attention_decode_noalloc(d.out, d.query, d.k_cache, d.v_cache, d.tables,
                                           d.lens, scale=c.scale, max_seq_len=c.max_seq_len)
    assert e.value.status == -9
