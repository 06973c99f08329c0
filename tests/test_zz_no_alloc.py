"""gqa_decode_noalloc against gqa_decode (needs an MI355X).

The no-allocation entry point keeps its split partials in the library's
static device scratch.  Two calls in a row, the second smaller than the
first, must each equal gqa_decode on the same inputs (the same kernels and
plan, so bit for bit) and stay within the tolerance of the oracle; a plan
whose partials exceed the scratch is refused before any device work.
"""
import numpy as np
import pytest
import torch

import gqa_inputs as gi
import gqa_kv_cache_amd as gqa
from oracle import reference as orc
from tests.gpu_util import bits, from_dev, to_dev
from tests.helpers import bf16_tol_ok, f32_tol_ok

pytestmark = pytest.mark.gpu


def _both(c, num_splits):
    q, k, v = to_dev(c.q), to_dev(c.k), to_dev(c.v)
    sl = torch.from_numpy(c.seqlens).cuda()
    want = gqa.decode(q, k, v, sl, c.scale, num_splits=num_splits)
    out = torch.full_like(q, float("nan"))
    got = gqa.decode_noalloc(q, k, v, sl, out, c.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return want, got


def test_two_calls_second_smaller():
    big = gi.decode_case(4, 32, 8, 128, 1000, [1000, 999, 3, 640], "bf16", q_seed=61, kv_seed=62,
                         invalid="nan", name="noalloc_big")
    small = gi.decode_case(2, 16, 2, 64, 300, [300, 77], "bf16", q_seed=63, kv_seed=64,
                           invalid="nan", name="noalloc_small")
    for c in (big, small):
        B, Hq, d = c.q.shape
        Lmax, Hkv = c.k.shape[1], c.k.shape[2]
        assert gqa.decode_num_splits(B, Hq, Hkv, d, Lmax, gqa.BF16, 0) > 1  # the scratch is used
        want, got = _both(c, 0)
        assert np.array_equal(bits(got), bits(want)), c.name
        ok, err = bf16_tol_ok(from_dev(got), orc.decode(c.q, c.k, c.v, c.seqlens, c.scale))
        assert ok, (c.name, err)


def test_fp32_and_forced_splits():
    c = gi.tiny_decode(2)
    for splits in (3, 5):
        want, got = _both(c, splits)
        assert np.array_equal(bits(got), bits(want))
        ok, err = f32_tol_ok(from_dev(got), orc.decode(c.q, c.k, c.v, c.seqlens, c.scale))
        assert ok, err


def test_plan_above_the_scratch_is_refused():
    """8 x 64 heads x 1024 pieces x (128 + 2) x 4 bytes = 272 MB of partials:
    refused on the host, before any launch; out keeps its contents."""
    c = gi.decode_case(8, 64, 1, 128, 1024, [1024] * 8, "bf16", q_seed=65, kv_seed=66)
    q, k, v = to_dev(c.q), to_dev(c.k), to_dev(c.v)
    sl = torch.from_numpy(c.seqlens).cuda()
    assert gqa.decode_workspace_size(8, 64, 1, 128, 1024, gqa.BF16, 1024) > (16 << 20)
    out = torch.full_like(q, 3.0)
    with pytest.raises(gqa.GqaError) as e:
        gqa.decode_noalloc(q, k, v, sl, out, c.scale, num_splits=1024)
    assert e.value.status == gqa.Status.ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool(torch.all(out == 3.0))
    # the same plan within the limit runs
    want, got = _both(c, 16)
    assert np.array_equal(bits(got), bits(want))


def test_captured_in_a_graph():
    """The callers it is for: capture a split decode through the entry point
    once, then replay it after eager calls (of both entry points, on the
    same stream) and after in-place changes of q; every replay equals an
    eager gqa_decode of the same inputs bit for bit."""
    c = gi.decode_case(4, 32, 8, 128, 1000, [1000, 999, 3, 640], "bf16", q_seed=67, kv_seed=68,
                       invalid="nan")
    q, k, v = to_dev(c.q), to_dev(c.k), to_dev(c.v)
    sl = torch.from_numpy(c.seqlens).cuda()
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gqa.decode_noalloc(q, k, v, sl, out, c.scale, num_splits=3)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gqa.decode_noalloc(q, k, v, sl, out, c.scale, num_splits=3)
    other = to_dev(gi.decode_case(4, 32, 8, 128, 1000, [1000, 999, 3, 640], "bf16", q_seed=69,
                                  kv_seed=68).q)
    for i in range(4):
        src = other if i % 2 else to_dev(c.q)
        q.copy_(src)
        want = bits(gqa.decode(src, k, v, sl, c.scale, num_splits=3))
        scratch_user = torch.empty_like(q)
        gqa.decode_noalloc(other, k, v, sl, scratch_user, c.scale, num_splits=5)  # reuses the scratch
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), want), i
