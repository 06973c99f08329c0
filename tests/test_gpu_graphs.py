"""The calls inside captured HIP graphs (needs an MI355X).

The library allocates nothing and issues no memset, so a decode step can be
captured once with its buffers and replayed.  Each replay runs after eager
work and a synchronisation and must equal the eager result bit for bit,
also after the inputs are changed in place between replays.
"""
import numpy as np
import pytest
import torch

import gqa_inputs as gi
import gqa_kv_cache_amd as gqa
from tests.gpu_util import bits, to_dev

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_decode_split_and_merge_in_a_graph():
    c = gi.decode_case(4, 32, 8, 128, 1000, [1000, 999, 3, 640], "bf16", q_seed=31, kv_seed=32,
                       invalid="nan")
    q, k, v = to_dev(c.q), to_dev(c.k), to_dev(c.v)
    sl = torch.from_numpy(c.seqlens).cuda()
    need = gqa.decode_workspace_size(4, 32, 8, 128, 1000, gqa.BF16, 3)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    g = _capture(lambda: gqa.decode(q, k, v, sl, c.scale, out=out, num_splits=3, workspace=ws))
    q_other = to_dev(gi.decode_case(4, 32, 8, 128, 1000, [1000, 999, 3, 640], "bf16", q_seed=33,
                                    kv_seed=32).q)
    for i in range(4):
        src = q_other if i % 2 else to_dev(c.q)
        q.copy_(src)
        want = gqa.decode(src, k, v, sl, c.scale, num_splits=3)  # eager, own buffers
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(want)), i


def test_decode_ex_append_fp8_paged_in_a_graph():
    c = gi.decode_ex_case(3, 2, 16, 4, 128, 256, [256, 97, 5], "bf16", seed=34, kv="fp8",
                          paged=True, block_size=16, window=50)
    dev8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = to_dev(c.q)
    k, v = dev8(c.k_pre), dev8(c.v_pre)
    kn, vn = dev8(c.k_new), dev8(c.v_new)
    sl = torch.from_numpy(c.seqlens).cuda()
    kw = dict(scale=c.scale, k_scale=dev8(c.k_scale), v_scale=dev8(c.v_scale),
              block_table=dev8(c.block_table), block_size=16, window=50, k_new=kn, v_new=vn)
    ws = torch.empty(8 << 20, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    g = _capture(lambda: gqa.decode_ex(q, k, v, sl, out=out, num_splits=2, workspace=ws, **kw))
    # eager reference on its own copies of the caches (the append writes them)
    k2, v2 = dev8(c.k_pre), dev8(c.v_pre)
    want = gqa.decode_ex(q, k2, v2, sl, num_splits=2, **kw)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(want)), i
        assert torch.equal(k, k2) and torch.equal(v, v2)


def test_prefill_with_window_in_a_graph():
    c = gi.prefill_case(2, 333, 16, 4, 128, "bf16", seed=35)
    q, k, v = to_dev(c.q), to_dev(c.k), to_dev(c.v)
    out = torch.empty_like(q)
    g = _capture(lambda: gqa.prefill(q, k, v, True, c.scale, out=out, window=100))
    q_other = to_dev(gi.prefill_case(2, 333, 16, 4, 128, "bf16", seed=36).q)
    for i in range(4):
        src = q_other if i % 2 else to_dev(c.q)
        q.copy_(src)
        want = gqa.prefill(src, k, v, True, c.scale, window=100)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(want)), i
