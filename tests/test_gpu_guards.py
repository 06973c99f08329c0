"""The GQA_CHECK_SEQLENS debug check of the device-side lengths (needs an MI355X).

With GQA_CHECK_SEQLENS=1 a decode call copies seqlens (and the block-table
entries a sequence uses) to the host and returns GQA_ERR_SHAPE before any
launch when one is out of range.  Every invalid case here is refused on the
host, so no kernel ever sees an invalid length; the outputs and caches keep
their canaries.  Valid inputs give the same bits with and without the check,
and the check stands aside while a stream is being captured.
"""
import numpy as np
import pytest
import torch

import gqa_inputs as gi
import gqa_kv_cache_amd as gqa
from tests.gpu_util import bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture
def checked(monkeypatch):
    monkeypatch.setenv("GQA_CHECK_SEQLENS", "1")


def _decode_inputs():
    c = gi.decode_case(2, 16, 4, 128, 300, [300, 17], "bf16", q_seed=71, kv_seed=72, invalid="nan")
    return c, to_dev(c.q), to_dev(c.k), to_dev(c.v)


@pytest.mark.parametrize("bad", [[300, 301], [-1, 17], [2 ** 31 - 1, 0]])
@pytest.mark.parametrize("entry", ["decode", "noalloc"])
def test_decode_refuses_out_of_range_lengths(checked, bad, entry):
    c, q, k, v = _decode_inputs()
    sl = torch.tensor(bad, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 5.0)
    with pytest.raises(gqa.GqaError) as e:
        if entry == "decode":
            gqa.decode(q, k, v, sl, c.scale, out=out, num_splits=3)
        else:
            gqa.decode_noalloc(q, k, v, sl, out, c.scale, num_splits=3)
    assert e.value.status == gqa.Status.ERR_SHAPE
    torch.cuda.synchronize()
    assert bool(torch.all(out == 5.0))


def test_valid_lengths_same_bits_with_and_without_check(monkeypatch):
    c, q, k, v = _decode_inputs()
    sl = torch.from_numpy(c.seqlens).cuda()
    monkeypatch.delenv("GQA_CHECK_SEQLENS", raising=False)
    plain = bits(gqa.decode(q, k, v, sl, c.scale, num_splits=3))
    monkeypatch.setenv("GQA_CHECK_SEQLENS", "1")
    checked = bits(gqa.decode(q, k, v, sl, c.scale, num_splits=3))
    out = torch.empty_like(q)
    checked_noalloc = bits(gqa.decode_noalloc(q, k, v, sl, out, c.scale, num_splits=3))
    torch.cuda.synchronize()
    assert np.array_equal(plain, checked) and np.array_equal(plain, checked_noalloc)


def _ex_inputs(paged):
    e = gi.decode_ex_case(2, 2, 16, 4, 128, 256, [256, 40], "bf16", seed=73, paged=paged,
                          block_size=32)
    d = dict(q=to_dev(e.q), k=to_dev(e.k_pre), v=to_dev(e.v_pre), kn=to_dev(e.k_new),
             vn=to_dev(e.v_new))
    return e, d


@pytest.mark.parametrize("case", ["length_below_tokens", "length_above_cache", "block_outside_pool",
                                  "negative_block"])
def test_decode_ex_refuses_bad_lengths_and_blocks(checked, case):
    paged = case.endswith("pool") or case.startswith("negative")
    e, d = _ex_inputs(paged)
    sl = e.seqlens.copy()
    bt = None if e.block_table is None else e.block_table.copy()
    if case == "length_below_tokens":
        sl[1] = 1                       # T = 2 new tokens need at least 2 rows
    elif case == "length_above_cache":
        sl[0] = 257
    elif case == "block_outside_pool":
        bt[1, 1] = e.k.shape[0]         # row 32..63 of sequence 1 (length 40) is used
    else:
        bt[0, 7] = -3
    kw = {}
    if bt is not None:
        kw = dict(block_table=torch.from_numpy(bt).cuda(), block_size=32)
    out = torch.full_like(d["q"], 5.0)
    k_before, v_before = d["k"].clone(), d["v"].clone()
    with pytest.raises(gqa.GqaError) as err:
        gqa.decode_ex(d["q"], d["k"], d["v"], torch.from_numpy(sl).cuda(), scale=e.scale,
                      k_new=d["kn"], v_new=d["vn"], out=out, num_splits=3, **kw)
    assert err.value.status == gqa.Status.ERR_SHAPE
    torch.cuda.synchronize()
    assert bool(torch.all(out == 5.0))
    # nothing was appended
    assert torch.equal(d["k"].view(torch.int16), k_before.view(torch.int16))
    assert torch.equal(d["v"].view(torch.int16), v_before.view(torch.int16))


def test_check_stands_aside_under_graph_capture(checked):
    """A captured call cannot wait for a copy: the check is skipped there,
    the capture succeeds and its replays equal an eager (checked) call."""
    c, q, k, v = _decode_inputs()
    sl = torch.from_numpy(c.seqlens).cuda()
    need = gqa.decode_workspace_size(2, 16, 4, 128, 300, gqa.BF16, 3)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    want = bits(gqa.decode(q, k, v, sl, c.scale, num_splits=3))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gqa.decode(q, k, v, sl, c.scale, out=out, num_splits=3, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gqa.decode(q, k, v, sl, c.scale, out=out, num_splits=3, workspace=ws)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), want)
