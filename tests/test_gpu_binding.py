"""Argument refusals of the Python binding and of the C library (needs an
MI355X for device tensors).  Every case is refused before any launch: the
binding's own checks raise ValueError or TypeError, the library's return a
status that the binding raises as GqaError.  Outputs keep their canaries."""
import pytest
import torch

import gqa_kv_cache_amd as gqa

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _decode_args(B=2, Hq=8, Hkv=2, d=128, L=64, dtype=torch.bfloat16):
    q = torch.randn(B, Hq, d, device=DEV).to(dtype)
    k = torch.randn(B, L, Hkv, d, device=DEV).to(dtype)
    v = torch.randn(B, L, Hkv, d, device=DEV).to(dtype)
    sl = torch.full((B,), L, dtype=torch.int32, device=DEV)
    return q, k, v, sl


def _canary(q):
    return torch.full_like(q, 7.0)


def test_binding_refuses_strided_and_host_tensors():
    q, k, v, sl = _decode_args()
    out = _canary(q)
    with pytest.raises(ValueError, match="contiguous"):
        gqa.decode(q.transpose(0, 1).contiguous().transpose(0, 1), k, v, sl, out=out)
    with pytest.raises(ValueError, match="contiguous"):
        gqa.decode(q, k[:, ::2], v[:, ::2], sl, out=out)
    with pytest.raises(ValueError, match="device tensor"):
        gqa.decode(q, k, v, sl.cpu(), out=out)
    with pytest.raises(ValueError, match="contiguous"):
        gqa.prefill(q.view(2, 1, 8, 128).expand(2, 3, 8, 128), k[:, :3], v[:, :3])
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))


def test_binding_refuses_types_and_shapes():
    q, k, v, sl = _decode_args()
    out = _canary(q)
    with pytest.raises(TypeError, match="int32"):
        gqa.decode(q, k, v, sl.long(), out=out)
    with pytest.raises(TypeError, match="one dtype"):
        gqa.decode(q, k.float(), v.float(), sl, out=out)
    with pytest.raises(ValueError, match="inconsistent"):
        gqa.decode(q, k[:1].contiguous(), v[:1].contiguous(), sl, out=out)
    with pytest.raises(ValueError, match="out must match"):
        gqa.decode(q, k, v, sl, out=torch.empty(2, 8, 64, dtype=q.dtype, device=DEV))
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))


@pytest.mark.parametrize("Hq,Hkv,d,status", [(8, 3, 128, "ERR_GROUP"), (8, 2, 96, "ERR_HEADDIM"),
                                             (130, 2, 128, "ERR_UNSUPPORTED")])
def test_library_refuses_heads(Hq, Hkv, d, status):
    q, k, v, sl = _decode_args(Hq=Hq, Hkv=Hkv, d=d)
    out = _canary(q)
    with pytest.raises(gqa.GqaError) as e:
        gqa.decode(q, k, v, sl, out=out)
    assert e.value.status == getattr(gqa.Status, status)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))


def test_library_refuses_a_short_workspace():
    q, k, v, sl = _decode_args(L=1000)
    need = gqa.decode_workspace_size(2, 8, 2, 128, 1000, gqa.BF16, 4)
    assert need > 0
    out = _canary(q)
    ws = torch.empty(need - 1, dtype=torch.uint8, device=DEV)
    with pytest.raises(gqa.GqaError) as e:
        gqa.decode(q, k, v, sl, out=out, num_splits=4, workspace=ws)
    assert e.value.status == gqa.Status.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))


def test_library_refuses_prefill_arguments():
    q = torch.randn(1, 40, 8, 128, device=DEV).to(torch.bfloat16)
    k = torch.randn(1, 40, 2, 128, device=DEV).to(torch.bfloat16)
    out = _canary(q)
    with pytest.raises(gqa.GqaError) as e:      # a window needs the causal mask
        gqa.prefill(q, k, k.clone(), causal=False, window=8, out=out)
    assert e.value.status == gqa.Status.ERR_UNSUPPORTED
    with pytest.raises(gqa.GqaError) as e:      # prefill computes in bf16 only
        gqa.prefill(q.float(), k.float(), k.float(), out=out.float())
    assert e.value.status == gqa.Status.ERR_DTYPE
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
