"""The torch helpers of the binding reject caller-given tensors that the
kernels would index out of bounds (wrong shape, dtype, layout or device)
before anything is enqueued, and accept the right ones."""
import pytest
import torch

import io_aware_tiled_02_amd as fa

pytestmark = pytest.mark.gpu


def _qkv(B=1, H=2, L=70, d=64, dtype=torch.bfloat16):
    g = torch.Generator(device="cpu").manual_seed(5)
    return [torch.randn(B, H, L, d, generator=g).to(dtype).to("cuda") for _ in range(3)]


def test_forward_rejects_bad_outputs():
    print("[binding] forward: bad out / lse", flush=True)
    q, k, v = _qkv()
    B, H, L, d = q.shape
    bad_out = [torch.empty(B, H, L - 1, d, dtype=q.dtype, device="cuda"),
               torch.empty(B, H, L, d, dtype=torch.float16, device="cuda"),
               torch.empty(B, H, d, L, dtype=q.dtype, device="cuda").transpose(2, 3),
               torch.empty(B, H, L, d, dtype=q.dtype)]
    for out in bad_out:
        with pytest.raises(ValueError):
            fa.forward(q, k, v, 0.125, out=out)
    bad_lse = [torch.empty(B, H, L - 1, device="cuda"), torch.empty(B, H, L, dtype=torch.float64, device="cuda"),
               torch.empty(B, H, L)]
    for lse in bad_lse:
        with pytest.raises(ValueError):
            fa.forward(q, k, v, 0.125, lse=lse)
    out = torch.empty_like(q)
    lse = torch.empty(B, H, L, device="cuda")
    o2, l2 = fa.forward(q, k, v, 0.125, out=out, lse=lse)
    torch.cuda.synchronize()
    assert o2 is out and l2 is lse and torch.isfinite(lse).all()


def test_backward_and_splitkv_reject_bad_tensors():
    print("[binding] backward / split-K/V: bad lse, out, workspace", flush=True)
    q, k, v = _qkv()
    B, H, L, d = q.shape
    o, lse = fa.forward(q, k, v, 0.125)
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, lse[:, :, :-1].contiguous(), torch.randn_like(q), 0.125)
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, lse.double(), torch.randn_like(q), 0.125)
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, lse, torch.randn(B, H, L, d, device="cuda"), 0.125)   # dout float32
    qd = q[:, :, :1].contiguous()
    with pytest.raises(ValueError):
        fa.forward_splitkv(qd, k, v, 0.125, out=torch.empty(B, H, 2, d, dtype=q.dtype, device="cuda"))
    with pytest.raises(ValueError):
        fa.forward_splitkv(qd, k, v, 0.125, lse=torch.empty(B, H, 1, dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        fa.forward_splitkv(qd, k, v, 0.125, workspace=torch.empty(1 << 16, dtype=torch.uint8))


def test_fp8_helpers_reject_bad_tensors():
    print("[binding] quantize_fp8 / forward_fp8: bad codes, scales, out", flush=True)
    q, k, v = _qkv(d=128)
    B, H, L, d = q.shape
    with pytest.raises(ValueError):
        fa.quantize_fp8(q, 32, x8=torch.empty(B, H, L, d, dtype=torch.int8, device="cuda"))
    with pytest.raises(ValueError):
        fa.quantize_fp8(q, 32, scales=torch.empty(B * H, 2, device="cuda"))          # needs ceil(70/32) = 3
    with pytest.raises(ValueError):
        fa.quantize_fp8(q, 0)
    q8, sq = fa.quantize_fp8(q, 32)
    k8, sk = fa.quantize_fp8(k, 32)
    with pytest.raises(ValueError):
        fa.forward_fp8(q8, k8, sq.double(), sk, v, 0.1, False, 32, 32)
    with pytest.raises(ValueError):
        fa.forward_fp8(q8, k8, sq, sk, v, 0.1, False, 32, 32, out=torch.empty(B, H, L, d, device="cuda"))
    with pytest.raises(ValueError):
        fa.forward_fp8(q8, k8, sq, sk, v, 0.1, False, 32, 32, lse=torch.empty(B, H, L + 1, device="cuda"))
    o, lse = fa.forward_fp8(q8, k8, sq, sk, v, 0.1, False, 32, 32)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
