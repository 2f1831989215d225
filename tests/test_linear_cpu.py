"""Host-side checks of the Float8BlockwiseLinear wrapper and the gated FFN
module (no GPU needed): argument validation happens before any kernel call,
with clear messages."""

import pytest
import torch

import blockwise_scaled_fp8_bs_amd as bs
from blockwise_scaled_fp8_bs_amd import Float8BlockwiseLinear, float8_blockwise_linear, swap_linear_layers


def test_rejects_dims_that_are_not_multiples_of_128():
    w = torch.zeros((256, 384), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="tokens M = 100"):
        float8_blockwise_linear(torch.zeros((100, 384), dtype=torch.bfloat16), w)
    with pytest.raises(ValueError, match="in_features K = 200"):
        float8_blockwise_linear(torch.zeros((128, 200), dtype=torch.bfloat16), torch.zeros((256, 200), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out_features N = 100"):
        Float8BlockwiseLinear(128, 100)


def test_rejects_wrong_dtype_layout_and_device():
    w = torch.zeros((256, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="bfloat16"):
        float8_blockwise_linear(torch.zeros((128, 128), dtype=torch.float32), w)
    with pytest.raises(ValueError, match="contiguous"):
        float8_blockwise_linear(torch.zeros((128, 256), dtype=torch.bfloat16)[:, :128], w)
    with pytest.raises(ValueError, match="features"):
        float8_blockwise_linear(torch.zeros((128, 256), dtype=torch.bfloat16), w)
    with pytest.raises(ValueError, match="GPU"):
        float8_blockwise_linear(torch.zeros((2, 64, 128), dtype=torch.bfloat16), w)


def test_swap_replaces_bias_free_linears_only():
    m = torch.nn.Sequential(torch.nn.Linear(128, 256, bias=False), torch.nn.ReLU(),
                            torch.nn.Sequential(torch.nn.Linear(256, 128, bias=False)),
                            torch.nn.Linear(128, 128, bias=True))
    ref = [m[0].weight.detach().clone(), m[2][0].weight.detach().clone()]
    swap_linear_layers(m)
    assert isinstance(m[0], Float8BlockwiseLinear) and isinstance(m[2][0], Float8BlockwiseLinear)
    assert isinstance(m[3], torch.nn.Linear)
    assert torch.equal(m[0].weight, ref[0].to(torch.bfloat16)) and torch.equal(m[2][0].weight, ref[1].to(torch.bfloat16))
    with pytest.raises(ValueError, match="bias"):
        Float8BlockwiseLinear.from_linear(torch.nn.Linear(128, 128))


# ---- the gated FFN module: argument checks (no GPU needed) ----

def _ffn_args(M=256, D=256, H=512, dtype=torch.bfloat16):
    x = torch.zeros((M, D), dtype=dtype)
    return x, torch.zeros((H, D), dtype=dtype), torch.zeros((H, D), dtype=dtype), torch.zeros((D, H), dtype=dtype)


def test_gated_ffn_rejects_bad_arguments():
    x, w1, w2, wo = _ffn_args()
    with pytest.raises(ValueError, match="bfloat16"):
        bs.float8_blockwise_gated_ffn(x.float(), w1, w2, wo)
    with pytest.raises(ValueError, match="contiguous"):
        bs.float8_blockwise_gated_ffn(x.t(), w1, w2, wo)
    with pytest.raises(ValueError, match="w1 and w2"):
        bs.float8_blockwise_gated_ffn(x, w1, w2[:384], wo)
    with pytest.raises(ValueError, match="out_proj must be"):
        bs.float8_blockwise_gated_ffn(x, w1, w2, wo[:, :384].contiguous())
    with pytest.raises(ValueError, match="features"):
        bs.float8_blockwise_gated_ffn(torch.zeros((256, 384), dtype=torch.bfloat16), w1, w2, wo)
    x6, a6, b6, o6 = _ffn_args(H=640)
    with pytest.raises(ValueError, match="multiple of 512"):
        bs.float8_blockwise_gated_ffn(x6, a6, b6, o6)
    x1, a1, b1, o1 = _ffn_args(M=200)
    with pytest.raises(ValueError, match="multiple of 128"):
        bs.float8_blockwise_gated_ffn(x1, a1, b1, o1)
    with pytest.raises(ValueError, match="GPU"):
        bs.float8_blockwise_gated_ffn(x, w1, w2, wo)


def test_gated_ffn_module_shapes_and_conversion():
    with pytest.raises(ValueError, match="multiple of 512"):
        bs.Float8BlockwiseGatedFFN(256, 640)
    lin = [torch.nn.Linear(256, 512, bias=False), torch.nn.Linear(256, 512, bias=False),
           torch.nn.Linear(512, 256, bias=False)]
    m = bs.Float8BlockwiseGatedFFN.from_linears(*lin)
    assert (m.dim, m.hidden) == (256, 512)
    assert m.w1.dtype == torch.bfloat16 and tuple(m.out_proj.shape) == (256, 512)
    assert torch.equal(m.w2, lin[1].weight.detach().to(torch.bfloat16))
    with pytest.raises(ValueError, match="biases"):
        bs.Float8BlockwiseGatedFFN.from_linears(torch.nn.Linear(256, 512), lin[1], lin[2])


# ---- the MXFP8 layers: argument checks (no GPU needed) ----

def test_mx_linear_rejects_bad_arguments():
    w = torch.zeros((256, 384), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="tokens = 100"):
        bs.float8_mx_linear(torch.zeros((100, 384), dtype=torch.bfloat16), w)
    with pytest.raises(ValueError, match="out_features = 96"):
        bs.float8_mx_linear(torch.zeros((128, 384), dtype=torch.bfloat16), torch.zeros((96, 384), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="bfloat16"):
        bs.float8_mx_linear(torch.zeros((128, 384)), w)
    with pytest.raises(ValueError, match="contiguous"):
        bs.float8_mx_linear(torch.zeros((128, 768), dtype=torch.bfloat16)[:, :384], w)
    with pytest.raises(ValueError, match="features"):
        bs.float8_mx_linear(torch.zeros((128, 256), dtype=torch.bfloat16), w)
    with pytest.raises(ValueError, match="GPU"):
        bs.float8_mx_linear(torch.zeros((128, 384), dtype=torch.bfloat16), w)
    with pytest.raises(ValueError, match="in_features = 200"):
        bs.Float8MXLinear(200, 128)
    with pytest.raises(ValueError, match="bias"):
        bs.Float8MXLinear.from_linear(torch.nn.Linear(128, 128))


def test_mx_grouped_mm_rejects_bad_arguments():
    x = torch.zeros((512, 256), dtype=torch.bfloat16)
    w = torch.zeros((4, 384, 256), dtype=torch.bfloat16)
    ends = torch.tensor([128, 256, 384, 512], dtype=torch.int32)
    with pytest.raises(ValueError, match="3-D"):
        bs.mx_grouped_mm(x, w[0], ends)
    with pytest.raises(ValueError, match=r"x must be \[M, 256\]"):
        bs.mx_grouped_mm(torch.zeros((512, 128), dtype=torch.bfloat16), w, ends)
    with pytest.raises(ValueError, match="group_end"):
        bs.mx_grouped_mm(x, w, ends.long())
    with pytest.raises(ValueError, match="group_end"):
        bs.mx_grouped_mm(x, w, ends[:3])
    with pytest.raises(ValueError, match="tokens = 500"):
        bs.mx_grouped_mm(torch.zeros((500, 256), dtype=torch.bfloat16), w, ends)
    with pytest.raises(ValueError, match="GPU"):
        bs.mx_grouped_mm(x, w, ends)


def test_mx_linear_module_conversion():
    lin = torch.nn.Linear(256, 128, bias=False)
    m = bs.Float8MXLinear.from_linear(lin)
    assert m.weight.dtype == torch.bfloat16 and tuple(m.weight.shape) == (128, 256)
    assert torch.equal(m.weight, lin.weight.detach().to(torch.bfloat16))
    assert "mxfp8" in repr(m)
