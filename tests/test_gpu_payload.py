"""GPU parity of the expert-parallel payloads (MXFP4 dispatch, FP8-blockwise
combine) against the oracle: payload bytes bit-exact, unpacked rows
bit-exact (bf16), at hidden sizes of the layers here, with zero blocks,
subnormal-range blocks, huge values and mixed magnitudes."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_cases import say

pytestmark = pytest.mark.gpu

mlr = pytest.importorskip("moe_layer_router_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mlr.lib()


def _rows(T, D, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((T, D), generator=g) * torch.exp2(torch.randint(-20, 20, (T, 1), generator=g).float())
    if T > 3:
        x[0, :64] = 0.0                                   # zero blocks
        x[1, 32:160] = torch.randn(128, generator=g) * 1e-39   # subnormal range
        x[2, :32] = 3.0e38                                # near the bf16 maximum
        x[3, ::7] = -x[3, ::7] * 1000.0                   # mixed magnitudes inside blocks
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8_block"])
@pytest.mark.parametrize("T,D", [(1, 128), (37, 4096), (300, 7168), (5, 16384), (0, 4096)])
def test_payload_matches_oracle(fmt, T, D):
    say("payload", fmt, T, D)
    x = _rows(T, D, 100 + T + D)
    xg = x.cuda()
    p = mlr.ep_pack(xg, fmt)
    y = mlr.ep_unpack(p, D, fmt)
    torch.cuda.synchronize()
    assert p.shape == (T, mlr.ep_payload_bytes(D, fmt))
    if T == 0:
        return
    xf = synth.bf16_to_f32_np(x)
    if fmt == "mxfp4":
        ref_p = O.mxfp4_payload(xf.astype(np.float64))
        ref_y = O.bf16_round(O.mxfp4_unpack(ref_p, D).astype(np.float32))
    else:
        ref_p = O.fp8_block_payload(xf)
        ref_y = O.fp8_block_unpack(ref_p, D)
    assert np.array_equal(p.cpu().numpy(), ref_p)
    got = y.view(torch.int16).cpu().numpy()
    want = O.bf16_bits(ref_y).astype(np.int16)
    assert np.array_equal(got, want)


def test_payload_round_trip_bytes_at_the_page_shape():
    """Hidden 7168 (the DeepSeek-R1 layer): 3808 + 7392 bytes per token, the
    page's 11,200-byte quantized round trip against 28,672 in bf16."""
    D = 7168
    assert mlr.ep_payload_bytes(D, "mxfp4") + mlr.ep_payload_bytes(D, "fp8_block") == 11200
    x = _rows(64, D, 7).cuda()
    p4, p8 = mlr.ep_pack(x, "mxfp4"), mlr.ep_pack(x, "fp8_block")
    assert p4.numel() + p8.numel() == 64 * 11200 and 2 * 2 * x.numel() == 64 * 28672


def test_mxfp4_codes_on_every_bf16_value():
    """Every bf16 value of magnitude up to 4 as an element of a block whose
    amax is 4 (scale 2^0, so the element is encoded as is), and every bf16
    value in (4, 8) in blocks of amax 7.5 (the saturating range): codes and
    scales bit-exact against the oracle's E2M1 encoder."""
    bits = np.arange(0, 1 << 15, dtype=np.uint32)                      # non-negative bf16 patterns
    vals = (bits << 16).view(np.float32)
    small = vals[np.isfinite(vals) & (vals <= 4.0)]
    mid = vals[np.isfinite(vals) & (vals > 4.0) & (vals < 8.0)]
    def blocks(v, head):
        v = np.concatenate([v, -v])
        n = -(-len(v) // 31) * 31
        v = np.concatenate([v, np.zeros(n - len(v), np.float32)]).reshape(-1, 31)
        return np.concatenate([np.full((len(v), 1), head, np.float32), v], axis=1)
    b = np.concatenate([blocks(small, 4.0), blocks(mid, 7.5)])
    D = 4096
    n = -(-b.size // D) * D
    x = np.concatenate([b.reshape(-1), np.zeros(n - b.size, np.float32)]).reshape(-1, D)
    say("mxfp4 every bf16 value", x.shape)
    p = mlr.ep_pack(torch.from_numpy(x).to(torch.bfloat16).cuda(), "mxfp4")
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), O.mxfp4_payload(x.astype(np.float64)))
