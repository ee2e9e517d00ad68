"""moe_forward_noalloc (the entry for callers that cannot allocate) against
moe_forward on the same inputs: the same kernels, so y must be bitwise
equal.  Two calls in a row on one layer, the second with fewer tokens (the
scratch array keeps the first call's intermediates), in every arithmetic
mode and both kernel families; sizes beyond the array are refused before
anything runs."""

import ctypes

import pytest
import torch

import synth
from tests.gpu_cases import REDUCED, build_case, say

pytestmark = pytest.mark.gpu

mlr = pytest.importorskip("moe_layer_router_amd")
from moe_layer_router_amd import _lib as L  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mlr.lib()


def _noalloc(layer, x, logits, block_m, y):
    return L.lib().moe_forward_noalloc(ctypes.byref(layer.desc), x.data_ptr(),
                                       None if logits is None else logits.data_ptr(), x.shape[0], block_m,
                                       y.data_ptr(), torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("name,block_m,T2", [("qwen3_235b_decode_ptpc", 0, 7), ("tiny_bf16", 0, 5),
                                             ("deepseek_r1_block_fp8_small", 0, 3),
                                             ("qwen3_235b_prefill_ptpc_r", 0, 101),
                                             ("deepseek_r1_block_fp8_r", 128, 77),
                                             ("e512_top10_shared_r", 16, 9), ("qwen3_235b_decode_mxfp4_r", 0, 7)])
def test_noalloc_equals_moe_forward(name, block_m, T2):
    w = REDUCED[name]
    say("noalloc", name, block_m, T2)
    c = build_case(w)
    need = c.layer.desc and L.lib().moe_forward_workspace_size(ctypes.byref(c.layer.desc), w.T, block_m)
    assert 0 < need <= L.NOALLOC_SCRATCH_BYTES, need
    for T in (w.T, T2):
        x = c.x[:T].contiguous()
        lg = None if c.logits is None else c.logits[:T].contiguous()
        ref = c.layer.forward(x, lg, block_m=block_m)
        y = torch.full((T, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
        L.check("moe_forward_noalloc", _noalloc(c.layer, x, lg, block_m, y))
        torch.cuda.synchronize()
        say("T", T, "equal", bool(torch.equal(y.view(torch.int16), ref.view(torch.int16))))
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), (name, T)


def test_noalloc_refuses_what_does_not_fit():
    w = synth.get("qwen3_235b_decode_ptpc").replace(T=4096, E=16)
    say("noalloc too large")
    c = build_case(w, cache_experts=False)
    need = L.lib().moe_forward_workspace_size(ctypes.byref(c.layer.desc), w.T, 0)
    assert need > L.NOALLOC_SCRATCH_BYTES
    y = torch.full((w.T, w.D), 7.0, dtype=torch.bfloat16, device="cuda")
    assert _noalloc(c.layer, c.x, c.logits, 0, y) == L.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))                    # nothing ran
    # T = 0 is a no-op; invalid arguments are reported as by moe_forward
    assert _noalloc(c.layer, c.x[:0], c.logits[:0], 0, y) == L.MOE_OK
    assert _noalloc(c.layer, c.x[:4].contiguous(), c.logits[:4].contiguous(), 48, y) == L.MOE_ERR_UNSUPPORTED
