"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/moe.h declares, and its host-only functions and
argument validation behave as documented."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from tests.conftest import ROOT

mlr = pytest.importorskip("moe_layer_router_amd")
from moe_layer_router_amd import _lib as L  # noqa: E402


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int32_t|int64_t|size_t|char\s*\*|const char\s*\*)\s*\*?\s*"
                                 r"(moe_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 14, names
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES), set(names) ^ set(L.SIGNATURES)


def test_status_strings():
    for s in range(5):
        assert L.status_str(s)
    assert L.status_str(99) == "unknown status"


@pytest.mark.parametrize("T,k,E,ns,B", [(0, 8, 128, 0, 32), (1, 1, 1, 0, 1), (64, 2, 8, 0, 32),
                                        (8192, 8, 128, 0, 128), (32, 8, 128, 0, 32), (4096, 8, 256, 1, 64),
                                        (8192, 10, 512, 0, 1)])
def test_max_rows_matches_oracle(T, k, E, ns, B):
    assert L.lib().moe_permute_max_rows(T, k, E, ns, B) == O.permute_max_rows(T, k, E, ns, B)


def test_max_rows_rejects_bad_input():
    assert L.lib().moe_permute_max_rows(-1, 8, 128, 0, 32) == -1
    assert L.lib().moe_permute_max_rows(4, 8, 128, 2, 32) == -1


def _desc(**kw):
    d = dict(D=512, I=256, E=16, top_k=4, n_shared=0, scoring=0, n_groups=1, topk_groups=1, renormalize=1,
             route_scale=1.0, quant=1, weight_layout=1, w13=1 << 20, w13_scale=1 << 21, w2=1 << 22, w2_scale=1 << 23,
             router_w=None, sel_bias=None)
    d.update(kw)
    return L.LayerDesc(**d)


def test_validation_happens_before_any_launch():
    lib = L.lib()
    bad = ctypes.c_void_p(0)
    # NULL device pointers with T > 0 -> invalid argument, nothing enqueued
    assert lib.moe_route_topk(None, 4, 8, 2, 0, 1, 1, None, 1, 1.0, None, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route_topk(None, 4, 8, 9, 0, 1, 1, None, 1, 1.0, None, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route_topk(None, 4, 8, 17, 0, 1, 1, None, 1, 1.0, None, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route_topk(None, 4, 2048, 8, 0, 1, 1, None, 1, 1.0, None, None, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_topk(None, 4, 64, 8, 1, 7, 2, None, 1, 1.0, None, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route_topk(None, 4, 64, 8, 1, 8, 1, None, 1, 1.0, None, None, None) == L.MOE_ERR_INVALID_ARG
    # T = 0 is a valid no-op even with NULL buffers
    assert lib.moe_route_topk(None, 0, 8, 2, 0, 1, 1, None, 1, 1.0, None, None, None) == L.MOE_OK
    assert lib.moe_quant_ptpc_fp8(None, 0, 256, 0, None, None, None, None) == L.MOE_OK
    assert lib.moe_quant_ptpc_fp8(None, 4, 256, 64, None, None, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_quant_ptpc_fp8(None, 4, 200, 128, None, None, None, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_permute_align(None, 4, 2, 8, 0, 0, None, None, None, None, None, None, None) \
        == L.MOE_ERR_INVALID_ARG
    assert lib.moe_unpermute_combine(None, 2, None, None, 4, 2, 0, 256, None, None) == L.MOE_ERR_INVALID_ARG
    # a token gathers at most MOE_MAX_TOPK + 1 rows: the check comes before the pointer checks
    assert lib.moe_unpermute_combine(None, 1, None, None, 4, 17, 1, 256, None, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_unpermute_combine(None, 1, None, None, 4, 18, 0, 256, None, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_unpermute_combine(None, 1, None, None, 4, 16, 1, 256, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_unpermute_combine(None, 1, None, None, 4, 17, 0, 256, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_unpermute_combine(None, 1, None, None, 0, 17, 1, 256, None, None) == L.MOE_ERR_UNSUPPORTED
    # input validation: argument errors come back before its kernels are enqueued
    fake = ctypes.c_void_p(256)      # never dereferenced: every call below is refused first
    assert lib.moe_validate_inputs(None, 4, 256, None, 8, None, 2, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_validate_inputs(None, -1, 256, None, 8, None, 2, fake, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_validate_inputs(fake, 4, 0, None, 8, None, 2, fake, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_validate_inputs(None, 4, 256, fake, 0, None, 2, fake, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_validate_inputs(None, 4, 256, None, 0, fake, 2, fake, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_validate_inputs(None, 4, 256, None, 8, fake, 0, fake, None) == L.MOE_ERR_INVALID_ARG


def test_gemm_byte_ranges_are_checked_before_any_launch():
    """The LDS-tiled GEMMs address rows with 32-bit byte offsets.  A layer
    whose shapes exceed them is rejected by moe_forward before it enqueues
    its first kernel (routing), and has no workspace size."""
    lib = L.lib()
    # bf16, D = I = 16384, T = 70000: T*D*2 bytes >= 4 GiB
    d = _desc(D=16384, I=16384, E=8, top_k=2, quant=0, weight_layout=0, w13_scale=None, w2_scale=None)
    assert lib.moe_forward_workspace_size(ctypes.byref(d), 70000, 256) == 0
    lay = L.WsLayout()
    assert lib.moe_workspace_layout(ctypes.byref(d), 70000, 256, ctypes.byref(lay)) == L.MOE_ERR_UNSUPPORTED
    # pointers that would fault if anything were launched: nothing is
    assert lib.moe_forward(ctypes.byref(d), 1 << 24, 1 << 27, 70000, 256, 1 << 25, 1 << 26, 1 << 40, None) \
        == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_grouped_gemm_gateup_silu(ctypes.byref(d), 1, None, 70000, 256, 1, 1, 1, None, 1, None) \
        == L.MOE_ERR_UNSUPPORTED
    # FP8 PTPC at D = 4096, I = 16384: max_rows * I bytes of act codes >= 4 GiB
    d8 = _desc(D=4096, I=16384, E=128, top_k=8)
    assert lib.moe_forward_workspace_size(ctypes.byref(d8), 40000, 128) == 0
    assert lib.moe_grouped_gemm_down(ctypes.byref(d8), 1, 1, 40000, 128, 1, 1, None, 1, None) \
        == L.MOE_ERR_UNSUPPORTED
    # the weight-streaming kernels (block_m 16) use 64-bit addresses
    assert lib.moe_forward_workspace_size(ctypes.byref(d8), 64, 16) > 0


def test_layer_validation_and_workspace():
    lib = L.lib()
    d = _desc()
    assert lib.moe_forward_workspace_size(ctypes.byref(d), 100, 64) > 0
    # unsupported shapes / block sizes
    assert lib.moe_forward_workspace_size(ctypes.byref(_desc(I=200)), 100, 64) == 0
    assert lib.moe_forward_workspace_size(ctypes.byref(d), 100, 48) == 0
    assert lib.moe_forward_workspace_size(ctypes.byref(_desc(quant=2)), 100, 128) > 0
    assert lib.moe_forward_workspace_size(ctypes.byref(_desc(quant=2)), 100, 256) > 0
    assert lib.moe_forward_workspace_size(ctypes.byref(d), 100, 16) > 0
    assert lib.moe_forward_workspace_size(ctypes.byref(d), 64, 16) > 0
    assert lib.moe_forward_workspace_size(ctypes.byref(d), 100, 8) == 0
    # the automatic block size streams weights while the mean rows per expert stay small
    assert lib.moe_default_block_m(ctypes.byref(d), 64) == 16
    # 16 rows per expert: the weight-streaming kernels; 32 rows per expert: 32-row tiles
    assert lib.moe_default_block_m(ctypes.byref(_desc(E=128, top_k=8)), 256) == 16
    assert lib.moe_default_block_m(ctypes.byref(_desc(E=128, top_k=8)), 512) == 32
    assert lib.moe_default_block_m(ctypes.byref(_desc(quant=3, I=512, E=128, top_k=8)), 256) == 32
    assert lib.moe_default_block_m(ctypes.byref(_desc(quant=3, I=512, E=128, top_k=8)), 32) == 16
    assert lib.moe_default_block_m(ctypes.byref(_desc(E=128, top_k=8)), 8192) == 256
    # about 143 rows per expert (the DeepSeek-R1-shaped batch): one 192-row tile; MXFP4 stays at 128
    r1 = dict(E=256, top_k=8, n_shared=1, scoring=1, n_groups=8, topk_groups=4)
    assert lib.moe_default_block_m(ctypes.byref(_desc(quant=2, **r1)), 4096) == 192
    assert lib.moe_default_block_m(ctypes.byref(_desc(quant=3, I=512, **r1)), 4096) == 128
    assert lib.moe_default_block_m(ctypes.byref(_desc(quant=0, weight_layout=0, w13_scale=None, w2_scale=None,
                                                       **r1)), 4096) == 256
    assert lib.moe_forward(ctypes.byref(_desc(I=200)), None, None, 4, 0, None, None, 0, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_forward(ctypes.byref(_desc(w13=None)), None, None, 4, 0, None, None, 0, None) \
        == L.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(ctypes.byref(_desc(quant=7)), None, None, 4, 0, None, None, 0, None) \
        == L.MOE_ERR_INVALID_ARG
    # weight layouts: blocked needs an FP8 mode; unknown layouts are rejected
    assert lib.moe_forward_workspace_size(ctypes.byref(_desc(weight_layout=0)), 100, 64) > 0
    assert lib.moe_forward_workspace_size(ctypes.byref(_desc(quant=0, weight_layout=1, w13_scale=None,
                                                             w2_scale=None)), 100, 64) == 0
    assert lib.moe_forward(ctypes.byref(_desc(weight_layout=2)), None, None, 4, 0, None, None, 0, None) \
        == L.MOE_ERR_INVALID_ARG
    assert lib.moe_quant_weight_fp8(None, 1, 24, 128, 1, 1, None, None, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_quant_weight_fp8(None, 1, 32, 128, 1, 3, None, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_quant_weight_fp8(None, 1, 32, 128, 1, 1, None, None, None) == L.MOE_ERR_INVALID_ARG
    # no logits and no router weight
    assert lib.moe_forward(ctypes.byref(d), 1 << 24, None, 4, 0, 1 << 25, 1 << 26, 1 << 30, None) \
        == L.MOE_ERR_INVALID_ARG
    # workspace too small is reported before anything runs
    need = lib.moe_forward_workspace_size(ctypes.byref(d), 4, 0)
    assert lib.moe_forward(ctypes.byref(d), 1 << 24, 1 << 27, 4, 0, 1 << 25, 1 << 26, need - 1, None) \
        == L.MOE_ERR_WORKSPACE
    # misaligned workspace
    assert lib.moe_forward(ctypes.byref(d), 1 << 24, 1 << 27, 4, 0, 1 << 25, (1 << 26) + 8, need, None) \
        == L.MOE_ERR_INVALID_ARG
    # T = 0: no-op
    assert lib.moe_forward(ctypes.byref(d), None, None, 0, 0, None, None, 0, None) == L.MOE_OK


def test_workspace_layout_is_disjoint_and_aligned():
    lib = L.lib()
    for d, T in [(_desc(), 300), (_desc(quant=0, weight_layout=0, w13_scale=None, w2_scale=None), 64),
                 (_desc(quant=2, n_shared=1, scoring=1, n_groups=4, topk_groups=2, route_scale=2.5), 77)]:
        lay = L.WsLayout()
        assert lib.moe_workspace_layout(ctypes.byref(d), T, 0, ctypes.byref(lay)) == L.MOE_OK
        offs = sorted(getattr(lay, n) for n, _ in L.WsLayout._fields_[:16] if getattr(lay, n) >= 0)
        assert all(o % 256 == 0 for o in offs)
        assert len(set(offs)) == len(offs)
        assert lay.total == lib.moe_forward_workspace_size(ctypes.byref(d), T, 0)
        assert lay.max_rows == O.permute_max_rows(T, d.top_k, d.E, d.n_shared, lay.block_m)


def test_unblock_weights_inverts_the_blocked_byte_order():
    """unblock_weights (host side) undoes the blocked code layout the header
    documents: blocks of 16 rows x 128 bytes, each line holding one 64-byte
    K half of two consecutive rows."""
    torch = pytest.importorskip("torch")
    from moe_layer_router_amd import unblock_weights
    rng = np.random.default_rng(5)
    n, N, K = 2, 48, 384
    rowmajor = rng.integers(0, 256, size=(n, N, K), dtype=np.uint8)
    blocked = np.zeros(n * N * K, np.uint8)
    for e in range(n):
        for r in range(N):
            for k in range(K):
                r16, c = r % 16, k % 128
                j = (e * (N // 16) + r // 16) * (K // 128) + k // 128
                o = (r16 // 2 + 8 * (c // 64)) * 128 + ((r16 % 2) * 4 + (c % 64) // 16) * 16 + c % 16
                blocked[j * 2048 + o] = rowmajor[e, r, k]
    got = unblock_weights(torch.from_numpy(blocked.reshape(n, N, K)))
    assert np.array_equal(got.numpy(), rowmajor)
    # the first line of a block holds bytes 0..63 of rows 0 and 1
    assert np.array_equal(blocked[:64], rowmajor[0, 0, :64]) and np.array_equal(blocked[64:128], rowmajor[0, 1, :64])


def test_ep_payload_sizes_and_validation():
    """Payload row sizes match the oracle's closed forms (host-only call), and
    bad arguments are rejected before anything is enqueued."""
    lib = L.lib()
    for D in (128, 4096, 7168, 16384):
        b = O.ep_payload_bytes(D)
        assert lib.moe_ep_payload_bytes(D, L.PAYLOAD_MXFP4) == b["mxfp4"]
        assert lib.moe_ep_payload_bytes(D, L.PAYLOAD_FP8_BLOCK) == b["fp8_block"]
    for D in (0, -128, 96, 7000, 65536 + 128):
        assert lib.moe_ep_payload_bytes(D, L.PAYLOAD_MXFP4) == -1
    assert lib.moe_ep_payload_bytes(4096, 7) == -1
    assert lib.moe_ep_pack_payload(None, 4, 4096, L.PAYLOAD_MXFP4, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_ep_pack_payload(None, -1, 4096, L.PAYLOAD_MXFP4, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_ep_pack_payload(None, 4, 100, L.PAYLOAD_FP8_BLOCK, None, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_ep_unpack_payload(None, 4, 4096, 3, None, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_ep_pack_payload(None, 0, 4096, L.PAYLOAD_MXFP4, None, None) == L.MOE_OK
    assert lib.moe_ep_unpack_payload(None, 0, 4096, L.PAYLOAD_FP8_BLOCK, None, None) == L.MOE_OK
