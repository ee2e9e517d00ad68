"""GPU test of the debug input validation: moe_validate_inputs counts Inf and
NaN in x (bf16) and the logits and routed ids outside [0, E) exactly as
torch counts them on the host, and with the switch on the binding refuses
such inputs before it enqueues the forward or the permutation."""

import pytest
import torch

from tests.gpu_cases import REDUCED, build_case, say

pytestmark = pytest.mark.gpu

mlr = pytest.importorskip("moe_layer_router_amd")
ops = pytest.importorskip("moe_layer_router_amd.ops")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mlr.lib()


def _planted(T=300, D=512, E=64, k=6):
    g = torch.Generator().manual_seed(11)
    x = torch.randn((T, D), generator=g).to(torch.bfloat16)
    lg = torch.randn((T, E), generator=g)
    ids = torch.randint(0, E, (T, k), generator=g, dtype=torch.int32)
    fx = x.view(-1)
    for i, v in [(5, float("nan")), (1000, float("inf")), (T * D - 1, float("-inf")), (7, float("nan"))]:
        fx[i] = v
    fl = lg.view(-1)
    for i, v in [(0, float("inf")), (T * E // 2, float("nan"))]:
        fl[i] = v
    fi = ids.view(-1)
    for i, v in [(3, -1), (17, E), (T * k - 1, 2 * E), (40, -2 ** 31)]:
        fi[i] = v
    return x, lg, ids, E


def test_validate_counts_match_torch():
    x, lg, ids, E = _planted()
    want = {"x_nonfinite": int((~torch.isfinite(x.float())).sum()),
            "logits_nonfinite": int((~torch.isfinite(lg)).sum()),
            "ids_out_of_range": int(((ids < 0) | (ids >= E)).sum())}
    assert want == {"x_nonfinite": 4, "logits_nonfinite": 2, "ids_out_of_range": 4}
    got = mlr.validate_inputs(x.cuda(), lg.cuda(), ids.cuda())
    say("validate", got)
    assert got == want
    assert mlr.validate_inputs(x=x.cuda()) == {"x_nonfinite": 4, "logits_nonfinite": 0, "ids_out_of_range": 0}
    assert mlr.validate_inputs(ids=ids.cuda(), E=E)["ids_out_of_range"] == 4
    clean = mlr.validate_inputs(torch.zeros((3, 512), dtype=torch.bfloat16, device="cuda"),
                                torch.zeros((3, E), device="cuda"), torch.zeros((3, 6), dtype=torch.int32,
                                                                                device="cuda"))
    assert clean == {"x_nonfinite": 0, "logits_nonfinite": 0, "ids_out_of_range": 0}
    assert mlr.validate_inputs(x=x[:0].cuda()) == {"x_nonfinite": 0, "logits_nonfinite": 0, "ids_out_of_range": 0}


def test_validate_switch_refuses_bad_inputs(monkeypatch):
    w = REDUCED["tiny_bf16"]
    c = build_case(w)
    monkeypatch.setattr(ops, "VALIDATE", True)
    y = c.layer.forward(c.x, c.logits)                     # clean inputs pass and run
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y.float()).all())
    x = c.x.clone()
    x[1, 2] = float("nan")
    with pytest.raises(ValueError, match="non-finite"):
        c.layer.forward(x, c.logits)
    lg = torch.zeros((w.T, w.E), dtype=torch.float32, device="cuda")   # given logits in place of the router's
    lg[0, 0] = float("inf")
    with pytest.raises(ValueError, match="non-finite"):
        c.layer.forward(c.x, lg)
    ids = torch.zeros((4, 2), dtype=torch.int32, device="cuda")
    ids[2, 1] = w.E
    with pytest.raises(ValueError, match="outside"):
        mlr.permute_align(ids, w.E, 0, 32)
