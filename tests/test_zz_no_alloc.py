"""bl_ffn_step_noalloc (the FFN step on the library's fixed per-device scratch)
against bl_ffn_step with a caller workspace: the same bits on consecutive
calls, the later ones on smaller inputs, and shapes past the scratch
rejected."""
import numpy as np
import pytest

import ternary_weight_linear_quant_amd as bl
from ternary_weight_linear_quant_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")


def _weights(wid, K, N_ff):
    out = []
    for i, (n, k) in enumerate([(N_ff, K), (N_ff, K), (K, N_ff)]):
        pk, g = bl.quantize_weights(torch.from_numpy(wl.weights(wid, i, n, k)).to(DEV))
        out += [pk, g]
    return out


def _x(wid, M, K):
    return torch.from_numpy(wl.activations(wid, 7, M, K).view(np.int16)).to(DEV) \
        .view(torch.bfloat16)


def test_noalloc_matches_workspace_call_on_consecutive_calls():
    K, N_ff = 2560, 6912
    W = _weights(2, K, N_ff)
    gain = torch.from_numpy(wl.rms_gain(2, 3, N_ff).view(np.int16)).to(DEV).view(torch.bfloat16)
    # Largest first (the four-launch sequence fills most of the scratch), then
    # the three- and two-launch steps on smaller inputs.
    for M, kind, g in [(40, "relu2", None), (16, "swiglu", gain), (4, "relu2", gain),
                       (1, "relu2", None)]:
        x = _x(2, M, K)
        ref = bl.ffn_step(x, *W, kind=kind, subln_gain=g)
        got = bl.ffn_step_noalloc(x, *W, kind=kind, subln_gain=g)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), (M, kind)


def test_noalloc_second_call_smaller_on_70b_shapes():
    K, N_ff = 8192, 28672
    W = _weights(5, K, N_ff)
    for M in (25, 3):
        x = _x(5, M, K)
        ref = bl.ffn_step(x, *W)
        got = bl.ffn_step_noalloc(x, *W)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), M


def test_noalloc_rejects_shapes_past_the_scratch():
    K, N_ff = 8192, 28672
    W = _weights(5, K, N_ff)
    with pytest.raises(bl.BitLinearError, match="INVALID_ARG"):
        bl.ffn_step_noalloc(_x(5, 26, K), *W)
