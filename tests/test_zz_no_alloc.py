"""The allocation-free MoE FFN entry point against the workspace one, through the
C ABI: two calls in a row (the benchmark's one-GPU FFN share, then a smaller
problem in the same scratch array) must each equal moe_ffn_fp8 bit for bit on
every written row, and leave rows outside the experts untouched."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_precision_05_amd as bsg
from block_scaled_precision_05_amd import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
FILL = 0x7FC1


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _operands(w):
    t = w.tensors
    G, two_i, hidden = t["W13"].shape
    inter = two_i // 2
    M = t["A"].shape[0]
    sfa = bsg.ensure_packed(t["sfa"], M, hidden // 128)
    sfw13 = torch.stack([bsg.ensure_packed(x, (two_i + 127) // 128, hidden // 128)
                         for x in t["sfw13"]])
    sfw2 = torch.stack([bsg.ensure_packed(x, (hidden + 127) // 128, inter // 128)
                        for x in t["sfw2"]])
    return t, G, M, hidden, inter, sfa, sfw13, sfw2


def _noalloc(w, rule):
    t, G, M, hidden, inter, sfa, sfw13, sfw2 = _operands(w)
    D = torch.full((M, hidden), FILL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    f = bsg.lib().moe_ffn_fp8_noalloc
    A, W13, W2 = t["A"].view(torch.uint8), t["W13"].view(torch.uint8), t["W2"].view(torch.uint8)
    st = f(A.data_ptr(), A.stride(0), sfa.data_ptr(), sfa.stride(0),
           W13.data_ptr(), W13.stride(1), W13.stride(0), sfw13.data_ptr(), sfw13.stride(1),
           sfw13.stride(0),
           W2.data_ptr(), W2.stride(1), W2.stride(0), sfw2.data_ptr(), sfw2.stride(1),
           sfw2.stride(0),
           t["offsets"].data_ptr(), G, M, hidden, inter, D.data_ptr(), D.stride(0),
           bsg.SCALE_RULES[rule], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == bsg.BSG_OK, bsg.status_string(st)
    return D


def _with_workspace(w, rule):
    t, G, M, hidden, inter, sfa, sfw13, sfw2 = _operands(w)
    D = torch.full((M, hidden), FILL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    bsg.moe_ffn_fp8(t["A"], sfa, t["W13"], sfw13, t["W2"], sfw2, t["offsets"], rule=rule, out=D)
    return D


def _same(w, D, Dref, what):
    torch.cuda.synchronize()
    got = D.view(torch.int16).cpu().numpy()
    want = Dref.view(torch.int16).cpu().numpy()
    off = w.tensors["offsets"].cpu().numpy()
    lo, hi = int(off[0]), int(off[-1])
    bad = int(np.sum(got[lo:hi] != want[lo:hi]))
    assert bad == 0, f"{what}: {bad} outputs differ from moe_ffn_fp8"
    assert np.all(got[:lo] == FILL) and np.all(got[hi:] == FILL)
    assert not np.any(got[lo:hi] == FILL)
    _say(f"  {what}: {hi - lo} rows x {got.shape[1]} bit-identical to moe_ffn_fp8")


@pytest.mark.parametrize("rule", ["ceil", "ocp_mx"])
def test_noalloc_equals_workspace_call_twice_in_a_row(rule):
    _say(f"moe_ffn_fp8_noalloc, rule {rule}: FFN share (48 + 1 experts, 7168/2048), then small")
    big = workloads.make("moe_ffn", device=DEV)
    assert big.tensors["A"].shape[0] * 2048 <= 64 << 20
    D1 = _noalloc(big, rule)
    _same(big, D1, _with_workspace(big, rule), "first call (FFN share)")
    del D1
    small = workloads.moe_ffn(71, device=DEV, hidden=512, inter=384, counts=[130, 0, 256, 37],
                              align=1)
    D2 = _noalloc(small, rule)
    _same(small, D2, _with_workspace(small, rule), "second call (423 rows, inter 384)")
