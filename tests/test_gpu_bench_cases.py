"""The benchmark's timed calls that go straight to the C entry points (the quantiser
and the MQA logits) pass raw device pointers; the tensors behind them must live as
long as the call does.  Each case runs once, then the caching allocator is emptied
and the memory it released is written over; a second run must give the same bits."""
import gc

import pytest
import torch

import bench

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.mark.parametrize("kind", ["quant_fp8", "mqa_decode_fp4"])
def test_direct_calls_keep_their_inputs(kind):
    print(f"[gpu-test] bench case {kind}: inputs kept alive across allocator reuse", flush=True)
    call = bench.make_case(kind, DEV)[0]
    held = call.__defaults__[0]
    out = held[1] if kind == "quant_fp8" else held[-1]
    call()
    torch.cuda.synchronize()
    first = out.clone()
    out.fill_(0)
    gc.collect()
    torch.cuda.empty_cache()
    junk = [torch.full((n,), 0x5A, dtype=torch.uint8, device=DEV) for n in (1 << 29, 1 << 20, 1 << 14)]
    call()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), first.view(torch.uint8))
    del junk
