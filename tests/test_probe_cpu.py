"""Host-side checks of libbsg_probe.so (include/bsg_probe.h) that need no GPU: it
loads, exports what its header declares, and rejects bad arguments before any HIP
call."""
import os
import re

from block_scaled_precision_05_amd import probe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "bsg_probe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_probe_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert names == ["bsg_probe_mfma"]
    lib = probe.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_probe_validation():
    f = probe.lib().bsg_probe_mfma
    P = 0x10000
    bad = [(3, 1, 1, 1, P), (-1, 1, 1, 1, P), (0, 1, 0, 1, P), (0, 1, 65536, 1, P),
           (0, 1, 1, -1, P), (0, 1, 1, (1 << 24) + 1, P), (0, 1, 1, 1, 0), (2, 1, 1, 1, P + 2)]
    for kind, seed, wg, iters, out in bad:
        assert f(kind, seed, wg, iters, out, None) == 1, (kind, wg, iters, out)


def test_probe_flop_count():
    # 8 waves x 16 MFMAs a round; BF16 32x32x16, FP8 / FP4 32x32x64
    assert probe.flops_per_call("bf16", 1, 1) == 8 * 16 * 32 * 32 * 16 * 2
    assert probe.flops_per_call("fp4", 256, 10) == 256 * 8 * 16 * 10 * 32 * 32 * 64 * 2
