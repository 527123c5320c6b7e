"""The GEMM kernels' ring barriers wait with explicit vmcnt counts that a compile-time
replay of each wave's load order derives.  Those counts are exact only if the compiled
code issues every copy and scale-word load the replay expects, in the k-step it expects:
a load the compiler dropped or merged would let a wave pass a barrier before its stage
landed.  This test disassembles the gfx950 code of the built libbsg.so (the LLVM tools
under /opt/rocm, no GPU needed) and checks, for every GEMM instantiation, that each
steady stage loop issues per barrier interval the copies and scale loads of an
independent Python model of the schedule, and, in the waves that issue the copies,
waits for the count that model gives."""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_scaled_precision_05_amd", "libbsg.so")
LLVM = "/opt/rocm/llvm/bin"
BF16, FP8, FP4 = 0, 1, 2


def _tools_present():
    return all(os.path.exists(os.path.join(LLVM, t))
               for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump"))


def disassemble(lib):
    """Device code of every bundle in the library's fat binary, as text."""
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fat.bin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", f".hip_fatbin={fat}", lib],
                       check=True, capture_output=True)
        data = open(fat, "rb").read()
        magic = b"__CLANG_OFFLOAD_BUNDLE__"
        starts = [m.start() for m in re.finditer(re.escape(magic), data)] + [len(data)]
        text = []
        for k in range(len(starts) - 1):
            part = os.path.join(d, f"b{k}.bin")
            with open(part, "wb") as f:
                f.write(data[starts[k]:starts[k + 1]])
            co = os.path.join(d, f"b{k}.o")
            r = subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--type=o",
                                "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={part}",
                                f"--output={co}", "--unbundle"], capture_output=True)
            if r.returncode != 0 or not os.path.exists(co) or os.path.getsize(co) == 0:
                continue
            r = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", co],
                               check=True, capture_output=True, text=True)
            text.append(r.stdout)
        return "\n".join(text)


def copying_waves(kind, wm, wn, grouped):
    """Waves that issue the copies: with eight waves the upper row only, except in the
    dense FP8 kernel, where every wave does."""
    nw = wm * wn
    return nw // 2 if nw > 4 and (kind != FP8 or grouped) else nw


class Schedule:
    """Python model of the kernel template's paired copy schedule (gemm_kernel.h):
    per k-step the chunk of copies (and, at a pair's first chunks, the scale loads)
    a wave issues, and the vmcnt each barrier of a copying wave waits for.  copies:
    the wave is one of the copying waves; scales: it loads scale words (it runs
    MFMAs)."""

    def __init__(self, kind, bm, bn, wm, wn, sb, ns, sv, scales=True, grouped=False, copies=True):
        nwc = copying_waves(kind, wm, wn, grouped)
        nc = sb // 16
        self.J = nc // 4 if kind == FP8 else nc // 2
        rows_per_copy = 1024 // sb
        a_loads = -(-(bm // rows_per_copy) // nwc)
        b_loads = -(-(bn // rows_per_copy) // nwc)
        self.n_dma = a_loads + b_loads
        self.copies = copies
        tn, tm = bn // wn, bm // wm
        fn, fm = tn // 32, tm // 32
        wide, b_row = bool(sv & 1), kind == FP8 and bool(sv & 2)
        one_b = not b_row and tn <= 128 and 128 % tn == 0 and bn % 128 == 0
        nsb = (1 if one_b else fn) if kind == FP8 else fn
        sw = 0 if kind == BF16 else (1 if kind == FP8 else nc // 4)
        perm_b = kind == FP4
        nsc = (1 + (1 if perm_b else nsb)) * sw if wide else (fm + nsb) * sw
        self.nsc = nsc if scales else 0
        self.shared = kind == FP8
        self.ns = ns
        self.U = 2 * ns if ns % 2 else ns
        self.p0 = (ns - 1) % 2
        self.qpc = self.n_dma // (2 * self.J)

    def chunk_at(self, g):
        return (g - (self.p0 * self.J + self.J - 1)) % (2 * self.J)

    def pair_start(self, g):
        return (g - self.chunk_at(g) - (self.J - 1)) // self.J

    def chunk(self, g):
        """(scale loads, copies) of the chunk due at k-step g."""
        c = self.chunk_at(g)
        sc = self.nsc if (c == 0 or (c == 1 and not self.shared)) else 0
        return sc, (2 * self.qpc if self.copies else 0)

    def interval(self, s):
        """(copies, scale loads) a wave issues between the barriers of stages s-1 and
        s: the chunk of the k-step holding barrier s-1 (issued after it) and those of
        stage s's k-steps before its barrier."""
        J = self.J
        gs = [(s - 1) * J + J - 1] + [s * J + j for j in range(J - 1)]
        sc = sum(self.chunk(g)[0] for g in gs)
        cp = sum(self.chunk(g)[1] for g in gs)
        return cp, sc

    def wait(self, s):
        """vmcnt at the barrier of stage s in the steady state: the loads issued
        after the last copy of stage s+1 (a copying wave)."""
        ns, J, qpc = self.ns, self.J, self.qpc
        issued, last = 0, None
        st = s + 1
        for g in range(-(ns + 2) * J, s * J + J - 1):
            c = self.chunk_at(g)
            t = self.pair_start(g) + ns - 1
            if t < 0:
                continue
            issued += self.chunk(g)[0]
            for _ in range(qpc):
                if t == st:
                    last = issued
                issued += 1
                if t + 1 == st:
                    last = issued
                issued += 1
        return issued - 1 - last


def kernels(dis):
    """{template args: [(address, instruction, comment)]} for every gemm_kernel."""
    out, cur = {}, None
    for line in dis.splitlines():
        m = re.match(r"^[0-9a-f]+ <(_Z\S+)>:", line)
        if m:
            name = m.group(1)
            t = re.search(r"gemm_kernelI(.*?)EEEvNS_8GemmArgsE", name)
            cur = None
            if t:
                args = tuple(int(x) for x in re.findall(r"L[ib](\d+)E", t.group(1) + "E"))
                cur = out.setdefault(args, [])
            continue
        if cur is None:
            continue
        m = re.match(r"^\s+(\S.*?)\s*//\s*([0-9A-F]+):(.*)$", line)
        if m:
            cur.append((int(m.group(2), 16), m.group(1), m.group(3)))
    return out


def stage_loops(ins, per_round):
    """Bodies of the branch-free backward loops that hold a whole round of barriers:
    the steady stage loops (every stage of the steady loop runs the same straight-line
    code)."""
    loops = []
    for addr, text, note in ins:
        if not text.startswith("s_cbranch_"):
            continue
        # objdump names the target as <kernel+offset>, the offset from the kernel start
        mt = re.search(r"<\S+\+0x([0-9a-f]+)>", note)
        if not mt:
            continue
        target = ins[0][0] + int(mt.group(1), 16)
        if target >= addr:
            continue
        body = [t for a, t, _ in ins if target <= a <= addr]
        if any(t.startswith(("s_cbranch", "s_branch", "s_setpc")) for t in body[:-1]):
            continue
        if sum(1 for t in body if t.startswith("s_barrier")) == per_round:
            loops.append(body)
    return loops


def observed(body):
    """Per barrier of a loop body: (copies, scale loads, vmcnt) issued since the
    previous barrier, the wait being the last vmcnt before the barrier (63 when the
    barrier's wait leaves vmcnt out).  The body is a cycle: what follows its last
    barrier runs before its first one on the next trip."""
    res, cp, sc, wait = [], 0, 0, None
    for t in body:
        if t.startswith("buffer_load"):
            if " lds" in t:
                cp += 1
            else:
                sc += 1
        elif t.startswith("s_waitcnt"):
            m = re.search(r"vmcnt\((\d+)\)", t)
            wait = int(m.group(1)) if m else 63
        elif t.startswith("s_barrier"):
            res.append([cp, sc, wait])
            cp, sc, wait = 0, 0, None
    if res:
        res[0][0] += cp
        res[0][1] += sc
        if res[0][2] is None:
            res[0][2] = wait
    return [(c, s_, 63 if w is None else w) for c, s_, w in res]


def rotations(seq):
    return [tuple(seq[i:] + seq[:i]) for i in range(len(seq))]


@pytest.fixture(scope="module")
def dis():
    if not _tools_present() or not os.path.exists(LIB):
        pytest.skip("the ROCm LLVM tools or the built library are missing")
    return disassemble(LIB)


def test_every_gemm_instantiation_found(dis):
    ks = kernels(dis)
    # dense BF16/FP8/FP4, grouped FP8/BF16/FP4 and the masked and SwiGLU variants
    assert len(ks) >= 60
    assert all(len(v) > 100 for v in ks.values())


def test_steady_loops_issue_and_wait_what_the_schedule_says(dis):
    """Copying waves: copies, scale loads and vmcnt per barrier interval as the model
    says.  The other waves issue no copies and wait for none (their scale words are
    waited for by the compiler where it decodes them): their loops must issue exactly
    the model's scale loads and no copy."""
    checked = 0
    for args, ins in kernels(dis).items():
        kind, bm, bn, wm, wn, sb, ns, pr, grouped, sv, koff, epi = args
        assert pr == 1, args
        nw, nwc = wm * wn, copying_waves(kind, wm, wn, grouped)
        # (model, its waits checked, whether it runs MFMAs)
        models = [(Schedule(kind, bm, bn, wm, wn, sb, ns, sv, True, grouped, True), True, True)]
        if nwc < nw:
            models.append((Schedule(kind, bm, bn, wm, wn, sb, ns, sv, True, grouped, False), False, True))
        if grouped and wm > 1 and nw > 4:
            # the lower row of waves runs an expert's half-height last tile without
            # MFMAs and without scale loads
            models.append((Schedule(kind, bm, bn, wm, wn, sb, ns, sv, False, grouped, nwc == nw),
                           nwc == nw, False))
        U = models[0][0].U
        keys = []   # per model: the rotations of its per-barrier sequence
        for m, waits, _ in models:
            seq = [m.interval(s) + ((m.wait(s),) if waits else ()) for s in range(U, 2 * U)]
            keys.append(set(rotations(seq)))
        loops = stage_loops(ins, U)
        assert loops, f"no steady stage loop found in gemm_kernel{args}"
        matched = [False] * len(models)
        for body in loops:
            got = tuple(observed(body))
            hit = False
            for i, (_, waits, _) in enumerate(models):
                if (got if waits else tuple(x[:2] for x in got)) in keys[i]:
                    matched[i] = hit = True
            assert hit, f"gemm_kernel{args}: loop issues/waits {got}"
        # every variant of the tile body has its loop (BF16's two waves without copies
        # load no scale words either, so one loop can stand for both)
        assert all(matched), (args, matched)
        checked += 1
    assert checked >= 60


def test_model_matches_the_known_fp4_schedule():
    """The waits the kernel template derives for dense FP4, read off its assembly: a
    copying wave (the upper row issues every copy, eight a stage) waits for 20 and 13
    at alternate barriers, the 13 after the interval that holds a pair's two
    scale-load chunks (four loads); dense FP8, where every wave copies (four a stage),
    for 10 and 7."""
    m = Schedule(FP4, 256, 256, 2, 4, 64, 5, 1)
    assert [m.wait(s) for s in range(10, 14)] == [20, 13, 20, 13]
    assert [m.interval(s) for s in range(10, 14)] == [(8, 0), (8, 4), (8, 0), (8, 4)]
    m = Schedule(FP4, 256, 256, 2, 4, 64, 5, 1, copies=False)
    assert [m.interval(s) for s in range(10, 14)] == [(0, 0), (0, 4), (0, 0), (0, 4)]
    m = Schedule(FP8, 256, 256, 2, 4, 64, 5, 1)
    assert [m.wait(s) for s in range(10, 12)] == [10, 7]
