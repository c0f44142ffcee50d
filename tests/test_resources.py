"""Code-generation checks on the built kernels (CPU only, no device calls).

The pages ask that the matmul tests also check for stack frames and register
spills in the generated kernels (issue "Automate performant Hopper matmul",
task list).  Here that is done two ways on the gfx950 build of libmm.so:

* the compiler's resource remarks, which the build writes next to the
  library: LDS within the 160 KiB one workgroup can hold, no dynamic stack,
  registers within the file, and spills within a recorded budget;
* the disassembly of the library's own gfx950 code object: no scratch access
  in any K loop (a loop that issues MFMAs and holds no loop that does), so
  the spills the 256-accumulator kernels do have stay in per-tile code.
"""
import os
import re
import shutil
import subprocess

import pytest

from dense_bf16_gemm_amd import build

LDS_MAX = 160 * 1024
REG_FILE = 512  # VGPRs + AGPRs per lane at one wave per SIMD

# Kernels that keep a 256 x 256 tile's 256 fp32 accumulators per lane in the
# AGPRs leave a few values of the per-tile bookkeeping (tile bases, epilogue
# pointers) in scratch; every other kernel has none.  The budget is a little
# above the present counts (at most 7 VGPR and 6 SGPR dwords): a change that
# spills more fails here and is looked at.
SPILL_BUDGET_256ACC = {"VGPRs Spill": 8, "SGPRs Spill": 8, "ScratchSize [bytes/lane]": 32}
# The bias-staging slab instance (selected only by configuration) keeps the
# staging state in scalar registers across its K loop; its scalar spills go
# to vector-register lanes outside the loop (test_no_lane_spills_in_mfma_loops).
SPILL_BUDGET_OVERRIDE = {
    "_ZN3mmk12gemm_nt_slabILi256ELi256ELi2ELi2ELb0ELb0ELb0ELb0ELb0ELb1ELb0EEEvNS_10GemmParamsE":
        {"SGPRs Spill": 12},
}


def _tool(name: str) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "llvm", "bin", name)
    if os.path.exists(path):
        return path
    found = shutil.which(name)
    assert found, f"{name} not found under {rocm}/llvm/bin or on PATH"
    return found


@pytest.fixture(scope="module")
def remarks():
    assert os.path.exists(build.LIB), "libmm.so is not built"
    assert os.path.exists(build.REMARKS), "the build's resource remarks are missing"
    r = build.resource_usage()
    assert r, "no kernels in the resource remarks"
    return r


@pytest.fixture(scope="module")
def disassembly(tmp_path_factory):
    """{kernel symbol: [(address, mnemonic, branch target or None)]} of the
    gfx950 code object inside libmm.so."""
    d = tmp_path_factory.mktemp("co")
    fatbin, co = str(d / "fatbin.bin"), str(d / "gfx950.co")
    subprocess.run([_tool("llvm-objcopy"), "--dump-section", f".hip_fatbin={fatbin}", build.LIB],
                   check=True, capture_output=True)
    subprocess.run([_tool("clang-offload-bundler"), "--type=o", "--unbundle", f"--input={fatbin}",
                    f"--output={co}", f"--targets=hipv4-amdgcn-amd-amdhsa--{build.ARCH}"],
                   check=True, capture_output=True)
    text = subprocess.run([_tool("llvm-objdump"), "-d", f"--mcpu={build.ARCH}", co],
                          check=True, capture_output=True, text=True).stdout
    head = re.compile(r"^([0-9a-f]+) <(\S+)>:$")
    insn = re.compile(r"^\s+(\S+).*//\s*([0-9A-Fa-f]+):[0-9A-Fa-f ]*(?:<(\S+?)(?:\+0x([0-9a-f]+))?>)?\s*$")
    funcs, starts, cur = {}, {}, None
    for line in text.splitlines():
        m = head.match(line)
        if m:
            cur = m.group(2)
            starts[cur] = int(m.group(1), 16)
            funcs[cur] = []
            continue
        m = insn.match(line)
        if cur is None or not m:
            continue
        mnem, addr = m.group(1), int(m.group(2), 16)
        target = None
        if mnem.startswith(("s_branch", "s_cbranch")) and m.group(3) in starts:
            target = starts[m.group(3)] + int(m.group(4) or "0", 16)
        funcs[cur].append((addr, mnem, target))
    return funcs


def _is_mfma(mnem: str) -> bool:
    return mnem.startswith(("v_mfma", "v_smfmac"))


def _blocks(code):
    """Basic blocks of one kernel: {start address: (instructions, successors)}."""
    addrs = [a for (a, _, _) in code]
    leaders = {addrs[0]}
    for i, (a, mnem, t) in enumerate(code):
        if mnem.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            if t is not None:
                leaders.add(t)
            if i + 1 < len(code):
                leaders.add(code[i + 1][0])
    blocks, cur = {}, None
    for i, (a, mnem, t) in enumerate(code):
        if a in leaders:
            cur = a
            blocks[cur] = ([], [])
        ins, succ = blocks[cur]
        ins.append(mnem)
        nxt = code[i + 1][0] if i + 1 < len(code) else None
        ends = nxt is None or nxt in leaders
        if mnem.startswith("s_branch"):
            succ.append(t)
        elif mnem.startswith("s_cbranch"):
            succ += [t, nxt]
        elif mnem.startswith(("s_endpgm", "s_setpc")):
            pass
        elif ends and nxt is not None:
            succ.append(nxt)
    return {k: (ins, [x for x in succ if x in blocks or x in leaders]) for k, (ins, succ) in blocks.items()}


def _sccs(nodes, edges):
    """Strongly connected components (Tarjan, iterative) of the subgraph on
    `nodes` with successor lists `edges`."""
    index, low, on, stack, out, n = {}, {}, set(), [], [], 0
    for root in nodes:
        if root in index:
            continue
        work = [(root, iter(edges[root]))]
        index[root] = low[root] = n
        n += 1
        stack.append(root)
        on.add(root)
        while work:
            v, it = work[-1]
            for w in it:
                if w not in nodes:
                    continue
                if w not in index:
                    index[w] = low[w] = n
                    n += 1
                    stack.append(w)
                    on.add(w)
                    work.append((w, iter(edges[w])))
                    break
                if w in on:
                    low[v] = min(low[v], index[w])
            else:
                work.pop()
                if work:
                    low[work[-1][0]] = min(low[work[-1][0]], low[v])
                if low[v] == index[v]:
                    comp = set()
                    while True:
                        w = stack.pop()
                        on.discard(w)
                        comp.add(w)
                        if w == v:
                            break
                    out.append(comp)
    return out


def _loop_forest(code):
    """Loops of the control-flow graph, outermost first, as (block starts,
    child loops, blocks): a loop is a strongly connected component; the loops
    nested in it are found again after removing the edges that re-enter its
    entry blocks (this also handles loops with several entries, which the
    compiler makes here)."""
    blocks = _blocks(code)
    succ = {k: v[1] for k, v in blocks.items()}

    def walk(nodes, edges):
        loops = []
        for comp in _sccs(nodes, edges):
            if len(comp) == 1:
                (v,) = comp
                if v not in edges[v]:
                    continue
            heads = {v for v in comp if any(v in succ[u] for u in blocks if u not in comp)}
            inner = {u: [w for w in edges[u] if w in comp and w not in heads] for u in comp}
            loops.append((comp, walk(comp, inner)))
        return loops

    return walk(set(blocks), succ), blocks


def _k_loops(code):
    """The K loops, as instruction lists: loops that issue MFMAs in their own
    blocks and contain no loop that issues MFMAs.  (A tile loop that also
    holds a peeled last k-step issues MFMAs itself but has its K loop inside.)"""
    forest, blocks = _loop_forest(code)

    def has_mfma(comp):
        return any(_is_mfma(m) for b in comp for m in blocks[b][0])

    out = []

    def visit(comp, children):
        for (c, ch) in children:
            visit(c, ch)
        if any(has_mfma(c) for (c, _) in children):
            return
        if has_mfma(comp):
            out.append([m for b in sorted(comp) for m in blocks[b][0]])

    for (comp, children) in forest:
        visit(comp, children)
    return out


def _code(listing):
    """Instruction tuples from (address, mnemonic, branch target) rows."""
    return [(a, m, t) for (a, m, t) in listing]


# Hand-made control flow for the checker itself: a tile loop (entered at 8)
# with a per-tile scratch reload and a peeled MFMA, around a K loop whose
# cycle B -> C -> B is entered at B from the tile loop.
TILE_AND_K = [
    (0, "s_cmp_eq_u32", None),
    (4, "s_cbranch_scc1", 44),
    (8, "scratch_load_dword", None),     # tile loop: per-tile reload
    (12, "v_mfma_f32_16x16x32_bf16", None),  # peeled k-step
    (16, "s_nop", None),
    (20, "v_mfma_f32_16x16x32_bf16", None),  # K loop, block B
    (24, "s_barrier", None),
    (28, "v_mfma_f32_16x16x32_bf16", None),  # block C
    (32, "s_cbranch_scc1", 20),          # back to B
    (36, "s_cbranch_scc1", 8),           # next tile
    (40, "s_nop", None),
    (44, "s_endpgm", None),
]


def test_checker_finds_k_loops_on_known_control_flow():
    loops = _k_loops(_code(TILE_AND_K))
    assert loops == [["v_mfma_f32_16x16x32_bf16", "s_barrier", "v_mfma_f32_16x16x32_bf16",
                      "s_cbranch_scc1"]]
    # a scratch access planted in the K loop is seen
    planted = [(a, "scratch_load_dword" if a == 24 else m, t) for (a, m, t) in TILE_AND_K]
    assert any(m.startswith("scratch_") for body in _k_loops(_code(planted)) for m in body)
    # the K cycle entered at two blocks (from the tile loop at B, and at C by
    # a branch from the tile loop's head) is still one K loop without the
    # tile loop's reload
    two_entry = [(a, m, t) for (a, m, t) in TILE_AND_K]
    two_entry[4] = (16, "s_cbranch_vccz", 28)
    loops = _k_loops(_code(two_entry))
    assert len(loops) == 1 and not any(m.startswith("scratch_") for m in loops[0])
    assert sum(_is_mfma(m) for m in loops[0]) == 2
    # a loop with no MFMA inside the K loop leaves the K loop checked
    spin = [(a, m, t) for (a, m, t) in TILE_AND_K]
    spin[6] = (24, "s_cbranch_scc0", 24)  # a one-block loop at 24
    spin.insert(7, (26, "scratch_load_dword", None))
    loops = _k_loops(_code(spin))
    assert len(loops) == 1 and any(m.startswith("scratch_") for m in loops[0])


def test_remarks_match_the_built_code_object(remarks, disassembly):
    kernels = {k for k in disassembly if k.startswith("_ZN3mmk")}
    assert set(remarks) == kernels, "resource remarks and libmm.so come from different builds"


def test_lds_registers_and_stack(remarks):
    for name, r in remarks.items():
        assert r["LDS Size [bytes/block]"] <= LDS_MAX, name
        assert r.get("Dynamic Stack", 0) == 0, name
        assert r["VGPRs"] + r["AGPRs"] <= REG_FILE, name
        assert r["Occupancy [waves/SIMD]"] >= 1, name


def test_spills_within_budget(remarks):
    for name, r in remarks.items():
        if r["AGPRs"] >= 256:
            for key, cap in SPILL_BUDGET_256ACC.items():
                cap = SPILL_BUDGET_OVERRIDE.get(name, {}).get(key, cap)
                assert r[key] <= cap, (name, key, r[key])
        else:
            for key in SPILL_BUDGET_256ACC:
                assert r[key] == 0, (name, key, r[key])


def test_no_scratch_in_mfma_loops(disassembly):
    checked = 0
    for name, code in disassembly.items():
        if not any(_is_mfma(m) for (_, m, _) in code):
            continue
        k_loops = _k_loops(code)
        assert k_loops, f"{name}: no K loop found"
        for body in k_loops:
            assert not any(m.startswith("scratch_") for m in body), name
        checked += 1
    assert checked >= 10


def test_no_lane_spills_in_mfma_loops(disassembly):
    """Scalar-register spills (to and from vector-register lanes) stay out of
    every K loop as well."""
    for name, code in disassembly.items():
        if not any(_is_mfma(m) for (_, m, _) in code):
            continue
        for body in _k_loops(code):
            assert not any(m in ("v_writelane_b32", "v_readlane_b32") for m in body), name


def test_headline_kernel_k_loop_shape(disassembly):
    """The 256 x 256 slab kernel's K loop: 128 MFMAs per 64-k super-step (a
    multiple of it if unrolled), one barrier per super-step, no scratch."""
    name = "_ZN3mmk12gemm_nt_slabILi256ELi256ELi2ELi2ELb0ELb0ELb0ELb0ELb0ELb0ELb0EEEvNS_10GemmParamsE"
    code = disassembly[name]
    loops = _k_loops(code)
    assert len(loops) == 1, len(loops)
    body = loops[0]
    n_mfma = sum(_is_mfma(m) for m in body)
    n_bar = sum(m == "s_barrier" for m in body)
    assert n_mfma % 128 == 0 and n_bar == n_mfma // 128, (n_mfma, n_bar)
    assert all(m == "v_mfma_f32_16x16x32_bf16" for m in body if _is_mfma(m))
