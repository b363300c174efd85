"""The decode kernels' tile loop, as compiled for gfx950 (host-side check of the device
assembly, no GPU): at the head of the innermost loop the next tile's loads are issued
without first waiting for every outstanding load. A `s_waitcnt vmcnt(0)` there would
request a tile only once the previous one had arrived, leaving one tile in flight while the
matrix products run (it cost the 8B batch 58.5 against 55.9 us on MI355X). The compiler
placed such a wait when the loop rebuilt 64-bit per-lane tile addresses, or compared block
ids in 64 bits, in registers that loads were still filling; the kernels now read tiles
through per-tile buffer resources at fixed lane offsets. Also checked: the tile loads of
the 16-token kernels carry the non-temporal hint."""
import os
import re
import subprocess
import tempfile

import pytest

from paged_kv_cache_28_amd import build as B


def _asm(src: str) -> str:
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        flags = [f for f in B.common_flags() if f != "-fPIC"]
        r = subprocess.run([hipcc] + flags + ["--cuda-device-only", "-S", "-o", out,
                                              os.path.join(B.CSRC, src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


@pytest.fixture(scope="module")
def asm16():
    return _asm("decode.hip")


def _kernels(asm: str, pattern: str):
    names = re.findall(r"^(_ZN3pkv\w+):", asm, re.M)
    for nm in names:
        if re.search(pattern, nm):
            i = asm.index(nm + ":")
            yield nm, asm[i:asm.index("s_endpgm", i)]


def _blocks(body: str):
    """Basic blocks of a kernel's listing: (name, innermost loop or None, loops it heads
    with their ancestors, lines). The compiler annotates each block with its loop
    ("in Loop: Header=BBx Depth=d") and each loop header with its ancestors ("Parent Loop")."""
    blocks = []
    cur = None
    for ln in body.split("\n"):
        m = re.match(r"^(\.LBB\w+):|^; %bb\.(\d+):", ln)
        if m:
            name = m.group(1)[2:] if m.group(1) else "bb" + m.group(2)   # .LBBx_y -> BBx_y
            cur = {"name": name, "loop": None, "parents": [], "lines": []}
            blocks.append(cur)
            lm = re.search(r"in Loop: Header=(BB\w+) Depth", ln)
            if lm:
                cur["loop"] = lm.group(1)
            pm = re.search(r"Parent Loop (BB\w+) Depth", ln)
            if pm:
                cur["parents"].append(pm.group(1))
            if re.search(r"Loop Header: Depth=", ln):
                cur["loop"] = cur["name"]
            continue
        if cur is None:
            continue
        pm = re.search(r"^\s*;\s*Parent Loop (BB\w+) Depth", ln)
        if pm:
            cur["parents"].append(pm.group(1))
        if re.search(r"Loop Header: Depth=", ln):
            cur["loop"] = cur["name"]
        cur["lines"].append(ln)
    return blocks


def _tile_loops(body: str):
    """(waits, first load) of the tile loops: the deepest loops that issue buffer loads in
    their own blocks; the memory waits from the loop's header to its first buffer load."""
    blocks = _blocks(body)
    parent = {}
    for b in blocks:
        if b["loop"] == b["name"]:
            parent[b["name"]] = b["parents"][-1] if b["parents"] else None

    def chain(loop):
        out = []
        while loop is not None:
            out.append(loop)
            loop = parent.get(loop)
        return out

    depth = {L: len(chain(L)) for L in parent}
    owner = {}    # loop -> indices of its blocks (nested loops' blocks included)
    for i, b in enumerate(blocks):
        for L in chain(b["loop"]) if b["loop"] else []:
            owner.setdefault(L, []).append(i)
    is_load = lambda l: re.search(r"\bbuffer_load_dwordx[24]\b", l)   # noqa: E731
    own_loads = {L: any(is_load(l) for i in idx if blocks[i]["loop"] == L for l in blocks[i]["lines"])
                 for L, idx in owner.items()}
    cands = [L for L, v in own_loads.items() if v]
    if not cands:
        return
    deepest = max(depth[L] for L in cands)
    for L in cands:
        if depth[L] != deepest:
            continue
        waits = []
        for i in sorted(owner[L]):
            for l in blocks[i]["lines"]:
                if "s_waitcnt" in l and "vmcnt" in l:
                    waits.append(l.strip())
                if is_load(l):
                    yield waits, l.strip()
                    break
            else:
                continue
            break


# decode_mfma_kernel (single pass / partitions), 16-bit and FP8 caches, with and without
# the fused append, and decode_split_kernel over FP8 caches (over 16-bit caches it keeps
# one tile in flight, so its wait for the tile is a full one)
PATTERNS = [r"decode_mfma_kernelINS_6bf16_tELi128ES1_Li4ELb1ELb0ELi16E",
            r"decode_mfma_kernelINS_6bf16_tELi128ES1_Li4ELb0ELb0ELi16E",
            r"decode_mfma_kernelINS_5f16_tELi128ES1_Li4ELb0ELb0ELi16E",
            r"decode_mfma_kernelINS_6bf16_tELi128ES1_Li4ELb1ELb1ELi16E",
            r"decode_split_kernelINS_6bf16_tELi128ES1_Lb1ELi16E"]


@pytest.mark.parametrize("pattern", PATTERNS)
def test_tile_loop_keeps_loads_in_flight(asm16, pattern):
    found = list(_kernels(asm16, pattern))
    assert found, f"no kernel matches {pattern}"
    for nm, body in found:
        loops = list(_tile_loops(body))
        assert loops, f"{nm}: no tile loop reads through a buffer resource"
        for waits, ld in loops:
            assert "vmcnt(0)" not in " ".join(waits), (nm, waits, ld)
            assert ld.endswith(" nt"), (nm, ld)   # the non-temporal hint


@pytest.mark.parametrize("src", ["decode.hip", "decode_bs8.hip", "decode_bs32.hip"])
def test_decode_kernels_keep_tiles_in_registers(src, asm16):
    """No decode kernel uses scratch memory: tiles, queries and the new token's rows stay in
    registers (a select between two such arrays, for one, would make the compiler keep
    both in scratch and load through a pointer, with a wait for every tile). Every block
    size's translation unit, the whole-block kernels included."""
    asm = asm16 if src == "decode.hip" else _asm(src)
    names = re.findall(r"^(_ZN3pkv\w*decode\w+):", asm, re.M)
    assert names
    for nm in names:
        i = asm.index(nm + ":")
        m = re.search(r"ScratchSize: (\d+)", asm[i:])
        assert m and m.group(1) == "0", (nm, m.group(1) if m else None)
