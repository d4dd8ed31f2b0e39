"""Code-generation checks of the decode and prefill kernels' inner loops (CPU only: hipcc
cross-compiles).

The decode kernel keeps two 32-key steps in registers: the next step's K/V loads are meant to
be in flight while the current step computes.  Vector-memory waits count in issue order, so a
wait for all loads (``s_waitcnt vmcnt(0)``) inside the step loop drains the other register set
too and leaves one step loading at a time.  That happened when the block-table lookups were
vector loads (the compiler cannot prove a plain table pointer unwritten once the kernel stores
its outputs): every lookup's use waited for every load in flight, and the decode after the
chunked prefill (8 sequences x 4096 keys) ran 7% slower, with every output still correct.  These
tests compile ``decode.hip`` for gfx950 and check the step loop of the head-size-128 kernels that
the benchmarks time: no full wait, the block-table lookups are scalar loads, and no single-dword
vector load (the K/V loads are 8 or 16 bytes wide).  The prefill kernel's tile loop reads the block
table the same way (its full waits are its own, for each wave's tile copies before the barrier):
there the checks are the scalar lookups and the absence of single-dword vector loads.
"""

import os
import re
import subprocess

import pytest

from paged_attention_block_amd import build as pa_build

CSRC = os.path.join(os.path.dirname(pa_build.__file__), "csrc")

# decode_bf16_kernel<D, ALIBI, CASCADE, FP8, FUSED> instantiations, head size 128
KERNELS = {
    "plain": "_ZN2pa18decode_bf16_kernelILi128ELb0ELb0ELb0ELb0EEEvNS_10DecodeArgsE",
    "alibi": "_ZN2pa18decode_bf16_kernelILi128ELb1ELb0ELb0ELb0EEEvNS_10DecodeArgsE",
    "fp8": "_ZN2pa18decode_bf16_kernelILi128ELb0ELb0ELb1ELb0EEEvNS_10DecodeArgsE",
    "cascade": "_ZN2pa18decode_bf16_kernelILi128ELb0ELb1ELb0ELb0EEEvNS_10DecodeArgsE",
}


def _hipcc():
    try:
        return pa_build.hipcc()
    except RuntimeError:
        return None


def _device_asm(tmp_path_factory, source):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / (source + ".s"))
    cmd = [cc, *pa_build.FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, source), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    return _device_asm(tmp_path_factory, "decode.hip")


@pytest.fixture(scope="module")
def prefill_asm(tmp_path_factory):
    return _device_asm(tmp_path_factory, "prefill.hip")


def _functions(asm):
    """{symbol: body} for every function of the assembly listing."""
    out = {}
    for part in re.split(r"\n(?=_Z\S+:)", asm):
        m = re.match(r"(_Z\S+):", part)
        if m:
            out[m.group(1)] = part
    return out


def _loops(body, depth):
    """{header: [instructions]} for the loops of a function at one nesting depth, from the
    compiler's loop comments (a header block is marked 'Loop Header: Depth=<depth>', the other
    blocks of the loop 'in Loop: Header=<header> Depth=<depth>')."""
    blocks, cur = [], None
    for line in body.split("\n"):
        m = re.match(r"\.(LBB\d+_\d+):(.*)", line)
        if m:
            cur = [m.group(1)[1:], m.group(2), []]
            blocks.append(cur)
        elif cur is not None:
            if line.strip().startswith(";"):
                cur[1] += line
            elif line.strip():
                cur[2].append(line.strip())
    loops = {b[0]: list(b[2]) for b in blocks if f"Loop Header: Depth={depth}" in b[1]}
    for b in blocks:
        m = re.search(rf"in Loop: Header=(BB\d+_\d+) Depth={depth}\b", b[1])
        if m and m.group(1) in loops:
            loops[m.group(1)].extend(b[2])
    return loops


def _step_loop(asm, symbol):
    fns = _functions(asm)
    assert symbol in fns, f"{symbol} not in the listing"
    loops = _loops(fns[symbol], 3)
    assert loops, f"no innermost loop found in {symbol}"
    # the step loop is the innermost loop that issues the K/V loads
    return max(loops.values(), key=lambda ins: sum(i.startswith("global_load_dwordx") for i in ins))


@pytest.mark.parametrize("kind", sorted(KERNELS))
def test_step_loop_keeps_loads_in_flight(decode_asm, kind):
    ins = _step_loop(decode_asm, KERNELS[kind])
    kv_loads = [i for i in ins if i.startswith("global_load_dwordx")]
    assert len(kv_loads) >= 16, f"{kind}: expected the K/V loads of two steps in the loop, got {len(kv_loads)}"
    drains = [i for i in ins if i.startswith("s_waitcnt") and re.search(r"\bvmcnt\(0\)", i)]
    assert not drains, f"{kind}: the step loop waits for every load in flight: {drains}"
    assert any(i.startswith("s_load_dword") for i in ins), f"{kind}: the block-table lookups are not scalar loads"
    dword = [i for i in ins if re.match(r"global_load_dword\s", i)]
    assert not dword, f"{kind}: single-dword vector loads in the step loop (table lookups?): {dword}"


def test_prefill_tile_loop_reads_the_table_with_scalar_loads(prefill_asm):
    fns = {k: v for k, v in _functions(prefill_asm).items() if "prefill_bf16_kernelILi128" in k}
    assert fns, "no head-size-128 prefill kernel in the listing"
    for symbol, body in fns.items():
        loops = [ins for d in (1, 2, 3) for ins in _loops(body, d).values()]
        tile = [ins for ins in loops if any(i.startswith("v_mfma") for i in ins)]
        assert tile, f"{symbol}: no loop with MFMAs"
        ins = max(tile, key=lambda x: sum(i.startswith("v_mfma") for i in x))
        assert any(i.startswith("s_load_dword") for i in ins), f"{symbol}: the block-table lookups are not scalar loads"
        dword = [i for i in ins if re.match(r"global_load_dword\s", i)]
        assert not dword, f"{symbol}: single-dword vector loads in the tile loop: {dword}"
