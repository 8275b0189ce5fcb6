"""Properties of the built GPU code (CPU only): the gfx950 code objects of
this repository's own build, taken out of the objects `build()` leaves in
_build/ and disassembled with ROCm's LLVM tools.

Each property guards against a compiler outcome that costs speed without
changing any result, so no parity test would notice it:
  * no kernel makes a function call (HIP's threadIdx/blockIdx compile to
    calls into the device library under this build's floating-point flags,
    and each callee starts by waiting for every outstanding memory
    operation);
  * the forward's main loop waits for no vector-memory operation: its K/V
    copies run ahead into the rings, and a wait the compiler places for a
    load it tracks (vmcnt counts the copies too) would make every tile
    position wait for copies started in the same position;
  * the kernels the benchmark times keep everything in registers (no
    scratch memory);
  * the matrix-core probe's loop holds its products and the loop counter
    and nothing else (the compiler is free to recompute the operands inside
    the loop instead of holding them, which would measure the vector ALU);
  * the 8-bit forward zeroes no register for its probability conversions
    (each P word is built by two 2-byte conversions; a zeroed start costs a
    vector move per word on a loop the vector ALU bounds);
  * the forward's K/V copies are non-temporal exactly in the instantiations
    for single-reader grids (a decode step), where that streams faster, and
    plain everywhere else, where it would evict tiles other workgroups read.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build", "attn")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def code_object(name, tmp):
    """The gfx950 code object inside _build/attn/<name>.o."""
    obj = os.path.join(BUILD, name + ".o")
    if not os.path.exists(obj):
        pytest.skip(f"{obj} is not built (run build() first)")
    for tool in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump", "llvm-readelf"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip(f"{tool} not available")
    fb, junk, co = (os.path.join(tmp, name + s) for s in (".fatbin", ".host.o", ".co"))
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fb}", obj, junk],
                   check=True, capture_output=True)
    subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                    f"--targets={TARGET}", f"--input={fb}", f"--output={co}"], check=True, capture_output=True)
    return co


def kernels(co):
    """{kernel symbol: [instruction, ...]} from the disassembly."""
    out = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--no-show-raw-insn", "--no-leading-addr",
                          co], check=True, capture_output=True, text=True).stdout
    ks, cur = {}, None
    for line in out.splitlines():
        m = re.match(r"^<(\S+)>:$", line)
        if m:
            cur = ks.setdefault(m.group(1), []) if "kernel" in m.group(1) else None
            continue
        if cur is not None and line.startswith("\t"):
            cur.append(line.strip().split("//")[0].strip())
    return ks


def metadata(co):
    """{kernel symbol: {field: int}} from the code object's notes."""
    out = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", co], check=True, capture_output=True,
                         text=True).stdout
    md = {}
    for blk in out.split("  - .")[1:]:
        m = re.search(r"\.name:\s+(\S+)", blk)
        if not m:
            continue
        md[m.group(1)] = {k: int(v) for k, v in re.findall(r"\.(\w+):\s+(\d+)\s*$", blk, flags=re.M)}
    return md


@pytest.fixture(scope="module")
def objects(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("code"))
    return {n: code_object(n, tmp) for n in ("attn_fwd", "attn_decode", "attn_bwd", "attn_std", "attn_probe")}


def test_tools_found():
    assert shutil.which("llvm-objdump", path=LLVM)


def test_no_kernel_makes_a_call(objects):
    for name, co in objects.items():
        ks = kernels(co)
        assert ks, name
        for k, ins in ks.items():
            calls = [i for i in ins if i.startswith(("s_swappc", "s_call"))]
            assert not calls, f"{k} makes {len(calls)} call(s)"


def segments(ins):
    """Straight-line runs of instructions between branches."""
    seg = []
    for i in ins:
        seg.append(i)
        if i.startswith(("s_cbranch", "s_branch", "s_setpc", "s_endpgm")):
            yield seg
            seg = []
    if seg:
        yield seg


def test_forward_loop_waits_for_no_memory_operation(objects):
    """Every run of instructions holding a whole position's products (16
    32x32x16 products with 16-bit operands, 8 32x32x64 ones with 8-bit
    operands) -- the main loop's body -- contains no vmcnt wait; the waits
    for the copies sit only at the barriers between positions."""
    ks = {k: v for n in ("attn_fwd", "attn_decode") for k, v in kernels(objects[n]).items() if "fwd_kernel" in k}
    assert len(ks) >= 38 + 22
    for k, ins in ks.items():
        nmm = 8 if "fp8" in k else 16
        bodies = [s for s in segments(ins) if sum(i.startswith("v_mfma") for i in s) >= nmm]
        assert len(bodies) >= 10, f"{k}: {len(bodies)} loop bodies found"
        for b in bodies:
            waits = [i for i in b if i.startswith("s_waitcnt") and "vmcnt" in i]
            assert not waits, f"{k}: a loop body waits for memory: {waits}"


BENCHED = [
    # the benchmark's step (7B layer, bf16, d = 128, causal) and the other
    # workloads' kernels
    r"fwd_kernelIDF16bDF16bLi128ELb1ELb0E",
    r"fwd_kernelIDF16_DF16_Li64ELb0ELb0E",
    r"dq_kernelIDF16bDF16bLi128ELb1ELb0E",
    r"dkdv_kernelIDF16bDF16bLi128ELb1ELb0E",
    r"fwd_kernelINS_7fp8e4m3EDF16bLi128ELb1ELb0E",
]


def test_benchmarked_kernels_use_no_scratch(objects):
    md = {}
    for co in objects.values():
        md.update(metadata(co))
    for pat in BENCHED:
        hits = [k for k in md if re.search(pat, k)]
        assert hits, pat
        for k in hits:
            assert md[k].get("private_segment_fixed_size", 0) == 0, (k, md[k])
            assert md[k].get("vgpr_spill_count", 0) == 0, (k, md[k])


def test_every_forward_and_standard_kernel_uses_no_scratch(objects):
    for name in ("attn_fwd", "attn_decode", "attn_std"):
        for k, m in metadata(objects[name]).items():
            assert m.get("private_segment_fixed_size", 0) == 0, (k, m)


def test_dropout_dq_loop_uses_no_scratch(objects):
    """The dq kernel with dropout (bf16, d = 128, causal) forms its dP seed
    before each chain instead of holding it, so its loop keeps everything in
    registers (holding the seed cost 22 scratch accesses per key block)."""
    ks = kernels(objects["attn_bwd"])
    hits = [k for k in ks if re.search(r"dq_kernelIDF16bDF16bLi128ELb1ELb1E", k)]
    assert hits
    for k in hits:
        for seg in segments(ks[k]):
            if sum(i.startswith("v_mfma") for i in seg) >= 8:
                assert not [i for i in seg if i.startswith("scratch_")], k


def test_probe_loop_is_products_only(objects):
    ks = {k: v for k, v in kernels(objects["attn_probe"]).items() if "mfma_probe_kernel" in k}
    assert len(ks) == 1
    (ins,) = ks.values()
    loops = [s for s in segments(ins) if sum(i.startswith("v_mfma") for i in s) == 16]
    assert len(loops) == 1
    body = loops[0]
    # the loop starts after the last accumulator initialisation
    start = max(n for n, i in enumerate(body) if not i.startswith(("v_mfma", "s_"))) + 1
    rest = [i.split()[0] for i in body[start:] if not i.startswith("v_mfma")]
    assert set(rest) <= {"s_nop", "s_add_i32", "s_sub_i32", "s_cmp_lg_u32", "s_cmp_eq_u32", "s_cbranch_scc1",
                         "s_cbranch_scc0"}, rest
    assert sum(i.startswith("v_mfma_f32_32x32x16_bf16") for i in body[start:]) == 16
    md = metadata(objects["attn_probe"])
    (m,) = [v for k, v in md.items() if "mfma_probe_kernel" in k]
    assert m.get("private_segment_fixed_size", 0) == 0 and m.get("vgpr_spill_count", 0) == 0


def test_fp8_probability_words_start_from_no_zeroed_register(objects):
    """In every run of instructions that converts 8-bit probabilities, no
    register a conversion writes was set to 0 first (an earlier form of the
    kernel did so for every P word: 80 such moves per kernel)."""
    ks = {k: v for n in ("attn_fwd", "attn_decode") for k, v in kernels(objects[n]).items()
          if "fwd_kernel" in k and "fp8" in k}
    assert len(ks) >= 12
    for k, ins in ks.items():
        ncvt = 0
        for seg in segments(ins):
            cvt = [i for i in seg if i.startswith("v_cvt_pk_fp8_f32")]
            if not cvt:
                continue
            ncvt += len(cvt)
            dests = {i.split()[1].rstrip(",") for i in cvt}
            zeroed = [i for i in seg if re.fullmatch(r"v_mov_b32_e32 v\d+, 0", i) and i.split()[1].rstrip(",") in dests]
            assert not zeroed, (k, zeroed[:4])
        assert ncvt >= 16, k


def test_forward_copies_are_non_temporal_only_for_single_reader_grids(objects):
    def copies(ins):
        c = [i for i in ins if i.startswith("buffer_load_dwordx4") and i.endswith(" lds")]
        return sum(" nt lds" in i for i in c), sum(" nt lds" not in i for i in c)

    for name, want_nt in (("attn_fwd", False), ("attn_decode", True)):
        ks = {k: v for k, v in kernels(objects[name]).items() if "fwd_kernel" in k}
        assert ks, name
        for k, ins in ks.items():
            nt, plain = copies(ins)
            assert nt + plain >= 8, k
            assert (plain == 0) if want_nt else (nt == 0), (name, k, nt, plain)
