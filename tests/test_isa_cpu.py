"""CPU-only: the device code in libbqd.so, disassembled.

Every code object bundled into the library is a gfx950 one, and its
instructions stay inside two rules the kernels are written to:
- no packed fp32 VALU arithmetic (the packed add, multiply and fused
  multiply-add on float pairs): the build turns the target feature off, and no
  source writes them by hand;
- the only scalar-unit memory instructions are loads (kernel arguments,
  uniform values) and the real-time counter reads: nothing is written through
  the scalar data cache.  Every scalar mnemonic must match the allowlist below,
  so anything outside it fails the test and has to be looked at.
"""
import os
import re
import struct
import subprocess

import pytest

import bit_quantized_decode_amd as bqd

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
OBJDUMP = os.path.join(ROCM, "llvm", "bin", "llvm-objdump")
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

# scalar ALU, compare, branch and program-control forms, and scalar loads
SCALAR_OK = re.compile(
    r"s_(?:add|addc|sub|subb|and|or|xor|andn2|orn2|nand|nor|xnor|not|mov|movk|cmov|cmovk|cmp|cmpk|"
    r"cselect|lshl|lshr|ashr|lshl\d_add|bfe|bfm|bcnt0|bcnt1|ff0|ff1|flbit|brev|abs|absdiff|min|max|"
    r"mul|mul_hi|mulk|addk|sext|bitcmp0|bitcmp1|bitset0|bitset1|pack_ll|pack_lh|pack_hh|"
    r"branch|cbranch|barrier|waitcnt|nop|endpgm|sleep|setprio|getpc|setpc|swappc|set_gpr_idx|"
    r"and_saveexec|or_saveexec|xor_saveexec|andn2_saveexec|orn2_saveexec|nand_saveexec|"
    r"nor_saveexec|xnor_saveexec|andn1_saveexec|orn1_saveexec|andn1_wrexec|andn2_wrexec|"
    r"load|buffer_load|memtime|memrealtime|getreg|setreg|sendmsg|trap|icache_inv|wqm|quadmask|"
    r"movreln|movrels|bitreplicate|rfe|setkill|denorm_mode|round_mode|inst_prefetch|"
    r"code_end|sethalt|ttracedata|incperflevel|decperflevel|dcache_inv)(?:_\w+)?$")
PACKED_F32 = {"v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"}


def _code_objects(path):
    """(target id, bytes) of every entry of every offload bundle in the file."""
    data = open(path, "rb").read()
    out, pos = [], 0
    while True:
        start = data.find(BUNDLE_MAGIC, pos)
        if start < 0:
            return out
        (n,) = struct.unpack_from("<Q", data, start + len(BUNDLE_MAGIC))
        p = start + len(BUNDLE_MAGIC) + 8
        for _ in range(n):
            off, size, id_len = struct.unpack_from("<QQQ", data, p)
            p += 24
            target = data[p:p + id_len].decode()
            p += id_len
            out.append((target, data[start + off:start + off + size]))
        pos = start + 1


@pytest.fixture(scope="module")
def mnemonics(tmp_path_factory):
    assert os.path.exists(bqd.LIB_PATH), "libbqd.so is not built"
    objs = [(t, b) for t, b in _code_objects(bqd.LIB_PATH) if "amdgcn" in t]
    assert objs, "no device code objects in libbqd.so"
    for target, _ in objs:
        assert target.endswith("--gfx950"), target
    seen = set()
    d = tmp_path_factory.mktemp("isa")
    for k, (_, blob) in enumerate(objs):
        f = d / f"{k}.co"
        f.write_bytes(blob)
        r = subprocess.run([OBJDUMP, "-d", str(f)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        for line in r.stdout.splitlines():
            m = re.match(r"\s+([sv]_\w+)", line)
            if m:
                seen.add(m.group(1))
    return seen


def test_device_code_disassembles(mnemonics):
    assert any(m.startswith("v_mfma") for m in mnemonics)  # the batch kernels' products
    assert "s_endpgm" in mnemonics


def test_no_packed_fp32_arithmetic(mnemonics):
    assert not (mnemonics & PACKED_F32), sorted(mnemonics & PACKED_F32)


def test_scalar_unit_only_loads_memory(mnemonics):
    odd = sorted(m for m in mnemonics if m.startswith("s_") and not SCALAR_OK.match(m))
    assert not odd, odd
