"""Properties of the gfx950 code the matrix-core kernels compile to (CPU only:
hipcc cross-compiles to assembly, nothing runs).

* No wait for all outstanding vector-memory operations right next to an LDS
  read, in the kernels that pipeline their operand copies (forward NA,
  projection GEMM).  They read one LDS buffer while the copy of the next
  block or chunk fills the other; when the compiler cannot tell the two
  buffers apart (it loses track once an address is derived through too many
  steps), it makes the read wait for that copy, which stalls every tile on
  the next block's loads.  (The fused block kernel loads its x operands into
  registers for its own next products; waits for those are expected, and so
  is a full wait that no further load follows before the loop branches back
  or the kernel ends: the last steps of a unit need every load in flight.)
* No vector-register spills and no scratch memory, in every matrix-core
  kernel: forward, projection, fused block, backward.  (Scalar registers may
  spill into vector-register lanes, which costs no memory traffic.)
* No LDS access through flat (generic) addresses.
* No packed-FP32 arithmetic (the build disables it).
"""
import os
import re
import shutil
import subprocess

import pytest

from vision_transformer_local_amd import build as B

SOURCES = ["na2d_mfma.hip", "na2d_dense.hip", "na2d_stream.hip", "na2d_linear.hip",
           "na2d_block.hip", "na2d_backward_mfma.hip"]
PIPELINED = {"na2d_mfma.hip", "na2d_dense.hip", "na2d_stream.hip", "na2d_linear.hip"}
KERNEL = re.compile(r"^(_ZN4na2d12_GLOBAL__N_1\d+\w*(?:mfma_kernel|block_fused_kernel|"
                    r"bwd_query_mfma|bwd_key_mfma)\S*):", re.M)


def _asm(src, tmp_path):
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [B.HIPCC] + [f for f in B.COMMON if f not in ("-fPIC",)] + [
        "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(asm):
    for m in KERNEL.finditer(asm):
        end = asm.index(".Lfunc_end", m.end())
        yield m.group(1), asm[m.end():end].split("\n")


def _loads_follow(ops, i):
    """Whether a vector-memory load is issued after ops[i] before a branch
    back to an earlier label (the loop's next iteration) or the end of the
    kernel, scanning the code in its layout order."""
    labels = {}
    for j, op in enumerate(ops):
        if op.endswith(":"):
            labels[op[:-1]] = j
    for op in ops[i + 1:]:
        mnem = op.split()[0]
        if mnem.startswith(("buffer_load", "global_load")):
            return True
        if mnem == "s_endpgm":
            return False
        if mnem.startswith(("s_branch", "s_cbranch")):
            target = op.split()[-1]
            if labels.get(target, len(ops)) <= i:
                return False
    return False


def _metadata(asm, name):
    meta = asm[asm.index(".amdgpu_metadata"):]
    for block in meta.split("- .agpr_count")[1:]:
        if name in block:
            return block
    raise AssertionError("no metadata for " + name)


@pytest.mark.parametrize("src", SOURCES)
def test_kernel_code_properties(src, tmp_path):
    asm = _asm(src, tmp_path)
    kernels = list(_kernels(asm))
    assert kernels, "no kernels found in " + src
    for name, body in kernels:
        ops = [l.split(";")[0].strip() for l in body]
        ops = [o for o in ops if o and (not o.startswith(".") or o.startswith(".LBB"))]
        for i, op in enumerate(ops):
            if op.endswith(":"):
                continue
            if src in PIPELINED and re.fullmatch(r"s_waitcnt vmcnt\(0\)", op):
                near = [o.split()[0] for o in ops[max(0, i - 2):i + 3]]
                assert not (any(o.startswith("ds_read") for o in near)
                            and _loads_follow(ops, i)), (
                    "%s: full vector-memory wait next to an LDS read: %s" % (name, near))
            mnem = op.split()[0]
            assert not mnem.startswith("flat_"), "%s: flat access %s" % (name, op)
            assert mnem not in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"), (
                "%s: packed fp32 %s" % (name, op))
        meta = _metadata(asm, name)
        for key in (".vgpr_spill_count", ".private_segment_fixed_size"):
            m = re.search(re.escape(key) + r":\s+(\d+)", meta)
            assert m is not None, key
            assert int(m.group(1)) == 0, "%s: %s = %s" % (name, key, m.group(1))
