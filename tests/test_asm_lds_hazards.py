"""No inline-asm LDS read of the device code is left in flight.

Compiles every device source to gfx950 assembly with the library's own flags
and checks that each inline-asm statement holding an LDS read waits for it
(s_waitcnt lgkmcnt(0)) before it ends, and that no instruction touches a
register an asm read has not yet filled; the two checks are exercised on
hand-written snippets first.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from mixture_experts_ffn_06_amd import build as B

from tests.asm_lds_hazards import scan, unwaited_reads

SAFE = """
_Zkern:
	;;#ASMSTART
	ds_read_b128 v[4:7], v1 offset:0
	;;#ASMEND
	;;#ASMSTART
	ds_read_b128 v[8:11], v1 offset:16
	;;#ASMEND
	v_add_u32_e32 v2, v3, v12
	s_waitcnt lgkmcnt(0)
	v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]
	s_endpgm
"""

# a copy of an in-flight destination before the wait
HAZARD_COPY = SAFE.replace("v_add_u32_e32 v2, v3, v12", "v_accvgpr_write_b32 a9, v6")
# an in-flight destination reused as the next read's address
HAZARD_ADDR = SAFE.replace("ds_read_b128 v[8:11], v1 offset:16", "ds_read_b128 v[8:11], v5 offset:16")
# a wait for only some of the reads does not clear the most recent ones
HAZARD_PARTIAL = SAFE.replace("s_waitcnt lgkmcnt(0)", "s_waitcnt lgkmcnt(1)")
# ... but it does clear the older ones (reads complete in order)
SAFE_PARTIAL = SAFE.replace("v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]",
                            "v_mov_b32 v20, v4").replace("s_waitcnt lgkmcnt(0)", "s_waitcnt lgkmcnt(1)")


def test_scanner_on_snippets():
    h, n, f = scan(SAFE)
    assert (h, n, f) == ([], 2, 1)
    h, _, _ = scan(HAZARD_COPY)
    assert [x[3] for x in h] == [("v", 6)]
    h, _, _ = scan(HAZARD_ADDR)
    assert [x[3] for x in h] == [("v", 5)]
    h, _, _ = scan(HAZARD_PARTIAL)
    assert {x[3] for x in h} == {("v", r) for r in range(8, 12)}
    h, _, _ = scan(SAFE_PARTIAL)
    assert h == []


def _asm(src: str) -> str:
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    r = subprocess.run([B.HIPCC, *flags, *B.file_flags(src), "-x", "hip", "--cuda-device-only", "-S",
                        os.path.join(B.CSRC, src), "-o", "-"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stderr}")
    return r.stdout


# an asm statement that issues its reads and waits for them
WAITED = """
_Zkern:
	;;#ASMSTART
	ds_read_b32 v4, v1 offset:0
	ds_read_b32 v5, v1 offset:64
	s_waitcnt lgkmcnt(0)
	;;#ASMEND
	v_add_u32_e32 v2, v4, v5
	s_endpgm
"""
# the same reads with the wait in a later statement
SPLIT = WAITED.replace("\ts_waitcnt lgkmcnt(0)\n\t;;#ASMEND\n",
                       "\t;;#ASMEND\n\t;;#ASMSTART\n\ts_waitcnt lgkmcnt(0)\n\t;;#ASMEND\n")
# a wait before the last read does not cover it
EARLY = WAITED.replace("\tds_read_b32 v5, v1 offset:64\n\ts_waitcnt lgkmcnt(0)\n",
                       "\ts_waitcnt lgkmcnt(0)\n\tds_read_b32 v5, v1 offset:64\n")


def test_unwaited_reads_on_snippets():
    assert unwaited_reads(WAITED) == ([], 1)
    bad, n = unwaited_reads(SPLIT)
    assert n == 1 and len(bad) == 1
    bad, n = unwaited_reads(EARLY)
    assert n == 1 and len(bad) == 1
    assert unwaited_reads(SAFE)[0] and unwaited_reads(SAFE)[1] == 2


@pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not installed")
def test_device_code_has_no_asm_lds_read_in_flight():
    srcs = sorted(f for f in os.listdir(B.CSRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(len(srcs)) as ex:
        texts = list(ex.map(_asm, srcs))
    n_asm = {}
    for src, text in zip(srcs, texts):
        hazards, n_reads, n_fn = scan(text)
        bad, n_stmt = unwaited_reads(text)
        assert n_fn > 0, src
        assert not bad, f"{src}: {[(f, ln) for f, ln, _ in bad[:5]]}"
        assert not hazards, f"{src}: {hazards[:5]}"
        n_asm[src] = n_stmt
    # the ring GEMMs read LDS with ordinary loads only; the MX streaming
    # kernel's grouped reads are asm statements with their own wait
    assert n_asm["gateup.hip"] == 0 and n_asm["grouped.hip"] == 0
    assert n_asm["small_m.hip"] > 0
