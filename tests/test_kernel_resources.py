"""Every kernel compiles for gfx950 without a private (scratch) segment and
without reading the dispatch packet.  Either would come from a private array
indexed at run time: the compiler then places it in scratch, or in LDS
addressed by the flat thread id, which every workgroup reads from the
dispatch packet at its start (host-resident queue memory, a multi-microsecond
stall under load).  CPU only: compiles to assembly, launches nothing."""
import os
import re
import shutil
import subprocess

import pytest

from linear_attention_recurrent_gdn_amd import _build

pytestmark = pytest.mark.skipif(shutil.which(_build.hipcc()) is None and not os.path.exists(_build.hipcc()),
                                reason="hipcc not available")


def kernel_descriptors(asm: str):
    out = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm, re.S):
        fields = dict(re.findall(r"\.(amdhsa_\w+) (\S+)", m.group(2)))
        out[m.group(1)] = fields
    return out


@pytest.mark.parametrize("src", [os.path.basename(p) for p in _build.sources()])
def test_no_scratch_no_dispatch_packet(src, tmp_path):
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    out = tmp_path / (src + ".s")
    cmd = [_build.hipcc(), *flags, "--cuda-device-only", "-S", f"-I{_build.INCLUDE}", f"-I{_build.CSRC}",
           os.path.join(_build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kds = kernel_descriptors(out.read_text())
    if src != "lq_api.hip":  # the API file is host code
        assert kds, f"no kernels found in {src}"
    for name, f in kds.items():
        assert f.get("amdhsa_private_segment_fixed_size") == "0", (name, f.get("amdhsa_private_segment_fixed_size"))
        assert f.get("amdhsa_user_sgpr_dispatch_ptr") == "0", name
