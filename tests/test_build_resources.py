"""Register budget of the timed chunk loops (host only: compiles device code to
assembly with hipcc, runs nothing).

A spilled value that the compiler reloads inside a chunk loop comes with a
`s_waitcnt vmcnt(0)`, which also waits for the next chunk's tile copies or the
previous chunk's output stores in flight: the per-channel gate's output pass
once lost 6 % that way.  These instances must keep every value in registers
(no scratch)."""
import os
import re
import shutil
import subprocess

import pytest

from chunkwise_recurrence_amd.build import COMMON, HIPCC

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunkwise_recurrence_amd", "csrc")

# (translation unit, mangled-name fragment of the instance): the output passes
# of the retnet_bf16 (per-head decay) and gla_bf16 (per-channel gate) workloads,
# and the delta rule's column pass (its compute waves hold 250 registers)
INSTANCES = [
    ("la_chunk_stripe_dk128_c1", "chunk_stripe_kernelILi128ELi4ELi2ELi64ELi1ELb0ELb0ELb0E"),
    ("la_chunk_stripe_dk128_c3", "chunk_stripe_kernelILi128ELi4ELi2ELi64ELi3ELb0ELb0ELb0E"),
    ("la_delta", "delta_chunk_cols_kernelILi128EE"),
    ("la_delta", "delta_chunk_cols_kernelILi64EE"),
]


def _kernel_fields(asm: str):
    """{kernel symbol: {amdhsa field: value}} from a device assembly listing."""
    out, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"\s*\.amdhsa_kernel (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.match(r"\s*\.amdhsa_(\w+) (\d+)", line)
        if m and cur is not None:
            out[cur][m.group(1)] = int(m.group(2))
        if line.strip() == ".end_amdhsa_kernel":
            cur = None
    return out


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    """Device assembly of the translation units above, compiled in parallel."""
    from concurrent.futures import ThreadPoolExecutor
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("asm")
    args = [a for a in COMMON if a != "-fPIC"]

    def compile_unit(unit):
        out = d / (unit + ".s")
        r = subprocess.run([HIPCC, *args, "--cuda-device-only", "-S",
                            os.path.join(CSRC, unit + ".hip"), "-o", str(out)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return unit, _kernel_fields(out.read_text())

    units = sorted({u for u, _ in INSTANCES})
    with ThreadPoolExecutor(len(units)) as ex:
        return dict(ex.map(compile_unit, units))


@pytest.mark.parametrize("unit,fragment", INSTANCES)
def test_output_pass_has_no_scratch(listings, unit, fragment):
    fields = listings[unit]
    hits = {k: v for k, v in fields.items() if fragment in k}
    assert len(hits) == 1, sorted(fields)
    (name, f), = hits.items()
    assert f["private_segment_fixed_size"] == 0, \
        f"{name}: {f['private_segment_fixed_size']} bytes of scratch"
