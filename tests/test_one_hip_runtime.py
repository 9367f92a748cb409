"""One HIP runtime per process (no GPU needed).

PyTorch's ROCm build brings its own libamdhip64; importing the binding must not
map a second copy next to it, whatever the import order, because two HIP
runtimes in one process each open the device and the second can fail to.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
import sys
sys.path.insert(0, {root!r})
{imports}
maps = open('/proc/self/maps').read().splitlines()
paths = sorted(set(l.split()[-1] for l in maps if 'libamdhip64' in l))
print(len(paths), paths)
"""


def _hip_runtimes(imports: str):
    code = PROBE.format(root=ROOT, imports=imports)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    return out.stdout.strip()


def test_binding_imported_before_torch():
    assert _hip_runtimes("import decode_attention_paged_04_amd\nimport torch").startswith("1 ")


def test_binding_imported_after_torch():
    assert _hip_runtimes("import torch\nimport decode_attention_paged_04_amd").startswith("1 ")
