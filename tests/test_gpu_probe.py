"""The benchmark's streaming probe kernels (libkvprobe.so) do what their
ceilings claim: the copy reproduces its source, the fill writes its value,
at every variant and at sizes that leave a ragged last workgroup."""

import pytest
import torch

from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant", [0, 1, 2, 3])
def test_probe_copy_fill_read(variant):
    import bench
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    probes = bench.Probes(stream)
    for n in (16, 4096 + 48, (1 << 20) + 16 * 37):
        say("probe variant", variant, "bytes", n)
        src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV)
        dst = torch.zeros(n + 64, dtype=torch.uint8, device=DEV)
        probes.copy(src, dst[:n], variant)
        probes.read(src, variant)
        torch.cuda.synchronize()
        assert torch.equal(dst[:n], src) and torch.all(dst[n:] == 0)
        probes.fill(dst[:n], variant, 0x01020304)
        torch.cuda.synchronize()
        assert torch.equal(dst[:n].view(torch.int32), torch.full((n // 4,), 0x01020304, dtype=torch.int32,
                                                                  device=DEV))
        assert torch.all(dst[n:] == 0)
