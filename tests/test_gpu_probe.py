"""The benchmark's matrix-core rate probe (libllmint8_probe.so, a measurement
helper built beside the product library, not part of it) keeps its work: the
checksums are deterministic and not all zero."""
from __future__ import annotations

import pytest

torch = pytest.importorskip("torch")
import bench  # noqa: E402

pytestmark = pytest.mark.gpu


def test_probe_runs_and_is_deterministic():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[case] probe blocks=8 iters=50", flush=True)
    stream = torch.cuda.current_stream()
    outs = []
    for _ in range(2):
        out = torch.zeros(8 * 256, dtype=torch.int32, device="cuda")
        ops = bench.probe_mfma_i8(8, 50, out, stream)
        torch.cuda.synchronize()
        outs.append(out.cpu())
    assert ops == 8 * 4 * 50 * 4 * 65536
    assert torch.equal(outs[0], outs[1])
    assert bool((outs[0] != 0).any())
