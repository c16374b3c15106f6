"""The matrix-core rate probe (a measurement helper of the benchmark, not part of
the method) runs through the C ABI and keeps its work: the checksums are
deterministic and not all zero."""
from __future__ import annotations

import pytest

torch = pytest.importorskip("torch")
import mixed_precision_int8_amd as m8  # noqa: E402

pytestmark = pytest.mark.gpu


def test_probe_runs_and_is_deterministic():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[case] probe blocks=8 iters=50", flush=True)
    outs = []
    for _ in range(2):
        out = torch.zeros(8 * 256, dtype=torch.int32, device="cuda")
        ops = m8.llmint8_probe_mfma_i8(8, 50, out)
        torch.cuda.synchronize()
        outs.append(out.cpu())
    assert ops == 8 * 4 * 50 * 4 * 65536
    assert torch.equal(outs[0], outs[1])
    assert bool((outs[0] != 0).any())
