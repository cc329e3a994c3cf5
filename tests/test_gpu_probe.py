"""The measurement probes bench.py reads its ceilings from: the copy moves every byte
(temporal, nontemporal and write-through stores), and the streaming read of a zero-filled source never
writes its sink."""

import numpy as np
import pytest

from gpu_helpers import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 3 << 20])
@pytest.mark.parametrize("policy", [0, 1, 2])
def test_probe_copy_and_read(nbytes, policy):
    import torch
    from combine_router_softmax_expert_amd import binding as B

    log(f"[probe] {nbytes} bytes policy={policy}")
    src = torch.from_numpy(np.random.default_rng(nbytes).integers(0, 256, nbytes, dtype=np.uint8)).cuda()
    dst = torch.full((nbytes + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    B.moe_probe_copy(src, dst[:nbytes], policy)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    B.moe_probe_read(torch.zeros(nbytes, dtype=torch.uint8, device="cuda"), sink, policy == 1)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert (dst[nbytes:] == 0x5A).all()          # nothing past the end
    assert (sink == 0).all()
