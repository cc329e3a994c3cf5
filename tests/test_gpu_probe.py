"""The measurement probes bench.py reads its ceilings from: the copy moves every byte
(temporal, nontemporal and write-through stores), the row gather puts every row where its permutation says
(out-of-range entries clamped), and the streaming read of a zero-filled source never writes its sink."""

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


@pytest.mark.parametrize("rows,row_bytes", [(1, 16), (577, 14336), (300, 4096 + 48),
                                            (9400, 14336)])   # 135 MB: the streaming shape for nontemporal gathers
@pytest.mark.parametrize("policy", [0, 1, 2])
def test_probe_gather(rows, row_bytes, policy):
    import torch
    from combine_router_softmax_expert_amd import binding as B

    log(f"[probe] gather {rows} rows of {row_bytes} bytes policy={policy}")
    rng = np.random.default_rng(rows * 7 + policy)
    src_rows = rows + 3
    src = torch.from_numpy(rng.integers(0, 256, (src_rows, row_bytes), dtype=np.uint8)).cuda()
    perm = rng.permutation(src_rows)[:rows].astype(np.int32)
    if rows > 2:
        perm[0], perm[1] = -5, src_rows + 9          # clamped to the first and last source row
    dst = torch.full((rows + 1, row_bytes), 0x5A, dtype=torch.uint8, device="cuda")
    B.moe_probe_gather(src, dst[:rows], torch.from_numpy(perm).cuda(), policy)
    torch.cuda.synchronize()
    want = src.cpu().numpy()[np.clip(perm, 0, src_rows - 1)]
    assert np.array_equal(dst[:rows].cpu().numpy(), want)
    assert (dst[rows:] == 0x5A).all()            # nothing past the last row
