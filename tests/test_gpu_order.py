"""The order a record's replays run in (dao_grad_order), on the GPU: a
counting sort by decreasing step count that keeps equal bins in index order.

Bins are ((s_max + 1) - min(count, s_max + 1)) >> shift with the smallest
shift that leaves at most 4096 bins (a negative count, a failed trajectory,
counts as 0).  The expected order is numpy's stable argsort of those bins.
The order sits in the workspace after the queue counter and the 4096 bin
offsets (256-byte aligned regions): bytes [16640, 16640 + 4 n)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PERM_OFFSET = 256 + 4096 * 4


def expected(count, s_max):
    shift = 0
    while ((s_max + 1) >> shift) + 1 > 4096:
        shift += 1
    c = np.clip(count.astype(np.int64), 0, s_max + 1)
    return np.argsort(((s_max + 1) - c) >> shift, kind="stable")


@pytest.mark.parametrize("n,s_max,hi", [(1, 8, 8), (1000, 70, 70), (1025, 6, 9),
                                        (64 * 1024 + 37, 1000, 1000),
                                        (300_000, 20_000, 20_000), (200_000, 8191, 300),
                                        # one bin of real counts; exactly 4096 bins (12 bits);
                                        # the first s_max that needs a shift
                                        (5000, 0, 0), (70_000, 4094, 4094), (70_000, 4095, 4095)])
def test_order_is_a_stable_sort_by_bin(n, s_max, hi):
    from differentiable_adaptive_ode_amd import _lib

    print(f"[order] n={n} s_max={s_max}", flush=True)
    rng = np.random.default_rng(n + s_max)
    count = rng.integers(-1, hi + 1, n).astype(np.int32)  # many ties, a few failed
    cnt = torch.tensor(count, device=DEV)
    status = torch.zeros(n, dtype=torch.int32, device=DEV)
    h = torch.zeros(1, dtype=torch.float64, device=DEV)  # not read by the order
    rec = _lib.dao_record(s_max, None, h.data_ptr(), cnt.data_ptr(), None, status.data_ptr())
    ids = _lib.SYSTEMS["lorenz63"], 0, 0
    nb = _lib.dao_grad_workspace_size(*ids, n, s_max)
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    for rep in range(2):
        _lib.check(_lib.dao_grad_order(*ids, n, rec, s_max, ws.data_ptr(), nb,
                                       torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        perm = ws[PERM_OFFSET:PERM_OFFSET + 4 * n].cpu().numpy().view(np.int32)
        assert np.array_equal(perm, expected(count, s_max)), rep
