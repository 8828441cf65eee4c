"""route_pack_noalloc -- route_pack for callers that cannot allocate device memory (its workspace is a
library-owned device array) -- called through the C ABI and checked against route_pack's outputs bit
for bit, on two calls in a row with the second one smaller, plus the size limit it enforces."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_fp4_quant_amd as fp4

pytestmark = pytest.mark.gpu


def _table(seed, T, E, top, repeats=False):
    """A routing table from the device router over random logits; with `repeats`, some ids are
    duplicated within a token or dropped (outside [0, E)), which takes route_pack's slower path."""
    rng = np.random.default_rng([20261203, seed])
    logits = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
    ids, w = fp4.route_softmax_topk(logits, top)
    if repeats:
        ids_h = ids.cpu().numpy()
        ids_h[::7, -1] = ids_h[::7, 0]
        ids_h[3::11, 1] = E + 5
        ids_h[5::13, 0] = -1
        ids = torch.from_numpy(ids_h).cuda()
    return ids, w


def _noalloc(ids, w, E):
    """One route_pack_noalloc call through ctypes; outputs start poisoned so unwritten entries show."""
    T, top = ids.shape
    dev = ids.device
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    row_ids = torch.full((T * top,), -7, dtype=torch.int32, device=dev)
    pair_rows = torch.full((T, top), -7, dtype=torch.int32, device=dev)
    row_w = torch.full((T * top,), float("nan"), dtype=torch.float32, device=dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = fp4.lib().route_pack_noalloc(p(ids), p(w), T, top, E, p(offsets), p(row_ids), p(pair_rows), p(row_w),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, fp4.lib().fp4moe_last_error().decode()
    return offsets, row_ids, pair_rows, row_w


def _same(got, want):
    offs_g, rid_g, pr_g, rw_g = (t.cpu().numpy() for t in got)
    offs_w, rid_w, pr_w, rw_w = (t.cpu().numpy() for t in want)
    R = int(offs_w[-1])
    assert np.array_equal(offs_g, offs_w)
    assert np.array_equal(rid_g[:R], rid_w[:R])
    assert np.array_equal(pr_g, pr_w)
    assert np.array_equal(rw_g[:R].view(np.uint32), rw_w[:R].view(np.uint32))


@pytest.mark.parametrize("repeats", [False, True], ids=["topk", "repeats"])
def test_noalloc_matches_route_pack(repeats):
    # the prefill router's size first, then a smaller call: the second must not see the first's data
    for seed, T, E, top in [(1, 8192, 256, 8), (2, 300, 64, 4)]:
        ids, w = _table(seed + (10 if repeats else 0), T, E, top, repeats)
        got = _noalloc(ids, w, E)
        want = fp4.route_pack(ids, E, w)
        torch.cuda.synchronize()
        _same(got, want)


def test_noalloc_rejects_oversize():
    # 256 experts: at most 65,472 tokens fit the 1 MiB array; nothing is launched for a larger call
    big = ctypes.c_void_p(0x1000)
    rc = fp4.lib().route_pack_noalloc(big, None, 70000, 8, 256, big, big, big, None, None)
    assert rc == fp4.EINVAL
    assert "scratch" in fp4.lib().fp4moe_last_error().decode()
    assert fp4.route_pack_workspace_size(65472, 256) <= 1 << 20 < fp4.route_pack_workspace_size(65536, 256)
