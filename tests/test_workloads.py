"""Structure of the seeded synthetic workloads (routing tables, shapes, determinism)."""
import numpy as np

import workloads


def _check_routing(row_ids, offsets, T, E, top):
    assert offsets.dtype == np.int32 and row_ids.dtype == np.int32
    assert offsets[0] == 0 and offsets[-1] == T * top and np.all(np.diff(offsets) >= 0)
    assert np.array_equal(np.bincount(row_ids, minlength=T), np.full(T, top))
    for e in range(E):
        seg = row_ids[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)             # ascending tokens, each at most once per expert


def test_route_topk_ties_to_lower_id():
    logits = np.array([[1.0, 3.0, 3.0, 0.0], [2.0, 2.0, 2.0, 2.0]])
    row_ids, offsets = workloads.route_topk(logits, 2)
    assert list(offsets) == [0, 1, 3, 4, 4]          # t0 -> {1, 2}, t1 -> {0, 1}
    assert list(row_ids) == [1, 0, 1, 0]


def test_small_grouped_structure():
    wl = workloads.grouped_random(0, T=40, E=8, top=3, n=64, k=256, kinds=[0, 1] * 4,
                                  empty_experts=(5,))
    _check_routing(wl.row_ids, wl.offsets, 40, 8, 3)
    assert wl.offsets[6] == wl.offsets[5]
    for e in range(8):
        gs = workloads.GROUP_SIZE[int(wl.kinds[e])]
        assert wl.w_of(e).shape == (64, 128) and wl.s_of(e).shape == (64, 256 // gs)
    assert np.all(wl.scale2[wl.kinds == 1] == 0.0)


def test_config3_routing_loads():
    rng = workloads.rng_for(3)
    T, E = 512, 256
    rng.standard_normal((T, 7168), dtype=np.float32)           # same draw order as config3()
    logits = rng.standard_normal((T, E), dtype=np.float32)
    row_ids, offsets = workloads.route_topk(logits, 8)
    _check_routing(row_ids, offsets, T, E, 8)
    loads = np.diff(offsets)
    assert loads.sum() == 4096 and loads.min() >= 1 and loads.max() <= 40


def test_zipf_router_is_skewed():
    wl = workloads.grouped_random(2, T=2048, E=64, top=4, n=16, k=128, zipf=1.1)
    loads = np.diff(wl.offsets)
    _check_routing(wl.row_ids, wl.offsets, 2048, 64, 4)
    assert loads.max() > 8 * loads.mean() / 4 and loads.max() <= 2048


def test_determinism():
    a, b = workloads.config0(), workloads.config0()
    assert np.array_equal(a.x, b.x) and np.array_equal(a.expert.w, b.expert.w)
    assert np.array_equal(a.expert.s, b.expert.s)
    c2 = workloads.config2()
    n_big = int(np.sum(np.abs(c2.x) > 2.5))                     # |0.5 N(0,1)| > 2.5 is ~never drawn
    assert 250 <= n_big <= 328                                   # so these are the 328 x40 entries
