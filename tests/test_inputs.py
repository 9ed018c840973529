"""The seeded workload generators: determinism and the recipes' statistics."""
import numpy as np
import pytest

from lora_inputs import (make_workload, bf16_round, bf16_to_f32, lognormal_lengths, zipf_ids,
                         CONFIG_NAMES)


def test_bf16_round_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    got = bf16_to_f32(bf16_round(v))
    assert list(got) == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0 + 2 ** -7]


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_deterministic_and_seed_sensitive(name):
    small = dict(d_in=64, d_out=48, T=64, n_slots=16, r=8, n_req=4, n_decode=16, prefill_len=8,
                 shapes=[("q", 64, 48), ("down", 48, 64)])
    a = make_workload(name, **small)
    b = make_workload(name, **small)
    c = make_workload(name, seed=77, **small)
    assert np.array_equal(a.ids, b.ids) and np.array_equal(a.active, b.active)
    p, q = a.projections[0], b.projections[0]
    w0a, w0b = p.w0(), q.w0()
    if isinstance(w0a, tuple):
        assert np.array_equal(w0a[0], w0b[0]) and np.array_equal(w0a[1], w0b[1])
    else:
        assert np.array_equal(w0a, w0b)
    assert np.array_equal(a.x(p), b.x(q))
    s = a.touched_slots()[0]
    assert all(np.array_equal(u, v) for u, v in zip(p.slot(s), q.slot(s)))
    assert not np.array_equal(a.x(p), c.x(c.projections[0]))


def test_decode_recipe():
    w = make_workload("decode_bgmv")
    assert w.T == 256 and (w.ids == -1).sum() == 64
    p = w.projections[0]
    assert (p.d_in, p.d_out, p.n_slots, p.r_cap) == (4096, 4096, 64, 16)
    live = w.ids[w.ids >= 0]
    # Zipf(1.1) over 64 ids: id 0 is by far the most frequent
    counts = np.bincount(live, minlength=64)
    assert counts[0] == counts.max() and counts[0] > 0.15 * len(live)
    A, Bt = p.slot(0)
    a = bf16_to_f32(A).astype(np.float64)
    assert abs(a.std() - 0.02) < 0.001 and a.shape == (16, 4096)


def test_prefill_recipe():
    w = make_workload("prefill_sgmv")
    assert w.T == 8192 and len(w.request_lengths) == 32 and w.request_lengths.sum() == 8192
    p = w.projections[0]
    assert set(np.unique(p.slot_rank)) <= {8, 16, 32, 64}
    assert np.allclose(p.slot_scale * p.slot_rank, 32.0)
    # requests are contiguous runs of one adapter id
    starts = np.concatenate([[0], np.cumsum(w.request_lengths)[:-1]])
    for s, n in zip(starts, w.request_lengths):
        assert len(set(w.ids[s:s + n])) == 1


def test_llama_layer_recipe():
    w = make_workload("llama_layer", n_slots=64)
    assert w.T == 2048
    assert [(p.d_in, p.d_out) for p in w.projections] == [
        (4096, 4096), (4096, 1024), (4096, 1024), (4096, 4096), (4096, 14336), (4096, 14336), (14336, 4096)]
    assert w.active[:1536].all() and w.active[1536:].sum() == 256
    assert (w.ids >= 0).all()


def test_fp8_recipe_small():
    w = make_workload("fp8_fused", d_in=256, d_out=96, T=32, n_slots=8)
    codes, s = w.projections[0].w0()
    assert codes.dtype == np.uint8 and codes.shape == (96, 256) and s.shape == (96,)
    assert np.all((codes & 0x7F) != 0x7F)                        # no NaN codes
    assert np.all(np.any((codes & 0x7F) == 0x7E, axis=1))        # amax -> 448 in every row


def test_lognormal_lengths_sum_and_min():
    g = np.random.default_rng(0)
    for n, tot in [(32, 8192), (5, 7), (10, 10), (3, 1000)]:
        l = lognormal_lengths(g, n, 5.5, 0.8, tot)
        assert l.sum() == tot and l.min() >= 1


def test_zipf_probabilities():
    g = np.random.default_rng(0)
    ids = zipf_ids(g, 8, 1.1, 200000)
    p = np.arange(1, 9) ** -1.1
    p /= p.sum()
    emp = np.bincount(ids, minlength=8) / len(ids)
    assert np.abs(emp - p).max() < 0.005
