"""The seeded generator: known-answer Philox vectors, rounding, determinism,
and the structure of its draws (hot sets, clustered runs, pool hits)."""
import json
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        out = synth.philox([int(x, 16) for x in v["ctr"]], [int(x, 16) for x in v["key"]])
        assert [int(x) for x in out] == [int(x, 16) for x in v["out"]]


def test_normals_moments_and_determinism():
    z = synth.normals(5, synth.TAG_K, 0, 0, 200000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert np.array_equal(z[1000:1100], synth.normals(5, synth.TAG_K, 0, 0, 100, off=1000))
    assert not np.array_equal(z[:100], synth.normals(6, synth.TAG_K, 0, 0, 100))
    assert not np.array_equal(z[:100], synth.normals(5, synth.TAG_K, 0, 0, 100, attempt=1))


def test_quantize_round_to_nearest_even():
    B, H = synth.BF16, synth.F16
    assert synth.quantize(1.0, B) == 0x3F80
    assert synth.quantize(1.0 + 2 ** -8, B) == 0x3F80          # tie -> even
    assert synth.quantize(1.0 + 3 * 2 ** -8, B) == 0x3F82      # tie -> even (up)
    assert synth.quantize(1.0 + 2 ** -8 + 2 ** -20, B) == 0x3F81
    assert synth.quantize(-2.0, B) == 0xC000
    assert synth.quantize(1.0, H) == 0x3C00
    assert synth.quantize(1.0 + 2 ** -11, H) == 0x3C00          # tie -> even
    assert synth.quantize(1.0 + 3 * 2 ** -11, H) == 0x3C02
    assert synth.quantize(2 ** -24, H) == 0x0001                # smallest subnormal
    assert synth.quantize(2 ** -25, H) == 0x0000                # tie -> even (zero)
    assert synth.quantize(3 * 2 ** -25, H) == 0x0002
    assert synth.quantize(65504.0, H) == 0x7BFF
    assert synth.quantize(65520.0, H) == 0x7C00                 # rounds to inf
    # agreement with numpy's own float16 rounding on random values
    x = np.random.default_rng(0).standard_normal(2000) * 3
    ref = x.astype(np.float32).astype(np.float16).view(np.uint16)
    assert [synth.quantize(v, H) for v in x] == ref.tolist()


def test_kv_block_regeneration_matches_full_fill():
    s = synth.spec(1, ctx=200)
    rq = synth.request_draws(s)[0]
    q = synth.gen_q(s, 0, 0)
    qhat = synth.gen_qhat(s, q)
    hot = synth.hot_mask(s, 0, 0, rq)
    att = np.zeros(rq.nb, np.uint8)
    att[3] = 2
    full = synth.gen_kv(s, synth.TAG_K, 0, 0, rq.ctx, hot=hot, attempts=att, qhat=qhat)
    base = synth.gen_kv(s, synth.TAG_K, 0, 0, rq.ctx, hot=hot, qhat=qhat)
    synth.regen_block(s, synth.TAG_K, 0, 0, rq.ctx, 3, bool(hot[3]), 2, qhat, base)
    assert np.array_equal(full, base)


def test_qhat_unit_vectors_and_planting_direction():
    s = synth.spec(2, B=1, ctx=64)
    q = synth.gen_q(s, 0, 0)
    qhat = synth.gen_qhat(s, q)
    assert np.allclose(np.linalg.norm(qhat, axis=1), 1.0)
    u = synth.decode(q, s.dtype).reshape(s.Hkv, s.G, s.d).sum(axis=1)
    assert np.allclose(qhat, u / np.linalg.norm(u, axis=1, keepdims=True))


def test_choose_distinct_sorted():
    c = synth.choose(3, synth.TAG_HOT, 0, 0, 1024, 51)
    assert len(set(c.tolist())) == 51 and np.all(np.diff(c) > 0) and c.min() >= 0 and c.max() < 1024


def test_clustered_runs_structure():
    for r in range(20):
        nb = int(synth.uniform_int(9, 1, 0, r, 0, 256, 4096))
        k = max(1, int(0.15 * nb))
        mask, m = synth.runs_mask(9, 0, r, nb, k)
        assert mask.sum() == k
        edges = np.diff(np.concatenate([[0], mask.astype(int), [0]]))
        starts, ends = np.flatnonzero(edges == 1), np.flatnonzero(edges == -1)
        assert len(starts) == m
        assert np.all(ends - starts <= 8) and np.all(ends - starts >= 1)


def test_variable_workload_draws():
    s = synth.spec(4)
    reqs = synth.request_draws(s)
    assert len(reqs) == 32
    for rq in reqs:
        assert 8192 <= rq.ctx <= 131072 and rq.nb == -(-rq.ctx // 32)
        assert 1 <= rq.k <= round(0.15 * rq.nb) + 1 and rq.k >= int(0.02 * rq.nb) - 1
    assert len({rq.ctx for rq in reqs}) > 20


def test_pool_hits_quarter():
    s = synth.spec(5)
    rq = synth.request_draws(s)[0]
    hits = synth.pool_hits(s, 0, 0, rq)
    assert hits.sum() == 256
