"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against the pages' printed numbers (fixtures in
tests/golden/), exact rational arithmetic, closed forms, invariants, or a
library routine (numpy relayout, numpy argpartition, torch SDPA in fp64).
The set is chosen so that a dropped term, a wrong index or group mapping, a
transposed operand, a wrong divisor or a wrong tie rule fails at least one.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F16, BF16 = oracle.F16, oracle.BF16


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(x: np.ndarray, dtype: int) -> np.ndarray:
    """float values -> storage bits via numpy (independent of both C modules)."""
    if dtype == F16:
        return np.asarray(x, np.float16).view(np.uint16)
    f = np.asarray(x, np.float32).view(np.uint32)
    # round to nearest even into the top 16 bits
    r = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def _vals(bits, dtype):
    bits = np.asarray(bits, np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rn32(fr: Fraction) -> np.float32:
    """Exact round-to-nearest-even of a rational to float32."""
    f = np.float32(float(fr))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        dist = abs(Fraction(float(c)) - fr)
        key = (dist, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _rand_bits(rng, shape, dtype, scale=1.0):
    return _bits(rng.standard_normal(shape) * scale, dtype)


# ------------------------------------------------------------ page numbers

def test_widen_known_patterns():
    assert oracle.widen(0x3C00, F16) == 1.0
    assert oracle.widen(0x0001, F16) == 2.0 ** -24
    assert oracle.widen(0x7BFF, F16) == 65504.0
    assert oracle.widen(0xC000, F16) == -2.0
    assert oracle.widen(0x3F80, BF16) == 1.0
    assert oracle.widen(0xC000, BF16) == -2.0
    assert oracle.widen(0x0001, BF16) == 2.0 ** -133


def test_kv_cache_bytes_page_example():
    g = _golden("page_kv_size.json")
    b = oracle.kv_cache_bytes(g["L"], g["Hkv"], g["d"], g["S"], g["es"])
    assert round(b / 1e9, 1) == g["gb_printed"]


def test_rec_bytes_page_formula():
    g = _golden("page_record_bytes.json")
    assert oracle.rec_bytes(g["Hkv"], g["bs"], g["d"], g["es"]) == g["bytes"]
    # the two record sizes of the workloads: 16 KiB (2 KV heads, 16 tokens, fp16)
    # and 128 KiB (8 KV heads, 32 tokens, bf16)
    assert oracle.rec_bytes(2, 16, 128, 2) == 16 * 1024
    assert oracle.rec_bytes(8, 32, 128, 2) == 128 * 1024


def test_page_solohead_example_counts():
    g = _golden("page_solohead_example.json")
    sets = np.array(g["head_sets"], np.int32)
    counts = [3, 3, 3]
    assert oracle.union_count(sets, counts) == g["union_blocks"]
    assert oracle.headwise_transfers(sets, counts) == g["per_head_transfers"]
    cons = np.array(g["consensus_blocks"], np.int32)
    first, ln = oracle.runs(cons)
    assert len(first) == g["consensus_transfers"]
    assert round(100 * (1 - len(cons) / g["union_blocks"])) == g["reduction_percent"]


# ------------------------------------------------------------------ digest

@pytest.mark.parametrize("dtype", [F16, BF16])
def test_digest_constant_block(dtype):
    # ctx = 21 with bs = 8: blocks of 8, 8 and 5 valid tokens
    Hkv, d, bs, ctx = 2, 8, 8, 21
    vals = np.array([0.75, -3.5, 1.0 / 3.0], np.float64)
    c = _bits(vals, dtype)
    K = np.empty((ctx, Hkv, d), np.uint16)
    for t in range(ctx):
        K[t] = c[t // bs]
    D = oracle.digest(K, dtype, bs)
    assert D.shape == (3, Hkv, d)
    for b in range(3):
        assert np.all(D[b] == np.float32(_vals(c[b], dtype)))


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_digest_exact_rounding_full_blocks(dtype):
    rng = np.random.default_rng(7)
    Hkv, d, bs, ctx = 2, 4, 16, 64
    K = _rand_bits(rng, (ctx, Hkv, d), dtype)
    D = oracle.digest(K, dtype, bs)
    V = _vals(K, dtype)
    for b in range(ctx // bs):
        for g in range(Hkv):
            for j in range(d):
                exact = sum(Fraction(float(V[t, g, j])) for t in range(b * bs, (b + 1) * bs)) / bs
                assert D[b, g, j] == _rn32(exact), (b, g, j)


def test_digest_partial_block_within_one_ulp():
    rng = np.random.default_rng(8)
    Hkv, d, bs, ctx = 1, 16, 32, 37  # last block holds 5 tokens
    K = _rand_bits(rng, (ctx, Hkv, d), BF16)
    D = oracle.digest(K, BF16, bs)
    V = _vals(K, BF16)
    for j in range(d):
        exact = sum(Fraction(float(V[t, 0, j])) for t in range(32, 37)) / 5
        got = Fraction(float(D[1, 0, j]))
        ulp = abs(Fraction(float(np.spacing(np.float32(float(exact))))))
        assert abs(got - exact) <= ulp / 2 + Fraction(1, 10 ** 30)


def test_digest_block_indexing():
    Hkv, d, bs, ctx = 3, 8, 4, 16
    K = np.zeros((ctx, Hkv, d), np.uint16)
    K[9, 2, 5] = _bits(np.array([2.0]), F16)[0]  # token 9 -> block 2, head 2, dim 5
    D = oracle.digest(K, F16, bs)
    nz = np.argwhere(D != 0)
    assert nz.tolist() == [[2, 2, 5]]
    assert D[2, 2, 5] == np.float32(0.5)


# ------------------------------------------------------------------- score

def test_score_bruteforce_exact():
    rng = np.random.default_rng(11)
    Hq, Hkv, d, nb = 4, 2, 8, 5
    q = _rand_bits(rng, (Hq, d), BF16)
    D = rng.standard_normal((nb, Hkv, d)).astype(np.float32)
    S = oracle.score(q, BF16, D)
    qv = _vals(q, BF16)
    G = Hq // Hkv
    for b in range(nb):
        exact = Fraction(0)
        mag = 0.0
        for h in range(Hq):
            for j in range(d):
                term = Fraction(float(qv[h, j])) * Fraction(float(D[b, h // G, j]))
                exact += term
                mag += abs(float(term))
        assert abs(Fraction(S[b]) - exact) <= Fraction(1e-13) * Fraction(mag)


def test_score_gqa_floor_mapping():
    # Hq = 8, Hkv = 4 (G = 2): head 5 belongs to KV head floor(5/2) = 2,
    # not 5 mod 4 = 1
    Hq, Hkv, d, nb = 8, 4, 4, 3
    q = np.zeros((Hq, d), np.uint16)
    q[5] = _bits(np.ones(d), F16)
    D = np.zeros((nb, Hkv, d), np.float32)
    D[1, 2, :] = 1.0
    D[2, 1, :] = 1.0
    S = oracle.score(q, F16, D)
    assert S.tolist() == [0.0, 4.0, 0.0]
    Sg = oracle.score_headwise(q, F16, D)
    assert Sg[2].tolist() == [0.0, 4.0, 0.0] and not Sg[[0, 1, 3]].any()


def test_score_presum_identity_and_headwise_sum():
    rng = np.random.default_rng(12)
    Hq, Hkv, d, nb = 32, 8, 128, 40
    q = _rand_bits(rng, (Hq, d), BF16)
    D = (rng.standard_normal((nb, Hkv, d)) / 5).astype(np.float32)
    S = oracle.score(q, BF16, D)
    u = _vals(q, BF16).reshape(Hkv, Hq // Hkv, d).sum(axis=1)  # u_g = sum of the group's heads
    S2 = np.einsum("gj,bgj->b", u, D.astype(np.float64))
    assert np.allclose(S, S2, rtol=1e-12, atol=1e-12)
    Sg = oracle.score_headwise(q, BF16, D)
    assert np.allclose(Sg.sum(axis=0), S, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ select

def test_select_bruteforce_random():
    rng = np.random.default_rng(13)
    for trial in range(50):
        nb = int(rng.integers(1, 60))
        k = int(rng.integers(1, 70))
        S = np.round(rng.standard_normal(nb), 1)  # coarse values force ties
        sel = oracle.select(S, k)
        want = sorted(sorted(range(nb), key=lambda b: (-S[b], b))[:min(k, nb)])
        assert sel.tolist() == want


def test_select_ties_lower_id_and_signed_zero():
    S = np.array([1.0, 0.0, -0.0, 0.0, 2.0, -1.0])
    assert oracle.select(S, 2).tolist() == [0, 4]
    assert oracle.select(S, 3).tolist() == [0, 1, 4]   # ties among zeros: lowest id first
    assert oracle.select(S, 4).tolist() == [0, 1, 2, 4]  # -0.0 ranks with +0.0 by id


def test_select_k_clamp_and_reject():
    S = np.array([3.0, 1.0, 2.0])
    assert oracle.select(S, 10).tolist() == [0, 1, 2]
    with pytest.raises(ValueError):
        oracle.select(S, 0)


def test_select_matches_argpartition():
    rng = np.random.default_rng(14)
    S = rng.standard_normal(4096)
    k = 614
    sel = oracle.select(S, k)
    ref = np.sort(np.argpartition(-S, k)[:k])
    assert sel.tolist() == ref.tolist()


# ------------------------------------------------------------------ recall

def test_runs_hand_examples():
    sel = np.array([1, 2, 3, 7, 8, 10], np.int32)
    f, ln = oracle.runs(sel)
    assert f.tolist() == [0, 3, 5] and ln.tolist() == [3, 2, 1]
    hit = np.zeros(16, np.uint8)
    hit[2] = 1
    f, ln = oracle.runs(sel, hit)
    assert f.tolist() == [0, 2, 3, 5] and ln.tolist() == [1, 1, 2, 1]
    hit[:] = 1
    f, ln = oracle.runs(sel, hit)
    assert len(f) == 0


def test_runs_properties_random():
    rng = np.random.default_rng(15)
    for trial in range(100):
        nb = int(rng.integers(1, 200))
        k = int(rng.integers(1, nb + 1))
        sel = np.sort(rng.choice(nb, k, replace=False)).astype(np.int32)
        hit = (rng.random(nb) < 0.25).astype(np.uint8)
        f, ln = oracle.runs(sel, hit)
        covered = []
        for a, n in zip(f, ln):
            ids = sel[a:a + n]
            assert np.all(np.diff(ids) == 1) and not hit[ids].any()
            covered += ids.tolist()
            # maximal: the next rank is not the next block, or is resident
            if a + n < k:
                nxt = sel[a + n]
                assert nxt != ids[-1] + 1 or hit[nxt]
        assert sorted(covered) == [b for b in sel.tolist() if not hit[b]]
        assert oracle.headwise_transfers(sel[None, :], [k], hit) == len(covered)


def test_records_vs_numpy_relayout():
    rng = np.random.default_rng(16)
    Hkv, d, bs, ctx = 3, 8, 4, 14
    K = rng.integers(0, 65535, (ctx, Hkv, d), dtype=np.uint16)
    V = rng.integers(0, 65535, (ctx, Hkv, d), dtype=np.uint16)
    rec = oracle.records(K, V, bs)
    nb = -(-ctx // bs)
    pad = lambda X: np.concatenate([X, np.zeros((nb * bs - ctx, Hkv, d), np.uint16)])
    Kb = pad(K).reshape(nb, bs, Hkv, d).transpose(0, 2, 1, 3)
    Vb = pad(V).reshape(nb, bs, Hkv, d).transpose(0, 2, 1, 3)
    assert np.array_equal(rec, np.stack([Kb, Vb], axis=2))


# --------------------------------------------------------------- attention

def _torch_sdpa_f64(q, K, V, dtype, tokens):
    import torch
    Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(_vals(q, dtype)).reshape(1, Hq, 1, d)
    kt = torch.from_numpy(_vals(K[tokens], dtype)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(_vals(V[tokens], dtype)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    return o.reshape(Hq, d).numpy()


def _small_case(seed, dtype=BF16, Hq=8, Hkv=2, d=32, bs=8, ctx=45):
    rng = np.random.default_rng(seed)
    q = _rand_bits(rng, (Hq, d), dtype)
    K = _rand_bits(rng, (ctx, Hkv, d), dtype)
    V = _rand_bits(rng, (ctx, Hkv, d), dtype)
    return q, K, V


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_dense_vs_torch_sdpa(dtype):
    q, K, V = _small_case(21, dtype)
    out = oracle.dense_f64(q, K, V, dtype)
    ref = _torch_sdpa_f64(q, K, V, dtype, np.arange(K.shape[0]))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_sparse_vs_sdpa_on_gathered_tokens():
    q, K, V = _small_case(22)  # ctx 45, bs 8: block 5 holds 5 valid tokens
    sel = np.array([0, 2, 3, 5], np.int32)
    toks = np.concatenate([np.arange(b * 8, min(b * 8 + 8, 45)) for b in sel])
    out = oracle.attend_f64(q, K, V, BF16, 8, sel)
    ref = _torch_sdpa_f64(q, K, V, BF16, toks)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    out32 = oracle.attend_f32(q, K, V, BF16, 8, sel)
    assert np.abs(out32 - ref).max() < 1e-5


def test_attend_all_blocks_equals_dense():
    q, K, V = _small_case(23, ctx=61)
    nb = -(-61 // 8)
    out = oracle.attend_f64(q, K, V, BF16, 8, np.arange(nb, dtype=np.int32))
    assert np.abs(out - oracle.dense_f64(q, K, V, BF16)).max() <= 1e-6
    assert np.array_equal(oracle.attend_f64(q, K, V, BF16, 8, None), out)


def test_softmax_weights_sum_to_one():
    q, K, V = _small_case(24)
    _, ws = oracle.attend_f64(q, K, V, BF16, 8, np.array([1, 4, 5], np.int32), want_wsum=True)
    assert np.allclose(ws, 1.0, rtol=0, atol=1e-12)


def test_attend_q_zero_gives_mean_of_selected_values():
    q, K, V = _small_case(25)
    q[:] = 0
    sel = np.array([1, 5], np.int32)
    toks = np.concatenate([np.arange(8, 16), np.arange(40, 45)])
    G = 4
    mean = _vals(V[toks], BF16).mean(axis=0)  # [Hkv][d]
    out = oracle.attend_f64(q, K, V, BF16, 8, sel)
    for h in range(8):
        assert np.allclose(out[h], mean[h // G], rtol=1e-12, atol=1e-14)


def test_attend_constant_values():
    q, K, V = _small_case(26)
    c = _bits(np.array([0.375, -1.25]), BF16)
    V[:, 0, :] = c[0]
    V[:, 1, :] = c[1]
    out = oracle.attend_f32(q, K, V, BF16, 8, np.array([0, 3], np.int32))
    assert np.allclose(out[:4], 0.375, rtol=1e-6) and np.allclose(out[4:], -1.25, rtol=1e-6)


def test_headwise_attention_with_equal_sets_equals_solohead():
    q, K, V = _small_case(27)
    sel = np.array([0, 2, 5], np.int32)
    a = oracle.attend_f32(q, K, V, BF16, 8, sel)
    b = oracle.attend_headwise_f32(q, K, V, BF16, 8, np.stack([sel, sel]))
    assert np.array_equal(a, b)
    # and different sets per KV head change only that group's heads
    c = oracle.attend_headwise_f32(q, K, V, BF16, 8, np.stack([sel, np.array([1, 3, 4], np.int32)]))
    assert np.array_equal(c[:4], a[:4]) and not np.array_equal(c[4:], a[4:])


def test_attend_f32_close_to_f64():
    q, K, V = _small_case(28, d=128, ctx=300)
    sel = np.array([3, 9, 10, 11, 30, 37], np.int32)
    a = oracle.attend_f32(q, K, V, BF16, 8, sel)
    b = oracle.attend_f64(q, K, V, BF16, 8, sel)
    assert np.abs(a - b).max() < 1e-5


# ---------------------------------------------------- workload conditioning

def test_gap_enforcement_and_planted_recovery():
    from tests import workloads
    s = synth.spec(2, B=2, ctx=8192, hot=13, k=16)
    for r, rq in enumerate(synth.request_draws(s)):
        sl = workloads.make_slice(s, 0, r, rq)
        gap, _ = workloads.boundary(sl.S, sl.K)
        assert gap >= workloads.MIN_GAP
        # planted blocks sit about 8 standard deviations above the rest at
        # these shapes; recovering them is a sanity rate of the generator
        hot = set(np.flatnonzero(sl.lr.hot).tolist())
        assert len(hot & set(sl.sel.tolist())) >= 0.9 * len(hot)


def test_gap_enforcement_redraws_a_tight_boundary():
    from tests import workloads
    s = synth.spec(1, ctx=512, hot=4, k=8)
    rq = synth.request_draws(s)[0]
    lr = synth.gen_layer_request(s, 0, 0, rq)
    plain = workloads.condition(s, lr, enforce=False)
    # demand a gap just above the natural one: the boundary block must be re-drawn
    lr2 = synth.gen_layer_request(s, 0, 0, rq)
    want = plain.gap + 1e-6
    sl = workloads.condition(s, lr2, min_gap=want)
    assert sl.redraws >= 1 and sl.gap >= want
    assert lr2.attempts.sum() == sl.redraws


# ----------------------------------------------------------- consensus rule

def test_consensus_bruteforce_and_special_cases():
    rng = np.random.default_rng(31)
    Hq, Hkv, d, nb = 8, 4, 8, 6
    q = _rand_bits(rng, (Hq, d), BF16)
    D = rng.standard_normal((nb, Hkv, d)).astype(np.float32)
    qv = _vals(q, BF16)
    G = Hq // Hkv
    for lam in (0.0, 0.5, 1.0):
        S = oracle.score_consensus(q, BF16, D, lam)
        for b in range(nb):
            per = [sum(Fraction(float(qv[h, j])) * Fraction(float(D[b, g, j]))
                       for h in range(g * G, (g + 1) * G) for j in range(d)) for g in range(Hkv)]
            exact = max(per) + Fraction(lam) * sum(per) / Hkv
            assert abs(Fraction(S[b]) - exact) <= Fraction(1e-12) * (1 + abs(exact))
    # lambda = 0 is the per-block max over KV heads; one KV head gives (1 + lambda) * S
    Sg = oracle.score_headwise(q, BF16, D)
    assert np.array_equal(oracle.score_consensus(q, BF16, D, 0.0), Sg.max(axis=0))
    q1 = _rand_bits(rng, (4, d), BF16)
    D1 = rng.standard_normal((nb, 1, d)).astype(np.float32)
    assert np.allclose(oracle.score_consensus(q1, BF16, D1, 0.5), 1.5 * oracle.score(q1, BF16, D1),
                       rtol=1e-14, atol=0)


def test_group_consensus_bruteforce_and_special_cases():
    """Consensus within each GQA group: exact rational brute force; lambda = 0
    is the max over the group's query heads; the lambda term is the headwise
    score / G; a group of identical heads gives (1 + lambda) * their score."""
    rng = np.random.default_rng(33)
    Hq, Hkv, d, nb = 8, 2, 8, 5
    G = Hq // Hkv
    q = _rand_bits(rng, (Hq, d), BF16)
    D = rng.standard_normal((nb, Hkv, d)).astype(np.float32)
    qv = _vals(q, BF16)
    for lam in (0.0, 0.5, 1.0):
        S = oracle.score_group_consensus(q, BF16, D, lam)
        assert S.shape == (Hkv, nb)
        for g in range(Hkv):
            for b in range(nb):
                per = [sum(Fraction(float(qv[h, j])) * Fraction(float(D[b, g, j])) for j in range(d))
                       for h in range(g * G, (g + 1) * G)]
                exact = max(per) + Fraction(lam) * sum(per) / G
                assert abs(Fraction(S[g, b]) - exact) <= Fraction(1e-12) * (1 + abs(exact))
    S0, S1 = oracle.score_group_consensus(q, BF16, D, 0.0), oracle.score_group_consensus(q, BF16, D, 1.0)
    assert np.allclose((S1 - S0) * G, oracle.score_headwise(q, BF16, D), rtol=1e-12, atol=1e-12)
    qs = q.copy()
    for g in range(Hkv):
        qs[g * G:(g + 1) * G] = q[g * G]
    Sh = oracle.score_headwise(qs, BF16, D)
    assert np.allclose(oracle.score_group_consensus(qs, BF16, D, 0.5), 1.5 * Sh / G, rtol=1e-13, atol=1e-13)


def _softmax_mass_scipy(q, K, dtype, bs, sets):
    """Independent form: logits by a numpy matmul, softmax by scipy, summed
    over the selected tokens of each head's set."""
    from scipy.special import softmax
    Hq, d = q.shape
    ctx, Hkv, _ = K.shape
    G = Hq // Hkv
    qv, Kv = _vals(q, dtype), _vals(K, dtype)
    out = np.empty(Hq)
    for h in range(Hq):
        g = h // G
        p = softmax((Kv[:, g, :] @ qv[h]) / np.sqrt(d))
        chosen = np.isin(np.arange(ctx) // bs, sets[0 if len(sets) == 1 else g])
        out[h] = p[chosen].sum()
    return out


def test_attention_mass_vs_scipy_softmax():
    q, K, _ = _small_case(41, ctx=61)  # bs 8: last block holds 5 tokens
    shared = np.array([0, 3, 7], np.int32)
    m = oracle.attention_mass(q, K, BF16, 8, shared)
    assert np.allclose(m, _softmax_mass_scipy(q, K, BF16, 8, [shared]), rtol=0, atol=1e-12)
    per = np.array([[1, 2, 7], [0, 4, 6]], np.int32)
    m = oracle.attention_mass(q, K, BF16, 8, per)
    assert np.allclose(m, _softmax_mass_scipy(q, K, BF16, 8, list(per)), rtol=0, atol=1e-12)
    # per-KV-head sets with equal rows are the shared set
    assert np.array_equal(oracle.attention_mass(q, K, BF16, 8, np.stack([shared, shared])),
                          oracle.attention_mass(q, K, BF16, 8, shared))


def test_attention_mass_complement_and_mixture_identity():
    """mass(S) + mass(complement) = 1, and the dense output is the mass-weighted
    mix of the sparse outputs over S and its complement (ties the mass to the
    attention oracle, itself pinned to torch's SDPA)."""
    q, K, V = _small_case(42, ctx=70)  # 9 blocks of 8, the last holds 6 tokens
    nb = 9
    S = np.array([1, 2, 5, 8], np.int32)
    C = np.setdiff1d(np.arange(nb, dtype=np.int32), S)
    mS = oracle.attention_mass(q, K, BF16, 8, S)
    mC = oracle.attention_mass(q, K, BF16, 8, C)
    assert np.allclose(mS + mC, 1.0, rtol=0, atol=1e-12)
    assert np.all((mS > 0) & (mS < 1))
    mix = mS[:, None] * oracle.attend_f64(q, K, V, BF16, 8, S) + \
        mC[:, None] * oracle.attend_f64(q, K, V, BF16, 8, C)
    assert np.allclose(mix, oracle.dense_f64(q, K, V, BF16), rtol=0, atol=1e-12)
    # every block selected keeps all of the mass; counts limit the set
    assert np.array_equal(oracle.attention_mass(q, K, BF16, 8, np.arange(nb, dtype=np.int32)),
                          np.ones(q.shape[0]))
    assert np.array_equal(oracle.attention_mass(q, K, BF16, 8, np.array([[1, 2, 5, 8]], np.int32),
                                                counts=[2]),
                          oracle.attention_mass(q, K, BF16, 8, np.array([1, 2], np.int32)))
