"""Pins for the float64 oracle: each test checks it against something other than itself.

Brute force (pure Python, math.fsum, its own visibility predicate and head mapping), closed
forms, hand-derived worked examples, torch's float64 attention as a library special case,
permutation invariance and reductions.  The planted-mistake tests at the end swap one oracle
helper for a plausible wrong one and require that some pin goes red, so the pins are known
to discriminate.
"""
import itertools
import json
import math
import os
import random

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from oracle import pages as opages

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


# ----------------------------------------------------------------------------- bf16
def test_bf16_widen_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x4049], np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -2.0
    assert got[2] == 2.0 ** -133                      # smallest bf16 subnormal: 2^-126 * 2^-7
    assert got[3] == math.inf and got[4] == -math.inf
    assert got[5] == 0.0 and math.copysign(1.0, got[6]) == -1.0
    assert got[7] == 3.140625                         # 0x4049 = 1.5703125 * 2
    assert np.isnan(oracle.bf16_bits_to_f64(np.array([0x7FC0, 0xFFC1], np.uint16))).all()


def test_bf16_narrow_round_to_nearest_even():
    one = 1.0
    ulp = 2.0 ** -7                                   # bf16 spacing just above 1.0
    cases = {
        one: 0x3F80,
        one + ulp / 2: 0x3F80,                        # tie -> even (mantissa 0)
        one + 3 * ulp / 2: 0x3F82,                    # tie -> even (mantissa 2)
        one + ulp / 2 + 2.0 ** -20: 0x3F81,           # just above the tie -> up
        3.0e38 * 2: 0x7F80,                           # float32 overflow -> inf
        -0.0: 0x8000,
    }
    for x, want in cases.items():
        assert int(oracle.f64_to_bf16_bits(np.array([x]))[0]) == want, x
    # agrees with torch's own float32 -> bf16 rounding on random values
    x = np.random.default_rng(0).standard_normal(10000) * 100
    tb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (oracle.f64_to_bf16_bits(x) == tb).all()


# ----------------------------------------------------------------------------- brute force
def brute_attention(q, k, v, lengths, window, scale=None):
    """Pure-Python attention written from the definition, sharing no code with the oracle:
    its own loops, its own visibility predicate and head mapping, math.exp and math.fsum."""
    S, R, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    out = []
    for s in range(S):
        L = lengths[s]
        Hkv = len(k[s][0])
        c = 1.0 / math.sqrt(D) if scale is None else scale
        rows_out = []
        for r in range(R):
            pos = L - R + r
            heads_out = []
            for h in range(Hq):
                g = (h * Hkv) // Hq                      # contiguous groups, written differently
                keys = [j for j in range(L) if j <= pos and (window <= 0 or j > pos - window)]
                sc = [c * math.fsum(q[s][r][h][d] * k[s][j][g][d] for d in range(D)) for j in keys]
                top = max(sc)
                w = [math.exp(x - top) for x in sc]
                tot = math.fsum(w)
                heads_out.append([math.fsum(w[i] * v[s][keys[i]][g][d] for i in range(len(keys))) / tot
                                  for d in range(D)])
            rows_out.append(heads_out)
        out.append(rows_out)
    return np.array(out)


def _random_case(rng, S, R, Hkv, G, D, lengths):
    q = rng.standard_normal((S, R, Hkv * G, D))
    ks = [rng.standard_normal((L, Hkv, D)) for L in lengths]
    vs = [rng.standard_normal((L, Hkv, D)) for L in lengths]
    return q, ks, vs


@pytest.mark.parametrize("seed", range(12))
def test_oracle_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 3))
    R = int(rng.integers(1, 5))
    Hkv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([1, 3, 8]))
    lengths = [int(rng.integers(R, 41)) for _ in range(S)]
    window = int(rng.choice([0, 0, 1, 3, 7, 50]))
    q, ks, vs = _random_case(rng, S, R, Hkv, G, D, lengths)
    got = oracle.attend(q, ks, vs, lengths, window)
    want = brute_attention(q.tolist(), [x.tolist() for x in ks], [x.tolist() for x in vs], lengths, window)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed,scale", [(101, 0.02), (102, 0.3), (103, 1.7)])
def test_oracle_matches_brute_force_at_a_given_scale(seed, scale):
    # a caller-given scale replaces 1/sqrt(d): the oracle must use it (and not the default)
    rng = np.random.default_rng(seed)
    lengths = [int(rng.integers(4, 30)) for _ in range(2)]
    q, ks, vs = _random_case(rng, 2, 3, 2, 2, 8, lengths)
    got = oracle.attend(q, ks, vs, lengths, 0, scale=scale)
    want = brute_attention(q.tolist(), [x.tolist() for x in ks], [x.tolist() for x in vs], lengths, 0, scale=scale)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    assert np.abs(got - oracle.attend(q, ks, vs, lengths, 0)).max() > 1e-3


# ----------------------------------------------------------------------------- closed forms
def test_one_key_gives_v_exactly():
    rng = np.random.default_rng(1)
    for D in (1, 7, 128, 512):
        q = rng.standard_normal((1, 1, 4, D)) * 10
        k = rng.standard_normal((1, 1, D))
        v = rng.standard_normal((1, 1, D))
        out = oracle.attend(q, [k], [v], [1])
        assert (out[0, 0] == v[0, 0][None, :]).all()


def test_zero_query_gives_mean_of_visible_rows():
    rng = np.random.default_rng(2)
    L, R, W, D = 33, 4, 9, 5
    q = np.zeros((1, R, 2, D))
    k = rng.standard_normal((L, 2, D))
    v = rng.standard_normal((L, 2, D))
    for window in (0, W):
        out = oracle.attend(q, [k], [v], [L], window)
        for r in range(R):
            p = L - R + r
            first = 0 if window == 0 else p - window + 1
            for h in range(2):
                want = [math.fsum(v[j, h, d] for j in range(first, p + 1)) / (p + 1 - first) for d in range(D)]
                np.testing.assert_allclose(out[0, r, h], want, rtol=1e-14, atol=1e-15)


def test_golden_worked_examples():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 6
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)[None]
        k = np.array(c["k"], dtype=np.float64)
        v = np.array(c["v"], dtype=np.float64)
        out = oracle.attend(q, [k], [v], [k.shape[0]], c["window"], c["scale"])
        np.testing.assert_allclose(out[0], np.array(c["expected"]), rtol=1e-12, atol=1e-12, err_msg=c["name"])


# ----------------------------------------------------------------------------- library special case
@pytest.mark.parametrize("seed,window", [(0, 0), (1, 0), (2, 5), (3, 17), (4, 1)])
def test_oracle_matches_torch_sdpa_float64(seed, window):
    rng = np.random.default_rng(100 + seed)
    S, R, Hkv, G, D = 2, 5, 2, 4, 16
    lengths = [37, 64]
    q, ks, vs = _random_case(rng, S, R, Hkv, G, D, lengths)
    got = oracle.attend(q, ks, vs, lengths, window)
    for s, L in enumerate(lengths):
        qt = torch.from_numpy(q[s]).permute(1, 0, 2)                    # [Hq][R][D]
        kt = torch.from_numpy(ks[s]).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq][L][D]
        vt = torch.from_numpy(vs[s]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        pos = torch.arange(L - R, L)[:, None]
        j = torch.arange(L)[None, :]
        mask = j <= pos
        if window > 0:
            mask &= j > pos - window
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        np.testing.assert_allclose(got[s], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- reductions
def test_verify_row_equals_decode_at_its_length():
    rng = np.random.default_rng(3)
    L, R, Hkv, G, D = 50, 8, 2, 4, 8
    q, ks, vs = _random_case(rng, 1, R, Hkv, G, D, [L])
    for window in (0, 6):
        full = oracle.attend(q, ks, vs, [L], window)
        for r in range(R):
            p = L - R + r
            one = oracle.attend(q[:, r:r + 1], [ks[0][:p + 1]], [vs[0][:p + 1]], [p + 1], window)
            np.testing.assert_allclose(full[0, r], one[0, 0], rtol=1e-13, atol=1e-14)


def test_chunked_prefill_equals_unchunked():
    rng = np.random.default_rng(4)
    L, Hkv, G, D, C = 96, 2, 2, 8, 32
    q, ks, vs = _random_case(rng, 1, L, Hkv, G, D, [L])
    for window in (0, 40):
        whole = oracle.attend(q, ks, vs, [L], window)
        for c0 in range(0, L, C):
            part = oracle.attend(q[:, c0:c0 + C], [ks[0][:c0 + C]], [vs[0][:c0 + C]], [c0 + C], window)
            np.testing.assert_allclose(whole[0, c0:c0 + C], part[0], rtol=1e-13, atol=1e-14)


def test_window_at_least_length_is_full_causal():
    rng = np.random.default_rng(5)
    L, R = 30, 3
    q, ks, vs = _random_case(rng, 1, R, 1, 2, 4, [L])
    np.testing.assert_array_equal(oracle.attend(q, ks, vs, [L], 0), oracle.attend(q, ks, vs, [L], L))


def test_output_lies_within_visible_rows():
    rng = np.random.default_rng(6)
    L, R, D = 45, 4, 6
    q, ks, vs = _random_case(rng, 1, R, 1, 2, D, [L])
    q *= 20
    for window in (0, 7):
        out = oracle.attend(q, ks, vs, [L], window)
        for r in range(R):
            p = L - R + r
            lo = 0 if window == 0 else p - window + 1
            vis = vs[0][lo:p + 1, 0]
            assert (out[0, r] >= vis.min(axis=0) - 1e-12).all()
            assert (out[0, r] <= vis.max(axis=0) + 1e-12).all()


# ----------------------------------------------------------------------------- pages
def test_slot_of_matches_enumeration():
    table = [5, 2, 7, 0]
    for P, ring in [(1, 0), (3, 0), (37, 0), (3, 2), (5, 3)]:
        # enumerate the slots in order: logical page idx, then slot within it
        n = len(table) if not ring else ring
        expected = {}
        j = 0
        for idx in itertools.count():
            for sl in range(P):
                expected[j] = (table[idx % n] if ring else table[idx], sl)
                j += 1
            if j >= (len(table) * P if not ring else 4 * n * P):
                break
        for jj, want in expected.items():
            assert opages.slot_of(jj, table, P, ring) == want


@pytest.mark.parametrize("P,ring", [(1, 0), (3, 0), (37, 0), (64, 0), (512, 0), (4, 3), (37, 2)])
def test_rows_put_then_gather_round_trip(P, ring):
    rng = np.random.default_rng(P * 10 + ring)
    Hkv, D = 2, 4
    L_final = 130 if P < 512 else 700
    n_pages = ring if ring else -(-L_final // P)
    N = n_pages + 9
    table = rng.permutation(N)[:n_pages]
    pages = np.full((N, Hkv, P, D), np.nan)
    hist = rng.standard_normal((L_final, Hkv, D))
    L = 0
    while L < L_final:
        R = int(min(rng.integers(1, 20), L_final - L))
        L += R
        pages = opages.rows_put(pages, table, L, hist[L - R:L], P, ring)
    got = oracle.gather_linear(pages, table, L_final, P, ring)
    if ring:
        got, first = got
        assert first == max(0, L_final - ring * P)
        np.testing.assert_array_equal(got, hist[first:])
    else:
        np.testing.assert_array_equal(got, hist)
    # pages the table never names are untouched (still NaN)
    others = np.setdiff1d(np.arange(N), table)
    assert np.isnan(pages[others]).all()


def test_gather_is_invariant_under_page_shuffles():
    rng = np.random.default_rng(7)
    P, Hkv, D, L = 37, 2, 8, 300
    n = -(-L // P)
    hist = rng.standard_normal((L, Hkv, D))
    q = rng.standard_normal((1, 3, Hkv * 4, D))
    outs = []
    for order in (np.arange(n + 5), rng.permutation(n + 5), rng.permutation(n + 5)):
        table = order[:n]
        pages = np.full((n + 5, Hkv, P, D), np.nan)
        pages = opages.rows_put(pages, table, L, hist, P)
        lin = oracle.gather_linear(pages, table, L, P)
        outs.append(oracle.attend(q, [lin], [lin * 0.5], [L]))
    assert all((o == outs[0]).all() for o in outs[1:])
    assert np.isfinite(outs[0]).all()


# ----------------------------------------------------------------------------- lease model
def test_lease_model_partitions_the_pool():
    rng = random.Random(11)
    N, S = 50, 5
    order = list(range(N))
    rng.shuffle(order)
    m = oracle.LeaseModel(N, S, order)
    handed = []
    for _ in range(400):
        s = rng.randrange(S)
        if rng.random() < 0.7:
            n = rng.randrange(0, 12)
            before = (list(m.free), [list(x) for x in m.leased])
            try:
                got = m.lease(s, n)
                handed.extend(got)
            except oracle.NoPages:
                assert n > len(before[0])
                assert (list(m.free), [list(x) for x in m.leased]) == before   # nothing changed
        else:
            m.release(s)
        leased = [p for lst in m.leased for p in lst]
        assert len(set(leased)) == len(leased)                                  # no page twice
        assert sorted(leased + list(m.free)) == list(range(N))                  # a partition
    # hand-out follows the queue: the first leases take free_order's ids in order
    m2 = oracle.LeaseModel(N, S, order)
    assert m2.lease(0, 3) == order[:3] and m2.lease(1, 2) == order[3:5]
    m2.release(0)
    assert list(m2.free)[-3:] == order[:3]


def _share_sequence(model_cls=None):
    """The hand-worked share/release sequence: True when every step gives the derived lists."""
    m = (model_cls or oracle.LeaseModel)(8, 3)
    ok = m.lease(0, 4) == [0, 1, 2, 3]
    m.share(0, 1, 3)
    ok &= m.leased[1] == [0, 1, 2] and list(m.free) == [4, 5, 6, 7]
    ok &= m.lease(1, 2) == [4, 5]
    m.release(0)
    ok &= list(m.free) == [6, 7, 3]
    m.release(1)
    ok &= list(m.free) == [6, 7, 3, 0, 1, 2, 4, 5]
    return bool(ok and m.lease(2, 3) == [6, 7, 3])


class _ReleaseFreesShared(oracle.LeaseModel):
    """Planted mistake: a release returns every page of the stream, held elsewhere or not."""
    def release(self, stream):
        self.free.extend(self.leased[stream])
        self.leased[stream] = []


def test_planted_share_mistake_turns_the_share_sequence_red():
    assert _share_sequence()
    assert not _share_sequence(_ReleaseFreesShared)


def test_shared_pages_follow_the_hand_worked_sequence():
    # 8 pages in identity order, 3 streams; each expected list is derived from the rules:
    m = oracle.LeaseModel(8, 3)
    assert m.lease(0, 4) == [0, 1, 2, 3]           # queue front
    m.share(0, 1, 3)                               # stream 1 takes stream 0's first 3 pages
    assert m.leased[1] == [0, 1, 2] and list(m.free) == [4, 5, 6, 7]
    assert m.lease(1, 2) == [4, 5]                 # its own pages follow the shared ones
    assert m.leased[1] == [0, 1, 2, 4, 5]
    m.release(0)                                   # 0, 1, 2 are still held by stream 1: only 3 returns
    assert list(m.free) == [6, 7, 3] and [m.holders(i) for i in range(8)] == [1, 1, 1, 0, 1, 1, 0, 0]
    m.release(1)                                   # the last holder: all of stream 1's pages, in its order
    assert list(m.free) == [6, 7, 3, 0, 1, 2, 4, 5]
    assert m.lease(2, 3) == [6, 7, 3]
    with pytest.raises(ValueError):
        m.share(2, 2, 1)                           # not with itself
    m.share(2, 0, 2)
    with pytest.raises(ValueError):
        m.share(2, 0, 1)                           # stream 0 already holds pages
    with pytest.raises(ValueError):
        m.share(2, 1, 4)                           # more than stream 2 holds


def test_rows_before_the_stream_get_zeros_and_leave_the_others_alone():
    # a call with more rows than the stream's length: rows at negative positions see no key (a
    # stream of length 0 has only such rows); the rows at positions >= 0 are those of a call
    # with exactly L rows
    rng = np.random.default_rng(77)
    Hkv, G, D, L, R = 2, 4, 16, 3, 5
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    q = rng.standard_normal((R, Hkv * G, D))
    out = oracle.attend_stream(q, k, v, R, length=L)
    assert (out[:R - L] == 0).all()
    assert np.array_equal(out[R - L:], oracle.attend_stream(q[R - L:], k, v, L, length=L))
    empty = oracle.attend_stream(q[:1], k[:0], v[:0], 1, length=0)
    assert empty.shape == (1, Hkv * G, D) and (empty == 0).all()


def test_shared_pages_partition_the_pool():
    rng = random.Random(23)
    N, S = 40, 6
    m = oracle.LeaseModel(N, S)
    for _ in range(600):
        s = rng.randrange(S)
        r = rng.random()
        if r < 0.5:
            try:
                m.lease(s, rng.randrange(0, 8))
            except oracle.NoPages:
                pass
        elif r < 0.75:
            empty = [d for d in range(S) if not m.leased[d] and d != s]
            if empty:
                m.share(s, rng.choice(empty), rng.randrange(0, len(m.leased[s]) + 1))
        else:
            m.release(s)
        for lst in m.leased:
            assert len(set(lst)) == len(lst)                                   # no page twice in a list
        held = set(p for lst in m.leased for p in lst)
        free = list(m.free)
        assert len(set(free)) == len(free) and not held & set(free)           # free pages are not held
        assert sorted(held | set(free)) == list(range(N))                      # nothing lost
        assert all((m.holders(p) == 0) == (p in set(free)) for p in range(N))


# ----------------------------------------------------------------------------- planted mistakes
def _pins_pass():
    try:
        for seed in range(6):
            test_oracle_matches_brute_force(seed)
        test_golden_worked_examples()
        test_verify_row_equals_decode_at_its_length()
        test_zero_query_gives_mean_of_visible_rows()
        for seed, window in [(0, 0), (2, 5)]:
            test_oracle_matches_torch_sdpa_float64(seed, window)
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name,patch", [
    ("interleaved_gqa", ("kv_head_of", lambda h, group: h % max(1, group))),
    ("window_one_short", ("visible_range", lambda p, w: (0 if w <= 0 else max(0, p - w + 2), p + 1))),
    ("causal_off_by_one", ("row_position", lambda L, R, r: L - R + r - 1)),
    ("decode_sees_future", ("visible_range", lambda p, w: (0 if w <= 0 else max(0, p - w + 1), p + 2))),
])
def test_planted_mistakes_turn_pins_red(monkeypatch, name, patch):
    assert _pins_pass()
    attr, fn = patch
    monkeypatch.setattr(oatt, attr, fn)
    assert not _pins_pass(), f"planted mistake {name} was not caught"


def test_planted_wrong_scale_turns_pins_red(monkeypatch):
    real = oatt.attend_stream

    def wrong(q, k, v, rows, window=0, scale=None, length=None):
        d = np.asarray(q).shape[-1]
        return real(q, k, v, rows, window, 1.0 / d if scale is None else scale, length)
    monkeypatch.setattr(oatt, "attend_stream", wrong)
    assert not _pins_pass()


# ----------------------------------------------------------------------------- tree windows
def _random_tree(rng, R):
    """Parents of a draft tree flattened into R window slots, parents before children: slot 0
    is the pending token (no parent in the window), parent[i] < i."""
    return [-1] + [int(rng.integers(0, i)) for i in range(1, R)]


def _ancestor_set(parent, r):
    out = {r}
    while parent[r] >= 0:
        r = parent[r]
        out.add(r)
    return out


def brute_tree_attention(q, k, v, L, R, anc, window=0):
    """Pure Python over one stream; row r sees key j iff j <= its slot, j is inside the window,
    and j lies before the window or is one of r's ancestor slots (given as sets, not bits)."""
    Hq, D, Hkv = len(q[0]), len(q[0][0]), len(k[0])
    c = 1.0 / math.sqrt(D)
    out = []
    for r in range(R):
        pos = L - R + r
        rows = []
        for h in range(Hq):
            g = (h * Hkv) // Hq
            keys = [j for j in range(L) if j <= pos and (window <= 0 or j > pos - window)
                    and (j < L - R or (j - (L - R)) in anc[r])]
            if not keys:
                rows.append([0.0] * D)
                continue
            sc = [c * math.fsum(q[r][h][d] * k[j][g][d] for d in range(D)) for j in keys]
            top = max(sc)
            w = [math.exp(x - top) for x in sc]
            tot = math.fsum(w)
            rows.append([math.fsum(w[i] * v[keys[i]][g][d] for i in range(len(keys))) / tot for d in range(D)])
        out.append(rows)
    return np.array(out)


def _tree_case(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(2, 9))
    Hkv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([1, 3, 8]))
    L = int(rng.integers(R, 30))
    window = int(rng.choice([0, 0, 2, 5]))
    parent = _random_tree(rng, R)
    anc = [_ancestor_set(parent, r) for r in range(R)]
    masks = [sum(1 << i for i in a) for a in anc]
    q = rng.standard_normal((R, Hkv * G, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    return q, k, v, L, R, anc, masks, window


def _tree_pins_pass():
    for seed in range(6):
        q, k, v, L, R, anc, masks, window = _tree_case(seed)
        got = oracle.attend_stream_tree(q, k, v, R, masks, window)
        want = brute_tree_attention(q.tolist(), k.tolist(), v.tolist(), L, R, anc, window)
        if not np.allclose(got, want, rtol=1e-12, atol=1e-13):
            return False
    return True


@pytest.mark.parametrize("seed", range(10))
def test_tree_oracle_matches_brute_force(seed):
    q, k, v, L, R, anc, masks, window = _tree_case(seed)
    got = oracle.attend_stream_tree(q, k, v, R, masks, window)
    want = brute_tree_attention(q.tolist(), k.tolist(), v.tolist(), L, R, anc, window)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_chain_tree_equals_causal_verify():
    rng = np.random.default_rng(3)
    R, L = 8, 40
    q = rng.standard_normal((R, 8, 16))
    k = rng.standard_normal((L, 2, 16))
    v = rng.standard_normal((L, 2, 16))
    chain = [(1 << (r + 1)) - 1 for r in range(R)]
    np.testing.assert_allclose(oracle.attend_stream_tree(q, k, v, R, chain), oracle.attend_stream(q, k, v, R),
                               rtol=1e-13, atol=1e-14)


def test_tree_bits_above_the_row_are_ignored():
    rng = np.random.default_rng(4)
    R, L = 6, 25
    q = rng.standard_normal((R, 4, 8))
    k = rng.standard_normal((L, 1, 8))
    v = rng.standard_normal((L, 1, 8))
    everything = [0xFF] * R
    np.testing.assert_allclose(oracle.attend_stream_tree(q, k, v, R, everything), oracle.attend_stream(q, k, v, R),
                               rtol=1e-13, atol=1e-14)


def test_tree_row_seeing_only_itself_is_a_decode_without_the_other_drafts():
    rng = np.random.default_rng(5)
    R, L, r = 5, 30, 3
    q = rng.standard_normal((R, 4, 8))
    k = rng.standard_normal((L, 2, 8))
    v = rng.standard_normal((L, 2, 8))
    masks = [(1 << (i + 1)) - 1 for i in range(R)]
    masks[r] = 1 << r
    got = oracle.attend_stream_tree(q, k, v, R, masks)[r]
    keep = list(range(L - R)) + [L - R + r]             # the prefix and the row's own slot
    want = oracle.attend_stream(q[r:r + 1], k[keep], v[keep], 1)[0]
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-14)


def test_tree_row_with_no_visible_key_is_zero():
    q = np.ones((2, 2, 4))
    k = np.ones((2, 1, 4))
    v = np.ones((2, 1, 4))
    out = oracle.attend_stream_tree(q, k, v, 2, [0b01, 0b00])     # L == R: no prefix; row 1 sees nothing
    assert np.all(out[1] == 0) and np.allclose(out[0], 1.0)


def test_planted_reversed_tree_bits_turn_pins_red(monkeypatch):
    assert _tree_pins_pass()
    real = oatt.tree_keys

    def reversed_bits(length, rows, r, mask, window=0):
        flipped = sum(((mask >> i) & 1) << (rows - 1 - i) for i in range(rows))
        return real(length, rows, r, flipped, window)
    monkeypatch.setattr(oatt, "tree_keys", reversed_bits)
    assert not _tree_pins_pass()


def test_planted_tree_without_the_prefix_turns_pins_red(monkeypatch):
    assert _tree_pins_pass()
    real = oatt.tree_keys

    def no_prefix(length, rows, r, mask, window=0):
        return [j for j in real(length, rows, r, mask, window) if j >= length - rows]
    monkeypatch.setattr(oatt, "tree_keys", no_prefix)
    assert not _tree_pins_pass()


# ----------------------------------------------------------------------------- kept states
def test_copy_pages_then_gather_reads_the_same_stream():
    rng = np.random.default_rng(11)
    N, Hkv, P, D, L = 12, 2, 5, 3, 17
    pages = rng.standard_normal((N, Hkv, P, D))
    src = [7, 2, 9, 4]                          # the stream's table: ceil(17 / 5) = 4 pages
    dst = [0, 11, 5, 8]                         # freshly leased pages for the kept state
    before = opages.gather_linear(pages, src, L, P)
    copied = oracle.copy_pages(pages, src, dst)
    np.testing.assert_array_equal(opages.gather_linear(copied, dst, L, P), before)
    # the source pages and every page outside dst are untouched
    untouched = [i for i in range(N) if i not in dst]
    np.testing.assert_array_equal(copied[untouched], pages[untouched])


def test_copy_pages_reads_sources_before_any_write():
    pages = np.arange(4 * 1 * 2 * 1, dtype=np.float64).reshape(4, 1, 2, 1)
    out = oracle.copy_pages(pages, [0, 1], [1, 2])           # page 1 is a source and a destination
    np.testing.assert_array_equal(out[1], pages[0])
    np.testing.assert_array_equal(out[2], pages[1])          # the old page 1, not the copy of page 0
    np.testing.assert_array_equal(oracle.copy_pages(pages, [0, 9], [3, 1])[1], pages[1])   # 9 outside: skipped


# ----------------------------------------------------------------------------- contiguous leases
def _run_lease_golden(model_cls=None):
    """Drive a lease model through the hand-worked sequence of tests/golden/contiguous_leases.json
    (TensorFold PR #1620, first review: the full layers in one unbroken run of pages while the
    pool has space to spare); AssertionError on the first difference."""
    fx = json.load(open(os.path.join(os.path.dirname(GOLDEN), "contiguous_leases.json")))
    m = (model_cls or oracle.LeaseModel)(fx["num_pages"], fx["max_streams"])
    for st in fx["steps"]:
        if st["op"] == "policy":
            m.set_policy(st["policy"])
            continue
        if st["op"] == "release":
            m.release(st["stream"])
        else:
            try:
                got = m.lease(st["stream"], st["n"])
            except oracle.NoPages:
                got = "no_pages"
            assert got == st["expect"], (st, got)
        if "free_after" in st:
            assert list(m.free) == st["free_after"], (st, list(m.free))
    assert m.leased == fx["final_leased"]


def test_contiguous_leases_follow_the_hand_worked_sequence():
    _run_lease_golden()


def _has_run(free, n):
    free = set(free)
    return any(all(a + k in free for k in range(n)) for a in free)


@pytest.mark.parametrize("seed", range(4))
def test_contiguous_leases_keep_runs_while_the_pool_has_them(seed):
    rng = random.Random(100 + seed)
    N, S = 64, 6
    m = oracle.LeaseModel(N, S)
    m.set_policy("contiguous")
    for _ in range(500):
        s = rng.randrange(S)
        if rng.random() < 0.75:
            n = rng.randrange(1, 6)
            free_before = set(m.free)
            newest = m.leased[s][-1] if m.leased[s] else None
            try:
                got = m.lease(s, n)
            except oracle.NoPages:
                assert n > len(free_before)
                continue
            assert set(got) <= free_before and len(set(got)) == n
            ext = None if newest is None else list(range(newest + 1, newest + n + 1))
            if ext is not None and set(ext) <= free_before:
                assert got == ext                                   # the stream's own run grows
            elif _has_run(free_before, n):
                assert got == list(range(got[0], got[0] + n))       # still one run of adjacent ids
            else:
                assert got == sorted(free_before)[:n]
        else:
            m.release(s)
        leased = [p for lst in m.leased for p in lst]
        assert len(set(leased)) == len(leased)
        assert sorted(leased + list(m.free)) == list(range(N))


def test_interleaved_growth_in_an_empty_pool_stays_in_few_runs():
    # 4 streams grow one page at a time in turn until each holds 12 of 64 pages: the
    # placements leave each stream room behind it, so every table is a single run
    m = oracle.LeaseModel(64, 4)
    m.set_policy("contiguous")
    for _ in range(12):
        for s in range(4):
            m.lease(s, 1)
    for lst in m.leased:
        assert lst == list(range(lst[0], lst[0] + 12))


class _StartAtRunStart(oracle.LeaseModel):
    def _contiguous_ids(self, stream, n):
        mine = self.leased[stream]
        free = set(self.free)
        if mine and all(mine[-1] + k in free for k in range(1, n + 1)):
            return [mine[-1] + k for k in range(1, n + 1)]
        for a, b in sorted(self._free_runs(), key=lambda r: (-(r[1] - r[0]), r[0])):
            if b - a >= n:
                return list(range(a, a + n))
        return sorted(free)[:n]


class _TieToHighest(oracle.LeaseModel):
    def _free_runs(self):
        return list(reversed(super()._free_runs()))


class _FallbackInQueueOrder(oracle.LeaseModel):
    def _contiguous_ids(self, stream, n):
        got = super()._contiguous_ids(stream, n)
        if got == sorted(set(self.free))[:n] and not _has_run(self.free, n):
            return list(self.free)[:n]
        return got


class _NoExtension(oracle.LeaseModel):
    def _contiguous_ids(self, stream, n):
        saved = self.leased[stream]
        self.leased[stream] = []
        try:
            return super()._contiguous_ids(stream, n)
        finally:
            self.leased[stream] = saved


@pytest.mark.parametrize("cls", [_StartAtRunStart, _TieToHighest, _FallbackInQueueOrder, _NoExtension])
def test_planted_lease_mistakes_turn_the_golden_sequence_red(cls):
    with pytest.raises(AssertionError):
        _run_lease_golden(cls)
