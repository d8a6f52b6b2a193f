"""Pins for the CPU oracle: it is checked against things other than itself.

* brute-force dense causal softmax attention in float64 (when k covers every
  block, MSA is exactly dense causal attention);
* a brute-force lexsort over exactly computed block maxima (integer inputs make
  every float32 sum exact, and produce many ties);
* closed forms: planted index keys with a known selection, all-tie inputs whose
  selection is {0..m-1}, uniform attention whose output is a block average;
* invariances: exact rescaling of Q_idx, decode = last prefill row, ragged
  packing = independent sequences, attention independent of id order;
* the figure's head -> index-query mapping (tests/golden).
"""
import json
import os

import numpy as np
import pytest

from block_sparse_gqa_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def make(seqlens_q, seqlens_k, H, h, d, di, B, k, q=None, kk=None, v=None, q_idx=None, k_idx=None, seed=0):
    """Inputs of arbitrary shape; any tensor not given is drawn N(0,1)."""
    base = synth.custom(seqlens_q, seqlens_k, H, h, d, di, B, k, seed=seed)
    for name, val in (("q", q), ("k", kk), ("v", v), ("q_idx", q_idx), ("k_idx", k_idx)):
        if val is not None:
            bits = synth.f32_to_bf16_bits(np.asarray(val, np.float32))
            assert np.array_equal(synth.bf16_bits_to_f32(bits), np.asarray(val, np.float32)), \
                "test values must be exact in bf16"
            setattr(base, name, bits.reshape(getattr(base, name).shape))
    return base


def f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def dense_causal_reference(inp):
    """Textbook causal GQA softmax attention in float64 (bottom-right aligned)."""
    wl = inp.wl
    H, h, d = wl.num_heads, wl.num_kv_heads, wl.head_dim
    G = H // h
    q, k, v = f64(inp.q), f64(inp.k), f64(inp.v)
    out = np.zeros((wl.total_q, H, d))
    lse = np.zeros((wl.total_q, H))
    for s in range(len(wl.seqlens_q)):
        q0, q1 = inp.cu_seqlens_q[s], inp.cu_seqlens_q[s + 1]
        k0, k1 = inp.cu_seqlens_k[s], inp.cu_seqlens_k[s + 1]
        lq, lk = q1 - q0, k1 - k0
        for r in range(lq):
            p = lk - lq + r
            for head in range(H):
                g = head // G
                logits = k[k0:k0 + p + 1, g, :] @ q[q0 + r, head, :] * wl.scale
                m = logits.max()
                w = np.exp(logits - m)
                out[q0 + r, head] = w @ v[k0:k0 + p + 1, g, :] / w.sum()
                lse[q0 + r, head] = m + np.log(w.sum())
    return out, lse


def bruteforce_topk(inp):
    """Exact block maxima (float64 of integer-valued products) and a full lexsort."""
    wl = inp.wl
    h, B, K = wl.num_kv_heads, wl.block_size, wl.top_k
    qi, ki = f64(inp.q_idx), f64(inp.k_idx)
    ids = np.full((wl.total_q, h, K), -1, np.int32)
    kth = np.full((wl.total_q, h, 2), np.nan)
    for s in range(len(wl.seqlens_q)):
        q0, q1 = inp.cu_seqlens_q[s], inp.cu_seqlens_q[s + 1]
        k0, k1 = inp.cu_seqlens_k[s], inp.cu_seqlens_k[s + 1]
        lq, lk = q1 - q0, k1 - k0
        for r in range(lq):
            p = lk - lq + r
            E = p // B + 1
            for g in range(h):
                sc = ki[k0:k0 + p + 1] @ qi[q0 + r, g]
                S = np.array([sc[j * B:min((j + 1) * B, p + 1)].max() for j in range(E)])
                order = np.lexsort((np.arange(E), -S))
                m = min(K, E)
                ids[q0 + r, g, :m] = np.sort(order[:m])
                if E > K:
                    kth[q0 + r, g] = S[order[K - 1]], S[order[K]]
    return ids, kth


DENSE_CASES = [
    # seqlens_q, seqlens_k, H, h, d, d_idx, B
    ((200,), (200,), 4, 4, 32, 16, 16),
    ((130, 77, 93), (130, 77, 93), 6, 2, 64, 32, 64),
    ((64, 65), (64, 65), 8, 2, 16, 8, 16),
    ((1, 1, 1), (150, 64, 1), 8, 2, 32, 16, 64),
    ((5, 40), (45, 40), 3, 1, 16, 16, 16),
]


@pytest.mark.parametrize("case", DENSE_CASES)
def test_equals_dense_attention_when_k_covers_all_blocks(oracle_lib, case):
    sq, sk, H, h, d, di, B = case
    nblk = max(sk) // B + 1
    inp = make(sq, sk, H, h, d, di, B, nblk + 2, seed=7)
    ids, _, _ = oracle_lib.index_topk(inp)
    out, lse = oracle_lib.sparse_attention(inp, ids)
    ref, ref_lse = dense_causal_reference(inp)
    np.testing.assert_allclose(out, ref, rtol=1e-5, atol=2e-6)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-6, atol=1e-5)


@pytest.mark.parametrize("case", [((300,), (300,), 2, 8, 16, 3), ((97, 1, 160), (97, 33, 160), 3, 4, 16, 5),
                                  ((1, 1), (500, 257), 2, 8, 32, 7)])
def test_topk_equals_bruteforce_lexsort(oracle_lib, case):
    sq, sk, h, di, B, K = case
    rng = np.random.default_rng(3)
    tq, tk = sum(sq), sum(sk)
    q_idx = rng.integers(-3, 4, size=(tq, h, di)).astype(np.float32)
    k_idx = rng.integers(-3, 4, size=(tk, di)).astype(np.float32)
    inp = make(sq, sk, h * 2, h, 16, di, B, K, q_idx=q_idx, k_idx=k_idx)
    ids, kth, tie = oracle_lib.index_topk(inp)
    ref_ids, ref_kth = bruteforce_topk(inp)
    np.testing.assert_array_equal(ids, ref_ids)
    np.testing.assert_array_equal(np.isnan(kth), np.isnan(ref_kth))
    m = ~np.isnan(ref_kth)
    np.testing.assert_array_equal(kth[m], ref_kth[m].astype(np.float32))
    a, b = ref_kth[..., 0], ref_kth[..., 1]
    with np.errstate(invalid="ignore"):
        ref_tie = (a - b) <= 1e-3 * np.maximum(np.abs(a), np.abs(b))
    np.testing.assert_array_equal(tie, np.where(np.isnan(a), False, ref_tie))
    assert tie.any(), "integer scores should produce exact ties"


@pytest.mark.parametrize("case", [((300,), (300,), 2, 8, 16), ((97, 1, 160), (97, 33, 160), 3, 4, 16),
                                  ((1, 1), (500, 257), 2, 8, 32), ((70,), (70,), 1, 4, 64)])
def test_block_scores_equal_bruteforce_maxima(oracle_lib, case):
    """The oracle's Block Max Pool of one (row, group), value by value, against exact block maxima of
    integer-valued scores (so float64 and float32 agree exactly): causal rows, a diagonal block cut at
    the row's position, partial last blocks, decode rows and ragged packing.  Scores of 0 must come
    back as +0.0 whatever the sign of the products' zero."""
    sq, sk, h, di, B = case
    rng = np.random.default_rng(11)
    tq, tk = sum(sq), sum(sk)
    q_idx = rng.integers(-3, 4, size=(tq, h, di)).astype(np.float32)
    k_idx = rng.integers(-3, 4, size=(tk, di)).astype(np.float32)
    k_idx[::5] = -0.0                     # rows of negative zeros: products -0.0 * x
    inp = make(sq, sk, h * 2, h, 16, di, B, 2, q_idx=q_idx, k_idx=k_idx)
    qi, ki = f64(inp.q_idx), f64(inp.k_idx)
    checked = 0
    for s in range(len(sq)):
        q0, k0 = inp.cu_seqlens_q[s], inp.cu_seqlens_k[s]
        lq, lk = sq[s], sk[s]
        for r in range(lq):
            p = lk - lq + r
            for g in range(h):
                sc = ki[k0:k0 + p + 1] @ qi[q0 + r, g]
                ref = np.array([sc[j * B:min((j + 1) * B, p + 1)].max() for j in range(p // B + 1)])
                got = oracle_lib.block_scores(inp, int(q0 + r), g)
                np.testing.assert_array_equal(got, ref.astype(np.float32))
                assert not np.signbit(got[got == 0]).any()
                checked += 1
    assert checked == tq * h


def _planted(n, h, B, K, values, di=8):
    """Q_idx[., g] = e_g; K_idx zero except one planted token per (group, block)."""
    q_idx = np.zeros((n, h, di), np.float32)
    for g in range(h):
        q_idx[:, g, g] = 1.0
    k_idx = np.zeros((n, di), np.float32)
    offs = {}
    for (g, j), val in values.items():
        t = j * B + (7 * j + 3 * g) % B
        assert t < n
        k_idx[t, g] = val
        offs[(g, j)] = t
    return q_idx, k_idx, offs


def test_planted_selection_closed_form(oracle_lib):
    n, h, B, K = 640, 2, 32, 4
    nblk = n // B
    rng = np.random.default_rng(5)
    values = {}
    for g in range(h):
        for j in range(nblk):
            if (j + g) % 3 == 0:
                values[(g, j)] = float(rng.choice(np.arange(1, 200)))  # exact in bf16
    q_idx, k_idx, offs = _planted(n, h, B, K, values)
    inp = make((n,), (n,), h * 3, h, 16, 8, B, K, q_idx=q_idx, k_idx=k_idx)
    ids, _, _ = oracle_lib.index_topk(inp)
    for p in range(n):
        E = p // B + 1
        for g in range(h):
            visible = [(val, j) for (gg, j), val in values.items() if gg == g and offs[(gg, j)] <= p]
            visible.sort(key=lambda x: (-x[0], x[1]))
            chosen = [j for _, j in visible[:K]]
            zeros = [j for j in range(E) if j not in {jj for _, jj in visible}]
            chosen += zeros[:max(0, min(K, E) - len(chosen))]
            expect = sorted(chosen) + [-1] * (K - min(K, E))
            assert list(ids[p, g]) == expect, (p, g)


def test_all_ties_select_lowest_ids_including_signed_zeros(oracle_lib):
    n, h, B, K, di = 260, 2, 16, 5, 8
    q_idx = -np.ones((n, h, di), np.float32)
    q_idx[:, 1, :] = 1.0
    k_idx = np.zeros((n, di), np.float32)
    inp = make((n,), (n,), 4, h, 16, di, B, K, q_idx=q_idx, k_idx=k_idx)
    # half of the blocks hold -0.0 index keys, so scores are a mix of +0.0 and -0.0
    kb = inp.k_idx.copy()
    for j in range(0, n // B + 1, 2):
        kb[j * B:(j + 1) * B] = 0x8000
    inp.k_idx = kb
    ids, _, tie = oracle_lib.index_topk(inp)
    for p in range(n):
        E = p // B + 1
        m = min(K, E)
        assert list(ids[p, 0]) == list(range(m)) + [-1] * (K - m)
        assert list(ids[p, 1]) == list(range(m)) + [-1] * (K - m)
    assert tie[K * B:].all()
    # constant non-zero index keys: every block score is identical
    inp2 = make((n,), (n,), 4, h, 16, di, B, K, q_idx=np.ones((n, h, di), np.float32),
                k_idx=np.full((n, di), 0.5, np.float32))
    ids2, _, _ = oracle_lib.index_topk(inp2)
    np.testing.assert_array_equal(ids2, ids)


def test_exact_rescaling_of_index_query_keeps_selection(oracle_lib):
    inp = synth.custom((700,), (700,), 8, 4, 16, 32, 32, 6, seed=11)
    ids, _, _ = oracle_lib.index_topk(inp)
    doubled = synth.f32_to_bf16_bits(2.0 * synth.bf16_bits_to_f32(inp.q_idx))
    inp.q_idx = doubled
    ids2, _, _ = oracle_lib.index_topk(inp)
    np.testing.assert_array_equal(ids, ids2)


def test_selection_invariants_and_group_sharing(oracle_lib):
    inp = synth.custom((333, 190), (333, 190), 12, 4, 32, 16, 16, 7, seed=2)
    ids, _, _ = oracle_lib.index_topk(inp)
    for row in range(inp.wl.total_q):
        s = 0 if row < 333 else 1
        p = row - inp.cu_seqlens_q[s]
        E = p // 16 + 1
        m = min(7, E)
        for g in range(4):
            sel = ids[row, g]
            assert (sel[m:] == -1).all()
            assert (np.diff(sel[:m]) > 0).all()
            assert sel[0] >= 0 and sel[m - 1] < E
    # heads of one group see exactly that group's blocks: with Q = 0 every visible
    # token of the selection gets the same weight, and V = block id makes the
    # output the mean block id of the group's selection.
    wl = inp.wl
    tok_block = np.concatenate([np.arange(n) // 16 for n in wl.seqlens_k]).astype(np.float32)
    v = np.repeat(tok_block[:, None, None], 4, axis=1).repeat(32, axis=2)
    v = v + np.arange(4, dtype=np.float32)[None, :, None] * 32.0   # < 256: exact in bf16
    inp.v = synth.f32_to_bf16_bits(v)
    inp.q = np.zeros_like(inp.q)
    out, _ = oracle_lib.sparse_attention(inp, ids)
    for row in (0, 17, 200, 332, 333 + 100, 333 + 189):
        s = 0 if row < 333 else 1
        p = row - inp.cu_seqlens_q[s]
        for head in range(12):
            g = head // 3
            toks = [t for j in ids[row, g] if j >= 0 for t in range(j * 16, min(j * 16 + 16, p + 1))]
            expect = np.mean([t // 16 for t in toks]) + 32.0 * g
            np.testing.assert_allclose(out[row, head], expect, rtol=1e-5)


def test_figure_head_to_index_query_mapping(oracle_lib):
    with open(os.path.join(GOLDEN, "figure_gqa_6_heads_2_index_queries.json")) as f:
        fig = json.load(f)
    H, h = fig["num_heads"], fig["num_index_queries"]
    n, B, K = 256, 32, 2
    # group 0 plants its keys in blocks {1, 5}, group 1 in blocks {2, 6}
    values = {(0, 1): 9.0, (0, 5): 8.0, (1, 2): 9.0, (1, 6): 8.0}
    q_idx, k_idx, _ = _planted(n, h, B, K, values)
    v = np.zeros((n, h, 16), np.float32)
    v[:, :, 0] = (np.arange(n) // B)[:, None]
    inp = make((n,), (n,), H, h, 16, 8, B, K, q_idx=q_idx, k_idx=k_idx,
               q=np.zeros((n, H, 16), np.float32), v=v)
    ids, _, _ = oracle_lib.index_topk(inp)
    assert list(ids[n - 1, 0]) == [1, 5] and list(ids[n - 1, 1]) == [2, 6]
    out, _ = oracle_lib.sparse_attention(inp, ids)
    mean_block = {0: 3.0, 1: 4.0}   # uniform weights over two full blocks
    for head in range(H):
        assert out[n - 1, head, 0] == pytest.approx(mean_block[fig["selection_of_head"][head]])


def test_decode_equals_last_prefill_row(oracle_lib):
    n = 517
    pre = synth.custom((n,), (n,), 8, 2, 64, 32, 64, 3, seed=4)
    ids, _, _ = oracle_lib.index_topk(pre)
    out, lse = oracle_lib.sparse_attention(pre, ids)
    dec = synth.custom((1,), (n,), 8, 2, 64, 32, 64, 3, seed=4)
    dec.k, dec.v, dec.k_idx = pre.k, pre.v, pre.k_idx
    dec.q, dec.q_idx = pre.q[n - 1:n], pre.q_idx[n - 1:n]
    dids, _, _ = oracle_lib.index_topk(dec)
    dout, dlse = oracle_lib.sparse_attention(dec, dids)
    np.testing.assert_array_equal(dids[0], ids[n - 1])
    np.testing.assert_array_equal(dout[0], out[n - 1])
    np.testing.assert_array_equal(dlse[0], lse[n - 1])


def test_ragged_packing_equals_independent_sequences(oracle_lib):
    lens = (90, 200, 33)
    packed = synth.custom(lens, lens, 6, 3, 32, 16, 32, 4, seed=8)
    ids, _, _ = oracle_lib.index_topk(packed)
    out, _ = oracle_lib.sparse_attention(packed, ids)
    for s, n in enumerate(lens):
        a, b = packed.cu_seqlens_q[s], packed.cu_seqlens_q[s + 1]
        one = synth.custom((n,), (n,), 6, 3, 32, 16, 32, 4)
        one.q, one.k, one.v = packed.q[a:b], packed.k[a:b], packed.v[a:b]
        one.q_idx, one.k_idx = packed.q_idx[a:b], packed.k_idx[a:b]
        ids1, _, _ = oracle_lib.index_topk(one)
        out1, _ = oracle_lib.sparse_attention(one, ids1)
        np.testing.assert_array_equal(ids1, ids[a:b])
        np.testing.assert_array_equal(out1, out[a:b])


def test_attention_does_not_depend_on_id_order(oracle_lib):
    inp = synth.custom((400,), (400,), 8, 2, 64, 32, 32, 6, seed=9)
    ids, _, _ = oracle_lib.index_topk(inp)
    out, lse = oracle_lib.sparse_attention(inp, ids)
    rng = np.random.default_rng(0)
    perm = np.stack([rng.permutation(6) for _ in range(400 * 2)]).reshape(400, 2, 6)
    shuffled = np.take_along_axis(ids, perm, axis=2)
    out2, lse2 = oracle_lib.sparse_attention(inp, shuffled)
    np.testing.assert_allclose(out2, out, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(lse2, lse, rtol=1e-6)


def test_near_tie_flag(oracle_lib):
    n, h, B, K, di = 320, 2, 32, 2, 8
    # score = hi + lo, both exact in bf16, the sum exact in float32
    # group 0: k-th = 1000, (k+1)-th = 992 + 7.5 = 999.5 -> within 1e-3 relative (near tie)
    # group 1: k-th = 1000, (k+1)-th = 992              -> not a near tie
    planted = {0: {1: (1024.0, 0.0), 3: (1000.0, 0.0), 6: (992.0, 7.5)},
               1: {1: (1024.0, 0.0), 3: (1000.0, 0.0), 6: (992.0, 0.0)}}
    q_idx = np.zeros((n, h, di), np.float32)
    k_idx = np.zeros((n, di), np.float32)
    for g in range(h):
        q_idx[:, g, 2 * g] = q_idx[:, g, 2 * g + 1] = 1.0
        for j, (hi, lo) in planted[g].items():
            k_idx[j * B + 5 + g, 2 * g] = hi
            k_idx[j * B + 5 + g, 2 * g + 1] = lo
    inp = make((n,), (n,), 4, h, 16, di, B, K, q_idx=q_idx, k_idx=k_idx)
    ids, kth, tie = oracle_lib.index_topk(inp)
    last = n - 1
    assert list(ids[last, 0]) == [1, 3] and list(ids[last, 1]) == [1, 3]
    assert tie[last, 0] and not tie[last, 1]
    assert kth[last, 0, 0] == 1000.0 and kth[last, 0, 1] == 999.5
    assert kth[last, 1, 1] == 992.0


def test_oracle_rejects_ineligible_or_duplicate_ids(oracle_lib):
    inp = synth.custom((100,), (100,), 2, 1, 16, 16, 16, 2, seed=1)
    ids = np.full((100, 1, 2), -1, np.int32)
    ids[:, 0, 0] = 0
    oracle_lib.sparse_attention(inp, ids)
    bad = ids.copy()
    bad[10, 0, 1] = 5          # row 10 sees blocks 0 only
    with pytest.raises(ValueError):
        oracle_lib.sparse_attention(inp, bad)
    dup = ids.copy()
    dup[50, 0, 1] = 0
    with pytest.raises(ValueError):
        oracle_lib.sparse_attention(inp, dup)


# ---------------------------------------------------------------------------
# Forced blocks (attention-sink and local-window option; 0, 0 = plain TopK).


def bruteforce_forced(inp, sink, local):
    """Exact block maxima (float64 of integer-valued products); forced blocks,
    then a lexsort of the rest."""
    wl = inp.wl
    h, B, K = wl.num_kv_heads, wl.block_size, wl.top_k
    qi, ki = f64(inp.q_idx), f64(inp.k_idx)
    ids = np.full((wl.total_q, h, K), -1, np.int32)
    for s in range(len(wl.seqlens_q)):
        q0, q1 = inp.cu_seqlens_q[s], inp.cu_seqlens_q[s + 1]
        k0, k1 = inp.cu_seqlens_k[s], inp.cu_seqlens_k[s + 1]
        lq, lk = q1 - q0, k1 - k0
        for r in range(lq):
            p = lk - lq + r
            E = p // B + 1
            forced = sorted(set(range(min(sink, E))) | set(range(max(0, E - local), E)))
            rest = np.array([j for j in range(E) if j not in forced], np.int64)
            for g in range(h):
                sc = ki[k0:k0 + p + 1] @ qi[q0 + r, g]
                S = np.array([sc[j * B:min((j + 1) * B, p + 1)].max() for j in range(E)])
                order = rest[np.lexsort((rest, -S[rest]))] if len(rest) else rest
                m = min(K, E)
                keep = sorted(forced + order[:m - len(forced)].tolist())
                ids[q0 + r, g, :m] = keep
    return ids


@pytest.mark.parametrize("sink,local", [(1, 0), (0, 1), (1, 2), (2, 3)])
def test_forced_blocks_equal_bruteforce(oracle_lib, sink, local):
    sq, sk, h, di, B, K = (97, 1, 160), (97, 33, 160), 3, 4, 16, 5
    rng = np.random.default_rng(11)
    q_idx = rng.integers(-3, 4, size=(sum(sq), h, di)).astype(np.float32)
    k_idx = rng.integers(-3, 4, size=(sum(sk), di)).astype(np.float32)
    inp = make(sq, sk, h * 2, h, 16, di, B, K, q_idx=q_idx, k_idx=k_idx)
    ids, _, _ = oracle_lib.index_topk(inp, sink=sink, local=local)
    np.testing.assert_array_equal(ids, bruteforce_forced(inp, sink, local))


def test_forced_blocks_closed_forms(oracle_lib):
    n, h, B, K = 640, 2, 32, 4
    rng = np.random.default_rng(2)
    inp = make((n,), (n,), 4, h, 16, 8, B, K, seed=4)
    plain, _, _ = oracle_lib.index_topk(inp)
    # nothing forced: plain TopK
    np.testing.assert_array_equal(oracle_lib.index_topk(inp, sink=0, local=0)[0], plain)
    # sink + local = k: once E exceeds k the selection is the forced set, whatever the scores
    ids, kth, tie = oracle_lib.index_topk(inp, sink=1, local=3)
    for p in range(n):
        E = p // B + 1
        if E > K:
            assert list(ids[p, 0]) == [0, E - 3, E - 2, E - 1], p
            assert np.isnan(kth[p, 0]).all() and not tie[p].any()
    # planted scores on non-forced blocks: forced blocks plus the best planted ones
    values = {(g, j): float(rng.choice(np.arange(1, 200))) for g in range(h) for j in range(2, n // B - 2)}
    q_idx, k_idx, offs = _planted(n, h, B, K, values)
    inp = make((n,), (n,), h * 3, h, 16, 8, B, K, q_idx=q_idx, k_idx=k_idx)
    ids, _, _ = oracle_lib.index_topk(inp, sink=1, local=1)
    p = n - 1
    E = p // B + 1
    for g in range(h):
        ranked = sorted(((val, j) for (gg, j), val in values.items() if gg == g and 0 < j < E - 1),
                        key=lambda x: (-x[0], x[1]))
        assert list(ids[p, g]) == sorted([0, E - 1] + [j for _, j in ranked[:K - 2]])


def test_forced_blocks_invariants(oracle_lib):
    inp = make((300, 45), (300, 45), 8, 2, 32, 16, 16, 6, seed=9)
    sink, local = 2, 2
    ids, _, _ = oracle_lib.index_topk(inp, sink=sink, local=local)
    for row in range(inp.wl.total_q):
        s = 0 if row < 300 else 1
        p = row - inp.cu_seqlens_q[s]
        E = p // 16 + 1
        forced = set(range(min(sink, E))) | set(range(max(0, E - local), E))
        for g in range(2):
            sel = set(ids[row, g][ids[row, g] >= 0].tolist())
            assert forced <= sel and len(sel) == min(6, E)
            S = oracle_lib.block_scores(inp, row, g)
            kept = [S[j] for j in sel - forced]
            dropped = [S[j] for j in set(range(E)) - sel]
            if kept and dropped:
                assert min(kept) >= max(dropped)
    with pytest.raises(ValueError):
        oracle_lib.index_topk(inp, sink=4, local=3)   # more forced blocks than k


# ---------------------------------------------------------------------------
# Backward of the sparse branch (selection fixed): torch float64 autograd of
# masked softmax attention is the independent reference.


def autograd_reference(inp, ids, dout_bits, out_bits=None):
    """dq, dk, dv of sum(O * dO) for attention restricted to the visible tokens
    of each group's selected blocks, by float64 autograd (per sequence).

    With ``out_bits`` (a given forward output, bf16 bits) the loss gains
    sum_rows c * lse, where lse is the row's log-sum-exp of the scaled logits
    and c = dO.O - dO.out is held constant.  Since d lse / d s_t = P_t, this
    turns every dS_t = P_t (dP_t - dO.O) into P_t (dP_t - dO.out): the gradient
    a backward computes when it forms D from the output it is given."""
    torch = pytest.importorskip("torch")
    wl = inp.wl
    H, h, d, B = wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    G = H // h
    q = torch.tensor(f64(inp.q), requires_grad=True)
    k = torch.tensor(f64(inp.k), requires_grad=True)
    v = torch.tensor(f64(inp.v), requires_grad=True)
    dout = torch.tensor(f64(dout_bits))
    loss = 0
    for s in range(len(wl.seqlens_q)):
        q0, q1 = inp.cu_seqlens_q[s], inp.cu_seqlens_q[s + 1]
        k0, k1 = inp.cu_seqlens_k[s], inp.cu_seqlens_k[s + 1]
        lq, lk = q1 - q0, k1 - k0
        mask = np.zeros((lq, h, lk), bool)
        for r in range(lq):
            p = lk - lq + r
            for g in range(h):
                for j in ids[q0 + r, g]:
                    if j >= 0:
                        mask[r, g, j * B:min((j + 1) * B, p + 1)] = True
        m = torch.tensor(np.repeat(mask, G, axis=1))                    # [lq, H, lk]
        kk = k[k0:k1].repeat_interleave(G, dim=1)                       # [lk, H, d]
        vv = v[k0:k1].repeat_interleave(G, dim=1)
        logits = torch.einsum("rhd,thd->rht", q[q0:q1], kk) * wl.scale
        logits = logits.masked_fill(~m, float("-inf"))
        p_ = torch.softmax(logits, dim=-1)
        o = torch.einsum("rht,thd->rhd", p_, vv)
        loss = loss + (o * dout[q0:q1]).sum()
        if out_bits is not None:
            given = torch.tensor(f64(out_bits[q0:q1]))
            c = ((o.detach() - given) * dout[q0:q1]).sum(dim=-1)            # [lq, H]
            loss = loss + (c * torch.logsumexp(logits, dim=-1)).sum()
    loss.backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


BWD_CASES = [
    # seqlens_q, seqlens_k, H, h, d, d_idx, B, k
    ((130, 77), (130, 77), 6, 2, 32, 16, 16, 3),     # sparse, ragged, partial blocks, G = 3
    ((96,), (96,), 4, 4, 16, 16, 16, 8),             # k covers every block: dense causal, G = 1
    ((1, 40), (70, 60), 8, 2, 16, 8, 16, 2),          # a decode row and a chunk with prior context
]


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward_equals_autograd(oracle_lib, case):
    sq, sk, H, h, d, di, B, K = case
    inp = make(sq, sk, H, h, d, di, B, K, seed=13)
    ids, _, _ = oracle_lib.index_topk(inp)
    rng = np.random.default_rng(4)
    dout = synth.f32_to_bf16_bits(rng.standard_normal(inp.q.shape).astype(np.float32))
    dq, dk, dv = oracle_lib.sparse_attention_backward(inp, ids, dout)
    rq, rk, rv = autograd_reference(inp, ids, dout)
    for got, ref, name in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        np.testing.assert_allclose(got, ref, rtol=2e-4, atol=2e-5 * np.abs(ref).max(), err_msg=name)


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward_with_given_output_equals_autograd(oracle_lib, case):
    """The backward handed the forward's output rounded to bf16 (as a caller passes it) forms
    D = dO.out from it; autograd of sum(O dO) + sum c lse with c = dO.(O - out) is the same
    gradient.  The rounding must also change the result (the given output is really used)."""
    sq, sk, H, h, d, di, B, K = case
    inp = make(sq, sk, H, h, d, di, B, K, seed=17)
    ids, _, _ = oracle_lib.index_topk(inp)
    o, _ = oracle_lib.sparse_attention(inp, ids)
    out_bits = synth.f32_to_bf16_bits(o.astype(np.float32))
    rng = np.random.default_rng(6)
    dout = synth.f32_to_bf16_bits(rng.standard_normal(inp.q.shape).astype(np.float32))
    got = oracle_lib.sparse_attention_backward(inp, ids, dout, out=out_bits)
    ref = autograd_reference(inp, ids, dout, out_bits=out_bits)
    for g_, r_, name in zip(got, ref, ("dq", "dk", "dv")):
        np.testing.assert_allclose(g_, r_, rtol=2e-4, atol=2e-5 * np.abs(r_).max(), err_msg=name)
    exact = oracle_lib.sparse_attention_backward(inp, ids, dout)
    assert not np.array_equal(exact[0], got[0])
    np.testing.assert_array_equal(exact[2], got[2])    # dv does not involve D


def test_backward_untouched_tokens_get_zero(oracle_lib):
    """Tokens no row selects (and rows' unselected blocks) receive zero dk/dv."""
    inp = make((200,), (200,), 4, 2, 16, 8, 16, 1, seed=2)
    ids, _, _ = oracle_lib.index_topk(inp)
    dout = synth.f32_to_bf16_bits(np.random.default_rng(1).standard_normal(inp.q.shape).astype(np.float32))
    _, dk, dv = oracle_lib.sparse_attention_backward(inp, ids, dout)
    for g in range(2):
        used = np.zeros(200, bool)
        for r in range(200):
            j = ids[r, g, 0]
            used[j * 16:min(j * 16 + 16, r + 1)] = True
        assert not dk[~used, g].any() and not dv[~used, g].any()
        assert dv[used, g].any()
