"""Pins for the CPU oracle: checks against facts fixed outside the oracle.

Each test pins the oracle to something other than itself: hand-derived worked
examples (tests/golden), a textbook special case written with complex
arithmetic, closed forms, invariants the pages' identity implies, brute-force
index enumeration, and torch / numpy rounding routines.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rope_complex(x, theta, pos):
    """RoPE as complex multiplication: (x_i + i x_{i+D/2}) * exp(i pos theta^(-2i/D))."""
    x = np.asarray(x, np.float64)
    h = x.shape[-1] // 2
    z = x[..., :h] + 1j * x[..., h:]
    w = theta ** (-2.0 * np.arange(h) / x.shape[-1])
    z = z * np.exp(1j * pos * w)
    return np.concatenate([z.real, z.imag], axis=-1)


def textbook_decode(q, K, V):
    """o = softmax(q K^T / sqrt(d)) V for one query row (MagicPIG notes, sec. 3 definition)."""
    s = K @ q / math.sqrt(q.shape[0])
    p = np.exp(s - s.max())
    return (p / p.sum()) @ V


def _golden_pool(g):
    """Pack a golden example's blocks into a one-head plane + one-worker table."""
    D = g["D"]
    Ks, Vs, starts, lens, tb, to = [], [], [], [], [], []
    slot = 0
    for blk in g["blocks"]:
        n = len(blk["K"])
        starts.append(slot)
        lens.append(n)
        Ks += blk["K"]
        Vs += blk["V"]
        tb.append(blk["id"])
        to.append(blk["view_offset"])
        slot += n
    K = np.array(Ks, np.float64).reshape(-1, D)
    V = np.array(Vs, np.float64).reshape(-1, D)
    return K, V, np.array(starts, np.int64), np.array(lens, np.int32), np.array(tb), np.array(to)


@pytest.mark.parametrize("name", ["hand_d2_two_blocks.json", "hand_d4_pairing.json"])
@pytest.mark.parametrize("form", [oracle.FORM_DEFINITION, oracle.FORM_METHOD])
def test_hand_examples(name, form):
    g = _load(name)
    K, V, starts, lens, tb, to = _golden_pool(g)
    out, rc = oracle.attn_one(form, np.array(g["q"]), K, V, tb, to, lens, starts, g["theta"])
    assert rc == oracle.HWO_OK
    np.testing.assert_allclose(out, g["expected_out"], rtol=0, atol=2e-10)


def test_hand_example_values_match_closed_form():
    g = _load("hand_d4_pairing.json")
    s = [math.sin(2) / 2, math.sin(1) / 2, 1.0]
    e = [math.exp(x) for x in s]
    np.testing.assert_allclose(s, g["expected_scores"], atol=1e-10)
    np.testing.assert_allclose([x / sum(e) for x in e] + [0.0], g["expected_out"], atol=1e-10)
    g = _load("hand_d2_two_blocks.json")
    s = [math.cos(1) / math.sqrt(2), 1 / math.sqrt(2)]
    e = [math.exp(x) for x in s]
    np.testing.assert_allclose(s, g["expected_scores"], atol=1e-10)
    np.testing.assert_allclose([x / sum(e) for x in e], g["expected_out"], atol=1e-10)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(1)
    for D, theta, pos in [(2, 10.0, 3.0), (8, 1e4, 17.0), (64, 1e4, 383.0), (128, 1e6, 50001.0),
                          (128, 1e6, -7.0)]:
        x = rng.standard_normal(D)
        # fp64 angle pos*w carries ~|pos| * 1e-16 of rounding on either route
        np.testing.assert_allclose(oracle.rope(x, theta, pos), rope_complex(x, theta, pos),
                                   rtol=0, atol=1e-13 * max(1.0, abs(pos)))


def test_alice_bob_tables():
    g = _load("alice_bob_tables.json")
    tb, to, ne = oracle.build_combined_tables(g["common_block"], g["worker_block"], g["block_len"])
    assert tb.tolist() == g["expected_tbl_block"]
    assert to.tolist() == g["expected_tbl_off"]
    assert ne.tolist() == g["expected_num_entries"]
    for w in range(2):
        assert oracle.query_position(tb[w], to[w], g["block_len"]) == g["expected_query_position"][w]


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8])
def test_tables_cover_the_view_without_gaps(W):
    rng = np.random.default_rng(100 + W)
    for trial in range(20):
        nb = W + 1 + int(rng.integers(0, 3))
        lens = rng.integers(0, 50, size=nb).astype(np.int32)
        ids = rng.permutation(nb)
        common, workers = int(ids[0]), ids[1:W + 1].astype(np.int32)
        tb, to, ne = oracle.build_combined_tables(common, workers, lens)
        assert (ne == W + 1).all()
        for w in range(W):
            row = tb[w].tolist()
            assert row[0] == common and to[w][0] == 0
            assert row[-1] == workers[w]
            assert row[1:-1] == [int(workers[v]) for v in range(W) if v != w]
            ends = to[w] + lens[tb[w]]
            assert (to[w][1:] == ends[:-1]).all()            # contiguous, no overlap
            assert ends[-1] == lens[[common] + list(workers)].sum()
            iq = oracle.query_position(tb[w], to[w], lens)
            nonempty = lens[tb[w]] > 0
            assert iq == (ends[nonempty].max() - 1 if nonempty.any() else -1)


def test_table_errors():
    with pytest.raises(ValueError):
        oracle.build_combined_tables(0, [1, 1], [3, 3, 3])      # same block twice
    with pytest.raises(ValueError):
        oracle.build_combined_tables(0, [0, 1], [3, 3, 3])      # worker block == common
    with pytest.raises(ValueError):
        oracle.build_combined_tables(0, [1, 5], [3, 3, 3])      # id out of range


def _random_view(rng, nblocks, D, maxlen=40, start_pad=3):
    lens = rng.integers(1, maxlen, size=nblocks).astype(np.int32)
    starts = np.zeros(nblocks, np.int64)
    slot = start_pad
    for b in range(nblocks):
        starts[b] = slot
        slot += int(lens[b]) + int(rng.integers(0, 5))
    S = slot + 2
    return lens, starts, S


@pytest.mark.parametrize("seed", range(6))
def test_definition_equals_method_form(seed):
    """The pages' identity: rotating the query by i_q - i_k equals re-encoding every key."""
    rng = np.random.default_rng(seed)
    D = [2, 8, 64, 128][seed % 4]
    theta = [1e4, 1e6][seed % 2]
    W, Hkv, G = 1 + seed % 3, 1 + seed % 2, 1 + (seed * 7) % 3
    Hq = Hkv * G
    nb = W + 1
    lens, starts, S = _random_view(rng, nb, D)
    tb, to, ne = oracle.build_combined_tables(0, np.arange(1, W + 1), lens)
    q = rng.standard_normal((W, Hq, D))
    K = rng.standard_normal((Hkv, S, D)) + rng.normal(0, 0.5, (Hkv, 1, D))
    V = rng.standard_normal((Hkv, S, D))
    od, rc1 = oracle.attn_decode(oracle.FORM_DEFINITION, q, K, V, tb, to, ne, lens, starts, theta)
    om, rc2 = oracle.attn_decode(oracle.FORM_METHOD, q, K, V, tb, to, ne, lens, starts, theta)
    assert rc1 == rc2 == oracle.HWO_OK
    assert np.abs(od - om).max() <= 1e-12 * max(1.0, np.abs(om).max())


@pytest.mark.parametrize("form", [oracle.FORM_DEFINITION, oracle.FORM_METHOD])
def test_one_block_is_textbook_decode_with_gqa(form):
    """One worker, one block at offset 0: ordinary decode with the query at L-1."""
    rng = np.random.default_rng(7)
    D, Hkv, G, L, theta = 16, 2, 3, 37, 1e4
    Hq = Hkv * G
    S, start = 50, 5
    K = rng.standard_normal((Hkv, S, D))
    V = rng.standard_normal((Hkv, S, D))
    q = rng.standard_normal((1, Hq, D))
    out, rc = oracle.attn_decode(form, q, K, V, [[0]], [[0]], [1], np.array([L], np.int32),
                                 np.array([start], np.int64), theta)
    assert rc == oracle.HWO_OK
    for h in range(Hq):
        g = h // G  # contiguous groups of q-heads share a kv head
        ref = textbook_decode(rope_complex(q[0, h], theta, L - 1), K[g, start:start + L],
                              V[g, start:start + L])
        np.testing.assert_allclose(out[0, h], ref, rtol=0, atol=1e-12)


def test_single_visible_token_returns_its_value_exactly():
    rng = np.random.default_rng(3)
    D = 8
    K = rng.standard_normal((1, 10, D))
    V = rng.standard_normal((1, 10, D))
    lens = np.array([0, 1, 0], np.int32)
    starts = np.array([0, 4, 7], np.int64)
    for form in (0, 1):
        out, rc = oracle.attn_decode(form, rng.standard_normal((1, 1, D)), K, V, [[0, 1, 2]],
                                     [[0, 0, 1]], [3], lens, starts, 1e4)
        assert rc == 0
        assert (out[0, 0] == V[0, 4]).all()


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(4)
    D = 16
    lens, starts, S = _random_view(rng, 3, D)
    K = rng.standard_normal((1, S, D))
    V = rng.standard_normal((1, S, D))
    tb, to, ne = oracle.build_combined_tables(0, [1, 2], lens)
    out, rc = oracle.attn_decode(1, np.zeros((2, 1, D)), K, V, tb, to, ne, lens, starts, 1e6)
    assert rc == 0
    vis = np.concatenate([V[0, starts[b]:starts[b] + lens[b]] for b in range(3)])
    np.testing.assert_allclose(out[0, 0], vis.mean(0), atol=1e-13)
    np.testing.assert_allclose(out[1, 0], vis.mean(0), atol=1e-13)


@pytest.mark.parametrize("form", [0, 1])
def test_shifting_every_offset_changes_nothing(form):
    rng = np.random.default_rng(5)
    D = 32
    lens, starts, S = _random_view(rng, 4, D)
    K = rng.standard_normal((2, S, D))
    V = rng.standard_normal((2, S, D))
    q = rng.standard_normal((3, 4, D))
    tb, to, ne = oracle.build_combined_tables(0, [1, 2, 3], lens)
    a, _ = oracle.attn_decode(form, q, K, V, tb, to, ne, lens, starts, 1e4)
    b, _ = oracle.attn_decode(form, q, K, V, tb, to + 1234, ne, lens, starts, 1e4)
    assert np.abs(a - b).max() <= 1e-10


def test_table_entry_order_is_irrelevant():
    rng = np.random.default_rng(6)
    D = 32
    lens, starts, S = _random_view(rng, 4, D)
    K = rng.standard_normal((1, S, D))
    V = rng.standard_normal((1, S, D))
    q = rng.standard_normal((3, 2, D))
    tb, to, ne = oracle.build_combined_tables(0, [1, 2, 3], lens)
    a, _ = oracle.attn_decode(1, q, K, V, tb, to, ne, lens, starts, 1e6)
    perm = [3, 0, 2, 1]
    b, _ = oracle.attn_decode(1, q, K, V, tb[:, perm], to[:, perm], ne, lens, starts, 1e6)
    assert np.abs(a - b).max() <= 1e-13


def test_large_logit_selects_that_token():
    rng = np.random.default_rng(8)
    D, theta = 16, 1e4
    lens = np.array([20, 9], np.int32)
    starts = np.array([0, 32], np.int64)
    K = rng.standard_normal((1, 64, D))
    V = rng.standard_normal((1, 64, D))
    q = rng.standard_normal(D)
    # view: block 0 at 0, block 1 at 20 -> i_q = 28; make token 5 of block 0 dominate
    delta = 28 - 0
    qr = rope_complex(q, theta, delta)
    K[0, 5] = 1000.0 * math.sqrt(D) * qr / (qr @ qr)
    out, rc = oracle.attn_one(1, q, K[0], V[0], [0, 1], [0, 20], lens, starts, theta)
    assert rc == 0
    np.testing.assert_allclose(out, V[0, 5], atol=1e-9)


def test_no_visible_token_and_duplicates_are_errors():
    D = 4
    K = np.zeros((1, 8, D))
    out, rc = oracle.attn_one(1, np.ones(D), K[0], K[0], [0, 1], [0, 0], np.array([0, 0], np.int32),
                              np.array([0, 4], np.int64), 1e4)
    assert rc == oracle.HWO_ENOTOKENS and (out == 0).all()
    _, rc = oracle.attn_one(1, np.ones(D), K[0], K[0], [0, 0], [0, 3], np.array([3, 3], np.int32),
                            np.array([0, 4], np.int64), 1e4)
    assert rc == oracle.HWO_EINVAL


def test_round_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(9)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
    ])
    # exact ties: 1 + (2k+1) 2^-8 and their negatives
    ties = np.array([(1 + (2 * k + 1) * 2.0 ** -8) * s for k in range(64) for s in (1, -1)],
                    np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.round_bf16(float(v)) for v in x])
    assert (got == ref).all()


def test_round_bf16_is_single_rounding_from_double():
    # 1 + 2^-8 + 2^-30 lies just above a bf16 tie: correct rounding goes up.
    # Going through float32 first would drop 2^-30 and round the tie to even (down).
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.round_bf16(x) == 1.0 + 2.0 ** -7
    assert oracle.round_f32(1.0 + 2.0 ** -30) == 1.0
    assert oracle.round_f32(1.0 + 2.0 ** -23) == 1.0 + 2.0 ** -23


def _append_fixture(rng, dtype_round):
    L, Hkv, D, S = 2, 2, 8, 96
    starts = np.array([0, 32, 64], np.int64)
    caps = np.array([32, 32, 32], np.int32)
    lens = np.array([11, 7, 5], np.int32)
    K = np.vectorize(dtype_round)(rng.standard_normal((L, Hkv, S, D)))
    # V encodes (layer, head, slot, dim) so every move is visible bit for bit
    l, g, s, d = np.meshgrid(np.arange(L), np.arange(Hkv), np.arange(S), np.arange(D),
                             indexing="ij")
    V = (l * 1_000_000 + g * 10_000 + s * 10 + d).astype(np.float64)
    return L, Hkv, D, S, starts, caps, lens, K, V


@pytest.mark.parametrize("dtype", [oracle.HWO_BF16, oracle.HWO_F32])
def test_append_moves_and_rerotates(dtype):
    rnd = oracle.round_bf16 if dtype == oracle.HWO_BF16 else oracle.round_f32
    rng = np.random.default_rng(10)
    L, Hkv, D, S, starts, caps, lens, K, V = _append_fixture(rng, rnd)
    K0, V0, lens0 = K.copy(), V.copy(), lens.copy()
    theta, src, dst = 1e4, 2, 0
    rc = oracle.block_append(K, V, starts, caps, lens, src, dst, theta, dtype)
    assert rc == oracle.HWO_OK
    assert lens.tolist() == [16, 7, 0]
    ld, ls = int(lens0[dst]), int(lens0[src])
    moved = np.zeros(S, bool)
    moved[starts[dst] + ld: starts[dst] + ld + ls] = True
    # every untouched slot is bit-identical
    assert (K[:, :, ~moved] == K0[:, :, ~moved]).all()
    assert (V[:, :, ~moved] == V0[:, :, ~moved]).all()
    # V is copied exactly to slot len_dst + j
    for j in range(ls):
        assert (V[:, :, starts[dst] + ld + j] == V0[:, :, starts[src] + j]).all()
    # K: the key stored at local j now sits at local ld + j, i.e. rotated by ld,
    # and is the correctly rounded value of the exact rotation
    half_ulp = 2.0 ** -9 if dtype == oracle.HWO_BF16 else 2.0 ** -24
    for j in range(ls):
        exact = rope_complex(K0[:, :, starts[src] + j], theta, ld)
        got = K[:, :, starts[dst] + ld + j]
        assert (np.abs(got - exact) <= half_ulp * 2.0 ** np.ceil(np.log2(np.abs(exact))) + 0).all()
        assert (np.vectorize(rnd)(got) == got).all()


def test_append_review_invariant():
    """A src block right after common in worker v's view: attention is unchanged by the append."""
    rng = np.random.default_rng(11)
    D, Hkv, Hq, theta = 32, 2, 4, 1e4
    S = 160
    starts = np.array([0, 64, 128], np.int64)   # common, worker0, worker1
    caps = np.array([64, 32, 32], np.int32)
    lens = np.array([21, 9, 13], np.int32)
    K = np.vectorize(oracle.round_f32)(rng.standard_normal((1, Hkv, S, D)))
    V = rng.standard_normal((1, Hkv, S, D))
    q = rng.standard_normal((2, Hq, D))
    tb, to, ne = oracle.build_combined_tables(0, [1, 2], lens)
    # worker 0's view is [common, worker1, worker0]: worker1's block follows common
    before, _ = oracle.attn_decode(1, q, K[0], V[0], tb, to, ne, lens, starts, theta)
    rc = oracle.block_append(K, V, starts, caps, lens, 2, 0, theta, oracle.HWO_F32)
    assert rc == 0 and lens.tolist() == [34, 9, 0]
    tb2, to2, ne2 = oracle.build_combined_tables(0, [1, 2], lens)
    after, _ = oracle.attn_decode(1, q, K[0], V[0], tb2, to2, ne2, lens, starts, theta)
    np.testing.assert_allclose(after[0], before[0], rtol=0, atol=2e-6)
    # the definition form agrees as well
    after_d, _ = oracle.attn_decode(0, q, K[0], V[0], tb2, to2, ne2, lens, starts, theta)
    np.testing.assert_allclose(after_d[0], before[0], rtol=0, atol=2e-6)


def test_append_errors():
    rng = np.random.default_rng(12)
    L, Hkv, D, S, starts, caps, lens, K, V = _append_fixture(rng, oracle.round_f32)
    assert oracle.block_append(K, V, starts, caps, lens, 1, 1, 1e4, 0) == oracle.HWO_EINVAL
    assert oracle.block_append(K, V, starts, caps, lens, 1, 3, 1e4, 0) == oracle.HWO_EINVAL
    lens[0] = 30
    K0 = K.copy()
    assert oracle.block_append(K, V, starts, caps, lens, 1, 0, 1e4, 0) == oracle.HWO_ECAPACITY
    assert (K == K0).all() and lens.tolist() == [30, 7, 5]


# ------------------------------------------------------- token write (a new token)
@pytest.mark.parametrize("dtype", [oracle.HWO_F32, oracle.HWO_BF16])
def test_token_write_encodes_at_local_position(dtype):
    """The new token's key lands in slot len-1 of its block encoded at that local
    position (key design 1), correctly rounded; its value rounded; nothing else moves."""
    rnd = oracle.round_bf16 if dtype == oracle.HWO_BF16 else oracle.round_f32
    rng = np.random.default_rng(20)
    Hkv, D, theta = 2, 16, 1e4
    starts = np.array([0, 64, 96], np.int64)
    lens = np.array([40, 5, 17], np.int32)
    S = 128
    K = np.vectorize(rnd)(rng.standard_normal((Hkv, S, D)))
    V = np.vectorize(rnd)(rng.standard_normal((Hkv, S, D)))
    K0, V0 = K.copy(), V.copy()
    blocks = np.array([2, 1], np.int32)
    kn = rng.standard_normal((2, Hkv, D))
    vn = rng.standard_normal((2, Hkv, D))
    assert oracle.block_write(K, V, starts, lens, blocks, kn, vn, theta, dtype) == oracle.HWO_OK
    assert lens.tolist() == [40, 5, 17]
    written = np.zeros(S, bool)
    half_ulp = 2.0 ** -9 if dtype == oracle.HWO_BF16 else 2.0 ** -24
    for i, b in enumerate(blocks):
        slot = starts[b] + lens[b] - 1
        written[slot] = True
        exact = rope_complex(kn[i], theta, lens[b] - 1)
        got = K[:, slot]
        assert (np.abs(got - exact) <= half_ulp * 2.0 ** np.ceil(np.log2(np.abs(exact)))).all()
        assert (np.vectorize(rnd)(got) == got).all()
        if dtype == oracle.HWO_F32:
            assert (got == exact.astype(np.float32)).all()  # numpy's own rounding to nearest even
            assert (V[:, slot] == vn[i].astype(np.float32)).all()
        else:
            assert (np.abs(V[:, slot] - vn[i]) <= half_ulp * 2.0 ** np.ceil(np.log2(np.abs(vn[i])))).all()
    assert (K[:, ~written] == K0[:, ~written]).all() and (V[:, ~written] == V0[:, ~written]).all()


def test_tokens_written_one_by_one_attend_like_textbook_decode():
    """Build one block by writing raw keys token by token (advance, then write);
    attention of one worker with one block at offset 0 is textbook decode over
    the raw keys with RoPE at absolute positions 0..n-1 and the query at n-1."""
    rng = np.random.default_rng(21)
    Hkv, D, theta, n = 1, 8, 1e4, 23
    starts = np.array([0], np.int64)
    S = 32
    K = np.zeros((Hkv, S, D))
    V = np.zeros((Hkv, S, D))
    lens = np.array([0], np.int32)
    raw_k = rng.standard_normal((n, D))
    raw_v = rng.standard_normal((n, D))
    for t in range(n):
        lens[0] += 1  # the slot reserved for token t
        rc = oracle.block_write(K, V, starts, lens, np.array([0], np.int32), raw_k[t][None, None],
                                raw_v[t][None, None], theta, oracle.HWO_F32)
        assert rc == oracle.HWO_OK
    q = rng.standard_normal(D)
    tb, to, ne = np.array([[0]], np.int32), np.array([[0]], np.int32), np.array([1], np.int32)
    got, rc = oracle.attn_one(oracle.FORM_METHOD, q, K[0], V[0], tb[0], to[0], lens, starts, theta)
    assert rc == 0
    Kabs = np.stack([rope_complex(raw_k[t], theta, t) for t in range(n)])
    ref = textbook_decode(rope_complex(q, theta, n - 1), Kabs, V[0, :n])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-6)


def test_token_write_errors():
    K = np.zeros((1, 32, 8))
    V = np.zeros((1, 32, 8))
    starts = np.array([0], np.int64)
    one = np.ones((1, 1, 8))
    assert oracle.block_write(K, V, starts, np.array([3], np.int32), np.array([1], np.int32), one,
                              one, 1e4, 0) == oracle.HWO_EINVAL
    assert oracle.block_write(K, V, starts, np.array([0], np.int32), np.array([0], np.int32), one,
                              one, 1e4, 0) == oracle.HWO_ENOTOKENS
    assert (K == 0).all() and (V == 0).all()


# ------------------------------------------------- interleaved layout (NEXT-2)
def test_interleaved_tables_hand_example():
    """Step-level sync only (the notes' layout ablation): each worker sees the
    common history and its own block, nothing of the others' current steps."""
    tb, to, ne = oracle.build_interleaved_tables(0, [1, 2], np.array([10, 3, 4], np.int32))
    assert ne.tolist() == [2, 2]
    assert tb[:, :2].tolist() == [[0, 1], [0, 2]]
    assert to[:, :2].tolist() == [[0, 10], [0, 10]]


def test_interleaved_equals_combined_with_other_steps_empty():
    """Worker w's interleaved view is its combined view with every other
    worker's current block emptied (empty blocks add no tokens and no offset)."""
    rng = np.random.default_rng(30)
    D, Hkv, Hq, theta, W = 16, 2, 4, 1e4, 3
    starts = np.array([0, 64, 96, 128], np.int64)
    lens = np.array([50, 7, 19, 12], np.int32)
    S = 160
    K = rng.standard_normal((Hkv, S, D))
    V = rng.standard_normal((Hkv, S, D))
    q = rng.standard_normal((W, Hq, D))
    tb, to, ne = oracle.build_interleaved_tables(0, [1, 2, 3], lens)
    inter, rc = oracle.attn_decode(1, q, K, V, tb, to, ne, lens, starts, theta)
    assert rc == 0
    for w in range(W):
        l2 = lens.copy()
        for v in range(W):
            if v != w:
                l2[1 + v] = 0
        tb2, to2, ne2 = oracle.build_combined_tables(0, [1, 2, 3], l2)
        comb, rc = oracle.attn_decode(1, q, K, V, tb2, to2, ne2, l2, starts, theta)
        assert rc == 0
        np.testing.assert_allclose(inter[w], comb[w], rtol=0, atol=1e-12)


# ------------------------------------------------- multi-token query chunks (NEXT-3)
def test_chunk_of_one_token_is_decode():
    rng = np.random.default_rng(40)
    D, Hkv, Hq, theta = 16, 2, 4, 1e4
    starts = np.array([0, 64, 96], np.int64)
    lens = np.array([50, 9, 13], np.int32)
    K = rng.standard_normal((Hkv, 128, D))
    V = rng.standard_normal((Hkv, 128, D))
    q = rng.standard_normal((2, Hq, D))
    tb, to, ne = oracle.build_combined_tables(0, [1, 2], lens)
    dec, rc = oracle.attn_decode(1, q, K, V, tb, to, ne, lens, starts, theta)
    ch, rc2 = oracle.attn_chunk(1, q[:, None], K, V, tb, to, ne, lens, starts, theta)
    assert rc == 0 and rc2 == 0
    assert np.array_equal(ch[:, 0], dec)


@pytest.mark.parametrize("form", [0, 1])
def test_chunk_row_equals_decode_on_the_truncated_view(form):
    """Row j of a chunk of n sits lag = n-1-j tokens before the end of its
    worker's own block (the last entry of a combined view): it equals decode
    on the same view with that block shortened by lag."""
    rng = np.random.default_rng(41)
    D, Hkv, Hq, theta, n = 16, 2, 4, 1e4, 5
    starts = np.array([0, 64, 96], np.int64)
    lens = np.array([40, 11, 14], np.int32)
    K = rng.standard_normal((Hkv, 128, D))
    V = rng.standard_normal((Hkv, 128, D))
    q = rng.standard_normal((2, n, Hq, D))
    tb, to, ne = oracle.build_combined_tables(0, [1, 2], lens)
    ch, rc = oracle.attn_chunk(form, q, K, V, tb, to, ne, lens, starts, theta)
    assert rc == 0
    for w in range(2):
        for j in range(n):
            l2 = lens.copy()
            l2[1 + w] -= n - 1 - j
            tb2, to2, ne2 = oracle.build_combined_tables(0, [1, 2], l2)
            ref, rc = oracle.attn_decode(form, q[:, j], K, V, tb2, to2, ne2, l2, starts, theta)
            assert rc == 0
            np.testing.assert_allclose(ch[w, j], ref[w], rtol=0, atol=1e-12)


def test_chunk_one_block_is_causal_textbook_attention():
    """One worker, one block at offset 0, the last n tokens as queries: row j
    is textbook attention with RoPE at absolute positions over tokens
    0..L-n+j (a causal mask)."""
    rng = np.random.default_rng(42)
    D, theta, L, n = 8, 1e4, 30, 6
    raw = rng.standard_normal((L, D))
    K = np.stack([rope_complex(raw[t], theta, t) for t in range(L)])[None]  # stored at local t
    V = rng.standard_normal((1, L + 2, D))
    K = np.concatenate([K, np.zeros((1, 2, D))], axis=1)
    q = rng.standard_normal((1, n, 1, D))
    lens = np.array([L], np.int32)
    tb, to, ne = np.zeros((1, 1), np.int32), np.zeros((1, 1), np.int32), np.array([1], np.int32)
    got, rc = oracle.attn_chunk(1, q, K, V, tb, to, ne, lens, np.array([0], np.int64), theta)
    assert rc == 0
    for j in range(n):
        p = L - n + j
        Kabs = np.stack([rope_complex(raw[t], theta, t) for t in range(p + 1)])
        ref = textbook_decode(rope_complex(q[0, j, 0], theta, p), Kabs, V[0, :p + 1])
        np.testing.assert_allclose(got[0, j, 0], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------- FP8 E4M3 pools (NEXT-4)
def _e4m3_table():
    """Every finite non-negative E4M3 value with its code (codes 0x00..0x7e)."""
    return [(c, oracle.e4m3_value(c)) for c in range(0x7f)]


def test_e4m3_codes_match_torch():
    """All 256 codes decode as torch's float8_e4m3fn (a library routine) does."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2  # 0x7f and 0xff
    assert (got[~nan] == ref[~nan]).all()
    assert oracle.e4m3_value(0x7e) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6 and oracle.e4m3_value(0x38) == 1.0


def _nearest_even_brute(x, table):
    """Nearest value by exhaustive search; equidistant candidates go to the even code."""
    a = abs(x)
    best = None
    for c, v in table:
        d = abs(a - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c, v)
    v = min(best[2], 448.0)
    return math.copysign(v, x) if v != 0.0 else math.copysign(0.0, x)


def test_round_e4m3_brute_force():
    rng = np.random.default_rng(30)
    table = _e4m3_table()
    xs = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.uniform(-4, 2.6, 3000),
        rng.uniform(-448, 448, 500),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 300),       # subnormal range
    ])
    for x in xs:
        assert oracle.round_e4m3(float(x)) == _nearest_even_brute(float(x), table), x


def test_round_e4m3_ties_and_saturation():
    table = _e4m3_table()
    for (c0, v0), (c1, v1) in zip(table[:-1], table[1:]):
        mid = (v0 + v1) / 2.0  # exact in double
        want = v0 if c0 % 2 == 0 else v1
        assert oracle.round_e4m3(mid) == want and oracle.round_e4m3(-mid) == -want
    # past the largest finite value: 464 is the tie between 448 (even code) and
    # 480 (not representable); larger magnitudes saturate to 448
    for x, want in [(448.0, 448.0), (464.0, 448.0), (465.0, 448.0), (1e9, 448.0),
                    (-500.0, -448.0), (math.inf, 448.0), (2.0 ** -10, 0.0),
                    (3 * 2.0 ** -11, 2.0 ** -9)]:
        assert oracle.round_e4m3(x) == want, x
    assert math.isnan(oracle.round_e4m3(math.nan))


def test_round_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(31)
    x = np.concatenate([rng.standard_normal(20000) * 30.0, rng.standard_normal(2000) * 1e-3]
                       ).astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.round_e4m3(float(v)) for v in x])
    assert (got == ref).all()


def _fp8_grid(x, s):
    """True where every x / s is an E4M3 value."""
    r = np.vectorize(oracle.round_e4m3)(x / s)
    return (r == x / s).all()


def test_append_fp8_moves_and_rerotates():
    """FP8 pool: a moved key is s * (the E4M3 value nearest to its exact rotation / s),
    values move bit for bit, nothing else changes."""
    rng = np.random.default_rng(32)
    L, Hkv, D, S = 2, 2, 8, 96
    starts = np.array([0, 32, 64], np.int64)
    caps = np.array([32, 32, 32], np.int32)
    lens = np.array([11, 7, 5], np.int32)
    ks = np.array([[0.02, 0.05], [0.011, 0.3]])
    codes = rng.integers(0, 0x7f, (L, Hkv, S, D)) | (rng.integers(0, 2, (L, Hkv, S, D)) << 7)
    K = np.vectorize(oracle.e4m3_value)(codes) * ks[:, :, None, None]
    l, g, s, d = np.meshgrid(np.arange(L), np.arange(Hkv), np.arange(S), np.arange(D),
                             indexing="ij")
    V = (l * 1_000_000 + g * 10_000 + s * 10 + d).astype(np.float64)
    K0, V0, lens0 = K.copy(), V.copy(), lens.copy()
    theta, src, dst = 1e4, 2, 0
    assert oracle.block_append(K, V, starts, caps, lens, src, dst, theta, oracle.HWO_FP8,
                               k_scale=ks) == oracle.HWO_OK
    assert lens.tolist() == [16, 7, 0]
    ld, ls = int(lens0[dst]), int(lens0[src])
    moved = np.zeros(S, bool)
    moved[starts[dst] + ld: starts[dst] + ld + ls] = True
    assert (K[:, :, ~moved] == K0[:, :, ~moved]).all() and (V[:, :, ~moved] == V0[:, :, ~moved]).all()
    table = _e4m3_table()
    for j in range(ls):
        assert (V[:, :, starts[dst] + ld + j] == V0[:, :, starts[src] + j]).all()
        exact = rope_complex(K0[:, :, starts[src] + j], theta, ld)
        got = K[:, :, starts[dst] + ld + j]
        for li in range(L):
            for gi in range(Hkv):
                sc = ks[li, gi]
                want = [sc * _nearest_even_brute(x / sc, table) for x in exact[li, gi]]
                # the exact rotation lies off every rounding boundary here, so the
                # brute-force nearest value is the unique answer
                assert np.allclose(got[li, gi], want, rtol=0, atol=0), (j, li, gi)


def test_append_fp8_needs_positive_scales():
    rng = np.random.default_rng(33)
    L, Hkv, D, S, starts, caps, lens, K, V = _append_fixture(rng, oracle.round_f32)
    assert oracle.block_append(K, V, starts, caps, lens, 1, 0, 1e4, oracle.HWO_FP8) == oracle.HWO_EINVAL
    bad = np.array([[1.0, 0.0], [1.0, 1.0]])
    assert oracle.block_append(K, V, starts, caps, lens, 1, 0, 1e4, oracle.HWO_FP8,
                               k_scale=bad) == oracle.HWO_EINVAL


def test_token_write_fp8():
    """FP8 pool: the new key is s_k * e4m3(rho(k, p) / s_k) at slot len-1, the value
    s_v * e4m3(v / s_v), both the brute-force nearest grid values."""
    rng = np.random.default_rng(34)
    Hkv, D, theta = 2, 16, 1e4
    starts = np.array([0, 64, 96], np.int64)
    lens = np.array([40, 5, 17], np.int32)
    S = 128
    K = np.zeros((Hkv, S, D))
    V = np.zeros((Hkv, S, D))
    ks, vs = np.array([0.01, 0.04]), np.array([0.02, 0.005])
    blocks = np.array([2, 1], np.int32)
    kn = rng.standard_normal((2, Hkv, D))
    vn = rng.standard_normal((2, Hkv, D)) * 0.5
    assert oracle.block_write(K, V, starts, lens, blocks, kn, vn, theta, oracle.HWO_FP8,
                              k_scale=ks, v_scale=vs) == oracle.HWO_OK
    table = _e4m3_table()
    written = np.zeros(S, bool)
    for i, b in enumerate(blocks):
        slot = starts[b] + lens[b] - 1
        written[slot] = True
        exact = rope_complex(kn[i], theta, lens[b] - 1)
        for g in range(Hkv):
            want_k = [ks[g] * _nearest_even_brute(x / ks[g], table) for x in exact[g]]
            want_v = [vs[g] * _nearest_even_brute(x / vs[g], table) for x in vn[i, g]]
            assert (K[g, slot] == want_k).all() and (V[g, slot] == want_v).all()
    assert (K[:, ~written] == 0).all() and (V[:, ~written] == 0).all()
    assert oracle.block_write(K, V, starts, lens, blocks, kn, vn, theta, oracle.HWO_FP8,
                              k_scale=ks) == oracle.HWO_EINVAL
