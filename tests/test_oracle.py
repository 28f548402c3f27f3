"""Pins for the float64 oracle: facts that do not come from the oracle itself.

Each test ties an oracle function to a hand-derived fixture, a closed form, a
library routine or an invariant of the method, so that a dropped term, a wrong
sign or index, or a transposed operand inside the oracle fails at least one of
them (tests/test_oracle_mutations.py plants such mistakes and checks that).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (copy_blocks_ref, decode_gqa_ref, decode_ref, gather_sequence_kv, swap_blocks_ref,
                    lse_merge_ref, reshape_and_cache_ref, split_decode_ref)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers that build paged inputs WITHOUT the oracle's gather: contiguous
# per-sequence K/V are generated first, then written block by block into the
# pool at table-chosen physical ids (the inverse mapping, written block-wise).
# --------------------------------------------------------------------------

def _paged_from_contiguous(Kc, Vc, lens, num_blocks, bs, rng, poison=np.nan):
    """Kc, Vc: lists (per sequence) of [H, L_s, D] float64 arrays."""
    S = len(Kc)
    H, D = Kc[0].shape[0], Kc[0].shape[2]
    need = [-(-L // bs) for L in lens]
    width = max(1, max(need))
    ids = rng.permutation(num_blocks)
    assert sum(need) <= num_blocks
    tables = -np.ones((S, width), dtype=np.int64)
    k_pool = np.full((num_blocks, H, bs, D), poison)
    v_pool = np.full((num_blocks, H, bs, D), poison)
    cursor = 0
    for s in range(S):
        for j in range(need[s]):
            p = ids[cursor]
            cursor += 1
            tables[s, j] = p
            lo = j * bs
            hi = min(lo + bs, lens[s])
            k_pool[p, :, : hi - lo, :] = Kc[s][:, lo:hi, :]
            v_pool[p, :, : hi - lo, :] = Vc[s][:, lo:hi, :]
    return k_pool, v_pool, tables


def _random_case(seed, lens=(1, 7, 16, 33), H=3, D=8, bs=4, spare=5):
    rng = np.random.default_rng(seed)
    Kc = [rng.standard_normal((H, L, D)) for L in lens]
    Vc = [rng.standard_normal((H, L, D)) for L in lens]
    q = rng.standard_normal((len(lens), H, D))
    nb = sum(-(-L // bs) for L in lens) + spare
    k_pool, v_pool, tables = _paged_from_contiguous(Kc, Vc, list(lens), nb, bs, rng)
    return q, Kc, Vc, k_pool, v_pool, tables, np.array(lens), bs


# --------------------------------------------------------------------------
# hand-worked fixture
# --------------------------------------------------------------------------

def _load_golden():
    with open(os.path.join(GOLDEN, "decode_hand_worked.json")) as f:
        return json.load(f)


def test_golden_hand_worked_cases():
    g = _load_golden()
    k_pool = np.array(g["k_pool"], dtype=np.float64)
    v_pool = np.array(g["v_pool"], dtype=np.float64)
    tables = np.array(g["block_tables"])
    lens = np.array(g["context_lens"])
    for case in g["cases"]:
        q = np.array(case["q"], dtype=np.float64)
        out = decode_ref(q, k_pool, v_pool, tables, lens, case["scale"], g["block_size"])
        np.testing.assert_allclose(out, np.array(case["expected"]), rtol=0, atol=1e-12,
                                   err_msg=case["name"])


def test_golden_gather_order():
    g = _load_golden()
    k_pool = np.array(g["k_pool"], dtype=np.float64)
    v_pool = np.array(g["v_pool"], dtype=np.float64)
    K, V = gather_sequence_kv(k_pool, v_pool, g["block_tables"][0], 3, 0, g["block_size"])
    np.testing.assert_array_equal(K, [[1, 0], [0, 1], [-1, -1]])
    np.testing.assert_array_equal(V, [[1, 2], [3, 4], [5, 9]])


# --------------------------------------------------------------------------
# library routine: contiguous attention (torch SDPA, float64, CPU)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_sdpa_on_contiguous_cache(seed):
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(seed)
    scale = 0.37
    out = decode_ref(q, k_pool, v_pool, tables, lens, scale, bs)
    for s, L in enumerate(lens):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[s][:, None, :]),          # [H, 1, D]
            torch.from_numpy(np.ascontiguousarray(Kc[s])),  # [H, L, D]
            torch.from_numpy(np.ascontiguousarray(Vc[s])),
            scale=scale)[:, 0, :].numpy()
        np.testing.assert_allclose(out[s], ref, rtol=0, atol=1e-12)
        assert np.all(np.isfinite(out[s]))


def test_gather_round_trip_of_blockwise_scatter():
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(5)
    for s, L in enumerate(lens):
        for h in range(Kc[s].shape[0]):
            K, V = gather_sequence_kv(k_pool, v_pool, tables[s], L, h, bs)
            np.testing.assert_array_equal(K, Kc[s][h])
            np.testing.assert_array_equal(V, Vc[s][h])


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_single_token_returns_its_value_row_exactly():
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(3, lens=(1, 1, 1))
    out = decode_ref(q, k_pool, v_pool, tables, lens, 1.3, bs)
    for s in range(3):
        np.testing.assert_array_equal(out[s], Vc[s][:, 0, :])


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(11)
    H, D, bs, L = 2, 6, 4, 13
    key = rng.standard_normal((H, 1, D))
    Kc = [np.repeat(key, L, axis=1)]
    Vc = [rng.standard_normal((H, L, D))]
    k_pool, v_pool, tables = _paged_from_contiguous(Kc, Vc, [L], 8, bs, rng)
    q = rng.standard_normal((1, H, D))
    out = decode_ref(q, k_pool, v_pool, tables, [L], 0.9, bs)
    np.testing.assert_allclose(out[0], Vc[0].mean(axis=1), rtol=0, atol=1e-14)


def test_zero_scale_gives_mean_of_values():
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(4)
    out = decode_ref(q, k_pool, v_pool, tables, lens, 0.0, bs)
    for s in range(len(lens)):
        np.testing.assert_allclose(out[s], Vc[s].mean(axis=1), rtol=0, atol=1e-14)


def test_two_tokens_logistic_closed_form():
    rng = np.random.default_rng(12)
    H, D, bs = 2, 5, 16
    Kc = [rng.standard_normal((H, 2, D))]
    Vc = [rng.standard_normal((H, 2, D))]
    k_pool, v_pool, tables = _paged_from_contiguous(Kc, Vc, [2], 3, bs, rng)
    q = rng.standard_normal((1, H, D))
    scale = 0.61
    out = decode_ref(q, k_pool, v_pool, tables, [2], scale, bs)
    for h in range(H):
        z1 = scale * float(np.dot(q[0, h], Kc[0][h, 0]))
        z2 = scale * float(np.dot(q[0, h], Kc[0][h, 1]))
        a = 1.0 / (1.0 + math.exp(z2 - z1))   # logistic(z1 - z2)
        b = 1.0 / (1.0 + math.exp(z1 - z2))
        np.testing.assert_allclose(out[0, h], a * Vc[0][h, 0] + b * Vc[0][h, 1],
                                   rtol=0, atol=1e-14)


def test_dominant_score_selects_its_row_and_stays_finite():
    # Scores near 1e4: without the max subtraction exp() would overflow.
    rng = np.random.default_rng(13)
    H, D, bs, L = 1, 4, 4, 9
    Kc = [rng.standard_normal((H, L, D)) * 0.01]
    Kc[0][0, 6] = np.array([100.0, 0, 0, 0])
    Vc = [rng.standard_normal((H, L, D))]
    k_pool, v_pool, tables = _paged_from_contiguous(Kc, Vc, [L], 4, bs, rng)
    q = np.array([[[100.0, 0, 0, 0]]])
    out = decode_ref(q, k_pool, v_pool, tables, [L], 1.0, bs)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out[0, 0], Vc[0][0, 6], rtol=0, atol=1e-12)


def test_empty_context_gives_zero_row():
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(6)
    lens = lens.copy()
    lens[2] = 0
    out = decode_ref(q, k_pool, v_pool, tables, lens, 0.5, bs)
    np.testing.assert_array_equal(out[2], 0.0)
    assert np.all(np.isfinite(out))


# --------------------------------------------------------------------------
# invariants of paging
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1])
def test_physical_block_permutation_is_invisible(seed):
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(seed)
    base = decode_ref(q, k_pool, v_pool, tables, lens, 0.5, bs)
    rng = np.random.default_rng(100 + seed)
    perm = rng.permutation(k_pool.shape[0])      # new position of old block b is perm[b]
    k2 = np.empty_like(k_pool)
    v2 = np.empty_like(v_pool)
    k2[perm] = k_pool
    v2[perm] = v_pool
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    out = decode_ref(q, k2, v2, t2, lens, 0.5, bs)
    np.testing.assert_array_equal(out, base)


def test_shared_prefix_equals_private_copies():
    rng = np.random.default_rng(21)
    H, D, bs = 2, 8, 4
    prefix_blocks = 3
    S = 4
    suffix = [0, 1, 5, 8]
    nb = prefix_blocks + sum(-(-n // bs) for n in suffix) + S * prefix_blocks + 2
    k_pool = np.full((nb, H, bs, D), np.nan)
    v_pool = np.full((nb, H, bs, D), np.nan)
    k_pool[:prefix_blocks] = rng.standard_normal((prefix_blocks, H, bs, D))
    v_pool[:prefix_blocks] = rng.standard_normal((prefix_blocks, H, bs, D))
    width = prefix_blocks + 2
    shared = -np.ones((S, width), dtype=np.int64)
    private = -np.ones((S, width), dtype=np.int64)
    nxt = prefix_blocks
    for s in range(S):
        shared[s, :prefix_blocks] = np.arange(prefix_blocks)
        for j in range(prefix_blocks):          # private copy of every prefix block
            k_pool[nxt] = k_pool[j]
            v_pool[nxt] = v_pool[j]
            private[s, j] = nxt
            nxt += 1
        for j in range(-(-suffix[s] // bs)):
            k_pool[nxt] = rng.standard_normal((H, bs, D))
            v_pool[nxt] = rng.standard_normal((H, bs, D))
            shared[s, prefix_blocks + j] = nxt
            private[s, prefix_blocks + j] = nxt
            nxt += 1
    lens = np.array([prefix_blocks * bs + n for n in suffix])
    q = rng.standard_normal((S, H, D))
    a = decode_ref(q, k_pool, v_pool, shared, lens, 0.4, bs)
    b = decode_ref(q, k_pool, v_pool, private, lens, 0.4, bs)
    np.testing.assert_array_equal(a, b)
    assert np.all(np.isfinite(a))


def test_poisoned_tail_and_unreferenced_blocks_do_not_matter():
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(7)   # poison = NaN already
    out = decode_ref(q, k_pool, v_pool, tables, lens, 0.5, bs)
    assert np.all(np.isfinite(out))
    k_inf = np.where(np.isnan(k_pool), np.inf, k_pool)
    v_inf = np.where(np.isnan(v_pool), -np.inf, v_pool)
    out2 = decode_ref(q, k_inf, v_inf, tables, lens, 0.5, bs)
    np.testing.assert_array_equal(out, out2)


def test_torch_storage_dtypes_upcast_exactly():
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(8)
    for dt in (torch.float16, torch.bfloat16, torch.float32):
        kt = torch.from_numpy(k_pool).to(dt)
        vt = torch.from_numpy(v_pool).to(dt)
        qt = torch.from_numpy(q).to(dt)
        out_t = decode_ref(qt, kt, vt, torch.from_numpy(tables).int(), torch.from_numpy(lens).int(), 0.5, bs)
        out_n = decode_ref(qt.double().numpy(), kt.double().numpy(), vt.double().numpy(), tables, lens, 0.5, bs)
        np.testing.assert_array_equal(out_t, out_n)


# --------------------------------------------------------------------------
# split-context log-sum-exp merge
# --------------------------------------------------------------------------

@pytest.mark.parametrize("P", [4, 8, 12, 32, 64])
def test_split_decode_equals_unsplit(P):
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(9, lens=(1, 5, 17, 40, 63))
    ref = decode_ref(q, k_pool, v_pool, tables, lens, 0.8, bs)
    out, parts = split_decode_ref(q, k_pool, v_pool, tables, lens, 0.8, bs, P)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    for s, L in enumerate(lens):
        assert len(parts[s][0]) == -(-int(L) // P)


def test_lse_merge_single_partial_is_identity_and_empty_is_none():
    o = np.array([0.25, -1.5, 3.0])
    np.testing.assert_array_equal(lse_merge_ref([(2.0, 5.0, o)]), o)
    assert lse_merge_ref([]) is None
    np.testing.assert_array_equal(lse_merge_ref([(1.0, 0.0, o * 9), (7.0, 2.0, o)]), o)


def test_lse_merge_two_partials_closed_form():
    # partition A: one token with score a; partition B: one token with score b.
    a, b = 3.0, -1.0
    va, vb = np.array([1.0, 0.0]), np.array([0.0, 1.0])
    got = lse_merge_ref([(a, 1.0, va), (b, 1.0, vb)])
    wa = 1.0 / (1.0 + math.exp(b - a))
    np.testing.assert_allclose(got, wa * va + (1 - wa) * vb, rtol=0, atol=1e-15)


def test_split_rejects_bad_partition():
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(0)
    with pytest.raises(ValueError):
        split_decode_ref(q, k_pool, v_pool, tables, lens, 1.0, bs, 6)


# --------------------------------------------------------------------------
# cache writes and block copies
# --------------------------------------------------------------------------

def test_reshape_and_cache_hand_slots_read_back_in_order():
    # table [5, 2, 7] with block_size 4: tokens 0..9 go to these slots (by hand)
    slots = [20, 21, 22, 23, 8, 9, 10, 11, 28, 29]
    H, D, bs, nb = 2, 3, 4, 9
    rng = np.random.default_rng(30)
    k_pool = torch.full((nb, H, bs, D), float("nan"), dtype=torch.float16)
    v_pool = torch.full((nb, H, bs, D), float("nan"), dtype=torch.float16)
    k_new = torch.from_numpy(rng.standard_normal((10, H, D))).half()
    v_new = torch.from_numpy(rng.standard_normal((10, H, D))).half()
    k2, v2 = reshape_and_cache_ref(k_pool, v_pool, k_new, v_new, slots, bs)
    for h in range(H):
        K, V = gather_sequence_kv(k2, v2, [5, 2, 7], 10, h, bs)
        np.testing.assert_array_equal(K, k_new[:, h].double().numpy())
        np.testing.assert_array_equal(V, v_new[:, h].double().numpy())
    # every byte not written stays as it was (NaN here), inputs unmodified
    written = torch.zeros((nb, bs), dtype=torch.bool)
    for s in slots:
        written[s // bs, s % bs] = True
    assert torch.isnan(k2.permute(0, 2, 1, 3)[~written]).all()
    assert torch.isnan(k_pool).all()


def test_reshape_and_cache_negative_slot_writes_nothing():
    H, D, bs, nb = 1, 2, 2, 3
    k_pool = torch.zeros((nb, H, bs, D), dtype=torch.float32)
    v_pool = torch.zeros((nb, H, bs, D), dtype=torch.float32)
    k_new = torch.ones((2, H, D))
    v_new = torch.ones((2, H, D)) * 2
    k2, v2 = reshape_and_cache_ref(k_pool, v_pool, k_new, v_new, [-1, 5], bs)
    assert k2.sum() == 2 and v2.sum() == 4
    assert (k2[2, 0, 1] == 1).all() and (v2[2, 0, 1] == 2).all()


def test_copy_blocks_bytes_and_isolation():
    rng = np.random.default_rng(31)
    nb, H, bs, D = 6, 2, 4, 3
    k_pool = torch.from_numpy(rng.standard_normal((nb, H, bs, D))).to(torch.bfloat16)
    v_pool = torch.from_numpy(rng.standard_normal((nb, H, bs, D))).to(torch.bfloat16)
    mapping = [[1, 4], [1, 5], [0, 2]]
    k2, v2 = copy_blocks_ref(k_pool, v_pool, mapping)
    for src, dst in mapping:
        assert torch.equal(k2[dst].view(torch.int16), k_pool[src].view(torch.int16))
        assert torch.equal(v2[dst].view(torch.int16), v_pool[src].view(torch.int16))
    for b in (0, 1, 3):
        assert torch.equal(k2[b].view(torch.int16), k_pool[b].view(torch.int16))
        assert torch.equal(v2[b].view(torch.int16), v_pool[b].view(torch.int16))


def test_copy_on_write_keeps_decode_bit_identical():
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(32, spare=8)
    before = decode_ref(q, k_pool, v_pool, tables, lens, 0.5, bs)
    used = set(int(x) for x in tables.ravel() if x >= 0)
    free = [b for b in range(k_pool.shape[0]) if b not in used]
    # privatise logical block 0 of sequences 1 and 3 into fresh blocks
    mapping = [[int(tables[1, 0]), free[0]], [int(tables[3, 0]), free[1]]]
    k2, v2 = copy_blocks_ref(k_pool, v_pool, mapping)
    t2 = tables.copy()
    t2[1, 0] = free[0]
    t2[3, 0] = free[1]
    after = decode_ref(q, k2, v2, t2, lens, 0.5, bs)
    np.testing.assert_array_equal(after, before)


def test_swap_out_and_back_restores_the_cache_and_the_decode():
    """Swapping sequence 2's blocks out to a host pool, reusing its device
    blocks for other data, then swapping them back (into different device
    blocks, with the table repointed) leaves decode bit-identical."""
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(33, spare=8)
    before = decode_ref(q, k_pool, v_pool, tables, lens, 0.5, bs)
    nb = -(-int(lens[2]) // bs)
    blocks = [int(b) for b in tables[2, :nb]]
    host_k = np.zeros((nb + 3,) + k_pool.shape[1:])
    host_v = np.zeros((nb + 3,) + v_pool.shape[1:])
    out_map = [[b, i + 1] for i, b in enumerate(blocks)]  # host slots 1..nb
    hk, hv = swap_blocks_ref(host_k, host_v, k_pool, v_pool, out_map)
    for src, dst in out_map:
        assert np.array_equal(hk[dst], k_pool[src]) and np.array_equal(hv[dst], v_pool[src])
    assert not hk[0].any() and not hk[nb + 1:].any()       # untouched host slots
    # the device blocks are overwritten, then the data comes back elsewhere
    used = set(int(x) for x in tables.ravel() if x >= 0)
    free = [b for b in range(k_pool.shape[0]) if b not in used][:nb]
    k2, v2 = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    k2[blocks] = np.nan
    v2[blocks] = np.nan
    in_map = [[1 + i, f] for i, f in enumerate(free)]
    k3, v3 = swap_blocks_ref(k2, v2, hk, hv, in_map)
    t2 = tables.copy()
    t2[2, :nb] = free
    after = decode_ref(q, k3, v3, t2, lens, 0.5, bs)
    np.testing.assert_array_equal(after, before)


@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 3), (8, 2), (3, 3)])
def test_gqa_decode_matches_torch_sdpa_with_grouped_heads(H, Hkv):
    """torch's scaled_dot_product_attention with enable_gqa (float64, on the
    contiguous cache) is an independent implementation of grouped heads."""
    rng = np.random.default_rng(40 + H + Hkv)
    lens = [1, 9, 20]
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(41, lens=lens, H=Hkv, D=8, bs=4)
    q = rng.standard_normal((len(lens), H, 8))
    out = decode_gqa_ref(q, k_pool, v_pool, tables, lens, 0.6, bs)
    for s, L in enumerate(lens):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[s][None, :, None, :]), torch.from_numpy(Kc[s][None]),
            torch.from_numpy(Vc[s][None]), scale=0.6, enable_gqa=True)[0, :, 0, :].numpy()
        np.testing.assert_allclose(out[s], ref, rtol=0, atol=1e-12)


def test_gqa_decode_equals_mha_decode_on_repeated_heads():
    q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(42, H=2, D=8, bs=4)
    q4 = np.random.default_rng(43).standard_normal((len(lens), 6, 8))
    got = decode_gqa_ref(q4, k_pool, v_pool, tables, lens, 0.3, bs)
    want = decode_ref(q4, np.repeat(k_pool, 3, axis=1), np.repeat(v_pool, 3, axis=1), tables, lens, 0.3, bs)
    np.testing.assert_array_equal(got, want)
    # one query head per K/V head is plain decode
    np.testing.assert_array_equal(decode_gqa_ref(q, k_pool, v_pool, tables, lens, 0.3, bs),
                                  decode_ref(q, k_pool, v_pool, tables, lens, 0.3, bs))
    with pytest.raises(ValueError):
        decode_gqa_ref(q4[:, :5], k_pool, v_pool, tables, lens, 0.3, bs)
