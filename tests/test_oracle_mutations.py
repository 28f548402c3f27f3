"""Plant plausible mistakes in copies of the oracle and check the pins catch them.

Each mutant below is the oracle's decode / merge / cache-write arithmetic with
one deliberate slip (a swapped index, a dropped term, a flipped sign, a
transposed operand, an off-by-one).  ``_decode_pins`` runs the same kinds of
checks as tests/test_oracle.py (hand-worked fixture, torch SDPA on a
contiguous cache, a dominant score, NaN poison) against a decode function
passed in; the unmutated oracle must pass and every mutant must fail.  Runs on
the CPU only.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.paged_attention as opa
from oracle import decode_ref, lse_merge_ref, reshape_and_cache_ref, copy_blocks_ref

from test_oracle import _random_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decode_hand_worked.json")


def _decode_pins(fn) -> bool:
    """True when ``fn`` (same signature as decode_ref) passes every pin."""
    try:
        with np.errstate(all="ignore"):
            g = json.load(open(GOLDEN))
            kp = np.array(g["k_pool"], dtype=np.float64)
            vp = np.array(g["v_pool"], dtype=np.float64)
            for case in g["cases"]:
                out = fn(np.array(case["q"], dtype=np.float64), kp, vp,
                         np.array(g["block_tables"]), np.array(g["context_lens"]),
                         case["scale"], g["block_size"])
                if not np.allclose(out, case["expected"], rtol=0, atol=1e-12):
                    return False
            q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(0)
            out = fn(q, k_pool, v_pool, tables, lens, 0.37, bs)
            for s in range(len(lens)):
                ref = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(q[s][:, None, :]), torch.from_numpy(Kc[s]),
                    torch.from_numpy(Vc[s]), scale=0.37)[:, 0, :].numpy()
                if not np.allclose(out[s], ref, rtol=0, atol=1e-12):
                    return False
            # dominant score: large logits must neither overflow nor blur
            Kd = np.zeros((1, 1, 4, 2))
            Kd[0, 0, 2] = [100.0, 0.0]
            Vd = np.arange(8, dtype=np.float64).reshape(1, 1, 4, 2)
            out = fn(np.array([[[100.0, 0.0]]]), Kd, Vd, np.array([[0]]), np.array([4]), 1.0, 4)
            if not (np.all(np.isfinite(out)) and np.allclose(out[0, 0], Vd[0, 0, 2], atol=1e-12)):
                return False
        return True
    except (IndexError, ValueError, FloatingPointError, OverflowError):
        return False


# ---- mutants of decode -----------------------------------------------------

def _make_decode(score_fn=None, gather_fn=None, combine_fn=None, length_fn=None):
    def fn(q, k_pool, v_pool, block_tables, context_lens, scale, block_size):
        qf = opa._as_f64(q)
        S, H, D = qf.shape
        tables = opa._as_int(block_tables)
        lens = opa._as_int(context_lens)
        out = np.zeros((S, H, D))
        for s in range(S):
            L = int(lens[s]) if length_fn is None else length_fn(int(lens[s]))
            if L <= 0:
                continue
            for h in range(H):
                if gather_fn is None:
                    K, V = opa.gather_sequence_kv(k_pool, v_pool, tables[s], L, h, block_size)
                else:
                    K, V = gather_fn(k_pool, v_pool, tables, s, L, h, block_size)
                z = (scale * (K @ qf[s, h])) if score_fn is None else score_fn(K, qf[s, h], scale)
                if combine_fn is None:
                    w = np.exp(z - z.max())
                    out[s, h] = (w @ V) / w.sum()
                else:
                    out[s, h] = combine_fn(z, K, V)
        return out
    return fn


def _gather_swapped_index(k_pool, v_pool, tables, s, L, h, bs):
    t = np.arange(L)
    phys = tables[s][t % bs]
    rows = t // bs
    return k_pool[phys, h, rows].astype(np.float64), v_pool[phys, h, rows].astype(np.float64)


def _gather_wrong_sequence(k_pool, v_pool, tables, s, L, h, bs):
    t = np.arange(L)
    phys = tables[0][t // bs]
    return k_pool[phys, h, t % bs].astype(np.float64), v_pool[phys, h, t % bs].astype(np.float64)


def _gather_head_zero(k_pool, v_pool, tables, s, L, h, bs):
    return opa.gather_sequence_kv(k_pool, v_pool, tables[s], L, 0, bs)


DECODE_MUTANTS = {
    "block and row index swapped": _make_decode(gather_fn=_gather_swapped_index),
    "table of the wrong sequence": _make_decode(gather_fn=_gather_wrong_sequence),
    "always head 0": _make_decode(gather_fn=_gather_head_zero),
    "scale dropped": _make_decode(score_fn=lambda K, q, sc: K @ q),
    "score sign flipped": _make_decode(score_fn=lambda K, q, sc: -sc * (K @ q)),
    "scale squared": _make_decode(score_fn=lambda K, q, sc: sc * sc * (K @ q)),
    "no normalisation": _make_decode(combine_fn=lambda z, K, V: np.exp(z - z.max()) @ V),
    "no max subtraction": _make_decode(combine_fn=lambda z, K, V: (np.exp(z) @ V) / np.exp(z).sum()),
    "K used as values": _make_decode(combine_fn=lambda z, K, V: (np.exp(z - z.max()) @ K) / np.exp(z - z.max()).sum()),
    "one token too many": _make_decode(length_fn=lambda L: L + 1),
    "one token too few": _make_decode(length_fn=lambda L: L - 1),
}


def test_unmutated_oracle_passes_the_pins():
    assert _decode_pins(decode_ref)


@pytest.mark.parametrize("name", sorted(DECODE_MUTANTS))
def test_decode_mutant_is_caught(name):
    assert not _decode_pins(DECODE_MUTANTS[name]), name


# ---- mutants of the log-sum-exp merge ----------------------------------------

def _merge_pins(merge) -> bool:
    o1, o2 = np.array([1.0, 0.0]), np.array([0.0, 1.0])
    ok = np.allclose(merge([(2.0, 5.0, o1)]), o1)
    wa = 1.0 / (1.0 + math.exp(-1.0 - 3.0))
    ok &= np.allclose(merge([(3.0, 1.0, o1), (-1.0, 1.0, o2)]), wa * o1 + (1 - wa) * o2)
    # unequal l: partition A has 3 tokens of score 0, partition B 1 token of score 0
    ok &= np.allclose(merge([(0.0, 3.0, o1), (0.0, 1.0, o2)]), 0.75 * o1 + 0.25 * o2)
    return bool(ok)


def _merge_without_l(partials):
    M = max(m for m, _, _ in partials)
    return sum(math.exp(m - M) * o for m, _, o in partials) / sum(math.exp(m - M) for m, _, _ in partials)


def _merge_sign_flipped(partials):
    M = max(m for m, _, _ in partials)
    return (sum(l * math.exp(M - m) * o for m, l, o in partials)
            / sum(l * math.exp(M - m) for m, l, _ in partials))


def test_merge_pins():
    assert _merge_pins(lse_merge_ref)
    assert not _merge_pins(_merge_without_l)
    assert not _merge_pins(_merge_sign_flipped)


# ---- mutants of the cache write and block copy --------------------------------

def _reshape_pins(write) -> bool:
    slots = [20, 21, 22, 23, 8, 9, 10, 11, 28, 29]     # table [5, 2, 7], block_size 4
    H, D, bs, nb = 2, 3, 4, 9
    k = torch.zeros((nb, H, bs, D))
    v = torch.zeros((nb, H, bs, D))
    kn = torch.arange(10 * H * D, dtype=torch.float32).reshape(10, H, D) + 1
    k2, v2 = write(k, v, kn, -kn, slots, bs)
    ok = True
    for h in range(H):
        K, V = opa.gather_sequence_kv(k2, v2, [5, 2, 7], 10, h, bs)
        ok &= np.array_equal(K, kn[:, h].double().numpy())
        ok &= np.array_equal(V, -kn[:, h].double().numpy())
    return bool(ok)


def _reshape_rows_swapped(k_pool, v_pool, k_new, v_new, slots, bs):
    k, v = k_pool.clone(), v_pool.clone()
    for i, s in enumerate(slots):
        row, block = divmod(s, bs)
        if block < k.shape[0] and row < bs:
            k[block, :, row] = k_new[i]
            v[block, :, row] = v_new[i]
    return k, v


def _reshape_head0_only(k_pool, v_pool, k_new, v_new, slots, bs):
    k, v = k_pool.clone(), v_pool.clone()
    for i, s in enumerate(slots):
        b, r = divmod(s, bs)
        k[b, 0, r] = k_new[i, 0]
        v[b, 0, r] = v_new[i, 0]
    return k, v


def test_reshape_pins():
    assert _reshape_pins(reshape_and_cache_ref)
    assert not _reshape_pins(_reshape_rows_swapped)
    assert not _reshape_pins(_reshape_head0_only)


def _copy_pins(copy) -> bool:
    k = torch.arange(6 * 2 * 2 * 2, dtype=torch.float32).reshape(6, 2, 2, 2)
    v = -k
    k2, v2 = copy(k, v, [[1, 4], [0, 2]])
    return bool(torch.equal(k2[4], k[1]) and torch.equal(v2[4], v[1]) and torch.equal(k2[2], k[0])
                and torch.equal(v2[2], v[0]) and torch.equal(k2[1], k[1]) and torch.equal(k2[0], k[0]))


def _copy_reversed(k_pool, v_pool, mapping):
    return copy_blocks_ref(k_pool, v_pool, [[d, s] for s, d in mapping])


def _copy_k_only(k_pool, v_pool, mapping):
    k2, _ = copy_blocks_ref(k_pool, v_pool, mapping)
    return k2, v_pool.clone()


def test_copy_pins():
    assert _copy_pins(copy_blocks_ref)
    assert not _copy_pins(_copy_reversed)
    assert not _copy_pins(_copy_k_only)


# ---- mutants of the swap between pools ----------------------------------------

from oracle import swap_blocks_ref  # noqa: E402


def _swap_pins(swap) -> bool:
    """Out to a host pool and back into other device blocks restores the data;
    untouched destination blocks keep theirs."""
    try:
        dk = torch.arange(8 * 2 * 2 * 2, dtype=torch.float32).reshape(8, 2, 2, 2)
        dv = -dk - 1
        hk, hv = torch.zeros(4, 2, 2, 2), torch.zeros(4, 2, 2, 2)
        hk2, hv2 = swap(hk, hv, dk, dv, [[5, 1], [2, 3]])
        if not (torch.equal(hk2[1], dk[5]) and torch.equal(hv2[3], dv[2]) and not hk2[0].any()
                and not hk2[2].any()):
            return False
        dk3, dv3 = swap(dk, dv, hk2, hv2, [[1, 6], [3, 7]])
        return bool(torch.equal(dk3[6], dk[5]) and torch.equal(dv3[7], dv[2])
                    and torch.equal(dk3[:6], dk[:6]) and torch.equal(dv3[:6], dv[:6]))
    except (IndexError, RuntimeError):
        return False


def _swap_reversed(dk, dv, sk, sv, mapping):
    return swap_blocks_ref(dk, dv, sk, sv, [[d, s] for s, d in mapping])


def _swap_k_only(dk, dv, sk, sv, mapping):
    k2, _ = swap_blocks_ref(dk, dv, sk, sv, mapping)
    return k2, dv.clone()


def _swap_dst_off_by_one(dk, dv, sk, sv, mapping):
    return swap_blocks_ref(dk, dv, sk, sv, [[s, d - 1] for s, d in mapping])


def test_swap_pins():
    assert _swap_pins(swap_blocks_ref)
    for mutant in (_swap_reversed, _swap_k_only, _swap_dst_off_by_one):
        assert not _swap_pins(mutant), mutant.__name__



# ---- mutants of the grouped-query head mapping ---------------------------------

from oracle import decode_gqa_ref  # noqa: E402
from test_oracle import _random_case as _rc  # noqa: E402


def _gqa_pins(fn) -> bool:
    try:
        q, Kc, Vc, k_pool, v_pool, tables, lens, bs = _rc(44, lens=(3, 17), H=2, D=4, bs=4)
        q6 = np.random.default_rng(45).standard_normal((2, 6, 4))
        out = fn(q6, k_pool, v_pool, tables, lens, 0.5, bs)
        for s in range(2):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q6[s][None, :, None, :]), torch.from_numpy(Kc[s][None]),
                torch.from_numpy(Vc[s][None]), scale=0.5, enable_gqa=True)[0, :, 0, :].numpy()
            if not np.allclose(out[s], ref, rtol=0, atol=1e-12):
                return False
        return True
    except (IndexError, ValueError):
        return False


def _gqa_with_map(head_of):
    def fn(q, k_pool, v_pool, block_tables, context_lens, scale, block_size):
        qf = opa._as_f64(q)
        S, H, D = qf.shape
        Hkv = k_pool.shape[1]
        out = np.zeros((S, H, D))
        for s in range(S):
            L = int(context_lens[s])
            for h in range(H):
                K, V = opa.gather_sequence_kv(k_pool, v_pool, block_tables[s], L, head_of(h, H, Hkv),
                                              block_size)
                z = scale * (K @ qf[s, h])
                w = np.exp(z - z.max())
                out[s, h] = (w @ V) / w.sum()
        return out
    return fn


def test_gqa_pins():
    assert _gqa_pins(decode_gqa_ref)
    assert _gqa_pins(_gqa_with_map(lambda h, H, Hkv: h // (H // Hkv)))   # the builder, no slip
    for name, m in (("interleaved h % Hkv", lambda h, H, Hkv: h % Hkv),
                    ("group of the next head", lambda h, H, Hkv: min((h + 1) // (H // Hkv), Hkv - 1)),
                    ("always K/V head 0", lambda h, H, Hkv: 0)):
        assert not _gqa_pins(_gqa_with_map(m)), name
