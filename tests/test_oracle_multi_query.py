"""Pins of the multi-token-query and latent-cache oracles (oracle/multi_query.py)
to facts outside them — torch's attention with its own causal mask, reductions
to the already pinned decode, invariants of causal attention, closed forms —
and mutants that each pin set must catch (CPU only)."""

import numpy as np
import pytest
import torch

import oracle.paged_attention as opa
from oracle import decode_gqa_ref, mla_decode_ref, prefill_ref

from test_oracle import _random_case


def _sdpa(q, k, v, scale, causal=False):
    """torch attention, float64: q [H, Lq, D], k [Hkv, L, D], v [Hkv, L, Dv]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        scale=scale, is_causal=causal, enable_gqa=True)[0].numpy()


def _prefill_case(seed, lens=(5, 12, 1, 20), Hkv=2, G=3, D=8, bs=4, tq=None):
    """Paged pools built by an independent block-wise scatter (test_oracle's
    helper), queries for the last Tq_s tokens of every sequence."""
    q1, Kc, Vc, k_pool, v_pool, tables, lens, bs = _random_case(seed, lens=lens, H=Hkv, D=D, bs=bs)
    rng = np.random.default_rng(seed + 1000)
    tq = list(lens) if tq is None else list(tq)
    qs = np.concatenate([[0], np.cumsum(tq)]).astype(np.int64)
    q = rng.standard_normal((int(qs[-1]), Hkv * G, D))
    return q, Kc, Vc, k_pool, v_pool, tables, lens, qs, bs


# ---------------------------------------------------------------- the pins --

def _prefill_pins(fn) -> bool:
    """True when ``fn`` (prefill_ref's signature) passes every pin below."""
    try:
        with np.errstate(all="ignore"):
            # (1) whole context new (Tq = L): torch's own causal mask, grouped heads
            q, Kc, Vc, kp, vp, tables, lens, qs, bs = _prefill_case(1)
            out = fn(q, kp, vp, tables, lens, qs, 0.45, bs)
            for s, L in enumerate(lens):
                ref = _sdpa(q[qs[s]:qs[s + 1]].transpose(1, 0, 2).copy(), Kc[s], Vc[s], 0.45, causal=True)
                if not np.allclose(out[qs[s]:qs[s + 1]], ref.transpose(1, 0, 2), rtol=0, atol=1e-12):
                    return False
            # (2) one query token per sequence is grouped-query decode
            q, Kc, Vc, kp, vp, tables, lens, qs, bs = _prefill_case(2, tq=(1, 1, 1, 1))
            if not np.array_equal(fn(q, kp, vp, tables, lens, qs, 0.7, bs),
                                  decode_gqa_ref(q, kp, vp, tables, lens, 0.7, bs)):
                return False
            # (3) speculative verification: row i is a decode at length p_i + 1
            tq = (3, 5, 1, 4)
            q, Kc, Vc, kp, vp, tables, lens, qs, bs = _prefill_case(3, tq=tq)
            out = fn(q, kp, vp, tables, lens, qs, 0.6, bs)
            for s, L in enumerate(lens):
                for i in range(tq[s]):
                    p = int(L) - tq[s] + i
                    one = decode_gqa_ref(q[qs[s] + i][None], kp, vp, tables[s:s + 1], np.array([p + 1]),
                                         0.6, bs)[0]
                    if not np.allclose(out[qs[s] + i], one, rtol=0, atol=1e-13):
                        return False
            # (4) prefix property: a chunk's rows equal those rows of the
            # whole-context prefill
            full_q, _, _, kp, vp, tables, lens, full_qs, bs = _prefill_case(4)
            full = fn(full_q, kp, vp, tables, lens, full_qs, 0.5, bs)
            tq = (2, 4, 1, 7)
            rows = np.concatenate([np.arange(full_qs[s + 1] - tq[s], full_qs[s + 1]) for s in range(4)])
            chunk_qs = np.concatenate([[0], np.cumsum(tq)])
            part = fn(full_q[rows], kp, vp, tables, lens, chunk_qs, 0.5, bs)
            if not np.allclose(part, full[rows], rtol=0, atol=1e-13):
                return False
        return True
    except (IndexError, ValueError):
        return False


def _prefill_mutant(pos=lambda L, Tq, i: L - Tq + i, keys=lambda p, L: p + 1,
                    head=lambda h, G, Hkv: h // G, row=lambda i, Tq: i):
    def fn(q, k_pool, v_pool, block_tables, context_lens, query_start, scale, block_size):
        qf = opa._as_f64(q)
        T, H, D = qf.shape
        Hkv = k_pool.shape[1]
        G = H // Hkv
        qs = opa._as_int(query_start)
        out = np.zeros((T, H, D))
        for s in range(len(context_lens)):
            L = int(context_lens[s])
            Tq = int(qs[s + 1] - qs[s])
            for h in range(H):
                K, V = opa.gather_sequence_kv(k_pool, v_pool, block_tables[s], L, head(h, G, Hkv),
                                              block_size)
                for i in range(Tq):
                    n = keys(pos(L, Tq, i), L)
                    if n <= 0:
                        raise ValueError("no visible key")
                    z = scale * (K[:n] @ qf[qs[s] + row(i, Tq), h])
                    w = np.exp(z - z.max())
                    out[qs[s] + i, h] = (w @ V[:n]) / w.sum()
        return out
    return fn


def test_prefill_oracle_passes_its_pins():
    assert _prefill_pins(prefill_ref)
    assert _prefill_pins(_prefill_mutant())    # the mutant builder without a slip


@pytest.mark.parametrize("name,mutant", [
    ("a token does not see itself", _prefill_mutant(keys=lambda p, L: p)),
    ("one key too many", _prefill_mutant(keys=lambda p, L: min(p + 2, L))),
    ("no causal mask", _prefill_mutant(keys=lambda p, L: L)),
    ("top-left alignment", _prefill_mutant(pos=lambda L, Tq, i: i)),
    ("positions reversed", _prefill_mutant(pos=lambda L, Tq, i: L - 1 - i)),
    ("interleaved head groups", _prefill_mutant(head=lambda h, G, Hkv: h % Hkv)),
    ("query rows shifted", _prefill_mutant(row=lambda i, Tq: (i + 1) % Tq)),
])
def test_each_prefill_mutant_is_caught(name, mutant):
    assert not _prefill_pins(mutant), name


def test_prefill_rejects_inconsistent_query_layout():
    q, _, _, kp, vp, tables, lens, qs, bs = _prefill_case(5, tq=(1, 2, 1, 2))
    with pytest.raises(ValueError):   # last boundary is not the number of rows
        prefill_ref(q, kp, vp, tables, lens, qs - np.array([0, 0, 0, 0, 1]), 0.5, bs)
    with pytest.raises(ValueError):   # more query tokens than context (L = 1)
        prefill_ref(q, kp, vp, tables, lens, np.array([0, 1, 2, 4, 6]), 0.5, bs)


def test_prefill_sequences_without_queries_produce_nothing():
    q, _, _, kp, vp, tables, lens, qs, bs = _prefill_case(6, tq=(0, 3, 0, 2))
    out = prefill_ref(q, kp, vp, tables, lens, qs, 0.5, bs)
    assert out.shape == (5, 6, 8) and np.all(np.isfinite(out))


# ------------------------------------------------------------ latent cache --

def _latent_case(seed, lens=(1, 9, 20), H=4, Dqk=24, bs=4, spare=3):
    """Latent rows generated contiguously, then written block by block into a
    [num_blocks, bs, Dqk] pool at permuted ids (NaN elsewhere)."""
    rng = np.random.default_rng(seed)
    C = [rng.standard_normal((L, Dqk)) for L in lens]
    need = [-(-L // bs) for L in lens]
    nb = sum(need) + spare
    ids = rng.permutation(nb)
    tables = -np.ones((len(lens), max(need)), dtype=np.int64)
    pool = np.full((nb, bs, Dqk), np.nan)
    cur = 0
    for s, L in enumerate(lens):
        for j in range(need[s]):
            tables[s, j] = ids[cur]
            rows = C[s][j * bs:(j + 1) * bs]
            pool[ids[cur], :len(rows)] = rows
            cur += 1
    q = rng.standard_normal((len(lens), H, Dqk))
    return q, C, pool, tables, np.array(lens), bs


def _mla_pins(fn) -> bool:
    try:
        with np.errstate(all="ignore"):
            q, C, pool, tables, lens, bs = _latent_case(7)
            Dv = 16
            out = fn(q, pool, tables, lens, 0.3, bs, Dv)
            for s in range(len(lens)):
                ref = _sdpa(q[s][:, None, :], C[s][None], C[s][None, :, :Dv], 0.3)[:, 0, :]
                if not np.allclose(out[s], ref, rtol=0, atol=1e-12):
                    return False
            # one token: its latent part; zero scale: the mean latent
            if not np.array_equal(out[0], np.repeat(C[0][:, :Dv], 4, axis=0)):
                return False
            z = fn(q, pool, tables, lens, 0.0, bs, Dv)
            if not np.allclose(z[2], np.repeat(C[2][:, :Dv].mean(axis=0)[None], 4, axis=0), atol=1e-13):
                return False
        return True
    except (IndexError, ValueError):
        return False


def _mla_mutant(value_tail=False, latent_scores=False, block_shift=0):
    def fn(q, kv_pool, block_tables, context_lens, scale, block_size, v_dim):
        qf = opa._as_f64(q)
        S, H, Dqk = qf.shape
        out = np.zeros((S, H, v_dim))
        for s in range(S):
            L = int(context_lens[s])
            t = np.arange(L)
            blocks = np.asarray(block_tables[s])[t // block_size + block_shift * (t >= block_size)]
            C = np.asarray(kv_pool, dtype=np.float64)[blocks, t % block_size]
            Vv = C[:, -v_dim:] if value_tail else C[:, :v_dim]
            for h in range(H):
                z = scale * ((C[:, :v_dim] @ qf[s, h, :v_dim]) if latent_scores else (C @ qf[s, h]))
                w = np.exp(z - z.max())
                out[s, h] = (w @ Vv) / w.sum()
        return out
    return fn


def test_mla_oracle_passes_its_pins():
    assert _mla_pins(mla_decode_ref)
    assert _mla_pins(_mla_mutant())


@pytest.mark.parametrize("name,mutant", [
    ("value from the tail of the row", _mla_mutant(value_tail=True)),
    ("scores over the latent part only", _mla_mutant(latent_scores=True)),
    ("blocks after the first shifted", _mla_mutant(block_shift=-1)),
])
def test_each_mla_mutant_is_caught(name, mutant):
    assert not _mla_pins(mutant), name


def test_mla_empty_context_and_bad_width():
    q, C, pool, tables, lens, bs = _latent_case(8)
    out = mla_decode_ref(q, pool, tables, np.array([0, 9, 20]), 0.3, bs, 16)
    assert np.all(out[0] == 0)
    with pytest.raises(ValueError):
        mla_decode_ref(q, pool, tables, lens, 0.3, bs, 25)
