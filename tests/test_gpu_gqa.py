"""GPU parity of grouped-query decode (pa_decode_gqa) against the float64
oracle (decode_gqa_ref), through the C ABI: every group width the kernels
build (tile loads shared by 4 or 2 query heads — groups of 8 and more 4 at a
time — and 1: each head reads its own K/V head), multi-query (one K/V head),
16-bit and 8-bit caches with fp16 and bf16 queries, the default split and
explicit partitions, ragged NaN-poisoned batches."""

import numpy as np
import pytest
import torch

import paged_kv_cache_186_amd as pa
from paged_kv_cache_186_amd import workloads as W
from oracle import decode_gqa_ref, dequant_ref
from gpu_support import DEV, announce, assert_close, bits

pytestmark = pytest.mark.gpu


def _gqa_workload(lens, H, Hkv, D, bs, dtype, seed, poison=True):
    rng = np.random.default_rng(seed)
    nb = sum(-(-L // bs) for L in lens) + len(lens) + 4
    m = W.BlockManager(nb, bs, free_order=rng.permutation(nb).tolist())
    for s, L in enumerate(lens):
        m.allocate(s)
        m.append_slots(s, L)
    width = max(1, max(-(-L // bs) for L in lens))
    w = W.PagedWorkload("gqa", dtype, H, D, bs, nb, 0.9 / np.sqrt(D), m, list(range(len(lens))),
                        width, seed, DEV)
    W.fill_values(w, poison=False)
    w.k_pool = w.k_pool[:, :Hkv].contiguous()
    w.v_pool = w.v_pool[:, :Hkv].contiguous()
    if poison:
        W.poison_unreferenced(w)
    return w


def _run(w, kv=None, partition_size=0):
    out = torch.empty_like(w.q)
    bt, cl = w.block_tables().to(DEV), w.context_lens().to(DEV)
    if kv is None:
        pa.pa_decode_gqa(out, w.q, w.k_pool, w.v_pool, bt, cl, w.scale, w.block_size,
                         partition_size=partition_size)
    else:
        kc, vc, ks, vs = kv
        pa.pa_decode_gqa(out, w.q, kc, vc, bt, cl, w.scale, w.block_size, k_scales=ks, v_scales=vs,
                         partition_size=partition_size)
    torch.cuda.synchronize()
    return out


def _oracle(w, kv=None, fmt=None):
    if kv is None:
        k, v = w.k_pool.cpu(), w.v_pool.cpu()
    else:
        kc, vc, ks, vs = kv
        k = dequant_ref(kc.cpu().view(torch.uint8).numpy(), ks.cpu().numpy(), fmt)
        v = dequant_ref(vc.cpu().view(torch.uint8).numpy(), vs.cpu().numpy(), fmt)
    return decode_gqa_ref(w.q.cpu(), k, v, w.block_tables_np(), w.context_lens_np(), w.scale, w.block_size)


LENS = [0, 1, 900, 2, 0, 333, 17, 2500, 1]


@pytest.mark.parametrize("H,Hkv", [(32, 4), (32, 1), (16, 4), (8, 4), (12, 4), (8, 8)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_group_widths_16bit_cache(H, Hkv, dtype):
    """(32,4) and (32,1): groups of 8 and 32, served 4 heads per tile load;
    (16,4): 4; (8,4): 2;
    (12,4): groups of 3, one head per load; (8,8): plain multi-head."""
    announce(f"gqa H={H} Hkv={Hkv} dtype={dtype}")
    w = _gqa_workload(LENS, H, Hkv, 128, 16, dtype, 50 + H + Hkv)
    ref = _oracle(w)
    for part in (0, 64):
        out = _run(w, partition_size=part)
        assert_close(out, ref, dtype, f"H={H} Hkv={Hkv} partition={part}")
        for s in (0, 4):
            assert not out[s].any()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("H,Hkv", [(32, 4), (16, 8), (8, 2)])
def test_group_widths_8bit_cache(fmt, H, Hkv):
    announce(f"gqa fp8 {fmt} H={H} Hkv={Hkv}")
    w = _gqa_workload(LENS, H, Hkv, 128, 16, torch.float16, 60 + H + Hkv)
    kv = W.fp8_pools(w, fmt)
    ref = _oracle(w, kv, fmt)
    for part in (0, 128):
        assert_close(_run(w, kv, part), ref, torch.float16, f"{fmt} H={H} Hkv={Hkv} partition={part}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("D,bs", [(128, 16), (128, 32), (64, 32)])
def test_bf16_queries_over_8bit_cache(fmt, D, bs):
    """bf16 queries and output over an 8-bit cache with groups of 8 (4 heads
    per tile load); at D = 128 and block 32 this kernel holds part of its
    state in scratch (the register file is full), which must not change the
    result."""
    announce(f"gqa bf16 over {fmt} D={D} bs={bs}")
    w = _gqa_workload(LENS, 32, 4, D, bs, torch.bfloat16, 75 + D + bs)
    kv = W.fp8_pools(w, fmt)
    ref = _oracle(w, kv, fmt)
    for part in (0, 128):
        assert_close(_run(w, kv, part), ref, torch.bfloat16, f"bf16 {fmt} D={D} bs={bs} partition={part}")


@pytest.mark.parametrize("D,bs", [(64, 16), (64, 32), (128, 32)])
def test_head_dims_and_block_sizes(D, bs):
    announce(f"gqa D={D} bs={bs}")
    w = _gqa_workload(LENS, 16, 2, D, bs, torch.float16, 70 + D + bs)
    assert_close(_run(w), _oracle(w), torch.float16, f"D={D} bs={bs}")
    kv = W.fp8_pools(w, "e4m3")
    assert_close(_run(w, kv), _oracle(w, kv, "e4m3"), torch.float16, f"fp8 D={D} bs={bs}")


def test_fp32_queries_one_head_per_load():
    announce("gqa fp32")
    w = _gqa_workload([5, 300, 0, 41], 8, 2, 64, 16, torch.float32, 80)
    assert_close(_run(w), _oracle(w), torch.float32, "fp32 gqa")


def test_layer_shape_with_8_kv_heads():
    """The layer shape (8 sequences, lengths in [1, 2048], block 16, fp16) with
    32 query heads over 8 K/V heads — 4 query heads per K/V head."""
    announce("gqa layer shape 32/8")
    w = W.layer_shape(0, device=DEV, poison=True)
    w.k_pool = w.k_pool[:, :8].contiguous()
    w.v_pool = w.v_pool[:, :8].contiguous()
    assert_close(_run(w), _oracle(w), torch.float16, "layer shape gqa")


@pytest.mark.parametrize("Hkv", [8, 1])
def test_continuous_batching_with_grouped_heads(Hkv):
    """The continuous-batching workload (64 sequences, log-normal lengths,
    block 32, fp16) with 32 query heads over 8 K/V heads or one (multi-query),
    whole output against the oracle."""
    announce(f"gqa continuous batching 32/{Hkv}")
    w = W.continuous_batching(0, device=DEV, poison=True)
    w.k_pool = w.k_pool[:, :Hkv].contiguous()
    w.v_pool = w.v_pool[:, :Hkv].contiguous()
    assert_close(_run(w), _oracle(w), torch.float16, f"continuous batching gqa {Hkv}")


def test_long_context_with_8_kv_heads_sampled_heads():
    """One 131072-token context (8192 scattered blocks, fp16) with 32 query
    heads over 8 K/V heads, the benchmark's size and launch: sampled query
    heads of every group position against the oracle (one K/V head each)."""
    announce("gqa long context 32/8")
    w = W.long_context(0, batch=1, device=DEV)
    w.k_pool = w.k_pool[:, :8].contiguous()
    w.v_pool = w.v_pool[:, :8].contiguous()
    torch.cuda.empty_cache()
    out = _run(w)
    tables, lens = w.block_tables_np(), w.context_lens_np()
    for h in (0, 5, 14, 27, 31):  # group positions 0, 1, 2, 3, 3
        hk = h // 4
        ref = decode_gqa_ref(w.q[:, h:h + 1].cpu(), w.k_pool[:, hk:hk + 1].cpu(), w.v_pool[:, hk:hk + 1].cpu(),
                             tables, lens, w.scale, w.block_size)
        assert_close(out[:, h:h + 1], ref, torch.float16, f"long context gqa head {h}")


def test_gqa_agrees_with_mha_on_repeated_kv_heads():
    """The grouped kernel (groups of 8 served 4 heads per tile load) and plain
    multi-head decode over K/V heads repeated 8 times compute the same
    attention; their splits differ (rows of 4 heads vs single heads), so they
    agree within the tolerance, not bit for bit, and both match the oracle."""
    announce("gqa vs repeated-head mha")
    w = _gqa_workload(LENS, 32, 4, 128, 16, torch.float16, 90, poison=False)
    gqa = _run(w)
    out = torch.empty_like(w.q)
    kr = w.k_pool.repeat_interleave(8, dim=1).contiguous()
    vr = w.v_pool.repeat_interleave(8, dim=1).contiguous()
    pa.pa_decode(out, w.q, kr, vr, w.block_tables().to(DEV), w.context_lens().to(DEV), w.scale,
                 w.block_size)
    torch.cuda.synchronize()
    ref = _oracle(w)
    assert_close(gqa, ref, torch.float16, "gqa")
    assert_close(out, ref, torch.float16, "mha on repeated heads")
    assert float((gqa.float() - out.float()).abs().max()) <= 2 * 3e-3


def test_one_workspace_serves_grouped_plain_and_partitioned_calls():
    """Every decode call lays out the same counter region for the same
    num_seqs * num_heads, so one zero-filled workspace serves grouped (tile
    loads shared by 4 heads), partitioned and plain calls in any order, and
    every call leaves the counters zero."""
    announce("gqa: one workspace for grouped, partitioned and plain calls")
    w = _gqa_workload(LENS, 32, 1, 128, 16, torch.float16, 95)
    S, H = w.num_seqs, w.num_heads
    need = max(pa.pa_decode_gqa_workspace_size(S, H, 1, 128, w.table_width, 16, p, torch.float16,
                                               torch.float16) for p in (0, 64))
    need = max(need, pa.pa_decode_workspace_size(S, H, 128, w.table_width, 16, 0))
    ws = pa.new_workspace(need, DEV)
    bt, cl = w.block_tables().to(DEV), w.context_lens().to(DEV)
    ref = _oracle(w)
    kr = w.k_pool.repeat_interleave(32, dim=1).contiguous()
    vr = w.v_pool.repeat_interleave(32, dim=1).contiguous()
    for it, kind in enumerate(("gqa", "gqa64", "mha", "gqa", "mha64", "gqa64", "gqa")):
        out = torch.empty_like(w.q)
        part = 64 if kind.endswith("64") else 0
        if kind.startswith("gqa"):
            pa.pa_decode_gqa(out, w.q, w.k_pool, w.v_pool, bt, cl, w.scale, 16, partition_size=part,
                             workspace=ws)
        else:
            pa.pa_decode(out, w.q, kr, vr, bt, cl, w.scale, 16, partition_size=part, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[: 4 * S * H].view(torch.int32).abs().sum()) == 0, f"counters after call {it}"
        assert_close(out, ref, torch.float16, f"call {it} ({kind})")


@pytest.mark.parametrize("Hkv", [4, 2, 1])
def test_grouped_split_shares_between_rows(Hkv):
    """Grouped heads with many short rows and about as many units as waves
    (shares that fall between rows' units, waves walking many row segments)."""
    announce(f"decode gqa shares between rows Hkv={Hkv}")
    rng = np.random.default_rng(21)
    lens = rng.choice([0, 1, 5, 16, 17, 40, 130], size=400).tolist()
    w = _gqa_workload(lens, 8, Hkv, 128, 16, torch.float16, 21)
    ref = _oracle(w)
    first = _run(w)
    assert_close(first, ref, torch.float16, f"gqa shares between rows Hkv={Hkv}")
    assert torch.equal(bits(_run(w)), bits(first)), "second call differs"
