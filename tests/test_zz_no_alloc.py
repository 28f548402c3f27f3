"""pa_decode_noalloc (the decode entry point that allocates nothing: its
partials and arrival counters live in the library's static per-GPU scratch)
against pa_decode with a caller workspace, through the C ABI.

Both run the same kernels with the same split, so their outputs must agree
bit for bit; each is also held to the oracle's tolerance.  Calls follow one
another with different sizes (larger, then smaller, then the partitioned
kernel, then smaller again), so a call that found the previous call's
partials on its counters would show up here.  Last, the call is captured in
a HIP graph (it allocates nothing) and every replay, with eager calls of
other sizes in between, must equal the eager result.
"""

import pytest
import torch

import paged_kv_cache_186_amd as pa
from paged_kv_cache_186_amd import workloads as W
from gpu_support import DEV, announce, assert_close, bits, oracle_decode

pytestmark = pytest.mark.gpu


def _on_device(w):
    w.q, w.k_pool, w.v_pool = w.q.to(DEV), w.k_pool.to(DEV), w.v_pool.to(DEV)
    w.device = DEV
    return w


def _both(w, partition_size=0):
    tables, lens = w.block_tables().to(DEV), w.context_lens().to(DEV)
    ref_out = torch.empty_like(w.q)
    pa.pa_decode(ref_out, w.q, w.k_pool, w.v_pool, tables, lens, w.scale, w.block_size,
                 partition_size=partition_size)
    out = torch.full_like(w.q, float("nan"))
    pa.pa_decode_noalloc(out, w.q, w.k_pool, w.v_pool, tables, lens, w.scale, w.block_size,
                         partition_size=partition_size)
    torch.cuda.synchronize()
    return out, ref_out


def test_noalloc_equals_workspace_decode_over_calls_of_changing_size():
    big = _on_device(W.layer_shape(1, poison=True))
    small = _on_device(W.tiny(0, poison=True))
    ref_big, ref_small = oracle_decode(big), oracle_decode(small)
    for i, (w, part, ref) in enumerate([(big, 0, ref_big), (small, 0, ref_small), (big, 64, ref_big),
                                        (small, 16, ref_small), (small, 0, ref_small)]):
        announce(f"noalloc call {i}: {w.name} partition {part}")
        out, want = _both(w, part)
        assert torch.equal(bits(out), bits(want)), f"call {i} differs from pa_decode"
        assert_close(out, ref, w.dtype, f"noalloc call {i} ({w.name}, partition {part})")


def test_noalloc_long_context_default_split():
    announce("noalloc long_context b1")
    w = W.long_context(0, batch=1, device=DEV)
    out, want = _both(w)
    assert torch.equal(bits(out), bits(want))
    del w
    torch.cuda.empty_cache()


def test_noalloc_graph_replays():
    announce("noalloc graph capture")
    w = _on_device(W.layer_shape(2))
    small = _on_device(W.tiny(1))
    tables, lens = w.block_tables().to(DEV), w.context_lens().to(DEV)
    out = torch.empty_like(w.q)

    def call():
        pa.pa_decode_noalloc(out, w.q, w.k_pool, w.v_pool, tables, lens, w.scale, w.block_size)
    call()
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(want))
        _both(small)                      # eager calls of another size in between
    assert_close(want, oracle_decode(w), torch.float16, "noalloc graph")
