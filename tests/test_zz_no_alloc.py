"""The allocation-free decode entry point (paged_attention_decode_noalloc)
against paged_attention_decode with a workspace of its own, through the C
ABI (needs an MI355X).  Two calls in a row on the shared static scratch, the
second with a smaller input (so stale partials and dispatch entries of the
first are in the array), then the first again; each output bit for bit equal
to the allocating entry point's and within tolerance of the oracle."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from workloads import make_prefix_case, make_private_case

from gpu_helpers import REGRESS, TOL, DeviceCase, max_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_386_amd as pa
    pa.lib()
    yield
    torch.cuda.synchronize()


def _noalloc(dc, ps):
    import paged_kv_cache_386_amd as pa
    out = torch.full(dc.case.q.shape, 7.0, dtype=torch.float32, device="cuda")
    pa.paged_attention_decode_noalloc(dc.q, dc.k_cache, dc.v_cache, dc.block_tables,
                                      dc.context_lens, float(dc.case.scale), out,
                                      max_context_len=dc.max_context_len, partition_size=ps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _cases():
    rng = np.random.default_rng(31)
    lens = np.clip(np.rint(rng.lognormal(np.log(1024), 1.0, 160)), 1, 4096).astype(int)
    big = make_prefix_case("noalloc-big", lens, 16, 1024, 32, 8, 128, 16, "bf16", 31)
    small = make_private_case("noalloc-small", rng.integers(1, 3000, size=20).tolist(), 8, 2, 128,
                              16, "bf16", 32)
    return big, small


def test_noalloc_matches_allocating_decode():
    import paged_kv_cache_386_amd as pa
    big, small = _cases()
    runs = [(big, 2048), (small, 512), (big, 2048)]
    for case, ps in runs:
        need = pa.workspace_size(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                 case.head_dim, case.max_context_len, ps)
        P = pa.num_partitions(case.num_seqs, case.num_kv_heads, case.max_context_len, ps)
        say(f"noalloc {case.name}: S={case.num_seqs} P={P} workspace {need} bytes "
            f"(scratch {pa.noalloc_scratch_bytes()})")
        assert 0 < need <= pa.noalloc_scratch_bytes() and P > 1
        dc = DeviceCase(case)
        dc.run_edits()
        got = _noalloc(dc, ps)
        want = dc.run_decode(ps).cpu().numpy()
        torch.cuda.synchronize()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), case.name
        kc, vc = case.k_cache, case.v_cache
        if case.has_step:
            kc, vc = O.copy_blocks(case.copy_pairs, kc, vc)
            kc, vc = O.kv_cache_write(case.k_new, case.v_new, case.slot_mapping, kc, vc,
                                      case.block_size)
        ref = O.paged_attention_decode(case.q, kc, vc, case.block_tables, case.context_lens,
                                       case.scale, case.block_size, case.dtype)
        err = max_err(got, ref)
        say(f"noalloc {case.name}: max abs err {err:.3e}")
        assert err <= TOL["bf16"] and err <= REGRESS["bf16"]


def test_noalloc_rejects_too_large_on_host():
    """A call whose workspace exceeds the scratch returns PA_ERR_SCRATCH from
    the host check; the device buffers here are sized for the call, with
    empty contexts, so nothing could read out of bounds either way."""
    import paged_kv_cache_386_amd as pa
    S, Hq, Hkv, D, B, max_ctx = 4096, 64, 8, 128, 16, 65536
    assert pa.workspace_size(S, Hq, Hkv, D, max_ctx, 0) > pa.noalloc_scratch_bytes()
    q = torch.zeros((S, Hq, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, Hkv, B, D), dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros((S, max_ctx // B), dtype=torch.int32, device="cuda")
    lens = torch.zeros(S, dtype=torch.int32, device="cuda")
    out = torch.full((S, Hq, D), 7.0, dtype=torch.float32, device="cuda")
    say("noalloc: too-large call")
    with pytest.raises(pa.PagedAttnError) as e:
        pa.paged_attention_decode_noalloc(q, kc, kc, tables, lens, 0.1, out,
                                          max_context_len=max_ctx)
    assert e.value.status == -12
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
