"""The continuously batched decode loop of serving_loop.py on the device
calls of pagedattn.h (needs an MI355X): the block manager's slots, copy pairs,
block tables and lengths drive copy_blocks, kv_cache_write and
paged_attention_decode for many steps, with forks, finishes, admissions and
preemption; the pool must hold each sequence's recorded tokens bit for bit and
decode must match the oracle's dense attention over them.  The same for the
native engine, with and without its host planning (shared-prefix groups and
dispatch list), and over FP8 / INT8 pools."""
import numpy as np
import pytest
import torch

from gpu_helpers import bits, say, to_torch
from serving_loop import Loop, drive

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_386_amd as pa
    pa.lib()
    yield
    torch.cuda.synchronize()


class DeviceBackend:
    def new_pool(self, NB, Hkv, B, D, dtype):
        self.dtype = dtype
        if dtype == "bf16":
            self.k = torch.full((NB, Hkv, B, D), 0x7FC0, dtype=torch.int16,
                                device="cuda").view(torch.bfloat16)
        else:
            self.k = torch.full((NB, Hkv, B, D), float("nan"), dtype=torch.float32,
                                device="cuda")
        self.v = self.k.clone()

    def write(self, k, v, slots):
        import paged_kv_cache_386_amd as pa
        pa.kv_cache_write(to_torch(k, self.dtype), to_torch(v, self.dtype),
                          torch.from_numpy(np.ascontiguousarray(slots)).cuda(), self.k, self.v)

    def copy(self, pairs):
        import paged_kv_cache_386_amd as pa
        pa.copy_blocks(torch.from_numpy(np.ascontiguousarray(pairs)).cuda(), self.k, self.v)

    def decode(self, q, tables, lens, scale, partition_size):
        import paged_kv_cache_386_amd as pa
        n, Hq, D = q.shape
        out = torch.empty((n, Hq, D), dtype=torch.float32, device="cuda")
        pa.paged_attention_decode(to_torch(q, self.dtype), self.k, self.v,
                                  torch.from_numpy(np.ascontiguousarray(tables)).cuda(),
                                  torch.from_numpy(np.ascontiguousarray(lens)).cuda(),
                                  float(scale), out, max_context_len=int(lens.max()),
                                  partition_size=partition_size)
        return out.cpu().numpy()

    def pool_bits(self):
        return bits(self.k), bits(self.v)


@pytest.mark.parametrize("dtype,Hq,Hkv,D,B", [
    ("bf16", 32, 8, 128, 16),   # matrix-core path, groups of 4
    ("bf16", 16, 2, 128, 16),   # matrix-core path, groups of 8
    ("bf16", 8, 4, 128, 32),    # vector path, pairs
    ("f32", 8, 2, 64, 16),      # vector path, fp32
])
@pytest.mark.parametrize("ps", [0, 64])
def test_serving_loop_matches_oracle(dtype, Hq, Hkv, D, B, ps):
    say(f"serving loop {dtype} Hq={Hq} Hkv={Hkv} D={D} B={B} ps={ps}")
    loop = Loop(DeviceBackend(), dtype, Hq, Hkv, D, B, NB=1024, max_blocks=64,
                seed=D + B + Hq + ps)
    drive(loop, steps=14, partition_size=ps, max_prompt=500, sync=torch.cuda.synchronize)
    assert loop.copies > 0  # copy-on-write happened


def test_serving_loop_preempts_when_the_pool_is_full():
    say("serving loop with preemption")
    loop = Loop(DeviceBackend(), "bf16", 32, 8, 128, 16, NB=60, max_blocks=64, seed=11)
    drive(loop, steps=20, partition_size=0, max_prompt=200, admit_p=0.8,
          sync=torch.cuda.synchronize)
    assert loop.preempted > 0


@pytest.mark.parametrize("host_plan", [True, False])
@pytest.mark.parametrize("dtype,Hq,Hkv,D,B,NB,ps", [
    ("bf16", 32, 8, 128, 16, 800, 0),   # matrix-core decode, automatic partitions
    ("bf16", 16, 2, 128, 16, 800, 64),  # groups of 8, forced 64-token partitions
    ("f32", 8, 2, 64, 16, 800, 0),      # vector decode
    ("bf16", 32, 8, 128, 16, 90, 0),    # small pool: preemption and recompute
])
def test_engine_steps_match_oracle(dtype, Hq, Hkv, D, B, NB, ps, host_plan):
    """The native engine (scheduler, block manager, one index copy and four
    device calls per step) over a stream of requests with parallel samples:
    after every step the pool holds each batch row's tokens bit for bit and
    decode matches dense attention over them; with host_plan, the step's
    decode reads the forked samples' shared prompt blocks once per group in
    the order planned on the host."""
    from serving_loop import EngineHarness, drive_engine
    say(f"engine {dtype} Hq={Hq} Hkv={Hkv} D={D} B={B} NB={NB} ps={ps} plan={host_plan}")
    h = EngineHarness("device", dtype, Hq, Hkv, D, B, NB, max_batch=48, max_ctx=400,
                      seed=NB + D, partition_size=ps, host_plan=host_plan)
    drive_engine(h, num_requests=36, seed=NB + D, max_prompt=300, max_new=40)
    assert h.copies > 0
    if NB < 100:
        assert h.preempted > 0
    if host_plan and dtype == "bf16":
        assert h.groups_seen > 0
    h.eng.close()


@pytest.mark.parametrize("kv8", ["fp8", "int8"])
@pytest.mark.parametrize("Hq,Hkv,NB,ps,D", [(32, 8, 800, 0, 128), (8, 8, 800, 64, 128),
                                            (32, 8, 90, 0, 128), (16, 4, 90, 0, 64)])
def test_engine_8bit_pools(kv8, Hq, Hkv, NB, ps, D):
    """The engine over an FP8 / INT8 pool: bfloat16 token rows quantised by
    its writes; after every step the pool holds the oracle's codes of each
    row's tokens and decode matches dense attention over their dequantised
    values (forks sharing prompt blocks, copy-on-write, preemption in the
    small pools; head_dim 64 on the vector decode kernel)."""
    from serving_loop import EngineHarness, drive_engine
    say(f"engine {kv8} Hq={Hq} Hkv={Hkv} NB={NB} ps={ps} D={D}")
    h = EngineHarness("device", "bf16", Hq, Hkv, D, 16, NB, max_batch=48, max_ctx=400,
                      seed=NB + Hq, partition_size=ps, kv8=kv8)
    drive_engine(h, num_requests=36, seed=NB + Hq, max_prompt=300, max_new=40)
    assert h.copies > 0
    if NB < 100:
        assert h.preempted > 0
    h.eng.close()
