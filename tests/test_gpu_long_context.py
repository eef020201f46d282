"""Long contexts with dominant tiles (needs an MI355X).

At 10^4 - 10^5 tokens an ordinary N(0, 1) workload cannot show a lost or
repeated 16-token tile: the output moves by about 1e-3, inside the bf16
tolerance.  Here every query head of a sequence carries the same query u, and
a few chosen tiles get keys whose scores exceed every other score by more
than 35 (natural-log units), all of them equal.  The softmax then gives each
token of those tiles the same weight and the rest less than 1e-15 in all, so
the exact result is the plain mean of the V rows of the chosen tiles (a
closed form: no oracle call).  A tile dropped, read twice or read from the
wrong block moves the output by about 0.05.

The chosen tiles are the ones where the walk changes state: the first and
last tile of a partition (including a ragged last tile), and the tiles where a
wave's block ids roll over to the next group of 64 (each of the 4 waves
takes every 4th tile of its partition, so wave w's 64th and 65th tiles are
partition tiles 4*63 + w and 4*64 + w, and likewise 127/128).  Each length
runs unsplit, with the automatic partitions and with 8192-token partitions,
over every kernel family: bfloat16 on the matrix cores (G = 4, 8) and on the
vector ALU (G = 1, 2), and FP8 / INT8 pools.
"""
import numpy as np
import pytest
import torch

from oracle import fp8
from workloads.generate import BF16_QNAN, E4M3_QNAN, bf16_bits_from_f32, draw_e4m3_codes

from gpu_helpers import say, to_torch

D = 128
TILE = 16
SPIKE = 40.0  # score of a spike token, natural-log units (others are about N(0, 1))
NSEQ = 4
K_SCALE = {"fp8": 0.25, "int8": 0.25}
V_SCALE = {"fp8": 0.5, "int8": 0.03}


@pytest.fixture(scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_386_amd as pa
    pa.lib()
    yield
    torch.cuda.synchronize()


class Base:
    """NSEQ sequences of L tokens on one KV head, private blocks in a random
    permutation of the pool, the pool's values random (N(0, 1) bfloat16, or
    random 8-bit codes), slots past L and a spare block poisoned."""

    def __init__(self, kind, L, B, seed):
        rng = np.random.default_rng(seed)
        nblk = -(-L // B)
        NB = NSEQ * nblk + 1
        perm = rng.permutation(NB).astype(np.int32)
        self.tables = np.ascontiguousarray(perm[:NSEQ * nblk].reshape(NSEQ, nblk))
        shape = (NB, 1, B, D)
        if kind == "bf16":
            self.k = bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))
            self.v = bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))
            nan = BF16_QNAN
        elif kind == "fp8":
            self.k = draw_e4m3_codes(rng, shape)
            self.v = draw_e4m3_codes(rng, shape)
            nan = E4M3_QNAN
        else:
            self.k = rng.integers(-127, 128, size=shape, dtype=np.int8)
            self.v = rng.integers(-127, 128, size=shape, dtype=np.int8)
            nan = -128
        for a in (self.k, self.v):
            a[perm[-1]] = nan
            if L % B:
                a[self.tables[:, -1], :, L % B:] = nan
        self.u = bf16_bits_from_f32(rng.standard_normal((NSEQ, D), dtype=np.float32))
        self.kind, self.L, self.B = kind, L, B
        self.scale = np.float32(1.0 / np.sqrt(D))

    def slots(self, s, tiles):
        """(block, offset) of every token of the given tiles of sequence s."""
        pos = np.concatenate([np.arange(TILE * t, min(TILE * t + TILE, self.L)) for t in tiles])
        return self.tables[s, pos // self.B], pos % self.B

    def spike_key(self, s):
        u = (self.u[s].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        if self.kind == "bf16":
            c = SPIKE / (float(self.scale) * float(u @ u))
            return bf16_bits_from_f32((c * u).astype(np.float32))
        if self.kind == "fp8":
            return np.where(u > 0, 0x7E, 0xFE).astype(np.uint8)  # +-448
        return np.where(u > 0, 127, -127).astype(np.int8)

    def v_values(self, blk, off):
        rows = self.v[blk, 0, off]
        if self.kind == "bf16":
            return (rows.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        if self.kind == "fp8":
            return fp8.e4m3_decode(rows) * np.float64(V_SCALE["fp8"])
        return rows.astype(np.float64) * np.float64(np.float32(V_SCALE["int8"]))


def spike_tiles(L, ps_eff):
    """Tiles where the walk changes state, for partitions of ps_eff tokens."""
    ntiles = -(-L // TILE)
    per = ps_eff // TILE
    nparts = -(-ntiles // per)
    tiles = set()
    for p in sorted({0, 1, nparts - 1}):
        if p >= nparts:
            continue
        first = p * per
        n = min(per, ntiles - first)
        tiles |= {first, first + n - 1}
        for j, w in ((63, 0), (64, 1), (127, 2), (128, 3)):
            if 4 * j + w < n:
                tiles.add(first + 4 * j + w)
    return sorted(tiles)


def run(base, G, k, ps):
    import paged_kv_cache_386_amd as pa
    Hq = G
    q = np.repeat(base.u[:, None, :], Hq, axis=1)
    dq = to_torch(q, "bf16")
    tables = torch.from_numpy(base.tables).cuda()
    lens = torch.from_numpy(np.full(NSEQ, base.L, np.int32)).cuda()
    out = torch.full((NSEQ, Hq, D), 7.0, dtype=torch.float32, device="cuda")
    if base.kind == "bf16":
        pa.paged_attention_decode(dq, to_torch(k, "bf16"), to_torch(base.v, "bf16"), tables, lens,
                                  float(base.scale), out, max_context_len=base.L,
                                  partition_size=ps)
    else:
        dec = pa.paged_attention_decode_fp8 if base.kind == "fp8" else pa.paged_attention_decode_int8
        dec(dq, torch.from_numpy(k).cuda(), torch.from_numpy(base.v).cuda(), tables, lens,
            float(base.scale), K_SCALE[base.kind], V_SCALE[base.kind], out,
            max_context_len=base.L, partition_size=ps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.gpu
@pytest.mark.usefixtures("_gpu")
@pytest.mark.parametrize("L", [9000, 32768, 131071])
@pytest.mark.parametrize("kind,G", [("bf16", 4), ("bf16", 8), ("bf16", 1), ("bf16", 2),
                                    ("fp8", 4), ("fp8", 8), ("int8", 1)])
def test_dominant_tiles_at_walk_boundaries(kind, G, L):
    import paged_kv_cache_386_amd as pa
    B = 512 if (L == 32768 and G == 8) else 16
    say(f"spike {kind} G={G} L={L} B={B}: generating")
    base = Base(kind, L, B, seed=L % 1000 + 10 * G + len(kind))
    for ps in (0, -1, 8192):
        ps_eff = pa.partition_tokens(NSEQ, 1, L, ps)
        tiles = spike_tiles(L, ps_eff)
        k = base.k.copy()
        want = np.zeros((NSEQ, D))
        for s in range(NSEQ):
            blk, off = base.slots(s, tiles)
            k[blk, 0, off] = base.spike_key(s)
            want[s] = base.v_values(blk, off).mean(axis=0)
        say(f"spike {kind} G={G} L={L} B={B} ps={ps} (partition {ps_eff}): tiles {tiles}")
        got = run(base, G, k, ps)
        err = float(np.abs(got - want[:, None, :]).max())
        say(f"spike {kind} G={G} L={L} ps={ps}: max abs err {err:.3e}")
        assert np.isfinite(got).all()
        assert err <= 1e-4, f"ps={ps}: max abs err {err} (tiles {tiles})"


def test_spike_construction_is_dominant():
    """The closed form holds for the inputs built here: on the CPU, each
    spike key's score exceeds the largest other score by more than 30."""
    for kind in ("bf16", "fp8", "int8"):
        base = Base(kind, 2000, 16, 3)
        u = (base.u[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        if kind == "bf16":
            kf = (base.k[base.tables[0], 0].astype(np.uint32) << 16).view(np.float32)
            ks = (base.spike_key(0).astype(np.uint32) << 16).view(np.float32)
            sc = 1.0
        elif kind == "fp8":
            kf, ks, sc = fp8.e4m3_decode(base.k[base.tables[0], 0]), fp8.e4m3_decode(
                base.spike_key(0)), K_SCALE[kind]
        else:
            kf, ks, sc = base.k[base.tables[0], 0].astype(np.float64), base.spike_key(0).astype(
                np.float64), K_SCALE[kind]
        others = float(base.scale) * sc * (kf.reshape(-1, D)[:2000] @ u)
        spike = float(base.scale) * sc * float(ks.astype(np.float64) @ u)
        assert spike - others.max() > 30, (kind, spike, others.max())
