"""kv_cache_append through the C ABI against the oracle (needs an MI355X): the
pools it leaves must equal, bit for bit, those of the oracle's copy_blocks
followed by its write (stored rows, or FP8 / INT8 quantisation), on the
orderings that the one-launch form has to resolve -- a token writing a
copy's destination, a token writing a copy's source (with and without a
token on the same position of the destination), several copies of one
source, random mixes, skipped pairs and slots -- at block sizes 1, 16, 512
and 1024 (a copy's skip mask then spans all its 32 words), and on the
full-size GQA prefix and fork steps."""
import zlib

import numpy as np
import pytest
import torch

from oracle import fp8, int8
from oracle import oracle as O
from workloads import make_case
from workloads.generate import bf16_bits_from_f32

from gpu_helpers import check_indices, say, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_386_amd as pa
    pa.lib()


def _pool(rng, shape, dt):
    """Random bits of the pool's element type (NaN patterns included: the
    copies and stored rows must keep every bit)."""
    if dt == "bf16":
        return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    if dt == "f32":
        return rng.integers(0, 1 << 32, size=shape, dtype=np.uint32).view(np.float32)
    if dt == "fp8":
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    return rng.integers(-128, 128, size=shape, dtype=np.int8)


def _rows(rng, shape, dt):
    """New token rows: values for quantised writes, any bits for stored ones."""
    if dt == "bf16":
        return bf16_bits_from_f32((rng.standard_normal(shape) * 3).astype(np.float32))
    if dt == "f32":
        return (rng.standard_normal(shape) * 3).astype(np.float32)
    return _pool(rng, shape, dt)


def _dev(a):
    if a.dtype == np.uint16:
        return to_torch(a, "bf16")
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _host(t, like):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(like.dtype)


def _expected(pairs, k, v, slots, kc, vc, B, src, kv, ks, vs):
    """The oracle: the valid pairs copied in order, then the writes of the
    tokens whose slot lies in the pool."""
    NB = kc.shape[0]
    p = pairs.reshape(-1, 2)
    ok = (p >= 0).all(1) & (p < NB).all(1) & (p[:, 0] != p[:, 1])
    wk, wv = O.copy_blocks(p[ok], kc, vc)
    sl = np.where(slots < NB * B, slots, -1).astype(np.int32)
    if src == kv:
        return O.kv_cache_write(k, v, sl, wk, wv, B)
    mod = fp8.kv_cache_write_fp8 if kv == "fp8" else int8.kv_cache_write_int8
    return mod(k, v, sl, wk, wv, B, src, ks, vs)


def _run(pairs, k, v, slots, kc, vc, B, src, kv, ks=0.5, vs=0.25, host_pairs=True):
    import paged_kv_cache_386_amd as pa
    dk, dv = _dev(kc), _dev(vc)
    dp = torch.from_numpy(np.ascontiguousarray(pairs.reshape(-1, 2).astype(np.int32))).cuda()
    say(f"append src={src} kv={kv} B={B} pairs={len(dp)} tokens={len(slots)}")
    pa.kv_cache_append(dp if len(dp) else None, _dev(k) if len(slots) else None,
                       _dev(v) if len(slots) else None,
                       torch.from_numpy(slots.astype(np.int32)).cuda() if len(slots) else None,
                       dk, dv, k_scale=ks, v_scale=vs,
                       host_pairs=pairs.reshape(-1, 2) if host_pairs else None)
    torch.cuda.synchronize()
    wk, wv = _expected(pairs, k, v, slots, kc, vc, B, src, kv, ks, vs)
    gk, gv = _host(dk, kc), _host(dv, vc)
    assert np.array_equal(gk.view(np.uint8), wk.view(np.uint8))
    assert np.array_equal(gv.view(np.uint8), wv.view(np.uint8))


def _scenario(rng, NB, B, kind):
    """Pairs and slots for one ordering case (block ids < NB, distinct dsts,
    no dst a src, distinct slots)."""
    ids = rng.permutation(NB)
    slots = []
    if kind == "cow":
        # each copy's destination gets the appending token
        srcs, dsts = ids[:6], ids[6:12]
        pairs = np.stack([srcs, dsts], 1)
        slots += [int(d) * B + int(rng.integers(B)) for d in dsts]
        slots += [int(b) * B + int(rng.integers(B)) for b in ids[12:16]]
    elif kind == "fork":
        # one source, three copies; the parent writes position q of the
        # source; siblings 0 and 1 write q of their copies, sibling 2 does not
        s, d = int(ids[0]), ids[1:4]
        pairs = np.stack([np.full(3, s), d], 1)
        q = int(rng.integers(B))
        slots += [s * B + q, int(d[0]) * B + q, int(d[1]) * B + q]
        # a second source written at another position with no sibling writes
        s2, d2 = int(ids[4]), int(ids[5])
        pairs = np.concatenate([pairs, [[s2, d2]]])
        slots += [s2 * B + int(rng.integers(B))]
    elif kind == "mixed":
        P = min(NB // 3, 40)
        srcs = rng.choice(ids[:NB // 2], size=P)  # sources may repeat
        dsts = ids[NB // 2:NB // 2 + P]
        pairs = np.stack([srcs, dsts], 1)
        T = min(NB * B // 2, 700)
        slots = rng.choice(NB * B, size=T, replace=False).tolist()
    else:  # skipped pairs and slots mixed with valid ones
        pairs = np.array([[ids[0], ids[1]], [ids[2], ids[2]], [-1, ids[3]], [ids[4], NB],
                          [ids[5], ids[6]]])
        slots = [int(ids[1]) * B, -1, NB * B, int(ids[5]) * B + B - 1, int(ids[7]) * B]
    return np.asarray(pairs, np.int64).reshape(-1, 2), np.asarray(slots, np.int64)


DTYPES = [("bf16", "bf16"), ("f32", "f32"), ("bf16", "fp8"), ("f32", "fp8"), ("bf16", "int8"),
          ("f32", "int8"), ("fp8", "fp8"), ("int8", "int8")]


@pytest.mark.parametrize("src,kv", DTYPES)
@pytest.mark.parametrize("kind", ["cow", "fork", "mixed", "skipped"])
def test_append_matches_copy_then_write(src, kv, kind):
    rng = np.random.default_rng(zlib.crc32(f"{src}/{kv}/{kind}".encode()))
    NB, Hkv, B, D = 48, 2, 16, 128
    pairs, slots = _scenario(rng, NB, B, kind)
    kc = _pool(rng, (NB, Hkv, B, D), kv)
    vc = _pool(rng, (NB, Hkv, B, D), kv)
    k = _rows(rng, (len(slots), Hkv, D), src)
    v = _rows(rng, (len(slots), Hkv, D), src)
    _run(pairs, k, v, slots, kc, vc, B, src, kv, host_pairs=kind != "skipped")


@pytest.mark.parametrize("B", [1, 16, 512, 1024])
@pytest.mark.parametrize("src,kv", [("bf16", "bf16"), ("bf16", "fp8")])
def test_append_block_sizes(B, src, kv):
    rng = np.random.default_rng(B)
    NB, Hkv, D = 40, 4, 64 if kv == "bf16" else 128
    for kind in ("cow", "fork", "mixed"):
        pairs, slots = _scenario(rng, NB, B, kind)
        kc = _pool(rng, (NB, Hkv, B, D), kv)
        vc = _pool(rng, (NB, Hkv, B, D), kv)
        k = _rows(rng, (len(slots), Hkv, D), src)
        v = _rows(rng, (len(slots), Hkv, D), src)
        _run(pairs, k, v, slots, kc, vc, B, src, kv)


def test_append_only_copies_or_only_writes():
    rng = np.random.default_rng(11)
    NB, Hkv, B, D = 20, 2, 16, 128
    kc = _pool(rng, (NB, Hkv, B, D), "bf16")
    vc = _pool(rng, (NB, Hkv, B, D), "bf16")
    pairs = np.array([[1, 5], [2, 6], [1, 7]])
    none = np.zeros(0, np.int64)
    _run(pairs, np.zeros((0, Hkv, D), np.uint16), np.zeros((0, Hkv, D), np.uint16), none,
         kc, vc, B, "bf16", "bf16")
    slots = np.array([3, 40, 41, 319])
    k = _rows(rng, (4, Hkv, D), "bf16")
    v = _rows(rng, (4, Hkv, D), "bf16")
    _run(np.zeros((0, 2), np.int64), k, v, slots, kc, vc, B, "bf16", "bf16")


@pytest.mark.parametrize("cfg", [2, 4])
def test_append_full_size_steps(cfg):
    """The GQA prefix step (copy-on-write of shared blocks, 256 new tokens)
    and the fork step (a parent writing the block its siblings copy), whole
    pools compared."""
    import paged_kv_cache_386_amd as pa
    c = make_case(cfg)
    check_indices(c)
    dk, dv = to_torch(c.k_cache, c.dtype), to_torch(c.v_cache, c.dtype)
    say(f"append full size cfg{cfg}: pairs={len(c.copy_pairs)} tokens={len(c.slot_mapping)}")
    pairs = np.ascontiguousarray(c.copy_pairs.reshape(-1, 2).astype(np.int32))
    pa.kv_cache_append(torch.from_numpy(pairs).cuda(), to_torch(c.k_new, c.dtype),
                       to_torch(c.v_new, c.dtype), torch.from_numpy(c.slot_mapping).cuda(),
                       dk, dv, host_pairs=pairs)
    torch.cuda.synchronize()
    wk, wv = O.copy_blocks(c.copy_pairs, c.k_cache, c.v_cache)
    wk, wv = O.kv_cache_write(c.k_new, c.v_new, c.slot_mapping, wk, wv, c.block_size)
    assert np.array_equal(_host(dk, wk), wk)
    assert np.array_equal(_host(dv, wv), wv)
