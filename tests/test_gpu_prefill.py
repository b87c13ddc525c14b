"""GPU parity of chunked prefill (``pa_prefill``, through the C ABI) against the fp64 oracle.

Every sequence appends a chunk of new tokens (written with ``pa_write_kv``) to its cached context
and each new token attends causally up to its own position. Tolerances as for decode: max-abs
2e-3 (fp16 / bf16 cache, fp32 accumulation) or 2e-2 (fp8 cache) against the oracle, plus half an
ulp of a 16-bit output at the reference value.

Cases: every supported dtype pairing, group size (1, 4, 8, 16 query heads per kv head) and head
size, chunks spanning several 64-row tiles with ragged tails, empty chunks and empty contexts,
one-token chunks (the decode step), a chunk as long as its sequence (a prompt into an empty
cache), negative, zero and large scales, NaN-poisoned unused memory, placement invariance, and a
full-size chunked-prefill batch checked on sampled rows.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_318_amd import lib
from paged_kv_cache_318_amd.step import workspace_for
from workloads import make_prefill, make_workload
from workloads.device import to_numpy_f64, torch_dtype, upload

pytestmark = pytest.mark.gpu

TOL = {"f16": 2e-3, "bf16": 2e-3, "fp8": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    lib.load()
    yield
    torch.cuda.synchronize()


def _half_ulp(ref, out_dt):
    if out_dt == "f32":
        return 0.0
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    mant = {"f16": 10, "bf16": 7}[out_dt]
    return 0.5 * 2.0 ** (e - mant)


def assert_close(got, want, cache_dt, out_dt, what=""):
    """Max-abs error within the cache dtype's tolerance, plus half an ulp of a 16-bit output type
    where |o_ref| >= 1 (there the output's own rounding exceeds the tolerance's margin); the number
    of elements that needed that allowance is printed."""
    assert got.shape == want.shape
    err = np.abs(got - want)
    allow = np.where(np.abs(want) >= 1.0, _half_ulp(want, out_dt), 0.0)
    bad = ~(err <= TOL[cache_dt] + allow)
    if out_dt != "f32" and not bad.any():
        print(f"[half-ulp allowance] {what}: {int((err > TOL[cache_dt]).sum())} of {err.size} "
              f"{out_dt} outputs ({int((np.abs(want) >= 1.0).sum())} with |o_ref| >= 1)")
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(np.isfinite(err), err, np.inf)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; max err "
                             f"{np.nanmax(err):.3e} at {i} (got {got[i]}, want {want[i]})")


def _check_inputs(w):
    """Host-side bounds check of every index the kernels will follow."""
    B, NB = w.block_size, w.num_blocks
    qs = w.query_start
    assert qs[0] == 0 and np.all(np.diff(qs) >= 0) and qs[-1] == w.q.shape[0]
    for s in range(w.num_seqs):
        nb = -(-int(w.lens[s]) // B)
        assert nb <= w.tables.shape[1]
        assert np.all((w.tables[s, :nb] >= 0) & (w.tables[s, :nb] < NB))
        assert qs[s + 1] - qs[s] <= w.lens[s]
    assert np.all((w.slots >= 0) & (w.slots < NB * B))


def run_gpu(w, out_dt=None, max_query_len=None, return_pools=False):
    _check_inputs(w)
    d = upload(w)
    qs = torch.from_numpy(np.ascontiguousarray(w.query_start, dtype=np.int32)).cuda()
    out_dt = out_dt or w.q_dtype
    T = w.q.shape[0]
    out = torch.empty(T, w.num_heads, w.head_dim, dtype=torch_dtype(out_dt), device="cuda")
    lib.pa_write_kv(d.k_new, d.v_new, d.k_cache, d.v_cache, d.slots, d.k_scale, d.v_scale)
    mql = max_query_len or max(1, int(np.diff(w.query_start).max(initial=0)))
    lib.pa_prefill(out, d.q, d.k_cache, d.v_cache, d.tables, d.lens, qs, w.scale, mql,
                   d.k_scale, d.v_scale)
    torch.cuda.synchronize()
    res = to_numpy_f64(out)
    return (res, d) if return_pools else res


def run_oracle(w, tokens=None):
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    ks = None if w.k_scale is None else w.k_scale.copy()
    vs = None if w.v_scale is None else w.v_scale.copy()
    oracle.write_kv(kp, vp, w.k_new, w.v_new, w.slots, w.block_size, w.dtype, ks, vs, w.new_dtype)
    return oracle.prefill(w.q, kp, vp, w.tables, w.lens, w.query_start, w.block_size, w.scale,
                          w.dtype, w.q_dtype, ks, vs, tokens=tokens)


CTX = [0, 5, 40, 300, 16, 1000, 77]
NEW = [19, 1, 64, 3, 100, 33, 0]
COMBOS = [  # cache, q, Hq, Hkv, D
    ("f16", "f16", 4, 4, 128), ("bf16", "bf16", 8, 2, 128), ("bf16", "bf16", 16, 2, 64),
    ("f16", "f16", 16, 1, 128), ("bf16", "bf16", 32, 2, 128), ("fp8", "bf16", 8, 2, 128),
    ("fp8", "f16", 4, 4, 64), ("fp8", "bf16", 32, 4, 128),
]


@pytest.mark.parametrize("dt,B,D", [("bf16", 16, 128), ("f16", 8, 64), ("f32", 32, 128),
                                    ("fp8", 16, 128), ("fp8", 32, 64)])
def test_chunk_write_bit_exact(dt, B, D):
    """pa_write_kv of prefill chunks: whole blocks (values transposed through LDS and stored as
    whole rows), the partial first and last blocks of each chunk, and an empty chunk -- byte for
    byte against the oracle's write."""
    w = make_prefill([0, 5, 40, 3 * B], [3 * B + 5, 1, 64, 2 * B], num_heads=4, num_kv_heads=4,
                     head_dim=D, dtype=dt, block_size=B, seed=B + D)
    _check_inputs(w)
    d = upload(w)
    lib.pa_write_kv(d.k_new, d.v_new, d.k_cache, d.v_cache, d.slots, d.k_scale, d.v_scale)
    torch.cuda.synchronize()
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    oracle.write_kv(kp, vp, w.k_new, w.v_new, w.slots, B, w.dtype, w.k_scale, w.v_scale,
                    w.new_dtype)

    def host(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16) if dt == "bf16" else t.cpu().numpy()
    assert np.array_equal(host(d.k_cache).view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(host(d.v_cache).view(np.uint8), vp.view(np.uint8))


@pytest.mark.parametrize("cdt,qdt,hq,hkv,D", COMBOS)
def test_prefill_parity(cdt, qdt, hq, hkv, D):
    w = make_prefill(CTX, NEW, num_heads=hq, num_kv_heads=hkv, head_dim=D, dtype=cdt, q_dtype=qdt,
                     seed=hq * 100 + D)
    ref = run_oracle(w)
    got = run_gpu(w, out_dt="f32")
    assert_close(got, ref, cdt, "f32", f"{cdt}/{qdt} Hq={hq} Hkv={hkv} D={D}")
    got16 = run_gpu(w, out_dt=qdt)
    assert_close(got16, ref, cdt, qdt, "16-bit output")


@pytest.mark.parametrize("B", [8, 32])
@pytest.mark.parametrize("cdt,qdt,hq,hkv,D", [("bf16", "bf16", 8, 2, 128), ("f16", "f16", 16, 2, 64),
                                              ("fp8", "bf16", 8, 2, 128), ("fp8", "f16", 4, 4, 64)])
def test_prefill_parity_other_block_sizes(cdt, qdt, hq, hkv, D, B):
    """Block sizes 8 and 32: an iteration's two 16-token tiles come from four blocks or from one;
    fp8 at B = 8 stages each block's value tile as stored and reads per-lane scales."""
    w = make_prefill(CTX, NEW, num_heads=hq, num_kv_heads=hkv, head_dim=D, dtype=cdt, q_dtype=qdt,
                     block_size=B, seed=hq * 100 + D + B)
    ref = run_oracle(w)
    assert_close(run_gpu(w, out_dt="f32"), ref, cdt, "f32", f"{cdt}/{qdt} Hq={hq} Hkv={hkv} D={D} B={B}")
    assert_close(run_gpu(w, out_dt=qdt), ref, cdt, qdt, f"16-bit output B={B}")


@pytest.mark.parametrize("scale", [-0.125, 0.0, 2.0])
@pytest.mark.parametrize("cdt,qdt", [("bf16", "bf16"), ("f16", "f16"), ("fp8", "bf16")])
def test_prefill_scale_sign_and_size(cdt, qdt, scale):
    """Any finite scale: negative (16-bit caches carry its sign in the query operand), zero (equal
    weights: the mean of the attended values) and large (nearly one-hot weights whose running max
    jumps by far more than the rescale slack from one tile to the next)."""
    w = make_prefill(CTX, NEW, num_heads=8, num_kv_heads=2, head_dim=128, dtype=cdt, q_dtype=qdt,
                     seed=700 + int(8 * scale))
    w.scale = scale
    ref = run_oracle(w)
    assert_close(run_gpu(w, out_dt="f32"), ref, cdt, "f32", f"{cdt}/{qdt} scale={scale}")


@pytest.mark.parametrize("B", [8, 32])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_poison_invariance_other_block_sizes_bit_exact(dtype, B):
    """Free blocks and unused slots filled with NaN or huge values change no output bit at block
    sizes 8 and 32 either (blocks past a group's last query stand in as real ones)."""
    outs = []
    for poison in ("nan", "big"):
        w = make_prefill([40, 333, 7, 0], [20, 70, 9, 45], num_heads=8, num_kv_heads=2, head_dim=128,
                         dtype=dtype, block_size=B, seed=15, poison=poison)
        outs.append(run_gpu(w, out_dt="f32"))
    assert np.all(np.isfinite(outs[0])) and np.array_equal(outs[0], outs[1])


def test_prompt_into_empty_cache_and_long_chunks():
    """Chunks as long as their sequences (several 64-row tiles per kv head, ragged last tile)."""
    w = make_prefill([0, 0, 0], [257, 64, 1], num_heads=8, num_kv_heads=2, head_dim=128,
                     dtype="bf16", seed=11)
    assert_close(run_gpu(w, out_dt="f32"), run_oracle(w), "bf16", "f32", "prompts")


def test_one_token_chunks_are_the_decode_step():
    """A chunk of one token per sequence is the decode step: pa_prefill and pa_decode agree on
    the same cache (both within tolerance of the oracle, and of each other)."""
    lens = [1, 17, 40, 333, 1024]
    w = make_workload(lens, num_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", seed=12)
    d = upload(w)
    lib.pa_write_kv(d.k_new, d.v_new, d.k_cache, d.v_cache, d.slots)
    S = w.num_seqs
    qs = torch.arange(S + 1, dtype=torch.int32, device="cuda")
    pre = torch.empty(S, w.num_heads, w.head_dim, dtype=torch.float32, device="cuda")
    dec = torch.empty_like(pre)
    lib.pa_prefill(pre, d.q, d.k_cache, d.v_cache, d.tables, d.lens, qs, w.scale, 1)
    ws = workspace_for(d.q, d.k_cache, d.tables, w.block_size)
    lib.pa_decode(dec, d.q, d.k_cache, d.v_cache, d.tables, d.lens, w.scale, workspace=ws)
    torch.cuda.synchronize()
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    oracle.write_kv(kp, vp, w.k_new, w.v_new, w.slots, w.block_size, w.dtype, in_dtype=w.new_dtype)
    ref = oracle.decode(w.q, kp, vp, w.tables, w.lens, w.block_size, w.scale, w.dtype)
    assert_close(to_numpy_f64(pre), ref, "bf16", "f32", "prefill of one token")
    assert np.max(np.abs(to_numpy_f64(pre) - to_numpy_f64(dec))) <= TOL["bf16"]


def test_empty_chunks_and_generous_max_query_len():
    w = make_prefill([10, 0, 50, 3], [0, 5, 0, 2], num_heads=4, num_kv_heads=1, head_dim=64,
                     dtype="f16", seed=13)
    assert_close(run_gpu(w, out_dt="f32", max_query_len=300), run_oracle(w), "f16", "f32",
                 "empty chunks")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_poison_and_placement_invariance_bit_exact(dtype):
    """Unused slots and free blocks (NaN, huge values or random bits) and where the blocks sit do
    not change a single output bit."""
    outs = []
    for poison, ps in (("nan", 0), ("big", 0), ("random", 1)):
        w = make_prefill([40, 333, 7], [20, 70, 9], num_heads=8, num_kv_heads=2, head_dim=128,
                         dtype=dtype, seed=14, poison=poison)
        if ps:  # same logical data, other physical blocks: permute the pool and remap the tables
            perm = np.random.default_rng(ps).permutation(w.num_blocks)
            inv = np.argsort(perm)
            w.k_pool, w.v_pool = w.k_pool[perm].copy(), w.v_pool[perm].copy()
            if w.k_scale is not None:
                w.k_scale, w.v_scale = w.k_scale[perm].copy(), w.v_scale[perm].copy()
            w.tables = np.where(w.tables >= 0, inv[np.maximum(w.tables, 0)], -1).astype(np.int32)
            w.slots = (inv[w.slots // w.block_size] * w.block_size + w.slots % w.block_size).astype(np.int32)
        outs.append(run_gpu(w, out_dt="f32"))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_bf16_values_beyond_fp16_range():
    """bf16 has fp32's exponent range: two context tokens hold +-70144 (past fp16's largest value)
    in two dims here. The rows that attend them are finite and match the oracle within 2e-3 plus
    2^-14 of sum_t p_t |v_t| (the oracle run on |V|), and every other row has the very bits it has
    without the large values (a column's arithmetic depends on its own data alone)."""
    ctx, new = [300, 40, 1000], [64, 19, 100]
    kw = dict(num_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", seed=31)
    base = make_prefill(ctx, new, **kw)
    w = make_prefill(ctx, new, **kw)
    B, G = w.block_size, w.num_heads // w.num_kv_heads
    big = [(0, 1, 150), (2, 0, 900)]  # (sequence, kv head, context position)
    for s, h, p in big:
        blk = int(w.tables[s, p // B])
        w.v_pool[blk, h, 3, p % B] = 0x4789   # +70144
        w.v_pool[blk, h, 77, p % B] = 0xC789  # -70144
    out0 = run_gpu(base, out_dt="f32")
    out = run_gpu(w, out_dt="f32")
    ref = run_oracle(w)
    mag = run_oracle(dataclasses.replace(w, v_pool=w.v_pool & np.uint16(0x7FFF),
                                         v_new=w.v_new & np.uint16(0x7FFF)))
    qs = w.query_start
    hit = np.zeros(out.shape[:2], dtype=bool)  # [token row, query head] attends a large value
    for s, h, p in big:
        L, n = int(w.lens[s]), int(qs[s + 1] - qs[s])
        for t in range(int(qs[s]), int(qs[s + 1])):
            if L - n + (t - int(qs[s])) >= p:
                hit[t, h * G:(h + 1) * G] = True
    assert hit.any() and (~hit).any()
    assert np.all(np.isfinite(out[hit]))
    err = np.abs(out[hit] - ref[hit])
    lim = 2e-3 + 2.0 ** -14 * mag[hit]
    assert np.all(err <= lim), f"max err {err.max():.3e}, worst ratio {np.max(err / lim):.3f}"
    assert_close(out[~hit], ref[~hit], "bf16", "f32", "rows without large values")
    assert np.array_equal(out[~hit], out0[~hit])


def test_full_size_chunked_prefill_sampled_rows():
    """16 sequences append 512-token chunks to contexts of 0..3584 tokens (32 query / 8 kv heads,
    bf16): the shape the prefill bench times, checked on every sequence's first, middle and last
    rows and a seeded sample of the rest."""
    rng = np.random.default_rng(15)
    ctx = rng.integers(0, 3584, endpoint=True, size=16)
    w = make_prefill(ctx, [512] * 16, num_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                     seed=15)
    got = run_gpu(w, out_dt="f32")
    qs = w.query_start
    rows = set(rng.choice(w.q.shape[0], size=48, replace=False).tolist())
    for s in range(16):
        rows |= {int(qs[s]), int((qs[s] + qs[s + 1]) // 2), int(qs[s + 1] - 1)}
    rows = sorted(rows)
    ref = run_oracle(w, tokens=rows)
    assert_close(got[rows], ref[rows], "bf16", "f32", "full-size sampled rows")


def _rows_for_prefix(tokens, Hq, Hkv, D, dt):
    """Synthetic per-position q, k, v that depend on the whole prefix (as a model's would): row p
    is drawn from a generator seeded by the digest of tokens[:p+1]."""
    import hashlib
    from workloads import round_to
    q = np.empty((len(tokens), Hq, D), np.float32)
    k = np.empty((len(tokens), Hkv, D), np.float32)
    v = np.empty((len(tokens), Hkv, D), np.float32)
    h = hashlib.sha256()
    for p, t in enumerate(tokens):
        h.update(int(t).to_bytes(8, "little"))
        rng = np.random.default_rng(int.from_bytes(h.digest()[:8], "little"))
        q[p] = rng.standard_normal((Hq, D), dtype=np.float32)
        k[p] = rng.standard_normal((Hkv, D), dtype=np.float32)
        v[p] = rng.standard_normal((Hkv, D), dtype=np.float32)
    return round_to(q, dt), round_to(k, dt), round_to(v, dt)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_prefix_cache_end_to_end_reuses_blocks_bit_exact(dt):
    """Request A prefills its whole prompt and indexes its full blocks; request B shares A's
    40-token system prompt, finds its first 32 tokens (2 full blocks) cached, and prefills only
    the rest over them. B's rows equal (bit for bit) a run that prefills B's whole prompt into
    fresh blocks, and the oracle within tolerance (bf16 weights as hi part + remainder, fp16
    weights as one operand)."""
    from paged_kv_cache_318_amd.blocks import CachingBlockPool
    Hq, Hkv, D, B = 8, 2, 128, 16
    rng = np.random.default_rng(21)
    system = rng.integers(0, 32000, size=40).tolist()
    pa_ = system + rng.integers(0, 32000, size=60).tolist()
    pb_ = system + rng.integers(0, 32000, size=30).tolist()
    NB = 32
    pool = CachingBlockPool(NB, B, free_order=rng.permutation(NB).tolist())
    tdt = torch_dtype(dt)
    kc = torch.full((NB, Hkv, B, D), float("nan"), dtype=tdt, device="cuda")
    vc = torch.full((NB, Hkv, D, B), float("nan"), dtype=tdt, device="cuda")
    scale = D ** -0.5

    def bf(a):
        if dt == "f16":
            return torch.from_numpy(np.ascontiguousarray(a)).cuda()
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    def run(seq, tokens, start):
        """Write positions start.. of ``tokens`` and prefill their rows; returns f32 rows."""
        q, k, v = _rows_for_prefix(tokens, Hq, Hkv, D, dt)
        table = pool.tables[seq]
        slots = np.array([table[p // B] * B + p % B for p in range(start, len(tokens))], np.int32)
        lib.pa_write_kv(bf(k[start:]), bf(v[start:]), kc, vc, torch.from_numpy(slots).cuda())
        out = torch.empty(len(tokens) - start, Hq, D, dtype=torch.float32, device="cuda")
        tab = torch.from_numpy(pool.block_table([seq])).cuda()
        lens = torch.tensor([len(tokens)], dtype=torch.int32, device="cuda")
        qs = torch.tensor([0, len(tokens) - start], dtype=torch.int32, device="cuda")
        lib.pa_prefill(out, bf(q[start:]), kc, vc, tab, lens, qs, scale, len(tokens) - start)
        torch.cuda.synchronize()
        return out.cpu().numpy(), q, k, v

    assert pool.add_sequence_cached(0, pa_) == 0
    run(0, pa_, 0)
    pool.register(0, pa_)
    cached = pool.add_sequence_cached(1, pb_)
    assert cached == 32 and pool.tables[1][:2] == pool.tables[0][:2]
    got, q, k, v = run(1, pb_, cached)
    assert pool.add_sequence(2, len(pb_)) and pool.tables[2][0] not in pool.tables[0]
    full, _, _, _ = run(2, pb_, 0)
    assert np.array_equal(got, full[cached:])
    # oracle: B's whole prompt in B's blocks (the shared ones hold A's identical prefix)
    nan = np.float16(np.nan) if dt == "f16" else np.uint16(0x7FC0)
    kp = np.full((NB, Hkv, B, D), nan, k.dtype)
    vp = np.full((NB, Hkv, D, B), nan, v.dtype)
    slots = np.array([pool.tables[1][p // B] * B + p % B for p in range(len(pb_))], np.int32)
    oracle.write_kv(kp, vp, k, v, slots, B, dt)
    ref = oracle.prefill(q[cached:], kp, vp, pool.block_table([1]), np.array([len(pb_)]),
                         np.array([0, len(pb_) - cached]), B, scale, dt)
    assert_close(got.astype(np.float64), ref, dt, "f32", "prefix-cached request")
