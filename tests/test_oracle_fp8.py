"""Pins of the oracle's fp8 dequantisation (CPU only).

The 8-bit KV cache ("PagedAttention", Ultralytics glossary, section "関連手法") stores keys and
values as OCP E4M3 codes with one fp32 scale per (physical block, kv head), separate for keys and
values: the real value of a stored code c in block b, kv head g is e4m3(c) * scale[b][g]. These
tests tie the oracle's reading of that to things outside it:

* closed forms on a pool whose physical block ids differ from the logical positions and whose key
  and value scales differ per block -- a single token gives its own dequantised value, a zero
  query gives the mean of the dequantised values, and a huge score scale picks the block whose
  *key* scale is largest. Indexing the scales by logical block, or swapping the key and value
  scales, changes every one of these answers;
* the same decode over a float pool built block by block with PyTorch's float8_e4m3fn decoder
  (no table involved);
* the quantisation effect: the same draws stored as bf16 and as fp8 differ, element by element and
  in the attention output, by no more than half an E4M3 step (plus bf16's own rounding) allows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload

B, D, HKV = 4, 4, 2
TABLE = [4, 1, 3]            # logical block j lives in physical block TABLE[j]
NB = 6


def torch_e4m3(codes) -> np.ndarray:
    """float64 value of E4M3 codes, decoded by PyTorch (independent of the oracle's table)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _scales():
    """Key and value scales [NB][HKV], chosen so that the block with the largest key scale among
    the sequence's physical blocks (head 0: physical 1 = logical 1; head 1: physical 4 = logical 0)
    is neither the one a logical index would pick (k_scale[0..2]: logical 0 for head 0, logical 2
    for head 1) nor the one the value scales would pick (v_scale[TABLE]: the same)."""
    ks = np.full((NB, HKV), 0.75, np.float32)
    vs = np.full((NB, HKV), 0.6, np.float32)
    ks[4] = [0.5, 3.0]
    ks[1] = [2.0, 0.125]
    ks[3] = [1.0, 1.0]
    ks[0] = [3.0, 0.0625]        # unused block: a logical-index reading would take it
    ks[2] = [0.1, 4.0]
    vs[4] = [4.0, 0.5]
    vs[1] = [0.2, 0.375]
    vs[3] = [1.0, 1.5]
    vs[0] = [7.0, 9.0]
    vs[2] = [5.0, 11.0]
    return ks, vs


def _pool(k_codes, v_codes, L):
    """fp8 pool holding one sequence's codes [L][HKV][D] at TABLE; other slots hold NaN codes."""
    kp = np.full((NB, HKV, B, D), 0x7F, np.uint8)
    vp = np.full((NB, HKV, D, B), 0x7F, np.uint8)
    for t in range(L):
        kp[TABLE[t // B], :, t % B, :] = k_codes[t]
        vp[TABLE[t // B], :, :, t % B] = v_codes[t]
    tables = np.array([TABLE + [-1]], np.int32)
    return kp, vp, tables, np.array([L], np.int32)


def _random_codes(rng, L):
    """Finite E4M3 codes of moderate magnitude (exponent fields 3..10), random signs."""
    exp = rng.integers(3, 11, size=(L, HKV, D))
    man = rng.integers(0, 8, size=(L, HKV, D))
    sgn = rng.integers(0, 2, size=(L, HKV, D))
    return ((sgn << 7) | (exp << 3) | man).astype(np.uint8)


def _both_routes(q, kp, vp, tables, lens, scale, ks, vs):
    """The oracle's two decode routes, fp8 cache, bf16-free float queries (q given as float32)."""
    args = (q, kp, vp, tables, lens, B, scale, "fp8", "f32", ks, vs)
    return oracle.decode(*args), oracle.decode_blockwise(*args)


def _dequant(codes_tok, scales_phys, t):
    """Real value of token t: torch-decoded code times the scale of its *physical* block."""
    return torch_e4m3(codes_tok) * scales_phys[TABLE[t // B]][:, None].astype(np.float64)


def test_fp8_single_token_is_its_dequantised_value():
    """L = 1: the output of every query head is the token's value, e4m3(code) * v_scale[pb][g]."""
    rng = np.random.default_rng(21)
    ks, vs = _scales()
    kc, vc = _random_codes(rng, 1), _random_codes(rng, 1)
    kp, vp, tables, lens = _pool(kc, vc, 1)
    q = rng.standard_normal((1, 2 * HKV, D)).astype(np.float32)
    want = _dequant(vc[0], vs, 0)                         # [HKV][D]
    for out in _both_routes(q, kp, vp, tables, lens, 0.7, ks, vs):
        for h in range(2 * HKV):
            np.testing.assert_array_equal(out[0, h], want[h // 2])


@pytest.mark.parametrize("L", [5, 9, 12])
def test_fp8_zero_query_is_the_mean_of_dequantised_values(L):
    """q = 0: equal weights, so the output is the mean over t < L of e4m3(v_code) * v_scale[pb(t)]
    -- with pb(t) the physical block the table names, and the *value* scale."""
    rng = np.random.default_rng(30 + L)
    ks, vs = _scales()
    kc, vc = _random_codes(rng, L), _random_codes(rng, L)
    kp, vp, tables, lens = _pool(kc, vc, L)
    q = np.zeros((1, HKV, D), np.float32)
    want = np.mean([_dequant(vc[t], vs, t) for t in range(L)], axis=0)
    for out in _both_routes(q, kp, vp, tables, lens, 1.0, ks, vs):
        np.testing.assert_allclose(out[0], want, rtol=1e-14, atol=1e-15)


def test_fp8_huge_scale_picks_the_block_with_the_largest_key_scale():
    """Every key code is 1.0 and the query is positive, so token t's score is proportional to
    k_scale[pb(t)][g]; with a huge score scale the weights go to the block whose key scale is
    largest (ties inside it share equally). Head 0 must pick logical block 1 (physical 1, key
    scale 2.0) and head 1 logical block 0 (physical 4, key scale 3.0); a logical-index reading or
    the value scales would pick logical block 0 for head 0 and logical block 2 for head 1."""
    L = 11                                                # blocks 0, 1 full; block 2 has 3 tokens
    rng = np.random.default_rng(40)
    ks, vs = _scales()
    kc = np.full((L, HKV, D), 0x38, np.uint8)             # e4m3 0x38 = 1.0
    assert torch_e4m3(np.array([0x38]))[0] == 1.0
    vc = _random_codes(rng, L)
    kp, vp, tables, lens = _pool(kc, vc, L)
    q = np.full((1, HKV, D), 0.5, np.float32)
    winners = {0: 1, 1: 0}                                # head -> logical block
    want = np.empty((HKV, D))
    for g, j in winners.items():
        toks = [t for t in range(j * B, min(L, (j + 1) * B))]
        want[g] = np.mean([_dequant(vc[t], vs, t)[g] for t in toks], axis=0)
    for out in _both_routes(q, kp, vp, tables, lens, 1e3, ks, vs):
        np.testing.assert_allclose(out[0], want, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 8)])
def test_fp8_decode_equals_decode_of_a_torch_dequantised_pool(hq, hkv):
    """Every physical block of the generator's fp8 pool is dequantised with PyTorch's decoder and
    that block's own key / value scale (no table involved); the oracle's fp8 decode must equal its
    float decode of that pool."""
    w = make_workload([1, 7, 16, 17, 40, 63], num_heads=hq, num_kv_heads=hkv, head_dim=16,
                      block_size=8, dtype="fp8", seed=50, poison="random")
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    ks, vs = w.k_scale.copy(), w.v_scale.copy()
    oracle.write_kv(kp, vp, w.k_new, w.v_new, w.slots, w.block_size, "fp8", ks, vs, w.new_dtype)
    kf = torch_e4m3(kp) * ks[:, :, None, None].astype(np.float64)
    vf = torch_e4m3(vp) * vs[:, :, None, None].astype(np.float64)
    ref = oracle.decode(w.q, kf, vf, w.tables, w.lens, w.block_size, w.scale, "f32", w.q_dtype)
    assert np.all(np.isfinite(ref))
    for fn in (oracle.decode, oracle.decode_blockwise):
        got = fn(w.q, kp, vp, w.tables, w.lens, w.block_size, w.scale, "fp8", w.q_dtype, ks, vs)
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------------------------
# Quantisation effect: the same draws stored as bf16 and as fp8
# ----------------------------------------------------------------------------------------------

U_BF16 = 2.0 ** -8      # unit roundoff of bf16 (8 significant bits)
U_E4M3 = 2.0 ** -4      # of E4M3 normals (4 significant bits)
HALF_SUB = 2.0 ** -10   # half the E4M3 subnormal step (2^-9)


def element_bound(b, s):
    """Bound on |fp8 value - bf16 value| of one element whose bf16 value is b, stored in a block of
    scale s. Both come from the same float32 draw x with |x| <= |b| / (1 - U_BF16):
      fp8: y = fl32(x / s) (relative error 2^-24), rounded to E4M3 (at most U_E4M3 |y| for
           normals, HALF_SUB below them), times s; |y| beyond 448 saturates to 448;
      bf16: |x - b| <= U_BF16 |x|.
    The rounding terms add; saturation adds what lies beyond 448 s."""
    x = np.abs(b) / (1.0 - U_BF16)
    rnd = (U_E4M3 * (1 + 2.0 ** -24) + 2.0 ** -24 + U_BF16) * x + HALF_SUB * s
    sat = np.maximum(0.0, x - 448.0 * s)
    return rnd + sat


def _twins(lens, hq, hkv, Dh, B_, seed):
    """The same seeded draws stored as fp8 (+ scales) and as bf16: identical lengths, tables,
    queries and new tokens (the generator draws in the same order for both)."""
    kw = dict(num_heads=hq, num_kv_heads=hkv, head_dim=Dh, block_size=B_, seed=seed)
    w8 = make_workload(lens, dtype="fp8", q_dtype="bf16", **kw)
    wb = make_workload(lens, dtype="bf16", **kw)
    assert np.array_equal(w8.tables, wb.tables) and np.array_equal(w8.q, wb.q)
    assert np.array_equal(w8.k_new, wb.k_new)
    return w8, wb


def _pools_after_write(w):
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    ks = None if w.k_scale is None else w.k_scale.copy()
    vs = None if w.v_scale is None else w.v_scale.copy()
    oracle.write_kv(kp, vp, w.k_new, w.v_new, w.slots, w.block_size, w.dtype, ks, vs, w.new_dtype)
    return kp, vp, ks, vs


def quantisation_effect(w8, wb, seqs=None):
    """(max |fp8 output - bf16 output|, max of the derived bound, elements checked) over the given
    sequences; raises if any dequantised element or output element breaks its bound."""
    kp8, vp8, ks, vs = _pools_after_write(w8)
    kpb, vpb, _, _ = _pools_after_write(wb)
    seqs = range(w8.num_seqs) if seqs is None else seqs
    o8 = oracle.decode(w8.q, kp8, vp8, w8.tables, w8.lens, w8.block_size, w8.scale, "fp8",
                       "bf16", ks, vs, seqs=seqs)
    ob = oracle.decode(wb.q, kpb, vpb, wb.tables, wb.lens, wb.block_size, wb.scale, "bf16",
                       seqs=seqs)
    G = w8.num_heads // w8.num_kv_heads
    q64 = oracle.to_f64(w8.q, "bf16")
    worst_err, worst_bound, n = 0.0, 0.0, 0
    for s in seqs:
        L = int(w8.lens[s])
        K8, V8 = oracle.sequence_kv(kp8, vp8, w8.tables[s], L, w8.block_size, "fp8", ks, vs)
        Kb, Vb = oracle.sequence_kv(kpb, vpb, wb.tables[s], L, wb.block_size, "bf16")
        # the scale each token was stored with: its physical block's (from the table)
        phys = np.array([w8.tables[s][t // w8.block_size] for t in range(L)])
        eK = element_bound(Kb, ks[phys][:, :, None].astype(np.float64))
        eV = element_bound(Vb, vs[phys][:, :, None].astype(np.float64))
        assert np.all(np.abs(K8 - Kb) <= eK), f"sequence {s}: a dequantised key is off"
        assert np.all(np.abs(V8 - Vb) <= eV), f"sequence {s}: a dequantised value is off"
        for h in range(w8.num_heads):
            g = h // G
            # score error <= scale * sum_d |q_d| eK[t, d]; weights then move by at most a factor
            # exp(+-2 delta), so the output moves by (exp(2 delta) - 1) max|v| + max eV
            delta = float(w8.scale * (eK[:, g, :] @ np.abs(q64[s, h])).max())
            bound = math.expm1(2 * delta) * np.abs(Vb[:, g, :]).max(axis=0) + eV[:, g, :].max(axis=0)
            err = np.abs(o8[s, h] - ob[s, h])
            assert np.all(err <= bound), f"sequence {s}, head {h}: output beyond the bound"
            worst_err = max(worst_err, float(err.max()))
            worst_bound = max(worst_bound, float(bound.max()))
            n += err.size
    return worst_err, worst_bound, n


@pytest.mark.parametrize("hq,hkv,Dh,B_", [(4, 2, 16, 8), (8, 2, 64, 16), (4, 4, 128, 16)])
def test_fp8_quantisation_effect_within_half_an_e4m3_step(hq, hkv, Dh, B_):
    w8, wb = _twins([1, 9, 16, 33, 130, 400], hq, hkv, Dh, B_, seed=60 + Dh)
    err, bound, n = quantisation_effect(w8, wb)
    assert n > 0 and 0.0 < err < bound


def test_fp8_quantisation_effect_fp8_workload_shape():
    """The fp8 KV decode workload's shape (32 query / 8 kv heads x 128, block size 16, contexts of
    16K..32K tokens), on two of its sequences: the fp8 outputs stay within the bound of the bf16
    ones. The observed figure is reported with the design notes."""
    rng = np.random.default_rng(5)
    lens = rng.integers(16384, 32768, endpoint=True, size=2)
    w8, wb = _twins(lens, 32, 8, 128, 16, seed=5)
    err, bound, n = quantisation_effect(w8, wb)
    print(f"fp8 vs bf16 cache, 2 sequences of {lens.tolist()} tokens: max |diff| {err:.3e} "
          f"over {n} output elements (derived bound {bound:.3e})")
    assert err < 0.1
