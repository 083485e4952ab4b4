"""Pins of the oracle's paged decode attention and split-K merge.

Pinned against: brute-force contiguous attention written as plain Python
loops (math.exp, no numpy), placement invariance, closed-form special cases
(one token, zero query, equal keys, one dominant key), the GQA head mapping,
the log-sum-exp merge identity, and library conversions of the 16-bit
formats. A planted mistake in a copy of the oracle must fail a pin.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention, pool

BS = 16


# --------------------------------------------------------------- helpers ----
def brute_attention(q, k, v, scale, group):
    """Textbook softmax attention with Python floats. q: [Hq][D]; k, v: [L][Hkv][D]."""
    out = []
    for h in range(len(q)):
        g = h // group
        scores = [scale * sum(qd * kd for qd, kd in zip(q[h], k[t][g])) for t in range(len(k))]
        top = max(scores)
        e = [math.exp(s - top) for s in scores]
        tot = sum(e)
        dim = len(q[h])
        out.append([sum(e[t] * v[t][g][d] for t in range(len(k))) / tot for d in range(dim)])
    return out


def f16_bits(rng, shape):
    return rng.standard_normal(shape).astype(np.float16).view(np.uint16)


def build_paged(rng, lengths, hkv, dim, num_blocks, extra_perm=True):
    """Place each sequence's logical K/V into randomly chosen physical blocks.

    Returns (pool6, tables, logical_k_raw, logical_v_raw). Unused blocks and
    unused tail slots hold fp16 NaN bits so any stray read poisons the result.
    """
    pool6 = np.full((1, 2, num_blocks, hkv, BS, dim), 0x7E00, dtype=np.uint16)
    need = sum(-(-l // BS) for l in lengths)
    ids = rng.permutation(num_blocks)[:need] if extra_perm else np.arange(need)
    maxb = max(-(-l // BS) for l in lengths)
    tables = np.full((len(lengths), maxb + 2), -1, dtype=np.int32)
    ks, vs, pos = [], [], 0
    for i, length in enumerate(lengths):
        k = f16_bits(rng, (length, hkv, dim))
        v = f16_bits(rng, (length, hkv, dim))
        ks.append(k)
        vs.append(v)
        nb = -(-length // BS)
        for j in range(nb):
            b = int(ids[pos]); pos += 1
            tables[i, j] = b
            lo, hi = j * BS, min((j + 1) * BS, length)
            pool6[0, 0, b, :, : hi - lo, :] = k[lo:hi].transpose(1, 0, 2)
            pool6[0, 1, b, :, : hi - lo, :] = v[lo:hi].transpose(1, 0, 2)
    return pool6, tables, ks, vs


def f64(raw):
    return raw.view(np.float16).astype(np.float64)


# ------------------------------------------------------------------ pins ----
def check_against_brute_force(decode_fn, seed=0):
    rng = np.random.default_rng(seed)
    for hq, hkv, dim, lengths in [(2, 2, 8, [1, 5, 16, 17, 33]),
                                  (4, 2, 4, [3, 32, 40]),
                                  (4, 1, 6, [20, 7])]:
        pool6, tables, ks, vs = build_paged(rng, lengths, hkv, dim, num_blocks=16)
        q = rng.standard_normal((len(lengths), hq, dim))
        scale = 1.0 / math.sqrt(dim)
        got = decode_fn(pool6, 0, q, tables, np.array(lengths), scale, "f16")
        for i, length in enumerate(lengths):
            ref = brute_attention(q[i].tolist(), f64(ks[i]).tolist(), f64(vs[i]).tolist(),
                                  scale, hq // hkv)
            assert np.allclose(got[i], np.array(ref), rtol=1e-12, atol=1e-12), (hq, hkv, length)


def test_paged_decode_matches_brute_force():
    check_against_brute_force(attention.paged_decode)


def test_placement_invariance_is_bitwise():
    rng = np.random.default_rng(3)
    lengths = [37, 1, 64, 15]
    a = build_paged(rng, lengths, 2, 16, 32, extra_perm=True)
    # Same logical data as in a, placed in other physical blocks.
    pool_b = np.full_like(a[0], 0x7E00)
    tables_b = np.full_like(a[1], -1)
    ids = np.random.default_rng(7).permutation(32)
    pos = 0
    for i, length in enumerate(lengths):
        for j in range(-(-length // BS)):
            nb = int(ids[pos]); pos += 1
            tables_b[i, j] = nb
            pool_b[0, :, nb] = a[0][0, :, a[1][i, j]]
    assert not np.array_equal(tables_b, a[1])
    q = rng.standard_normal((len(lengths), 4, 16))
    out_a = attention.paged_decode(a[0], 0, q, a[1], np.array(lengths), 0.25, "f16")
    out_b = attention.paged_decode(pool_b, 0, q, tables_b, np.array(lengths), 0.25, "f16")
    assert np.array_equal(out_a, out_b)


def test_single_token_gives_its_value_exactly():
    rng = np.random.default_rng(4)
    pool6, tables, ks, vs = build_paged(rng, [1, 1], 2, 8, 8)
    q = rng.standard_normal((2, 4, 8)) * 10
    out = attention.paged_decode(pool6, 0, q, tables, np.array([1, 1]), 0.3, "f16")
    for i in range(2):
        for h in range(4):
            assert np.array_equal(out[i, h], f64(vs[i])[0, h // 2])


def test_zero_query_and_equal_keys_give_mean_value():
    rng = np.random.default_rng(5)
    lengths = [19, 48]
    pool6, tables, ks, vs = build_paged(rng, lengths, 1, 8, 8)
    out = attention.paged_decode(pool6, 0, np.zeros((2, 1, 8)), tables, np.array(lengths),
                                 0.5, "f16")
    for i in range(2):
        assert np.allclose(out[i, 0], f64(vs[i])[:, 0].mean(axis=0), rtol=1e-13, atol=1e-15)
    # Equal keys: overwrite every K slot of sequence 0 with one key.
    key = f16_bits(rng, (8,))
    for j in range(2):
        pool6[0, 0, tables[0, j], 0] = key
    q = rng.standard_normal((2, 1, 8))
    out = attention.paged_decode(pool6, 0, q, tables, np.array(lengths), 0.5, "f16")
    assert np.allclose(out[0, 0], f64(vs[0])[:, 0].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(6)
    lengths = [40]
    pool6, tables, ks, vs = build_paged(rng, lengths, 1, 8, 8)
    k = f64(ks[0])[:, 0]
    q = rng.standard_normal((1, 1, 8))
    s = k @ q[0, 0]
    target = int(np.argmax(s))
    gap = s[target] - np.sort(s)[-2]
    q *= 60.0 / gap  # top score now exceeds every other by 60
    out = attention.paged_decode(pool6, 0, q, tables, np.array(lengths), 1.0, "f16")
    assert np.allclose(out[0, 0], f64(vs[0])[target, 0], atol=1e-9)


def check_gqa_mapping(decode_fn):
    """Each kv head's V is a constant c_g, so query head h must output c_{h // G}."""
    hq, hkv, dim = 8, 2, 4
    lengths = [21]
    pool6 = np.zeros((1, 2, 4, hkv, BS, dim), dtype=np.uint16)
    tables = np.array([[2, 0]], dtype=np.int32)
    consts = np.array([1.5, -3.0], dtype=np.float16)
    rng = np.random.default_rng(8)
    for g in range(hkv):
        pool6[0, 0, :, g] = f16_bits(rng, (4, BS, dim))
        pool6[0, 1, :, g] = consts[g].view(np.uint16)
    q = rng.standard_normal((1, hq, dim))
    out = decode_fn(pool6, 0, q, tables, np.array(lengths), 0.5, "f16")
    for h in range(hq):
        assert np.allclose(out[0, h], float(consts[h // (hq // hkv)]), rtol=1e-14), h


def test_gqa_head_mapping():
    check_gqa_mapping(attention.paged_decode)


def test_large_scores_do_not_overflow():
    rng = np.random.default_rng(9)
    pool6, tables, ks, vs = build_paged(rng, [30], 1, 8, 4)
    q = rng.standard_normal((1, 1, 8)) * 1e4
    out = attention.paged_decode(pool6, 0, q, tables, np.array([30]), 1.0, "f16")
    assert np.all(np.isfinite(out))


def check_split_merge(partials_fn, merge_fn):
    rng = np.random.default_rng(10)
    hq, hkv, dim = 4, 2, 8
    for length in (1, 15, 16, 17, 100, 513):
        k = f64(f16_bits(rng, (length, hkv, dim)))
        v = f64(f16_bits(rng, (length, hkv, dim)))
        q = rng.standard_normal((hq, dim))
        whole = attention.attend(q, k, v, 0.35)
        for ps in (16, 32, 64, 512, 1024):
            m, l, o = partials_fn(q, k, v, 0.35, ps)
            assert m.shape[0] == -(-length // ps)
            assert np.allclose(merge_fn(m, l, o), whole, rtol=1e-12, atol=1e-12), (length, ps)


def test_split_merge_identity():
    check_split_merge(attention.partials, attention.merge)


def test_partials_definition_on_one_partition():
    """With one partition, m is the max score, l sums exp(s - m), o is the attention."""
    rng = np.random.default_rng(11)
    k = f64(f16_bits(rng, (10, 1, 4)))
    v = f64(f16_bits(rng, (10, 1, 4)))
    q = rng.standard_normal((1, 4))
    m, l, o = attention.partials(q, k, v, 1.0, 16)
    s = [sum(a * b for a, b in zip(q[0], k[t, 0])) for t in range(10)]
    assert m[0, 0] == pytest.approx(max(s), rel=1e-14)
    assert l[0, 0] == pytest.approx(sum(math.exp(x - max(s)) for x in s), rel=1e-13)
    assert np.allclose(o[0, 0], attention.attend(q, k, v, 1.0)[0], rtol=1e-13)


def test_bf16_and_f16_decoding_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = pool.raw_to_f64(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    ref = ref.numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(ours), fin)
    assert np.array_equal(ours[fin], ref[fin])
    ours16 = pool.raw_to_f64(bits, "f16")
    ref16 = torch.from_numpy(bits.view(np.int16).copy()).view(torch.float16).to(torch.float64)
    fin16 = np.isfinite(ref16.numpy())
    assert np.array_equal(ours16[fin16], ref16.numpy()[fin16])
    assert pool.raw_to_f64(np.uint16(0x3F80), "bf16") == 1.0
    assert pool.raw_to_f64(np.uint16(0xC000), "bf16") == -2.0
    assert pool.raw_to_f64(np.uint16(0x3C00), "f16") == 1.0


def test_zero_length_sequence_gives_zeros():
    rng = np.random.default_rng(12)
    pool6, tables, ks, vs = build_paged(rng, [5], 1, 4, 4)
    out = attention.paged_decode(pool6, 0, np.ones((2, 1, 4)), np.vstack([tables, tables]),
                                 np.array([5, 0]), 1.0, "f16")
    assert np.array_equal(out[1], np.zeros((1, 4)))


# --------------------------------------------------- planted mistakes ----
def _mutant_decode(kind):
    def decode(pool6, layer, q, tables, lens, scale, kv_dtype, k_scale=None, v_scale=None):
        out = np.zeros(q.shape)
        for i in range(q.shape[0]):
            length = int(lens[i])
            if kind == "off_by_one_tail":
                length = max(length - 1, 1)
            kr, vr = attention.gather(pool6, layer, tables[i], length)
            k, v = f64(kr), f64(vr)
            hq, hkv = q.shape[1], k.shape[1]
            for h in range(hq):
                g = h % hkv if kind == "gqa_modulo" else h // (hq // hkv)
                sc = 1.0 if kind == "no_scale" else scale
                if kind == "k_for_v":
                    v = k
                s = (k[:, g] @ q[i, h]) * sc
                p = np.exp(s - s.max())
                out[i, h] = (p @ v[:, g]) / p.sum()
        return out
    return decode


@pytest.mark.parametrize("kind", ["off_by_one_tail", "no_scale", "k_for_v"])
def test_planted_mistakes_fail_brute_force(kind):
    with pytest.raises(AssertionError):
        check_against_brute_force(_mutant_decode(kind))


def test_planted_gqa_mistake_fails_mapping_pin():
    with pytest.raises(AssertionError):
        check_gqa_mapping(_mutant_decode("gqa_modulo"))


def test_planted_merge_mistake_fails_identity():
    def bad_merge(m, l, o):
        w = l  # forgets the exp(m_p - M) factor
        return (w[:, :, None] * o).sum(axis=0) / w.sum(axis=0)[:, None]
    with pytest.raises(AssertionError):
        check_split_merge(attention.partials, bad_merge)


# ----------------------------------------------- FP8 (E4M3) KV cache pins ----
# [P2] "vLLM 也不是银弹：真实部署中的坑", third pitfall: an FP8 KV cache. Each kv
# head has its own K scale and V scale, and a stored code means
# decode(code) * scale. The brute force below dequantises through torch's
# float8_e4m3fn conversion (a library routine, not the oracle's table) and
# attends with Python floats. The scales differ per head and between K and V
# by large factors, so applying a scale to the wrong operand or head moves
# every output far outside the tolerance.
FP8_K_SCALE = np.array([0.01, 0.37, 0.055], dtype=np.float32)
FP8_V_SCALE = np.array([0.25, 4.0, 0.8], dtype=np.float32)


def e4m3_codes(rng, shape):
    """Random finite E4M3 codes (never the NaN codes 0x7F / 0xFF)."""
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)


def build_paged_e4m3(rng, lengths, hkv, dim, num_blocks):
    """As build_paged, for a uint8 E4M3 pool; unused slots hold NaN codes."""
    pool6 = np.full((1, 2, num_blocks, hkv, BS, dim), 0x7F, dtype=np.uint8)
    ids = rng.permutation(num_blocks)
    maxb = max(-(-l // BS) for l in lengths)
    tables = np.full((len(lengths), maxb + 1), -1, dtype=np.int32)
    ks, vs, pos = [], [], 0
    for i, length in enumerate(lengths):
        k = e4m3_codes(rng, (length, hkv, dim))
        v = e4m3_codes(rng, (length, hkv, dim))
        ks.append(k)
        vs.append(v)
        for j in range(-(-length // BS)):
            b = int(ids[pos]); pos += 1
            tables[i, j] = b
            lo, hi = j * BS, min((j + 1) * BS, length)
            pool6[0, 0, b, :, : hi - lo, :] = k[lo:hi].transpose(1, 0, 2)
            pool6[0, 1, b, :, : hi - lo, :] = v[lo:hi].transpose(1, 0, 2)
    return pool6, tables, ks, vs


def torch_dequant(codes, scales):
    """[L, Hkv, D] codes -> nested Python floats, code value x its head's scale."""
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return (vals * scales.astype(np.float64)[None, :, None]).tolist()


def check_fp8_against_brute_force(decode_fn, seed=21):
    rng = np.random.default_rng(seed)
    for hq, hkv, dim, lengths in [(3, 3, 8, [1, 9, 16, 35]),
                                  (6, 3, 4, [17, 40]),
                                  (2, 2, 16, [50])]:
        ksc, vsc = FP8_K_SCALE[:hkv], FP8_V_SCALE[:hkv]
        pool6, tables, ks, vs = build_paged_e4m3(rng, lengths, hkv, dim, num_blocks=24)
        q = rng.standard_normal((len(lengths), hq, dim))
        scale = 1.0 / math.sqrt(dim)
        got = decode_fn(pool6, 0, q, tables, np.array(lengths), scale, "e4m3",
                        k_scale=ksc, v_scale=vsc)
        for i, length in enumerate(lengths):
            ref = brute_attention(q[i].tolist(), torch_dequant(ks[i], ksc),
                                  torch_dequant(vs[i], vsc), scale, hq // hkv)
            assert np.allclose(got[i], np.array(ref), rtol=1e-12, atol=1e-12), (hq, hkv, length)


def test_fp8_paged_decode_matches_brute_force():
    check_fp8_against_brute_force(attention.paged_decode)


def test_fp8_single_token_gives_scaled_value_exactly():
    """L = 1: the output is the stored V code times that head's V scale."""
    rng = np.random.default_rng(22)
    pool6, tables, ks, vs = build_paged_e4m3(rng, [1], 3, 8, 4)
    q = rng.standard_normal((1, 3, 8))
    out = attention.paged_decode(pool6, 0, q, tables, np.array([1]), 0.3, "e4m3",
                                 k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    ref = np.array(torch_dequant(vs[0], FP8_V_SCALE))[0]
    assert np.array_equal(out[0], ref)


def _fp8_mutant(kind):
    """paged_decode with one planted mistake in the FP8 scale handling."""
    def decode(pool6, layer, q, tables, lens, scale, kv_dtype, k_scale=None, v_scale=None):
        if kind == "swap_scales":
            k_scale, v_scale = v_scale, k_scale
        elif kind == "k_scale_for_both":
            v_scale = k_scale
        elif kind == "reversed_heads":
            k_scale, v_scale = k_scale[::-1].copy(), v_scale[::-1].copy()
        elif kind == "v_unscaled":
            v_scale = np.ones_like(v_scale)
        return attention.paged_decode(pool6, layer, q, tables, lens, scale, kv_dtype,
                                      k_scale=k_scale, v_scale=v_scale)
    return decode


@pytest.mark.parametrize("kind", ["swap_scales", "k_scale_for_both", "reversed_heads",
                                  "v_unscaled"])
def test_planted_fp8_scale_mistakes_fail_brute_force(kind):
    with pytest.raises(AssertionError):
        check_fp8_against_brute_force(_fp8_mutant(kind))
