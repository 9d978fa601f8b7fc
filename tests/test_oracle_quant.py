"""Pins of the oracle's FP8 KV rows (oracle/quant.py): the E4M3 code table
against the OCP 8-bit floating point definition (closed forms and the
format's named values), round-to-nearest-even against brute force over every
code, the per-row power-of-two scale against its defining inequality, the
quantisation error against the format's half-ulp bound, and FP8 paged
attention against the online-softmax oracle run on the read-back values.
CPU only."""
import math

import numpy as np
import pytest

import oracle
from oracle import quant


def test_named_e4m3_values():
    # OCP FP8 E4M3: bias 7, largest finite S.1111.110 = 448, NaN S.1111.111,
    # smallest normal 2^-6, smallest subnormal 2^-9, no infinities.
    named = {0x00: 0.0, 0x38: 1.0, 0x3F: 1.875, 0x40: 2.0, 0xC0: -2.0, 0x7E: 448.0,
             0xFE: -448.0, 0x08: 2.0 ** -6, 0x07: 7 * 2.0 ** -9, 0x01: 2.0 ** -9,
             0x30: 0.5, 0x77: 240.0}
    for code, val in named.items():
        assert quant.e4m3_decode(code) == val, hex(code)
        assert quant.e4m3_encode(val) == code, hex(code)
    assert math.isnan(quant.e4m3_decode(0x7F)) and math.isnan(quant.e4m3_decode(0xFF))
    assert quant.e4m3_encode(-0.0) == 0x80 and quant.e4m3_encode(0.0) == 0x00
    finite = [quant.e4m3_decode(c) for c in range(256) if c not in (0x7F, 0xFF)]
    assert len(set(finite)) == 253            # +0 and -0 compare equal
    assert max(finite) == 448.0 and min(finite) == -448.0


def test_every_code_round_trips():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert quant.e4m3_encode(quant.e4m3_decode(c)) == c


def _brute_force(x):
    best, best_d = None, None
    for c in range(0x7F):                     # non-negative finite codes
        d = abs(quant.e4m3_decode(c) - abs(x))
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | (0x80 if math.copysign(1.0, x) < 0 else 0)


def test_round_to_nearest_even_against_brute_force():
    rng = np.random.default_rng(3)
    xs = list(rng.uniform(-448, 448, 300)) + list(rng.uniform(-0.02, 0.02, 300))
    # exact midpoints between neighbouring codes (the ties)
    for c in range(0x7D):
        xs.append((quant.e4m3_decode(c) + quant.e4m3_decode(c + 1)) / 2)
    for x in xs:
        x = float(np.float32(x))
        assert quant.e4m3_encode(x) == _brute_force(x), x
    assert quant.e4m3_encode(1.0625) == 0x38 and quant.e4m3_encode(1.1875) == 0x3A
    assert quant.e4m3_encode(1.5 * 2.0 ** -9) == 0x02 and quant.e4m3_encode(0.5 * 2.0 ** -9) == 0x00


def test_row_scale_is_the_smallest_fitting_power_of_two():
    rng = np.random.default_rng(4)
    for _ in range(500):
        row = (rng.standard_normal(128) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32)
        e = quant.row_scale_exponent(row)
        amax = float(np.abs(row).max())
        assert amax <= 448.0 * 2.0 ** e
        assert amax > 448.0 * 2.0 ** (e - 1)
    for k in (-20, 0, 3, 40):
        assert quant.row_scale_exponent(np.array([448.0 * 2.0 ** k], np.float32)) == k
        assert quant.row_scale_exponent(np.array([449.0 * 2.0 ** k], np.float32)) == k + 1
    assert quant.row_scale_exponent(np.zeros(8, np.float32)) == 0


def test_quantisation_error_within_half_ulp():
    rng = np.random.default_rng(5)
    for _ in range(50):
        row = (rng.standard_normal(128) * rng.uniform(0.01, 100)).astype(np.float32)
        codes, sb = quant.quantize_row(row)
        back = quant.dequantize(codes[None], np.array([sb]))[0]
        e = sb - 127
        y = np.abs(row.astype(np.float64)) / 2.0 ** e
        ulp = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 1e-300))) - 3), 2.0 ** -9)
        assert np.all(np.abs(back - row) <= 0.5 * ulp * 2.0 ** e + 0.0)
        assert np.abs(row).max() / 2.0 ** e > 224.0      # the top code range is used
        assert not np.any(codes == 0x80)


def test_negative_zero_codes_are_stored_as_zero():
    row = np.array([-0.0, -1e-9, 3.0, -5.0], dtype=np.float32)
    codes, sb = quant.quantize_row(row)
    assert codes[0] == 0x00 and codes[1] == 0x00 and sb == 127 - 6


def test_fp8_attention_matches_online_oracle_on_read_back_values():
    rng = np.random.default_rng(6)
    N, H, bs, D, hq = 12, 2, 4, 16, 4
    kc, vc, ks, vs = quant.new_fp8_pool(N, H, bs, D)
    m = oracle.BlockManager(N, bs, rng.permutation(N))
    lens = [7, 1, 12]
    for b, L in enumerate(lens):
        slots = m.allocate_for_prefill(b, L)
        k = (rng.standard_normal((L, H, D)) * 3).astype(np.float32)
        v = rng.standard_normal((L, H, D)).astype(np.float32)
        quant.write_kv_fp8(k, v, slots, kc, vc, ks, vs, bs)
    q = rng.standard_normal((3, hq, D)).astype(np.float32)
    tabs = m.block_tables([0, 1, 2], 3, -1)
    got = quant.decode_attention_fp8(q, "f32", kc, vc, ks, vs, tabs, lens, 0.25)
    # the read-back values as a float32 pool (exact: E4M3 * 2^e fits float32)
    kf = quant.dequantize(kc, ks).astype(np.float32)
    vf = quant.dequantize(vc, vs).astype(np.float32)
    for b, L in enumerate(lens):
        ref = oracle.decode_attention_online(q[b], kf, vf, m.block_table(b), L, 0.25, "f32")
        assert np.abs(got[b] - ref).max() < 1e-12
    # untouched rows keep the poison pattern
    used = {pb for b in range(3) for pb in m.block_table(b)}
    for pb in set(range(N)) - used:
        assert np.all(kc[pb] == 0x7F) and np.all(ks[pb] == 0xFF)


def test_array_quantiser_equals_the_scalar_definition():
    rng = np.random.default_rng(8)
    rows = [(rng.standard_normal(64) * 10.0 ** rng.uniform(-8, 8)).astype(np.float32) for _ in range(60)]
    rows.append(np.zeros(64, np.float32))
    rows.append(np.array([-0.0] * 32 + [1.0] * 32, np.float32))
    ties = np.array([(quant.e4m3_decode(c) + quant.e4m3_decode(c + 1)) / 2 for c in range(0x70, 0x7D)],
                    np.float32)
    rows.append(np.concatenate([ties, -ties, np.full(64 - 2 * len(ties), 448.0, np.float32)]))
    rows.append(np.array([2.0 ** -140, -(2.0 ** -135)] + [0.0] * 62, np.float32))   # float32 subnormals
    arr = np.stack(rows)
    codes, sbytes = quant.quantize_rows(arr)
    for i, r in enumerate(rows):
        c, sb = quant.quantize_row(r)
        assert np.array_equal(codes[i], c) and sbytes[i] == sb, i


def _fp8_pool_with_spread_scales(rng, N, H, bs, D):
    """An 8-bit pool whose blocks hold rows of very different magnitudes, so
    that codes read with another block's scale bytes give other values."""
    kc, vc, ks, vs = quant.new_fp8_pool(N, H, bs, D)
    for b in range(N):
        mag = 2.0 ** (3 * b - 12)
        k = (rng.standard_normal((bs, H, D)) * mag).astype(np.float32)
        v = (rng.standard_normal((bs, H, D)) * mag * 0.5).astype(np.float32)
        quant.write_kv_fp8(k, v, [b * bs + o for o in range(bs)], kc, vc, ks, vs, bs)
    return kc, vc, ks, vs


def test_fp8_block_copy_keeps_every_read_back_value():
    """Copy-on-write of an 8-bit block ([impl-detail] "Copy-on-Write机制"):
    the new block reads back exactly the shared block's values, the
    attention of a table through it is unchanged, and no other block moves.
    Copying codes without their scale bytes fails the first check."""
    rng = np.random.default_rng(9)
    N, H, bs, D = 8, 2, 4, 16
    kc, vc, ks, vs = _fp8_pool_with_spread_scales(rng, N, H, bs, D)
    before = [(kc[b].copy(), vc[b].copy(), ks[b].copy(), vs[b].copy()) for b in range(N)]
    pairs = [(1, 6), (4, 2)]
    q = np.asarray(rng.standard_normal((1, 2 * H, D)), dtype=np.float32).astype(np.float16)
    ref = quant.decode_attention_fp8(q, "f16", kc, vc, ks, vs, np.array([[1, 4]]), [2 * bs - 1], 0.25)
    quant.copy_blocks_fp8(pairs, kc, vc, ks, vs)
    for s, d in pairs:
        assert not np.array_equal(quant.dequantize(before[d][0], before[d][2]),
                                  quant.dequantize(kc[s], ks[s]))     # the copy changes something
        assert np.array_equal(quant.dequantize(kc[d], ks[d]), quant.dequantize(kc[s], ks[s]))
        assert np.array_equal(quant.dequantize(vc[d], vs[d]), quant.dequantize(vc[s], vs[s]))
        assert np.array_equal(kc[d], kc[s]) and np.array_equal(vs[d], vs[s])
    for b in set(range(N)) - {d for _, d in pairs}:
        assert all(np.array_equal(x, y) for x, y in zip((kc[b], vc[b], ks[b], vs[b]), before[b]))
    out = quant.decode_attention_fp8(q, "f16", kc, vc, ks, vs, np.array([[6, 2]]), [2 * bs - 1], 0.25)
    assert np.array_equal(out, ref)


def test_fp8_swap_staging_round_trip():
    """Swap of 8-bit blocks ([impl-detail] "异构内存支持"): staged entry j
    holds block ids[j]'s codes and scale bytes (K half, then V half), reads
    back as that block's values, and scattering it onto other blocks
    reproduces every value there."""
    rng = np.random.default_rng(10)
    N, H, bs, D = 9, 3, 4, 8
    kc, vc, ks, vs = _fp8_pool_with_spread_scales(rng, N, H, bs, D)
    ids = [7, 0, 3]
    codes, scales = quant.gather_blocks_fp8(ids, kc, vc, ks, vs)
    assert codes.shape == (3, 2, H, bs, D) and scales.shape == (3, 2, H, bs)
    for j, b in enumerate(ids):
        assert np.array_equal(quant.dequantize(codes[j, 0], scales[j, 0]), quant.dequantize(kc[b], ks[b]))
        assert np.array_equal(quant.dequantize(codes[j, 1], scales[j, 1]), quant.dequantize(vc[b], vs[b]))
    want = [(quant.dequantize(kc[b], ks[b]), quant.dequantize(vc[b], vs[b])) for b in ids]
    dst = [2, 8, 5]
    quant.scatter_blocks_fp8(codes, scales, dst, kc, vc, ks, vs)
    for (wk, wv), b in zip(want, dst):
        assert np.array_equal(quant.dequantize(kc[b], ks[b]), wk)
        assert np.array_equal(quant.dequantize(vc[b], vs[b]), wv)


def _fp8_prefill_case(seed):
    rng = np.random.default_rng(seed)
    N, H, bs, D, hq = 24, 2, 4, 16, 6
    kc, vc, ks, vs = quant.new_fp8_pool(N, H, bs, D)
    order = rng.permutation(N)
    mgr = oracle.BlockManager(N, bs, order)
    lens = [13, 5, 9]
    for b, L in enumerate(lens):
        rows_k = (rng.standard_normal((L, H, D)) * 2.0 ** rng.integers(-4, 5, (L, H, 1))).astype(np.float32)
        rows_v = (rng.standard_normal((L, H, D)) * 2.0 ** rng.integers(-4, 5, (L, H, 1))).astype(np.float32)
        quant.write_kv_fp8(rows_k, rows_v, mgr.allocate_for_prefill(b, L), kc, vc, ks, vs, bs)
    tables = mgr.block_tables([0, 1, 2], 4, -1)
    return rng, (kc, vc, ks, vs), tables, lens, hq, D


def test_fp8_prefill_one_row_chunks_equal_fp8_decode():
    """A one-row chunk (the row at the last position sees every key) is
    decode attention: the 8-bit prefill oracle equals the 8-bit decode
    oracle there."""
    rng, pool, tables, lens, hq, D = _fp8_prefill_case(21)
    q = np.asarray(rng.standard_normal((3, hq, D)), dtype=np.float32).astype(np.float16)
    pre = quant.prefill_attention_fp8(q, "f16", [0, 1, 2, 3], *pool, tables, lens, 0.3)
    dec = quant.decode_attention_fp8(q, "f16", *pool, tables, lens, 0.3)
    np.testing.assert_allclose(pre, dec, rtol=0, atol=1e-13)


def test_fp8_prefill_equals_16bit_prefill_on_the_read_back_values():
    """On a 16-bit pool holding exactly the read-back values (every one is a
    bf16 number here: E4M3 codes times 2^e), the 8-bit prefill oracle equals
    the 16-bit prefill oracle; reading K's scale bytes for V fails."""
    rng, (kc, vc, ks, vs), tables, lens, hq, D = _fp8_prefill_case(22)
    kd, vd = quant.dequantize(kc, ks), quant.dequantize(vc, vs)
    written = np.isfinite(kd)
    as_bf16 = []
    for x in (kd, vd):
        f = np.where(np.isfinite(x), x, 0.0).astype(np.float32)
        assert np.array_equal(f.astype(np.float64), np.where(np.isfinite(x), x, 0.0))
        bits = f.view(np.uint32)
        assert not np.any(bits & 0xFFFF), "read-back values must be bf16 numbers"
        as_bf16.append((bits >> 16).astype(np.uint16))
    assert written.any()
    n = [2, 5, 9]                                      # chunk rows: the last n_b positions
    q = np.asarray(rng.standard_normal((sum(n), hq, D)), dtype=np.float32)
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)   # bf16 queries by truncation (exact values)
    q_start = np.concatenate([[0], np.cumsum(n)])
    got = quant.prefill_attention_fp8(qb, "bf16", q_start, kc, vc, ks, vs, tables, lens, 0.25)
    want = oracle.prefill_attention(qb, q_start, as_bf16[0], as_bf16[1], tables, lens, 0.25, "bf16")
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    bad = quant.prefill_attention_fp8(qb, "bf16", q_start, kc, vc, ks, ks, tables, lens, 0.25)
    assert np.abs(bad - want).max() > 1e-3


def test_non_finite_elements_take_the_nan_code_and_leave_the_scale_to_the_finite_ones():
    """A row holding an infinity and a NaN, worked by hand: the largest
    finite magnitude is 2 = 2^1, so e = 1 - 8 = -7 and x * 2^7 is coded:
    1 -> 128 = 2^7 -> (7 + 7) << 3 = 0x70; 2 -> 2^8 -> 0x78; -2 -> 0xF8;
    0.5 -> 2^6 -> 0x68; 0 -> 0x00; -inf -> 0xFF; +inf and NaN -> 0x7F.
    The scalar and the array encoders agree, and the NaN codes read back as
    NaN."""
    row = np.array([1.0, 2.0, -np.inf, np.nan, 0.5, -2.0, np.inf, 0.0], dtype=np.float32)
    want = [0x70, 0x78, 0xFF, 0x7F, 0x68, 0xF8, 0x7F, 0x00]
    codes, sb = quant.quantize_row(row)
    assert list(codes) == want and sb == 127 - 7
    c2, s2 = quant.quantize_rows(row[None])
    assert list(c2[0]) == want and int(s2[0]) == 127 - 7
    back = quant.dequantize(c2, s2)[0]
    assert np.isnan(back[[2, 3, 6]]).all()
    assert back[[0, 1, 4, 5, 7]].tolist() == [1.0, 2.0, 0.5, -2.0, 0.0]
    # a row with no finite nonzero element takes e = 0
    c3, s3 = quant.quantize_rows(np.array([[np.nan, -np.inf, 0.0, 0.0]], dtype=np.float32))
    assert list(c3[0]) == [0x7F, 0xFF, 0, 0] and int(s3[0]) == 127
