"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks an oracle function against a library routine, an exhaustive
or boundary-focused brute force, a closed form, a hand-worked fixture under
tests/golden/ (with its citation), an invariant, or an exact-arithmetic
derivation.  None of them needs a GPU.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f32_from_bits(u):
    return np.asarray(u, np.uint32).view(np.float32)


def bits(f):
    return np.asarray(f, np.float32).view(np.uint32)


# --------------------------------------------------------------------------
# bf16 rounding: every fp32 input against torch's own conversion
# --------------------------------------------------------------------------

def _bf16_chunk(start, step):
    u = np.arange(step, dtype=np.uint32) + np.uint32(start)
    f = u.view(np.float32)
    ours = oracle.bf16_round(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    diff = np.nonzero(ours != ref)[0]
    # torch keeps NaN payloads; the oracle canonicalises NaN to 0x7FC0.  Nothing else may differ.
    nan_count = int(np.count_nonzero(((u & 0x7F800000) == 0x7F800000) & ((u & 0x7FFFFF) != 0)))
    return (bool(np.all(np.isnan(f[diff]))) and bool(np.all(ours[diff] == 0x7FC0)),
            len(diff) <= nan_count, start)


def test_bf16_round_all_fp32_inputs_match_torch():
    from concurrent.futures import ThreadPoolExecutor
    step = 1 << 26
    with ThreadPoolExecutor(4) as ex:
        for only_nan, count_ok, start in ex.map(lambda s: _bf16_chunk(s, step), range(0, 1 << 32, step)):
            assert only_nan and count_ok, hex(start)
    nan_in = f32_from_bits(np.array([0x7FC00000, 0x7F800001, 0xFFFFFFFF], np.uint32))
    assert np.all(oracle.bf16_round(nan_in) == 0x7FC0)


# --------------------------------------------------------------------------
# E4M3: decode table, encoder against a brute-force nearest search
# --------------------------------------------------------------------------

def e4m3_exact_value(code):
    """OCP E4M3 (FN) value from the bit fields, as an exact fraction."""
    e, m = (code >> 3) & 15, code & 7
    if e == 0:
        return Fraction(m, 512)
    return Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


def test_e4m3_decode_all_finite_codes():
    for c in range(127):
        assert Fraction(oracle.e4m3_value(c)) == e4m3_exact_value(c)
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x38) == 1.0
    # strictly increasing: the encoder relies on it
    vals = [oracle.e4m3_value(c) for c in range(127)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


E4M3_VALUES = np.array([float(e4m3_exact_value(c)) for c in range(127)])


def brute_e4m3(x):
    """Nearest of the 127 finite E4M3 values by exhaustive search, ties to the even code."""
    x = np.asarray(x, np.float64)
    d = np.abs(x[:, None] - E4M3_VALUES[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among the (at most two) nearest codes, prefer the even one
    idx = np.where(cand.sum(axis=1) > 1,
                   np.argmax(cand & (np.arange(127)[None, :] % 2 == 0), axis=1),
                   np.argmax(cand, axis=1))
    return idx.astype(np.uint8)


def neighbourhood(points, ulps=3):
    """fp32 values within +-ulps of each point (points as fp32)."""
    p = bits(np.asarray(points, np.float32)).astype(np.int64)
    offs = np.arange(-ulps, ulps + 1)
    u = (p[:, None] + offs[None, :]).ravel()
    u = u[(u >= 0) & (u < 0x7F800000)]
    return f32_from_bits(u.astype(np.uint32))


def test_e4m3_encoder_vs_bruteforce_at_every_boundary_and_random():
    mids = (E4M3_VALUES[1:] + E4M3_VALUES[:-1]) / 2
    pts = np.concatenate([neighbourhood(E4M3_VALUES), neighbourhood(mids.astype(np.float32), 4),
                          neighbourhood([448.0, 464.0, 480.0, 2.0 ** -10, 2.0 ** -9], 8)])
    g = np.random.Generator(np.random.PCG64(11))
    rand = np.concatenate([
        g.uniform(0, 500, 200000).astype(np.float32),
        f32_from_bits(g.integers(0, 0x7F800000, 200000, dtype=np.uint32)),  # every exponent
        np.exp2(g.uniform(-20, 10, 200000)).astype(np.float32)])
    x = np.concatenate([pts, rand])
    x = x[x < 1e6]  # beyond that brute force distances stop being informative; covered below
    assert np.array_equal(oracle.e4m3_encode(x), brute_e4m3(x))
    big = np.array([448.0, 449.0, 463.99, 464.0, 500.0, 1e6, 3.4e38, np.inf], np.float32)
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(np.array([0.0, -0.0, 2.0 ** -10, 1e-30], np.float32)) == 0)
    assert oracle.e4m3_encode(np.array([2.0 ** -10 * 1.0000001], np.float32))[0] == 1


def test_e4m3_encoder_monotone_over_a_dense_sweep():
    u = np.arange(0, 0x44000000, 97, dtype=np.uint32)  # every 97th pattern up to 512
    c = oracle.e4m3_encode(f32_from_bits(u))
    assert np.all(np.diff(c.astype(np.int32)) >= 0)


# --------------------------------------------------------------------------
# E2M1: the interval table and a brute-force nearest search
# --------------------------------------------------------------------------

E2M1_MAG = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def brute_e2m1(v):
    v = np.asarray(v, np.float32)
    a = np.abs(v.astype(np.float64))
    d = np.abs(a[:, None] - E2M1_MAG[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    mag = np.where(cand.sum(axis=1) > 1, np.argmax(cand & (np.arange(8)[None, :] % 2 == 0), axis=1),
                   np.argmax(cand, axis=1))
    return (mag | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def test_e2m1_interval_table():
    # closed/open intervals of round-to-nearest-even with saturation at 6
    cases = [(0.0, 0), (0.25, 0), (0.2500001, 1), (0.5, 1), (0.7499999, 1), (0.75, 2), (1.25, 2),
             (1.2500001, 3), (1.7499999, 3), (1.75, 4), (2.5, 4), (2.5000002, 5), (3.4999998, 5),
             (3.5, 6), (5.0, 6), (5.0000005, 7), (6.0, 7), (7.0, 7), (1e30, 7), (np.inf, 7)]
    v = np.array([c[0] for c in cases], np.float32)
    want = np.array([c[1] for c in cases], np.uint8)
    assert np.array_equal(oracle.e2m1_encode(v), want)
    assert np.array_equal(oracle.e2m1_encode(-v), want | 8)
    assert oracle.e2m1_encode(np.array([-0.0], np.float32))[0] == 8
    for c in range(16):
        assert oracle.e2m1_value(c) == (-1 if c & 8 else 1) * E2M1_MAG[c & 7]


def test_e2m1_encoder_vs_bruteforce():
    mids = (E2M1_MAG[1:] + E2M1_MAG[:-1]) / 2
    pts = np.concatenate([neighbourhood(E2M1_MAG, 4), neighbourhood(mids.astype(np.float32), 6)])
    allbf16 = f32_from_bits(np.arange(65536, dtype=np.uint32) << 16)
    allbf16 = allbf16[np.isfinite(allbf16)]
    g = np.random.Generator(np.random.PCG64(12))
    rand = np.concatenate([g.uniform(-7, 7, 300000).astype(np.float32),
                           f32_from_bits(g.integers(0, 0x7F800000, 100000, dtype=np.uint32))])
    v = np.concatenate([pts, -pts, allbf16, rand])
    # fp64 distances are exact below 2^50; beyond, every value saturates to 6
    small = np.abs(v) < 2.0 ** 50
    assert np.array_equal(oracle.e2m1_encode(v[small]), brute_e2m1(v[small]))
    assert np.array_equal(oracle.e2m1_encode(v[~small]), np.where(np.signbit(v[~small]), 15, 7))


# --------------------------------------------------------------------------
# swizzled scale layout
# --------------------------------------------------------------------------

def pages_nested_index(r, g, width):
    """The swizzled index as the FastVideo branch compare's quant_probe nests it:
    row tile, then 4-block group, then r%32, then (r/32)%4, then g%4."""
    return (((((r // 128) * (width // 64) + g // 4) * 32 + r % 32) * 4 + (r // 32) % 4) * 4 + g % 4)


def test_scale_offset_hand_worked_cases():
    data = json.load(open(os.path.join(GOLDEN, "hand_worked_blocks.json")))["scale_offsets"]
    for c in data["cases"]:
        assert oracle.scale_offset(c["r"], c["b"], c["k"]) == c["offset"], c


@pytest.mark.parametrize("k", [64, 128, 192, 7168, 19456])
def test_scale_offset_equals_pages_nesting_and_is_a_bijection(k):
    m = 300
    pad = oracle.padded_rows(m)
    offs = oracle.scale_offsets(np.arange(pad), k)
    r = np.arange(pad)[:, None]
    g = np.arange(k // 16)[None, :]
    assert np.array_equal(offs, pages_nested_index(r, g, k))
    for rr, bb in [(0, 0), (pad - 1, k // 16 - 1), (129, 7 % (k // 16))]:
        assert oracle.scale_offset(rr, bb, k) == offs[rr, bb]
    flat = np.sort(offs.ravel())
    assert np.array_equal(flat, np.arange(pad * k // 16))


def test_padded_rows():
    assert [oracle.padded_rows(m) for m in (0, 1, 127, 128, 129, 63240, 300000)] == \
        [0, 128, 128, 128, 256, 63360, 300032]


# --------------------------------------------------------------------------
# the block quantizer: hand-worked blocks, padding, dequantization bound
# --------------------------------------------------------------------------

def _block_values(vals):
    out = []
    for v in vals:
        out.append(-0.0 if v == "-0" else float(v))
    return np.array(out, np.float32)


def test_hand_worked_blocks():
    data = json.load(open(os.path.join(GOLDEN, "hand_worked_blocks.json")))
    for blk in data["blocks"]:
        row = np.zeros(64, np.float32)
        row[:16] = _block_values(blk["values"])
        y = oracle.bf16_round(row).reshape(1, 64)
        codes, sb = oracle.quantize_rows(y, blk["global_amax"])
        assert sb[0, 0] == blk["scale_code"], blk["name"]
        assert codes[0, :8].tobytes().hex() == blk["packed_hex"], blk["name"]
        nib = np.stack([codes[0, :8] & 15, codes[0, :8] >> 4], axis=1).ravel()
        assert list(nib) == blk["codes"], blk["name"]


def test_padding_rows_are_zero():
    p = json.load(open(os.path.join(GOLDEN, "hand_worked_blocks.json")))["padding"]
    g = np.random.Generator(np.random.PCG64(3))
    x = oracle.bf16_round(g.standard_normal((p["m"], p["k"])).astype(np.float32) + 3.0)
    codes, scales = oracle.nvfp4_quantize(x, 10.0)
    assert codes.size == p["codes_bytes"] and scales.size == p["scale_bytes"]
    nz = np.nonzero(scales.ravel())[0]
    assert list(nz) == p["nonzero_scale_offsets"]


def test_dequantization_error_bound():
    g = np.random.Generator(np.random.PCG64(4))
    n, k = 512, 256
    x = g.standard_normal((n, k)).astype(np.float32) * np.exp2(g.integers(-6, 2, (n, 1))).astype(np.float32)
    y = oracle.bf16_round(x)
    yf = oracle.bf16_to_f32(y).astype(np.float64)
    amax = 8.0
    gsf = oracle.global_scale(amax)
    assert gsf == np.float32(2688.0) / np.float32(amax)
    codes, sb = oracle.quantize_rows(y, amax)
    q = np.stack([codes & 15, codes >> 4], axis=-1).reshape(n, k)
    qv = np.vectorize(oracle.e2m1_value)(q)
    dec = np.vectorize(oracle.e4m3_value)(sb)
    dec_e = np.repeat(dec, 16, axis=1)
    s_e = np.repeat(sb, 16, axis=1)
    ok = (s_e != 0) & (s_e != 0x7E)
    deq = qv * dec_e / float(gsf)
    spacing = np.where(np.abs(qv) < 2, 0.5, np.where(np.abs(qv) < 4, 1.0, 2.0))
    # half a code spacing in the block's units, plus the two fp32 roundings (inv and y*inv);
    # |v| <= 6 holds since the scale rounds to nearest with relative error <= 2^-4 ...
    bound = 0.5 * spacing * dec_e / float(gsf) + 2.0 ** -22 * np.abs(yf)
    v_over = np.abs(yf) * float(gsf) / dec_e
    sel = ok & (v_over <= 6.0)
    assert sel.sum() > 0.9 * sel.size
    assert np.all(np.abs(yf - deq)[sel] <= bound[sel])
    # ... which this checks directly: per normal-scale block max|v| <= 6 / (1 - 2^-4)
    blocks_amax = np.abs(yf).reshape(n, k // 16, 16).max(axis=2)
    normal = (sb >= 0x08) & (sb < 0x7E)
    assert np.all((blocks_amax * float(gsf) / dec)[normal] <= 6.0 / (1 - 2.0 ** -4))


# --------------------------------------------------------------------------
# RMSNorm statistic and the adaLN rounding chain
# --------------------------------------------------------------------------

def test_rstd_equal_values_row_is_exact():
    k = 7168
    for c in [1.0, 0.5, 3.0, 0.125]:
        x = oracle.bf16_round(np.full(k, c, np.float32))
        # K * c^2 is exact in fp32 here, so the tree sums exactly and ms = c^2
        want = np.float32(1.0) / np.sqrt(np.float32(c * c) + np.float32(1e-6))
        assert oracle.rms_rstd(x, 1e-6) == want


def test_rstd_zero_row():
    for eps in [1e-6, 1e-5, 0.25]:
        assert oracle.rms_rstd(np.zeros(2048, np.uint16), eps) == \
            np.float32(1.0) / np.sqrt(np.float32(eps))


def test_rstd_close_to_fp64():
    g = np.random.Generator(np.random.PCG64(5))
    for k in [512, 2048, 7168]:
        x = oracle.bf16_round(g.standard_normal(k).astype(np.float32) * 3)
        xf = oracle.bf16_to_f32(x).astype(np.float64)
        ref = 1.0 / np.sqrt(np.mean(xf * xf) + 1e-6)
        assert abs(oracle.rms_rstd(x, 1e-6) / ref - 1) < 1e-6


def test_rstd_tree_order_is_the_documented_one():
    """Rows whose fp32 sum depends on the order of the additions.  Lane L holds
    chunk L (k = 512 gives one chunk per lane).  Lane 0 holds 2^24 (x = 4096);
    two other lanes hold 1.0.  In fp32, 2^24 + 1 rounds back to 2^24 (tie to
    even), while 1 + 1 = 2 and 2^24 + 2 are exact.  The butterfly pairs lanes
    (0,1),(2,3) at distance 1, then (0,2) at distance 2:
      ones on lanes 1 and 3: (2^24+1) -> 2^24, then 2^24 + 1 -> 2^24;
      ones on lanes 2 and 3: 1 + 1 = 2 first, then 2^24 + 2 exactly.
    A sequential left-to-right sum gives 2^24 in both cases."""
    k = 512

    def row(lanes):
        x = np.zeros(k, np.float32)
        x[0] = 4096.0
        for L in lanes:
            x[8 * L] = 1.0
        return oracle.bf16_round(x)

    eps = np.float32(1e-6)
    want13 = np.float32(1.0) / np.sqrt(np.float32(2.0 ** 24 / 512) + eps)
    want23 = np.float32(1.0) / np.sqrt(np.float32((2.0 ** 24 + 2) / 512) + eps)
    assert want13 != want23
    assert oracle.rms_rstd(row([1, 3]), 1e-6) == want13
    assert oracle.rms_rstd(row([2, 3]), 1e-6) == want23


def test_adaln_chain_reduces_to_bf16_of_x_times_rstd():
    """With w = 1, scale = 0 and shift = 0 every later rounding is exact, so
    y = bf16(x * rstd); checked with torch's fp32 multiply and bf16 cast."""
    g = np.random.Generator(np.random.PCG64(6))
    n, k = 8, 2048
    x = oracle.bf16_round(g.standard_normal((n, k)).astype(np.float32))
    w = oracle.bf16_round(np.ones(k, np.float32))
    tab = np.zeros((2, 2, k), np.uint16)
    res = oracle.rms_adaln_rows(x, w, tab, np.zeros(n, np.int32), 1e-6, 4.0, want_y=True)
    xt = torch.from_numpy(oracle.bf16_to_f32(x).copy())
    rt = torch.from_numpy(res["rstd"].copy())[:, None]
    want = (xt * rt).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(res["y"], want)


def test_adaln_chain_single_element_by_hand():
    """One element traced through the chain with torch fp32 ops, each result cast to bf16."""
    k = 512
    g = np.random.Generator(np.random.PCG64(7))
    x = oracle.bf16_round(g.standard_normal((1, k)).astype(np.float32))
    w = oracle.bf16_round((1 + 0.1 * g.standard_normal(k)).astype(np.float32))
    tab = oracle.bf16_round((0.1 * g.standard_normal((3, 2, k))).astype(np.float32))
    res = oracle.rms_adaln_rows(x, w, tab, np.array([2], np.int32), 1e-6, 4.0, want_y=True)
    B = torch.bfloat16

    def t(a):
        return torch.from_numpy(oracle.bf16_to_f32(a).copy())

    n = (t(x[0]) * torch.tensor(res["rstd"][0])).to(B).float()
    nw = (n * t(w)).to(B).float()
    opl = (1.0 + t(tab[2, 1])).to(B).float()
    mm = (nw * opl).to(B).float()
    y = (mm + t(tab[2, 0])).to(B)
    assert np.array_equal(res["y"][0], y.view(torch.int16).numpy().view(np.uint16))


def test_frame_index_out_of_range_zeroes_the_row_and_sets_status():
    k = 512
    g = np.random.Generator(np.random.PCG64(8))
    x = oracle.bf16_round(g.standard_normal((3, k)).astype(np.float32))
    w = oracle.bf16_round(np.ones(k, np.float32))
    tab = oracle.bf16_round((0.1 * g.standard_normal((2, 2, k))).astype(np.float32))
    res = oracle.rms_adaln_rows(x, w, tab, np.array([0, 2, -1], np.int32), 1e-6, 4.0, want_y=True,
                                scales_rows=128)
    assert res["status"] & 1
    assert not res["codes"][1:].any() and not res["scale_bytes"][1:].any() and not res["y"][1:].any()
    assert res["codes"][0].any()
    ok = oracle.rms_adaln_rows(x[:1], w, tab, np.array([1], np.int32), 1e-6, 4.0)
    assert ok["status"] == 0


# --------------------------------------------------------------------------
# fp32 residual stream + RMSNorm with an fp32 weight
# --------------------------------------------------------------------------

def test_rms_sum_f32_equal_values_row_is_exact():
    for k, c in [(512, 1.0), (7168, 0.5), (2048, 3.0), (7168, 1.25)]:
        # every partial sum is a multiple of c^2 below 2^24 ulps: exact in any order
        assert oracle.rms_sum_f32(np.full(k, c, np.float32)) == np.float32(k * c * c)
    assert oracle.rms_rstd_f32(np.zeros(1024, np.float32), 0.25) == np.float32(2.0)


def test_rms_sum_f32_tree_order_is_the_documented_one():
    """k = 512: lane L owns quads L and L + 64, i.e. elements 4L..4L+3 and 256+4L..256+4L+3.
    2^24 + 1 rounds back to 2^24 in fp32 (tie to even) while 2^24 + 2 is exact, so the
    grouping of the additions is visible in the sum."""
    k = 512

    def row(**ones):
        h = np.zeros(k, np.float32)
        h[0] = 4096.0                       # lane 0, quad 0, element 0: 4096^2 = 2^24
        for idx in ones["at"]:
            h[idx] = 1.0
        return h

    big, big2 = np.float32(2.0 ** 24), np.float32(2.0 ** 24 + 2)
    # lanes 1 and 3 (butterfly distance 1 pairs 0+1 and 2+3, so each 1 meets 2^24 alone)
    assert oracle.rms_sum_f32(row(at=[4, 12])) == big
    # lanes 2 and 3: 1 + 1 = 2 at distance 1, then 2^24 + 2 at distance 2
    assert oracle.rms_sum_f32(row(at=[8, 12])) == big2
    # one lane, the same element position in its two quads: one accumulator, so
    # fma(1, 1, 2^24) = 2^24; then the other element's accumulator adds 1 -> 2^24
    assert oracle.rms_sum_f32(row(at=[256, 1])) == big
    # both ones in another element position of lane 0: a1 = 2, then (2^24 + 2) exact
    assert oracle.rms_sum_f32(row(at=[1, 257])) == big2
    # ones in elements 2 and 3 of lane 0: the lane folds (a0 + a1) + (a2 + a3), so 1 + 1
    # first; a left-to-right fold would lose both ones against 2^24
    assert oracle.rms_sum_f32(row(at=[2, 3])) == big2


def test_rms_sum_f32_uses_fused_multiply_add():
    """Element 0 of lane 0 takes 2^-12 (quad 0) then 1 + 2^-12 (quad 64): with a fused
    multiply-add the accumulator is 2^-24 + (1 + 2^-11 + 2^-24) = 1 + 2^-11 + 2^-23
    exactly; rounding the square first would give 1 + 2^-11 (the 2^-24 tie goes to even)."""
    h = np.zeros(512, np.float32)
    h[0], h[256] = 2.0 ** -12, 1.0 + 2.0 ** -12
    assert oracle.rms_sum_f32(h) == np.float32(1.0 + 2.0 ** -11 + 2.0 ** -23)


def test_rms_rstd_f32_close_to_fp64():
    g = np.random.Generator(np.random.PCG64(41))
    for k in [512, 2048, 7168]:
        h = (g.standard_normal(k) * 3).astype(np.float32)
        ref = 1.0 / np.sqrt(np.mean(h.astype(np.float64) ** 2) + 1e-6)
        assert abs(oracle.rms_rstd_f32(h, 1e-6) / ref - 1) < 1e-6


def _residual_case(seed, n=4, k=1024):
    g = np.random.Generator(np.random.PCG64(seed))
    h = (g.standard_normal((n, k)) * 2).astype(np.float32)
    o = oracle.bf16_round(g.standard_normal((n, k)).astype(np.float32))
    bias = oracle.bf16_round((0.5 * g.standard_normal(k)).astype(np.float32))
    scale = (0.3 * g.standard_normal(k)).astype(np.float32)
    gamma = (1 + 0.1 * g.standard_normal(k)).astype(np.float32)
    return h, o, bias, scale, gamma


def _t16(a_u16):
    return torch.from_numpy(a_u16.view(np.int16).copy()).view(torch.bfloat16)


def test_residual_update_matches_torch_eager_ops():
    h, o, bias, scale, gamma = _residual_case(42)
    for b in (bias, None):
        res = oracle.residual_rms_rows(h, o, b, scale, gamma, 1e-6, 8.0)
        t = _t16(o) + _t16(b) if b is not None else _t16(o)      # bf16 tensor add
        want = torch.from_numpy(h) + t.float() * torch.from_numpy(scale)
        assert np.array_equal(res["h"].view(np.uint32), want.numpy().view(np.uint32))


def test_residual_norm_output_matches_torch_eager_ops():
    h, o, bias, scale, gamma = _residual_case(43)
    res = oracle.residual_rms_rows(h, o, bias, scale, gamma, 1e-6, 8.0, want_y=True)
    hn = torch.from_numpy(res["h"])
    rstd = torch.from_numpy(res["rstd"])[:, None]
    want = ((hn * rstd) * torch.from_numpy(gamma)).to(torch.bfloat16)
    assert np.array_equal(res["y"], want.view(torch.int16).numpy().view(np.uint16))
    # rstd is the fixed-tree statistic of the updated rows
    for i in range(h.shape[0]):
        assert res["rstd"][i] == oracle.rms_rstd_f32(res["h"][i], 1e-6)
    # without a residual the stream is only read
    plain = oracle.residual_rms_rows(h, None, None, None, gamma, 1e-6, 8.0)
    assert np.array_equal(plain["h"], h)
    assert plain["rstd"][0] == oracle.rms_rstd_f32(h[0], 1e-6)


def test_residual_norm_hand_worked_block():
    """h' = 1.5 + bf16(0.25 + 0.25) * 1 = 2 everywhere (k = 512), eps = 0: sum = 2048 exactly,
    rstd = 1 / sqrt(4) = 0.5 and y = bf16(1 * gamma).  gamma's first block holds the first
    block of hand_worked_blocks.json, whose codes and scale code follow at gsf = 1."""
    blk = json.load(open(os.path.join(GOLDEN, "hand_worked_blocks.json")))["blocks"][0]
    k = 512
    gamma = np.ones(k, np.float32)
    gamma[:16] = _block_values(blk["values"])
    h = np.full((1, k), 1.5, np.float32)
    o = oracle.bf16_round(np.full((1, k), 0.25, np.float32))
    bias = oracle.bf16_round(np.full(k, 0.25, np.float32))
    res = oracle.residual_rms_rows(h, o, bias, np.ones(k, np.float32), gamma, 0.0, blk["global_amax"])
    assert np.all(res["h"] == 2.0) and res["rstd"][0] == 0.5
    assert res["scale_bytes"][0, 0] == blk["scale_code"]
    assert res["codes"][0, :8].tobytes().hex() == blk["packed_hex"]
    # every other block is all ones: amax 1 -> the E4M3 code of 1/6 = 1.333.. * 2^-3, which
    # rounds to 1.375 * 2^-3 = 0.171875 (exponent field 4, mantissa 3: 0x23), and
    # 1 * (1 / 0.171875) = 5.818.. lies above 5 -> code 7 (6)
    assert np.all(res["scale_bytes"][0, 1:] == 0x23)
    assert np.all(res["codes"][0, 8:] == 0x77)


def _adaln_fold_case(seed, n=6, k=1024, frames=3):
    g = np.random.Generator(np.random.PCG64(seed))
    h = (g.standard_normal((n, k)) * 2).astype(np.float32)
    o = oracle.bf16_round(g.standard_normal((n, k)).astype(np.float32))
    bias = oracle.bf16_round((0.5 * g.standard_normal(k)).astype(np.float32))
    gate = oracle.bf16_round((0.3 * g.standard_normal((frames, k))).astype(np.float32))
    w = oracle.bf16_round((1 + 0.1 * g.standard_normal(k)).astype(np.float32))
    tab = oracle.bf16_round((0.1 * g.standard_normal((frames, 2, k))).astype(np.float32))
    idx = (np.arange(n) * frames // n).astype(np.int32)[::-1].copy()
    return h, o, bias, gate, w, tab, idx


def test_gated_residual_update_is_the_stream_update_with_the_frame_gate():
    h, o, bias, gate, w, tab, idx = _adaln_fold_case(51)
    res = oracle.residual_rms_adaln_rows(h, o, bias, gate, w, tab, idx, 1e-6, 8.0)
    for i, t in enumerate(idx):
        ref = oracle.residual_rms_rows(h[i:i + 1], o[i:i + 1], bias, oracle.bf16_to_f32(gate[t]),
                                       np.ones(h.shape[1], np.float32), 1e-6, 8.0)
        assert np.array_equal(res["h"][i].view(np.uint32), ref["h"][0].view(np.uint32))
        assert res["rstd"][i] == ref["rstd"][0]
    # and against torch's eager ops directly (bf16 tensor add, fp32 product and add)
    gt = _t16(gate[idx]).float()
    want = torch.from_numpy(h) + (_t16(o) + _t16(bias)).float() * gt
    assert np.array_equal(res["h"].view(np.uint32), want.numpy().view(np.uint32))


def test_gated_residual_adaln_chain_matches_torch_eager_ops():
    h, o, bias, gate, w, tab, idx = _adaln_fold_case(52)
    res = oracle.residual_rms_adaln_rows(h, o, None, gate, w, tab, idx, 1e-6, 8.0, want_y=True)
    B = torch.bfloat16
    hn = torch.from_numpy(res["h"])
    rstd = torch.from_numpy(res["rstd"])[:, None]
    shift = _t16(tab[idx, 0]).float()
    scale = _t16(tab[idx, 1]).float()
    n_ = (hn * rstd).to(B).float()
    nw = (n_ * _t16(w).float()).to(B).float()
    opl = (1.0 + scale).to(B).float()
    mm = (nw * opl).to(B).float()
    y = (mm + shift).to(B)
    assert np.array_equal(res["y"], y.view(torch.int16).numpy().view(np.uint16))
    # the gate comes from the first table, shift and scale from the second: exchanging
    # the gate table with the scale rows changes the result
    other = oracle.residual_rms_adaln_rows(h, o, None, np.ascontiguousarray(tab[:, 1]), w,
                                           np.stack([tab[:, 0], gate], axis=1), idx, 1e-6, 8.0, want_y=True)
    assert not np.array_equal(other["y"], res["y"])


def test_gated_residual_out_of_range_frame_leaves_the_row():
    h, o, bias, gate, w, tab, idx = _adaln_fold_case(53)
    idx[[1, 4]] = [3, -1]
    res = oracle.residual_rms_adaln_rows(h, o, bias, gate, w, tab, idx, 1e-6, 8.0, want_y=True)
    assert res["status"] == 1
    for i in (1, 4):
        assert np.array_equal(res["h"][i], h[i])
        assert res["rstd"][i] == oracle.rms_rstd_f32(h[i], 1e-6)
        assert not res["codes"][i].any() and not res["scale_bytes"][i].any() and not res["y"][i].any()
    ok = [0, 2, 3, 5]
    part = oracle.residual_rms_adaln_rows(h[ok], o[ok], bias, gate, w, tab, idx[ok], 1e-6, 8.0, want_y=True)
    assert part["status"] == 0
    for key in ("codes", "scale_bytes", "y", "h", "rstd"):
        assert np.array_equal(part[key], res[key][ok]), key


# --------------------------------------------------------------------------
# fp16 codec, fp16 SiLU table, channels-last RMSNorm + SiLU -> NVFP4
# --------------------------------------------------------------------------

def _f16_chunk(start, step):
    u = np.arange(step, dtype=np.uint32) + np.uint32(start)
    f = u.view(np.float32)
    ours = oracle.f16_round(f)
    ref = torch.from_numpy(f).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    diff = np.nonzero(ours != ref)[0]
    nan_count = int(np.count_nonzero(((u & 0x7F800000) == 0x7F800000) & ((u & 0x7FFFFF) != 0)))
    return (bool(np.all(np.isnan(f[diff]))) and bool(np.all(ours[diff] == 0x7E00)),
            len(diff) <= nan_count, start)


def test_f16_round_all_fp32_inputs_match_torch():
    from concurrent.futures import ThreadPoolExecutor
    step = 1 << 26
    with ThreadPoolExecutor(8) as ex:
        for only_nan, count_ok, start in ex.map(lambda s: _f16_chunk(s, step), range(0, 1 << 32, step)):
            assert only_nan and count_ok, hex(start)


def test_f16_decode_is_numpy_float16():
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((u >> 10) & 0x1F) != 0x1F
    # every finite pattern decodes and re-encodes to itself
    assert np.array_equal(oracle.f16_round(oracle.f16_to_f32(u[finite])), u[finite])


def test_silu_table_f16_equals_exact_decimal_derivation():
    assert np.array_equal(oracle.silu_table_f16(), oracle.silu_exact_f16())


def test_silu_table_f16_special_values():
    t = oracle.silu_table_f16()
    assert t[0x0000] == 0x0000 and t[0x8000] == 0x8000 and t[0x7C00] == 0x7C00 and t[0xFC00] == 0x8000
    # silu(1) = 0.7310585..: fp16 0x39D9 = 0.73095703125 (next 0x39DA = 0.7314453125);
    # silu(-20) = -4.12e-8 rounds to the smallest subnormal -2^-24 (0x8001), silu(-25) to -0
    assert t[0x3C00] == 0x39D9
    assert t[0xCD00] == 0x8001 and t[0xCE40] == 0x8000


def _rms_silu_case(seed, n=6, c=192):
    g = np.random.Generator(np.random.PCG64(seed))
    x = oracle.f16_round((g.standard_normal((n, c)) * 2).astype(np.float32))
    gamma = oracle.f16_round((1 + 0.3 * g.standard_normal(c)).astype(np.float32))
    return x, gamma


def test_rms_f16row_statistic():
    for c in (96, 192, 384):
        for v in (1.0, 0.5, 3.0):
            x = oracle.f16_round(np.full(c, v, np.float32))
            assert oracle.rms_rstd_f16row(x, 1e-6) == np.float32(1.0) / np.sqrt(np.float32(v * v) + np.float32(1e-6))
        g = np.random.Generator(np.random.PCG64(c))
        x = oracle.f16_round((g.standard_normal(c) * 3).astype(np.float32))
        xf = oracle.f16_to_f32(x).astype(np.float64)
        ref = 1.0 / np.sqrt(np.mean(xf * xf) + 1e-6)
        assert abs(oracle.rms_rstd_f16row(x, 1e-6) / ref - 1) < 1e-6


def test_rms_f16row_tree_over_padded_slots():
    """c = 96: 12 chunks in 16 slots.  Chunk 0 holds 4096 (4096^2 = 2^24) and two other
    chunks 1.0 each: 2^24 + 1 rounds back to 2^24 in fp32, 1 + 1 = 2 and 2^24 + 2 are exact,
    so the pairing of the butterfly shows in the sum (as in the bf16 row statistic)."""
    c = 96

    def total(ones, first=0):
        x = np.zeros(c, np.float32)
        x[0] = 4096.0
        for ch in ones:
            x[8 * ch + first] = 1.0
        return oracle.rms_sum_f16row(oracle.f16_round(x))

    big, big2 = np.float32(2.0 ** 24), np.float32(2.0 ** 24 + 2)
    assert total([1, 3]) == big and total([2, 3]) == big2
    # chunks 8 and 9 meet chunk 0 only at distance 8, after pairing with each other
    assert total([8, 9]) == big2
    # within a chunk: elements 2 and 3 pair before meeting element 0 ((q0+q1)+(q2+q3))
    x = np.zeros(c, np.float32)
    x[0], x[2], x[3] = 4096.0, 1.0, 1.0
    assert oracle.rms_sum_f16row(oracle.f16_round(x)) == big2
    x[3], x[1] = 0.0, 1.0
    assert oracle.rms_sum_f16row(oracle.f16_round(x)) == big     # (2^24 + 1) + 1, both lost
    # the padding slots add +0: the c = 96 row equals the same chunks in a c = 128 row
    g = np.random.Generator(np.random.PCG64(5))
    v = oracle.f16_round(g.standard_normal(96).astype(np.float32) * 5)
    assert oracle.rms_sum_f16row(v) == oracle.rms_sum_f16row(np.concatenate([v, np.zeros(32, np.uint16)]))


def test_rms_silu_chain_matches_torch_eager_ops():
    # 2048 rows: enough elements (~390k) that some fp32 products x * rstd round onto an fp16
    # midpoint, where one fused rounding to fp16 would differ from the two of the chain
    x, gamma = _rms_silu_case(61, n=2048)
    res = oracle.rms_silu_rows(x, gamma, 1e-6, 4.0, want_y=True)
    H = torch.float16
    xt = torch.from_numpy(x.view(np.int16).copy()).view(H)
    gt = torch.from_numpy(gamma.view(np.int16).copy()).view(H)
    rstd = torch.from_numpy(res["rstd"])[:, None]
    nn = (xt.float() * rstd).to(H)
    a = nn * gt                                       # fp16 tensor multiply
    a16 = a.view(torch.int16).numpy().view(np.uint16)
    want = oracle.silu_table_f16()[a16]
    assert np.array_equal(res["y"], want)
    # the table entries used are the correctly rounded silu of a (torch's own silu in fp64)
    ref = torch.nn.functional.silu(a.double()).to(H).view(torch.int16).numpy().view(np.uint16)
    assert np.mean(ref == want) > 0.999


def test_rms_silu_hand_worked_block():
    """x = 2 in every channel, eps = 0: sum = 4c exactly, rstd = 1/2, nn = 1, a = gamma, and
    y = silu(gamma).  gamma's first block holds 96, 80, ..., 12 (silu rounds each back to
    itself in fp16) and four zeros; global_amax = 43008 gives gsf = 1/16, block amax 96 ->
    scale 96/6/16 = 1.0 (0x38), inverse 1/16: v = 6, 5, 4, 3.5, 3, 2.5, 2, 1.75, 1.5, 1.25,
    1, 0.75 -> codes 7, 6, 6, 6, 5, 4, 4, 4, 3, 2, 2, 2 (ties to even), then 0, 0, 0, 0."""
    c = 192
    vals = [96, 80, 64, 56, 48, 40, 32, 28, 24, 20, 16, 12, 0, 0, 0, 0]
    gamma = np.full(c, 16.0, np.float32)
    gamma[:16] = vals
    x = oracle.f16_round(np.full((1, c), 2.0, np.float32))
    res = oracle.rms_silu_rows(x, oracle.f16_round(gamma), 0.0, 43008.0, want_y=True)
    assert res["rstd"][0] == 0.5
    assert np.array_equal(oracle.f16_to_f32(res["y"][0, :16]), np.array(vals, np.float32))
    nib = [7, 6, 6, 6, 5, 4, 4, 4, 3, 2, 2, 2, 0, 0, 0, 0]
    want = bytes(nib[2 * i] | (nib[2 * i + 1] << 4) for i in range(8))
    assert res["codes"][0, :8].tobytes() == want and res["scale_bytes"][0, 0] == 0x38
    # the other blocks: all 16 -> amax 16, scale 16/6/16 = 1/6 -> 0x23 (0.171875), v = 5.818 -> 7
    assert np.all(res["scale_bytes"][0, 1:] == 0x23) and np.all(res["codes"][0, 8:] == 0x77)


# --------------------------------------------------------------------------
# LayerNorm + adaLN -> per-tensor FP8 E4M3
# --------------------------------------------------------------------------

def _torch_fp8(v_f32):
    t = torch.from_numpy(np.ascontiguousarray(v_f32, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_signed_encoder_matches_torch_saturating_conversion():
    g = np.random.Generator(np.random.PCG64(71))
    vals = [g.standard_normal(200000).astype(np.float32) * s for s in (1e-3, 0.05, 1.0, 30.0, 300.0, 1e4)]
    # every E4M3 value, its midpoints with the neighbours and a few ulps around them, both signs
    grid = np.array([oracle.e4m3_value(c) for c in range(127)], np.float64)
    mids = (grid[:-1] + grid[1:]) / 2
    pts = np.concatenate([grid, mids, [448.0, 464.0, 480.0, 1e30, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11]])
    pts32 = pts.astype(np.float32)
    u = pts32.view(np.uint32)
    near = np.concatenate([(u.astype(np.int64) + d).astype(np.uint32).view(np.float32) for d in range(-3, 4)])
    near = near[np.isfinite(near)]          # stepping down from +0 wraps to NaN patterns
    allv = np.concatenate(vals + [near, -near, np.array([0.0, -0.0], np.float32)])
    assert np.array_equal(oracle.e4m3_encode_signed(allv), _torch_fp8(allv))
    assert oracle.e4m3_encode_signed(np.array([-0.0], np.float32))[0] == 0x80
    assert list(oracle.e4m3_encode_signed(np.array([1e30, -1e30], np.float32))) == [0x7E, 0xFE]


def test_tree_sum_f32_order():
    """The SUM tree: lane 0 holds 2^24 (chunk 0, element 0); 2^24 + 1 rounds back to 2^24
    (tie to even), 1 + 1 = 2 and 2^24 + 2 are exact (k = 512: one chunk per lane)."""
    def total(ones):
        v = np.zeros(512, np.float32)
        v[0] = 2.0 ** 24
        for i in ones:
            v[i] = 1.0
        return oracle.tree_sum_f32(v)
    big, big2 = np.float32(2.0 ** 24), np.float32(2.0 ** 24 + 2)
    assert total([8, 24]) == big            # lanes 1 and 3: each one meets 2^24 alone
    assert total([16, 24]) == big2          # lanes 2 and 3 pair first
    assert total([2, 3]) == big2            # elements 2, 3 of lane 0 pair within the lane
    assert total([1, 2]) == big             # (2^24 + 1) loses it, then (1 + 0) is added to 2^24
    v = np.zeros(1024, np.float32)
    v[0], v[512] = 2.0 ** -12, 1.0 + 2.0 ** -12     # lane 0, element 0, chunks 0 and 64
    assert oracle.tree_sum_f32(v, squares=True) == np.float32(1.0 + 2.0 ** -11 + 2.0 ** -23)   # fma


def _ln_case(seed, n=5, k=1024):
    g = np.random.Generator(np.random.PCG64(seed))
    x = oracle.f16_round((g.standard_normal((n, k)) * 3 + 0.5).astype(np.float32))
    scale = (0.2 * g.standard_normal(k)).astype(np.float32)
    shift = (0.2 * g.standard_normal(k)).astype(np.float32)
    return x, scale, shift


def test_ln_statistics():
    x, scale, shift = _ln_case(72)
    res = oracle.ln_adaln_fp8_rows(x, scale, shift, 1e-6, 0.05)
    xf = oracle.f16_to_f32(x).astype(np.float64)
    mean = xf.mean(axis=1)
    var = xf.var(axis=1)
    assert np.all(np.abs(res["mean"] - mean) <= 1e-6 * np.abs(xf).max())
    assert np.all(np.abs(res["rstd"] / (1.0 / np.sqrt(var + 1e-6)) - 1) < 1e-6)
    # a constant row: mean exact, var 0, rstd = 1 / sqrt(eps)
    c = oracle.f16_round(np.full((1, 512), 1.5, np.float32))
    r = oracle.ln_adaln_fp8_rows(c, np.zeros(512, np.float32), np.zeros(512, np.float32), 0.25, 1.0)
    assert r["mean"][0] == 1.5 and r["rstd"][0] == 2.0 and not np.any(r["codes"] & 0x7F)


def test_ln_statistics_follow_the_documented_trees():
    """Hand-derived rows (k = 512, one chunk per lane; k = 1024 for the variance) whose mean
    and variance tell the documented trees from other orders.  Mean: 2048 in lane 0 with two
    2^-13 (half an fp32 ulp of 2048: alone each is lost, tie to even) where the tree pairs them
    first (elements 2 and 3 of lane 0; lanes 2 and 3) or not (lanes 1 and 3; elements 1 and 2).
    Variance: 64 and -64 in lane 0 (chunks 0 and 64) and +-2^-6 likewise in lanes 2 and 3, so
    the mean is exactly 0; the squares' tree gives 8192 + 2^-10, a left-to-right sum 8192."""
    zeros = np.zeros(1024, np.float32)

    def mean_of(smalls):
        v = np.zeros((1, 512), np.float32)
        v[0, 0] = 2048.0
        v[0, smalls] = 2.0 ** -13
        r = oracle.ln_adaln_fp8_rows(oracle.f16_round(v), zeros[:512], zeros[:512], 0.0, 1.0)
        return r["mean"][0]
    lost, kept = np.float32(2048.0 / 512), np.float32((2048.0 + 2.0 ** -12) / 512)
    assert mean_of([2, 3]) == kept and mean_of([16, 24]) == kept
    assert mean_of([1, 2]) == lost and mean_of([8, 24]) == lost
    v = np.zeros((1, 1024), np.float32)
    v[0, 0], v[0, 512] = 64.0, -64.0
    v[0, 16], v[0, 528], v[0, 24], v[0, 536] = 2.0 ** -6, -(2.0 ** -6), 2.0 ** -6, -(2.0 ** -6)
    r = oracle.ln_adaln_fp8_rows(oracle.f16_round(v), zeros, zeros, 0.0, 1.0)
    assert r["mean"][0] == 0.0
    assert r["rstd"][0] == np.float32(1.0) / np.sqrt(np.float32(8.0 + 2.0 ** -20))


def test_ln_adaln_chain_and_codes_match_torch_eager_ops():
    x, scale, shift = _ln_case(73)
    act = 0.03
    res = oracle.ln_adaln_fp8_rows(x, scale, shift, 1e-6, act)
    xt = torch.from_numpy(oracle.f16_to_f32(x))
    d = xt - torch.from_numpy(res["mean"])[:, None]
    y = ((d * torch.from_numpy(res["rstd"])[:, None]) * (1.0 + torch.from_numpy(scale))) + torch.from_numpy(shift)
    assert np.array_equal(res["y"].view(np.uint32), y.numpy().view(np.uint32))
    inv = np.float32(1.0) / np.float32(act)
    assert oracle.fp8_inverse_scale(act) == inv
    assert np.array_equal(res["codes"], _torch_fp8((y * torch.tensor(inv)).numpy()))


def test_ln_adaln_hand_worked_row():
    """x = +1, -1 alternating: mean 0, var 1; eps = 0 gives rstd 1, y = +-1 with no
    modulation, and act_scale 1 codes them 0x38 (1.0) and 0xB8 (-1.0)."""
    x = oracle.f16_round(np.tile([1.0, -1.0], 256).reshape(1, 512).astype(np.float32))
    z = np.zeros(512, np.float32)
    res = oracle.ln_adaln_fp8_rows(x, z, z, 0.0, 1.0)
    assert res["mean"][0] == 0.0 and res["rstd"][0] == 1.0
    assert list(res["codes"][0, :4]) == [0x38, 0xB8, 0x38, 0xB8]
    # shift 2, scale 1: y = +-1 * 2 + 2 = 4 or 0 -> 0x48 (4.0) and 0x00
    res = oracle.ln_adaln_fp8_rows(x, np.ones(512, np.float32), np.full(512, 2.0, np.float32), 0.0, 1.0)
    assert list(res["codes"][0, :2]) == [0x48, 0x00]


# --------------------------------------------------------------------------
# SiLU table and the SwiGLU producer
# --------------------------------------------------------------------------

def test_silu_table_equals_exact_decimal_derivation():
    assert np.array_equal(oracle.silu_table(), oracle.silu_exact())


def test_silu_table_special_values():
    t = oracle.silu_table()
    assert t[0x0000] == 0x0000 and t[0x8000] == 0x8000
    assert t[0x7F80] == 0x7F80 and t[0xFF80] == 0x8000 and t[0x7FC1] == 0x7FC0
    # silu(1) = 0.7310585..., bf16 0x3F3B = 0.73046875; silu(-1) = -0.268941..., 0xBE8A = -0.26953125
    assert t[0x3F80] == 0x3F3B and t[0xBF80] == 0xBE8A


def test_swiglu_with_unit_up_returns_the_table():
    gate = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((gate >> 7) & 0xFF) != 0xFF
    gate = gate[finite][: (finite.sum() // 64) * 64].reshape(-1, 64)
    up = np.full(gate.shape, 0x3F80, np.uint16)
    res = oracle.swiglu_rows(up, gate, 4.0, want_y=True)
    assert np.array_equal(res["y"], oracle.silu_table()[gate])


def test_swiglu_product_rounding_vs_torch():
    g = np.random.Generator(np.random.PCG64(9))
    up = oracle.bf16_round(g.standard_normal((4, 256)).astype(np.float32))
    gate = oracle.bf16_round(g.standard_normal((4, 256)).astype(np.float32))
    res = oracle.swiglu_rows(up, gate, 4.0, want_y=True)
    s = torch.from_numpy(oracle.bf16_to_f32(oracle.silu_table()[gate]).copy())
    u = torch.from_numpy(oracle.bf16_to_f32(up).copy())
    want = (s * u).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(res["y"], want)


# --------------------------------------------------------------------------
# SwiGLU of a packed projection with a bias (value-first and paired columns)
# --------------------------------------------------------------------------

def _f32_list(vals):
    return np.array([-0.0 if v == "-0" else float(v) for v in vals], np.float32)


def _pack_columns(value, gate, interleaved):
    """[n, f] value and gate halves -> one [n, 2f] projection in the given column order."""
    n, f = value.shape
    out = np.empty((n, 2 * f), value.dtype)
    if interleaved:
        out[:, 0::2], out[:, 1::2] = value, gate
    else:
        out[:, :f], out[:, f:] = value, gate
    return out


def _torch_bf16_add(a_u16, b_u16):
    """bf16 + bf16 by torch on the CPU (fp32 sum, nearest-even to bf16)."""
    a = torch.from_numpy(a_u16.view(np.int16).copy()).view(torch.bfloat16)
    b = torch.from_numpy(b_u16.view(np.int16).copy()).view(torch.bfloat16)
    return (a + b).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("interleaved", [False, True])
def test_swiglu_packed_hand_worked_blocks(interleaved):
    d = json.load(open(os.path.join(GOLDEN, "swiglu_packed_blocks.json")))
    f, cols = d["f"], d["columns"]
    half = {}
    for key in ("value", "value_bias", "gate", "gate_bias"):
        row = np.zeros((1, f), np.float32)
        row[0, :cols] = _f32_list(d[key])
        half[key] = oracle.bf16_round(row)
    proj = _pack_columns(half["value"], half["gate"], interleaved)
    bias = _pack_columns(half["value_bias"], half["gate_bias"], interleaved).reshape(-1)
    res = oracle.swiglu_packed_rows(proj, bias, interleaved, d["global_amax"], want_y=True)
    want = bytes.fromhex(d["codes_hex"]) + bytes(f // 2 - len(d["codes_hex"]) // 2)
    assert res["codes"][0].tobytes() == want
    assert list(res["scale_bytes"][0]) == d["scale_codes"]


def _random_projection(seed, n, f):
    g = np.random.Generator(np.random.PCG64(seed))
    proj = oracle.bf16_round(g.standard_normal((n, 2 * f)).astype(np.float32))
    # bias values of the same scale, so that most sums need rounding and some tie
    bias = oracle.bf16_round((0.5 * g.standard_normal(2 * f)).astype(np.float32))
    return proj, bias


@pytest.mark.parametrize("interleaved", [False, True])
def test_swiglu_packed_without_bias_is_the_two_pointer_form(interleaved):
    n, f = 6, 192
    proj_vf, _ = _random_projection(31, n, f)
    value, gate = proj_vf[:, :f], proj_vf[:, f:]
    proj = _pack_columns(value, gate, interleaved)
    got = oracle.swiglu_packed_rows(proj, None, interleaved, 7.5, want_y=True, scales_rows=128)
    ref = oracle.swiglu_rows(value, gate, 7.5, want_y=True, scales_rows=128)
    for key in ("codes", "scale_bytes", "y", "scales"):
        assert np.array_equal(got[key], ref[key]), key


@pytest.mark.parametrize("interleaved", [False, True])
def test_swiglu_packed_bias_is_a_bf16_add_before_silu(interleaved):
    n, f = 6, 256
    proj_vf, bias_vf = _random_projection(32, n, f)
    value, gate = proj_vf[:, :f], proj_vf[:, f:]
    bv, bg = bias_vf[:f], bias_vf[f:]
    proj = _pack_columns(value, gate, interleaved)
    bias = _pack_columns(bv[None], bg[None], interleaved).reshape(-1)
    got = oracle.swiglu_packed_rows(proj, bias, interleaved, 9.0, want_y=True)
    ref = oracle.swiglu_rows(_torch_bf16_add(value, np.broadcast_to(bv, value.shape)),
                             _torch_bf16_add(gate, np.broadcast_to(bg, gate.shape)), 9.0, want_y=True)
    for key in ("codes", "scale_bytes", "y"):
        assert np.array_equal(got[key], ref[key]), key
    # the bias changes the result (a dropped bias would pass the test above only by accident)
    plain = oracle.swiglu_packed_rows(proj, None, interleaved, 9.0, want_y=True)
    assert not np.array_equal(plain["y"], got["y"])


@pytest.mark.parametrize("interleaved", [False, True])
def test_swiglu_packed_negative_zero_bias_is_no_bias(interleaved):
    n, f = 4, 128
    proj, _ = _random_projection(33, n, f)
    proj[0, :8] = 0x0000          # x + (-0) = x also for both zeros
    proj[0, 8:16] = 0x8000
    bias = np.full(2 * f, 0x8000, np.uint16)
    got = oracle.swiglu_packed_rows(proj, bias, interleaved, 5.0, want_y=True)
    ref = oracle.swiglu_packed_rows(proj, None, interleaved, 5.0, want_y=True)
    for key in ("codes", "scale_bytes", "y"):
        assert np.array_equal(got[key], ref[key]), key


# --------------------------------------------------------------------------
# whole-tensor quantize equals per-row quantize placed by the layout
# --------------------------------------------------------------------------

def test_tensor_quantize_matches_rows_and_layout():
    g = np.random.Generator(np.random.PCG64(10))
    m, k = 261, 192
    x = oracle.bf16_round(g.standard_normal((m, k)).astype(np.float32))
    codes, scales = oracle.nvfp4_quantize(x, 5.0)
    c2, sb = oracle.quantize_rows(x, 5.0)
    assert np.array_equal(codes, c2)
    offs = oracle.scale_offsets(np.arange(m), k)
    assert np.array_equal(scales.ravel()[offs], sb)
    mask = np.ones(scales.size, bool)
    mask[offs.ravel()] = False
    assert not scales.ravel()[mask].any()


# --------------------------------------------------------------------------
# per-call (dynamic) global amax
# --------------------------------------------------------------------------

def test_dynamic_global_scale_special_cases():
    f32 = np.float32
    fmax = float(np.finfo(np.float32).max)
    # positive amax with a finite quotient: the static rule 2688 / amax (IEEE fp32)
    for a in [2688.0, 1.0, 63.25, 1.0e-35, fmax]:
        want = float(f32(2688.0) / f32(a))
        assert oracle.dynamic_global_scale(a) == want
    # zero, negative zero, a quotient that overflows, non-finite amax: scale 0
    assert np.isinf(f32(2688.0) / f32(1e-38))
    for a in [0.0, -0.0, 1e-38, float(2.0 ** -133), float("inf"), float("nan")]:
        assert oracle.dynamic_global_scale(a) == 0.0


def test_max_abs_vs_numpy():
    g = np.random.Generator(np.random.PCG64(77))
    x = oracle.bf16_round((g.standard_normal(5000) * 3).astype(np.float32))
    x[17] = 0x8000                       # -0
    x[18] = 0x0001                       # smallest positive subnormal
    x[19] = 0xC2F7                       # -123.5
    want = float(np.abs(oracle.bf16_to_f32(x)).max())
    assert oracle.max_abs(x) == want == 123.5
    assert oracle.max_abs(np.array([0x8000, 0x0000], np.uint16)) == 0.0


def test_dynamic_quantize_is_static_quantize_at_the_measured_amax():
    g = np.random.Generator(np.random.PCG64(78))
    x = oracle.bf16_round((g.standard_normal((300, 192)) * np.linspace(0.1, 5, 192)).astype(np.float32))
    codes, scales, amax = oracle.nvfp4_quantize_dynamic(x)
    assert amax == float(np.abs(oracle.bf16_to_f32(x)).max())
    c2, s2 = oracle.nvfp4_quantize(x, amax)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)


def test_dynamic_quantize_block_holding_the_max_gets_the_top_scale():
    # gsf * (amax * fp32(1/6)) rounds to 448 for the block holding the global maximum, so
    # its scale code is 0x7E and the maximal element encodes as magnitude 6 (code 7)
    g = np.random.Generator(np.random.PCG64(79))
    for trial in range(20):
        x = oracle.bf16_round(g.standard_normal((8, 64)).astype(np.float32) * np.float32(10.0 ** g.uniform(-30, 30)))
        codes, scales, amax = oracle.nvfp4_quantize_dynamic(x)
        xf = oracle.bf16_to_f32(x)
        r, c = np.unravel_index(int(np.argmax(np.abs(xf))), xf.shape)
        b = c // 16
        assert scales.reshape(-1)[oracle.scale_offset(r, b, 64)] == 0x7E
        nib = (codes[r, c // 2] >> (4 * (c % 2))) & 0xF
        assert nib & 0x7 == 7 and (nib >> 3) == (1 if xf[r, c] < 0 else 0)


@pytest.mark.parametrize("pattern", [0x0000, 0x8000, 0x0001, 0x8005])
def test_dynamic_quantize_all_zero_or_subnormal_tensor(pattern):
    # an all-(+/-)zero tensor, and one whose amax is so small that 2688 / amax overflows:
    # scale 0, so every code is the sign of the value and every scale byte is 0
    x = np.full((130, 64), pattern, np.uint16)
    x[::3, ::5] = 0x0000
    codes, scales, amax = oracle.nvfp4_quantize_dynamic(x)
    assert oracle.dynamic_global_scale(amax) == 0.0
    sign = (x >> 15).astype(np.uint8) * 8
    assert np.array_equal(codes, sign[:, 0::2] | (sign[:, 1::2] << 4))
    assert not scales.any()


def test_dynamic_swiglu_packed_is_static_at_its_own_amax():
    proj, bias = _random_projection(34, 5, 128)
    for interleaved in (False, True):
        dyn = oracle.swiglu_packed_dynamic(proj, bias, interleaved, want_y=True, scales_rows=128)
        y = oracle.swiglu_packed_rows(proj, bias, interleaved, 1.0, want_y=True)["y"]
        assert dyn["amax"] == float(np.abs(oracle.bf16_to_f32(y)).max())
        ref = oracle.swiglu_packed_rows(proj, bias, interleaved, dyn["amax"], want_y=True, scales_rows=128)
        for key in ("codes", "scales", "y"):
            assert np.array_equal(dyn[key], ref[key]), key


def test_dynamic_residual_rms_is_static_at_its_own_amax():
    h, o, bias, scale, gamma = _residual_case(44, n=5, k=512)
    dyn = oracle.residual_rms_dynamic(h, o, bias, scale, gamma, 1e-6, want_y=True, scales_rows=128)
    y = oracle.residual_rms_rows(h, o, bias, scale, gamma, 1e-6, 1.0, want_y=True)["y"]
    assert dyn["amax"] == float(np.abs(oracle.bf16_to_f32(y)).max())
    ref = oracle.residual_rms_rows(h, o, bias, scale, gamma, 1e-6, dyn["amax"], want_y=True, scales_rows=128)
    for key in ("codes", "scales", "y", "h", "rstd"):
        assert np.array_equal(dyn[key], ref[key]), key


def test_dynamic_gated_residual_adaln_is_static_at_its_own_amax():
    h, o, bias, gate, w, tab, idx = _adaln_fold_case(54, n=5, k=512)
    dyn = oracle.residual_rms_adaln_dynamic(h, o, bias, gate, w, tab, idx, 1e-6, want_y=True, scales_rows=128)
    ref = oracle.residual_rms_adaln_rows(h, o, bias, gate, w, tab, idx, 1e-6, dyn["amax"], want_y=True,
                                         scales_rows=128)
    assert dyn["amax"] == float(np.abs(oracle.bf16_to_f32(ref["y"])).max())
    for key in ("codes", "scales", "y", "h", "rstd"):
        assert np.array_equal(dyn[key], ref[key]), key


def test_dynamic_rms_silu_is_static_at_its_own_amax():
    x, gamma = _rms_silu_case(62, n=9)
    dyn = oracle.rms_silu_dynamic(x, gamma, 1e-6, want_y=True)
    ref = oracle.rms_silu_rows(x, gamma, 1e-6, dyn["amax"], want_y=True)
    assert dyn["amax"] == float(np.abs(oracle.f16_to_f32(ref["y"])).max())
    for key in ("codes", "scale_bytes", "y", "rstd"):
        assert np.array_equal(dyn[key], ref[key]), key


def test_dynamic_ln_adaln_fp8():
    x, scale, shift = _ln_case(74, n=7)
    dyn = oracle.ln_adaln_fp8_dynamic(x, scale, shift, 1e-6)
    assert dyn["amax"] == float(np.abs(dyn["y"]).max())
    assert dyn["act_scale"] == np.float32(dyn["amax"]) / np.float32(448.0)
    ref = oracle.ln_adaln_fp8_rows(x, scale, shift, 1e-6, dyn["act_scale"])
    assert np.array_equal(ref["codes"], dyn["codes"])
    # the element holding the maximum saturates to +-448
    i = np.unravel_index(np.argmax(np.abs(dyn["y"])), dyn["y"].shape)
    assert dyn["codes"][i] & 0x7F == 0x7E
    # an all-zero tensor: scale 0, inverse 0, every code a zero (mean 0, y = shift = 0)
    z = np.zeros(512, np.float32)
    zero = oracle.ln_adaln_fp8_dynamic(np.zeros((2, 512), np.uint16), z, z, 1e-6)
    assert zero["act_scale"] == 0.0 and not np.any(zero["codes"] & 0x7F)


def test_dynamic_rms_adaln_and_swiglu_are_static_at_their_own_amax():
    g = np.random.Generator(np.random.PCG64(80))
    m, k, t = 70, 1024, 3
    x = oracle.bf16_round(g.standard_normal((m, k)).astype(np.float32))
    w = oracle.bf16_round((1 + 0.1 * g.standard_normal(k)).astype(np.float32))
    tab = oracle.bf16_round((0.1 * g.standard_normal((t, 2, k))).astype(np.float32))
    idx = (np.arange(m) * t // m).astype(np.int32)
    dyn = oracle.rms_adaln_dynamic(x, w, tab, idx, 1e-6, want_y=True, scales_rows=oracle.padded_rows(m))
    assert dyn["amax"] == float(np.abs(oracle.bf16_to_f32(dyn["y"])).max())
    st = oracle.rms_adaln_rows(x, w, tab, idx, 1e-6, dyn["amax"], scales_rows=oracle.padded_rows(m))
    assert np.array_equal(dyn["codes"], st["codes"]) and np.array_equal(dyn["scales"], st["scales"])
    assert (dyn["scale_bytes"] == 0x7E).any()

    proj = oracle.bf16_round(g.standard_normal((m, 2 * 256)).astype(np.float32))
    dyn = oracle.swiglu_dynamic(proj[:, :256], proj[:, 256:], want_y=True, scales_rows=oracle.padded_rows(m))
    assert dyn["amax"] == float(np.abs(oracle.bf16_to_f32(dyn["y"])).max())
    st = oracle.swiglu_rows(proj[:, :256], proj[:, 256:], dyn["amax"], scales_rows=oracle.padded_rows(m))
    assert np.array_equal(dyn["codes"], st["codes"]) and np.array_equal(dyn["scales"], st["scales"])
    assert (dyn["scale_bytes"] == 0x7E).any()
