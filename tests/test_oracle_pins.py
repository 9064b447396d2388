"""Pins of the CPU oracle against things other than itself.

Every check here compares the oracle with a value the pages print, a closed
form, exact rational arithmetic (``fractions.Fraction``), an independent
numpy formulation or brute force on tiny inputs.  They are chosen so that a
plausible mistake anywhere in the oracle (a reversed bit order, a dropped -1
offset, a reciprocal instead of a division, round-half-away instead of
half-even, a swapped scale byte, a transposed operand or a wrong group index)
fails at least one of them.  CPU only.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- helpers
def _f32_nearest(value: Fraction) -> np.float32:
    """The binary32 nearest to an exact rational, ties to even (from the
    definition of IEEE round-to-nearest, independent of any FPU division)."""
    if value == 0:
        return np.float32(0.0)
    guess = np.float32(float(value))
    cands = [np.nextafter(guess, np.float32(-np.inf)), guess, np.nextafter(guess, np.float32(np.inf))]
    best = None
    for c in cands:
        dist = abs(Fraction(float(c)) - value)
        key = (dist, int(np.array(c, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def _digit_decode(byte: int):
    """Weight values of a code byte via its base-4 digits (least significant
    digit = weight 4b+0), an independent route to the same table."""
    digits = np.base_repr(byte, base=4).zfill(4)[::-1]
    return [int(d) - 1 for d in digits]


def _block(codes32, scale_f16):
    """One raw 34-byte block: fp16 scale bytes (little-endian) then codes."""
    sb = np.array([scale_f16], dtype=np.float16).view(np.uint8)
    return np.concatenate([sb, np.asarray(codes32, dtype=np.uint8)])


def _dense_weights(raw, n, k):
    """(c-1)*ws as float64 [n][k] by numpy slicing of the raw blocks."""
    g = k // 128
    blocks = raw[:, : g * 34].reshape(n, g, 34)
    ws = blocks[:, :, :2].copy().view(np.float16).astype(np.float64).reshape(n, g)
    codes = blocks[:, :, 2:].astype(np.int64)                       # [n][g][32]
    fields = np.stack([(codes >> (2 * s)) & 3 for s in range(4)], axis=-1)  # [n][g][32][4]
    vals = (fields - 1).reshape(n, g, 128).astype(np.float64)
    return (vals * ws[:, :, None]).reshape(n, k), (fields - 1).reshape(n, g * 128)


# ---------------------------------------------------------------- decode
def test_code_table_fixture_matches_add_xor_mapping():
    """The fixture's code table agrees with the pages' add/XOR byte trick."""
    table = {int(r[1]): int(r[2]) for r in _read_fixture("code_values.txt") if r[0] == "code"}
    for c in range(4):
        signed = np.array([(c + 0x7F) ^ 0x80], dtype=np.uint8).view(np.int8)[0]
        assert table[c] == int(signed)


def test_decode_fixture_bytes():
    for row in _read_fixture("code_values.txt"):
        if row[0] != "byte":
            continue
        byte = int(row[1], 16)
        expected = [int(v) for v in row[2:]]
        assert list(oracle.decode_byte(byte)) == expected, hex(byte)


def test_decode_all_256_bytes_against_base4_digits():
    for byte in range(256):
        assert list(oracle.decode_byte(byte)) == _digit_decode(byte)


def test_decode_block_weight_order():
    """Weight i of a block is field i%4 of code byte i//4 (brute force over a
    block whose bytes are all distinct)."""
    codes = np.arange(32, dtype=np.uint8) * 7 + 3
    vals = oracle.decode_block_codes(codes)
    for i in range(128):
        assert vals[i] == _digit_decode(int(codes[i // 4]))[i % 4]


# ---------------------------------------------------------------- worked example
def test_worked_example():
    fx = {r[0]: r[1:] for r in _read_fixture("worked_example.txt")}
    weights = [int(v) for v in fx["weights"]]
    acts = [int(v) for v in fx["activations"]]
    act_scale = np.float32(float(fx["act_scale"][0]))
    w_scale = np.float16(float(fx["weight_scale"][0]))
    # Encode the four weights in code byte 0 by hand (code = value + 1, field s
    # at bits 2s); every other weight of the block is 0 (code 1, byte 0x55).
    byte0 = sum((w + 1) << (2 * s) for s, w in enumerate(weights))
    assert byte0 == 0xA4
    codes = np.full(32, 0x55, dtype=np.uint8)
    codes[0] = byte0
    raw = _block(codes, w_scale)[None, :]
    q = np.zeros((1, 128), dtype=np.int8)
    q[0, :4] = acts
    xs = np.array([[act_scale]], dtype=np.float32)
    y, bound = oracle.matmul_raw(q, xs, raw, 1, 128)
    assert int(fx["dot"][0]) == int(np.dot(weights, acts))
    expected = float(fx["contribution"][0])
    assert abs(y[0, 0] - expected) <= bound[0, 0]
    # FP32 rounding of the scaled dot is exactly the printed 1.5.
    assert np.float32(y[0, 0]) == np.float32(expected)
    # And the FP64 value is exactly dot * fp32(0.1) * 0.5.
    assert Fraction(y[0, 0]) == 30 * Fraction(float(act_scale)) * Fraction(1, 2)


# ---------------------------------------------------------------- prepare
@pytest.mark.parametrize("n,k,pad", [(3, 128, 0), (5, 512, 6), (7, 1024, 1)])
def test_prepare_planes_layout(n, k, pad):
    raw = workloads.make_raw_weights(n, k, seed=11 + n, codes="ternary+3", row_pad=pad)
    planes = oracle.prepare_planes(raw, n, k)
    g = k // 128
    assert planes.size == n * g * 34                      # same storage size
    blocks = raw[:, : g * 34].reshape(n, g, 34)
    codes = planes[: n * k // 4].reshape(n, g, 32)
    scales = planes[n * k // 4:].reshape(n, g, 2)
    assert np.array_equal(codes, blocks[:, :, 2:])
    assert np.array_equal(scales, blocks[:, :, :2])
    # Round trip back to raw blocks.
    back = np.concatenate([scales, codes], axis=2).reshape(n, g * 34)
    assert np.array_equal(back, raw[:, : g * 34])


@pytest.mark.parametrize("n,k,pad", [(3, 128, 0), (17, 384, 6), (32, 1024, 1), (5, 640, 0)])
def test_prepare_tiles_preserves_every_value(n, k, pad):
    """The tile layout moves every code and scale to the address its
    definition names and nothing else: read back in weight order with an
    independent numpy gather (the inverse of the C scatter), the codes and
    scales equal the raw blocks' fields, and all padding is code 1 / scale 0."""
    raw = workloads.make_raw_weights(n, k, seed=21 + n, codes="ternary+3", row_pad=pad)
    tiles = oracle.prepare_tiles(raw, n, k)
    g = k // 128
    t, s8 = -(-n // 16), -(-g // 8)
    assert tiles.size == t * s8 * 4352
    blocks = raw[:, : g * 34].reshape(n, g, 34)
    # Raw codes in weight order: weight 4b + s of a block is field s of byte b.
    raw_codes = ((blocks[:, :, 2:, None] >> (2 * np.arange(4))) & 3).reshape(n, k)
    units = tiles.reshape(t, s8, 4352)
    # Unit code bytes: [b][kb][j][u][v], field s of byte v of dword u = weight
    # 128*(8sb + 2b + u//2) + 64*(u%2) + 16*kb + 4s + v of row 16t + j.
    code = units[:, :, :4096].reshape(t, s8, 4, 4, 16, 2, 2, 4)   # t, sb, b, kb, j, ug, uh, v
    fields = (code[..., None] >> (2 * np.arange(4))) & 3         # ..., v, s
    w = fields.transpose(0, 4, 1, 2, 5, 6, 3, 8, 7).reshape(t * 16, s8 * 1024)  # [row][sb, b, ug, uh, kb, s, v]
    assert np.array_equal(w[:n, :k], raw_codes)
    assert np.all(w[n:] == 1) and np.all(w[:, k:] == 1)
    sc = units[:, :, 4096:].reshape(t, s8, 16, 8, 2).transpose(0, 2, 1, 3, 4).reshape(t * 16, s8 * 8, 2)
    assert np.array_equal(sc[:n, :g], blocks[:, :, :2])
    assert np.all(sc[n:] == 0) and np.all(sc[:, g:] == 0)


# ---------------------------------------------------------------- quantiser
def _bf16(values):
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    assert torch.equal(t.float(), torch.tensor(np.asarray(values, dtype=np.float32))), "not bf16-exact"
    return workloads.bf16_bits(t)


def test_quantiser_closed_forms():
    for row in _read_fixture("quantiser_closed_forms.txt"):
        e, v, expect = int(row[0]), float(row[1]), int(row[2])
        group = np.zeros(128, dtype=np.float64)
        group[0] = 127.0 * 2.0 ** e
        group[5] = v * 2.0 ** e
        q, xs = oracle.quantize_act_i8(_bf16(group)[None, :])
        assert xs[0, 0] == np.float32(2.0 ** e)
        assert q[0, 5] == expect, row
        assert q[0, 0] == 127


def test_quantiser_exhaustive_power_of_two_scale():
    """Every bf16 value in [-127, 127] against round_half_even, scale 1."""
    vals = torch.arange(-(1 << 15), 1 << 15, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    vals = vals[torch.isfinite(vals) & (vals.abs() <= 127)].numpy().astype(np.float64)
    pad = (-len(vals)) % 127
    vals = np.concatenate([vals, np.zeros(pad)])
    groups = vals.reshape(-1, 127)
    x = np.concatenate([np.full((groups.shape[0], 1), 127.0), groups], axis=1)
    q, xs = oracle.quantize_act_i8(_bf16(x))
    assert np.all(xs == 1.0)
    expect = np.array([[round(Fraction(v)) for v in row] for row in x], dtype=np.int64)
    assert np.array_equal(q.astype(np.int64), expect)


def test_quantiser_zero_group_and_amax():
    x = np.zeros((2, 256))
    x[1, 128:] = np.arange(-3, 5, 1 / 16)
    q, xs = oracle.quantize_act_i8(_bf16(x))
    assert xs[0, 0] == 0.0 and np.signbit(xs[0, 0]) == False  # noqa: E712
    assert xs[0, 1] == 0.0 and xs[1, 0] == 0.0
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0)
    bits = _bf16(x)
    vals = torch.tensor(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    grp = vals[1, 128:]
    imax = int(np.argmax(np.abs(grp)))
    assert q[1, 128 + imax] == (127 if grp[imax] > 0 else -127)


def _exact_quantise(values_f32):
    """Quantise one group with exact rational arithmetic: the scale is the
    binary32 nearest amax/127, each quotient the binary32 nearest x/scale."""
    amax = max(abs(Fraction(float(v))) for v in values_f32)
    scale = _f32_nearest(amax / 127)
    div = Fraction(float(scale)) if scale > 0 else Fraction(1)
    q = []
    for v in values_f32:
        r = round(Fraction(float(_f32_nearest(Fraction(float(v)) / div))))
        q.append(max(-127, min(127, r)))
    return np.array(q, dtype=np.int64), scale


@pytest.mark.parametrize("dist,seed", [("normal", 1), ("normal+outliers", 2), ("laplace", 3)])
def test_quantiser_exact_rational(dist, seed):
    x = workloads.make_activations(3, 1024, seed, dist)
    q, xs = oracle.quantize_act_i8(workloads.bf16_bits(x))
    xf = x.float().numpy()
    for m in range(3):
        for g in range(8):
            eq, es = _exact_quantise(xf[m, g * 128:(g + 1) * 128])
            assert xs[m, g].view(np.uint32) == np.float32(es).view(np.uint32)
            assert np.array_equal(q[m, g * 128:(g + 1) * 128].astype(np.int64), eq)


def test_quantiser_divides_not_reciprocal():
    """Groups where amax/127 (one rounding) and amax*fl(1/127) differ: the
    oracle must give the correctly rounded quotient."""
    recip = np.float32(1.0) / np.float32(127.0)
    found = 0
    gen = np.random.default_rng(5)
    while found < 20:
        amax = np.float32(torch.tensor(float(gen.uniform(0.5, 40))).to(torch.bfloat16).float().item())
        exact = _f32_nearest(Fraction(float(amax)) / 127)
        if np.float32(amax * recip) == exact:
            continue
        found += 1
        group = torch.zeros(128, dtype=torch.float32)
        group[3] = -float(amax)
        group[7] = float(amax) / 3
        group = group.to(torch.bfloat16)
        q, xs = oracle.quantize_act_i8(workloads.bf16_bits(group)[None, :])
        assert xs[0, 0] == exact
        eq, _ = _exact_quantise(group.float().numpy())
        assert np.array_equal(q[0].astype(np.int64), eq)


def test_quantiser_subnormal_scale():
    """A group of tiny bf16 values gives an FP32-subnormal scale."""
    tiny = np.array([2.0 ** -130, -3 * 2.0 ** -131, 2.0 ** -126, 5 * 2.0 ** -133])
    group = np.zeros(128)
    group[:4] = tiny
    q, xs = oracle.quantize_act_i8(_bf16(group)[None, :])
    eq, es = _exact_quantise(torch.tensor(group, dtype=torch.float32).to(torch.bfloat16).float().numpy())
    assert xs[0, 0] == es and xs[0, 0] < np.finfo(np.float32).tiny
    assert np.array_equal(q[0].astype(np.int64), eq)


def test_quantiser_sign_symmetry_and_dtypes():
    x = workloads.make_activations(2, 512, 9, "normal")
    q, xs = oracle.quantize_act_i8(workloads.bf16_bits(x))
    qn, xsn = oracle.quantize_act_i8(workloads.bf16_bits(-x))
    assert np.array_equal(qn, -q) and np.array_equal(xsn, xs)
    # The same values given as f16 (exact for these magnitudes? not always) and f32.
    q32, xs32 = oracle.quantize_act_i8(x.float().numpy(), dtype="f32")
    assert np.array_equal(q32, q) and np.array_equal(xs32, xs)
    xh = x.float().to(torch.float16)
    qh, xsh = oracle.quantize_act_i8(xh.view(torch.int16).numpy().view(np.uint16), dtype="f16")
    xhf = xh.float().numpy()
    for m in range(2):
        for g in range(4):
            eq, es = _exact_quantise(xhf[m, g * 128:(g + 1) * 128])
            assert xsh[m, g] == es and np.array_equal(qh[m, g * 128:(g + 1) * 128].astype(np.int64), eq)


def test_quantiser_row_stride():
    x = workloads.make_activations(3, 640, 4, "normal")
    bits = workloads.bf16_bits(x)
    q_full, xs_full = oracle.quantize_act_i8(bits)
    q_part, xs_part = oracle.quantize_act_i8(bits, k=384)
    assert np.array_equal(q_part, q_full[:, :384]) and np.array_equal(xs_part, xs_full[:, :3])


# ---------------------------------------------------------------- matmul
@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (2, 3, 256), (3, 5, 512), (4, 2, 384)])
def test_matmul_exact_rational_brute_force(m, n, k):
    raw = workloads.make_raw_weights(n, k, seed=100 + k + n, codes="ternary+3", row_pad=3)
    x = workloads.make_activations(m, k, 200 + m, "laplace")
    q, xs = oracle.quantize_act_i8(workloads.bf16_bits(x))
    y, bound = oracle.matmul_raw(q, xs, raw, n, k)
    g = k // 128
    for mi in range(m):
        for ni in range(n):
            exact = Fraction(0)
            for kk in range(k):
                blk = raw[ni, (kk // 128) * 34:(kk // 128) * 34 + 34]
                ws = Fraction(float(blk[:2].copy().view(np.float16)[0]))
                w = _digit_decode(int(blk[2 + (kk % 128) // 4]))[kk % 4]
                exact += Fraction(int(q[mi, kk])) * Fraction(float(xs[mi, kk // 128])) * w * ws
            err = abs(Fraction(y[mi, ni]) - exact)
            assert err <= abs(exact) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 30), (mi, ni)
    assert np.all(bound >= 1e-6)
    assert g >= 1


def test_matmul_dense_identity():
    """The oracle equals dequantise-then-matmul in float64 (the pages' own
    FP64 reconstruction check, Test 8: within 1e-12)."""
    m, n, k = 3, 40, 1024
    raw = workloads.make_raw_weights(n, k, seed=21, codes="ternary+3")
    x = workloads.make_activations(m, k, 22, "normal+outliers")
    q, xs = oracle.quantize_act_i8(workloads.bf16_bits(x))
    y, bound = oracle.matmul_raw(q, xs, raw, n, k)
    dense, _ = _dense_weights(raw, n, k)
    act = q.astype(np.float64) * np.repeat(xs.astype(np.float64), 128, axis=1)
    ref = act @ dense.T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_matmul_bound_is_sum_of_group_magnitudes():
    m, n, k = 2, 6, 768
    raw = workloads.make_raw_weights(n, k, seed=31, codes="ternary")
    x = workloads.make_activations(m, k, 32, "normal")
    q, xs = oracle.quantize_act_i8(workloads.bf16_bits(x))
    _, bound = oracle.matmul_raw(q, xs, raw, n, k)
    _, vals = _dense_weights(raw, n, k)
    g = k // 128
    ws = raw[:, : g * 34].reshape(n, g, 34)[:, :, :2].copy().view(np.float16).astype(np.float64).reshape(n, g)
    dots = (q.astype(np.int64).reshape(m, 1, g, 128) * vals.reshape(1, n, g, 128)).sum(-1)  # [m][n][g]
    mag = np.abs(dots * xs.astype(np.float64)[:, None, :] * ws[None, :, :]).sum(-1)
    np.testing.assert_allclose(bound, 1e-5 * mag + 1e-6, rtol=1e-12)


def test_matmul_invariants():
    m, n, k = 3, 7, 640
    raw = workloads.make_raw_weights(n, k, seed=41, codes="ternary+3")
    x = workloads.make_activations(m, k, 42, "normal")
    q, xs = oracle.quantize_act_i8(workloads.bf16_bits(x))
    y, _ = oracle.matmul_raw(q, xs, raw, n, k)
    g = k // 128
    # Doubling every weight scale (fp16 exponent + 1) doubles y exactly.
    raw2 = raw.copy()
    sc = raw2[:, : g * 34].reshape(n, g, 34)[:, :, :2].copy().view(np.float16)
    raw2.reshape(n, g, 34)[:, :, :2] = (sc.astype(np.float32) * 2).astype(np.float16).view(np.uint8).reshape(n, g, 2)
    y2, _ = oracle.matmul_raw(q, xs, raw2, n, k)
    assert np.array_equal(y2, 2 * y)
    # Negating the activations negates y exactly.
    yn, _ = oracle.matmul_raw(-q, xs, raw, n, k)
    assert np.array_equal(yn, -y)
    # Permuting weight rows permutes outputs; a column does not depend on others.
    perm = np.array([3, 0, 6, 1, 5, 2, 4])
    yp, _ = oracle.matmul_raw(q, xs, raw[perm], n, k)
    assert np.array_equal(yp, y[:, perm])
    y1, _ = oracle.matmul_raw(q[1:2], xs[1:2], raw, n, k)
    assert np.array_equal(y1[0], y[1])


def test_matmul_sample_matches_full():
    m, n, k = 2, 9, 256
    raw = workloads.make_raw_weights(n, k, seed=51, codes="ternary")
    x = workloads.make_activations(m, k, 52, "normal")
    q, xs = oracle.quantize_act_i8(workloads.bf16_bits(x))
    y, bound = oracle.matmul_raw(q, xs, raw, n, k)
    mi = np.array([0, 1, 1, 0])
    ni = np.array([8, 0, 4, 3])
    ys, bs = oracle.matmul_raw_sample(q, xs, raw, n, k, mi, ni)
    assert np.array_equal(ys, y[mi, ni]) and np.array_equal(bs, bound[mi, ni])


def test_quantised_projection_error_sanity():
    """Not parity: the quantised result stays near the unquantised product
    (relative RMS under the pages' 0.03 gate)."""
    m, n, k = 2, 64, 2048
    raw = workloads.make_raw_weights(n, k, seed=61, codes="ternary")
    x = workloads.make_activations(m, k, 62, "normal")
    q, xs = oracle.quantize_act_i8(workloads.bf16_bits(x))
    y, _ = oracle.matmul_raw(q, xs, raw, n, k)
    dense, _ = _dense_weights(raw, n, k)
    ref = x.double().numpy() @ dense.T
    rel = np.sqrt(((y - ref) ** 2).sum() / (ref ** 2).sum())
    assert rel < 0.03


# ---------------------------------------------------------------- smaller activation groups
# Page "Kernel experiments: recorded evidence", section C (Diagram 3, Tests 8
# and 9): the same weights, activations quantised per 64 or 32 elements.
@pytest.mark.parametrize("agroup", [64, 32])
def test_agroup_closed_forms(agroup):
    """Each activation group gets its own power-of-two scale: group a holds
    127 * 2^e_a, so xs = 2^e_a exactly and q = round_half_even(x / 2^e_a),
    with the values placed so that a shifted group index would read another
    group's scale."""
    k = 256
    per = k // agroup
    exps = [(-3 + 2 * a) % 7 - 3 for a in range(per)]
    x = np.zeros((1, k))
    picks = [1.5, 2.5, -2.5, 0.5, 3.25, -7.0, 126.5, 17.75]
    for a in range(per):
        x[0, a * agroup] = 127.0 * 2.0 ** exps[a]
        for j, v in enumerate(picks[: agroup // 8]):
            x[0, a * agroup + 1 + 3 * j] = v * 2.0 ** exps[a]
    q, xs = oracle.quantize_act_i8_g(_bf16(x), agroup)
    assert xs.shape == (1, per)
    for a in range(per):
        assert xs[0, a] == np.float32(2.0 ** exps[a])
        for i in range(agroup):
            val = Fraction(float(x[0, a * agroup + i])) / Fraction(2) ** exps[a]
            assert q[0, a * agroup + i] == round(val), (a, i)


@pytest.mark.parametrize("agroup", [64, 32])
def test_agroup_exact_rational(agroup):
    """Every activation group against exact rational quantisation."""
    x = workloads.make_activations(2, 512, 40 + agroup, "normal+outliers")
    q, xs = oracle.quantize_act_i8_g(workloads.bf16_bits(x), agroup)
    xf = x.float().numpy()
    for m in range(2):
        for a in range(512 // agroup):
            eq, es = _exact_quantise(xf[m, a * agroup:(a + 1) * agroup])
            assert xs[m, a].view(np.uint32) == np.float32(es).view(np.uint32)
            assert np.array_equal(q[m, a * agroup:(a + 1) * agroup].astype(np.int64), eq)


def test_agroup_128_is_the_group_128_definition_and_equal_amax_groups_agree():
    x = workloads.make_activations(3, 640, 12, "laplace")
    bits = workloads.bf16_bits(x)
    q, xs = oracle.quantize_act_i8(bits)
    q1, xs1 = oracle.quantize_act_i8_g(bits, 128)
    assert np.array_equal(q, q1) and np.array_equal(xs.view(np.uint32), xs1.view(np.uint32))
    # When every 32-group of a 128-group holds the same amax, the smaller
    # groups reproduce the group-128 codes and repeat its scale.
    xv = x.float().numpy().copy()
    for g in range(640 // 32):
        xv[:, g * 32] = 9.0  # above every other |x| of this Laplace(0, 0.5) draw
    bits = _bf16(xv)
    q, xs = oracle.quantize_act_i8(bits)
    for agroup in (64, 32):
        qa, xsa = oracle.quantize_act_i8_g(bits, agroup)
        assert np.array_equal(qa, q)
        assert np.array_equal(xsa, np.repeat(xs, 128 // agroup, axis=1))


@pytest.mark.parametrize("agroup,m,n,k", [(64, 1, 2, 128), (64, 2, 3, 256), (32, 2, 2, 256), (32, 1, 3, 384)])
def test_agroup_matmul_exact_rational_brute_force(agroup, m, n, k):
    raw = workloads.make_raw_weights(n, k, seed=300 + k + n + agroup, codes="ternary+3", row_pad=2)
    x = workloads.make_activations(m, k, 301 + m, "laplace")
    q, xs = oracle.quantize_act_i8_g(workloads.bf16_bits(x), agroup)
    y, bound = oracle.matmul_raw_g(q, xs, raw, n, k, agroup)
    for mi in range(m):
        for ni in range(n):
            exact = Fraction(0)
            for kk in range(k):
                blk = raw[ni, (kk // 128) * 34:(kk // 128) * 34 + 34]
                ws = Fraction(float(blk[:2].copy().view(np.float16)[0]))
                w = _digit_decode(int(blk[2 + (kk % 128) // 4]))[kk % 4]
                exact += Fraction(int(q[mi, kk])) * Fraction(float(xs[mi, kk // agroup])) * w * ws
            err = abs(Fraction(y[mi, ni]) - exact)
            assert err <= abs(exact) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 30), (mi, ni)
    assert np.all(bound >= 1e-6)


@pytest.mark.parametrize("agroup", [128, 64, 32])
def test_agroup_matmul_dense_identity_and_sample(agroup):
    m, n, k = 2, 24, 1024
    raw = workloads.make_raw_weights(n, k, seed=23, codes="ternary+3")
    x = workloads.make_activations(m, k, 24, "normal+outliers")
    q, xs = oracle.quantize_act_i8_g(workloads.bf16_bits(x), agroup)
    y, bound = oracle.matmul_raw_g(q, xs, raw, n, k, agroup)
    dense, _ = _dense_weights(raw, n, k)
    act = q.astype(np.float64) * np.repeat(xs.astype(np.float64), agroup, axis=1)
    np.testing.assert_allclose(y, act @ dense.T, rtol=1e-12, atol=1e-12)
    if agroup == 128:
        y0, b0 = oracle.matmul_raw(q, xs, raw, n, k)
        assert np.array_equal(y, y0) and np.array_equal(bound, b0)
    mi = np.array([0, 1, 1, 0]); ni = np.array([0, 5, 23, 17])
    ys, bs = oracle.matmul_raw_sample_g(q, xs, raw, n, k, agroup, mi, ni)
    assert np.array_equal(ys, y[mi, ni]) and np.array_equal(bs, bound[mi, ni])


def test_agroup_smaller_groups_reduce_error():
    """Smaller activation groups quantise more finely: the dequantised
    activations' relative RMS error falls from 128 to 64 to 32 on data with
    outliers (the direction Test 8 reports; a sanity property, not parity)."""
    x = workloads.make_activations(4, 2048, 77, "normal+outliers")
    xf = x.float().numpy().astype(np.float64)
    errs = []
    for agroup in (128, 64, 32):
        q, xs = oracle.quantize_act_i8_g(workloads.bf16_bits(x), agroup)
        deq = q.astype(np.float64) * np.repeat(xs.astype(np.float64), agroup, axis=1)
        errs.append(np.sqrt(((deq - xf) ** 2).sum() / (xf ** 2).sum()))
    assert errs[0] > errs[1] > errs[2], errs


def test_agroup_rejects_bad_groups():
    x = np.zeros((1, 256), dtype=np.float32)
    for bad in (0, 16, 96, 256):
        with pytest.raises(ValueError):
            oracle.quantize_act_i8_g(x, bad, "f32")
