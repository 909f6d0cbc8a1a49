"""Pins of the float64 oracle against facts that do not come from the oracle:
hand-assembled blobs, hand-worked cases, closed forms, brute force, and
textbook identities.  CPU only."""
import itertools
import json
import math
import os
import subprocess
import sys
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import blobkit

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


SMALL = oracle.Dims(H=256, I=256, E=8, K=4, bits=4)


# ---- bf16 and format ----------------------------------------------------------

def test_bf16_decode_exact():
    assert oracle.lib().or_bf16(0x3F80) == 1.0
    assert oracle.lib().or_bf16(0xC000) == -2.0
    assert oracle.lib().or_bf16(0x3C00) == 2.0 ** -7
    assert oracle.lib().or_bf16(0x3F81) == 1.0 + 2.0 ** -7
    assert oracle.lib().or_bf16(0x7F7F) == float.fromhex("0x1.fep+127")
    assert oracle.lib().or_bf16(0x0001) == 2.0 ** -133  # smallest subnormal


def test_blob_size_matches_page_expert_size():
    facts = _gold("page_facts.json")
    d4 = oracle.Dims(H=facts["hidden"]["value"], I=1024, E=512, K=4, bits=4)
    assert oracle.blob_bytes(d4) == 7_077_888
    assert oracle.blob_bytes(d4) == facts["expert_mib_4bit"]["value"] * 2 ** 20
    d2 = oracle.Dims(H=4096, I=1024, E=512, K=4, bits=2)
    assert oracle.blob_bytes(d2) == 3_932_160
    # 60 x 512 experts: the 2-bit stack is about 90 GB smaller (pages: ~89 GB saved)
    saving_gb = 60 * 512 * (7_077_888 - 3_932_160) / 1e9
    assert abs(saving_gb - facts["saving_gb_2bit"]["value"]) < 10


def test_section_offsets_by_hand():
    # H = I = 256, 4-bit: code sections 256 rows x 128 B = 32768 B;
    # (s,z) sections 256 rows x 4 groups x 4 B = 4096 B
    want = [0, 32768, 65536, 98304, 102400, 106496, 110592]
    assert [oracle.section_offset(SMALL, s) for s in range(7)] == want
    # 2-bit, H=512, I=256: gate/up codes 256 x 512/16 x 4 = 32768 B,
    # down codes 512 x 256/16 x 4 = 32768 B, gate/up sb 256 x 8 x 4 = 8192,
    # down sb 512 x 4 x 4 = 8192
    d2 = oracle.Dims(H=512, I=256, E=4, K=2, bits=2)
    want2 = [0, 32768, 65536, 98304, 106496, 114688, 122880]
    assert [oracle.section_offset(d2, s) for s in range(7)] == want2


def _random_codes_blob(d, rng, s_of=None):
    bits = d.bits
    qmax = 2 ** bits
    qg = rng.integers(0, qmax, (d.I, d.H))
    qu = rng.integers(0, qmax, (d.I, d.H))
    qd = rng.integers(0, qmax, (d.H, d.I))

    def sb(rows, cols):
        if s_of is None:
            return (np.ones((rows, cols // 64), np.float32), np.zeros((rows, cols // 64), np.float32))
        return s_of(rows, cols // 64)
    blob = blobkit.assemble(d.H, d.I, bits, qg, qu, qd, sb(d.I, d.H), sb(d.I, d.H), sb(d.H, d.I))
    return blob, (qg, qu, qd)


@pytest.mark.parametrize("bits", [4, 2])
def test_code_positions_all_elements(bits):
    d = oracle.Dims(H=512, I=256, E=4, K=2, bits=bits)
    rng = np.random.default_rng(7)
    blob, qs = _random_codes_blob(d, rng)
    assert blob.size == oracle.blob_bytes(d)
    for which in range(3):
        # s = 1, z = 0: the dequantised matrix is the code matrix itself
        np.testing.assert_array_equal(oracle.dequant_matrix(d, blob, which), qs[which])
    assert oracle.code(d, blob, 0, 3, 5) == qs[0][3, 5]
    assert oracle.code(d, blob, 2, 511, 255) == qs[2][511, 255]


def test_code_bit_order_hand_word():
    # one gate row whose first word is 0x76543210: codes 0..7 in order
    d = SMALL
    qg = np.zeros((d.I, d.H), int)
    qg[0, :8] = [0, 1, 2, 3, 4, 5, 6, 7]
    z = np.zeros
    sb = (np.ones((256, 4), np.float32), z((256, 4), np.float32))
    blob = blobkit.assemble(256, 256, 4, qg, z((256, 256), int), z((256, 256), int), sb, sb, sb)
    assert bytes(blob[:4]) == bytes([0x10, 0x32, 0x54, 0x76])
    assert [oracle.code(d, blob, 0, 0, c) for c in range(8)] == list(range(8))


def test_scale_bias_per_group_and_row():
    # H != I so that a row or group index computed from the wrong dimension
    # lands on another word; every (s, z) pair is distinct, so reading the word
    # of another row or group (c / 128 in place of c / 64, r / 2 in place of r)
    # gives a different value somewhere
    d = oracle.Dims(H=512, I=256, E=4, K=2, bits=4)
    rng = np.random.default_rng(3)
    drawn = {}

    def s_of(rows, groups):
        # exact bf16 values: scales k 2^-10 (k = 1..127), biases j 2^-12
        n = rows * groups
        s = (1 + rng.permutation(np.arange(n) % 127)) * 2.0 ** -10
        z = (rng.permutation(np.arange(n) % 255) - 127) * 2.0 ** -12
        s = s.reshape(rows, groups).astype(np.float32)
        z = z.reshape(rows, groups).astype(np.float32)
        drawn[len(drawn)] = (s, z)
        return s, z
    blob, qs = _random_codes_blob(d, rng, s_of)
    assert len(drawn) == 3  # gate, up, down, in that order
    for which, rows, cols in [(0, d.I, d.H), (1, d.I, d.H), (2, d.H, d.I)]:
        s, z = drawn[which]
        assert s.shape == (rows, cols // 64)
        # the (s, z) pair of every (row, group), through the oracle's accessor
        for r in range(rows):
            for g in range(cols // 64):
                c = 64 * g + (r * 7 + g * 13) % 64  # any column of the group
                assert oracle.scale_bias(d, blob, which, r, c) == (float(s[r, g]), float(z[r, g]))
        # and every element of the dequantised matrix against s q + z built
        # here from the drawn arrays (exact in float64)
        want = (np.repeat(s.astype(np.float64), 64, axis=1) * qs[which]
                + np.repeat(z.astype(np.float64), 64, axis=1))
        np.testing.assert_array_equal(oracle.dequant_matrix(d, blob, which), want)


def test_dequant_closed_forms():
    hw = 256
    for q, s, z, want in [(0, 0.0078125, -0.0625, -0.0625),        # q=0 -> z
                          (15, 0.0078125, -0.0625, 15 * 0.0078125 - 0.0625),
                          (9, 0.0, 0.03125, 0.03125),              # s=0 -> z
                          (15, 0.015625, 0.0, 0.234375)]:
        blob = blobkit.constant_blob(hw, hw, 4, q, s, z)
        assert oracle.dequant(SMALL, blob, 0, 0, 0) == want
        assert oracle.dequant(SMALL, blob, 2, 255, 255) == want
        if s != 0:
            # round trip: the code is recovered exactly
            assert (oracle.dequant(SMALL, blob, 1, 7, 9) - z) / s == q


def test_dequant_f32_is_one_rounding_of_exact_value():
    # s = 1 + 2^-7 (bf16 exact), z = 2^-30 * (1 + 2^-7): s*15 + z needs ~37 bits
    s = 1 + 2 ** -7
    z = 2 ** -30 * (1 + 2 ** -7)
    blob = blobkit.constant_blob(256, 256, 4, 15, s, z)
    exact = Fraction(s) * 15 + Fraction(z)
    assert Fraction(oracle.dequant(SMALL, blob, 0, 0, 0)) == exact
    want32 = np.float32(float(exact))  # float(exact) is exact here (< 53 bits)
    got32 = oracle.lib().or_dequant_f32(oracle.Dims(256, 256, 8, 4).c(), blob.ctypes.data_as(
        oracle._u8p), 0, 0, 0)
    assert np.float32(got32) == want32
    assert float(want32) != float(exact)  # a real rounding happened
    Wf = oracle.dequant_matrix_f32(SMALL, blob, 0)
    assert Wf[3, 4] == want32


def test_dequant_inexact_aborts():
    # scale 2^60 and bias 2^-60 cannot be summed exactly in double: the
    # oracle must refuse instead of returning a rounded weight
    code = r"""
import sys; sys.path.insert(0, %r)
import oracle
from tests import blobkit
blob = blobkit.constant_blob(256, 256, 4, 3, 2.0**60, 2.0**-60)
oracle.dequant(oracle.Dims(256, 256, 8, 4), blob, 0, 0, 0)
print("NOT ABORTED")
""" % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert r.returncode != 0
    assert "inexact dequant" in r.stderr
    assert "NOT ABORTED" not in r.stdout


# ---- routing -------------------------------------------------------------------

def test_router_matches_numpy_matvec():
    d = oracle.Dims(H=512, I=256, E=32, K=4)
    rng = np.random.default_rng(11)
    W = synth.f32_to_bf16(rng.standard_normal((32, 512)) * 0.02)
    x = synth.f32_to_bf16(rng.standard_normal(512))
    got = oracle.router_logits(d, W, x)
    want = oracle.bf16_to_f64(W) @ oracle.bf16_to_f64(x)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-15)


def test_router_one_hot():
    d = oracle.Dims(H=256, I=256, E=16, K=4)
    rng = np.random.default_rng(5)
    W = synth.f32_to_bf16(rng.standard_normal((16, 256)) * 0.02)
    x = np.zeros(256, np.uint16)
    x[37] = 0x4040  # 3.0
    got = oracle.router_logits(d, W, x)
    np.testing.assert_array_equal(got, 3.0 * oracle.bf16_to_f64(W[:, 37]))


@pytest.mark.parametrize("case", ["route_2_1_0_m1_k2", "route_ties_k2", "route_all_k4"])
def test_route_hand_worked(case):
    c = _gold("hand_worked.json")[case]
    d = oracle.Dims(H=256, I=256, E=len(c["logits"]), K=c["K"])
    ids, w, gap = oracle.route_logits(d, np.array(c["logits"]))
    assert list(ids) == c["ids"]
    np.testing.assert_allclose(w, c["w"], rtol=1e-15)
    assert gap == c["gap"]


def test_topk_brute_force_small_E():
    rng = np.random.default_rng(123)
    E, K = 16, 4
    d = oracle.Dims(H=256, I=256, E=E, K=K)
    for trial in range(50):
        logits = rng.standard_normal(E) * (1 + trial % 3)
        ids, w, gap = oracle.route_logits(d, logits)
        best = max(itertools.combinations(range(E), K), key=lambda s: sum(logits[list(s)]))
        assert set(ids) == set(best)
        assert all(logits[ids[i]] >= logits[ids[i + 1]] for i in range(K - 1))
        srt = np.sort(logits)[::-1]
        assert gap == pytest.approx(np.min(srt[:K] - srt[1:K + 1]), rel=0, abs=0)


def test_renormalised_weights_identities():
    rng = np.random.default_rng(9)
    for E, K in [(16, 4), (512, 4), (8, 8), (9, 1)]:
        d = oracle.Dims(H=256, I=256, E=E, K=K)
        logits = rng.standard_normal(E) * 1.4
        ids, w, _ = oracle.route_logits(d, logits)
        sel = logits[ids]
        soft_sel = np.exp(sel - sel.max()) / np.sum(np.exp(sel - sel.max()))
        np.testing.assert_allclose(w, soft_sel, rtol=1e-13)   # = softmax over the kept logits
        assert abs(np.sum(w) - 1) < 1e-15
        if K == E:  # K = E: the full softmax
            full = np.exp(logits - logits.max())
            full /= full.sum()
            np.testing.assert_allclose(w, full[ids], rtol=1e-13)
        if K == 1:
            assert w[0] == 1.0


def test_route_permutation_equivariance():
    rng = np.random.default_rng(21)
    E, K = 64, 4
    d = oracle.Dims(H=256, I=256, E=E, K=K)
    logits = rng.standard_normal(E)
    perm = rng.permutation(E)
    ids, w, _ = oracle.route_logits(d, logits)
    ids_p, w_p, _ = oracle.route_logits(d, logits[perm])
    # expert perm[i] of the permuted list is expert i's original index
    np.testing.assert_array_equal(perm[ids_p], ids)
    np.testing.assert_allclose(w_p, w, rtol=1e-15)


# ---- SwiGLU and the expert MLP --------------------------------------------------

def test_silu_values():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(_gold("hand_worked.json")["silu_1"]["value"], rel=1e-15)
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.silu(-40.0)) < 1e-15
    assert oracle.silu(-1.0) == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)


def _per_matrix_constant_blob(H, I, gate, up, down):
    def mats(rows, cols, p):
        return (np.full((rows, cols), p["q"]),
                (np.full((rows, cols // 64), p["s"], np.float32),
                 np.full((rows, cols // 64), p["z"], np.float32)))
    qg, sg = mats(I, H, gate)
    qu, su = mats(I, H, up)
    qd, sd = mats(H, I, down)
    return blobkit.assemble(H, I, 4, qg, qu, qd, sg, su, sd)


@pytest.mark.parametrize("case", ["expert_saturated", "expert_silu_1"])
def test_expert_closed_form(case):
    c = _gold("hand_worked.json")[case]
    d = oracle.Dims(H=c["H"], I=c["I"], E=4, K=2)
    blob = _per_matrix_constant_blob(c["H"], c["I"], c["gate"], c["up"], c["down"])
    x = np.full(c["H"], c["x"])
    y = oracle.expert(d, blob, x)
    np.testing.assert_allclose(y, c["y"], rtol=1e-15)


def test_expert_matches_numpy_on_dequantised_matrices():
    d = oracle.Dims(H=512, I=256, E=4, K=2)
    p = synth.BlobParams(seed=77, H=512, I=256)
    blob = synth.blob_host(p, 0, 1)
    rng = np.random.default_rng(4)
    x = synth.f32_to_bf16(synth.rms_normalise(rng.standard_normal(512)))
    xd = oracle.bf16_to_f64(x)
    G = oracle.dequant_matrix(d, blob, 0)
    U = oracle.dequant_matrix(d, blob, 1)
    D = oracle.dequant_matrix(d, blob, 2)
    assert D.shape == (512, 256)
    g, u = G @ xd, U @ xd
    h = g / (1 + np.exp(-g)) * u
    want = D @ h
    y, hh = oracle.expert(d, blob, x, want_h=True)
    np.testing.assert_allclose(hh, h, rtol=1e-11, atol=1e-12 * np.abs(h).max())
    np.testing.assert_allclose(y, want, rtol=1e-11, atol=1e-12 * np.abs(want).max())


def test_group_factorisation_identity():
    # sum_c (s q_c + z) x_c = s sum_c q_c x_c + z sum_c x_c over one group of
    # 64: the algebra a dequantising GEMV may use in place of per-weight FMAs
    rng = np.random.default_rng(8)
    for _ in range(20):
        q = rng.integers(0, 16, 64).astype(np.float64)
        x = rng.standard_normal(64)
        s, z = rng.uniform(0.005, 0.02), rng.uniform(-0.08, 0.08)
        lhs = np.sum((s * q + z) * x)
        rhs = s * np.sum(q * x) + z * np.sum(x)
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


# ---- layer ---------------------------------------------------------------------

def _layer_inputs(E, K, T, H=256, I=256, seed=31):
    d = oracle.Dims(H=H, I=I, E=E, K=K)
    p = synth.BlobParams(seed=seed, H=H, I=I)
    router = synth.router_weights(seed, 0, E, H)
    blobs = {e: synth.blob_host(p, 0, e) for e in range(E)}
    shared = synth.blob_host(p, 0, 100000)
    x = synth.tokens(seed, 0, T, H)
    return d, router, blobs, shared, x


def test_identical_experts_combine_to_one_expert():
    # sum_k w_k = 1, so K copies of the same expert give that expert's output
    d, router, blobs, shared, x = _layer_inputs(E=8, K=4, T=2)
    same = blobs[0]
    y, ids, w, _, _ = oracle.layer(d, router, {e: same for e in range(8)}, shared, x)
    for t in range(2):
        want = oracle.expert(d, same, x[t]) + oracle.expert(d, shared, x[t])
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_zero_shared_expert_leaves_routed_sum():
    d, router, blobs, shared, x = _layer_inputs(E=8, K=4, T=1)
    zero = blobkit.constant_blob(256, 256, 4, 5, 0.0, 0.0)
    y, ids, w, _, _ = oracle.layer(d, router, blobs, zero, x)
    want = sum(w[0, k] * oracle.expert(d, blobs[ids[0, k]], x[0]) for k in range(4))
    np.testing.assert_allclose(y[0], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    d0 = oracle.Dims(H=256, I=256, E=8, K=4, has_shared=0)
    y0, _, _, _, _ = oracle.layer(d0, router, blobs, None, x)
    np.testing.assert_allclose(y0[0], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_batched_layer_equals_per_token_layers():
    d, router, blobs, shared, x = _layer_inputs(E=8, K=2, T=3)
    yb, idsb, wb, lb, gb = oracle.layer(d, router, blobs, shared, x)
    for t in range(3):
        y1, ids1, w1, l1, g1 = oracle.layer(d, router, blobs, shared, x[t:t + 1])
        np.testing.assert_array_equal(y1[0], yb[t])
        np.testing.assert_array_equal(ids1[0], idsb[t])


def test_expert_forward_invalid_id_contributes_zero():
    d, router, blobs, shared, x = _layer_inputs(E=8, K=2, T=1)
    ids = np.array([[3, 99]], np.int32)
    w = np.array([[0.6, 0.4]])
    y = oracle.expert_forward(d, blobs, shared, x, ids, w)
    want = 0.6 * oracle.expert(d, blobs[3], x[0]) + oracle.expert(d, shared, x[0])
    np.testing.assert_allclose(y[0], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


# ---- generator, read back through the oracle's own parser -----------------------

@pytest.mark.parametrize("bits", [4, 2])
def test_generated_blob_ranges_through_oracle_parser(bits):
    # a section-offset or field-order mistake in either the generator or the
    # oracle would put code bits where scales are read (or vice versa)
    d = oracle.Dims(H=4096, I=1024, E=16, K=4, bits=bits)
    p = synth.BlobParams(seed=5, bits=bits)
    blob = synth.blob_host(p, 2, 9)
    assert blob.size == oracle.blob_bytes(d)
    rng = np.random.default_rng(0)
    for which, rows, cols in [(0, 1024, 4096), (1, 1024, 4096), (2, 4096, 1024)]:
        for _ in range(200):
            r, c = int(rng.integers(rows)), int(rng.integers(cols))
            s, z = oracle.scale_bias(d, blob, which, r, c)
            # bounds widened by half a bf16 ulp (values are rounded to bf16)
            assert 0.005 * (1 - 2 ** -8) <= s <= 0.02 * (1 + 2 ** -8)
            assert -0.08 * (1 + 2 ** -8) <= z <= 0.08 * (1 + 2 ** -8)
    W = oracle.dequant_matrix(d, blob, 2)
    G = oracle.dequant_matrix(d, blob, 0)
    # codes uniform: the per-group mean of q is near (2^b - 1)/2
    q = np.array([oracle.code(d, blob, 0, 0, c) for c in range(4096)])
    hist = np.bincount(q, minlength=2 ** bits)
    expect = 4096 / 2 ** bits
    chi2 = float(np.sum((hist - expect) ** 2 / expect))
    assert chi2 < 60  # dof 15 (or 3): far below this for a uniform source
    assert np.isfinite(W).all() and np.isfinite(G).all()


# ---- residual stream and pre-MoE norm -------------------------------------------

def test_f64_to_bf16_rounds_to_nearest_even():
    # bf16 keeps 8 significant bits: around 1.0 the spacing is 2^-7
    assert oracle.f64_to_bf16(1.0) == 0x3F80
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80        # tie -> even (1.0)
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82    # tie -> even (1 + 2^-6)
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 0x3F81  # above the tie
    assert oracle.f64_to_bf16(-2.5) == 0xC020
    # just off a tie by less than half an fp32 step: a rounding through fp32
    # would first land on the tie and then go to the even neighbour
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81   # above -> up
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0 ** -8 - 2.0 ** -30) == 0x3F81  # below -> down
    assert oracle.f64_to_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == 0xBF81
    # subnormals (spacing 2^-133) and the top of the range
    assert oracle.f64_to_bf16(2.0 ** -133) == 0x0001
    assert oracle.f64_to_bf16(2.0 ** -134) == 0x0000              # tie -> even (0)
    assert oracle.f64_to_bf16(1.5 * 2.0 ** -134) == 0x0001
    assert oracle.f64_to_bf16(3 * 2.0 ** -134) == 0x0002          # tie -> even
    assert oracle.f64_to_bf16(2.0 ** -126) == 0x0080               # smallest normal
    assert oracle.f64_to_bf16(float.fromhex("0x1.fep127")) == 0x7F7F   # largest finite
    assert oracle.f64_to_bf16(float.fromhex("0x1.ffp127")) == 0x7F80   # tie -> even (inf)
    assert oracle.f64_to_bf16(0.0) == 0x0000
    assert oracle.f64_to_bf16(-0.0) == 0x8000


def test_f64_to_bf16_is_the_nearest_value_by_brute_force():
    # against the definition: among all finite bf16 patterns of the value's
    # sign, the one nearest to v (exact rational distances), ties to an even
    # last bit
    from fractions import Fraction
    pos = np.arange(0x0000, 0x7F80, dtype=np.uint32)
    vals = [Fraction(float(v)) for v in (pos << 16).view(np.float32)]
    rng = np.random.default_rng(17)
    cases = list(rng.uniform(0.5, 4.0, 300)) + list(2.0 ** rng.uniform(-135, 127, 300))
    # values exactly on and next to ties
    for b in rng.integers(1, 0x7F7F, 200):
        lo, hi = vals[b], vals[b + 1]
        mid = (lo + hi) / 2
        cases += [float(mid), float(mid) * (1 + 2.0 ** -40), float(mid) * (1 - 2.0 ** -40)]
    import bisect
    for v in cases:
        fv = Fraction(v)
        i = bisect.bisect_left(vals, fv)
        cand = [j for j in (i - 1, i) if 0 <= j < len(vals)]
        best = min(cand, key=lambda j: (abs(vals[j] - fv), j & 1))
        assert oracle.f64_to_bf16(v) == best, (v, hex(best))


def test_rmsnorm_hand_worked():
    # r = (3, 4, 0, 0): mean r^2 = 25/4, rms = 2.5, x = (1.2, 1.6, 0, 0);
    # bf16(1.2) = 1.203125 (0x3F9A), bf16(1.6) = 1.6015625 (0x3FCD) by hand
    x = oracle.rmsnorm_bf16(np.array([3.0, 4.0, 0.0, 0.0], np.float32))
    assert x.tolist() == [0x3F9A, 0x3FCD, 0, 0]


def test_rmsnorm_constant_and_sign():
    # a constant vector c has rms |c|: x = sign(c) / sqrt(1 + eps / c^2) -> +-1.0 in bf16
    for c in (2.5, -0.75, 1000.0):
        x = oracle.rmsnorm_bf16(np.full(256, c, np.float32))
        assert set(x.tolist()) == {0x3F80 if c > 0 else 0xBF80}


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(7)
    r = (rng.standard_normal(4096) * 37.0).astype(np.float32)
    x = synth.bf16_to_f32(oracle.rmsnorm_bf16(r)).astype(np.float64)
    # mean of x^2 is 1 up to the bf16 rounding of each element (< 2^-8 relative)
    assert abs(np.mean(x * x) - 1.0) < 2.0 ** -8
    # the norm removes a positive scale (up to eps and ties: at most one bf16 ulp)
    x8 = synth.bf16_to_f32(oracle.rmsnorm_bf16(r * np.float32(8.0))).astype(np.float64)
    assert np.all(np.abs(x8 - x) <= np.abs(x) * 2.0 ** -7 + 1e-30)
    # and equals the direct definition, element by element, before rounding
    ref = r.astype(np.float64) / math.sqrt(np.mean(r.astype(np.float64) ** 2) + oracle.RMS_EPS)
    assert np.all(np.abs(x - ref) <= np.abs(ref) * 2.0 ** -8)


def test_residual_layer_is_norm_then_layer_then_add():
    d, router, blobs, shared, _ = _layer_inputs(E=8, K=4, T=2)
    rng = np.random.default_rng(3)
    r = (rng.standard_normal((2, 256)) * 5.0).astype(np.float32)
    r_out, x, y, ids, w, _, _ = oracle.residual_layer(d, router, blobs, shared, r)
    np.testing.assert_array_equal(x, oracle.rmsnorm_bf16(r))
    y2, ids2, _, _, _ = oracle.layer(d, router, blobs, shared, x)
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(r_out, r.astype(np.float64) + y2)


def test_residual_layer_with_zero_experts_keeps_the_residual():
    # s = z = 0 in every matrix: every expert outputs 0, so r_out = r exactly
    d, router, _, _, _ = _layer_inputs(E=8, K=4, T=1)
    zero = blobkit.constant_blob(256, 256, 4, 9, 0.0, 0.0)
    r = np.linspace(-3, 3, 256, dtype=np.float32)[None]
    r_out, _, y, _, _, _, _ = oracle.residual_layer(d, router, {e: zero for e in range(8)}, zero, r)
    assert np.all(y == 0.0)
    np.testing.assert_array_equal(r_out, r.astype(np.float64))


def test_threads_do_not_change_results():
    # output rows on several threads: every row is the same sequential sum
    d, router, blobs, shared, x = _layer_inputs(E=8, K=4, T=2)
    try:
        oracle.set_threads(1)
        y1, ids1, w1, l1, g1 = oracle.layer(d, router, blobs, shared, x)
        oracle.set_threads(4)
        assert oracle.get_threads() == 4
        y4, ids4, w4, l4, g4 = oracle.layer(d, router, blobs, shared, x)
    finally:
        oracle.set_threads(1)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(l1, l4)
    np.testing.assert_array_equal(ids1, ids4)
