"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values printed on the
pages (fixtures under tests/golden/, each with its citation), library routines that
compute the same thing (torch's float8_e4m3fn, numpy's stable argsort and matmul),
brute force over all candidates, closed forms and invariants. Each is chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a transposed
operand, a wrong tie rule) fails at least one of them.
"""
import itertools
import os

import numpy as np
import pytest
import torch

import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line)
    return out


# ---------------------------------------------------------------- E2M1 --------------------
def test_e2m1_decode_matches_page_grid(orc):
    grid = {int(a): float(b) for a, b in (r.split() for r in _rows("e2m1_grid.txt"))}
    for c in range(16):
        mag = grid[c & 7]
        expect = -mag if (c & 8) else mag
        assert orc.e2m1_decode(c) == expect, c


def test_e2m1_encode_is_nearest_on_dense_sweep(orc):
    grid = np.array(sorted({abs(orc.e2m1_decode(c)) for c in range(8)}))
    xs = np.concatenate([np.linspace(-8, 8, 20001, dtype=np.float32),
                         np.float32([1e-30, -1e-30, 7.999, 100.0, -100.0, 6.0, -6.0])])
    for x in xs:
        c = orc.e2m1_encode(x)
        got = orc.e2m1_decode(c)
        best = np.min(np.abs(np.concatenate([grid, -grid]) - float(x)))
        assert abs(got - float(x)) == pytest.approx(best, abs=0), (x, c)
        # the sign follows the input, and zero is never negative
        if got != 0:
            assert np.sign(got) == np.sign(x)
        else:
            assert c == 0


def test_e2m1_ties_follow_stated_reading(orc):
    for r in _rows("e2m1_ties.txt"):
        v, code = r.split()
        assert orc.e2m1_encode(float(v)) == int(code), v


def test_e2m1_saturates_for_any_magnitude(orc):
    # every magnitude past 5 is nearest to 6 (code 7), however large, also where the distances to 4 and
    # to 6 are not separable in double precision; NaN encodes to 0 (no comparison holds)
    for x in (5.0000005, 6.0, 7.0, 1e10, 2.0 ** 54, 2.0 ** 60, 1e30, 3.4e38, float("inf")):
        assert orc.e2m1_encode(x) == 7, x
        assert orc.e2m1_encode(-x) == 15, x
    assert orc.e2m1_encode(float("nan")) == 0


def test_e2m1_idempotent_and_monotone(orc):
    for c in range(16):
        want = 0 if c == 8 else c
        assert orc.e2m1_encode(orc.e2m1_decode(c)) == want
    xs = np.linspace(-7, 7, 5001, dtype=np.float32)
    vals = [orc.e2m1_decode(orc.e2m1_encode(x)) for x in xs]
    assert all(a <= b for a, b in zip(vals, vals[1:]))
    assert orc.e2m1_encode(-0.0) == 0 and orc.e2m1_encode(-0.2) == 0


# ---------------------------------------------------------------- E4M3 --------------------
def test_e4m3_decode_matches_torch_float8_e4m3fn(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = orc.e4m3_decode(c)
        if np.isnan(ref[c]):
            assert np.isnan(got), c
        else:
            assert got == ref[c], c


def test_e4m3_max_is_page_value(orc):
    facts = dict(r.split() for r in _rows("e4m3_facts.txt"))
    finite = [orc.e4m3_decode(c) for c in range(128) if not np.isnan(orc.e4m3_decode(c))]
    assert max(finite) == float(facts["e4m3_max"])
    assert orc.e4m3_decode(0x7E) == 448.0
    assert max(abs(orc.e2m1_decode(c)) for c in range(16)) == float(facts["e2m1_max"])


def test_e4m3_encode_matches_torch_rounding(orc):
    rng = np.random.default_rng(0)
    # log-uniform over the whole finite range plus exact midpoints between adjacent codes
    xs = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 20000)).astype(np.float32)
    vals = np.array([orc.e4m3_decode(c) for c in range(0x7F)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    xs = np.concatenate([xs, mids, np.float32([0.0, 448.0, 2.0 ** -9, 2.0 ** -10, 2.0 ** -6])])
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, r in zip(xs, ref):
        assert orc.e4m3_encode(x) == r, x
    # saturation (the reading): anything above 448 stays at 448
    assert orc.e4m3_encode(460.0) == 0x7E and orc.e4m3_encode(1e30) == 0x7E


# ----------------------------------------------------- Eq. 5 scales and the quantizer ------
def test_global_scale_closed_form(orc):
    for amax in [1.0, 6.0, 0.02345, 123.456, 3e-5]:
        g = orc.global_scale(amax)
        assert g == pytest.approx(448.0 * 6.0 / amax, rel=1e-6)
    assert orc.global_scale(0.0) == 1.0


@pytest.mark.parametrize("dist", ["normal", "student_t"])
def test_quantizer_pins(orc, dist):
    T, K = 64, 512
    x = gen.normal(5, 99, T * K) if dist == "normal" else gen.student_t(5, 99, T * K)
    x = x.reshape(T, K)
    g = orc.global_scale_of(x)
    q, s = orc.quantize_rows(x, g)
    # Eq. 5: the block holding the tensor amax gets the largest scale code and its max element -> +-6
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert s[r, c // 32] == 0x7E
    code = (q[r, c // 2] >> (4 * (c % 2))) & 15
    assert code & 7 == 7
    assert (code >> 3) == (1 if x[r, c] < 0 else 0)
    # dequantized value = e2m1 * e4m3 / gamma is within half a grid step of x (no saturation below amax)
    deq = orc.dequant(q, s) / np.float64(g)
    sv = np.array([orc.e4m3_decode(v) for v in range(256)])[s].repeat(32, axis=1) / np.float64(g)
    mags = np.abs(orc.dequant(q, s) / sv.clip(1e-300) / np.float64(g))
    err = np.abs(deq - x.astype(np.float64))
    assert np.all(err <= sv * 1.0 + 1e-12)  # never more than one full step
    nz = sv > 0
    # nearest-point property: error <= half the spacing of the two grid points around x/s
    xs = np.abs(x.astype(np.float64)[nz] / sv[nz])
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    nearest = np.min(np.abs(xs[:, None] - grid[None, :]), axis=1)
    assert np.allclose(np.abs(mags[nz] - xs), nearest, atol=1e-5 * 6)


def test_quantizer_zero_block_and_underflow(orc):
    x = np.zeros((2, 64), np.float32)
    x[1, 40] = 1000.0
    x[1, 0] = 1e-7  # tiny block: scale underflows -> all codes 0
    g = orc.global_scale_of(x)
    q, s = orc.quantize_rows(x, g)
    assert np.all(q[0] == 0) and np.all(s[0] == 0)
    assert s[1, 0] == 0 and np.all(q[1, :16] == 0)
    assert s[1, 1] == 0x7E


# ----------------------------------------------------------------- pruning ----------------
PATTERNS = [p for p in itertools.combinations(range(4), 2)]


def test_six_patterns():
    # paper Section 3.2: paired 4:8 has m = 8 and P = 6 admissible patterns
    assert len(PATTERNS) == 6


def test_prune_keeps_max_energy_pattern(orc):
    rng = np.random.default_rng(1)
    w = rng.standard_normal((64, 256)).astype(np.float32)
    w[0, :8] = [1, 1, 1, 1, 0, 0, 0, 0]  # tie: pairs 0 and 1 equal, kept by the lower-index rule
    w[1, :8] = [0, 0, 3, 0, 0, 0, 0, 3]
    p = orc.prune_paired48(w)
    for r in range(w.shape[0]):
        for g in range(w.shape[1] // 8):
            x = w[r, 8 * g:8 * g + 8].astype(np.float64)
            y = p[r, 8 * g:8 * g + 8]
            nrm = [x[2 * i] ** 2 + x[2 * i + 1] ** 2 for i in range(4)]
            best = max(nrm[a] + nrm[b] for a, b in PATTERNS)
            kept = [i for i in range(4) if np.any(y[2 * i:2 * i + 2] != 0)]
            assert len(kept) <= 2
            assert sum(nrm[i] for i in kept) == pytest.approx(best, rel=1e-12, abs=0)
            for i in range(4):  # kept pairs unchanged, others zero
                if i in kept:
                    assert np.array_equal(y[2 * i:2 * i + 2], w[r, 8 * g + 2 * i:8 * g + 2 * i + 2])
    assert np.array_equal(p[0, :8], np.float32([1, 1, 1, 1, 0, 0, 0, 0]))
    assert np.count_nonzero(p[1, :8]) == 2


# ------------------------------------------------------- pair-bitmask storage -------------
def test_pair_bitmask_worked_examples(orc):
    for r in _rows("pair_bitmask_examples.txt"):
        d, pk, m = (part.strip() for part in r.split("|"))
        dense = np.array([int(v, 16) for v in d.split()], np.uint8)[None, :]
        packed, mask = orc.pack(dense)
        assert packed[0].tolist() == [int(v, 16) for v in pk.split()]
        assert mask[0, 0] == int(m, 16)
        assert np.array_equal(orc.unpack(packed, mask), dense)


def _random_valid_dense(rng, rows, K):
    dense = np.zeros((rows, K // 2), np.uint8)
    for r in range(rows):
        for c in range(K // 8):
            keep = PATTERNS[rng.integers(6)]
            for i in keep:
                dense[r, 4 * c + i] = rng.integers(0, 256)  # may be 0: exercises the tie rule
    return dense


def test_pack_roundtrip_and_mask_invariant(orc):
    rng = np.random.default_rng(2)
    dense = _random_valid_dense(rng, 32, 512)
    packed, mask = orc.pack(dense)
    assert np.array_equal(orc.unpack(packed, mask), dense)
    nibs = np.concatenate([mask & 15, mask >> 4], axis=None)
    assert set(np.unique(nibs).tolist()) <= {0x3, 0x5, 0x6, 0x9, 0xA, 0xC}
    # canonical form: pack(unpack(S)) == S
    p2, m2 = orc.pack(orc.unpack(packed, mask))
    assert np.array_equal(p2, packed) and np.array_equal(m2, mask)


def test_pack_rejects_three_nonzero_bytes_and_bad_nibbles(orc):
    dense = np.zeros((1, 16), np.uint8)
    dense[0, :3] = [1, 2, 3]
    with pytest.raises(orc.OracleError):
        orc.pack(dense)
    packed = np.zeros((1, 8), np.uint8)
    mask = np.array([[0x37, 0x33]], np.uint8)  # nibble 7 has three bits
    with pytest.raises(orc.OracleError):
        orc.unpack(packed, mask)


def test_storage_bits_per_weight(orc):
    bits = float(dict(r.split() for r in _rows("storage_bits.txt"))["bits_per_weight"])
    N, K = 64, 256
    w = gen.normal(3, 7, N * K, 0.02).reshape(1, N, K)
    W = orc.compress(w)
    nbytes = W["packed"].nbytes + W["mask"].nbytes + W["scale"].nbytes
    assert nbytes * 8 / (N * K) == bits


# ------------------------------------------------------------ compression -----------------
def test_compress_feasible_set_and_error(orc):
    E, N, K = 2, 32, 256
    w = gen.normal(11, 12, E * N * K, 0.02).reshape(E, N, K)
    W = orc.compress(w)
    pr = orc.prune_paired48(w)
    for e in range(E):
        # Eq. 5 tensor scale of the pruned weights
        assert W["gscale"][e] == orc.global_scale(np.abs(pr[e]).max())
        deq = orc.dequant_weights(W, e) / np.float64(W["gscale"][e])
        # Eq. 6: every 8-group matches one admissible pattern (the zero pattern of S)
        z = deq.reshape(N, K // 8, 4, 2)
        assert np.all((np.abs(z).sum(-1) != 0).sum(-1) <= 2)
        assert np.all(deq[pr[e] == 0] == 0)
        # values: block-relative error of the quantizer
        rel = np.linalg.norm(deq - pr[e]) / np.linalg.norm(pr[e])
        assert rel < 0.12
        # each 32-block's values lie on s_b * G (UE4M3 scale times the E2M1 grid)
        dense = orc.unpack(W["packed"][e], W["mask"][e])
        codes = np.stack([dense & 15, dense >> 4], -1).reshape(N, K)
        grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
        sb = np.array([orc.e4m3_decode(v) for v in range(256)])[W["scale"][e]].repeat(32, axis=1)
        assert np.allclose(orc.dequant_weights(W, e), np.where(codes & 8, -1, 1) * grid[codes & 7] * sb)


# ---------------------------------------------------------------- routing -----------------
def test_route_matches_stable_argsort(orc):
    ids, _ = gen.route_zipf(4, 300, 16, 4, 1.1, 3)
    R = orc.route(ids, 16)
    flat = ids.ravel()
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(R["sorted_slot"], order)
    assert np.array_equal(R["counts"], np.bincount(flat, minlength=16))
    assert np.array_equal(R["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=16))]))
    assert np.array_equal(R["slot_pos"][R["sorted_slot"]], np.arange(flat.size))
    assert R["counts"][np.setdiff1d(np.arange(16), np.unique(flat))].sum() == 0


def test_route_rejects_out_of_range(orc):
    with pytest.raises(orc.OracleError):
        orc.route(np.array([[0, 5]], np.int32), 4)


def test_dispatch_quantize_equals_quantize_of_gathered_rows(orc):
    T, K, E, k = 40, 128, 6, 3
    x = gen.student_t(8, 1, T * K).reshape(T, K)
    ids, _ = gen.route_uniform(8, T, E, k)
    R = orc.route(ids, E)
    gam = np.array([orc.global_scale_of(x) * f for f in (1, 0.5, 2, 1, 0.25, 4)], np.float32)
    q, s = orc.dispatch_quantize(x, R["sorted_slot"], k, R["offsets"], gam)
    tok = R["sorted_slot"] // k
    ex = np.repeat(np.arange(E), R["counts"])
    q2, s2 = orc.quantize_rows(x[tok], gam, ex)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


# ------------------------------------------------------------------- GEMM -----------------
def _small_problem(orc, E=3, N=48, K=128, T=20, k=2, seed=21):
    w = gen.normal(seed, 1, E * N * K, 0.02).reshape(E, N, K)
    W = orc.compress(w)
    x = gen.normal(seed, 2, T * K).reshape(T, K)
    ids, _ = gen.route_uniform(seed, T, E, k)
    R = orc.route(ids, E)
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    q, s = orc.dispatch_quantize(x, R["sorted_slot"], k, R["offsets"], ga)
    return W, q, s, ga, R


def test_grouped_gemm_vs_numpy_matmul(orc):
    W, q, s, ga, R = _small_problem(orc)
    y = orc.grouped_gemm(W, q, s, ga, R["offsets"])
    X = orc.dequant(q, s)
    off = R["offsets"]
    for e in range(W["E"]):
        Wd = orc.dequant_weights(W, e)
        ref = X[off[e]:off[e + 1]] @ Wd.T / (np.float64(W["gscale"][e]) * np.float64(ga[e]))
        assert np.allclose(y[off[e]:off[e + 1]], ref, rtol=1e-12, atol=1e-12)
    # row subsets give the same rows
    rl = np.array([off[-1] - 1, 0, 3], np.int64)
    assert np.array_equal(orc.grouped_gemm(W, q, s, ga, off, rl), y[rl])


def test_grouped_gemm_one_hot_activation_reads_weight_column(orc):
    W, q, s, ga, R = _small_problem(orc)
    # activation row with a single nonzero E2M1 code (1.0 at column 37, scale code 1.0)
    q1 = np.zeros_like(q)
    s1 = np.zeros_like(s)
    q1[:, 37 // 2] = 2 << 4  # column 37 is odd -> high nibble; code 2 = 1.0
    s1[:, 37 // 32] = 0x38  # E4M3 1.0
    y = orc.grouped_gemm(W, q1, s1, ga, R["offsets"])
    off = R["offsets"]
    for e in range(W["E"]):
        col = orc.dequant_weights(W, e)[:, 37] / (np.float64(W["gscale"][e]) * np.float64(ga[e]))
        for p in range(off[e], off[e + 1]):
            assert np.array_equal(y[p], col)


# ------------------------------------------- split gate / up tensor scales (model card) ------
def test_split_scales_power_of_two_halves(orc):
    """Up half = 8 x gate half: each linear's Eq. 5 scale absorbs the factor exactly, so the codes of
    the two halves are identical, gamma_up = gamma_gate / 8 and the up outputs are 8 x the gate
    outputs; each half also equals the matmul definition with its own scale."""
    rng = np.random.default_rng(31)
    E, N, K = 3, 64, 256
    g = (rng.standard_normal((E, N // 2, K)) * 0.02).astype(np.float32)
    w = np.concatenate([g, g * np.float32(8.0)], axis=1)
    W = orc.compress_split(w)
    assert W["gscale"].shape == (E, 2)
    assert np.array_equal(W["gscale"][:, 1] * np.float32(8.0), W["gscale"][:, 0])
    for key in ("packed", "mask", "scale"):
        assert np.array_equal(W[key][:, :N // 2], W[key][:, N // 2:]), key
    x = rng.standard_normal((24, K)).astype(np.float32)
    ids = np.stack([rng.choice(E, 2, replace=False) for _ in range(12)]).astype(np.int32)
    R = orc.route(ids, E)
    ga = np.full(E, orc.global_scale_of(x[:12]), np.float32)
    q, s = orc.dispatch_quantize(x[:12], R["sorted_slot"], 2, R["offsets"], ga)
    y = orc.grouped_gemm(W, q, s, ga, R["offsets"])
    assert y.shape == (24, N)
    assert np.array_equal(y[:, N // 2:], 8.0 * y[:, :N // 2])
    X = orc.dequant(q, s)
    off = R["offsets"]
    for h, Wh in enumerate(orc.split_halves(W)):
        for e in range(E):
            ref = X[off[e]:off[e + 1]] @ orc.dequant_weights(Wh, e).T / (np.float64(W["gscale"][e, h]) * np.float64(ga[e]))
            assert np.allclose(y[off[e]:off[e + 1], h * (N // 2):(h + 1) * (N // 2)], ref, rtol=1e-12, atol=1e-12)


def test_split_scales_equal_amax_reduce_to_one_scale(orc):
    """Halves with the same tensor amax: the split compression and GEMM equal the single-scale ones."""
    rng = np.random.default_rng(32)
    E, N, K = 2, 64, 256
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    w[:, 3, 5] = 0.5
    w[:, N // 2 + 7, 9] = -0.5
    Ws, W1 = orc.compress_split(w), orc.compress(w)
    for key in ("packed", "mask", "scale"):
        assert np.array_equal(Ws[key], W1[key]), key
    assert np.array_equal(Ws["gscale"][:, 0], W1["gscale"]) and np.array_equal(Ws["gscale"][:, 1], W1["gscale"])
    x = rng.standard_normal((8, K)).astype(np.float32)
    ids = np.array([[0, 1]] * 8, np.int32)
    R = orc.route(ids, E)
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    q, s = orc.dispatch_quantize(x, R["sorted_slot"], 2, R["offsets"], ga)
    assert np.array_equal(orc.grouped_gemm(Ws, q, s, ga, R["offsets"]), orc.grouped_gemm(W1, q, s, ga, R["offsets"]))


# ----------------------------------------------------------- SwiGLU / combine ---------------
def test_swiglu_closed_form(orc):
    from scipy.special import expit
    rng = np.random.default_rng(3)
    y13 = rng.standard_normal((7, 10)) * 4
    h = orc.swiglu(y13)
    g, u = y13[:, :5], y13[:, 5:]
    assert np.allclose(h, g * expit(g) * u, rtol=1e-14)
    z = np.zeros((1, 4))
    z[0, 2:] = 5.0
    assert np.all(orc.swiglu(z) == 0.0)


def test_combine_special_cases(orc):
    T, k, H = 9, 3, 16
    rng = np.random.default_rng(4)
    ids = np.stack([rng.permutation(5)[:k] for _ in range(T)]).astype(np.int32)
    R = orc.route(ids, 5)
    row = rng.standard_normal(H)
    y = np.tile(row, (T * k, 1))  # identical expert outputs
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    out = orc.combine(y, R["slot_pos"], w)
    assert np.allclose(out, np.outer(w.astype(np.float64).sum(1), row), rtol=1e-12)
    y2 = rng.standard_normal((T * k, H))
    out2 = orc.combine(y2, R["slot_pos"], w)
    ref = np.einsum("tj,tjh->th", w.astype(np.float64), y2[R["slot_pos"].reshape(T, k)])
    assert np.allclose(out2, ref, rtol=1e-12)


def test_mlp_chain_matches_step_by_step(orc):
    cfg = gen.CONFIGS["t_mlp"]
    H, I2, I = cfg.K, cfg.N, cfg.N // 2
    w13 = np.stack([gen.weights_expert(cfg, 0, e, I2, H) for e in range(cfg.E)])
    w2 = np.stack([gen.weights_expert(cfg, 1, e, H, I) for e in range(cfg.E)])
    W13, W2 = orc.compress(w13), orc.compress(w2)
    x = gen.activations(cfg, 0, cfg.T, H)
    ids, wts = gen.routing(cfg)
    R = orc.route(ids, cfg.E)
    ga = np.full(cfg.E, orc.global_scale_of(x), np.float32)
    q, s = orc.dispatch_quantize(x, R["sorted_slot"], cfg.k, R["offsets"], ga)
    gh = np.full(cfg.E, orc.global_scale(20.0), np.float32)
    M = orc.expert_mlp(W13, W2, q, s, ga, gh, R["offsets"])
    y13 = orc.grouped_gemm(W13, q, s, ga, R["offsets"])
    assert np.array_equal(M["y13"], y13)
    h = orc.swiglu(y13)
    ex = np.repeat(np.arange(cfg.E), R["counts"])
    hq, hs = orc.quantize_rows(h.astype(np.float32), gh, ex)
    assert np.array_equal(M["hq"], hq) and np.array_equal(M["hs"], hs)
    y2 = orc.grouped_gemm(W2, hq, hs, gh, R["offsets"])
    assert np.array_equal(M["y2"], y2)
    # the requantized h is close to h (NVFP4 relative error)
    assert orc.rel_frobenius(orc.dequant(hq, hs) / np.float64(gh[0]), h) < 0.12


# ---------------------------------------------------------------- dense NVFP4 control ------
def test_dense_gemm_on_unpacked_sparse_weights_equals_sparse_gemm(orc):
    """The dense control computes the same product as the sparse GEMM when its weights are the
    sparse weights written out densely (model card round trip: unpack gives dense NVFP4 bytes)."""
    cfg = gen.CONFIGS["c0"]
    w = np.stack([gen.weights_expert(cfg, 0, e, cfg.N, cfg.K) for e in range(cfg.E)])
    W = orc.compress(w)
    Wd = dict(codes=orc.unpack(W["packed"], W["mask"]), scale=W["scale"], gscale=W["gscale"], E=cfg.E, N=cfg.N,
              K=cfg.K)
    x = gen.activations(cfg, 0, cfg.T, cfg.K)
    ids, _ = gen.routing(cfg)
    R = orc.route(ids, cfg.E)
    ga = np.full(cfg.E, orc.global_scale_of(x), np.float32) * np.linspace(0.5, 2.0, cfg.E).astype(np.float32)
    q, s = orc.dispatch_quantize(x, R["sorted_slot"], cfg.k, R["offsets"], ga)
    ys = orc.grouped_gemm(W, q, s, ga, R["offsets"])
    yd = orc.dense_grouped_gemm(Wd, q, s, ga, R["offsets"])
    assert orc.rel_frobenius(yd, ys) < 1e-12


def test_dense_compress_and_one_hot_column(orc):
    """Dense compression keeps every weight (no pruning): the block holding the tensor amax gets the
    largest scale code 448 (Eq. 5), the reconstruction error is the quantizer's, and a one-hot
    activation reads back one dequantized weight column."""
    rng = np.random.default_rng(5)
    E, N, K = 2, 64, 256
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    Wd = orc.compress_dense(w)
    for e in range(E):
        r, c = np.unravel_index(np.argmax(np.abs(w[e])), w[e].shape)
        assert Wd["scale"][e, r, c // 32] == 0x7E
        deq = orc.dequant(Wd["codes"][e], Wd["scale"][e]) / np.float64(Wd["gscale"][e])
        assert np.count_nonzero(deq) > 0.9 * N * K                  # dense: no paired-4:8 zeros
        assert orc.rel_frobenius(deq, w[e]) < 0.12
    # one token routed to expert 1 whose activation is 1.0 at K index 37 and 0 elsewhere
    x = np.zeros((1, K), np.float32)
    x[0, 37] = 1.0
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    q, s = orc.quantize_rows(x, ga[0])
    y = orc.dense_grouped_gemm(Wd, q, s, ga, np.array([0, 0, 1]))
    col = orc.dequant(Wd["codes"][1], Wd["scale"][1])[:, 37] / np.float64(Wd["gscale"][1])
    assert np.allclose(y[0], col, rtol=1e-12, atol=0)
