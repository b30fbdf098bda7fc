"""GPU parity of every step of the path against the CPU oracle, through the C ABI binding.

Bars: bit-exact for packing, permutation, quantized codes and scales; rel-Frobenius <= 1e-3 for
fp32 GEMM outputs against the fp64 oracle on identical operands; bf16 outputs against the oracle
rounded to bf16 (the only difference is fp32 accumulation order, far below 1e-3)."""
import numpy as np
import pytest
import torch

import gen
import oracle as orc

from gpu_cases import (DEV, OracleWeights, dev, device_weights, gamma_h_table, host, sample_expert_rows,
                       sample_rows, sample_tile_rows, say, single_case)

pytestmark = pytest.mark.gpu

mq = pytest.importorskip("sparse_precision_grouped_amd")

GEMM_TOL = 1e-3   # relative Frobenius error of a GEMM output block against the fp64 oracle
ROW_TOL = 1e-5    # relative error of every single fp32 output row: a few wrong elements in one row fail
                  # here even where the block's norm would hide them (fp32 accumulation alone: ~1e-7)


def bf16_round(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def gemm_gate(got, ref, what="gemm"):
    """fp32 GEMM outputs against the fp64 oracle: the block's rel-Frobenius error <= GEMM_TOL and each
    row's own relative error <= ROW_TOL (a row whose reference is zero must be zero)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = orc.rel_frobenius(got, ref)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    nz = den > 0
    row = float((num[nz] / den[nz]).max()) if nz.any() else 0.0
    say(what, "rel-Frobenius %.3g, max row %.3g, rows %d" % (err, row, got.shape[0]))
    assert np.all(num[~nz] == 0), what
    assert err <= GEMM_TOL, what
    assert row <= ROW_TOL, what
    return err


def rows_of(t, rows):
    """Rows of a device tensor, gathered on the device and copied to the host."""
    return host(t.index_select(0, torch.from_numpy(np.asarray(rows, np.int64)).to(t.device)))


def requant_gate(ws, rows_all, I, gh, rows, experts, M=None):
    """The fused SwiGLU + requantization against the oracle's quantizer (paper Section 3.4, Eq. 3 + 5;
    Appendix D.1): on the fp32 h the kernel itself requantized (F_DUMP_H), the h codes, block scales and
    the f16 operand copy must be byte-identical to the oracle's. With M (the oracle's own chain on the
    same rows), the kernel's h must also match the oracle's fp64 h within GEMM_TOL; the fraction of h
    codes that differ from the oracle's chain (rounding-boundary flips) is returned as a reported number."""
    hq, hs, _ = mq.mlp_workspace_views(ws, rows_all, I, dump=True)
    hk, h = mq.mlp_h_views(ws, rows_all, I)
    h_g = rows_of(h, rows)
    qo, so = orc.quantize_rows(h_g, gh, experts)
    hq_g, hs_g = rows_of(hq, rows), rows_of(hs, rows)
    assert np.array_equal(hq_g, qo), "h codes"
    assert np.array_equal(hs_g, so), "h block scales"
    assert np.array_equal(rows_of(hk, rows).view(np.uint16), _xk_reference(qo, so).view(np.uint16)), "h f16 copy"
    say("requantized h: codes, scales and f16 copy of %d rows byte-identical to the oracle's quantizer" % len(rows))
    if M is None:
        return None
    e_h = orc.rel_frobenius(h_g, M["h"])
    flips = float(np.mean(orc.dequant(hq_g, hs_g) != orc.dequant(M["hq"], M["hs"])))
    say("h rel-Frobenius vs the oracle's fp64 h %.3g; h codes differing from the oracle's chain: %.2e" % (e_h, flips))
    assert e_h <= GEMM_TOL
    return flips


def h_row_absmax(ws, rows_all, I, rows):
    """max |h| of each given row of the dumped fp32 h (a max: exact however it is computed)."""
    _, h = mq.mlp_h_views(ws, rows_all, I)
    idx = torch.from_numpy(np.asarray(rows, np.int64)).to(h.device)
    return host(h.index_select(0, idx).abs().amax(dim=1))


def calibration_gate(gcal, acal, row_absmax, experts, E, gh_oracle=None):
    """MOESQ_F_CALIBRATE against the kernel's own fp32 h (F_DUMP_H of the same kernel family, all rows):
    amax_h[e] is the largest |h| over expert e's rows exactly (0 without rows) and gamma_h[e] is Eq. 5
    of it exactly; against the oracle's scale from its fp64 h within 1e-5 (a max moves by at most the
    error of h)."""
    gcal, acal = host(gcal), host(acal)
    ref = np.zeros(E, np.float32)
    np.maximum.at(ref, np.asarray(experts), np.asarray(row_absmax, np.float32))
    assert np.array_equal(acal, ref), "amax_h"
    for e in range(E):
        assert gcal[e] == np.float32(orc.global_scale(float(acal[e]))), e
    if gh_oracle is not None:
        has = np.bincount(np.asarray(experts), minlength=E) > 0
        rel = np.abs(gcal[has].astype(np.float64) / gh_oracle[has] - 1.0)
        say("calibrated gamma_h vs the oracle's: max rel %.3g over %d experts" % (rel.max(), has.sum()))
        assert rel.max() <= 1e-5


def oracle_gamma_h(W13o, qo, so, ga, off):
    """The oracle's per-expert intermediate scale: Eq. 5 over the largest |h| (fp32) of each expert's
    rows, h from its own gate_up GEMM and SwiGLU (the reading the workloads use)."""
    h = orc.swiglu(orc.grouped_gemm(W13o, qo, so, ga, off)).astype(np.float32)
    E = len(off) - 1
    amax = np.zeros(E, np.float32)
    np.maximum.at(amax, orc.expert_of_rows(off, np.arange(h.shape[0])), np.abs(h).max(axis=1))
    return np.array([orc.global_scale(float(a)) for a in amax], np.float32)


# ---------------------------------------------------------------- generator ------------------
def test_gen_device_bitexact():
    say("gen device vs host")
    n = 1 << 20
    out = torch.empty(n, dtype=torch.float32, device=DEV)
    gen.gpu_fill_normal(out, 99, gen.weight_stream(0, 3), 0.02, start=12345)
    assert np.array_equal(host(out), gen.normal(99, gen.weight_stream(0, 3), n, 0.02, start=12345))
    out2 = torch.empty(1 << 16, dtype=torch.float32, device=DEV)
    gen.gpu_fill_student_t(out2, 7, gen.act_stream(1), 4)
    assert np.array_equal(host(out2), gen.student_t(7, gen.act_stream(1), 1 << 16, 4))


# ---------------------------------------------------------------- compression ----------------
@pytest.mark.parametrize("name,proj", [("c0", 0), ("t_mlp", 0), ("t_mlp", 1), ("c1", 0)])
def test_compress_bitexact(name, proj):
    c = single_case(name, proj) if proj == 0 else None
    if c is None:
        cfg = gen.CONFIGS[name]
        E, N, K = cfg.E, cfg.N2, cfg.K2
        w = np.stack([gen.weights_expert(cfg, 1, e, N, K) for e in range(E)])
        Wd = mq.moesq_compress_weights(dev(w))
        W = orc.compress(w)
    else:
        Wd, Wo = c["Wd"], c["Wo"]
        W = Wo.as_dict()
    say("compress", name, proj)
    assert np.array_equal(host(Wd.gscale), W["gscale"])
    assert np.array_equal(host(Wd.scale), W["scale"])
    assert np.array_equal(host(Wd.mask), W["mask"])
    assert np.array_equal(host(Wd.packed), W["packed"])


def test_compress_edge_patterns():
    """Zero groups, pairs that quantize to 0x00 (pack tie rule), ties in pair norms, and a tiny block
    whose scale underflows."""
    say("compress edge patterns")
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((2, 64, 256)) * 0.02).astype(np.float32)
    w[0, 0, :32] = 0.0                          # all-zero block
    w[0, 1, :8] = [1e-9, 1e-9, 0.3, 0.3, 0, 0, 0.3, 0.3]  # kept pair far below the block scale -> 0x00
    w[0, 2, :8] = [0.1, 0.1, 0.1, 0.1, 0.1, 0.1, 0.1, 0.1]  # four equal pairs: lower two kept
    w[1, 3, 32:64] = 1e-12                      # underflowing scale
    w[1, 5, 100] = 1.0                          # tensor amax
    Wd = mq.moesq_compress_weights(dev(w))
    W = orc.compress(w)
    for key in ("packed", "mask", "scale"):
        assert np.array_equal(host(getattr(Wd, key)), W[key]), key
    assert np.array_equal(host(Wd.gscale), W["gscale"])
    dense = mq.moesq_unpack_weights(Wd)
    assert np.array_equal(host(dense), orc.unpack(W["packed"], W["mask"]))


def _kernel_layout_reference(packed, mask, scale):
    """The kernel weight layout built with numpy from its definition (a byte permutation plus the
    per-pair nibble interleave), independent of the device prepack: units of 4 fragments (64 rows)
    per 256-K super-step; lane l = 16c + r of fragment j owns packed bytes [1024 j + 16 l, +16),
    index codes [4096 + 16 l + 4 j, +4) and scale codes [5120 + 8 l + 2 j, +2)."""
    E, N, K4 = packed.shape
    K = K4 * 4
    nss = K // 256
    G = N // 64
    out = np.zeros((E, G, nss, 5632), np.uint8)
    pk = packed.reshape(E, N // 16, 16, nss, 4, 16)            # [e, rb, r, ss, c, 16 bytes]
    b0, b1 = pk[..., 0::2], pk[..., 1::2]
    sh = np.empty_like(pk)
    sh[..., 0::2] = (b0 & 15) | ((b1 & 15) << 4)
    sh[..., 1::2] = (b0 >> 4) | (b1 & 0xF0)
    frag = sh.transpose(0, 1, 3, 4, 2, 5).reshape(E, G, 4, nss, 1024)          # [e, g, j, ss, lane*16]
    out[..., :4096] = frag.transpose(0, 1, 3, 2, 4).reshape(E, G, nss, 4096)
    # mask nibbles -> pair-index codes i | j << 2, nibble order (g0, g2, g4, g6, g1, g3, g5, g7)
    code = np.zeros(16, np.uint32)
    for i, j in ((0, 1), (0, 2), (1, 2), (0, 3), (1, 3), (2, 3)):
        code[(1 << i) | (1 << j)] = i | (j << 2)
    mk = mask.reshape(E, N // 16, 16, nss, 4, 4).transpose(0, 1, 3, 4, 2, 5).astype(np.uint32)
    word = mk[..., 0] | (mk[..., 1] << 8) | (mk[..., 2] << 16) | (mk[..., 3] << 24)
    nib = [code[(word >> (4 * g)) & 15] for g in range(8)]
    order = [0, 2, 4, 6, 1, 3, 5, 7]
    cw = sum(nib[order[kk]] << np.uint32(4 * kk) for kk in range(8)).astype(np.uint32)
    cw = cw.reshape(E, G, 4, nss, 64).transpose(0, 1, 3, 4, 2)                  # [e, g, ss, lane, j]
    out[..., 4096:5120] = np.ascontiguousarray(cw).view(np.uint8).reshape(E, G, nss, 1024)
    sc = scale.reshape(E, N // 16, 16, nss, 4, 2).transpose(0, 1, 3, 4, 2, 5)  # [e, rb, ss, c, r, 2]
    sc = sc.reshape(E, G, 4, nss, 64, 2).transpose(0, 1, 3, 4, 2, 5)           # [e, g, ss, lane, j, 2]
    out[..., 5120:] = sc.reshape(E, G, nss, 512)
    return out.reshape(-1)


@pytest.mark.parametrize("name", ["c0", "t_zipf"])
def test_prepack_kernel_layout(name):
    c = single_case(name)
    say("prepack", name)
    Wd = c["Wd"]
    ref = _kernel_layout_reference(host(Wd.packed), host(Wd.mask), host(Wd.scale))
    assert np.array_equal(host(Wd.kl), ref)


def test_unpack_roundtrip_and_bad_nibble():
    c = single_case("c0")
    say("unpack c0")
    dense = mq.moesq_unpack_weights(c["Wd"])
    W = c["Wo"].as_dict()
    assert np.array_equal(host(dense), orc.unpack(W["packed"], W["mask"]))
    bad = mq.Weights(c["Wd"].packed.clone(), c["Wd"].mask.clone(), c["Wd"].scale, c["Wd"].gscale)
    bad.mask[0, 0, 0] = 0x37                          # nibble 7: three bits
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    mq.moesq_unpack_weights(bad, dev_status=st)
    assert int(host(st)[0]) == mq.ERR_PATTERN


# ---------------------------------------------------------------- routing --------------------
def _route_check(ids, E):
    rt = mq.moesq_route_permute(dev(ids.astype(np.int32)), E)
    R = orc.route(ids, E)
    for key in ("counts", "offsets", "sorted_slot", "slot_pos"):
        assert np.array_equal(host(rt[key]), R[key]), key
    return rt


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4", "t_zipf"])
def test_route_bitexact(name):
    cfg = gen.CONFIGS[name]
    say("route", name)
    ids, _ = gen.routing(cfg)
    _route_check(ids, cfg.E)


def test_route_edge_cases():
    say("route edges")
    _route_check(np.zeros((1, 1), np.int32), 4)                                    # T = 1, k = 1
    _route_check(np.full((3000, 1), 7, np.int32), 8)                               # all slots to one expert
    _route_check(np.tile(np.arange(8, dtype=np.int32), (2000, 1)), 384)            # 16000 slots, multi-block
    ids, _ = gen.route_zipf(3, 9000, 384, 8, 1.1, 0)                                # 72000 slots, uneven chunks
    _route_check(ids, 384)
    # ids out of range are dropped and reported
    ids = np.array([[0, 1], [5, 2], [1, -1]], np.int32)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    rt = mq.moesq_route_permute(dev(ids), 4, dev_status=st)
    assert int(host(st)[0]) == mq.ERR_INVALID_ARG
    sp = host(rt["slot_pos"])
    assert sp[2] == -1 and sp[5] == -1
    assert host(rt["offsets"])[-1] == 4
    assert np.array_equal(host(rt["counts"]), [1, 2, 1, 0])


# ---------------------------------------------------------------- activation quantization ----
@pytest.mark.parametrize("name", ["c0", "c1", "t_zipf", "t_mlp"])
def test_quantize_dispatch_bitexact(name):
    c = single_case(name)
    say("quantize", name)
    R, k = c["R"], c["k"]
    rt = mq.moesq_route_permute(dev(c["ids"]), c["E"])
    ga = c["ga"] * np.linspace(0.5, 2.0, c["E"]).astype(np.float32)   # distinct per-expert scales
    q, s = mq.moesq_quantize_act(dev(c["x"]), dev(ga), slot_pos=rt["slot_pos"], k=k, offsets=rt["offsets"])
    qo, so = orc.dispatch_quantize(c["x"], R["sorted_slot"], k, R["offsets"], ga)
    assert np.array_equal(host(q), qo)
    assert np.array_equal(host(s), so)


def _xk_reference(q, s):
    """The f16 operand copy from its definition: exact dequantized values, each 8-group stored in
    the order (0, 2, 4, 6, 1, 3, 5, 7)."""
    v = orc.dequant(q, s)
    R, K = v.shape
    g = v.reshape(R, K // 8, 8)[:, :, [0, 2, 4, 6, 1, 3, 5, 7]]
    return g.reshape(R, K).astype(np.float16)


@pytest.mark.parametrize("name", ["c0", "t_zipf"])
def test_quantize_f16_operand_copy(name):
    c = single_case(name)
    say("quantize xk", name)
    R, k = c["R"], c["k"]
    rt = mq.moesq_route_permute(dev(c["ids"]), c["E"])
    q, s, xk = mq.moesq_quantize_act(dev(c["x"]), dev(c["ga"]), slot_pos=rt["slot_pos"], k=k,
                                     offsets=rt["offsets"], xk=True)
    qo, so = orc.dispatch_quantize(c["x"], R["sorted_slot"], k, R["offsets"], c["ga"])
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    assert np.array_equal(host(xk).view(np.uint16), _xk_reference(qo, so).view(np.uint16))


def test_quantize_plain_and_bf16_and_zero():
    say("quantize plain / bf16 / zeros")
    x = gen.student_t(3, gen.act_stream(9), 37 * 512).reshape(37, 512)
    x[3] = 0.0
    x[4, :32] = 1e-30
    g = np.float32(orc.global_scale_of(x))
    q, s = mq.moesq_quantize_act(dev(x), dev(np.array([g], np.float32)))
    qo, so = orc.quantize_rows(x, g)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    q2, s2 = mq.moesq_quantize_act(xb.to(DEV), dev(np.array([g], np.float32)))
    qo2, so2 = orc.quantize_rows(xb.to(torch.float32).numpy(), g)
    assert np.array_equal(host(q2), qo2) and np.array_equal(host(s2), so2)
    # tensor scales far outside the data's range: 1e33 saturates every block scale at 448 and puts the
    # quotients near 1e30 (the quantizer's plain-division path), 1e-38 makes every scale and code 0
    for gx in (1e33, 1e-38):
        q3, s3 = mq.moesq_quantize_act(dev(x), dev(np.array([gx], np.float32)))
        qo3, so3 = orc.quantize_rows(x, np.float32(gx))
        assert np.array_equal(host(q3), qo3) and np.array_equal(host(s3), so3), gx


def _route_quantize_check(ids, x, E, ga, xk=False, bf16=False):
    """moesq_route_quantize against the oracle's routing + dispatch quantizer, and byte for byte
    against the two separate calls it replaces."""
    ids = ids.astype(np.int32)
    T, k = ids.shape
    xd = dev(x)
    if bf16:
        xd = xd.to(torch.bfloat16)
        x = xd.float().cpu().numpy()
    out = mq.moesq_route_quantize(dev(ids), E, xd, dev(ga), xk=True if xk else None)
    rt, q, s = out[:3]
    R = orc.route(ids, E)
    for key in ("counts", "offsets", "sorted_slot", "slot_pos"):
        assert np.array_equal(host(rt[key]), R[key]), key
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], k, R["offsets"], ga)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    rt2 = mq.moesq_route_permute(dev(ids), E)
    q2, s2, xk2 = mq.moesq_quantize_act(xd, dev(ga), slot_pos=rt2["slot_pos"], k=k, offsets=rt2["offsets"], xk=True)
    assert np.array_equal(host(q), host(q2)) and np.array_equal(host(s), host(s2))
    if xk:
        assert np.array_equal(host(out[3]).view(np.uint16), host(xk2).view(np.uint16))
        assert np.array_equal(host(out[3]).view(np.uint16), _xk_reference(qo, so).view(np.uint16))


@pytest.mark.parametrize("name", ["c0", "c1", "t_zipf", "t_mlp"])
def test_route_quantize_bitexact(name):
    c = single_case(name)
    say("route+quantize", name, "T*k", c["ids"].size)
    ga = c["ga"] * np.linspace(0.5, 2.0, c["E"]).astype(np.float32)   # distinct per-expert scales
    _route_quantize_check(c["ids"], c["x"], c["E"], ga, xk=True)


def test_route_quantize_edges():
    """The single-launch limit (T*k = 2048) and one past it (two launches), k = 1 and k = 32, one
    expert, ragged K (not a multiple of 512), bf16 input, skewed routing, and an empty batch."""
    rng = np.random.default_rng(17)

    def case(T, k, E, K, zipf=False, bf16=False):
        say("route+quantize edge T", T, "k", k, "E", E, "K", K)
        if zipf:
            ids, _ = gen.route_zipf(5, T, E, k, 1.2, 0)
        else:
            ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        x = gen.student_t(11, gen.act_stream(T + K), T * K).reshape(T, K)
        ga = (np.float32(orc.global_scale_of(x)) * np.linspace(0.7, 1.3, E)).astype(np.float32)
        _route_quantize_check(ids, x, E, ga, xk=(K % 256 == 0), bf16=bf16)

    case(256, 8, 128, 2048)            # T*k = 2048: the fused kernel's limit
    case(257, 8, 128, 2048)            # one token more: routing kernels + quantizer
    case(2, 32, 64, 7168)              # k = 32, K = 14 chunks of 512
    case(40, 1, 1, 96)                 # one expert, ragged K
    case(64, 8, 512, 1024, zipf=True)  # the routing path's largest E, skewed counts
    case(24, 6, 60, 2048, bf16=True)
    case(300, 40, 64, 64)              # k = 40 > 32: routing kernels + quantizer
    # empty batch: offsets and counts still written (zeros)
    cnt = torch.full((8,), 5, dtype=torch.int32, device=DEV)
    off = torch.full((9,), 5, dtype=torch.int32, device=DEV)
    empty = lambda *shape: torch.empty(shape, dtype=torch.int32, device=DEV)  # noqa: E731
    rt = dict(counts=cnt, offsets=off, sorted_slot=empty(0), slot_pos=empty(0))
    mq.moesq_route_quantize(empty(0, 2), 8, torch.zeros((0, 64), device=DEV), dev(np.ones(8, np.float32)), rt=rt)
    assert not host(cnt).any() and not host(off).any()


def test_route_quantize_invalid_ids():
    """Ids outside [0, E): both paths drop the slot (slot_pos = -1), report MOESQ_ERR_INVALID_ARG and
    write the valid copies to the same rows."""
    say("route+quantize invalid ids")
    ids = np.array([[0, 1], [5, 2], [1, -1], [3, 0]], np.int32)
    E, K = 4, 64
    x = gen.student_t(12, gen.act_stream(1), 4 * K).reshape(4, K)
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    q = torch.zeros((8, K // 2), dtype=torch.uint8, device=DEV)
    s = torch.zeros((8, K // 32), dtype=torch.uint8, device=DEV)
    rt, q, s = mq.moesq_route_quantize(dev(ids), E, dev(x), dev(ga), q=q, s=s, dev_status=st)
    assert int(host(st)[0]) == mq.ERR_INVALID_ARG
    st2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    rt2 = mq.moesq_route_permute(dev(ids), E, dev_status=st2)
    q2 = torch.zeros_like(q)
    s2 = torch.zeros_like(s)
    mq.moesq_quantize_act(dev(x), dev(ga), slot_pos=rt2["slot_pos"], k=2, offsets=rt2["offsets"], q=q2, s=s2)
    assert int(host(st2)[0]) == mq.ERR_INVALID_ARG
    n_ok = int(host(rt2["offsets"])[-1])
    assert n_ok == 6
    for key in ("counts", "offsets", "slot_pos"):
        assert np.array_equal(host(rt[key]), host(rt2[key])), key
    assert np.array_equal(host(rt["sorted_slot"])[:n_ok], host(rt2["sorted_slot"])[:n_ok])
    assert np.array_equal(host(q), host(q2)) and np.array_equal(host(s), host(s2))


def _route_quantize_dyn_check(ids, x, E, bf16=False):
    """moesq_route_quantize_dyn: the tensor scale against the oracle's Eq. 5 over all of x, the codes
    against the oracle's dispatch quantizer with that scale, and every output byte for byte against
    moesq_global_scale + moesq_route_quantize."""
    ids = ids.astype(np.int32)
    T, k = ids.shape
    xd = dev(x)
    if bf16:
        xd = xd.to(torch.bfloat16)
        x = xd.float().cpu().numpy()
    rt, q, s, xk, g = mq.moesq_route_quantize_dyn(dev(ids), E, xd, xk=True)
    gam = np.float32(orc.global_scale_of(x))
    assert np.all(host(g) == gam)
    R = orc.route(ids, E)
    for key in ("counts", "offsets", "sorted_slot", "slot_pos"):
        assert np.array_equal(host(rt[key]), R[key]), key
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], k, R["offsets"], np.full(E, gam, np.float32))
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    ga2 = mq.moesq_global_scale(xd).expand(E).contiguous()
    rt2, q2, s2, xk2 = mq.moesq_route_quantize(dev(ids), E, xd, ga2, xk=True)
    assert np.array_equal(host(q), host(q2)) and np.array_equal(host(s), host(s2))
    assert np.array_equal(host(xk.view(torch.int16)), host(xk2.view(torch.int16)))


def test_route_quantize_dynamic_scale():
    """The dynamic activation tensor scale: in the single launch (c1's 16 fp32 tokens of 2048, 128 KiB),
    past the token-byte budget (amax pre-pass, then the single-launch routing), past the routing's
    single launch (pre-pass, routing kernels, quantizer), bf16 tokens, one token, all-zero tokens."""
    c = single_case("c1")
    say("route+quantize dynamic scale c1")
    _route_quantize_dyn_check(c["ids"], c["x"], c["E"])
    rng = np.random.default_rng(29)

    def case(T, k, E, K, bf16=False, zero=False):
        say("route+quantize dynamic scale T", T, "k", k, "E", E, "K", K, "bf16", bf16, "zero", zero)
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        x = gen.student_t(31, gen.act_stream(T + K), T * K).reshape(T, K)
        if zero:
            x[:] = 0.0
        _route_quantize_dyn_check(ids, x, E, bf16=bf16)

    case(64, 8, 128, 2048)              # 512 KiB of tokens: pre-pass + single-launch routing
    case(64, 8, 384, 7168, bf16=True)   # the decode MLP's tokens
    case(300, 8, 64, 256)               # T*k > 2048: pre-pass + routing kernels + quantizer
    case(1, 4, 16, 512)
    case(8, 2, 8, 256, zero=True)       # amax 0: gamma = 1, every code 0


def test_global_scale_bitexact():
    say("global scale")
    for x in (gen.student_t(4, gen.act_stream(2), 300 * 256).reshape(300, 256),
              gen.normal(4, gen.act_stream(3), 5 * 4096).reshape(5, 4096), np.zeros((2, 64), np.float32),
              gen.normal(5, gen.act_stream(4), 7 * 37).reshape(7, 37),          # K % 8 != 0: element path
              gen.student_t(6, gen.act_stream(5), 64 * 7168).reshape(64, 7168)):
        g = mq.moesq_global_scale(dev(x))
        assert host(g)[0] == np.float32(orc.global_scale_of(x))
        gb = mq.moesq_global_scale(torch.from_numpy(x).to(torch.bfloat16).to(DEV))
        assert host(gb)[0] == np.float32(orc.global_scale_of(torch.from_numpy(x).to(torch.bfloat16).float().numpy()))


# ---------------------------------------------------------------- grouped GEMM ---------------
def _gemm_inputs(c):
    R, k = c["R"], c["k"]
    qo, so = orc.dispatch_quantize(c["x"], R["sorted_slot"], k, R["offsets"], c["ga"])
    return qo, so


_ref_cache = {}


def _oracle_gemm_all_rows(c, key):
    """The oracle's grouped GEMM over every routed row of a single-projection case (computed once)."""
    if key not in _ref_cache:
        qo, so = _gemm_inputs(c)
        off = c["R"]["offsets"]
        rows = np.arange(int(off[-1]))
        Wo = c["Wo"].ensure(np.flatnonzero(np.diff(off) > 0))
        say("oracle grouped GEMM over all", rows.size, "rows of", key)
        _ref_cache[key] = orc.grouped_gemm(Wo.as_dict(), qo, so, c["ga"], off, rows)
    return _ref_cache[key]


@pytest.mark.parametrize("name,proj", [("c0", 0), ("c1", 0), ("t_zipf", 0), ("c2", 0)])
@pytest.mark.parametrize("flags", ["decode", "decode_xk", "prefill", "prefill_xk"])
def test_grouped_gemm_parity(name, proj, flags):
    """Every routed row of every single-projection workload, including the Qwen3-30B-A3B prefill at its
    full 32,768 rows, in both kernel families and both activation operands, fp32 and bf16 outputs."""
    c = single_case(name, proj)
    say("gemm", name, proj, flags)
    qo, so = _gemm_inputs(c)
    off = c["R"]["offsets"]
    fl = mq.F_FORCE_DECODE if flags.startswith("decode") else mq.F_FORCE_PREFILL
    xk = dev(_xk_reference(qo, so)) if flags.endswith("_xk") else None
    y = mq.moesq_grouped_gemm(c["Wd"], dev(qo), dev(so), dev(c["ga"]), dev(off), y_dtype=torch.float32, flags=fl,
                              xk=xk)
    yb = mq.moesq_grouped_gemm(c["Wd"], dev(qo), dev(so), dev(c["ga"]), dev(off), y_dtype=torch.bfloat16,
                               flags=fl, xk=xk)
    ref = _oracle_gemm_all_rows(c, (name, proj))
    rows = int(off[-1])
    gemm_gate(host(y)[:rows], ref, "gemm %s %s" % (name, flags))
    gotb = host(yb.to(torch.float32))[:rows]
    assert orc.rel_frobenius(gotb, bf16_round(ref)) <= GEMM_TOL


def _weights_bitexact(Wd, Wo, experts, what):
    """Device-compressed weights (drawn on the device) byte for byte against the oracle's compression of
    the generator's host draw, for the given experts: packed values, masks, block scales, tensor scales."""
    idx = torch.tensor(experts, dtype=torch.long, device=DEV)
    for key in ("packed", "mask", "scale", "gscale"):
        got = host(getattr(Wd, key).index_select(0, idx))
        assert np.array_equal(got, getattr(Wo, key)[experts]), (what, key)
    say(what, "weights of experts", experts, "byte-identical")


@pytest.mark.parametrize("proj", [0, 1])
@pytest.mark.parametrize("flags", ["auto", "prefill"])
def test_grouped_gemm_parity_c3_full_size(proj, flags):
    """Kimi-shaped decode projections at full size (E=384; gate_up K=7168 N=4096, down K=2048
    N=7168, 512 routed rows), in the launch the benchmark uses (auto = weight streaming) and in the
    tiled kernel; the oracle evaluates every output column of every row of 24 sampled experts, whose
    device-compressed weights are also compared byte for byte with the oracle's compression."""
    c = single_case("c3", proj, x_tag=proj)
    say("gemm c3 full size proj", proj, flags)
    qo, so = _gemm_inputs(c)
    off = c["R"]["offsets"]
    fl = 0 if flags == "auto" else mq.F_FORCE_PREFILL
    y = mq.moesq_grouped_gemm(c["Wd"], dev(qo), dev(so), dev(c["ga"]), dev(off), y_dtype=torch.float32, flags=fl)
    rows, experts = sample_expert_rows(off, n_experts=24, per_expert=64)
    say("sampled experts", experts, "rows", rows.size)
    Wo = c["Wo"].ensure(experts)
    if flags == "auto":
        _weights_bitexact(c["Wd"], Wo, experts, "c3 proj %d" % proj)
    ref = orc.grouped_gemm(Wo.as_dict(), qo, so, c["ga"], off, rows)
    gemm_gate(host(y)[rows], ref, "c3 proj %d %s" % (proj, flags))


def test_grouped_gemm_deterministic_and_variants_agree():
    c = single_case("t_zipf")
    say("gemm determinism t_zipf")
    qo, so = _gemm_inputs(c)
    args = (c["Wd"], dev(qo), dev(so), dev(c["ga"]), dev(c["R"]["offsets"]))
    y1 = host(mq.moesq_grouped_gemm(*args, y_dtype=torch.float32))
    y2 = host(mq.moesq_grouped_gemm(*args, y_dtype=torch.float32))
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("kernel", ["streaming", "tiled"])
def test_every_call_deterministic(kernel):
    """Every call of the path, run twice on the same inputs, gives bitwise-identical outputs (no
    atomics decide a result): routing + quantization (fixed and dynamic scale), the one-call decode
    step, the MLP on both kernel families (with its fp32 gate_up dump and the h codes) and the
    combine."""
    cfg = gen.CONFIGS["t_mlp"]
    say("determinism", kernel)
    E, H, I2, I, T, k = cfg.E, cfg.K, cfg.N, cfg.N // 2, cfg.T, cfg.k
    kf = mq.F_FORCE_DECODE if kernel == "streaming" else mq.F_FORCE_PREFILL
    w13 = np.stack([gen.weights_expert(cfg, 0, e, I2, H) for e in range(E)])
    w2 = np.stack([gen.weights_expert(cfg, 1, e, H, I) for e in range(E)])
    W13, W2 = mq.moesq_compress_weights(dev(w13)), mq.moesq_compress_weights(dev(w2))
    x = dev(gen.activations(cfg, 0, T, H))
    ids, wts = gen.routing(cfg)
    ids_d, wts_d = dev(ids), dev(wts)
    ga = mq.moesq_global_scale(x).expand(E).contiguous()
    gh = torch.full((E,), cfg.gamma_h, dtype=torch.float32, device=DEV)

    def run():
        out = {}
        rt, q, s, xk = mq.moesq_route_quantize(ids_d, E, x, ga, xk=True)
        out.update(q=q, s=s, xk=xk.view(torch.int16), slot_pos=rt["slot_pos"], offsets=rt["offsets"])
        rtd, qd, sd, gd = mq.moesq_route_quantize_dyn(ids_d, E, x)
        out.update(qd=qd, sd=sd, gd=gd)
        y2, ws = mq.moesq_expert_mlp(W13, W2, q, s, ga, gh, rt["offsets"], y_dtype=torch.float32,
                                     flags=mq.F_DUMP_GATEUP | kf)
        hq, hs, dump = mq.mlp_workspace_views(ws, T * k, I, dump=True)
        out.update(y2=y2, hq=hq.clone(), hs=hs.clone(), dump=dump.clone())
        out["comb"] = mq.moesq_unpermute_combine(y2, rt["slot_pos"], wts_d, out_dtype=torch.float32)
        rtg, qg, sg, yg = mq.moesq_route_quantize_gemm(ids_d[:1], x[:1], ga, W13)
        out.update(yg=yg.view(torch.int16), qg=qg)
        torch.cuda.synchronize()
        return {key: host(v).copy() for key, v in out.items()}

    a, b = run(), run()
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_grouped_gemm_edge_cases():
    """All rows to one expert, T = 1 / k = 1, all-zero activations."""
    c = single_case("c0")
    say("gemm edges c0")
    E, K, N = c["E"], c["K"], c["N"]
    W = c["Wo"].as_dict()
    for ids in (np.full((70, 1), 2, np.int32), np.array([[3]], np.int32)):
        R = orc.route(ids, E)
        x = gen.activations(c["cfg"], 5, ids.shape[0], K)
        ga = np.full(E, orc.global_scale_of(x), np.float32)
        qo, so = orc.dispatch_quantize(x, R["sorted_slot"], ids.shape[1], R["offsets"], ga)
        for fl in (mq.F_FORCE_DECODE, mq.F_FORCE_PREFILL):
            y = mq.moesq_grouped_gemm(c["Wd"], dev(qo), dev(so), dev(ga), dev(R["offsets"]), y_dtype=torch.float32,
                                      flags=fl)
            ref = orc.grouped_gemm(W, qo, so, ga, R["offsets"])
            gemm_gate(host(y), ref, "gemm edge T=%d k=%d" % ids.shape)
    qz = np.zeros((16, K // 2), np.uint8)
    sz = np.zeros((16, K // 32), np.uint8)
    off = np.array([0, 4, 4, 10, 16], np.int32)
    y = mq.moesq_grouped_gemm(c["Wd"], dev(qz), dev(sz), dev(c["ga"]), dev(off), y_dtype=torch.float32)
    assert np.all(host(y) == 0)


@pytest.mark.parametrize("flags", ["decode", "decode_xk", "prefill", "prefill_xk"])
def test_grouped_gemm_token_count_boundaries(flags):
    """Experts whose token counts sit on and around every block boundary of both kernels (16-token
    fragments, the 64-token skip groups and 128-token tiles of the tiled kernel, its B read-ahead
    within a group) and an empty expert, with N = 640 (a partial 512-row block) and K = 512: each
    configuration against the oracle."""
    counts = np.array([0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257], np.int64)
    E, K, N = counts.size, 512, 640
    say("gemm token-count boundaries", flags)
    rng = np.random.default_rng(77)
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    Wo, Wd = orc.compress(w), mq.moesq_compress_weights(dev(w))
    rows = int(counts.sum())
    ids = np.repeat(np.arange(E, dtype=np.int32), counts).reshape(rows, 1)
    R = orc.route(ids, E)
    x = gen.student_t(71, gen.act_stream(3), rows * K).reshape(rows, K)
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], 1, R["offsets"], ga)
    fl = mq.F_FORCE_DECODE if flags.startswith("decode") else mq.F_FORCE_PREFILL
    xk = dev(_xk_reference(qo, so)) if flags.endswith("_xk") else None
    y = mq.moesq_grouped_gemm(Wd, dev(qo), dev(so), dev(ga), dev(R["offsets"]), y_dtype=torch.float32, flags=fl,
                              xk=xk)
    ref = orc.grouped_gemm(Wo, qo, so, ga, R["offsets"])
    gemm_gate(host(y), ref, "gemm token-count boundaries %s" % flags)
    # every expert on its own (a small expert's error is not hidden by the large ones)
    off = R["offsets"]
    for e in range(E):
        if counts[e]:
            assert orc.rel_frobenius(host(y)[off[e]:off[e + 1]], ref[off[e]:off[e + 1]]) <= GEMM_TOL, e


@pytest.mark.parametrize("flags", ["decode", "decode_xk", "prefill", "prefill_xk"])
def test_grouped_gemm_smallest_shapes(flags):
    """The smallest weight shapes the kernels take: N = 64 (one 64-row group: a single fragment group of
    the streaming kernel, one wave's rows of a 512-row tile) and K = 256 (one super-step), with a single
    expert (E = 1, three token tiles) and with an empty expert next to a 129-token one."""
    say("gemm smallest shapes", flags)
    rng = np.random.default_rng(123)
    fl = mq.F_FORCE_DECODE if flags.startswith("decode") else mq.F_FORCE_PREFILL
    for counts in (np.array([300]), np.array([0, 129])):
        E, N, K = counts.size, 64, 256
        w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
        Wo, Wd = orc.compress(w), mq.moesq_compress_weights(dev(w))
        rows = int(counts.sum())
        ids = np.repeat(np.arange(E, dtype=np.int32), counts).reshape(rows, 1)
        R = orc.route(ids, E)
        x = gen.student_t(91, gen.act_stream(E), rows * K).reshape(rows, K)
        ga = np.full(E, orc.global_scale_of(x), np.float32)
        qo, so = orc.dispatch_quantize(x, R["sorted_slot"], 1, R["offsets"], ga)
        xk = dev(_xk_reference(qo, so)) if flags.endswith("_xk") else None
        y = mq.moesq_grouped_gemm(Wd, dev(qo), dev(so), dev(ga), dev(R["offsets"]), y_dtype=torch.float32, flags=fl,
                                  xk=xk)
        gemm_gate(host(y), orc.grouped_gemm(Wo, qo, so, ga, R["offsets"]), "gemm E=%d N=64 K=256 %s" % (E, flags))


@pytest.mark.parametrize("n_full", [1000, 1024])
def test_grouped_gemm_many_full_tiles(n_full):
    """The tiled kernel at the largest expert count it takes (E = 1024, N = 64, K = 256) with n_full
    experts of 129 tokens (one full token tile and a 1-token partial tile each) and the rest empty. Its
    workgroups look up the expert of a full token tile in an LDS table when the table fits beside the
    tile tables (1018 entries at E = 1024): 1000 full tiles take the table, 1024 the binary search over
    the tile prefix. Sampled rows (every nonempty expert's first and last row among them) against the
    oracle."""
    say("gemm many full tiles", n_full)
    E, N, K = 1024, 64, 256
    counts = np.zeros(E, np.int64)
    counts[:n_full] = 129
    rng = np.random.default_rng(2024)
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    Wo, Wd = orc.compress(w), mq.moesq_compress_weights(dev(w))
    rows = int(counts.sum())
    ids = np.repeat(np.arange(E, dtype=np.int32), counts).reshape(rows, 1)
    R = orc.route(ids, E)
    x = gen.student_t(93, gen.act_stream(5), rows * K).reshape(rows, K)
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], 1, R["offsets"], ga)
    y = mq.moesq_grouped_gemm(Wd, dev(qo), dev(so), dev(ga), dev(R["offsets"]), y_dtype=torch.float32,
                              flags=mq.F_FORCE_PREFILL)
    sr = sample_rows(R["offsets"], 4096, seed=n_full)
    gemm_gate(host(y)[sr], orc.grouped_gemm(Wo, qo, so, ga, R["offsets"], sr), "gemm E=1024 full tiles %d" % n_full)


# ------------------------------------------------- dispatch + GEMM in one call --------------
def _rqg_check(ids, x, E, ga, Wd, Wo=None, bf16=False, y_dtype=torch.float32, oracle_rows=None):
    """moesq_route_quantize_gemm byte for byte against moesq_route_quantize + moesq_grouped_gemm (the
    two calls it replaces, with the f16 operand copy), and its y against the oracle's GEMM on the
    oracle's routing and quantization."""
    ids = ids.astype(np.int32)
    T, k = ids.shape
    xd = dev(x)
    if bf16:
        xd = xd.to(torch.bfloat16)
        x = xd.float().cpu().numpy()
    gad = dev(ga)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    rt, q, s, xk, y = mq.moesq_route_quantize_gemm(dev(ids), xd, gad, Wd, xk=True, y_dtype=y_dtype, dev_status=st)
    st2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    rt2, q2, s2, xk2 = mq.moesq_route_quantize(dev(ids), E, xd, gad, xk=True, dev_status=st2)
    y2 = mq.moesq_grouped_gemm(Wd, q2, s2, gad, rt2["offsets"], y_dtype=y_dtype, xk=xk2)
    assert int(host(st)[0]) == int(host(st2)[0])
    n_ok = int(host(rt2["offsets"])[-1])
    for key in ("counts", "offsets", "slot_pos"):
        assert np.array_equal(host(rt[key]), host(rt2[key])), key
    assert np.array_equal(host(rt["sorted_slot"])[:n_ok], host(rt2["sorted_slot"])[:n_ok])
    assert np.array_equal(host(q)[:n_ok], host(q2)[:n_ok]) and np.array_equal(host(s)[:n_ok], host(s2)[:n_ok])
    assert np.array_equal(host(xk.view(torch.int16))[:n_ok], host(xk2.view(torch.int16))[:n_ok])
    bits = torch.int32 if y_dtype == torch.float32 else torch.int16
    assert np.array_equal(host(y.view(bits))[:n_ok], host(y2.view(bits))[:n_ok])
    if Wo is None:
        return y
    R = orc.route(ids, E)
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], k, R["offsets"], ga)
    assert np.array_equal(host(q)[:n_ok], qo) and np.array_equal(host(s)[:n_ok], so)
    rows = np.arange(n_ok) if oracle_rows is None else oracle_rows
    ref = orc.grouped_gemm(Wo, qo, so, ga, R["offsets"], rows)
    got = host(y.to(torch.float32))[rows]
    if y_dtype == torch.float32:
        gemm_gate(got, ref, "route_quantize_gemm")
    else:
        err = orc.rel_frobenius(got, bf16_round(ref))
        say("route_quantize_gemm bf16 rel-Frobenius", err)
        assert err <= GEMM_TOL
    return y


@pytest.mark.parametrize("name,T", [("c0", None), ("c1", None), ("c1", 2), ("c1", 1)])
def test_route_quantize_gemm_parity(name, T):
    """The one-call decode step on the benchmark's decode configuration (E=128, K=2048, N=1536, top-8)
    at its 16 tokens (two launches) and at 2 and 1 tokens (one launch), and the small case, with
    distinct per-expert activation scales."""
    c = single_case(name)
    ids, x = c["ids"][:T], c["x"][:T]
    say("route_quantize_gemm", name, "T", ids.shape[0])
    ga = (c["ga"] * np.linspace(0.5, 2.0, c["E"])).astype(np.float32)
    off = orc.route(ids, c["E"])["offsets"]
    Wo = c["Wo"].ensure(np.flatnonzero(np.diff(off) > 0)).as_dict()
    for ydt in (torch.float32, torch.bfloat16):
        _rqg_check(ids, x, c["E"], ga, c["Wd"], Wo, y_dtype=ydt)


def test_route_quantize_gemm_edges():
    """Multi-pass experts (more tokens than one LDS pass holds), bf16 input, split tensor scales,
    invalid ids, the one-launch limits (2 T*k = E, K = 2048) and one past each (two calls), and the
    smallest K."""
    rng = np.random.default_rng(23)

    def case(T, k, E, N, K, zipf=False, bf16=False, split=False, bad=False, oracle=True):
        say("route_quantize_gemm edge T", T, "k", k, "E", E, "N", N, "K", K, "zipf", zipf, "split", split, "bad", bad)
        if zipf:
            ids, _ = gen.route_zipf(9, T, E, k, 1.3, 0)
        else:
            ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        if bad:
            ids[1, 0] = E
            ids[T - 1, k - 1] = -3
        x = gen.student_t(13, gen.act_stream(T + K + N), T * K).reshape(T, K)
        ga = (np.float32(orc.global_scale_of(x)) * np.linspace(0.8, 1.25, E)).astype(np.float32)
        w = (np.random.default_rng(T + N).standard_normal((E, N, K)) * 0.02).astype(np.float32)
        if split:
            w[:, N // 2:] *= np.float32(3.0)
            Wd, Wo = mq.moesq_compress_weights(dev(w), split_halves=True), orc.compress_split(w)
        else:
            Wd, Wo = mq.moesq_compress_weights(dev(w)), orc.compress(w)
        _rqg_check(ids, x, E, ga, Wd, Wo if (oracle and not bad) else None, bf16=bf16)

    case(40, 1, 320, 128, 512, zipf=True)         # hot experts: many tokens, several LDS passes
    case(2, 4, 64, 256, 2048, bf16=True)
    case(2, 8, 128, 256, 256, split=True)
    case(3, 3, 80, 64, 256, bad=True)             # ids outside [0, E)
    case(48, 1, 96, 64, 2048)                     # 2 T*k = E: one launch
    case(49, 1, 96, 64, 2048)                     # one token more: two calls
    case(16, 8, 128, 64, 2048)                    # the decode benchmark's batch shape: two calls
    case(17, 4, 4, 64, 256)                       # T*k > 16 E: two calls, tiled GEMM
    case(2, 4, 64, 64, 2304)                     # 2 T*k <= E but K > 2048: two calls


def test_empty_batch_one_call_and_dynamic_scale():
    """T = 0 through the one-call step and the dynamic-scale dispatch: counts and offsets are written
    as zeros, nothing else is touched, the dynamic scale of an empty tensor is Eq. 5's 1."""
    say("empty batch: route_quantize_gemm, route_quantize_dyn")
    c = single_case("c0")
    E, K = c["E"], c["K"]
    empty = lambda *shape: torch.empty(shape, dtype=torch.int32, device=DEV)  # noqa: E731
    for call in ("gemm", "dyn"):
        cnt = torch.full((E,), 5, dtype=torch.int32, device=DEV)
        off = torch.full((E + 1,), 5, dtype=torch.int32, device=DEV)
        rt = dict(counts=cnt, offsets=off, sorted_slot=empty(0), slot_pos=empty(0))
        x = torch.zeros((0, K), device=DEV)
        if call == "gemm":
            mq.moesq_route_quantize_gemm(empty(0, c["k"]), x, dev(c["ga"]), c["Wd"], rt=rt)
        else:
            g = torch.full((E,), 7.0, device=DEV)
            mq.moesq_route_quantize_dyn(empty(0, c["k"]), E, x, gamma_out=g, rt=rt)
            assert np.all(host(g) == 1.0)
        assert not host(cnt).any() and not host(off).any(), call


@pytest.mark.parametrize("T", [2, 16])
def test_route_quantize_gemm_graph_replays(T):
    """The one-call step (one launch at 2 tokens, two at 16) captured in a HIP graph and replayed with
    eager work in between: every replay reproduces the eager outputs bit for bit."""
    c = single_case("c1")
    say("route_quantize_gemm graph replays c1 T", T)
    ids_d, x_d, ga_d = dev(c["ids"][:T]), dev(c["x"][:T]), dev(c["ga"])
    xk = True if T > 2 else None
    out = mq.moesq_route_quantize_gemm(ids_d, x_d, ga_d, c["Wd"], xk=xk)
    rt, q, s, y = out[0], out[1], out[2], out[-1]
    xk = out[3] if T > 2 else None
    ref = [host(t.view(torch.int16) if t.dtype == torch.bfloat16 else t).copy() for t in (y, q, rt["slot_pos"])]

    def step():
        mq.moesq_route_quantize_gemm(ids_d, x_d, ga_d, c["Wd"], rt=rt, q=q, s=s, xk=xk, y=y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        y.zero_()
        q.zero_()
        rt["slot_pos"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(t.view(torch.int16) if t.dtype == torch.bfloat16 else t) for t in (y, q, rt["slot_pos"])]
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), i
        _ = torch.ones(1024, device=DEV).sum()


# ---------------------------------------------------------------- combine --------------------
COMBINE_CASES = [
    # (T, k, H, E, drop): drop marks copies that have no row (slot_pos = -1: an invalid id, or a slot
    # over the capacity), which the combine skips
    (50, 4, 512, 9, "none"),
    (37, 10, 7168, 13, "some"),   # two groups of 8 copies, the second partial; the Kimi hidden size
    (19, 8, 1032, 11, "groups"),  # a token with no row at all; 129 threads per token (a partial block)
]


@pytest.mark.parametrize("case", COMBINE_CASES, ids=["k4", "k10_drops", "k8_empty_tokens"])
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16])
def test_combine_parity(ydt, case):
    T, k, H, E, drop = case
    say("combine", ydt, case)
    ids, w = gen.route_uniform(11, T, E, k)
    R = orc.route(ids, E)
    sp = R["slot_pos"].reshape(T, k).copy()
    if drop == "some":
        sp[::3, 1] = -1          # dropped copies inside the first group of 8
        sp[5, :] = -1            # a token with no row
        sp[7, 8:] = -1           # the partial second group empty
    elif drop == "groups":
        sp[2, :] = -1
        sp[3, ::2] = -1
    sp = sp.reshape(-1)
    y = gen.normal(3, gen.act_stream(3), T * k * H).reshape(T * k, H)
    yt = torch.from_numpy(y).to(ydt)
    # the oracle on the same rows, a dropped copy pointing at an extra zero row
    y64 = np.vstack([yt.to(torch.float64).numpy(), np.zeros((1, H))])
    sp_ref = np.where(sp < 0, T * k, sp).astype(np.int32)
    ref = orc.combine(y64, sp_ref, w)
    out = mq.moesq_unpermute_combine(yt.to(DEV), dev(sp), dev(w), out_dtype=torch.float32)
    got = host(out)
    assert orc.rel_frobenius(got, ref) <= 1e-6
    # per element: k fp32 products summed in fp32 are within (k + 1) 2^-24 of the sum of |products|
    mag = orc.combine(np.abs(y64), sp_ref, np.abs(w))
    assert np.all(np.abs(got - ref) <= (k + 1) * 2.0 ** -24 * mag)
    empty = (sp.reshape(T, k) < 0).all(1)
    assert empty.any() == (drop != "none") and np.all(got[empty] == 0.0)
    outb = mq.moesq_unpermute_combine(yt.to(DEV), dev(sp), dev(w), out_dtype=torch.bfloat16)
    assert orc.rel_frobenius(host(outb.float()), bf16_round(ref)) <= 1e-3


# ---------------------------------------------------------------- MLP --------------------------
def _mlp_stage_gates(W2o, y, ws, rows_all, I, ga_unused, gh, off, M, what, rows=None):
    """Stage gates of one moesq_expert_mlp call (run with F_DUMP_GATEUP | F_DUMP_H) against the oracle
    chain M on the same rows: gate_up outputs (fp32 dump) within tolerance; the requantized h byte for
    byte on the kernel's own h; the down GEMM on the kernel's own h codes within tolerance; the end-to-end
    chain error and the h code flips against the oracle's independent chain are reported (they include
    rounding-boundary flips of h codes, so they are not the gate)."""
    rows = np.arange(rows_all) if rows is None else rows
    hq, hs, dump = mq.mlp_workspace_views(ws, rows_all, I, dump=True)
    gemm_gate(rows_of(dump, rows), M["y13"], what + " gate_up")
    flips = requant_gate(ws, rows_all, I, gh, rows, orc.expert_of_rows(off, rows), M)
    # the down GEMM on the kernel's own codes (other rows zero: rows are independent)
    hq_k = np.zeros((int(off[-1]), I // 2), np.uint8)
    hs_k = np.zeros((int(off[-1]), I // 32), np.uint8)
    hq_k[rows], hs_k[rows] = rows_of(hq, rows), rows_of(hs, rows)
    gemm_gate(rows_of(y, rows), orc.grouped_gemm(W2o, hq_k, hs_k, gh, off, rows), what + " down on the kernel's h")
    chain = orc.rel_frobenius(rows_of(y, rows), M["y2"])
    say(what, "end-to-end rel-Frobenius against the oracle's chain %.3g (h code flips %.2e)" % (chain, flips))
    assert chain <= 1e-2   # a sanity bound: flips move single outputs by one E2M1 step
    return chain


@pytest.mark.parametrize("kernel", ["tiled", "streaming"])
def test_mlp_parity_tiny(kernel):
    """The routed-expert MLP on both kernel families (t_mlp has 32 rows per expert: tiled by default;
    MOESQ_F_FORCE_DECODE runs both GEMMs by weight streaming with the SwiGLU + requant epilogue), with a
    distinct intermediate scale per expert from the oracle's own h; the calibration call against the
    kernel's h and the oracle's scales."""
    cfg = gen.CONFIGS["t_mlp"]
    say("mlp t_mlp", kernel)
    kf = mq.F_FORCE_DECODE if kernel == "streaming" else 0
    E, H, I2, I, T, k = cfg.E, cfg.K, cfg.N, cfg.N // 2, cfg.T, cfg.k
    w13 = np.stack([gen.weights_expert(cfg, 0, e, I2, H) for e in range(E)])
    w2 = np.stack([gen.weights_expert(cfg, 1, e, H, I) for e in range(E)])
    W13o, W2o = orc.compress(w13), orc.compress(w2)
    W13, W2 = mq.moesq_compress_weights(dev(w13)), mq.moesq_compress_weights(dev(w2))
    x = gen.activations(cfg, 0, T, H)
    ids, wts = gen.routing(cfg)
    R = orc.route(ids, E)
    off = R["offsets"]
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], k, off, ga)
    gh = oracle_gamma_h(W13o, qo, so, ga, off)
    assert len(set(gh.tolist())) == E   # one scale per expert
    M = orc.expert_mlp(W13o, W2o, qo, so, ga, gh, off)
    rows = int(off[-1])
    y, ws = mq.moesq_expert_mlp(W13, W2, dev(qo), dev(so), dev(ga), dev(gh), dev(off), y_dtype=torch.float32,
                                flags=mq.F_DUMP_GATEUP | mq.F_DUMP_H | kf)
    y_xk, _ = mq.moesq_expert_mlp(W13, W2, dev(qo), dev(so), dev(ga), dev(gh), dev(off),
                                  y_dtype=torch.float32, xk=dev(_xk_reference(qo, so)), flags=kf)
    assert np.array_equal(host(y_xk), host(y))   # same operands, same kernel order of operations
    _mlp_stage_gates(W2o, y, ws, rows, I, ga, gh, off, M, "t_mlp " + kernel)
    # down GEMM alone on the oracle's h codes: identical operands
    yd = mq.moesq_grouped_gemm(W2, dev(M["hq"]), dev(M["hs"]), dev(gh), dev(off), y_dtype=torch.float32, flags=kf)
    gemm_gate(host(yd), M["y2"], "down on the oracle's h")
    out = mq.moesq_unpermute_combine(y, dev(R["slot_pos"]), dev(wts), out_dtype=torch.float32)
    assert orc.rel_frobenius(host(out), orc.combine(M["y2"], R["slot_pos"], wts)) <= 1e-2
    # calibration of the intermediate scales, on the same kernel family
    gcal, acal = mq.moesq_calibrate_gamma_h(W13, W2, dev(qo), dev(so), dev(ga), dev(off), flags=kf)
    all_rows = np.arange(rows)
    calibration_gate(gcal, acal, h_row_absmax(ws, rows, I, all_rows), orc.expert_of_rows(off, all_rows), E, gh)


@pytest.mark.parametrize("I", [512, 1024])
def test_mlp_streaming_block_renumbering(I):
    """The weight-streaming MLP gate_up renumbers its workgroups (pairs sharing a unit's mask and scale
    lines on one XCD) when I/32 is a multiple of 16: its smallest cases (16 and 32 column blocks)
    against the oracle, gate_up outputs and the requantized h, with the NVFP4 codes and the f16
    operand copy."""
    E, H, T, k = 4, 256, 32, 2
    say("mlp streaming renumbering I", I)
    rng = np.random.default_rng(I)
    w13 = (rng.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    W13o, W2o = orc.compress(w13), orc.compress(w2)
    W13, W2 = mq.moesq_compress_weights(dev(w13)), mq.moesq_compress_weights(dev(w2))
    x = gen.student_t(70, gen.act_stream(I), T * H).reshape(T, H)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    R = orc.route(ids, E)
    off = R["offsets"]
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], k, off, ga)
    gh = oracle_gamma_h(W13o, qo, so, ga, off)
    M = orc.expert_mlp(W13o, W2o, qo, so, ga, gh, off)
    rows = int(off[-1])
    y, ws = mq.moesq_expert_mlp(W13, W2, dev(qo), dev(so), dev(ga), dev(gh), dev(off), y_dtype=torch.float32,
                                flags=mq.F_DUMP_GATEUP | mq.F_DUMP_H | mq.F_FORCE_DECODE)
    _mlp_stage_gates(W2o, y, ws, rows, I, ga, gh, off, M, "streaming I=%d" % I)
    # the f16-operand form (one activation stage in registers): the same operands, the same result bits
    y_xk, _ = mq.moesq_expert_mlp(W13, W2, dev(qo), dev(so), dev(ga), dev(gh), dev(off),
                                  y_dtype=torch.float32, xk=dev(_xk_reference(qo, so)), flags=mq.F_FORCE_DECODE)
    assert np.array_equal(host(y_xk), host(y))


@pytest.mark.parametrize("kernel", ["streaming", "tiled"])
def test_mlp_token_count_boundaries(kernel):
    """The routed-expert MLP with expert token counts on and around the kernels' block boundaries
    (16, 64, 128 tokens) and an empty expert: gate_up outputs, requantized h and the chain against
    the oracle, with the NVFP4 codes and the f16 operand copy (bit-identical to each other), and the
    calibration (the empty expert gets amax 0, gamma 1)."""
    counts = np.array([0, 1, 16, 17, 63, 64, 65, 127, 128, 129, 200], np.int64)
    E, H, I = counts.size, 256, 512
    say("mlp token-count boundaries", kernel)
    kf = mq.F_FORCE_DECODE if kernel == "streaming" else mq.F_FORCE_PREFILL
    rng = np.random.default_rng(78)
    w13 = (rng.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    W13o, W2o = orc.compress(w13), orc.compress(w2)
    W13, W2 = mq.moesq_compress_weights(dev(w13)), mq.moesq_compress_weights(dev(w2))
    rows = int(counts.sum())
    ids = np.repeat(np.arange(E, dtype=np.int32), counts).reshape(rows, 1)
    R = orc.route(ids, E)
    off = R["offsets"]
    x = gen.student_t(72, gen.act_stream(5), rows * H).reshape(rows, H)
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], 1, off, ga)
    gh = oracle_gamma_h(W13o, qo, so, ga, off)
    M = orc.expert_mlp(W13o, W2o, qo, so, ga, gh, off)
    y, ws = mq.moesq_expert_mlp(W13, W2, dev(qo), dev(so), dev(ga), dev(gh), dev(off), y_dtype=torch.float32,
                                flags=mq.F_DUMP_GATEUP | mq.F_DUMP_H | kf)
    _mlp_stage_gates(W2o, y, ws, rows, I, ga, gh, off, M, "boundaries " + kernel)
    y_xk, _ = mq.moesq_expert_mlp(W13, W2, dev(qo), dev(so), dev(ga), dev(gh), dev(off),
                                  y_dtype=torch.float32, xk=dev(_xk_reference(qo, so)), flags=kf)
    assert np.array_equal(host(y_xk), host(y))
    gcal, acal = mq.moesq_calibrate_gamma_h(W13, W2, dev(qo), dev(so), dev(ga), dev(off), flags=kf,
                                           xk=dev(_xk_reference(qo, so)))
    all_rows = np.arange(rows)
    calibration_gate(gcal, acal, h_row_absmax(ws, rows, I, all_rows), orc.expert_of_rows(off, all_rows), E, gh)
    assert host(acal)[0] == 0 and host(gcal)[0] == 1.0   # the empty expert


@pytest.mark.parametrize("kernel", ["streaming", "tiled"])
def test_requant_extreme_intermediate_scales(kernel):
    """The requantization of h with intermediate scales far outside the calibrated range: expert 0's
    gamma_h = 1e33 (every block scale saturates at 448 and h / s reaches ~1e30: the epilogue's
    plain-division path), expert 1's 1e-38 (every block scale encodes to 0, so do the codes), the rest
    calibrated. Codes, block scales and the f16 copy against the oracle's quantizer on the kernel's own
    fp32 h, byte for byte, in both kernel families."""
    cfg = gen.CONFIGS["t_mlp"]
    say("requant extreme gamma_h", kernel)
    kf = mq.F_FORCE_DECODE if kernel == "streaming" else mq.F_FORCE_PREFILL
    E, H, I2, I, T, k = cfg.E, cfg.K, cfg.N, cfg.N // 2, cfg.T, cfg.k
    w13 = np.stack([gen.weights_expert(cfg, 0, e, I2, H) for e in range(E)])
    w2 = np.stack([gen.weights_expert(cfg, 1, e, H, I) for e in range(E)])
    W13, W2 = mq.moesq_compress_weights(dev(w13)), mq.moesq_compress_weights(dev(w2))
    x = gen.activations(cfg, 0, T, H)
    ids, _ = gen.routing(cfg)
    R = orc.route(ids, E)
    off = R["offsets"]
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], k, off, ga)
    gh = oracle_gamma_h(orc.compress(w13), qo, so, ga, off)
    gh[0], gh[1] = np.float32(1e33), np.float32(1e-38)
    rows = int(off[-1])
    assert off[1] > off[0] and off[2] > off[1]
    y, ws = mq.moesq_expert_mlp(W13, W2, dev(qo), dev(so), dev(ga), dev(gh), dev(off), y_dtype=torch.float32,
                                flags=mq.F_DUMP_GATEUP | mq.F_DUMP_H | kf)
    requant_gate(ws, rows, I, gh, np.arange(rows), orc.expert_of_rows(off, np.arange(rows)))
    hq, hs, _ = mq.mlp_workspace_views(ws, rows, I, dump=True)
    assert np.all(host(hs)[:off[1]] == 0x7E)                       # saturated block scales
    assert not np.any(host(hs)[off[1]:off[2]]) and not np.any(host(hq)[off[1]:off[2]])  # zero scales, zero codes


@pytest.mark.parametrize("kernel", ["streaming", "tiled"])
def test_split_tensor_scales(kernel):
    """Gate and up kept as separate linears, each with its own Eq. 5 tensor scale (the model card's
    checkpoint): device compression of the [2E, N/2, K] view against the oracle's compress_split
    (bit-exact), the grouped GEMM on the split weights, and the MLP whose gate_up carries them, on
    both kernel families."""
    cfg = gen.CONFIGS["t_mlp"]
    say("split tensor scales", kernel)
    E, H, I2, I, T, k = cfg.E, cfg.K, cfg.N, cfg.N // 2, cfg.T, cfg.k
    kf = mq.F_FORCE_DECODE if kernel == "streaming" else mq.F_FORCE_PREFILL
    w13 = np.stack([gen.weights_expert(cfg, 0, e, I2, H) for e in range(E)])
    w13[:, I:] *= np.float32(3.0)  # the up projection at another magnitude: its own tensor scale
    w2 = np.stack([gen.weights_expert(cfg, 1, e, H, I) for e in range(E)])
    W13 = mq.moesq_compress_weights(dev(w13), split_halves=True)
    W13o = orc.compress_split(w13)
    for key in ("packed", "mask", "scale", "gscale"):
        assert np.array_equal(host(getattr(W13, key)), W13o[key]), key
    assert np.all(W13o["gscale"][:, 0] != W13o["gscale"][:, 1])
    W2 = mq.moesq_compress_weights(dev(w2))
    W2o = orc.compress(w2)
    x = gen.activations(cfg, 0, T, H)
    ids, _ = gen.routing(cfg)
    R = orc.route(ids, E)
    off = R["offsets"]
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], k, off, ga)
    gh = oracle_gamma_h(W13o, qo, so, ga, off)
    y = host(mq.moesq_grouped_gemm(W13, dev(qo), dev(so), dev(ga), dev(off), y_dtype=torch.float32, flags=kf))
    ref = orc.grouped_gemm(W13o, qo, so, ga, off)
    for h in (slice(0, I), slice(I, I2)):
        gemm_gate(y[:, h], ref[:, h], "split scales gate_up half")
    y2, ws = mq.moesq_expert_mlp(W13, W2, dev(qo), dev(so), dev(ga), dev(gh), dev(off), y_dtype=torch.float32,
                                 flags=mq.F_DUMP_GATEUP | mq.F_DUMP_H | kf)
    M = orc.expert_mlp(W13o, W2o, qo, so, ga, gh, off)
    _mlp_stage_gates(W2o, y2, ws, int(off[-1]), I, ga, gh, off, M, "split scales " + kernel)


def _small_weights(E, N, K, seed):
    """Seeded N(0, 0.02) weights compressed on the device and by the oracle."""
    w = (np.random.default_rng(seed).standard_normal((E, N, K)) * 0.02).astype(np.float32)
    return mq.moesq_compress_weights(dev(w)), orc.compress(w)


def _capacity_rows(R, ids, C):
    """The oracle's routing mapped into the fixed-capacity layout: expected slot positions, and for
    every placed slot its capacity row and its contiguous (prefix-layout) row."""
    E = R["counts"].size
    e = ids.ravel().astype(np.int64)
    r = R["slot_pos"].astype(np.int64) - R["offsets"][e]
    exp = np.where(r < C, e * C + r, -1).astype(np.int32)
    keep = exp >= 0
    return exp, exp[keep].astype(np.int64), R["slot_pos"][keep].astype(np.int64)


@pytest.mark.parametrize("kernel", ["streaming", "tiled"])
def test_capacity_layout_gemm(kernel):
    """The fixed-capacity layout (expert e owns rows [e C, (e+1) C), counts on the device): routing
    into it, the scatter quantizer with per-expert scales, and the grouped GEMM, against the oracle's
    contiguous results mapped row by row; experts below, at zero and over the capacity."""
    say("capacity layout gemm", kernel)
    E, N, K, T, k, C = 16, 256, 512, 64, 4, 20
    kf = mq.F_FORCE_DECODE if kernel == "streaming" else mq.F_FORCE_PREFILL
    Wd, W = _small_weights(E, N, K, 41)
    ids, _ = gen.route_zipf(41, T, E, k, 1.1, 2)
    x = gen.student_t(41, gen.act_stream(5), T * K).reshape(T, K)
    ga = (np.float32(orc.global_scale_of(x)) * np.linspace(0.8, 1.25, E)).astype(np.float32)
    R = orc.route(ids, E)
    exp, cap_rows, pre_rows = _capacity_rows(R, ids, C)
    rc = mq.moesq_route_capacity(dev(ids), E, C)
    assert np.array_equal(host(rc["counts"]), R["counts"])
    assert np.array_equal(host(rc["slot_pos"]), exp)
    q, s = mq.moesq_quantize_act(dev(x), dev(ga), slot_pos=rc["slot_pos"], k=k, rows=E * C, capacity_experts=E)
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], k, R["offsets"], ga)
    assert np.array_equal(host(q)[cap_rows], qo[pre_rows]) and np.array_equal(host(s)[cap_rows], so[pre_rows])
    y = host(mq.moesq_grouped_gemm(Wd, q, s, dev(ga), rc["counts"], y_dtype=torch.float32, flags=mq.F_CAPACITY | kf))
    ref = orc.grouped_gemm(W, qo, so, ga, R["offsets"], pre_rows)
    assert orc.rel_frobenius(y[cap_rows], ref) <= GEMM_TOL


@pytest.mark.parametrize("kernel", ["streaming", "tiled"])
def test_capacity_layout_mlp_and_combine(kernel):
    """The routed-expert MLP in the fixed-capacity layout and the combine of its outputs (slots over
    the capacity are dropped and contribute nothing); the requantized h byte for byte on the kernel's
    h, and the calibration over the capacity rows."""
    cfg = gen.CONFIGS["t_mlp"]
    say("capacity layout mlp", kernel)
    E, H, I2, I, T, k = cfg.E, cfg.K, cfg.N, cfg.N // 2, cfg.T, cfg.k
    C = 32
    kf = mq.F_FORCE_DECODE if kernel == "streaming" else mq.F_FORCE_PREFILL
    w13 = np.stack([gen.weights_expert(cfg, 0, e, I2, H) for e in range(E)])
    w2 = np.stack([gen.weights_expert(cfg, 1, e, H, I) for e in range(E)])
    W13, W2 = mq.moesq_compress_weights(dev(w13)), mq.moesq_compress_weights(dev(w2))
    W13o, W2o = orc.compress(w13), orc.compress(w2)
    x = gen.activations(cfg, 0, T, H)
    ids, wts = gen.routing(cfg)
    R = orc.route(ids, E)
    exp, cap_rows, pre_rows = _capacity_rows(R, ids, C)
    assert (R["counts"] > C).any() and (R["counts"] < C).any()
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], k, R["offsets"], ga)
    # the oracle's scales over the rows the capacity layout keeps
    h_keep = orc.swiglu(orc.grouped_gemm(W13o, qo, so, ga, R["offsets"], pre_rows)).astype(np.float32)
    amax = np.zeros(E, np.float32)
    np.maximum.at(amax, cap_rows // C, np.abs(h_keep).max(axis=1))
    gh = np.array([orc.global_scale(float(a)) for a in amax], np.float32)
    rc = mq.moesq_route_capacity(dev(ids), E, C)
    assert np.array_equal(host(rc["slot_pos"]), exp)
    q, s = mq.moesq_quantize_act(dev(x), dev(ga), slot_pos=rc["slot_pos"], k=k, rows=E * C, capacity_experts=E)
    y2, ws = mq.moesq_expert_mlp(W13, W2, q, s, dev(ga), dev(gh), rc["counts"], y_dtype=torch.float32,
                                 flags=mq.F_DUMP_GATEUP | mq.F_DUMP_H | mq.F_CAPACITY | kf)
    hq, hs, dump = mq.mlp_workspace_views(ws, E * C, I, dump=True)
    M = orc.expert_mlp(W13o, W2o, qo, so, ga, gh, R["offsets"], pre_rows)
    gemm_gate(rows_of(dump, cap_rows), M["y13"], "capacity gate_up")
    flips = requant_gate(ws, E * C, I, gh, cap_rows, (cap_rows // C).astype(np.int32), M)
    # the down GEMM on the kernel's own codes, placed at the oracle's contiguous rows
    hq_k = np.zeros((int(R["offsets"][-1]), I // 2), np.uint8)
    hs_k = np.zeros((int(R["offsets"][-1]), I // 32), np.uint8)
    hq_k[pre_rows], hs_k[pre_rows] = rows_of(hq, cap_rows), rows_of(hs, cap_rows)
    gemm_gate(rows_of(y2, cap_rows), orc.grouped_gemm(W2o, hq_k, hs_k, gh, R["offsets"], pre_rows),
              "capacity down on the kernel's h")
    err = orc.rel_frobenius(rows_of(y2, cap_rows), M["y2"])
    say("capacity MLP y2 end-to-end rel-Frobenius", err, "h flips", flips)
    assert err <= 1e-2
    gcal, acal = mq.moesq_calibrate_gamma_h(W13, W2, q, s, dev(ga), rc["counts"], flags=mq.F_CAPACITY | kf)
    calibration_gate(gcal, acal, h_row_absmax(ws, E * C, I, cap_rows), cap_rows // C, E, gh)
    # combine over the capacity layout: the oracle on the same rows, dropped slots pointing at a zero row
    out = host(mq.moesq_unpermute_combine(y2, rc["slot_pos"], dev(wts), out_dtype=torch.float32))
    y_ext = np.concatenate([host(y2).astype(np.float64), np.zeros((1, H))])
    sp = np.where(exp >= 0, exp, E * C).astype(np.int32)
    assert orc.rel_frobenius(out, orc.combine(y_ext, sp, wts)) <= 1e-6


@pytest.mark.parametrize("name", ["c4", "c3_mlp"])
def test_mlp_parity_full_size(name):
    """The Kimi-shaped routed-expert MLP at full size (E=384, H=7168, I=2048, top-8): c4 (T=8192, Zipf,
    tiled kernels) and c3_mlp (T=64, uniform, bf16 tokens, weight-streaming kernels), with the f16
    operand copy from the quantizer and the per-expert intermediate scales of the oracle-only table
    (golden/gamma_h.txt). Stage by stage on the rows of sampled experts (c4: 16 experts, the busiest one
    on the first and last row of every 128-token tile): device-compressed weights (byte for byte),
    activation codes (all rows, bit-exact), gate_up (fp32 dump), the requantized h (byte for byte on the
    kernel's h), the down GEMM on the kernel's and on the oracle's h codes, the end-to-end chain
    (reported), the calibration call over all rows, and the combine."""
    cfg = gen.CONFIGS[name]
    E, H, I2, I, T, k = cfg.E, cfg.K, cfg.N, cfg.N // 2, cfg.T, cfg.k
    say("mlp", name, "full size: weights")
    W13, _ = device_weights(cfg, 0, E, I2, H, host_draw=False)
    W2, _ = device_weights(cfg, 1, E, H, I, host_draw=False)
    say("mlp", name, ": inputs")
    x = gen.activations(cfg, 0, T, H)
    xd = dev(x)
    if cfg.x_bf16:  # the oracle quantizes the same bf16 values
        xd = xd.to(torch.bfloat16)
        x = xd.float().cpu().numpy()
    ids, wts = gen.routing(cfg)
    R = orc.route(ids, E)
    off = R["offsets"]
    rows_all = int(off[-1])
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    gh, _, table_rows = gamma_h_table(name)
    assert np.array_equal(table_rows, R["counts"])   # the table was made for this routing
    qo, so = orc.dispatch_quantize(x, R["sorted_slot"], k, off, ga)
    say("mlp", name, ": quantize on the device")
    rt = mq.moesq_route_permute(dev(ids), E)
    q, s, xk = mq.moesq_quantize_act(xd, dev(ga), slot_pos=rt["slot_pos"], k=k, offsets=rt["offsets"], xk=True)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    say("mlp", name, ": expert MLP")
    y, ws = mq.moesq_expert_mlp(W13, W2, q, s, dev(ga), dev(gh), rt["offsets"], y_dtype=torch.float32,
                                flags=mq.F_DUMP_GATEUP | mq.F_DUMP_H, xk=xk)
    if name == "c4":
        rows, experts = sample_tile_rows(off, n_experts=16, per_expert=64)
    else:
        rows, experts = sample_expert_rows(off, n_experts=24, per_expert=8)
    say("mlp", name, ": oracle on experts", experts, "rows", rows.size)
    W13o = OracleWeights(cfg, 0, E, I2, H).ensure(experts)
    W2o = OracleWeights(cfg, 1, E, H, I).ensure(experts)
    _weights_bitexact(W13, W13o, experts, name + " gate_up")
    _weights_bitexact(W2, W2o, experts, name + " down")
    W13o, W2o = W13o.as_dict(), W2o.as_dict()
    M = orc.expert_mlp(W13o, W2o, qo, so, ga, gh, off, rows)
    _mlp_stage_gates(W2o, y, ws, rows_all, I, ga, gh, off, M, name, rows)
    # down GEMM alone on the oracle's h codes (other rows zero: rows are independent)
    hq_o = np.zeros((rows_all, I // 2), np.uint8)
    hs_o = np.zeros((rows_all, I // 32), np.uint8)
    hq_o[rows], hs_o[rows] = M["hq"], M["hs"]
    yd = mq.moesq_grouped_gemm(W2, dev(hq_o), dev(hs_o), dev(gh), dev(off), y_dtype=torch.float32)
    gemm_gate(rows_of(yd, rows), M["y2"], name + " down on the oracle's h")
    # calibration over all rows (the same kernel family and operand as the MLP call above)
    gcal, acal = mq.moesq_calibrate_gamma_h(W13, W2, q, s, dev(ga), rt["offsets"], xk=xk)
    all_rows = np.arange(rows_all)
    calibration_gate(gcal, acal, h_row_absmax(ws, rows_all, I, all_rows), orc.expert_of_rows(off, all_rows), E, gh)
    del y, ws, yd
    # combine at full size on a generated expert output, sampled tokens
    say("mlp", name, ": combine")
    y2 = gen.normal(5, gen.act_stream(12), rows_all * H).reshape(rows_all, H)
    yt = torch.from_numpy(y2).to(torch.bfloat16)
    out = host(mq.moesq_unpermute_combine(yt.to(DEV), rt["slot_pos"], dev(wts), out_dtype=torch.float32))
    toks = np.sort(np.random.default_rng(1).choice(T, 64, replace=False))
    sp = R["slot_pos"].reshape(T, k)[toks].ravel()
    # the sampled tokens as a problem of their own: their k rows each, in (token, slot) order
    ref = orc.combine(yt[torch.from_numpy(sp)].to(torch.float64).numpy(), np.arange(sp.size, dtype=np.int32),
                      wts[toks])
    assert orc.rel_frobenius(out[toks], ref) <= 1e-6


# ---------------------------------------------------------------- dense NVFP4 control ----------
def _dense_layout_reference(codes, scale):
    """The dense control's kernel layout built with numpy from its definition: per 64-row group and
    256-K super-step a 9216-byte unit; lane l = 16c + r of fragment j owns 32 code bytes at
    2048 j + 32 l (words of 8-groups g(S, h) = 8 (c>>1) + 2 S + (c&1) + 16 h in the order S0h0, S0h1,
    ..., S3h1, nibbles reordered to 0,2,4,6,1,3,5,7) and 4 scale bytes at 8192 + 16 l + 4 j (blocks
    2q, 4+2q, 2q+1, 5+2q of the super-step, q = c>>1)."""
    E, N, K2 = codes.shape
    K = 2 * K2
    nss, G = K // 256, N // 64
    words = np.ascontiguousarray(codes.reshape(E, N, nss, 32, 4)).view(np.uint32)[..., 0]   # [e, row, ss, group]
    order = [0, 2, 4, 6, 1, 3, 5, 7]
    reo = np.zeros_like(words)
    for i, src in enumerate(order):
        reo |= ((words >> np.uint32(4 * src)) & np.uint32(15)) << np.uint32(4 * i)
    out = np.zeros((E, G, nss, 9216), np.uint8)
    rows = reo.reshape(E, G, 4, 16, nss, 32)            # [e, g, j, r, ss, group]
    sc = scale.reshape(E, G, 4, 16, nss, 8)             # [e, g, j, r, ss, block]
    for c in range(4):
        q = c >> 1
        for S in range(4):
            for h in range(2):
                grp = 8 * q + 2 * S + (c & 1) + 16 * h
                wv = rows[..., grp].transpose(0, 1, 4, 2, 3)                                # [e, g, ss, j, r]
                for j in range(4):
                    off = 2048 * j + 32 * (16 * c) + 4 * (2 * S + h)
                    byt = np.ascontiguousarray(wv[:, :, :, j, :]).view(np.uint8).reshape(E, G, nss, 16, 4)
                    for r in range(16):
                        out[:, :, :, off + 32 * r: off + 32 * r + 4] = byt[:, :, :, r, :]
        blocks = [2 * q, 4 + 2 * q, 2 * q + 1, 5 + 2 * q]
        for j in range(4):
            for r in range(16):
                l = 16 * c + r
                for b, blk in enumerate(blocks):
                    out[:, :, :, 8192 + 16 * l + 4 * j + b] = sc[:, :, j, r, :, blk]
    return out.reshape(-1)


def _dense_case(name):
    key = ("dense", name)
    if key in _dense_cache:
        return _dense_cache[key]
    c = single_case(name)
    cfg, E, N, K = c["cfg"], c["E"], c["N"], c["K"]
    w = np.stack([gen.weights_expert(cfg, 0, e, N, K) for e in range(E)])
    Wo = orc.compress_dense(w)
    Wg = mq.compress_dense_weights(dev(w))
    out = dict(c, Wdo=Wo, Wdg=Wg)
    _dense_cache[key] = out
    return out


_dense_cache = {}


@pytest.mark.parametrize("name", ["c0", "t_zipf"])
def test_dense_compress_and_layout(name):
    c = _dense_case(name)
    say("dense compress + layout", name)
    Wg, Wo = c["Wdg"], c["Wdo"]
    assert np.array_equal(host(Wg.codes), Wo["codes"])
    assert np.array_equal(host(Wg.scale), Wo["scale"])
    assert np.array_equal(host(Wg.gscale), Wo["gscale"])
    assert np.array_equal(host(Wg.kl), _dense_layout_reference(Wo["codes"], Wo["scale"]))


@pytest.mark.parametrize("name", ["c0", "t_zipf", "c1", "c2"])
@pytest.mark.parametrize("flags", ["decode", "decode_xk", "prefill", "prefill_xk"])
def test_dense_gemm_parity(name, flags):
    """The dense NVFP4 control on every routed row (c2: all 32,768)."""
    c = _dense_case(name)
    say("dense gemm", name, flags)
    qo, so = _gemm_inputs(c)
    off = c["R"]["offsets"]
    fl = mq.F_FORCE_DECODE if flags.startswith("decode") else mq.F_FORCE_PREFILL
    xk = dev(_xk_reference(qo, so)) if flags.endswith("_xk") else None
    y = mq.moesq_dense_grouped_gemm(c["Wdg"], dev(qo), dev(so), dev(c["ga"]), dev(off), y_dtype=torch.float32,
                                    flags=fl, xk=xk)
    key = ("dense", name)
    if key not in _ref_cache:
        _ref_cache[key] = orc.dense_grouped_gemm(c["Wdo"], qo, so, c["ga"], off)
    rows = int(off[-1])
    gemm_gate(host(y)[:rows], _ref_cache[key], "dense gemm %s %s" % (name, flags))


def test_dense_kernel_on_unpacked_sparse_weights_matches_sparse_kernel():
    """The dense control on the sparse weights written out densely gives the sparse kernel's result
    (same values; only the MFMA instruction and summation order differ)."""
    c = single_case("t_zipf")
    say("dense vs sparse kernels t_zipf")
    qo, so = _gemm_inputs(c)
    off = c["R"]["offsets"]
    Wd = c["Wd"]
    dense = mq.moesq_unpack_weights(Wd)
    Wdd = mq.DenseWeights(dense, Wd.scale, Wd.gscale).prepack()
    for fl in (mq.F_FORCE_DECODE, mq.F_FORCE_PREFILL):
        ys = host(mq.moesq_grouped_gemm(Wd, dev(qo), dev(so), dev(c["ga"]), dev(off), y_dtype=torch.float32, flags=fl))
        yd = host(mq.moesq_dense_grouped_gemm(Wdd, dev(qo), dev(so), dev(c["ga"]), dev(off), y_dtype=torch.float32,
                                              flags=fl))
        assert orc.rel_frobenius(yd, ys) <= 1e-5


# ---------------------------------------------------------------- graph replay -----------------
@pytest.mark.parametrize("fused,streaming_xk", [(False, False), (True, False), (True, True)])
def test_graph_replays_match_eager_step(fused, streaming_xk):
    """The benchmark times HIP-graph replays of a whole step. Capture the t_mlp chain (route ->
    scatter-quantize -> MLP -> combine; routing and quantization as two calls or as one; the tiled
    MLP on the NVFP4 codes, or the weight-streaming MLP on the quantizer's f16 copy as the decode
    layer runs it) once, replay it several times with eager work and synchronization in between, and
    compare every replay with the eager result, bit for bit."""
    cfg = gen.CONFIGS["t_mlp"]
    say("graph replay t_mlp fused", fused, "streaming_xk", streaming_xk)
    E, H, I2, I, T, k = cfg.E, cfg.K, cfg.N, cfg.N // 2, cfg.T, cfg.k
    w13 = np.stack([gen.weights_expert(cfg, 0, e, I2, H) for e in range(E)])
    w2 = np.stack([gen.weights_expert(cfg, 1, e, H, I) for e in range(E)])
    W13, W2 = mq.moesq_compress_weights(dev(w13)), mq.moesq_compress_weights(dev(w2))
    x = dev(gen.activations(cfg, 0, T, H))
    ids, wts = gen.routing(cfg)
    ids_d, wts_d = dev(ids), dev(wts)
    ga = mq.moesq_global_scale(x).expand(E).contiguous()
    gh = torch.full((E,), cfg.gamma_h, dtype=torch.float32, device=DEV)
    rows = T * k
    rt = mq.moesq_route_permute(ids_d, E)
    q = torch.empty((rows, H // 2), dtype=torch.uint8, device=DEV)
    s = torch.empty((rows, H // 32), dtype=torch.uint8, device=DEV)
    ws = mq.mlp_workspace(rows, I, False, DEV)
    y2 = torch.empty((rows, H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    xk = torch.empty((rows, H), dtype=torch.float16, device=DEV) if streaming_xk else None
    kf = mq.F_FORCE_DECODE if streaming_xk else 0

    def step():
        if fused:
            mq.moesq_route_quantize(ids_d, E, x, ga, rt=rt, q=q, s=s, xk=xk)
        else:
            mq.moesq_route_permute(ids_d, E, rt["counts"], rt["offsets"], rt["sorted_slot"], rt["slot_pos"])
            mq.moesq_quantize_act(x, ga, slot_pos=rt["slot_pos"], k=k, offsets=rt["offsets"], q=q, s=s)
        mq.moesq_expert_mlp(W13, W2, q, s, ga, gh, rt["offsets"], y=y2, workspace=ws, xk=xk, flags=kf)
        mq.moesq_unpermute_combine(y2, rt["slot_pos"], wts_d, out=out)

    step()
    ref = host(out.view(torch.int16)).copy()
    ref_q = host(q).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.zero_()
        q.zero_()
        rt["slot_pos"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out.view(torch.int16)), ref), i
        assert np.array_equal(host(q), ref_q), i
        _ = torch.ones(1024, device=DEV).sum()          # unrelated eager work between replays
