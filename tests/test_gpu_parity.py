"""GPU parity of every step against the CPU oracle, through the C ABI.

Integer results (routing ids, counts, offsets, permutation maps, MXFP8 codes
and scales) must match bit for bit; bf16 outputs within a max relative error
of 1e-2; MXFP8 GEMM outputs within 2e-2 relative L2 of the oracle fed the
identical quantised operands.  Shapes are small enough for the oracle but
span several 256-wide tiles with ragged tails and empty groups.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from dropless_moe_expert_amd import inputs
from gpu_util import (BF16_TOL, MX_TOL, W_RTOL, bf16, check_route_fused, dev, host_u16, max_rel_err, rel_l2,
                      say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    from dropless_moe_expert_amd import ops as _ops
    _ops.load_library()
    return _ops


# ------------------------------------------------------------------- routing

@pytest.mark.parametrize("T,E,K,renorm", [(300, 8, 2, 1), (1000, 128, 8, 1), (77, 256, 8, 1), (64, 4, 1, 1),
                                          (50, 32, 32, 1), (129, 60, 5, 0), (0, 8, 2, 1),
                                          # E not a multiple of the lane's chunk: one load per logit
                                          (513, 130, 9, 0), (300, 7, 7, 1),
                                          # more picks than lanes per token: several slots per lane
                                          (1000, 64, 16, 1), (16384, 128, 8, 1)])
def test_route_topk(ops, T, E, K, renorm):
    say("route", T, E, K, renorm)
    rng = np.random.default_rng(T * 7 + E)
    l = rng.standard_normal((T, E)).astype(np.float32)
    if T:
        l[:, ::3] = np.round(l[:, ::3] * 2) / 2     # many exact ties
    ids_ref, w_ref = orc.route_topk(l, K, renormalize=bool(renorm))
    ids, w = ops.route_topk(dev(torch.from_numpy(l)), K, renormalize=bool(renorm))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=W_RTOL, atol=1e-30)


@pytest.mark.parametrize("E,K", [(8, 2), (128, 8), (200, 20)])
def test_route_topk_signed_zeros_and_infinities(ops, E, K):
    """-0 and +0 are equal logits (the lower expert first), -inf logits are
    picked after every finite one and among themselves by index, and a row
    of only -inf picks the K lowest experts with NaN weights, as the oracle
    does."""
    say("route special", E, K)
    rng = np.random.default_rng(E)
    T = 96
    l = rng.standard_normal((T, E)).astype(np.float32)
    l[0::4, ::2] = 0.0
    l[0::4, 1::2] = -0.0
    l[1::4, : E - K // 2] = -np.inf             # fewer finite logits than picks
    l[2::4] = -np.inf
    l[3::4, ::3] = np.float32(3.0)
    ids_ref, w_ref = orc.route_topk(l, K)
    ids, w = ops.route_topk(dev(torch.from_numpy(l)), K)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_array_equal(ids_ref[2], np.arange(K))
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=W_RTOL, atol=1e-30)


# -------------------------------------------------------------- fused router

@pytest.mark.parametrize("T,d,E,K,renorm,bias_std", [
    (256, 128, 8, 2, 1, 0.0),      # 16-token blocks, experts padded to 32
    (1000, 256, 60, 6, 0, 1.5),    # 32-token blocks, ragged tail, E not a multiple of 16
    (777, 512, 128, 8, 1, 1.5),    # 64-token blocks, ragged tail
    (300, 96, 256, 20, 1, 1.0),    # 256 experts, d not a multiple of a stage, 32-slot lists
    (70, 32, 1, 1, 1, 0.0),        # one expert, the smallest d
    (64, 64, 16, 16, 0, 0.0),      # K = E
    (33, 4096, 32, 32, 1, 0.5),    # K = E = 32, long contraction
    (0, 64, 8, 2, 1, 0.0),
])
def test_route_fused(ops, T, d, E, K, renorm, bias_std):
    say("route fused", T, d, E, K, renorm, bias_std)
    rng = np.random.default_rng(T * 13 + E * 7 + d)
    x = bf16(rng, T, d)
    wr = bf16(rng, E, d, scale=1.0 / np.sqrt(d))
    bias = torch.from_numpy((rng.standard_normal(E) * bias_std).astype(np.float32)) if bias_std else None
    n_near, _ = check_route_fused(ops, x, wr, bias, K, bool(renorm))
    assert n_near <= max(2, T // 50), n_near


def test_route_fused_ties_and_tiny_workload(ops):
    """Exact ties (duplicated router rows score identically on both sides:
    the lower expert comes first) and the tiny workload's router, whose bias
    keeps expert 7 empty."""
    say("route fused ties")
    rng = np.random.default_rng(5)
    T, d, E, K = 200, 128, 16, 4
    w = rng.standard_normal((E, d)).astype(np.float32) / np.sqrt(d)
    w[1::2] = w[0::2]                 # experts 2j and 2j + 1 identical
    wr = inputs.to_bf16(w)
    x = bf16(rng, T, d)
    _, out = check_route_fused(ops, x, wr, None, K)
    lg = out["logits"].cpu().numpy()
    assert np.array_equal(lg[:, 0::2], lg[:, 1::2])
    ids = out["topk_ids"].cpu().numpy()
    pos = {(t, int(e)): k for t in range(T) for k, e in enumerate(ids[t])}
    for t in range(T):
        for e in ids[t]:
            if e % 2 == 1:            # the odd twin is picked only after its even twin
                assert (t, int(e) - 1) in pos and pos[(t, int(e) - 1)] < pos[(t, int(e))]
    c = inputs.WORKLOADS["tiny"]
    x = inputs.workload("tiny", weights=False).x
    wr = inputs.router_weights(c["seed"], c["E"], c["d"])
    _, out = check_route_fused(ops, x, wr, inputs.expert_bias("tiny"), c["K"])
    assert not np.any(out["topk_ids"].cpu().numpy() == 7)


def test_route_fused_nan_and_unfused_agreement(ops):
    """A NaN in a token row raises the flag and scores -inf for that token
    (the lowest experts are then picked, as moe_route_topk does); on the same
    logits, moe_route_topk returns the fused kernel's ids."""
    say("route fused nan")
    rng = np.random.default_rng(9)
    T, d, E, K = 100, 256, 64, 8
    x = bf16(rng, T, d)
    x[17, 5] = float("nan")
    wr = bf16(rng, E, d, scale=1.0 / 16)
    flag = ops.new_flag("cuda")
    out = ops.route_fused(dev(x), dev(wr), K, keep_logits=True, flag=flag)
    ids2, w2 = ops.route_topk(out["logits"], K)
    torch.cuda.synchronize()
    assert int(flag.item()) & ops.FLAG_NAN_LOGIT
    ids = out["topk_ids"].cpu().numpy()
    assert ids[17].tolist() == list(range(K))
    assert np.all(np.isneginf(out["logits"][17].cpu().numpy()))
    np.testing.assert_array_equal(ids, ids2.cpu().numpy())
    ok = np.arange(T) != 17
    np.testing.assert_allclose(out["topk_w"].cpu().numpy()[ok], w2.cpu().numpy()[ok], rtol=W_RTOL)


# ------------------------------------------------------------------- permute

@pytest.mark.parametrize("T,E,K,d", [(256, 8, 2, 128), (3000, 128, 8, 64), (1, 4, 2, 8), (2049, 256, 8, 24),
                                     (700, 5, 1, 4096), (0, 8, 2, 16)])
def test_permute(ops, T, E, K, d):
    say("permute", T, E, K, d)
    rng = np.random.default_rng(T + E * 3)
    ids = np.array([rng.permutation(E)[:K] for _ in range(T)], dtype=np.int32).reshape(T, K)
    if T > 10:
        ids[: T // 3] = np.sort(ids[: T // 3], axis=1)     # skew: low experts more popular
    x = bf16(rng, T, d)
    sizes, offs, src, dst = orc.permute(ids, E)
    xp_ref = orc.gather_rows(x, src, K)
    out = ops.permute(dev(x), dev(torch.from_numpy(ids)), E)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["group_sizes"].cpu().numpy(), sizes)
    np.testing.assert_array_equal(out["group_offsets"].cpu().numpy(), offs)
    np.testing.assert_array_equal(out["perm_src"].cpu().numpy(), src)
    np.testing.assert_array_equal(out["perm_dst"].cpu().numpy(), dst)
    np.testing.assert_array_equal(host_u16(out["x_perm"]), xp_ref)


@pytest.mark.parametrize("T,E,K,d", [(256, 8, 2, 128), (3000, 128, 8, 64), (1, 4, 2, 32), (513, 6, 3, 96),
                                     (0, 8, 2, 32)])
def test_permute_mxfp8(ops, T, E, K, d):
    """Permute writing MXFP8 rows: maps as moe_permute, codes and scales bit
    for bit those of quantising the oracle's permuted bf16 rows."""
    say("permute mxfp8", T, E, K, d)
    rng = np.random.default_rng(T + 7 * E)
    ids = np.array([rng.permutation(E)[:K] for _ in range(T)], dtype=np.int32).reshape(T, K)
    x = bf16(rng, T, d, scale=3.0)
    sizes, offs, src, dst = orc.permute(ids, E)
    xq_ref, xs_ref = orc.mxfp8_quantize(orc.gather_rows(x, src, K), 0)
    out = ops.permute_mxfp8(dev(x), dev(torch.from_numpy(ids)), E)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["group_sizes"].cpu().numpy(), sizes)
    np.testing.assert_array_equal(out["group_offsets"].cpu().numpy(), offs)
    np.testing.assert_array_equal(out["perm_src"].cpu().numpy(), src)
    np.testing.assert_array_equal(out["perm_dst"].cpu().numpy(), dst)
    np.testing.assert_array_equal(out["xq"].cpu().numpy(), xq_ref.reshape(T * K, d))
    np.testing.assert_array_equal(out["xs"].cpu().numpy(), xs_ref.reshape(T * K, d // 32))


def test_routed_layer_mxfp8(ops):
    """The routed MXFP8 forward (permute writing MXFP8, gate/up quantising its
    output, down, combine) against the oracle applying the same quantisation
    at the same points."""
    say("routed mxfp8 layer")
    T, d, E, K, f = 600, 256, 8, 2, 256
    L = inputs.routed_layer("mx", T, d, E, K, f, 71, bias_std=1.0)
    lg, x, w1p, w2 = dev(L.logits), dev(L.x), dev(L.w1p), dev(L.w2)
    w1q, w1s = ops.quantize_weights(w1p)
    w2q, w2s = ops.quantize_weights(w2)
    w1k = ops.pack_weights_mxfp8(w1q, w1s, ops.MOE_EPI_SWIGLU)
    w2k = ops.pack_weights_mxfp8(w2q, w2s)
    y, parts = ops.moe_forward_mxfp8(lg, x, w1k, w2k, K)
    torch.cuda.synchronize()
    ids, w = orc.route_topk(L.logits, K)
    sizes, offs, src, dst = orc.permute(ids, E)
    xq, xs = orc.mxfp8_quantize(orc.gather_rows(L.x, src, K), 0)
    q1, s1 = orc.mxfp8_quantize(orc.u16(L.w1p).reshape(-1, d), 0)
    q2, s2 = orc.mxfp8_quantize(orc.u16(L.w2).reshape(-1, f), 0)
    h = orc.mx_grouped_gemm(xq, xs, q1.reshape(E, 2 * f, d), s1.reshape(E, 2 * f, d // 32), sizes, swiglu=True)
    hq, hs = orc.mxfp8_quantize(h, 0)
    yp = orc.mx_grouped_gemm(hq, hs, q2.reshape(E, d, f), s2.reshape(E, d, f // 32), sizes)
    y_ref = orc.unpermute_combine(yp, w, dst, T, K)
    np.testing.assert_array_equal(parts["ids"].cpu().numpy(), ids)
    np.testing.assert_array_equal(parts["xq"].cpu().numpy(), xq)
    assert rel_l2(y, y_ref) <= MX_TOL


def test_permute_maps_only_and_deterministic(ops):
    rng = np.random.default_rng(5)
    T, E, K = 5000, 64, 6
    ids = dev(torch.from_numpy(np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)))
    a = ops.permute(None, ids, E)
    b = ops.permute(None, ids, E)
    for k in ("group_sizes", "group_offsets", "perm_src", "perm_dst"):
        assert torch.equal(a[k], b[k])


# ------------------------------------------------------------------- grouped GEMM

SIZES = [np.array([0, 300, 1, 0, 517], np.int32),            # empty first/middle, ragged tails
         np.array([256, 255, 257, 0], np.int32),               # tile edges, empty last
         np.array([5], np.int32),
         np.array([0, 0, 0], np.int32)]                         # nothing to do


@pytest.mark.parametrize("si", range(len(SIZES)))
@pytest.mark.parametrize("N,Kd", [(512, 192), (264, 64)])
def test_grouped_gemm_nk(ops, si, N, Kd):
    sizes = SIZES[si]
    say("gg nk", sizes.tolist(), N, Kd)
    rng = np.random.default_rng(si * 10 + N)
    G, M = sizes.size, int(sizes.sum())
    m_cap = M + 37                                           # rows past the groups must stay untouched
    A, B = bf16(rng, m_cap, Kd), bf16(rng, G, N, Kd, scale=Kd ** -0.5)
    ref = orc.grouped_gemm(A, B, sizes)
    C = torch.full((m_cap + 64, N), 7.0, dtype=torch.bfloat16, device="cuda")
    ops.grouped_gemm(dev(A), dev(B), dev(torch.from_numpy(sizes)), out=C[:m_cap])
    torch.cuda.synchronize()
    if M:
        assert max_rel_err(C[:M], ref) <= BF16_TOL
    assert torch.all(C[M:] == 7.0)
    # fp32 output
    C32 = ops.grouped_gemm(dev(A), dev(B), dev(torch.from_numpy(sizes)), out_dtype=torch.float32)
    if M:
        r = orc.bf16_to_f64(ref)
        assert np.abs(C32[:M].cpu().double().numpy() - r).max() <= 1e-2 * np.abs(r).max()


@pytest.mark.parametrize("f,Kd", [(384, 128), (200, 64), (128, 320)])
def test_grouped_gemm_swiglu(ops, f, Kd):
    sizes = np.array([3, 0, 400, 129, 0, 1], np.int32)
    say("gg swiglu", f, Kd)
    rng = np.random.default_rng(f + Kd)
    G, M = sizes.size, int(sizes.sum())
    A, W = bf16(rng, M, Kd), bf16(rng, G, 2 * f, Kd, scale=Kd ** -0.5)
    h_ref, gu_ref = orc.gemm_swiglu(A, W, sizes, keep_gu=True)
    h, gu = ops.grouped_gemm(dev(A), dev(W), dev(torch.from_numpy(sizes)), epilogue=ops.MOE_EPI_SWIGLU,
                             keep_aux=True)
    torch.cuda.synchronize()
    assert max_rel_err(h, h_ref) <= BF16_TOL
    assert max_rel_err(gu, gu_ref) <= BF16_TOL


@pytest.mark.parametrize("N,Kd", [(512, 192), (264, 64), (8, 128)])
def test_grouped_gemm_packed_weights(ops, N, Kd):
    """Weights in the packed tile-stage layout give the oracle's result and the
    very bits of the plain [G, N, K] layout (same products, same order)."""
    sizes = np.array([0, 300, 1, 0, 517, 256], np.int32)
    say("gg packed", N, Kd)
    rng = np.random.default_rng(N + 3 * Kd)
    G, M = sizes.size, int(sizes.sum())
    A, B = bf16(rng, M, Kd), bf16(rng, G, N, Kd, scale=Kd ** -0.5)
    ref = orc.grouped_gemm(A, B, sizes)
    Bd, sz = dev(B), dev(torch.from_numpy(sizes))
    P = ops.pack_weights(Bd)
    C = ops.grouped_gemm(dev(A), P, sz)
    C_plain = ops.grouped_gemm(dev(A), Bd, sz)
    C32 = ops.grouped_gemm(dev(A), P, sz, out_dtype=torch.float32)
    C32_plain = ops.grouped_gemm(dev(A), Bd, sz, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert max_rel_err(C, ref) <= BF16_TOL
    assert torch.equal(C, C_plain) and torch.equal(C32, C32_plain)


@pytest.mark.parametrize("f,Kd", [(384, 128), (200, 64), (8, 64)])
def test_grouped_gemm_packed_weights_swiglu(ops, f, Kd):
    sizes = np.array([3, 0, 400, 129, 0, 1], np.int32)
    say("gg packed swiglu", f, Kd)
    rng = np.random.default_rng(7 * f + Kd)
    G, M = sizes.size, int(sizes.sum())
    A, W = bf16(rng, M, Kd), bf16(rng, G, 2 * f, Kd, scale=Kd ** -0.5)
    h_ref, gu_ref = orc.gemm_swiglu(A, W, sizes, keep_gu=True)
    Wd, sz = dev(W), dev(torch.from_numpy(sizes))
    P = ops.pack_weights(Wd, ops.MOE_EPI_SWIGLU)
    h, gu = ops.grouped_gemm(dev(A), P, sz, epilogue=ops.MOE_EPI_SWIGLU, keep_aux=True)
    h2, gu2 = ops.grouped_gemm(dev(A), Wd, sz, epilogue=ops.MOE_EPI_SWIGLU, keep_aux=True)
    torch.cuda.synchronize()
    assert max_rel_err(h, h_ref) <= BF16_TOL and max_rel_err(gu, gu_ref) <= BF16_TOL
    assert torch.equal(h, h2) and torch.equal(gu, gu2)
    with pytest.raises(ops.MoeError):          # packed for SwiGLU, used without it
        ops.grouped_gemm(dev(A), P, sz)


@pytest.mark.parametrize("N,Kd", [(256, 128), (200, 320), (8, 64)])
def test_grouped_gemm_kn_dgrad(ops, N, Kd):
    sizes = np.array([0, 260, 7, 0, 300], np.int32)
    say("gg kn", N, Kd)
    rng = np.random.default_rng(N * Kd)
    G, M = sizes.size, int(sizes.sum())
    dC = bf16(rng, M, Kd)
    B = bf16(rng, G, Kd, N, scale=Kd ** -0.5)                 # [G, K, N]: weight of a forward C = A B^T
    # oracle: dA = dC @ W with W = B[g] as [Kd(=forward N), N(=forward K)]
    ref = orc.grouped_dgrad(dC, B, sizes)
    out = ops.grouped_gemm(dev(dC), dev(B), dev(torch.from_numpy(sizes)), b_layout=ops.MOE_B_KN)
    torch.cuda.synchronize()
    assert max_rel_err(out, ref) <= BF16_TOL


@pytest.mark.parametrize("P,Q", [(136, 264), (256, 64), (8, 8)])
def test_grouped_gemm_wgrad(ops, P, Q):
    sizes = np.array([0, 70, 300, 0, 5, 64], np.int32)
    say("gg wgrad", P, Q)
    rng = np.random.default_rng(P + Q)
    G, M = sizes.size, int(sizes.sum())
    X, Y = bf16(rng, M + 9, P), bf16(rng, M + 9, Q)
    ref = orc.grouped_wgrad(X[:M], Y[:M], sizes)              # [G, P, Q]
    out = ops.grouped_gemm_wgrad(dev(X), dev(Y), dev(torch.from_numpy(sizes)))
    torch.cuda.synchronize()
    assert max_rel_err(out, ref) <= BF16_TOL
    for g in np.nonzero(sizes == 0)[0]:
        assert torch.all(out[g] == 0)


@pytest.mark.parametrize("P,Q,out_dtype", [(256, 256, "bf16"), (512, 768, "bf16"), (512, 264, "f32")])
def test_grouped_gemm_wgrad_many_groups(ops, P, Q, out_dtype):
    """300 groups, most of one or two stages, runs of empty groups between
    and at the ends, and one long group: every group against the oracle on
    its own scale (so a short group's error shows), empty ones exactly
    zero, and a repeat bit for bit.  Full 256 x 256 tiles and a partial
    column tile; bf16 and fp32 outputs."""
    rng = np.random.default_rng(P * 7 + Q)
    sizes = rng.integers(0, 41, 300).astype(np.int32)
    sizes[rng.random(300) < 0.25] = 0
    sizes[:3] = 0
    sizes[-4:] = 0
    sizes[150] = 2000
    sizes[151:160] = 0
    G, M = sizes.size, int(sizes.sum())
    say("gg wgrad many groups", P, Q, out_dtype, G, M)
    X, Y = bf16(rng, M + 5, P), bf16(rng, M + 5, Q)
    ref = orc.grouped_wgrad(X[:M], Y[:M], sizes)
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    S = dev(torch.from_numpy(sizes))
    out = ops.grouped_gemm_wgrad(dev(X), dev(Y), S, out_dtype=dt)
    again = ops.grouped_gemm_wgrad(dev(X), dev(Y), S, out_dtype=dt)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    got = out.float().cpu().numpy().astype(np.float64)
    want = orc.bf16_to_f64(ref)
    for g in range(G):
        if sizes[g] == 0:
            assert not np.any(got[g]), g
        else:   # each group against its own scale, so a short group's error shows
            assert np.abs(got[g] - want[g]).max() <= BF16_TOL * np.abs(want[g]).max(), g


def test_grouped_gemm_wgrad_queues(ops):
    # The weight-gradient kernel takes tiles from per-launch counters that its
    # last workgroup resets: consecutive launches of different shapes (a grid
    # of fewer than 8 workgroups, then many groups of skewed sizes, so
    # workgroups take tiles from other queues) must each match the oracle, and
    # a repeated launch must match bit for bit.
    rng = np.random.default_rng(97)
    cases = [(8, 8, np.array([3, 0, 40], np.int32)),
             (136, 264, np.concatenate([[900, 0, 0], rng.integers(0, 120, 37)]).astype(np.int32)),
             (8, 8, np.array([3, 0, 40], np.int32))]
    first = None
    for i, (P, Q, sizes) in enumerate(cases):
        say("gg wgrad queues", i, P, Q, sizes.size)
        G, M = sizes.size, int(sizes.sum())
        r = np.random.default_rng(P + Q + G)
        X, Y = bf16(r, M + 3, P), bf16(r, M + 3, Q)
        ref = orc.grouped_wgrad(X[:M], Y[:M], sizes)
        out = ops.grouped_gemm_wgrad(dev(X), dev(Y), dev(torch.from_numpy(sizes)))
        again = ops.grouped_gemm_wgrad(dev(X), dev(Y), dev(torch.from_numpy(sizes)))
        torch.cuda.synchronize()
        assert max_rel_err(out, ref) <= BF16_TOL
        assert torch.equal(out, again)
        for g in np.nonzero(sizes == 0)[0]:
            assert torch.all(out[g] == 0)
        if i == 0:
            first = out
        if i == 2:
            assert torch.equal(out, first)


def test_grouped_gemm_wgrad_graph_replay_and_slot_wrap(ops):
    """The weight gradients' tile queues carry each call's epoch and are
    zeroed by the call's last workgroup: a captured call (whose epoch repeats
    on every replay) replayed with eager calls in between, and 140 eager
    calls in a row (every one of the 64 slots reused twice), all equal the
    first eager result bit for bit, in bf16 and in MXFP8."""
    rng = np.random.default_rng(131)
    sizes = np.concatenate([[700, 0], rng.integers(0, 90, 21)]).astype(np.int32)
    G, M = sizes.size, int(sizes.sum())
    say("gg wgrad graph + slots", G, M)
    P, Q = 136, 264
    Xh, Yh = bf16(rng, M + 3, P), bf16(rng, M + 3, Q)
    X, Y = dev(Xh), dev(Yh)
    S = dev(torch.from_numpy(sizes))
    ref = orc.grouped_wgrad(Xh[:M], Yh[:M], sizes)
    XqT, XsT = ops.mxfp8_quantize_transposed(X, S)
    YqT, YsT = ops.mxfp8_quantize_transposed(Y, S)
    calls = {"bf16": lambda: ops.grouped_gemm_wgrad(X, Y, S),
             "mxfp8": lambda: ops.grouped_gemm_wgrad_mxfp8(XqT, XsT, YqT, YsT, S, M + 3)}
    for name, call in calls.items():
        eager = call()
        torch.cuda.synchronize()
        if name == "bf16":
            assert max_rel_err(eager, ref) <= BF16_TOL
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            call()
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            out = call()
        for rep in range(4):
            out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), (name, rep)
            between = call()
            torch.cuda.synchronize()
            assert torch.equal(between, eager), (name, rep)
        for i in range(140):
            got = call()
        torch.cuda.synchronize()
        assert torch.equal(got, eager), name
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), name


# ------------------------------------------------------------------- MXFP8

@pytest.mark.parametrize("R,C", [(300, 256), (1, 32), (1000, 7168 // 4)])
def test_mxfp8_quantize_axis0(ops, R, C):
    say("mx q0", R, C)
    rng = np.random.default_rng(R + C)
    x32 = (rng.standard_normal((R, C)) * np.exp(rng.uniform(-30, 30, (R, 1)))).astype(np.float32)
    x32[0, :32] = 0.0
    if R > 2:
        x32[1, :32] = -0.0
        x32[2, :32] = np.float32(1e-39)     # subnormal block
    x = inputs.to_bf16(x32)
    q_ref, s_ref = orc.mxfp8_quantize(x, 0)
    q, s = ops.mxfp8_quantize(dev(x), 0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


def test_mxfp8_quantize_axis0_valid_rows_only(ops):
    rng = np.random.default_rng(9)
    sizes = np.array([3, 0, 40], np.int32)
    x = bf16(rng, 60, 64)
    q_ref, s_ref = orc.mxfp8_quantize(x[:43], 0)
    q = torch.full((60, 64), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((60, 2), 0xCD, dtype=torch.uint8, device="cuda")
    L = ops.lib()
    xd, sd = dev(x), dev(torch.from_numpy(sizes))     # keep both alive until the kernel has run
    st = L.mxfp8_group_quantize(ops._ptr(xd), 60, 64, 0, ops._ptr(sd), 3, ops._ptr(q), ops._ptr(s), None,
                                ops._stream(q.device))
    torch.cuda.synchronize()
    assert st == 0
    np.testing.assert_array_equal(q[:43].cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s[:43].cpu().numpy(), s_ref)
    assert torch.all(q[43:] == 0xAB) and torch.all(s[43:] == 0xCD)


def test_mxfp8_quantize_axis1_grouped(ops):
    say("mx q1")
    rng = np.random.default_rng(10)
    sizes = np.array([0, 5, 32, 33, 0, 70, 1], np.int32)
    M, C = int(sizes.sum()), 48
    x = inputs.to_bf16((rng.standard_normal((M, C)) * 3).astype(np.float32))
    q_ref, s_ref = orc.mxfp8_quantize(x, 1, sizes)
    q, s = ops.mxfp8_quantize(dev(x), 1, dev(torch.from_numpy(sizes)))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s[: s_ref.shape[0]].cpu().numpy(), s_ref)


def _to_transposed(q, s, sizes, k_cap):
    """The oracle's axis-1 codes/scales laid out as mxfp8_quantize_transposed
    stores them (groups 64-aligned along each column's row of positions); the
    padding positions are zero codes and, for blocks with no rows, scale 0."""
    C = q.shape[1]
    qT = np.zeros((C, k_cap), np.uint8)
    sT = np.zeros((C, k_cap // 32), np.uint8)
    o = P = K = 0
    for n in sizes:
        n = int(n)
        qT[:, K:K + n] = q[o:o + n].T
        nb = (n + 31) // 32
        sT[:, K // 32:K // 32 + nb] = s[P:P + nb].T
        o, P, K = o + n, P + nb, K + (n + 63) // 64 * 64
    return qT, sT, K


def test_mxfp8_quantize_transposed(ops):
    rng = np.random.default_rng(12)
    # grouped: empty groups, short last blocks, a group of exactly 64 rows
    sizes = np.array([0, 5, 64, 33, 0, 70, 1], np.int32)
    M, C = int(sizes.sum()), 56
    say("mx qT grouped", M, C)
    x = inputs.to_bf16((rng.standard_normal((M + 7, C)) * 3).astype(np.float32))
    q_ref, s_ref = orc.mxfp8_quantize(x[:M], 1, sizes)
    qT, sT = ops.mxfp8_quantize_transposed(dev(x), dev(torch.from_numpy(sizes)))
    torch.cuda.synchronize()
    want_q, want_s, used = _to_transposed(q_ref, s_ref, sizes, qT.shape[1])
    np.testing.assert_array_equal(qT[:, :used].cpu().numpy(), want_q[:, :used])
    np.testing.assert_array_equal(sT[:, :used // 32].cpu().numpy(), want_s[:, :used // 32])
    # both layouts from one read (cols % 32 == 0): the axis-0 part as the axis-0 oracle
    x2 = inputs.to_bf16((rng.standard_normal((M + 7, 96)) * 3).astype(np.float32))
    q_ref, s_ref = orc.mxfp8_quantize(x2[:M], 1, sizes)
    q0_ref, s0_ref = orc.mxfp8_quantize(x2[:M], 0)
    qT, sT, q0, s0 = ops.mxfp8_quantize_transposed(dev(x2), dev(torch.from_numpy(sizes)), rows_too=True)
    torch.cuda.synchronize()
    want_q, want_s, used = _to_transposed(q_ref, s_ref, sizes, qT.shape[1])
    np.testing.assert_array_equal(qT[:, :used].cpu().numpy(), want_q[:, :used])
    np.testing.assert_array_equal(sT[:, :used // 32].cpu().numpy(), want_s[:, :used // 32])
    np.testing.assert_array_equal(q0[:M].cpu().numpy(), q0_ref)
    np.testing.assert_array_equal(s0[:M].cpu().numpy(), s0_ref)
    # batched (weights): G batches of 128 rows, each one group
    G, R, C2 = 3, 128, 96
    say("mx qT batched", G, R, C2)
    w = inputs.to_bf16((rng.standard_normal((G, R, C2)) * 0.05).astype(np.float32))
    qT, sT, q0, s0 = ops.mxfp8_quantize_transposed(dev(w), rows_too=True)
    torch.cuda.synchronize()
    for g in range(G):
        q_ref, s_ref = orc.mxfp8_quantize(w[g], 1, np.array([R], np.int32))
        np.testing.assert_array_equal(qT[g].cpu().numpy(), q_ref.T)
        np.testing.assert_array_equal(sT[g].cpu().numpy(), s_ref.T)
        q_ref, s_ref = orc.mxfp8_quantize(w[g], 0)
        np.testing.assert_array_equal(q0[g].cpu().numpy(), q_ref)
        np.testing.assert_array_equal(s0[g].cpu().numpy(), s_ref)


@pytest.mark.parametrize("T,E,K,C", [(150, 9, 3, 96), (8192, 64, 8, 512)])
def test_mxfp8_quantize_gathered(ops, T, E, K, C):
    # the permuted rows quantised both ways straight from their tokens, as
    # the oracle quantises its own x_perm (no weights) and its own
    # combine-backward dy_perm (weights), bit for bit; the oracle's perm_src
    # drives the gather.  The second case gives every workgroup several
    # tiles (the prefetch of the next tile's pairs and rows); the last
    # expert receives no token.
    rng = np.random.default_rng(T + C)
    ids = np.stack([rng.choice(E - 1, K, replace=False) for _ in range(T)]).astype(np.int32)
    sizes, _, src, dst = orc.permute(ids, E)
    assert sizes[-1] == 0
    M = T * K
    say("mx gathered", T, E, K, C)
    x = bf16(rng, T, C, scale=3.0)
    w = rng.dirichlet(np.ones(K), T).astype(np.float32)
    refs = {
        False: orc.gather_rows(x, src, K),
        True: orc.combine_backward(x, np.zeros((M, C), np.uint16), w, dst, K)[0],
    }
    S, SRC = dev(torch.from_numpy(sizes)), dev(torch.from_numpy(src))
    for weighted, ref in refs.items():
        q_ref, s_ref = orc.mxfp8_quantize(ref, 1, sizes)
        q0_ref, s0_ref = orc.mxfp8_quantize(ref, 0)
        tw = dev(torch.from_numpy(w)) if weighted else None
        for rows_too in (False, True):
            got = ops.mxfp8_quantize_gathered(dev(x), SRC, K, S, topk_w=tw, rows_too=rows_too)
            torch.cuda.synchronize()
            want_q, want_s, used = _to_transposed(q_ref, s_ref, sizes, got[0].shape[1])
            np.testing.assert_array_equal(got[0][:, :used].cpu().numpy(), want_q[:, :used])
            np.testing.assert_array_equal(got[1][:, :used // 32].cpu().numpy(), want_s[:, :used // 32])
            if rows_too:
                np.testing.assert_array_equal(got[2].cpu().numpy(), q0_ref)
                np.testing.assert_array_equal(got[3].cpu().numpy(), s0_ref)


def test_swiglu_backward_mxfp8(ops):
    # dgu delivered only as MXFP8 codes equals quantising the bf16 dgu, bit for bit
    rng = np.random.default_rng(44)
    sizes = np.array([3, 0, 70, 130], np.int32)
    M, f = int(sizes.sum()), 48
    say("swiglu bwd mxfp8", M, f)
    gu = dev(inputs.to_bf16((rng.standard_normal((M + 4, 2 * f)) * 2).astype(np.float32)))
    dh = dev(inputs.to_bf16(rng.standard_normal((M + 4, f)).astype(np.float32)))
    S = dev(torch.from_numpy(sizes))
    dgu = ops.swiglu_backward(gu, dh, S)
    want = ops.mxfp8_quantize_transposed(dgu, S, rows_too=True)
    got = ops.swiglu_backward_mxfp8(gu, dh, S)
    torch.cuda.synchronize()
    used = int(((sizes + 63) // 64 * 64).sum())
    assert torch.equal(got[0][:, :used], want[0][:, :used])
    assert torch.equal(got[1][:, :used // 32], want[1][:, :used // 32])
    assert torch.equal(got[2][:M], want[2][:M]) and torch.equal(got[3][:M], want[3][:M])
    ref = orc.swiglu_backward(host_u16(gu)[:M], host_u16(dh)[:M])
    assert max_rel_err(dgu[:M], ref) <= BF16_TOL


@pytest.mark.parametrize("P,Q", [(136, 264), (256, 64)])
def test_grouped_gemm_wgrad_mxfp8(ops, P, Q):
    # group-aware MXFP8 weight gradient: operands quantised down their rows by
    # the transposed quantiser (bit-exact with the oracle, tested above), the
    # GEMM against the oracle on the identical codes; groups that are empty,
    # shorter than a block, and longer than the 8 stages one scale piece covers
    rng = np.random.default_rng(P + 3 * Q)
    sizes = np.array([0, 5, 600, 33, 0, 130, 64, 1], np.int32)
    G, M = sizes.size, int(sizes.sum())
    say("gg wgrad mxfp8", P, Q, M)
    A = inputs.to_bf16((rng.standard_normal((M + 5, P)) * 2).astype(np.float32))
    B = inputs.to_bf16((rng.standard_normal((M + 5, Q)) * 0.5).astype(np.float32))
    aq, as_ = orc.mxfp8_quantize(A[:M], 1, sizes)
    bq, bs = orc.mxfp8_quantize(B[:M], 1, sizes)
    ref = orc.mx_grouped_wgrad(aq, as_, bq, bs, sizes)
    S = dev(torch.from_numpy(sizes))
    AqT, AsT = ops.mxfp8_quantize_transposed(dev(A), S)
    BqT, BsT = ops.mxfp8_quantize_transposed(dev(B), S)
    out = ops.grouped_gemm_wgrad_mxfp8(AqT, AsT, BqT, BsT, S, M + 5)
    again = ops.grouped_gemm_wgrad_mxfp8(AqT, AsT, BqT, BsT, S, M + 5)
    torch.cuda.synchronize()
    got = out.cpu()
    for g in range(G):
        if sizes[g] == 0:
            assert torch.all(got[g] == 0)
        else:
            assert rel_l2(got[g], ref[g]) <= MX_TOL, g
    assert torch.equal(out, again)


@pytest.mark.parametrize("swiglu", [False, True])
def test_grouped_gemm_mxfp8(ops, swiglu):
    sizes = np.array([0, 300, 1, 0, 260], np.int32)
    say("gg mxfp8", swiglu)
    rng = np.random.default_rng(11 + swiglu)
    G, M, N, Kd = sizes.size, int(sizes.sum()), 512, 384
    A, B = bf16(rng, M, Kd), bf16(rng, G, N, Kd, scale=Kd ** -0.5)
    aq, as_ = orc.mxfp8_quantize(A, 0)
    bq, bs = orc.mxfp8_quantize(orc.u16(B).reshape(-1, Kd), 0)
    bq, bs = bq.reshape(G, N, Kd), bs.reshape(G, N, Kd // 32)
    ref = orc.mx_grouped_gemm(aq, as_, bq, bs, sizes, swiglu=swiglu)
    t = lambda a: dev(torch.from_numpy(np.ascontiguousarray(a)))
    out = ops.grouped_gemm_mxfp8(t(aq), t(as_), t(bq), t(bs), t(sizes),
                                 epilogue=ops.MOE_EPI_SWIGLU if swiglu else ops.MOE_EPI_NONE)
    torch.cuda.synchronize()
    assert rel_l2(out[:M], ref) <= MX_TOL
    assert max_rel_err(out[:M], ref) <= 2 * BF16_TOL
    # the packed weight layout (codes and scales together) gives the same bits
    epi = ops.MOE_EPI_SWIGLU if swiglu else ops.MOE_EPI_NONE
    P = ops.pack_weights_mxfp8(t(bq), t(bs), epi)
    out_p = ops.grouped_gemm_mxfp8(t(aq), t(as_), P, None, t(sizes), epilogue=epi)
    torch.cuda.synchronize()
    assert torch.equal(out_p[:M], out[:M])


@pytest.mark.parametrize("packed", [False, True])
def test_grouped_gemm_mxfp8_fused_quant(ops, packed):
    """SwiGLU + MXFP8 quantisation in the gate/up GEMM's epilogue: codes and
    scales equal quantising the unfused bf16 h, bit for bit (several tiles,
    ragged tails, empty groups); against the oracle within the MXFP8 bound."""
    sizes = np.array([300, 0, 1, 517, 0, 33], np.int32)
    say("gg mxfp8 fused quant", packed)
    rng = np.random.default_rng(23 + packed)
    G, M, f, Kd = sizes.size, int(sizes.sum()), 320, 256
    A, B = bf16(rng, M, Kd), bf16(rng, G, 2 * f, Kd, scale=Kd ** -0.5)
    aq, as_ = orc.mxfp8_quantize(A, 0)
    bq, bs = orc.mxfp8_quantize(orc.u16(B).reshape(-1, Kd), 0)
    bq, bs = bq.reshape(G, 2 * f, Kd), bs.reshape(G, 2 * f, Kd // 32)
    t = lambda a: dev(torch.from_numpy(np.ascontiguousarray(a)))
    W = ops.pack_weights_mxfp8(t(bq), t(bs), ops.MOE_EPI_SWIGLU) if packed else t(bq)
    Ws = None if packed else t(bs)
    h = ops.grouped_gemm_mxfp8(t(aq), t(as_), W, Ws, t(sizes), epilogue=ops.MOE_EPI_SWIGLU)
    hq, hs = ops.mxfp8_quantize(h, 0, t(sizes))
    fq, fs = ops.grouped_gemm_mxfp8(t(aq), t(as_), W, Ws, t(sizes), epilogue=ops.MOE_EPI_SWIGLU_MXFP8)
    torch.cuda.synchronize()
    assert torch.equal(fq[:M], hq[:M]) and torch.equal(fs[:M], hs[:M])
    # oracle: its own h, quantised by its own rule; compare dequantised values
    h_ref = orc.mx_grouped_gemm(aq, as_, bq, bs, sizes, swiglu=True)
    q_ref, s_ref = orc.mxfp8_quantize(h_ref, 0)
    deq = lambda q, sc: orc.e4m3_to_f64(q) * np.exp2(np.repeat(sc.astype(np.float64) - 127, 32, axis=1))
    got = deq(fq[:M].cpu().numpy(), fs[:M].cpu().numpy())
    ref = deq(q_ref, s_ref)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= MX_TOL


@pytest.mark.parametrize("N,Kd", [(8, 128), (264, 256)])
def test_grouped_gemm_mxfp8_packed_narrow(ops, N, Kd):
    """Packed MXFP8 weights with a partial last n-tile (padding rows are zero)."""
    sizes = np.array([3, 0, 257], np.int32)
    say("gg mxfp8 packed", N, Kd)
    rng = np.random.default_rng(N + Kd)
    G, M = sizes.size, int(sizes.sum())
    A, B = bf16(rng, M, Kd), bf16(rng, G, N, Kd, scale=Kd ** -0.5)
    aq, as_ = orc.mxfp8_quantize(A, 0)
    bq, bs = orc.mxfp8_quantize(orc.u16(B).reshape(-1, Kd), 0)
    bq, bs = bq.reshape(G, N, Kd), bs.reshape(G, N, Kd // 32)
    ref = orc.mx_grouped_gemm(aq, as_, bq, bs, sizes, swiglu=False)
    t = lambda a: dev(torch.from_numpy(np.ascontiguousarray(a)))
    P = ops.pack_weights_mxfp8(t(bq), t(bs))
    out = ops.grouped_gemm_mxfp8(t(aq), t(as_), P, None, t(sizes))
    torch.cuda.synchronize()
    assert rel_l2(out[:M], ref) <= MX_TOL


# ------------------------------------------------------------------- combine and backward helpers

@pytest.mark.parametrize("T,K,d,weighted", [(300, 2, 128, True), (100, 8, 2048, True), (64, 4, 24, False)])
def test_unpermute_combine(ops, T, K, d, weighted):
    say("combine", T, K, d, weighted)
    rng = np.random.default_rng(T + K + d)
    E = 16
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    _, _, src, dst = orc.permute(ids, E)
    yp = bf16(rng, T * K, d)
    w = rng.dirichlet(np.ones(K), T).astype(np.float32) if weighted else None
    ref = orc.unpermute_combine(yp, w, dst, T, K)
    out = ops.unpermute_combine(dev(yp), None if w is None else dev(torch.from_numpy(w)),
                                dev(torch.from_numpy(dst)), T, K)
    torch.cuda.synchronize()
    assert max_rel_err(out, ref) <= BF16_TOL


def test_combine_backward_and_swiglu_backward(ops):
    say("combine bwd")
    rng = np.random.default_rng(21)
    T, K, d, E, f = 200, 4, 256, 12, 96
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    sizes, _, src, dst = orc.permute(ids, E)
    yp, dy = bf16(rng, T * K, d), bf16(rng, T, d)
    w = rng.dirichlet(np.ones(K), T).astype(np.float32)
    dyp_ref, dw_ref = orc.combine_backward(dy, yp, w, dst, K)
    dyp, dw = ops.combine_backward(dev(dy), dev(yp), dev(torch.from_numpy(w)), dev(torch.from_numpy(dst)), K)
    _, dw_only = ops.combine_backward(dev(dy), dev(yp), dev(torch.from_numpy(w)), dev(torch.from_numpy(dst)), K,
                                      weights_only=True)
    torch.cuda.synchronize()
    q_mx, s_mx, dw_mx = ops.combine_backward_mxfp8(dev(dy), dev(yp), dev(torch.from_numpy(w)),
                                                   dev(torch.from_numpy(dst)), K)
    torch.cuda.synchronize()
    # dy_perm: the exact product rounded once to bf16, bit for bit
    np.testing.assert_array_equal(host_u16(dyp), dyp_ref)
    assert torch.equal(dw_only, dw) and torch.equal(dw_mx, dw)
    # and delivered as MXFP8 rows: the oracle's codes of the oracle's dy_perm
    q_ref, s_ref = orc.mxfp8_quantize(dyp_ref, 0)
    np.testing.assert_array_equal(q_mx.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s_mx.cpu().numpy(), s_ref)
    np.testing.assert_allclose(dw.cpu().numpy(), dw_ref, rtol=1e-3, atol=1e-3 * np.abs(dw_ref).max())
    M = T * K
    gu, dh = bf16(rng, M, 2 * f, scale=2.0), bf16(rng, M, f)
    dgu_ref = orc.swiglu_backward(gu, dh)
    dgu = ops.swiglu_backward(dev(gu), dev(dh), dev(torch.from_numpy(sizes)))
    torch.cuda.synchronize()
    assert max_rel_err(dgu, dgu_ref) <= BF16_TOL


# ------------------------------------------------------------------- the tiny layer end to end

def test_tiny_layer_forward_backward(ops):
    say("tiny layer")
    L = inputs.workload("tiny")
    y_ref, saved_ref = orc.layer_forward(L.logits, L.x, L.w1p, L.w2, L.K, keep=True)
    g_ref = orc.layer_backward(L.dy, saved_ref, L.w1p, L.w2, L.K)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    y, saved = ops.moe_forward(dev(L.logits), dev(L.x), dev(L.w1p), dev(L.w2), L.K, keep=True, flag=flag)
    grads = ops.moe_backward(dev(L.dy), saved, dev(L.w1p), dev(L.w2), L.K, flag=flag, fused=False)
    fused = ops.moe_backward(dev(L.dy), saved, dev(L.w1p), dev(L.w2), L.K, flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    # SwiGLU's backward formed in the data-gradient GEMM's epilogue gives the
    # same bits as the GEMM's stored dh followed by the elementwise kernel
    assert fused["dh"] is None
    for k in ("dy_perm", "dgu", "dx_perm", "dx", "dw2", "dw1p"):
        assert torch.equal(fused[k], grads[k]), k
    np.testing.assert_array_equal(saved["ids"].cpu().numpy(), saved_ref["ids"])
    np.testing.assert_array_equal(saved["group_sizes"].cpu().numpy(), saved_ref["sizes"])
    assert saved_ref["sizes"][7] == 0
    np.testing.assert_array_equal(saved["perm_dst"].cpu().numpy(), saved_ref["perm_dst"])
    np.testing.assert_array_equal(host_u16(saved["x_perm"]), saved_ref["x_perm"])
    assert max_rel_err(saved["h"], saved_ref["h"]) <= BF16_TOL
    assert max_rel_err(saved["y_perm"], saved_ref["y_perm"]) <= BF16_TOL
    assert max_rel_err(y, y_ref) <= BF16_TOL
    for k in ("dy_perm", "dh", "dgu", "dx_perm", "dx", "dw2", "dw1p"):
        assert max_rel_err(grads[k], g_ref[k]) <= BF16_TOL, k
    dw = grads["dw"].cpu().numpy()
    np.testing.assert_allclose(dw, g_ref["dw"], rtol=1e-2, atol=1e-2 * np.abs(g_ref["dw"]).max())
    # expert 7 received nothing: its weight gradients are exact zeros
    assert torch.all(grads["dw2"][7] == 0) and torch.all(grads["dw1p"][7] == 0)


def test_tiny_layer_forward_backward_mxfp8(ops):
    # the training step with every GEMM in MXFP8 (the weight gradients
    # group-aware along the tokens) against the oracle that quantises the
    # same way, step by step
    say("tiny layer mxfp8")
    L = inputs.workload("tiny")
    y_ref, saved_ref = orc.layer_forward_mxfp8(L.logits, L.x, L.w1p, L.w2, L.K)
    g_ref = orc.layer_backward_mxfp8(L.dy, saved_ref, L.w1p, L.w2, L.K)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    wk = ops.quantize_weights_mxfp8_train(dev(L.w1p), dev(L.w2), flag=flag)
    y, saved = ops.moe_forward_mxfp8_train(dev(L.logits), dev(L.x), wk, L.K, flag=flag, fused=False)
    y_f, saved_f = ops.moe_forward_mxfp8_train(dev(L.logits), dev(L.x), wk, L.K, flag=flag)
    grads = ops.moe_backward_mxfp8(dev(L.dy), saved, wk, L.K, flag=flag, fused=False)
    fused = ops.moe_backward_mxfp8(dev(L.dy), saved_f, wk, L.K, flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    # the quantisers that gather their rows (x, dy) or form them (dgu)
    # themselves change no bit downstream
    assert saved_f["x_perm"] is None and fused["dy_perm"] is None and fused["dgu"] is None
    assert torch.equal(y_f, y)
    used = int(((saved_ref["sizes"] + 63) // 64 * 64).sum())   # written positions of the transposed codes
    for k in ("xT", "hT"):
        assert torch.equal(saved_f[k][:, :used], saved[k][:, :used]), k
    for k in ("xsT", "hsT"):
        assert torch.equal(saved_f[k][:, :used // 32], saved[k][:, :used // 32]), k
    M_all = int(saved_ref["sizes"].sum())
    for k in ("h", "gu", "y_perm"):
        assert torch.equal(saved_f[k][:M_all], saved[k][:M_all]), k
    for k in ("dw", "dh", "dw2", "dx_perm", "dw1p", "dx"):
        assert torch.equal(fused[k], grads[k]), k
    np.testing.assert_array_equal(saved["group_sizes"].cpu().numpy(), saved_ref["sizes"])
    M = int(saved_ref["sizes"].sum())
    for k, got in (("gu", saved["gu"]), ("h", saved["h"]), ("y_perm", saved["y_perm"])):
        assert rel_l2(got[:M], saved_ref[k]) <= MX_TOL, k
    assert rel_l2(y, y_ref) <= MX_TOL
    for k in ("dy_perm", "dh", "dgu", "dx_perm"):
        assert rel_l2(grads[k][:M], g_ref[k]) <= MX_TOL, k
    for k in ("dx", "dw2", "dw1p"):
        assert rel_l2(grads[k], g_ref[k]) <= MX_TOL, k
    assert torch.all(grads["dw2"][7] == 0) and torch.all(grads["dw1p"][7] == 0)


# ------------------------------------------------------------------- data errors: flags, bounds

def test_flags_bad_ids_stay_in_bounds(ops):
    say("flags ids")
    T, E, K, d = 100, 8, 2, 16
    rng = np.random.default_rng(31)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    ids[5, 0] = 9
    ids[7, 1] = -3
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = ops.permute(dev(bf16(rng, T, d)), dev(torch.from_numpy(ids)), E, flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & ops.FLAG_BAD_EXPERT_ID
    dst = out["perm_dst"].cpu().numpy()
    assert dst.min() >= 0 and dst.max() < T * K
    assert int(out["group_sizes"].sum()) == T * K
    np.testing.assert_array_equal(np.sort(dst), np.arange(T * K))


def test_flags_bad_sizes(ops):
    say("flags sizes")
    rng = np.random.default_rng(32)
    m_cap, Kd, N = 300, 64, 64
    A, B = bf16(rng, m_cap, Kd), bf16(rng, 3, N, Kd)
    buf = torch.full((m_cap + 40, N), 3.0, dtype=torch.bfloat16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    sizes = np.array([100, -5, 250], np.int32)        # negative, and 350 > m_cap
    ops.grouped_gemm(dev(A), dev(B), dev(torch.from_numpy(sizes)), out=buf[:m_cap], flag=flag)
    torch.cuda.synchronize()
    f = int(flag.item())
    assert f & ops.FLAG_NEGATIVE_SIZE and f & ops.FLAG_ROWS_OVER_CAP
    assert torch.all(buf[m_cap:] == 3.0)
    ref = orc.grouped_gemm(A, B, np.array([100, 0, 200], np.int32))   # the clamped reading
    assert max_rel_err(buf[:m_cap], ref) <= BF16_TOL


def test_flags_wgrad_sizes_past_int32(ops):
    """Weight-gradient sizes whose sum passes 2^31 (and a negative one): the
    offsets are summed in 64 bits and clamped to the rows given, so the
    flags rise and the first group contracts every given row while the rest
    are empty (zeros), the clamped reading of the oracle; no row outside the
    operands is read."""
    say("flags wgrad sizes")
    rng = np.random.default_rng(33)
    m_cap, P, Q = 300, 64, 64
    X, Y = bf16(rng, m_cap, P), bf16(rng, m_cap, Q)
    sizes = np.array([2 ** 30, 2 ** 30, 100, -7], np.int32)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = ops.grouped_gemm_wgrad(dev(X), dev(Y), dev(torch.from_numpy(sizes)), flag=flag)
    torch.cuda.synchronize()
    f = int(flag.item())
    assert f & ops.FLAG_NEGATIVE_SIZE and f & ops.FLAG_ROWS_OVER_CAP
    ref = orc.grouped_wgrad(X, Y, np.array([m_cap, 0, 0, 0], np.int32))
    assert max_rel_err(out, ref) <= BF16_TOL
    for g in (1, 2, 3):
        assert torch.all(out[g] == 0)


def test_flag_nan_logit(ops):
    l = torch.randn(4, 8)
    l[2, 3] = float("nan")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids, _ = ops.route_topk(dev(l), 2, flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & ops.FLAG_NAN_LOGIT
    assert 3 not in ids[2].tolist()


# ------------------------------------------------------------------- graph capture: sizes stay on the device

def test_forward_graph_replay_follows_new_routing(ops):
    say("graph replay")
    T, d, E, K, f = 512, 128, 8, 2, 256
    L = inputs.routed_layer("g", T, d, E, K, f, 51, bias_std=1.0)
    logits, x, w1p, w2 = dev(L.logits), dev(L.x), dev(L.w1p), dev(L.w2)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            ops.moe_forward(logits, x, w1p, w2, K)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y, _ = ops.moe_forward(logits, x, w1p, w2, K)
    rng = np.random.default_rng(52)
    for rep in range(3):
        new = rng.standard_normal((T, E)).astype(np.float32) + np.array([3.0 * (rep == 1)] + [0] * (E - 1),
                                                                          np.float32)
        logits.copy_(torch.from_numpy(new))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_ref, _ = orc.layer_forward(new, L.x, L.w1p, L.w2, K)
        assert max_rel_err(y, y_ref) <= BF16_TOL, rep
        # an eager call between replays agrees bit for bit with the replay
        y_eager, _ = ops.moe_forward(logits, x, w1p, w2, K)
        torch.cuda.synchronize()
        assert torch.equal(y_eager, y)


def test_grouped_gemm_bitwise_deterministic(ops):
    rng = np.random.default_rng(61)
    sizes = dev(torch.from_numpy(np.array([100, 0, 700, 3], np.int32)))
    A, B = dev(bf16(rng, 803, 256)), dev(bf16(rng, 4, 512, 256))
    c1 = ops.grouped_gemm(A, B, sizes, epilogue=ops.MOE_EPI_SWIGLU)
    c2 = ops.grouped_gemm(A, B, sizes, epilogue=ops.MOE_EPI_SWIGLU)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


# ------------------------------------------------------------------- split tail

# three m-tiles over eight groups: the grid (sized by the groups' upper bound)
# is more than twice the two n-tiles' six tiles, so with K = 2048 (64 stages)
# every tile of the one round is split along K in three
SPLIT_SIZES = np.array([300, 0, 0, 0, 0, 0, 0, 40], np.int32)


@pytest.mark.parametrize("mode", ["nk", "packed_swiglu", "kn", "f32"])
def test_grouped_gemm_split_tail(ops, mode):
    """Tiles of a short last round split along K, their fp32 partials added in
    split order by the last to arrive: the oracle's result, the same bits on
    every call, and the unsplit kernel's result within rounding."""
    sizes, N, Kd = SPLIT_SIZES, 512, 2048
    say("gg split tail", mode)
    rng = np.random.default_rng(71 + len(mode))
    G, M = sizes.size, int(sizes.sum())
    sz = dev(torch.from_numpy(sizes))
    A = bf16(rng, M, Kd)
    if mode == "kn":
        B = bf16(rng, G, Kd, N, scale=Kd ** -0.5)
        ref = orc.grouped_dgrad(A, B, sizes)
        run = lambda split: ops.grouped_gemm(dev(A), dev(B), sz, b_layout=ops.MOE_B_KN, split=split)
    elif mode == "packed_swiglu":
        B = bf16(rng, G, N, Kd, scale=Kd ** -0.5)
        ref, _ = orc.gemm_swiglu(A, B, sizes, keep_gu=True)
        P = ops.pack_weights(dev(B), ops.MOE_EPI_SWIGLU)
        run = lambda split: ops.grouped_gemm(dev(A), P, sz, epilogue=ops.MOE_EPI_SWIGLU, split=split)
    else:
        B = bf16(rng, G, N, Kd, scale=Kd ** -0.5)
        ref = orc.grouped_gemm(A, B, sizes)
        odt = torch.float32 if mode == "f32" else torch.bfloat16
        run = lambda split: ops.grouped_gemm(dev(A), dev(B), sz, out_dtype=odt, split=split)
    c1, c2, c0 = run(True), run(True), run(False)
    torch.cuda.synchronize()
    if mode == "f32":
        r = orc.bf16_to_f64(ref)
        assert np.abs(c1.cpu().double().numpy() - r).max() <= 1e-2 * np.abs(r).max()
        assert torch.allclose(c1, c0, rtol=1e-5, atol=1e-5 * float(c0.abs().max()))
    else:
        assert max_rel_err(c1, ref) <= BF16_TOL
        # one bf16 rounding apart at most: the two sum the same products in another order
        d = (c1.float() - c0.float()).abs()
        assert float(d.max()) <= 2 ** -7 * float(c0.float().abs().max())
    assert torch.equal(c1, c2)


def test_grouped_gemm_split_tail_after_whole_rounds(ops):
    """592 tiles on a 256-workgroup grid (eight groups of about 1,024 rows,
    N = 4096): two whole rounds, then 80 tiles split in three.  The whole
    output against the unsplit kernel, sampled rows of every group (those
    of the split tiles included) against the oracle."""
    sizes = np.array([1010, 1050, 980, 1030, 1000, 1044, 1040, 1038], np.int32)
    N, Kd = 4096, 2048
    say("gg split tail after whole rounds")
    rng = np.random.default_rng(77)
    G, M = sizes.size, int(sizes.sum())
    A, B = bf16(rng, M, Kd), bf16(rng, G, N, Kd, scale=Kd ** -0.5)
    Ad, Bd, sz = dev(A), dev(B), dev(torch.from_numpy(sizes))
    c1 = ops.grouped_gemm(Ad, Bd, sz)
    c0 = ops.grouped_gemm(Ad, Bd, sz, split=False)
    torch.cuda.synchronize()
    d = (c1.float() - c0.float()).abs()
    assert float(d.max()) <= 2 ** -7 * float(c0.float().abs().max())
    off = np.concatenate([[0], np.cumsum(sizes)])
    rows = np.unique(np.concatenate([np.linspace(off[g], off[g + 1] - 1, 6).astype(np.int64) for g in range(G)]))
    ref = orc.grouped_gemm(A, B, sizes, rows=rows)
    assert max_rel_err(c1[torch.from_numpy(rows).cuda()], ref) <= BF16_TOL


@pytest.mark.parametrize("case", ["ragged", "split_tail", "empty"])
def test_grouped_gemm_swiglu_bwd_epilogue(ops, case):
    """SwiGLU's backward formed in the data-gradient GEMM's epilogue: the
    oracle's dgu from the oracle's dh, the same bits as the stored dh
    followed by moe_swiglu_backward, rows past the groups not written.
    ragged: empty groups, one-row and partial tiles, a partial column tile
    (f = 200); split_tail: one round of tiles split along K in three;
    empty: every group empty, nothing written."""
    if case == "ragged":
        sizes, f, Kd = np.array([0, 37, 256, 1, 0, 300, 129, 0], np.int32), 200, 192
    elif case == "empty":
        sizes, f, Kd = np.zeros(4, np.int32), 64, 64
    else:
        sizes, f, Kd = SPLIT_SIZES, 512, 2048
    say("gg swiglu bwd epilogue", case)
    rng = np.random.default_rng(83 + len(case))
    G, M = sizes.size, int(sizes.sum())
    m_cap = M + 40
    A, B = bf16(rng, m_cap, Kd), bf16(rng, G, Kd, f, scale=Kd ** -0.5)
    gu = bf16(rng, m_cap, 2 * f, scale=2.0)
    Ad, Bd, gud, sz = dev(A), dev(B), dev(gu), dev(torch.from_numpy(sizes))
    if M == 0:
        out = torch.full((m_cap, 2 * f), 3.0, dtype=torch.bfloat16, device="cuda")
        ops.grouped_gemm(Ad, Bd, sz, b_layout=ops.MOE_B_KN, epilogue=ops.MOE_EPI_SWIGLU_BWD, aux=gud, out=out)
        torch.cuda.synchronize()
        assert torch.all(out == 3.0)
        return
    dh_ref = orc.grouped_dgrad(A[:M], B, sizes)
    dgu_ref = orc.swiglu_backward(gu[:M], dh_ref)
    out = torch.full((m_cap, 2 * f), 3.0, dtype=torch.bfloat16, device="cuda")
    r = ops.grouped_gemm(Ad, Bd, sz, b_layout=ops.MOE_B_KN, epilogue=ops.MOE_EPI_SWIGLU_BWD, aux=gud, out=out)
    again = ops.grouped_gemm(Ad, Bd, sz, b_layout=ops.MOE_B_KN, epilogue=ops.MOE_EPI_SWIGLU_BWD, aux=gud)
    dh = ops.grouped_gemm(Ad, Bd, sz, b_layout=ops.MOE_B_KN)
    dgu = ops.swiglu_backward(gud, dh, sz)
    torch.cuda.synchronize()
    assert r is out
    assert max_rel_err(out[:M], dgu_ref) <= BF16_TOL
    assert torch.equal(out[:M], dgu[:M]) and torch.equal(again[:M], out[:M])
    assert torch.all(out[M:] == 3.0)
    assert torch.equal(gud, dev(gu))   # the pre-activations are only read


@pytest.mark.parametrize("mode", ["nk", "packed", "packed_swiglu", "fused_quant"])
def test_grouped_gemm_mxfp8_split_tail(ops, mode):
    """The MXFP8 kernel's split tail (K = 4096: 64 stages, three ranges per
    tile): the oracle's result on the same codes, the same bits on every
    call, the unsplit kernel's result within rounding; with the quantising
    epilogue, codes and scales of the split run's h equal quantising its own
    bf16 h."""
    sizes, N, Kd = SPLIT_SIZES, 512, 4096
    say("gg mxfp8 split tail", mode)
    rng = np.random.default_rng(81 + len(mode))
    G, M = sizes.size, int(sizes.sum())
    A, B = bf16(rng, M, Kd), bf16(rng, G, N, Kd, scale=Kd ** -0.5)
    aq, as_ = orc.mxfp8_quantize(A, 0)
    bq, bs = orc.mxfp8_quantize(orc.u16(B).reshape(-1, Kd), 0)
    bq, bs = bq.reshape(G, N, Kd), bs.reshape(G, N, Kd // 32)
    t = lambda a: dev(torch.from_numpy(np.ascontiguousarray(a)))
    sz = t(sizes)
    swi = mode != "nk" and mode != "packed"
    ref = orc.mx_grouped_gemm(aq, as_, bq, bs, sizes, swiglu=swi)
    epi = ops.MOE_EPI_SWIGLU if swi else ops.MOE_EPI_NONE
    Bw, Bsc = (ops.pack_weights_mxfp8(t(bq), t(bs), epi), None) if mode.startswith("packed") else (t(bq), t(bs))
    if mode == "fused_quant":
        run = lambda split: ops.grouped_gemm_mxfp8(t(aq), t(as_), Bw, Bsc, sz, epilogue=ops.MOE_EPI_SWIGLU_MXFP8,
                                                   split=split)
        (q1, s1), (q2, s2) = run(True), run(True)
        h = ops.grouped_gemm_mxfp8(t(aq), t(as_), Bw, Bsc, sz, epilogue=ops.MOE_EPI_SWIGLU)
        qh, sh = ops.mxfp8_quantize(h, 0)
        torch.cuda.synchronize()
        assert torch.equal(q1, q2) and torch.equal(s1, s2)
        assert torch.equal(q1[:M], qh[:M]) and torch.equal(s1[:M], sh[:M])
        assert rel_l2(h[:M], ref) <= MX_TOL
        return
    run = lambda split: ops.grouped_gemm_mxfp8(t(aq), t(as_), Bw, Bsc, sz, epilogue=epi, split=split)
    c1, c2, c0 = run(True), run(True), run(False)
    torch.cuda.synchronize()
    assert rel_l2(c1[:M], ref) <= MX_TOL and max_rel_err(c1[:M], ref) <= 2 * BF16_TOL
    assert torch.equal(c1, c2)
    d = (c1[:M].float() - c0[:M].float()).abs()
    assert float(d.max()) <= 2 ** -7 * float(c0[:M].float().abs().max())


def test_grouped_gemm_mxfp8_split_tail_after_whole_rounds(ops):
    """592 MXFP8 tiles on a 256-workgroup grid (eight groups of about 1,024
    rows, N = 4096, K = 4096): two whole rounds, then 80 tiles split in
    three; the whole output against the unsplit kernel, sampled rows of every
    group against the oracle."""
    sizes = np.array([1010, 1050, 980, 1030, 1000, 1044, 1040, 1038], np.int32)
    N, Kd = 4096, 4096
    say("gg mxfp8 split tail after whole rounds")
    rng = np.random.default_rng(83)
    G, M = sizes.size, int(sizes.sum())
    A, B = bf16(rng, M, Kd), bf16(rng, G, N, Kd, scale=Kd ** -0.5)
    aq, as_ = ops.mxfp8_quantize(dev(A), 0)
    bq, bs = ops.mxfp8_quantize(dev(B).reshape(-1, Kd), 0)
    bq, bs = bq.reshape(G, N, Kd), bs.reshape(G, N, Kd // 32)
    sz = dev(torch.from_numpy(sizes))
    c1 = ops.grouped_gemm_mxfp8(aq, as_, bq, bs, sz)
    c0 = ops.grouped_gemm_mxfp8(aq, as_, bq, bs, sz, split=False)
    torch.cuda.synchronize()
    d = (c1.float() - c0.float()).abs()
    assert float(d.max()) <= 2 ** -7 * float(c0.float().abs().max())
    off = np.concatenate([[0], np.cumsum(sizes)])
    rows = np.unique(np.concatenate([np.linspace(off[g], off[g + 1] - 1, 6).astype(np.int64) for g in range(G)]))
    h = lambda x: x.cpu().numpy()
    ref = orc.mx_grouped_gemm(h(aq), h(as_), h(bq), h(bs), sizes, rows=rows)
    assert rel_l2(c1[torch.from_numpy(rows).cuda()], ref) <= MX_TOL


def test_grouped_gemm_split_tail_graph_replay(ops):
    """A captured call replayed with group sizes that do and do not split its
    last round (the split decision is taken on the device) matches an eager
    call bit for bit on every replay."""
    N, Kd, G = 512, 2048, 8
    rng = np.random.default_rng(75)
    m_cap = 1024
    A, B = dev(bf16(rng, m_cap, Kd)), dev(bf16(rng, G, N, Kd, scale=Kd ** -0.5))
    sz = dev(torch.from_numpy(SPLIT_SIZES.copy()))
    out = torch.empty((m_cap, N), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            ops.grouped_gemm(A, B, sz, out=out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.grouped_gemm(A, B, sz, out=out)
    for sizes in ([300, 0, 0, 0, 0, 0, 0, 40], [1000, 0, 0, 0, 0, 0, 0, 24], [128] * 8, [0, 0, 0, 1, 0, 0, 0, 0]):
        say("split replay", sizes)
        sizes = np.array(sizes, np.int32)
        M = int(sizes.sum())
        sz.copy_(torch.from_numpy(sizes))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = ops.grouped_gemm(A, B, sz)
        torch.cuda.synchronize()
        assert torch.equal(out[:M], eager[:M])
        ref = orc.grouped_gemm(A[:M], B, sizes)
        assert max_rel_err(out[:M], ref) <= BF16_TOL


# ------------------------------------------------------------------- guard bands

def _guarded(shape, dtype, fill):
    """A tensor of `shape` at the front of a buffer with a 4 KB tail; every
    element starts at `fill` (checked as raw bits afterwards)."""
    n = int(np.prod(shape))
    tail = 4096 // torch.empty((), dtype=dtype).element_size()
    buf = torch.full((n + tail,), fill, dtype=dtype, device="cuda")
    return buf[:n].view(*shape), buf


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else (t.view(torch.int32) if t.element_size() == 4 else t)


def _untouched(buf, start, fill):
    ref = torch.full((1,), fill, dtype=buf.dtype, device=buf.device)
    return bool(torch.all(_bits(buf[start:]) == _bits(ref)[0]).item())


def test_guard_bands_every_output(ops):
    """Rows past sum(group_sizes) and a 4 KB tail after every output keep their
    sentinel, for every grouped GEMM variant and the bandwidth kernels (empty
    groups first, in the middle and last; ragged group tails)."""
    say("guard bands")
    rng = np.random.default_rng(61)
    sizes = np.array([0, 130, 0, 300, 1, 0], np.int32)
    G, M = sizes.size, int(sizes.sum())
    m_cap, Kd, N, f = M + 37, 128, 256, 128
    S = dev(torch.from_numpy(sizes))
    A = dev(bf16(rng, m_cap, Kd))
    W = dev(bf16(rng, G, N, Kd, scale=Kd ** -0.5))
    W1 = dev(bf16(rng, G, 2 * f, Kd, scale=Kd ** -0.5))
    Wkn = dev(bf16(rng, G, Kd, N, scale=Kd ** -0.5))
    nan16 = float("nan")
    cases = []
    out, buf = _guarded((m_cap, N), torch.bfloat16, nan16)
    ops.grouped_gemm(A, W, S, out=out)
    cases.append(("nk plain", out, buf, M * N))
    out, buf = _guarded((m_cap, N), torch.float32, nan16)
    ops.grouped_gemm(A, W, S, out=out, out_dtype=torch.float32)
    cases.append(("nk f32", out, buf, M * N))
    out, buf = _guarded((m_cap, N), torch.bfloat16, nan16)
    ops.grouped_gemm(A, ops.pack_weights(W), S, out=out)
    cases.append(("packed plain", out, buf, M * N))
    out, buf = _guarded((m_cap, f), torch.bfloat16, nan16)
    ops.grouped_gemm(A, ops.pack_weights(W1, ops.MOE_EPI_SWIGLU), S, epilogue=ops.MOE_EPI_SWIGLU, out=out)
    cases.append(("packed swiglu", out, buf, M * f))
    out, buf = _guarded((m_cap, f), torch.bfloat16, nan16)
    aux, abuf = _guarded((m_cap, 2 * f), torch.bfloat16, nan16)
    ops.grouped_gemm(A, W1, S, epilogue=ops.MOE_EPI_SWIGLU, out=out, aux=aux, keep_aux=True)
    cases.append(("swiglu h", out, buf, M * f))
    cases.append(("swiglu aux", aux, abuf, M * 2 * f))
    out, buf = _guarded((m_cap, N), torch.bfloat16, nan16)
    ops.grouped_gemm(A, Wkn, S, b_layout=ops.MOE_B_KN, out=out)
    cases.append(("kn dgrad", out, buf, M * N))
    # MXFP8: plain, SwiGLU, quantising SwiGLU (codes and scales)
    aq, as_ = ops.mxfp8_quantize(A, 0)
    wq, ws = ops.quantize_weights(W)
    w1q, w1s = ops.quantize_weights(W1)
    out, buf = _guarded((m_cap, N), torch.bfloat16, nan16)
    ops.grouped_gemm_mxfp8(aq, as_, ops.pack_weights_mxfp8(wq, ws), None, S, out=out)
    cases.append(("mxfp8 plain", out, buf, M * N))
    P1 = ops.pack_weights_mxfp8(w1q, w1s, ops.MOE_EPI_SWIGLU)
    out, buf = _guarded((m_cap, f), torch.bfloat16, nan16)
    ops.grouped_gemm_mxfp8(aq, as_, P1, None, S, epilogue=ops.MOE_EPI_SWIGLU, out=out)
    cases.append(("mxfp8 swiglu", out, buf, M * f))
    q, qbuf = _guarded((m_cap, f), torch.uint8, 0xA5)
    sc, sbuf = _guarded((m_cap, f // 32), torch.uint8, 0xA5)
    ops.grouped_gemm_mxfp8(aq, as_, P1, None, S, epilogue=ops.MOE_EPI_SWIGLU_MXFP8, out=q, out_scale=sc)
    cases.append(("mxfp8 fused codes", q, qbuf, M * f))
    cases.append(("mxfp8 fused scales", sc, sbuf, M * (f // 32)))
    # quantiser over the valid rows only
    # (the binding allocates: call the library directly to quantise into the guarded buffers)
    q, qbuf = _guarded((m_cap, Kd), torch.uint8, 0xA5)
    sc, sbuf = _guarded((m_cap, Kd // 32), torch.uint8, 0xA5)
    st = ops.lib().mxfp8_group_quantize(ops._ptr(A), m_cap, Kd, 0, ops._ptr(S), G, ops._ptr(q), ops._ptr(sc), None,
                                        ops._stream(A.device))
    assert st == 0
    cases.append(("quantize codes", q, qbuf, M * Kd))
    cases.append(("quantize scales", sc, sbuf, M * (Kd // 32)))
    # weight gradient: every group written (empty ones as zeros), nothing past C
    Y = dev(bf16(rng, m_cap, N))
    out, buf = _guarded((G, Kd, N), torch.bfloat16, nan16)
    ops.grouped_gemm_wgrad(A, Y, S, out=out)
    cases.append(("wgrad", out, buf, G * Kd * N))
    torch.cuda.synchronize()
    for name, o, b, valid in cases:
        assert _untouched(b, valid, 0xA5 if b.dtype == torch.uint8 else nan16), name
    # the valid parts were written (no sentinel left in them)
    for name, o, b, valid in cases:
        if b.dtype in (torch.bfloat16, torch.float32):
            assert not bool(torch.isnan(b[:valid]).any().item()), name
    # wgrad of the empty groups: exact zeros
    for g in np.nonzero(sizes == 0)[0]:
        assert bool(torch.all(out[int(g)] == 0).item())
    # permute and combine: exactly T*K rows / T rows, nothing past them
    T, K, E, d = 97, 2, 5, 64
    ids = dev(torch.from_numpy(rng.integers(0, E, size=(T, K)).astype(np.int32)))
    ids[:, 1] = (ids[:, 0] + 1) % E
    x = dev(bf16(rng, T, d))
    p = ops.permute(x, ids, E)
    xp, xbuf = _guarded((T * K, d), torch.bfloat16, nan16)
    ws_bytes = ops.lib().moe_permute_workspace_bytes(T, E, K)
    wsb = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    st = ops.lib().moe_permute(ops._ptr(x), ops._ptr(ids), T, d, E, K, ops._ptr(p["group_sizes"]),
                               ops._ptr(p["group_offsets"]), ops._ptr(p["perm_src"]), ops._ptr(p["perm_dst"]),
                               ops._ptr(xp), ops._ptr(wsb), ws_bytes, None, ops._stream(x.device))
    assert st == 0
    y, ybuf = _guarded((T, d), torch.bfloat16, nan16)
    ops.unpermute_combine(xp, None, p["perm_dst"], T, K, out=y)
    torch.cuda.synchronize()
    assert _untouched(xbuf, T * K * d, nan16) and _untouched(ybuf, T * d, nan16)
    assert not bool(torch.isnan(xbuf[: T * K * d]).any().item()) and not bool(torch.isnan(ybuf[: T * d]).any().item())


# -------------------------------------------------------------------- MXFP4

def _mx4_layout(q, s):
    """Oracle MXFP4 (one code per byte [R, C], scales [R, C/32]) -> the boundary's
    layout (two codes per byte, element 2i low; scales [C/128, R, 4]): data movement only."""
    R, C = q.shape
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    st = np.ascontiguousarray(s.reshape(R, C // 128, 4).transpose(1, 0, 2))
    return packed, st


@pytest.mark.parametrize("R,C,scale", [(300, 384, 1.0), (1, 128, 1e-3), (77, 1024, 300.0)])
def test_mxfp4_quantize(ops, R, C, scale):
    """Codes and scales bit for bit the oracle's, with exact E2M1 ties, zeros
    and signed zeros, saturation and tiny blocks mixed in."""
    say("mxfp4 quantize", R, C, scale)
    rng = np.random.default_rng(R + C)
    x = (rng.standard_normal((R, C)) * scale).astype(np.float32)
    if R > 2:
        x[0, :32] = np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, 4, 3, 2, 1.5, 1, 0.5] * 2) * scale
        x[1, :32] = 0.0
        x[1, 32:64] = -0.0
        x[2, 64:96] = 1e-30
    xb = inputs.to_bf16(x)
    q_ref, s_ref = _mx4_layout(*orc.mxfp4_quantize(xb))
    q, s = ops.mxfp4_quantize(dev(xb))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)


@pytest.mark.parametrize("swiglu,sizes,N,Kd", [
    (False, [0, 300, 1, 0, 260], 512, 384),      # several m-tiles, empty groups, 3 stages
    (False, [513, 7], 200, 128),                 # partial n-tile, one stage (fewer than the pipeline depth)
    (True, [300, 0, 1, 517, 0, 33], 272, 256),   # SwiGLU, f = 136: partial output tile
    (False, [260, 3], 256, 640),                 # five stages: the stage buffers wrap around
])
def test_grouped_gemm_mxfp4(ops, swiglu, sizes, N, Kd):
    """The MXFP4 grouped GEMM on the oracle's own codes and scales (moved into
    the boundary's layout) against the oracle's exact-dequantisation GEMM."""
    sizes = np.array(sizes, np.int32)
    say("gg mxfp4", swiglu, sizes.tolist(), N, Kd)
    rng = np.random.default_rng(31 + N + Kd)
    G, M = sizes.size, int(sizes.sum())
    A, B = bf16(rng, M, Kd), bf16(rng, G, N, Kd, scale=Kd ** -0.5)
    aq, as_ = orc.mxfp4_quantize(A)
    bq, bs = orc.mxfp4_quantize(orc.u16(B).reshape(-1, Kd))
    ref = orc.mx4_grouped_gemm(aq, as_, bq.reshape(G, N, Kd), bs.reshape(G, N, Kd // 32), sizes, swiglu=swiglu)
    apk, ast = _mx4_layout(aq, as_)
    bpk, bst = _mx4_layout(bq, bs)
    t = lambda a: dev(torch.from_numpy(np.ascontiguousarray(a)))
    out = ops.grouped_gemm_mxfp4(t(apk), t(ast), t(bpk.reshape(G, N, Kd // 2)), t(bst), t(sizes),
                                 epilogue=ops.MOE_EPI_SWIGLU if swiglu else ops.MOE_EPI_NONE)
    torch.cuda.synchronize()
    assert rel_l2(out[:M], ref) <= MX_TOL
    assert max_rel_err(out[:M], ref) <= 2 * BF16_TOL
    # the device quantiser feeding the same GEMM gives the same bits
    q1, s1 = ops.mxfp4_quantize(dev(A))
    q2, s2 = ops.mxfp4_quantize(dev(B))
    out2 = ops.grouped_gemm_mxfp4(q1, s1, q2, s2, t(sizes), epilogue=ops.MOE_EPI_SWIGLU if swiglu else ops.MOE_EPI_NONE)
    torch.cuda.synchronize()
    assert torch.equal(out2[:M], out[:M])


def test_routed_layer_mxfp4(ops):
    """The routed MXFP4 forward (route, permute, quantise, gate/up + SwiGLU,
    quantise h, down, combine) against the oracle applying the same
    quantisation at the same points (its own h quantised by its own rule)."""
    say("routed mxfp4 layer")
    T, d, E, K, f = 600, 256, 8, 2, 256
    L = inputs.routed_layer("mx4", T, d, E, K, f, 73, bias_std=1.0)
    lg, x, w1p, w2 = dev(L.logits), dev(L.x), dev(L.w1p), dev(L.w2)
    y, parts = ops.moe_forward_mxfp4(lg, x, ops.mxfp4_quantize(w1p), ops.mxfp4_quantize(w2), K)
    torch.cuda.synchronize()
    ids, w = orc.route_topk(L.logits, K)
    sizes, offs, src, dst = orc.permute(ids, E)
    xq, xs = orc.mxfp4_quantize(orc.gather_rows(L.x, src, K))
    q1, s1 = orc.mxfp4_quantize(orc.u16(L.w1p).reshape(-1, d))
    q2, s2 = orc.mxfp4_quantize(orc.u16(L.w2).reshape(-1, f))
    h = orc.mx4_grouped_gemm(xq, xs, q1.reshape(E, 2 * f, d), s1.reshape(E, 2 * f, d // 32), sizes, swiglu=True)
    hq, hs = orc.mxfp4_quantize(h)
    yp = orc.mx4_grouped_gemm(hq, hs, q2.reshape(E, d, f), s2.reshape(E, d, f // 32), sizes)
    y_ref = orc.unpermute_combine(yp, w, dst, T, K)
    np.testing.assert_array_equal(parts["ids"].cpu().numpy(), ids)
    np.testing.assert_array_equal(parts["group_sizes"].cpu().numpy(), sizes)
    assert rel_l2(parts["h"][:T * K], h) <= MX_TOL
    assert rel_l2(y, y_ref) <= MX_TOL


# ------------------------------------------------------------------- NaN and infinities

def _plant_nonfinite(rng, x: torch.Tensor, n: int) -> torch.Tensor:
    """x (bf16, CPU) with n entries replaced by +-NaN / +-inf bit patterns."""
    bits = x.clone().view(torch.int16).numpy().view(np.uint16).copy()
    flat = bits.reshape(-1)
    pos = rng.choice(flat.size, size=n, replace=False)
    flat[pos] = rng.choice(np.array([0x7FC0, 0xFFC0, 0x7F80, 0xFF80], np.uint16), size=n)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)


def test_quantizers_nonfinite(ops):
    """A block holding a NaN or an infinity: scale 0xFF and NaN codes with each
    value's sign (E2M1: code 7 with the sign), other blocks untouched - bit
    for bit the oracle's, in every quantiser that writes MX codes."""
    rng = np.random.default_rng(31)
    R, C = 200, 256
    x = _plant_nonfinite(rng, bf16(rng, R, C, scale=2.0), 40)
    say("nonfinite mx q0")
    q_ref, s_ref = orc.mxfp8_quantize(x, 0)
    assert (s_ref == 0xFF).sum() >= 30
    q, s = ops.mxfp8_quantize(dev(x), 0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    # axis 1, grouped, and the transposed layout with the row-wise codes
    sizes = np.array([37, 0, 100, 63], np.int32)
    M = int(sizes.sum())
    say("nonfinite mx q1 / qT", M)
    q_ref, s_ref = orc.mxfp8_quantize(x[:M], 1, sizes)
    assert (s_ref == 0xFF).any()
    S = dev(torch.from_numpy(sizes))
    q1, s1 = ops.mxfp8_quantize(dev(x), 1, S)
    qT, sT, q0, s0 = ops.mxfp8_quantize_transposed(dev(x), S, rows_too=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q1[:M].cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s1[:s_ref.shape[0]].cpu().numpy(), s_ref)
    want_q, want_s, used = _to_transposed(q_ref, s_ref, sizes, qT.shape[1])
    np.testing.assert_array_equal(qT[:, :used].cpu().numpy(), want_q[:, :used])
    np.testing.assert_array_equal(sT[:, :used // 32].cpu().numpy(), want_s[:, :used // 32])
    q0_ref, s0_ref = orc.mxfp8_quantize(x[:M], 0)
    np.testing.assert_array_equal(q0[:M].cpu().numpy(), q0_ref)
    np.testing.assert_array_equal(s0[:M].cpu().numpy(), s0_ref)
    # the dispatch writing MXFP8 rows
    T, E, K = 64, 8, 2
    say("nonfinite permute mxfp8", T, E, K)
    ids = np.array([rng.permutation(E)[:K] for _ in range(T)], dtype=np.int32)
    xt = x[:T]
    _, _, src, _ = orc.permute(ids, E)
    xq_ref, xs_ref = orc.mxfp8_quantize(orc.gather_rows(xt, src, K), 0)
    out = ops.permute_mxfp8(dev(xt), dev(torch.from_numpy(ids)), E)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["xq"].cpu().numpy(), xq_ref.reshape(T * K, C))
    np.testing.assert_array_equal(out["xs"].cpu().numpy(), xs_ref.reshape(T * K, C // 32))
    # MXFP4
    say("nonfinite mxfp4")
    q_ref, s_ref = _mx4_layout(*orc.mxfp4_quantize(x))
    q4, s4 = ops.mxfp4_quantize(dev(x))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q4.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s4.cpu().numpy(), s_ref)
