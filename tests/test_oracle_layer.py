"""Pins of the oracle's layer steps: routing, permutation, grouped GEMMs,
SwiGLU, combine and the backward.

Pins used (none re-runs the oracle's own code path):
* the softmax worked example printed on the pages (golden fixture);
* numpy's stable argsort / bincount / cumsum for the permutation;
* numpy fp64 matmuls with a correct-rounding bound (|bf16 - exact| <= half
  an ulp) for every GEMM;
* a dense brute force (every expert on every token, masked by the routing)
  for the whole dropless forward;
* torch's silu and autograd for the activation and the backward.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

from dropless_moe_expert_amd import inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return 2.0 ** (e - 7)


def assert_correctly_rounded(orc, got_bits, exact, slack=1e-9):
    """got must be the bf16 nearest to exact: within half an ulp of it."""
    got = orc.bf16_to_f64(got_bits)
    err = np.abs(got - exact)
    bound = 0.5 * _ulp_bf16(exact) * (1 + slack) + 1e-300
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} values not correctly rounded; worst {err[bad].max()} vs {bound[bad].min()}"


# --------------------------------------------------------------------------- routing

def test_softmax_worked_example(orc):
    g = json.load(open(os.path.join(GOLD, "softmax_example.json")))
    s = np.array([g["scores"]], np.float32)
    ids, w = orc.route_topk(s, K=4)          # K = E: renormalised top-K equals the full softmax
    assert list(ids[0]) == [1, 3, 0, 2]      # selection order = descending score
    full = dict(zip(ids[0], w[0]))
    got = [full[i] for i in range(4)]
    np.testing.assert_allclose(got, g["softmax"], atol=0.5 * 10 ** -g["printed_decimals"])
    # top-2 of the same row: experts 1 and 3, renormalised from the printed values
    ids2, w2 = orc.route_topk(s, K=2)
    assert list(ids2[0]) == [1, 3]
    p = np.array(g["softmax"])
    np.testing.assert_allclose(w2[0], [p[1] / (p[1] + p[3]), p[3] / (p[1] + p[3])], atol=2e-3)
    # non-renormalised weights are the full-softmax probabilities
    ids3, w3 = orc.route_topk(s, K=2, renormalize=False)
    np.testing.assert_allclose(w3[0], [p[1], p[3]], atol=0.5e-3)


def test_route_ties_and_invariants(orc):
    ids, w = orc.route_topk(np.array([[1.0, 1.0, 1.0, 1.0], [0.0, 5.0, 5.0, -1.0]], np.float32), K=2)
    assert ids.tolist() == [[0, 1], [1, 2]]
    np.testing.assert_allclose(w, [[0.5, 0.5], [0.5, 0.5]], rtol=0, atol=0)
    rng = np.random.default_rng(7)
    for T, E, K in [(300, 8, 2), (200, 128, 8), (50, 256, 8), (64, 4, 1), (32, 16, 16)]:
        l = rng.standard_normal((T, E)).astype(np.float32)
        l[:, ::3] = np.round(l[:, ::3])               # plenty of ties
        ids, w = orc.route_topk(l, K)
        # independent selection: lexicographic sort on (-logit, expert index)
        for t in range(T):
            order = np.lexsort((np.arange(E), -l[t].astype(np.float64)))
            assert ids[t].tolist() == order[:K].tolist()
        np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
        sm = scipy.special.softmax(l.astype(np.float64), axis=1)
        sel = np.take_along_axis(sm, ids, axis=1)
        np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=2e-7)


# --------------------------------------------------------------------------- permutation

def test_route_logits_closed_forms(orc):
    """Router scores: a hand-worked 2x2 by 2x3 product, one-hot tokens (which
    read one column of the router weight each: a transposed operand or a wrong
    index shows), zero tokens (bias only) and linearity in the bias."""
    bf = inputs.to_bf16
    x = bf(np.array([[1.0, 2.0], [3.0, 4.0]], np.float32))
    w = bf(np.array([[1.0, 0.0], [1.0, 1.0], [0.0, -1.0]], np.float32))
    # by hand: [1*1+2*0, 1*1+2*1, 1*0+2*(-1)] and [3, 3+4, -4]
    assert orc.route_logits(x, w).tolist() == [[1.0, 3.0, -2.0], [3.0, 7.0, -4.0]]
    b = np.array([0.5, -2.0, 8.0], np.float32)
    assert orc.route_logits(x, w, b).tolist() == [[1.5, 1.0, 6.0], [3.5, 5.0, 4.0]]

    rng = np.random.default_rng(7)
    T, d, E = 9, 40, 6
    cols = rng.integers(0, d, T)
    onehot = np.zeros((T, d), np.float32)
    onehot[np.arange(T), cols] = 1.0
    wr = bf(rng.standard_normal((E, d)).astype(np.float32))
    bias = rng.standard_normal(E).astype(np.float32)
    got = orc.route_logits(bf(onehot), wr, bias)
    wf = orc.bf16_to_f64(wr)
    want = wf[:, cols].T + bias.astype(np.float64)[None, :]
    assert np.array_equal(got, want)
    assert np.array_equal(orc.route_logits(bf(np.zeros((3, d), np.float32)), wr, bias),
                          np.tile(bias.astype(np.float64), (3, 1)))


@pytest.mark.parametrize("T,E,K", [(256, 8, 2), (1000, 128, 8), (17, 5, 1), (3, 256, 8), (1, 1, 1)])
def test_permute_is_stable_counting_sort(orc, T, E, K):
    rng = np.random.default_rng(T * 31 + E)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    sizes, offs, src, dst = orc.permute(ids, E)
    flat = ids.ravel()
    np.testing.assert_array_equal(sizes, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offs, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    np.testing.assert_array_equal(src, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(dst[src], np.arange(T * K))
    np.testing.assert_array_equal(src[dst], np.arange(T * K))
    # within an expert, token indices ascend
    for e in range(E):
        tok = src[offs[e]:offs[e + 1]] // K
        assert np.all(np.diff(tok) > 0)


def test_gather_and_unweighted_combine_roundtrip(orc):
    """combine(permute(x), w = 1) = K * x (exact: K*x is a bf16 value for K a power of two)."""
    rng = np.random.default_rng(11)
    for K in (1, 2, 4, 8):
        T, E, d = 40, 16, 24
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
        x = inputs.to_bf16(rng.standard_normal((T, d)).astype(np.float32))
        sizes, offs, src, dst = orc.permute(ids, E)
        xp = orc.gather_rows(x, src, K)
        y = orc.unpermute_combine(xp, None, dst, T, K)
        np.testing.assert_array_equal(orc.bf16_to_f64(y), K * orc.bf16_to_f64(x))


# --------------------------------------------------------------------------- GEMMs

def _bf16(rng, *shape, scale=1.0):
    return inputs.to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def test_grouped_gemm_vs_numpy(orc):
    rng = np.random.default_rng(12)
    sizes = np.array([3, 0, 17, 1, 0, 9], np.int32)
    M, N, Kd = int(sizes.sum()), 24, 40
    A, B = _bf16(rng, M, Kd), _bf16(rng, len(sizes), N, Kd)
    C = orc.grouped_gemm(A, B, sizes)
    a, b = orc.bf16_to_f64(A), orc.bf16_to_f64(B)
    o = 0
    for e, s in enumerate(sizes):
        exact = a[o:o + s] @ b[e].T
        assert_correctly_rounded(orc, C[o:o + s], exact)
        o += s
    # the row subset gives the same rows
    rows = np.array([0, 5, M - 1, 20])
    np.testing.assert_array_equal(orc.grouped_gemm(A, B, sizes, rows=rows), C[rows])


def test_grouped_gemm_identity_copies_rows(orc):
    rng = np.random.default_rng(13)
    sizes = np.array([4, 0, 6], np.int32)
    Kd = 32
    A = _bf16(rng, 10, Kd)
    B = torch.eye(Kd, dtype=torch.bfloat16).expand(3, Kd, Kd).contiguous()
    np.testing.assert_array_equal(orc.grouped_gemm(A, B, sizes), orc.u16(A))


def test_swiglu_vs_torch(orc):
    """E = 1, K = 1 reduces to a dense SwiGLU FFN; torch (fp64) is the reference."""
    rng = np.random.default_rng(14)
    M, f, Kd = 37, 48, 64
    A, W = _bf16(rng, M, Kd), _bf16(rng, 1, 2 * f, Kd, scale=0.3)
    h, gu = orc.gemm_swiglu(A, W, np.array([M], np.int32), keep_gu=True)
    a = torch.from_numpy(orc.bf16_to_f64(A))
    w = torch.from_numpy(orc.bf16_to_f64(W))[0]
    g, u = a @ w[:f].T, a @ w[f:].T
    exact = (torch.nn.functional.silu(g) * u).numpy()
    assert_correctly_rounded(orc, h, exact, slack=1e-6)
    assert_correctly_rounded(orc, gu, torch.cat([g, u], 1).numpy())


def test_dense_brute_force_equals_dropless(orc):
    """Every expert on every token, masked by the routing, equals the dropless forward bit for bit."""
    for (T, d, E, K, f, seed) in [(64, 32, 8, 2, 48, 21), (40, 64, 16, 4, 32, 22), (30, 32, 5, 1, 16, 23)]:
        L = inputs.routed_layer("t", T, d, E, K, f, seed, bias_std=1.0)
        y, kept = orc.layer_forward(L.logits, L.x, L.w1p, L.w2, K, keep=True)
        x = orc.bf16_to_f64(L.x)
        w1, w2 = orc.bf16_to_f64(L.w1p), orc.bf16_to_f64(L.w2)
        ids, wt = kept["ids"], kept["w"]
        # dense: all experts for all tokens
        ye = np.empty((E, T, d))
        for e in range(E):
            g, u = x @ w1[e, :f].T, x @ w1[e, f:].T
            h = orc.bf16_to_f64(orc.f64_to_bf16(scipy.special.expit(g) * g * u))
            ye[e] = orc.bf16_to_f64(orc.f64_to_bf16(h @ w2[e].T))
        mask = np.zeros((T, E))
        for t in range(T):
            for k in range(K):
                mask[t, ids[t, k]] = wt[t, k]
        # sum in the oracle's k order for bit-exactness
        acc = np.zeros((T, d))
        for k in range(K):
            acc += wt[:, k:k + 1].astype(np.float64) * ye[ids[:, k], np.arange(T)]
        np.testing.assert_array_equal(orc.f64_to_bf16(acc), y)
        # expert order with a 0/1-weighted mask: within one bf16 ulp
        acc2 = np.einsum("te,etd->td", mask, ye)
        assert np.all(np.abs(orc.bf16_to_f64(y) - acc2) <= _ulp_bf16(acc2) + 1e-30)


def test_identical_experts_reduce_to_dense_ffn(orc):
    T, d, E, K, f = 48, 32, 8, 2, 40
    L = inputs.routed_layer("t", T, d, E, K, f, 31)
    L.w1p = L.w1p[:1].expand(E, -1, -1).contiguous()
    L.w2 = L.w2[:1].expand(E, -1, -1).contiguous()
    y, _ = orc.layer_forward(L.logits, L.x, L.w1p, L.w2, K)
    x = orc.bf16_to_f64(L.x)
    w1, w2 = orc.bf16_to_f64(L.w1p[0]), orc.bf16_to_f64(L.w2[0])
    h = orc.bf16_to_f64(orc.f64_to_bf16(torch.nn.functional.silu(torch.from_numpy(x @ w1[:f].T)).numpy() * (x @ w1[f:].T)))
    dense = orc.bf16_to_f64(orc.f64_to_bf16(h @ w2.T))
    # weights sum to one: y = bf16(sum_k w_k * dense) is within one ulp of dense
    assert np.all(np.abs(orc.bf16_to_f64(y) - dense) <= _ulp_bf16(dense) + 1e-30)


def test_zero_token_expert_changes_nothing(orc):
    L = inputs.workload("tiny")
    y, kept = orc.layer_forward(L.logits, L.x, L.w1p, L.w2, L.K, keep=True)
    assert kept["sizes"][7] == 0
    w1p = L.w1p.clone(); w1p[7] = 1e30
    w2 = L.w2.clone(); w2[7] = -1e30
    y2, _ = orc.layer_forward(L.logits, L.x, w1p.to(torch.bfloat16), w2.to(torch.bfloat16), L.K)
    np.testing.assert_array_equal(y, y2)


def test_mx_grouped_gemm_vs_torch_dequant(orc):
    rng = np.random.default_rng(15)
    sizes = np.array([5, 0, 12, 1], np.int32)
    M, N, Kd = int(sizes.sum()), 16, 96
    A, B = _bf16(rng, M, Kd), _bf16(rng, len(sizes), N, Kd, scale=0.1)
    aq, as_ = orc.mxfp8_quantize(A, 0)
    bq, bs = orc.mxfp8_quantize(orc.u16(B).reshape(-1, Kd), 0)
    bq, bs = bq.reshape(len(sizes), N, Kd), bs.reshape(len(sizes), N, Kd // 32)

    def deq(q, s):
        v = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return v * np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=-1)

    a, b = deq(aq, as_), deq(bq, bs)
    C = orc.mx_grouped_gemm(aq, as_, bq, bs, sizes)
    o = 0
    for e, s in enumerate(sizes):
        assert_correctly_rounded(orc, C[o:o + s], a[o:o + s] @ b[e].T)
        o += s
    # SwiGLU variant: first half gate, second half up
    H = orc.mx_grouped_gemm(aq, as_, bq, bs, sizes, swiglu=True)
    o = 0
    for e, s in enumerate(sizes):
        gu = a[o:o + s] @ b[e].T
        g, u = gu[:, :N // 2], gu[:, N // 2:]
        assert_correctly_rounded(orc, H[o:o + s], torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u, 1e-6)
        o += s


# E2M1 by the format's definition (sign, 2 exponent bits with bias 1, one
# mantissa bit; exponent 0 is subnormal: 0.5 * m), written out by hand
E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_decode_encode(orc):
    dec = orc.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    assert dec.tolist() == E2M1_VALUES
    assert np.array_equal(np.signbit(dec), np.array([c >= 8 for c in range(16)]))
    # every code round-trips
    assert orc.f64_to_e2m1(dec).tolist() == list(range(16))
    # ties go to the even mantissa bit; past 6 saturates; the sign of zero is kept
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 6.5: 7, 1e30: 7, 0.2: 0, 0.3: 1,
             -0.3: 9, -0.0: 8, -0.1: 8, 2.9: 5, 4.9: 6, 5.1: 7}
    got = orc.f64_to_e2m1(np.array(list(cases.keys())))
    assert got.tolist() == list(cases.values())
    # brute force: the code is a nearest representable value of the same sign
    v = np.linspace(-7.5, 7.5, 6001)
    c = orc.f64_to_e2m1(v)
    a, dec = np.abs(v), np.abs(orc.e2m1_to_f64(c))
    mags = np.array(E2M1_VALUES[:8])
    dist = np.abs(a[:, None] - mags[None, :]).min(axis=1)
    inside = a <= 6
    assert np.array_equal(np.abs(dec - a)[inside], dist[inside])
    assert np.all(dec[~inside] == 6.0)
    assert np.all((c >= 8) == np.signbit(v))


def test_mx4_block_closed_forms(orc):
    bf = inputs.to_bf16
    row = np.zeros((4, 32), np.float32)
    row[0, :8] = [6.0, -4.0, 3.0, 1.5, 0.5, -0.0, 2.0, 1.0]   # amax 6: scale 2^0, every value on the grid
    row[1, 0] = 1.0                                            # amax 1: scale 2^-2, 1.0 -> 4.0 (code 6)
    row[1, 1] = 0.1                                            # 0.4 -> 0.5 (code 1)
    row[2, 0] = 7.0                                            # amax 7: scale 2^0, 7 saturates to 6
    q, s = orc.mxfp4_quantize(bf(row))
    assert s[:, 0].tolist() == [127, 125, 127, 0]
    assert q[0, :8].tolist() == [7, 14, 5, 3, 1, 8, 4, 2]
    assert q[1, :2].tolist() == [6, 1]
    assert q[2, 0] == 7 and q[3].tolist() == [0] * 32
    # large and tiny blocks: the scale follows floor(log2 amax) - 2 across the exponent range
    big = np.zeros((3, 32), np.float32)
    big[0, 0], big[1, 0], big[2, 0] = 2.0 ** 100, 2.0 ** -100, 3.0 * 2.0 ** 20
    _, s = orc.mxfp4_quantize(bf(big))
    assert s[:, 0].tolist() == [127 + 98, 127 - 102, 127 + 19]   # 3 * 2^20 = 1.5 * 2^21


def test_mx4_grouped_gemm_vs_numpy_dequant(orc):
    rng = np.random.default_rng(16)
    sizes = np.array([7, 0, 13, 2], np.int32)
    M, N, Kd = int(sizes.sum()), 16, 128
    A, B = _bf16(rng, M, Kd), _bf16(rng, len(sizes), N, Kd, scale=0.1)
    aq, as_ = orc.mxfp4_quantize(A)
    bq, bs = orc.mxfp4_quantize(orc.u16(B).reshape(-1, Kd))
    bq, bs = bq.reshape(len(sizes), N, Kd), bs.reshape(len(sizes), N, Kd // 32)
    table = np.array(E2M1_VALUES)

    def deq(q, s):
        return table[q] * np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=-1)

    a, b = deq(aq, as_), deq(bq, bs)
    C = orc.mx4_grouped_gemm(aq, as_, bq, bs, sizes)
    o = 0
    for e, s in enumerate(sizes):
        assert_correctly_rounded(orc, C[o:o + s], a[o:o + s] @ b[e].T)
        o += s
    H = orc.mx4_grouped_gemm(aq, as_, bq, bs, sizes, swiglu=True)
    o = 0
    for e, s in enumerate(sizes):
        gu = a[o:o + s] @ b[e].T
        g, u = gu[:, :N // 2], gu[:, N // 2:]
        assert_correctly_rounded(orc, H[o:o + s], torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u, 1e-6)
        o += s


def test_mx_grouped_wgrad_vs_torch_dequant(orc):
    # operands quantised down their rows, blocks restarting at every group
    # (a 40-row group has a short second block); the contraction runs over
    # each group's rows of the dequantised values; an empty group gives zeros
    rng = np.random.default_rng(18)
    sizes = np.array([40, 0, 7, 33], np.int32)
    M, P, Q = int(sizes.sum()), 24, 40
    A, B = _bf16(rng, M, P), _bf16(rng, M, Q, scale=0.2)
    aq, as_ = orc.mxfp8_quantize(A, 1, sizes)
    bq, bs = orc.mxfp8_quantize(B, 1, sizes)

    def deq(q, s):
        v = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        out = np.zeros_like(v)
        o, pb = 0, 0
        for n in sizes:
            for i in range(n):
                out[o + i] = v[o + i] * 2.0 ** (s[pb + i // 32].astype(np.float64) - 127)
            o, pb = o + n, pb + (n + 31) // 32
        return out

    a, b = deq(aq, as_), deq(bq, bs)
    C = orc.mx_grouped_wgrad(aq, as_, bq, bs, sizes)
    o = 0
    for e, n in enumerate(sizes):
        assert_correctly_rounded(orc, C[e], a[o:o + n].T @ b[o:o + n])
        if n == 0:
            assert np.all(C[e] == 0)
        o += n


# --------------------------------------------------------------------------- backward

def test_backward_steps_vs_numpy(orc):
    rng = np.random.default_rng(16)
    sizes = np.array([0, 7, 3, 0, 12], np.int32)
    M, N, Kd = int(sizes.sum()), 20, 36
    dC, A, B = _bf16(rng, M, N), _bf16(rng, M, Kd), _bf16(rng, len(sizes), N, Kd)
    dA = orc.grouped_dgrad(dC, B, sizes)
    dB = orc.grouped_wgrad(dC, A, sizes)
    g, a, b = orc.bf16_to_f64(dC), orc.bf16_to_f64(A), orc.bf16_to_f64(B)
    o = 0
    for e, s in enumerate(sizes):
        assert_correctly_rounded(orc, dA[o:o + s], g[o:o + s] @ b[e])
        assert_correctly_rounded(orc, dB[e], g[o:o + s].T @ a[o:o + s])
        if s == 0:
            assert np.all(dB[e] == 0)
        o += s
    sub = orc.grouped_wgrad(dC, A, sizes, groups=[4, 1])
    np.testing.assert_array_equal(sub, dB[[4, 1]])


def test_swiglu_backward_vs_autograd(orc):
    rng = np.random.default_rng(17)
    M, f = 33, 40
    gu = _bf16(rng, M, 2 * f, scale=3.0)
    dh = _bf16(rng, M, f)
    dgu = orc.swiglu_backward(gu, dh)
    t = torch.from_numpy(orc.bf16_to_f64(gu)).requires_grad_(True)
    h = torch.nn.functional.silu(t[:, :f]) * t[:, f:]
    h.backward(torch.from_numpy(orc.bf16_to_f64(dh)))
    assert_correctly_rounded(orc, dgu, t.grad.numpy(), slack=1e-6)


def test_layer_backward_vs_autograd(orc):
    """The composed backward against autograd of the unrounded dense layer (fp64).

    The oracle rounds its stored tensors to bf16; autograd does not, so the two
    agree to a few bf16 ulps relative to each tensor's scale."""
    T, d, E, K, f = 48, 32, 6, 2, 24
    L = inputs.routed_layer("t", T, d, E, K, f, 41, bias_std=0.5, dy=True)
    y, saved = orc.layer_forward(L.logits, L.x, L.w1p, L.w2, K, keep=True)
    grads = orc.layer_backward(L.dy, saved, L.w1p, L.w2, K)
    ids, wt = saved["ids"], saved["w"]
    x = torch.from_numpy(orc.bf16_to_f64(L.x)).requires_grad_(True)
    w1 = torch.from_numpy(orc.bf16_to_f64(L.w1p)).requires_grad_(True)
    w2 = torch.from_numpy(orc.bf16_to_f64(L.w2)).requires_grad_(True)
    wv = torch.from_numpy(wt.astype(np.float64)).requires_grad_(True)
    out = torch.zeros(T, d, dtype=torch.float64)
    for k in range(K):
        e = torch.from_numpy(ids[:, k].astype(np.int64))
        g = torch.einsum("td,tfd->tf", x, w1[e, :f])
        u = torch.einsum("td,tfd->tf", x, w1[e, f:])
        yk = torch.einsum("tf,tdf->td", torch.nn.functional.silu(g) * u, w2[e])
        out = out + wv[:, k:k + 1] * yk
    out.backward(torch.from_numpy(orc.bf16_to_f64(L.dy)))

    def rel(a, b):
        b = np.asarray(b)
        return np.abs(a - b).max() / np.abs(b).max()

    assert rel(orc.bf16_to_f64(y), out.detach().numpy()) < 1e-2
    assert rel(orc.bf16_to_f64(grads["dx"]), x.grad.numpy()) < 2e-2
    assert rel(orc.bf16_to_f64(grads["dw1p"]), w1.grad.numpy()) < 2e-2
    assert rel(orc.bf16_to_f64(grads["dw2"]), w2.grad.numpy()) < 2e-2
    assert rel(grads["dw"], wv.grad.numpy()) < 2e-2


def test_finite_difference_dx(orc):
    """A finite-difference check (fp64, central) of one input-gradient entry per token."""
    T, d, E, K, f = 6, 8, 3, 2, 8
    L = inputs.routed_layer("t", T, d, E, K, f, 43, dy=True)
    _, saved = orc.layer_forward(L.logits, L.x, L.w1p, L.w2, K, keep=True)
    grads = orc.layer_backward(L.dy, saved, L.w1p, L.w2, K)
    ids, wt = saved["ids"], saved["w"]
    w1, w2 = orc.bf16_to_f64(L.w1p), orc.bf16_to_f64(L.w2)
    dy = orc.bf16_to_f64(L.dy)

    def loss(xt, t):
        s = 0.0
        for k in range(K):
            e = ids[t, k]
            g, u = w1[e, :f] @ xt, w1[e, f:] @ xt
            s += wt[t, k] * dy[t] @ (w2[e] @ (scipy.special.expit(g) * g * u))
        return s

    x = orc.bf16_to_f64(L.x)
    dx = orc.bf16_to_f64(grads["dx"])
    eps = 1e-5
    for t in range(T):
        j = t % d
        xp, xm = x[t].copy(), x[t].copy()
        xp[j] += eps
        xm[j] -= eps
        fd = (loss(xp, t) - loss(xm, t)) / (2 * eps)
        assert abs(dx[t, j] - fd) <= 2e-2 * max(1.0, abs(fd)), (t, dx[t, j], fd)


# --------------------------------------------------------------------------- workloads

def test_workload_structure(orc):
    L = inputs.workload("tiny")
    ids, _ = orc.route_topk(L.logits, L.K)
    sizes, *_ = orc.permute(ids, L.E)
    assert sizes[7] == 0 and sizes.sum() == L.T * L.K
    S = inputs.workload("dsv3_share", weights=False)
    s = S.group_sizes.numpy()
    assert s.sum() == 24576 and (s == 0).sum() >= 2 and s.max() > 0.15 * 24576
    F = inputs.routed_layer("finegrained", 16384, 8, 128, 8, 8, 5, bias_std=1.5, weights=False)
    ids, _ = orc.route_topk(F.logits, 8)
    sizes, *_ = orc.permute(ids, 128)
    assert (sizes == 0).sum() >= 1
