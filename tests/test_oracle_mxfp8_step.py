"""Pin of the oracle's MXFP8 training step (``layer_forward_mxfp8`` and
``layer_backward_mxfp8``, with ``_quant_experts``).

Group-aware MXFP8 quantisation of the expert matmuls is one of the building
blocks named on the page "NVIDIA Accelerates Dropless MoE Training in JAX
Using Transformer Engine" (section "What specialized optimizations are
required for dropless MoE?"; MXFP8 block scaling in "Optimization 1").  The
oracle composes its pinned steps with one choice per GEMM of the axis each
operand is quantised along: every operand along that GEMM's contraction
(activations and h along their rows, weights along d for gate/up and along f
for down; the data gradients' weights down their output axis; both
weight-gradient operands down the tokens, 32-blocks restarting at every
expert's first row).

This module rebuilds every MXFP8 operand without the oracle's quantiser:
the block exponent from numpy's frexp of the block amax (floor(log2 amax)
minus 8, the largest E4M3 exponent), the codes from torch's float8_e4m3fn
cast of the clamped, scaled values, dequantised by torch.  It contracts them
in numpy fp64 and requires every oracle output to be the correctly rounded
bf16 of that (within half an ulp).  A quantisation along the wrong axis, a
missing transpose or a wrong operand changes the dequantised values, and
with them the products, far beyond half an ulp; one case below is built so
that its 32-blocks are lossless along one axis and lossy along the other,
and a planted axis swap in the oracle is shown to fail the check.
"""
import numpy as np
import pytest
import torch

from dropless_moe_expert_amd import inputs

# ---------------------------------------------------------------------------- helpers


def _f64(orc, bits):
    return orc.bf16_to_f64(bits)


def mx_dequant(v: np.ndarray, axis: int, group_sizes=None) -> np.ndarray:
    """Values after MXFP8 quantisation of the fp64 array v (bf16 values) with
    32-blocks along `axis`; with group_sizes the blocks restart at every
    group's first index along that axis (a short last block is padded with
    zeros for its amax).  Scale 2^e, e = floor(log2 amax) - 8 clamped to
    [-127, 127]; codes = torch float8_e4m3fn cast of clamp(v / 2^e, +-448);
    an all-zero block stays zero."""
    x = np.moveaxis(np.asarray(v, np.float64), axis, -1)
    n = x.shape[-1]
    out = np.zeros_like(x)
    if group_sizes is None:
        spans = [(0, n)]
    else:
        o = np.concatenate([[0], np.cumsum(np.asarray(group_sizes, np.int64))])
        spans = [(int(o[g]), int(o[g + 1])) for g in range(len(o) - 1)]
    for s, e in spans:
        for b0 in range(s, e, 32):
            blk = x[..., b0:min(b0 + 32, e)]
            amax = np.abs(blk).max(axis=-1, keepdims=True)
            _, ex = np.frexp(amax)                         # amax = m 2^ex, m in [0.5, 1)
            sexp = np.clip(ex - 1 - 8, -127, 127).astype(np.float64)
            scaled = np.clip(blk * 2.0 ** (-sexp), -448.0, 448.0)   # exact: bf16 value times 2^k
            codes = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn)
            deq = codes.to(torch.float64).numpy() * 2.0 ** sexp
            out[..., b0:min(b0 + 32, e)] = np.where(amax > 0, deq, 0.0)
    return np.moveaxis(out, -1, axis)


def _ulp_bf16(v):
    a = np.abs(v)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -126)
    return 2.0 ** (e - 7)


def check_rounded(orc, name, got_bits, exact, slack=1e-9):
    """got (bf16 bits) must be the bf16 nearest to exact (fp64)."""
    got = _f64(orc, got_bits)
    assert got.shape == exact.shape, (name, got.shape, exact.shape)
    err = np.abs(got - exact)
    bound = 0.5 * _ulp_bf16(exact) * (1 + slack) + 1e-300
    bad = err > bound
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {bad.size} values not the correctly rounded bf16 "
                           f"of the rebuilt MXFP8 product; worst error {err[bad].max():.3e}")


def group_of_rows(sizes):
    return np.repeat(np.arange(len(sizes)), np.asarray(sizes, np.int64))


def rebuild_and_check(orc, logits, x, w1p, w2, dy, K):
    """Runs the oracle's MXFP8 step and checks each output against the
    independent rebuild; returns the number of values checked."""
    y, sv = orc.layer_forward_mxfp8(logits, x, w1p, w2, K)
    bw = orc.layer_backward_mxfp8(dy, sv, w1p, w2, K)
    E = w1p.shape[0]
    f = w1p.shape[1] // 2
    T = logits.shape[0]
    sizes = np.asarray(sv["sizes"], np.int64)
    grp = group_of_rows(sizes)
    dst = np.asarray(sv["perm_dst"], np.int64).reshape(T, K)
    w = np.asarray(sv["w"], np.float64)
    W1 = _f64(orc, orc.u16(w1p))            # [E, 2f, d]
    W2 = _f64(orc, orc.u16(w2))             # [E, d, f]
    xp = _f64(orc, sv["x_perm"])
    n = 0

    # forward: gate/up on X and W1p quantised along d
    Xq = mx_dequant(xp, 1)
    W1q = np.stack([mx_dequant(W1[e], 1) for e in range(E)])
    gu = np.einsum("rk,rnk->rn", Xq, W1q[grp])
    check_rounded(orc, "gu", sv["gu"], gu)
    g, u = gu[:, :f], gu[:, f:]
    with np.errstate(over="ignore"):       # exp(-g) = inf for very negative g: silu = -0
        h = g / (1.0 + np.exp(-g)) * u
    check_rounded(orc, "h", sv["h"], h)
    # down on h (the oracle's bf16 h) and W2 quantised along f
    Hq = mx_dequant(_f64(orc, sv["h"]), 1)
    W2q = np.stack([mx_dequant(W2[e], 1) for e in range(E)])
    yp = np.einsum("rk,rnk->rn", Hq, W2q[grp])
    check_rounded(orc, "y_perm", sv["y_perm"], yp)
    Yp = _f64(orc, sv["y_perm"])
    check_rounded(orc, "y", y, np.einsum("tk,tkd->td", w, Yp[dst]))
    n += gu.size + h.size + yp.size

    # backward
    dyv = _f64(orc, orc.u16(dy))
    dyp = np.zeros_like(Yp)
    dyp[dst.ravel()] = (w[:, :, None] * dyv[:, None, :]).reshape(-1, dyv.shape[1])
    check_rounded(orc, "dy_perm", bw["dy_perm"], dyp)
    DYP = _f64(orc, bw["dy_perm"])
    # data gradient of down: dy_perm along d, W2 quantised down d (its output axis)
    W2t = np.stack([mx_dequant(W2[e], 0) for e in range(E)])     # [E, d, f], blocks down d
    dh = np.einsum("rk,rkn->rn", mx_dequant(DYP, 1), W2t[grp])
    check_rounded(orc, "dh", bw["dh"], dh)
    # weight gradient of down: both operands down the tokens, blocks restart per expert
    A = mx_dequant(DYP, 0, sizes)
    B = mx_dequant(_f64(orc, sv["h"]), 0, sizes)
    o = np.concatenate([[0], np.cumsum(sizes)])
    dw2 = np.stack([A[o[e]:o[e + 1]].T @ B[o[e]:o[e + 1]] for e in range(E)])
    check_rounded(orc, "dw2", bw["dw2"], dw2)
    # SwiGLU backward from the kept bf16 pre-activations
    G = _f64(orc, sv["gu"])
    gg, uu, dd = G[:, :f], G[:, f:], _f64(orc, bw["dh"])
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-gg))
    dgu = np.concatenate([dd * uu * s * (1 + gg * (1 - s)), dd * gg * s], axis=1)
    check_rounded(orc, "dgu", bw["dgu"], dgu)
    DGU = _f64(orc, bw["dgu"])
    # data gradient of gate/up: dgu along 2f, W1p quantised down 2f
    W1t = np.stack([mx_dequant(W1[e], 0) for e in range(E)])     # [E, 2f, d], blocks down 2f
    dxp = np.einsum("rk,rkn->rn", mx_dequant(DGU, 1), W1t[grp])
    check_rounded(orc, "dx_perm", bw["dx_perm"], dxp)
    # weight gradient of gate/up
    A = mx_dequant(DGU, 0, sizes)
    B = mx_dequant(xp, 0, sizes)
    dw1p = np.stack([A[o[e]:o[e + 1]].T @ B[o[e]:o[e + 1]] for e in range(E)])
    check_rounded(orc, "dw1p", bw["dw1p"], dw1p)
    for e in np.nonzero(sizes == 0)[0]:
        assert not _f64(orc, bw["dw1p"][e]).any() and not _f64(orc, bw["dw2"][e]).any()
    DXP = _f64(orc, bw["dx_perm"])
    check_rounded(orc, "dx", bw["dx"], DXP[dst].sum(axis=1))
    n += dh.size + dw2.size + dgu.size + dxp.size + dw1p.size
    return n


def _layer(seed, T, d, E, K, f, empty=None):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if empty is not None:
        lg[:, empty] -= 1e4
    x = inputs.to_bf16(rng.standard_normal((T, d)).astype(np.float32))
    w1p = inputs.to_bf16((rng.standard_normal((E, 2 * f, d)) / np.sqrt(d)).astype(np.float32))
    w2 = inputs.to_bf16((rng.standard_normal((E, d, f)) / np.sqrt(f)).astype(np.float32))
    dy = inputs.to_bf16(rng.standard_normal((T, d)).astype(np.float32))
    return lg, x, w1p, w2, dy


def _one_axis_lossless(rng, E, R, C):
    """[E, R, C] bf16 whose 32-blocks along C are exact in MXFP8 and whose
    32-blocks along R are not: row r holds (1 + k/8) 2^(r % 32 - 16) with
    k in 0..6 (one exponent per row: a block along C needs no more than
    E4M3's 3 mantissa bits at scale 2^(r % 32 - 24)); down a column the
    magnitudes span 2^31, so the small rows fall below E4M3's range."""
    k = rng.integers(0, 7, size=(E, R, C))
    sgn = rng.choice([-1.0, 1.0], size=(E, R, C))
    p = (np.arange(R) % 32 - 16).astype(np.float64)[None, :, None]
    return inputs.to_bf16((sgn * (1 + k / 8.0) * 2.0 ** p).astype(np.float32))


# ---------------------------------------------------------------------------- tests


def test_rebuilt_quantiser_matches_closed_forms():
    """The independent quantiser of this module: power-of-two blocks round
    trip, the amax element lands in [256, 448] after scaling, a zero block
    stays zero, and group restarts change the block split."""
    v = np.array([[2.0 ** -3, -2.0 ** 5, 0.0, 2.0 ** 7] + [0.0] * 28])
    assert np.array_equal(mx_dequant(v, 1), v)
    rng = np.random.default_rng(3)
    a = rng.standard_normal((4, 64)) * 7
    q = mx_dequant(a, 1)
    for b in range(2):
        blk = a[:, 32 * b:32 * b + 32]
        amax = np.abs(blk).max(axis=1)
        scale = 2.0 ** (np.floor(np.log2(amax)) - 8)
        top = np.abs(q[:, 32 * b:32 * b + 32]).max(axis=1) / scale
        assert ((top >= 256) & (top <= 448)).all()
    assert not mx_dequant(np.zeros((3, 32)), 1).any()
    col = rng.standard_normal((40, 3))
    col[:20] *= 1e-3
    whole = mx_dequant(col, 0)                      # one block of 32 + one of 8
    split = mx_dequant(col, 0, [20, 20])            # blocks restart at row 20
    assert not np.array_equal(whole, split)
    assert np.array_equal(split[:20], mx_dequant(col[:20], 0))


def test_one_axis_lossless_construction():
    rng = np.random.default_rng(11)
    W = _one_axis_lossless(rng, 1, 64, 64)[0].float().double().numpy()
    assert np.array_equal(mx_dequant(W, 1), W)                   # blocks along C: exact
    lossy = mx_dequant(W, 0) != W                                 # blocks down R: not
    assert lossy.mean() > 0.2


@pytest.mark.parametrize("seed,T,d,E,K,f,empty", [
    (1, 80, 64, 4, 2, 64, 3),       # groups of ~40 rows: blocks restart mid-tile; expert 3 empty
    (2, 48, 96, 6, 3, 32, None),    # K = 3, short groups
])
def test_mxfp8_step_rebuilt_independently(orc, seed, T, d, E, K, f, empty):
    lg, x, w1p, w2, dy = _layer(seed, T, d, E, K, f, empty)
    n = rebuild_and_check(orc, lg, x, w1p, w2, dy, K)
    assert n > 0
    if empty is not None:
        ids, _ = orc.route_topk(lg, K)
        assert not (ids == empty).any()


def _structured(seed=5, T=64, d=64, E=3, K=2, f=32):
    rng = np.random.default_rng(seed)
    lg, x, _, _, dy = _layer(seed, T, d, E, K, f)
    w1p = _one_axis_lossless(rng, E, 2 * f, d)     # exact along d (forward), lossy along 2f (dgrad)
    w2 = _one_axis_lossless(rng, E, d, f)          # exact along f (forward), lossy along d (dgrad)
    return lg, x, w1p, w2, dy, K


def test_mxfp8_step_one_axis_lossless_weights(orc):
    lg, x, w1p, w2, dy, K = _structured()
    rebuild_and_check(orc, lg, x, w1p, w2, dy, K)


def _prequantised(orc, w, axis):
    """bf16 [E, R, C] holding w's values after MXFP8 quantisation with
    32-blocks along `axis` of each expert (0: down R, 1: along C)."""
    wb = orc.u16(w)
    deq = np.stack([mx_dequant(_f64(orc, wb[e]), axis) for e in range(wb.shape[0])])
    return torch.from_numpy(deq.astype(np.float32)).to(torch.bfloat16)


def test_planted_axis_swap_is_caught(orc, monkeypatch):
    """Mistakes planted in the oracle's weight quantisation (on the CPU) must
    fail the rebuild check: (a) the forward weights quantised down R before
    their blocks along C, on weights exact along C only; (b) the data
    gradients' weights quantised along C before their blocks down R, on
    random weights."""
    real = orc._quant_experts

    def fwd_down_r(w, axis):
        return real(_prequantised(orc, w, 0), 0) if axis == 0 else real(w, axis)

    def bwd_along_c(w, axis):
        return real(_prequantised(orc, w, 1), 1) if axis == 1 else real(w, axis)

    lg, x, w1p, w2, dy, K = _structured()
    rebuild_and_check(orc, lg, x, w1p, w2, dy, K)         # the real oracle passes
    monkeypatch.setattr(orc, "_quant_experts", fwd_down_r)
    with pytest.raises(AssertionError, match="not the correctly rounded"):
        rebuild_and_check(orc, lg, x, w1p, w2, dy, K)
    lg, x, w1p, w2, dy = _layer(7, 64, 64, 3, 2, 32)
    monkeypatch.setattr(orc, "_quant_experts", bwd_along_c)
    with pytest.raises(AssertionError, match="not the correctly rounded"):
        rebuild_and_check(orc, lg, x, w1p, w2, dy, K)
