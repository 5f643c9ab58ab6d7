"""GPU parity of every path the benchmark times, at the size it times and
through the same calls (packed weights, fused quantising epilogues, the
routed MXFP8 / MXFP4 layers, the fine-grained MXFP8 training step).

The oracle's inputs are the generator's, never a GPU output.  Floating-point
results are checked on sampled rows and tokens, and the weight gradients of
the smallest, the median, the largest and an empty expert of the fine-grained
workload over their whole contraction (all of the expert's rows) on selected
output columns: selecting columns commutes with the GEMMs that produce them
and with MXFP8 quantisation down the tokens (its 32-blocks run down each
column on their own) or along a weight row, so the oracle computes exactly
those entries of the full result.  Integer results (codes, scales, maps) are
compared over whole tensors where the oracle can make them.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from dropless_moe_expert_amd import inputs
from gpu_util import BF16_TOL, MX_TOL, host_u16, mre_u16, rel_l2_u16, rows_of, sample_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    from dropless_moe_expert_amd import ops as _ops
    _ops.load_library()
    return _ops


def _deq_mx8(q, s):
    """E4M3 codes [R, C] and E8M0 scales [R, C/32] -> values."""
    return orc.e4m3_to_f64(q) * np.repeat(orc.e8m0_to_f64(s), 32, axis=1)


def _quant_rows_experts(w_u16, experts, rows_sel=None):
    """MXFP8 codes/scales along the last axis of the listed experts' weight
    rows (all rows, or rows_sel), as [G, R, C] / [G, R, C/32] with zeros for
    experts not listed."""
    G, R, C = w_u16.shape
    rsel = np.arange(R) if rows_sel is None else np.asarray(rows_sel)
    q = np.zeros((G, rsel.size, C), np.uint8)
    s = np.zeros((G, rsel.size, C // 32), np.uint8)
    for e in experts:
        q[e], s[e] = orc.mxfp8_quantize(np.ascontiguousarray(w_u16[e][rsel]), 0)
    return q, s


# ------------------------------------------------------------------ expert share (headline)

def test_dsv3_share_bf16_packed_full(ops):
    """The headline step exactly as timed: packed weights, gate/up + SwiGLU
    then down."""
    say("full bench path: dsv3 share bf16 packed")
    L = inputs.workload("dsv3_share")
    s = L.group_sizes.numpy()
    dev = torch.device("cuda")
    x, sz = L.x_perm.to(dev), L.group_sizes.to(dev)
    w1, w2 = L.w1p.to(dev), L.w2.to(dev)
    w1k, w2k = ops.pack_weights(w1, ops.MOE_EPI_SWIGLU), ops.pack_weights(w2)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    h = torch.empty((L.M, L.f), dtype=torch.bfloat16, device=dev)
    y = torch.empty((L.M, L.d), dtype=torch.bfloat16, device=dev)
    ops.grouped_gemm(x, w1k, sz, epilogue=ops.MOE_EPI_SWIGLU, out=h, flag=flag)
    ops.grouped_gemm(h, w2k, sz, out=y, flag=flag)
    y_plain, h_plain = ops.expert_mlp(x, sz, w1, w2)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    # packed weights change the load order only: the same bits as the plain layout
    assert torch.equal(h, h_plain) and torch.equal(y, y_plain)
    rows = sample_rows(s, 48, 11)
    h_ref, _ = orc.gemm_swiglu(L.x_perm, L.w1p, s, rows=rows)
    H = np.zeros((L.M, L.f), np.uint16)
    H[rows] = h_ref
    y_ref = orc.grouped_gemm(H, L.w2, s, rows=rows)
    assert mre_u16(rows_of(h, rows), h_ref) <= BF16_TOL
    assert mre_u16(rows_of(y, rows), y_ref) <= BF16_TOL


def test_dsv3_share_mxfp8_packed_fused_full(ops):
    """The MXFP8 share exactly as timed: X quantised, packed weights, the
    gate/up GEMM quantising h in its epilogue (K = 7168), the down GEMM."""
    say("full bench path: dsv3 share mxfp8 packed + fused quantise")
    L = inputs.workload("dsv3_mxfp8")
    s = L.group_sizes.numpy()
    dev = torch.device("cuda")
    x, sz = L.x_perm.to(dev), L.group_sizes.to(dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    w1q, w1s = ops.quantize_weights(L.w1p.to(dev))
    w2q, w2s = ops.quantize_weights(L.w2.to(dev))
    w1k = ops.pack_weights_mxfp8(w1q, w1s, ops.MOE_EPI_SWIGLU)
    w2k = ops.pack_weights_mxfp8(w2q, w2s)
    xq, xs = ops.mxfp8_quantize(x, 0, sz, flag=flag)
    hq, hs = ops.grouped_gemm_mxfp8(xq, xs, w1k, None, sz, epilogue=ops.MOE_EPI_SWIGLU_MXFP8, flag=flag)
    y = ops.grouped_gemm_mxfp8(hq, hs, w2k, None, sz, flag=flag)
    # the unfused pair on the same packed weights: bf16 h, then the quantiser
    h = ops.grouped_gemm_mxfp8(xq, xs, w1k, None, sz, epilogue=ops.MOE_EPI_SWIGLU, flag=flag)
    hq2, hs2 = ops.mxfp8_quantize(h, 0, sz, flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    assert torch.equal(hq, hq2) and torch.equal(hs, hs2)
    rows = sample_rows(s, 24, 12)
    xq_ref, xs_ref = orc.mxfp8_quantize(L.x_perm, 0)
    np.testing.assert_array_equal(xq.cpu().numpy(), xq_ref)
    np.testing.assert_array_equal(xs.cpu().numpy(), xs_ref)
    experts = sorted(set(np.repeat(np.arange(L.E), s)[rows].tolist()))
    w1q_ref, w1s_ref = _quant_rows_experts(orc.u16(L.w1p), experts)
    h_ref = orc.mx_grouped_gemm(xq_ref, xs_ref, w1q_ref, w1s_ref, s, swiglu=True, rows=rows)
    assert rel_l2_u16(rows_of(h, rows), h_ref) <= MX_TOL
    hq_ref, hs_ref = orc.mxfp8_quantize(h_ref, 0)
    got = _deq_mx8(hq[torch.from_numpy(rows).to(dev)].cpu().numpy(), hs[torch.from_numpy(rows).to(dev)].cpu().numpy())
    want = _deq_mx8(hq_ref, hs_ref)
    assert np.linalg.norm(got - want) / np.linalg.norm(want) <= MX_TOL
    HQ = np.zeros((L.M, L.f), np.uint8)
    HS = np.zeros((L.M, L.f // 32), np.uint8)
    HQ[rows], HS[rows] = hq_ref, hs_ref
    w2q_ref, w2s_ref = _quant_rows_experts(orc.u16(L.w2), experts)
    y_ref = orc.mx_grouped_gemm(HQ, HS, w2q_ref, w2s_ref, s, rows=rows)
    assert rel_l2_u16(rows_of(y, rows), y_ref) <= MX_TOL


# ------------------------------------------------------------------ Mixtral-shaped routed layers

def _routed_sample(L, n_tokens, seed):
    ids, w = orc.route_topk(L.logits, L.K)
    sizes, offs, src, dst = orc.permute(ids, L.E)
    rng = np.random.default_rng(seed)
    tokens = np.unique(np.concatenate([[0, L.T - 1], rng.choice(L.T, n_tokens - 2, replace=False)]))
    rows = np.unique(dst.reshape(L.T, L.K)[tokens].ravel().astype(np.int64))
    return ids, w, sizes, src, dst, tokens, rows


def test_mixtral_mxfp8_layer_full(ops):
    """The routed MXFP8 layer exactly as timed: route, permute writing MXFP8
    rows, gate/up quantising h, down, combine."""
    say("full bench path: mixtral mxfp8 layer")
    L = inputs.workload("mixtral")
    dev = torch.device("cuda")
    lg, x = L.logits.to(dev), L.x.to(dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    w1q, w1s = ops.quantize_weights(L.w1p.to(dev))
    w1k = ops.pack_weights_mxfp8(w1q, w1s, ops.MOE_EPI_SWIGLU)
    del w1q, w1s
    w2q, w2s = ops.quantize_weights(L.w2.to(dev))
    w2k = ops.pack_weights_mxfp8(w2q, w2s)
    del w2q, w2s
    y, sv = ops.moe_forward_mxfp8(lg, x, w1k, w2k, L.K, flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    ids, w, sizes, src, dst, tokens, rows = _routed_sample(L, 8, 21)
    np.testing.assert_array_equal(sv["ids"].cpu().numpy(), ids)
    np.testing.assert_array_equal(sv["perm_dst"].cpu().numpy(), dst)
    M = L.T * L.K
    xp_rows = orc.gather_rows(L.x, src[rows], L.K)
    xq_r, xs_r = orc.mxfp8_quantize(xp_rows, 0)
    XQ = np.zeros((M, L.d), np.uint8)
    XS = np.zeros((M, L.d // 32), np.uint8)
    XQ[rows], XS[rows] = xq_r, xs_r
    np.testing.assert_array_equal(sv["xq"][torch.from_numpy(rows).to(dev)].cpu().numpy(), xq_r)
    np.testing.assert_array_equal(sv["xs"][torch.from_numpy(rows).to(dev)].cpu().numpy(), xs_r)
    experts = sorted(set(np.repeat(np.arange(L.E), sizes)[rows].tolist()))
    w1q_ref, w1s_ref = _quant_rows_experts(orc.u16(L.w1p), experts)
    h_ref = orc.mx_grouped_gemm(XQ, XS, w1q_ref, w1s_ref, sizes, swiglu=True, rows=rows)
    del w1q_ref, w1s_ref
    hq_ref, hs_ref = orc.mxfp8_quantize(h_ref, 0)
    got = _deq_mx8(sv["hq"][torch.from_numpy(rows).to(dev)].cpu().numpy(),
                   sv["hs"][torch.from_numpy(rows).to(dev)].cpu().numpy())
    want = _deq_mx8(hq_ref, hs_ref)
    assert np.linalg.norm(got - want) / np.linalg.norm(want) <= MX_TOL
    HQ = np.zeros((M, L.f), np.uint8)
    HS = np.zeros((M, L.f // 32), np.uint8)
    HQ[rows], HS[rows] = hq_ref, hs_ref
    w2q_ref, w2s_ref = _quant_rows_experts(orc.u16(L.w2), experts)
    yp = orc.mx_grouped_gemm(HQ, HS, w2q_ref, w2s_ref, sizes, rows=rows)
    YP = np.zeros((M, L.d), np.uint16)
    YP[rows] = yp
    y_ref = orc.unpermute_combine(YP, w, dst, L.T, L.K)[tokens]
    assert rel_l2_u16(rows_of(y, tokens), y_ref) <= MX_TOL


def test_mixtral_mxfp4_layer_full(ops):
    """The routed MXFP4 layer exactly as timed: route, permute, quantise the
    rows, gate/up + SwiGLU, quantise h, down, combine."""
    say("full bench path: mixtral mxfp4 layer")
    L = inputs.workload("mixtral")
    dev = torch.device("cuda")
    lg, x = L.logits.to(dev), L.x.to(dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    w1 = ops.mxfp4_quantize(L.w1p.to(dev))
    w2 = ops.mxfp4_quantize(L.w2.to(dev))
    y, sv = ops.moe_forward_mxfp4(lg, x, w1, w2, L.K, flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    ids, w, sizes, src, dst, tokens, rows = _routed_sample(L, 8, 22)
    np.testing.assert_array_equal(sv["perm_dst"].cpu().numpy(), dst)
    M = L.T * L.K
    xq_r, xs_r = orc.mxfp4_quantize(orc.gather_rows(L.x, src[rows], L.K))
    XQ = np.zeros((M, L.d), np.uint8)
    XS = np.zeros((M, L.d // 32), np.uint8)
    XQ[rows], XS[rows] = xq_r, xs_r
    # the boundary layout of the sampled rows: two codes per byte, stage-major scales
    rd = torch.from_numpy(rows).to(dev)
    np.testing.assert_array_equal(sv["xq"][rd].cpu().numpy(), (xq_r[:, 0::2] | (xq_r[:, 1::2] << 4)).astype(np.uint8))
    np.testing.assert_array_equal(sv["xs"][:, rd].cpu().numpy(), xs_r.reshape(-1, L.d // 128, 4).transpose(1, 0, 2))
    experts = sorted(set(np.repeat(np.arange(L.E), sizes)[rows].tolist()))

    def quant4(w_u16):
        G, R, C = w_u16.shape
        q = np.zeros((G, R, C), np.uint8)
        s = np.zeros((G, R, C // 32), np.uint8)
        for e in experts:
            q[e], s[e] = orc.mxfp4_quantize(np.ascontiguousarray(w_u16[e]))
        return q, s

    w1q_ref, w1s_ref = quant4(orc.u16(L.w1p))
    h_ref = orc.mx4_grouped_gemm(XQ, XS, w1q_ref, w1s_ref, sizes, swiglu=True, rows=rows)
    del w1q_ref, w1s_ref
    assert rel_l2_u16(rows_of(sv["h"], rows), h_ref) <= MX_TOL
    hq_r, hs_r = orc.mxfp4_quantize(h_ref)
    HQ = np.zeros((M, L.f), np.uint8)
    HS = np.zeros((M, L.f // 32), np.uint8)
    HQ[rows], HS[rows] = hq_r, hs_r
    w2q_ref, w2s_ref = quant4(orc.u16(L.w2))
    yp = orc.mx4_grouped_gemm(HQ, HS, w2q_ref, w2s_ref, sizes, rows=rows)
    YP = np.zeros((M, L.d), np.uint16)
    YP[rows] = yp
    y_ref = orc.unpermute_combine(YP, w, dst, L.T, L.K)[tokens]
    assert rel_l2_u16(rows_of(y, tokens), y_ref) <= MX_TOL


# ------------------------------------------------------------------ fine-grained training steps

def _fg_experts(sizes):
    """The smallest non-empty, the median, the largest and an empty expert."""
    nz = np.nonzero(sizes)[0]
    order = nz[np.argsort(sizes[nz], kind="stable")]
    return [int(order[0]), int(order[len(order) // 2]), int(order[-1])], int(np.nonzero(sizes == 0)[0][0])


def _fg_reference_inputs(L):
    ids, w = orc.route_topk(L.logits, L.K)
    sizes, offs, src, dst = orc.permute(ids, L.E)
    M = L.T * L.K
    # dy_perm = w * dy gathered to the rows (its weight-gradient output is not used here)
    dyp, _ = orc.combine_backward(L.dy, np.zeros((M, L.d), np.uint16), w, dst, L.K)
    return ids, w, sizes, offs, src, dst, dyp


def test_finegrained_bf16_wgrad_all_sizes_full(ops):
    """bf16 weight gradients of the smallest, median and largest (12,876
    rows, about 400 K-stages through the tile queues) and an empty expert,
    over all of each expert's rows, on 16 columns of dW2 and 16 rows of dW1p."""
    say("full bench path: finegrained bf16 wgrad, every expert size")
    L = inputs.workload("finegrained")
    dev = torch.device("cuda")
    lg, x, w1, w2, dy = (t.to(dev) for t in (L.logits, L.x, L.w1p, L.w2, L.dy))
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    _, sv = ops.moe_forward(lg, x, w1, w2, L.K, keep=True, flag=flag)
    g = ops.moe_backward(dy, sv, w1, w2, L.K, flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    ids, w, sizes, offs, src, dst, dyp = _fg_reference_inputs(L)
    experts, empty = _fg_experts(sizes)
    assert sizes[experts[-1]] > 10000
    rng = np.random.default_rng(41)
    f, d = L.f, L.d
    W1, W2 = orc.u16(L.w1p), orc.u16(L.w2)
    for e in experts:
        er = np.arange(offs[e], offs[e + 1], dtype=np.int64)
        n = er.size
        one = np.array([n], np.int32)
        xp = orc.gather_rows(L.x, src[er], L.K)
        dy_e = dyp[er]
        qs = np.sort(rng.choice(f, 16, replace=False))
        js = np.sort(rng.choice(f, 8, replace=False))
        # dW2[e][:, qs] = sum_r dy_perm[r]^T h[r, qs]
        h_q, _ = orc.gemm_swiglu(xp, W1[e][np.concatenate([qs, f + qs])][None], one)
        dw2 = orc.grouped_wgrad(dy_e, h_q, one)[0]
        assert mre_u16(host_u16(g["dw2"][e][:, torch.from_numpy(qs).to(dev)]), dw2) <= BF16_TOL, e
        # dW1p[e][(js, f + js), :] = sum_r dgu[r, (js, f + js)]^T x_perm[r]
        _, gu_j = orc.gemm_swiglu(xp, W1[e][np.concatenate([js, f + js])][None], one, keep_gu=True)
        dh_j = orc.grouped_dgrad(dy_e, np.ascontiguousarray(W2[e][:, js])[None], one)
        dgu_j = orc.swiglu_backward(gu_j, dh_j)
        dw1 = orc.grouped_wgrad(dgu_j, xp, one)[0]
        sel = torch.from_numpy(np.concatenate([js, f + js])).to(dev)
        assert mre_u16(host_u16(g["dw1p"][e][sel]), dw1) <= BF16_TOL, e
    assert torch.all(g["dw2"][empty] == 0) and torch.all(g["dw1p"][empty] == 0)


def test_finegrained_mxfp8_step_full(ops):
    """The fine-grained MXFP8 training step exactly as timed (weights
    quantised both ways and packed, forward keeping the pre-activations,
    backward with the SwiGLU backward writing MXFP8): sampled tokens through
    forward and backward, and the weight gradients of the smallest, median,
    largest and an empty expert over all their rows on selected columns."""
    say("full bench path: finegrained mxfp8 step")
    L = inputs.workload("finegrained")
    dev = torch.device("cuda")
    lg, x, w1, w2, dy = (t.to(dev) for t in (L.logits, L.x, L.w1p, L.w2, L.dy))
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    wk = ops.quantize_weights_mxfp8_train(w1, w2, flag=flag)
    y, sv = ops.moe_forward_mxfp8_train(lg, x, wk, L.K, flag=flag)
    g = ops.moe_backward_mxfp8(dy, sv, wk, L.K, flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    ids, w, sizes, offs, src, dst, dyp = _fg_reference_inputs(L)
    np.testing.assert_array_equal(sv["perm_dst"].cpu().numpy(), dst)
    M, f, d = L.T * L.K, L.f, L.d
    W1, W2 = orc.u16(L.w1p), orc.u16(L.w2)
    grp = np.repeat(np.arange(L.E), sizes)

    # ---- sampled tokens, forward and backward
    rng = np.random.default_rng(43)
    tokens = np.unique(np.concatenate([[0, L.T - 1], rng.choice(L.T, 6, replace=False)]))
    rows = np.unique(dst.reshape(L.T, L.K)[tokens].ravel().astype(np.int64))
    experts = sorted(set(grp[rows].tolist()))
    XP = np.zeros((M, d), np.uint16)
    XP[rows] = orc.gather_rows(L.x, src[rows], L.K)
    xq, xs = orc.mxfp8_quantize(XP, 0)
    w1q, w1s = _quant_rows_experts(W1, experts)
    h_r = orc.mx_grouped_gemm(xq, xs, w1q, w1s, sizes, swiglu=True, rows=rows)
    assert rel_l2_u16(rows_of(sv["h"], rows), h_r) <= MX_TOL
    H = np.zeros((M, f), np.uint16)
    H[rows] = h_r
    hq, hs = orc.mxfp8_quantize(H, 0)
    w2q, w2s = _quant_rows_experts(W2, experts)
    yp_r = orc.mx_grouped_gemm(hq, hs, w2q, w2s, sizes, rows=rows)
    YP = np.zeros((M, d), np.uint16)
    YP[rows] = yp_r
    assert rel_l2_u16(rows_of(sv["y_perm"], rows), yp_r) <= MX_TOL
    y_ref = orc.unpermute_combine(YP, w, dst, L.T, L.K)[tokens]
    assert rel_l2_u16(rows_of(y, tokens), y_ref) <= MX_TOL
    # backward: dh on the weight quantised down d, dgu, dx_perm on W1p quantised down 2f
    # dy_perm reaches the GEMMs only as MXFP8, quantised as it is gathered:
    # its row codes are the oracle's codes of the oracle's dy_perm rows
    DYP = np.zeros((M, d), np.uint16)
    DYP[rows] = dyp[rows]
    dq, ds = orc.mxfp8_quantize(DYP, 0)
    _, _, gq0, gs0 = ops.mxfp8_quantize_gathered(dy, sv["perm_src"], L.K, sv["group_sizes"], topk_w=sv["w"],
                                                 rows_too=True)
    sel = torch.from_numpy(rows).to(dev)
    np.testing.assert_array_equal(gq0[sel].cpu().numpy(), dq[rows])
    np.testing.assert_array_equal(gs0[sel].cpu().numpy(), ds[rows])
    del gq0, gs0
    w2tq = np.zeros((L.E, f, d), np.uint8)
    w2ts = np.zeros((L.E, f, d // 32), np.uint8)
    w1tq = np.zeros((L.E, d, 2 * f), np.uint8)
    w1ts = np.zeros((L.E, d, 2 * f // 32), np.uint8)
    for e in experts:
        w2tq[e], w2ts[e] = (a[0] for a in orc._quant_experts(L.w2[e:e + 1], 1))
        w1tq[e], w1ts[e] = (a[0] for a in orc._quant_experts(L.w1p[e:e + 1], 1))
    dh_r = orc.mx_grouped_gemm(dq, ds, w2tq, w2ts, sizes, rows=rows)
    assert rel_l2_u16(rows_of(g["dh"], rows), dh_r) <= MX_TOL
    gu_r = orc.mx_grouped_gemm(xq, xs, w1q, w1s, sizes, rows=rows)     # pre-activations, MXFP8 operands
    assert rel_l2_u16(rows_of(sv["gu"], rows), gu_r) <= MX_TOL
    dgu_r = orc.swiglu_backward(gu_r, dh_r)
    DGU = np.zeros((M, 2 * f), np.uint16)
    DGU[rows] = dgu_r
    gq, gs = orc.mxfp8_quantize(DGU, 0)
    dxp_r = orc.mx_grouped_gemm(gq, gs, w1tq, w1ts, sizes, rows=rows)
    assert rel_l2_u16(rows_of(g["dx_perm"], rows), dxp_r) <= MX_TOL
    DXP = np.zeros((M, d), np.uint16)
    DXP[rows] = dxp_r
    dx_ref = orc.unpermute_combine(DXP, None, dst, L.T, L.K)[tokens]
    assert rel_l2_u16(rows_of(g["dx"], tokens), dx_ref) <= MX_TOL
    del w1q, w1s, w2q, w2s, w1tq, w1ts, w2tq, w2ts, XP, H, YP, DYP, DGU, DXP

    # ---- weight gradients over all rows of four experts, selected columns
    wexp, empty = _fg_experts(sizes)
    for e in wexp:
        er = np.arange(offs[e], offs[e + 1], dtype=np.int64)
        n = er.size
        one = np.array([n], np.int32)
        xp = orc.gather_rows(L.x, src[er], L.K)
        xq_e, xs_e = orc.mxfp8_quantize(xp, 0)
        qs = np.sort(rng.choice(f, 16, replace=False))
        js = np.sort(rng.choice(f, 8, replace=False))
        # h[:, qs] from the MXFP8 gate/up (weight rows quantised along d), then dW2[e][:, qs]
        wq, ws_ = orc.mxfp8_quantize(np.ascontiguousarray(W1[e][np.concatenate([qs, f + qs])]), 0)
        h_q = orc.mx_grouped_gemm(xq_e, xs_e, wq[None], ws_[None], one, swiglu=True)
        aq, as_ = orc.mxfp8_quantize(dyp[er], 1, one)
        bq, bs = orc.mxfp8_quantize(h_q, 1, one)
        dw2 = orc.mx_grouped_wgrad(aq, as_, bq, bs, one)[0]
        assert rel_l2_u16(host_u16(g["dw2"][e][:, torch.from_numpy(qs).to(dev)]), dw2) <= MX_TOL, e
        # dgu[:, (js, f + js)]: pre-activations of those columns and dh[:, js]
        # from dy_perm (along d) times W2[e][:, js] quantised down d
        wq, ws_ = orc.mxfp8_quantize(np.ascontiguousarray(W1[e][np.concatenate([js, f + js])]), 0)
        gu_j = orc.mx_grouped_gemm(xq_e, xs_e, wq[None], ws_[None], one)
        dq_e, ds_e = orc.mxfp8_quantize(dyp[er], 0)
        tq, ts = (a[0] for a in orc._quant_experts(L.w2[e:e + 1], 1))      # [f, d], blocks along d
        dh_j = orc.mx_grouped_gemm(dq_e, ds_e, np.ascontiguousarray(tq[js])[None],
                                   np.ascontiguousarray(ts[js])[None], one)
        dgu_j = orc.swiglu_backward(gu_j, dh_j)
        aq, as_ = orc.mxfp8_quantize(dgu_j, 1, one)
        bq, bs = orc.mxfp8_quantize(xp, 1, one)
        dw1 = orc.mx_grouped_wgrad(aq, as_, bq, bs, one)[0]
        sel = torch.from_numpy(np.concatenate([js, f + js])).to(dev)
        assert rel_l2_u16(host_u16(g["dw1p"][e][sel]), dw1) <= MX_TOL, e
    assert torch.all(g["dw2"][empty] == 0) and torch.all(g["dw1p"][empty] == 0)
