"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.

Integer results (routing ids, counts, offsets, permutation maps, MXFP8 codes
and scales) are compared over the whole tensors.  Floating-point outputs are
compared on sampled rows / tokens / weight-gradient groups that the oracle
computes one by one from the generator's inputs (never from GPU outputs):
every group's first and last row plus random rows, every sampled token's K
rows, the smallest, a middle-sized and an empty expert for the weight
gradients.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from dropless_moe_expert_amd import inputs
from gpu_util import BF16_TOL, MX_TOL, W_RTOL, host_u16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    from dropless_moe_expert_amd import ops as _ops
    _ops.load_library()
    return _ops


def mre(got_u16, ref_u16):
    g, r = orc.bf16_to_f64(got_u16), orc.bf16_to_f64(ref_u16)
    return float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-30))


def rel_l2(got_u16, ref_u16):
    g, r = orc.bf16_to_f64(got_u16), orc.bf16_to_f64(ref_u16)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))


def sample_rows(sizes, n_extra, seed):
    offs = np.concatenate([[0], np.cumsum(sizes)])
    rows = []
    for g in range(len(sizes)):
        if sizes[g] > 0:
            rows += [offs[g], offs[g + 1] - 1]
    rng = np.random.default_rng(seed)
    rows += list(rng.choice(int(offs[-1]), size=n_extra, replace=False))
    return np.unique(np.array(rows, np.int64))


def rows_of(t: torch.Tensor, rows) -> np.ndarray:
    return host_u16(t[torch.from_numpy(np.asarray(rows, np.int64)).to(t.device)])


def check_routing(ops, L, ids, w, p):
    """Routing and permutation bit-exact over all tokens."""
    ids_ref, w_ref = orc.route_topk(L.logits, L.K)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=W_RTOL, atol=1e-30)
    sizes, offs, src, dst = orc.permute(ids_ref, L.E)
    np.testing.assert_array_equal(p["group_sizes"].cpu().numpy(), sizes)
    np.testing.assert_array_equal(p["group_offsets"].cpu().numpy(), offs)
    np.testing.assert_array_equal(p["perm_src"].cpu().numpy(), src)
    np.testing.assert_array_equal(p["perm_dst"].cpu().numpy(), dst)
    return ids_ref, w_ref, sizes, src, dst


def sampled_forward(L, sizes, src, dst, w_ref, tokens, keep_gu=False):
    """Oracle y for the sampled tokens (and the h / y_perm / gu of their rows)."""
    rows = np.unique(np.concatenate([dst.reshape(L.T, L.K)[t] for t in tokens]).astype(np.int64))
    xp = orc.gather_rows(L.x, src, L.K)
    h_rows, gu_rows = orc.gemm_swiglu(xp, L.w1p, sizes, rows=rows, keep_gu=keep_gu)
    M = L.T * L.K
    H = np.zeros((M, L.f), np.uint16)
    H[rows] = h_rows
    yp_rows = orc.grouped_gemm(H, L.w2, sizes, rows=rows)
    YP = np.zeros((M, L.d), np.uint16)
    YP[rows] = yp_rows
    y = orc.unpermute_combine(YP, w_ref, dst, L.T, L.K)
    return rows, xp, H, YP, h_rows, gu_rows, y[tokens]


def test_mixtral_forward_full(ops):
    say("full: mixtral forward")
    L = inputs.workload("mixtral")
    dev = torch.device("cuda")
    lg, x, w1, w2 = (t.to(dev) for t in (L.logits, L.x, L.w1p, L.w2))
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    y, saved = ops.moe_forward(lg, x, w1, w2, L.K, keep=True, flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    ids_ref, w_ref, sizes, src, dst = check_routing(ops, L, saved["ids"], saved["w"], saved)
    assert abs(int(sizes.max()) - 1024) < 200 and sizes.sum() == L.T * L.K
    np.testing.assert_array_equal(rows_of(saved["x_perm"], np.arange(0, L.T * L.K, 97)),
                                  orc.gather_rows(L.x, src, L.K)[::97])
    tokens = np.unique(np.concatenate([[0, L.T - 1], np.random.default_rng(1).choice(L.T, 14, replace=False)]))
    rows, _, _, _, h_rows, _, y_tok = sampled_forward(L, sizes, src, dst, w_ref, tokens)
    assert mre(rows_of(saved["h"], rows), h_rows) <= BF16_TOL
    assert mre(rows_of(y, tokens), y_tok) <= BF16_TOL


def test_dsv3_share_bf16_full(ops):
    say("full: dsv3 share bf16")
    L = inputs.workload("dsv3_share")
    s = L.group_sizes.numpy()
    assert (s == 0).sum() >= 2 and s.max() > 0.15 * L.M
    dev = torch.device("cuda")
    x, w1, w2, sz = L.x_perm.to(dev), L.w1p.to(dev), L.w2.to(dev), L.group_sizes.to(dev)
    y, h = ops.expert_mlp(x, sz, w1, w2)
    torch.cuda.synchronize()
    rows = sample_rows(s, 40, 3)
    h_ref, _ = orc.gemm_swiglu(L.x_perm, L.w1p, s, rows=rows)
    H = np.zeros((L.M, L.f), np.uint16)
    H[rows] = h_ref
    y_ref = orc.grouped_gemm(H, L.w2, s, rows=rows)
    assert mre(rows_of(h, rows), h_ref) <= BF16_TOL
    assert mre(rows_of(y, rows), y_ref) <= BF16_TOL


def test_dsv3_share_mxfp8_full(ops):
    say("full: dsv3 share mxfp8")
    L = inputs.workload("dsv3_mxfp8")
    s = L.group_sizes.numpy()
    dev = torch.device("cuda")
    x, w1, w2, sz = L.x_perm.to(dev), L.w1p.to(dev), L.w2.to(dev), L.group_sizes.to(dev)
    # quantisation of the activations: codes and scales bit-exact over the whole tensor
    xq, xs = ops.mxfp8_quantize(x, 0, sz)
    xq_ref, xs_ref = orc.mxfp8_quantize(L.x_perm, 0)
    np.testing.assert_array_equal(xs.cpu().numpy(), xs_ref)
    np.testing.assert_array_equal(xq.cpu().numpy(), xq_ref)
    # weights: a few experts, bit-exact
    w1q, w1s = ops.quantize_weights(w1)
    w2q, w2s = ops.quantize_weights(w2)
    for e in (0, int(np.argmax(s)), L.E - 1):
        q_ref, s_ref = orc.mxfp8_quantize(orc.u16(L.w1p[e]), 0)
        np.testing.assert_array_equal(w1q[e].cpu().numpy(), q_ref)
        np.testing.assert_array_equal(w1s[e].cpu().numpy(), s_ref)
    y, parts = ops.expert_mlp_mxfp8(x, sz, w1q, w1s, w2q, w2s)
    torch.cuda.synchronize()
    # oracle: identical quantisation of X and of the weights, its own H quantised by its own rule
    rows = sample_rows(s, 24, 4)
    w1q_ref, w1s_ref = orc.mxfp8_quantize(orc.u16(L.w1p).reshape(-1, L.d), 0)
    w1q_ref, w1s_ref = w1q_ref.reshape(L.E, 2 * L.f, L.d), w1s_ref.reshape(L.E, 2 * L.f, L.d // 32)
    h_ref = orc.mx_grouped_gemm(xq_ref, xs_ref, w1q_ref, w1s_ref, s, swiglu=True, rows=rows)
    assert rel_l2(rows_of(parts["h"], rows), h_ref) <= MX_TOL
    hq_ref, hs_ref = orc.mxfp8_quantize(h_ref, 0)
    HQ = np.zeros((L.M, L.f), np.uint8)
    HS = np.zeros((L.M, L.f // 32), np.uint8)
    HQ[rows], HS[rows] = hq_ref, hs_ref
    w2q_ref, w2s_ref = orc.mxfp8_quantize(orc.u16(L.w2).reshape(-1, L.f), 0)
    w2q_ref, w2s_ref = w2q_ref.reshape(L.E, L.d, L.f), w2s_ref.reshape(L.E, L.d, L.f // 32)
    y_ref = orc.mx_grouped_gemm(HQ, HS, w2q_ref, w2s_ref, s, rows=rows)
    assert rel_l2(rows_of(y, rows), y_ref) <= MX_TOL
    # and against the bf16 oracle: MXFP8 stays close to the unquantised layer
    hb, _ = orc.gemm_swiglu(L.x_perm, L.w1p, s, rows=rows)
    assert rel_l2(rows_of(parts["h"], rows), hb) <= 0.1


def test_finegrained_forward_backward_full(ops):
    say("full: finegrained forward+backward")
    L = inputs.workload("finegrained")
    dev = torch.device("cuda")
    lg, x, w1, w2, dy = (t.to(dev) for t in (L.logits, L.x, L.w1p, L.w2, L.dy))
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    y, saved = ops.moe_forward(lg, x, w1, w2, L.K, keep=True, flag=flag)
    g = ops.moe_backward(dy, saved, w1, w2, L.K, flag=flag, fused=False)
    dgu_fused = ops.moe_backward(dy, saved, w1, w2, L.K, flag=flag)["dgu"]
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    rows_all = int(saved["group_sizes"].sum())
    assert torch.equal(dgu_fused[:rows_all], g["dgu"][:rows_all])
    del dgu_fused
    ids_ref, w_ref, sizes, src, dst = check_routing(ops, L, saved["ids"], saved["w"], saved)
    assert (sizes == 0).sum() >= 1
    tokens = np.unique(np.concatenate([[0, L.T - 1], np.random.default_rng(5).choice(L.T, 10, replace=False)]))
    rows, xp, H, YP, h_rows, gu_rows, y_tok = sampled_forward(L, sizes, src, dst, w_ref, tokens, keep_gu=True)
    assert mre(rows_of(saved["h"], rows), h_rows) <= BF16_TOL
    assert mre(rows_of(saved["gu"], rows), gu_rows) <= BF16_TOL
    assert mre(rows_of(y, tokens), y_tok) <= BF16_TOL
    # backward, sampled tokens: combine backward needs y_perm of the token's rows only
    dyp_ref, dw_ref = orc.combine_backward(L.dy, YP, w_ref, dst, L.K)
    tk_rows = dst.reshape(L.T, L.K)[tokens].ravel()
    assert mre(rows_of(g["dy_perm"], tk_rows), dyp_ref[tk_rows]) <= BF16_TOL
    dw_gpu = g["dw"].cpu().numpy()[tokens]
    np.testing.assert_allclose(dw_gpu, dw_ref[tokens], rtol=1e-2, atol=1e-2 * np.abs(dw_ref[tokens]).max())
    dh_rows = orc.grouped_dgrad(dyp_ref, L.w2, sizes, rows=rows)
    assert mre(rows_of(g["dh"], rows), dh_rows) <= BF16_TOL
    dgu_rows = orc.swiglu_backward(gu_rows, dh_rows)
    assert mre(rows_of(g["dgu"], rows), dgu_rows) <= BF16_TOL
    DGU = np.zeros((L.T * L.K, 2 * L.f), np.uint16)
    DGU[rows] = dgu_rows
    dxp_rows = orc.grouped_dgrad(DGU, L.w1p, sizes, rows=rows)
    assert mre(rows_of(g["dx_perm"], rows), dxp_rows) <= BF16_TOL
    DXP = np.zeros((L.T * L.K, L.d), np.uint16)
    DXP[rows] = dxp_rows
    dx_ref = orc.unpermute_combine(DXP, None, dst, L.T, L.K)[tokens]
    assert mre(rows_of(g["dx"], tokens), dx_ref) <= BF16_TOL
    # weight gradients of a small, a middle-sized and an empty expert (full contraction over their rows)
    nz = np.nonzero(sizes)[0]
    order = nz[np.argsort(sizes[nz])]
    experts = [int(order[0]), int(order[len(order) // 2])]
    empty = int(np.nonzero(sizes == 0)[0][0])
    offs = np.concatenate([[0], np.cumsum(sizes)])
    for e in experts:
        er = np.arange(offs[e], offs[e + 1], dtype=np.int64)
        he, gue = orc.gemm_swiglu(xp, L.w1p, sizes, rows=er, keep_gu=True)
        He = np.zeros((L.T * L.K, L.f), np.uint16)
        He[er] = he
        dw2_ref = orc.grouped_wgrad(dyp_ref, He, sizes, groups=[e])[0]
        assert mre(host_u16(g["dw2"][e]), dw2_ref) <= BF16_TOL, e
        dhe = orc.grouped_dgrad(dyp_ref, L.w2, sizes, rows=er)
        dgue = orc.swiglu_backward(gue, dhe)
        DG = np.zeros((L.T * L.K, 2 * L.f), np.uint16)
        DG[er] = dgue
        dw1_ref = orc.grouped_wgrad(DG, xp, sizes, groups=[e])[0]
        assert mre(host_u16(g["dw1p"][e]), dw1_ref) <= BF16_TOL, e
    assert torch.all(g["dw2"][empty] == 0) and torch.all(g["dw1p"][empty] == 0)


@pytest.mark.parametrize("name", ["mixtral", "finegrained"])
def test_route_fused_full(ops, name):
    """The fused router at the routed workloads' full sizes (every token: the
    oracle's fp64 scores take a few seconds), with its dispatch maps."""
    from gpu_util import check_route_fused
    c = inputs.WORKLOADS[name]
    say("route fused full", name)
    x = inputs.workload(name, weights=False).x
    wr = inputs.router_weights(c["seed"], c["E"], c["d"])
    n_near, _ = check_route_fused(ops, x, wr, inputs.expert_bias(name), c["K"])
    assert n_near <= c["T"] // 200, n_near


def test_dsv3_share_mxfp4_full(ops):
    """The expert share in MXFP4 at full size, in the benchmark's launch
    configuration: the activations' codes and scales bit-exact over the whole
    tensor, weights of three experts bit-exact, both GEMMs on sampled rows
    against the oracle fed its own quantisation (H quantised by its own rule)."""
    say("full: dsv3 share mxfp4")
    L = inputs.workload("dsv3_share")
    s = L.group_sizes.numpy()
    dev = torch.device("cuda")
    x, w1, w2, sz = L.x_perm.to(dev), L.w1p.to(dev), L.w2.to(dev), L.group_sizes.to(dev)

    def boundary(q, sc):   # oracle layout -> two codes per byte, stage-major scales (data movement only)
        R, C = q.shape
        return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8), sc.reshape(R, C // 128, 4).transpose(1, 0, 2)

    xq, xs = ops.mxfp4_quantize(x)
    xq_ref, xs_ref = orc.mxfp4_quantize(L.x_perm)
    pq, ps = boundary(xq_ref, xs_ref)
    np.testing.assert_array_equal(xq.cpu().numpy(), pq)
    np.testing.assert_array_equal(xs.cpu().numpy(), ps)
    w1q, w1s = ops.mxfp4_quantize(w1)
    w2q, w2s = ops.mxfp4_quantize(w2)
    rows_w1 = 2 * L.f
    for e in (0, int(np.argmax(s)), L.E - 1):
        q_ref, s_ref = boundary(*orc.mxfp4_quantize(orc.u16(L.w1p[e])))
        np.testing.assert_array_equal(w1q[e].cpu().numpy(), q_ref)
        np.testing.assert_array_equal(w1s[:, e * rows_w1:(e + 1) * rows_w1].cpu().numpy(), s_ref)
    h = ops.grouped_gemm_mxfp4(xq, xs, w1q, w1s, sz, epilogue=ops.MOE_EPI_SWIGLU)
    hq, hs = ops.mxfp4_quantize(h)
    y = ops.grouped_gemm_mxfp4(hq, hs, w2q, w2s, sz)
    torch.cuda.synchronize()
    rows = sample_rows(s, 24, 5)
    w1q_ref, w1s_ref = orc.mxfp4_quantize(orc.u16(L.w1p).reshape(-1, L.d))
    w1q_ref, w1s_ref = w1q_ref.reshape(L.E, 2 * L.f, L.d), w1s_ref.reshape(L.E, 2 * L.f, L.d // 32)
    h_ref = orc.mx4_grouped_gemm(xq_ref, xs_ref, w1q_ref, w1s_ref, s, swiglu=True, rows=rows)
    assert rel_l2(rows_of(h, rows), h_ref) <= MX_TOL
    hq_ref, hs_ref = orc.mxfp4_quantize(h_ref)
    HQ = np.zeros((L.M, L.f), np.uint8)
    HS = np.zeros((L.M, L.f // 32), np.uint8)
    HQ[rows], HS[rows] = hq_ref, hs_ref
    w2q_ref, w2s_ref = orc.mxfp4_quantize(orc.u16(L.w2).reshape(-1, L.f))
    w2q_ref, w2s_ref = w2q_ref.reshape(L.E, L.d, L.f), w2s_ref.reshape(L.E, L.d, L.f // 32)
    y_ref = orc.mx4_grouped_gemm(HQ, HS, w2q_ref, w2s_ref, s, rows=rows)
    assert rel_l2(rows_of(y, rows), y_ref) <= MX_TOL
