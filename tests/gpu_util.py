"""Helpers shared by the GPU tests (inputs from the seeded generators, host
copies for the oracle, error measures)."""
import sys

import numpy as np
import torch

import oracle as orc
from dropless_moe_expert_amd import inputs


def say(*a):
    """Name the case on stdout before a GPU step (survives a crash)."""
    print("[gpu case]", *a, flush=True)
    sys.stdout.flush()


def dev(t):
    return t.contiguous().cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16(rng: np.random.Generator, *shape, scale=1.0) -> torch.Tensor:
    return inputs.to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def max_rel_err(got: torch.Tensor, ref_u16: np.ndarray) -> float:
    """max |got - ref| / max |ref| over the whole tensor (bf16 outputs)."""
    g = orc.bf16_to_f64(host_u16(got))
    r = orc.bf16_to_f64(ref_u16)
    assert g.shape == r.shape, (g.shape, r.shape)
    denom = np.abs(r).max()
    return float(np.abs(g - r).max() / (denom if denom > 0 else 1.0))


def rel_l2(got: torch.Tensor, ref_u16: np.ndarray) -> float:
    g = orc.bf16_to_f64(host_u16(got))
    r = orc.bf16_to_f64(ref_u16)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))


BF16_TOL = 1e-2     # max relative error of bf16 outputs
MX_TOL = 2e-2       # relative L2 of MXFP8 outputs against the identically quantised oracle
W_RTOL = 1e-6       # routing weights: a few fp32 ulps (exp differs between libms)


def check_route_fused(ops, x: torch.Tensor, wr: torch.Tensor, bias, K: int, renorm: bool = True):
    """The fused router against the oracle's scores and selection.

    logits: |gpu - oracle| <= d * 2^-24 * sum_k |x_k w_ek| + 2^-23 |l| (fp32
    accumulation of d exact bf16 products, plus the bias add).  ids: wherever
    the oracle's sorted scores of a token's top K + 1 are separated by more
    than twice the largest logit error of its row (plus an fp32 rounding of
    the scores), the ids equal the oracle's exactly; for the other tokens the
    picks form a valid top-K within that margin.  Weights: within the error
    that the logit error implies, the oracle's on exactly matching tokens,
    and a softmax of the kernel's own logits elsewhere.  The dispatch maps of
    permute_routed equal moe_permute's on the same ids bit for bit, and the
    oracle's wherever all ids match.  Returns (n near-tie tokens, outputs)."""
    T, d = x.shape
    E = wr.shape[0]
    out = ops.route_fused(dev(x), dev(wr), K, bias=None if bias is None else dev(bias), renormalize=renorm,
                          keep_logits=True)
    pr = ops.permute_routed(dev(x), out["topk_ids"], E, out["ws"])
    torch.cuda.synchronize()
    ids = out["topk_ids"].cpu().numpy()
    w = out["topk_w"].cpu().numpy().astype(np.float64)
    lg = out["logits"].cpu().numpy().astype(np.float64)
    L = orc.route_logits(x, wr, bias)
    absx = np.abs(orc.bf16_to_f64(x))
    absw = np.abs(orc.bf16_to_f64(wr))
    bound = d * 2.0 ** -24 * (absx @ absw.T) + 2.0 ** -23 * np.abs(L)
    err = np.abs(lg - L)
    assert np.all(err <= bound), float((err - bound).max())
    if T == 0:
        return 0, out
    margin = 2.0 * err.max(axis=1) + 2.0 ** -22 * np.abs(L).max(axis=1)
    order = np.argsort(-L, axis=1, kind="stable")
    top = np.take_along_axis(L, order[:, :min(K + 1, E)], axis=1)
    gaps = top[:, :-1] - top[:, 1:] if top.shape[1] > 1 else np.full((T, 1), np.inf)
    clear = np.all(gaps > margin[:, None], axis=1)
    ids_ref, w_ref = orc.route_topk(L.astype(np.float32), K, renormalize=renorm)
    np.testing.assert_array_equal(ids[clear], ids_ref[clear])
    rtol = 4.0 * err.max() + 4.0 * W_RTOL
    np.testing.assert_allclose(w[clear], w_ref[clear], rtol=rtol, atol=1e-30)
    for t in np.nonzero(~clear)[0]:
        s = ids[t]
        assert len(set(s.tolist())) == K and s.min() >= 0 and s.max() < E
        rest = np.setdiff1d(np.arange(E), s)
        if rest.size:
            assert L[t, s].min() >= L[t, rest].max() - margin[t]
        assert np.all(L[t, s][:-1] >= L[t, s][1:] - margin[t])
        m = lg[t, s[0]]
        den = np.exp(lg[t, s] - m).sum() if renorm else np.exp(lg[t] - m).sum()
        np.testing.assert_allclose(w[t], np.exp(lg[t, s] - m) / den, rtol=1e-5)
    # dispatch maps: against moe_permute on the same ids, and the oracle's when every id matches
    ref = ops.permute(dev(x), out["topk_ids"], E)
    torch.cuda.synchronize()
    for k in ("group_sizes", "group_offsets", "perm_src", "perm_dst"):
        np.testing.assert_array_equal(pr[k].cpu().numpy(), ref[k].cpu().numpy(), err_msg=k)
    np.testing.assert_array_equal(host_u16(pr["x_perm"]), host_u16(ref["x_perm"]))
    if np.array_equal(ids, ids_ref):
        sizes, offs, src, dst = orc.permute(ids_ref, E)
        np.testing.assert_array_equal(pr["group_sizes"].cpu().numpy(), sizes)
        np.testing.assert_array_equal(pr["group_offsets"].cpu().numpy(), offs)
        np.testing.assert_array_equal(pr["perm_src"].cpu().numpy(), src)
        np.testing.assert_array_equal(pr["perm_dst"].cpu().numpy(), dst)
        np.testing.assert_array_equal(host_u16(pr["x_perm"]), orc.gather_rows(x, src, K))
    return int((~clear).sum()), out


# ---------------------------------------------------------------- full-size sampling helpers

def mre_u16(got_u16, ref_u16) -> float:
    """max |got - ref| / max |ref| of two bf16 bit arrays."""
    g, r = orc.bf16_to_f64(got_u16), orc.bf16_to_f64(ref_u16)
    assert g.shape == r.shape, (g.shape, r.shape)
    return float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-30))


def rel_l2_u16(got_u16, ref_u16) -> float:
    g, r = orc.bf16_to_f64(got_u16), orc.bf16_to_f64(ref_u16)
    assert g.shape == r.shape, (g.shape, r.shape)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))


def sample_rows(sizes, n_extra, seed):
    """Every non-empty group's first and last row plus n_extra random rows."""
    offs = np.concatenate([[0], np.cumsum(sizes)])
    rows = []
    for g in range(len(sizes)):
        if sizes[g] > 0:
            rows += [offs[g], offs[g + 1] - 1]
    rng = np.random.default_rng(seed)
    rows += list(rng.choice(int(offs[-1]), size=n_extra, replace=False))
    return np.unique(np.array(rows, np.int64))


def rows_of(t: torch.Tensor, rows) -> np.ndarray:
    """bf16 rows of a device tensor as uint16 bits on the host."""
    return host_u16(t[torch.from_numpy(np.asarray(rows, np.int64)).to(t.device)])
