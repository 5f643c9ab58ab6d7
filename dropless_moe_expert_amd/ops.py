"""Python binding of libmoe.so: argument marshalling only.

Every step of the layer runs in the library's HIP kernels.  torch supplies
device memory and the current HIP stream; this module allocates outputs,
checks dtypes and shapes, passes raw pointers through ``ctypes`` and turns a
non-zero status into an exception.  There is no CPU fallback: without the
built library (or without a GPU) every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libmoe.so")

MOE_DTYPE_BF16, MOE_DTYPE_MXFP8, MOE_DTYPE_MXFP4 = 0, 1, 2
MOE_RAGGED_M, MOE_RAGGED_K = 0, 1
MOE_B_NK, MOE_B_KN, MOE_B_PACKED = 0, 1, 2
MOE_EPI_NONE, MOE_EPI_SWIGLU, MOE_EPI_SWIGLU_MXFP8, MOE_EPI_SWIGLU_BWD = 0, 1, 2, 3
MOE_OUT_BF16, MOE_OUT_F32 = 0, 1

FLAG_BAD_EXPERT_ID = 0x1
FLAG_ROWS_OVER_CAP = 0x2
FLAG_NEGATIVE_SIZE = 0x4
FLAG_NAN_LOGIT = 0x8

EXPORTS = (
    "moe_abi_version", "moe_status_string", "moe_route_topk", "moe_permute_workspace_bytes", "moe_permute",
    "moe_permute_mxfp8", "moe_permute_noalloc", "grouped_gemm_workspace_bytes", "grouped_gemm", "moe_unpermute_combine",
    "moe_combine_backward", "moe_combine_backward_mxfp8",
    "moe_swiglu_backward", "moe_swiglu_backward_mxfp8", "mxfp8_group_quantize", "mxfp8_quantize_transposed",
    "mxfp8_quantize_gathered",
    "moe_pack_weights_bytes",
    "moe_pack_weights",
    "moe_pack_weights_mxfp8_bytes", "moe_pack_weights_mxfp8",
    "moe_route_fused_workspace_bytes", "moe_route_fused", "moe_permute_routed", "mxfp4_quantize",
    # measurement only (include/moe_bench.h)
    "moe_bench_mfma_flops", "moe_bench_mfma_ceiling",
)


class MoeError(RuntimeError):
    pass


class GGDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("ragged", ctypes.c_int32), ("b_layout", ctypes.c_int32),
                ("epilogue", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("G", ctypes.c_int32),
                ("M", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("m_cap", ctypes.c_int64)]


_lock = threading.Lock()
_lib = None


def load_library(path: str = LIB_PATH, require_gpu: bool = True):
    """dlopen libmoe.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise MoeError(f"{path} is not built; run dropless_moe_expert_amd.build.build()")
        if require_gpu and not torch.cuda.is_available():
            raise MoeError("no GPU visible: the dropless MoE kernels run only on an MI355X (gfx950)")
        L = ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)
        P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        sig = {
            "moe_abi_version": (ctypes.c_int, []),
            "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "moe_route_topk": (ctypes.c_int, [P, i64, i32, i32, i32, P, P, P, P]),
            "moe_permute_workspace_bytes": (sz, [i64, i32, i32]),
            "moe_permute": (ctypes.c_int, [P, P, i64, i32, i32, i32, P, P, P, P, P, P, sz, P, P]),
            "moe_permute_mxfp8": (ctypes.c_int, [P, P, i64, i32, i32, i32, P, P, P, P, P, P, P, sz, P, P]),
            "moe_permute_noalloc": (ctypes.c_int, [P, P, i64, i32, i32, i32, P, P, P, P, P, P, P]),
            "grouped_gemm_workspace_bytes": (sz, [ctypes.POINTER(GGDesc)]),
            "grouped_gemm": (ctypes.c_int, [ctypes.POINTER(GGDesc), P, P, P, P, P, P, P, P, sz, P, P]),
            "moe_unpermute_combine": (ctypes.c_int, [P, P, P, i64, i32, i32, P, P]),
            "moe_combine_backward": (ctypes.c_int, [P, P, P, P, i64, i32, i32, P, P, P]),
            "moe_swiglu_backward": (ctypes.c_int, [P, P, i64, i32, P, i32, P, P]),
            "mxfp8_group_quantize": (ctypes.c_int, [P, i64, i32, i32, P, i32, P, P, P, P]),
            "mxfp8_quantize_transposed": (ctypes.c_int, [P, i64, i32, P, i32, i64, P, P, P, P, P, P]),
            "moe_swiglu_backward_mxfp8": (ctypes.c_int, [P, P, i64, i32, P, i32, i64, P, P, P, P, P, P]),
            "mxfp8_quantize_gathered": (ctypes.c_int, [P, P, P, i64, i32, i32, P, i32, i64, P, P, P, P, P, P]),
            "moe_combine_backward_mxfp8": (ctypes.c_int, [P, P, P, P, i64, i32, i32, P, P, P, P]),
            "moe_pack_weights_bytes": (sz, [i32, i32, i32, i32]),
            "moe_pack_weights": (ctypes.c_int, [P, i32, i32, i32, i32, P, sz, P]),
            "moe_pack_weights_mxfp8_bytes": (sz, [i32, i32, i32, i32]),
            "moe_pack_weights_mxfp8": (ctypes.c_int, [P, P, i32, i32, i32, i32, P, sz, P]),
            "moe_route_fused_workspace_bytes": (sz, [i64, i32, i32]),
            "moe_route_fused": (ctypes.c_int, [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, sz, P, P]),
            "moe_permute_routed": (ctypes.c_int, [P, P, i64, i32, i32, i32, P, P, P, P, P, P, sz, P, P]),
            "mxfp4_quantize": (ctypes.c_int, [P, i64, i32, P, P, P]),
            "moe_bench_mfma_flops": (i64, [i64, i32]),
            "moe_bench_mfma_ceiling": (ctypes.c_int, [i32, i32, P, i64, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
        if require_gpu:
            _check_single_hip_runtime()
        return _lib


def _check_single_hip_runtime() -> None:
    """libmoe.so must bind to the HIP runtime torch already loaded."""
    try:
        with open("/proc/self/maps") as f:
            paths = {l.split()[-1] for l in f if "libamdhip64" in l}
    except OSError:  # pragma: no cover
        return
    if len(paths) > 1:
        raise MoeError(f"two HIP runtimes are mapped ({sorted(paths)}); streams and pointers would not be shared")


def lib():
    return _lib if _lib is not None else load_library()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().moe_status_string(status).decode()
        raise MoeError(f"{what}: status {status} ({msg})")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise MoeError("tensors must be on the GPU")
            if not t.is_contiguous():
                raise MoeError("tensors must be contiguous")
    return ts[0].device


def new_flag(device) -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=device)


# ------------------------------------------------------------------ steps

def route_topk(logits: torch.Tensor, K: int, renormalize: bool = True, flag: Optional[torch.Tensor] = None):
    """-> (topk_ids int32 [T,K], topk_w fp32 [T,K])."""
    assert logits.dtype == torch.float32 and logits.dim() == 2
    dev = _dev(logits)
    T, E = logits.shape
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    _check(lib().moe_route_topk(_ptr(logits), T, E, K, int(renormalize), _ptr(ids), _ptr(w), _ptr(flag),
                                _stream(dev)), "moe_route_topk")
    return ids, w


def permute(x: Optional[torch.Tensor], topk_ids: torch.Tensor, E: int, flag: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None):
    """-> dict(group_sizes, group_offsets, perm_src, perm_dst, x_perm)."""
    assert topk_ids.dtype == torch.int32 and topk_ids.dim() == 2
    dev = _dev(topk_ids, x)
    T, K = topk_ids.shape
    d = 0 if x is None else x.shape[1]
    if x is not None:
        assert x.dtype == torch.bfloat16 and x.shape[0] == T
    M = T * K
    out = dict(
        group_sizes=torch.empty(E, dtype=torch.int32, device=dev),
        group_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        perm_src=torch.empty(M, dtype=torch.int32, device=dev),
        perm_dst=torch.empty(M, dtype=torch.int32, device=dev),
        x_perm=None if x is None else torch.empty((M, d), dtype=torch.bfloat16, device=dev),
    )
    need = lib().moe_permute_workspace_bytes(T, E, K)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(lib().moe_permute(_ptr(x), _ptr(topk_ids), T, d, E, K, _ptr(out["group_sizes"]),
                             _ptr(out["group_offsets"]), _ptr(out["perm_src"]), _ptr(out["perm_dst"]),
                             _ptr(out["x_perm"]), _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _ptr(flag), _stream(dev)), "moe_permute")
    return out


def permute_noalloc(x: Optional[torch.Tensor], topk_ids: torch.Tensor, E: int, flag: Optional[torch.Tensor] = None,
                    out: Optional[dict] = None):
    """moe_permute_noalloc: moe_permute's outputs, workspace in the library's
    static device memory (no allocation inside the call).  `out` may supply
    the output tensors (keys as returned), so that nothing at all is
    allocated."""
    assert topk_ids.dtype == torch.int32 and topk_ids.dim() == 2
    dev = _dev(topk_ids, x)
    T, K = topk_ids.shape
    d = 0 if x is None else x.shape[1]
    if x is not None:
        assert x.dtype == torch.bfloat16 and x.shape[0] == T
    M = T * K
    if out is None:
        out = dict(
            group_sizes=torch.empty(E, dtype=torch.int32, device=dev),
            group_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
            perm_src=torch.empty(M, dtype=torch.int32, device=dev),
            perm_dst=torch.empty(M, dtype=torch.int32, device=dev),
            x_perm=None if x is None else torch.empty((M, d), dtype=torch.bfloat16, device=dev),
        )
    _check(lib().moe_permute_noalloc(_ptr(x), _ptr(topk_ids), T, d, E, K, _ptr(out["group_sizes"]),
                                     _ptr(out["group_offsets"]), _ptr(out["perm_src"]), _ptr(out["perm_dst"]),
                                     _ptr(out["x_perm"]), _ptr(flag), _stream(dev)), "moe_permute_noalloc")
    return out


def permute_mxfp8(x: torch.Tensor, topk_ids: torch.Tensor, E: int, flag: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None):
    """Permute with MXFP8 output -> dict(group_sizes, group_offsets, perm_src,
    perm_dst, xq uint8 [T*K, d], xs uint8 [T*K, d/32])."""
    assert topk_ids.dtype == torch.int32 and topk_ids.dim() == 2 and x.dtype == torch.bfloat16
    dev = _dev(topk_ids, x)
    T, K = topk_ids.shape
    d = x.shape[1]
    M = T * K
    out = dict(
        group_sizes=torch.empty(E, dtype=torch.int32, device=dev),
        group_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        perm_src=torch.empty(M, dtype=torch.int32, device=dev),
        perm_dst=torch.empty(M, dtype=torch.int32, device=dev),
        xq=torch.empty((M, d), dtype=torch.uint8, device=dev),
        xs=torch.empty((M, d // 32), dtype=torch.uint8, device=dev),
    )
    need = lib().moe_permute_workspace_bytes(T, E, K)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(lib().moe_permute_mxfp8(_ptr(x), _ptr(topk_ids), T, d, E, K, _ptr(out["group_sizes"]),
                                   _ptr(out["group_offsets"]), _ptr(out["perm_src"]), _ptr(out["perm_dst"]),
                                   _ptr(out["xq"]), _ptr(out["xs"]), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _ptr(flag), _stream(dev)),
           "moe_permute_mxfp8")
    return out


def route_fused(x: torch.Tensor, w_router: torch.Tensor, K: int, bias: Optional[torch.Tensor] = None,
                renormalize: bool = True, keep_logits: bool = False, histogram: bool = True,
                flag: Optional[torch.Tensor] = None):
    """Fused router: logits = x w_router^T (+ bias), top-K, softmax weights and
    (histogram=True) the dispatch histogram for permute_routed.
    -> dict(topk_ids int32 [T,K], topk_w fp32 [T,K], logits fp32 [T,E] or None,
            ws uint8 workspace or None)."""
    assert x.dtype == torch.bfloat16 and w_router.dtype == torch.bfloat16
    assert x.dim() == 2 and w_router.dim() == 2 and x.shape[1] == w_router.shape[1]
    assert x.is_contiguous() and w_router.is_contiguous()
    dev = _dev(x, w_router, bias)
    T, d = x.shape
    E = w_router.shape[0]
    if bias is not None:
        assert bias.dtype == torch.float32 and bias.shape == (E,) and bias.is_contiguous()
    out = dict(topk_ids=torch.empty((T, K), dtype=torch.int32, device=dev),
               topk_w=torch.empty((T, K), dtype=torch.float32, device=dev),
               logits=torch.empty((T, E), dtype=torch.float32, device=dev) if keep_logits else None,
               ws=None)
    nbytes = 0
    if histogram:
        nbytes = max(int(lib().moe_route_fused_workspace_bytes(T, E, K)), 256)
        out["ws"] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(lib().moe_route_fused(_ptr(x), _ptr(w_router), _ptr(bias), T, d, E, K, int(renormalize),
                                 _ptr(out["topk_ids"]), _ptr(out["topk_w"]), _ptr(out["logits"]), _ptr(out["ws"]),
                                 nbytes, _ptr(flag), _stream(dev)), "moe_route_fused")
    return out


def permute_routed(x: Optional[torch.Tensor], topk_ids: torch.Tensor, E: int, ws: torch.Tensor,
                   flag: Optional[torch.Tensor] = None):
    """moe_permute's outputs from route_fused's histogram (ws is consumed)."""
    assert topk_ids.dtype == torch.int32 and topk_ids.dim() == 2 and ws is not None
    dev = _dev(topk_ids, x, ws)
    T, K = topk_ids.shape
    d = 0 if x is None else x.shape[1]
    M = T * K
    out = dict(
        group_sizes=torch.empty(E, dtype=torch.int32, device=dev),
        group_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        perm_src=torch.empty(M, dtype=torch.int32, device=dev),
        perm_dst=torch.empty(M, dtype=torch.int32, device=dev),
        x_perm=None if x is None else torch.empty((M, d), dtype=torch.bfloat16, device=dev),
    )
    _check(lib().moe_permute_routed(_ptr(x), _ptr(topk_ids), T, d, E, K, _ptr(out["group_sizes"]),
                                    _ptr(out["group_offsets"]), _ptr(out["perm_src"]), _ptr(out["perm_dst"]),
                                    _ptr(out["x_perm"]), _ptr(ws), ws.numel() * ws.element_size(), _ptr(flag),
                                    _stream(dev)), "moe_permute_routed")
    return out


class PackedWeights:
    """Expert weights [G, N, K] rewritten by moe_pack_weights (bf16) or
    moe_pack_weights_mxfp8 for one epilogue; usable only as B of the forward
    grouped GEMM of that dtype with that epilogue."""

    def __init__(self, data: torch.Tensor, G: int, N: int, K: int, epilogue: int, mxfp8: bool = False):
        self.data, self.G, self.N, self.K, self.epilogue, self.mxfp8 = data, G, N, K, epilogue, mxfp8

    @property
    def shape(self):
        return (self.G, self.N, self.K)

    @property
    def device(self):
        return self.data.device


def pack_weights(W: torch.Tensor, epilogue: int = MOE_EPI_NONE) -> PackedWeights:
    """Pack W bf16 [G, N, K] (B_NK) for the forward GEMM with this epilogue."""
    dev = _dev(W)
    assert W.dtype == torch.bfloat16 and W.dim() == 3 and W.is_contiguous()
    G, N, Kd = W.shape
    need = lib().moe_pack_weights_bytes(G, N, Kd, epilogue)
    if need == 0:
        raise MoeError(f"moe_pack_weights: unsupported shape {tuple(W.shape)} / epilogue {epilogue}")
    data = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().moe_pack_weights(_ptr(W), G, N, Kd, epilogue, _ptr(data), need, _stream(dev)), "moe_pack_weights")
    return PackedWeights(data, G, N, Kd, epilogue)


def pack_weights_mxfp8(Bq: torch.Tensor, Bs: torch.Tensor, epilogue: int = MOE_EPI_NONE) -> PackedWeights:
    """Pack MXFP8 weights (codes uint8 [G, N, K], scales uint8 [G, N, K/32])."""
    dev = _dev(Bq, Bs)
    assert Bq.dtype == torch.uint8 and Bs.dtype == torch.uint8 and Bq.dim() == 3
    G, N, Kd = Bq.shape
    assert tuple(Bs.shape) == (G, N, Kd // 32)
    need = lib().moe_pack_weights_mxfp8_bytes(G, N, Kd, epilogue)
    if need == 0:
        raise MoeError(f"moe_pack_weights_mxfp8: unsupported shape {tuple(Bq.shape)} / epilogue {epilogue}")
    data = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().moe_pack_weights_mxfp8(_ptr(Bq), _ptr(Bs), G, N, Kd, epilogue, _ptr(data), need, _stream(dev)),
           "moe_pack_weights_mxfp8")
    return PackedWeights(data, G, N, Kd, epilogue, mxfp8=True)


_gemm_ws = {}   # device index -> the ragged-M calls' workspace (one per device)


def _gemm_workspace(d: "GGDesc", dev: torch.device) -> Optional[torch.Tensor]:
    """The library's workspace for this call (grouped_gemm_workspace_bytes),
    allocated once per device and shared by this module's calls, which run
    on the device's current stream one after another."""
    need = lib().grouped_gemm_workspace_bytes(ctypes.byref(d))
    if need == 0:
        return None
    ws = _gemm_ws.get(dev.index)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        _gemm_ws[dev.index] = ws
    return ws


def grouped_gemm(A: torch.Tensor, B, group_sizes: torch.Tensor, *, b_layout: int = MOE_B_NK,
                 epilogue: int = MOE_EPI_NONE, out_dtype: torch.dtype = torch.bfloat16, keep_aux: bool = False,
                 out: Optional[torch.Tensor] = None, aux: Optional[torch.Tensor] = None,
                 flag: Optional[torch.Tensor] = None, split: bool = True):
    """Ragged-M grouped GEMM, bf16.  A [m_cap, K]; B [G, N, K] (NK), [G, K, N]
    (KN) or PackedWeights.  Returns C [m_cap, N] (or [m_cap, N/2] with SwiGLU)
    and, with keep_aux, the pre-activations [m_cap, N].  With
    MOE_EPI_SWIGLU_BWD (KN): aux = the forward's pre-activations [m_cap, 2N]
    (read), returns [dg | du] [m_cap, 2N] from dh = bf16(A Bop).  Rows past
    sum(group_sizes) are left untouched.  split: pass the library its
    workspace, so that a short last round of tiles is split along K."""
    packed = isinstance(B, PackedWeights)
    Bt = B.data if packed else B
    dev = _dev(A, Bt, group_sizes)
    assert A.dtype == torch.bfloat16 and group_sizes.dtype == torch.int32
    m_cap, Kd = A.shape
    if packed:
        if B.mxfp8 or B.epilogue != epilogue or B.K != Kd or b_layout != MOE_B_NK:
            raise MoeError("packed weights used with another epilogue, K or layout than they were packed for")
        b_layout = MOE_B_PACKED
    else:
        assert B.dtype == torch.bfloat16
    G = B.shape[0]
    N = B.shape[2] if b_layout == MOE_B_KN else B.shape[1]
    ncols = N // 2 if epilogue == MOE_EPI_SWIGLU else 2 * N if epilogue == MOE_EPI_SWIGLU_BWD else N
    if epilogue == MOE_EPI_SWIGLU_BWD and (aux is None or aux.shape != (m_cap, 2 * N)):
        raise MoeError("MOE_EPI_SWIGLU_BWD reads the forward's pre-activations: aux [m_cap, 2N]")
    if out is None:
        out = torch.empty((m_cap, ncols), dtype=out_dtype, device=dev)
    if keep_aux and aux is None:
        aux = torch.empty((m_cap, N), dtype=torch.bfloat16, device=dev)
    d = GGDesc(MOE_DTYPE_BF16, MOE_RAGGED_M, b_layout, epilogue,
               MOE_OUT_F32 if out_dtype == torch.float32 else MOE_OUT_BF16, G, 0, N, Kd, m_cap)
    ws = _gemm_workspace(d, dev) if split else None
    _check(lib().grouped_gemm(ctypes.byref(d), _ptr(A), None, _ptr(Bt), None, _ptr(group_sizes), _ptr(out),
                              _ptr(aux), _ptr(ws), ws.numel() if ws is not None else 0, _ptr(flag), _stream(dev)),
           "grouped_gemm")
    return (out, aux) if keep_aux else out


def grouped_gemm_wgrad(X: torch.Tensor, Y: torch.Tensor, group_sizes: torch.Tensor, *,
                       out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                       flag: Optional[torch.Tensor] = None):
    """Ragged-K grouped GEMM: C[g] = sum over group g's rows r of X[r]^T Y[r] -> [G, P, Q]."""
    dev = _dev(X, Y, group_sizes)
    m_cap, P = X.shape
    Q = Y.shape[1]
    G = group_sizes.numel()
    if out is None:
        out = torch.empty((G, P, Q), dtype=out_dtype, device=dev)
    d = GGDesc(MOE_DTYPE_BF16, MOE_RAGGED_K, MOE_B_NK, MOE_EPI_NONE,
               MOE_OUT_F32 if out_dtype == torch.float32 else MOE_OUT_BF16, G, P, Q, 0, m_cap)
    _check(lib().grouped_gemm(ctypes.byref(d), _ptr(X), None, _ptr(Y), None, _ptr(group_sizes), _ptr(out), None,
                              None, 0, _ptr(flag), _stream(dev)), "grouped_gemm (ragged K)")
    return out


def grouped_gemm_wgrad_mxfp8(AqT: torch.Tensor, AsT: torch.Tensor, BqT: torch.Tensor, BsT: torch.Tensor,
                             group_sizes: torch.Tensor, m_cap: int, *, out: Optional[torch.Tensor] = None,
                             flag: Optional[torch.Tensor] = None):
    """MXFP8 weight gradient: C[g] = sum over group g's rows of a[r]^T b[r] -> bf16 [G, P, Q],
    from mxfp8_quantize_transposed(a, group_sizes) (codes [P, k_cap]) and the same of b ([Q, k_cap])."""
    dev = _dev(AqT, AsT, BqT, BsT, group_sizes)
    P, k_cap = AqT.shape
    Q = BqT.shape[0]
    G = group_sizes.numel()
    if out is None:
        out = torch.empty((G, P, Q), dtype=torch.bfloat16, device=dev)
    d = GGDesc(MOE_DTYPE_MXFP8, MOE_RAGGED_K, MOE_B_NK, MOE_EPI_NONE, MOE_OUT_BF16, G, P, Q, k_cap, m_cap)
    _check(lib().grouped_gemm(ctypes.byref(d), _ptr(AqT), _ptr(AsT), _ptr(BqT), _ptr(BsT), _ptr(group_sizes),
                              _ptr(out), None, None, 0, _ptr(flag), _stream(dev)), "grouped_gemm (MXFP8, ragged K)")
    return out


def mxfp4_quantize(x: torch.Tensor):
    """bf16 [rows, cols] (or [G, N, K] weights, quantised as G*N rows) ->
    (codes uint8 [..., cols/2], two E2M1 codes per byte, element 2i in the low
    nibble; scales uint8 [cols/128, rows, 4], stage-major E8M0 per 32)."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous()
    dev = _dev(x)
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    codes = torch.empty(tuple(x.shape[:-1]) + (cols // 2,), dtype=torch.uint8, device=dev)
    scales = torch.empty((cols // 128, rows, 4), dtype=torch.uint8, device=dev)
    _check(lib().mxfp4_quantize(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(dev)), "mxfp4_quantize")
    return codes, scales


def grouped_gemm_mxfp4(Aq: torch.Tensor, As: torch.Tensor, Bq: torch.Tensor, Bs: torch.Tensor,
                       group_sizes: torch.Tensor, *, epilogue: int = MOE_EPI_NONE,
                       out: Optional[torch.Tensor] = None, flag: Optional[torch.Tensor] = None):
    """MXFP4 ragged-M grouped GEMM from mxfp4_quantize's outputs: Aq [m_cap, K/2],
    As [K/128, m_cap, 4], Bq [G, N, K/2], Bs [K/128, G*N, 4] -> bf16 [m_cap, N]
    (N/2 with MOE_EPI_SWIGLU: rows [0, N/2) of each expert are the gate)."""
    dev = _dev(Aq, As, Bq, Bs, group_sizes)
    m_cap, Kh = Aq.shape
    G, N = Bq.shape[0], Bq.shape[1]
    ncols = N // 2 if epilogue == MOE_EPI_SWIGLU else N
    if out is None:
        out = torch.empty((m_cap, ncols), dtype=torch.bfloat16, device=dev)
    d = GGDesc(MOE_DTYPE_MXFP4, MOE_RAGGED_M, MOE_B_NK, epilogue, MOE_OUT_BF16, G, 0, N, 2 * Kh, m_cap)
    _check(lib().grouped_gemm(ctypes.byref(d), _ptr(Aq), _ptr(As), _ptr(Bq), _ptr(Bs), _ptr(group_sizes), _ptr(out),
                              None, None, 0, _ptr(flag), _stream(dev)), "grouped_gemm (mxfp4)")
    return out


def grouped_gemm_mxfp8(Aq: torch.Tensor, As: torch.Tensor, Bq, Bs: Optional[torch.Tensor],
                       group_sizes: torch.Tensor, *, epilogue: int = MOE_EPI_NONE,
                       out: Optional[torch.Tensor] = None, out_scale: Optional[torch.Tensor] = None,
                       keep_aux: bool = False, flag: Optional[torch.Tensor] = None, split: bool = True):
    """MXFP8 ragged-M grouped GEMM.  Aq uint8 [m_cap, K], As uint8 [m_cap, K/32],
    Bq uint8 [G, N, K] with Bs uint8 [G, N, K/32], or Bq = PackedWeights from
    pack_weights_mxfp8 (Bs None) -> bf16 [m_cap, N] (or N/2 with SwiGLU).
    With MOE_EPI_SWIGLU_MXFP8 (weights packed for MOE_EPI_SWIGLU, or
    unpacked) -> (codes uint8 [m_cap, N/2], scales uint8 [m_cap, N/64]): the
    SwiGLU output quantised as mxfp8_quantize(h, 0) would.  keep_aux (with
    MOE_EPI_SWIGLU) -> (h, pre-activations bf16 [m_cap, N]).  split: pass
    the library its workspace (a short last round of tiles split along K)."""
    packed = isinstance(Bq, PackedWeights)
    m_cap, Kd = Aq.shape
    fused = epilogue == MOE_EPI_SWIGLU_MXFP8
    if packed:
        want = MOE_EPI_SWIGLU if fused else epilogue
        if not Bq.mxfp8 or Bq.epilogue != want or Bq.K != Kd:
            raise MoeError("packed weights used with another dtype, epilogue or K than they were packed for")
        dev = _dev(Aq, As, Bq.data, group_sizes)
        Bt, layout = Bq.data, MOE_B_PACKED
    else:
        dev = _dev(Aq, As, Bq, Bs, group_sizes)
        Bt, layout = Bq, MOE_B_NK
    G, N = Bq.shape[0], Bq.shape[1]
    ncols = N // 2 if epilogue != MOE_EPI_NONE else N
    if fused:
        if out is None:
            out = torch.empty((m_cap, ncols), dtype=torch.uint8, device=dev)
        if out_scale is None:
            out_scale = torch.empty((m_cap, ncols // 32), dtype=torch.uint8, device=dev)
    elif out is None:
        out = torch.empty((m_cap, ncols), dtype=torch.bfloat16, device=dev)
    aux = None
    if keep_aux:
        if epilogue != MOE_EPI_SWIGLU:
            raise MoeError("keep_aux needs the SwiGLU epilogue")
        aux = torch.empty((m_cap, N), dtype=torch.bfloat16, device=dev)
    d = GGDesc(MOE_DTYPE_MXFP8, MOE_RAGGED_M, layout, epilogue, MOE_OUT_BF16, G, 0, N, Kd, m_cap)
    ws = _gemm_workspace(d, dev) if split else None
    _check(lib().grouped_gemm(ctypes.byref(d), _ptr(Aq), _ptr(As), _ptr(Bt), None if packed else _ptr(Bs),
                              _ptr(group_sizes), _ptr(out), _ptr(out_scale) if fused else _ptr(aux), _ptr(ws),
                              ws.numel() if ws is not None else 0, _ptr(flag), _stream(dev)), "grouped_gemm (mxfp8)")
    if fused:
        return out, out_scale
    return (out, aux) if keep_aux else out


def unpermute_combine(y_perm: torch.Tensor, topk_w: Optional[torch.Tensor], perm_dst: torch.Tensor, T: int, K: int,
                      out: Optional[torch.Tensor] = None):
    dev = _dev(y_perm, perm_dst, topk_w)
    d = y_perm.shape[1]
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    _check(lib().moe_unpermute_combine(_ptr(y_perm), _ptr(topk_w), _ptr(perm_dst), T, d, K, _ptr(out),
                                       _stream(dev)), "moe_unpermute_combine")
    return out


def combine_backward(dy: torch.Tensor, y_perm: torch.Tensor, topk_w: torch.Tensor, perm_dst: torch.Tensor, K: int,
                     weights_only: bool = False):
    """-> (dy_perm bf16 [T*K, d], d_topk_w fp32 [T, K]); weights_only: dy_perm
    is not formed (None), as when mxfp8_quantize_gathered delivers it quantised."""
    dev = _dev(dy, y_perm, topk_w, perm_dst)
    T, d = dy.shape
    dyp = None if weights_only else torch.empty((T * K, d), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((T, K), dtype=torch.float32, device=dev)
    _check(lib().moe_combine_backward(_ptr(dy), _ptr(y_perm), _ptr(topk_w), _ptr(perm_dst), T, d, K, _ptr(dyp),
                                      _ptr(dw), _stream(dev)), "moe_combine_backward")
    return dyp, dw


def combine_backward_mxfp8(dy: torch.Tensor, y_perm: torch.Tensor, topk_w: torch.Tensor, perm_dst: torch.Tensor,
                           K: int):
    """-> (dy_perm row codes uint8 [T*K, d], their scales [T*K, d/32],
    d_topk_w fp32 [T, K]): combine_backward with dy_perm quantised along its
    rows as it is formed (mxfp8_quantize(dy_perm, 0) bit for bit)."""
    dev = _dev(dy, y_perm, topk_w, perm_dst)
    T, d = dy.shape
    q = torch.empty((T * K, d), dtype=torch.uint8, device=dev)
    sc = torch.empty((T * K, d // 32), dtype=torch.uint8, device=dev)
    dw = torch.empty((T, K), dtype=torch.float32, device=dev)
    _check(lib().moe_combine_backward_mxfp8(_ptr(dy), _ptr(y_perm), _ptr(topk_w), _ptr(perm_dst), T, d, K, _ptr(q),
                                            _ptr(sc), _ptr(dw), _stream(dev)), "moe_combine_backward_mxfp8")
    return q, sc, dw


def swiglu_backward(gu: torch.Tensor, dh: torch.Tensor, group_sizes: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None):
    dev = _dev(gu, dh, group_sizes)
    m_cap, f = dh.shape
    if out is None:
        out = torch.empty((m_cap, 2 * f), dtype=torch.bfloat16, device=dev)
    G = 0 if group_sizes is None else group_sizes.numel()
    _check(lib().moe_swiglu_backward(_ptr(gu), _ptr(dh), m_cap, f, _ptr(group_sizes), G, _ptr(out),
                                     _stream(dev)), "moe_swiglu_backward")
    return out


def mxfp8_quantize(x: torch.Tensor, axis: int = 0, group_sizes: Optional[torch.Tensor] = None,
                   flag: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """-> (codes uint8 [rows, cols], scales uint8): axis 0 [rows, cols/32]; axis 1 [rows/32 + G, cols]."""
    dev = _dev(x, group_sizes)
    assert x.dtype == torch.bfloat16
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if axis == 0:
        s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    else:
        s = torch.empty((rows // 32 + group_sizes.numel(), cols), dtype=torch.uint8, device=dev)
    G = 0 if group_sizes is None else group_sizes.numel()
    _check(lib().mxfp8_group_quantize(_ptr(x), rows, cols, axis, _ptr(group_sizes), G, _ptr(q), _ptr(s), _ptr(flag),
                                      _stream(dev)), "mxfp8_group_quantize")
    return q, s


def k_cap_for(m_cap: int, G: int) -> int:
    """Positions per row of the grouped transposed layout: room for every
    group starting 64-aligned."""
    return (m_cap + 63 * G + 63) // 64 * 64


def mxfp8_quantize_transposed(x: torch.Tensor, group_sizes: Optional[torch.Tensor] = None,
                              flag: Optional[torch.Tensor] = None, rows_too: bool = False):
    """Blocks of 32 down the columns, codes stored column-contiguous.
    x [rows, cols] with group_sizes -> (qT uint8 [cols, k_cap], scaleT [cols, k_cap/32]);
    x [G, rows, cols] without -> (qT [G, cols, rows], scaleT [G, cols, rows/32]).
    rows_too: also the axis-0 codes and scales of the same rows (as
    mxfp8_quantize(x, 0)), from the same read: returns (qT, scaleT, q, scale)."""
    dev = _dev(x, group_sizes)
    assert x.dtype == torch.bfloat16
    if group_sizes is not None:
        rows, cols = x.shape
        G = group_sizes.numel()
        k_cap = k_cap_for(rows, G)
        q = torch.empty((cols, k_cap), dtype=torch.uint8, device=dev)
        s = torch.empty((cols, k_cap // 32), dtype=torch.uint8, device=dev)
    else:
        G, rows, cols = x.shape
        k_cap = 0
        q = torch.empty((G, cols, rows), dtype=torch.uint8, device=dev)
        s = torch.empty((G, cols, rows // 32), dtype=torch.uint8, device=dev)
    q0 = s0 = None
    if rows_too:
        q0 = torch.empty(x.shape, dtype=torch.uint8, device=dev)
        s0 = torch.empty(tuple(x.shape[:-1]) + (cols // 32,), dtype=torch.uint8, device=dev)
    _check(lib().mxfp8_quantize_transposed(_ptr(x), rows, cols, _ptr(group_sizes), G, k_cap, _ptr(q), _ptr(s),
                                           _ptr(q0), _ptr(s0), _ptr(flag), _stream(dev)), "mxfp8_quantize_transposed")
    return (q, s, q0, s0) if rows_too else (q, s)


def mxfp8_quantize_gathered(x: torch.Tensor, perm_src: torch.Tensor, K: int, group_sizes: torch.Tensor,
                            topk_w: Optional[torch.Tensor] = None, flag: Optional[torch.Tensor] = None,
                            rows_too: bool = False):
    """mxfp8_quantize_transposed(x_perm, group_sizes, rows_too=...) without
    x_perm: row r is x[perm_src[r] // K] (moe_permute's x_perm), or with
    topk_w that row times topk_w.flatten()[perm_src[r]] rounded to bf16
    (moe_combine_backward's dy_perm for dy = x).  x bf16 [T, cols]."""
    dev = _dev(x, perm_src, group_sizes, topk_w)
    assert x.dtype == torch.bfloat16 and perm_src.dtype == torch.int32
    T, cols = x.shape
    M = T * K
    G = group_sizes.numel()
    k_cap = k_cap_for(M, G)
    q = torch.empty((cols, k_cap), dtype=torch.uint8, device=dev)
    s = torch.empty((cols, k_cap // 32), dtype=torch.uint8, device=dev)
    q0 = s0 = None
    if rows_too:
        q0 = torch.empty((M, cols), dtype=torch.uint8, device=dev)
        s0 = torch.empty((M, cols // 32), dtype=torch.uint8, device=dev)
    _check(lib().mxfp8_quantize_gathered(_ptr(x), _ptr(perm_src), _ptr(topk_w), T, K, cols, _ptr(group_sizes), G,
                                         k_cap, _ptr(q), _ptr(s), _ptr(q0), _ptr(s0), _ptr(flag), _stream(dev)),
           "mxfp8_quantize_gathered")
    return (q, s, q0, s0) if rows_too else (q, s)


def swiglu_backward_mxfp8(gu: torch.Tensor, dh: torch.Tensor, group_sizes: torch.Tensor,
                          flag: Optional[torch.Tensor] = None):
    """SwiGLU backward delivered as MXFP8 only: (qT, scaleT, q, scale) equal to
    mxfp8_quantize_transposed(swiglu_backward(gu, dh), group_sizes, rows_too=True)."""
    dev = _dev(gu, dh, group_sizes)
    m_cap, f = dh.shape
    G = group_sizes.numel()
    k_cap = k_cap_for(m_cap, G)
    qT = torch.empty((2 * f, k_cap), dtype=torch.uint8, device=dev)
    sT = torch.empty((2 * f, k_cap // 32), dtype=torch.uint8, device=dev)
    q = torch.empty((m_cap, 2 * f), dtype=torch.uint8, device=dev)
    sc = torch.empty((m_cap, 2 * f // 32), dtype=torch.uint8, device=dev)
    _check(lib().moe_swiglu_backward_mxfp8(_ptr(gu), _ptr(dh), m_cap, f, _ptr(group_sizes), G, k_cap, _ptr(qT),
                                           _ptr(sT), _ptr(q), _ptr(sc), _ptr(flag), _stream(dev)),
           "moe_swiglu_backward_mxfp8")
    return qT, sT, q, sc


# ------------------------------------------------------------------ measurement only

def bench_mfma_ceiling(random_operands: bool, iters: int, blocks: int, device) -> Tuple[torch.Tensor, int]:
    """Enqueues the MFMA ceiling kernel (include/moe_bench.h) on the current
    stream; returns its sink tensor and the FLOPs of the call."""
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=device)
    _check(lib().moe_bench_mfma_ceiling(int(bool(random_operands)), iters, _ptr(sink), blocks, _stream(sink.device)),
           "moe_bench_mfma_ceiling")
    return sink, int(lib().moe_bench_mfma_flops(blocks, iters))


# ------------------------------------------------------------------ the layer

def moe_forward(logits: torch.Tensor, x: torch.Tensor, w1p: torch.Tensor, w2: torch.Tensor, K: int,
                keep: bool = False, flag: Optional[torch.Tensor] = None):
    """Router top-K -> permute -> GEMM + SwiGLU -> GEMM -> combine.  Returns y
    [T, d] and, if keep, the intermediates the backward needs."""
    E = w1p.shape[0]
    T = x.shape[0]
    ids, w = route_topk(logits, K, flag=flag)
    p = permute(x, ids, E, flag=flag)
    if keep:
        h, gu = grouped_gemm(p["x_perm"], w1p, p["group_sizes"], epilogue=MOE_EPI_SWIGLU, keep_aux=True, flag=flag)
    else:
        h, gu = grouped_gemm(p["x_perm"], w1p, p["group_sizes"], epilogue=MOE_EPI_SWIGLU, flag=flag), None
    y_perm = grouped_gemm(h, w2, p["group_sizes"], flag=flag)
    y = unpermute_combine(y_perm, w, p["perm_dst"], T, K)
    if not keep:
        return y, None
    return y, dict(ids=ids, w=w, h=h, gu=gu, y_perm=y_perm, **p)


def moe_forward_mxfp8(logits: torch.Tensor, x: torch.Tensor, w1k, w2k, K: int,
                      flag: Optional[torch.Tensor] = None):
    """The routed layer on MXFP8 operands: router top-K -> permute writing
    MXFP8 rows -> gate/up GEMM quantising its SwiGLU output -> down GEMM ->
    combine.  w1k / w2k: PackedWeights from pack_weights_mxfp8 (gate/up packed
    for MOE_EPI_SWIGLU).  Returns y [T, d] bf16 and the intermediates."""
    T = x.shape[0]
    ids, w = route_topk(logits, K, flag=flag)
    p = permute_mxfp8(x, ids, w1k.G, flag=flag)
    hq, hs = grouped_gemm_mxfp8(p["xq"], p["xs"], w1k, None, p["group_sizes"], epilogue=MOE_EPI_SWIGLU_MXFP8,
                                flag=flag)
    y_perm = grouped_gemm_mxfp8(hq, hs, w2k, None, p["group_sizes"], flag=flag)
    y = unpermute_combine(y_perm, w, p["perm_dst"], T, K)
    return y, dict(ids=ids, w=w, hq=hq, hs=hs, y_perm=y_perm, **p)


def moe_forward_mxfp4(logits: torch.Tensor, x: torch.Tensor, w1: tuple, w2: tuple, K: int,
                      flag: Optional[torch.Tensor] = None):
    """The routed layer on MXFP4 operands: router top-K -> permute -> quantise
    the permuted rows -> gate/up GEMM with SwiGLU -> quantise h -> down GEMM ->
    combine.  w1 / w2: (codes, scales) from mxfp4_quantize of the [E, 2f, d]
    gate/up weight and the [E, d, f] down weight.  Returns y [T, d] bf16 and
    the intermediates."""
    T = x.shape[0]
    E = w1[0].shape[0]
    ids, w = route_topk(logits, K, flag=flag)
    p = permute(x, ids, E, flag=flag)
    xq, xs = mxfp4_quantize(p["x_perm"])
    h = grouped_gemm_mxfp4(xq, xs, w1[0], w1[1], p["group_sizes"], epilogue=MOE_EPI_SWIGLU, flag=flag)
    hq, hs = mxfp4_quantize(h)
    y_perm = grouped_gemm_mxfp4(hq, hs, w2[0], w2[1], p["group_sizes"], flag=flag)
    y = unpermute_combine(y_perm, w, p["perm_dst"], T, K)
    return y, dict(ids=ids, w=w, xq=xq, xs=xs, h=h, hq=hq, hs=hs, y_perm=y_perm, **p)


def moe_backward(dy: torch.Tensor, saved: dict, w1p: torch.Tensor, w2: torch.Tensor, K: int,
                 flag: Optional[torch.Tensor] = None, fused: bool = True):
    """Backward of moe_forward (routing weights' gradient included, router
    logits' not).  fused: the down projection's data gradient forms SwiGLU's
    backward in its epilogue (dh is not written; None in the result); else
    dh is written and moe_swiglu_backward reads it (the same bits)."""
    sizes, dst = saved["group_sizes"], saved["perm_dst"]
    T = dy.shape[0]
    dyp, dw = combine_backward(dy, saved["y_perm"], saved["w"], dst, K)
    if fused:
        dh = None
        dgu = grouped_gemm(dyp, w2, sizes, b_layout=MOE_B_KN, epilogue=MOE_EPI_SWIGLU_BWD, aux=saved["gu"],
                           flag=flag)
    else:
        dh = grouped_gemm(dyp, w2, sizes, b_layout=MOE_B_KN, flag=flag)       # dY_perm [M,d] x W2_e [d,f]
        dgu = swiglu_backward(saved["gu"], dh, sizes)
    dw2 = grouped_gemm_wgrad(dyp, saved["h"], sizes, flag=flag)                # [E, d, f]
    dxp = grouped_gemm(dgu, w1p, sizes, b_layout=MOE_B_KN, flag=flag)          # dGU [M,2f] x W1p_e [2f,d]
    dw1p = grouped_gemm_wgrad(dgu, saved["x_perm"], sizes, flag=flag)          # [E, 2f, d]
    dx = unpermute_combine(dxp, None, dst, T, K)
    return dict(dy_perm=dyp, dw=dw, dh=dh, dw2=dw2, dgu=dgu, dx_perm=dxp, dw1p=dw1p, dx=dx)


def quantize_weights_mxfp8_train(w1p: torch.Tensor, w2: torch.Tensor, flag: Optional[torch.Tensor] = None):
    """The four MXFP8 weight operands of a training step, packed: W1p [E, 2f, d]
    and W2 [E, d, f] quantised along their forward contraction (for the
    forward GEMMs) and along their output axis (for the data gradients, via
    the transposed quantiser: W2^T [E, f, d] blocks along d, W1p^T [E, d, 2f]
    blocks along 2f)."""
    q1t, s1t, q1, s1 = mxfp8_quantize_transposed(w1p, flag=flag, rows_too=True)
    q2t, s2t, q2, s2 = mxfp8_quantize_transposed(w2, flag=flag, rows_too=True)
    return dict(w1k=pack_weights_mxfp8(q1, s1, MOE_EPI_SWIGLU), w2k=pack_weights_mxfp8(q2, s2),
                w2tk=pack_weights_mxfp8(q2t, s2t), w1tk=pack_weights_mxfp8(q1t, s1t))


def moe_forward_mxfp8_train(logits: torch.Tensor, x: torch.Tensor, wk: dict, K: int,
                            flag: Optional[torch.Tensor] = None, fused: bool = True):
    """The routed layer on MXFP8 operands, keeping what the backward needs:
    route -> permute -> quantise -> gate/up GEMM + SwiGLU (bf16 h and
    pre-activations) -> quantise h -> down GEMM -> combine.  wk from
    quantize_weights_mxfp8_train.  fused: no bf16 x_perm (None): the row
    codes come from permute_mxfp8, the transposed ones from
    mxfp8_quantize_gathered; else permute writes bf16 x_perm and
    mxfp8_quantize_transposed reads it."""
    T = x.shape[0]
    ids, w = route_topk(logits, K, flag=flag)
    # x and h quantised both ways: along their rows for the forward GEMMs,
    # down the tokens (kept) for the weight gradients
    if fused:
        # the dispatch quantises each token row once for its K rows, the
        # transposed codes come from the rows gathered from x
        p = permute_mxfp8(x, ids, wk["w1k"].G, flag=flag)
        sizes = p["group_sizes"]
        xq, xs = p.pop("xq"), p.pop("xs")
        p["x_perm"] = None
        xT, xsT = mxfp8_quantize_gathered(x, p["perm_src"], K, sizes, flag=flag)
    else:
        p = permute(x, ids, wk["w1k"].G, flag=flag)
        sizes = p["group_sizes"]
        xT, xsT, xq, xs = mxfp8_quantize_transposed(p["x_perm"], sizes, flag=flag, rows_too=True)
    h, gu = grouped_gemm_mxfp8(xq, xs, wk["w1k"], None, sizes, epilogue=MOE_EPI_SWIGLU, keep_aux=True, flag=flag)
    hT, hsT, hq, hs = mxfp8_quantize_transposed(h, sizes, flag=flag, rows_too=True)
    y_perm = grouped_gemm_mxfp8(hq, hs, wk["w2k"], None, sizes, flag=flag)
    y = unpermute_combine(y_perm, w, p["perm_dst"], T, K)
    return y, dict(ids=ids, w=w, h=h, gu=gu, y_perm=y_perm, xT=xT, xsT=xsT, hT=hT, hsT=hsT, **p)


def moe_backward_mxfp8(dy: torch.Tensor, saved: dict, wk: dict, K: int, flag: Optional[torch.Tensor] = None,
                       fused: bool = True):
    """Backward of moe_forward_mxfp8_train with MXFP8 GEMMs: the data gradients
    quantise their left operands along the contraction and use the weights
    quantised along their output axis; the weight gradients quantise both
    operands down the tokens, blocks restarting at every expert's rows
    (group-aware MXFP8).  Combine, SwiGLU backward and the dx fold stay bf16;
    fused: dy_perm (the combine's backward) and dgu (the SwiGLU backward)
    are delivered as MXFP8 only, by mxfp8_quantize_gathered and
    swiglu_backward_mxfp8 (both None in the result)."""
    sizes, dst = saved["group_sizes"], saved["perm_dst"]
    T = dy.shape[0]
    m_cap = saved["h"].shape[0]
    if fused:
        # dy_perm's row codes as the combine's backward forms it, its
        # transposed codes from dy gathered and weighted again
        dyp = None
        q, sc, dw = combine_backward_mxfp8(dy, saved["y_perm"], saved["w"], dst, K)
        aT, asT = mxfp8_quantize_gathered(dy, saved["perm_src"], K, sizes, topk_w=saved["w"], flag=flag)
    else:
        dyp, dw = combine_backward(dy, saved["y_perm"], saved["w"], dst, K)
        aT, asT, q, sc = mxfp8_quantize_transposed(dyp, sizes, flag=flag, rows_too=True)
    dh = grouped_gemm_mxfp8(q, sc, wk["w2tk"], None, sizes, flag=flag)                    # [M, f]
    dw2 = grouped_gemm_wgrad_mxfp8(aT, asT, saved["hT"], saved["hsT"], sizes, m_cap, flag=flag)  # [E, d, f]
    if fused:
        dgu = None
        aT, asT, q, sc = swiglu_backward_mxfp8(saved["gu"], dh, sizes, flag=flag)
    else:
        dgu = swiglu_backward(saved["gu"], dh, sizes)
        aT, asT, q, sc = mxfp8_quantize_transposed(dgu, sizes, flag=flag, rows_too=True)
    dxp = grouped_gemm_mxfp8(q, sc, wk["w1tk"], None, sizes, flag=flag)                   # [M, d]
    dw1p = grouped_gemm_wgrad_mxfp8(aT, asT, saved["xT"], saved["xsT"], sizes, m_cap, flag=flag)  # [E, 2f, d]
    dx = unpermute_combine(dxp, None, dst, T, K)
    return dict(dy_perm=dyp, dw=dw, dh=dh, dw2=dw2, dgu=dgu, dx_perm=dxp, dw1p=dw1p, dx=dx)


def expert_mlp(x_perm: torch.Tensor, group_sizes: torch.Tensor, w1p: torch.Tensor, w2: torch.Tensor,
               flag: Optional[torch.Tensor] = None, h: Optional[torch.Tensor] = None,
               y: Optional[torch.Tensor] = None):
    """The expert share alone (rows already permuted): GEMM + SwiGLU, then GEMM."""
    h = grouped_gemm(x_perm, w1p, group_sizes, epilogue=MOE_EPI_SWIGLU, out=h, flag=flag)
    return grouped_gemm(h, w2, group_sizes, out=y, flag=flag), h


def expert_mlp_mxfp8(x_perm: torch.Tensor, group_sizes: torch.Tensor, w1q, w1s, w2q, w2s,
                     flag: Optional[torch.Tensor] = None, fused: bool = False):
    """MXFP8 expert share: quantise X, GEMM + SwiGLU, quantise H, GEMM.  Weights
    come pre-quantised ([G, N, K] codes with [G, N, K/32] scales), or packed
    (PackedWeights from pack_weights_mxfp8, with w1s = w2s = None).  fused:
    the gate/up GEMM quantises H in its epilogue (no bf16 H)."""
    xq, xs = mxfp8_quantize(x_perm, 0, group_sizes, flag=flag)
    if fused:
        hq, hs = grouped_gemm_mxfp8(xq, xs, w1q, w1s, group_sizes, epilogue=MOE_EPI_SWIGLU_MXFP8, flag=flag)
        h = None
    else:
        h = grouped_gemm_mxfp8(xq, xs, w1q, w1s, group_sizes, epilogue=MOE_EPI_SWIGLU, flag=flag)
        hq, hs = mxfp8_quantize(h, 0, group_sizes, flag=flag)
    y = grouped_gemm_mxfp8(hq, hs, w2q, w2s, group_sizes, flag=flag)
    return y, dict(xq=xq, xs=xs, h=h, hq=hq, hs=hs)


def quantize_weights(w: torch.Tensor):
    """[G, N, K] bf16 -> (codes [G, N, K], scales [G, N, K/32]) along K."""
    G, N, Kd = w.shape
    q, s = mxfp8_quantize(w.reshape(G * N, Kd), 0)
    return q.view(G, N, Kd), s.view(G, N, Kd // 32)
