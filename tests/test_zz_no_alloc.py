"""moe_permute_noalloc (the permute for callers that cannot allocate: its
workspace lives in the library's static device memory) against moe_permute,
through the C ABI: every output bit for bit, on two calls in a row with the
second smaller, outputs pre-filled so that a missing write shows."""
import numpy as np
import pytest
import torch

from gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    from dropless_moe_expert_amd import ops as _ops
    _ops.load_library()
    return _ops


def _case(rng, T, E, K, d):
    ids = np.array([rng.permutation(E)[:K] for _ in range(T)], dtype=np.int32).reshape(T, K)
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    return dev(x), dev(torch.from_numpy(ids))


def _filled(T, E, K, d):
    M = T * K
    return dict(group_sizes=torch.full((E,), -7, dtype=torch.int32, device="cuda"),
                group_offsets=torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
                perm_src=torch.full((M,), -7, dtype=torch.int32, device="cuda"),
                perm_dst=torch.full((M,), -7, dtype=torch.int32, device="cuda"),
                x_perm=torch.full((M, d), 3.0, dtype=torch.bfloat16, device="cuda"))


def test_permute_noalloc_matches_permute(ops):
    rng = np.random.default_rng(77)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    # fine-grained routing shape, then a smaller Mixtral-like call (second call smaller)
    for T, E, K, d in [(16384, 128, 8, 256), (1000, 8, 2, 512)]:
        say("permute noalloc", T, E, K, d)
        x, ids = _case(rng, T, E, K, d)
        want = ops.permute(x, ids, E, flag=flag)
        got = ops.permute_noalloc(x, ids, E, flag=flag, out=_filled(T, E, K, d))
        torch.cuda.synchronize()
        for k in ("group_sizes", "group_offsets", "perm_src", "perm_dst"):
            assert torch.equal(got[k], want[k]), k
        assert torch.equal(got["x_perm"].view(torch.int16), want["x_perm"].view(torch.int16))
        assert int(flag.item()) == 0
    # maps only (x = NULL)
    say("permute noalloc maps only")
    x, ids = _case(rng, 300, 16, 4, 64)
    want = ops.permute(None, ids, 16)
    got = ops.permute_noalloc(None, ids, 16)
    torch.cuda.synchronize()
    for k in ("group_sizes", "group_offsets", "perm_src", "perm_dst"):
        assert torch.equal(got[k], want[k]), k


def test_permute_noalloc_rejects_past_its_scratch(ops):
    # 2^20 + 256 pairs with E = 256 need more than the 8 MiB of static scratch;
    # the check is on the host, before any launch
    L = ops.lib()
    fake = 1 << 20
    T = (1 << 17) + 32
    assert L.moe_permute_workspace_bytes(T, 256, 8) > (8 << 20)
    assert L.moe_permute_noalloc(None, fake, T, 0, 256, 8, fake, fake, fake, fake, None, None, None) == 4
