"""GPU: qdot_attn_decode_kv4_noalloc (the attention call whose workspace is
the library's static device array, for callers that cannot allocate)
against qdot_attn_decode_kv4 with a caller workspace: the same kernels, so
the outputs must be bitwise equal; both also against the oracle at the
attention tests' bar.  Two calls in a row, the second smaller, so the second
runs on what the first left in the array; the first at the array's limit."""
import math

import numpy as np
import pytest

import oracle
from quant_integer_dot_amd import binding as qd

from gpu_util import dev, to_dev
from test_gpu_attn import D, case, check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qd.load()


def largest_T(Hq):
    """Longest context whose workspace fits the static array."""
    per_chunk = Hq * (D + 2) * 4
    return QDOT_LIMIT // per_chunk * 256


QDOT_LIMIT = qd.QDOT_ATTN_NOALLOC_BYTES


def test_noalloc_equals_workspace_call_twice():
    import torch
    cases = [(4, 1, largest_T(4)), (8, 2, 700)]   # the second smaller than the first
    assert qd.qdot_attn_kv4_workspace_bytes(4, cases[0][2]) <= QDOT_LIMIT
    assert qd.qdot_attn_kv4_workspace_bytes(4, cases[0][2] + 256) > QDOT_LIMIT
    for Hq, Hkv, T in cases:
        scale = np.float32(1 / math.sqrt(D))
        K, V, xqd, xq = case(Hq, Hkv, T, 500 + Hq)
        Kd, Vd = to_dev(K), to_dev(V)
        out_na = torch.full((Hq, D), float("nan"), dtype=torch.float32, device=dev())
        qd.qdot_attn_decode_kv4_noalloc(xqd, Hq, Kd, Vd, Hkv, T, D, scale, out_na)
        torch.cuda.synchronize()
        nb = qd.qdot_attn_kv4_workspace_bytes(Hq, T)
        ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device=dev())
        out_ws = torch.full((Hq, D), float("nan"), dtype=torch.float32, device=dev())
        qd.qdot_attn_decode_kv4(xqd, Hq, Kd, Vd, Hkv, T, D, scale, out_ws, ws, nb)
        torch.cuda.synchronize()
        a, b = out_na.cpu().numpy(), out_ws.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"T={T}: no-alloc != workspace call"
        o64, sc = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
        check(a, o64, V, sc, Hq, Hkv, f"no-alloc Hq={Hq} T={T}")
