"""fa_fwd_splitkv_noalloc (the key-split forward pass with its parts in the
library's fixed per-GPU scratch) against fa_fwd_splitkv with a caller
workspace, through the C ABI: two calls in a row, the second smaller, each
bit-equal to the existing entry point and within the bf16 bar of the oracle."""
import numpy as np
import pytest

from exact_attention_07_amd import gen
from oracle import attention_fp64
from tests.gpu_util import compare, out_to_f64, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_07_amd import api as a
    a.lib()
    return a


CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal, nsplit: the first needs more scratch than the second
    (4, 32, 8, 1, 9000, 128, True, 0),
    (2, 8, 2, 3, 2100, 64, False, 5),
]


def test_noalloc_matches_workspace_entry_point_twice(api):
    for i, (B, Hq, Hkv, Nq, Nk, d, causal, nsplit) in enumerate(CASES):
        w = gen.workload(B, Hq, Hkv, Nq, Nk, d, causal=causal)
        print(f"case: noalloc {w.name} nsplit={nsplit}", flush=True)
        x = gen.make_inputs(w, (31, i))
        q, k, v = (to_device(x[t], "bf16") for t in "qkv")
        need = api.splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal, nsplit)
        assert 0 < need <= 32 * 1024 * 1024, need
        ws = torch.empty(need // 4, dtype=torch.float32, device="cuda")
        o_ref = torch.empty_like(q)
        lse_ref = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        api.fa_fwd_splitkv(q, k, v, o_ref, lse_ref, w.softmax_scale, causal, nsplit, ws)
        o = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        api.fa_fwd_splitkv_noalloc(q, k, v, o, lse, w.softmax_scale, causal, nsplit)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), w.name
        assert torch.equal(lse, lse_ref), w.name
        oq, ok_, ov = (to_f64(x[t], "bf16") for t in "qkv")
        o64, l64 = attention_fp64(oq, ok_, ov, w.softmax_scale, causal)
        compare(out_to_f64(o), lse.cpu().numpy().astype(np.float64), o64, l64, what=w.name)
