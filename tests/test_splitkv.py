"""GPU parity of fa_fwd_splitkv (keys split into ranges, parts merged on the GPU) against the fp64 oracle.

* The merged result against the full definition, element by element, at the
  bf16 tolerances: decoding shapes (one to a few query rows over long,
  ragged key sequences; MHA, GQA, MQA; causal and not) and prefill shapes
  split over keys, for the library's own split count and explicit ones.
* The parts the kernel leaves in the workspace against the definition over
  each key range (attention_keys_fp64), which pins the range arithmetic and
  the layout the header documents.
* The decoding workload at full size (B8 Hq32 Hkv8, 32768 keys) in the
  launch configuration the benchmark times, on every row.
"""
import math

import numpy as np
import pytest

from exact_attention_07_amd import gen
from oracle import attention_fp64, attention_keys_fp64
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


def ranges(nk, nsplit):
    """Key ranges of an explicit split count: equal numbers of 64-key tiles."""
    tiles = math.ceil(nk / 64)
    want = min(nsplit, tiles)
    if want <= 1:
        return [(0, nk)]
    tps = math.ceil(tiles / want)
    return [(a * 64, min((a + tps) * 64, nk)) for a in range(0, tiles, tps)]


CASES = [
    # B, Hq, Hkv, Nq, Nk, d
    (2, 8, 2, 1, 4099, 128),     # decoding, GQA 4, ragged keys
    (1, 6, 6, 3, 2500, 64),      # three queries, MHA
    (1, 4, 1, 17, 3000, 256),    # MQA, 17 queries
    (3, 16, 2, 1, 1000, 128),    # GQA 8 (eight-wave workgroups)
    (1, 4, 2, 300, 1500, 128),   # prefill over several query blocks
    (1, 32, 1, 1, 3000, 128),    # 32 query heads packed into one wave
    (3, 6, 2, 10, 2000, 64),     # 3 heads x 10 rows packed
    (1, 4, 2, 16, 700, 256),     # 2 heads x 16 rows: every column
    (2, 64, 8, 8, 1500, 128),    # 8 heads x 8 rows: two waves of 4 heads
    (1, 24, 2, 10, 900, 64),     # 12 heads x 10 rows: four waves of 3 heads
    (1, 16, 1, 16, 700, 128),    # 16 heads x 16 rows: eight waves of 2 heads
    (1, 8, 1, 12, 500, 256),     # 8 heads x 12 rows: four waves of 2 heads
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nsplit", [0, 1, 3, 7, 1000])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_splitkv_matches_the_oracle(api, case, nsplit, causal):
    B, Hq, Hkv, Nq, Nk, d = case
    w = gen.workload(B, Hq, Hkv, Nq, Nk, d, causal=causal)
    x = gen.make_inputs(w, (sum(case), nsplit, int(causal), 11))
    print(f"case: splitkv {w.name} nsplit={nsplit}", flush=True)
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    o, lse = api.attention_splitkv(q, k, v, causal=causal, nsplit=nsplit)
    torch.cuda.synchronize()
    qf, kf, vf = (to_f64(x[t], "bf16") for t in "qkv")
    o_ref, lse_ref = attention_fp64(qf, kf, vf, w.softmax_scale, causal)
    compare(out_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, what=w.name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case,nsplit", [((2, 8, 2, 1, 4099, 128), 5), ((1, 4, 2, 300, 1500, 128), 4),
                                         ((1, 2, 2, 150, 90, 64), 2)],
                         ids=["decode", "prefill", "nq_gt_nk"])
def test_splitkv_parts_in_the_workspace(api, case, nsplit, causal):
    B, Hq, Hkv, Nq, Nk, d = case
    w = gen.workload(B, Hq, Hkv, Nq, Nk, d, causal=causal)
    x = gen.make_inputs(w, (sum(case), nsplit, int(causal), 12))
    print(f"case: splitkv parts {w.name} nsplit={nsplit}", flush=True)
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    rs = ranges(Nk, nsplit)
    nbytes = api.splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal, nsplit)
    rows = B * Hq * Nq
    assert nbytes == len(rs) * rows * (d + 1) * 4
    guard = 1024
    buf = torch.full((nbytes // 4 + guard,), 7.0, dtype=torch.float32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
    api.fa_fwd_splitkv(q, k, v, o, lse, w.softmax_scale, causal, nsplit, buf[: nbytes // 4])
    torch.cuda.synchronize()
    assert (buf[nbytes // 4:] == 7.0).all(), "writes past the workspace"
    ws = buf[: nbytes // 4].cpu().numpy().astype(np.float64)
    o_parts = ws[: len(rs) * rows * d].reshape(len(rs), B, Hq, Nq, d)
    l_parts = ws[len(rs) * rows * d:].reshape(len(rs), B, Hq, Nq)
    qf, kf, vf = (to_f64(x[t], "bf16") for t in "qkv")
    for s, (k0, k1) in enumerate(rs):
        o_ref, lse_ref = attention_keys_fp64(qf, kf, vf, w.softmax_scale, causal, k0, k1)
        compare(o_parts[s], l_parts[s], o_ref, lse_ref, what=f"{w.name} part {s} keys [{k0}, {k1})")
    o_all, lse_all = attention_fp64(qf, kf, vf, w.softmax_scale, causal)
    compare(out_to_f64(o), lse.cpu().numpy().astype(np.float64), o_all, lse_all, what=w.name)


def test_splitkv_agrees_with_fa_fwd(api):
    w = gen.workload(1, 8, 2, 64, 6000, 128, causal=True)
    x = gen.make_inputs(w, (13,))
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    o1, l1 = api.attention(q, k, v, causal=True)
    o2, l2 = api.attention_splitkv(q, k, v, causal=True, nsplit=6)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
    assert (l1 - l2).abs().max().item() <= 1e-3


def test_splitkv_workspace_errors(api):
    q = torch.zeros(1, 8, 1, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 4096, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(api.FaError) as e:
        api.fa_fwd_splitkv(q, k, k, o, None, 0.1, False, 4, None)
    assert e.value.status == 9
    small = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(api.FaError) as e:
        api.fa_fwd_splitkv(q, k, k, o, None, 0.1, False, 4, small)
    assert e.value.status == 9


def test_decode_workload_full_size(api):
    """The decoding workload the benchmark times (GQA B8 Hq32 Hkv8, one query
    over 32768 keys, d = 128, causal), in its launch configuration (the
    library's own split count), against the oracle on every one of its 256
    rows."""
    w, x = gen.make_config("decode")
    print(f"case: splitkv full size {w.name}", flush=True)
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    o, lse = api.attention_splitkv(q, k, v, causal=w.causal, scale=w.softmax_scale, nsplit=0)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_fp64(*(to_f64(x[t], "bf16") for t in "qkv"), w.softmax_scale, w.causal)
    compare(out_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, what=w.name)
