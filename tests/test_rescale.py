"""How often the threshold rule skips the output rescaling, on the standing
workloads' own rows (CPU, the tile-by-tile fp64 model of the kernels' online
softmax).

"FlashAttention-4震撼发布" (first algorithmic improvement) reports that about
90 % of the output rescalings are skipped; the pages give no rule.  The
kernels rescale a wave's 32 rows only when some row's running maximum has
grown by more than TAU = 8 (log2 units) since the maximum its exponentials
use; oracle.online_fp64 takes the same decision per group of 32 rows and
64-key tile and counts it.  A sample of 32-row groups of the causal GQA
long-context workload and of the outlier-channel workload is run over all
the keys the rows see (the kernels' tile boundaries), with TAU = 8 and with
TAU = 0 (the classic rule: every growth of the maximum rescales).  The result
must stay exact whatever the rule (checked against the two-pass oracle)."""
import numpy as np
import pytest

from exact_attention_07_amd import gen
from oracle import attention_fp64, online_fp64
from oracle.formats import bf16_bits_to_f64


def _skip_fraction(w, x, groups, tau):
    events = decisions = 0
    g = w.Hq // w.Hkv
    for b, h, p0 in groups:
        q = bf16_bits_to_f64(x["q"][b:b + 1, h:h + 1, p0:p0 + 32])
        nk = p0 + 32 if w.causal else w.Nk
        k = bf16_bits_to_f64(x["k"][b:b + 1, h // g:h // g + 1, :nk])
        v = bf16_bits_to_f64(x["v"][b:b + 1, h // g:h // g + 1, :nk])
        # Nq = 32 rows against nk keys: bottom-right causal alignment puts
        # row i at position p0 + i, as in the full problem
        o, lse, (ev, dec) = online_fp64(q, k, v, w.softmax_scale, w.causal, 64, tau, group=32)
        if tau == 8.0 and (b, h, p0) == groups[0]:
            o_ref, lse_ref = attention_fp64(q, k, v, w.softmax_scale, w.causal)
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)
        events += ev
        decisions += dec
    return 1.0 - events / decisions, events, decisions


@pytest.mark.parametrize("cfg", [3, 4])
def test_threshold_rule_skips_most_rescalings(cfg):
    w, x = gen.make_config(cfg)
    rng = np.random.default_rng(cfg)
    n = 8 if cfg == 3 else 4
    groups = [(int(rng.integers(w.B)), int(rng.integers(w.Hq)), 32 * int(rng.integers(w.Nq // 32))) for _ in range(n)]
    groups[0] = (0, 0, w.Nq - 32)   # the longest causal row range
    skip8, ev8, dec8 = _skip_fraction(w, x, groups, 8.0)
    skip0, ev0, dec0 = _skip_fraction(w, x, groups, 0.0)
    print(f"{w.name}: TAU=8 skips {skip8:.4f} of rescalings ({ev8} of {dec8} group-tile steps rescale); "
          f"TAU=0 skips {skip0:.4f} ({ev0} of {dec0})")
    assert skip8 >= 0.9
    assert skip0 < skip8
