"""fp64 CPU oracle for exact attention (forward pass and its gradient).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only the test-suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP path.

Contents
  attention.attention_fp64      plain definition, S and P materialised (two passes)
  attention.attention_rows_fp64 the same definition for a chosen set of query rows
  attention.online_fp64         tile-by-tile online softmax with a rescale threshold
  attention.attention_keys_fp64 the definition over one key range (a part of split attention)
  attention.merge_fp64          exact combination of parts over disjoint key ranges
  attention.attention_backward_fp64  gradients dQ, dK, dV of the definition for a given dO
  formats                       bf16 / OCP e4m3 decoding and e4m3 round-to-nearest-even
  fp8                           Hadamard rotation and the per-tensor e4m3 quantisation step
"""
from .attention import (attention_backward_fp64, attention_fp64, attention_keys_fp64, attention_rows_fp64, kv_head_of,
                        merge_fp64, online_fp64)
from . import formats, fp8

__all__ = ["attention_fp64", "attention_rows_fp64", "attention_keys_fp64", "merge_fp64", "online_fp64", "kv_head_of",
           "attention_backward_fp64", "formats", "fp8"]
