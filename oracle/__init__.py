"""fp64 CPU oracle for shared-latent MLA attention.  TEST INFRASTRUCTURE ONLY.

This package is the independent reference that the HIP path is checked
against.  Only the test-suite, the package entry's smoke check and the
benchmark's CPU-baseline leg may import or call it; the product path never
does, and it shares no code with the HIP kernels or their binding.

It computes the plain definitions the pages state, in float64 NumPy on the
bfloat16-rounded inputs, with a two-pass exact softmax (full score row, max,
exp, sum, divide).  Matrix products are done with NumPy's ``@``; no blocking,
fusion or reordering is added beyond iterating over independent rows.

Functions and the passages they follow:

* :func:`attention`   -- softmax(scale * Q K^T + causal mask) V with the
  log-sum-exp per row (TT-NN ``ring_mla`` description and "Returns";
  Ascend ``RingMLAOperation`` members ``prevLse``, ``qkScale``, ``maskType``,
  ``softmaxLse``).
* :func:`dense_mla`   -- the shared-latent form: one KV head whose full width
  is the key and whose first ``head_dim_v`` columns are the value (TT-NN
  ``ring_mla`` description and ``head_dim_v``; TensorRT-LLM ``mla.py``,
  ``MLA.__init__`` building the absorbed backend with
  ``head_dim = kv_lora_rank + qk_rope_head_dim``, ``num_kv_heads=1``,
  ``v_head_dim = kv_lora_rank``).
* :func:`merge`       -- fold of two partial results over disjoint key sets
  through their log-sum-exp (TensorRT-LLM ``mla.py``,
  ``forward_context_with_chunked_prefill`` and its FP4 twin's docstring:
  partial outputs merged with their softmax stats; Ascend ``calcType``:
  ``prevOut``/``prevLse`` folded into the new output).
* :func:`ring`        -- successive KV chunks on one device folded in ring
  order (TensorRT-LLM ``forward_context_with_chunked_prefill``: cached chunks
  with a FULL mask, the current chunk CAUSAL last; Ascend ``calcType``:
  first ring step without prev).
* :func:`split_mla`   -- the split query/key ring step with separate V,
  per-sequence ``seqLen`` and optional prev fold (Ascend
  ``AtbRingMLAGetWorkspaceSize`` member table).
* :func:`sparse_mla`  -- per-query attention over the top-k listed latent
  cache rows (NKI ``mla_sparse_attention_cte_kernel``, "Parameters" and
  "Returns").
* :func:`mx4_pack`    -- the MX 4-pack column order of the sparse output
  (NKI ``mla_sparse_attention_cte_kernel``, "Returns" and "Notes").
* :func:`vup`         -- the V-up projection of the latent output by the
  per-head ``v_b_proj`` weight (TensorRT-LLM ``mla.py``,
  ``forward_absorption_context`` and ``forward_absorption_generation``).
* :func:`decode_mla`  -- token generation: each sequence's newest query over
  its valid cache rows (Mojo ``mha_single_batch_pipelined``: seq_len = 1,
  ``num_keys``; split-K with a separate reduction).
* :func:`e4m3_decode`, :func:`dense_mla_fp8` -- the FP8 form: e4m3 codes
  decoded from the OCP FP8 definition, dequantised by their per-tensor scales
  and attended as :func:`dense_mla` (TensorRT-LLM ``mla.py``,
  ``forward_absorption_context`` with the fused FP8 query and the FP8 latent
  cache; the output stays bf16).  :func:`attention_weights` returns the exact
  softmax weights from which the tests bound the effect of the kernel's FP8
  P.V product.

Every function is pinned by ``tests/test_oracle.py`` against brute force on
tiny inputs, ``torch.nn.functional.scaled_dot_product_attention`` in float64,
closed forms, hand-worked values and the chunking invariants.
"""
from .mla_fp8 import attention_weights, dense_mla_fp8, e4m3_decode
from .mla_ref import (attention, decode_mla, dense_mla, merge, mx4_pack, ring, ring_order, split_mla,
                      sparse_mla, vup)

__all__ = ["attention", "attention_weights", "decode_mla", "dense_mla", "dense_mla_fp8", "e4m3_decode", "merge",
           "mx4_pack", "ring", "ring_order", "split_mla", "sparse_mla", "vup"]
