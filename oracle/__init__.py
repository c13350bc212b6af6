"""CPU oracle for one batched codec-LM decode step.

TEST INFRASTRUCTURE, NOT THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The GPU library never routes
through it, and it shares no code with ``codec_language_model_amd``: it
imports only numpy and works on the unpaged, logical arrays a caller would
hold (except ``kv``, which defines the paged append itself).

Each function is the plain definition of what the step computes, written out
with explicit loops over streams, heads and queries:

* ``kv``        - appending new K/V rows into the paged cache (16-token blocks,
                  "Dynamic Token-Level Batching", Optimizing Streaming
                  Text-to-Speech Models for Sub-50 Millisecond Latency).
* ``attention`` - single- or K-query GQA softmax attention over each stream's
                  cache ("Token generation under a frame budget", TTS Serving,
                  in depth: one decode step per frame reads the KV cache).
* ``head``      - the codebook logit projection (TontaubeV1, audio head
                  paragraph and codec paragraph for the vocabulary sizes).
* ``sampling``  - greedy argmax and temperature sampling with a supplied
                  uniform; masking of logits outside the target vocabulary
                  (TontaubeV1 Section 3.3).
* ``step``      - the chained step: append, attention, o in the step's
                  element type, head, token choice or verification.
* ``verify``    - speculative accept/reject with residual resampling
                  ("Speculative Decoding for Acoustic Tokens", Optimizing
                  Streaming Text-to-Speech Models ...).

Precision: attention and the head accumulate in float64 (the pages fix no
precision).  Sampling and verification decide integers, so they compute in
float32, the precision the GPU kernels decide in.
"""

from .attention import attend, attention_weights, decode_attention
from .head import codebook_head, codebook_head_mlp, mish
from .kv import gather_logical, kv_cache_append
from .rope import rope, rope_kv_cache_append
from . import fp8
from .sampling import argmax_token, inverse_cdf, sample_or_argmax, sample_token
from .verify import spec_verify, spec_verify_stream, target_probs
from .step import decode_step, round_to_bf16

__all__ = [
    "attend", "attention_weights", "decode_attention", "codebook_head",
    "gather_logical", "kv_cache_append", "argmax_token", "inverse_cdf",
    "sample_or_argmax", "sample_token", "spec_verify", "spec_verify_stream",
    "codebook_head_mlp", "mish", "rope", "rope_kv_cache_append",
    "target_probs", "decode_step", "round_to_bf16",
]
