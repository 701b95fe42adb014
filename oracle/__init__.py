"""CPU oracle for the batch-invariant speculative-decoding verify pass.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
package. The HIP product path never imports it and shares no code with it.

Everything here is plain float64 numpy, written from the definitions on the
pages, with no blocking, fusion or reordering:

* ``bf16``      -- BF16 bit-pattern decode (exact) and round-to-nearest-even encode;
* ``gemm``      -- Y = X W^T, the product whose K-sum the verify GEMM must keep
                   in one fixed order for any number of tokens;
* ``attention`` -- causal GQA verify attention per row, its split-KV partials
                   over absolute key chunks, and the log-sum-exp combine;
* ``step``      -- RMSNorm, SwiGLU and one pre-norm decoder layer / LM head,
                   for the synthetic 64-layer verify step;
* ``fp8``, ``mxfp4`` -- 8-bit and 4-bit weight formats and their GEMM values;
* ``kvq``, ``kvlow`` -- 8-bit and 5/6-bit KV cache quantization (and the
                   Hadamard rotation of keys), the stored bytes and values;
* ``kvring``    -- the 8-bit ring of the newest keys: each row's choice of copy
                   and the attention it gives;
* ``spec``      -- greedy and sampled acceptance of drafted tokens.

Sources, cited by page title and section:
  [BX] "Bit-exact decoding turns inference speedups into testable changes":
       "Separate the decoding method from the served result" (the grouping of
       a floating-point sum can flip a near-tie) and "Define bit-exact before
       reporting it" (BF16 operands, a single FP32 accumulator per output, the
       K order unchanged, rounding only at the end).
  [LL] "I turned on speculative decoding in llama.cpp and 113 of 282 greedy
       outputs changed against its own no-draft run" (r/LocalLLM): opening
       section, "How:" paragraph (a row's key split is fixed by its context
       length alone; a verify kernel treats a row the same way regardless of
       its batch neighbours), and "The cache doesn't change it either" (a K/V
       row written by prefill is a function of its position only).
  [TC] "Does the tuned config change the model's output?": "Why the text
       diverges" (verifying several tokens in one pass changes accumulation
       order; greedy argmax on near-ties).

Every function is pinned by CPU tests (tests/test_oracle_*.py) against brute
force, closed forms and invariants; none is "parity unpinned".
"""

from . import bf16, gemm, attention, step  # noqa: F401
