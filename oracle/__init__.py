"""CPU oracle for the Orthrus draft/verify step (TEST INFRASTRUCTURE ONLY).

This package is a plain, slow, fp64 numpy statement of what one Orthrus decode
step computes.  It exists to check the HIP library and nothing else: only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may import
it.  The product path (the C-ABI library and its Python binding) never imports,
links or calls anything here, and nothing here imports the product path.

Sources.  The method is described on five web pages; the only methodological
one is the gist.science technical summary of "Orthrus: Memory-Efficient
Parallel Token Generation via Dual-View Diffusion" (written in Dutch), cited
below as [gist §x].  The co-author's post #21 in the Hacker News thread
"Orthrus-Qwen3: up to 7.8x tokens/forward on Qwen3, identical output
distribution" is cited as [HN #21] (post #26 of the same thread as
[HN #26]).  The paper abstract (codewithpapers and fugumt pages) is cited as
[abstract], the author profile page as [profile].

Modules:
  attention  - page-table gather + dense masked softmax attention (draft mask,
               verify mask)
  consensus  - vocabulary argmax, longest-prefix acceptance, cache commit
  lmhead     - LM-head projection of the final hidden states and the greedy
               token of every row
  sampling   - consensus at temperature > 0 (speculative sampling, a stated
               reading; the pages give only the greedy rule)
  fp8        - an e4m3 KV cache: the format, quantisation with per-head
               scales, and attention over the decoded values (a stated
               reading; the pages describe no quantised cache)
  toy        - a tiny fp64 Qwen3-style decoder with a diffusion view, the
               Orthrus loop and plain greedy decoding

Parity status of each function is stated in its docstring ("pinned by ...").
"""
from .attention import from_bf16, gather_context, block_attention, attention_weights  # noqa: F401
from .consensus import argmax_rows, accept, commit_kv  # noqa: F401
