"""CPU oracle for MLA decode over a paged latent KV cache — TEST INFRASTRUCTURE.

This package is the slow, plainly written reference the HIP path is checked against. Only the test
suite, the package smoke check and the CPU-baseline leg of the benchmark may import it; the product
path never calls it and shares no code with it.

Everything is computed in float64 with numpy on dense, unpaged rows:

- fp8.py       e4m3fn and ue8m0 decoding from their bit definitions, row dequantisation
- attention.py absorbed (MQA-form) attention with visible sets, sink and log-sum-exp
- merge.py     log-sum-exp merge of split partials and the sink fold
- brute.py     pure-Python loops for tiny cases
- mha.py       the expanded (MHA-form) computation, used only to pin the absorbed form
- paging.py    reads a paged cache back into dense rows
- plan.py      the split/work-unit plan, integer arithmetic
- kvwrite.py   writing new tokens' rows into the paged cache (bf16 copy, fp8 quantisation)
- absorb.py    per-head weight absorption before (W_UK) and up-projection after (W_UV) the decode
- swa_runs.py  sliding windows of cache slots compressed into at most two runs per token
- gather.py    context rows of a chunk of requests gathered into a dense workspace
- chunks.py    packing requests' context rows into workspace-sized chunks (host plan)
- sparse_prefill.py  prefill tokens attending over their own index lists into a flat buffer,
                with the per-row maximum logit

Parity status of each function is stated in its module docstring.
"""
