"""fp64 CPU oracle for PCP-sharded MLA prefill attention with an attention sink.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg do. It
shares no code with the HIP library (no kernels, headers, helpers or tables); the
two meet only at the seeded input bytes.

What it computes, and where the pages fix it:

* ``partition``: the DualChunkSwap split of each prefill into 2*P contiguous chunks,
  rank r receiving chunks r and 2P-1-r; decode rows replicated on every rank
  ("[Core] Add MRV2 virtual-batch PCP for MLA", sections "PCP algorithm" and
  "DualChunkSwap partitioning", with the PCP=4 figure).
* ``attention``: single-pass causal softmax attention of absorbed MLA (one shared
  latent KV head: key = latent || rope, value = latent) with and without a per-head
  sink logit, computed straight from the definition in fp64, unsharded. Each rank's
  partial equals the no-sink rows because every rank holds the full all-gathered
  latent KV ("[Core] Add MRV2 virtual-batch PCP for MLA", "DualChunkSwap
  partitioning": K/V, or the latent KV for MLA, are all-gathered).
* ``merge``: the log-sum-exp merge of per-rank partial (O, LSE) with the sink
  applied once in the final denominator ("[DeepSeekV4][PCP] Enable context-parallel
  prefill for hybrid KV and MegaMoE", "Purpose" and "Main challenges").
* ``numerics``: exact bf16 decode, bf16 round-to-nearest-even, OCP E4M3FN decode and
  nearest-even encode.
* ``kvcache``: paged addressing of a cache of 64-row blocks and fp8 quantise-on-insert with
  one fp32 scale per block ("[Feature][PCP] Add DeepSeek-V4.1-Flash support", "vLLM Launch
  Arguments": fp8 MLA KV cache, block size 64).

Every function is pinned by tests marked ``not gpu`` against brute force, closed
forms, library special cases and the pages' worked partition pictures.
"""
from . import numerics, partition, attention, merge, kvcache  # noqa: F401
