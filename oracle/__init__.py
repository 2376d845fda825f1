"""CPU oracle for the W4A16 paged-KV decode step (test infrastructure only).

This package is the plain, slow, obviously-correct definition of what the GPU
library computes, written in numpy float64. It exists to check the GPU path.
Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import it; the library itself never does, and it shares no code with the
HIP kernels or their host runtime. Inputs come from ``workloads`` (seeded
draws); nothing here is read back from the GPU except the values under test.

Sources (page title, section):
  * "How to build your own LLM runtime from scratch" (aikraft.ru digest of a
    Towards Data Science article), "Architectural decisions and
    optimizations": 28 layers, hidden 3584, 28 attention heads with GQA 7:1;
    symmetric group-wise INT4 weights with group 128; RMSNorm and lm_head kept
    in FP16; 16-token KV pages (4 KiB per head slice).
  * "Building a Custom LLM Inference Runtime on H100", "The KV Cache and
    PagedAttention": the cache is split into pages, handled like virtual
    memory; "The Three Critical Bugs", Bug 1: each logical token position maps
    to a physical block.
  * Where the pages are silent the readings are: groups run along the input
    dimension; dequantised weight = q * s with q in [-8, 7]; RoPE is
    rotate-half with base 1e6; softmax scale 1/sqrt(D); KV head of q head h is
    h // (Hq / Hkv); the token being decoded sits at position ctx - 1 and its
    K/V are written before attention; every stored tensor is rounded once to
    IEEE binary16 (round to nearest even).

Modules:
  decode   -- the paged decode step, layer by layer (the oracle proper)
  dense    -- brute-force dense re-statement (no pages, dense weights,
              repeat-kv multi-head attention) used to cross-check ``decode``
  packing  -- reads the packed weight formats of the library back into (q, s)
  generate -- greedy token loop over ``decode`` (argmax, positions advancing
              across page boundaries, optional teacher forcing)
  prefill  -- a prompt through the model at once (every row the decode step
              of its token at its position; causal attention over the pages)
  quantize -- the symmetric INT4 group-128 quantiser (fp16 -> q, s)
  w4a8     -- the W4A8 variant of the projections (INT8 activations, integer
              inner sums), measured against the W4A16 path
  runs     -- whole synthetic workloads through the above
"""
