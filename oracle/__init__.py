"""CPU oracle for the paged-attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything in this package; only
the tests, the smoke check and the CPU-baseline leg of the benchmark use it.

The oracle is plain numpy, fp64 wherever floating point is involved, and is
written from the two source texts on the subject:

* LESSON  -- "vLLM Serving Internals: PagedAttention, Continuous Batching,
  Chunked Prefill" (AI Engineering from Scratch, Phase 17, Lesson 04; read in
  its Turkish, Chinese, Persian and Portuguese renderings).
* ARTICLE -- "vLLM推理引擎架构：PagedAttention机制与高吞吐推理" (vLLM inference
  engine architecture: the PagedAttention mechanism and high-throughput
  inference), lpnh.cn.

Modules:
  codecs         bf16 / fp8 e4m3fn storage formats (decode and encode)
  allocator      FIFO block pool, per-sequence block tables, slot mapping
  cache          scatter of new K/V into the paged cache layout
  attention      gather through block tables + softmax attention (decode and
                 causal prefill chunks)
  fragmentation  KV-cache waste accounting
  scheduler      iteration-level continuous batching with chunked prefill
"""
