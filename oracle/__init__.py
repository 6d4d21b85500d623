"""CPU oracle for the window+sink chunk-attention KV path.

TEST INFRASTRUCTURE ONLY. Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg
of `bench.py` may import anything from this package. The product path (the HIP library and
its Python binding) never imports, calls or falls back to it.

Everything here is plain NumPy in float64 (integers for the FP4 codec), written from the
definitions of the method, with no blocking, fusion or reordering beyond what the
definitions state. It shares no code with the HIP path; the only module both sides use is
the seeded input generator, which holds none of the arithmetic.

Modules
  ring       the per-layer cache: sink slots, window ring, the visible-frame set
  attention  explicit masked softmax attention over concatenated keys
  fp4        the e2m1 / e8m0 block codec of the FP4 KV store
  model      a whole-stream model: chunk attention, commit, recache, export

Sources (pages, by title and section):
  [LL]   "英伟达LongLive框架：实时交互式生成长达4分钟视频" (yunpan.plus), 方法 §1 KV 重缓存,
         §2 流式长视频微调, §3 高效长推理 (short-window attention; frame sink)
  [NEWS] "英伟达LONGLIVE框架发布：单GPU实时生成240秒交互式长视频" (paooo.com), LONGLIVE的技术原理
  [INFRA] "为什么视频生成是一个基础设施问题" (NVIDIA blog, Chinese translation), §3, §4, §5
  [DIST] LongLive 2.0 distributed inference (blog.hotdry.top), "NVFP4 量化与 KV Cache 压缩的工程实现",
         "序列并行与注意力汇聚的协同设计"
  [PIPE] "LongLive 长视频生成数据流水线架构与存储优化实践" (blog.hotdry.top), 三、NVFP4 量化
  [OCP]  OCP Microscaling Formats (MX) v1.0 specification: FP4 E2M1 element and E8M0 scale
         encodings (an external published definition; the pages only say "FP4")

Where the pages are silent, each function states the reading it takes. Parity pins: every function here is checked by `tests/test_oracle_*.py` against
brute force, library routines (torch CPU fp64 scaled_dot_product_attention), closed forms
and invariants. No function in this package is "parity unpinned".
"""
