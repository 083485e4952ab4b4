"""CPU oracle for the paged KV cache and paged decode attention.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
reference written in numpy / float64. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``paged_kv_cache_450_amd`` and its HIP library) never imports, links or calls
anything here, and this package never imports the product path: the two share
no code, no headers, no tables and no constants.

Sources. The pages are cited by title and section:

* [P2] "vLLM 推理加速原理详解：大模型服务吞吐量为何能提升 10 倍"
  (fudengji.cn/article/275). Sections used:
  - "真正吃显存的是 KV Cache，不是模型权重" (KV cache size closed form);
  - "PagedAttention：把操作系统的虚拟内存搬进 GPU" (fixed-size physical
    blocks, page table, on-demand allocation, shared blocks, the kernel that
    reads KV from non-contiguous blocks);
  - "连续批处理：别再等最慢的那个请求了" (the scheduler's block-manager
    calls: free a finished request's table, count free blocks, can_allocate,
    allocate);
  - "vLLM 也不是银弹：真实部署中的坑", third pitfall (FP8 KV cache).
* [P3] "突破大模型推理瓶颈：vLLM框架核心技术深度解剖与实战指南", section 2.4
  (FP32 accumulation).

Modules:

* ``fp8``       - OCP E4M3 ("fn") codec from the format definition.
* ``pool``      - pool layout, byte sizes, the KV-size closed form, append.
* ``attention`` - gather through the block table, softmax(q K^T * scale) V,
                  split-K partials and their merge.
* ``allocator`` - ``AllocatorModel``: the refcounted block manager and the
                  per-sequence slot bookkeeping.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against something other than itself (brute force, closed forms, library
routines, the pages' printed numbers). Nothing is "parity unpinned".
"""

from . import fp8, pool, attention, allocator  # noqa: F401
