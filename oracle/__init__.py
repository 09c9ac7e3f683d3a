"""CPU oracle for causal GQA prefill attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by ``__graft_entry__.smoke()`` and by
the CPU-baseline leg of ``bench.py``. The product library never imports, links or calls it,
and it imports nothing from the product package.

Two independent implementations live here:

* ``attention_ref.c`` -- the plain definition in fp64 C (OpenMP over rows), built into
  ``liboracle.so`` by :func:`build`. It reads the paged KV pool through the page table and
  is what GPU results are compared against.
* :func:`dense_attention_np` -- numpy fp64 brute force on a dense (un-paged) K/V with an
  explicit boolean mask; used only on tiny inputs to pin the C code.

Sources for what is computed: causal scaled-dot-product attention softmax(QK^T/sqrt(d) +
causal mask)V over a paged KV cache, the prefill operation of the sglang PR #46351 page
(Motivation); the right-aligned causal placement of a query block against its KV
segment (sglang PR #46351, "Fix" section, and the author's reply on tail alignment); fixed
KV splits whose partial states are combined afterwards (model-serving-minefield issue #73,
correction comment, "What the flag actually does in this build", item 2).
"""
from .oracle import (  # noqa: F401
    build,
    dense_attention_np,
    e4m3_decode_table,
    library_path,
    merge_states,
    num_threads,
    paged_prefill,
)
