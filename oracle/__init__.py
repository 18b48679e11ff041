"""CPU oracle for attention over a paged KV cache (plain numpy, float64).

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import or run anything in this package.  The
HIP library never calls it, and it shares no code with the library: it is the
plain definition of what the library must compute, written out slowly so that
it can be checked against the pages by eye.

Pages it follows (cited by title and section):

* «FlashAttention y FlashInfer: los dos grandes backends de atención en GPU»
  - §Flujo de datos, the ``get_kv_cache_shape`` listing: pool shape
    ``(num_blocks, 2, block_size, num_kv_heads, head_size)``, dim 1 = K/V slot,
    block size a multiple of 16;
  - §Responsabilidades: Q/out are ``[num_tokens, num_heads, head_size]``; the
    metadata carries ``query_start_loc``, ``seq_lens`` and the block table; the
    FlashInfer builder splits decodes from prefills and moves decodes to the front;
    the new tokens' K/V are written into the cache by an operation of its own.
* «El especialista del plato estrella: el backend de atención de vLLM»
  - §Por qué prefill y decode son problemas opuestos: prefill = many queries
    against many keys, decode = one query against all accumulated keys;
  - §Cómo lee el backend el KV paginado: K/V are gathered through the block
    table from fixed-size blocks scattered in memory;
  - §Qué aporta FlashInfer (eq. "lecturas"): cascade attention computes the
    shared prefix once and combines it with each request's own suffix.
* «AttentionBackend: capa de abstracción de backends de atención»
  - §Motivación de diseño and §Límites y fallos: partial attentions are combined
    through their softmax log-sum-exp, whose base (natural log here) must match.
* FP8 KV cache: «FlashAttention y FlashInfer», §Motivación de diseño and
  §Límites y fallos (an ``fp8_e4m3`` cache and per-head quantisation scales);
  the format and the readings are in :mod:`oracle.fp8`.

Every public function has a pin in ``tests/`` that checks it against something
other than itself (closed forms, invariants, brute force, a library special
case, or the pages' own worked numbers).  Nothing here is "parity unpinned".
"""
from .attention import (  # noqa: F401
    attention,
    attention_rows,
    cascade_attention,
    cascade_prefix_reads,
    decode_intensity,
    gather,
    kv_cache_shape,
    merge_states,
    metadata,
    slot_mapping,
    to_f64,
    write_kv,
)
from .layout import kv_cache_stride_order, logical_pool  # noqa: F401
from .fp8 import (  # noqa: F401
    dequantize_pool,
    e4m3_decode,
    e4m3_encode,
    quantize,
    scales_per_head,
    write_kv_fp8,
)
