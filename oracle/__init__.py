"""Plain, slow CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (``paged_kv_cache_forward_amd``) never imports it,
and this package imports nothing from the product path: the two share no code.

Everything here is written for a reader to check by eye against the pages it
follows, not for speed: NumPy in float64, one sequence (and one KV head) at a
time, no blocking, fusion or reordering beyond what the definitions state.

Pages followed (cited by title and section throughout the package):

  [HADA]  "vLLM PagedAttention: eine Revolution für den Durchsatz bei der
          LLM-Inferenz" (de.news.hada.io) -- bullets "Continuous Batching",
          "Chunked Prefill", "Prefix Caching".
  [SLAVA] "Was ändert PagedAttention an der KV-Speicherzuweisung für LLMs?"
          (slavadubrov.com) -- lead paragraph; section "Ungenutzten Platz in
          Blöcken berechnen"; section "Gemeinsame Nutzung erfordert mehr als
          Speicherzuweisung".
  [AIU]   "PagedAttention et vLLM" (aiunderstanding.org) -- sections
          "Aperçu", "Plongée profonde", "Mise en œuvre dans le monde réel",
          "Questions fréquemment posées".
  [ART]   "Внутреннее устройство vLLM: как работает высокопроизводительный
          инференс LLM" (artificials.ru) -- paragraphs on paged attention,
          chunked prefill, prefix caching and the forward pass ("super-batch").

Modules:
  numerics   -- widening of stored element formats (fp32, bf16 bits) to float64
  blocks     -- block counts and unused-slot accounting (closed forms)
  alloc      -- RefAllocator: block allocator with refcounts, copy-on-write
                and the prefix cache
  prefix     -- chained FNV-1a 64 block hashes for prefix caching
  quant      -- fp8 (E4M3 codes, power-of-two row scales) cache format: encode,
                decode, quantised write and dequantised gather
  cache      -- cache write through a slot mapping; whole-block copies
  attention  -- paged attention over a varlen super-batch; split/merge pieces

Parity status: every function is pinned by ``tests/test_oracle_*.py``:
``numerics.to_f64`` by torch's own bfloat16/float32 conversions over every
bf16 bit pattern and by values the formats fix; the rest by closed forms, the
worked allocation example printed on [SLAVA], invariances, and a float64
library attention routine fed through torch's conversions.  Planted mistakes
in each module fail a pin (``tests/test_oracle_mutations.py``).  None is
"parity unpinned".
"""

from .numerics import to_f64
from .blocks import blocks_needed, unused_slots, unused_fraction
from .alloc import RefAllocator, OutOfBlocks
from .prefix import fnv1a64, block_hash, chain
from .quant import (
    decode_e4m3,
    encode_e4m3,
    row_exponent,
    quantize_rows,
    dequantize_rows,
    fp8_pool,
    ref_write_kv_fp8,
    gather_logical_fp8,
)
from .cache import ref_write_kv, ref_copy_blocks
from .attention import (
    gather_logical,
    ref_paged_attention,
    ref_partition_state,
    ref_lse_merge,
    ref_split_attention_row,
)

__all__ = [
    "to_f64",
    "blocks_needed",
    "unused_slots",
    "unused_fraction",
    "RefAllocator",
    "OutOfBlocks",
    "fnv1a64",
    "block_hash",
    "chain",
    "decode_e4m3",
    "encode_e4m3",
    "row_exponent",
    "quantize_rows",
    "dequantize_rows",
    "fp8_pool",
    "ref_write_kv_fp8",
    "gather_logical_fp8",
    "ref_write_kv",
    "ref_copy_blocks",
    "gather_logical",
    "ref_paged_attention",
    "ref_partition_state",
    "ref_lse_merge",
    "ref_split_attention_row",
]
