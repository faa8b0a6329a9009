"""Plain float64 CPU oracle of DeepSeek-V4 compressed-attention decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, headers,
tables or helpers with the HIP library; it imports nothing but NumPy.

Source of every definition: the page "DeepSeek-V4 deep dive" (gangliao.me,
2026), cited by section, equation or table, plus the V4-Flash model record
(phantomic12.github.io) and the V4.1-Flash diagram page (flozi.net) for the
cache row layouts.  Where the pages are silent the reading used is stated in
the docstring of the function that takes it.

Modules
-------
rope        partial RoPE on the last 64 dims, YaRN frequency blend
codec       FP8-MX32 (528 B / 132 B rows) and MXFP4-E4M3/16 (288 B rows), bf16
compressor  learned gated pooling compressor, bulk and streaming forms
indexer     lightning-indexer scores
topk        deterministic top-k selection
attention   index lists, shared-KV MQA with sink, CSA and HCA decode
cache_bytes closed-form cache and work arithmetic printed on the pages
pipeline    the tiny whole-path case (hidden states -> attention output)
"""

from . import rope, codec, compressor, indexer, topk, attention, cache_bytes, pipeline  # noqa: F401
