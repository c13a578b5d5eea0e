"""CPU oracle for the copy-span splice forward -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy implementation of everything the splice path
computes.  Only the test-suite, the package smoke check and the benchmark's
CPU-baseline leg may import it; the GPU library never does, and this package
imports nothing from the GPU library.  It shares no code, tables or constants
with the HIP kernels.

Sources (the pages this follows):

* "Copy-as-Decode: Grammar-Constrained Parallel Prefill for LLM Editing"
  (Z. Liu): §2.4 (one forward over the span with the existing KV cache
  replaces N decode steps), §2.3 (masked argmax at decision points), the
  appendix paragraph "Position-encoding correctness" (the splice advances
  absolute positions exactly like N decode steps), §3 "Kernel
  microbenchmark" (the autoregressive comparator: N one-token forwards that
  each append to the cache), and Fig. 1 (acceptance is 1 inside a copy op).
* "CopyLoop: Fast Looped Transformer Decoding via Context Copying and Shallow
  Screening" (W. Du, S. Chung): §2 "Block Construction" (suffix match, lengths
  four down to one, up to K copied tokens), "Shallow Screening" (longest
  prefix agreeing with the predecessor's shallow prediction), "Full-Depth
  Verification" (sequential acceptance, first mismatch supplies the
  correction, a full match adds one token), "Concurrent Pipeline" (each
  depth uses its own KV states).

The decoder itself (RMSNorm, rotary positions, GQA attention, SwiGLU) is not
spelled out on the pages beyond "Llama-style"; the readings taken here are
listed in each function's docstring.

Pins (tests/test_oracle_*.py): splice == N sequential decode steps; an
independent library implementation of the Llama decoder (HF transformers,
float64, eager attention, DynamicCache); closed forms of the building blocks;
brute force for the suffix matcher and the masked argmax; planted acceptance.
"""
from .decoder import (Config, KVCache, rms_norm, rope_rotate, decode_step,
                      splice, sequential, prefill, final_logits)
from .decision import masked_argmax, acceptance, top2_margin
from .suffix import suffix_match
from .looped import looped_splice
from .batched import batched_splice
from .copyloop import loop_step, copyloop_decode, greedy_decode
from .cad_program import program_decode

__all__ = ["Config", "KVCache", "rms_norm", "rope_rotate", "decode_step", "splice",
           "sequential", "prefill", "final_logits", "masked_argmax", "acceptance",
           "top2_margin", "suffix_match", "looped_splice", "batched_splice",
           "loop_step", "copyloop_decode", "greedy_decode", "program_decode"]
