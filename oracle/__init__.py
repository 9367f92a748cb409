"""Float64 CPU oracle for one paged grouped-query-attention decode step.

TEST INFRASTRUCTURE. This package is the checker, not the product: only the
test suite, the package's smoke check and the benchmark's CPU-baseline leg
may import it. The HIP library never calls into it and shares no code with
it; the two meet only at the seeded inputs of ``workloads.py``.

What it computes, and which passage each part follows (pages are cited by
title and section; section tags of the first page are its own §/Tab. tags):

* ``numerics``  -- exact bf16 <-> float64 conversion and round-to-nearest-even
  to bf16 (the precision the pages name for weights and KV, "The KV Cache Is
  the New Memory Wall" review §2.1; froggydisk "LLM에서 KV 캐시는 얼마나
  생길까", FP8 format table).
* ``footprint`` -- KV bytes per token, per request and per decode step; FLOPs
  and arithmetic intensity of the step (froggydisk, size of one token;
  review §2.1, §3.1-§3.2, Tab. 8).
* ``paged``     -- block-table addressing over 16-token blocks and the
  library's documented pool layout (froggydisk, PagedAttention paragraph and
  its block-table example).
* ``attention`` -- softmax(q K^T / sqrt(d_h)) V per query head with grouped KV
  heads, its log-sum-exp, per-chunk partials and their merge (froggydisk,
  section "KV 캐시란": scores scaled by sqrt(128), softmax, weighted sum of the
  V rows; 4 query heads per KV head).
* ``e4m3``      -- the FP8 E4M3 format: decode of all 256 codes, nearest-even
  encode with saturation at 448, and per-(block, head) absmax/448 scales
  (froggydisk, FP8 KV cache paragraph and format table).
* ``scores``    -- the cumulative attention score, layer- and head-averaged
  (gist.science summary of "Not all thinking needs HBM", methodology 2).

Every function here is pinned by ``tests/test_oracle_*.py`` against values
the pages print, closed forms, library routines (torch's float8/bfloat16
casts and scaled_dot_product_attention) or brute force on tiny inputs.
"""
from . import numerics, footprint, paged, attention, e4m3, scores  # noqa: F401
