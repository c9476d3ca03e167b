"""Plain fp64 CPU oracle for DeepSeek-V2 Multi-head Latent Attention decode.

TEST INFRASTRUCTURE ONLY. Only `tests/`, `__graft_entry__.smoke()` and the
benchmark's CPU-baseline leg may import this package. The library (the HIP
path and its Python binding) never imports it, and this package imports
nothing from the library: the two share no code.

What it computes, and where the pages say so:
  * the latent cache: per token only c_KV (d_c = 512) and one decoupled RoPE
    key shared by all heads (d_R = 64) are stored -- DeepSeek-V2 reading card
    (ai-papers.xuzou.cn), "Bottlenecks" and "Method adaptation"; discosf
    explainer, "long-context bottleneck" and "decoupled RoPE" sections;
  * decode in the *unabsorbed* form: per head, K = W_UK c and V = W_UV^T c are
    expanded explicitly and textbook softmax attention runs over all cached
    tokens of the sequence (discosf explainer, "long-context bottleneck":
    each generated token attends to the K/V of all previous tokens; the
    up-projection recovers K/V from the latent). The absorbed form the method
    uses reaches the same result by associativity (same section: W_UK folds
    into the query side, W_UV into the output side);
  * prefill (many queries per sequence): the same attention per query token
    over the rows up to its own position (causal); the pages report prompt
    throughput beside generation (DeepSeek-V2 reading card, "Evidence");
  * append: c_KV = W_DKV h and k_pe = RoPE(W_KR h), stored in the cache dtype;
    RoPE optionally with YaRN frequencies (discosf explainer, "decoupled RoPE
    and YaRN" section, with the formula of the published YaRN method).

Readings where the pages are silent are listed in the package's modules next
to the code that takes them.
"""
from .numerics import (round_bf16, round_f32, e4m3_decode, e4m3_encode,
                       E4M3_MAX, e4m3_value_table, e2m3_decode, e2m3_encode, e2m3_value_table,
                       E2M3_MAX, MX_BLOCK, mx_block_exponent, pack6, unpack6)
from .mla import (D_C, D_R, D_ROW, D_NOPE, D_V, softmax_scale, rope_inv_freq,
                  yarn_inv_freq, yarn_softmax_factor, rope_rotate, paged_rows, append_rows_exact, quantize_rows,
                  fp6_rows,
                  decode_head, decode_problem, decode_sampled, attention_weights,
                  prefill_head, prefill_positions, prefill_problem,
                  mla_cache_elements_per_token, mha_cache_elements_per_token,
                  gqa_equivalent_groups, cache_bytes)

__all__ = [n for n in dir() if not n.startswith("_")]
