"""Closed-form cache and work arithmetic printed on the pages (oracle).

Test infrastructure only.  Every function restates a count the pages print,
so that the tests can pin each figure:

* V4-Flash model record (phantomic12.github.io): naive GQA reading
  layers * kv_heads * head_dim * 2 (K and V) * 2 (bf16) = 88,064 B/token;
  HCA charges head_dim * 2 * 2 / 128 ~ 16.0 B/token/layer; FP8 row 528 B,
  FP4 row 288 B.
* V2 model record: 60 * (512 + 64) * 2 = 69,120 B/token against the naive
  60 * 128 * 128 * 2 * 2 = 3,932,160 B.
* "DeepSeek-V4 deep dive" section 3.1 (mixed 448 FP8 + 64 BF16 = 576 B),
  section 6.1 (4.5 B and 160 B per token per layer; 4.7 MB and 168 MB per
  layer at 1M), section 9.2 (whole-model cache at 1M, window 73,728 B per
  layer, GQA8 baseline ~2%, V3.2 at 788 B/token/layer), section 6.1 / 9.3
  (keys read per query) and section 6.2 (multiply-adds per query).
"""

import math

CTX_1M = 1_048_576
WINDOW = 128
HEAD_DIM = 512
INDEX_DIM = 128

MODELS = {
    # layers by type (section 2.2), heads, top-k (section 1 / configs)
    "pro": {"layers": 61, "csa": 30, "hca": 31, "swa": 0, "heads": 128, "topk": 1024},
    "flash": {"layers": 43, "csa": 21, "hca": 20, "swa": 2, "heads": 64, "topk": 512},
}


def naive_gqa_bytes_per_token(layers=43, kv_heads=1, head_dim=HEAD_DIM, dtype_bytes=2):
    return layers * kv_heads * head_dim * 2 * dtype_bytes


def hca_naive_bytes_per_token_layer(head_dim=HEAD_DIM, ratio=128, dtype_bytes=2):
    """K and V counted separately in bf16, divided by the ratio."""
    return head_dim * 2 * dtype_bytes / ratio


def mla_bytes_per_token(layers=60, latent=512, rope=64, dtype_bytes=2):
    return layers * (latent + rope) * dtype_bytes


def naive_mha_bytes_per_token(layers=60, heads=128, head_dim=128, dtype_bytes=2):
    return layers * heads * head_dim * 2 * dtype_bytes


def mixed_entry_bytes(nope=448, rope=64):
    """448 dims FP8 + 64 RoPE dims BF16, scale bytes ignored."""
    return nope * 1 + rope * 2


def fp4_index_key_bytes(dim=INDEX_DIM):
    return dim // 2  # scale bytes ignored, as on the page


def fp8_mx32_row_bytes(dim=HEAD_DIM):
    return dim + dim // 32


def fp4_e4m3_16_row_bytes(dim=HEAD_DIM):
    return dim // 2 + dim // 16


def per_token_layer_bytes(kind):
    e = mixed_entry_bytes()
    if kind == "hca":
        return e / 128
    if kind == "csa":
        return (e + fp4_index_key_bytes()) / 4
    raise ValueError(kind)


def layer_bytes_at(kind, ctx=CTX_1M):
    e = mixed_entry_bytes()
    if kind == "hca":
        return (ctx // 128) * e
    if kind == "csa":
        return (ctx // 4) * (e + fp4_index_key_bytes())
    raise ValueError(kind)


def window_bytes_per_layer():
    return WINDOW * mixed_entry_bytes()


def model_cache_bytes(model, ctx=CTX_1M):
    m = MODELS[model]
    csa = m["csa"] * layer_bytes_at("csa", ctx)
    hca = m["hca"] * layer_bytes_at("hca", ctx)
    win = m["layers"] * window_bytes_per_layer()
    return {"csa": csa, "hca": hca, "window": win, "total": csa + hca + win}


def v32_cache_bytes(ctx=CTX_1M, layers=61, per_token_layer=656 + 132):
    return layers * per_token_layer * ctx


def gqa8_cache_bytes(ctx=CTX_1M, layers=61, kv_heads=8, head_dim=128, dtype_bytes=2):
    return layers * 2 * kv_heads * head_dim * dtype_bytes * ctx


def keys_per_query(kind, ctx, topk=None):
    if kind == "hca":
        return WINDOW + ctx // 128
    if kind == "csa":
        return WINDOW + min(topk, ctx // 4)
    if kind == "swa":
        return WINDOW
    raise ValueError(kind)


def sparsity_start(topk, ratio=4):
    """First position t whose visible block count floor((t+1)/r) exceeds k."""
    return (topk + 1) * ratio - 1


def macs_per_query(kind, model="pro", ctx=CTX_1M):
    m = MODELS[model]
    if kind == "csa_attention":
        return keys_per_query("csa", ctx, m["topk"]) * m["heads"] * (HEAD_DIM + HEAD_DIM)
    if kind == "indexer":
        return (ctx // 4) * 64 * INDEX_DIM
    if kind == "hca_attention":
        return keys_per_query("hca", ctx) * m["heads"] * 2 * HEAD_DIM
    raise ValueError(kind)


def share_read(model, ctx=CTX_1M):
    return MODELS[model]["topk"] / (ctx // 4)


def ceil_div(a, b):
    return -(-a // b)


def log2(x):
    return math.log2(x)
