"""fp64 CPU oracle for exact attention. Test infrastructure only: the library never imports it."""
from .attention import (attention_ref, attention_rows, combine_ref, decode_ref, kv_head_of,
                        online_ref, split_partials_ref, visible_keys, widen_bf16)

__all__ = ["attention_ref", "attention_rows", "combine_ref", "decode_ref", "kv_head_of",
           "online_ref", "split_partials_ref", "visible_keys", "widen_bf16"]
