"""cp_slot_map_amd: attention over a context-parallel striped paged KV pool on AMD Instinct MI355X (gfx950).

The compute lives in ``libcpattn.so`` (hand-written HIP, C ABI in include/cpattn.h); this package is its PyTorch
binding (``api``) and a pool builder (``pool``) that writes a batch into the stripe pools through the library's own
write path.
"""
from .api import (slot_map, slot_map_rank, kv_write, paged_attn_partial, paged_attn_workspace_size, own_token_attn,
                  lse_merge, debug_gather_stripe, version)

__all__ = ["slot_map", "slot_map_rank", "kv_write", "paged_attn_partial", "paged_attn_workspace_size",
           "own_token_attn", "lse_merge", "debug_gather_stripe", "version"]
