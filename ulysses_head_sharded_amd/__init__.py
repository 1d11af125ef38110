"""MI355X-native per-rank hot path of DeepSpeed-Ulysses sequence parallelism.

pack (seq->head send side) -> head-sharded attention -> unpack (head->seq
receive side), as hand-written HIP kernels for gfx950 behind the C ABI in
include/ulysses.h.  Importing the package loads nothing; the binding loads
libulysses.so on first use and raises if it has not been built.
"""
from .binding import (  # noqa: F401
    ULYS_BF16, ULYS_F32, UlyssesError, attn_fwd, pack_seq2head, ulys_abi_version,
    ulys_attn_fwd, ulys_attn_fwd_ws, ulys_attn_fwd_workspace_size, ulys_pack_seq2head, ulys_status_string, ulys_unpack_head2seq,
    unpack_head2seq)
