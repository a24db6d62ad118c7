"""Gated DeltaNet mixer hot path for AMD Instinct MI355X (gfx950).

The computation runs in libgdn.so (hand-written HIP kernels behind the C ABI
declared in include/gdn.h); this package only binds it to torch tensors.
"""
from ._binding import (GDN_ALGO_AUTO, GDN_ALGO_CHUNKED, GDN_ALGO_SEQUENTIAL, GDN_BF16, GDN_F32,
                       GDNError, gdn_abi_version, gdn_conv_silu, gdn_decode_rows,
                       gdn_decode_rows_multi, gdn_dims, gdn_gate_proj,
                       gdn_gate_proj_workspace_bytes,
                       gdn_gated_rmsnorm, gdn_linear, gdn_linear_kernel, gdn_linear_tune,
                       gdn_linear_workspace_bytes,
                       gdn_mixer_prefill, gdn_mixer_prefill_workspace_bytes,
                       gdn_prefill, gdn_prefill_noalloc, gdn_prefill_slots,
                       gdn_prefill_slots_workspace_bytes, gdn_prefill_workspace_bytes,
                       gdn_status_str, lib, LIB_PATH)

__all__ = ["GDN_ALGO_AUTO", "GDN_ALGO_CHUNKED", "GDN_ALGO_SEQUENTIAL", "GDN_BF16", "GDN_F32",
           "GDNError", "gdn_abi_version", "gdn_conv_silu", "gdn_decode_rows",
           "gdn_decode_rows_multi", "gdn_dims", "gdn_gate_proj",
           "gdn_gate_proj_workspace_bytes",
           "gdn_gated_rmsnorm", "gdn_linear", "gdn_linear_kernel", "gdn_linear_tune", "gdn_linear_workspace_bytes", "gdn_mixer_prefill", "gdn_mixer_prefill_workspace_bytes",
           "gdn_prefill", "gdn_prefill_noalloc", "gdn_prefill_slots",
           "gdn_prefill_slots_workspace_bytes",
           "gdn_prefill_workspace_bytes", "gdn_status_str",
           "lib", "LIB_PATH"]
