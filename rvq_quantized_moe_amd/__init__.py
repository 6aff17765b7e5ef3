"""RVQ-LUT Mixture-of-Experts expert forward for MI355X (gfx950).

Python binding of librvq.so: see include/rvq.h for the C ABI.  PyTorch is used
only for device memory and streams; every step of the path runs in the
library's HIP kernels.
"""
from ._lib import (BF16, F16, F32, ExpertBank, ExpertPool, RecordHeader, RvqError, bank_crc32, check_device_status,
                   expert_gemv, gemv_workspace_bytes, lib, lut_build, make_batch_workspace, make_moe_workspace,
                   moe_batch_decode, moe_block_decode, moe_decode_routed, moe_layer_forward, moe_workspace_bytes,
                   pack_codes, packed_bytes, record_bytes, record_check, record_header, rmsnorm, router_topk,
                   rvq_encode, rvq_fit, set_wait_limit, status_string, stream_copy, stream_read, workspace_init, write_records)

__all__ = ["BF16", "F16", "F32", "ExpertBank", "ExpertPool", "RecordHeader", "RvqError", "bank_crc32",
           "check_device_status", "expert_gemv", "gemv_workspace_bytes", "lib", "lut_build", "make_batch_workspace",
           "make_moe_workspace", "moe_batch_decode", "moe_block_decode", "moe_decode_routed", "moe_layer_forward",
           "moe_workspace_bytes", "pack_codes", "packed_bytes", "record_bytes", "record_check", "record_header",
           "rmsnorm", "router_topk", "rvq_encode", "rvq_fit", "set_wait_limit", "status_string", "stream_copy", "stream_read",
           "workspace_init",
           "write_records"]
