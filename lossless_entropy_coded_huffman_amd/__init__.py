"""Lossless Huffman-coded LLM weights, decompressed on AMD MI355X (gfx950).

BF16 weights keep sign and mantissa raw and have their exponent byte Huffman
coded (DFloat11); uint8 and uint4 quantised weights are Huffman coded whole
(EntroLLM; uint4 packed two per byte).  Encoding runs in the C++ host library, decompression in HIP
kernels; both sit behind the C ABI in include/dfh.h, which ``dfh`` binds
with the same names.  ``synth`` draws the seeded synthetic workloads.
"""
from .dfh import (  # noqa: F401
    KIND_BF16, KIND_U4, KIND_U8, MAX_LEN, SECTION_NAMES, DEVERR_CODE, DEVERR_COUNT, ENCODE_SCRATCH_BYTES, DFError,
    Container,
    DeviceContainer, compress, compress_device, compress_device_batch, df_build_codebook, df_build_tables, df_encode_device, df_encode_device_noalloc,
    df_encode_layout, df_encode_workspace_bytes, df_histogram_device, df_symbol_device, df_container_free,
    df_container_info,
    df_container_load, df_container_save, df_container_section, df_container_validate,
    df_decompress, df_decompress_batch, df_decompress_checked, df_encode, df_histogram,
    df_status_string, lib, output_bytes, to_device,
)
