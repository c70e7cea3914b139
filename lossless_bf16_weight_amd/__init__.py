"""Lossless BF16 weight decompression (DFloat11-style) for AMD MI355X.

The exponent byte of every BF16 weight is stored as a canonical,
length-limited prefix code; sign and fraction are kept as a raw byte.  The
HIP library `libdf11.so` decodes containers back into bit-identical BF16
tensors in GPU memory.  See include/df11.h for the C ABI and the container
layout.
"""
from ._lib import (ABI_VERSION, FLAG_SHA256, DF11Error, Plan, bw_control, check, container_bound, decode,  # noqa: F401
                   decode_batch, encode, encode_device, encode_device_batch, lib, nf12_decode, nf12_decode_batch, nf12_encode, nf12_validate,
                   sha256, validate, validate_status, verify, verify_decoded, verify_status)
