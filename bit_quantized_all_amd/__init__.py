"""MI355X (gfx950) block-quantization codec and compressed-domain reduction.

The kernels live in ``csrc/`` and are built into ``libqr.so``; ``qr`` is the
ctypes binding of the C ABI declared in ``include/qr.h``.
"""
from .qr import (FORMATS, MAX_RANKS, QR_ERR_ALIAS, QR_ERR_ALIGN, QR_ERR_ARG, QR_ERR_HIP,  # noqa: F401
                 QR_ERR_SIZE, QR_ERR_UNSUPPORTED, QR_OK, QRError, TILE_VALUES, lib, qr_decode, qr_encode,
                 qr_packed_bytes, qr_reduce_compressed, qr_reduce_compressed_mixed, qr_status_string)
