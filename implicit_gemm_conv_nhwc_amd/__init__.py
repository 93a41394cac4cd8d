"""implicit_gemm_conv_nhwc_amd -- the resident image-VAE decoder's NHWC
implicit-GEMM convolution path on MI355X (gfx950).

The compute lives in ``libigconv.so`` (HIP, built from ``csrc/``; C ABI in
``include/ig_conv.h``). This package is its ctypes binding plus a helper
that uploads and packs a decoder's weights into the descriptor
``decoder_forward`` takes. PyTorch supplies device memory and the stream.
"""

from ._lib import (  # noqa: F401
    AttnW,
    ConvW,
    DecoderDesc,
    IgError,
    ResnetW,
    UpW,
    combine,
    conv3x3_nhwc,
    conv3x3_gn_stats_nhwc,
    conv3x3_guard_out_nhwc,
    conv3x3_norm_nhwc,
    conv3x3_out_nchw,
    conv3x3_up2_nhwc,
    conv_gn_partials_bytes,
    conv_nhwc_ex,
    band_plan,
    set_clock_probe,
    decoder_bands_workspace_bytes,
    decoder_forward,
    decoder_forward_bands,
    decoder_workspace_bytes,
    dupup_add,
    gemm1x1,
    gemm1x1_acc,
    attention_f16,
    attention_workspace_bytes,
    groupnorm_silu_f16,
    groupnorm_silu_f16_from_partials,
    groupnorm_silu_f16_noalloc,
    groupnorm_workspace_bytes,
    guard_cast,
    last_error,
    latent_to_nhwc_f16,
    lib,
    nhwc_to_nchw,
    pack_conv_weights,
    plane_shape,
    rmsnorm_silu_f16,
    rmsnorm_silu_guard_cast_f16,
    softmax_rows_f16,
    version,
    zero_rows_f16,
)
from .decoder import DeviceDecoder, cpad  # noqa: F401
