"""Seeded synthetic inputs and the layer lists of the measured workloads.

This package holds no arithmetic of the convolution method: it draws random
numbers, casts them to the storage type and describes layer shapes. Both the
GPU path (tests, benchmark) and the CPU oracle consume the same bytes from it.
"""
from .inputs import (  # noqa: F401
    ConvSpec,
    PoolSpec,
    conv1_single,
    conv2_stem,
    conv2_stem_bf16,
    conv3_pointwise,
    conv4_ifnet_block,
    conv5_resnet18d,
    conv_flops,
    ifnet_deconv,
    large_map,
    random_conv_case,
    random_deconv_case,
    random_map,
    to_storage,
)
