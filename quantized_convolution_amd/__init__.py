"""quantized_convolution_amd: group-wise fully quantized 8-bit Winograd
convolution F(4,3) / F(6,3) with diagonal transform scales, on MI355X.

The compute path is the HIP library libwino_q8_conv.so (C ABI declared in
include/wino_q8_conv.h); `binding` marshals torch tensors into it. Importing
this package does not load the library; the first call does, and raises if
it has not been built.
"""
from .binding import (Plan, Wq8Error, load, wq8_conv_forward, wq8_direct_conv, wq8_direct_forward,
                      wq8_direct_quantize_x, wq8_direct_weights_prepare, wq8_plan_bt_codes, wq8_plan_matrices,
                      wq8_stage1, wq8_stage2, wq8_stage2_i32, wq8_stage3, wq8_stage23,
                      wq8_weights_prepare)

__all__ = ["Plan", "Wq8Error", "load", "wq8_conv_forward", "wq8_direct_conv", "wq8_direct_forward",
           "wq8_direct_quantize_x", "wq8_direct_weights_prepare", "wq8_plan_bt_codes", "wq8_plan_matrices", "wq8_stage1",
           "wq8_stage2", "wq8_stage2_i32", "wq8_stage3", "wq8_stage23", "wq8_weights_prepare"]
