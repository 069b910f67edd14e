// Internal launchers behind the C ABI (svgemm.h).  Each enqueues its kernels
// on `stream` and returns hipGetLastError(); argument checks are done by the
// caller in svgemm.hip before any of these is reached.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

hipError_t svg_launch_act_rht_quant(const float* X, int M, int K, const int8_t* signs, int8_t* xq,
                                    float* x_scale, hipStream_t stream);
hipError_t svg_launch_rot_quant_w4(const float* W, int N, int K, const int8_t* signs, int group,
                                   bool z4, uint8_t* wq, uint16_t* w_scale, void* w_zero,
                                   float* w_rot, hipStream_t stream);
hipError_t svg_launch_rot_quant_w8(const float* W, int N, int K, const int8_t* signs, int8_t* wq,
                                   uint16_t* w_scale, float* w_rot, hipStream_t stream);
hipError_t svg_launch_w4a8(const int8_t* xq, const float* x_scale, int M, int K, const uint8_t* wq,
                           const uint16_t* w_scale, const void* w_zero, bool z4, int group, int N,
                           float* y, int32_t* dbg, hipStream_t stream);
hipError_t svg_launch_w8a8(const int8_t* xq, const float* x_scale, int M, int K, const int8_t* wq,
                           const uint16_t* w_scale, int N, float* y, int32_t* dbg,
                           hipStream_t stream);

// Largest M served by the dot-product (GEMV) kernels; larger M use MFMA.
constexpr int kGemvMaxM = 2;
