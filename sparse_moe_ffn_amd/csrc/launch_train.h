// Host launchers of the training-side kernels (k_train.hip).  Shapes and
// pointers are validated by the C ABI before these are called.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mm {

// Bias step of the aux-loss-free balancing over T*k expert ids (E <= 4096).
hipError_t launch_bias_update(int64_t Tk, int E, const int32_t* idx, float lambda, float* bias,
                              int32_t* load, hipStream_t st);

// Drop-and-pad tables from the stable count sort (offsets, perm, inv).
hipError_t launch_drop_pad(int64_t Tk, int E, int64_t C, const int32_t* idx, const int32_t* offsets,
                           const int32_t* perm, const int32_t* inv, int32_t* buf, int32_t* offsets_c,
                           int32_t* perm_c, int32_t* inv_c, hipStream_t st);

// eq. (6) fake quantisation, forward and/or straight-through backward;
// groups of 32 or one group per row; cols a multiple of 4 (32 for groups).
hipError_t launch_fake_quant(int64_t rows, int64_t cols, int bits, bool row_group, const float* x,
                             float* xbar, const float* gout, float* gin, hipStream_t st);

}  // namespace mm

namespace mm {

// dst[r] = scale[perm[r]] * src[perm[r] / k] (d a multiple of 4).
hipError_t launch_gather_rows(int64_t R, int64_t d, int k, const int32_t* perm, const float* scale,
                              const float* src, float* dst, hipStream_t st);

// QAT forward of the experts over expert-ordered rows (d, h multiples of 16).
hipError_t launch_expert_train_forward(int E, int d, int h, int64_t R, const int32_t* off,
                                       const float* xs, const float* wgu, const float* wd, float* gu,
                                       float* abar, float* f, hipStream_t st);

// Its backward; dabar [R][h] and dgu [R][2h] are scratch.
hipError_t launch_expert_backward(int E, int d, int h, int64_t R, const int32_t* off, const float* xs,
                                  const float* wgu, const float* wd, const float* gu,
                                  const float* abar, const float* df, float* dxs, float* dwgu,
                                  float* dwd, float* dabar, float* dgu, hipStream_t st);

}  // namespace mm

namespace mm {

// Router backward of the training step (E <= 64, E and d multiples of 4 and 16).
hipError_t launch_router_backward(int64_t T, int d, int E, int k, int gating, const float* x,
                                  const float* wr, const float* bias, const int32_t* idx,
                                  const float* f, const int32_t* inv, const float* dy, float lambda_z,
                                  float* dz, float* dwr, float* dx, hipStream_t st);

}  // namespace mm
