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
