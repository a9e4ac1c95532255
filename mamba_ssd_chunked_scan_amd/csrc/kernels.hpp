// kernels.hpp -- host-side launchers of the libssd kernels (internal interface
// between the C ABI in api.cpp and the .hip translation units).  Every launcher
// assumes its arguments were validated by api.cpp and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace ssd {

enum DType { DT_F32 = 0, DT_BF16 = 1 };

hipError_t launch_varlen_meta(const Geo& g, const int32_t* cu_seqlens, int32_t* meta,
                              hipStream_t s);

hipError_t launch_chunk_cumsum(const Geo& g, TArg dt, int dt_dtype, const float* A,
                               const float* dt_bias, int softplus, int clamp, float dt_min,
                               float dt_max, float* cs, float* dt_out, hipStream_t s);

hipError_t launch_bmm_chunk(const Geo& g, TArg C, TArg B, int in_dtype, float* CB,
                            hipStream_t s);

hipError_t launch_chunk_state(const Geo& g, TArg x, TArg B, int in_dtype, const float* cs,
                              void* states, int st_dtype, hipStream_t s);

hipError_t launch_state_passing(const Geo& g, const void* states, int st_dtype,
                                const float* cs, const float* h0, void* states_out,
                                float* hfinal, hipStream_t s);

// Chunk states and the inter-chunk scan in one pass (bf16 inputs): writes the
// carry-in states (K, H, P, N) in the state dtype and the final states.
hipError_t launch_state_scan(const Geo& g, TArg x, TArg B, const float* cs, const float* h0,
                             void* hin, int st_dtype, float* hfinal, hipStream_t s);

hipError_t launch_chunk_scan(const Geo& g, const float* CB, TArg x, TArg C, int in_dtype,
                             const float* cs, const void* states, int st_dtype,
                             const float* D, TArg z, TArg out, int out_dtype, hipStream_t s);

}  // namespace ssd
