// Host-side launchers of the AVQ kernels (internal to libavq).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace avq {

// Raise a kernel's dynamic-LDS limit when a launch needs more than the
// default; remembers the largest size set per kernel so the attribute call is
// made once per size class, not on every launch.
hipError_t raise_lds_limit(const void* kernel, size_t bytes);

size_t assign_smem_bytes(int dtype, int d, int M0, int C);
size_t attention_smem_bytes(int dtype, int d, int M0, int C, int P, int block_q, bool importance);

// Parent rows of the attention kernel's operands: M0 padded to whole 64-row
// passes (padding rows carry zero values and count 0).
__host__ __device__ constexpr int attn_parent_rows(int M0) { return (M0 + 63) & ~63; }

// Children rows staged in LDS per chunk by the attention kernel.
template <int D>
struct AttnTraits {
  static constexpr int kChunkRows = 64;
};

// zeroes nv floats of vsum, nk floats of ksum (both multiples of 4) and nc ints of counts
hipError_t launch_zero(float* vsum, int64_t nv, float* ksum, int64_t nk, int* counts, int64_t nc, hipStream_t st);
hipError_t launch_assign(int dtype, const void* K, const void* V, const void* cb, int BH, int H, int N, int d, int M0,
                         int C, float* vsum, int* counts, int* assign, float* ksum, hipStream_t st);
size_t attention_workspace_bytes(int dtype, int d, int M0, int C, int BH);
// stages of launch_attention: the value fragments of the workspace, the attention kernel
constexpr int kAttnPrep = 1;
constexpr int kAttnKernel = 2;
hipError_t launch_attention(int dtype, const void* Q, const void* cb, const float* vsum, const int* counts, int BH, int H,
                            int N, int d, int M0, int C, int P, int bq, float scale, float* Y, int* topp,
                            float* importance, void* ws, bool approx, const int* order, int stages, float* clear_v,
                            int* clear_c, hipStream_t st);
hipError_t launch_codebook_update(const float* ksum, const int* counts, int B, int H, int d, int M0, int C,
                                  float decay, float* S, float* Nm, float* cb, hipStream_t st);

}  // namespace avq
