// Device-side building blocks shared by the two AVQ kernels (gfx950 / CDNA4).
//
// MFMA conventions used throughout (32x32 output tiles, wave64):
//   * An operand of v_mfma_f32_32x32x{16,2}: lane l supplies row (l % 32) of
//     A (or column (l % 32) of B) and a slice of E consecutive contraction
//     elements; lanes l and l + 32 ("halves" h = l / 32) hold the two slices
//     of one k-step.  The contraction pairs slot j of half h in A with slot j
//     of half h in B, so any consistent labelling of the slices works.
//   * The 16 accumulator registers of lane l hold column (l % 32) and rows
//     row_of(r, h) = 8 * (r / 4) + 4 * h + (r % 4), r = 0..15.
// The attention kernel computes logits transposed (rows = codewords,
// columns = queries) so that every lane owns one query and 16 codewords per
// 32-row block; the same registers then feed the weighted value sum as the B
// operand without any data movement.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace avq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// bfloat16 inputs: logits on bf16 MFMA; weighted value sums on fp16 MFMA with
// value sums scaled by a power of two per staged chunk.
struct TBF16 {
  using in_t = __bf16;
  using frag_t = bf16x8;
  using pv_t = _Float16;
  using pvfrag_t = f16x8;
  static constexpr int E = 8;
  static constexpr bool kScaleValues = true;
  __device__ static inline f32x16 mma_in(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline f32x16 mma_pv(pvfrag_t a, pvfrag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline pvfrag_t pack_pv(const float* x) {
    pvfrag_t v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (_Float16)x[j];
    return v;
  }
  __device__ static inline float to_f32(in_t x) { return (float)x; }
};

// float inputs: every contraction on fp32 MFMA.
struct TF32 {
  using in_t = float;
  using frag_t = float;
  using pv_t = float;
  using pvfrag_t = float;
  static constexpr int E = 1;
  static constexpr bool kScaleValues = false;
  __device__ static inline f32x16 mma_in(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline f32x16 mma_pv(pvfrag_t a, pvfrag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline pvfrag_t pack_pv(const float* x) { return x[0]; }
  __device__ static inline float to_f32(in_t x) { return x; }
};

// accumulator register r of half h holds output row row_of(r, h)
__device__ __forceinline__ int row_of(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }
// inverse: output row rho is register r_of_row(rho) of half h_of_row(rho)
__device__ __forceinline__ int h_of_row(int rho) { return (rho >> 2) & 1; }
__device__ __forceinline__ int r_of_row(int rho) { return 4 * (rho >> 3) + (rho & 3); }
// Column of a codeword in the staged (transposed) value tile: the codeword
// that sits at accumulator register (r, h) of a 32-row block is stored at
// position col_of(r, h), so that the E registers of one k-step are E
// consecutive columns.
__device__ __forceinline__ int col_of(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }
__device__ __forceinline__ int r_of_col(int q) { return 8 * (q >> 4) + (q & 7); }
__device__ __forceinline__ int h_of_col(int q) { return (q >> 3) & 1; }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// ---- cross-lane helpers -------------------------------------------------
// value of the same register in lane l ^ 32
__device__ __forceinline__ float xhalf_partner(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(p[0]) : __uint_as_float(p[1]);
}
__device__ __forceinline__ int xhalf_partner(int x) {
  auto p = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return (threadIdx.x & 32) ? (int)p[0] : (int)p[1];
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xhalf_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
constexpr int DPP_ROW_MIRROR = 0x140;       // lane i <- 15 - i within 16
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <- 7 - i within 8
constexpr int DPP_QP_3210 = 0x1B;           // lane i <- 3 - i within 4
constexpr int DPP_QP_1032 = 0xB1;           // lane i <- i ^ 1

// Reduce-scatter over the 16 lanes of a DPP row: on entry v[0..16) per lane,
// on exit v[0] of lane i holds the sum over the row of register (i % 16).
// Each butterfly step forms both candidate sums with the partner's value
// moved by DPP (folded into the add) and keeps the one for this lane's half.
template <int CTRL, int HALF>
__device__ __forceinline__ void rs_step(float* v, bool lo) {
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const float a = v[i] + dpp<CTRL>(v[i]);                // kept by the lower lanes
    const float b = v[HALF + i] + dpp<CTRL>(v[HALF + i]);  // kept by the upper lanes
    v[i] = lo ? a : b;
  }
}
__device__ __forceinline__ void rs_row16(float* v, int lane) {
  rs_step<DPP_ROW_MIRROR, 8>(v, (lane & 15) < 8);      // partner 15 - i
  rs_step<DPP_ROW_HALF_MIRROR, 4>(v, (lane & 7) < 4);  // partner 7 - i within 8
  rs_step<DPP_QP_3210, 2>(v, (lane & 3) < 2);          // partner 3 - i within 4
  rs_step<DPP_QP_1032, 1>(v, (lane & 1) == 0);         // partner i ^ 1
}

// Sum over the 32 lanes of each half of 32 registers: on exit v[0] of lane l
// holds the half's total of register (l % 32).
__device__ __forceinline__ void rs_half32(float* v, int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[16 + i]), false, false);
    v[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  rs_row16(v, lane);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ void atomic_add_f32(float* p, float v) { unsafeAtomicAdd(p, v); }

// Workgroup barrier for LDS traffic only: this wave's LDS accesses are complete
// before it and visible after it.  Unlike __syncthreads() it does not wait for
// the wave's global loads and stores still in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Global -> LDS copy of one fragment per lane (no registers): lane l's BYTES
// at gptr land at lds_base + l * BYTES.  Counted by vmcnt; readers wait for it
// and, across waves, for a barrier.
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void* gptr, void* lds_base) {
  static_assert(BYTES == 16 || BYTES == 4, "fragment size");
  if constexpr (BYTES == 16)
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

}  // namespace avq
