// Codebook update step of the training recipe ("AVQ-Attention: Adaptive
// Vector-Quantized Attention", App. A, Eq. 11 and Eq. 12; Sec. 4.1, Fig. 2):
// EMA statistics of every codeword, parents moved to their means, children
// projected back onto the parent-child constraint by the mass-weighted
// least-squares solution.
//
// The batch statistics are the per-(batch, head) key sums and counts of the
// aggregation call run with the keys in place of the values (parents over
// their whole cell, children over the keys that moved to them); this kernel
// folds them over the batch into the head's EMA state.  The work is a few
// floats per codeword: the kernel is bound by launch and HBM latency, not by
// arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "avq_launch.h"

namespace avq {
namespace {

constexpr int kMaxChildren = 16;

// One wave per (head, parent): the parent and its C children.  Every
// codeword's mass is the same in all lanes; lane t holds dimension t of a
// 64-dimension chunk.  The wave reads and writes only its own rows of S, N
// and the codebook, so the update is in place.
__global__ __launch_bounds__(256) void codebook_update_kernel(const float* __restrict__ ksum,
                                                              const int* __restrict__ counts, int B, int H, int d,
                                                              int M0, int C, float decay, float* __restrict__ S,
                                                              float* __restrict__ Nm, float* __restrict__ cb) {
  const int lane = threadIdx.x & 63;
  const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
  if (gw >= H * M0) return;
  const int h = gw / M0, p = gw % M0;
  const int64_t Mt = (int64_t)M0 * (1 + C);
  const float keep = decay, take = 1.0f - decay;
  float* Sh = S + (int64_t)h * Mt * d;
  float* Nh = Nm + (int64_t)h * Mt;
  float* cbh = cb + (int64_t)h * Mt * d;
  const int64_t c0 = M0 + (int64_t)p * C;
  auto row = [&](int i) -> int64_t { return i == 0 ? (int64_t)p : c0 + i - 1; };  // i = 0: the parent

  // Eq. 11 for the masses of the group
  float n[1 + kMaxChildren];
#pragma unroll
  for (int i = 0; i <= kMaxChildren; ++i) {
    n[i] = 0.0f;
    if (i <= C) {
      int cnt = 0;
      for (int b = 0; b < B; ++b) cnt += counts[((int64_t)b * H + h) * Mt + row(i)];
      n[i] = keep * Nh[row(i)] + take * (float)cnt;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i <= kMaxChildren; ++i)
      if (i <= C) Nh[row(i)] = n[i];
  }
  // Eq. 12's share of the residual for each child, 1 / (N_c sigma) with
  // sigma = sum 1 / N_c, taken relative to the lightest child (every ratio is
  // then at most one, so no reciprocal of a tiny mass can overflow); children
  // without mass take the whole residual between them, the limit of Eq. 12
  float share[kMaxChildren];
  {
    int zeros = 0;
    float nmin = INFINITY;
#pragma unroll
    for (int c = 0; c < kMaxChildren; ++c)
      if (c < C) {
        const float m = n[1 + c];
        if (m > 0.0f) nmin = fminf(nmin, m); else ++zeros;
      }
    float usum = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxChildren; ++c) {
      const float m = n[1 + c];
      share[c] = (c < C && m > 0.0f) ? nmin / m : 0.0f;
      usum += share[c];
    }
#pragma unroll
    for (int c = 0; c < kMaxChildren; ++c) {
      const float m = n[1 + c];
      if (zeros == 0) share[c] = share[c] / usum;
      else share[c] = (c < C && !(m > 0.0f)) ? 1.0f / (float)zeros : 0.0f;
    }
  }

  for (int t0 = 0; t0 < d; t0 += 64) {
    const int t = t0 + lane;
    if (t >= d) break;
    // Eq. 11 for the key sums, then the means
    float mean[1 + kMaxChildren];
#pragma unroll
    for (int i = 0; i <= kMaxChildren; ++i) {
      mean[i] = 0.0f;
      if (i <= C) {
        float ks = 0.0f;
        for (int b = 0; b < B; ++b) ks += ksum[(((int64_t)b * H + h) * Mt + row(i)) * d + t];
        const float s = keep * Sh[row(i) * d + t] + take * ks;
        Sh[row(i) * d + t] = s;
        // a codeword without mass keeps its position
        mean[i] = n[i] > 0.0f ? s / n[i] : cbh[row(i) * d + t];
      }
    }
    cbh[(int64_t)p * d + t] = mean[0];
    if (C == 0) continue;
    float delta = 0.0f;  // Eq. 12's residual: sum of the child means minus C times the parent
#pragma unroll
    for (int c = 0; c < kMaxChildren; ++c)
      if (c < C) delta += mean[1 + c];
    delta = fmaf(-(float)C, mean[0], delta);
#pragma unroll
    for (int c = 0; c < kMaxChildren; ++c)
      if (c < C) cbh[(c0 + c) * d + t] = fmaf(-share[c], delta, mean[1 + c]);
  }
}

}  // namespace

hipError_t launch_codebook_update(const float* ksum, const int* counts, int B, int H, int d, int M0, int C,
                                  float decay, float* S, float* Nm, float* cb, hipStream_t st) {
  const int64_t waves = (int64_t)H * M0;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  hipLaunchKernelGGL(codebook_update_kernel, dim3(blocks), dim3(256), 0, st, ksum, counts, B, H, d, M0, C, decay, S,
                     Nm, cb);
  return hipGetLastError();
}

}  // namespace avq
