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

// One wave per (head, parent): the parent and its C children (C <= W).  Lane
// t holds dimension t of a 64-dimension chunk; the masses are gathered one
// codeword per lane and broadcast.  The work per wave is a few hundred bytes,
// so the kernel is bound by memory latency: every load is issued before any
// is used -- the counts first, then the first chunk's key sums, EMA sums and
// positions, four batch entries at a time -- so that a wave waits for memory
// about once.  Rows past C repeat the parent's and batch entries past B
// repeat the last, and are masked.  The wave reads and writes only its own
// rows of S, N and the codebook, so the update is in place.
template <int W>
__global__ __launch_bounds__(256) void codebook_update_kernel(const float* __restrict__ ksum,
                                                              const int* __restrict__ counts, int B, int H, int d,
                                                              int M0, int C, float decay, float* __restrict__ S,
                                                              float* __restrict__ Nm, float* __restrict__ cb) {
  constexpr int BU = 4;  // batch entries per group of loads
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
  // codeword i of the group: 0 the parent, 1 + c child c; past C the parent again
  auto row = [&](int i) -> int64_t { return (i == 0 || i > C) ? (int64_t)p : c0 + i - 1; };
  const int64_t bstride = (int64_t)H * Mt;  // between the batch entries of one head
  const int blast = B > 0 ? B - 1 : 0;

  // the counts and the old mass of codeword `lane` of the group
  const int64_t rl = row(lane <= C ? lane : 0);
  const float nold = Nh[rl];
  auto load_counts = [&](int b, int* cv) {
#pragma unroll
    for (int j = 0; j < BU; ++j) cv[j] = counts[(int64_t)h * Mt + rl + (int64_t)min(b + j, blast) * bstride];
  };
  // the first batch entries' counts, summed after the chunk's loads are
  // issued (with B = 0 there are none, and counts and ksum may be NULL)
  int cv0[BU] = {0, 0, 0, 0};
  if (B > 0) load_counts(0, cv0);

  // this lane's dimension of every codeword of the group, for one chunk
  float sv[1 + W], pv[1 + W], ks[1 + W];
  auto load_chunk = [&](int t) {
    const float* kb = ksum + ((int64_t)h * Mt) * d + t;
#pragma unroll
    for (int i = 0; i <= W; ++i) {
      sv[i] = Sh[row(i) * d + t];
      pv[i] = cbh[row(i) * d + t];
      ks[i] = 0.0f;
    }
    for (int b = 0; b < B; b += BU) {
      float kv[BU][1 + W];
#pragma unroll
      for (int j = 0; j < BU; ++j)
#pragma unroll
        for (int i = 0; i <= W; ++i) kv[j][i] = kb[((int64_t)min(b + j, blast) * bstride + row(i)) * d];
#pragma unroll
      for (int j = 0; j < BU; ++j)
#pragma unroll
        for (int i = 0; i <= W; ++i) ks[i] += b + j < B ? kv[j][i] : 0.0f;
    }
  };
  const int tl = lane < d ? lane : d - 1;
  load_chunk(tl);
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < BU; ++j) cnt += j < B ? cv0[j] : 0;
  for (int b = BU; b < B; b += BU) {
    int cv[BU];
    load_counts(b, cv);
#pragma unroll
    for (int j = 0; j < BU; ++j) cnt += b + j < B ? cv[j] : 0;
  }

  // Eq. 11 for the masses, broadcast: n[i] is the mass of codeword i (0 past C)
  const float nl = lane <= C ? keep * nold + take * (float)cnt : 0.0f;
  if (lane <= C) Nh[rl] = nl;
  float n[1 + W];
#pragma unroll
  for (int i = 0; i <= W; ++i) n[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(nl), i));
  // Eq. 12's share of the residual for each child, 1 / (N_c sigma) with
  // sigma = sum 1 / N_c, taken relative to the lightest child (every ratio is
  // then at most one, so no reciprocal of a tiny mass can overflow); children
  // without mass take the whole residual between them, the limit of Eq. 12
  float share[W];
  {
    int zeros = 0;
    float nmin = INFINITY;
#pragma unroll
    for (int c = 0; c < W; ++c)
      if (c < C) {
        if (n[1 + c] > 0.0f) nmin = fminf(nmin, n[1 + c]); else ++zeros;
      }
    float usum = 0.0f;
#pragma unroll
    for (int c = 0; c < W; ++c) {
      share[c] = (c < C && n[1 + c] > 0.0f) ? nmin / n[1 + c] : 0.0f;
      usum += share[c];
    }
#pragma unroll
    for (int c = 0; c < W; ++c) {
      if (zeros == 0) share[c] = share[c] / usum;
      else share[c] = (c < C && !(n[1 + c] > 0.0f)) ? 1.0f / (float)zeros : 0.0f;
    }
  }

  for (int t0 = 0; t0 < d; t0 += 64) {
    const int t = t0 + lane;
    if (t0 > 0) load_chunk(t < d ? t : d - 1);
    if (t < d) {
      // Eq. 11 for the key sums, then the means (a codeword without mass keeps
      // its position)
      float mean[1 + W];
#pragma unroll
      for (int i = 0; i <= W; ++i) {
        const float sn = keep * sv[i] + take * ks[i];
        mean[i] = n[i] > 0.0f ? sn / n[i] : pv[i];
        if (i <= C) Sh[row(i) * d + t] = sn;
      }
      cbh[(int64_t)p * d + t] = mean[0];
      if (C > 0) {
        float delta = 0.0f;  // Eq. 12's residual: sum of the child means minus C times the parent
#pragma unroll
        for (int c = 0; c < W; ++c)
          if (c < C) delta += mean[1 + c];
        delta = fmaf(-(float)C, mean[0], delta);
#pragma unroll
        for (int c = 0; c < W; ++c)
          if (c < C) cbh[(c0 + c) * d + t] = fmaf(-share[c], delta, mean[1 + c]);
      }
    }
  }
}

}  // namespace

hipError_t launch_codebook_update(const float* ksum, const int* counts, int B, int H, int d, int M0, int C,
                                  float decay, float* S, float* Nm, float* cb, hipStream_t st) {
  const int64_t waves = (int64_t)H * M0;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  if (C <= 4)
    hipLaunchKernelGGL(codebook_update_kernel<4>, dim3(blocks), dim3(256), 0, st, ksum, counts, B, H, d, M0, C, decay,
                       S, Nm, cb);
  else if (C <= 8)
    hipLaunchKernelGGL(codebook_update_kernel<8>, dim3(blocks), dim3(256), 0, st, ksum, counts, B, H, d, M0, C, decay,
                       S, Nm, cb);
  else
    hipLaunchKernelGGL(codebook_update_kernel<16>, dim3(blocks), dim3(256), 0, st, ksum, counts, B, H, d, M0, C,
                       decay, S, Nm, cb);
  return hipGetLastError();
}

}  // namespace avq
