// Kernel 1 of the AVQ-Attention forward pass: two-level VQ assignment of the
// keys and per-codeword value sums and key counts ("AVQ-Attention: Adaptive
// Vector-Quantized Attention", Sec. 4.2 and Algorithm 1; Eq. 2 and 3).
//
// One workgroup (4 waves) owns a chunk of consecutive keys of one (batch,
// head).  Design for CDNA4:
//   * Parent distances ||c||^2 - 2 k.c come from MFMA: parents of the head
//     are staged once in LDS as the A operand, keys are streamed from HBM
//     straight into B-operand registers (64 keys per wave step) and stay
//     there for the child search.
//   * Child distances: the distinct parents of the wave's 64 keys are packed
//     four (C <= 8) at a time into a 32-row block of their children, one MFMA
//     block per group; each key then reads the C distances of its own parent
//     from registers.  Parent and child distances use the same formula.
//   * Aggregation without per-key global atomics: keys are counting-sorted in
//     LDS by (parent, slot), then 8 streams walk the sorted keys with one lane
//     per pair/quad of value dimensions, accumulate runs in registers and
//     issue one coalesced atomic row update per run.  Counts are flushed from
//     the LDS histogram.  Heavy-tailed occupancy therefore costs one atomic
//     row update per chunk per codeword, not per key.
#include "avq_device.h"
#include "avq_launch.h"

namespace avq {

namespace {

template <class T>
struct VecLoad;
template <>
struct VecLoad<TBF16> {
  // EPL consecutive bf16 values -> float
  template <int EPL>
  __device__ static inline void load(const __bf16* p, float* out) {
    if constexpr (EPL == 2) {
      uint32_t u = *(const uint32_t*)p;
      out[0] = __uint_as_float(u << 16);
      out[1] = __uint_as_float(u & 0xFFFF0000u);
    } else {
      uint2 u = *(const uint2*)p;
      out[0] = __uint_as_float(u.x << 16);
      out[1] = __uint_as_float(u.x & 0xFFFF0000u);
      out[2] = __uint_as_float(u.y << 16);
      out[3] = __uint_as_float(u.y & 0xFFFF0000u);
    }
  }
};
template <>
struct VecLoad<TF32> {
  template <int EPL>
  __device__ static inline void load(const float* p, float* out) {
    if constexpr (EPL == 2) {
      f32x2 v = *(const f32x2*)p;
      out[0] = v[0];
      out[1] = v[1];
    } else {
      f32x4 v = *(const f32x4*)p;
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = v[i];
    }
  }
};

}  // namespace

// W: width of a child slot in accumulator registers (C <= W, W in {4,8,16}).
template <class T, int D, int W>
__global__ __launch_bounds__(256) void assign_aggregate_kernel(
    const typename T::in_t* __restrict__ K, const typename T::in_t* __restrict__ V,
    const typename T::in_t* __restrict__ cb, int H, int N, int M0, int C, int chunk,
    float* __restrict__ vsum, int* __restrict__ counts, int* __restrict__ assign) {
  using in_t = typename T::in_t;
  using frag_t = typename T::frag_t;
  constexpr int E = T::E;
  constexpr int KS = D / (2 * E);            // k-steps over the head dimension
  constexpr int LDP = D + 16 / sizeof(in_t); // padded LDS row of a parent
  constexpr int S = 32 / W;                  // child slots per 32-row block
  constexpr int EPL = D / 32;                // value elements per lane in the walk

  extern __shared__ __align__(16) unsigned char smem[];
  const int Mt = M0 * (1 + C);
  const int M0p = (M0 + 31) & ~31;
  const int NB = M0 * (C + 1);
  in_t* sPar = (in_t*)smem;
  float* sNorm = (float*)(sPar + (size_t)M0p * LDP);
  int* sHist = (int*)(sNorm + Mt);
  int* sScan = sHist + NB;
  unsigned short* sBin = (unsigned short*)(sScan + 8);
  unsigned short* sSorted = sBin + chunk;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, hh = lane >> 5;
  const int bh = blockIdx.y, h = bh % H;
  const int cstart = blockIdx.x * chunk;
  const int nval = min(chunk, N - cstart);
  const in_t* cbh = cb + (int64_t)h * Mt * D;
  const in_t* Kb = K + (int64_t)bh * N * D;
  const in_t* Vb = V + (int64_t)bh * N * D;

  // ---- stage parents, codeword norms, clear the histogram ---------------
  for (int i = tid; i < M0p * (D / E); i += 256) {
    const int row = i / (D / E), col = (i % (D / E)) * E;
    const int src = row < M0 ? row : 0;
    frag_t v = *(const frag_t*)(cbh + (int64_t)src * D + col);
    *(frag_t*)(sPar + row * LDP + col) = v;
  }
  for (int r = tid; r < Mt; r += 256) {
    const frag_t* c = (const frag_t*)(cbh + (int64_t)r * D);
    float acc = 0.0f;
    for (int t = 0; t < D / E; ++t) {
      frag_t v = c[t];
      if constexpr (E == 1) {
        float x = T::to_f32(v);
        acc = fmaf(x, x, acc);
      } else {
#pragma unroll
        for (int j = 0; j < E; ++j) {
          float x = T::to_f32(v[j]);
          acc = fmaf(x, x, acc);
        }
      }
    }
    sNorm[r] = acc;
  }
  for (int i = tid; i < NB; i += 256) sHist[i] = 0;
  __syncthreads();

  // ---- assignment, 64 keys per wave step ---------------------------------
  const int keys_per_wave = chunk / 4;
  const int nblkP = M0p / 32;
  for (int it = 0; it < keys_per_wave; it += 64) {
    const int kbase = cstart + wave * keys_per_wave + it;
    if (kbase >= N) break;
    frag_t kf[2][KS];
    int key[2];
    bool kval[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      key[g] = kbase + g * 32 + ql;
      kval[g] = key[g] < N;
      const in_t* kp = Kb + (int64_t)(kval[g] ? key[g] : N - 1) * D + E * hh;
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[g][s] = *(const frag_t*)(kp + s * 2 * E);
    }
    // nearest parent: first minimum of ||c||^2 - 2 k.c
    float best[2] = {INFINITY, INFINITY};
    int bidx[2] = {0, 0};
    for (int blk = 0; blk < nblkP; ++blk) {
      f32x16 a0 = zero16(), a1 = zero16();
      const in_t* ap = sPar + (blk * 32 + ql) * LDP + E * hh;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        frag_t a = *(const frag_t*)(ap + s * 2 * E);
        a0 = T::mma_in(a, kf[0][s], a0);
        a1 = T::mma_in(a, kf[1][s], a1);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = blk * 32 + row_of(r, hh);
        const float nrm = row < M0 ? sNorm[row] : INFINITY;
        const float d0 = nrm - 2.0f * a0[r];
        const float d1 = nrm - 2.0f * a1[r];
        if (d0 < best[0]) { best[0] = d0; bidx[0] = row; }
        if (d1 < best[1]) { best[1] = d1; bidx[1] = row; }
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float pb = xhalf_partner(best[g]);
      const int pi = xhalf_partner(bidx[g]);
      if (pb < best[g] || (pb == best[g] && pi < bidx[g])) { best[g] = pb; bidx[g] = pi; }
    }

    // children of the distinct parents, S parents per MFMA block
    float dch[2] = {INFINITY, INFINITY};
    int cst[2] = {-1, -1};
    bool need0 = kval[0], need1 = kval[1];
    const int rr = r_of_row(ql), hr = h_of_row(ql);
    const int srow = 2 * (rr / W) + hr, crow = rr % W;  // slot and child of this lane's A row
    while (true) {
      uint64_t b0 = __ballot(need0), b1 = __ballot(need1);
      if ((b0 | b1) == 0) break;
      int gpar[S];
      int ng = 0, slot0 = -1, slot1 = -1;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        gpar[s] = -1;
        b0 = __ballot(need0);
        b1 = __ballot(need1);
        if ((b0 | b1) == 0) break;
        const int p = b0 ? __builtin_amdgcn_readlane(bidx[0], __builtin_ctzll(b0))
                         : __builtin_amdgcn_readlane(bidx[1], __builtin_ctzll(b1));
        gpar[s] = p;
        ng = s + 1;
        if (need0 && bidx[0] == p) { slot0 = s; need0 = false; }
        if (need1 && bidx[1] == p) { slot1 = s; need1 = false; }
      }
      int prow = -1;
#pragma unroll
      for (int s = 0; s < S; ++s)
        if (s == srow && s < ng) prow = gpar[s];
      const int crow_idx = (prow >= 0 && crow < C) ? M0 + prow * C + crow : 0;
      const in_t* cp = cbh + (int64_t)crow_idx * D + E * hh;
      f32x16 c0 = zero16(), c1 = zero16();
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        frag_t a = *(const frag_t*)(cp + s * 2 * E);
        c0 = T::mma_in(a, kf[0][s], c0);
        c1 = T::mma_in(a, kf[1][s], c1);
      }
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int slot = g ? slot1 : slot0;
        if (slot >= 0 && (slot & 1) == hh) {
          const int gg = slot >> 1;
          const int base = M0 + bidx[g] * C;
          float dmin = INFINITY;
          int cmin = -1;
#pragma unroll
          for (int c = 0; c < W; ++c) {
            if (c < C) {
              float v = g ? c1[c] : c0[c];
#pragma unroll
              for (int gi = 1; gi < 16 / W; ++gi)
                if (gg == gi) v = g ? c1[gi * W + c] : c0[gi * W + c];
              const float dist = sNorm[base + c] - 2.0f * v;
              if (dist < dmin) { dmin = dist; cmin = c; }
            }
          }
          dch[g] = dmin;
          cst[g] = cmin;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float pd = xhalf_partner(dch[g]);
      const int pc = xhalf_partner(cst[g]);
      if (cst[g] < 0) { dch[g] = pd; cst[g] = pc; }
    }
    // lane half hh records key group hh
    const int a_ = hh ? bidx[1] : bidx[0];
    const float db_ = hh ? best[1] : best[0];
    const float dc_ = hh ? dch[1] : dch[0];
    const int cs_ = hh ? cst[1] : cst[0];
    const int k_ = hh ? key[1] : key[0];
    if (hh ? kval[1] : kval[0]) {
      const bool moved = cs_ >= 0 && dc_ < db_;
      const int bin = a_ * (C + 1) + (moved ? 1 + cs_ : 0);
      sBin[k_ - cstart] = (unsigned short)bin;
      atomicAdd(&sHist[bin], 1);
      if (assign) assign[(int64_t)bh * N + k_] = moved ? M0 + a_ * C + cs_ : a_;
    }
  }
  __syncthreads();

  // ---- counts, and bin offsets for the counting sort ----------------------
  // thread t owns parent t (M0 <= 256): bins t*(C+1) .. t*(C+1)+C
  int mycount = 0;
  if (tid < M0) {
    for (int sl = 0; sl <= C; ++sl) mycount += sHist[tid * (C + 1) + sl];
    if (mycount > 0) {
      atomicAdd(&counts[(int64_t)bh * Mt + tid], mycount);
      for (int sl = 1; sl <= C; ++sl) {
        const int c = sHist[tid * (C + 1) + sl];
        if (c) atomicAdd(&counts[(int64_t)bh * Mt + M0 + tid * C + sl - 1], c);
      }
    }
  }
  const int incl = wave_incl_scan(mycount, lane);
  if (lane == 63) sScan[wave] = incl;
  __syncthreads();
  int off = incl - mycount;
  for (int w = 0; w < wave; ++w) off += sScan[w];
  if (tid < M0) {
    for (int sl = 0; sl <= C; ++sl) {
      const int b = tid * (C + 1) + sl;
      const int c = sHist[b];
      sHist[b] = off;
      off += c;
    }
  }
  __syncthreads();
  for (int k = tid; k < nval; k += 256) {
    const int pos = atomicAdd(&sHist[sBin[k]], 1);
    sSorted[pos] = (unsigned short)k;
  }
  __syncthreads();

  // ---- value sums: 8 streams walk the sorted keys ---------------------------
  const int stream = wave * 2 + hh;
  const int per = (nval + 7) / 8;
  const int p0 = stream * per;
  const int p1 = min(nval, p0 + per);
  const int col = ql * EPL;
  float pacc[EPL], cacc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) { pacc[e] = 0.0f; cacc[e] = 0.0f; }
  int pcur = -1, ccur = -1;
  float* vsb = vsum + (int64_t)bh * Mt * D + col;
  constexpr int U = 8;
  for (int pos = p0; pos < p1; pos += U) {
    float vb[U][EPL];
    int bb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pp = pos + u;
      const int k = sSorted[pp < p1 ? pp : p0];
      bb[u] = pp < p1 ? (int)sBin[k] : -1;
      VecLoad<T>::template load<EPL>(Vb + (int64_t)(cstart + k) * D + col, vb[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = bb[u];
      if (b < 0) break;
      const int p = b / (C + 1);
      const int sl = b - p * (C + 1);
      if (p != pcur) {
        if (pcur >= 0) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) atomic_add_f32(vsb + (int64_t)pcur * D + e, pacc[e]);
        }
        pcur = p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) pacc[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) pacc[e] += vb[u][e];
      if (sl > 0) {
        if (b != ccur) {
          if (ccur >= 0) {
            const int cp = ccur / (C + 1);
            const int crow = M0 + cp * C + (ccur - cp * (C + 1)) - 1;
#pragma unroll
            for (int e = 0; e < EPL; ++e) atomic_add_f32(vsb + (int64_t)crow * D + e, cacc[e]);
          }
          ccur = b;
#pragma unroll
          for (int e = 0; e < EPL; ++e) cacc[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) cacc[e] += vb[u][e];
      }
    }
  }
  if (pcur >= 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) atomic_add_f32(vsb + (int64_t)pcur * D + e, pacc[e]);
  }
  if (ccur >= 0) {
    const int cp = ccur / (C + 1);
    const int crow = M0 + cp * C + (ccur - cp * (C + 1)) - 1;
#pragma unroll
    for (int e = 0; e < EPL; ++e) atomic_add_f32(vsb + (int64_t)crow * D + e, cacc[e]);
  }
}

__global__ __launch_bounds__(256) void zero_kernel(f32x4* __restrict__ a, int64_t na4, int* __restrict__ b, int64_t nb) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < na4; i += stride) a[i] = z;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nb; i += stride) b[i] = 0;
}

size_t assign_smem_bytes(int dtype, int d, int M0, int C, int chunk) {
  const size_t es = dtype == 0 ? 4 : 2;
  const size_t ldp = d + 16 / es;
  const size_t M0p = (M0 + 31) & ~31;
  const size_t Mt = (size_t)M0 * (1 + C);
  const size_t NB = (size_t)M0 * (C + 1);
  return M0p * ldp * es + Mt * 4 + NB * 4 + 8 * 4 + (size_t)chunk * 2 * 2;
}

template <class T, int D, int W>
static hipError_t launch_assign_t(const void* K, const void* V, const void* cb, int BH, int H, int N, int M0, int C,
                                  int chunk, float* vsum, int* counts, int* assign, hipStream_t st) {
  const size_t smem = assign_smem_bytes(std::is_same<T, TF32>::value ? 0 : 1, D, M0, C, chunk);
  auto kern = assign_aggregate_kernel<T, D, W>;
  hipError_t e = raise_lds_limit((const void*)kern, smem);
  if (e != hipSuccess) return e;
  dim3 grid((N + chunk - 1) / chunk, BH);
  hipLaunchKernelGGL(kern, grid, dim3(256), smem, st, (const typename T::in_t*)K, (const typename T::in_t*)V,
                     (const typename T::in_t*)cb, H, N, M0, C, chunk, vsum, counts, assign);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_assign_w(const void* K, const void* V, const void* cb, int BH, int H, int N, int M0, int C,
                                  int chunk, float* vsum, int* counts, int* assign, hipStream_t st) {
  if (C <= 4) return launch_assign_t<T, D, 4>(K, V, cb, BH, H, N, M0, C, chunk, vsum, counts, assign, st);
  if (C <= 8) return launch_assign_t<T, D, 8>(K, V, cb, BH, H, N, M0, C, chunk, vsum, counts, assign, st);
  return launch_assign_t<T, D, 16>(K, V, cb, BH, H, N, M0, C, chunk, vsum, counts, assign, st);
}

hipError_t launch_zero(float* vsum, int64_t nv, int* counts, int64_t nc, hipStream_t st) {
  const int64_t work = nv / 4 > nc ? nv / 4 : nc;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (f32x4*)vsum, nv / 4, counts, nc);
  return hipGetLastError();
}

hipError_t launch_assign(int dtype, const void* K, const void* V, const void* cb, int BH, int H, int N, int d, int M0,
                         int C, int chunk, float* vsum, int* counts, int* assign, hipStream_t st) {
  if (dtype == 0) {
    if (d == 64) return launch_assign_w<TF32, 64>(K, V, cb, BH, H, N, M0, C, chunk, vsum, counts, assign, st);
    return launch_assign_w<TF32, 128>(K, V, cb, BH, H, N, M0, C, chunk, vsum, counts, assign, st);
  }
  if (d == 64) return launch_assign_w<TBF16, 64>(K, V, cb, BH, H, N, M0, C, chunk, vsum, counts, assign, st);
  return launch_assign_w<TBF16, 128>(K, V, cb, BH, H, N, M0, C, chunk, vsum, counts, assign, st);
}

}  // namespace avq
