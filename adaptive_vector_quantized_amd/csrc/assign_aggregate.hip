// Kernel 1 of the AVQ-Attention forward pass: two-level VQ assignment of the
// keys and per-codeword value sums and key counts ("AVQ-Attention: Adaptive
// Vector-Quantized Attention", Sec. 4.2 and Algorithm 1; Eq. 2 and 3).
//
// One workgroup (4 waves) owns a chunk of consecutive keys of one (batch,
// head).  Design for CDNA4:
//   * Parent distances ||c||^2 - 2 k.c come from MFMA: parents of the head
//     are staged once in LDS as the A operand (their norms are reduced from
//     LDS; a large codebook passes through LDS 64 parents at a time instead,
//     when that fits more workgroups on a CU), keys are streamed from HBM
//     straight into B-operand registers (64 keys per wave step) and stay
//     there for the child search.
//   * Child distances: the distinct parents of the wave's 64 keys are packed
//     S = 32 / W at a time into a 32-row block of their children, one MFMA
//     block per group; the children's norms come from the same operand
//     registers, so no codeword is read twice.  Each key then reads the C
//     distances of its own parent from registers.
//   * Aggregation without per-key atomics: the codewords the chunk touches
//     get compact slots; every wave loads the values of its own keys in
//     natural (coalesced) order straight into registers, issued right after
//     the assignment so their latency overlaps the slot bookkeeping.  The
//     value sums are then a matrix product on MFMA, (one-hot key -> slot)^T
//     x V, 32 slots at a time: with one lane per value column and the keys
//     of a lane half along K, the loaded registers already are the B
//     operand.  The four waves' partial tiles are added in LDS and each
//     touched codeword costs one coalesced atomic row update per chunk.
#include <algorithm>
#include <type_traits>

#include "avq_device.h"
#include "avq_launch.h"

namespace avq {

namespace {

// EPL consecutive input elements of one value row as they sit in registers
template <class T, int EPL>
struct RawV;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <>
struct RawV<TBF16, 2> { using t = uint32_t; };
template <>
struct RawV<TBF16, 4> { using t = u32x2; };
template <>
struct RawV<TF32, 2> { using t = f32x2; };
template <>
struct RawV<TF32, 4> { using t = f32x4; };

// Raw buffer load (bounds-checked by the descriptor: reads past num_records
// return zero).  Word 3 of the descriptor is the gfx9-family raw-access value.
// voff: per-lane byte offset, soff: wave-uniform byte offset.  The values are
// read exactly once, so the load is a streaming (non-temporal) one.
constexpr int kNonTemporal = 2;  // cache-policy bit of the buffer load
template <class R>
__device__ __forceinline__ R buf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  if constexpr (sizeof(R) == 4)
    return __builtin_bit_cast(R, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNonTemporal));
  else if constexpr (sizeof(R) == 8)
    return __builtin_bit_cast(R, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kNonTemporal));
  else
    return __builtin_bit_cast(R, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNonTemporal));
}
constexpr int kBufWord3 = 0x00020000;

// acc + the squared norm of one fragment (bf16 pairs on v_dot2: the products
// are exact in fp32)
template <class T>
__device__ __forceinline__ float frag_sumsq(typename T::frag_t v, float acc) {
  if constexpr (T::E == 1) {
    const float x = T::to_f32(v);
    return fmaf(x, x, acc);
  } else {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
#pragma unroll
    for (int j = 0; j < T::E / 2; ++j) {
      const bf16x2 x = {v[2 * j], v[2 * j + 1]};
      acc = __builtin_amdgcn_fdot2_f32_bf16(x, x, acc, false);
    }
    return acc;
  }
}

}  // namespace

// LDS layout of one workgroup (byte offsets; every array 16-byte aligned)
struct AssignLds {
  unsigned par, norm, cn, list, stage, hist, scan, slot, row, bin, ks, acc, total;
};

static size_t al16(size_t x) { return (x + 15) & ~(size_t)15; }

template <class T, int D>
struct AssignShape {
  static constexpr int EPL = D / 32;  // value elements per lane (32 lanes per key)
  static constexpr int kVgprPerKey = EPL * (int)sizeof(typename T::in_t) / 4;
  static constexpr int KPW = 128 / kVgprPerKey;  // keys per wave: 64 registers of values
  static constexpr int kChunk = 4 * KPW;         // keys per workgroup
  static constexpr int LDP = D + 16 / (int)sizeof(typename T::in_t);  // padded LDS row of a parent
  static constexpr int ACC_D = D < 64 ? D : 64;  // value columns per pass of the partial tiles
  // waves per SIMD the registers are set for: the whole codebook in LDS, or 64 parents at a time
  static constexpr int kWavesLds = (D == 64 && T::E > 1) ? 4 : 2;
  static constexpr int kWavesL2 = T::E > 1 ? (D == 64 ? 4 : 3) : (D == 64 ? 3 : 2);
};

// parents_lds: all the parents' codewords are staged in LDS (else 64 at a time)
static AssignLds assign_lds(int es, int d, int M0, int C, int chunk, bool parents_lds) {
  const size_t M0p = (M0 + 31) & ~31;
  const size_t Mt = (size_t)M0 * (1 + C);
  const size_t NB = (size_t)M0 * (C + 1);
  const size_t ldp = d + 16 / es;
  size_t o = 0, at[13];
  // assignment phase only
  at[0] = o; o = al16(o + (parents_lds ? M0p * ldp * es : 0));  // parents, padded rows
  at[1] = o; o = al16(o + M0p * 4);                // parent norms
  at[2] = o; o = al16(o + 4 * 32 * 4);             // child-block norms, per wave
  at[3] = o; o = al16(o + 4 * 64 * 4);             // distinct parents of a wave step
  at[12] = o; o = al16(o + (parents_lds ? 0 : (size_t)64 * d * es));  // one 64-parent pass (from L2)
  // aggregation phase only: four partial value tiles (up to 64 columns) over
  // the same bytes
  at[9] = 0;
  o = std::max(o, al16((size_t)4 * 32 * (d < 64 ? d : 64) * 4));
  at[4] = o; o = al16(o + NB * 4);                 // key count per (parent, child slot)
  at[5] = o; o = al16(o + 8 * 4);                  // scan partials
  at[6] = o; o = al16(o + Mt * 2);                 // codeword -> slot
  at[7] = o; o = al16(o + Mt * 2);                 // slot -> codeword
  at[8] = o; o = al16(o + (size_t)chunk * 2);      // parent << 5 | child slot of every key
  at[11] = o; o = al16(o + (size_t)chunk * 4);     // parent slot | child slot << 16 of every key
  at[10] = o;
  AssignLds L;
  L.par = (unsigned)at[0]; L.norm = (unsigned)at[1]; L.cn = (unsigned)at[2]; L.list = (unsigned)at[3];
  L.stage = (unsigned)at[12];
  L.hist = (unsigned)at[4]; L.scan = (unsigned)at[5]; L.slot = (unsigned)at[6]; L.row = (unsigned)at[7];
  L.bin = (unsigned)at[8]; L.ks = (unsigned)at[11]; L.acc = (unsigned)at[9]; L.total = (unsigned)at[10];
  return L;
}

// W: width of a child slot in accumulator registers (C <= W, W in {4,8,16}).
// PL: all parents' codewords staged in LDS; else they pass through a shared
// 64-parent LDS buffer (large codebooks: the LDS then holds more workgroups
// per CU).
template <class T, int D, int W, bool PL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PL ? AssignShape<T, D>::kWavesLds
                                                                          : AssignShape<T, D>::kWavesL2))) void
assign_aggregate_kernel(const typename T::in_t* __restrict__ K, const typename T::in_t* __restrict__ V,
                        const typename T::in_t* __restrict__ cb, int H, int N, int M0, int C,
                        AssignLds L, float* __restrict__ vsum, int* __restrict__ counts, int* __restrict__ assign,
                        float* __restrict__ ksum) {
  using in_t = typename T::in_t;
  using frag_t = typename T::frag_t;
  using Sh = AssignShape<T, D>;
  using raw_t = typename RawV<T, Sh::EPL>::t;
  constexpr int E = T::E;
  constexpr int KS = D / (2 * E);  // k-steps over the head dimension
  constexpr int LDP = Sh::LDP;
  constexpr int S = 32 / W;        // child slots per 32-row block
  constexpr int EPL = Sh::EPL;
  constexpr int KPW = Sh::KPW;
  constexpr int chunk = Sh::kChunk;

  extern __shared__ __align__(16) unsigned char smem[];
  const int Mt = M0 * (1 + C);
  const int M0p = (M0 + 31) & ~31;
  const int NB = M0 * (C + 1);
  in_t* sPar = (in_t*)(smem + L.par);
  float* sNorm = (float*)(smem + L.norm);
  float* sCN = (float*)(smem + L.cn);
  int* sList = (int*)(smem + L.list);
  int* sHist = (int*)(smem + L.hist);
  int* sScan = (int*)(smem + L.scan);
  unsigned short* sSlot = (unsigned short*)(smem + L.slot);
  unsigned short* sRow = (unsigned short*)(smem + L.row);
  unsigned short* sBin = (unsigned short*)(smem + L.bin);
  uint32_t* sKS = (uint32_t*)(smem + L.ks);
  float* sAcc = (float*)(smem + L.acc);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, hh = lane >> 5;
  // the chunks of one (batch, head) on one XCD when possible (consecutive
  // workgroup ids go to the XCDs round robin)
  int bh, ci;
  {
    const int nch = (N + chunk - 1) / chunk;
    const int L = blockIdx.x;
    const int BH = gridDim.x / nch;
    if ((BH & 7) == 0) {
      bh = (L / (8 * nch)) * 8 + (L & 7);
      ci = (L >> 3) % nch;
    } else {
      bh = L / nch;
      ci = L % nch;
    }
  }
  const int h = bh % H;
  const int cstart = ci * chunk;
  const int nval = min(chunk, N - cstart);
  const in_t* cbh = cb + (int64_t)h * Mt * D;
  const in_t* Kb = K + (int64_t)bh * N * D;
  const in_t* Vb = V + (int64_t)bh * N * D;

  // ---- stage parents, clear the histogram, parent norms -----------------
  // The first 32 keys of this wave's first step are requested right after
  // the first round of set-up loads (the parents' rows when they are all held
  // in LDS, else the first round of norm reads), straight into their operand
  // registers: they stream in during the set-up instead of after it, and the
  // wait for those loads does not wait for them (the counter retires in
  // order).  With parents read from L2 at four waves per SIMD the registers
  // do not allow it (the early keys would spill).
  constexpr bool kEarlyKeys = PL || Sh::kWavesL2 < 4;
  frag_t kf0[KS];
  auto request_first_keys = [&]() {
    const int kl = wave * KPW + ql;  // chunk-relative key of this lane
    const in_t* kp = Kb + (int64_t)(kl < nval ? cstart + kl : cstart) * D + E * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) kf0[s] = *(const frag_t*)(kp + s * 2 * E);
  };
  if constexpr (PL) {
    constexpr int NF = D / E;  // fragments per parent row
    const int nfr = M0p * NF;  // a multiple of 256: every thread owns one or more whole rounds
    // the first two rounds, both loads unconditional (a single round repeats
    // the first), so that neither is moved to its store
    const int i1 = nfr > 256 ? tid + 256 : tid;
    // (padding rows past M0 repeat row M0 - 1: their norm is +inf, never chosen)
    const frag_t pre0 = *(const frag_t*)(cbh + (int64_t)min(tid / NF, M0 - 1) * D + (tid % NF) * E);
    const frag_t pre1 = *(const frag_t*)(cbh + (int64_t)min(i1 / NF, M0 - 1) * D + (i1 % NF) * E);
    __builtin_amdgcn_sched_barrier(0);
    request_first_keys();
    __builtin_amdgcn_sched_barrier(0);
    *(frag_t*)(sPar + (tid / NF) * LDP + (tid % NF) * E) = pre0;
    *(frag_t*)(sPar + (i1 / NF) * LDP + (i1 % NF) * E) = pre1;
    for (int i = tid + 512; i < M0p * NF; i += 256) {
      const int row = i / NF, col = (i % NF) * E;
      const int src = row < M0 ? row : 0;
      *(frag_t*)(sPar + row * LDP + col) = *(const frag_t*)(cbh + (int64_t)src * D + col);
    }
  }
  for (int i = tid; i < NB; i += 256) sHist[i] = 0;
  lds_barrier();
  // 4 lanes per row (M0p * 4 is a multiple of 64, so whole waves take part);
  // rows read from L2 are requested NI at a time before any is summed, so a
  // workgroup waits for them about once per NI rows instead of once each
  constexpr int NI = PL ? 1 : (E == 8 ? 4 : 1);
  constexpr int QF = D / 4 / E;  // fragments per row quarter
  for (int i0 = tid; i0 < M0p * 4; i0 += 256 * NI) {
    frag_t v[NI][QF];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int i = i0 + 256 * n, row = min(i >> 2, M0p - 1), q = i & 3;
      const in_t* pr = PL ? sPar + row * LDP + q * (D / 4) : cbh + (int64_t)(row < M0 ? row : 0) * D + q * (D / 4);
#pragma unroll
      for (int t = 0; t < QF; ++t) v[n][t] = *(const frag_t*)(pr + t * E);
    }
    if constexpr (!PL && kEarlyKeys) {
      if (i0 == tid) {  // the first round (every thread takes part: M0p >= 64 here)
        __builtin_amdgcn_sched_barrier(0);
        request_first_keys();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int i = i0 + 256 * n, row = i >> 2, q = i & 3;
      float acc = 0.0f;
#pragma unroll
      for (int t = 0; t < QF; ++t) acc = frag_sumsq<T>(v[n][t], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      if (q == 0 && row < M0p) sNorm[row] = row < M0 ? acc : INFINITY;
    }
  }
  if constexpr (!PL && kEarlyKeys) {
    if (tid >= M0p * 4) request_first_keys();  // (a thread the loop above skipped)
  }
  lds_barrier();

  // ---- assignment, 64 keys per wave step ---------------------------------
  const int nblkP = M0p / 32;
  const int rr = r_of_row(ql), hr = h_of_row(ql);
  const int srow = 2 * (rr / W) + hr, crow = rr % W;  // slot and child of this lane's A row
  int* list = sList + wave * 64;
  float* cn = sCN + wave * 32;
  // Parents read from L2 pass through LDS 64 at a time, one copy shared by
  // the four waves (instead of each wave reading every parent from L2): each
  // wave copies its share global -> LDS; the whole pass is visible after a
  // wait and a barrier; after the pass's MFMAs a barrier frees the buffer for
  // the next pass (or the first one of the next step).  Every wave then runs
  // every step and pass, a wave past the end of the keys with all of its keys
  // masked, so that all of them reach every barrier.
  frag_t* sPS = (frag_t*)(smem + L.stage);
  const int npass = (nblkP + 1) / 2;
  auto stage_pass = [&](int ps) {
    for (int u = wave; u < 2 * KS; u += 4) {
      const int b = u / KS, s = u % KS;
      const int prow = min(ps * 64 + b * 32 + ql, M0 - 1);
      lds_dma<(int)sizeof(frag_t)>(cbh + (int64_t)prow * D + s * 2 * E + E * hh, sPS + u * 64);
    }
  };
  if constexpr (!PL) stage_pass(0);
  for (int it = 0; it < KPW; it += 64) {
    const int kloc = wave * KPW + it;  // first key of the step, chunk-relative
    if constexpr (PL) {
      if (kloc >= nval) break;
    }
    frag_t kf[2][KS];
    int key[2];
    bool kval[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      key[g] = cstart + kloc + g * 32 + ql;
      kval[g] = it + g * 32 + ql < KPW && kloc + g * 32 + ql < nval;
      if (kEarlyKeys && g == 0 && it == 0) {  // requested during the set-up
#pragma unroll
        for (int s = 0; s < KS; ++s) kf[0][s] = kf0[s];
        continue;
      }
      const in_t* kp = Kb + (int64_t)(kval[g] ? key[g] : cstart) * D + E * hh;
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[g][s] = *(const frag_t*)(kp + s * 2 * E);
    }
    // nearest parent: first minimum of ||c||^2 - 2 k.c
    float best[2] = {INFINITY, INFINITY};
    int bidx[2] = {0, 0};
    auto parent_block = [&](int blk, auto frag_at) {
      f32x16 a0 = zero16(), a1 = zero16();
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const frag_t a = frag_at(s);
        a0 = T::mma_in(a, kf[0][s], a0);
        a1 = T::mma_in(a, kf[1][s], a1);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = blk * 32 + row_of(r, hh);
        const float nrm = sNorm[row];
        const float d0 = nrm - 2.0f * a0[r];
        const float d1 = nrm - 2.0f * a1[r];
        if (d0 < best[0]) { best[0] = d0; bidx[0] = row; }
        if (d1 < best[1]) { best[1] = d1; bidx[1] = row; }
      }
    };
    if constexpr (PL) {
      for (int blk = 0; blk < nblkP; ++blk) {
        const in_t* ap = sPar + (blk * 32 + ql) * LDP + E * hh;
        parent_block(blk, [&](int s) { return *(const frag_t*)(ap + s * 2 * E); });
      }
    } else {
      // rows past M0 (norm +inf) are never chosen; they repeat row M0 - 1
      for (int ps = 0; ps < npass; ++ps) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int blk = ps * 2 + b;
          if (blk < nblkP) parent_block(blk, [&](int s) { return sPS[(b * KS + s) * 64 + lane]; });
        }
        lds_barrier();
        const int next = ps + 1 < npass ? ps + 1 : (it + 64 < KPW ? 0 : -1);
        if (next >= 0) stage_pass(next);
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float pb = xhalf_partner(best[g]);
      const int pi = xhalf_partner(bidx[g]);
      if (pb < best[g] || (pb == best[g] && pi < bidx[g])) { best[g] = pb; bidx[g] = pi; }
    }

    // distinct parents of the step, in order of first appearance (none to
    // look at when the codebook has no children)
    int idx[2] = {-1, -1};
    int n = 0;
    if (C > 0) {
      bool need0 = kval[0], need1 = kval[1];
      while (true) {
        const uint64_t b0 = __ballot(need0), b1 = __ballot(need1);
        if ((b0 | b1) == 0) break;
        const int p = b0 ? __builtin_amdgcn_readlane(bidx[0], __builtin_ctzll(b0))
                         : __builtin_amdgcn_readlane(bidx[1], __builtin_ctzll(b1));
        if (need0 && bidx[0] == p) { idx[0] = n; need0 = false; }
        if (need1 && bidx[1] == p) { idx[1] = n; need1 = false; }
        if (lane == 0) list[n] = p;
        ++n;
      }
    }
    __builtin_amdgcn_wave_barrier();

    // children of S distinct parents per MFMA block; their norms from the
    // same operand registers
    float dch[2] = {INFINITY, INFINITY};
    int cst[2] = {-1, -1};
    const int nblkC = (n + S - 1) / S;
    for (int blk = 0; blk < nblkC; ++blk) {
      const int li = blk * S + srow;
      const int prow = li < n ? list[li] : -1;
      const int crow_idx = (prow >= 0 && crow < C) ? M0 + prow * C + crow : 0;
      const in_t* cp = cbh + (int64_t)crow_idx * D + E * hh;
      frag_t a[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) a[s] = *(const frag_t*)(cp + s * 2 * E);
      float nrm = 0.0f;
#pragma unroll
      for (int s = 0; s < KS; ++s) nrm = frag_sumsq<T>(a[s], nrm);
      nrm += xhalf_partner(nrm);
      if (hh == 0) cn[ql] = nrm;
      f32x16 c0 = zero16(), c1 = zero16();
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        c0 = T::mma_in(a[s], kf[0][s], c0);
        c1 = T::mma_in(a[s], kf[1][s], c1);
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int sl = idx[g] - blk * S;
        if (sl >= 0 && sl < S && (sl & 1) == hh) {
          const int gg = sl >> 1;
          // the norms of the W rows this lane's registers gg * W .. hold: rows
          // row_of(gg * W + c, hh), four consecutive rows per quad of c, all
          // read before any is used
          float nr[W];
#pragma unroll
          for (int q = 0; q < W / 4; ++q) {
            const f32x4 n4 = *(const f32x4*)(cn + 2 * gg * W + 8 * q + 4 * hh);
#pragma unroll
            for (int u = 0; u < 4; ++u) nr[4 * q + u] = n4[u];
          }
          float dmin = INFINITY;
          int cmin = -1;
#pragma unroll
          for (int c = 0; c < W; ++c) {
            float v = g ? c1[c] : c0[c];
#pragma unroll
            for (int gi = 1; gi < 16 / W; ++gi)
              if (gg == gi) v = g ? c1[gi * W + c] : c0[gi * W + c];
            const float dist = nr[c] - 2.0f * v;
            if (c < C && dist < dmin) {  // children past C are padding rows
              dmin = dist;
              cmin = c;
            }
          }
          dch[g] = dmin;
          cst[g] = cmin;
        }
      }
      __builtin_amdgcn_wave_barrier();
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
      const int sl = moved ? 1 + cs_ : 0;
      sBin[k_ - cstart] = (unsigned short)((a_ << 5) | sl);  // sl <= C <= 16, a_ < 512
      atomicAdd(&sHist[a_ * (C + 1) + sl], 1);
      if (assign) assign[(int64_t)bh * N + k_] = moved ? M0 + a_ * C + cs_ : a_;
    }
  }

  // ---- values of this wave's keys into registers ------------------------
  // Half hh of the wave owns the KH consecutive keys from wave * KPW + hh *
  // KH; lane ql of the half holds dims EPL*ql .. EPL*ql+EPL-1 of every one of them.  Keys
  // past the end of the sequence read as zero (descriptor bound).
  constexpr int KH = KPW / 2;
  raw_t vr[KH];
  auto load_rows = [&](const in_t* src) {
    const int w0 = __builtin_amdgcn_readfirstlane(wave * KPW);
    const int nk = __builtin_amdgcn_readfirstlane(max(0, min(KPW, nval - w0)));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src + (int64_t)(cstart + w0) * D), 0, nk * D * (int)sizeof(in_t), kBufWord3);
    const int voff = (hh * KH * D + ql * EPL) * (int)sizeof(in_t);
#pragma unroll
    for (int u = 0; u < KH; ++u) vr[u] = buf_load<raw_t>(rs, voff, u * D * (int)sizeof(in_t));
  };
  load_rows(Vb);
  lds_barrier();

  // ---- slots: thread t owns parents t and t + 256 (M0 <= 512) and their C children
  constexpr int kPPT = 2;  // parents per thread
  int nz = 0, pcount[kPPT] = {0, 0};
#pragma unroll
  for (int k = 0; k < kPPT; ++k) {
    const int par = tid + 256 * k;
    if (par < M0) {
#pragma unroll 1
      for (int sl = 0; sl <= C; ++sl) {
        const int c = sHist[par * (C + 1) + sl];
        pcount[k] += c;
        nz += (sl > 0 && c > 0);
      }
      nz += pcount[k] > 0;
    }
  }
  const int incl = wave_incl_scan(nz, lane);
  if (lane == 63) sScan[wave] = incl;
  lds_barrier();
  int off = incl - nz;
  int nslots = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    off += w < wave ? sScan[w] : 0;
    nslots += sScan[w];
  }
#pragma unroll
  for (int k = 0; k < kPPT; ++k) {
    const int par = tid + 256 * k;
    if (par < M0 && pcount[k] > 0) {
      sSlot[par] = (unsigned short)off;
      sRow[off++] = (unsigned short)par;
#pragma unroll 1
      for (int sl = 1; sl <= C; ++sl) {
        if (sHist[par * (C + 1) + sl] > 0) {
          const int r = M0 + par * C + sl - 1;
          sSlot[r] = (unsigned short)off;
          sRow[off++] = (unsigned short)r;
        }
      }
    }
  }
  lds_barrier();
  // slots of every key: parent slot | child slot << 16 (0xFFFF: the key stayed)
  for (int k = tid; k < nval; k += 256) {
    const int x = sBin[k];
    const int p = x >> 5, sl = x & 31;
    const uint32_t cs = sl ? (uint32_t)sSlot[M0 + p * C + sl - 1] : 0xFFFFu;
    sKS[k] = (uint32_t)sSlot[p] | (cs << 16);
  }
  lds_barrier();

  // ---- value sums on MFMA: (one-hot of key -> slot)^T x V -------------------
  // Slots are taken 32 at a time (M = slots).  K = keys: a k-step takes E
  // keys of each half's segment (the A and B operands of lane (m/n, hh) both
  // refer to segment hh), so the registers already hold B = V with keys along
  // K, one block of N = 32 columns per value element i (dim EPL*n + i).  A
  // key contributes to the slot of its parent and, if it moved, of its child.
  // Each wave reduces its own keys; the four partial tiles meet in LDS and
  // one atomic row update per touched codeword goes to HBM.
  // With ksum the same sums are then formed for the keys (reloaded into the
  // same registers; the chunk's keys were read moments before, mostly from L2):
  // the per-codeword key sums of the codebook update (App. A, Eq. 11).
  float* tile = sAcc;  // [4 waves][32 slots][D]
  // one-hot A operand of the wave in LDS, over the bytes of its partial tile:
  // [half][k-step][slot row][E keys] (bf16 1.0 or 0; fp32 for E = 1)
  using oh_t = typename std::conditional<E == 8, unsigned short, float>::type;
  constexpr int ACC_D = Sh::ACC_D;    // columns of a partial tile per pass
  constexpr int NPASS = D / ACC_D;
  oh_t* oh = (oh_t*)(tile + wave * 32 * ACC_D);
  constexpr int OHN = 2 * KH * 32;  // entries
  auto aggregate = [&](float* dst) {
    float* vsb = dst + (int64_t)bh * Mt * D;
    for (int sb = 0; sb * 32 < nslots; ++sb) {
      // clear, then every key marks the rows of its parent and child slots
      for (int i = lane; i < OHN * (int)sizeof(oh_t) / 16; i += 64) ((u32x4*)oh)[i] = u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_wave_barrier();
      for (int kk = lane; kk < KPW; kk += 64) {
        const int kl = wave * KPW + kk;
        if (kl < nval) {
          const uint32_t x = sKS[kl];
          const int h2 = kk / KH, u = kk % KH;
          const int base = ((h2 * (KH / E) + u / E) * 32) * E + u % E;
          const oh_t one = E == 8 ? (oh_t)0x3F80 : (oh_t)1.0f;
          const int ps = (int)(x & 0xFFFFu) - 32 * sb, cs = (int)(x >> 16) - 32 * sb;
          if (ps >= 0 && ps < 32) oh[base + ps * E] = one;
          if (cs >= 0 && cs < 32) oh[base + cs * E] = one;  // 0xFFFF (stayed) is never in range
        }
      }
      __builtin_amdgcn_wave_barrier();
      f32x16 acc[EPL];
  #pragma unroll
      for (int i = 0; i < EPL; ++i) acc[i] = zero16();
  #pragma unroll
      for (int t = 0; t < KH / E; ++t) {
        const oh_t* ap = oh + ((hh * (KH / E) + t) * 32 + ql) * E;
        frag_t a;
        if constexpr (E == 8)
          a = __builtin_bit_cast(frag_t, *(const u32x4*)ap);
        else
          a = *ap;
  #pragma unroll
        for (int i = 0; i < EPL; ++i) {
          frag_t b;
          if constexpr (E == 8) {
            // element i of E consecutive keys, two bf16 per dword
            u32x4 w;
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint32_t lo, hi;
              if constexpr (EPL == 2) {
                lo = vr[8 * t + 2 * q];
                hi = vr[8 * t + 2 * q + 1];
              } else {
                lo = vr[8 * t + 2 * q][i >> 1];
                hi = vr[8 * t + 2 * q + 1][i >> 1];
              }
              w[q] = (i & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
            }
            b = __builtin_bit_cast(frag_t, w);
          } else {
            b = vr[t][i];
          }
          acc[i] = T::mma_in(a, b, acc[i]);
        }
      }
      // partial tile of this wave (over its one-hot operand): row = slot within
      // the block, col = dim; ACC_D dims per pass (lane ql holds dims EPL*ql ..)
      const int nrow = min(32, nslots - 32 * sb);
  #pragma unroll
      for (int pass = 0; pass < NPASS; ++pass) {
        if (pass > 0) lds_barrier();  // the previous pass's tiles are summed
        __builtin_amdgcn_wave_barrier();
        if (NPASS == 1 || (EPL * ql) / ACC_D == pass) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            float* tr = tile + (wave * 32 + row_of(r, hh)) * ACC_D + (EPL * ql) % ACC_D;
            if constexpr (EPL == 2) {
              *(f32x2*)tr = f32x2{acc[0][r], acc[1][r]};
            } else {
              *(f32x4*)tr = f32x4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
            }
          }
        }
        lds_barrier();
        // one row per wave instruction: consecutive lanes, consecutive floats
        for (int i = tid; i < nrow * ACC_D; i += 256) {
          const int row = i / ACC_D, c = i % ACC_D;
          float sum = tile[row * ACC_D + c];
  #pragma unroll
          for (int w = 1; w < 4; ++w) sum += tile[(w * 32 + row) * ACC_D + c];
          atomic_add_f32(vsb + (int64_t)sRow[32 * sb + row] * D + pass * ACC_D + c, sum);
        }
      }
      if ((sb + 1) * 32 < nslots) lds_barrier();  // the next block rewrites the tiles
    }
  };
  aggregate(vsum);
  if (ksum != nullptr) {
    lds_barrier();  // the last block's tiles are summed before they hold one-hot operands again
    load_rows(Kb);
    aggregate(ksum);
  }

  // ---- counts --------------------------------------------------------------
  // (from the histogram, still intact in LDS: no register stays live across
  // the aggregation for them)
  int* cnt = counts + (int64_t)bh * Mt;
#pragma unroll
  for (int k = 0; k < kPPT; ++k) {
    const int par = tid + 256 * k;
    if (par < M0) {
      int total = 0;
#pragma unroll 1
      for (int sl = 0; sl <= C; ++sl) {
        const int c = sHist[par * (C + 1) + sl];
        total += c;
        if (sl > 0 && c) atomicAdd(&cnt[M0 + par * C + sl - 1], c);
      }
      if (total) atomicAdd(&cnt[par], total);
    }
  }
}

__global__ __launch_bounds__(256) void zero_kernel(f32x4* __restrict__ a, int64_t na4, f32x4* __restrict__ a2,
                                                   int64_t na24, int* __restrict__ b, int64_t nb) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < na4; i += stride) a[i] = z;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < na24; i += stride) a2[i] = z;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nb; i += stride) b[i] = 0;
}

template <class T, int D>
static AssignLds lds_of(int M0, int C, bool parents_lds) {
  return assign_lds((int)sizeof(typename T::in_t), D, M0, C, AssignShape<T, D>::kChunk, parents_lds);
}

// Parents in LDS unless reading them from L2 at least doubles the workgroups
// that share a CU (a workgroup puts one wave on each SIMD, so waves per SIMD
// = workgroups); the L2 reads cost more than one extra workgroup gains.
template <class T, int D>
static bool parents_in_lds(int M0, int C) {
  constexpr size_t kLdsPerCu = 160 * 1024;
  using Sh = AssignShape<T, D>;
  const size_t lp = lds_of<T, D>(M0, C, true).total, lg = lds_of<T, D>(M0, C, false).total;
  const size_t wp = std::min<size_t>(kLdsPerCu / lp, Sh::kWavesLds);
  const size_t wg = std::min<size_t>(kLdsPerCu / lg, Sh::kWavesL2);
  return wg < 2 * wp;
}

template <class T, int D>
static size_t smem_of(int M0, int C) {
  return lds_of<T, D>(M0, C, parents_in_lds<T, D>(M0, C)).total;
}

size_t assign_smem_bytes(int dtype, int d, int M0, int C) {
  if (dtype == 0) return d == 64 ? smem_of<TF32, 64>(M0, C) : smem_of<TF32, 128>(M0, C);
  return d == 64 ? smem_of<TBF16, 64>(M0, C) : smem_of<TBF16, 128>(M0, C);
}

template <class T, int D, int W, bool PL>
static hipError_t launch_assign_t(const void* K, const void* V, const void* cb, int BH, int H, int N, int M0, int C,
                                  float* vsum, int* counts, int* assign, float* ksum, hipStream_t st) {
  using Sh = AssignShape<T, D>;
  const AssignLds L = lds_of<T, D>(M0, C, PL);
  auto kern = assign_aggregate_kernel<T, D, W, PL>;
  hipError_t e = raise_lds_limit((const void*)kern, L.total);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)(((N + Sh::kChunk - 1) / Sh::kChunk) * BH));
  hipLaunchKernelGGL(kern, grid, dim3(256), L.total, st, (const typename T::in_t*)K, (const typename T::in_t*)V,
                     (const typename T::in_t*)cb, H, N, M0, C, L, vsum, counts, assign, ksum);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_assign_w(const void* K, const void* V, const void* cb, int BH, int H, int N, int M0, int C,
                                  float* vsum, int* counts, int* assign, float* ksum, hipStream_t st) {
  if (parents_in_lds<T, D>(M0, C)) {
    if (C <= 4) return launch_assign_t<T, D, 4, true>(K, V, cb, BH, H, N, M0, C, vsum, counts, assign, ksum, st);
    if (C <= 8) return launch_assign_t<T, D, 8, true>(K, V, cb, BH, H, N, M0, C, vsum, counts, assign, ksum, st);
    return launch_assign_t<T, D, 16, true>(K, V, cb, BH, H, N, M0, C, vsum, counts, assign, ksum, st);
  }
  if (C <= 4) return launch_assign_t<T, D, 4, false>(K, V, cb, BH, H, N, M0, C, vsum, counts, assign, ksum, st);
  if (C <= 8) return launch_assign_t<T, D, 8, false>(K, V, cb, BH, H, N, M0, C, vsum, counts, assign, ksum, st);
  return launch_assign_t<T, D, 16, false>(K, V, cb, BH, H, N, M0, C, vsum, counts, assign, ksum, st);
}

hipError_t launch_zero(float* vsum, int64_t nv, float* ksum, int64_t nk, int* counts, int64_t nc, hipStream_t st) {
  const int64_t work = std::max(std::max(nv / 4, nk / 4), nc);
  int64_t blocks = (work + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (f32x4*)vsum, nv / 4, (f32x4*)ksum, nk / 4,
                     counts, nc);
  return hipGetLastError();
}

hipError_t launch_assign(int dtype, const void* K, const void* V, const void* cb, int BH, int H, int N, int d, int M0,
                         int C, float* vsum, int* counts, int* assign, float* ksum, hipStream_t st) {
  if (dtype == 0) {
    if (d == 64) return launch_assign_w<TF32, 64>(K, V, cb, BH, H, N, M0, C, vsum, counts, assign, ksum, st);
    return launch_assign_w<TF32, 128>(K, V, cb, BH, H, N, M0, C, vsum, counts, assign, ksum, st);
  }
  if (d == 64) return launch_assign_w<TBF16, 64>(K, V, cb, BH, H, N, M0, C, vsum, counts, assign, ksum, st);
  return launch_assign_w<TBF16, 128>(K, V, cb, BH, H, N, M0, C, vsum, counts, assign, ksum, st);
}

}  // namespace avq
