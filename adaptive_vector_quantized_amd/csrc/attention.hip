// Kernel 2 of the AVQ-Attention forward pass: count-weighted attention over
// the parent codewords, per-tile importance, top-P selection and the child
// correction ("AVQ-Attention: Adaptive Vector-Quantized Attention",
// Sec. 4.3 and Algorithm 2; Eq. 6-9; Sec. C and D).
//
// Two launches on the caller's stream:
//
//  1. attention_prep_kernel, once per (batch, head): the value sums are
//     scaled by one power of two per (batch, head) (so that the largest
//     magnitude lands in [2^14, 2^15) and fp16 keeps 11 significant bits of
//     every value without overflow) and written to the workspace as fp16
//     MFMA operand fragments, in exactly the order the attention kernel keeps
//     them in LDS.  fp32 inputs keep fp32 values (scale 1).
//
//  2. attention_kernel.  A workgroup owns a contiguous range of query tiles
//     of one (batch, head); one wave handles 32 queries of a tile.  The
//     parents' codeword and value fragments are copied into LDS once per
//     workgroup (up to 64 parents; beyond, the codewords pass through a
//     64-parent LDS buffer shared by the workgroup's waves, and the value
//     fragments are read from L2 at d = 128 and at d = 64 beyond 256
//     parents); per tile, the selected
//     parents' children are copied into LDS by asynchronous buffer loads (no
//     registers held, one wait).  The output goes out in streaming stores.
//
// Per tile.  Logits are computed transposed on MFMA (rows = codewords,
// columns = queries): each lane owns one query and 16 codewords per 32-row
// block, so the stabiliser, the denominator and the rescaling are per-lane
// scalars, the parent logit of Eq. 8 is a sum over registers of one lane, and
// the weights feed the weighted-value MFMA as its B operand in place.  The
// importance of Eq. 7 is reduced over the 32 query lanes by a butterfly
// reduce-scatter (permlane16 swap and DPP mirrors), then over the waves in
// LDS; every wave ranks the parents itself, so the selection needs no second
// barrier.
//
// The stabiliser follows Eq. 18 (max over non-empty codewords) but is only
// raised when a new maximum exceeds it by more than 2^8: weights then stay in
// [-2^8, 2^8], exactly representable ranges for the fp16 operand, and most
// rescaling of the accumulators is skipped.  Empty codewords get logit -inf
// (weight exactly 0), and a selected parent without keys gets a bounded
// recovered weight, so no inf * 0 can arise (Sec. D).
//
// Children of a selected parent occupy W (8 or 16) consecutive accumulator
// registers of one lane half, so S = 32 / W parents share a 32-row block.
#include <algorithm>
#include <atomic>
#include <cfloat>

#include "avq_device.h"
#include "avq_launch.h"

namespace avq {

namespace {

template <class T, int OFF>
__device__ __forceinline__ typename T::pvfrag_t pack_at(const f32x16& v) {
  if constexpr (T::E == 8) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = v[OFF + j];
    return T::pack_pv(x);
  } else {
    return v[OFF];
  }
}

template <class T, int KV>
__device__ __forceinline__ typename T::pvfrag_t pv_operand(const f32x16& v, int k) {
  if constexpr (KV == 2) {
    return k == 0 ? pack_at<T, 0>(v) : pack_at<T, 8>(v);
  } else {
    return v[k];
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// power of two sigma with max / sigma in [2^14, 2^15)
__device__ __forceinline__ float value_scale(float mx) {
  if (!(mx > 0.0f)) return 1.0f;
  int e;
  frexpf(mx, &e);
  return ldexpf(1.0f, e - 15);
}

__device__ __forceinline__ float absmax4(f32x4 v) {
  return fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
}

// parent index of value column c (columns are in accumulator-register order)
__device__ __forceinline__ int parent_of_col(int c) {
  const int q = c & 31;
  return 32 * (c >> 5) + row_of(r_of_col(q), h_of_col(q));
}

// lds_dma (avq_device.h) through a buffer descriptor (base and size in scalar
// registers, a 32-bit byte offset per lane): a fragment at or past the
// descriptor's size reads as zeros.
constexpr int kBufWord3 = 0x00020000;     // word 3 of a raw gfx9-family descriptor
constexpr int kOutOfRange = 0x7FFFFFF0;   // a byte offset past any descriptor here
template <int BYTES>
__device__ __forceinline__ void lds_dma_buf(__amdgpu_buffer_rsrc_t rs, int voff, void* lds_base) {
  static_assert(BYTES == 16 || BYTES == 4, "fragment size");
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_base, 4, voff, 0, 0, 0);
}

// Zero fill of the caller's value sums and counts by the attention kernel,
// spread over its whole grid (plain stores): once the preparation has run,
// the kernel reads neither, and the next accumulating assignment call adds
// into them.
__device__ __forceinline__ void clear_buffers(float* v, int64_t n4, int* c, int64_t nc) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v != nullptr)
    for (int64_t i = t; i < n4; i += stride) ((f32x4*)v)[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (c != nullptr)
    for (int64_t i = t; i < nc; i += stride) c[i] = 0;
}

// Top-P of Alg. 2 over the importances one wave holds (parent j = 64 g + lane
// in u[g]; non-negative floats as bit patterns, so integer order is value
// order).  A radix search on the bits, from the top, raises a threshold thr
// while at least P values reach it; it stops early once exactly P do (they
// are then the answer), else it ends at the P-th largest value.  The chosen
// set is everything above thr plus the lowest-index parents equal to it (the
// tie rule of the oracle), written ascending to out[0..P).
template <int NG>
__device__ __forceinline__ void select_top(const uint32_t (&u)[NG], int M0, int P, int lane, int* out, int* gout) {
  uint32_t thr = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int g = 0; g < NG; ++g) cnt += __popcll(__ballot(u[g] >= cand));
    thr = cnt >= P ? cand : thr;
    if (cnt == P) break;
  }
  int above = 0;
#pragma unroll
  for (int g = 0; g < NG; ++g) above += __popcll(__ballot(u[g] > thr));
  const uint64_t below_me = (1ull << lane) - 1ull;
  int eq_before = 0, before = 0;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const bool valid = g * 64 + lane < M0;
    const bool eq = valid && u[g] == thr;
    const uint64_t meq = __ballot(eq);
    const bool sel = (valid && u[g] > thr) || (eq && eq_before + __popcll(meq & below_me) < P - above);
    const uint64_t msk = __ballot(sel);
    if (sel) {
      const int pos = before + __popcll(msk & below_me);
      out[pos] = g * 64 + lane;
      if (gout) gout[pos] = g * 64 + lane;
    }
    before += __popcll(msk);
    eq_before += __popcll(meq);
  }
}

}  // namespace

// ---- workspace layout ---------------------------------------------------------
// [0, align256(4*BH))         scale sigma of every (batch, head)
// then per (batch, head), align256(bytes) each:
//   parent value fragments    (M0p/32 blocks) x [KV][2][D] fragments
//   child value fragments     M0 parents x [W/E][D] fragments
// A fragment is E consecutive operand elements (8 fp16, or 1 fp32).
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
constexpr int kYRow = 36;  // floats per staged output row (32 dims + 4 to spread LDS banks)

// Workspace: [BH] value scales | [BH] value operand fragments | [BH][slices]
// partial maxima of |vsum| (one per slice of kMaxSlice4 float4 of a head's
// value sums) | [BH][Mt] a copy of the counts (the attention kernel reads
// the counts from here, so that the caller's counts are free once the
// preparation has run).
constexpr int kMaxThreads = 256;               // threads of the partial-maximum kernel
constexpr int kMaxPer = 4;                     // float4 loads per thread
constexpr int kMaxSlice4 = kMaxThreads * kMaxPer;
struct AttnWs {
  size_t sig_bytes, per_bh, pmax_off, counts_off, total;
  int slices;
};
static AttnWs attn_ws(int dtype, int d, int M0, int C, int BH) {
  AttnWs w;
  const size_t pes = dtype == 0 ? 4 : 2;
  const size_t M0p = attn_parent_rows(M0);
  const size_t W = C == 0 ? 0 : C <= 8 ? 8 : 16;  // a flat codebook has no child fragments
  const size_t n4 = (size_t)M0 * (1 + C) * d / 4;
  w.sig_bytes = align256((size_t)BH * 4);
  w.per_bh = align256((M0p * d + (size_t)M0 * W * d) * pes);
  w.slices = (int)((n4 + kMaxSlice4 - 1) / kMaxSlice4);
  w.pmax_off = w.sig_bytes + (size_t)BH * w.per_bh;
  w.counts_off = w.pmax_off + align256((size_t)BH * w.slices * 4);
  w.total = w.counts_off + align256((size_t)BH * M0 * (1 + C) * 4);
  return w;
}

size_t attention_workspace_bytes(int dtype, int d, int M0, int C, int BH) { return attn_ws(dtype, d, M0, C, BH).total; }

// Prep: attention_prep_kernel, one round of loads per thread; every block of
// a (batch, head) issues the gathers of its own fragments (at most kPrepFrag
// per thread), forms the head's maximum |value sum|, then scales, packs and
// stores.  For a small head every block forms the maximum itself from the
// head's value sums (a few hundred KB, read from L2): one launch, no wait
// between blocks.  For a large head, where those repeated reads would cost
// more than a launch, attention_absmax_kernel first takes the maximum of each
// slice of kMaxSlice4 float4 (every value sum read once) and the blocks then
// combine the slices' maxima.
constexpr int kPrepThreads = 512;
constexpr int kPrepFrag = 2;   // fragments per thread
constexpr int kPrepMax = 18;   // f32x4 loads in flight per thread for the maximum
constexpr size_t kPrepRepeatBytes = 8u << 20;  // repeated reads of one head's sums beyond which the maximum is split

__global__ __launch_bounds__(kMaxThreads) void attention_absmax_kernel(const float* __restrict__ vsum, int n4,
                                                                       int slices, float* __restrict__ pmax) {
  __shared__ float red[kMaxThreads / 64];
  const int bh = blockIdx.x / slices, sl = blockIdx.x % slices;
  const f32x4* v = (const f32x4*)vsum + (int64_t)bh * n4;
  const int tid = threadIdx.x;
  f32x4 x[kMaxPer];
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) {
    const int i = sl * kMaxSlice4 + u * kMaxThreads + tid;
    x[u] = i < n4 ? v[i] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  float mx = 0.0f;
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) mx = fmaxf(mx, absmax4(x[u]));
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int w = 1; w < kMaxThreads / 64; ++w) mx = fmaxf(mx, red[w]);
    pmax[blockIdx.x] = mx;
  }
}

template <class T, int D, int W>
__global__ __launch_bounds__(kPrepThreads) void attention_prep_kernel(const float* __restrict__ vsum,
                                                                      const int* __restrict__ counts, int BH, int M0,
                                                                      int C, int parts, unsigned char* __restrict__ ws,
                                                                      size_t sig_bytes, size_t per_bh,
                                                                      const float* __restrict__ pmax, int slices,
                                                                      int* __restrict__ counts_copy) {
  using pvfrag_t = typename T::pvfrag_t;
  constexpr int E = T::E;
  constexpr int KV = 16 / E;
  constexpr int NWV = kPrepThreads / 64;
  __shared__ float red[NWV];
  // the blocks of one (batch, head) on one XCD when possible (consecutive
  // block ids go to the XCDs round robin): the head's sums are then read from
  // HBM once and from that XCD's L2 afterwards
  int bh, part;
  {
    const int L = blockIdx.x;
    if ((BH & 7) == 0) {
      bh = (L / (8 * parts)) * 8 + (L & 7);
      part = (L >> 3) % parts;
    } else {
      bh = L / parts;
      part = L % parts;
    }
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Mt = M0 * (1 + C);
  const int M0p = attn_parent_rows(M0);
  const float* vs = vsum + (int64_t)bh * Mt * D;
  // this block's share of the head's counts, copied for the attention kernel
  for (int i = part * kPrepThreads + tid; i < Mt; i += parts * kPrepThreads)
    counts_copy[(int64_t)bh * Mt + i] = counts[(int64_t)bh * Mt + i];
  const int nP = (M0p / 32) * KV * 2 * D;           // parent fragments
  const int nF = nP + (C > 0 ? M0 * (W / E) * D : 0);  // + child fragments
  // gathers of this thread's fragments (unscaled)
  float x[kPrepFrag][E];
#pragma unroll
  for (int k = 0; k < kPrepFrag; ++k) {
    const int f = (k * parts + part) * kPrepThreads + tid;
    if (f < nP) {
      const int d = f % D, t = f / D;
      const int hh = t % 2, bk = t / 2, kk = bk % KV, b = bk / KV;
      const int c0 = b * 32 + 16 * ((kk * E) >> 3) + 8 * hh + ((kk * E) & 7);
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int p = parent_of_col(c0 + j);
        x[k][j] = p < M0 ? vs[(int64_t)p * D + d] : 0.0f;
      }
    } else if (f < nF) {
      const int g2 = f - nP;
      const int d = g2 % D, t = g2 / D;
      const int g = t % (W / E), p = t / (W / E);
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int c = g * E + j;
        x[k][j] = c < C ? vs[(int64_t)(M0 + p * C + c) * D + d] : 0.0f;
      }
    }
  }
  float sig = 1.0f;
  if constexpr (T::kScaleValues) {
    float mx = 0.0f;
    if (pmax != nullptr) {
      for (int i = tid; i < slices; i += kPrepThreads) mx = fmaxf(mx, pmax[(int64_t)bh * slices + i]);
    } else {
      const int n4 = Mt * (D / 4);
      for (int i0 = tid; i0 < n4; i0 += kPrepThreads * kPrepMax) {
        f32x4 v[kPrepMax];
#pragma unroll
        for (int u = 0; u < kPrepMax; ++u) {
          const int i = i0 + u * kPrepThreads;
          v[u] = ((const f32x4*)vs)[i < n4 ? i : 0];
        }
#pragma unroll
        for (int u = 0; u < kPrepMax; ++u) mx = fmaxf(mx, absmax4(v[u]));
      }
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NWV; ++w) mx = fmaxf(mx, red[w]);
    sig = value_scale(mx);
  }
  if (part == 0 && tid == 0) ((float*)ws)[bh] = sig;
  const float inv = 1.0f / sig;
  pvfrag_t* pf = (pvfrag_t*)(ws + sig_bytes + (size_t)bh * per_bh);
#pragma unroll
  for (int k = 0; k < kPrepFrag; ++k) {
    const int f = (k * parts + part) * kPrepThreads + tid;
    if (f < nF) {
#pragma unroll
      for (int j = 0; j < E; ++j) x[k][j] *= inv;
      pf[f] = T::pack_pv(x[k]);
    }
  }
}

// PL: the parents' codewords are all held in LDS (M0 <= 64); else they pass
// through a one-pass (64-parent) LDS buffer that the workgroup's waves share.
// VL: the parents' value fragments are held in LDS (d = 64 up to 256
// parents); else they are read from L2 at their MFMAs (at d = 128 beyond 64
// parents and at d = 64 beyond 256, where the LDS then holds two workgroups)
template <class T, int D, int W, bool PL, bool VL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attention_kernel(
    const typename T::in_t* __restrict__ Q, const typename T::in_t* __restrict__ cb, const int* __restrict__ counts,
    const unsigned char* __restrict__ ws, size_t sig_bytes, size_t per_bh, int H, int BH, int N, int M0, int C, int P,
    int bq, int tiles_per_wg, int wgs_per_bh, float sl2, float* __restrict__ Y, int* __restrict__ topp,
    float* __restrict__ importance, int approx, const int* __restrict__ order, float* __restrict__ clear_v,
    int64_t clear_v4, int* __restrict__ clear_c, int64_t clear_nc) {
  using in_t = typename T::in_t;
  using frag_t = typename T::frag_t;
  using pvfrag_t = typename T::pvfrag_t;
  constexpr int E = T::E;
  constexpr int KS = D / (2 * E);   // logit k-steps over the head dimension
  constexpr int DB = D / 32;        // 32-row blocks of the output dimension
  constexpr int S = 32 / W;         // parents per 32-row child block
  constexpr int KV = 16 / E;        // weighted-value k-steps per 32-row block
  constexpr int CH = AttnTraits<D>::kChunkRows;
  constexpr int NCB = CH / 32;
  constexpr int FA = KS * 64;       // codeword fragments per 32-row block
  constexpr int FV = KV * 2 * D;    // value fragments per 32-codeword block
  constexpr int BA = (int)sizeof(frag_t);
  constexpr int BV = (int)sizeof(pvfrag_t);
  constexpr float kLazy = 8.0f;

  extern __shared__ __align__(16) unsigned char smem[];
  const int nthreads = blockDim.x;
  const int nw = nthreads >> 6;
  const int Mt = M0 * (1 + C);
  const int M0p = attn_parent_rows(M0);
  const int nblkP = M0p / 32;
  const int Pp = P > 0 ? P : 1;
  constexpr bool parents_lds = PL;
  constexpr bool values_lds = VL;
  frag_t* sPC = (frag_t*)smem;                                        // [nblkP*FA] if parents_lds, else one pass [2*FA]
  pvfrag_t* sPV = (pvfrag_t*)(sPC + (parents_lds ? nblkP * FA : 2 * FA));  // [nblkP*FV] if values_lds
  // the children's arrays exist only when P > 0, the importance partials only
  // when importances are formed
  const bool need_imp = (P > 0) || (importance != nullptr);
  const int nCH = P > 0 ? CH : 0;
  // the chunk buffers exist with children, and also without them when the
  // parents' value fragments are not held in LDS (they then carry the staged
  // passes' values)
  const int nCBbuf = (P > 0 || !values_lds) ? NCB : 0;
  frag_t* sCC = (frag_t*)(sPV + (values_lds ? nblkP * FV : 0));       // [NCB*FA]
  pvfrag_t* sCV = (pvfrag_t*)(sCC + nCBbuf * FA);                     // [NCB*FV]
  float* sNp = (float*)(sCV + nCBbuf * FV);                           // [M0p] counts
  float* sNc = sNp + M0p;                                             // [CH]
  float* sBp = sNc + nCH;                                             // [M0p] 0 or -inf (empty)
  float* sBc = sBp + M0p;                                             // [CH]
  float* sW = sBc + nCH;                                              // [M0p][4] partials per wave
  int* sSel = (int*)(sW + (need_imp ? M0p * 4 : 0));                  // [nw][Pp]
  int* sFlag = sSel + nw * Pp;                                        // [2] all parents hold keys; chunk needs masks
  float* sPass = (float*)(sFlag + 2);                                 // [8] keys of the parents of each 64-parent pass
  float* sY = (float*)(smem + ((((unsigned char*)(sFlag + 12) - smem) + 15) & ~15));  // [nw][32][kYRow] output staging

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, hh = lane >> 5;
  // Workgroups of one (batch, head) on one XCD when possible (consecutive
  // workgroup ids go to the XCDs round robin): its data then lives in one L2.
  int bh, g;
  {
    const int L = blockIdx.x;
    if ((BH & 7) == 0) {
      const int k = L >> 3;
      bh = (k / wgs_per_bh) * 8 + (L & 7);
      g = k % wgs_per_bh;
    } else {
      bh = L / wgs_per_bh;
      g = L % wgs_per_bh;
    }
  }
  // this workgroup's share of the requested zero fill, first (measured: it
  // costs least issued before anything else)
  clear_buffers(clear_v, clear_v4, clear_c, clear_nc);
  const int h = bh % H;
  const int ntiles = (N + bq - 1) / bq;
  const int tile0 = g * tiles_per_wg;
  const int tile1 = min(ntiles, tile0 + tiles_per_wg);
  if (tile0 >= tile1) return;
  const in_t* cbh = cb + (int64_t)h * Mt * D;
  const int* nb = counts + (int64_t)bh * Mt;
  const in_t* Qb = Q + (int64_t)bh * N * D;
  float* Yb = Y + (int64_t)bh * N * D;
  const float sig = ((const float*)ws)[bh];
  const pvfrag_t* pvf = (const pvfrag_t*)(ws + sig_bytes + (size_t)bh * per_bh);
  const pvfrag_t* cvf = pvf + nblkP * FV;
  // descriptors of the head's codebook and of the child value fragments
  const __amdgpu_buffer_rsrc_t cb_rs = __builtin_amdgcn_make_buffer_rsrc((void*)cbh, 0, Mt * D * (int)sizeof(in_t), kBufWord3);
  const __amdgpu_buffer_rsrc_t cv_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)cvf, 0, C > 0 ? M0 * (W / E) * D * BV : 0, kBufWord3);
  const int nPT = (M0 + 63) / 64;

  // ---- once per workgroup: parents into LDS -----------------------------------
  if constexpr (parents_lds) {
    for (int u = wave; u < nblkP * KS; u += nw) {
      const int b = u / KS, s = u % KS;
      const int j = b * 32 + ql;
      lds_dma<BA>(cbh + (int64_t)(j < M0 ? j : 0) * D + s * 2 * E + E * hh, sPC + u * 64);
    }
  }
  if constexpr (values_lds)
    for (int u = wave; u < nblkP * FV / 64; u += nw) lds_dma<BV>(pvf + u * 64 + lane, sPV + u * 64);
  if (tid == 0) sFlag[0] = 1;
  // importance partials: slots of absent waves (and of parents past M0) stay zero
  if (need_imp)
    for (int i = tid; i < M0p * 4; i += nthreads) sW[i] = 0.0f;
  __syncthreads();
  for (int c = tid; c < M0p; c += nthreads) {  // a wave covers the 64 columns of one pass
    const int j = parent_of_col(c);
    const float n = j < M0 ? (float)nb[j] : 0.0f;
    sNp[c] = n;
    sBp[c] = n > 0.0f ? 0.0f : -INFINITY;
    if (j < M0 && !(n > 0.0f)) sFlag[0] = 0;
    if (approx) {
      const float tot = wave_sum(n);
      if (lane == 0) sPass[(c - lane) / 64] = tot;
    }
  }
  // Token row of the query at tile position pos, -1 for none: the position
  // itself, or with a query order the row it names (a name outside [0, N)
  // makes the position empty, like the positions past N of the last tile).
  // The order entries are fetched one tile ahead of the query loads that use
  // them, so that those loads never wait for them.
  auto order_at = [&](int pos) -> int { return (order != nullptr && pos < N) ? order[pos] : pos; };
  auto query_row = [&](int pos, int entry) -> int {
    if (pos >= N) return -1;
    if (order == nullptr) return pos;
    return (entry >= 0 && entry < N) ? entry : -1;
  };
  const int qpos0 = tile0 * bq + wave * 32 + ql;
  frag_t qf[KS];
  int qrow = query_row(qpos0, order_at(qpos0));
  int entry_n = order_at(qpos0 + bq);  // the order entry of this lane's query in the next tile
  {
    const in_t* qp = Qb + (int64_t)(qrow >= 0 ? qrow : 0) * D + E * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *(const frag_t*)(qp + s * 2 * E);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const bool all_parents = sFlag[0] != 0;

  // Output staging: a wave's 32 rows x 32 dims in LDS, written out by
  // store_rows with eight whole 128-byte row segments per store instruction,
  // as streaming (non-temporal) stores: the output is never read back here,
  // and keeping it out of L2 leaves L2 to the codewords and value fragments.
  float* yw = sY + wave * 32 * kYRow;
  auto store_rows = [&](int q0, int db, int row) {
    __builtin_amdgcn_wave_barrier();
    const int r0 = lane >> 3, c4 = (lane & 7) * 4;
    const float* src = yw + r0 * kYRow + c4;
    if (order != nullptr) {
      // rows scattered by the query order: each 8-lane group still writes one
      // whole 128-byte segment of its row; lane r of the wave holds the row of
      // the wave's r-th query
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = __shfl(row, r0 + 8 * k);
        if (r >= 0)
          __builtin_nontemporal_store(*(const f32x4*)(src + 8 * k * kYRow), (f32x4*)(Yb + (int64_t)r * D + db * 32 + c4));
      }
      return;
    }
    float* dst = Yb + (int64_t)(q0 + r0) * D + db * 32 + c4;
    if (q0 + 32 <= N) {
#pragma unroll
      for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(*(const f32x4*)(src + 8 * k * kYRow), (f32x4*)(dst + 8 * k * D));
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (q0 + r0 + 8 * k < N)
          __builtin_nontemporal_store(*(const f32x4*)(src + 8 * k * kYRow), (f32x4*)(dst + 8 * k * D));
    }
  };

  // One pass of 64 parents' codeword fragments in LDS when they are not all
  // held there: every wave copies its share (global -> LDS, no registers);
  // wait_pass makes the whole pass visible, release_pass (after the pass's
  // logits) lets the buffer be refilled -- with the next pass, or the first
  // pass again for the second (importance) pass or the next tile -- while
  // the rest of the pass runs.
  auto stage_pass = [&](int pt2) {
    for (int u = wave; u < 2 * KS; u += nw) {
      const int b = u / KS, s = u % KS;
      const int j = pt2 * 64 + b * 32 + ql;
      lds_dma<BA>(cbh + (int64_t)(j < M0 ? j : 0) * D + s * 2 * E + E * hh, sPC + u * 64);
    }
  };
  auto wait_pass = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  auto release_pass = [&](int next) {
    lds_barrier();
    if (next >= 0) stage_pass(next);
  };
  if constexpr (!parents_lds) stage_pass(0);
  // Parents' value fragments that are not held in LDS: the first pass's value
  // products read them from the two chunk buffers (idle until the children,
  // each exactly one 64-parent pass of value fragments in size), shared by
  // the workgroup's waves, instead of every wave reading them from L2.  Pass pt uses buffer pt % 2; the copy
  // of pass pt + 1 is issued right after pass pt's opening barrier (every
  // wave is then done with pass pt - 1, the buffer's last user) and waited
  // for by pass pt + 1's opening wait and barrier; only pass 0's own copy
  // needs a wait of its own.
  constexpr bool vstage = !values_lds;
  pvfrag_t* const vbuf[2] = {sCV, (pvfrag_t*)sCC};
  auto stage_values = [&](int pt2) {
    pvfrag_t* dst = vbuf[pt2 & 1];
    for (int u = wave; u < 2 * FV / 64; u += nw) lds_dma<BV>(pvf + pt2 * 2 * FV + u * 64 + lane, dst + u * 64);
  };

  // ---- query tiles ------------------------------------------------------------
  for (int tile = tile0; tile < tile1; ++tile) {
    const bool qv = qrow >= 0;
    // the next tile's queries, a whole tile ahead of their use (d = 64; at
    // d = 128 they are loaded at the end of the tile, saving registers)
    constexpr bool kEarlyQ = D == 64;
    frag_t qn[KS];
    int qrow_n = -1;
    auto load_next_q = [&]() {
      const int pos = (tile + 1) * bq + wave * 32 + ql;
      qrow_n = query_row(pos, entry_n);
      const in_t* qp = Qb + (int64_t)(qrow_n >= 0 ? qrow_n : 0) * D + E * hh;
#pragma unroll
      for (int s = 0; s < KS; ++s) qn[s] = *(const frag_t*)(qp + s * 2 * E);
      entry_n = order_at(pos + bq);
    };
    if constexpr (kEarlyQ) load_next_q();

    f32x16 xacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) xacc[db] = zero16();
    float zp = 0.0f;  // denominator over this lane half's codewords
    // stabiliser of the scaled (log2-domain) logits; finite from the start so
    // that an all-empty pass (logits -inf) gives weights exp2(-inf) = 0 and the
    // first real maximum rescales the (zero) accumulators by exp2(-huge) = 0
    float m = -FLT_MAX;
    f32x16 lg[2];

    // parents (Alg. 2, the pass over the parent codewords), 64 per pass (the padding rows past M0 have
    // count 0 and logit -inf); parents not all held in LDS pass through a
    // one-pass LDS buffer shared by the workgroup's waves (staged_pass)
    const bool second_pass = need_imp && !approx && !parents_lds;
    for (int pt = 0; pt < nPT; ++pt) {
      const int j0 = pt * 64;
      if constexpr (!parents_lds) wait_pass();
      if (vstage) {
        if (pt == 0) stage_values(0);
        if (pt + 1 < nPT) stage_values(pt + 1);
      }
      // empty parents and padding rows (count 0) get logit -inf: their bias
      // enters as the initial value of the accumulator (zero when every
      // parent of the pass holds keys)
      const bool pass_masked = !all_parents || j0 + 64 > M0;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int bb = parents_lds ? pt * 2 + b : b;
        lg[b] = zero16();
        if (pass_masked) {
          const f32x4* bp = (const f32x4*)(sBp + j0 + b * 32 + 8 * hh);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 b4 = bp[(q >> 1) * 4 + (q & 1)];
#pragma unroll
            for (int u = 0; u < 4; ++u) lg[b][q * 4 + u] = b4[u];
          }
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) lg[b] = T::mma_in(sPC[(bb * KS + s) * 64 + lane], qf[s], lg[b]);
      }
      if constexpr (!parents_lds)
        release_pass(pt + 1 < nPT ? pt + 1 : (second_pass || tile + 1 < tile1) ? 0 : -1);
      float tm = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) tm = fmaxf(tm, lg[b][r]);
      tm = xhalf_max(tm) * sl2;
      if (tm > m + kLazy) {
        if (pt > 0) {  // (the first pass finds the accumulators still zero)
          const float f = fast_exp2(m - tm);
          zp *= f;
#pragma unroll
          for (int db = 0; db < DB; ++db) xacc[db] *= f;
        }
        m = tm;
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const f32x4* np4 = (const f32x4*)(sNp + j0 + b * 32 + 8 * hh);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 n4 = np4[(q >> 1) * 4 + (q & 1)];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float a = fast_exp2(fmaf(lg[b][q * 4 + u], sl2, -m));
            lg[b][q * 4 + u] = a;
            zp = fmaf(a, n4[u], zp);
          }
        }
      }
      if (vstage && pt == 0) {  // pass 0's value fragments have landed
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      const pvfrag_t* vsrc = vstage ? vbuf[pt & 1] : values_lds ? sPV + pt * 2 * FV : pvf + pt * 2 * FV;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int k = 0; k < KV; ++k) {
          const pvfrag_t bf = pv_operand<T, KV>(lg[b], k);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            xacc[db] = T::mma_pv(vsrc[((b * KV + k) * 2 + hh) * D + ql + 32 * db], bf, xacc[db]);
        }
      }
      if constexpr (!parents_lds) {
        if (approx && need_imp) {
          // App. B, Eq. 13-14: this pass's importances with the extrapolated
          // denominator N / N_seen * (the part of Z formed so far), from the
          // weights still in registers; no second pass over the parents
          float nseen = 0.0f, ntot = 0.0f;
          for (int p2 = 0; p2 < nPT; ++p2) {
            const float c = sPass[p2];
            ntot += c;
            if (p2 <= pt) nseen += c;
          }
          const float zs = xhalf_sum(zp);
          const float rz = (qv && nseen > 0.0f) ? nseen / (ntot * zs) : 0.0f;
          float t[32];
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) t[b * 16 + r] = lg[b][r] * rz;
          rs_half32(t, lane);
          const int j = j0 + 32 * (ql >> 4) + row_of(ql & 15, hh);
          if (j < M0) sW[j * 4 + wave] = t[0] * sNp[j0 + 32 * (ql >> 4) + col_of(ql & 15, hh)];
        }
      }
    }

    // importance (Eq. 7) and top-P (Alg. 2, the parent choice)
    if (need_imp) {
      const float rz = qv ? 1.0f / xhalf_sum(zp) : 0.0f;
      if constexpr (parents_lds) {
        // one pass (M0 <= 64): its weights are still in registers; the count
        // n_j of Eq. 7 is a factor of the whole sum over the tile's queries,
        // applied once after the reduction
        float t[32];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) t[b * 16 + r] = lg[b][r] * rz;
        rs_half32(t, lane);
        const int j = 32 * (ql >> 4) + row_of(ql & 15, hh);
        if (j < M0) sW[j * 4 + wave] = t[0] * sNp[32 * (ql >> 4) + col_of(ql & 15, hh)];
      } else if (!approx) {
        // Second pass over the parents with the final stabiliser and
        // denominator (the exact Z of Eq. 7).  Its logits are formed
        // untransposed (the MFMA operands swapped: rows = this wave's queries,
        // columns = parents), so that a lane holds one parent for 16 queries
        // and the sum over the wave's queries is a sum over its registers and
        // the two lane halves.  Each register's query (row row_of(r, hh))
        // brings its stabiliser and 1/z, read once per tile from a table of
        // the wave's 32 queries in its own output-staging rows (idle until the
        // output).
        if (hh == 0) {
          yw[ql] = m;
          yw[32 + ql] = rz;
        }
        float mr[16], rr[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 a = *(const f32x4*)(yw + 8 * q + 4 * hh);
          const f32x4 c = *(const f32x4*)(yw + 32 + 8 * q + 4 * hh);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            mr[4 * q + u] = a[u];
            rr[4 * q + u] = c[u];
          }
        }
        // this lane's parent column in the count and bias arrays (stored by
        // staged value column)
        const int ccol = col_of(r_of_row(ql), h_of_row(ql));
        for (int pt = 0; pt < nPT; ++pt) {
          const int j0 = pt * 64;
          wait_pass();
          f32x16 l2[2];
          const bool pass_masked = !all_parents || j0 + 64 > M0;
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            // empty parents and padding columns at -inf, as in the first pass
            const float bj = pass_masked ? sBp[j0 + b * 32 + ccol] : 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) l2[b][r] = bj;
#pragma unroll
            for (int s = 0; s < KS; ++s) l2[b] = T::mma_in(qf[s], sPC[(b * KS + s) * 64 + lane], l2[b]);
          }
          release_pass(pt + 1 < nPT ? pt + 1 : tile + 1 < tile1 ? 0 : -1);
          // the stabiliser bounds every logit of a parent with keys (exp2 of
          // at most the lazy margin) and the others are -inf: every term is
          // finite, and exactly 0 for a parent without keys
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            float acc = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc = fmaf(fast_exp2(fmaf(l2[b][r], sl2, -mr[r])), rr[r], acc);
            acc = xhalf_sum(acc);
            const int j = j0 + b * 32 + ql;
            if (hh == 0 && j < M0) sW[j * 4 + wave] = acc * sNp[j0 + b * 32 + ccol];
          }
        }
      }
      lds_barrier();
      // every wave forms the totals and its own copy of the selection; the
      // importance of parent 64 g + lane as a bit pattern (0 past M0: never
      // above a threshold search candidate), loaded for as many groups as the
      // parents fill
      auto imp_bits = [&](int g) -> uint32_t {
        if (g * 64 >= M0) return 0u;
        const f32x4 p4 = *(const f32x4*)(sW + (g * 64 + lane) * 4);  // j < M0p
        return __float_as_uint((p4[0] + p4[1]) + (p4[2] + p4[3]));
      };
      if (importance && wave == 0)
        for (int g = 0; g * 64 < M0; ++g)
          if (g * 64 + lane < M0)
            importance[((int64_t)bh * ntiles + tile) * M0 + g * 64 + lane] = __uint_as_float(imp_bits(g));
      if (P > 0) {
        int* gout = (topp && wave == 0) ? topp + ((int64_t)bh * ntiles + tile) * P : nullptr;
        if (parents_lds || M0 <= 64) {
          uint32_t u1[1] = {imp_bits(0)};
          select_top<1>(u1, M0, P, lane, sSel + wave * Pp, gout);
        } else if (M0 <= 128) {
          uint32_t u2[2] = {imp_bits(0), imp_bits(1)};
          select_top<2>(u2, M0, P, lane, sSel + wave * Pp, gout);
        } else if (M0 <= 256) {
          uint32_t u4[4] = {imp_bits(0), imp_bits(1), imp_bits(2), imp_bits(3)};
          select_top<4>(u4, M0, P, lane, sSel + wave * Pp, gout);
        } else {
          uint32_t u8[8];
#pragma unroll
          for (int g = 0; g < 8; ++g) u8[g] = imp_bits(g);
          select_top<8>(u8, M0, P, lane, sSel + wave * Pp, gout);
        }
        __builtin_amdgcn_wave_barrier();
      } else {
        lds_barrier();  // partials are rewritten by the next tile; no staging barrier follows
      }
    }


    // children of the selected parents (Alg. 2, the refinement loop; Eq. 8-9), CH rows per chunk
    if (P > 0) {
      const int* sel = sSel + wave * Pp;
      const float sl2C = sl2 / (float)C;  // Eq. 8's mean folded into the logit scale
      for (int cs = 0; cs < P; cs += NCB * S) {
        if (cs > 0) lds_barrier();  // readers of the previous chunk are done
        // codeword fragments: one DMA per (block, k-step); lane = (row, half).
        // Slots past P and rows past C read zeros (offsets out of range).
        {
          const int r = r_of_row(ql), hr = h_of_row(ql);
          const int s_row = 2 * (r / W) + hr, c_row = r % W;
          for (int u = wave; u < NCB * KS; u += nw) {
            const int b = u / KS, s = u % KS;
            const int gs = cs + b * S + s_row;
            const bool ok = gs < P && c_row < C;
            const int voff = ((M0 + sel[ok ? gs : 0] * C + c_row) * D + s * 2 * E + E * hh) * (int)sizeof(in_t);
            lds_dma_buf<BA>(cb_rs, ok ? voff : kOutOfRange, sCC + u * 64);
          }
        }
        // value fragments: one DMA per (block, k-step, half, 64 dims); lane = dim
        for (int u = wave; u < NCB * KV * 2 * (D / 64); u += nw) {
          const int dc = u % (D / 64), t = u / (D / 64);
          const int h2 = t % 2, bk = t / 2, k = bk % KV, b = bk / KV;
          const int r = k * E;
          const int gs = cs + b * S + 2 * (r / W) + h2, gg = (r % W) / E;
          const int p = gs < P ? sel[gs] : sel[0];
          lds_dma_buf<BV>(cv_rs, (((p * (W / E) + gg) * D + dc * 64 + lane) * BV), sCV + ((b * KV + k) * 2 + h2) * D + dc * 64);
        }
        // counts and biases of the chunk's NCB * 32 = 64 rows (one per lane of
        // wave 0), and whether any row is empty (then the chunk takes masks)
        static_assert(NCB * 32 == 64, "one chunk row per lane of wave 0");
        if (wave == 0) {
          const int b = lane >> 5, qq = lane & 31;
          const int r = r_of_col(qq), hc = h_of_col(qq);
          const int gs = cs + b * S + 2 * (r / W) + hc, cc = r % W;
          const float n = (gs < P && cc < C) ? (float)nb[M0 + sel[gs] * C + cc] : 0.0f;
          sNc[lane] = n;
          sBc[lane] = n > 0.0f ? 0.0f : -INFINITY;
          const bool any_empty = __builtin_amdgcn_ballot_w64(!(n > 0.0f)) != 0;
          if (lane == 0) sFlag[1] = any_empty ? 1 : 0;
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's staging copies have landed
        lds_barrier();
        const bool chunk_masked = __builtin_amdgcn_readfirstlane(sFlag[1]) != 0;

        // logits of the whole chunk
        f32x16 cl[NCB];
#pragma unroll
        for (int b = 0; b < NCB; ++b) {
          cl[b] = zero16();
#pragma unroll
          for (int s = 0; s < KS; ++s) cl[b] = T::mma_in(sCC[(b * KS + s) * 64 + lane], qf[s], cl[b]);
        }
        // Eq. 8: the parent logit is the mean of its C child logits, taken
        // before any masking; the W - C padding rows have zero codewords and
        // add nothing
        float sp[NCB][16 / W];
#pragma unroll
        for (int b = 0; b < NCB; ++b)
#pragma unroll
          for (int g2 = 0; g2 < 16 / W; ++g2) {
            float acc = cl[b][g2 * W];
#pragma unroll
            for (int c = 1; c < W; ++c) acc += cl[b][g2 * W + c];
            sp[b][g2] = acc;
            // formed here, before the masks, so that the unmasked logits are
            // dead once they are masked in place
            asm volatile("" : "+v"(sp[b][g2]));
          }
        // children without keys, padding rows and slots past P: logit -inf
        // (weight exactly 0); a chunk without such rows skips the masks
        if (chunk_masked) {
#pragma unroll
          for (int b = 0; b < NCB; ++b) {
            const f32x4* bc = (const f32x4*)(sBc + b * 32 + 8 * hh);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 b4 = bc[(q >> 1) * 4 + (q & 1)];
#pragma unroll
              for (int u = 0; u < 4; ++u) cl[b][q * 4 + u] += b4[u];
            }
          }
        }
        float tm = -INFINITY;
#pragma unroll
        for (int b = 0; b < NCB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) tm = fmaxf(tm, cl[b][r]);
        tm = xhalf_max(tm) * sl2;
        if (tm > m + kLazy) {
          const float f = fast_exp2(m - tm);
          zp *= f;
#pragma unroll
          for (int db = 0; db < DB; ++db) xacc[db] *= f;
          m = tm;
        }
#pragma unroll
        for (int b = 0; b < NCB; ++b) {
          const f32x4* nc = (const f32x4*)(sNc + b * 32 + 8 * hh);
#pragma unroll
          for (int g2 = 0; g2 < 16 / W; ++g2) {
            // a slot beyond P contributes nothing; an empty selected parent
            // gets a bounded weight (its children carry zero values and counts)
            const bool slot_ok = cs + b * S + 2 * g2 + hh < P;
            const float ap = slot_ok ? fast_exp2(fminf(fmaf(sp[b][g2], sl2C, -m), kLazy + 1.0f)) : 0.0f;
#pragma unroll
            for (int q = (g2 * W) / 4; q < (g2 * W + W) / 4; ++q) {
              const f32x4 n4 = nc[(q >> 1) * 4 + (q & 1)];
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                // empty and padding children: weight 0 - ap against zero
                // values and counts, so they add exactly nothing
                const float da = fast_exp2(fmaf(cl[b][q * 4 + u], sl2, -m)) - ap;
                cl[b][q * 4 + u] = da;
                zp = fmaf(da, n4[u], zp);
              }
            }
          }
#pragma unroll
          for (int k = 0; k < KV; ++k) {
            const pvfrag_t bf = pv_operand<T, KV>(cl[b], k);
#pragma unroll
            for (int db = 0; db < DB; ++db)
              xacc[db] = T::mma_pv(sCV[((b * KV + k) * 2 + hh) * D + ql + 32 * db], bf, xacc[db]);
          }
        }
      }
    }

    // the next tile's queries, taken before this tile's output stores are
    // issued (a wait for the loads then never waits for those stores)
    if constexpr (!kEarlyQ) load_next_q();
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = qn[s];
    const int qrow_t = qrow;
    qrow = qrow_n;

    // Y = x / z (Alg. 2, the final normalisation).  A lane holds 4-float runs of its query's
    // row; the wave's output goes through LDS 32 dims at a time.
    const float zt = xhalf_sum(zp);
    const float f = qv ? sig / zt : 0.0f;
    const int q0 = tile * bq + wave * 32;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x16& a = xacc[db];
        const f32x4 o = {a[4 * i] * f, a[4 * i + 1] * f, a[4 * i + 2] * f, a[4 * i + 3] * f};
        *(f32x4*)(yw + ql * kYRow + 8 * i + 4 * hh) = o;
      }
      store_rows(q0, db, qrow_t);
    }
  }
}

// ---- software-pipelined kernel for at most 64 parents (bf16, d = 64, P > 0) --
// The same arithmetic as attention_kernel with all parents in LDS, with the
// tile loop reordered so that the waits of one tile overlap the work of the
// next: while the children of tile t are being copied into LDS, every wave
// runs the parent pass of tile t + 1 (its weighted values go to a second set
// of accumulators), and the next queries are loaded as soon as the current
// ones are dead.  The children of a whole tile (up to kPipeBlocks 32-row
// blocks) are staged at once, so a tile takes two workgroup barriers: one
// after which the staged children (and the next tile's importance partials)
// are visible, one after which every wave is done with them.  Per tile t:
//   (a) parent pass of t + 1, importance partials of t + 1
//   (b) wait for this wave's copies; barrier
//   (c) children of t (later stages, when P needs more than kPipeBlocks
//       blocks, are copied and waited for in place); load the queries of t + 2
//   (d) top-P of t + 1
//   (h) output of t
//   (e) barrier; (f) copy the children of t + 1, load their counts
// The parents' logits start their MFMA accumulation from the parents' bias
// (0, or -inf for a parent without keys), so the mask costs no instruction.
// Children are masked only when needed: their logits' unmasked maximum is
// formed first, and only if it exceeds the stabiliser by more than the lazy
// margin (a rare event) are empty children masked out of the maximum.
// Otherwise every child weight is at most 2^8, and the children that must not
// contribute (no keys, padding rows, slots past P) carry exactly zero values
// and counts, so they add nothing.
constexpr int kPipeBlocks = 4;

size_t attention_pipe_smem_bytes(int d, int P, int block_q) {
  const size_t es = 2;  // bf16 codewords, fp16 value fragments
  const size_t nw = block_q / 32;
  size_t b = 2 * (size_t)64 * d * es;             // parents' codeword and value fragments
  b += 2 * (size_t)kPipeBlocks * 32 * d * es;     // staged children's codeword and value fragments
  b += 2 * 64 * 4 + 2 * kPipeBlocks * 32 * 4;     // counts and biases
  b += 64 * 4 * 4;                                // importance partials
  b += nw * (size_t)P * 4 + 16;                   // selections, flags
  b = (b + 15) & ~(size_t)15;
  b += nw * 32 * kYRow * 4;                       // output staging
  return b;
}

template <class T, int D, int W>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attention_pipe_kernel(
    const typename T::in_t* __restrict__ Q, const typename T::in_t* __restrict__ cb, const int* __restrict__ counts,
    const unsigned char* __restrict__ ws, size_t sig_bytes, size_t per_bh, int H, int BH, int N, int M0, int C, int P,
    int bq, int tiles_per_wg, int wgs_per_bh, float sl2, float* __restrict__ Y, int* __restrict__ topp,
    float* __restrict__ importance, const int* __restrict__ order, float* __restrict__ clear_v, int64_t clear_v4,
    int* __restrict__ clear_c, int64_t clear_nc) {
  using in_t = typename T::in_t;
  using frag_t = typename T::frag_t;
  using pvfrag_t = typename T::pvfrag_t;
  constexpr int E = T::E;
  constexpr int KS = D / (2 * E);
  constexpr int DB = D / 32;
  constexpr int S = 32 / W;
  constexpr int KV = 16 / E;
  constexpr int FA = KS * 64;
  constexpr int FV = KV * 2 * D;
  constexpr int BA = (int)sizeof(frag_t);
  constexpr int BV = (int)sizeof(pvfrag_t);
  constexpr int SB = kPipeBlocks;
  constexpr float kLazy = 8.0f;
  static_assert(SB % 2 == 0, "children are processed two blocks at a time");

  extern __shared__ __align__(16) unsigned char smem[];
  const int nw = blockDim.x >> 6;
  const int Mt = M0 * (1 + C);
  const int nCB = ((P + S - 1) / S + 1) & ~1;  // child blocks of a tile, even
  const int nStage = (nCB + SB - 1) / SB;
  frag_t* sPC = (frag_t*)smem;                        // [2 * FA]
  pvfrag_t* sPV = (pvfrag_t*)(sPC + 2 * FA);          // [2 * FV]
  frag_t* sCC = (frag_t*)(sPV + 2 * FV);              // [SB * FA]
  pvfrag_t* sCV = (pvfrag_t*)(sCC + SB * FA);         // [SB * FV]
  float* sNp = (float*)(sCV + SB * FV);               // [64] parent counts, by value column
  float* sBp = sNp + 64;                              // [64] 0 or -inf
  float* sNc = sBp + 64;                              // [SB * 32] staged children's counts, by column
  float* sBc = sNc + SB * 32;                         // [SB * 32] 0 or -inf
  float* sW = sBc + SB * 32;                          // [64][4] importance partials per wave
  int* sSel = (int*)(sW + 256);                       // [nw][P] selection (every wave its own copy)
  int* sFlag = sSel + nw * P;                         // [0] stage has rows to mask
  float* sY = (float*)(smem + ((((unsigned char*)(sFlag + 4) - smem) + 15) & ~15));  // [nw][32][kYRow]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, hh = lane >> 5;
  int bh, g;
  {
    const int L = blockIdx.x;
    if ((BH & 7) == 0) {
      const int k = L >> 3;
      bh = (k / wgs_per_bh) * 8 + (L & 7);
      g = k % wgs_per_bh;
    } else {
      bh = L / wgs_per_bh;
      g = L % wgs_per_bh;
    }
  }
  // this workgroup's share of the requested zero fill, first (measured: it
  // costs least issued before anything else)
  clear_buffers(clear_v, clear_v4, clear_c, clear_nc);
  const int h = bh % H;
  const int ntiles = (N + bq - 1) / bq;
  const int tile0 = g * tiles_per_wg;
  const int tile1 = min(ntiles, tile0 + tiles_per_wg);
  if (tile0 >= tile1) return;
  const in_t* cbh = cb + (int64_t)h * Mt * D;
  const int* nb = counts + (int64_t)bh * Mt;
  const in_t* Qb = Q + (int64_t)bh * N * D;
  float* Yb = Y + (int64_t)bh * N * D;
  const float sig = ((const float*)ws)[bh];
  const pvfrag_t* pvf = (const pvfrag_t*)(ws + sig_bytes + (size_t)bh * per_bh);
  const pvfrag_t* cvf = pvf + 2 * FV;
  const __amdgpu_buffer_rsrc_t cb_rs = __builtin_amdgcn_make_buffer_rsrc((void*)cbh, 0, Mt * D * (int)sizeof(in_t), kBufWord3);
  const __amdgpu_buffer_rsrc_t cv_rs = __builtin_amdgcn_make_buffer_rsrc((void*)cvf, 0, M0 * (W / E) * D * BV, kBufWord3);
  const float sl2C = sl2 / (float)C;  // Eq. 8's mean folded into the logit scale

  // ---- once per workgroup: parents into LDS -------------------------------------
  for (int u = wave; u < 2 * KS; u += nw) {
    const int b = u / KS, s = u % KS;
    const int j = b * 32 + ql;
    lds_dma<BA>(cbh + (int64_t)(j < M0 ? j : 0) * D + s * 2 * E + E * hh, sPC + u * 64);
  }
  for (int u = wave; u < 2 * FV / 64; u += nw) lds_dma<BV>(pvf + u * 64 + lane, sPV + u * 64);
  // importance partials: slots of absent waves and of parents past M0 stay zero
  for (int i = tid; i < 256; i += blockDim.x) sW[i] = 0.0f;
  if (tid < 64) {
    const int j = parent_of_col(tid);
    const float n = j < M0 ? (float)nb[j] : 0.0f;
    sNp[tid] = n;
    sBp[tid] = n > 0.0f ? 0.0f : -INFINITY;
  }

  // queries: rows of tile positions (an order gathers them; entries are
  // fetched a tile ahead of the loads that use them)
  auto order_at = [&](int pos) -> int { return (order != nullptr && pos < N) ? order[pos] : pos; };
  auto query_row = [&](int pos, int entry) -> int {
    if (pos >= N) return -1;
    if (order == nullptr) return pos;
    return (entry >= 0 && entry < N) ? entry : -1;
  };
  auto load_q = [&](frag_t (&qq)[KS], int row) {
    const in_t* qp = Qb + (int64_t)(row >= 0 ? row : 0) * D + E * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) qq[s] = *(const frag_t*)(qp + s * 2 * E);
  };
  auto qpos = [&](int t) { return t * bq + wave * 32 + ql; };

  float* yw = sY + wave * 32 * kYRow;
  auto store_rows = [&](int q0, int db, int row) {
    __builtin_amdgcn_wave_barrier();
    const int r0 = lane >> 3, c4 = (lane & 7) * 4;
    const float* src = yw + r0 * kYRow + c4;
    if (order != nullptr) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = __shfl(row, r0 + 8 * k);
        if (r >= 0)
          __builtin_nontemporal_store(*(const f32x4*)(src + 8 * k * kYRow), (f32x4*)(Yb + (int64_t)r * D + db * 32 + c4));
      }
      return;
    }
    float* dst = Yb + (int64_t)(q0 + r0) * D + db * 32 + c4;
    if (q0 + 32 <= N) {
#pragma unroll
      for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(*(const f32x4*)(src + 8 * k * kYRow), (f32x4*)(dst + 8 * k * D));
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (q0 + r0 + 8 * k < N)
          __builtin_nontemporal_store(*(const f32x4*)(src + 8 * k * kYRow), (f32x4*)(dst + 8 * k * D));
    }
  };

  // Parent pass of one tile (Alg. 2, Eq. 6; Eq. 18 with its lazy stabiliser)
  // and, from the weights still in registers, this wave's importance
  // partials (Eq. 7) in sW.
  auto parent_pass = [&](const frag_t (&qq)[KS], bool qv, f32x16 (&xa)[DB], float& zz, float& mm) {
#pragma unroll
    for (int db = 0; db < DB; ++db) xa[db] = zero16();
    f32x16 lg[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const f32x4* bp = (const f32x4*)(sBp + b * 32 + 8 * hh);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 b4 = bp[(q >> 1) * 4 + (q & 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) lg[b][q * 4 + u] = b4[u];
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) lg[b] = T::mma_in(sPC[(b * KS + s) * 64 + lane], qq[s], lg[b]);
    }
    float tm = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) tm = fmaxf(tm, lg[b][r]);
    // the first (only) pass: the accumulators are zero, no rescaling
    mm = fmaxf(xhalf_max(tm) * sl2, -FLT_MAX);
    float z = 0.0f;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const f32x4* np4 = (const f32x4*)(sNp + b * 32 + 8 * hh);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 n4 = np4[(q >> 1) * 4 + (q & 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float a = fast_exp2(fmaf(lg[b][q * 4 + u], sl2, -mm));
          lg[b][q * 4 + u] = a;
          z = fmaf(a, n4[u], z);
        }
      }
#pragma unroll
      for (int k = 0; k < KV; ++k) {
        const pvfrag_t bf = pv_operand<T, KV>(lg[b], k);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          xa[db] = T::mma_pv(sPV[((b * KV + k) * 2 + hh) * D + ql + 32 * db], bf, xa[db]);
      }
    }
    zz = z;
    // Eq. 7: A / z summed over the wave's 32 queries; the count n_j is a
    // factor of the whole sum, applied after the reduction
    const float rz = qv ? 1.0f / xhalf_sum(z) : 0.0f;
    float t[32];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) t[b * 16 + r] = lg[b][r] * rz;
    rs_half32(t, lane);
    const int j = 32 * (ql >> 4) + row_of(ql & 15, hh);
    if (j < M0) sW[j * 4 + wave] = t[0] * sNp[32 * (ql >> 4) + col_of(ql & 15, hh)];
  };

  // Top-P of one tile (Alg. 2, the parent choice) from the importance
  // partials of every wave, formed by wave 0 alone into sSel; the other waves
  // read it after the barrier that follows every call.
  auto top_p = [&](int tile) {
    if (wave != 0) return;
    uint32_t u1[1];
    {
      const f32x4 p4 = *(const f32x4*)(sW + lane * 4);
      u1[0] = lane < M0 ? __float_as_uint((p4[0] + p4[1]) + (p4[2] + p4[3])) : 0u;
    }
    if (importance && lane < M0) importance[((int64_t)bh * ntiles + tile) * M0 + lane] = __uint_as_float(u1[0]);
    int* gout = topp ? topp + ((int64_t)bh * ntiles + tile) * P : nullptr;
    select_top<1>(u1, M0, P, lane, sSel, gout);
  };

  // Copies of one stage of the selected parents' children into LDS (this
  // wave's share): codeword fragments, value fragments.  Slots past P and
  // rows past C read zeros (offsets out of range).
  const int r_row = r_of_row(ql), h_row = h_of_row(ql);
  const int s_row = 2 * (r_row / W) + h_row, c_row = r_row % W;
  auto stage_issue = [&](int st) {
    const int* sel = sSel;
    const int b0 = st * SB;
    const int nb_st = min(SB, nCB - b0);
    for (int u = wave; u < nb_st * KS; u += nw) {
      const int b = u / KS, s = u % KS;
      const int gs = (b0 + b) * S + s_row;
      const bool ok = gs < P && c_row < C;
      const int voff = ((M0 + sel[ok ? gs : 0] * C + c_row) * D + s * 2 * E + E * hh) * (int)sizeof(in_t);
      lds_dma_buf<BA>(cb_rs, ok ? voff : kOutOfRange, sCC + u * 64);
    }
    for (int u = wave; u < nb_st * KV * 2 * (D / 64); u += nw) {
      const int dc = u % (D / 64), t = u / (D / 64);
      const int h2 = t % 2, bk = t / 2, k = bk % KV, b = bk / KV;
      const int r = k * E;
      const int gs = (b0 + b) * S + 2 * (r / W) + h2, gg = (r % W) / E;
      const int voff = gs < P ? ((sel[gs] * (W / E) + gg) * D + dc * 64 + lane) * BV : kOutOfRange;
      lds_dma_buf<BV>(cv_rs, voff, sCV + ((b * KV + k) * 2 + h2) * D + dc * 64);
    }
  };
  // counts of one stage's rows (wave 0; two rows per lane), loaded into
  // registers here and written to LDS by stage_counts_store
  auto stage_counts_load = [&](int st, int (&cn)[SB / 2]) {
    const int* sel = sSel;  // wave 0's copy
#pragma unroll
    for (int i = 0; i < SB / 2; ++i) {
      const int row = lane + 64 * i;
      const int b = st * SB + (row >> 5), qq = row & 31;
      const int r = r_of_col(qq), hc = h_of_col(qq);
      const int gs = b * S + 2 * (r / W) + hc, cc = r % W;
      cn[i] = (gs < P && cc < C) ? nb[M0 + sel[gs] * C + cc] : 0;
    }
  };
  auto stage_counts_store = [&](const int (&cn)[SB / 2]) {
    bool any_empty = false;
#pragma unroll
    for (int i = 0; i < SB / 2; ++i) {
      const float n = (float)cn[i];
      sNc[lane + 64 * i] = n;
      sBc[lane + 64 * i] = n > 0.0f ? 0.0f : -INFINITY;
      any_empty = any_empty || !(n > 0.0f);
    }
    const bool e = __builtin_amdgcn_ballot_w64(any_empty) != 0;
    if (lane == 0) sFlag[0] = e ? 1 : 0;
  };

  // The children of one staged stage (Alg. 2, the refinement loop; Eq. 8-9),
  // two 32-row blocks at a time, into the accumulators of the tile.
  auto children_stage = [&](int st, const frag_t (&qq)[KS], f32x16 (&xa)[DB], float& zz, float& mm) {
    const bool stage_masked = __builtin_amdgcn_readfirstlane(sFlag[0]) != 0;
    const int nb_st = min(SB, nCB - st * SB);
    for (int pb = 0; pb < nb_st; pb += 2) {
      f32x16 cl[2];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        cl[bb] = zero16();
#pragma unroll
        for (int s = 0; s < KS; ++s) cl[bb] = T::mma_in(sCC[((pb + bb) * KS + s) * 64 + lane], qq[s], cl[bb]);
      }
      // Eq. 8: the parent logit is the mean of its C child logits, taken
      // before any masking (padding rows have zero codewords)
      float sp[2][16 / W];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int g2 = 0; g2 < 16 / W; ++g2) {
          float acc = cl[bb][g2 * W];
#pragma unroll
          for (int c = 1; c < W; ++c) acc += cl[bb][g2 * W + c];
          // formed here, before the rare masking below, so that the unmasked
          // logits are dead once they are masked in place (formed after the
          // branch, they stay live across it and the merge copies all 32)
          asm volatile("" : "+v"(acc));
          sp[bb][g2] = acc;
        }
      float tm = -INFINITY;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tm = fmaxf(tm, cl[bb][r]);
      tm = xhalf_max(tm) * sl2;
      if (__builtin_amdgcn_ballot_w64(tm > mm + kLazy) != 0) {
        // rare: a child logit exceeds the stabiliser by more than the lazy
        // margin; Eq. 18 takes the maximum over children with keys only
        if (stage_masked) {
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            const f32x4* bc = (const f32x4*)(sBc + (pb + bb) * 32 + 8 * hh);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 b4 = bc[(q >> 1) * 4 + (q & 1)];
#pragma unroll
              for (int u = 0; u < 4; ++u) cl[bb][q * 4 + u] += b4[u];
            }
          }
          tm = -INFINITY;
#pragma unroll
          for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) tm = fmaxf(tm, cl[bb][r]);
          tm = xhalf_max(tm) * sl2;
        }
        if (tm > mm + kLazy) {
          const float f = fast_exp2(mm - tm);
          zz *= f;
#pragma unroll
          for (int db = 0; db < DB; ++db) xa[db] *= f;
          mm = tm;
        }
      }
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const f32x4* nc = (const f32x4*)(sNc + (pb + bb) * 32 + 8 * hh);
#pragma unroll
        for (int g2 = 0; g2 < 16 / W; ++g2) {
          const bool slot_ok = (st * SB + pb + bb) * S + 2 * g2 + hh < P;
          const float ap = slot_ok ? fast_exp2(fminf(fmaf(sp[bb][g2], sl2C, -mm), kLazy + 1.0f)) : 0.0f;
#pragma unroll
          for (int q = (g2 * W) / 4; q < (g2 * W + W) / 4; ++q) {
            const f32x4 n4 = nc[(q >> 1) * 4 + (q & 1)];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float da = fast_exp2(fmaf(cl[bb][q * 4 + u], sl2, -mm)) - ap;
              cl[bb][q * 4 + u] = da;
              zz = fmaf(da, n4[u], zz);
            }
          }
        }
#pragma unroll
        for (int k = 0; k < KV; ++k) {
          const pvfrag_t bf = pv_operand<T, KV>(cl[bb], k);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            xa[db] = T::mma_pv(sCV[(((pb + bb) * KV + k) * 2 + hh) * D + ql + 32 * db], bf, xa[db]);
        }
      }
    }
  };

  // children of a tile: stage 0 is staged already; later stages are copied
  // and waited for here
  auto children = [&](const frag_t (&qq)[KS], f32x16 (&xa)[DB], float& zz, float& mm) {
    children_stage(0, qq, xa, zz, mm);
    for (int st = 1; st < nStage; ++st) {
      lds_barrier();  // every wave is done with the previous stage
      stage_issue(st);
      if (wave == 0) {
        int cn[SB / 2];
        stage_counts_load(st, cn);
        stage_counts_store(cn);
      }
      __builtin_amdgcn_s_waitcnt(0);
      lds_barrier();
      children_stage(st, qq, xa, zz, mm);
    }
  };

  // Y = x / z (Alg. 2, the final normalisation), through LDS 32 dims at a time
  auto output = [&](int tile, const f32x16 (&xa)[DB], float zz, bool qv, int qrow_t) {
    const float zt = xhalf_sum(zz);
    const float f = qv ? sig / zt : 0.0f;
    const int q0 = tile * bq + wave * 32;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x16& a = xa[db];
        const f32x4 o = {a[4 * i] * f, a[4 * i + 1] * f, a[4 * i + 2] * f, a[4 * i + 3] * f};
        *(f32x4*)(yw + ql * kYRow + 8 * i + 4 * hh) = o;
      }
      store_rows(q0, db, qrow_t);
    }
  };

  // ---- prologue: tile0's parent pass, selection and child copies ----------------
  frag_t qA[KS], qB[KS];
  f32x16 xA[DB], xB[DB];
  float zA = 0.0f, mA = -FLT_MAX, zB = 0.0f, mB = -FLT_MAX;
  int rowA = query_row(qpos(tile0), order_at(qpos(tile0)));
  int rowB = -1;
  int entry_n = order_at(qpos(tile0 + 1));  // order entry of this lane's query in the next tile
  load_q(qA, rowA);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  parent_pass(qA, rowA >= 0, xA, zA, mA);
  if (tile0 + 1 < tile1) {
    rowB = query_row(qpos(tile0 + 1), entry_n);
    load_q(qB, rowB);
    entry_n = order_at(qpos(tile0 + 2));
  }
  lds_barrier();  // importance partials of tile0
  top_p(tile0);
  int cnt[SB / 2];
  lds_barrier();  // every wave has read the partials
  stage_issue(0);
  if (wave == 0) stage_counts_load(0, cnt);

  // ---- the pipelined tile loop (unrolled by two: the register sets swap roles) --
  auto step = [&](int t, frag_t (&qc)[KS], f32x16 (&xc)[DB], float& zc, float& mc, int& rowc,
                  frag_t (&qn)[KS], f32x16 (&xn)[DB], float& zn, float& mn, int& rown) {
    const bool more = t + 1 < tile1;
    // (a) the next tile's parent pass and importance partials
    if (more) parent_pass(qn, rown >= 0, xn, zn, mn);
    // (b) this wave's copies (and counts) of tile t have landed; barrier
    if (wave == 0) stage_counts_store(cnt);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    // (c) the children of tile t; then the queries of tile t + 2
    children(qc, xc, zc, mc);
    const int rowt = rowc;
    const bool qvt = rowc >= 0;
    if (t + 2 < tile1) {
      rowc = query_row(qpos(t + 2), entry_n);
      load_q(qc, rowc);
      entry_n = order_at(qpos(t + 3));
    }
    // (d) the next tile's selection
    if (more) top_p(t + 1);
    // (h) the output of tile t
    output(t, xc, zc, qvt, rowt);
    // (e) every wave is done with tile t's children and the partials; (f) the
    // next tile's child copies and counts
    if (more) {
      lds_barrier();
      stage_issue(0);
      if (wave == 0) stage_counts_load(0, cnt);
    }
  };
  for (int t = tile0; t < tile1; t += 2) {
    step(t, qA, xA, zA, mA, rowA, qB, xB, zB, mB, rowB);
    if (t + 1 < tile1) step(t + 1, qB, xB, zB, mB, rowB, qA, xA, zA, mA, rowA);
  }
}

size_t attention_smem_bytes(int dtype, int d, int M0, int C, int P, int block_q, bool importance) {
  const size_t es = dtype == 0 ? 4 : 2;   // input and value operand element (same width)
  const size_t M0p = attn_parent_rows(M0);
  const size_t nw = block_q / 32;
  const size_t CH = d == 64 ? AttnTraits<64>::kChunkRows : AttnTraits<128>::kChunkRows;
  (void)C;
  const size_t ch = P > 0 ? CH : 0;
  const bool values_lds = M0p <= 64 || (d == 64 && M0p <= 256);
  size_t b = (M0p <= 64 ? M0p : 64) * d * es;  // parents' codeword fragments (all, or one 64-parent pass)
  if (values_lds) b += M0p * d * es;         // parents' value fragments (else staged per pass)
  b += 2 * (P > 0 || !values_lds ? CH : 0) * d * es;  // chunk codeword and value fragments
  b += 2 * (M0p + ch) * 4;                    // counts and biases
  if (P > 0 || importance) b += M0p * 4 * 4;           // importance partials
  b += nw * (size_t)(P > 0 ? P : 1) * 4 + 48; // selections, flags, keys per pass
  b = (b + 15) & ~(size_t)15;
  b += nw * 32 * kYRow * 4;                   // output staging
  return b;
}

// Query tiles per workgroup: aim for about two resident workgroups per CU.
int attention_tiles_per_wg(int BH, int N, int bq) {
  // CU count of the current device, read once per device (only the split of
  // the work depends on it)
  static std::atomic<int> cu_cache[64];
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    cus = cu_cache[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
      cu_cache[dev].store(cus, std::memory_order_relaxed);
    }
  }
  const int T = (N + bq - 1) / bq;
  const int target = 2 * cus;
  int per_bh = (target + BH - 1) / (BH > 0 ? BH : 1);
  if (per_bh > T) per_bh = T;
  if (per_bh < 1) per_bh = 1;
  return (T + per_bh - 1) / per_bh;
}

template <class T, int D, int W, bool PL, bool VL>
static hipError_t launch_attn_t(const void* Q, const void* cb, const float* vsum, const int* counts, int BH, int H, int N,
                                int M0, int C, int P, int bq, float scale, float* Y, int* topp, float* importance,
                                void* ws, bool approx, const int* order, int stages, float* clear_v, int* clear_c, hipStream_t st) {
  const int dtype = std::is_same<T, TF32>::value ? 0 : 1;
  const AttnWs wl = attn_ws(dtype, D, M0, C, BH);
  const size_t sig_bytes = wl.sig_bytes, per_bh = wl.per_bh;
  if (stages & kAttnPrep) {
    constexpr int E = T::E, KV = 16 / E;
    const int M0p = attn_parent_rows(M0);
    const int nF = (M0p / 32) * KV * 2 * D + (C > 0 ? M0 * (W / E) * D : 0);
    const int per_part = kPrepThreads * kPrepFrag;
    const int parts = std::max(8, (nF + per_part - 1) / per_part);
    const size_t head_bytes = (size_t)M0 * (1 + C) * D * 4;
    float* pmax = nullptr;
    if (T::kScaleValues && (size_t)parts * head_bytes > kPrepRepeatBytes) {
      pmax = (float*)((unsigned char*)ws + wl.pmax_off);
      hipLaunchKernelGGL(attention_absmax_kernel, dim3(BH * wl.slices), dim3(kMaxThreads), 0, st, vsum,
                         M0 * (1 + C) * (D / 4), wl.slices, pmax);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((attention_prep_kernel<T, D, W>), dim3(BH * parts), dim3(kPrepThreads), 0, st, vsum, counts,
                       BH, M0, C, parts, (unsigned char*)ws, sig_bytes, per_bh, (const float*)pmax, wl.slices,
                       (int*)((unsigned char*)ws + wl.counts_off));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(stages & kAttnKernel)) return hipSuccess;
  // the kernel reads the counts from the workspace copy the preparation made
  const int* wcounts = (const int*)((const unsigned char*)ws + wl.counts_off);
  const int64_t Mt = (int64_t)M0 * (1 + C);
  const int64_t clear_v4 = clear_v ? (int64_t)BH * Mt * D / 4 : 0, clear_nc = clear_c ? (int64_t)BH * Mt : 0;
  const int tpw = attention_tiles_per_wg(BH, N, bq);
  const int T_ = (N + bq - 1) / bq;
  const int per = (T_ + tpw - 1) / tpw;
  const float sl2 = scale * 1.4426950408889634f;
  if constexpr (PL && VL && D == 64 && std::is_same<T, TBF16>::value) {
    if (P > 0) {
      // all parents in LDS and children to refine: the pipelined tile loop
      const size_t smem = attention_pipe_smem_bytes(D, P, bq);
      auto kern = attention_pipe_kernel<T, D, W>;
      hipError_t e = raise_lds_limit((const void*)kern, smem);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(per * BH), dim3(2 * bq), smem, st, (const typename T::in_t*)Q,
                         (const typename T::in_t*)cb, wcounts, (const unsigned char*)ws, sig_bytes, per_bh, H, BH,
                         N, M0, C, P, bq, tpw, per, sl2, Y, topp, importance, order, clear_v, clear_v4, clear_c,
                         clear_nc);
      return hipGetLastError();
    }
  }
  const size_t smem = attention_smem_bytes(dtype, D, M0, C, P, bq, importance != nullptr);
  auto kern = attention_kernel<T, D, W, PL, VL>;
  hipError_t e = raise_lds_limit((const void*)kern, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(per * BH), dim3(2 * bq), smem, st, (const typename T::in_t*)Q,
                     (const typename T::in_t*)cb, wcounts, (const unsigned char*)ws, sig_bytes, per_bh, H, BH, N, M0,
                     C, P, bq, tpw, per, sl2, Y, topp, importance, approx ? 1 : 0, order, clear_v, clear_v4, clear_c,
                     clear_nc);
  return hipGetLastError();
}

template <class T, int D, int W>
static hipError_t launch_attn_v(const void* Q, const void* cb, const float* vsum, const int* counts, int BH, int H, int N,
                                int M0, int C, int P, int bq, float scale, float* Y, int* topp, float* importance,
                                void* ws, bool approx, const int* order, int stages, float* clear_v, int* clear_c, hipStream_t st) {
  if (M0 <= 64)
    return launch_attn_t<T, D, W, true, true>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance,
                                              ws, approx, order, stages, clear_v, clear_c, st);
  // at d = 64 the values stay in LDS up to 256 parents; beyond, LDS-resident
  // values would leave one workgroup per CU, with nothing to cover the
  // staged parent passes' barriers (measured at 512 flat codewords: 211 us
  // against 177 us reading the values from L2 with two workgroups per CU)
  if constexpr (D == 64) {
    if (M0 <= 256)
      return launch_attn_t<T, D, W, false, true>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp,
                                                 importance, ws, approx, order, stages, clear_v, clear_c, st);
  }
  return launch_attn_t<T, D, W, false, false>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance,
                                              ws, approx, order, stages, clear_v, clear_c, st);
}

template <class T, int D>
static hipError_t launch_attn_w(const void* Q, const void* cb, const float* vsum, const int* counts, int BH, int H, int N,
                                int M0, int C, int P, int bq, float scale, float* Y, int* topp, float* importance,
                                void* ws, bool approx, const int* order, int stages, float* clear_v, int* clear_c, hipStream_t st) {
  if (C <= 8)
    return launch_attn_v<T, D, 8>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, ws, approx,
                                  order, stages, clear_v, clear_c, st);
  return launch_attn_v<T, D, 16>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, ws, approx,
                                 order, stages, clear_v, clear_c, st);
}

hipError_t launch_attention(int dtype, const void* Q, const void* cb, const float* vsum, const int* counts, int BH, int H,
                            int N, int d, int M0, int C, int P, int bq, float scale, float* Y, int* topp,
                            float* importance, void* ws, bool approx, const int* order, int stages, float* clear_v, int* clear_c, hipStream_t st) {
  if (dtype == 0) {
    if (d == 64) return launch_attn_w<TF32, 64>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, ws, approx, order, stages, clear_v, clear_c, st);
    return launch_attn_w<TF32, 128>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, ws, approx, order, stages, clear_v, clear_c, st);
  }
  if (d == 64) return launch_attn_w<TBF16, 64>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, ws, approx, order, stages, clear_v, clear_c, st);
  return launch_attn_w<TBF16, 128>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, ws, approx, order, stages, clear_v, clear_c, st);
}

}  // namespace avq
