// Kernel 2 of the AVQ-Attention forward pass: count-weighted attention over
// the parent codewords, per-tile importance, top-P selection and the child
// correction ("AVQ-Attention: Adaptive Vector-Quantized Attention",
// Sec. 4.3 and Algorithm 2; Eq. 6-9; Sec. C and D).
//
// One workgroup per (query tile, batch*head); one wave per 32 queries.
// Logits are computed transposed on MFMA (rows = codewords, columns =
// queries): each lane owns one query and 16 codewords per 32-row block, so
// the running max, the denominator and the rescaling are per-lane scalars,
// the parent logit of Eq. 8 is a sum over registers of one lane, and the
// weights feed the weighted-value MFMA as its B operand in place.
//
// Value sums of the codewords in use are staged per chunk (up to 128
// codewords) in LDS, transposed and, for bf16 inputs, converted to fp16
// after scaling by a power of two chosen from the chunk's largest magnitude;
// the accumulator carries the current scale and is re-expressed when the
// next chunk's scale differs (an exact power-of-two factor folded into the
// online-softmax rescale).
//
// Children are packed S = 32 / W parents per 32-row block (W = slot width,
// C <= W): the children of one selected parent occupy W consecutive
// accumulator registers of one lane half, in child order.
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

// Stage value sums and counts of ncols codewords into the transposed tile
// sV[D][LDV] and sN[ncols]; rowof(c) is the codebook row of column c or -1.
// Returns the scale sigma: staged values are vsum / sigma.
template <class T, int D, int LDV, class RowFn>
__device__ float stage_values(typename T::pv_t* sV, float* sN, float* sRed, const float* __restrict__ vs,
                              const int* __restrict__ nb, int ncols, RowFn rowof, int tid, int nthreads,
                              int lane, int wave, int nw) {
  using pv_t = typename T::pv_t;
  constexpr int C4 = D / 4;
  const int items = ncols * C4;
  float sig = 1.0f, inv = 1.0f;
  if constexpr (T::kScaleValues) {
    float mx = 0.0f;
    for (int i = tid; i < items; i += nthreads) {
      const int c = i / C4, q = (i % C4) * 4;
      const int row = rowof(c);
      if (row >= 0) {
        const f32x4 v = *(const f32x4*)(vs + (int64_t)row * D + q);
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
      }
    }
    mx = wave_max(mx);
    if (lane == 0) sRed[wave] = mx;
    __syncthreads();
    mx = 0.0f;
    for (int w = 0; w < nw; ++w) mx = fmaxf(mx, sRed[w]);
    if (mx > 0.0f) {
      int e;
      frexpf(mx, &e);  // mx < 2^e
      sig = ldexpf(1.0f, e - 15);
      inv = ldexpf(1.0f, 15 - e);
    }
  }
  for (int i = tid; i < items; i += nthreads) {
    const int c = i / C4, q = (i % C4) * 4;
    const int row = rowof(c);
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (row >= 0) v = *(const f32x4*)(vs + (int64_t)row * D + q);
#pragma unroll
    for (int j = 0; j < 4; ++j) sV[(q + j) * LDV + c] = (pv_t)(v[j] * inv);
  }
  for (int c = tid; c < ncols; c += nthreads) {
    const int row = rowof(c);
    sN[c] = row >= 0 ? (float)nb[row] : 0.0f;
  }
  __syncthreads();
  return sig;
}

}  // namespace

template <class T, int D, int W>
__global__ __launch_bounds__(256) void attention_kernel(
    const typename T::in_t* __restrict__ Q, const typename T::in_t* __restrict__ cb,
    const float* __restrict__ vsum, const int* __restrict__ counts, int H, int N, int M0, int C, int P, int bq,
    float sl2, float* __restrict__ Y, int* __restrict__ topp, float* __restrict__ importance) {
  using in_t = typename T::in_t;
  using frag_t = typename T::frag_t;
  using pv_t = typename T::pv_t;
  using pvfrag_t = typename T::pvfrag_t;
  constexpr int E = T::E;
  constexpr int KS = D / (2 * E);
  constexpr int DB = D / 32;
  constexpr int S = 32 / W;
  constexpr int LDV = 128 + 16 / sizeof(pv_t);
  constexpr int KV = 16 / E;  // weighted-value k-steps per 32-row block

  extern __shared__ __align__(16) unsigned char smem[];
  const int nthreads = blockDim.x;
  const int nw = nthreads >> 6;
  const int Mt = M0 * (1 + C);
  const int M0p = (M0 + 31) & ~31;
  pv_t* sV = (pv_t*)smem;
  float* sN = (float*)(sV + D * LDV);
  float* sW = sN + 128;
  float* sWt = sW + nw * M0p;
  float* sRed = sWt + M0p;
  int* sSel = (int*)(sRed + 8);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, hh = lane >> 5;
  const int bh = blockIdx.y, h = bh % H, tile = blockIdx.x;
  const int ntiles = gridDim.x;
  const int qi = tile * bq + wave * 32 + ql;
  const bool qv = qi < N;
  const in_t* cbh = cb + (int64_t)h * Mt * D;
  const float* vs = vsum + (int64_t)bh * Mt * D;
  const int* nb = counts + (int64_t)bh * Mt;

  frag_t qf[KS];
  {
    const in_t* qp = Q + ((int64_t)bh * N + (qv ? qi : N - 1)) * D + E * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *(const frag_t*)(qp + s * 2 * E);
  }

  f32x16 xacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) xacc[db] = zero16();
  float zp = 0.0f;        // denominator over this lane half's codewords
  float m = -INFINITY;    // running max of the log2-scaled logits
  float sig = 1.0f;       // xacc holds value sums divided by sig
  const bool need_imp = (P > 0) || (importance != nullptr);
  const int nPT = (M0 + 63) / 64;
  f32x16 lg[2];

  // ---- parents (Alg. 2 lines 2-7), in tiles of 64 --------------------------
  for (int pt = 0; pt < nPT; ++pt) {
    const int j0 = pt * 64;
    const int nblk = min(2, (M0 - j0 + 31) / 32);
    if (pt > 0) __syncthreads();
    const float sg = stage_values<T, D, LDV>(
        sV, sN, sRed, vs, nb, nblk * 32,
        [&](int c) {
          const int b = c >> 5, q = c & 31;
          const int j = j0 + 32 * b + row_of(r_of_col(q), h_of_col(q));
          return j < M0 ? j : -1;
        },
        tid, nthreads, lane, wave, nw);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      lg[b] = zero16();
      if (b < nblk) {
        const int j = j0 + 32 * b + ql;
        const in_t* ap = cbh + (int64_t)(j < M0 ? j : 0) * D + E * hh;
#pragma unroll
        for (int s = 0; s < KS; ++s) lg[b] = T::mma_in(*(const frag_t*)(ap + s * 2 * E), qf[s], lg[b]);
      }
    }
    float tm = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (b < nblk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          lg[b][r] *= sl2;
          if (sN[b * 32 + col_of(r, hh)] > 0.0f) tm = fmaxf(tm, lg[b][r]);
        }
      }
    }
    tm = xhalf_max(tm);
    const float mn = fmaxf(m, tm);
    if (mn != -INFINITY) {
      const float f = exp2f(m - mn);
      zp *= f;
      const float fx = f * (sig / sg);
#pragma unroll
      for (int db = 0; db < DB; ++db) xacc[db] *= fx;
      m = mn;
      sig = sg;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (b < nblk) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float n = sN[b * 32 + col_of(r, hh)];
            const float a = n > 0.0f ? exp2f(lg[b][r] - m) : 0.0f;
            lg[b][r] = a;
            zp = fmaf(a, n, zp);
          }
#pragma unroll
          for (int k = 0; k < KV; ++k) {
            pvfrag_t bf;
            if constexpr (KV == 2) bf = k == 0 ? pack_at<T, 0>(lg[b]) : pack_at<T, 8>(lg[b]);
            else bf = lg[b][k];
            const int cofs = b * 32 + 16 * ((k * E) >> 3) + 8 * hh + ((k * E) & 7);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const pvfrag_t af = *(const pvfrag_t*)(sV + (db * 32 + ql) * LDV + cofs);
              xacc[db] = T::mma_pv(af, bf, xacc[db]);
            }
          }
        }
      }
    } else {
      lg[0] = zero16();
      lg[1] = zero16();
    }
  }

  // ---- importance (Eq. 7, Alg. 2 line 8) and top-P (line 9) ----------------
  if (need_imp) {
    const float zt = xhalf_sum(zp);
    const float rz = qv ? 1.0f / zt : 0.0f;
    for (int pt = 0; pt < nPT; ++pt) {
      const int j0 = pt * 64;
      const int nblk = min(2, (M0 - j0 + 31) / 32);
      float t[32];
      if (nPT == 1) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            t[b * 16 + r] = b < nblk ? lg[b][r] * sN[b * 32 + col_of(r, hh)] * rz : 0.0f;
      } else {
        // second pass: logits again with the final max and denominator
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          f32x16 l2 = zero16();
          if (b < nblk) {
            const int j = j0 + 32 * b + ql;
            const in_t* ap = cbh + (int64_t)(j < M0 ? j : 0) * D + E * hh;
#pragma unroll
            for (int s = 0; s < KS; ++s) l2 = T::mma_in(*(const frag_t*)(ap + s * 2 * E), qf[s], l2);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = j0 + 32 * b + row_of(r, hh);
            const float n = (b < nblk && j < M0) ? (float)nb[j] : 0.0f;
            t[b * 16 + r] = n > 0.0f ? exp2f(l2[r] * sl2 - m) * n * rz : 0.0f;
          }
        }
      }
      if (nblk == 2) {
        rs_half32(t, lane);
        const int j = j0 + 32 * (ql >> 4) + row_of(ql & 15, hh);
        if (j < M0) sW[wave * M0p + j] = t[0];
      } else {
        rs_half16(t, lane);
        const int j = j0 + row_of(ql & 15, hh);
        if (ql < 16 && j < M0) sW[wave * M0p + j] = t[0];
      }
    }
    __syncthreads();
    for (int j = tid; j < M0; j += nthreads) {
      float s = 0.0f;
      for (int w = 0; w < nw; ++w) s += sW[w * M0p + j];
      sWt[j] = s;
      if (importance) importance[((int64_t)bh * ntiles + tile) * M0 + j] = s;
    }
    __syncthreads();
    if (P > 0) {
      if (wave == 0) {
        int before = 0;
        for (int jb = 0; jb < M0p; jb += 64) {
          const int j = jb + lane;
          bool sel = false;
          if (j < M0) {
            const float wj = sWt[j];
            int rank = 0;
            for (int jj = 0; jj < M0; ++jj) {
              const float wo = sWt[jj];
              rank += (wo > wj) || (wo == wj && jj < j);
            }
            sel = rank < P;
          }
          const uint64_t msk = __ballot(sel);
          if (sel) {
            const int pos = before + __popcll(msk & ((1ull << lane) - 1ull));
            sSel[pos] = j;
            if (topp) topp[((int64_t)bh * ntiles + tile) * P + pos] = j;
          }
          before += __popcll(msk);
        }
      }
      __syncthreads();
    }
  }

  // ---- children of the selected parents (Alg. 2 lines 10-19) ---------------
  if (P > 0) {
    const float invC = 1.0f / (float)C;
    const int nblkC = (P + S - 1) / S;
    const int rr = r_of_row(ql), hr = h_of_row(ql);
    const int s_row = 2 * (rr / W) + hr, c_row = rr % W;
    for (int cb0 = 0; cb0 < nblkC; cb0 += 4) {
      const int nbk = min(4, nblkC - cb0);
      __syncthreads();
      const float sg = stage_values<T, D, LDV>(
          sV, sN, sRed, vs, nb, nbk * 32,
          [&](int c) {
            const int b = c >> 5, q = c & 31;
            const int r = r_of_col(q), hc = h_of_col(q);
            const int gs = (cb0 + b) * S + 2 * (r / W) + hc, cc = r % W;
            return (gs < P && cc < C) ? M0 + sSel[gs] * C + cc : -1;
          },
          tid, nthreads, lane, wave, nw);
      f32x16 cl[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        cl[b] = zero16();
        if (b < nbk) {
          const int gs = (cb0 + b) * S + s_row;
          const int row = (gs < P && c_row < C) ? M0 + sSel[gs] * C + c_row : 0;
          const in_t* ap = cbh + (int64_t)row * D + E * hh;
#pragma unroll
          for (int s = 0; s < KS; ++s) cl[b] = T::mma_in(*(const frag_t*)(ap + s * 2 * E), qf[s], cl[b]);
        }
      }
      float tm = -INFINITY;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b < nbk) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            cl[b][r] *= sl2;
            if (sN[b * 32 + col_of(r, hh)] > 0.0f) tm = fmaxf(tm, cl[b][r]);
          }
        }
      }
      tm = xhalf_max(tm);
      const float mn = fmaxf(m, tm);
      const float f = exp2f(m - mn);
      zp *= f;
      const float fx = f * (sig / sg);
#pragma unroll
      for (int db = 0; db < DB; ++db) xacc[db] *= fx;
      m = mn;
      sig = sg;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b < nbk) {
#pragma unroll
          for (int g = 0; g < 16 / W; ++g) {
            float sp = 0.0f;
#pragma unroll
            for (int c = 0; c < W; ++c)
              if (c < C) sp += cl[b][g * W + c];
            const float ap = exp2f(sp * invC - m);
#pragma unroll
            for (int c = 0; c < W; ++c) {
              const float n = sN[b * 32 + col_of(g * W + c, hh)];
              const float da = (c < C && n > 0.0f) ? exp2f(cl[b][g * W + c] - m) - ap : 0.0f;
              cl[b][g * W + c] = da;
              zp = fmaf(da, n, zp);
            }
          }
#pragma unroll
          for (int k = 0; k < KV; ++k) {
            pvfrag_t bf;
            if constexpr (KV == 2) bf = k == 0 ? pack_at<T, 0>(cl[b]) : pack_at<T, 8>(cl[b]);
            else bf = cl[b][k];
            const int cofs = b * 32 + 16 * ((k * E) >> 3) + 8 * hh + ((k * E) & 7);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const pvfrag_t af = *(const pvfrag_t*)(sV + (db * 32 + ql) * LDV + cofs);
              xacc[db] = T::mma_pv(af, bf, xacc[db]);
            }
          }
        }
      }
    }
  }

  // ---- Y = x / z (Alg. 2 line 20) -------------------------------------------
  const float zt = xhalf_sum(zp);
  if (qv) {
    const float f = sig / zt;
    float* yp = Y + ((int64_t)bh * N + qi) * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 o = {xacc[db][4 * i] * f, xacc[db][4 * i + 1] * f, xacc[db][4 * i + 2] * f, xacc[db][4 * i + 3] * f};
        *(f32x4*)(yp + db * 32 + 8 * i) = o;
      }
  }
}

size_t attention_smem_bytes(int dtype, int d, int M0, int P, int block_q) {
  const size_t pes = dtype == 0 ? 4 : 2;
  const size_t ldv = 128 + 16 / pes;
  const size_t M0p = (M0 + 31) & ~31;
  const size_t nw = block_q / 32;
  return d * ldv * pes + 128 * 4 + nw * M0p * 4 + M0p * 4 + 8 * 4 + (size_t)(P > 0 ? P : 1) * 4;
}

template <class T, int D, int W>
static hipError_t launch_attn_t(const void* Q, const void* cb, const float* vsum, const int* counts, int BH, int H, int N,
                                int M0, int C, int P, int bq, float scale, float* Y, int* topp, float* importance,
                                hipStream_t st) {
  const size_t smem = attention_smem_bytes(std::is_same<T, TF32>::value ? 0 : 1, D, M0, P, bq);
  auto kern = attention_kernel<T, D, W>;
  hipError_t e = raise_lds_limit((const void*)kern, smem);
  if (e != hipSuccess) return e;
  dim3 grid((N + bq - 1) / bq, BH);
  const float sl2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(kern, grid, dim3(2 * bq), smem, st, (const typename T::in_t*)Q, (const typename T::in_t*)cb,
                     vsum, counts, H, N, M0, C, P, bq, sl2, Y, topp, importance);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_attn_w(const void* Q, const void* cb, const float* vsum, const int* counts, int BH, int H, int N,
                                int M0, int C, int P, int bq, float scale, float* Y, int* topp, float* importance,
                                hipStream_t st) {
  if (C <= 4) return launch_attn_t<T, D, 4>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, st);
  if (C <= 8) return launch_attn_t<T, D, 8>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, st);
  return launch_attn_t<T, D, 16>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, st);
}

hipError_t launch_attention(int dtype, const void* Q, const void* cb, const float* vsum, const int* counts, int BH, int H,
                            int N, int d, int M0, int C, int P, int bq, float scale, float* Y, int* topp,
                            float* importance, hipStream_t st) {
  if (dtype == 0) {
    if (d == 64) return launch_attn_w<TF32, 64>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, st);
    return launch_attn_w<TF32, 128>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, st);
  }
  if (d == 64) return launch_attn_w<TBF16, 64>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, st);
  return launch_attn_w<TBF16, 128>(Q, cb, vsum, counts, BH, H, N, M0, C, P, bq, scale, Y, topp, importance, st);
}

}  // namespace avq
