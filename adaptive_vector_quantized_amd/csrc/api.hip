// C interface of libavq: argument validation on the host, then the launches.
// The contract of every entry point is documented in include/avq.h.
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <unordered_map>

#include "../../include/avq.h"
#include "avq_launch.h"

namespace {

constexpr int kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_common(int B, int H, int N, int d, int M0, int C, int dtype) {
  if (dtype != AVQ_F32 && dtype != AVQ_BF16) return AVQ_ERR_DTYPE;
  if (B < 0 || H < 0 || N < 0) return AVQ_ERR_SHAPE;
  if (d < 1 || M0 < 1 || C < 0) return AVQ_ERR_SHAPE;
  if (d != 64 && d != 128) return AVQ_ERR_UNSUPPORTED;
  if (M0 > 512 || C > 16) return AVQ_ERR_UNSUPPORTED;
  if ((int64_t)B * H > 65535) return AVQ_ERR_UNSUPPORTED;
  return AVQ_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? AVQ_OK : AVQ_ERR_HIP; }

}  // namespace

namespace avq {

hipError_t raise_lds_limit(const void* kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  static std::mutex mu;
  static std::unordered_map<const void*, size_t> done;
  std::lock_guard<std::mutex> lock(mu);
  auto it = done.find(kernel);
  if (it != done.end() && it->second >= bytes) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done[kernel] = bytes;
  return e;
}

}  // namespace avq

namespace {

int assign_call(const void* K, const void* V, const void* codebook, int B, int H, int N, int d, int M0, int C,
                int dtype, float* vsum, int32_t* counts, int32_t* assign, float* ksum, bool with_keys, void* stream) {
  int rc = check_common(B, H, N, d, M0, C, dtype);
  if (rc != AVQ_OK) return rc;
  const int64_t BH = (int64_t)B * H;
  if (BH == 0) return AVQ_OK;
  if (!vsum || !counts || !codebook || (with_keys && !ksum)) return AVQ_ERR_NULL;
  if (N > 0 && (!K || !V)) return AVQ_ERR_NULL;
  if (!aligned16(vsum) || !aligned16(counts) || !aligned16(codebook) || (K && !aligned16(K)) ||
      (V && !aligned16(V)) || (assign && !aligned16(assign)) || (ksum && !aligned16(ksum)))
    return AVQ_ERR_ALIGN;
  if (avq::assign_smem_bytes(dtype, d, M0, C) > (size_t)kMaxLds) return AVQ_ERR_UNSUPPORTED;
  const int64_t Mt = (int64_t)M0 * (1 + C);
  hipStream_t st = (hipStream_t)stream;
  rc = from_hip(avq::launch_zero(vsum, BH * Mt * d, with_keys ? ksum : nullptr, with_keys ? BH * Mt * d : 0, counts,
                                 BH * Mt, st));
  if (rc != AVQ_OK || N == 0) return rc;
  return from_hip(avq::launch_assign(dtype, K, V, codebook, (int)BH, H, N, d, M0, C, vsum, counts, assign,
                                     with_keys ? ksum : nullptr, st));
}

}  // namespace

extern "C" {

int avq_assign_aggregate(const void* K, const void* V, const void* codebook, int B, int H, int N, int d, int M0, int C,
                         int dtype, float* vsum, int32_t* counts, int32_t* assign, void* stream) {
  return assign_call(K, V, codebook, B, H, N, d, M0, C, dtype, vsum, counts, assign, nullptr, false, stream);
}

int avq_assign_aggregate_kv(const void* K, const void* V, const void* codebook, int B, int H, int N, int d, int M0,
                            int C, int dtype, float* vsum, int32_t* counts, int32_t* assign, float* ksum,
                            void* stream) {
  return assign_call(K, V, codebook, B, H, N, d, M0, C, dtype, vsum, counts, assign, ksum, true, stream);
}

size_t avq_attention_workspace_size(int B, int H, int d, int M0, int C, int dtype) {
  if (check_common(B, H, 0, d, M0, C, dtype) != AVQ_OK) return 0;
  return avq::attention_workspace_bytes(dtype, d, M0, C, B * H);
}

}  // extern "C"

namespace {

int attention_call(const void* Q, const void* codebook, const float* vsum, const int32_t* counts, int B, int H, int N,
                   int d, int M0, int C, int dtype, int P, int block_q, float scale, float* Y, int32_t* topp,
                   float* importance, void* workspace, size_t workspace_bytes, void* stream, bool approx,
                   const int32_t* order, bool ordered) {
  int rc = check_common(B, H, N, d, M0, C, dtype);
  if (rc != AVQ_OK) return rc;
  if (P < 0 || P > M0 || (C == 0 && P > 0)) return AVQ_ERR_SHAPE;  // no children to refine with
  if (block_q != 32 && block_q != 64 && block_q != 128) return AVQ_ERR_UNSUPPORTED;
  if (!isfinite(scale) || !(scale > 0.0f)) return AVQ_ERR_SHAPE;
  const int64_t BH = (int64_t)B * H;
  if (BH == 0 || N == 0) return AVQ_OK;
  if (!Q || !codebook || !vsum || !counts || !Y || !workspace || (ordered && !order)) return AVQ_ERR_NULL;
  if (!aligned16(Q) || !aligned16(codebook) || !aligned16(vsum) || !aligned16(counts) || !aligned16(Y) ||
      !aligned16(workspace) || (topp && !aligned16(topp)) || (importance && !aligned16(importance)) ||
      ((uintptr_t)order & 3u) != 0)
    return AVQ_ERR_ALIGN;
  if (workspace_bytes < avq::attention_workspace_bytes(dtype, d, M0, C, (int)BH)) return AVQ_ERR_WORKSPACE;
  if (avq::attention_smem_bytes(dtype, d, M0, C, P, block_q, importance != nullptr) > (size_t)kMaxLds)
    return AVQ_ERR_UNSUPPORTED;
  return from_hip(avq::launch_attention(dtype, Q, codebook, vsum, counts, (int)BH, H, N, d, M0, C, P, block_q, scale,
                                        Y, topp, importance, workspace, approx, order, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int avq_attention_fwd(const void* Q, const void* codebook, const float* vsum, const int32_t* counts, int B, int H,
                      int N, int d, int M0, int C, int dtype, int P, int block_q, float scale, float* Y,
                      int32_t* topp, float* importance, void* workspace, size_t workspace_bytes, void* stream) {
  return attention_call(Q, codebook, vsum, counts, B, H, N, d, M0, C, dtype, P, block_q, scale, Y, topp, importance,
                        workspace, workspace_bytes, stream, false, nullptr, false);
}

int avq_attention_fwd_approx(const void* Q, const void* codebook, const float* vsum, const int32_t* counts, int B,
                             int H, int N, int d, int M0, int C, int dtype, int P, int block_q, float scale, float* Y,
                             int32_t* topp, float* importance, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return attention_call(Q, codebook, vsum, counts, B, H, N, d, M0, C, dtype, P, block_q, scale, Y, topp, importance,
                        workspace, workspace_bytes, stream, true, nullptr, false);
}

int avq_attention_fwd_ordered(const void* Q, const void* codebook, const float* vsum, const int32_t* counts, int B,
                              int H, int N, int d, int M0, int C, int dtype, int P, int block_q, float scale,
                              const int32_t* query_order, int approx_denominator, float* Y, int32_t* topp,
                              float* importance, void* workspace, size_t workspace_bytes, void* stream) {
  return attention_call(Q, codebook, vsum, counts, B, H, N, d, M0, C, dtype, P, block_q, scale, Y, topp, importance,
                        workspace, workspace_bytes, stream, approx_denominator != 0, query_order, true);
}

int avq_codebook_update(const float* ksum, const int32_t* counts, int B, int H, int d, int M0, int C, float decay,
                        float* S, float* Nema, float* codebook, void* stream) {
  if (B < 0 || H < 0 || d < 1 || M0 < 1 || C < 0) return AVQ_ERR_SHAPE;
  if (!(decay >= 0.0f && decay <= 1.0f)) return AVQ_ERR_SHAPE;  // NaN included
  if (C > 16 || (int64_t)H * M0 > (int64_t)1 << 30) return AVQ_ERR_UNSUPPORTED;
  if (H == 0) return AVQ_OK;
  if (!S || !Nema || !codebook || (B > 0 && (!ksum || !counts))) return AVQ_ERR_NULL;
  auto a4 = [](const void* q) { return ((uintptr_t)q & 3u) == 0; };
  if (!a4(S) || !a4(Nema) || !a4(codebook) || !a4(ksum) || !a4(counts)) return AVQ_ERR_ALIGN;
  return from_hip(avq::launch_codebook_update(ksum, counts, B, H, d, M0, C, decay, S, Nema, codebook,
                                              (hipStream_t)stream));
}

const char* avq_status_string(int status) {
  switch (status) {
    case AVQ_OK: return "ok";
    case AVQ_ERR_NULL: return "a required pointer is NULL";
    case AVQ_ERR_SHAPE: return "a size is out of range";
    case AVQ_ERR_DTYPE: return "unknown dtype";
    case AVQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case AVQ_ERR_UNSUPPORTED: return "unsupported size (d, M0, C, block_q, B*H or H*M0)";
    case AVQ_ERR_HIP: return "HIP runtime error";
    case AVQ_ERR_WORKSPACE: return "workspace smaller than avq_attention_workspace_size()";
    default: return "unknown status";
  }
}

int avq_version(void) { return 100; }

}  // extern "C"
