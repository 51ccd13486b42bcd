// C interface of libavq: argument validation on the host, then the launches.
// The contract of every entry point is documented in include/avq.h.
#include <math.h>
#include <stdint.h>

#include <map>
#include <mutex>

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

// The largest dynamic LDS size already allowed for each (device, kernel):
// the attribute is set once per device and kernel (and again only for a
// larger size), under a lock, since calls may come from several host threads.
hipError_t raise_lds_limit(const void* kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> done;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, kernel);
  auto it = done.find(key);
  if (it != done.end() && it->second >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done[key] = bytes;
  return e;
}

}  // namespace avq

namespace {

// zero: fill vsum, counts (and ksum) with zeros first; else add this batch's
// sums and counts to what they hold
int assign_call(const void* K, const void* V, const void* codebook, int B, int H, int N, int d, int M0, int C,
                int dtype, float* vsum, int32_t* counts, int32_t* assign, float* ksum, bool with_keys, void* stream,
                bool zero = true) {
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
  if (zero) {
    rc = from_hip(avq::launch_zero(vsum, BH * Mt * d, with_keys ? ksum : nullptr, with_keys ? BH * Mt * d : 0, counts,
                                   BH * Mt, st));
    if (rc != AVQ_OK) return rc;
  }
  if (N == 0) return AVQ_OK;
  return from_hip(avq::launch_assign(dtype, K, V, codebook, (int)BH, H, N, d, M0, C, vsum, counts, assign,
                                     with_keys ? ksum : nullptr, st));
}

}  // namespace

extern "C" {

int avq_assign_aggregate(const void* K, const void* V, const void* codebook, int B, int H, int N, int d, int M0, int C,
                         int dtype, float* vsum, int32_t* counts, int32_t* assign, void* stream) {
  return assign_call(K, V, codebook, B, H, N, d, M0, C, dtype, vsum, counts, assign, nullptr, false, stream);
}

int avq_assign_aggregate_accum(const void* K, const void* V, const void* codebook, int B, int H, int N, int d, int M0,
                               int C, int dtype, float* vsum, int32_t* counts, int32_t* assign, void* stream) {
  return assign_call(K, V, codebook, B, H, N, d, M0, C, dtype, vsum, counts, assign, nullptr, false, stream, false);
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

// stages: avq::kAttnPrep (value fragments from vsum, and a copy of counts,
// into the workspace) and/or avq::kAttnKernel (the attention kernel, from a
// prepared workspace, optionally zero-filling clear_v and clear_c); vsum and
// counts are needed by the first, Q, codebook and Y by the second
int attention_call(const void* Q, const void* codebook, const float* vsum, const int32_t* counts, int B, int H, int N,
                   int d, int M0, int C, int dtype, int P, int block_q, float scale, float* Y, int32_t* topp,
                   float* importance, void* workspace, size_t workspace_bytes, void* stream, bool approx,
                   const int32_t* order, bool ordered, bool validate_only = false,
                   int stages = avq::kAttnPrep | avq::kAttnKernel, float* clear_v = nullptr,
                   int32_t* clear_c = nullptr) {
  const bool prep = (stages & avq::kAttnPrep) != 0, kern = (stages & avq::kAttnKernel) != 0;
  int rc = check_common(B, H, N, d, M0, C, dtype);
  if (rc != AVQ_OK) return rc;
  if (kern) {
    if (P < 0 || P > M0 || (C == 0 && P > 0)) return AVQ_ERR_SHAPE;  // no children to refine with
    if (block_q != 32 && block_q != 64 && block_q != 128) return AVQ_ERR_UNSUPPORTED;
    if (!isfinite(scale) || !(scale > 0.0f)) return AVQ_ERR_SHAPE;
  }
  const int64_t BH = (int64_t)B * H;
  if (BH == 0) return AVQ_OK;
  if (kern && N == 0) {  // no queries: nothing to attend, only the requested clearing
    if (!clear_v && !clear_c) return AVQ_OK;
    if ((clear_v && !aligned16(clear_v)) || (clear_c && !aligned16(clear_c))) return AVQ_ERR_ALIGN;
    if (validate_only) return AVQ_OK;
    const int64_t Mt = (int64_t)M0 * (1 + C);
    return from_hip(avq::launch_zero(clear_v, clear_v ? BH * Mt * d : 0, nullptr, 0, clear_c, clear_c ? BH * Mt : 0,
                                     (hipStream_t)stream));
  }
  if (!workspace || (prep && (!vsum || !counts)) || (kern && (!Q || !codebook || !Y || (ordered && !order))))
    return AVQ_ERR_NULL;
  if ((Q && !aligned16(Q)) || (codebook && !aligned16(codebook)) || (vsum && !aligned16(vsum)) ||
      (counts && !aligned16(counts)) || (Y && !aligned16(Y)) || (clear_v && !aligned16(clear_v)) ||
      (clear_c && !aligned16(clear_c)) || !aligned16(workspace) || (topp && !aligned16(topp)) ||
      (importance && !aligned16(importance)) || ((uintptr_t)order & 3u) != 0)
    return AVQ_ERR_ALIGN;
  if (workspace_bytes < avq::attention_workspace_bytes(dtype, d, M0, C, (int)BH)) return AVQ_ERR_WORKSPACE;
  if (kern && avq::attention_smem_bytes(dtype, d, M0, C, P, block_q, importance != nullptr) > (size_t)kMaxLds)
    return AVQ_ERR_UNSUPPORTED;
  if (validate_only) return AVQ_OK;
  return from_hip(avq::launch_attention(dtype, Q, codebook, vsum, counts, (int)BH, H, N, d, M0, C, P, block_q, scale,
                                        Y, topp, importance, workspace, approx, order, stages, clear_v, clear_c,
                                        (hipStream_t)stream));
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

int avq_attention_prepare(const float* vsum, const int32_t* counts, int B, int H, int d, int M0, int C, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return attention_call(nullptr, nullptr, vsum, counts, B, H, 0, d, M0, C, dtype, 0, 32, 1.0f, nullptr, nullptr,
                        nullptr, workspace, workspace_bytes, stream, false, nullptr, false, false, avq::kAttnPrep);
}

int avq_attention_fwd_prepared(const void* Q, const void* codebook, int B, int H, int N, int d, int M0, int C,
                               int dtype, int P, int block_q, float scale, float* Y, int32_t* topp, float* importance,
                               const void* workspace, size_t workspace_bytes, float* clear_vsum,
                               int32_t* clear_counts, void* stream) {
  return attention_call(Q, codebook, nullptr, nullptr, B, H, N, d, M0, C, dtype, P, block_q, scale, Y, topp,
                        importance, const_cast<void*>(workspace), workspace_bytes, stream, false, nullptr, false,
                        false, avq::kAttnKernel, clear_vsum, clear_counts);
}

}  // extern "C"

// ---- the attention call without a caller workspace --------------------------
// Scratch for avq_attention_fwd_noalloc: the operands avq_attention_fwd keeps
// in its workspace (a value scale per (batch, head) and the value sums as fp16
// fragments), in a static array every GPU the library runs on holds from the
// library's load to the end of the process.  Host code never uses the array's
// name as an address: its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[AVQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// device address of this GPU's scratch (the current device), or nullptr
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int avq_attention_fwd_noalloc(const void* Q, const void* codebook, const float* vsum, const int32_t* counts, int B,
                              int H, int N, int d, int M0, int C, int dtype, int P, int block_q, float scale,
                              float* Y, int32_t* topp, float* importance, void* stream) {
  // the arguments of avq_attention_fwd are checked first (with a stand-in
  // workspace of the right size, so only the scratch limit is left)
  const size_t need = avq_attention_workspace_size(B, H, d, M0, C, dtype);
  static unsigned char probe[16] __attribute__((aligned(16)));
  int rc = attention_call(Q, codebook, vsum, counts, B, H, N, d, M0, C, dtype, P, block_q, scale, Y, topp,
                          importance, probe, need, stream, false, nullptr, false, /*validate_only=*/true);
  if (rc != AVQ_OK) return rc;
  if ((int64_t)B * H == 0 || N == 0) return AVQ_OK;
  if (need > (size_t)AVQ_NOALLOC_SCRATCH_BYTES) return AVQ_ERR_SCRATCH;
  void* ws = device_scratch();
  if (ws == nullptr) return AVQ_ERR_HIP;
  return attention_call(Q, codebook, vsum, counts, B, H, N, d, M0, C, dtype, P, block_q, scale, Y, topp, importance,
                        ws, need, stream, false, nullptr, false, false);
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
    case AVQ_ERR_SCRATCH: return "the call needs more than the library's static scratch (AVQ_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int avq_version(void) { return 100; }

}  // extern "C"
