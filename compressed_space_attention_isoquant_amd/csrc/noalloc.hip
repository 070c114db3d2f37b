// Decode attention for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// iq_decode_attention with its workspace in a fixed device array of this
// library instead of caller memory.
#include <mutex>

#include "iq.h"
#include "iq_internal.h"

namespace {

// Largest workspace the array serves (the layout of iq_decode_workspace_bytes;
// 64 sequences x 32 query / 4 KV heads at d = 128 need about 20 MiB).
constexpr size_t kScratchBytes = size_t(64) << 20;

// One copy per GPU, held from the library's load until the process ends.
// Host code never uses this name as an address: the device address of each
// GPU's copy comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void *g_scratch_address[kMaxDevices];   // per device, set on its first call
std::mutex g_scratch_mutex;

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current).
int scratch_address(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return IQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_address[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return IQ_ERR_HIP;
    g_scratch_address[dev] = p;
  }
  *ptr = g_scratch_address[dev];
  return IQ_OK;
}

}  // namespace

extern "C" int iq_decode_attention_noalloc(const iq_config *cfg, const void *q, int32_t q_dtype, int32_t batch,
                                           int32_t num_q_heads, const iq_cache *k, const iq_cache *v,
                                           const int32_t *kv_len, int64_t max_kv_len, float softmax_scale,
                                           void *out, int32_t out_dtype, float *lse_out, int32_t *argmax_out,
                                           hipStream_t stream) {
  size_t need = 0;
  const int st = iq::decode_workspace_check(cfg, batch, num_q_heads, max_kv_len, &need);
  if (st != IQ_OK) return st;
  if (need > kScratchBytes) return IQ_ERR_WORKSPACE;
  void *ws = nullptr;
  const int sst = scratch_address(&ws);
  if (sst != IQ_OK) return sst;
  // Every part of the workspace a call reads is written earlier in the same
  // call (plan, rotated queries, records), so nothing needs clearing.
  return iq_decode_attention(cfg, q, q_dtype, batch, num_q_heads, k, v, kv_len, max_kv_len, softmax_scale, out,
                             out_dtype, lse_out, argmax_out, ws, kScratchBytes, stream);
}
