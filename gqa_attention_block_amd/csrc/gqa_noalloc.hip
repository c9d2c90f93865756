// The decode block without a caller workspace (gqa_attention_block_decode_noalloc):
// for callers that cannot allocate device memory at all -- code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc.
//
// The block's workspace (RoPE'd q, gate logits, gated attention, the split-K
// partials) lives in one file-scope device array of fixed size.  The runtime
// places a copy of it on every GPU the library runs on when the code object
// is loaded there, and that copy stays until the process ends.  In host code
// the array's name is only a stand-in for the host: its device address comes
// from hipGetSymbolAddress, taken once per device with that device current,
// and that address is what the kernels receive.  Nothing here allocates.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gqa.h"
#include "gqa_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;   // 8 MiB per GPU
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];   // device address of each GPU's copy, or null before set-up

// The device address of the current device's scratch, looked up on the first
// call on that device.  Returns GQA_OK or GQA_ERR_GPU with the HIP error.
gqa_status scratch_for_current_device(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return gqa::report(GQA_ERR_GPU, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return gqa::report(GQA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                       kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return gqa::report(GQA_ERR_GPU, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                         hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status gqa_attention_block_decode_noalloc(const gqa_arch *arch, const gqa_layer_weights *weights,
                                              int is_full, const gqa_kv_seq *seqs, int32_t batch,
                                              const float *x_normed, float *out, void *stream) {
  size_t need = 0;
  gqa_status st = gqa::block_workspace_need(arch, weights, is_full, seqs, batch, &need);
  if (st != GQA_OK) return st;
  if (need > kScratchBytes)
    return gqa::report(GQA_ERR_WORKSPACE_TOO_SMALL,
                       "the block needs %zu bytes of scratch for these sequences; the static scratch of "
                       "gqa_attention_block_decode_noalloc holds %zu (use gqa_attention_block_decode with a "
                       "caller workspace)",
                       need, kScratchBytes);
  if (batch == 0) return gqa_attention_block_decode(arch, weights, is_full, seqs, batch, x_normed, out, nullptr, 0,
                                                    stream);
  void *ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != GQA_OK) return st;
  return gqa_attention_block_decode(arch, weights, is_full, seqs, batch, x_normed, out, ws, kScratchBytes, stream);
}

}  // extern "C"
