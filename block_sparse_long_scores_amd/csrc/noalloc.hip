// Allocation-free block selection: fp2_select_blocks with its workspace (the
// pooled query blocks) in a static device array of the library instead of a
// caller buffer, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
// The operation is the one fp2_select_blocks computes ("FlashPrefill V2:
// block-sparse prefill attention for long-context LLM serving", abstract:
// pattern discovery and max-based dynamic thresholding); the same kernels run.
//
// The array is a file-scope __device__ symbol: each GPU the library runs on
// holds its own copy for the life of the process.  Its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever handed to kernels.  The pool kernel writes
// every pooled query block the select kernel then reads, so nothing needs
// clearing between calls.  Every call on one GPU shares the array: calls that
// overlap in time on one GPU (different streams, or a captured graph replayed
// next to an eager call) race on it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "fp2.h"
#include "fp2_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per GPU
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_status[kMaxDevices];

}  // namespace

extern "C" fp2_status fp2_select_blocks_noalloc(const fp2_params* p, int32_t batch, int32_t seqlen_q,
                                                int32_t seqlen_k, const void* q, const void* k, const void* v,
                                                int32_t* block_idx, int32_t* block_cnt, float* pooled_k,
                                                float* pooled_v, void* stream) {
  const size_t need = fp2_select_workspace_size(p, batch, seqlen_q, seqlen_k);
  if (need == 0)  // invalid parameters or sizes: the regular entry point reports which
    return fp2_select_blocks(p, batch, seqlen_q, seqlen_k, q, k, v, block_idx, block_cnt, pooled_k, pooled_v,
                             nullptr, 0, stream);
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "fp2_select_blocks_noalloc: this call needs %zu bytes of scratch, the static scratch holds %zu "
             "(use fp2_select_blocks with a workspace)",
             need, kScratchBytes);
    return (fp2_status)fp2::set_last_error(FP2_EUNSUPPORTED, msg);
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    char msg[256];
    snprintf(msg, sizeof msg, "fp2_select_blocks_noalloc: no usable current device (%d): %s", dev,
             hipGetErrorString(e));
    return (fp2_status)fp2::set_last_error(FP2_EDEVICE, msg);
  }
  // set-up, once per device with that device current: the device address of
  // this GPU's copy of the array (the host-side name is not a device address)
  std::call_once(g_once[dev], [dev] { g_status[dev] = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch)); });
  if (g_status[dev] != hipSuccess || g_ptr[dev] == nullptr) {
    char msg[256];
    snprintf(msg, sizeof msg, "fp2_select_blocks_noalloc: hipGetSymbolAddress failed on device %d: %s", dev,
             hipGetErrorString(g_status[dev]));
    return (fp2_status)fp2::set_last_error(FP2_EDEVICE, msg);
  }
  return fp2_select_blocks(p, batch, seqlen_q, seqlen_k, q, k, v, block_idx, block_cnt, pooled_k, pooled_v,
                           g_ptr[dev], kScratchBytes, stream);
}
