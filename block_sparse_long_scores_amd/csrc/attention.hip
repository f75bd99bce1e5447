// Precision dispatch of the attention kernel (instantiated in attention_bf16.hip and
// attention_fp8.hip, which are compiled with different code-generation options).
#include "fp2_internal.h"

namespace fp2 {

size_t attention_lds_bytes(int D, int block, int nkb, int fp8) {
  return fp8 ? attention_lds_bytes_fp8(D, block, nkb) : attention_lds_bytes_bf16(D, block, nkb);
}

hipError_t launch_attention(const AttnArgs& a, int D, int block, int fp8, hipStream_t st) {
  return fp8 ? launch_attention_fp8(a, D, block, st) : launch_attention_bf16(a, D, block, st);
}

}  // namespace fp2
