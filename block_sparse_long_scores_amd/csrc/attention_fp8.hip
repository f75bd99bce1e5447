// fp8 instantiations of the attention kernel (attention_kernel.h).
#include "attention_kernel.h"

namespace fp2 {

size_t attention_lds_bytes_fp8(int D, int block, int nkb) {
  if (D == 128 && block == 128) return attn_lds_bytes<128, 128, true>(nkb);
  if (D == 128 && block == 64) return attn_lds_bytes<128, 64, true>(nkb);
  if (D == 64 && block == 128) return attn_lds_bytes<64, 128, true>(nkb);
  if (D == 64 && block == 64) return attn_lds_bytes<64, 64, true>(nkb);
  return 0;
}

hipError_t launch_attention_fp8(const AttnArgs& a, int D, int block, hipStream_t st) {
  if (D == 128 && block == 128) return launch_t<128, 128, true>(a, st);
  if (D == 128 && block == 64) return launch_t<128, 64, true>(a, st);
  if (D == 64 && block == 128) return launch_t<64, 128, true>(a, st);
  if (D == 64 && block == 64) return launch_t<64, 64, true>(a, st);
  return hipErrorNotSupported;
}

}  // namespace fp2
