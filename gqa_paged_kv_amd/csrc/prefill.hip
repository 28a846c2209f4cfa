// Causal GQA prefill (bf16 MFMA) -- placeholder until the MFMA kernel lands.
#include <hip/hip_runtime.h>
#include "../../include/gqa.h"
namespace gqa {
int launch_prefill(const void*, const void*, const void*, void*, int, int, int, int, int, float,
                   hipStream_t) {
  return GQA_ERR_UNSUPPORTED;
}
}  // namespace gqa
