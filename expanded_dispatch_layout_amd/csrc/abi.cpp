// Host-only entry points of libmoe_expand: status text and the capacity
// bound.  Nothing here touches the GPU.
#include <stdint.h>

#include "moe_expand.h"

extern "C" const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MOE_ERR_ALIGNMENT: return "a pointer or stride is not suitably aligned";
    case MOE_ERR_UNSUPPORTED: return "unsupported argument combination";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_SCRATCH:
      return "the sizes need more workspace than moe_expand_layout_noalloc's static scratch "
             "holds (MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

// Largest padded row total over every routing of rows*topk assignments onto
// num_experts experts with blocks rounded up to `align` rows (SGLang
// moe_runner/deep_gemm.py source, _get_compact_all_tokens): with
// n = min(A, E) non-empty experts each taking one assignment and one block,
// the other A - n assignments add one block per `align`.
extern "C" int64_t moe_expand_capacity(int64_t rows, int topk, int num_experts, int align) {
  if (rows < 0 || topk < 1 || num_experts < 1 || align < 1) return -1;
  const int64_t a = rows * (int64_t)topk;
  const int64_t n = a < num_experts ? a : num_experts;
  return (int64_t)align * (n + (a - n) / align);
}
