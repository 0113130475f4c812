// The decode GEMV's bfloat16 instances (the kernel is in mnb_gemv_kernel.h).
#include "mnb_gemv_kernel.h"

namespace mnb {

GemvFn gemv_pick_bf16(bool has_zp, bool has_bias, int CB, int J, int W, bool silu, int input, bool nts) {
    return pick_type<true>(has_zp, has_bias, CB, J, W, silu, input, nts);
}

GemvFn gemv_pick_rows_bf16(bool has_zp, bool has_bias, int MR, int J, int W, bool nts) {
    return pick_rows_type<true>(has_zp, has_bias, MR, J, W, nts);
}

}  // namespace mnb
