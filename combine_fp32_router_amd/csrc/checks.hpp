// Host-side argument checks shared by the C entry points of the product
// library (abi.cpp) and of the test-support library (harness.hip).  Each
// returns a moe_status code; nothing here touches the GPU.
#pragma once

#include <stdint.h>

#include "../../include/moe_route.h"

namespace moe {

inline bool aligned(const void *p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

constexpr int64_t kMaxSlots = int64_t(1) << 31;  // T*k must fit an int32 row index

// T*k >= kMaxSlots for T >= 0 and k >= 1, without forming T*k (a caller's
// T near the int64 range would overflow the product).
inline bool too_many_slots(int64_t T, int k) { return T > (kMaxSlots - 1) / k; }

inline int check_ek(int E, int k)
{
    if (E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK)
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

inline int check_rows(int64_t T, int H, int k, int quant)
{
    if (T < 0 || k < 1 || k > MOE_MAX_TOPK || H < 16 || H > MOE_MAX_HIDDEN || (H % 16) != 0 ||
        (quant != MOE_QUANT_BF16 && quant != MOE_QUANT_INT8 && quant != MOE_QUANT_INT4 &&
         quant != MOE_QUANT_FP8) ||
        (quant == MOE_QUANT_INT4 && (H % 32) != 0) || too_many_slots(T, k))
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

inline int check_er(int E, int R)
{
    if (E < 1 || E > MOE_MAX_EXPERTS || R < 1 || (E % R) != 0)
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

// Scale array of a quantised row buffer: required (4-byte aligned) when
// quant != bf16 and the call moves rows; ignored for bf16.
inline int check_scales(const void *scales, int quant)
{
    if (quant == MOE_QUANT_BF16)
        return MOE_OK;
    if (!scales)
        return MOE_ERR_NULL;
    if (!aligned(scales, 4))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

}  // namespace moe
