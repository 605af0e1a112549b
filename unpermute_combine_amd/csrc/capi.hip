// Host-only entry points of the C ABI: status names and the expert capacity.
#include "moe_common.h"

extern "C" const char *moe_status_string(moe_status s)
{
    switch (s) {
    case MOE_OK:
        return "ok";
    case MOE_ERR_INVALID:
        return "invalid argument";
    case MOE_ERR_UNSUPPORTED:
        return "unsupported size or combination";
    case MOE_ERR_HIP:
        return "HIP launch error";
    }
    return "unknown status";
}

// [Scratch] §18 ("从零理解 MoE 算子"): expert_capacity = ceil(tokens * top_k / num_experts *
// capacity_factor); the factor is the exact fraction cf_num / cf_den, the ceiling is integral.
extern "C" int64_t moe_expert_capacity(int64_t tokens, int32_t top_k, int32_t num_experts, int32_t cf_num,
                                       int32_t cf_den)
{
    if (tokens < 0 || top_k < 1 || num_experts < 1 || cf_num < 0 || cf_den < 1)
        return -1;
    if (tokens > (int64_t{1} << 40))
        return -1;
    const __int128 num = static_cast<__int128>(tokens) * top_k * cf_num;
    const __int128 den = static_cast<__int128>(num_experts) * cf_den;
    const __int128 cap = (num + den - 1) / den;
    return cap > 0x7fffffff ? -1 : static_cast<int64_t>(cap);
}
