// Host-side pool object behind lora_pool_t, shared by the C-ABI layer and
// the adapter slot cache (which owns pools whose tables it rewrites as
// adapters move in and out of slots).
#pragma once

#include <vector>

#include "lora_internal.hpp"

struct lora_pool_s {
    lora::PoolDev dev;
    lora_layout_t layout;
    lora_dtype_t dtype;
    std::vector<int32_t> ranks;   // host copy (param counts); a cache pool keeps it current
    void* tables;                 // one device allocation: ranks, a_off, b_off, scales, err
    bool owned_by_cache;          // lora_pool_destroy refuses cache-owned pools
};
