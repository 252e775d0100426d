// Host helpers shared by the library's C ABI sources (pool.cpp, kvs_mask.cpp).
#pragma once

#include "../../include/leyline.h"

namespace ll {

// Record a message for ll_last_error() on the calling thread; returns s.
ll_status fail(ll_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
const char* last_error();

}  // namespace ll
