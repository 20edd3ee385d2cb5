// Workspace alignment shared by the resolve and top-k layouts of libhisparse.
#pragma once

#include <stddef.h>

namespace hsp {

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace hsp
