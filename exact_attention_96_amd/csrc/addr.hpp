// 64-bit addresses through 32-bit lane moves.  A wave-uniform address is put in
// scalar registers with v_readfirstlane_b32, whose builtin takes and returns a
// signed 32-bit int, one word at a time.  Each word must be widened back as
// unsigned: a signed widening of the low word copies its bit 31 into the whole
// high word, and the load then reads from an address that was never allocated.
// Plain C++ (no HIP types), so that a host test can compile and check it.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define ATTN_HOST_DEVICE __host__ __device__
#else
#define ATTN_HOST_DEVICE
#endif

namespace attn {

ATTN_HOST_DEVICE inline int addr_lo_word(uint64_t a) { return (int)(uint32_t)a; }
ATTN_HOST_DEVICE inline int addr_hi_word(uint64_t a) { return (int)(uint32_t)(a >> 32); }
ATTN_HOST_DEVICE inline uint64_t addr_join(int lo, int hi) {
    return (uint64_t)(uint32_t)lo | ((uint64_t)(uint32_t)hi << 32);
}

}  // namespace attn
