// Device helpers shared by the kernels' translation units.  Not part of the
// C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

// d << L and d >> R of the code dword pair (d0, d1) taken as one 64-bit value
// (d0 low): one 64-bit shift yields both dwords' copies, where two 32-bit
// shifts did.  Bits that cross between the dwords land in bits [0, L) of the
// high dword of d << L and bits [32 - R, 32) of the low dword of d >> R.  The
// decodes read only bits [6, 12) and [22, 28) of d << 6, and bits [8, 12) and
// [24, 28) (ternary, binary: R = 4) or [4, 10) and [20, 26) (affine: R = 6)
// of d >> R, so the crossed bits are always masked off.
template <int L, int R>
__device__ __forceinline__ void shifts64(uint32_t d0, uint32_t d1, uint32_t (&l)[2], uint32_t (&r)[2]) {
    const uint64_t w = ((uint64_t)d1 << 32) | d0;
    uint64_t wl, wr;
    // written out: the compiler splits a right shift whose halves are used
    // apart into an alignbit and a 32-bit shift
    asm("v_lshlrev_b64 %0, %2, %1" : "=v"(wl) : "v"(w), "i"(L));
    asm("v_lshrrev_b64 %0, %2, %1" : "=v"(wr) : "v"(w), "i"(R));
    l[0] = (uint32_t)wl;
    l[1] = (uint32_t)(wl >> 32);
    r[0] = (uint32_t)wr;
    r[1] = (uint32_t)(wr >> 32);
}

}  // namespace tq
