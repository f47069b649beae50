// A 64-bit device address as the two 32-bit words that scalar registers hold, and back.  Host
// and device share these, so the split can be checked by an ordinary C++ compiler on the host.
// The lane-broadcast builtin (readfirstlane) returns int: a word taken through it goes back to
// unsigned before it is widened, or a low word >= 2^31 would sign-extend into the high word.
#pragma once

#ifdef __HIPCC__
#define AW_HD __host__ __device__ __forceinline__
#else
#define AW_HD inline
#endif

namespace dm {

AW_HD unsigned addr_lo(unsigned long long a) { return (unsigned)a; }
AW_HD unsigned addr_hi(unsigned long long a) { return (unsigned)(a >> 32); }
AW_HD unsigned long long addr_join(unsigned lo, unsigned hi) { return ((unsigned long long)hi << 32) | lo; }

}  // namespace dm
