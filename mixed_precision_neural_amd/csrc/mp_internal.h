// Internal helpers of libmp (HIP side only). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mp.h"

namespace mp {

// Native clang vectors (usable with the non-temporal builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Pointers in the global address space: loads and stores through them become
// global_* instructions rather than flat_* ones.
template <class T>
using gptr_t = __attribute__((address_space(1))) T*;
template <class T>
__device__ __forceinline__ gptr_t<T> global(T* p) {
    return (gptr_t<T>)(p);
}

// Records `e` as the thread's last HIP error and maps it to a status.
mp_status hip_status(hipError_t e, const char* where);

// Status of the most recent launch on this thread.
inline mp_status launch_status(const char* where) {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MP_OK : hip_status(e, where);
}

inline hipStream_t as_stream(mp_stream s) { return reinterpret_cast<hipStream_t>(s); }

// ---- binary16 helpers (device) -------------------------------------------
// Decode is exact (v_cvt_f32_f16 keeps subnormals); encode rounds to nearest
// even with gradual underflow and overflow to +-inf (v_cvt_f16_f32 under the
// default round-to-nearest mode, denormals enabled).
__device__ __forceinline__ float h2f(uint16_t h) {
    _Float16 x = __builtin_bit_cast(_Float16, h);
    return static_cast<float>(x);
}
// The FP32 value is pinned in a register first (an empty asm the optimiser
// cannot see through), so the conversion is never merged with the operation
// that produced the value: a mixed-precision v_fma_mix*_f16 would round the
// exact product once, where every caller means "round to FP32, then to
// binary16". Without the pin the compiler picks either form depending on the
// surrounding code, and two kernels evaluating the same expression can differ
// in the last bit when the FP32 result is a binary16 tie.
__device__ __forceinline__ uint16_t f2h(float f) {
    asm("" : "+v"(f));
    _Float16 x = static_cast<_Float16>(f);
    return __builtin_bit_cast(uint16_t, x);
}
// Two values at once, a in the low half: one v_cvt_pk_f16_f32, the same
// rounding per element as f2h (both inputs pinned the same way).
__device__ __forceinline__ uint32_t f2h2(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    asm("" : "+v"(a));
    asm("" : "+v"(b));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}
// 1 when either binary16 half of the word has an all-ones exponent (inf/NaN).
__device__ __forceinline__ uint32_t nonfinite2(uint32_t w) {
    return ((w & 0x7C00u) == 0x7C00u) | ((w & 0x7C000000u) == 0x7C000000u);
}
__device__ __forceinline__ uint32_t nonfinite1(uint16_t h) {
    return (h & 0x7C00u) == 0x7C00u;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// A device word the kernels update atomically or read as a whole (flags, scaler, maxima).
inline bool misaligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) != 0; }

}  // namespace mp
