// Measurement probes (libmp_probe.so): achievable HBM stream rates, and the
// shader clock and binary16 MFMA rate under a matrix-core load with constant
// or random operands. They give the measured
// denominators beside the datasheet peaks for the hot path's kernels, whose
// bounds the source names: point-wise work and weight updates limited by
// memory bandwidth or latency, dot products by arithmetic ("Mixed Precision
// Training", long-form analysis page, §3.4 "FP16 Arithmetic with FP32
// Accumulation" and §6.1 "Speedup Claims").
#include "mp_probe.h"
#include "mp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kPer = 4;                                 // 16-byte vectors in flight per lane
constexpr int64_t kBlockVecs = int64_t(kThreads) * kPer;   // 16 KiB per block and round

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ mp::u32x4 ld(const mp::u32x4* p) {
    if (NT) return __builtin_nontemporal_load(mp::global(p));
    return *mp::global(p);
}
template <bool NT>
__device__ __forceinline__ void st(mp::u32x4* p, mp::u32x4 v) {
    if (NT) __builtin_nontemporal_store(v, mp::global(p));
    else *mp::global(p) = v;
}

// One round covers kBlockVecs vectors from `base`: lane t takes base + t + 256 u.
template <int MODE, bool NT>
__global__ __launch_bounds__(kThreads) void hbm_kernel(const mp::u32x4* __restrict__ src,
                                                       mp::u32x4* __restrict__ dst, int64_t nvec,
                                                       int persistent) {
    const int t = threadIdx.x;
    const int64_t step = persistent ? int64_t(gridDim.x) * kBlockVecs : nvec;
    uint32_t acc = 0;
    for (int64_t base = int64_t(blockIdx.x) * kBlockVecs; base < nvec; base += step) {
        if (base + kBlockVecs <= nvec) {
            if (MODE == MP_PROBE_WRITE) {
                const mp::u32x4 v = {uint32_t(base), uint32_t(t), 0x3C003C00u, 0x3C003C00u};
#pragma unroll
                for (int u = 0; u < kPer; ++u) st<NT>(dst + base + t + u * kThreads, v);
            } else {
                mp::u32x4 v[kPer];
#pragma unroll
                for (int u = 0; u < kPer; ++u) v[u] = ld<NT>(src + base + t + u * kThreads);
#pragma unroll
                for (int u = 0; u < kPer; ++u) {
                    if (MODE == MP_PROBE_COPY) st<NT>(dst + base + t + u * kThreads, v[u]);
                    else acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
                }
            }
        } else {
            for (int64_t i = base + t; i < nvec; i += kThreads) {
                if (MODE == MP_PROBE_WRITE) st<NT>(dst + i, mp::u32x4{uint32_t(i), 0u, 0u, 0u});
                else if (MODE == MP_PROBE_COPY) st<NT>(dst + i, ld<NT>(src + i));
                else {
                    const mp::u32x4 v = ld<NT>(src + i);
                    acc ^= v.x ^ v.y ^ v.z ^ v.w;
                }
            }
        }
    }
    if (MODE == MP_PROBE_READ) {
        // the block's XOR, so that no load is dead code
        __shared__ uint32_t part[kThreads / 64];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
        if ((t & 63) == 0) part[t >> 6] = acc;
        __syncthreads();
        if (t == 0) {
            uint32_t x = 0;
            for (int w = 0; w < kThreads / 64; ++w) x ^= part[w];
            reinterpret_cast<uint32_t*>(dst)[blockIdx.x] = x;
        }
    }
}

// A 32-bit integer hash (two multiply-xorshift rounds) for the probe's operand data.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7FEB352Du;
    x ^= x >> 15;
    x *= 0x846CA68Bu;
    x ^= x >> 16;
    return x;
}

// Independent accumulator chains keep the matrix core issuing back to back with
// one wave per SIMD. A round is 16 x 32768 FLOP on eight chains of
// v_mfma_f32_32x32x16_f16 (two MFMAs each: operand pairs (a[j], b[j + 3]) then
// (a[j + 5], b[j]), indices mod 8), or on sixteen chains of
// v_mfma_f32_16x16x32_f16 (two each: (a[j mod 8], b[(j + 3 + j / 8) mod 8]) then
// (a[j + 5], b[j]), mod 8). CONSTANT: all eight A and B registers hold the same
// few small multiples of 2^-8 (almost no bits change between MFMAs). RANDOM:
// each of the sixteen registers holds its own random binary16 values (random
// sign and 10-bit mantissa, exponent 2^-3 .. 2^0, like unit-scale activations
// and weights), so consecutive MFMAs see unrelated operands, as in a GEMM.
template <int OPERANDS, int SHAPE>
__global__ __launch_bounds__(kThreads) void mfma_clock_kernel(int iters, uint64_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const uint32_t seed = probe_hash(uint32_t(blockIdx.x) * kThreads + threadIdx.x + 1u);
    half8 a[8], b[8];
#pragma unroll
    for (int p = 0; p < 8; ++p)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (OPERANDS == MP_PROBE_OPERANDS_CONSTANT) {
                a[p][i] = _Float16(0.00390625f * float((lane + i) & 3));
                b[p][i] = _Float16(0.00390625f * float((lane * 3 + i) & 3));
            } else {
                const uint32_t ya = probe_hash(seed ^ uint32_t(16 * p + i)), yb = probe_hash(seed ^ uint32_t(16 * p + 8 + i));
                a[p][i] = __builtin_bit_cast(_Float16, uint16_t((ya & 0x83FFu) | ((0xCu + ((ya >> 10) & 3u)) << 10)));
                b[p][i] = __builtin_bit_cast(_Float16, uint16_t((yb & 0x83FFu) | ((0xCu + ((yb >> 10) & 3u)) << 10)));
            }
        }
    float s = 0.0f;
    uint64_t c0, c1, r0, r1;
    if constexpr (SHAPE == MP_PROBE_MFMA_32X32X16) {
        floatx16 acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b[(j + 3) & 7], acc[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[(j + 5) & 7], b[j], acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[j][r];
    } else {
        floatx4 acc[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[j][r] = 0.0f;
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j & 7], b[(j + 3 + (j >> 3)) & 7], acc[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[(j + 5) & 7], b[j & 7], acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) s += acc[j][r];
    }
    c1 = __builtin_amdgcn_s_memtime();
    r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        uint64_t* o = out + 4 * int64_t(blockIdx.x);
        o[0] = c0;
        o[1] = c1;
        o[2] = r0;
        // the sums are finite; testing them keeps the MFMAs live
        o[3] = __builtin_isnan(s) ? 0 : r1;
    }
}

}  // namespace

extern "C" mp_status mp_probe_hbm(int32_t mode, const void* src, void* dst, size_t bytes, int32_t blocks,
                                  int32_t nontemporal, mp_stream stream) {
    if (mode != MP_PROBE_READ && mode != MP_PROBE_WRITE && mode != MP_PROBE_COPY) return MP_ERR_INVALID_ARGUMENT;
    if (bytes == 0 || bytes % 4096 != 0 || blocks < 0 || !dst || !mp::aligned16(dst)) return MP_ERR_INVALID_ARGUMENT;
    if (mode != MP_PROBE_WRITE && (!src || !mp::aligned16(src))) return MP_ERR_INVALID_ARGUMENT;
    const int64_t nvec = int64_t(bytes / 16);
    int64_t grid = blocks > 0 ? blocks : (nvec + kBlockVecs - 1) / kBlockVecs;
    if (grid > 0x7FFFFFFF) return MP_ERR_INVALID_ARGUMENT;
    const int persistent = blocks > 0;
    auto s = mp::as_stream(stream);
    auto in = static_cast<const mp::u32x4*>(src);
    auto out = static_cast<mp::u32x4*>(dst);
    const dim3 g{uint32_t(grid)};
    if (mode == MP_PROBE_READ) {
        if (nontemporal) hbm_kernel<MP_PROBE_READ, true><<<g, kThreads, 0, s>>>(in, out, nvec, persistent);
        else hbm_kernel<MP_PROBE_READ, false><<<g, kThreads, 0, s>>>(in, out, nvec, persistent);
    } else if (mode == MP_PROBE_WRITE) {
        if (nontemporal) hbm_kernel<MP_PROBE_WRITE, true><<<g, kThreads, 0, s>>>(in, out, nvec, persistent);
        else hbm_kernel<MP_PROBE_WRITE, false><<<g, kThreads, 0, s>>>(in, out, nvec, persistent);
    } else {
        if (nontemporal) hbm_kernel<MP_PROBE_COPY, true><<<g, kThreads, 0, s>>>(in, out, nvec, persistent);
        else hbm_kernel<MP_PROBE_COPY, false><<<g, kThreads, 0, s>>>(in, out, nvec, persistent);
    }
    return mp::launch_status("mp_probe_hbm");
}

extern "C" mp_status mp_probe_mfma_clock(int32_t blocks, int32_t iters, int32_t operands, int32_t shape,
                                         uint64_t* out, int32_t* realtime_khz, mp_stream stream) {
    if (blocks < 1 || iters < 1 || !out || !realtime_khz) return MP_ERR_INVALID_ARGUMENT;
    if (operands != MP_PROBE_OPERANDS_CONSTANT && operands != MP_PROBE_OPERANDS_RANDOM) return MP_ERR_INVALID_ARGUMENT;
    if (shape != MP_PROBE_MFMA_32X32X16 && shape != MP_PROBE_MFMA_16X16X32) return MP_ERR_INVALID_ARGUMENT;
    int dev = 0, khz = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess) return mp::hip_status(e, "mp_probe_mfma_clock");
    *realtime_khz = khz;
    const dim3 g{uint32_t(blocks)};
    auto st = mp::as_stream(stream);
    constexpr int kC = MP_PROBE_OPERANDS_CONSTANT, kR = MP_PROBE_OPERANDS_RANDOM;
    constexpr int k32 = MP_PROBE_MFMA_32X32X16, k16 = MP_PROBE_MFMA_16X16X32;
    if (shape == k32) {
        if (operands == kC) mfma_clock_kernel<kC, k32><<<g, kThreads, 0, st>>>(iters, out);
        else mfma_clock_kernel<kR, k32><<<g, kThreads, 0, st>>>(iters, out);
    } else {
        if (operands == kC) mfma_clock_kernel<kC, k16><<<g, kThreads, 0, st>>>(iters, out);
        else mfma_clock_kernel<kR, k16><<<g, kThreads, 0, st>>>(iters, out);
    }
    return mp::launch_status("mp_probe_mfma_clock");
}
