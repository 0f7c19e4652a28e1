// Gradient statistics for loss-scale method 2 on gfx950.
//
// Source: "Mixed Precision Training", long-form analysis page
// (paper-graph-ui.vercel.app), §3.4 "Choosing the scaling factor — the direct
// statistical approach" and the gradient-statistics recipe after it: the
// largest |gradient| over all layers, recorded over a short FP32 run, sets
// S = 65504 / g_max, or 65504 / (2 g_max) with one bit of headroom.
//
// Design (HBM-bound: 4 bytes per FP32 element or 2 per binary16, read once):
//   - The ragged tensor list is cut into chunks of 4096 elements; one
//     256-thread block reads one chunk with 16-byte non-temporal loads (the
//     data is read once; a scalar path for
//     unaligned tensors and tails), keeps |x| of the finite elements, and
//     reduces across the block.
//   - |x| of a finite float is non-negative, and non-negative floats order
//     like their bit patterns, so the block maximum is merged into the running
//     device maximum with one unsigned atomic max per block, skipped when the
//     running value is already at least as large (tens of thousands of blocks
//     contending for one word serialise at the cache otherwise; measured 1.2
//     against 3+ TB/s). A bounded grid walking several chunks per block
//     streamed slower (fewer loads in flight).
//   - A non-finite element is left out of the maximum and ORs a flag (one
//     atomic per block that saw one).
#include <string.h>

#include <new>
#include <vector>

#include "mp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int64_t kChunk = 4096;

struct DevTensor {
    const void* ptr;
    int64_t numel;
    int64_t chunk_begin;
    uint32_t vec;
    uint32_t pad;
};

}  // namespace

struct mp_tensor_list {
    DevTensor* d_desc = nullptr;
    uint32_t* d_chunk_tensor = nullptr;
    int32_t n = 0;
    int64_t chunks = 0;
    mp_dtype dtype = MP_F32;
    std::vector<DevTensor> h_desc;             // kept alive for the async upload
    std::vector<uint32_t> h_chunk_tensor;
    hipStream_t stream = nullptr;
};

namespace {

// |x| as a bit pattern when x is finite, else 0 with *bad = 1.
__device__ __forceinline__ uint32_t abs_bits_f32(uint32_t x, uint32_t& bad) {
    const uint32_t a = x & 0x7FFFFFFFu;
    const bool fin = a < 0x7F800000u;
    bad |= fin ? 0u : 1u;
    return fin ? a : 0u;
}
__device__ __forceinline__ uint32_t abs_bits_f16(uint16_t h, uint32_t& bad) {
    const uint32_t a = h & 0x7FFFu;
    const bool fin = a < 0x7C00u;
    bad |= fin ? 0u : 1u;
    return fin ? __float_as_uint(mp::h2f(uint16_t(a))) : 0u;   // exact widening
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// One 256-thread block per chunk: many blocks in flight keep HBM streaming.
// The block maximum goes into the running maximum with one atomic, skipped
// when the value already there is at least as large, which after the first
// blocks is nearly always the case.
template <bool F32>
__global__ __launch_bounds__(kThreads) void absmax_kernel(const DevTensor* __restrict__ desc,
                                                          const uint32_t* __restrict__ chunk_tensor,
                                                          uint32_t* amax_bits, uint32_t* nonfinite) {
    const uint32_t c = blockIdx.x;
    const DevTensor t = desc[chunk_tensor[c]];
    const int64_t begin = (int64_t(c) - t.chunk_begin) * kChunk;
    const int64_t rem = t.numel - begin;
    const int len = rem < kChunk ? int(rem) : int(kChunk);
    uint32_t m = 0, bad = 0;
    if (F32) {
        const uint32_t* x = static_cast<const uint32_t*>(t.ptr) + begin;
        if (t.vec && len == kChunk) {
            constexpr int kV = kChunk / 4 / kThreads;            // 16-byte vectors per thread (4)
            mp::u32x4 v[kV];
#pragma unroll
            for (int u = 0; u < kV; ++u)
                v[u] = __builtin_nontemporal_load(mp::global(reinterpret_cast<const mp::u32x4*>(x)) + threadIdx.x +
                                                  u * kThreads);
            // every load of the chunk is issued before any is used (left alone,
            // the scheduler waits for the first before issuing the third)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < kV; ++u)
                m = umax(umax(umax(m, abs_bits_f32(v[u].x, bad)), umax(abs_bits_f32(v[u].y, bad),
                                                                    abs_bits_f32(v[u].z, bad))),
                         abs_bits_f32(v[u].w, bad));
        } else {
            for (int e = threadIdx.x; e < len; e += kThreads) m = umax(m, abs_bits_f32(x[e], bad));
        }
    } else {
        const uint16_t* x = static_cast<const uint16_t*>(t.ptr) + begin;
        if (t.vec && len == kChunk) {
            constexpr int kV = kChunk / 8 / kThreads;            // 16-byte vectors per thread (2)
            mp::u32x4 v[kV];
#pragma unroll
            for (int u = 0; u < kV; ++u)
                v[u] = __builtin_nontemporal_load(mp::global(reinterpret_cast<const mp::u32x4*>(x)) + threadIdx.x +
                                                  u * kThreads);
            // every load of the chunk is issued before any is used (left alone,
            // the scheduler waits for the first before issuing the third)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < kV; ++u) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    m = umax(m, umax(abs_bits_f16(uint16_t(w[k]), bad), abs_bits_f16(uint16_t(w[k] >> 16), bad)));
            }
        } else {
            for (int e = threadIdx.x; e < len; e += kThreads) m = umax(m, abs_bits_f16(x[e], bad));
        }
    }
    // wave, then block maximum
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = umax(m, uint32_t(__shfl_xor(int(m), off, 64)));
    __shared__ uint32_t wave_max[kThreads / 64];
    if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
    const int any_bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) {
        uint32_t b = wave_max[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) b = umax(b, wave_max[w]);
        if (b > *reinterpret_cast<volatile uint32_t*>(amax_bits)) atomicMax(amax_bits, b);
        if (any_bad && nonfinite) atomicOr(nonfinite, 1u);
    }
}

// S = the largest power of two with S * headroom * amax <= 65504, in [1, 2^64]:
// halving from 2^64, every product of powers of two with amax is exact (or
// overflows to +inf and fails the test), so the comparison is exact.
__global__ void scaler_from_absmax_kernel(mp_scaler* s, const float* amax, float headroom,
                                          uint32_t dynamic, int32_t interval) {
    const float x = headroom * *amax;
    float S = 0x1p64f;
    while (S > 1.0f && S * x > 65504.0f) S = S * 0.5f;
    s->scale = S;
    s->inv_scale = __uint_as_float(0x7F000000u - __float_as_uint(S));   // exact reciprocal
    s->count = 0;
    s->growth_interval = interval;
    s->found_inf = 0;
    s->dynamic = dynamic;
    s->skipped_steps = 0;
    s->reserved = 0;
}

bool is_pow2_in_range(float v) {
    uint32_t b;
    memcpy(&b, &v, 4);
    const uint32_t e = (b >> 23) & 0xFF, m = b & 0x7FFFFF;
    return (b >> 31) == 0 && m == 0 && e >= 127 && e <= 127 + 64;
}

}  // namespace

extern "C" mp_status mp_tensor_list_create(const void* const* host_ptrs, const int64_t* host_numel,
                                           int32_t n, mp_dtype dtype, mp_tensor_list** out,
                                           mp_stream stream) {
    if (!out || n < 0 || (n > 0 && (!host_ptrs || !host_numel))) return MP_ERR_INVALID_ARGUMENT;
    if (dtype != MP_F32 && dtype != MP_F16) return MP_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    for (int32_t i = 0; i < n; ++i) {
        if (host_numel[i] < 0 || (host_numel[i] > 0 && !host_ptrs[i])) return MP_ERR_INVALID_ARGUMENT;
    }
    mp_tensor_list* L = new (std::nothrow) mp_tensor_list;
    if (!L) return MP_ERR_OUT_OF_MEMORY;
    L->n = n;
    L->dtype = dtype;
    L->stream = mp::as_stream(stream);
    int64_t chunks = 0;
    for (int32_t i = 0; i < n; ++i) {
        DevTensor d{};
        d.ptr = host_ptrs[i];
        d.numel = host_numel[i];
        d.chunk_begin = chunks;
        d.vec = mp::aligned16(host_ptrs[i]);
        const int64_t nc = (d.numel + kChunk - 1) / kChunk;
        for (int64_t k = 0; k < nc; ++k) L->h_chunk_tensor.push_back(uint32_t(i));
        chunks += nc;
        L->h_desc.push_back(d);
    }
    if (chunks > 0x7FFFFFFF) { delete L; return MP_ERR_INVALID_ARGUMENT; }
    L->chunks = chunks;
    if (chunks > 0) {
        hipError_t e = hipMalloc(&L->d_desc, sizeof(DevTensor) * L->h_desc.size());
        if (e == hipSuccess) e = hipMalloc(&L->d_chunk_tensor, sizeof(uint32_t) * size_t(chunks));
        if (e == hipSuccess)
            e = hipMemcpyAsync(L->d_desc, L->h_desc.data(), sizeof(DevTensor) * L->h_desc.size(),
                               hipMemcpyHostToDevice, L->stream);
        if (e == hipSuccess)
            e = hipMemcpyAsync(L->d_chunk_tensor, L->h_chunk_tensor.data(),
                               sizeof(uint32_t) * size_t(chunks), hipMemcpyHostToDevice, L->stream);
        if (e != hipSuccess) {
            mp_status st = mp::hip_status(e, "mp_tensor_list_create");
            if (L->d_desc) (void)hipFree(L->d_desc);
            if (L->d_chunk_tensor) (void)hipFree(L->d_chunk_tensor);
            delete L;
            return st;
        }
    }
    *out = L;
    return MP_OK;
}

extern "C" mp_status mp_tensor_list_destroy(mp_tensor_list* L) {
    if (!L) return MP_OK;
    mp_status st = MP_OK;
    if (L->chunks > 0) {
        hipError_t e = hipStreamSynchronize(L->stream);
        if (e != hipSuccess) st = mp::hip_status(e, "mp_tensor_list_destroy");
        (void)hipFree(L->d_desc);
        (void)hipFree(L->d_chunk_tensor);
    }
    delete L;
    return st;
}

extern "C" mp_status mp_absmax(const mp_tensor_list* L, float* amax, uint32_t* nonfinite,
                               mp_stream stream) {
    if (!L || !amax || mp::misaligned4(amax) || (nonfinite && mp::misaligned4(nonfinite)))
        return MP_ERR_INVALID_ARGUMENT;
    if (L->chunks == 0) return MP_OK;
    hipStream_t s = mp::as_stream(stream);
    uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
    const uint32_t chunks = uint32_t(L->chunks);
    if (L->dtype == MP_F32)
        absmax_kernel<true><<<chunks, kThreads, 0, s>>>(L->d_desc, L->d_chunk_tensor, bits, nonfinite);
    else
        absmax_kernel<false><<<chunks, kThreads, 0, s>>>(L->d_desc, L->d_chunk_tensor, bits, nonfinite);
    return mp::launch_status("mp_absmax");
}

extern "C" mp_status mp_scaler_init_from_absmax(mp_scaler* scaler, const float* amax, float headroom,
                                                int32_t dynamic, int32_t growth_interval,
                                                mp_stream stream) {
    if (!scaler || !amax || mp::misaligned4(scaler) || mp::misaligned4(amax) || !is_pow2_in_range(headroom))
        return MP_ERR_INVALID_ARGUMENT;
    if (dynamic && growth_interval < 1) return MP_ERR_INVALID_ARGUMENT;
    scaler_from_absmax_kernel<<<1, 1, 0, mp::as_stream(stream)>>>(scaler, amax, headroom, dynamic ? 1u : 0u,
                                                                  growth_interval);
    return mp::launch_status("mp_scaler_init_from_absmax");
}
