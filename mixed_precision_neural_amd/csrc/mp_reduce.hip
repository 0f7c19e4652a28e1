// Large reductions on gfx950: batch-normalization statistics and normalization,
// and the row softmax, reading and writing binary16 with FP32 arithmetic.
//
// Source: "Mixed Precision Training", long-form analysis page
// (paper-graph-ui.vercel.app), §3.4 "FP16 Arithmetic with FP32 Accumulation":
// large reductions (batch normalization's mean and variance over the batch and
// spatial positions, the softmax normalization constant) are summed in FP32
// from binary16 tensors, all of their arithmetic is FP32 and binary16 results
// are written back; these layers are memory-bound, so FP32 costs no time.
//
// Design (HBM-bound; 16-byte loads and stores where rows are 16-byte aligned,
// an element-wise path with the same arithmetic otherwise):
//   - Batch-norm statistics of x[rows, C]: a block owns a chunk of rows and up
//     to 256 groups of 8 channels; each thread sums d and d^2 in FP32 for its 8
//     channels over its rows of the chunk, d = x minus the thread's first value
//     of the channel (a shift inside the data), turns the sums into (count,
//     mean, M2) once, the block merges its row lanes with Chan's pairwise formula
//     in a fixed tree, and writes one (count, mean, M2) per channel and chunk
//     to the caller's workspace. A second kernel merges the chunks of each
//     channel in a fixed order (one block per channel) and writes mean and the
//     population variance M2 / rows. Results do not depend on timing.
//   - The normalization y = ((x - mean) * inv) * gamma + beta, inv = 1 /
//     sqrt(var + eps) per channel (correctly rounded square root and
//     division), one rounding per operation in that order, then
//     round-to-nearest-even binary16.
//   - Softmax of each row of x[rows, cols], two forms with the same per-thread
//     arithmetic: an online (max m, sum s of exp(x - m)) per thread, the
//     block's pairs merged by a butterfly in each wave and then the waves in
//     order, the row's pairs merged in a fixed order by every block of the row
//     (so all agree on (M, S) to the bit), and RNE16(exp(x - M) * (1 / S))
//     written. m starts at -FLT_MAX, so -inf entries give exp = 0 without NaN;
//     a NaN or +inf entry makes the row's sum NaN, and a row of only -inf
//     gives 0 / 0 = NaN.
//       Single read (x and y distinct, 16-byte rows, the whole grid at most one
//     block per compute unit): each block keeps its segment of up to 204,800
//     values in registers and exchanges its pair through the workspace, so x
//     is read once (below, "single-read softmax").
//       Two passes otherwise: one block per (row, 32K-value segment) writes its
//     pair to the workspace; a second kernel re-reads x and writes y.
#include <float.h>

#include <atomic>
#include <random>

#include "mp_internal.h"

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------ statistics
struct Moments {
    float n, mean, m2;
};

// Chan et al.'s pairwise update: the moments of the union of two disjoint sets.
__device__ __forceinline__ Moments merge(Moments a, Moments b) {
    if (b.n == 0.0f) return a;
    if (a.n == 0.0f) return b;
    const float n = a.n + b.n;
    const float fb = b.n * __builtin_amdgcn_rcpf(n);    // within 1 ulp: the statistics are bound-checked
    const float d = b.mean - a.mean;
    Moments r;
    r.n = n;
    r.mean = a.mean + d * fb;
    r.m2 = (a.m2 + b.m2) + (d * d) * (a.n * fb);
    return r;
}

// Loads VEC consecutive binary16 values as floats.
template <int VEC>
__device__ __forceinline__ void load_f16(const uint16_t* p, float (&v)[VEC]) {
    if constexpr (VEC == 8) {
        const mp::u32x4 w = *mp::global(reinterpret_cast<const mp::u32x4*>(p));
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = mp::h2f(uint16_t(w[k >> 1] >> ((k & 1) * 16)));
    } else {
        v[0] = mp::h2f(*mp::global(p));
    }
}

// Thread layout of the two batch-norm kernels: lanes (row lane rl, channel
// group g) over the block's channel groups; rows_per_iter row lanes.
struct BnLayout {
    int g, rl, lc, rp;
    bool active;
    __device__ __forceinline__ BnLayout(int groups_left) {
        lc = groups_left < kThreads ? groups_left : kThreads;
        rp = kThreads / lc;
        const int t = int(threadIdx.x);
        g = t % lc;
        rl = t / lc;
        active = rl < rp;
    }
};

// grid (chunks, channel blocks); ws: cnt[chunks], then mean[C][chunks], m2[C][chunks]
// (channel-major, so the final merge reads each channel's chunks contiguously).
template <int VEC>
__global__ __launch_bounds__(kThreads) void bn_partial_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                              int64_t C, int64_t ldx, int64_t rows_per_chunk,
                                                              float* __restrict__ ws) {
    const int64_t groups = C / VEC;
    const int64_t g0 = int64_t(blockIdx.y) * kThreads;
    const BnLayout L(int(groups - g0 < kThreads ? groups - g0 : kThreads));
    const int64_t r0 = int64_t(blockIdx.x) * rows_per_chunk;
    const int64_t r1 = r0 + rows_per_chunk < rows ? r0 + rows_per_chunk : rows;
    const int64_t c0 = (g0 + L.g) * VEC;

    // Sums of d = x - k and of d^2 over this lane's rows, k the lane's first value of
    // the channel (a shift inside the data keeps s2 - s1^2 / n free of large cancellation);
    // converted once to (n, mean, M2) for Chan's merges.
    float n = 0.0f, mean[VEC], m2[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) mean[k] = m2[k] = 0.0f;
    if (L.active && r0 + L.rl < r1) {
        float sh[VEC], s1[VEC], s2[VEC];
        load_f16<VEC>(x + (r0 + L.rl) * ldx + c0, sh);
#pragma unroll
        for (int k = 0; k < VEC; ++k) s1[k] = s2[k] = 0.0f;
        n = 1.0f;
        auto add = [&](const float (&v)[VEC]) {
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const float d = v[k] - sh[k];
                s1[k] = s1[k] + d;
                s2[k] = s2[k] + d * d;
            }
        };
        int64_t r = r0 + L.rl + L.rp;
        for (; r + 7 * L.rp < r1; r += 8 * L.rp) {                // eight rows' loads in flight
            float v[8][VEC];
#pragma unroll
            for (int u = 0; u < 8; ++u) load_f16<VEC>(x + (r + u * L.rp) * ldx + c0, v[u]);
#pragma unroll
            for (int u = 0; u < 8; ++u) add(v[u]);
            n += 8.0f;
        }
        for (; r < r1; r += L.rp) {
            float v[VEC];
            load_f16<VEC>(x + r * ldx + c0, v);
            add(v);
            n += 1.0f;
        }
        const float inv = 1.0f / n;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float q = s1[k] * inv;
            mean[k] = sh[k] + q;
            m2[k] = s2[k] - s1[k] * q;
        }
    }

    // merge the row lanes of each channel group in a fixed order. When the block's
    // channel groups divide a wave, a channel's lanes in one wave are lc apart: a
    // butterfly of shuffles merges them, then the waves' results go through LDS.
    // Otherwise a binary tree over rl in LDS.
    __shared__ float s_n[kThreads], s_mean[VEC][kThreads], s_m2[VEC][kThreads];
    const int t = int(threadIdx.x);
    if (L.lc < 64 && (64 % L.lc) == 0) {
        for (int off = L.lc; off < 64; off *= 2) {
            const float on = __shfl_xor(n, off);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const Moments m = merge({n, mean[k], m2[k]}, {on, __shfl_xor(mean[k], off), __shfl_xor(m2[k], off)});
                mean[k] = m.mean;
                m2[k] = m.m2;
            }
            n = n + on;
        }
        const int w = t >> 6;
        if ((t & 63) < L.lc) {                              // lane g of each wave
            s_n[w * L.lc + L.g] = n;
#pragma unroll
            for (int k = 0; k < VEC; ++k) { s_mean[k][w * L.lc + L.g] = mean[k]; s_m2[k][w * L.lc + L.g] = m2[k]; }
        }
        __syncthreads();
        if (t < L.lc) {
            Moments acc[VEC];
#pragma unroll
            for (int k = 0; k < VEC; ++k) acc[k] = {s_n[t], s_mean[k][t], s_m2[k][t]};
            for (int v = 1; v < kThreads / 64; ++v) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) acc[k] = merge(acc[k], {s_n[v * L.lc + t], s_mean[k][v * L.lc + t], s_m2[k][v * L.lc + t]});
            }
            const int64_t chunks = gridDim.x;
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                ws[chunks + (c0 + k) * chunks + blockIdx.x] = acc[k].mean;
                ws[chunks + chunks * C + (c0 + k) * chunks + blockIdx.x] = acc[k].m2;
            }
            if (blockIdx.y == 0 && t == 0) ws[blockIdx.x] = acc[0].n;
        }
        return;
    }
    s_n[t] = n;
#pragma unroll
    for (int k = 0; k < VEC; ++k) { s_mean[k][t] = mean[k]; s_m2[k][t] = m2[k]; }
    __syncthreads();
    for (int s = 1; s < L.rp; s *= 2) {
        if (L.active && (L.rl % (2 * s)) == 0 && L.rl + s < L.rp) {
            const int o = t + s * L.lc;
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const Moments m = merge({s_n[t], s_mean[k][t], s_m2[k][t]}, {s_n[o], s_mean[k][o], s_m2[k][o]});
                s_mean[k][t] = m.mean;
                s_m2[k][t] = m.m2;
            }
            s_n[t] = s_n[t] + s_n[o];
        }
        __syncthreads();
    }
    if (L.active && L.rl == 0) {
        const int64_t chunks = gridDim.x;
        float* wmean = ws + chunks;
        float* wm2 = ws + chunks + chunks * C;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            wmean[(c0 + k) * chunks + blockIdx.x] = s_mean[k][t];
            wm2[(c0 + k) * chunks + blockIdx.x] = s_m2[k][t];
        }
        if (blockIdx.y == 0 && L.g == 0) ws[blockIdx.x] = s_n[t];
    }
}

// One wave per channel: merges the chunks' moments in a fixed order. Lane t takes
// chunks t, t + 64, ... (up to eight, all loaded before the first merge; more only
// past kMaxChunks chunks), then a butterfly of shuffles merges the lanes; lane 0's
// result is stored.
__global__ __launch_bounds__(64) void bn_final_kernel(const float* __restrict__ ws, int64_t chunks, int64_t C,
                                                      float* __restrict__ mean, float* __restrict__ var) {
    const int64_t c = blockIdx.x;
    const int t = int(threadIdx.x);
    const float* wmean = ws + chunks + c * chunks;
    const float* wm2 = ws + chunks + chunks * C + c * chunks;
    Moments m[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {                       // a lane past the end reloads the last chunk
        const int64_t k = t + 64 * u < chunks ? t + 64 * u : chunks - 1;
        m[u] = {ws[k], wmean[k], wm2[k]};
    }
    __builtin_amdgcn_sched_barrier(0);     // keep the loads ahead of the merges
#pragma unroll
    for (int u = 0; u < 8; ++u)
        if (t + 64 * u >= chunks) m[u] = {0.0f, 0.0f, 0.0f};   // and contributes nothing
    Moments acc = m[0];
#pragma unroll
    for (int u = 1; u < 8; ++u) acc = merge(acc, m[u]);
    for (int64_t k = t + 512; k < chunks; k += 64) acc = merge(acc, {ws[k], wmean[k], wm2[k]});
    for (int off = 32; off > 0; off >>= 1)
        acc = merge(acc, {__shfl_xor(acc.n, off), __shfl_xor(acc.mean, off), __shfl_xor(acc.m2, off)});
    if (t == 0) {
        mean[c] = acc.mean;
        var[c] = acc.m2 / acc.n;
    }
}

// ------------------------------------------------------------------ normalization
template <int VEC>
__global__ __launch_bounds__(kThreads) void bn_apply_kernel(const uint16_t* x, int64_t rows, int64_t C,
                                                            int64_t ldx, const float* __restrict__ mean,
                                                            const float* __restrict__ var,
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ beta, float eps,
                                                            uint16_t* y, int64_t ldy,
                                                            int64_t rows_per_chunk) {
    const int64_t groups = C / VEC;
    const int64_t g0 = int64_t(blockIdx.y) * kThreads;
    const BnLayout L(int(groups - g0 < kThreads ? groups - g0 : kThreads));
    if (!L.active) return;
    const int64_t c0 = (g0 + L.g) * VEC;
    float mu[VEC], inv[VEC], ga[VEC], be[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        const float s = var[c0 + k] + eps;
        const float r = sqrtf(s);
        inv[k] = 1.0f / r;
        mu[k] = mean[c0 + k];
        ga[k] = gamma[c0 + k];
        be[k] = beta[c0 + k];
    }
    const int64_t r0 = int64_t(blockIdx.x) * rows_per_chunk;
    const int64_t r1 = r0 + rows_per_chunk < rows ? r0 + rows_per_chunk : rows;
    auto emit = [&](int64_t r, const float (&v)[VEC]) {
        uint16_t h[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float t = v[k] - mu[k];
            const float u = t * inv[k];
            const float w = u * ga[k];
            h[k] = mp::f2h(w + be[k]);
        }
        if constexpr (VEC == 8) {
            *mp::global(reinterpret_cast<mp::u32x4*>(y + r * ldy + c0)) =
                mp::u32x4{uint32_t(h[0]) | uint32_t(h[1]) << 16, uint32_t(h[2]) | uint32_t(h[3]) << 16,
                          uint32_t(h[4]) | uint32_t(h[5]) << 16, uint32_t(h[6]) | uint32_t(h[7]) << 16};
        } else {
            *mp::global(y + r * ldy + c0) = h[0];
        }
    };
    int64_t r = r0 + L.rl;
    for (; r + 7 * L.rp < r1; r += 8 * L.rp) {                      // eight rows' loads in flight
        float v[8][VEC];
#pragma unroll
        for (int u = 0; u < 8; ++u) load_f16<VEC>(x + (r + u * L.rp) * ldx + c0, v[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u) emit(r + u * L.rp, v[u]);
    }
    for (; r < r1; r += L.rp) {
        float v[VEC];
        load_f16<VEC>(x + r * ldx + c0, v);
        emit(r, v);
    }
}

// ------------------------------------------------------------------ softmax
struct MaxSum {
    float m, s;
};

__device__ __forceinline__ MaxSum merge(MaxSum a, MaxSum b) {
    const float m = fmaxf(a.m, b.m);
    return {m, a.s * __expf(a.m - m) + b.s * __expf(b.m - m)};
}

// Merges a wave's 64 pairs with a butterfly; every lane gets the same bits
// (merge is commutative bit for bit: max and a sum of two terms).
__device__ __forceinline__ MaxSum wave_merge(MaxSum v) {
#pragma unroll
    for (int off = 32; off > 0; off /= 2)
        v = merge(v, MaxSum{__shfl_xor(v.m, off), __shfl_xor(v.s, off)});
    return v;
}

// Merges the block's THREADS pairs; every thread gets the same bits: a
// butterfly within each wave, then the waves' results in a fixed order.
template <int THREADS = kThreads>
__device__ __forceinline__ MaxSum block_merge(MaxSum v) {
    v = wave_merge(v);
    __shared__ float s_m[THREADS / 64], s_s[THREADS / 64];
    const int w = int(threadIdx.x) >> 6;
    if ((threadIdx.x & 63) == 0) { s_m[w] = v.m; s_s[w] = v.s; }
    __syncthreads();
    MaxSum r = {s_m[0], s_s[0]};
#pragma unroll
    for (int k = 1; k < THREADS / 64; ++k) r = merge(r, MaxSum{s_m[k], s_s[k]});
    __syncthreads();
    return r;
}

// The online (max, sum of exp(x - max)) update of one thread over 8 values
// (a 16-byte vector) or one value.
__device__ __forceinline__ void online8(MaxSum& acc, const float (&e)[8]) {
    float vm = e[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) vm = fmaxf(vm, e[k]);
    if (vm > acc.m) {
        acc.s = acc.s * __expf(acc.m - vm);
        acc.m = vm;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) acc.s = acc.s + __expf(e[k] - acc.m);
}
__device__ __forceinline__ void online1(MaxSum& acc, float e) {
    if (e > acc.m) {
        acc.s = acc.s * __expf(acc.m - e);
        acc.m = e;
    }
    acc.s = acc.s + __expf(e - acc.m);
}

__device__ __forceinline__ void unpack8(mp::u32x4 w, float (&e)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = mp::h2f(uint16_t(w[k >> 1] >> ((k & 1) * 16)));
}

// Eight outputs RNE16(exp(e - m) * inv), packed.
__device__ __forceinline__ mp::u32x4 softmax_out8(const float (&e)[8], float m, float inv) {
    uint16_t h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = mp::f2h(__expf(e[k] - m) * inv);
    return mp::u32x4{uint32_t(h[0]) | uint32_t(h[1]) << 16, uint32_t(h[2]) | uint32_t(h[3]) << 16,
                     uint32_t(h[4]) | uint32_t(h[5]) << 16, uint32_t(h[6]) | uint32_t(h[7]) << 16};
}

// Segment seg of a row covers vectors [seg * seg_vecs, ...) of the row's full
// VEC-element vectors; the last segment also takes the row's tail elements.
struct Segment {
    int64_t v0, v1, tail0, tail1;
    __device__ __forceinline__ Segment(int64_t cols, int vec, int64_t seg_vecs) {
        const int64_t nvec = cols / vec;
        const int64_t seg = blockIdx.y;
        v0 = seg * seg_vecs;
        v1 = v0 + seg_vecs < nvec ? v0 + seg_vecs : nvec;
        const bool last = seg == int64_t(gridDim.y) - 1;
        tail0 = last ? nvec * vec : cols;
        tail1 = cols;
    }
};

// grid (rows, segments): one (max, sum) per (row, segment) in ws[row * segments + seg]
template <int VEC>
__global__ __launch_bounds__(kThreads) void softmax_partial_kernel(const uint16_t* __restrict__ x, int64_t cols,
                                                                   int64_t ldx, int64_t seg_vecs,
                                                                   float2* __restrict__ ws) {
    const int64_t row = blockIdx.x;
    const uint16_t* xr = x + row * ldx;
    const Segment sg(cols, VEC, seg_vecs);
    MaxSum acc = {-FLT_MAX, 0.0f};
    auto update = [&](const float (&e)[VEC]) {
        float vm = e[0];
#pragma unroll
        for (int k = 1; k < VEC; ++k) vm = fmaxf(vm, e[k]);
        if (vm > acc.m) {
            acc.s = acc.s * __expf(acc.m - vm);
            acc.m = vm;
        }
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc.s = acc.s + __expf(e[k] - acc.m);
    };
    int64_t v = sg.v0 + threadIdx.x;
    for (; v + 3 * kThreads < sg.v1; v += 4 * kThreads) {      // four loads in flight
        float e[4][VEC];
#pragma unroll
        for (int u = 0; u < 4; ++u) load_f16<VEC>(xr + (v + u * kThreads) * VEC, e[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u) update(e[u]);
    }
    for (; v < sg.v1; v += kThreads) {
        float e[VEC];
        load_f16<VEC>(xr + v * VEC, e);
        update(e);
    }
    for (int64_t j = sg.tail0 + threadIdx.x; j < sg.tail1; j += kThreads) {
        const float e = mp::h2f(*mp::global(xr + j));
        if (e > acc.m) {
            acc.s = acc.s * __expf(acc.m - e);
            acc.m = e;
        }
        acc.s = acc.s + __expf(e - acc.m);
    }
    const MaxSum r = block_merge(acc);
    if (threadIdx.x == 0) ws[row * gridDim.y + blockIdx.y] = make_float2(r.m, r.s);
}

template <int VEC>
__global__ __launch_bounds__(kThreads) void softmax_norm_kernel(const uint16_t* x, int64_t cols,
                                                                int64_t ldx, uint16_t* y, int64_t ldy,
                                                                int64_t seg_vecs, const float2* __restrict__ ws) {
    const int64_t row = blockIdx.x;
    const int64_t S = gridDim.y;
    // the row's pairs, merged in the same order by every block of the row
    MaxSum acc = {-FLT_MAX, 0.0f};
    for (int64_t k = threadIdx.x; k < S; k += kThreads) {
        const float2 p = ws[row * S + k];
        acc = merge(acc, MaxSum{p.x, p.y});
    }
    const MaxSum tot = block_merge(acc);
    const float inv = 1.0f / tot.s;
    const uint16_t* xr = x + row * ldx;
    uint16_t* yr = y + row * ldy;
    const Segment sg(cols, VEC, seg_vecs);
    auto emit = [&](int64_t v, const float (&e)[VEC]) {
        uint16_t h[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) h[k] = mp::f2h(__expf(e[k] - tot.m) * inv);
        if constexpr (VEC == 8) {
            *mp::global(reinterpret_cast<mp::u32x4*>(yr + v * VEC)) =
                mp::u32x4{uint32_t(h[0]) | uint32_t(h[1]) << 16, uint32_t(h[2]) | uint32_t(h[3]) << 16,
                          uint32_t(h[4]) | uint32_t(h[5]) << 16, uint32_t(h[6]) | uint32_t(h[7]) << 16};
        } else {
            *mp::global(yr + v) = h[0];
        }
    };
    int64_t v = sg.v0 + threadIdx.x;
    for (; v + 3 * kThreads < sg.v1; v += 4 * kThreads) {      // four loads in flight
        float e[4][VEC];
#pragma unroll
        for (int u = 0; u < 4; ++u) load_f16<VEC>(xr + (v + u * kThreads) * VEC, e[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u) emit(v + u * kThreads, e[u]);
    }
    for (; v < sg.v1; v += kThreads) {
        float e[VEC];
        load_f16<VEC>(xr + v * VEC, e);
        emit(v, e);
    }
    for (int64_t j = sg.tail0 + threadIdx.x; j < sg.tail1; j += kThreads)
        *mp::global(yr + j) = mp::f2h(__expf(mp::h2f(*mp::global(xr + j)) - tot.m) * inv);
}

// ------------------------------------------------------------------ single-read softmax
// When every row fits on chip in at most kResMaxParts blocks and the grid fits
// one block per compute unit, x is read once. Row r is cut into `parts`
// segments of seg_vecs 16-byte vectors, one 512-thread block each (two waves
// per SIMD, 256 registers each); thread t holds vectors i * 512 + t of its
// segment in registers, all loads issued before the first use. (Holding part
// of the segment in LDS instead, loaded straight from memory, was slower: at
// one block per compute unit that path delivered its share well after the
// register loads had delivered theirs.) Each block computes its segment's
// (max, sum) with the two-pass form's per-thread online update and block
// merge, publishes it in a workspace slot tagged with the call's 64-bit tag
// (release), and its first wave polls the row's other slots (relaxed loads,
// then one acquire fence). A slot that has not been published within the wait
// limit, measured on the wall clock, is computed by the waiting block itself
// from x, in the owner's per-thread order, so it has the owner's bits: the
// wait always ends, and a block that is not resident yet only costs time.
// Every block of a row then merges the row's pairs in the same fixed order
// (a lane per slot in order, then a butterfly), so all agree on (M, S) to the
// bit, and writes RNE16(exp(x - M) * (1 / S)) from the values it holds.
constexpr int kResThreads = 512;
constexpr int kResRegVecs = 50;                                         // 200 VGPRs of x per thread
constexpr int64_t kResVecs = int64_t(kResThreads) * kResRegVecs;        // 204,800 values per block
constexpr int kResMaxParts = 256;
constexpr int kResMaxBlocks = 1024;
constexpr int64_t kResMinPartVecs = 4096;                               // below this, fewer parts

struct ResSlot {
    float m, s;
    uint64_t tag;
};

// Eight binary16 -inf values: lanes past their segment load these instead of
// data, and exp(-inf - m) adds +0, so the (max, sum) needs no per-vector branch.
__device__ const mp::u32x4 g_neg_inf8 = {0xFC00FC00u, 0xFC00FC00u, 0xFC00FC00u, 0xFC00FC00u};

__device__ __forceinline__ const mp::u32x4* res_src(const mp::u32x4* xv, int v, int nv) {
    return v < nv ? xv + v : &g_neg_inf8;
}

// Segment p of a row: vectors [v0, v0 + nv) of the row's full vectors.
struct ResSeg {
    int64_t v0;
    int nv;
    __device__ __forceinline__ ResSeg(int p, int64_t seg_vecs, int64_t nvec) {
        v0 = p * seg_vecs;
        const int64_t v1 = v0 + seg_vecs < nvec ? v0 + seg_vecs : nvec;
        nv = v1 > v0 ? int(v1 - v0) : 0;
    }
};

// (max, sum) of segment p of the row computed from memory, in the per-thread
// order of the block that owns it: vectors i * 512 + t for i = 0, 1, ...,
// nvt - 1 (-inf values past the segment, as the owner loads them), then the
// row's tail values (last segment only).
__device__ MaxSum res_pair_from_memory(const uint16_t* xr, int p, int parts, int64_t seg_vecs, int64_t nvec,
                                       int64_t cols, int nvt) {
    const ResSeg sg(p, seg_vecs, nvec);
    const mp::u32x4* xv = reinterpret_cast<const mp::u32x4*>(xr) + sg.v0;
    const int t = int(threadIdx.x);
    MaxSum acc = {-FLT_MAX, 0.0f};
    for (int i = 0; i < nvt; i += 2) {                        // two loads in flight: the caller
        mp::u32x4 w[2];                                       // keeps its segment in registers
#pragma unroll
        for (int u = 0; u < 2; ++u) w[u] = *mp::global(res_src(xv, (i + u) * kResThreads + t, sg.nv));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (i + u < nvt) {                                // uniform
                float e[8];
                unpack8(w[u], e);
                online8(acc, e);
            }
        }
    }
    const int64_t tail0 = nvec * 8;
    if (p == parts - 1 && t < cols - tail0) online1(acc, mp::h2f(*mp::global(xr + tail0 + t)));
    return block_merge<kResThreads>(acc);
}

// grid rows * parts; block b handles segment b % parts of row b / parts.
// nvt: vectors per thread in use, ceil(seg_vecs / 512) <= 50; slots[b] is block b's.
__global__ __launch_bounds__(kResThreads) void softmax_resident_kernel(
        const uint16_t* __restrict__ x, int64_t cols, int64_t ldx, uint16_t* __restrict__ y, int64_t ldy,
        int parts, int64_t seg_vecs, int nvt, ResSlot* __restrict__ slots, uint64_t tag, int64_t wait_ticks) {
    __shared__ float2 s_pair[kResMaxParts];
    __shared__ int s_missing[kResMaxParts];
    __shared__ float2 s_tot;
    const int t = int(threadIdx.x);
    const int lane = t & 63, wave = t >> 6;
    const int64_t row = blockIdx.x / parts;
    const int part = int(blockIdx.x - row * parts);
    const int64_t nvec = cols / 8;
    const uint16_t* xr = x + row * ldx;
    uint16_t* yr = y + row * ldy;
    const ResSeg sg(part, seg_vecs, nvec);
    const mp::u32x4* xv = reinterpret_cast<const mp::u32x4*>(xr) + sg.v0;
    const int64_t tail0 = nvec * 8;
    const bool tail = part == parts - 1 && t < cols - tail0;

    // Every load of the segment is issued before the first use, all fifty
    // always, so the wait before each use is a static count; lanes past the
    // segment load -inf values, which leave the (max, sum) unchanged.
    mp::u32x4 r[kResRegVecs];
#pragma unroll
    for (int i = 0; i < kResRegVecs; ++i) r[i] = *mp::global(res_src(xv, i * kResThreads + t, sg.nv));
    // the tail value (a valid address for every thread, so the load needs no branch and
    // no early wait)
    const uint16_t th = *mp::global(xr + (tail ? tail0 + t : 0));

    MaxSum acc = {-FLT_MAX, 0.0f};
#pragma unroll
    for (int i = 0; i < kResRegVecs; ++i) {
        if (i < nvt) {                                        // uniform
            float e[8];
            unpack8(r[i], e);
            online8(acc, e);
        }
    }
    if (tail) online1(acc, mp::h2f(th));
    const MaxSum own = block_merge<kResThreads>(acc);

    if (parts == 1) {
        if (t == 0) s_tot = make_float2(own.m, own.s);
    } else {
        ResSlot* rs = slots + row * parts;
        if (t == 0) {
            rs[part].m = own.m;
            rs[part].s = own.s;
            __hip_atomic_store(&rs[part].tag, tag, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (wave == 0) {
            // lane l watches slots l, l + 64, l + 128, l + 192; a slot seen
            // tagged stays so for the rest of the call
            uint32_t seen = 0;
#pragma unroll
            for (int k = 0; k < kResMaxParts / 64; ++k) {
                const int j = lane + 64 * k;
                if (j >= parts || j == part) seen |= 1u << k;
            }
            // wait_ticks 0: compute every other slot here (never waits)
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            for (int it = 0; wait_ticks > 0 && it < (1 << 20); ++it) {
                // all four loads in flight before the first compare (a lane past
                // the row's blocks reads its own block's slot)
                uint64_t v[kResMaxParts / 64];
#pragma unroll
                for (int k = 0; k < kResMaxParts / 64; ++k) {
                    const int j = lane + 64 * k;
                    v[k] = __hip_atomic_load(&rs[j < parts ? j : part].tag, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int k = 0; k < kResMaxParts / 64; ++k)
                    if (v[k] == tag) seen |= 1u << k;
                if (__all(seen == (1u << (kResMaxParts / 64)) - 1)) break;
                if (int64_t(__builtin_amdgcn_s_memrealtime() - t0) >= wait_ticks) break;
                __builtin_amdgcn_s_sleep(2);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
            for (int k = 0; k < kResMaxParts / 64; ++k) {
                const int j = lane + 64 * k;
                if (j < parts) {
                    const bool have = j == part || (seen >> k & 1u);
                    s_missing[j] = !have;
                    s_pair[j] = j == part ? make_float2(own.m, own.s)
                                          : (have ? make_float2(rs[j].m, rs[j].s) : make_float2(0.0f, 0.0f));
                }
            }
        }
        __syncthreads();
        for (int j = 0; j < parts; ++j) {                    // uniform: every thread reads the same flag
            if (!s_missing[j]) continue;
            const MaxSum q = res_pair_from_memory(xr, j, parts, seg_vecs, nvec, cols, nvt);
            if (t == 0) s_pair[j] = make_float2(q.m, q.s);
        }
        __syncthreads();
        if (wave == 0) {
            MaxSum a = {-FLT_MAX, 0.0f};
            for (int j = lane; j < parts; j += 64) a = merge(a, MaxSum{s_pair[j].x, s_pair[j].y});
            a = wave_merge(a);
            if (lane == 0) s_tot = make_float2(a.m, a.s);
        }
    }
    __syncthreads();
    const float m = s_tot.x, inv = 1.0f / s_tot.y;
#if defined(__HIP_DEVICE_COMPILE__)
    // buffer stores bounded by the segment: a lane past it stores nothing
    const __amdgpu_buffer_rsrc_t ys = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<mp::u32x4*>(yr) + sg.v0, 0, sg.nv * 16, 0x00020000);
#pragma unroll
    for (int i = 0; i < kResRegVecs; ++i) {
        if (i < nvt) {                                        // uniform
            float e[8];
            unpack8(r[i], e);
            __builtin_amdgcn_raw_buffer_store_b128(softmax_out8(e, m, inv), ys,
                                                   (i * kResThreads + t) * 16, 0, 0);
        }
    }
#endif
    if (tail) *mp::global(yr + tail0 + t) = mp::f2h(__expf(mp::h2f(th) - m) * inv);
}

// ------------------------------------------------------------------ shapes
constexpr int64_t kMaxChunks = 512;

// Rows per chunk of the statistics kernel: at least four row iterations per
// thread, more when there would be over kMaxChunks chunks to merge.
int64_t bn_rows_per_chunk(int64_t rows, int64_t C, int vec) {
    const int64_t groups = C / vec > 0 ? C / vec : 1;
    const int64_t lc = groups < kThreads ? groups : kThreads;
    const int64_t rp = kThreads / lc;
    int64_t per = (rows + kMaxChunks - 1) / kMaxChunks;
    if (per < 4 * rp) per = 4 * rp;
    return (per + rp - 1) / rp * rp;
}

int bn_vec(const void* x, int64_t ldx, int64_t C, const void* y = nullptr, int64_t ldy = 0) {
    const bool ok = (C % 8) == 0 && (ldx % 8) == 0 && mp::aligned16(x) && (y == nullptr || (mp::aligned16(y) && (ldy % 8) == 0));
    return ok ? 8 : 1;
}

// The single-read form's launch: parts per row (0: use the two-pass form),
// vectors per segment, vectors per thread, and the wait limit in wall-clock
// ticks of the current device.
struct ResPlan {
    int64_t parts = 0, seg_vecs = 0, wait_ticks = 0;
    int nvt = 0;
};

constexpr int64_t kResMaxWaitUs = 100000;
std::atomic<int64_t> g_wait_us{200};

struct DeviceInfo {
    int cus = 0, wall_khz = 0;
};

// Compute units and wall-clock rate of the current device, queried once per
// device (both in one atomic word, so concurrent first calls are harmless).
mp_status device_info(DeviceInfo* out) {
    static std::atomic<uint64_t> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return mp::hip_status(e, "mp_softmax/hipGetDevice");
    if (dev < 0 || dev >= 64) return mp::hip_status(hipErrorInvalidDevice, "mp_softmax/device");
    uint64_t w = cache[dev].load();
    if (w == 0) {
        int cus = 0, khz = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
        if (e != hipSuccess) return mp::hip_status(e, "mp_softmax/hipDeviceGetAttribute");
        if (cus <= 0 || khz <= 0) return mp::hip_status(hipErrorInvalidValue, "mp_softmax/device attributes");
        w = uint64_t(uint32_t(cus)) << 32 | uint32_t(khz);
        cache[dev].store(w);
    }
    out->cus = int(w >> 32);
    out->wall_khz = int(w & 0xFFFFFFFFu);
    return MP_OK;
}

// A 64-bit tag no earlier call of this process used (an odd multiplier is a
// bijection), offset by a per-process random value so that slots left by
// another process or another use of the memory do not match by accident.
uint64_t res_next_tag() {
    static const uint64_t salt = [] {
        std::random_device rd;
        return (uint64_t(rd()) << 32) ^ uint64_t(rd());
    }();
    static std::atomic<uint64_t> calls{0};
    return salt + 0x9E3779B97F4A7C15ull * (calls.fetch_add(1) + 1);
}

mp_status res_plan(int64_t rows, int64_t cols, size_t workspace_bytes, ResPlan* p) {
    *p = ResPlan{};
    if (rows > kResMaxBlocks) return MP_OK;
    DeviceInfo d;
    const mp_status st = device_info(&d);
    if (st != MP_OK) return st;
    const int64_t blocks = d.cus < kResMaxBlocks ? d.cus : kResMaxBlocks;
    int64_t pmax = blocks / rows;
    if (pmax > kResMaxParts) pmax = kResMaxParts;
    const int64_t nvec = cols / 8;
    const int64_t pmin = nvec > 0 ? (nvec + kResVecs - 1) / kResVecs : 1;
    if (pmax < pmin) return MP_OK;
    int64_t parts = (nvec + kResMinPartVecs - 1) / kResMinPartVecs;
    if (parts > pmax) parts = pmax;
    if (parts < pmin) parts = pmin;
    if (parts < 1) parts = 1;
    const int64_t seg = (nvec + parts - 1) / parts;
    if (seg > 0) parts = (nvec + seg - 1) / seg;        // no empty segment
    if (workspace_bytes < size_t(rows * parts) * sizeof(ResSlot)) return MP_OK;
    p->parts = parts;
    p->seg_vecs = seg;
    p->nvt = int((seg + kResThreads - 1) / kResThreads);
    p->wait_ticks = g_wait_us.load() * d.wall_khz / 1000;
    return MP_OK;
}

int64_t softmax_segments(int64_t cols) {
    int64_t s = (cols + 32767) / 32768;
    return s < 1 ? 1 : (s > 1024 ? 1024 : s);
}

}  // namespace

// Enough for either path (the 16-byte path is chosen at launch from the pointers).
extern "C" size_t mp_bn_stats_workspace(int64_t rows, int64_t channels) {
    if (rows <= 0 || channels <= 0) return 0;
    int64_t c = 0;
    for (int vec : {1, 8}) {
        const int64_t per = bn_rows_per_chunk(rows, channels, vec);
        const int64_t k = (rows + per - 1) / per;
        c = k > c ? k : c;
    }
    return size_t(c * (2 * channels + 1)) * sizeof(float);
}

extern "C" mp_status mp_bn_stats(const uint16_t* x, int64_t rows, int64_t channels, int64_t ldx, float* mean,
                                 float* var, void* workspace, size_t workspace_bytes, mp_stream stream) {
    if (rows <= 0 || channels < 0 || ldx < channels) return MP_ERR_INVALID_ARGUMENT;
    if (channels == 0) return MP_OK;
    if (!x || !mean || !var || !workspace || workspace_bytes < mp_bn_stats_workspace(rows, channels))
        return MP_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(workspace) & 3) != 0) return MP_ERR_INVALID_ARGUMENT;   // FP32 moments
    hipStream_t s = mp::as_stream(stream);
    const int vec = bn_vec(x, ldx, channels);
    const int64_t per = bn_rows_per_chunk(rows, channels, vec);
    const int64_t chunks = (rows + per - 1) / per;
    const int64_t cblocks = (channels / vec + kThreads - 1) / kThreads;
    float* ws = static_cast<float*>(workspace);
    const dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(cblocks));
    if (vec == 8)
        bn_partial_kernel<8><<<grid, kThreads, 0, s>>>(x, rows, channels, ldx, per, ws);
    else
        bn_partial_kernel<1><<<grid, kThreads, 0, s>>>(x, rows, channels, ldx, per, ws);
    mp_status st = mp::launch_status("bn_partial_kernel");
    if (st != MP_OK) return st;
    bn_final_kernel<<<unsigned(channels), 64, 0, s>>>(ws, chunks, channels, mean, var);
    return mp::launch_status("bn_final_kernel");
}

extern "C" mp_status mp_bn_apply(const uint16_t* x, int64_t rows, int64_t channels, int64_t ldx, const float* mean,
                                 const float* var, const float* gamma, const float* beta, float eps, uint16_t* y,
                                 int64_t ldy, mp_stream stream) {
    if (rows < 0 || channels < 0 || ldx < channels || ldy < channels) return MP_ERR_INVALID_ARGUMENT;
    if (rows == 0 || channels == 0) return MP_OK;
    if (!x || !mean || !var || !gamma || !beta || !y) return MP_ERR_INVALID_ARGUMENT;
    hipStream_t s = mp::as_stream(stream);
    const int vec = bn_vec(x, ldx, channels, y, ldy);
    const int64_t groups = channels / vec;
    const int64_t per = 8 * (kThreads / (groups < kThreads ? groups : kThreads));   // eight rows per thread
    const dim3 grid(unsigned((rows + per - 1) / per), unsigned((channels / vec + kThreads - 1) / kThreads));
    if (vec == 8)
        bn_apply_kernel<8><<<grid, kThreads, 0, s>>>(x, rows, channels, ldx, mean, var, gamma, beta, eps, y, ldy, per);
    else
        bn_apply_kernel<1><<<grid, kThreads, 0, s>>>(x, rows, channels, ldx, mean, var, gamma, beta, eps, y, ldy, per);
    return mp::launch_status("bn_apply_kernel");
}

// Either form: the two-pass form's (max, sum) per (row, segment), or the
// single-read form's slots (one per block, at most kResMaxBlocks).
extern "C" size_t mp_softmax_workspace(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    const size_t two_pass = size_t(rows * softmax_segments(cols)) * sizeof(float2);
    const int64_t slots = rows * kResMaxParts < kResMaxBlocks ? rows * kResMaxParts : kResMaxBlocks;
    const size_t res = size_t(slots) * sizeof(ResSlot);
    return two_pass > res ? two_pass : res;
}

extern "C" int64_t mp_softmax_wait_us(int64_t us) {
    if (us < 0) return g_wait_us.load();
    return g_wait_us.exchange(us < kResMaxWaitUs ? us : kResMaxWaitUs);
}

extern "C" mp_status mp_softmax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint16_t* y, int64_t ldy,
                                void* workspace, size_t workspace_bytes, mp_stream stream) {
    if (rows < 0 || cols < 0 || ldx < cols || ldy < cols) return MP_ERR_INVALID_ARGUMENT;
    if (rows == 0 || cols == 0) return MP_OK;
    if (!x || !y || !workspace || workspace_bytes < mp_softmax_workspace(rows, cols)) return MP_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(workspace) & 7) != 0) return MP_ERR_INVALID_ARGUMENT;   // 64-bit slots
    if (rows > 0x7FFFFFFF) return MP_ERR_INVALID_ARGUMENT;
    hipStream_t s = mp::as_stream(stream);
    const int vec = (mp::aligned16(x) && mp::aligned16(y) && ldx % 8 == 0 && ldy % 8 == 0) ? 8 : 1;
    // The single-read form's per-call tag is a kernel argument: under stream
    // capture every replay of the graph would reuse it, and a block could take
    // the slots of an earlier replay for this one's. A captured call takes the
    // two-pass form, which keeps nothing between calls.
    hipStreamCaptureStatus capture = hipStreamCaptureStatusActive;
    if (hipStreamIsCapturing(s, &capture) != hipSuccess) {
        (void)hipGetLastError();                         // not a launch error of this call
        capture = hipStreamCaptureStatusActive;
    }
    if (vec == 8 && static_cast<const void*>(x) != static_cast<const void*>(y) &&
        capture == hipStreamCaptureStatusNone) {
        ResPlan p;
        mp_status st = res_plan(rows, cols, workspace_bytes, &p);
        if (st != MP_OK) return st;
        if (p.parts > 0) {
            softmax_resident_kernel<<<unsigned(rows * p.parts), kResThreads, 0, s>>>(
                x, cols, ldx, y, ldy, int(p.parts), p.seg_vecs, p.nvt, static_cast<ResSlot*>(workspace),
                res_next_tag(), p.wait_ticks);
            return mp::launch_status("softmax_resident_kernel");
        }
    }
    const int64_t S = softmax_segments(cols);
    const int64_t nvec = cols / vec;
    const int64_t seg_vecs = (nvec + S - 1) / S;
    const dim3 grid(static_cast<unsigned>(rows), static_cast<unsigned>(S));
    float2* ws = static_cast<float2*>(workspace);
    if (vec == 8)
        softmax_partial_kernel<8><<<grid, kThreads, 0, s>>>(x, cols, ldx, seg_vecs, ws);
    else
        softmax_partial_kernel<1><<<grid, kThreads, 0, s>>>(x, cols, ldx, seg_vecs, ws);
    mp_status st = mp::launch_status("softmax_partial_kernel");
    if (st != MP_OK) return st;
    if (vec == 8)
        softmax_norm_kernel<8><<<grid, kThreads, 0, s>>>(x, cols, ldx, y, ldy, seg_vecs, ws);
    else
        softmax_norm_kernel<1><<<grid, kThreads, 0, s>>>(x, cols, ldx, y, ldy, seg_vecs, ws);
    return mp::launch_status("softmax_norm_kernel");
}
