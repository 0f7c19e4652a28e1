// Point-wise activations and losses around the hot path.
//
// Source: "Mixed Precision Training", long-form analysis page
// (paper-graph-ui.vercel.app), §3.4 "FP16 Arithmetic with FP32 Accumulation"
// (point-wise ops may run in either precision and are bandwidth-bound; large
// reductions such as the softmax normaliser run in FP32) and "The Integrated
// Training Procedure", Step 3 (the loss is multiplied by the scale S before
// back-propagation, so every gradient below the loss carries the factor S).
//
// Point-wise kernels read binary16, compute in FP32 and write binary16, with
// 16-byte vectors when the buffers allow. The losses reduce in FP32 in a
// fixed order (per-block partials in a caller-owned workspace, then a single
// block), so the loss value is deterministic and calls with disjoint buffers
// share no device state; the loss gradient is S * dL/dy in FP32, rounded once
// to binary16. S is read from the device scaler, so no host round trip is
// needed.
#include "mp_act.h"
#include "mp_loss.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxPartials = 1024;    // blocks of a loss kernel = FP32 partials in the workspace

using mp::act_bwd1;
using mp::act_fwd1;

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xFFFFu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }

template <int KIND>
__global__ __launch_bounds__(kThreads) void act_fwd_kernel(const uint16_t* __restrict__ x,
                                                           uint16_t* __restrict__ y, int64_t n,
                                                           int vec) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    const int64_t i0 = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    int64_t tail = 0;
    if (vec) {
        const int64_t nv = n / 8;
        for (int64_t v = i0; v < nv; v += stride) {
            const uint4 a = reinterpret_cast<const uint4*>(x)[v];
            const uint32_t w[4] = {a.x, a.y, a.z, a.w};
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = uint32_t(act_fwd1<KIND>(uint16_t(lo16(w[k])))) |
                       (uint32_t(act_fwd1<KIND>(uint16_t(hi16(w[k])))) << 16);
            reinterpret_cast<uint4*>(y)[v] = make_uint4(o[0], o[1], o[2], o[3]);
        }
        tail = nv * 8;
    }
    for (int64_t e = tail + i0; e < n; e += stride) y[e] = act_fwd1<KIND>(x[e]);
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void act_bwd_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ dy,
                                                           uint16_t* __restrict__ dx, int64_t n,
                                                           int vec) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    const int64_t i0 = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    int64_t tail = 0;
    if (vec) {
        const int64_t nv = n / 8;
        for (int64_t v = i0; v < nv; v += stride) {
            const uint4 a = reinterpret_cast<const uint4*>(x)[v];
            const uint4 b = reinterpret_cast<const uint4*>(dy)[v];
            const uint32_t wx[4] = {a.x, a.y, a.z, a.w};
            const uint32_t wd[4] = {b.x, b.y, b.z, b.w};
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = uint32_t(act_bwd1<KIND>(uint16_t(lo16(wx[k])), uint16_t(lo16(wd[k])))) |
                       (uint32_t(act_bwd1<KIND>(uint16_t(hi16(wx[k])), uint16_t(hi16(wd[k])))) << 16);
            reinterpret_cast<uint4*>(dx)[v] = make_uint4(o[0], o[1], o[2], o[3]);
        }
        tail = nv * 8;
    }
    for (int64_t e = tail + i0; e < n; e += stride) dx[e] = act_bwd1<KIND>(x[e], dy[e]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Block sum in a fixed order: waves reduce with butterflies, then wave 0 adds
// the wave totals in index order.
__device__ float block_sum(float v) {
    __shared__ float ws[kThreads / 64];
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.0f;
    if (threadIdx.x == 0)
        for (int w = 0; w < kThreads / 64; ++w) t += ws[w];
    return t;
}

// One wave per row; the block's waves take rows wave, wave + total_waves, ...
// With m = max_c z_c at the first index a attaining it and r = sum_{c != a} exp(z_c - m):
//   log sum exp = m + log1p(r),   softmax_c = exp(z_c - m) / (1 + r),
// and for the label at the argmax softmax - 1 = -r / (1 + r). Excluding the argmax from
// the sum keeps the loss and the gradient accurate in FP32 when one class dominates.
__device__ __forceinline__ void argmax_merge(float& v, int64_t& i, float v2, int64_t i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__global__ __launch_bounds__(kThreads) void softmax_ce_kernel(const uint16_t* __restrict__ z,
                                                              const int32_t* __restrict__ labels,
                                                              int64_t B, int64_t C,
                                                              const mp_scaler* __restrict__ sc,
                                                              uint16_t* __restrict__ dz,
                                                              float* __restrict__ partials) {
    const float S = sc->scale;
    const float invB = 1.0f / float(B);
    const int lane = threadIdx.x & 63;
    const int64_t wave = int64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
    const int64_t waves = int64_t(gridDim.x) * (kThreads / 64);
    float part = 0.0f;
    for (int64_t b = wave; b < B; b += waves) {
        const uint16_t* row = z + b * C;
        float mx = -INFINITY;
        int64_t am = C;
        for (int64_t c = lane; c < C; c += 64) argmax_merge(mx, am, mp::h2f(row[c]), c);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float v2 = __shfl_xor(mx, off, 64);
            const int64_t i2 = __shfl_xor(am, off, 64);
            argmax_merge(mx, am, v2, i2);
        }
        float rest = 0.0f;
        for (int64_t c = lane; c < C; c += 64)
            if (c != am) rest += expf(mp::h2f(row[c]) - mx);
        rest = wave_sum(rest);
        const float denom = 1.0f + rest;
        const float l1p = log1pf(rest);
        const int32_t y = labels[b];
        if (lane == 0 && y >= 0 && y < C)
            part += (y == am) ? l1p : (mx - mp::h2f(row[y])) + l1p;
        for (int64_t c = lane; c < C; c += 64) {
            float d;
            if (c == y && c == am) {
                d = -rest / denom;
            } else {
                const float p = (c == am ? 1.0f : expf(mp::h2f(row[c]) - mx)) / denom;
                d = p - (c == y ? 1.0f : 0.0f);
            }
            dz[b * C + c] = mp::f2h(S * (d * invB));
        }
    }
    const float t = block_sum(part);
    if (threadIdx.x == 0) partials[blockIdx.x] = t;
}

__global__ __launch_bounds__(kThreads) void mse_kernel(const uint16_t* __restrict__ y,
                                                       const uint16_t* __restrict__ t, int64_t n,
                                                       float coef, const mp_scaler* __restrict__ sc,
                                                       uint16_t* __restrict__ dy, int vec,
                                                       float* __restrict__ partials) {
    const float S = sc->scale;
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    const int64_t i0 = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    float part = 0.0f;
    int64_t tail = 0;
    if (vec) {
        const int64_t nv = n / 8;
        for (int64_t v = i0; v < nv; v += stride) {
            const uint4 a = reinterpret_cast<const uint4*>(y)[v];
            const uint4 b = reinterpret_cast<const uint4*>(t)[v];
            const uint32_t wy[4] = {a.x, a.y, a.z, a.w};
            const uint32_t wt[4] = {b.x, b.y, b.z, b.w};
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float d0 = mp::h2f(uint16_t(lo16(wy[k]))) - mp::h2f(uint16_t(lo16(wt[k])));
                const float d1 = mp::h2f(uint16_t(hi16(wy[k]))) - mp::h2f(uint16_t(hi16(wt[k])));
                part += d0 * d0;
                part += d1 * d1;
                o[k] = uint32_t(mp::f2h(S * (coef * d0))) | (uint32_t(mp::f2h(S * (coef * d1))) << 16);
            }
            reinterpret_cast<uint4*>(dy)[v] = make_uint4(o[0], o[1], o[2], o[3]);
        }
        tail = nv * 8;
    }
    for (int64_t e = tail + i0; e < n; e += stride) {
        const float d = mp::h2f(y[e]) - mp::h2f(t[e]);
        part += d * d;
        dy[e] = mp::f2h(S * (coef * d));
    }
    const float s = block_sum(part);
    if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

// *loss = mul * sum(partials[0..count)): each thread adds its strided share in
// index order, then the block sum (fixed order).
__global__ __launch_bounds__(kThreads) void finish_kernel(const float* __restrict__ partials, int count,
                                                          float mul, float* loss) {
    float v = 0.0f;
    for (int i = threadIdx.x; i < count; i += kThreads) v += partials[i];
    const float t = block_sum(v);
    if (threadIdx.x == 0) *loss = t * mul;
}

uint32_t grid_for(int64_t work_items) {
    int64_t b = (work_items + kThreads - 1) / kThreads;
    if (b < 1) b = 1;
    if (b > kMaxPartials) b = kMaxPartials;
    return uint32_t(b);
}

}  // namespace

extern "C" mp_status mp_act_fwd(mp_act kind, const uint16_t* x, uint16_t* y, int64_t n,
                                mp_stream stream) {
    if (n < 0 || (n > 0 && (!x || !y))) return MP_ERR_INVALID_ARGUMENT;
    if (kind != MP_ACT_RELU && kind != MP_ACT_GELU) return MP_ERR_INVALID_ARGUMENT;
    if (n == 0) return MP_OK;
    const int vec = mp::aligned16(x) && mp::aligned16(y);
    const uint32_t grid = grid_for((n + 7) / 8);
    hipStream_t s = mp::as_stream(stream);
    if (kind == MP_ACT_RELU) act_fwd_kernel<MP_ACT_RELU><<<grid, kThreads, 0, s>>>(x, y, n, vec);
    else act_fwd_kernel<MP_ACT_GELU><<<grid, kThreads, 0, s>>>(x, y, n, vec);
    return mp::launch_status("mp_act_fwd");
}

extern "C" mp_status mp_act_bwd(mp_act kind, const uint16_t* x, const uint16_t* dy, uint16_t* dx,
                                int64_t n, mp_stream stream) {
    if (n < 0 || (n > 0 && (!x || !dy || !dx))) return MP_ERR_INVALID_ARGUMENT;
    if (kind != MP_ACT_RELU && kind != MP_ACT_GELU) return MP_ERR_INVALID_ARGUMENT;
    if (n == 0) return MP_OK;
    const int vec = mp::aligned16(x) && mp::aligned16(dy) && mp::aligned16(dx);
    const uint32_t grid = grid_for((n + 7) / 8);
    hipStream_t s = mp::as_stream(stream);
    if (kind == MP_ACT_RELU) act_bwd_kernel<MP_ACT_RELU><<<grid, kThreads, 0, s>>>(x, dy, dx, n, vec);
    else act_bwd_kernel<MP_ACT_GELU><<<grid, kThreads, 0, s>>>(x, dy, dx, n, vec);
    return mp::launch_status("mp_act_bwd");
}

namespace {
uint32_t ce_grid(int64_t B) { return grid_for((B + 3) / 4 * kThreads); }
uint32_t mse_grid(int64_t n) { return grid_for((n + 7) / 8); }
bool ws_ok(const void* ws, size_t bytes, uint32_t grid) {
    return ws && (reinterpret_cast<uintptr_t>(ws) & 3u) == 0 && bytes >= size_t(grid) * sizeof(float);
}
}  // namespace

extern "C" size_t mp_loss_softmax_ce_workspace(int64_t B, int64_t C) {
    if (B <= 0 || C <= 0) return 0;
    return size_t(ce_grid(B)) * sizeof(float);
}

extern "C" size_t mp_loss_mse_workspace(int64_t M, int64_t N) {
    if (M <= 0 || N <= 0) return 0;
    return size_t(mse_grid(M * N)) * sizeof(float);
}

extern "C" mp_status mp_loss_softmax_ce(const uint16_t* logits, const int32_t* labels, int64_t B,
                                        int64_t C, const mp_scaler* scaler, float* loss,
                                        uint16_t* dlogits, void* workspace, size_t workspace_bytes,
                                        mp_stream stream) {
    if (B < 0 || C < 0) return MP_ERR_INVALID_ARGUMENT;
    if (!scaler || !loss || mp::misaligned4(scaler) || mp::misaligned4(loss)) return MP_ERR_INVALID_ARGUMENT;
    if (B > 0 && C > 0 && (!logits || !labels || !dlogits)) return MP_ERR_INVALID_ARGUMENT;
    if (B == 0 || C == 0) return MP_OK;
    const uint32_t grid = ce_grid(B);
    if (!ws_ok(workspace, workspace_bytes, grid)) return MP_ERR_INVALID_ARGUMENT;
    float* partials = static_cast<float*>(workspace);
    hipStream_t s = mp::as_stream(stream);
    softmax_ce_kernel<<<grid, kThreads, 0, s>>>(logits, labels, B, C, scaler, dlogits, partials);
    if (mp_status st = mp::launch_status("mp_loss_softmax_ce")) return st;
    finish_kernel<<<1, kThreads, 0, s>>>(partials, int(grid), 1.0f / float(B), loss);
    return mp::launch_status("mp_loss_softmax_ce/finish");
}

namespace mp {
// The MSE loss with its partials in `partials` (at least loss_mse_partials(M, N) floats);
// the arguments are checked by the caller (loss_mse_args).
mp_status loss_mse_into(const uint16_t* y, const uint16_t* t, int64_t M, int64_t N, float c,
                        const mp_scaler* scaler, float* loss, uint16_t* dy, float* partials,
                        hipStream_t s) {
    const int64_t n = M * N;
    const double mn = double(M) * double(N);
    const float coef = float(2.0 * double(c) / mn);
    const int vec = mp::aligned16(y) && mp::aligned16(t) && mp::aligned16(dy);
    const uint32_t grid = mse_grid(n);
    mse_kernel<<<grid, kThreads, 0, s>>>(y, t, n, coef, scaler, dy, vec, partials);
    if (mp_status st = mp::launch_status("mp_loss_mse")) return st;
    finish_kernel<<<1, kThreads, 0, s>>>(partials, int(grid), float(double(c) / mn), loss);
    return mp::launch_status("mp_loss_mse/finish");
}

mp_status loss_mse_args(const uint16_t* y, const uint16_t* t, int64_t M, int64_t N,
                        const mp_scaler* scaler, const float* loss, const uint16_t* dy) {
    if (M < 0 || N < 0 || !scaler || !loss) return MP_ERR_INVALID_ARGUMENT;
    if (mp::misaligned4(scaler) || mp::misaligned4(loss)) return MP_ERR_INVALID_ARGUMENT;
    if (M > 0 && N > 0 && (!y || !t || !dy)) return MP_ERR_INVALID_ARGUMENT;
    return MP_OK;
}
size_t loss_mse_partials(int64_t M, int64_t N) { return M > 0 && N > 0 ? mse_grid(M * N) : 0; }
}  // namespace mp

extern "C" mp_status mp_loss_mse(const uint16_t* y, const uint16_t* t, int64_t M, int64_t N,
                                 float c, const mp_scaler* scaler, float* loss, uint16_t* dy,
                                 void* workspace, size_t workspace_bytes, mp_stream stream) {
    if (mp_status st = mp::loss_mse_args(y, t, M, N, scaler, loss, dy)) return st;
    if (M == 0 || N == 0) return MP_OK;
    if (!ws_ok(workspace, workspace_bytes, mse_grid(M * N))) return MP_ERR_INVALID_ARGUMENT;
    return mp::loss_mse_into(y, t, M, N, c, scaler, loss, dy, static_cast<float*>(workspace),
                             mp::as_stream(stream));
}
