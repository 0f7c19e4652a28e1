// The optimizer sweep of mixed-precision training on gfx950.
//
// Source: "Mixed Precision Training", long-form analysis page
// (paper-graph-ui.vercel.app), §3.4 "The Integrated Training Procedure":
//   Step 5 unscale the binary16 weight gradients (divide by the loss scale S);
//   Step 6 if any weight gradient is +-inf or NaN, skip the whole update;
//   Step 7 SGD with momentum on the FP32 masters, v = mu v + g, w = w - lr v
//   (or, through mp_step_opt, the Nesterov or Adagrad rule of mp_opt_kind);
//   the weight-decay paragraph: g = g + lambda w with the FP32 master w;
//   Step 1 the next iteration works on the nearest binary16 copy of w.
// §3.4 "Choosing the Loss Scaling Factor" gives the constant (method 1) and
// dynamic (method 3) rules that mp_scaler_update applies.
//
// Design (HBM-bound, 20 bytes per parameter on a clean step):
//   - The ragged tensor list is cut into fixed chunks of kChunk elements; one
//     256-thread block owns one chunk. A per-chunk tensor map in device
//     memory makes the block's lookup two scalar loads.
//   - The skip decision is global, so the sweep runs in two passes: a
//     read-only check pass over the gradients (wave ballot via
//     __syncthreads_or, one atomic OR per dirty block, early exit once the
//     flag is set), then the fused update pass, which reads the flag first and
//     leaves at once on an overflowing step. The update pass walks the chunks
//     in reverse so that its first blocks meet the gradients the check pass
//     read last, while they are still in the last-level cache.
//   - 16-byte vector loads/stores where a tensor's four base addresses are
//     16-byte aligned; a scalar path with identical arithmetic otherwise. The
//     update pass uses ordinary (temporal) loads and stores: on MI355X they
//     stream a 50/50 read/write mix faster than non-temporal ones, and two
//     16-byte vectors per thread per array beat deeper unrolling.
//   - The update is one IEEE FP32 operation per step in a fixed order; this
//     file is compiled with -ffp-contract=off, so no multiply-add is fused.
#include <string.h>

#include <new>
#include <vector>

#include "mp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;                       // elements per 16-byte binary16 vector
constexpr int kUnroll = 2;                    // vectors per thread per chunk
constexpr int64_t kChunk = int64_t(kThreads) * kVec * kUnroll;   // 4096 elements

struct DevParam {
    float* master;
    float* momentum;
    const uint16_t* grad;
    uint16_t* w16;
    int64_t numel;
    int64_t chunk_begin;
    uint32_t vec;
    uint32_t pad;
};

}  // namespace

struct mp_param_list {
    DevParam* d_desc = nullptr;
    uint32_t* d_chunk_tensor = nullptr;
    int32_t n = 0;
    int64_t numel = 0;
    int64_t chunks = 0;
    std::vector<DevParam> h_desc;              // kept alive for the async upload
    std::vector<uint32_t> h_chunk_tensor;
    hipStream_t stream = nullptr;
};

namespace {

// ---------------------------------------------------------------- check pass
__global__ __launch_bounds__(kThreads) void check_kernel(const DevParam* __restrict__ desc,
                                                         const uint32_t* __restrict__ chunk_tensor,
                                                         uint32_t* flag) {
    if (*reinterpret_cast<volatile uint32_t*>(flag)) return;      // already decided
    const uint32_t c = blockIdx.x;
    const DevParam p = desc[chunk_tensor[c]];
    const int64_t begin = (int64_t(c) - p.chunk_begin) * kChunk;
    const int64_t rem = p.numel - begin;
    const int len = rem < kChunk ? int(rem) : int(kChunk);
    const uint16_t* g = p.grad + begin;
    uint32_t bad = 0;
    if (p.vec && len == kChunk) {
        mp::u32x4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            x[u] = __builtin_nontemporal_load(
                mp::global(reinterpret_cast<const mp::u32x4*>(g)) + threadIdx.x + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            bad |= mp::nonfinite2(x[u].x) | mp::nonfinite2(x[u].y) | mp::nonfinite2(x[u].z) |
                   mp::nonfinite2(x[u].w);
    } else {
        for (int e = threadIdx.x; e < len; e += kThreads) bad |= mp::nonfinite1(g[e]);
    }
    if (__syncthreads_or(bad) && threadIdx.x == 0) atomicOr(flag, 1u);
}

// ---------------------------------------------------------------- update pass
struct Hyper {
    float lr, mu, wd, eps;
};

// One element, in the fixed order of the method (no contraction). `v` is the
// optimizer state: the velocity, or Adagrad's sum of squared gradients.
template <int OPT>
__device__ __forceinline__ void opt_elem(float& w, float& v, uint16_t h, float inv, const Hyper& hp,
                                         uint16_t& w16) {
    float gs = mp::h2f(h);      // Step 5: binary16 -> FP32 (exact)
    float g = gs * inv;         // Step 5: unscale (exact, power of two)
    float t1 = hp.wd * w;       // weight decay on the FP32 master
    g = g + t1;
    if (OPT == MP_OPT_ADAGRAD) {
        float t2 = g * g;       // accumulated squared gradient
        v = v + t2;
        float r = sqrtf(v);     // correctly rounded
        float d = r + hp.eps;
        float u = g / d;        // correctly rounded
        float t3 = hp.lr * u;
        w = w - t3;
    } else {
        float t2 = hp.mu * v;   // Step 7: momentum
        v = t2 + g;
        float st = v;
        if (OPT == MP_OPT_NESTEROV) {   // look-ahead step g + mu v
            float t4 = hp.mu * v;
            st = g + t4;
        }
        float t3 = hp.lr * st;  // Step 7: master update
        w = w - t3;
    }
    w16 = mp::f2h(w);           // Step 1: nearest binary16
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
    return uint32_t(lo) | (uint32_t(hi) << 16);
}

template <int OPT>
__global__ __launch_bounds__(kThreads) void update_kernel(const DevParam* __restrict__ desc,
                                                          const uint32_t* __restrict__ chunk_tensor,
                                                          const mp_scaler* __restrict__ scaler,
                                                          Hyper hp, uint32_t chunks) {
    if (scaler->found_inf) return;                               // Step 6: skip
    const float inv = scaler->inv_scale;
    const uint32_t c = chunks - 1u - blockIdx.x;                  // reverse walk
    const DevParam p = desc[chunk_tensor[c]];
    const int64_t begin = (int64_t(c) - p.chunk_begin) * kChunk;
    const int64_t rem = p.numel - begin;
    const int len = rem < kChunk ? int(rem) : int(kChunk);
    float* wp = p.master + begin;
    float* vp = p.momentum + begin;
    const uint16_t* gp = p.grad + begin;
    uint16_t* hp16 = p.w16 + begin;

    if (p.vec && len == kChunk) {
        mp::u32x4 g[kUnroll];
        mp::f32x4 w[kUnroll][2], v[kUnroll][2];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int e = (threadIdx.x + u * kThreads) * kVec;
            g[u] = *mp::global(reinterpret_cast<const mp::u32x4*>(gp + e));
            w[u][0] = *mp::global(reinterpret_cast<const mp::f32x4*>(wp + e));
            w[u][1] = *mp::global(reinterpret_cast<const mp::f32x4*>(wp + e + 4));
            v[u][0] = *mp::global(reinterpret_cast<const mp::f32x4*>(vp + e));
            v[u][1] = *mp::global(reinterpret_cast<const mp::f32x4*>(vp + e + 4));
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int e = (threadIdx.x + u * kThreads) * kVec;
            const uint32_t gw[4] = {g[u].x, g[u].y, g[u].z, g[u].w};
            float wv[8] = {w[u][0].x, w[u][0].y, w[u][0].z, w[u][0].w,
                           w[u][1].x, w[u][1].y, w[u][1].z, w[u][1].w};
            float vv[8] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w,
                           v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
            uint16_t hv[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint16_t h = uint16_t(gw[k >> 1] >> ((k & 1) * 16));
                opt_elem<OPT>(wv[k], vv[k], h, inv, hp, hv[k]);
            }
            *mp::global(reinterpret_cast<mp::f32x4*>(wp + e)) = mp::f32x4{wv[0], wv[1], wv[2], wv[3]};
            *mp::global(reinterpret_cast<mp::f32x4*>(wp + e + 4)) = mp::f32x4{wv[4], wv[5], wv[6], wv[7]};
            *mp::global(reinterpret_cast<mp::f32x4*>(vp + e)) = mp::f32x4{vv[0], vv[1], vv[2], vv[3]};
            *mp::global(reinterpret_cast<mp::f32x4*>(vp + e + 4)) = mp::f32x4{vv[4], vv[5], vv[6], vv[7]};
            *mp::global(reinterpret_cast<mp::u32x4*>(hp16 + e)) = mp::u32x4{pack2(hv[0], hv[1]), pack2(hv[2], hv[3]),
                                                  pack2(hv[4], hv[5]), pack2(hv[6], hv[7])};
        }
    } else {
        for (int e = threadIdx.x; e < len; e += kThreads) {
            float w = wp[e], v = vp[e];
            uint16_t h16;
            opt_elem<OPT>(w, v, gp[e], inv, hp, h16);
            wp[e] = w;
            vp[e] = v;
            hp16[e] = h16;
        }
    }
}

// ---------------------------------------------------------------- scaler
__global__ void scaler_init_kernel(mp_scaler* s, float scale, uint32_t dynamic, int32_t interval) {
    s->scale = scale;
    s->inv_scale = __uint_as_float(0x7F000000u - __float_as_uint(scale));
    s->count = 0;
    s->growth_interval = interval;
    s->found_inf = 0;
    s->dynamic = dynamic;
    s->skipped_steps = 0;
    s->reserved = 0;
}

__global__ void scaler_update_kernel(mp_scaler* s) {
    const uint32_t overflow = s->found_inf;
    float scale = s->scale;
    int32_t count = s->count;
    if (overflow) s->skipped_steps = s->skipped_steps + 1u;
    if (s->dynamic) {
        if (overflow) {
            scale = scale * 0.5f;                      // back-off factor 1/2
            if (scale < 1.0f) scale = 1.0f;
            count = 0;
        } else {
            count = count + 1;
            if (count >= s->growth_interval) {
                scale = scale * 2.0f;                  // growth factor 2
                if (scale > 0x1p64f) scale = 0x1p64f;
                count = 0;
            }
        }
    }
    s->scale = scale;
    s->count = count;
    // Exact reciprocal of a power of two in [1, 2^64]: negate the exponent.
    s->inv_scale = __uint_as_float(0x7F000000u - __float_as_uint(scale));
    s->found_inf = 0;
}

// ---------------------------------------------------------------- FP32 -> binary16
__global__ __launch_bounds__(kThreads) void round_kernel(const float* __restrict__ x,
                                                         uint16_t* __restrict__ y, int64_t n,
                                                         int vec) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (vec) {
        const int64_t nv = n / kVec;
        for (int64_t v = i; v < nv; v += stride) {
            const float4 a = reinterpret_cast<const float4*>(x)[2 * v];
            const float4 b = reinterpret_cast<const float4*>(x)[2 * v + 1];
            reinterpret_cast<uint4*>(y)[v] =
                make_uint4(pack2(mp::f2h(a.x), mp::f2h(a.y)), pack2(mp::f2h(a.z), mp::f2h(a.w)),
                           pack2(mp::f2h(b.x), mp::f2h(b.y)), pack2(mp::f2h(b.z), mp::f2h(b.w)));
        }
        for (int64_t e = nv * kVec + i; e < n; e += stride) y[e] = mp::f2h(x[e]);
    } else {
        for (int64_t e = i; e < n; e += stride) y[e] = mp::f2h(x[e]);
    }
}

bool is_pow2_scale(float s) {
    uint32_t b;
    memcpy(&b, &s, 4);
    const uint32_t e = (b >> 23) & 0xFF, m = b & 0x7FFFFF;
    return (b >> 31) == 0 && m == 0 && e >= 127 && e <= 127 + 64;
}

}  // namespace

// =========================================================================
extern "C" mp_status mp_param_list_create(const mp_param* host_params, int32_t n,
                                          mp_param_list** out, mp_stream stream) {
    if (!out || n < 0 || (n > 0 && !host_params)) return MP_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    for (int32_t i = 0; i < n; ++i) {
        const mp_param& q = host_params[i];
        if (q.numel < 0) return MP_ERR_INVALID_ARGUMENT;
        if (q.numel > 0 && (!q.master || !q.momentum || !q.grad || !q.weight16))
            return MP_ERR_INVALID_ARGUMENT;
    }
    mp_param_list* L = new (std::nothrow) mp_param_list;
    if (!L) return MP_ERR_OUT_OF_MEMORY;
    L->n = n;
    L->stream = mp::as_stream(stream);
    int64_t chunks = 0, numel = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mp_param& q = host_params[i];
        DevParam d{};
        d.master = q.master;
        d.momentum = q.momentum;
        d.grad = q.grad;
        d.w16 = q.weight16;
        d.numel = q.numel;
        d.chunk_begin = chunks;
        d.vec = mp::aligned16(q.master) && mp::aligned16(q.momentum) && mp::aligned16(q.grad) &&
                mp::aligned16(q.weight16);
        const int64_t nc = (q.numel + kChunk - 1) / kChunk;
        for (int64_t k = 0; k < nc; ++k) L->h_chunk_tensor.push_back(uint32_t(i));
        chunks += nc;
        numel += q.numel;
        L->h_desc.push_back(d);
    }
    if (chunks > 0x7FFFFFFF) { delete L; return MP_ERR_INVALID_ARGUMENT; }
    L->chunks = chunks;
    L->numel = numel;
    if (chunks > 0) {
        hipError_t e = hipMalloc(&L->d_desc, sizeof(DevParam) * L->h_desc.size());
        if (e == hipSuccess) e = hipMalloc(&L->d_chunk_tensor, sizeof(uint32_t) * size_t(chunks));
        if (e == hipSuccess)
            e = hipMemcpyAsync(L->d_desc, L->h_desc.data(), sizeof(DevParam) * L->h_desc.size(),
                               hipMemcpyHostToDevice, L->stream);
        if (e == hipSuccess)
            e = hipMemcpyAsync(L->d_chunk_tensor, L->h_chunk_tensor.data(),
                               sizeof(uint32_t) * size_t(chunks), hipMemcpyHostToDevice, L->stream);
        if (e != hipSuccess) {
            mp_status st = mp::hip_status(e, "mp_param_list_create");
            if (L->d_desc) (void)hipFree(L->d_desc);
            if (L->d_chunk_tensor) (void)hipFree(L->d_chunk_tensor);
            delete L;
            return st;
        }
    }
    *out = L;
    return MP_OK;
}

extern "C" mp_status mp_param_list_destroy(mp_param_list* L) {
    if (!L) return MP_OK;
    mp_status st = MP_OK;
    if (L->chunks > 0) {
        hipError_t e = hipStreamSynchronize(L->stream);
        if (e != hipSuccess) st = mp::hip_status(e, "mp_param_list_destroy");
        (void)hipFree(L->d_desc);
        (void)hipFree(L->d_chunk_tensor);
    }
    delete L;
    return st;
}

extern "C" int64_t mp_param_list_numel(const mp_param_list* L) { return L ? L->numel : 0; }

namespace {

mp_status run_step(const mp_param_list* L, int kind, const Hyper& hp, mp_scaler* scaler,
                   uint32_t flags, mp_stream stream) {
    if (flags & ~uint32_t(MP_GRADS_PRECHECKED | MP_CHECK_ONLY)) return MP_ERR_UNSUPPORTED;
    if (L->chunks == 0) return MP_OK;
    hipStream_t s = mp::as_stream(stream);
    const uint32_t chunks = uint32_t(L->chunks);
    if (!(flags & MP_GRADS_PRECHECKED)) {
        check_kernel<<<chunks, kThreads, 0, s>>>(L->d_desc, L->d_chunk_tensor, &scaler->found_inf);
        if (mp_status st = mp::launch_status("mp_step/check")) return st;
    }
    if (flags & MP_CHECK_ONLY) return MP_OK;
    switch (kind) {
        case MP_OPT_SGD:
            update_kernel<MP_OPT_SGD><<<chunks, kThreads, 0, s>>>(L->d_desc, L->d_chunk_tensor, scaler, hp, chunks);
            break;
        case MP_OPT_NESTEROV:
            update_kernel<MP_OPT_NESTEROV><<<chunks, kThreads, 0, s>>>(L->d_desc, L->d_chunk_tensor, scaler, hp,
                                                                      chunks);
            break;
        default:
            update_kernel<MP_OPT_ADAGRAD><<<chunks, kThreads, 0, s>>>(L->d_desc, L->d_chunk_tensor, scaler, hp,
                                                                     chunks);
            break;
    }
    return mp::launch_status("mp_step/update");
}

}  // namespace

extern "C" mp_status mp_step(const mp_param_list* L, mp_sgd hyper, mp_scaler* scaler,
                             uint32_t flags, mp_stream stream) {
    if (!L || !scaler || mp::misaligned4(scaler)) return MP_ERR_INVALID_ARGUMENT;
    const Hyper hp{hyper.lr, hyper.momentum, hyper.weight_decay, 0.0f};
    return run_step(L, MP_OPT_SGD, hp, scaler, flags, stream);
}

extern "C" mp_status mp_step_opt(const mp_param_list* L, mp_optim hyper, mp_scaler* scaler,
                                 uint32_t flags, mp_stream stream) {
    if (!L || !scaler || mp::misaligned4(scaler)) return MP_ERR_INVALID_ARGUMENT;
    if (hyper.kind != MP_OPT_SGD && hyper.kind != MP_OPT_NESTEROV && hyper.kind != MP_OPT_ADAGRAD)
        return MP_ERR_INVALID_ARGUMENT;
    if (hyper.kind == MP_OPT_ADAGRAD && !(hyper.eps > 0.0f && hyper.eps <= 3.4028235e38f))
        return MP_ERR_INVALID_ARGUMENT;
    const Hyper hp{hyper.lr, hyper.momentum, hyper.weight_decay, hyper.eps};
    return run_step(L, hyper.kind, hp, scaler, flags, stream);
}

extern "C" mp_status mp_scaler_init(mp_scaler* scaler, float init_scale, int32_t dynamic,
                                    int32_t growth_interval, mp_stream stream) {
    if (!scaler || mp::misaligned4(scaler) || !is_pow2_scale(init_scale)) return MP_ERR_INVALID_ARGUMENT;
    if (dynamic && growth_interval < 1) return MP_ERR_INVALID_ARGUMENT;
    scaler_init_kernel<<<1, 1, 0, mp::as_stream(stream)>>>(scaler, init_scale, dynamic ? 1u : 0u,
                                                           growth_interval);
    return mp::launch_status("mp_scaler_init");
}

extern "C" mp_status mp_scaler_update(mp_scaler* scaler, mp_stream stream) {
    if (!scaler || mp::misaligned4(scaler)) return MP_ERR_INVALID_ARGUMENT;
    scaler_update_kernel<<<1, 1, 0, mp::as_stream(stream)>>>(scaler);
    return mp::launch_status("mp_scaler_update");
}

extern "C" mp_status mp_round_f32_to_f16(const float* w32, uint16_t* w16, int64_t n,
                                         mp_stream stream) {
    if (n < 0 || (n > 0 && (!w32 || !w16))) return MP_ERR_INVALID_ARGUMENT;
    if (n == 0) return MP_OK;
    const int vec = mp::aligned16(w32) && mp::aligned16(w16);
    int64_t blocks = (n / kVec + kThreads - 1) / kThreads;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    round_kernel<<<uint32_t(blocks), kThreads, 0, mp::as_stream(stream)>>>(w32, w16, n, vec);
    return mp::launch_status("mp_round_f32_to_f16");
}
