// Dot-product layers of mixed-precision training on gfx950 MFMA.
//
// Source: "Mixed Precision Training", long-form analysis page
// (paper-graph-ui.vercel.app), §3.4 "FP16 Arithmetic with FP32 Accumulation":
// dot products take binary16 inputs, sum the products in FP32 and round the
// FP32 result to binary16 only when it is stored; §3.4 "The Integrated
// Training Procedure", Steps 2 and 4: forward, activation-gradient and
// weight-gradient products of every linear layer.
//
// One kernel template computes C[i, j] = sum_r A(i, r) * B(j, r) where each
// operand is either reduction-contiguous ("KC": A(i, r) = A[i * lda + r]) or
// reduction-strided ("MN": A(i, r) = A[r * lda + i]):
//   forward  Y  = X  W^T : A = X  (KC), B = W (KC), reduction over K
//   dgrad    dX = dY W   : A = dY (KC), B = W (MN), reduction over N
//   wgrad    dW = dY^T X : A = dY (MN), B = X (MN), reduction over M
//
// Per block: a BM x BN output tile, BK = 64 reduction slices staged through
// LDS in two buffers. Both operands are stored in LDS the same way, as rows of
// 64 reduction elements (128 bytes, eight 16-byte chunks, XOR-swizzled by row
// to keep the MFMA fragment reads free of bank conflicts). A KC operand is
// copied as 16-byte vectors; an MN operand is loaded as 8 x 8 blocks of
// 16-byte vectors and transposed in registers before it is written, so the
// inner loop is the same for all three layouts. Each wave owns a
// (BM / WAVES_M) x (BN / WAVES_N) sub-tile of 32 x 32 MFMA tiles
// (v_mfma_f32_32x32x16_f16: binary16 inputs, exact products, FP32 sums).
// Blocks are renumbered so that each XCD (blocks are dealt round-robin to the
// 8 XCDs) works on a compact group of tiles that share rows of A and B in its
// own L2.
#include "mp_internal.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;          // reduction slice per LDS stage
constexpr int kRowChunks = 8;    // 16-byte chunks per LDS row (64 binary16)

struct GemmArgs {
    const uint16_t* A;
    const uint16_t* B;
    void* C;
    int64_t lda, ldb, ldc;
    int64_t Mc, Nc, R;           // output rows, output columns, reduction length
    uint32_t* flag;              // nullable: OR 1 if any binary16 output is inf/NaN
    int a_vec, b_vec;            // 16-byte global loads allowed for A / B
    int tiles_m, tiles_n;
};

// Physical 16-byte chunk of logical chunk `c` in LDS row `row`.
__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row ^ (row >> 3)) & 7); }

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// Loads 8 consecutive binary16 values p[0..7], of which only the first `valid`
// exist (valid may be <= 0). `vec` allows one 16-byte load when all 8 exist.
__device__ __forceinline__ uint4 load8(const uint16_t* p, int64_t valid, int vec) {
    if (vec && valid >= 8) return *reinterpret_cast<const uint4*>(p);
    uint16_t t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = (i < valid) ? p[i] : uint16_t(0);
    return make_uint4(uint32_t(t[0]) | uint32_t(t[1]) << 16, uint32_t(t[2]) | uint32_t(t[3]) << 16,
                      uint32_t(t[4]) | uint32_t(t[5]) << 16, uint32_t(t[6]) | uint32_t(t[7]) << 16);
}

__device__ __forceinline__ uint32_t half_of(const uint4& v, int j) {
    const uint32_t w = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
    return (j & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// A tile of one operand in flight between global memory and LDS.
template <int ROWS, int NT, bool KC>
struct TileLoader {
    // KC: ROWS*8 chunks of 16 bytes; MN: ROWS 8x8 blocks of 8 chunks each.
    static constexpr int kItems = KC ? (ROWS * kRowChunks) : ROWS;
    static constexpr int kPer = (kItems + NT - 1) / NT;
    static constexpr int kRegs = KC ? kPer : kPer * 8;
    uint4 r[kRegs];

    // Rows of the tile are [row0, row0 + ROWS) of the operand's "index" space,
    // the reduction slice is [k0, k0 + 64).
    __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int64_t rows_total,
                                         int64_t R, int64_t row0, int64_t k0, int vec, int tid) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int q = tid + u * NT;
            if (KC) {
                const int row = q / kRowChunks, kc = q % kRowChunks;
                const int64_t gr = row0 + row, gk = k0 + kc * 8;
                if (q < kItems && gr < rows_total)
                    r[u] = load8(base + gr * ld + gk, R - gk, vec);
                else
                    r[u] = zero4();
            } else {
                const int mb = q % (ROWS / 8), rb = q / (ROWS / 8);
                const int64_t gm = row0 + mb * 8;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int64_t gk = k0 + rb * 8 + i;
                    if (q < kItems && gk < R)
                        r[u * 8 + i] = load8(base + gk * ld + gm, rows_total - gm, vec);
                    else
                        r[u * 8 + i] = zero4();
                }
            }
        }
    }

    __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int q = tid + u * NT;
            if (q >= kItems) continue;
            if (KC) {
                const int row = q / kRowChunks, kc = q % kRowChunks;
                lds[row * kRowChunks + swz(row, kc)] = r[u];
            } else {
                const int mb = q % (ROWS / 8), rb = q / (ROWS / 8);
                // r[u*8 + i] holds 8 consecutive index-space values at reduction
                // offset rb*8 + i; row j of the LDS tile wants the 8 reduction
                // values of index mb*8 + j.
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint4* in = &r[u * 8];
                    uint4 o;
                    o.x = half_of(in[0], j) | (half_of(in[1], j) << 16);
                    o.y = half_of(in[2], j) | (half_of(in[3], j) << 16);
                    o.z = half_of(in[4], j) | (half_of(in[5], j) << 16);
                    o.w = half_of(in[6], j) | (half_of(in[7], j) << 16);
                    const int row = mb * 8 + j;
                    lds[row * kRowChunks + swz(row, rb)] = o;
                }
            }
        }
    }
};

template <int BM, int BN, int WAVES_M, int WAVES_N, bool A_KC, bool B_KC, bool OUT_F16>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_kernel(GemmArgs g) {
    constexpr int NT = 64 * WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int kStage = (BM + BN) * kRowChunks;         // uint4 per LDS stage
    __shared__ uint4 lds[2 * kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;

    // ---- tile order: XCD-local groups, then 8-row groups of tiles
    const int nblk = g.tiles_m * g.tiles_n;
    int lb = blockIdx.x;
    if ((nblk & 7) == 0) lb = (lb & 7) * (nblk >> 3) + (lb >> 3);
    constexpr int kGroup = 8;
    const int per_group = kGroup * g.tiles_n;
    const int grp = lb / per_group;
    const int first_m = grp * kGroup;
    const int gsize = min(g.tiles_m - first_m, kGroup);
    const int tm = first_m + (lb % per_group) % gsize;
    const int tn = (lb % per_group) / gsize;
    const int64_t row0 = int64_t(tm) * BM, col0 = int64_t(tn) * BN;

    TileLoader<BM, NT, A_KC> la;
    TileLoader<BN, NT, B_KC> lb_;

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = int((g.R + kBK - 1) / kBK);
    if (nk > 0) {
        la.load(g.A, g.lda, g.Mc, g.R, row0, 0, g.a_vec, tid);
        lb_.load(g.B, g.ldb, g.Nc, g.R, col0, 0, g.b_vec, tid);
        la.store(lds, tid);
        lb_.store(lds + BM * kRowChunks, tid);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            const int64_t k0 = int64_t(kt + 1) * kBK;
            la.load(g.A, g.lda, g.Mc, g.R, row0, k0, g.a_vec, tid);
            lb_.load(g.B, g.ldb, g.Nc, g.R, col0, k0, g.b_vec, tid);
        }
        const uint4* sA = lds + cur * kStage;
        const uint4* sB = sA + BM * kRowChunks;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int chunk = 2 * kk + (lane >> 5);
            half8 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WTM + i * 32 + (lane & 31);
                af[i] = __builtin_bit_cast(half8, sA[row * kRowChunks + swz(row, chunk)]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * WTN + j * 32 + (lane & 31);
                bf[j] = __builtin_bit_cast(half8, sB[row * kRowChunks + swz(row, chunk)]);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            uint4* nA = lds + (cur ^ 1) * kStage;
            la.store(nA, tid);
            lb_.store(nA + BM * kRowChunks, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4
    uint32_t bad = 0;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t gc = col0 + wn * WTN + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t gr =
                    row0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (gr < g.Mc && gc < g.Nc) {
                    if (OUT_F16) {
                        const uint16_t h = mp::f2h(acc[i][j][r]);
                        bad |= mp::nonfinite1(h);
                        static_cast<uint16_t*>(g.C)[gr * g.ldc + gc] = h;
                    } else {
                        static_cast<float*>(g.C)[gr * g.ldc + gc] = acc[i][j][r];
                    }
                }
            }
        }
    if (OUT_F16 && g.flag) {
        if (__syncthreads_or(bad) && tid == 0) atomicOr(g.flag, 1u);
    }
}

template <int BM, int BN, int WM, int WN, bool A_KC, bool B_KC>
mp_status launch_cfg(GemmArgs a, bool f16, hipStream_t s, const char* name) {
    a.tiles_m = int((a.Mc + BM - 1) / BM);
    a.tiles_n = int((a.Nc + BN - 1) / BN);
    const uint32_t blocks = uint32_t(a.tiles_m) * uint32_t(a.tiles_n);
    if (f16)
        gemm_kernel<BM, BN, WM, WN, A_KC, B_KC, true><<<blocks, 64 * WM * WN, 0, s>>>(a);
    else
        gemm_kernel<BM, BN, WM, WN, A_KC, B_KC, false><<<blocks, 64 * WM * WN, 0, s>>>(a);
    return mp::launch_status(name);
}

template <bool A_KC, bool B_KC>
mp_status launch(GemmArgs a, bool f16, hipStream_t s, const char* name) {
    // Large outputs: 256 x 256 tiles, 4 waves of 128 x 128. Small outputs
    // (where a 256 x 256 grid would leave most of the 256 CUs idle): 64 x 64.
    const int64_t big_tiles = ((a.Mc + 255) / 256) * ((a.Nc + 255) / 256);
    if (big_tiles >= 128) return launch_cfg<256, 256, 2, 2, A_KC, B_KC>(a, f16, s, name);
    return launch_cfg<64, 64, 2, 2, A_KC, B_KC>(a, f16, s, name);
}

bool bad_matrix(const void* p, int64_t rows, int64_t cols, int64_t ld) {
    if (rows < 0 || cols < 0) return true;
    if (rows > 0 && cols > 0 && (!p || ld < cols)) return true;
    return false;
}

// 16-byte loads need a 16-byte aligned base and a row pitch of 8 elements.
int vec_ok(const void* p, int64_t ld) { return mp::aligned16(p) && (ld % 8) == 0; }

bool too_large(int64_t Mc, int64_t Nc) {
    // tile counts must fit a 32-bit grid
    return ((Mc + 63) / 64) * ((Nc + 63) / 64) > 0x7FFFFFFF;
}

}  // namespace

extern "C" mp_status mp_linear_fwd(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                                   void* Y, int64_t ldy, mp_dtype y_dtype, int64_t M, int64_t N,
                                   int64_t K, mp_stream stream) {
    if (M < 0 || N < 0 || K < 0) return MP_ERR_INVALID_ARGUMENT;
    if (y_dtype != MP_F16 && y_dtype != MP_F32) return MP_ERR_INVALID_ARGUMENT;
    if (M == 0 || N == 0) return MP_OK;
    if (bad_matrix(X, M, K, ldx) || bad_matrix(W, N, K, ldw) || bad_matrix(Y, M, N, ldy))
        return MP_ERR_INVALID_ARGUMENT;
    if (too_large(M, N)) return MP_ERR_INVALID_ARGUMENT;
    GemmArgs a{X, W, Y, ldx, ldw, ldy, M, N, K, nullptr, vec_ok(X, ldx), vec_ok(W, ldw), 0, 0};
    return launch<true, true>(a, y_dtype == MP_F16, mp::as_stream(stream), "mp_linear_fwd");
}

extern "C" mp_status mp_linear_dgrad(const uint16_t* dY, int64_t lddy, const uint16_t* W,
                                     int64_t ldw, void* dX, int64_t lddx, mp_dtype dx_dtype,
                                     int64_t M, int64_t N, int64_t K, mp_stream stream) {
    if (M < 0 || N < 0 || K < 0) return MP_ERR_INVALID_ARGUMENT;
    if (dx_dtype != MP_F16 && dx_dtype != MP_F32) return MP_ERR_INVALID_ARGUMENT;
    if (M == 0 || K == 0) return MP_OK;
    if (bad_matrix(dY, M, N, lddy) || bad_matrix(W, N, K, ldw) || bad_matrix(dX, M, K, lddx))
        return MP_ERR_INVALID_ARGUMENT;
    if (too_large(M, K)) return MP_ERR_INVALID_ARGUMENT;
    GemmArgs a{dY, W, dX, lddy, ldw, lddx, M, K, N, nullptr, vec_ok(dY, lddy), vec_ok(W, ldw), 0, 0};
    return launch<true, false>(a, dx_dtype == MP_F16, mp::as_stream(stream), "mp_linear_dgrad");
}

extern "C" mp_status mp_linear_wgrad(const uint16_t* dY, int64_t lddy, const uint16_t* X,
                                     int64_t ldx, void* dW, int64_t lddw, mp_dtype dw_dtype,
                                     int64_t M, int64_t N, int64_t K, uint32_t* found_inf,
                                     mp_stream stream) {
    if (M < 0 || N < 0 || K < 0) return MP_ERR_INVALID_ARGUMENT;
    if (dw_dtype != MP_F16 && dw_dtype != MP_F32) return MP_ERR_INVALID_ARGUMENT;
    if (dw_dtype == MP_F32 && found_inf) return MP_ERR_INVALID_ARGUMENT;
    if (N == 0 || K == 0) return MP_OK;
    if (bad_matrix(dY, M, N, lddy) || bad_matrix(X, M, K, ldx) || bad_matrix(dW, N, K, lddw))
        return MP_ERR_INVALID_ARGUMENT;
    if (too_large(N, K)) return MP_ERR_INVALID_ARGUMENT;
    GemmArgs a{dY, X, dW, lddy, ldx, lddw, N, K, M, found_inf, vec_ok(dY, lddy), vec_ok(X, ldx), 0, 0};
    return launch<false, false>(a, dw_dtype == MP_F16, mp::as_stream(stream), "mp_linear_wgrad");
}
