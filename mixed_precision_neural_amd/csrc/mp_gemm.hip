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
// LDS in two buffers; the next slice's global loads are in flight while the
// current slice feeds the MFMAs (v_mfma_f32_16x16x32_f16: binary16 inputs,
// exact products, FP32 sums; on random data it draws less power per FLOP than
// the 32 x 32 x 16 form, so the chip holds a higher clock under it). Each
// operand keeps its global layout in LDS, so every global load and LDS store
// is a plain 16-byte vector:
//   KC tile: ROWS rows of 64 reduction elements (128 bytes, 8 chunks of 16
//     bytes), chunk c of row r at r*8 + (c ^ (r & 7)); an MFMA fragment row is
//     one ds_read_b128, and the 16 rows x 4 chunks of a fragment read hit
//     every LDS bank once.
//   MN tile: 64 reduction rows of ROWS index elements, chunk c of row k at
//     k*ROWS/8 + (c ^ swz_mn(k)); an MFMA fragment is two ds_read_b64_tr_b16,
//     whose lane j of each 16-lane group collects element j of the four
//     8-byte pieces its group reads, i.e. four reduction values of one index
//     column.
// Whole 256 x 256 tiles take a loop unrolled over the two LDS stages: 8 waves
// of 128 x 64, two per SIMD, one of which loads the next slab straight from
// global memory into LDS (buffer loads with scalar slab offsets) while its
// partner only reads fragments and issues MFMAs; fragment addresses are a few
// per-lane registers plus immediates, and an explicit instruction order puts
// the loads and the next step's LDS reads between the MFMAs.
// Edge tiles and small grids use a general loop with clamped, zero-filled
// loads staged through registers.
// Blocks are renumbered so that each XCD (blocks are dealt round-robin to the
// 8 XCDs) works on a compact group of tiles that share rows of A and B in its
// own L2. Binary16 outputs are rounded into LDS and written back as whole
// 16-byte row pieces; the activation-fused modes apply the point-wise step to
// those pieces.
#include "mp_act.h"

#include <type_traits>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

constexpr int kBK = 64;          // reduction slice per LDS stage
constexpr int kRowChunks = 8;    // 16-byte chunks per KC row (64 binary16)

struct GemmArgs {
    const uint16_t* A;
    const uint16_t* B;
    void* C;
    int64_t lda, ldb, ldc;
    int64_t Mc, Nc, R;           // output rows, output columns, reduction length
    uint32_t* flag;              // nullable: OR 1 if any binary16 output is inf/NaN
    int a_vec, b_vec;            // 16-byte global loads allowed for A / B
    int c_vec;                   // 16-byte output stores allowed (aligned base, ldc % 8 == 0 / % 4 for FP32)
    void* C2;                    // kEpiAct: act(C); kEpiActD: act'(Z) (binary16), ldc2
    const uint16_t* Z;           // kEpiDact: saved pre-activation; kEpiMul: saved act' (binary16), ldz
    int64_t ldc2, ldz;
    int aux_vec;                 // 16-byte access allowed for C2 / Z
    int pipe_ok;                 // non-empty reduction, operand panels under 4 GB: the buffer-load main loop applies
    int tiles_m, tiles_n;
};

// Epilogue modes.
constexpr int kEpiF32 = 0;       // C = acc (FP32)
constexpr int kEpiF16 = 1;       // C = RNE16(acc)
constexpr int kEpiAct = 2;       // C = RNE16(acc), C2 = act(C)             (forward of an activated layer)
constexpr int kEpiDact = 3;      // C = act'(Z) * RNE16(acc), rounded once  (dgrad into an activated layer)
constexpr int kEpiActD = 4;      // Z = RNE16(acc) (not stored): C = act(Z), C2 = RNE16(act'(Z))
constexpr int kEpiMul = 5;       // C = RNE16(RNE16(acc) * D), D = Z the stored act'  (dgrad with act' saved)

__device__ __forceinline__ int swz_kc(int row) { return row & 7; }
template <int CHUNKS>
__device__ __forceinline__ int swz_mn(int krow) { return ((krow & 3) << 2 ^ ((krow >> 3) & 1) << 1) & (CHUNKS - 1); }

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// Loads of 8 consecutive binary16 values p[0..7]. The edge version never
// branches: every element is read through a clamped (always valid) address and
// zeroed afterwards when it lies outside [0, valid), so the loads of a tile
// stay in flight together instead of waiting one by one.
__device__ __forceinline__ uint4 load8_full(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ uint4 load8_edge(const uint16_t* p, const uint16_t* safe, int64_t valid) {
    uint32_t t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const bool ok = i < valid;
        const uint16_t v = *(ok ? p + i : safe);
        t[i] = ok ? uint32_t(v) : 0u;
    }
    return make_uint4(t[0] | t[1] << 16, t[2] | t[3] << 16, t[4] | t[5] << 16, t[6] | t[7] << 16);
}

// One operand's tile (ROWS index rows x 64 reduction elements) in flight from
// global memory to LDS: ROWS * 8 chunks of 16 bytes, kPer per thread.
template <int ROWS, int NT, bool KC>
struct TileLoader {
    static constexpr int kItems = ROWS * kRowChunks;
    static constexpr int kPer = kItems / NT;
    static constexpr int kMnChunks = ROWS / 8;       // chunks per MN row
    static_assert(kItems % NT == 0, "threads must divide the tile");
    uint4 r[kPer];

    // FULL: the whole tile is in bounds and 16-byte loads are allowed.
    template <bool FULL>
    __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int64_t rows_total,
                                         int64_t R, int64_t row0, int64_t k0, int tid) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int q = tid + u * NT;
            if (KC) {
                const int row = q / kRowChunks, kc = q % kRowChunks;
                const int64_t gr = row0 + row, gk = k0 + kc * 8;
                if (FULL) {
                    r[u] = load8_full(base + gr * ld + gk);
                } else {
                    const bool ok = gr < rows_total;
                    r[u] = load8_edge(base + (ok ? gr : 0) * ld + gk, base, ok ? R - gk : 0);
                }
            } else {
                const int k = q / kMnChunks, cb = q % kMnChunks;
                const int64_t gk = k0 + k, gm = row0 + cb * 8;
                if (FULL) {
                    r[u] = load8_full(base + gk * ld + gm);
                } else {
                    const bool ok = gk < R;
                    r[u] = load8_edge(base + (ok ? gk : 0) * ld + gm, base, ok ? rows_total - gm : 0);
                }
            }
        }
    }

    __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int q = tid + u * NT;
            if (KC) {
                const int row = q / kRowChunks, kc = q % kRowChunks;
                lds[row * kRowChunks + (kc ^ swz_kc(row))] = r[u];
            } else {
                const int k = q / kMnChunks, cb = q % kMnChunks;
                lds[k * kMnChunks + (cb ^ swz_mn<kMnChunks>(k))] = r[u];
            }
        }
    }
};

// MFMA fragment of index rows [r0, r0 + 16) for reduction step ks (32
// values) from one operand's LDS tile of ROWS index rows: lane l holds index
// r0 + (l & 15) and the 8 reduction values 32 ks + 8 (l >> 4) .. + 7.
template <int ROWS, bool KC>
__device__ __forceinline__ half8 frag(const uint4* tile, int r0, int ks, int lane) {
    if (KC) {
        const int row = r0 + (lane & 15);
        const int c = 4 * ks + (lane >> 4);
        return __builtin_bit_cast(half8, tile[row * kRowChunks + (c ^ swz_kc(row))]);
    } else {
        constexpr int kMnChunks = ROWS / 8;
        const int g4 = lane >> 4, ii = lane & 15;
        const int n = r0 + 4 * (ii & 3);
        short4_t v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int krow = 32 * ks + 8 * g4 + 4 * h + (ii >> 2);
            const int chunk = krow * kMnChunks + ((n >> 3) ^ swz_mn<kMnChunks>(krow));
            const __attribute__((address_space(3))) uint8_t* p =
                (const __attribute__((address_space(3))) uint8_t*)(tile + chunk) + ((n >> 2) & 1) * 8;
            v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p));
        }
        const short8_t w = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
        return __builtin_bit_cast(half8, w);
    }
}

// The reduction loop of one block.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool A_KC, bool B_KC, bool FULL, int FM, int FN>
__device__ __forceinline__ void reduce_tile(const GemmArgs& g, uint4* st0, uint4* st1, int64_t row0, int64_t col0,
                                            int tid, int lane, int wm, int wn,
                                            floatx4 (&acc)[FM][FN]) {
    constexpr int NT = 64 * WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    TileLoader<BM, NT, A_KC> la;
    TileLoader<BN, NT, B_KC> lb;
    const int nk = int((g.R + kBK - 1) / kBK);
    if (nk <= 0) return;
    la.template load<FULL>(g.A, g.lda, g.Mc, g.R, row0, 0, tid);
    lb.template load<FULL>(g.B, g.ldb, g.Nc, g.R, col0, 0, tid);
    la.store(st0, tid);
    lb.store(st0 + BM * kRowChunks, tid);
    __syncthreads();

    auto read_frags = [&](const uint4* st, int ks, half8 (&af)[FM], half8 (&bf)[FN]) {
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = frag<BM, A_KC>(st, wm * WTM + i * 16, ks, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = frag<BN, B_KC>(st + BM * kRowChunks, wn * WTN + j * 16, ks, lane);
    };
    // The two reduction steps of one slice.
    auto slice = [&](const uint4* st) {
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            half8 af[FM], bf[FN];
            read_frags(st, ks, af, bf);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[j], af[i], acc[i][j], 0, 0, 0);
        }
    };

    int kt = 0;
    for (; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int64_t k0 = int64_t(kt + 1) * kBK;
            la.template load<FULL>(g.A, g.lda, g.Mc, g.R, row0, k0, tid);
            lb.template load<FULL>(g.B, g.ldb, g.Nc, g.R, col0, k0, tid);
        }
        slice(cur ? st1 : st0);
        if (more) {
            uint4* nxt = cur ? st0 : st1;
            la.store(nxt, tid);
            lb.store(nxt + BM * kRowChunks, tid);
        }
        __syncthreads();
    }
}

// One operand's slab (ROWS index rows x 64 reduction elements) fetched by
// buffer loads that write LDS directly: lane i of such a load stores its 16
// bytes at the instruction's LDS address + 16 i, so each of the WAVES loading
// waves fills kPer whole 1 KB blocks of the operand's region, and lane i of
// block b fetches the global chunk that the fragment layout places at chunk
// 64 b + i (both swizzles are XORs, hence their own inverses). No registers
// hold the slab and no LDS store instructions are issued. The resource covers
// the operand's panel; each lane keeps a fixed 32-bit byte offset per block,
// and the slab is a scalar offset.
template <int ROWS, int WAVES, bool KC>
struct DmaLoader {
    static constexpr int kBlocks = ROWS * kRowChunks / 64;   // 1 KB blocks per slab
    static constexpr int kPer = kBlocks / WAVES;
    static constexpr int C = ROWS / 8;                       // 16-byte chunks per MN row
    static_assert(kBlocks % WAVES == 0, "the waves share the blocks evenly");
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t voff[kPer];
    uint32_t blk0;                                           // wave's first block, bytes (uniform)

    // panel: A(row0, 0) for KC, A(0, row0) for MN; wave: a wave-uniform index
    __device__ __forceinline__ void init(const uint16_t* panel, int64_t ld, int wave, int lane) {
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(panel), 0, -1, 0x00020000);
        blk0 = uint32_t(wave * kPer * 1024);
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            const int q = (wave * kPer + t) * 64 + lane;         // LDS chunk this lane fills
            if (KC) {
                const int row = q / kRowChunks, kc = (q % kRowChunks) ^ swz_kc(row);
                voff[t] = uint32_t((int64_t(row) * ld + kc * 8) * 2);
            } else {
                const int k = q / C, cb = (q % C) ^ swz_mn<C>(k);
                voff[t] = uint32_t((int64_t(k) * ld + cb * 8) * 2);
            }
        }
    }
    // region: the operand's part of the target stage; soff: the slab's byte offset in the panel
    __device__ __forceinline__ void fetch(__attribute__((address_space(3))) uint8_t* region, uint32_t soff) const {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
        for (int t = 0; t < kPer; ++t)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)(region + blk0 + t * 1024), 16, voff[t], soff, 0, 0);
#endif
    }
};

// Per-lane LDS byte addresses of one operand's MFMA fragments, folded so that
// everything but the lane-dependent XOR swizzle is an immediate offset of the
// ds_read (the stage, the 16-row blocks, the reduction step):
//   KC: fragment (i, ks) of a wave's rows R0 + 16 i + (lane & 15) is chunk
//       4 ks + lane / 16 of its row, stored at that chunk ^ (row & 7) =
//       (lane / 16 ^ lane & 7) ^ 4 ks: two addresses (ks), plus 2048 i.
//   MN: fragment (j, ks) of the wave's 16-column block j takes reduction rows
//       32 ks + 8 (lane / 16) + 4 h + (lane & 15) / 4 (h: its two transposing
//       reads). The chunk swizzle depends on the lane only (it leaves bits 2
//       and 5 of the reduction row alone), so one address per block j covers
//       both reads and both steps (h and ks immediates).
typedef const __attribute__((address_space(3))) uint8_t lds_u8;

template <int ROWS, bool KC, int NBLK>
struct FragAddr {
    static constexpr int kRegs = KC ? 2 : NBLK;
    static constexpr int C = ROWS / 8;                       // 16-byte chunks per MN reduction row
    uint32_t a[kRegs];
    // r0w: first index row of the wave's block (a multiple of 16); base: byte offset of the operand's stage 0
    __device__ __forceinline__ void init(int r0w, int lane, uint32_t base) {
        if (KC) {
            const int x = (lane >> 4) ^ (lane & 7);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) a[ks] = base + uint32_t((r0w + (lane & 15)) * 128 + 16 * (x ^ (4 * ks)));
        } else {
            const int g4 = lane >> 4, ii = lane & 15;
            const int k0 = 8 * g4 + (ii >> 2);
            const int sw = swz_mn<C>(k0);
#pragma unroll
            for (int j = 0; j < kRegs; ++j) {
                const int n = r0w + 16 * j + 4 * (ii & 3);
                a[j] = base + uint32_t(k0 * C * 16 + 16 * ((n >> 3) ^ sw) + 8 * (ii & 1));
            }
        }
    }
    // fragment idx (i for KC rows, j for MN columns) of reduction step ks; off: stage offset in bytes
    __device__ __forceinline__ half8 read(lds_u8* lds, int idx, int ks, uint32_t off) const {
        if (KC) {
            return *reinterpret_cast<const __attribute__((address_space(3))) half8*>(lds + a[ks] + 2048 * idx + off);
        } else {
            constexpr uint32_t kStep = 32 * C * 16, kHalf = 4 * C * 16;   // bytes per 32 and per 4 reduction rows
            const uint32_t o = a[idx] + ks * kStep + off;
            short4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(lds + o));
            short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(lds + o + kHalf));
            const short8_t w = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            return __builtin_bit_cast(half8, w);
        }
    }
};

// The reduction loop for whole 256 x 256 tiles (reduction a multiple of 128,
// 16-byte aligned rows, panels under 4 GB). Stage s is the LDS variable st[s]
// (A's slab at byte 0, B's at kAStage); slab kt lives in stage kt & 1. The two
// stages are separate variables so that the compiler can tell a fragment read
// of one stage from a load in flight into the other and waits for those loads
// only where this code says so. The loop is unrolled over the two stages, so
// every LDS address is one of a few per-lane registers plus an immediate. A
// slab is two reduction steps of 32. Each slab issues the next slab's loads
// into the other stage under its step 0, reads step 1's fragments under step
// 0's MFMAs, and waits for its loads half way into step 1 at the slab's one
// barrier; the rest of step 1's MFMAs follow the barrier and cover the next
// slab's step-0 fragment reads.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool A_KC, bool B_KC, int FM, int FN>
__device__ __forceinline__ void reduce_tile_pipe(const GemmArgs& g, uint4* st0, uint4* st1, int64_t row0,
                                                 int64_t col0, int lane, int wm, int wn,
                                                 floatx4 (&acc)[FM][FN]) {
    constexpr int WAVES = WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr uint32_t kAStage = BM * kRowChunks * 16;                    // bytes
    constexpr int kReads = FM * (A_KC ? 1 : 2) + FN * (B_KC ? 1 : 2);   // LDS reads per reduction step
    // With 8 waves, waves 0-3 (one per SIMD: a block's waves are dealt to the 4
    // SIMDs in turn) load the slabs and waves 4-7 only compute. A loading wave
    // stalls whenever the CU's vector-memory path is backed up; its partner's
    // MFMAs keep the SIMD's matrix core busy meanwhile. The loading waves run
    // at a higher issue priority so that their loads go out as early as possible.
    constexpr int kLoadWaves = WAVES == 8 ? 4 : WAVES;
    using LA = DmaLoader<BM, kLoadWaves, A_KC>;
    using LB = DmaLoader<BN, kLoadWaves, B_KC>;
    constexpr int kLoads = LA::kPer + LB::kPer;                          // loads per loading wave per slab
    constexpr int kMfma = FM * FN;                                       // MFMAs per reduction step
    // Step 1's MFMAs before the barrier (half): the loads, issued under step 0,
    // get 32 MFMAs before their wait; the other half of step 1 covers the next
    // slab's step-0 reads.
    constexpr int kPre = kMfma / 2;
    static_assert(FM == 8 && FN == 4 && WTM == 16 * FM && WTN == 16 * FN, "8 x 4 blocks of 16 x 16 per wave");
    static_assert(2 * kLoads <= kMfma && kReads <= kMfma, "loads and reads fit step 0");
    static_assert(kAStage <= 32768 && BN * kRowChunks * 16 <= 32768, "fragment offsets must fit the LDS immediate");
    const int nk = int(g.R / kBK);
    typedef __attribute__((address_space(3))) uint8_t lds8;
    lds8* s8[2] = {(lds8*)st0, (lds8*)st1};
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const bool loader = wave < kLoadWaves;
    FragAddr<BM, A_KC, FM> fa;
    FragAddr<BN, B_KC, FN> fb;
    fa.init(wm * WTM, lane, 0);
    fb.init(wn * WTN, lane, kAStage);
    // byte offset of slab kt within a panel: 64 elements along a KC row, 64 rows of an MN panel
    const uint32_t a_step = A_KC ? 2 * kBK : uint32_t(2 * kBK * g.lda);
    const uint32_t b_step = B_KC ? 2 * kBK : uint32_t(2 * kBK * g.ldb);
    // Step 1's fragments, read under step 0's MFMAs: B's first (every MFMA of
    // step 0 still uses its own), then A's in the order step 0 retires its
    // blocks.
    auto read_ba = [&](int stage, int ks, half8 (&af)[FM], half8 (&bf)[FN]) {
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = fb.read(s8[stage], j, ks, 0);
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = fa.read(s8[stage], i, ks, 0);
    };
    // The next slab's step-0 fragments, in the order its MFMAs consume them (A
    // block 0 with every B block first).
    auto read_ab = [&](int stage, int ks, half8 (&af)[FM], half8 (&bf)[FN]) {
        af[0] = fa.read(s8[stage], 0, ks, 0);
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = fb.read(s8[stage], j, ks, 0);
#pragma unroll
        for (int i = 1; i < FM; ++i) af[i] = fa.read(s8[stage], i, ks, 0);
    };
    // block (i, j) = (t / FN, t % FN): B's fragment first, so lane l of block
    // (i, j) accumulates output row 16 i + (l & 15), columns 16 j + 4 (l >> 4) .. + 3
    auto mfma = [&](const half8 (&af)[FM], const half8 (&bf)[FN], int from, int to) {
#pragma unroll
        for (int t = from; t < to; ++t)
            acc[t / FN][t % FN] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[t % FN], af[t / FN], acc[t / FN][t % FN], 0, 0, 0);
    };
    // vmcnt(0), expcnt and lgkmcnt left at their maxima: this wave's loads into LDS have landed
    auto wait_loads = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };

    half8 af[2][FM], bf[2][FN];
    // The whole loop, for loading (LD) and computing waves. Only a loading wave
    // builds its loaders, so a computing wave holds none of their registers.
    auto run = [&](auto ld_tag) {
        constexpr bool LD = decltype(ld_tag)::value;
        LA la;
        LB lb;
        if constexpr (LD) {
            la.init(A_KC ? g.A + row0 * g.lda : g.A + row0, g.lda, wave % kLoadWaves, lane);
            lb.init(B_KC ? g.B + col0 * g.ldb : g.B + col0, g.ldb, wave % kLoadWaves, lane);
        }
        auto fetch = [&](int kt, int stage) {
            la.fetch(s8[stage], uint32_t(kt) * a_step);
            lb.fetch(s8[stage] + kAStage, uint32_t(kt) * b_step);
        };
        // Prologue: slab 0 in stage 0, and its step-0 fragments.
        if constexpr (LD) fetch(0, 0);
        wait_loads();
        __syncthreads();
        read_ab(0, 0, af[0], bf[0]);

        // One slab in stage S; a loading wave loads its share of the next slab
        // (or, after the last, a copy of it) into the other stage. At the slab's
        // one barrier the next slab has landed in the other stage and every read
        // of stage S is done (all of step 1's fragments were read before it).
        auto slab = [&](int kt, auto s_tag) {
            constexpr int S = decltype(s_tag)::value;
            if constexpr (LD) fetch(kt + 1 < nk ? kt + 1 : kt, S ^ 1);
            read_ba(S, 1, af[1], bf[1]);
            mfma(af[0], bf[0], 0, kMfma);
            mfma(af[1], bf[1], 0, kPre);
            // Instruction order (groups are filled in program order): step 0's
            // MFMAs, each followed by its even share of step 1's fragment reads
            // and, in a loading wave, every other one by a load of the next slab;
            // then step 1's first kPre MFMAs.
#pragma unroll
            for (int m = 0; m < kMfma; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (LD && !(m & 1) && m / 2 < kLoads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                const int nr = (m + 1) * kReads / kMfma - m * kReads / kMfma;
#pragma unroll
                for (int r = 0; r < nr; ++r) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int m = 0; m < kPre; ++m) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            // The barrier stays exactly here: the scheduler would otherwise move
            // MFMAs across it.
            __builtin_amdgcn_sched_barrier(0);
            wait_loads();
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            read_ab(S ^ 1, 0, af[0], bf[0]);
            mfma(af[1], bf[1], kPre, kMfma);
#pragma unroll
            for (int m = 0; m < kMfma - kPre; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                const int nr = (m + 1) * kReads / (kMfma - kPre) - m * kReads / (kMfma - kPre);
#pragma unroll
                for (int r = 0; r < nr; ++r) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        };
        using C0 = std::integral_constant<int, 0>;
        using C1 = std::integral_constant<int, 1>;
        // nk is even here. One loop body for every slab: after the last slab the
        // "next" load re-reads that slab into the idle stage (1/nk extra loads),
        // which keeps the loop free of tail copies. Every wave passes one barrier
        // per slab.
        if constexpr (LD) __builtin_amdgcn_s_setprio(2);
        for (int kt = 0; kt < nk; kt += 2) {
            slab(kt, C0());
            slab(kt + 1, C1());
        }
        if constexpr (LD) __builtin_amdgcn_s_setprio(0);
    };
    if (loader)
        run(std::integral_constant<bool, true>());
    else
        run(std::integral_constant<bool, false>());
    // The last slab read its (unused) successor's first fragments from the
    // idle stage; the epilogue stages the output through both stages.
    __syncthreads();
}

// Applies the binary16 point-wise tail of the epilogue to one output element
// h = RNE16(acc) and stores it (z: the saved pre-activation for kEpiDact, the
// saved derivative for kEpiMul).
template <int EPI, int KIND>
__device__ __forceinline__ uint16_t epi_main(uint16_t h, uint16_t z) {
    if (EPI == kEpiDact) return mp::act_bwd1<KIND>(z, h);
    if (EPI == kEpiMul) return mp::f2h(mp::h2f(h) * mp::h2f(z));
    return h;
}
__device__ __forceinline__ uint16_t half_of(const uint4& v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return uint16_t(w >> (16 * (e & 1)));
}
__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) { return uint32_t(lo) | uint32_t(hi) << 16; }

// KIND (the activation of kEpiAct / kEpiDact, an mp_act value) is ignored by the other modes.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool A_KC, bool B_KC, int EPI, int KIND>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_kernel(GemmArgs g) {
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 16, FN = WTN / 16;            // 16 x 16 MFMA blocks per wave
    constexpr int kStage = (BM + BN) * kRowChunks;         // uint4 per LDS stage
    // the two stages of the reduction loop, as two variables (see reduce_tile_pipe)
    __shared__ uint4 lds0[kStage];
    __shared__ uint4 lds1[kStage];
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles must be whole pairs of MFMA blocks");

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

    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

    const bool full = g.a_vec && g.b_vec && (g.R % kBK) == 0 && row0 + BM <= g.Mc &&
                      col0 + BN <= g.Nc;
    bool done = false;
    if constexpr (BM == 256 && BN == 256) {
        if (full && g.pipe_ok) {
            reduce_tile_pipe<BM, BN, WAVES_M, WAVES_N, A_KC, B_KC, FM, FN>(g, lds0, lds1, row0, col0, lane, wm, wn, acc);
            done = true;
        }
    }
    if (done) {
    } else if (full)
        reduce_tile<BM, BN, WAVES_M, WAVES_N, A_KC, B_KC, true, FM, FN>(g, lds0, lds1, row0, col0, tid, lane,
                                                                      wm, wn, acc);
    else
        reduce_tile<BM, BN, WAVES_M, WAVES_N, A_KC, B_KC, false, FM, FN>(g, lds0, lds1, row0, col0, tid, lane,
                                                                       wm, wn, acc);

    // ---- epilogue. The MFMA takes B's fragment as its first operand, so the
    // accumulator of block (i, j) holds the transposed tile: lane l has output
    // row m = 16 i + (l & 15) and, in register r, column n = 16 j + 4 (l / 16) + r
    // (wave-local), i.e. four consecutive columns of one row.
    const int64_t wrow0 = row0 + wm * WTM, wcol0 = col0 + wn * WTN;
    if (EPI == kEpiF32) {
        float* C = static_cast<float*>(g.C);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int64_t gr = wrow0 + i * 16 + (lane & 15);
                const int64_t gc = wcol0 + j * 16 + 4 * (lane >> 4);
                if (gr >= g.Mc) continue;
                float* dst = C + gr * g.ldc + gc;
                if (g.c_vec && gc + 4 <= g.Nc) {
                    *reinterpret_cast<mp::f32x4*>(dst) = mp::f32x4{acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (gc + e < g.Nc) dst[e] = acc[i][j][e];
                }
            }
        return;
    }
    // Binary16 out, staged through LDS (free once the reduction has ended): each
    // wave rounds its WTM x WTN tile, writes it row-major into its own LDS region
    // with 8-byte stores (16-byte chunk c of row m at chunk c ^ (m mod chunks)),
    // then reads it back a 16-byte row piece per lane and stores whole rows.
    constexpr int kChunks = WTN / 8;                     // 16-byte chunks per staged row
    constexpr int kRowsPerPass = 64 / kChunks;
    static_assert(WTM % kRowsPerPass == 0, "whole passes");
    uint32_t bad = 0;
    constexpr int kWaveBytes = WTM * WTN * 2, kFit0 = kStage * 16 / kWaveBytes;
    static_assert(WAVES_M * WAVES_N <= 2 * kFit0, "each wave's staged tile lies within one stage");
    uint8_t* stage = wave < kFit0 ? reinterpret_cast<uint8_t*>(lds0) + size_t(wave) * kWaveBytes
                                  : reinterpret_cast<uint8_t*>(lds1) + size_t(wave - kFit0) * kWaveBytes;
    uint16_t* C = static_cast<uint16_t*>(g.C);
    // Whole wave tiles with 16-byte access everywhere take an unchecked path.
    const bool whole = g.c_vec && (EPI == kEpiF16 || g.aux_vec) && wrow0 + WTM <= g.Mc &&
                       wcol0 + WTN <= g.Nc;
    // Read-back passes in groups; the dgrad epilogue's saved pre-activation
    // values for a group are loaded one group ahead, the first group before the
    // staging writes, so their latency overlaps other work.
    constexpr int kPasses = WTM / kRowsPerPass;
    constexpr int kGrp = kPasses < 4 ? kPasses : 4;
    static_assert(kPasses % kGrp == 0, "whole groups");
    auto piece_row = [&](int p) { return p * kRowsPerPass + lane / kChunks; };
    auto piece_chunk = [&]() { return lane % kChunks; };
    uint4 za[kGrp], zb[kGrp];
    auto zload = [&](uint4 (&z)[kGrp], int p0) {
#pragma unroll
        for (int q = 0; q < kGrp; ++q)
            z[q] = *reinterpret_cast<const uint4*>(g.Z + (wrow0 + piece_row(p0 + q)) * g.ldz + wcol0 +
                                                   8 * piece_chunk());
    };
    constexpr bool kLoadZ = EPI == kEpiDact || EPI == kEpiMul;
    if (kLoadZ && whole) zload(za, 0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int m = i * 16 + (lane & 15);
            const int c = 2 * j + (lane >> 5);             // chunk of the 8 columns 16 j + 8 (l / 32) ..
            const uint2 v = make_uint2(mp::f2h2(acc[i][j][0], acc[i][j][1]), mp::f2h2(acc[i][j][2], acc[i][j][3]));
            *reinterpret_cast<uint2*>(stage + (m * kChunks + (c ^ (m & (kChunks - 1)))) * 16 + 8 * ((lane >> 4) & 1)) = v;
        }
    __syncthreads();
    auto staged = [&](int m, int c) {
        return *reinterpret_cast<const uint4*>(stage + (m * kChunks + (c ^ (m & (kChunks - 1)))) * 16);
    };
    if (whole) {
        auto group = [&](const uint4 (&z)[kGrp], int p0) {
#pragma unroll
            for (int q = 0; q < kGrp; ++q) {
                const int m = piece_row(p0 + q), c = piece_chunk();
                const uint4 v = staged(m, c);
                const int64_t gr = wrow0 + m, gc = wcol0 + 8 * c;
                uint16_t* dst = C + gr * g.ldc + gc;
                if (EPI == kEpiF16) {
                    *reinterpret_cast<uint4*>(dst) = v;
                    bad |= mp::nonfinite2(v.x) | mp::nonfinite2(v.y) | mp::nonfinite2(v.z) | mp::nonfinite2(v.w);
                } else if (EPI == kEpiAct) {
                    *reinterpret_cast<uint4*>(dst) = v;
                    uint16_t a[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = mp::act_fwd1<KIND>(half_of(v, e));
                    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(g.C2) + gr * g.ldc2 + gc) =
                        make_uint4(pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(a[4], a[5]), pack2(a[6], a[7]));
                } else if (EPI == kEpiActD) {
                    uint32_t a[4], d[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        mp::act_fwd_deriv2<KIND>(half_of(v, 2 * e), half_of(v, 2 * e + 1), a[e], d[e]);
                    *reinterpret_cast<uint4*>(dst) = make_uint4(a[0], a[1], a[2], a[3]);
                    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(g.C2) + gr * g.ldc2 + gc) =
                        make_uint4(d[0], d[1], d[2], d[3]);
                } else {
                    uint16_t d[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) d[e] = epi_main<EPI, KIND>(half_of(v, e), half_of(z[q], e));
                    *reinterpret_cast<uint4*>(dst) =
                        make_uint4(pack2(d[0], d[1]), pack2(d[2], d[3]), pack2(d[4], d[5]), pack2(d[6], d[7]));
                }
            }
        };
#pragma unroll 1
        for (int p0 = 0; p0 < kPasses; p0 += 2 * kGrp) {
            if (kLoadZ && p0 + kGrp < kPasses) zload(zb, p0 + kGrp);
            group(za, p0);
            if (p0 + kGrp < kPasses) {
                if (kLoadZ && p0 + 2 * kGrp < kPasses) zload(za, p0 + 2 * kGrp);
                group(zb, p0 + kGrp);
            }
        }
    } else {
#pragma unroll 1
        for (int p = 0; p < kPasses; ++p) {
            const int m = piece_row(p), c = piece_chunk();
            const uint4 v = staged(m, c);
            const int64_t gr = wrow0 + m, gc = wcol0 + 8 * c;
            if (gr >= g.Mc) continue;
            uint16_t* dst = C + gr * g.ldc + gc;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (gc + e < g.Nc) {
                    const uint16_t h = half_of(v, e);
                    if (EPI == kEpiF16) {
                        dst[e] = h;
                        bad |= mp::nonfinite1(h);
                    } else if (EPI == kEpiAct) {
                        dst[e] = h;
                        static_cast<uint16_t*>(g.C2)[gr * g.ldc2 + gc + e] = mp::act_fwd1<KIND>(h);
                    } else if (EPI == kEpiActD) {
                        uint16_t a, d;
                        mp::act_fwd_deriv1<KIND>(h, a, d);
                        dst[e] = a;
                        static_cast<uint16_t*>(g.C2)[gr * g.ldc2 + gc + e] = d;
                    } else {
                        dst[e] = epi_main<EPI, KIND>(h, g.Z[gr * g.ldz + gc + e]);
                    }
                }
        }
    }
    if (EPI == kEpiF16 && g.flag) {
        if (__syncthreads_or(bad) && tid == 0) atomicOr(g.flag, 1u);
    }
}

template <int BM, int BN, int WM, int WN, bool A_KC, bool B_KC, int EPI, int KIND>
mp_status launch_cfg(GemmArgs a, hipStream_t s, const char* name) {
    a.tiles_m = int((a.Mc + BM - 1) / BM);
    a.tiles_n = int((a.Nc + BN - 1) / BN);
    // buffer-load offsets within an operand's panel must stay below 2^32 bytes
    const auto panel_ok = [&](bool kc, int64_t ld) {
        const int64_t bytes = kc ? (int64_t(BM > BN ? BM : BN) * ld + a.R) * 2 : (a.R + 64) * ld * 2 + 512;
        return bytes < (int64_t(1) << 32);
    };
    // The buffer-load loop fetches slab 0 before it looks at the reduction length: it needs a
    // non-empty reduction (an empty one takes the general loop, which writes zeros).
    a.pipe_ok = int(a.R > 0 && a.R % (2 * kBK) == 0 && panel_ok(A_KC, a.lda) && panel_ok(B_KC, a.ldb));
    const uint32_t blocks = uint32_t(a.tiles_m) * uint32_t(a.tiles_n);
    gemm_kernel<BM, BN, WM, WN, A_KC, B_KC, EPI, KIND><<<blocks, 64 * WM * WN, 0, s>>>(a);
    return mp::launch_status(name);
}

template <bool A_KC, bool B_KC, int EPI, int KIND = 0>
mp_status launch(GemmArgs a, hipStream_t s, const char* name) {
    // Large outputs: 256 x 256 tiles of 8 waves of 128 x 64, two per SIMD,
    // split into loading and computing waves (reduce_tile_pipe). Small outputs
    // (where a 256 x 256 grid would leave most of the 256 CUs idle): 64 x 64.
    const int64_t big_tiles = ((a.Mc + 255) / 256) * ((a.Nc + 255) / 256);
    if (big_tiles >= 128) return launch_cfg<256, 256, 2, 4, A_KC, B_KC, EPI, KIND>(a, s, name);
    return launch_cfg<64, 64, 2, 2, A_KC, B_KC, EPI, KIND>(a, s, name);
}

bool bad_matrix(const void* p, int64_t rows, int64_t cols, int64_t ld) {
    if (rows < 0 || cols < 0) return true;
    if (rows > 0 && cols > 0 && (!p || ld < cols)) return true;
    return false;
}

// 16-byte loads need a 16-byte aligned base and a row pitch of 8 elements.
int vec_ok(const void* p, int64_t ld) { return mp::aligned16(p) && (ld % 8) == 0; }
// 16-byte output stores: 8 binary16 or 4 FP32 values per row piece.
int out_vec_ok(const void* p, int64_t ld, mp_dtype t) {
    return mp::aligned16(p) && (ld % (t == MP_F16 ? 8 : 4)) == 0;
}

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
    GemmArgs a{X, W, Y, ldx, ldw, ldy, M, N, K, nullptr, vec_ok(X, ldx), vec_ok(W, ldw),
               out_vec_ok(Y, ldy, y_dtype)};
    hipStream_t s = mp::as_stream(stream);
    if (y_dtype == MP_F16) return launch<true, true, kEpiF16>(a, s, "mp_linear_fwd");
    return launch<true, true, kEpiF32>(a, s, "mp_linear_fwd");
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
    GemmArgs a{dY, W, dX, lddy, ldw, lddx, M, K, N, nullptr, vec_ok(dY, lddy), vec_ok(W, ldw),
               out_vec_ok(dX, lddx, dx_dtype)};
    hipStream_t s = mp::as_stream(stream);
    if (dx_dtype == MP_F16) return launch<true, false, kEpiF16>(a, s, "mp_linear_dgrad");
    return launch<true, false, kEpiF32>(a, s, "mp_linear_dgrad");
}

extern "C" mp_status mp_linear_wgrad(const uint16_t* dY, int64_t lddy, const uint16_t* X,
                                     int64_t ldx, void* dW, int64_t lddw, mp_dtype dw_dtype,
                                     int64_t M, int64_t N, int64_t K, uint32_t* found_inf,
                                     mp_stream stream) {
    if (M < 0 || N < 0 || K < 0) return MP_ERR_INVALID_ARGUMENT;
    if (dw_dtype != MP_F16 && dw_dtype != MP_F32) return MP_ERR_INVALID_ARGUMENT;
    if (dw_dtype == MP_F32 && found_inf) return MP_ERR_INVALID_ARGUMENT;
    if (found_inf && mp::misaligned4(found_inf)) return MP_ERR_INVALID_ARGUMENT;
    if (N == 0 || K == 0) return MP_OK;
    if (bad_matrix(dY, M, N, lddy) || bad_matrix(X, M, K, ldx) || bad_matrix(dW, N, K, lddw))
        return MP_ERR_INVALID_ARGUMENT;
    if (too_large(N, K)) return MP_ERR_INVALID_ARGUMENT;
    GemmArgs a{dY, X, dW, lddy, ldx, lddw, N, K, M, found_inf, vec_ok(dY, lddy), vec_ok(X, ldx),
               out_vec_ok(dW, lddw, dw_dtype)};
    hipStream_t s = mp::as_stream(stream);
    if (dw_dtype == MP_F16) return launch<false, false, kEpiF16>(a, s, "mp_linear_wgrad");
    return launch<false, false, kEpiF32>(a, s, "mp_linear_wgrad");
}

extern "C" mp_status mp_linear_fwd_act(mp_act kind, const uint16_t* X, int64_t ldx, const uint16_t* W,
                                       int64_t ldw, uint16_t* Z, int64_t ldz, uint16_t* H, int64_t ldh,
                                       int64_t M, int64_t N, int64_t K, mp_stream stream) {
    if (kind != MP_ACT_RELU && kind != MP_ACT_GELU) return MP_ERR_INVALID_ARGUMENT;
    if (M < 0 || N < 0 || K < 0) return MP_ERR_INVALID_ARGUMENT;
    if (M == 0 || N == 0) return MP_OK;
    if (bad_matrix(X, M, K, ldx) || bad_matrix(W, N, K, ldw) || bad_matrix(Z, M, N, ldz) ||
        bad_matrix(H, M, N, ldh))
        return MP_ERR_INVALID_ARGUMENT;
    if (too_large(M, N)) return MP_ERR_INVALID_ARGUMENT;
    GemmArgs a{X, W, Z, ldx, ldw, ldz, M, N, K, nullptr, vec_ok(X, ldx), vec_ok(W, ldw),
               out_vec_ok(Z, ldz, MP_F16), H, nullptr, ldh, 0, out_vec_ok(H, ldh, MP_F16)};
    hipStream_t s = mp::as_stream(stream);
    if (kind == MP_ACT_RELU) return launch<true, true, kEpiAct, MP_ACT_RELU>(a, s, "mp_linear_fwd_act");
    return launch<true, true, kEpiAct, MP_ACT_GELU>(a, s, "mp_linear_fwd_act");
}

extern "C" mp_status mp_linear_dgrad_act(mp_act kind, const uint16_t* dY, int64_t lddy, const uint16_t* W,
                                         int64_t ldw, const uint16_t* Z, int64_t ldz, uint16_t* dZ,
                                         int64_t lddz, int64_t M, int64_t N, int64_t K, mp_stream stream) {
    if (kind != MP_ACT_RELU && kind != MP_ACT_GELU) return MP_ERR_INVALID_ARGUMENT;
    if (M < 0 || N < 0 || K < 0) return MP_ERR_INVALID_ARGUMENT;
    if (M == 0 || K == 0) return MP_OK;
    if (bad_matrix(dY, M, N, lddy) || bad_matrix(W, N, K, ldw) || bad_matrix(Z, M, K, ldz) ||
        bad_matrix(dZ, M, K, lddz))
        return MP_ERR_INVALID_ARGUMENT;
    if (too_large(M, K)) return MP_ERR_INVALID_ARGUMENT;
    GemmArgs a{dY, W, dZ, lddy, ldw, lddz, M, K, N, nullptr, vec_ok(dY, lddy), vec_ok(W, ldw),
               out_vec_ok(dZ, lddz, MP_F16), nullptr, Z, 0, ldz, vec_ok(Z, ldz)};
    hipStream_t s = mp::as_stream(stream);
    if (kind == MP_ACT_RELU) return launch<true, false, kEpiDact, MP_ACT_RELU>(a, s, "mp_linear_dgrad_act");
    return launch<true, false, kEpiDact, MP_ACT_GELU>(a, s, "mp_linear_dgrad_act");
}

extern "C" mp_status mp_linear_fwd_act_deriv(mp_act kind, const uint16_t* X, int64_t ldx, const uint16_t* W,
                                             int64_t ldw, uint16_t* H, int64_t ldh, uint16_t* D, int64_t ldd,
                                             int64_t M, int64_t N, int64_t K, mp_stream stream) {
    if (kind != MP_ACT_RELU && kind != MP_ACT_GELU) return MP_ERR_INVALID_ARGUMENT;
    if (M < 0 || N < 0 || K < 0) return MP_ERR_INVALID_ARGUMENT;
    if (M == 0 || N == 0) return MP_OK;
    if (bad_matrix(X, M, K, ldx) || bad_matrix(W, N, K, ldw) || bad_matrix(H, M, N, ldh) ||
        bad_matrix(D, M, N, ldd))
        return MP_ERR_INVALID_ARGUMENT;
    if (too_large(M, N)) return MP_ERR_INVALID_ARGUMENT;
    GemmArgs a{X, W, H, ldx, ldw, ldh, M, N, K, nullptr, vec_ok(X, ldx), vec_ok(W, ldw),
               out_vec_ok(H, ldh, MP_F16), D, nullptr, ldd, 0, out_vec_ok(D, ldd, MP_F16)};
    hipStream_t s = mp::as_stream(stream);
    if (kind == MP_ACT_RELU) return launch<true, true, kEpiActD, MP_ACT_RELU>(a, s, "mp_linear_fwd_act_deriv");
    return launch<true, true, kEpiActD, MP_ACT_GELU>(a, s, "mp_linear_fwd_act_deriv");
}

extern "C" mp_status mp_linear_dgrad_mul(const uint16_t* dY, int64_t lddy, const uint16_t* W, int64_t ldw,
                                         const uint16_t* D, int64_t ldd, uint16_t* dZ, int64_t lddz, int64_t M,
                                         int64_t N, int64_t K, mp_stream stream) {
    if (M < 0 || N < 0 || K < 0) return MP_ERR_INVALID_ARGUMENT;
    if (M == 0 || K == 0) return MP_OK;
    if (bad_matrix(dY, M, N, lddy) || bad_matrix(W, N, K, ldw) || bad_matrix(D, M, K, ldd) ||
        bad_matrix(dZ, M, K, lddz))
        return MP_ERR_INVALID_ARGUMENT;
    if (too_large(M, K)) return MP_ERR_INVALID_ARGUMENT;
    GemmArgs a{dY, W, dZ, lddy, ldw, lddz, M, K, N, nullptr, vec_ok(dY, lddy), vec_ok(W, ldw),
               out_vec_ok(dZ, lddz, MP_F16), nullptr, D, 0, ldd, vec_ok(D, ldd)};
    return launch<true, false, kEpiMul>(a, mp::as_stream(stream), "mp_linear_dgrad_mul");
}
