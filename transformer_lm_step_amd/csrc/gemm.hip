// Matrix products of the GPT-2 step on MFMA (gfx950).
//
//   acc[m][n] = sum_k A(m, k) * B(n, k)            (fp32 accumulation)
//
// A is stored either k-contiguous (A[m*lda + k]) or m-contiguous (A[k*lda + m]); B likewise
// n- or k-contiguous. That covers the three products of a Linear layer y = x W^T + b
// ("Code you'll write": c_attn, c_proj, c_fc, lm_head):
//   forward   y  = x W^T        A = x  [M,K] k-contig,  B = W [N,K] k-contig
//   input     dx = dy W         A = dy [M,K] k-contig,  B = W [K,N] n-contig
//   weight    dW = dy^T x       A = dy [K,M] m-contig,  B = x [K,N] n-contig   (K = tokens)
// and the epilogues fuse what follows each product in the step: bias, GELU-tanh, residual
// add, GELU derivative, gradient scaling/accumulation, split-K partials.
//
// Tiling: a 256-thread workgroup (4 waves in 2 x 2) owns a BM x BN output tile, each wave a
// (BM/2) x (BN/2) sub-tile of 16x16 MFMA blocks. The block tile is 128x128, 256x128 or
// 256x256: the larger the wave tile, the fewer LDS bytes each MFMA needs (LDS bandwidth, not
// the matrix cores, bounds the small tile on CDNA4). K advances 128 bytes per step (64 bf16
// / 32 fp32) through a double-buffered LDS stage whose rows are padded by 16 bytes, which
// keeps the 16-byte fragment reads conflict-free. Operands that are not k-contiguous are
// transposed in registers (8x8 bf16 / 4x4 fp32 blocks) on their way into LDS; the k block
// varies fastest across lanes so 8 lanes write one whole 128-byte row. Workgroups are
// renumbered so that each of the 8 XCDs (one L2 each) works on a contiguous, M-grouped range
// of tiles.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gpt2k {

constexpr int GTHREADS = 256;
constexpr int ROWB = 128 + 16;  // LDS bytes per tile row (128 data + 16 pad)

struct GemmArgs {
    const void* A; const void* B;
    int64_t lda, ldb;
    int M, N, K;
    int ksplit_len;             // K elements per split (multiple of the tile K)
    void* C; int64_t ldc;       // main output (storage type or fp32, per epilogue)
    void* C2;                   // second output (GELU activation)
    const float* bias;
    const float* resid; int64_t ldr;
    const void* aux; int64_t ldaux;   // pre-activation u for the GELU derivative
    float alpha;
    int beta;                   // 1: add into the fp32 output
    int64_t part_stride;        // split-K partial stride (elements)
};

template <int BM, int BN>
constexpr size_t lds_bytes() { return 2 * (size_t)(BM + BN) * ROWB; }

#ifndef GEMM_TILE_ORDER
#define GEMM_TILE_ORDER 0
#endif
// workgroup id -> (tile_m, tile_n): XCD-contiguous ranges, then groups of GROUP_M tile rows
DEV void tile_coords(int pid, int nwg, int num_m, int num_n, int& tm, int& tn) {
    if (GEMM_TILE_ORDER == 1) { tm = pid % num_m; tn = pid / num_m; return; }
    const int xcd = pid & 7, slot = pid >> 3;
    const int per = (nwg + 7) >> 3;
    int tall = nwg & 7;
    if (tall == 0) tall = 8;
    int logical = (xcd < tall) ? xcd * per + slot : tall * per + (xcd - tall) * (per - 1) + slot;
    const int GROUP_M = 8;
    const int in_group = GROUP_M * num_n;
    const int gid = logical / in_group;
    const int first_m = gid * GROUP_M;
    int gsz = num_m - first_m;
    if (gsz > GROUP_M) gsz = GROUP_M;
    const int r = logical - gid * in_group;
    tm = first_m + r % gsz;
    tn = r / gsz;
}

// Loads a ROWS x (128 bytes of K) tile of one operand into registers, then stores it to LDS
// as [row][k] (row = m or n). LAYOUT 0: k-contiguous source (16-byte chunks along k).
// LAYOUT 1: row-contiguous source, read as E x E element blocks (E = 16/sizeof(T)) and
// transposed in registers. Rows past the matrix edge are clamped to the last row (valid
// memory; those outputs are never stored); a partial K tile zero-fills k >= kend.
template <typename T, int LAYOUT, int ROWS>
struct TileLoader {
    static constexpr int E = 16 / sizeof(T);
    static constexpr int BK = 128 / sizeof(T);
    static constexpr int NCHUNK = ROWS * 8 / GTHREADS;               // LAYOUT 0
    static constexpr int KB = BK / E;                                 // LAYOUT 1: k blocks
    static constexpr int NBLK_TOTAL = KB * (ROWS / E);
    static constexpr int NB = (NBLK_TOTAL + GTHREADS - 1) / GTHREADS;
    uint4 r[LAYOUT == 0 ? NCHUNK : E * NB];

    template <bool MASK>
    DEV void load(const T* __restrict__ src, int64_t ld, int row0, int nrows, int k0, int kend, int tid) {
        if constexpr (LAYOUT == 0) {
#pragma unroll
            for (int i = 0; i < NCHUNK; ++i) {
                const int c = tid + i * GTHREADS;
                int gr = row0 + (c >> 3);
                if (gr >= nrows) gr = nrows - 1;
                const int gk = k0 + (c & 7) * E;
                if (!MASK || gk < kend)
                    r[i] = ld16(src + (int64_t)gr * ld + gk);
                else
                    r[i] = make_uint4(0, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int blk = tid + b * GTHREADS;
                const int kb = blk % KB, mb = blk / KB;
                int gm = row0 + mb * E;
                if (gm > nrows - E) gm = nrows - E;
#pragma unroll
                for (int q = 0; q < E; ++q) {
                    const int gk = k0 + kb * E + q;
                    if ((NBLK_TOTAL % GTHREADS == 0 || blk < NBLK_TOTAL) && (!MASK || gk < kend))
                        r[b * E + q] = ld16(src + (int64_t)gk * ld + gm);
                    else
                        r[b * E + q] = make_uint4(0, 0, 0, 0);
                }
            }
        }
    }
    DEV void store(char* lds, int tid) {
        if constexpr (LAYOUT == 0) {
#pragma unroll
            for (int i = 0; i < NCHUNK; ++i) {
                const int c = tid + i * GTHREADS;
                st16(lds + (c >> 3) * ROWB + (c & 7) * 16, r[i]);
            }
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int blk = tid + b * GTHREADS;
                if (NBLK_TOTAL % GTHREADS != 0 && blk >= NBLK_TOTAL) continue;
                const int kb = blk % KB, mb = blk / KB;
                uint4 in[8], out[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) in[q] = q < E ? r[b * E + q] : make_uint4(0, 0, 0, 0);
                transpose_block(in, out, (T*)nullptr);
#pragma unroll
                for (int j = 0; j < E; ++j) st16(lds + (mb * E + j) * ROWB + kb * 16, out[j]);
            }
        }
    }
};

template <typename T>
DEV typename FragT<T>::type load_frag(const char* lds, int row, int kstep, int lane) {
    // 8 consecutive k values of `row`; lane group (lane>>4) owns a k sub-range of the
    // 32-element k step
    const int off = row * ROWB + (kstep * 32 + (lane >> 4) * 8) * (int)sizeof(T);
    if constexpr (sizeof(T) == 2) {
        return __builtin_bit_cast(bf16x8, ld16(lds + off));
    } else {
        const float4 lo = *(const float4*)(lds + off);
        const float4 hi = *(const float4*)(lds + off + 16);
        return frag_from_halves(lo, hi);
    }
}

template <typename T, int ALAY, int BLAY, int EPI, int BM, int BN>
__global__ void __launch_bounds__(GTHREADS, (BM * BN > 128 * 128) ? 1 : 2) gemm_kernel(GemmArgs p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    constexpr int BK = 128 / sizeof(T);
    constexpr int KSTEPS = BK / 32;
    constexpr int TM = BM / 2, TN = BN / 2;     // wave tile
    constexpr int FM = TM / 16, FN = TN / 16;   // MFMA blocks per wave
    char* sA = smem;                            // [2][BM][ROWB]
    char* sB = smem + 2 * BM * ROWB;            // [2][BN][ROWB]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int num_m = (p.M + BM - 1) / BM, num_n = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, num_m, num_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = blockIdx.y * p.ksplit_len;
    int kend = kbeg + p.ksplit_len;
    if (kend > p.K) kend = p.K;
    const int ntiles = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

    const T* A = (const T*)p.A;
    const T* B = (const T*)p.B;
    TileLoader<T, ALAY, BM> la;
    TileLoader<T, BLAY, BN> lb;
    auto fetch = [&](int k0) {
        if (k0 + BK <= kend) {
            la.template load<false>(A, p.lda, m0, p.M, k0, kend, tid);
            lb.template load<false>(B, p.ldb, n0, p.N, k0, kend, tid);
        } else {
            la.template load<true>(A, p.lda, m0, p.M, k0, kend, tid);
            lb.template load<true>(B, p.ldb, n0, p.N, k0, kend, tid);
        }
    };

    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    if (ntiles > 0) {
        fetch(kbeg);
        la.store(sA, tid);
        lb.store(sB, tid);
    }
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < ntiles;
        if (more) fetch(kbeg + (kt + 1) * BK);
        const char* a_s = sA + cur * BM * ROWB;
        const char* b_s = sB + cur * BN * ROWB;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            typename FragT<T>::type af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = load_frag<T>(a_s, wm * TM + i * 16 + (lane & 15), ks, lane);
#pragma unroll
            for (int j = 0; j < FN; ++j) bfr[j] = load_frag<T>(b_s, wn * TN + j * 16 + (lane & 15), ks, lane);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) mma8(acc[i][j], af[i], bfr[j]);
        }
        if (more) {
            la.store(sA + (cur ^ 1) * BM * ROWB, tid);
            lb.store(sB + (cur ^ 1) * BN * ROWB, tid);
        }
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    // lane holds rows mb..mb+3 of column n for each (i, j) block
    const bool full = m0 + BM <= p.M && n0 + BN <= p.N;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * TN + j * 16 + (lane & 15);
        const bool nok = full || n < p.N;
        float bias = 0.f;
        if constexpr (EPI == EPI_BIAS_T || EPI == EPI_BIAS_RESID_F32 || EPI == EPI_BIAS_GELU)
            bias = (p.bias && nok) ? p.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int mb = m0 + wm * TM + i * 16 + (lane >> 4) * 4;
            float extra[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mb + r;
                const bool ok = full || (nok && m < p.M);
                extra[r] = 0.f;
                if constexpr (EPI == EPI_BIAS_RESID_F32) {
                    if (ok) extra[r] = p.resid[(int64_t)m * p.ldr + n];
                } else if constexpr (EPI == EPI_GELU_BWD) {
                    if (ok) extra[r] = to_f<T>(((const T*)p.aux)[(int64_t)m * p.ldaux + n]);
                } else if constexpr (EPI == EPI_F32) {
                    if (ok && p.beta) extra[r] = ((const float*)p.C)[(int64_t)m * p.ldc + n];
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mb + r;
                const bool ok = full || (nok && m < p.M);
                if (!ok) continue;
                const float v = acc[i][j][r];
                const int64_t o = (int64_t)m * p.ldc + n;
                if constexpr (EPI == EPI_BIAS_T) {
                    ((T*)p.C)[o] = from_f<T>(p.alpha * v + bias);
                } else if constexpr (EPI == EPI_BIAS_RESID_F32) {
                    ((float*)p.C)[o] = extra[r] + v + bias;
                } else if constexpr (EPI == EPI_BIAS_GELU) {
                    const T u = from_f<T>(v + bias);
                    ((T*)p.C)[o] = u;
                    ((T*)p.C2)[o] = from_f<T>(gelu_f(to_f<T>(u)));
                } else if constexpr (EPI == EPI_GELU_BWD) {
                    ((T*)p.C)[o] = from_f<T>(v * gelu_grad_f(extra[r]));
                } else if constexpr (EPI == EPI_F32) {
                    ((float*)p.C)[o] = extra[r] + p.alpha * v;
                } else {  // EPI_PARTIAL
                    ((float*)p.C)[(int64_t)blockIdx.y * p.part_stride + o] = v;
                }
            }
        }
    }
}

// ====================================================================== direct-load path
// bf16, A k-contiguous, K a multiple of 64. Tiles of k-contiguous operands go straight from
// global memory into LDS with global_load_lds_dwordx4 (lane i of a wave writes LDS bytes
// base + 16*i), so they cost no registers and no LDS-store instructions. The rows of such a
// tile are 128 bytes, unpadded; the 16-byte chunk c of row r sits in slot c ^ ((r >> 1) & 7),
// which keeps the 16-lane fragment reads free of bank conflicts. A transposed B operand
// (the input-gradient products) still goes through registers into a padded [n][k] tile.
// Two stages: the loads of tile kt+1 are issued right after the barrier that opens the
// multiplication of tile kt, and waited for before the next barrier; 68 KB of LDS per
// workgroup leaves room for two workgroups per CU.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

constexpr int DL_BK = 64;                       // bf16 elements per K step (128 bytes)
constexpr int DL_TILE = 128 * 128;              // bytes of a 128-row swizzled tile
constexpr int DL_TILE_PAD = 128 * ROWB;         // bytes of a 128-row padded tile

// s_waitcnt immediate waiting for vmcnt == 0 only (expcnt, lgkmcnt at their maxima)
constexpr int kWaitVm0 = (0x7 << 4) | (0xF << 8);

DEV int swz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// One direct load: this wave's 64 lanes each move 16 bytes from their global address to
// LDS address lds + 16 * lane. Written as inline asm (M0 and the load in one block, no
// register results): the compiler then does not make every later LDS read wait for it; the
// kernel orders the loads with explicit vmcnt waits and barriers instead. Loads the compiler
// does not know about only make its own vmcnt waits stricter (the counter drains in order).
DEV void dma16(const void* gaddr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(gaddr) : "memory");
}

// issue the direct loads of one 128-row x 64-k tile: 4 wave-instructions per wave, each
// covering 8 rows; lane l loads logical chunk (l & 7) ^ f(row) of row 8*(4w+i) + (l >> 3)
DEV void dl_issue(const bf16* __restrict__ tile, const int (&off)[4], char* lds, int wave) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)(lds + wave * 4096));
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(tile + off[i], base + i * 1024);
}
DEV void dl_offsets(int (&off)[4], int64_t ld, int row0, int nrows, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * (4 * wave + i) + (lane >> 3);
        int gr = row0 + r;
        if (gr >= nrows) gr = nrows - 1;   // clamped rows: valid memory, outputs discarded
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        off[i] = (int)((gr - row0) * ld) + c * 8;
    }
}

template <int BLAY, int EPI>
__global__ void __launch_bounds__(GTHREADS, 2) gemm_dl_kernel(GemmArgs p, const bf16* __restrict__ Ap,
                                                              const bf16* __restrict__ Bp) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    constexpr int BT = BLAY == 0 ? DL_TILE : DL_TILE_PAD;
    constexpr int STAGE = DL_TILE + BT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int num_m = (p.M + 127) / 128, num_n = (p.N + 127) / 128;
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, num_m, num_n, tm, tn);
    const int m0 = tm * 128, n0 = tn * 128;
    const int kbeg = blockIdx.y * p.ksplit_len;
    int kend = kbeg + p.ksplit_len;
    if (kend > p.K) kend = p.K;
    const int ntiles = kend > kbeg ? (kend - kbeg) / DL_BK : 0;

    const bf16* A = Ap + (int64_t)m0 * p.lda + kbeg;
    int offA[4];
    dl_offsets(offA, p.lda, m0, p.M, wave, lane);
    int offB[4];
    const bf16* Bd = Bp + (int64_t)n0 * p.ldb + kbeg;   // BLAY 0
    TileLoader<bf16, 1, 128> lb;                                        // BLAY 1
    if constexpr (BLAY == 0) dl_offsets(offB, p.ldb, n0, p.N, wave, lane);

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // issue the loads of tile kt into the stage at byte offset ST (compile-time, so the
    // compiler sees that a stage being filled is never the one being read)
    auto issue = [&](auto st_c, int kt) {
        constexpr int ST = decltype(st_c)::value;
        dl_issue(A + kt * DL_BK, offA, smem + ST, wave);
        if constexpr (BLAY == 0) dl_issue(Bd + kt * DL_BK, offB, smem + ST + DL_TILE, wave);
        else lb.template load<false>(Bp, p.ldb, n0, p.N, kbeg + kt * DL_BK, kend, tid);
    };
    // multiply the tile in stage CUR while the next tile (if any) loads into stage NXT
    auto step = [&](auto cur_c, auto nxt_c, int kt) {
        constexpr int CUR = decltype(cur_c)::value, NXT = decltype(nxt_c)::value;
        // tile kt is in LDS once this wave's loads have landed and every wave has passed
        // the barrier; a bare barrier keeps the compiler from draining later prefetches
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (kt + 1 < ntiles) issue(nxt_c, kt + 1);
        const char* a_s = smem + CUR;
        const char* b_s = smem + CUR + DL_TILE;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = __builtin_bit_cast(bf16x8, ld16(a_s + swz(wm * 64 + i * 16 + (lane & 15), ks * 4 + (lane >> 4))));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = wn * 64 + j * 16 + (lane & 15);
                if constexpr (BLAY == 0) bfr[j] = __builtin_bit_cast(bf16x8, ld16(b_s + swz(r, ks * 4 + (lane >> 4))));
                else bfr[j] = load_frag<bf16>(b_s, r, ks, lane);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) mma8(acc[i][j], af[i], bfr[j]);
        }
        if constexpr (BLAY == 1) {
            if (kt + 1 < ntiles) {
                // the transposed B tile of kt+1 goes through registers into the other stage,
                // which no wave reads before the next barrier
                __builtin_amdgcn_s_waitcnt(kWaitVm0);
                lb.store(smem + NXT + DL_TILE, tid);
            }
        }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, STAGE>;
    if (ntiles > 0) {
        issue(S0{}, 0);
        if constexpr (BLAY == 1) {
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
            lb.store(smem + DL_TILE, tid);
        }
    }
    for (int kt = 0; kt < ntiles; kt += 2) {
        step(S0{}, S1{}, kt);
        if (kt + 1 < ntiles) step(S1{}, S0{}, kt + 1);
    }

    // ---------------------------------------------------------------- epilogue
    const bool full = m0 + 128 <= p.M && n0 + 128 <= p.N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + j * 16 + (lane & 15);
        const bool nok = full || n < p.N;
        float bias = 0.f;
        if constexpr (EPI == EPI_BIAS_T || EPI == EPI_BIAS_RESID_F32 || EPI == EPI_BIAS_GELU)
            bias = (p.bias && nok) ? p.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int mb = m0 + wm * 64 + i * 16 + (lane >> 4) * 4;
            float extra[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mb + r;
                const bool ok = full || (nok && m < p.M);
                extra[r] = 0.f;
                if constexpr (EPI == EPI_BIAS_RESID_F32) {
                    if (ok) extra[r] = p.resid[(int64_t)m * p.ldr + n];
                } else if constexpr (EPI == EPI_GELU_BWD) {
                    if (ok) extra[r] = to_f<bf16>(((const bf16*)p.aux)[(int64_t)m * p.ldaux + n]);
                } else if constexpr (EPI == EPI_F32) {
                    if (ok && p.beta) extra[r] = ((const float*)p.C)[(int64_t)m * p.ldc + n];
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mb + r;
                const bool ok = full || (nok && m < p.M);
                if (!ok) continue;
                const float v = acc[i][j][r];
                const int64_t o = (int64_t)m * p.ldc + n;
                if constexpr (EPI == EPI_BIAS_T) {
                    ((bf16*)p.C)[o] = from_f<bf16>(p.alpha * v + bias);
                } else if constexpr (EPI == EPI_BIAS_RESID_F32) {
                    ((float*)p.C)[o] = extra[r] + v + bias;
                } else if constexpr (EPI == EPI_BIAS_GELU) {
                    const bf16 u = from_f<bf16>(v + bias);
                    ((bf16*)p.C)[o] = u;
                    ((bf16*)p.C2)[o] = from_f<bf16>(gelu_f(to_f<bf16>(u)));
                } else if constexpr (EPI == EPI_GELU_BWD) {
                    ((bf16*)p.C)[o] = from_f<bf16>(v * gelu_grad_f(extra[r]));
                } else if constexpr (EPI == EPI_F32) {
                    ((float*)p.C)[o] = extra[r] + p.alpha * v;
                } else {  // EPI_PARTIAL
                    ((float*)p.C)[(int64_t)blockIdx.y * p.part_stride + o] = v;
                }
            }
        }
    }
}

template <int BLAY>
constexpr size_t dl_lds_bytes() { return 2 * (size_t)(DL_TILE + (BLAY == 0 ? DL_TILE : DL_TILE_PAD)); }

template <int BLAY, int EPI>
static hipError_t launch_dl(const GemmArgs& a, int nsplit, hipStream_t s) {
    const int num_m = (a.M + 127) / 128, num_n = (a.N + 127) / 128;
    dim3 grid(num_m * num_n, nsplit);
    gemm_dl_kernel<BLAY, EPI><<<grid, dim3(GTHREADS), dl_lds_bytes<BLAY>(), s>>>(a, (const bf16*)a.A, (const bf16*)a.B);
    return hipGetLastError();
}

// out[m][n] = (beta ? out : 0) + alpha * sum_z part[z][m][n], z in order (deterministic)
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int nsplit, int64_t stride,
                                     float* __restrict__ out, int64_t n_elem, float alpha, int beta) {
    const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i4 >= n_elem) return;
    float4 s = *(const float4*)(part + i4);
    for (int z = 1; z < nsplit; ++z) {
        const float4 t = *(const float4*)(part + z * stride + i4);
        s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
    }
    float4 o;
    if (beta) {
        o = *(float4*)(out + i4);
        o.x += alpha * s.x; o.y += alpha * s.y; o.z += alpha * s.z; o.w += alpha * s.w;
    } else {
        o = make_float4(alpha * s.x, alpha * s.y, alpha * s.z, alpha * s.w);
    }
    *(float4*)(out + i4) = o;
}

size_t gemm_lds_bytes() { return lds_bytes<256, 256>(); }

// Tile choice. 256x128 and 256x256 tiles (one workgroup per CU) measured slower than
// 128x128 (two per CU) on every shape of the step, so 128x128 is the default; the larger
// tiles stay available through GemmDesc::bm/bn.
void gemm_pick_tile(int M, int N, int nsplit, int is_bf16, int* bm, int* bn) {
    const long cus = 256;
    auto tiles = [&](int tm, int tn) { return (long)((M + tm - 1) / tm) * ((N + tn - 1) / tn) * nsplit; };
    *bm = 128;
    *bn = 128;
    (void)tiles;
    (void)cus;
    (void)is_bf16;
}

template <typename T, int ALAY, int BLAY, int EPI, int BM, int BN>
static hipError_t launch(const GemmArgs& a, int nsplit, hipStream_t s) {
    const int num_m = (a.M + BM - 1) / BM, num_n = (a.N + BN - 1) / BN;
    dim3 grid(num_m * num_n, nsplit);
    gemm_kernel<T, ALAY, BLAY, EPI, BM, BN><<<grid, dim3(GTHREADS), lds_bytes<BM, BN>(), s>>>(a);
    return hipGetLastError();
}

template <typename T, int ALAY, int BLAY, int EPI>
static hipError_t launch_tiled(const GemmArgs& a, int nsplit, int bm, int bn, hipStream_t s) {
    if constexpr (sizeof(T) == 2) {
        if (bm == 256 && bn == 256) return launch<T, ALAY, BLAY, EPI, 256, 256>(a, nsplit, s);
        if (bm == 256 && bn == 128) return launch<T, ALAY, BLAY, EPI, 256, 128>(a, nsplit, s);
    }
    return launch<T, ALAY, BLAY, EPI, 128, 128>(a, nsplit, s);
}

template <typename T>
static hipError_t dispatch(const GemmDesc& d, hipStream_t s) {
    GemmArgs a{};
    a.A = d.A; a.B = d.B; a.lda = d.lda; a.ldb = d.ldb;
    a.M = d.M; a.N = d.N; a.K = d.K;
    a.C = d.C; a.ldc = d.ldc; a.C2 = d.C2; a.bias = d.bias; a.resid = d.resid; a.ldr = d.ldr;
    a.aux = d.aux; a.ldaux = d.ldaux; a.alpha = d.alpha; a.beta = d.beta;
    constexpr int BK = 128 / sizeof(T);
    int nsplit = d.nsplit < 1 ? 1 : d.nsplit;
    const int ktiles = (d.K + BK - 1) / BK;
    if (nsplit > ktiles) nsplit = ktiles;
    const int per = (ktiles + nsplit - 1) / nsplit;
    nsplit = (ktiles + per - 1) / per;
    a.ksplit_len = per * BK;
    int epi = d.epi;
    if (nsplit > 1) {
        // partials, then a fixed-order reduce into the fp32 output
        a.C = d.partial; a.ldc = d.N; a.part_stride = (int64_t)d.M * d.N;
        epi = EPI_PARTIAL;
    }
    int bm = d.bm, bn = d.bn;
    if (bm == 0) gemm_pick_tile(d.M, d.N, nsplit, sizeof(T) == 2, &bm, &bn);
    hipError_t e = hipSuccess;
    // direct-load path: bf16, A k-contiguous, every split a whole number of 64-wide K steps
    const bool dl = sizeof(T) == 2 && d.a_layout == 0 && bm == 128 && bn == 128 && d.K % DL_BK == 0 &&
                    a.ksplit_len % DL_BK == 0 && d.lda % 8 == 0 && (d.b_layout == 1 || d.ldb % 8 == 0) && !d.no_dl;
    if (dl) {
#define DL_CASE(BL, EP) if (d.b_layout == BL && epi == EP) e = launch_dl<BL, EP>(a, nsplit, s); else
        DL_CASE(0, EPI_BIAS_T)
        DL_CASE(0, EPI_BIAS_RESID_F32)
        DL_CASE(0, EPI_BIAS_GELU)
        DL_CASE(1, EPI_GELU_BWD)
        DL_CASE(1, EPI_F32)
        DL_CASE(1, EPI_BIAS_T)
        DL_CASE(1, EPI_PARTIAL)
        return hipErrorInvalidValue;
#undef DL_CASE
        goto reduce;
    }
#define GEMM_CASE(AL, BL, EP) \
    if (d.a_layout == AL && d.b_layout == BL && epi == EP) e = launch_tiled<T, AL, BL, EP>(a, nsplit, bm, bn, s); else
    GEMM_CASE(0, 0, EPI_BIAS_T)
    GEMM_CASE(0, 0, EPI_BIAS_RESID_F32)
    GEMM_CASE(0, 0, EPI_BIAS_GELU)
    GEMM_CASE(0, 1, EPI_GELU_BWD)
    GEMM_CASE(0, 1, EPI_F32)
    GEMM_CASE(0, 1, EPI_BIAS_T)
    GEMM_CASE(1, 1, EPI_F32)
    GEMM_CASE(1, 1, EPI_PARTIAL)
    GEMM_CASE(0, 1, EPI_PARTIAL)
    return hipErrorInvalidValue;
#undef GEMM_CASE
reduce:
    if (e != hipSuccess) return e;
    if (nsplit > 1) {
        if (d.epi != EPI_F32 || d.ldc != d.N) return hipErrorInvalidValue;
        const int64_t n = (int64_t)d.M * d.N;
        const int threads = 256;
        const int64_t blocks = (n / 4 + threads - 1) / threads;
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(threads), 0, s,
                           (const float*)d.partial, nsplit, (int64_t)d.M * d.N, (float*)d.C, n, d.alpha, d.beta);
        e = hipGetLastError();
    }
    return e;
}

hipError_t gemm(const GemmDesc& d, int is_bf16, hipStream_t s) {
    return is_bf16 ? dispatch<bf16>(d, s) : dispatch<float>(d, s);
}

template <typename T, int AL, int BL, int EP, int BM, int BN>
static void set_lds() {
    (void)hipFuncSetAttribute((const void*)gemm_kernel<T, AL, BL, EP, BM, BN>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes<BM, BN>());
}
template <typename T, int AL, int BL, int EP>
static void set_lds_all() {
    set_lds<T, AL, BL, EP, 128, 128>();
    if constexpr (sizeof(T) == 2) {
        set_lds<T, AL, BL, EP, 256, 128>();
        set_lds<T, AL, BL, EP, 256, 256>();
    }
}

template <int BL, int EP>
static void set_lds_dl() {
    (void)hipFuncSetAttribute((const void*)gemm_dl_kernel<BL, EP>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)dl_lds_bytes<BL>());
}

void gemm_setup() {
    set_lds_dl<0, EPI_BIAS_T>(); set_lds_dl<0, EPI_BIAS_RESID_F32>(); set_lds_dl<0, EPI_BIAS_GELU>();
    set_lds_dl<1, EPI_GELU_BWD>(); set_lds_dl<1, EPI_F32>(); set_lds_dl<1, EPI_BIAS_T>(); set_lds_dl<1, EPI_PARTIAL>();
    // allow the dynamic LDS size (above the 64 KiB default) for every instantiation
#define SETUP_T(T)                                                                                          \
    set_lds_all<T, 0, 0, EPI_BIAS_T>(); set_lds_all<T, 0, 0, EPI_BIAS_RESID_F32>();                        \
    set_lds_all<T, 0, 0, EPI_BIAS_GELU>(); set_lds_all<T, 0, 1, EPI_GELU_BWD>();                           \
    set_lds_all<T, 0, 1, EPI_F32>(); set_lds_all<T, 0, 1, EPI_BIAS_T>(); set_lds_all<T, 1, 1, EPI_F32>(); \
    set_lds_all<T, 1, 1, EPI_PARTIAL>(); set_lds_all<T, 0, 1, EPI_PARTIAL>();
    SETUP_T(bf16)
    SETUP_T(float)
#undef SETUP_T
}

}  // namespace gpt2k
