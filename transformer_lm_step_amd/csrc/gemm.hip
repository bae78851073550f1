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
// (BM/2) x (BN/2) sub-tile of 16x16 MFMA blocks. Two paths:
//  - LDS-streamed (bf16, whole 64-wide K tiles): both operands go from global memory straight
//    into LDS in their stored orientation; fragments of mn-contiguous operands are read with
//    the transposing LDS read of CDNA4. 128x128 or 128x192 tiles, two workgroups per CU.
//  - register-staged (fp32 check mode, ragged bf16 shapes): tiles pass through registers
//    into a padded LDS stage; operands that are not k-contiguous are transposed in registers.
// Workgroups are renumbered so that each of the 8 XCDs (one L2 each) works on a contiguous,
// M-grouped range of tiles.
#include <type_traits>

#include <hip/hip_ext.h>

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
    const void* aux; int64_t ldaux;   // pre-activation u for the GELU derivative
    float alpha;
    int beta;                   // 1: add into the fp32 output
    int64_t part_stride;        // split-K partial stride (elements)
    float* rowsum_part;         // [nsplit][M] row sums of A (a_layout 1), or null
    float* rowsum_out;          // with one split: the row sums of A written (beta: added) here directly
    int vec;                    // 1: full tiles may use 8/16-byte epilogue accesses
    int vec8;                   // 1: also 8-element (16-byte bf16) epilogue accesses
    const int32_t* c_row_dev;   // few-row products: output row offset from device memory, or null
    int64_t c_row_bytes;
    int c_row_max;
};

template <int BM, int BN>
constexpr size_t lds_bytes() { return 2 * (size_t)(BM + BN) * ROWB; }

#ifndef GEMM_TILE_ORDER
#define GEMM_TILE_ORDER 0
#endif
// Workgroups are dealt to the 8 XCDs round-robin by id (id & 7), the (id >> 3)-th on its XCD.
// This renumbering gives each XCD a contiguous range of logical tile numbers.
DEV int xcd_logical(int pid, int nwg) {
    const int xcd = pid & 7, slot = pid >> 3;
    const int per = (nwg + 7) >> 3;
    int tall = nwg & 7;
    if (tall == 0) tall = 8;
    return (xcd < tall) ? xcd * per + slot : tall * per + (xcd - tall) * (per - 1) + slot;
}
// workgroup id -> (tile_m, tile_n): XCD-contiguous ranges (unless the caller already numbered
// the tiles that way: remap = false), then groups of GROUP_M tile rows
DEV void tile_coords(int pid, int nwg, int num_m, int num_n, int& tm, int& tn, bool remap = true) {
    if (GEMM_TILE_ORDER == 1) { tm = pid % num_m; tn = pid / num_m; return; }
    const int logical = remap ? xcd_logical(pid, nwg) : pid;
    if (num_n <= 8) {
        // few column tiles: the tiles of one row panel are consecutive, so the blocks that share
        // an A panel start (and stream its K tiles) together
        tm = logical / num_n;
        tn = logical - tm * num_n;
        return;
    }
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

// ---------------------------------------------------------------- epilogue
// acc[i][j] holds, in lane l, rows mw + 16i + 4*(l>>4) + r (r = 0..3) of column
// nw + 16j + (l & 15). CHECK = false for tiles wholly inside the matrix: straight-line code.
template <typename T, int EPI, int FM, int FN, bool CHECK>
DEV void store_body(const GemmArgs& p, const floatx4 (&acc)[FM][FN], int mw, int nw, int lane) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = nw + j * 16 + (lane & 15);
        const bool nok = !CHECK || n < p.N;
        float bias = 0.f;
        if constexpr (EPI == EPI_BIAS_T || EPI == EPI_BIAS_GELU)
            bias = (p.bias && nok) ? p.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int mb = mw + i * 16 + (lane >> 4) * 4;
            float extra[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mb + r;
                const bool ok = !CHECK || (nok && m < p.M);
                extra[r] = 0.f;
                if constexpr (EPI == EPI_GELU_BWD) {
                    if (ok) extra[r] = to_f<T>(((const T*)p.aux)[(int64_t)m * p.ldaux + n]);
                } else if constexpr (EPI == EPI_F32) {
                    if (ok && p.beta) extra[r] = ((const float*)p.C)[(int64_t)m * p.ldc + n];
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mb + r;
                if (CHECK && !(nok && m < p.M)) continue;
                const float v = acc[i][j][r];
                const int64_t o = (int64_t)m * p.ldc + n;
                if constexpr (EPI == EPI_BIAS_T) {
                    ((T*)p.C)[o] = from_f<T>(p.alpha * v + bias);
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
template <typename T, int EPI, int FM, int FN>
DEV void store_tile(const GemmArgs& p, const floatx4 (&acc)[FM][FN], int mw, int nw, int lane, bool full) {
    if (full) store_body<T, EPI, FM, FN, false>(p, acc, mw, nw, lane);
    else store_body<T, EPI, FM, FN, true>(p, acc, mw, nw, lane);
}

template <typename T, int ALAY, int BLAY, int EPI, int BM, int BN>
__global__ void __launch_bounds__(GTHREADS, (BM * BN > 128 * 128) ? 1 : 2) gemm_kernel(GemmArgs p) {
    if (p.c_row_dev) p.C = (char*)p.C + (int64_t)min(max(*p.c_row_dev, 0), p.c_row_max) * p.c_row_bytes;
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

    store_tile<T, EPI, FM, FN>(p, acc, m0 + wm * TM, n0 + wn * TN, lane, m0 + BM <= p.M && n0 + BN <= p.N);
}

// ====================================================================== LDS-streamed bf16 path
// bf16 operands in either orientation, K a multiple of 64 per split. Each 64-k tile of an
// operand goes straight from global memory into LDS with global_load_lds_dwordx4 (lane i of
// a wave writes LDS bytes base + 16*i), in the orientation it has in global memory, so the
// loads cost no registers, no LDS-store instructions and no transposes:
//   k-contiguous operand, R rows:   LDS [R][64 k], 128-byte rows; the 16-byte chunk c of row
//                                   r sits in slot c ^ ((r >> 1) & 7)
//   mn-contiguous operand, R cols:  LDS [64 k][R], 2R-byte rows; the 16-byte chunk c of k-row
//                                   k sits in slot c ^ (2 * ((k & 3) | ((k >> 3) & 1) << 2))
// Each lane picks its global chunk so that the slot it writes holds the chunk the swizzle
// puts there; a row is still read whole by 8 (or R/8) consecutive lanes. Fragments
// (8 consecutive k of one row/column per lane) are read with ds_read_b128 from k-contiguous
// tiles and with two ds_read_b64_tr_b16 from mn-contiguous tiles: within each 16-lane group
// that instruction hands lane i element (i % 4) of the 8 bytes addressed by lane 4j + i/4 as
// its j-th value, so when the group addresses 4 k-rows x 16 columns every lane receives 4
// consecutive k of one column. Both swizzles make those reads free of bank conflicts.
// Two stages: the loads of tile kt+1 are issued right after the barrier that opens the
// multiplication of tile kt and are waited for (vmcnt) before the next barrier. (The few-row
// 128x64 tiles keep three: tile kt+2 is issued there, and the wait leaves tile kt+1's loads
// in flight.)
constexpr int MM_BK = 64;   // bf16 elements of K per tile (128 bytes)
// compute units of the device (set by gemm_setup; 256 on MI355X)
static int kGemmCUs = 256;

DEV int swz_k(int r) { return (r >> 1) & 7; }
DEV int swz_mn(int k) { return ((k & 3) | ((k >> 1) & 4)) << 1; }
// slot of 16-byte chunk ch in k-row k of an mn-contiguous tile with R columns (R/8 chunks):
// the XOR stays inside aligned groups of 16 chunks; a trailing group of 8 (R = 192) uses
// the low 3 bits of the swizzle only
template <int R>
DEV int mn_slot(int ch, int k) {
    constexpr int CPR = R / 8;
    if constexpr (CPR % 16 == 0) {
        return ch ^ swz_mn(k);
    } else {
        const int base = ch & ~15;
        return base + ((ch & 15) ^ (swz_mn(k) & (base + 16 <= CPR ? 15 : 7)));
    }
}

// byte offsets (from the tile's base address) of the R/32 direct loads one wave issues per
// tile; rows/columns past the matrix edge are clamped (valid memory, outputs discarded)
template <int LAY, int R>
DEV void mm_offsets(uint32_t (&off)[R / 32], int64_t ld, int row0, int dim, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < R / 32; ++i) {
        const int o = (wave * (R / 32) + i) * 64 + lane;   // 16-byte unit of the LDS tile
        if constexpr (LAY == 0) {
            const int r = o >> 3, c = (o & 7) ^ swz_k(r);
            const int rr = min(row0 + r, dim - 1) - row0;
            off[i] = (uint32_t)(rr * ld * 2 + c * 16);
        } else {
            constexpr int CPR = R / 8;
            const int k = o / CPR, c = mn_slot<R>(o % CPR, k);   // mn_slot is an involution
            const int col = min(row0 + c * 8, dim - 8) - row0;
            off[i] = (uint32_t)(k * ld * 2 + col * 2);
        }
    }
}
template <int R>
DEV void mm_issue(const void* base, const uint32_t (&off)[R / 32], uint32_t lds, int wave) {
#pragma unroll
    for (int i = 0; i < R / 32; ++i) dma16(base, off[i], lds + (wave * (R / 32) + i) * 1024);
}
// fragment of rows/columns rb..rb+15 with k = ks*32 + 8*(lane>>4) + 0..7
template <int LAY, int R>
DEV bf16x8 mm_frag(const char* t, int rb, int ks, int lane) {
    if constexpr (LAY == 0) {
        const int r = rb + (lane & 15), c = ks * 4 + (lane >> 4);
        return __builtin_bit_cast(bf16x8, ld16(t + r * 128 + ((c ^ swz_k(r)) << 4)));
    } else {
        const int g = lane >> 4, q = lane & 15;
        const int col = rb + 4 * (q & 3), ch = col >> 3, within = (col & 7) * 2;
        const int k0 = ks * 32 + 8 * g + (q >> 2), k1 = k0 + 4;
        return read_tr_pair(t + k0 * (2 * R) + (mn_slot<R>(ch, k0) << 4) + within,
                            t + k1 * (2 * R) + (mn_slot<R>(ch, k1) << 4) + within);
    }
}

// Epilogue of the LDS-streamed path. Its MFMAs take B as the first operand, so acc[i][j] is a
// block of C^T: lane l holds row m = mw + 16i + (l & 15) and the 4 consecutive columns
// n = nw + 16j + 4(l >> 4) + r, r = 0..3.
DEV bf16x4 to_bf16x4(float a, float b, float c, float d) {
    bf16x4 o;
    o[0] = (bf16)a; o[1] = (bf16)b; o[2] = (bf16)c; o[3] = (bf16)d;
    return o;
}
// Epilogues that read a second matrix (the residual, the saved pre-activation, or the output
// itself when accumulating) get that input as a value loaded ahead of time, so that a thread's
// loads of a whole staged half are in flight together instead of one after each store.
template <int EPI> struct EpiIn { typedef float4 T; };
template <> struct EpiIn<EPI_GELU_BWD> { typedef bf16x4 T; };
template <int EPI>
DEV bool epi_reads(const GemmArgs& p) {
    return EPI == EPI_GELU_BWD || (EPI == EPI_F32 && p.beta);
}
// 1 if the 4 columns n..n+3 of row m take the vector path
DEV bool epi_vec(const GemmArgs& p, int m, int n) { return m < p.M && p.vec && n + 3 < p.N; }
template <int EPI>
DEV typename EpiIn<EPI>::T epi_load(const GemmArgs& p, int m, int n) {
    if constexpr (EPI == EPI_GELU_BWD) return *(const bf16x4*)((const bf16*)p.aux + (int64_t)m * p.ldaux + n);
    else return *(const float4*)((const float*)p.C + (int64_t)m * p.ldc + n);
}

constexpr float kLog2eF = 1.4426950408889634f;

// Epilogue steps that depend on the column only: the scale alpha (plain output and gradient
// accumulation) and the bias.
template <int EPI>
constexpr bool epi_alpha() { return EPI == EPI_BIAS_T || EPI == EPI_LOGITS || EPI == EPI_F32; }
template <int EPI>
constexpr bool epi_bias() {
    return EPI == EPI_BIAS_T || EPI == EPI_LOGITS || EPI == EPI_BIAS_GELU;
}
// bias of columns n..n+3 (0 past the matrix edge or without a bias)
DEV float4 bias4(const GemmArgs& p, int n) {
    if (!p.bias) return make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.vec && n + 3 < p.N) return *(const float4*)(p.bias + n);
    float b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) b[r] = n + r < p.N ? p.bias[n + r] : 0.f;
    return make_float4(b[0], b[1], b[2], b[3]);
}
// accumulators of columns n..n+3 with alpha and the bias applied. BIAS: 0 no bias, 1 a bias
// known to be present with n..n+3 inside the matrix (one vector load), 2 checked (bias4).
template <int EPI, int BIAS = 2>
DEV float4 epi_pre(const GemmArgs& p, const float4& v, int n) {
    const float al = epi_alpha<EPI>() ? p.alpha : 1.f;
    float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (epi_bias<EPI>()) {
        if constexpr (BIAS == 1) b = *(const float4*)(p.bias + n);
        else if constexpr (BIAS == 2) b = bias4(p, n);
    }
    return make_float4(al * v.x + b.x, al * v.y + b.y, al * v.z + b.z, al * v.w + b.w);
}

// Epilogue on 4 consecutive columns n..n+3 of row m (v = accumulators): vector accesses when
// the 4 columns are inside the matrix and the rows are 16-byte friendly, else per element.
// `in` is epi_load(p, m, n) on the vector path of an epilogue that reads (unused otherwise).
// CHECK = false: the caller knows the chunk is inside the matrix and vector-friendly.
// PRE = true: v already has alpha and the bias applied (epi_pre).
template <int EPI, bool CHECK = true, bool PRE = false>
DEV void epi4(const GemmArgs& p, int m, int n, const float4& v4, const typename EpiIn<EPI>::T& in) {
    if (CHECK && m >= p.M) return;
    const float4 w4 = PRE ? v4 : epi_pre<EPI>(p, v4, n);
    const float v[4] = {w4.x, w4.y, w4.z, w4.w};
    const int64_t o = (int64_t)m * p.ldc + n;
    if (!CHECK || (p.vec && n + 3 < p.N)) {
        if constexpr (EPI == EPI_BIAS_T) {
            *(bf16x4*)((bf16*)p.C + o) = to_bf16x4(v[0], v[1], v[2], v[3]);
        } else if constexpr (EPI == EPI_BIAS_GELU) {
            const bf16x4 u = to_bf16x4(v[0], v[1], v[2], v[3]);
            *(bf16x4*)((bf16*)p.C + o) = u;
            *(bf16x4*)((bf16*)p.C2 + o) = to_bf16x4(gelu_f((float)u[0]), gelu_f((float)u[1]), gelu_f((float)u[2]),
                                                    gelu_f((float)u[3]));
        } else if constexpr (EPI == EPI_GELU_BWD) {
            const bf16x4 a = in;
            *(bf16x4*)((bf16*)p.C + o) = to_bf16x4(v[0] * gelu_grad_f((float)a[0]), v[1] * gelu_grad_f((float)a[1]),
                                                   v[2] * gelu_grad_f((float)a[2]), v[3] * gelu_grad_f((float)a[3]));
        } else if constexpr (EPI == EPI_F32) {
            float4 old = make_float4(0.f, 0.f, 0.f, 0.f);
            if (p.beta) old = in;
            *(float4*)((float*)p.C + o) = make_float4(old.x + v[0], old.y + v[1], old.z + v[2], old.w + v[3]);
        } else {  // EPI_PARTIAL
            *(float4*)((float*)p.C + (int64_t)blockIdx.y * p.part_stride + o) = w4;
        }
        return;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int nn = n + r;
        if (nn >= p.N) continue;
        const int64_t e = o + r;
        if constexpr (EPI == EPI_BIAS_T) {
            ((bf16*)p.C)[e] = (bf16)v[r];
        } else if constexpr (EPI == EPI_BIAS_GELU) {
            const bf16 u = (bf16)v[r];
            ((bf16*)p.C)[e] = u;
            ((bf16*)p.C2)[e] = (bf16)gelu_f((float)u);
        } else if constexpr (EPI == EPI_GELU_BWD) {
            ((bf16*)p.C)[e] = (bf16)(v[r] * gelu_grad_f((float)((const bf16*)p.aux)[(int64_t)m * p.ldaux + nn]));
        } else if constexpr (EPI == EPI_F32) {
            const float old = p.beta ? ((const float*)p.C)[e] : 0.f;
            ((float*)p.C)[e] = old + v[r];
        } else {  // EPI_PARTIAL
            ((float*)p.C)[(int64_t)blockIdx.y * p.part_stride + e] = v[r];
        }
    }
}

// Epilogues with bf16 outputs take 8 consecutive columns per thread, so each output row
// segment is written with 16-byte stores (measured 9-18% faster on the forward products than
// 8-byte stores: the epilogue's store instructions, not its bytes, were what it waited on).
template <int EPI>
constexpr bool epi_wide() {
    return EPI == EPI_BIAS_T || EPI == EPI_LOGITS || EPI == EPI_BIAS_GELU || EPI == EPI_GELU_BWD;
}
template <int EPI> struct EpiIn8 { typedef int T; };
template <> struct EpiIn8<EPI_GELU_BWD> { typedef bf16x8 T; };
DEV bool epi_vec8(const GemmArgs& p, int m, int n) { return m < p.M && p.vec8 && n + 7 < p.N; }

DEV bf16x8 to_bf16x8(const float (&v)[8]) {
    bf16x8 o;
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = (bf16)v[q];
    return o;
}
// epi4 on 8 consecutive columns n..n+7 (a: the first 4 values, b: the next 4, with alpha and
// the bias applied); `in` is the 8 saved pre-activations of the GELU derivative on the vector
// path

// 16-byte store that bypasses the caches (for outputs read again only much later or from HBM
// anyway)
DEV void st16_nt(void* p, const bf16x8& v) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), (u32x4*)p);
}
template <int EPI, bool CHECK = true>
DEV void epi8(const GemmArgs& p, int m, int n, const float4& a, const float4& b, const typename EpiIn8<EPI>::T& in) {
    if (CHECK && m >= p.M) return;
    if (!CHECK || (p.vec8 && n + 7 < p.N)) {
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        const int64_t o = (int64_t)m * p.ldc + n;
        float r[8];
        if constexpr (EPI == EPI_GELU_BWD) {
#pragma unroll
            for (int q = 0; q < 8; ++q) r[q] = v[q] * gelu_grad_f((float)in[q]);
            *(bf16x8*)((bf16*)p.C + o) = to_bf16x8(r);
        } else if constexpr (EPI == EPI_LOGITS) {
            st16_nt((bf16*)p.C + o, to_bf16x8(v));
        } else if constexpr (EPI == EPI_BIAS_T) {
            *(bf16x8*)((bf16*)p.C + o) = to_bf16x8(v);
        } else {  // EPI_BIAS_GELU
            const bf16x8 u = to_bf16x8(v);
            *(bf16x8*)((bf16*)p.C + o) = u;
#pragma unroll
            for (int q = 0; q < 8; ++q) r[q] = gelu_f((float)u[q]);
            *(bf16x8*)((bf16*)p.C2 + o) = to_bf16x8(r);
        }
        return;
    }
    // edge or unaligned: two 4-column chunks (their inputs loaded here)
    typename EpiIn<EPI>::T i0{}, i1{};
    if (epi_reads<EPI>(p)) {
        if (epi_vec(p, m, n)) i0 = epi_load<EPI>(p, m, n);
        if (epi_vec(p, m, n + 4)) i1 = epi_load<EPI>(p, m, n + 4);
    }
    epi4<EPI, true, true>(p, m, n, a, i0);
    epi4<EPI, true, true>(p, m, n + 4, b, i1);
}

// LDS-staged epilogues. The fp32 tile passes through LDS in two halves of 64 rows (the waves
// with wm == h write half h with 16-byte stores, conflict-free with rows padded by 16 bytes),
// then all threads apply the epilogue to chunks along the rows, so every global load and store
// of the epilogue covers whole row segments with 16-byte accesses.
//
// bf16 outputs: 8-column chunks. CHK: per-chunk edge checks; BIAS: as in epi_pre.
template <int EPI, int FM, int FN, int BN, bool CHK, int BIAS>
DEV void store_staged_bf16(const GemmArgs& p, const floatx4 (&acc)[FM][FN], char* smem, int m0, int n0, int wm,
                           int wn, int lane, int tid) {
    static_assert(epi_wide<EPI>(), "bf16-output epilogues only");
    constexpr int LDW = BN + 4;            // floats per staged row
    constexpr int CPR = BN / 8;            // chunks per row
    constexpr int NIT = 64 * CPR / GTHREADS;  // chunks per thread and half
    static_assert(64 * CPR % GTHREADS == 0, "whole chunks per thread");
    typedef typename EpiIn8<EPI>::T In;
    float* st = (float*)smem;
    float* stats = st + 64 * LDW;          // EPI_LOGITS: 64 rows x CPR (max, sum) pairs
    static_assert(EPI != EPI_LOGITS || 4 * 64 * LDW + 8 * 64 * CPR <= 2 * (128 + BN) * 128,
                  "staged rows and statistics fit in the main loop's LDS");
    lds_barrier();                         // every wave is done reading the last K tile
    // the two halves (a generic lambda called twice, so both are laid out straight)
    auto half = [&](auto hc) {
        constexpr int h = decltype(hc)::value;
        In in[NIT];
        if constexpr (EPI == EPI_GELU_BWD) {
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int k = tid + it * GTHREADS, r = k / CPR, c = k - r * CPR;
                const int m = m0 + 64 * h + r, n = n0 + 8 * c;
                if (!CHK || epi_vec8(p, m, n)) in[it] = *(const bf16x8*)((const bf16*)p.aux + (int64_t)m * p.ldaux + n);
            }
        }
        if (wm == h) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    *(float4*)(st + (16 * i + (lane & 15)) * LDW + wn * (BN / 2) + 16 * j + 4 * (lane >> 4)) =
                        make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
        lds_barrier();
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int k = tid + it * GTHREADS, r = k / CPR, c = k - r * CPR;
            const int m = m0 + 64 * h + r, n = n0 + 8 * c;
            const float4 a = epi_pre<EPI, BIAS>(p, *(const float4*)(st + r * LDW + 8 * c), n);
            const float4 b = epi_pre<EPI, BIAS>(p, *(const float4*)(st + r * LDW + 8 * c + 4), n + 4);
            epi8<EPI, CHK>(p, m, n, a, b, in[it]);
            if constexpr (EPI == EPI_LOGITS) {
                // softmax statistics of the 8 stored (bf16-rounded) values: max, sum exp(z - max)
                const float z[8] = {(float)(bf16)a.x, (float)(bf16)a.y, (float)(bf16)a.z, (float)(bf16)a.w,
                                    (float)(bf16)b.x, (float)(bf16)b.y, (float)(bf16)b.z, (float)(bf16)b.w};
                float mx = z[0];
#pragma unroll
                for (int q = 1; q < 8; ++q) mx = fmaxf(mx, z[q]);
                float sm = 0.f;
#pragma unroll
                for (int q = 0; q < 8; ++q) sm += __builtin_amdgcn_exp2f((z[q] - mx) * kLog2eF);
                ((float2*)stats)[r * CPR + c] = make_float2(mx, sm);
            }
        }
        lds_barrier();
        if constexpr (EPI == EPI_LOGITS) {
            // four threads per row (lanes 4r..4r+3 of a wave) merge a quarter of the row's chunk
            // statistics each, then combine with two butterfly steps
            static_assert(CPR % 4 == 0 && GTHREADS == 256, "a quarter row of chunks per thread");
            constexpr int CQ = CPR / 4;
            const int r = tid >> 2;
            const float2* rs = (const float2*)stats + r * CPR + (tid & 3) * CQ;
            float2 v[CQ];
#pragma unroll
            for (int c = 0; c < CQ; ++c) v[c] = rs[c];
            float mx = v[0].x;
#pragma unroll
            for (int c = 1; c < CQ; ++c) mx = fmaxf(mx, v[c].x);
#pragma unroll
            for (int o = 1; o < 4; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            float sm = 0.f;
#pragma unroll
            for (int c = 0; c < CQ; ++c) sm += v[c].y * __builtin_amdgcn_exp2f((v[c].x - mx) * kLog2eF);
#pragma unroll
            for (int o = 1; o < 4; o <<= 1) sm += __shfl_xor(sm, o);
            if ((tid & 3) == 0) {
                const int tiles = p.N / BN;
                ((float2*)p.C2)[(int64_t)(m0 + 64 * h + r) * tiles + n0 / BN] = make_float2(mx, sm);
            }
            lds_barrier();
        }
    };
    half(std::integral_constant<int, 0>{});
    half(std::integral_constant<int, 1>{});
}
// fp32 outputs (gradient output, split-K partials): 4-column chunks (already
// 16-byte accesses), alpha and the bias applied per chunk by epi4. Split-K partials of
// a tile inside the matrix skip the per-chunk checks. (Applying alpha and the bias ahead of
// epi4, as the bf16 form does, measured 9-12% slower here.)
template <int EPI, int FM, int FN, int BN>
DEV void store_staged_f32(const GemmArgs& p, const floatx4 (&acc)[FM][FN], char* smem, int m0, int n0, int wm,
                          int wn, int lane, int tid) {
    constexpr int LDW = BN + 4, CPR = BN / 4, NIT = 64 * CPR / GTHREADS;
    static_assert(64 * CPR % GTHREADS == 0, "whole chunks per thread");
    typedef typename EpiIn<EPI>::T In;
    float* st = (float*)smem;
    const bool reads = epi_reads<EPI>(p);
    const bool full = EPI == EPI_PARTIAL && m0 + 128 <= p.M && n0 + BN <= p.N && p.vec;
    lds_barrier();                       // every wave is done reading the last K tile
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // (the half as a lambda: the compiler then keeps all of a half's input loads in flight
        // together, measured faster than the same code written inline)
        auto half = [&](auto check) {
            constexpr bool CHK = decltype(check)::value;
            In in[NIT];
            if (reads) {
#pragma unroll
                for (int it = 0; it < NIT; ++it) {
                    const int k = tid + it * GTHREADS, r = k / CPR, c4 = k - r * CPR;
                    const int m = m0 + 64 * h + r, n = n0 + 4 * c4;
                    if (epi_vec(p, m, n)) in[it] = epi_load<EPI>(p, m, n);
                }
            }
            if (wm == h) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        *(float4*)(st + (16 * i + (lane & 15)) * LDW + wn * (BN / 2) + 16 * j + 4 * (lane >> 4)) =
                            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
            lds_barrier();
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int k = tid + it * GTHREADS, r = k / CPR, c4 = k - r * CPR;
                epi4<EPI, CHK>(p, m0 + 64 * h + r, n0 + 4 * c4, *(const float4*)(st + r * LDW + 4 * c4), in[it]);
            }
            lds_barrier();
        };
        if constexpr (EPI == EPI_PARTIAL) {
            if (full) half(std::false_type{});
            else half(std::true_type{});
        } else {
            half(std::true_type{});
        }
    }
}
// For bf16 outputs, a tile inside the matrix with vector-friendly rows takes a straight-line
// form without per-chunk checks or bias branches, so its LDS reads and stores are issued back
// to back. The choice is made once per tile: were the two forms to meet between the halves,
// the compiler would wait there for every store of the first half (a wait it places where
// paths with outstanding loads join).
template <int EPI, int FM, int FN, int BN>
DEV void store_staged(const GemmArgs& p, const floatx4 (&acc)[FM][FN], char* smem, int m0, int n0, int wm, int wn,
                      int lane, int tid) {
    if constexpr (epi_wide<EPI>()) {
        const bool full = m0 + 128 <= p.M && n0 + BN <= p.N && p.vec8;
        if constexpr (EPI == EPI_LOGITS) {  // whole tiles only (gemm_logits_tiles)
            if (p.bias) store_staged_bf16<EPI, FM, FN, BN, false, 1>(p, acc, smem, m0, n0, wm, wn, lane, tid);
            else store_staged_bf16<EPI, FM, FN, BN, false, 0>(p, acc, smem, m0, n0, wm, wn, lane, tid);
            return;
        }
        if (full && epi_bias<EPI>() && p.bias)
            store_staged_bf16<EPI, FM, FN, BN, false, 1>(p, acc, smem, m0, n0, wm, wn, lane, tid);
        else if (full)
            store_staged_bf16<EPI, FM, FN, BN, false, 0>(p, acc, smem, m0, n0, wm, wn, lane, tid);
        else
            store_staged_bf16<EPI, FM, FN, BN, true, 2>(p, acc, smem, m0, n0, wm, wn, lane, tid);
    } else {
        store_staged_f32<EPI, FM, FN, BN>(p, acc, smem, m0, n0, wm, wn, lane, tid);
    }
}

// K stages in LDS: two (one tile multiplied while the next is loaded), three for the
// few-row 128x64 tiles (72 KB, still two workgroups per CU), whose short main loops otherwise
// wait on each tile's load latency (B=4 MLP projection 44 -> 40 us)
template <int BM, int BN>
constexpr int mm_nst() { return BN == 64 ? 3 : 2; }
// s_waitcnt vmcnt(N) lgkmcnt(0), then the barrier (N of this wave's direct loads may stay in flight)
template <int N>
DEV void dma_wait_barrier_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((N >> 4) << 14));
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// One output tile of the LDS-streamed path: workgroup `pid` of `nwg` over the tiles of p, K
// split `split` (a plain launch passes blockIdx.x, gridDim.x, blockIdx.y; a grouped launch its
// product's own numbering).
template <int ALAY, int BLAY, int EPI, int BM, int BN, bool ROWSUM>
DEV void mm_tile(const GemmArgs& p, int pid, int nwg, int split, char* smem, bool remap = true) {
    constexpr int STAGE = (BM + BN) * 128;
    constexpr int TM = BM / 2, TN = BN / 2, FM = TM / 16, FN = TN / 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), wm = wave >> 1, wn = wave & 1;
    const int num_m = (p.M + BM - 1) / BM, num_n = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(pid, nwg, num_m, num_n, tm, tn, remap);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = split * p.ksplit_len;
    const int nt = min(p.ksplit_len, p.K - kbeg) / MM_BK;

    uint32_t offA[BM / 32], offB[BN / 32];
    mm_offsets<ALAY, BM>(offA, p.lda, m0, p.M, wave, lane);
    mm_offsets<BLAY, BN>(offB, p.ldb, n0, p.N, wave, lane);
    // tile kt of each operand starts at base + kt * step (bytes)
    const char* baseA = (const char*)p.A + 2 * (ALAY == 0 ? (int64_t)m0 * p.lda + kbeg : (int64_t)kbeg * p.lda + m0);
    const char* baseB = (const char*)p.B + 2 * (BLAY == 0 ? (int64_t)n0 * p.ldb + kbeg : (int64_t)kbeg * p.ldb + n0);
    const int64_t stepA = ALAY == 0 ? 2 * MM_BK : 2 * MM_BK * p.lda;
    const int64_t stepB = BLAY == 0 ? 2 * MM_BK : 2 * MM_BK * p.ldb;
    const uint32_t lds0 = lds_addr(smem);

    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    // row sums of A: the waves of the first column tile with wn == 0 multiply the A fragments
    // they read anyway by a fragment of ones (one more MFMA per fragment, fp32 accumulation);
    // every column of rs[i] then holds the sum over k of row 16i + (lane & 15)
    floatx4 rs[ROWSUM ? FM : 1];
#pragma unroll
    for (int i = 0; i < (ROWSUM ? FM : 1); ++i) rs[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    const bool do_rs = ROWSUM && (p.rowsum_part || p.rowsum_out) && tn == 0 && wn == 0;

    constexpr int NST = mm_nst<BM, BN>();
    if (nt > 0) {
        mm_issue<BM>(baseA, offA, lds0, wave);
        mm_issue<BN>(baseB, offB, lds0 + BM * 128, wave);
    }
    if (NST == 3 && nt > 1) {
        mm_issue<BM>(baseA + stepA, offA, lds0 + STAGE, wave);
        mm_issue<BN>(baseB + stepB, offB, lds0 + STAGE + BM * 128, wave);
    }
    for (int kt = 0; kt < nt; ++kt) {
        // tile kt is in LDS once this wave's loads have landed and every wave has passed the
        // barrier, which also retires every read of the stage refilled next; a bare barrier
        // (no fence) keeps the prefetch below in flight
        if constexpr (NST == 3) {
            // tiles kt and kt + 1 in flight: wait for all but tile kt + 1's loads
            if (kt + 1 < nt) dma_wait_barrier_vm<(BM + BN) / 32>();
            else dma_wait_barrier();
            if (kt + 2 < nt) {
                const uint32_t st = lds0 + ((kt + 2) % 3) * STAGE;
                mm_issue<BM>(baseA + (kt + 2) * stepA, offA, st, wave);
                mm_issue<BN>(baseB + (kt + 2) * stepB, offB, st + BM * 128, wave);
            }
        } else {
            dma_wait_barrier();
            if (kt + 1 < nt) {
                const uint32_t st = lds0 + ((kt + 1) & 1) * STAGE;
                mm_issue<BM>(baseA + (kt + 1) * stepA, offA, st, wave);
                mm_issue<BN>(baseB + (kt + 1) * stepB, offB, st + BM * 128, wave);
            }
        }
        const char* As = smem + (NST == 3 ? kt % 3 : kt & 1) * STAGE;
        const char* Bs = As + BM * 128;
        // raised priority while this wave multiplies: the other wave on the SIMD (from the other
        // workgroup) issues its loads in the gaps instead of interleaving its own MFMA chain
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = mm_frag<ALAY, BM>(As, wm * TM + 16 * i, ks, lane);
            if constexpr (ROWSUM) {
                if (do_rs) {
                    const bf16x8 ones = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
#pragma unroll
                    for (int i = 0; i < FM; ++i) mma8(rs[i], ones, af[i]);
                }
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) bfr[j] = mm_frag<BLAY, BN>(Bs, wn * TN + 16 * j, ks, lane);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) mma8(acc[i][j], bfr[j], af[i]);
        }
        __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (ROWSUM) {
        if (do_rs) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int m = m0 + wm * TM + 16 * i + (lane & 15);
                if (lane < 16 && m < p.M) {
                    if (p.rowsum_out) p.rowsum_out[m] = p.beta ? p.rowsum_out[m] + rs[i][0] : rs[i][0];
                    else p.rowsum_part[(int64_t)split * p.M + m] = rs[i][0];
                }
            }
        }
    }
    store_staged<EPI, FM, FN, BN>(p, acc, smem, m0, n0, wm, wn, lane, tid);
}

// Bounds of one workgroup per CU: the compiler then keeps the accumulators in AGPRs and uses the
// VGPRs for deeper load scheduling (measured 10-15% faster than a two-workgroup bound). Every
// instantiation stays at or below 256 registers in total, so two workgroups still share a CU.
// (The row-sum variant needs the explicit two-workgroup bound to stay within 256 registers.)
template <int ALAY, int BLAY, int EPI, int BM, int BN, bool ROWSUM = false>
__global__ void __launch_bounds__(GTHREADS, ROWSUM ? 2 : 1) gemm_mm_kernel(GemmArgs p) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    mm_tile<ALAY, BLAY, EPI, BM, BN, ROWSUM>(p, blockIdx.x, gridDim.x, blockIdx.y, smem);
}

// Grouped weight-gradient products: the launch's tiles are numbered XCD-first over the whole
// product list (each XCD takes a contiguous run of whole products, so a product's operand panels
// are fetched into one L2 instead of all eight); logical tile w runs tile w - tile0 of the
// product whose range [tile0, tile0 + ntiles) holds it (binary search over the sorted ranges).
// Every product takes the whole K, so there are no split-K partials.
template <int BN>
__global__ void __launch_bounds__(GTHREADS, 2) gemm_mm_group_kernel(GemmArgs base, const GroupProb* __restrict__ probs,
                                                                    int nprob) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int w = xcd_logical(blockIdx.x, gridDim.x);
    int lo = 0, hi = nprob - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (probs[mid].tile0 <= w) lo = mid;
        else hi = mid - 1;
    }
    const GroupProb g = probs[lo];
    GemmArgs p = base;
    p.A = g.A; p.B = g.B; p.C = g.C; p.lda = g.lda; p.ldb = g.ldb; p.ldc = g.ldc;
    p.M = g.M; p.N = g.N;
    p.rowsum_part = nullptr;
    p.rowsum_out = g.rowsum;
    mm_tile<1, 1, EPI_F32, 128, BN, true>(p, w - g.tile0, g.ntiles, 0, smem, false);
}

template <int BM, int BN>
constexpr size_t mm_lds_bytes() { return mm_nst<BM, BN>() * (size_t)(BM + BN) * 128; }

// Per-kernel timing: while the caller has handed over an event pair (gemm_time_next), the next
// product that is a single kernel records them at that kernel's own start and end
// (hipExtLaunchKernel), so the interval holds the kernel alone, as a kernel trace reports it.
static thread_local hipEvent_t t_ev0 = nullptr, t_ev1 = nullptr;
static thread_local bool t_ev_used = false;
void gemm_time_next(hipEvent_t start, hipEvent_t stop) {
    t_ev0 = start;
    t_ev1 = stop;
    t_ev_used = false;
}
bool gemm_time_taken() {
    const bool used = t_ev_used;
    t_ev0 = t_ev1 = nullptr;
    t_ev_used = false;
    return used;
}
// launch `kernel` with the handed-over events, if any are pending (true: launched)
static bool launch_timed(const void* kernel, dim3 grid, dim3 block, void** args, size_t lds, hipStream_t s,
                         hipError_t* err) {
    if (!t_ev0) return false;
    *err = hipExtLaunchKernel(kernel, grid, block, args, lds, s, t_ev0, t_ev1, 0);
    t_ev0 = t_ev1 = nullptr;
    t_ev_used = *err == hipSuccess;
    return true;
}

template <int ALAY, int BLAY, int EPI, int BM, int BN>
static hipError_t launch_mm(const GemmArgs& a, int nsplit, hipStream_t s) {
    const int num_m = (a.M + BM - 1) / BM, num_n = (a.N + BN - 1) / BN;
    dim3 grid(num_m * num_n, nsplit);
    if constexpr (ALAY == 1) {
        if (a.rowsum_part) {
            gemm_mm_kernel<ALAY, BLAY, EPI, BM, BN, true><<<grid, dim3(GTHREADS), mm_lds_bytes<BM, BN>(), s>>>(a);
            return hipGetLastError();
        }
    }
    if (nsplit == 1 && !a.rowsum_part) {   // one kernel: timed alone when events are pending
        void* args[] = {(void*)&a};
        hipError_t e;
        if (launch_timed((const void*)gemm_mm_kernel<ALAY, BLAY, EPI, BM, BN>, grid, dim3(GTHREADS), args,
                         mm_lds_bytes<BM, BN>(), s, &e))
            return e;
    }
    gemm_mm_kernel<ALAY, BLAY, EPI, BM, BN><<<grid, dim3(GTHREADS), mm_lds_bytes<BM, BN>(), s>>>(a);
    return hipGetLastError();
}


static bool mm_ok(const GemmDesc& d, int ksplit_len);

int gemm_group_tiles(int M, int N, int bn) { return ((M + 127) / 128) * ((N + bn - 1) / bn); }

bool gemm_group_ok(const GroupProb& g, int K) {
    auto al = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
    GemmDesc d;
    d.A = g.A; d.lda = g.lda; d.a_layout = 1;
    d.B = g.B; d.ldb = g.ldb; d.b_layout = 1;
    d.M = g.M; d.N = g.N; d.K = K;
    return mm_ok(d, K) && g.ldc % 4 == 0 && al(g.C) && (!g.rowsum || al(g.rowsum));
}

hipError_t gemm_grouped(const GroupProb* d_probs, int nprob, int total_tiles, int K, float alpha, int beta, int bn,
                        hipStream_t s) {
    if (nprob < 1 || total_tiles < 1 || K % MM_BK || (bn != 128 && bn != 192)) return hipErrorInvalidValue;
    GemmArgs a{};
    a.K = K;
    a.ksplit_len = K;
    a.alpha = alpha;
    a.beta = beta;
    a.vec = 1;
    void* args[] = {(void*)&a, (void*)&d_probs, (void*)&nprob};
    hipError_t e;
    if (bn == 192) {
        if (launch_timed((const void*)gemm_mm_group_kernel<192>, dim3(total_tiles), dim3(GTHREADS), args,
                         mm_lds_bytes<128, 192>(), s, &e))
            return e;
        gemm_mm_group_kernel<192><<<dim3(total_tiles), dim3(GTHREADS), mm_lds_bytes<128, 192>(), s>>>(a, d_probs, nprob);
    } else {
        if (launch_timed((const void*)gemm_mm_group_kernel<128>, dim3(total_tiles), dim3(GTHREADS), args,
                         mm_lds_bytes<128, 128>(), s, &e))
            return e;
        gemm_mm_group_kernel<128><<<dim3(total_tiles), dim3(GTHREADS), mm_lds_bytes<128, 128>(), s>>>(a, d_probs, nprob);
    }
    return hipGetLastError();
}

// out[m][n] = (beta ? out : 0) + alpha * sum_z part[z][m][n], z in order (deterministic).
// Workgroups past the matrix (when rs_out is set) reduce the row-sum partials the same way:
// rs_out[m] = (beta ? rs_out[m] : 0) + sum_z rs_part[z][m].
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int nsplit, int64_t stride,
                                     float* __restrict__ out, int64_t n_elem, float alpha, int beta, int mat_blocks,
                                     const float* __restrict__ rs_part, int rs_m, float* __restrict__ rs_out) {
    if ((int)blockIdx.x >= mat_blocks) {
        const int m = ((int)blockIdx.x - mat_blocks) * blockDim.x + threadIdx.x;
        if (m >= rs_m) return;
        float v = 0.f;
        for (int z = 0; z < nsplit; ++z) v += rs_part[(int64_t)z * rs_m + m];
        rs_out[m] = beta ? rs_out[m] + v : v;
        return;
    }
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

size_t gemm_lds_bytes() { return mm_lds_bytes<128, 192>(); }

// Tile of the register-staged path (fp32, and bf16 shapes the LDS-streamed path does not
// take): always 128x128.
void gemm_pick_tile(int M, int N, int nsplit, int is_bf16, int* bm, int* bn) {
    (void)M;
    (void)N;
    (void)nsplit;
    (void)is_bf16;
    *bm = 128;
    *bn = 128;
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
    (void)bm;
    (void)bn;
    return launch<T, ALAY, BLAY, EPI, 128, 128>(a, nsplit, s);
}

// Shapes the LDS-streamed path takes: whole 64-wide K tiles in every split, leading
// dimensions and mn-contiguous extents in multiples of 8 elements, 16-byte aligned bases,
// and per-lane tile offsets that fit in 32 bits.
static bool mm_ok(const GemmDesc& d, int ksplit_len) {
    if (d.K % MM_BK || ksplit_len % MM_BK || d.lda % 8 || d.ldb % 8) return false;
    if (((uintptr_t)d.A | (uintptr_t)d.B) & 15) return false;
    if (d.a_layout == 1 && (d.M % 8 || d.M < 8)) return false;
    if (d.b_layout == 1 && (d.N % 8 || d.N < 8)) return false;
    const int64_t lim = (int64_t)1 << 31;
    for (int64_t ld : {d.lda, d.ldb})
        if (255 * ld * 2 + 1024 >= lim) return false;
    return true;
}

// ====================================================================== skinny products
// Products with few rows (M <= SK_MAX_M: one new position per sequence when decoding), both
// operands k-contiguous, bf16 storage (the epilogue is the tiled path's): every weight row is
// streamed once by one wave (lanes take consecutive 16-byte chunks of k), the M activation rows
// come from cache, and each lane keeps M partial sums for its column. A fixed butterfly reduces
// them across the wave; a workgroup's four columns (one per wave) then meet in LDS and go
// through the same epilogue as the tiled path. (Splitting a column's k over several waves
// measured slower: at k = 768 most of their lanes have no chunk.)
constexpr int SK_MAX_M = 16;
constexpr int SK_THREADS = 256;
constexpr int SK_LN_MAX_K = 2048;   // LayerNorm-fused form: [SK_MAX_M][K] bf16 rows in LDS (64 KB)

template <typename T, int EPI, bool LDS_A>
DEV void skinny_body(const GemmArgs& p, const char* sa) {
    constexpr int E = 16 / sizeof(T);        // elements per 16-byte chunk
    __shared__ float res[SK_MAX_M][4];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = blockIdx.x * 4, n = n0 + wave;
    float acc[SK_MAX_M];
#pragma unroll
    for (int m = 0; m < SK_MAX_M; ++m) acc[m] = 0.f;
    if (n < p.N) {
        const T* w = (const T*)p.B + (int64_t)n * p.ldb;
        // every row's load is issued before any use (rows past M repeat row M - 1; their sums
        // are never stored), so a chunk costs one round trip, not one per row
        const T* arow[SK_MAX_M];
#pragma unroll
        for (int m = 0; m < SK_MAX_M; ++m)
            arow[m] = LDS_A ? (const T*)sa + (int64_t)min(m, p.M - 1) * p.K : (const T*)p.A + (int64_t)min(m, p.M - 1) * p.lda;
#pragma unroll 2
        for (int k = lane * E; k < p.K; k += 64 * E) {
            const uint4 wr = ld16(w + k);
            uint4 ar[SK_MAX_M];
#pragma unroll
            for (int m = 0; m < SK_MAX_M; ++m) ar[m] = ld16(arow[m] + k);
            const T* we = (const T*)&wr;
            float wf[E];
#pragma unroll
            for (int q = 0; q < E; ++q) wf[q] = to_f<T>(we[q]);
#pragma unroll
            for (int m = 0; m < SK_MAX_M; ++m) {
                const T* ae = (const T*)&ar[m];
                float s = 0.f;
#pragma unroll
                for (int q = 0; q < E; ++q) s += to_f<T>(ae[q]) * wf[q];
                acc[m] += s;
            }
        }
    }
#pragma unroll
    for (int m = 0; m < SK_MAX_M; ++m) acc[m] = wave_sum(acc[m]);
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < SK_MAX_M; ++m) res[m][wave] = acc[m];
    }
    __syncthreads();
    const int m = threadIdx.x;
    if (m < p.M) {
        GemmArgs q = p;
        if (p.c_row_dev) q.C = (char*)p.C + (int64_t)min(max(*p.c_row_dev, 0), p.c_row_max) * p.c_row_bytes;
        const float4 v = make_float4(res[m][0], res[m][1], res[m][2], res[m][3]);
        typename EpiIn<EPI>::T in;
        if (epi_reads<EPI>(q) && epi_vec(q, m, n0)) in = epi_load<EPI>(q, m, n0);
        epi4<EPI>(q, m, n0, v, in);
    }
}

template <typename T, int EPI>
__global__ void __launch_bounds__(SK_THREADS) gemm_skinny_kernel(GemmArgs p) {
    skinny_body<T, EPI, false>(p, nullptr);
}

// The few-row product of decoding with the residual add and LayerNorm that precede c_attn and
// c_fc fused in: every workgroup forms the M rows x + y of the residual stream (TX: its type;
// y the bf16 projection output, or none), normalizes them exactly as the LayerNorm kernel
// does (one wave per row, the same lane partition and summation order, so the same bits) into
// bf16 rows in LDS, and multiplies those; workgroup 0 also stores x + y as the new stream.
// 23 of a decoding step's 25 LayerNorm launches go away.
template <typename TX, int EPI, int NV>
__global__ void __launch_bounds__(SK_THREADS) gemm_skinny_ln_kernel(GemmArgs p, SkinnyLn ln) {
    extern __shared__ __attribute__((aligned(16))) char sk_a[];   // [M][K] bf16
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int C = p.K, nv = C >> 2;
    const bool store_x = blockIdx.x == 0 && ln.x_out;
    for (int m = wave; m < p.M; m += SK_THREADS / 64) {
        const int64_t ro = (int64_t)m * C;
        float4 v[NV];
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = lane + 64 * j;
            v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < nv) {
                float4 a = load4<TX>((const TX*)ln.x + ro + 4 * c);
                if (ln.y) {
                    const float4 d = load4<bf16>((const bf16*)ln.y + ro + 4 * c);
                    a = make_float4(a.x + d.x, a.y + d.y, a.z + d.z, a.w + d.w);
                }
                if (store_x) store4<TX>((TX*)ln.x_out + ro + 4 * c, a.x, a.y, a.z, a.w);
                v[j] = load4_rounded<TX>(a.x, a.y, a.z, a.w);
            }
            sum += (v[j].x + v[j].y) + (v[j].z + v[j].w);
        }
        const float mu = wave_sum(sum) / (float)C;
        float s2 = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = lane + 64 * j;
            if (c < nv) {
                const float a = v[j].x - mu, bb = v[j].y - mu, cc = v[j].z - mu, d = v[j].w - mu;
                s2 += (a * a + bb * bb) + (cc * cc + d * d);
            }
        }
        const float r = 1.0f / sqrtf(wave_sum(s2) / (float)C + LN_EPS);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = lane + 64 * j;
            if (c < nv) {
                const float4 ww = ((const float4*)ln.w)[c], bb = ((const float4*)ln.b)[c];
                store4<bf16>((bf16*)sk_a + ro + 4 * c, (v[j].x - mu) * r * ww.x + bb.x, (v[j].y - mu) * r * ww.y + bb.y,
                             (v[j].z - mu) * r * ww.z + bb.z, (v[j].w - mu) * r * ww.w + bb.w);
            }
        }
    }
    __syncthreads();
    skinny_body<bf16, EPI, true>(p, sk_a);
}

template <typename T>
static bool skinny_ok(const GemmDesc& d, int nsplit) {
    constexpr int E = 16 / sizeof(T);
    if (d.M > SK_MAX_M || d.a_layout != 0 || d.b_layout != 0 || nsplit != 1 || d.rowsum) return false;
    if (d.N > 16384) return false;   // very wide products (the vocabulary) fill the GPU on the tiled path
    if (d.epi != EPI_BIAS_T && d.epi != EPI_BIAS_GELU) return false;
    if (d.K % E || d.lda % E || d.ldb % E) return false;
    return (((uintptr_t)d.A | (uintptr_t)d.B) & 15) == 0;
}

template <typename T>
static hipError_t launch_skinny(const GemmArgs& a, int epi, hipStream_t s) {
    const dim3 grid((a.N + 3) / 4), blk(SK_THREADS);
    if (epi == EPI_BIAS_T) gemm_skinny_kernel<T, EPI_BIAS_T><<<grid, blk, 0, s>>>(a);
    else gemm_skinny_kernel<T, EPI_BIAS_GELU><<<grid, blk, 0, s>>>(a);
    return hipGetLastError();
}

template <typename TX, int EPI>
static void launch_skinny_ln(const GemmArgs& a, const SkinnyLn& ln, int nv4, size_t lds, hipStream_t s) {
    const dim3 grid((a.N + 3) / 4), blk(SK_THREADS);
#define SKL(NV) gemm_skinny_ln_kernel<TX, EPI, NV><<<grid, blk, lds, s>>>(a, ln)
    if (nv4 <= 64) SKL(1);
    else if (nv4 <= 128) SKL(2);
    else if (nv4 <= 192) SKL(3);
    else if (nv4 <= 256) SKL(4);
    else if (nv4 <= 320) SKL(5);
    else if (nv4 <= 384) SKL(6);
    else if (nv4 <= 448) SKL(7);
    else SKL(8);
#undef SKL
}

int gemm_skinny_ln_ok(const GemmDesc& d, int is_bf16) {
    if (!is_bf16 || !skinny_ok<bf16>(d, 1) || d.lda != d.K || d.K > SK_LN_MAX_K || d.K % 8) return 0;
    return 1;
}

hipError_t gemm_skinny_ln(const GemmDesc& d, const SkinnyLn& ln, int x_bf16, hipStream_t s) {
    if (!gemm_skinny_ln_ok(d, 1) || !ln.x || !ln.w || !ln.b) return hipErrorInvalidValue;
    auto al = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
    if (!al(ln.w) || !al(ln.b) || ((uintptr_t)ln.x & 7) || ((uintptr_t)ln.y & 7) || ((uintptr_t)ln.x_out & 7))
        return hipErrorInvalidValue;
    GemmArgs a{};
    a.A = nullptr; a.B = d.B; a.lda = d.K; a.ldb = d.ldb;
    a.M = d.M; a.N = d.N; a.K = d.K;
    a.C = d.C; a.ldc = d.ldc; a.C2 = d.C2; a.bias = d.bias;
    a.alpha = d.alpha; a.beta = d.beta;
    a.ksplit_len = d.K;
    a.vec = d.ldc % 4 == 0 && al(d.C) && al(d.C2) && al(d.bias);
    a.vec8 = a.vec && d.ldc % 8 == 0;
    a.c_row_dev = d.c_row_dev; a.c_row_bytes = d.c_row_bytes; a.c_row_max = d.c_row_max;
    const size_t lds = (size_t)d.M * d.K * 2;
    const int nv4 = d.K / 4;
    if (x_bf16) {
        if (d.epi == EPI_BIAS_T) launch_skinny_ln<bf16, EPI_BIAS_T>(a, ln, nv4, lds, s);
        else launch_skinny_ln<bf16, EPI_BIAS_GELU>(a, ln, nv4, lds, s);
    } else {
        if (d.epi == EPI_BIAS_T) launch_skinny_ln<float, EPI_BIAS_T>(a, ln, nv4, lds, s);
        else launch_skinny_ln<float, EPI_BIAS_GELU>(a, ln, nv4, lds, s);
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t dispatch(const GemmDesc& d, hipStream_t s) {
    GemmArgs a{};
    a.A = d.A; a.B = d.B; a.lda = d.lda; a.ldb = d.ldb;
    a.M = d.M; a.N = d.N; a.K = d.K;
    a.C = d.C; a.ldc = d.ldc; a.C2 = d.C2; a.bias = d.bias;
    a.aux = d.aux; a.ldaux = d.ldaux; a.alpha = d.alpha; a.beta = d.beta;
    a.rowsum_part = nullptr;
    a.rowsum_out = nullptr;
    constexpr int BK = 128 / sizeof(T);
    int nsplit = d.nsplit < 1 ? 1 : d.nsplit;
    const int ktiles = (d.K + BK - 1) / BK;
    if (nsplit > ktiles) nsplit = ktiles;
    const int per = (ktiles + nsplit - 1) / nsplit;
    nsplit = (ktiles + per - 1) / per;
    a.ksplit_len = per * BK;
    {
        // vector epilogue accesses need 4-element-aligned rows and 16-byte aligned bases
        auto al = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
        a.vec = d.ldc % 4 == 0 && d.ldaux % 4 == 0 && al(d.C) && al(d.C2) && al(d.bias) && al(d.aux) &&
                al(d.partial);
        a.vec8 = a.vec && d.ldc % 8 == 0 && d.ldaux % 8 == 0;
    }
    int epi = d.epi;
    if (epi == EPI_LOGITS && !gemm_logits_tiles(d, sizeof(T) == 2)) return hipErrorInvalidValue;
    a.c_row_dev = d.c_row_dev;
    a.c_row_bytes = d.c_row_bytes;
    a.c_row_max = d.c_row_max;
    if constexpr (sizeof(T) == 2) {
        if (skinny_ok<T>(d, nsplit)) return launch_skinny<T>(a, epi, s);
    }
    if (nsplit > 1 && d.c_row_dev) return hipErrorInvalidValue;   // a device row offset: one split only
    if (nsplit > 1) {
        // partials, then a fixed-order reduce into the fp32 output
        a.C = d.partial; a.ldc = d.N; a.part_stride = (int64_t)d.M * d.N;
        epi = EPI_PARTIAL;
    }
    int bm = d.bm, bn = d.bn;
    if (bm == 0) gemm_pick_tile(d.M, d.N, nsplit, sizeof(T) == 2, &bm, &bn);
    hipError_t e = hipSuccess;
    if constexpr (sizeof(T) == 2) {
        if (!d.no_dl && mm_ok(d, a.ksplit_len) && !d.c_row_dev) {
            if (d.rowsum && d.a_layout == 1) a.rowsum_part = d.rowsum_part;
            // 128x192 tiles (wave tile 64x96: fewer LDS bytes per MFMA) where, at the 128x192
            // tile's measured 1.15 times the rate per output of 128x128, they use the rounds of
            // 512 workgroups (two per CU) and the output area better: N = 768 gives 512 tiles
            // instead of 768, N = 2304 three rounds instead of 4.5, N = 50304 = 262 x 192; ragged
            // N = 6400 (1558M-shaped MLP) 3 rounds instead of 4 (c_fc 6.11 -> 5.92 ms per step);
            // N = 1600 at 4096 rows stays 128-wide (416 tiles against 288: 128x192 measured
            // slower there). 256x256 tiles measured slower everywhere.
            bool wide = false, narrow = false;
            if (epi == EPI_LOGITS) {
                wide = true;
            } else if (d.bn) {
                wide = d.bn == 192;
                narrow = d.bn == 64;
            } else if (nsplit == 1) {
                // fraction of the launched rounds' output area that is the product's own
                auto fill = [&](int bn) {
                    const int64_t nt = (d.N + bn - 1) / bn;
                    const int64_t blocks = (int64_t)((d.M + 127) / 128) * nt;
                    const int64_t rounds = (blocks + 511) / 512;
                    return (double)blocks / (double)(rounds * 512) * (double)d.N / (double)(nt * bn);
                };
                if (d.N % 64 == 0) wide = 1.15 * fill(192) >= fill(128);
                // 128x64 tiles (48 KB of LDS: three workgroups per CU) where 128-wide tiles
                // would leave CUs without a workgroup (few rows: a batch of 4 sequences, the
                // forward-only pass): more workgroups at more LDS bytes per MFMA
                const int64_t blocks128 = (int64_t)((d.M + 127) / 128) * ((d.N + 127) / 128);
                if (d.N % 64 == 0 && blocks128 < kGemmCUs) {
                    narrow = true;
                    wide = false;
                }
            }
#define MM_CASE(AL, BL, EP)                                                                   \
    if (d.a_layout == AL && d.b_layout == BL && epi == EP) e = launch_mm<AL, BL, EP, 128, 128>(a, nsplit, s); else
#define MM_CASE_WIDE(AL, BL, EP)                                                              \
    if (wide && d.a_layout == AL && d.b_layout == BL && epi == EP) e = launch_mm<AL, BL, EP, 128, 192>(a, nsplit, s); else
#define MM_CASE_NARROW(AL, BL, EP)                                                            \
    if (narrow && d.a_layout == AL && d.b_layout == BL && epi == EP) e = launch_mm<AL, BL, EP, 128, 64>(a, nsplit, s); else
            MM_CASE_WIDE(0, 0, EPI_BIAS_T)
            MM_CASE_WIDE(0, 0, EPI_LOGITS)
            MM_CASE_WIDE(0, 1, EPI_F32)
            MM_CASE_WIDE(0, 1, EPI_BIAS_T)
            MM_CASE_WIDE(0, 0, EPI_BIAS_GELU)
            MM_CASE_WIDE(0, 1, EPI_GELU_BWD)
            MM_CASE_WIDE(1, 1, EPI_PARTIAL)
            MM_CASE_WIDE(1, 1, EPI_F32)
            MM_CASE_NARROW(0, 0, EPI_BIAS_T)
            MM_CASE_NARROW(0, 0, EPI_BIAS_GELU)
            MM_CASE_NARROW(0, 1, EPI_BIAS_T)
            MM_CASE_NARROW(0, 1, EPI_GELU_BWD)
            MM_CASE(0, 0, EPI_BIAS_T)
            MM_CASE(0, 0, EPI_BIAS_GELU)
            MM_CASE(0, 1, EPI_GELU_BWD)
            MM_CASE(0, 1, EPI_F32)
            MM_CASE(0, 1, EPI_BIAS_T)
            MM_CASE(0, 1, EPI_PARTIAL)
            MM_CASE(1, 1, EPI_F32)
            MM_CASE(1, 1, EPI_PARTIAL)
            return hipErrorInvalidValue;
#undef MM_CASE
#undef MM_CASE_WIDE
#undef MM_CASE_NARROW
            goto reduce;
        }
    }
#define GEMM_CASE(AL, BL, EP) \
    if (d.a_layout == AL && d.b_layout == BL && epi == EP) e = launch_tiled<T, AL, BL, EP>(a, nsplit, bm, bn, s); else
    GEMM_CASE(0, 0, EPI_BIAS_T)
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
    if (nsplit > 1 || a.rowsum_part) {
        // one launch: the split-K partials (if split) and the row-sum partials (if requested)
        if (nsplit > 1 && (d.epi != EPI_F32 || d.ldc != d.N)) return hipErrorInvalidValue;
        const int64_t n = nsplit > 1 ? (int64_t)d.M * d.N : 0;
        const int threads = 256;
        const int mat_blocks = (int)((n / 4 + threads - 1) / threads);
        const int rs_blocks = a.rowsum_part ? (d.M + threads - 1) / threads : 0;
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)(mat_blocks + rs_blocks)), dim3(threads), 0, s,
                           (const float*)d.partial, nsplit, (int64_t)d.M * d.N, (float*)d.C, n, d.alpha, d.beta,
                           mat_blocks, (const float*)a.rowsum_part, d.M, d.rowsum);
        e = hipGetLastError();
    }
    return e;
}

int gemm_logits_tiles(const GemmDesc& d, int is_bf16) {
    const bool ok = is_bf16 && !d.no_dl && d.a_layout == 0 && d.b_layout == 0 && d.nsplit <= 1 &&
                    (d.bn == 0 || d.bn == 192) && d.M % 128 == 0 && d.N % 192 == 0 && d.ldc % 8 == 0 &&
                    (((uintptr_t)d.C | (uintptr_t)d.C2 | (uintptr_t)d.bias) & 15) == 0 && d.C2 &&
                    mm_ok(d, ((d.K + MM_BK - 1) / MM_BK) * MM_BK);
    return ok ? d.N / 192 : 0;
}

int gemm_fuses_rowsum(const GemmDesc& d, int is_bf16) {
    if (!is_bf16 || d.no_dl || d.a_layout != 1) return 0;
    // the same split and tile-K rules dispatch applies
    int nsplit = d.nsplit < 1 ? 1 : d.nsplit;
    const int ktiles = (d.K + MM_BK - 1) / MM_BK;
    if (nsplit > ktiles) nsplit = ktiles;
    const int per = (ktiles + nsplit - 1) / nsplit;
    return mm_ok(d, per * MM_BK) ? 1 : 0;
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
}

template <int AL, int BL, int EP, int BM, int BN>
static void set_lds_mm() {
    (void)hipFuncSetAttribute((const void*)gemm_mm_kernel<AL, BL, EP, BM, BN>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)mm_lds_bytes<BM, BN>());
}

void gemm_setup() {
    {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            kGemmCUs = cus;
    }
    set_lds_mm<0, 0, EPI_BIAS_T, 128, 64>(); set_lds_mm<0, 0, EPI_BIAS_GELU, 128, 64>();
    set_lds_mm<0, 1, EPI_BIAS_T, 128, 64>(); set_lds_mm<0, 1, EPI_GELU_BWD, 128, 64>();
    set_lds_mm<0, 0, EPI_BIAS_T, 128, 192>(); set_lds_mm<0, 0, EPI_LOGITS, 128, 192>();
    set_lds_mm<0, 1, EPI_F32, 128, 192>(); set_lds_mm<0, 1, EPI_BIAS_T, 128, 192>();
    set_lds_mm<0, 0, EPI_BIAS_GELU, 128, 192>(); set_lds_mm<0, 1, EPI_GELU_BWD, 128, 192>();
    set_lds_mm<1, 1, EPI_PARTIAL, 128, 192>(); set_lds_mm<1, 1, EPI_F32, 128, 192>();
    (void)hipFuncSetAttribute((const void*)gemm_mm_kernel<1, 1, EPI_PARTIAL, 128, 192, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)mm_lds_bytes<128, 192>());
    (void)hipFuncSetAttribute((const void*)gemm_mm_kernel<1, 1, EPI_F32, 128, 192, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)mm_lds_bytes<128, 192>());
    (void)hipFuncSetAttribute((const void*)gemm_mm_kernel<1, 1, EPI_PARTIAL, 128, 128, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)mm_lds_bytes<128, 128>());
    (void)hipFuncSetAttribute((const void*)gemm_mm_kernel<1, 1, EPI_F32, 128, 128, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)mm_lds_bytes<128, 128>());
    (void)hipFuncSetAttribute((const void*)gemm_mm_group_kernel<192>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)mm_lds_bytes<128, 192>());
    (void)hipFuncSetAttribute((const void*)gemm_mm_group_kernel<128>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)mm_lds_bytes<128, 128>());
    set_lds_mm<0, 0, EPI_BIAS_T, 128, 128>();
    set_lds_mm<0, 0, EPI_BIAS_GELU, 128, 128>(); set_lds_mm<0, 1, EPI_GELU_BWD, 128, 128>();
    set_lds_mm<0, 1, EPI_F32, 128, 128>(); set_lds_mm<0, 1, EPI_BIAS_T, 128, 128>();
    set_lds_mm<0, 1, EPI_PARTIAL, 128, 128>(); set_lds_mm<1, 1, EPI_F32, 128, 128>();
    set_lds_mm<1, 1, EPI_PARTIAL, 128, 128>();
    // allow the dynamic LDS size (above the 64 KiB default) for every instantiation
#define SETUP_T(T)                                                                                          \
    set_lds_all<T, 0, 0, EPI_BIAS_T>();                                                                     \
    set_lds_all<T, 0, 0, EPI_BIAS_GELU>(); set_lds_all<T, 0, 1, EPI_GELU_BWD>();                           \
    set_lds_all<T, 0, 1, EPI_F32>(); set_lds_all<T, 0, 1, EPI_BIAS_T>(); set_lds_all<T, 1, 1, EPI_F32>(); \
    set_lds_all<T, 1, 1, EPI_PARTIAL>(); set_lds_all<T, 0, 1, EPI_PARTIAL>();
    SETUP_T(bf16)
    SETUP_T(float)
#undef SETUP_T
}

}  // namespace gpt2k
