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
// Tiling: 128x128 output tile per 256-thread workgroup (4 waves in 2x2, 64x64 per wave as
// 4x4 MFMA 16x16 blocks); K advances 128 bytes per tile step (64 bf16 / 32 fp32) through a
// double-buffered LDS stage padded by 16 bytes per row. Operands that are not k-contiguous
// are transposed in registers (8x8 bf16 / 4x4 fp32 blocks) on their way into LDS, so every
// LDS fragment read is one or two 16-byte reads. Workgroups are renumbered so that each of
// the 8 XCDs (one L2 each) works on a contiguous, M-grouped range of tiles.
#include "common.h"
#include "kernels.h"

namespace gpt2k {

constexpr int GBM = 128, GBN = 128, GTHREADS = 256;
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

// workgroup id -> (tile_m, tile_n): XCD-contiguous ranges, then groups of GROUP_M tile rows
DEV void tile_coords(int pid, int nwg, int num_m, int num_n, int& tm, int& tn) {
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

template <typename T, int LAYOUT>
struct TileLoader {
    // Loads a 128 x (128 bytes of K) tile of one operand into registers, then stores it to
    // LDS as [row][k] (row = m or n). LAYOUT 0: k-contiguous source, LAYOUT 1: row index
    // contiguous (transposed on the way).
    static constexpr int E = 16 / sizeof(T);        // elements per 16 bytes
    static constexpr int BK = 128 / sizeof(T);      // k elements per tile step
    static constexpr int NCHUNK = 128 * 8 / GTHREADS;  // k-contig: 16B chunks per thread (4)
    static constexpr int NBLK_TOTAL = (BK / E) * (128 / E);  // transposed: ExE blocks
    static constexpr int NBLK = (NBLK_TOTAL + GTHREADS - 1) / GTHREADS;
    uint4 r[LAYOUT == 0 ? NCHUNK : 8 * NBLK];

    DEV void load(const T* __restrict__ src, int64_t ld, int row0, int nrows, int k0, int kend, int tid) {
        if constexpr (LAYOUT == 0) {
#pragma unroll
            for (int i = 0; i < NCHUNK; ++i) {
                const int c = tid + i * GTHREADS;
                const int row = c >> 3, col = (c & 7) * E;
                const int gr = row0 + row, gk = k0 + col;
                if (gr < nrows && gk < kend)
                    r[i] = ld16(src + (int64_t)gr * ld + gk);
                else
                    r[i] = make_uint4(0, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int b = 0; b < NBLK; ++b) {
                const int blk = tid + b * GTHREADS;
                const int mb = blk % (128 / E), kb = blk / (128 / E);
                const int gm = row0 + mb * E;
#pragma unroll
                for (int q = 0; q < E; ++q) {
                    const int gk = k0 + kb * E + q;
                    if (blk < NBLK_TOTAL && gm < nrows && gk < kend)
                        r[b * 8 + q] = ld16(src + (int64_t)gk * ld + gm);
                    else
                        r[b * 8 + q] = make_uint4(0, 0, 0, 0);
                }
            }
        }
    }
    DEV void store(char* lds, int tid) {
        if constexpr (LAYOUT == 0) {
#pragma unroll
            for (int i = 0; i < NCHUNK; ++i) {
                const int c = tid + i * GTHREADS;
                const int row = c >> 3, colb = (c & 7) * 16;
                st16(lds + row * ROWB + colb, r[i]);
            }
        } else {
#pragma unroll
            for (int b = 0; b < NBLK; ++b) {
                const int blk = tid + b * GTHREADS;
                if (blk >= NBLK_TOTAL) continue;
                const int mb = blk % (128 / E), kb = blk / (128 / E);
                uint4 in[8], out[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) in[q] = r[b * 8 + q];
                transpose_block(in, out, (T*)nullptr);
#pragma unroll
                for (int j = 0; j < E; ++j) st16(lds + (mb * E + j) * ROWB + kb * 16, out[j]);
            }
        }
    }
};

template <typename T>
DEV typename FragT<T>::type load_frag(const char* lds, int row, int kstep, int lane) {
    // 8 consecutive k values of `row`, lane group (lane>>4) owns k sub-range within a
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

template <typename T, int ALAY, int BLAY, int EPI>
__global__ void __launch_bounds__(GTHREADS, 2) gemm_kernel(GemmArgs p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* sA = smem;
    char* sB = smem + 2 * GBM * ROWB;
    constexpr int BK = 128 / sizeof(T);
    constexpr int KSTEPS = BK / 32;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int num_m = (p.M + GBM - 1) / GBM, num_n = (p.N + GBN - 1) / GBN;
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, num_m, num_n, tm, tn);
    const int m0 = tm * GBM, n0 = tn * GBN;
    const int kbeg = blockIdx.y * p.ksplit_len;
    int kend = kbeg + p.ksplit_len;
    if (kend > p.K) kend = p.K;
    const int ntiles = (kend - kbeg + BK - 1) / BK;

    const T* A = (const T*)p.A;
    const T* B = (const T*)p.B;
    TileLoader<T, ALAY> la;
    TileLoader<T, BLAY> lb;

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    if (ntiles > 0) {
        la.load(A, p.lda, m0, p.M, kbeg, kend, tid);
        lb.load(B, p.ldb, n0, p.N, kbeg, kend, tid);
        la.store(sA, tid);
        lb.store(sB, tid);
    }
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < ntiles;
        if (more) {
            la.load(A, p.lda, m0, p.M, kbeg + (kt + 1) * BK, kend, tid);
            lb.load(B, p.ldb, n0, p.N, kbeg + (kt + 1) * BK, kend, tid);
        }
        const char* a_s = sA + cur * GBM * ROWB;
        const char* b_s = sB + cur * GBN * ROWB;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            typename FragT<T>::type af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = load_frag<T>(a_s, wm * 64 + i * 16 + (lane & 15), ks, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = load_frag<T>(b_s, wn * 64 + j * 16 + (lane & 15), ks, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) mma8(acc[i][j], af[i], bfr[j]);
        }
        if (more) {
            la.store(sA + (cur ^ 1) * GBM * ROWB, tid);
            lb.store(sB + (cur ^ 1) * GBN * ROWB, tid);
        }
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + j * 16 + (lane & 15);
        if (n >= p.N) continue;
        float bias = 0.f;
        if constexpr (EPI == EPI_BIAS_T || EPI == EPI_BIAS_RESID_F32 || EPI == EPI_BIAS_GELU)
            bias = p.bias ? p.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
                if (m >= p.M) continue;
                const float v = acc[i][j][r];
                if constexpr (EPI == EPI_BIAS_T) {
                    ((T*)p.C)[(int64_t)m * p.ldc + n] = from_f<T>(p.alpha * v + bias);
                } else if constexpr (EPI == EPI_BIAS_RESID_F32) {
                    ((float*)p.C)[(int64_t)m * p.ldc + n] = p.resid[(int64_t)m * p.ldr + n] + v + bias;
                } else if constexpr (EPI == EPI_BIAS_GELU) {
                    const T u = from_f<T>(v + bias);
                    ((T*)p.C)[(int64_t)m * p.ldc + n] = u;
                    ((T*)p.C2)[(int64_t)m * p.ldc + n] = from_f<T>(gelu_f(to_f<T>(u)));
                } else if constexpr (EPI == EPI_GELU_BWD) {
                    const float u = to_f<T>(((const T*)p.aux)[(int64_t)m * p.ldaux + n]);
                    ((T*)p.C)[(int64_t)m * p.ldc + n] = from_f<T>(v * gelu_grad_f(u));
                } else if constexpr (EPI == EPI_F32) {
                    float* o = (float*)p.C + (int64_t)m * p.ldc + n;
                    *o = p.beta ? *o + p.alpha * v : p.alpha * v;
                } else {  // EPI_PARTIAL
                    ((float*)p.C)[(int64_t)blockIdx.y * p.part_stride + (int64_t)m * p.ldc + n] = v;
                }
            }
        }
    }
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

size_t gemm_lds_bytes() { return 2 * (size_t)(GBM + GBN) * ROWB; }

template <typename T, int ALAY, int BLAY, int EPI>
static hipError_t launch(const GemmArgs& a, int nsplit, hipStream_t s) {
    const int num_m = (a.M + GBM - 1) / GBM, num_n = (a.N + GBN - 1) / GBN;
    dim3 grid(num_m * num_n, nsplit);
    gemm_kernel<T, ALAY, BLAY, EPI><<<grid, dim3(GTHREADS), gemm_lds_bytes(), s>>>(a);
    return hipGetLastError();
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
    hipError_t e = hipSuccess;
#define GEMM_CASE(AL, BL, EP) \
    if (d.a_layout == AL && d.b_layout == BL && epi == EP) e = launch<T, AL, BL, EP>(a, nsplit, s); else
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

void gemm_setup() {
    // allow the dynamic LDS size (above the 64 KiB default) for every instantiation
#define SETUP(T, AL, BL, EP) \
    (void)hipFuncSetAttribute((const void*)gemm_kernel<T, AL, BL, EP>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)gemm_lds_bytes());
#define SETUP_T(T) \
    SETUP(T, 0, 0, EPI_BIAS_T) SETUP(T, 0, 0, EPI_BIAS_RESID_F32) SETUP(T, 0, 0, EPI_BIAS_GELU) \
    SETUP(T, 0, 1, EPI_GELU_BWD) SETUP(T, 0, 1, EPI_F32) SETUP(T, 0, 1, EPI_BIAS_T) \
    SETUP(T, 1, 1, EPI_F32) SETUP(T, 1, 1, EPI_PARTIAL) SETUP(T, 0, 1, EPI_PARTIAL)
    SETUP_T(bf16)
    SETUP_T(float)
#undef SETUP_T
#undef SETUP
}

}  // namespace gpt2k
