// Causal multi-head attention of the GPT-2 step, flash style (gfx950 MFMA).
//
// Per sequence b and head h: S = q k^T / sqrt(hs), future positions masked, P = softmax(S)
// row-wise, y = P v ("Code you'll write": F.scaled_dot_product_attention(q, k, v,
// is_causal=True) with the default scale). The T x T matrix never leaves the chip: keys and
// values stream through LDS in 64-row tiles and the softmax is kept online (running max and
// running sum, rescaling the partial output; chapter 2:00:19-2:06:39 describes the method).
// The forward stores the row log-sum-exp; the backward recomputes P from it.
//
// Layouts: qkv [B*T, 3C] with q | k | v and head h in columns h*hs..h*hs+hs of each third
// (the split/view of the attention excerpt, read in place: no transpose kernel); y, dy
// [B*T, C]; lse [B, H, T] fp32.
//
// MFMA data flow. A wave computes S^T = K Q^T: its 16x16 accumulator gives lane l the
// column query (l & 15) and the rows key 4*(l>>4)+i. That is exactly a B-operand fragment
// of a product that sums over keys, so O^T = V^T P^T takes P straight from registers, with
// the V^T fragment read in the matching key order from a transposed LDS copy of V. The
// backward uses the same device: dK/dV per key block (S = Q K^T so P sums over queries),
// and dQ per query block (S^T again) -- two kernels instead of atomics, so dQ is
// deterministic.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gpt2k {

constexpr int A_THREADS = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Workgroups are dealt to the 8 XCDs round-robin by linear id. Renumber the 2-D grid
// (x = block along the sequence, y = b*H + h) so that every block of one (b, h) lands on the
// same XCD and its K/V (or Q/dO) tiles are served from that XCD's L2.
DEV void xcd_remap(int& bx, int& by) {
    const int nx = gridDim.x, n = nx * gridDim.y;
    const int pid = blockIdx.y * nx + blockIdx.x;
    const int xcd = pid & 7, slot = pid >> 3;
    const int per = (n + 7) >> 3;
    int tall = n & 7;
    if (tall == 0) tall = 8;
    const int logical = (xcd < tall) ? xcd * per + slot : tall * per + (xcd - tall) * (per - 1) + slot;
    by = logical / nx;
    bx = logical % nx;
}

template <typename T, int COLS>
struct Tile {  // LDS tile of up to 64 rows x COLS elements, rows padded by 16 bytes
    static constexpr int STRIDE = COLS * (int)sizeof(T) + 16;
    static constexpr int BYTES = 64 * STRIDE;
};

// 8 consecutive elements (k sub-range of lane group g within a 32-wide k step)
template <typename T>
DEV typename FragT<T>::type frag_nat(const char* base, int stride, int row, int ks, int lane) {
    const char* p = base + row * stride + (ks * 32 + (lane >> 4) * 8) * (int)sizeof(T);
    if constexpr (sizeof(T) == 2) return __builtin_bit_cast(bf16x8, ld16(p));
    else return frag_from_halves(*(const float4*)p, *(const float4*)(p + 16));
}
// elements {32s + 4g + 0..3} and {32s + 16 + 4g + 0..3}: the key/query order of a fragment
// built from two 16x16 accumulator blocks
template <typename T>
DEV typename FragT<T>::type frag_perm(const char* base, int stride, int row, int s, int lane) {
    const int g = lane >> 4;
    const char* p1 = base + row * stride + (s * 32 + 4 * g) * (int)sizeof(T);
    const char* p2 = p1 + 16 * (int)sizeof(T);
    if constexpr (sizeof(T) == 2) return frag_from_halves(*(const uint2*)p1, *(const uint2*)p2);
    else return frag_from_halves(*(const float4*)p1, *(const float4*)p2);
}
template <typename T>
DEV typename FragT<T>::type frag_global(const T* p) {
    if constexpr (sizeof(T) == 2) return __builtin_bit_cast(bf16x8, ld16(p));
    else return frag_from_halves(*(const float4*)p, *(const float4*)(p + 4));
}
template <typename T>
DEV typename FragT<T>::type frag_zero() {
    typename FragT<T>::type f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = from_f<T>(0.f);
    return f;
}
// fragment from two accumulators: values 0..3 from a, 4..7 from b
template <typename T>
DEV typename FragT<T>::type frag_from_acc(const floatx4& a, const floatx4& b) {
    typename FragT<T>::type f;
#pragma unroll
    for (int j = 0; j < 4; ++j) { f[j] = from_f<T>(a[j]); f[4 + j] = from_f<T>(b[j]); }
    return f;
}
template <typename T>
DEV void store4v(T* p, const floatx4& v, float s) {
    if constexpr (sizeof(T) == 2) {
        bf16x4 o;
        o[0] = (bf16)(v[0] * s); o[1] = (bf16)(v[1] * s); o[2] = (bf16)(v[2] * s); o[3] = (bf16)(v[3] * s);
        *(bf16x4*)p = o;
    } else {
        *(float4*)p = make_float4(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
    }
}

// Stage `rows64` rows (64 max) x HS columns of a strided source into LDS, natural and/or
// transposed. Rows >= nvalid are zero. Natural: dst[r][c]. Transposed: dstT[c][r].
template <typename T, int HS>
DEV void stage_rows(const T* __restrict__ src, int64_t ld, int nvalid, char* nat, char* trn, int tid) {
    constexpr int E = 16 / sizeof(T);
    using TN = Tile<T, HS>;
    using TT = Tile<T, 64>;
    if (trn == nullptr) {
        constexpr int CPR = HS / E;  // 16-byte chunks per row
        for (int c = tid; c < 64 * CPR; c += A_THREADS) {
            const int r = c / CPR, cc = c % CPR;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (r < nvalid) v = ld16(src + (int64_t)r * ld + cc * E);
            st16(nat + r * TN::STRIDE + cc * 16, v);
        }
    } else {
        // the row block varies fastest across lanes: 8 lanes then fill one 128-byte row of
        // the transposed tile, so those stores are free of bank conflicts. There are at most
        // 256 blocks (64 rows x HS columns), one per thread.
        constexpr int RBN = 64 / E, NB = RBN * (HS / E);
        static_assert(NB <= A_THREADS, "one block per thread");
        // (bf16 with 32-wide heads, used only by small test models, keeps the column-fastest
        // order: hipcc 7.2 crashes on the other order for that instantiation)
        constexpr bool row_fast = !(sizeof(T) == 2 && HS == 32);
        if (tid < NB) {
            const int rb = row_fast ? tid % RBN : tid / (HS / E);
            const int cb = row_fast ? tid / RBN : tid % (HS / E);
            uint4 in[8], out[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int r = rb * E + q;
                in[q] = (q < E && r < nvalid) ? ld16(src + (int64_t)r * ld + cb * E) : make_uint4(0, 0, 0, 0);
            }
            if (nat) {
#pragma unroll
                for (int q = 0; q < E; ++q) st16(nat + (rb * E + q) * TN::STRIDE + cb * 16, in[q]);
            }
            transpose_block(in, out, (T*)nullptr);
#pragma unroll
            for (int j = 0; j < E; ++j) st16(trn + (cb * E + j) * TT::STRIDE + rb * 16, out[j]);
        }
    }
}

// ================================================================== forward
template <typename T, int HS>
__global__ void __launch_bounds__(A_THREADS) attn_fwd_kernel(const T* __restrict__ qkv, T* __restrict__ y,
                                                             float* __restrict__ lse, int T_, int H, float sc) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    using TK = Tile<T, HS>;
    using TV = Tile<T, 64>;
    char* sK = smem;
    char* sVt = smem + TK::BYTES;
    constexpr int KS = HS / 32, DB = HS / 16;

    int bx, by;
    xcd_remap(bx, by);
    const int nqb = (T_ + 127) / 128;
    const int qblk = nqb - 1 - bx;  // longest blocks first
    const int bh = by, b = bh / H, h = bh % H;
    const int C = H * HS;
    const int64_t ld = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * T_ * ld;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q0 = qblk * 128, qw0 = q0 + wave * 32;
    const int col = lane & 15, g = lane >> 4;

    typename FragT<T>::type qf[2][KS];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int q = qw0 + qb * 16 + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[qb][ks] = q < T_ ? frag_global<T>(base + (int64_t)q * ld + h * HS + ks * 32 + g * 8) : frag_zero<T>();
    }
    floatx4 o[DB][2];
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d][0] = o[d][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};

    int kend = q0 + 128 < T_ ? q0 + 128 : T_;
    const int nchunk = (kend + 63) / 64;
    const bool wave_live = qw0 < T_;
    for (int c = 0; c < nchunk; ++c) {
        const int k0 = c * 64;
        const int nvalid = T_ - k0 < 64 ? T_ - k0 : 64;
        __syncthreads();
        stage_rows<T, HS>(base + (int64_t)k0 * ld + C + h * HS, ld, nvalid, sK, nullptr, tid);
        stage_rows<T, HS>(base + (int64_t)k0 * ld + 2 * C + h * HS, ld, nvalid, nullptr, sVt, tid);
        __syncthreads();
        if (!wave_live || k0 > qw0 + 31) continue;
        floatx4 s[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            s[kb][0] = s[kb][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const auto kf = frag_nat<T>(sK, TK::STRIDE, kb * 16 + col, ks, lane);
                mma8(s[kb][0], kf, qf[0][ks]);
                mma8(s[kb][1], kf, qf[1][ks]);
            }
        }
        const bool need_mask = (k0 + 63 > qw0) || (k0 + 64 > T_);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int q = qw0 + qb * 16 + col;
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = s[kb][qb][i] * sc;
                    if (need_mask) {
                        const int key = k0 + kb * 16 + g * 4 + i;
                        if (key > q || key >= T_) v = -INFINITY;
                    }
                    s[kb][qb][i] = v;
                    mx = fmaxf(mx, v);
                }
            mx = group4_max(mx);
            const float mnew = fmaxf(mrun[qb], mx);
            const float alpha = mrun[qb] == -INFINITY ? 0.f : exp2f(mrun[qb] - mnew);
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = s[kb][qb][i] == -INFINITY ? 0.f : exp2f(s[kb][qb][i] - mnew);
                    s[kb][qb][i] = p;
                    ls += p;
                }
            lrun[qb] = lrun[qb] * alpha + ls;
            mrun[qb] = mnew;
#pragma unroll
            for (int d = 0; d < DB; ++d) o[d][qb] *= alpha;
        }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const auto p0 = frag_from_acc<T>(s[2 * st][0], s[2 * st + 1][0]);
            const auto p1 = frag_from_acc<T>(s[2 * st][1], s[2 * st + 1][1]);
#pragma unroll
            for (int d = 0; d < DB; ++d) {
                const auto vf = frag_perm<T>(sVt, TV::STRIDE, d * 16 + col, st, lane);
                mma8(o[d][0], vf, p0);
                mma8(o[d][1], vf, p1);
            }
        }
    }
    if (!wave_live) return;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int q = qw0 + qb * 16 + col;
        const float ltot = group4_sum(lrun[qb]);
        if (q >= T_) continue;
        const float inv = 1.0f / ltot;
        T* yr = y + ((int64_t)b * T_ + q) * C + h * HS;
#pragma unroll
        for (int d = 0; d < DB; ++d) store4v<T>(yr + d * 16 + g * 4, o[d][qb], inv);
        if (g == 0) lse[(int64_t)bh * T_ + q] = (mrun[qb] + log2f(ltot)) * kLn2;
    }
}

// ================================================================== backward
// D[b,h,t] = sum_d dy * y (row sums of dO o O, the softmax-gradient correction term)
template <typename T, int HS>
__global__ void attn_bwd_pre_kernel(const T* __restrict__ y, const T* __restrict__ dy, float* __restrict__ D,
                                    int BT, int T_, int H) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over BT*H
    if (i >= (int64_t)BT * H) return;
    const int row = (int)(i / H), h = (int)(i % H);
    const int C = H * HS;
    const T* a = y + (int64_t)row * C + h * HS;
    const T* b = dy + (int64_t)row * C + h * HS;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < HS; ++d) s += to_f<T>(a[d]) * to_f<T>(b[d]);
    const int bb = row / T_, t = row % T_;
    D[((int64_t)bb * H + h) * T_ + t] = s;
}

// dK, dV for 128 keys per workgroup (32 per wave), looping over 64-query chunks.
template <typename T, int HS>
__global__ void __launch_bounds__(A_THREADS) attn_bwd_dkv_kernel(const T* __restrict__ qkv, const T* __restrict__ dy,
                                                                 const float* __restrict__ lse,
                                                                 const float* __restrict__ D, T* __restrict__ dqkv,
                                                                 int T_, int H, float sc, float scale) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    using TN = Tile<T, HS>;
    using TT = Tile<T, 64>;
    char* sQ = smem;
    char* sQt = sQ + TN::BYTES;
    char* sO = sQt + TT::BYTES;     // dO natural
    char* sOt = sO + TN::BYTES;     // dO transposed
    float* sL = (float*)(sOt + TT::BYTES);
    float* sD = sL + 64;
    constexpr int KS = HS / 32, DB = HS / 16;

    int bx, by;
    xcd_remap(bx, by);
    const int kblk = bx;  // early key blocks see the most queries: launch them first
    const int bh = by, b = bh / H, h = bh % H;
    const int C = H * HS;
    const int64_t ld = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * T_ * ld;
    const T* dyb = dy + (int64_t)b * T_ * C;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int k0 = kblk * 128, kw0 = k0 + wave * 32;

    typename FragT<T>::type kf[2][KS], vf[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int key = kw0 + kb * 16 + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int64_t off = (int64_t)key * ld + h * HS + ks * 32 + g * 8;
            kf[kb][ks] = key < T_ ? frag_global<T>(base + off + C) : frag_zero<T>();
            vf[kb][ks] = key < T_ ? frag_global<T>(base + off + 2 * C) : frag_zero<T>();
        }
    }
    floatx4 dk[DB][2], dv[DB][2];
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dk[d][kb] = dv[d][kb] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int nqc = (T_ + 63) / 64;
    const bool wave_live = kw0 < T_;
    for (int qc = k0 / 64; qc < nqc; ++qc) {
        const int q0 = qc * 64;
        const int nvalid = T_ - q0 < 64 ? T_ - q0 : 64;
        __syncthreads();
        stage_rows<T, HS>(base + (int64_t)q0 * ld + h * HS, ld, nvalid, sQ, sQt, tid);
        stage_rows<T, HS>(dyb + (int64_t)q0 * C + h * HS, C, nvalid, sO, sOt, tid);
        if (tid < 64) {
            const bool ok = tid < nvalid;
            sL[tid] = ok ? lse[(int64_t)bh * T_ + q0 + tid] * kLog2e : 0.f;
            sD[tid] = ok ? D[(int64_t)bh * T_ + q0 + tid] : 0.f;
        }
        __syncthreads();
        if (!wave_live || q0 + 63 < kw0) continue;
        floatx4 s[4][2], dp[4][2];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[qb][kb] = dp[qb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const auto qa = frag_nat<T>(sQ, TN::STRIDE, qb * 16 + col, ks, lane);
                const auto oa = frag_nat<T>(sO, TN::STRIDE, qb * 16 + col, ks, lane);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    mma8(s[qb][kb], qa, kf[kb][ks]);
                    mma8(dp[qb][kb], oa, vf[kb][ks]);
                }
            }
        }
        // P and dS; rows q = q0 + 16qb + 4g + i, column key = kw0 + 16kb + col
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ql = qb * 16 + g * 4 + i;
                const int q = q0 + ql;
                const float L = sL[ql], Dq = sD[ql];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int key = kw0 + kb * 16 + col;
                    const float p = (key <= q && q < T_) ? exp2f(s[qb][kb][i] * sc - L) : 0.f;
                    s[qb][kb][i] = p;
                    dp[qb][kb][i] = p * (dp[qb][kb][i] - Dq);
                }
            }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            typename FragT<T>::type pf[2], df[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                pf[kb] = frag_from_acc<T>(s[2 * st][kb], s[2 * st + 1][kb]);
                df[kb] = frag_from_acc<T>(dp[2 * st][kb], dp[2 * st + 1][kb]);
            }
#pragma unroll
            for (int d = 0; d < DB; ++d) {
                const auto oat = frag_perm<T>(sOt, TT::STRIDE, d * 16 + col, st, lane);
                const auto qat = frag_perm<T>(sQt, TT::STRIDE, d * 16 + col, st, lane);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    mma8(dv[d][kb], oat, pf[kb]);
                    mma8(dk[d][kb], qat, df[kb]);
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
    }
    if (!wave_live) return;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int key = kw0 + kb * 16 + col;
        if (key >= T_) continue;
        T* r = dqkv + ((int64_t)b * T_ + key) * ld + h * HS;
#pragma unroll
        for (int d = 0; d < DB; ++d) {
            store4v<T>(r + C + d * 16 + g * 4, dk[d][kb], scale);
            store4v<T>(r + 2 * C + d * 16 + g * 4, dv[d][kb], 1.0f);
        }
    }
}

// dQ for 128 queries per workgroup (32 per wave), looping over 64-key chunks.
template <typename T, int HS>
__global__ void __launch_bounds__(A_THREADS) attn_bwd_dq_kernel(const T* __restrict__ qkv, const T* __restrict__ dy,
                                                                const float* __restrict__ lse,
                                                                const float* __restrict__ D, T* __restrict__ dqkv,
                                                                int T_, int H, float sc, float scale) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    using TN = Tile<T, HS>;
    using TT = Tile<T, 64>;
    char* sK = smem;
    char* sKt = sK + TN::BYTES;
    char* sV = sKt + TT::BYTES;
    constexpr int KS = HS / 32, DB = HS / 16;

    int bx, by;
    xcd_remap(bx, by);
    const int nqb = (T_ + 127) / 128;
    const int qblk = nqb - 1 - bx;
    const int bh = by, b = bh / H, h = bh % H;
    const int C = H * HS;
    const int64_t ld = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * T_ * ld;
    const T* dyb = dy + (int64_t)b * T_ * C;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int q0 = qblk * 128, qw0 = q0 + wave * 32;

    typename FragT<T>::type qf[2][KS], of[2][KS];
    float L[2], Dq[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int q = qw0 + qb * 16 + col;
        const bool ok = q < T_;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[qb][ks] = ok ? frag_global<T>(base + (int64_t)q * ld + h * HS + ks * 32 + g * 8) : frag_zero<T>();
            of[qb][ks] = ok ? frag_global<T>(dyb + (int64_t)q * C + h * HS + ks * 32 + g * 8) : frag_zero<T>();
        }
        L[qb] = ok ? lse[(int64_t)bh * T_ + q] * kLog2e : 0.f;
        Dq[qb] = ok ? D[(int64_t)bh * T_ + q] : 0.f;
    }
    floatx4 dq[DB][2];
#pragma unroll
    for (int d = 0; d < DB; ++d) dq[d][0] = dq[d][1] = floatx4{0.f, 0.f, 0.f, 0.f};

    int kend = q0 + 128 < T_ ? q0 + 128 : T_;
    const int nchunk = (kend + 63) / 64;
    const bool wave_live = qw0 < T_;
    for (int c = 0; c < nchunk; ++c) {
        const int k0 = c * 64;
        const int nvalid = T_ - k0 < 64 ? T_ - k0 : 64;
        __syncthreads();
        stage_rows<T, HS>(base + (int64_t)k0 * ld + C + h * HS, ld, nvalid, sK, sKt, tid);
        stage_rows<T, HS>(base + (int64_t)k0 * ld + 2 * C + h * HS, ld, nvalid, sV, nullptr, tid);
        __syncthreads();
        if (!wave_live || k0 > qw0 + 31) continue;
        floatx4 s[4][2], dp[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            s[kb][0] = s[kb][1] = dp[kb][0] = dp[kb][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const auto ka = frag_nat<T>(sK, TN::STRIDE, kb * 16 + col, ks, lane);
                const auto va = frag_nat<T>(sV, TN::STRIDE, kb * 16 + col, ks, lane);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    mma8(s[kb][qb], ka, qf[qb][ks]);
                    mma8(dp[kb][qb], va, of[qb][ks]);
                }
            }
        }
        // rows key = k0 + 16kb + 4g + i, column q = qw0 + 16qb + col
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int q = qw0 + qb * 16 + col;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = k0 + kb * 16 + g * 4 + i;
                    const float p = (key <= q && key < T_) ? exp2f(s[kb][qb][i] * sc - L[qb]) : 0.f;
                    dp[kb][qb][i] = p * (dp[kb][qb][i] - Dq[qb]);
                }
            }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const auto d0 = frag_from_acc<T>(dp[2 * st][0], dp[2 * st + 1][0]);
            const auto d1 = frag_from_acc<T>(dp[2 * st][1], dp[2 * st + 1][1]);
#pragma unroll
            for (int d = 0; d < DB; ++d) {
                const auto kat = frag_perm<T>(sKt, TT::STRIDE, d * 16 + col, st, lane);
                mma8(dq[d][0], kat, d0);
                mma8(dq[d][1], kat, d1);
            }
        }
    }
    if (!wave_live) return;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int q = qw0 + qb * 16 + col;
        if (q >= T_) continue;
        T* r = dqkv + ((int64_t)b * T_ + q) * ld + h * HS;
#pragma unroll
        for (int d = 0; d < DB; ++d) store4v<T>(r + d * 16 + g * 4, dq[d][qb], scale);
    }
}

// ================================================================== bf16, 64-wide heads
// Streamed tiles: each 64-row x 64-column bf16 tile (128-byte rows) of K, V, Q or dO goes
// from its strided rows in global memory straight into LDS by direct loads, two stages
// deep, so the next chunk's tiles are in flight while the current chunk is multiplied.
// Fragments whose k index runs along the tile's rows (V^T, Q^T, dO^T, K^T) come from the
// transposing LDS read; its row choice per 16-lane group also produces the key/query order
// of a fragment built from two 16x16 accumulator blocks, so no tile is ever transposed.
// The 16-byte chunk c of row r sits in slot c ^ ts_swz(r): row bits 1, 2, 3 flip the slot
// by 3, 4, 6. That keeps both reads free of bank conflicts, the 16-byte row reads (16 rows x
// 4 chunks per instruction) and the transposing 8-byte reads (8 rows x 2 chunks per
// half-wave): a probe of the two read patterns reads 0 conflict cycles for both, where a
// swizzle of row bits 1..3 into slot bits 1, 2, 0 left half of the 16-byte reads' cycles in
// conflicts (and the GEMM's (r >> 1) & 7 half of the transposing reads').
constexpr int TS_BYTES = 64 * 128;

DEV int ts_swz(int r) { return (-((r >> 1) & 1) & 3) ^ (-((r >> 2) & 1) & 4) ^ (-((r >> 3) & 1) & 6); }

// Byte offsets of this wave's share (rows 16w..16w+15) of a 64-row tile whose row r starts at
// src + r*ld; rows >= nrows repeat the last valid row (finite values, masked out by the
// callers). They depend only on nrows, so kernels compute the full-tile set once.
struct TsOff {
    uint32_t o[2];
};
DEV TsOff ts_offsets(int64_t ld, int nrows, int wave, int lane) {
    TsOff t;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 16 * wave + 8 * i + (lane >> 3);
        const int c = (lane & 7) ^ ts_swz(r);
        const int rr = min(r, nrows - 1);
        t.o[i] = (uint32_t)(rr * ld * 2 + c * 16);
    }
    return t;
}
DEV void ts_issue(const bf16* src, const TsOff& off, uint32_t lds, int wave) {
    dma16(src, off.o[0], lds + (2 * wave) * 1024);
    dma16(src, off.o[1], lds + (2 * wave + 1) * 1024);
}
// the tile of nrows valid rows: the precomputed full-tile offsets unless the tile is ragged
DEV void ts_load(const bf16* src, int64_t ld, int nrows, const TsOff& full, uint32_t lds, int wave, int lane) {
    if (nrows == 64) ts_issue(src, full, lds, wave);
    else ts_issue(src, ts_offsets(ld, nrows, wave, lane), lds, wave);
}
// rows rb..rb+15 (lane & 15), k = 32ks + 8(lane >> 4) + 0..7 along the row
DEV bf16x8 ts_nat(const char* t, int rb, int ks, int lane) {
    const int r = rb + (lane & 15), c = ks * 4 + (lane >> 4);
    return __builtin_bit_cast(bf16x8, ld16(t + r * 128 + ((c ^ ts_swz(r)) << 4)));
}
// column cb + (lane & 15); values 0..3 from rows r0 + 4(lane >> 4) + j, 4..7 from rows
// r1 + 4(lane >> 4) + j
DEV bf16x8 ts_tr(const char* t, int cb, int r0, int r1, int lane) {
    const int g = lane >> 4, q = lane & 15;
    const int colx = cb + 4 * (q & 3), ch = colx >> 3, within = (colx & 7) * 2;
    const int ra = r0 + 4 * g + (q >> 2), rb = r1 + 4 * g + (q >> 2);
    return read_tr_pair(t + ra * 128 + ((ch ^ ts_swz(ra)) << 4) + within,
                        t + rb * 128 + ((ch ^ ts_swz(rb)) << 4) + within);
}
DEV float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32: exp2(-inf) = 0

// A fragment times a scalar, rounded back to bf16. The kernels below fold the score scale
// log2(e)/sqrt(hs) into the operand they keep in registers (one more bf16 rounding of it), and
// start each score accumulator at minus the offset the exponential needs (the running maximum,
// or the base-2 log-sum-exp in the backward), so that the product itself gives the argument
// of exp2 and the softmax needs no multiply-add per score.
DEV bf16x8 frag_scaled(const bf16x8& f, float s) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)((float)f[e] * s);
    return r;
}
DEV floatx4 splat4(float v) { return floatx4{v, v, v, v}; }

// QB blocks of 16 queries per wave: 4 waves cover 64 * QB queries of one (batch, head)
template <int QB>
__global__ void __launch_bounds__(A_THREADS, QB <= 2 ? 3 : 2) attn_fwd_ts_kernel(const bf16* __restrict__ qkv,
                                                                                 bf16* __restrict__ y,
                                                                                 float* __restrict__ lse, int T_, int H,
                                                                                 float sc) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];  // [stage][K | V]
    constexpr int HS = 64, STAGE = 2 * TS_BYTES;
    int bx, by;
    xcd_remap(bx, by);
    constexpr int QW = 16 * QB, QBLK = 4 * QW;  // queries per wave, per workgroup
    const int nqb = (T_ + QBLK - 1) / QBLK;
    const int qblk = nqb - 1 - bx;  // longest blocks first
    const int bh = by, b = bh / H, h = bh % H;
    const int C = H * HS;
    const int64_t ld = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T_ * ld;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q0 = qblk * QBLK, qw0 = q0 + wave * QW;
    const int col = lane & 15, g = lane >> 4;
    const uint32_t lds0 = lds_addr(smem);

    bf16x8 qf[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int q = qw0 + qb * 16 + col;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            qf[qb][ks] = q < T_ ? frag_scaled(frag_global<bf16>(base + (int64_t)q * ld + h * HS + ks * 32 + g * 8), sc)
                                : frag_zero<bf16>();
    }
    // o: the output rows, unnormalized; lacc: the softmax denominators, accumulated by the
    // same products as o with a fragment of ones in place of V^T (every entry of lacc[qb] is
    // then the sum over the keys so far of query column (lane & 15)); mref: the reference
    // maxima (base 2) the exponentials are taken against; moff: the same, 0 while still
    // -inf, the value the score accumulators start from (negated)
    floatx4 o[4][QB], lacc[QB];
    float mref[QB], moff[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
        lacc[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
        mref[qb] = -INFINITY;
        moff[qb] = 0.f;
    }
    const bf16x8 ones = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};

    const int kend = min(q0 + QBLK, T_);
    const int nchunk = (kend + 63) / 64;
    const bool wave_live = qw0 < T_;
    const TsOff offkv = ts_offsets(ld, 64, wave, lane);
    auto issue = [&](int c) {
        const int k0 = c * 64, nv = min(64, T_ - k0);
        const uint32_t st = lds0 + (c & 1) * STAGE;
        ts_load(base + (int64_t)k0 * ld + C + h * HS, ld, nv, offkv, st, wave, lane);
        ts_load(base + (int64_t)k0 * ld + 2 * C + h * HS, ld, nv, offkv, st + TS_BYTES, wave, lane);
    };
    if (nchunk > 0) issue(0);
    for (int c = 0; c < nchunk; ++c) {
        dma_wait_barrier();
        if (c + 1 < nchunk) issue(c + 1);
        const int k0 = c * 64;
        // With one 16-query block per wave every wave needs every chunk up to the diagonal; a
        // wave past the sequence end computes on zero queries and stores nothing. Skipping it
        // here would make the compiler copy the accumulators on every iteration.
        if constexpr (QB > 1) {
            if (!wave_live || k0 > qw0 + QW - 1) continue;
        }
        const char* sK = smem + (c & 1) * STAGE;
        const char* sV = sK + TS_BYTES;
        // Every fragment of the chunk is read before it is needed: the V^T reads complete under
        // the score products and the softmax instead of stalling each output product in turn.
        // (Two of them go out with the K reads, the rest after the score products: the LDS
        // wait counter tracks at most 15 reads in flight, and the products wait only for K.)
        bf16x8 kf[4][2], vf[2][4];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) kf[kb][ks] = ts_nat(sK, kb * 16, ks, lane);
#pragma unroll
        for (int d = 0; d < 2; ++d) vf[0][d] = ts_tr(sV, d * 16, 0, 16, lane);
        floatx4 s[4][QB];
        __builtin_amdgcn_s_setprio(1);  // MFMA phase first; other waves run their softmax meanwhile
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb] = splat4(-moff[qb]);
        // k step outermost, so that the two products into one accumulator are four apart
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) mma8(s[kb][qb], kf[kb][ks], qf[qb][ks]);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int d = 2; d < 4; ++d) vf[0][d] = ts_tr(sV, d * 16, 0, 16, lane);
#pragma unroll
        for (int d = 0; d < 4; ++d) vf[1][d] = ts_tr(sV, d * 16, 32, 48, lane);
        // online softmax in the log2 domain: s holds scale * score - moff; max first, then one
        // exp2 per score; the causal and sequence-end mask only in the chunks that reach the
        // diagonal or the end (one wave-uniform branch around selects)
        if ((k0 + 63 > qw0) || (k0 + 64 > T_)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int lim = min(qw0 + qb * 16 + col, T_ - 1) - k0 - g * 4;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        s[kb][qb][i] = kb * 16 + i > lim ? -INFINITY : s[kb][qb][i];
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][qb][i]);
            mx = group4_max_swap(mx) + moff[qb];
            // Lazy rescaling: the reference maximum moves (and o and the denominators are
            // rescaled) only when some query of the wave has a score more than 2^8 above it,
            // so the exponentials stay <= 256 and the normalization o / l, which shares the
            // reference, is unchanged. The first chunk always sets it (mref = -inf).
            if (__builtin_amdgcn_ballot_w64(mx > mref[qb] + 8.f)) {
                const float mnew = fmaxf(mref[qb], mx);
                const float msafe = mnew == -INFINITY ? 0.f : mnew;
                const float alpha = exp2_raw(mref[qb] - msafe);
#pragma unroll
                for (int d = 0; d < 4; ++d) o[d][qb] *= alpha;
                lacc[qb] *= alpha;
                const float shift = msafe - moff[qb];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) s[kb][qb] -= shift;
                mref[qb] = mnew;
                moff[qb] = msafe;
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[kb][qb][i] = exp2_raw(s[kb][qb][i]);
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            bf16x8 pf[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                pf[qb] = frag_from_acc<bf16>(s[2 * st][qb], s[2 * st + 1][qb]);
                mma8(lacc[qb], ones, pf[qb]);
            }
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) mma8(o[d][qb], vf[st][d], pf[qb]);
        }
        __builtin_amdgcn_s_setprio(0);
    }
    if (!wave_live) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int q = qw0 + qb * 16 + col;
        const float ltot = lacc[qb][0];
        if (q >= T_) continue;
        const float inv = 1.0f / ltot;
        bf16* yr = y + ((int64_t)b * T_ + q) * C + h * HS;
#pragma unroll
        for (int d = 0; d < 4; ++d) store4v<bf16>(yr + d * 16 + g * 4, o[d][qb], inv);
        if (g == 0) lse[(int64_t)bh * T_ + q] = (mref[qb] + log2f(ltot)) * kLn2;
    }
}

// dK, dV for 64 * KBW keys per workgroup (16 * KBW per wave), streaming 64-query chunks of Q, dO,
// -lse, -D.
template <int KBW>
__global__ void __launch_bounds__(A_THREADS, KBW == 1 ? 3 : 2) attn_bwd_dkv_ts_kernel(const bf16* __restrict__ qkv,
                                                                    const bf16* __restrict__ dy,
                                                                    const float* __restrict__ neg_lse2,
                                                                    const float* __restrict__ neg_D,
                                                                    bf16* __restrict__ dqkv, int T_, int H, float sc,
                                                                    float scale) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];  // [stage][Q | dO | lse | D]
    constexpr int HS = 64, STAGE = 2 * TS_BYTES + 512;
    int bx, by;
    xcd_remap(bx, by);
    const int kblk = bx;  // early key blocks see the most queries: launch them first
    const int bh = by, b = bh / H, h = bh % H;
    const int C = H * HS;
    const int64_t ld = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T_ * ld;
    const bf16* dyb = dy + (int64_t)b * T_ * C;
    const float* lse_bh = neg_lse2 + (int64_t)bh * T_;   // minus the base-2 log-sum-exp
    const float* D_bh = neg_D + (int64_t)bh * T_;         // minus D
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4;
    constexpr int KW = 16 * KBW, KBLK = 4 * KW;   // keys per wave, per workgroup
    const int k0 = kblk * KBLK, kw0 = k0 + wave * KW;
    const uint32_t lds0 = lds_addr(smem);

    bf16x8 kf[KBW][2], vf[KBW][2];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
        const int key = kw0 + kb * 16 + col;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int64_t off = (int64_t)key * ld + h * HS + ks * 32 + g * 8;
            kf[kb][ks] = key < T_ ? frag_scaled(frag_global<bf16>(base + off + C), sc) : frag_zero<bf16>();
            vf[kb][ks] = key < T_ ? frag_global<bf16>(base + off + 2 * C) : frag_zero<bf16>();
        }
    }
    floatx4 dk[4][KBW], dv[4][KBW];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) dk[d][kb] = dv[d][kb] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int qc0 = k0 / 64, nqc = (T_ + 63) / 64;
    const bool wave_live = kw0 < T_;
    const TsOff offq = ts_offsets(ld, 64, wave, lane), offo = ts_offsets(C, 64, wave, lane);
    auto issue = [&](int qc) {
        const int q0 = qc * 64, nv = min(64, T_ - q0);
        const uint32_t st = lds0 + ((qc - qc0) & 1) * STAGE;
        ts_load(base + (int64_t)q0 * ld + h * HS, ld, nv, offq, st, wave, lane);
        ts_load(dyb + (int64_t)q0 * C + h * HS, C, nv, offo, st + TS_BYTES, wave, lane);
        const uint32_t voff = (uint32_t)min(lane, nv - 1) * 4;
        if (wave == 0) dma4(lse_bh + q0, voff, st + 2 * TS_BYTES);
        if (wave == 1) dma4(D_bh + q0, voff, st + 2 * TS_BYTES + 256);
    };
    if (qc0 < nqc) issue(qc0);
    for (int qc = qc0; qc < nqc; ++qc) {
        dma_wait_barrier();
        if (qc + 1 < nqc) issue(qc + 1);
        const int q0 = qc * 64;
        // as in the forward: with one 16-key block per wave no wave skips a chunk except past
        // the sequence end, where it computes masked zeros and stores nothing
        if constexpr (KBW > 1) {
            if (!wave_live || q0 + 63 < kw0) continue;
        }
        const char* sQ = smem + ((qc - qc0) & 1) * STAGE;
        const char* sO = sQ + TS_BYTES;
        const float* sL = (const float*)(sQ + 2 * TS_BYTES);
        const float* sD = sL + 64;
        // fragments read one k step ahead of their products, k step outermost (as in the dQ
        // kernel)
        bf16x8 qa[4], oa[4];
        // s = scale * score - L (base 2), dp = dP - D, per query row q0 + 16qb + 4g + i: the
        // offsets (-L and -D as the dQ kernel stored them) start the accumulators
        floatx4 s[4][KBW], dp[4][KBW];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
            const floatx4 nl = *(const floatx4*)(sL + qb * 16 + g * 4);
            const floatx4 nd = *(const floatx4*)(sD + qb * 16 + g * 4);
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) {
                s[qb][kb] = nl;
                dp[qb][kb] = nd;
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) {
                qa[qb] = ts_nat(sQ, qb * 16, ks, lane);
                oa[qb] = ts_nat(sO, qb * 16, ks, lane);
            }
            __builtin_amdgcn_s_setprio(1);  // MFMA phases at raised priority (see the forward)
#pragma unroll
            for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb) {
                    mma8(s[qb][kb], qa[qb], kf[kb][ks]);
                    mma8(dp[qb][kb], oa[qb], vf[kb][ks]);
                }
            __builtin_amdgcn_s_setprio(0);
        }
        // P and dS; rows q = q0 + 16qb + 4g + i, column key = kw0 + 16kb + col. Only chunks
        // that cross the diagonal or the end of the sequence are masked: the two forms are
        // compiled separately, so the others carry no compares or selects.
        auto p_ds = [&](auto masked) {
#pragma unroll
            for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int q = q0 + qb * 16 + g * 4 + i;
#pragma unroll
                    for (int kb = 0; kb < KBW; ++kb) {
                        const int key = kw0 + kb * 16 + col;
                        float a = s[qb][kb][i];
                        // masked entries get -inf added before the exponential (exp2(-inf) = 0):
                        // a select between two constants, which the compiler keeps branch-free
                        // (a select of the loaded value itself it turns into a branch per entry)
                        if constexpr (decltype(masked)::value) a += ((key <= q) & (q < T_)) ? 0.f : -INFINITY;
                        const float p = exp2_raw(a);
                        s[qb][kb][i] = p;
                        dp[qb][kb][i] *= p;
                    }
                }
        };
        if ((q0 < kw0 + KW) || (q0 + 64 > T_)) p_ds(std::true_type{});
        else p_ds(std::false_type{});
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            bf16x8 pf[KBW], df[KBW];
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) {
                pf[kb] = frag_from_acc<bf16>(s[2 * st][kb], s[2 * st + 1][kb]);
                df[kb] = frag_from_acc<bf16>(dp[2 * st][kb], dp[2 * st + 1][kb]);
            }
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const bf16x8 oat = ts_tr(sO, d * 16, 32 * st, 32 * st + 16, lane);
                const bf16x8 qat = ts_tr(sQ, d * 16, 32 * st, 32 * st + 16, lane);
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb) {
                    mma8(dv[d][kb], oat, pf[kb]);
                    mma8(dk[d][kb], qat, df[kb]);
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
    }
    if (!wave_live) return;
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
        const int key = kw0 + kb * 16 + col;
        if (key >= T_) continue;
        bf16* r = dqkv + ((int64_t)b * T_ + key) * ld + h * HS;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            store4v<bf16>(r + C + d * 16 + g * 4, dk[d][kb], scale);
            store4v<bf16>(r + 2 * C + d * 16 + g * 4, dv[d][kb], 1.0f);
        }
    }
}

// dQ for 64 * QBW queries per workgroup (16 * QBW per wave), streaming 64-key chunks of K and V.
template <int QBW>
__global__ void __launch_bounds__(A_THREADS, QBW == 1 ? 4 : 2) attn_bwd_dq_ts_kernel(const bf16* __restrict__ qkv,
                                                                   const bf16* __restrict__ y,
                                                                   const bf16* __restrict__ dy,
                                                                   const float* __restrict__ lse,
                                                                   float* __restrict__ D,
                                                                   bf16* __restrict__ dqkv, int T_, int H, float sc,
                                                                   float scale) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];  // [stage][K | V]
    constexpr int HS = 64, STAGE = 2 * TS_BYTES;
    int bx, by;
    xcd_remap(bx, by);
    constexpr int QW = 16 * QBW, QBLK = 4 * QW;   // queries per wave, per workgroup
    const int nqb = (T_ + QBLK - 1) / QBLK;
    const int qblk = nqb - 1 - bx;
    const int bh = by, b = bh / H, h = bh % H;
    const int C = H * HS;
    const int64_t ld = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T_ * ld;
    const bf16* dyb = dy + (int64_t)b * T_ * C;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int q0 = qblk * QBLK, qw0 = q0 + wave * QW;
    const uint32_t lds0 = lds_addr(smem);

    bf16x8 qf[QBW][2], of[QBW][2];
    float L[QBW], Dq[QBW];
    const bf16* yb = y + (int64_t)b * T_ * C;
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
        const int q = qw0 + qb * 16 + col;
        const bool ok = q < T_;
        float dsum = 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            qf[qb][ks] = ok ? frag_scaled(frag_global<bf16>(base + (int64_t)q * ld + h * HS + ks * 32 + g * 8), sc)
                            : frag_zero<bf16>();
            of[qb][ks] = ok ? frag_global<bf16>(dyb + (int64_t)q * C + h * HS + ks * 32 + g * 8) : frag_zero<bf16>();
            // D = sum_d dO o O of this query row (the softmax-gradient correction term): this
            // lane's 8 dimensions, then the 4 lane groups of the row
            const bf16x8 yf = ok ? frag_global<bf16>(yb + (int64_t)q * C + h * HS + ks * 32 + g * 8) : frag_zero<bf16>();
#pragma unroll
            for (int e = 0; e < 8; ++e) dsum += (float)of[qb][ks][e] * (float)yf[e];
        }
        dsum += __shfl_xor(dsum, 16);
        dsum += __shfl_xor(dsum, 32);
        L[qb] = ok ? lse[(int64_t)bh * T_ + q] * kLog2e : 0.f;
        Dq[qb] = ok ? dsum : 0.f;
        // for the dK/dV kernel, which runs next: -D, and after all B*H*T of them the log-sum-exp
        // already in base 2 and negated (one multiply per query here instead of one per score
        // there; negated, they are the accumulators' starting values as loaded)
        if (ok && g == 0) {
            D[(int64_t)bh * T_ + q] = -dsum;
            D[(int64_t)gridDim.y * T_ + (int64_t)bh * T_ + q] = -L[qb];
        }
    }
    floatx4 dq[4][QBW];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) dq[d][qb] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int kend = min(q0 + QBLK, T_);
    const int nchunk = (kend + 63) / 64;
    const bool wave_live = qw0 < T_;
    const TsOff offkv = ts_offsets(ld, 64, wave, lane);
    auto issue = [&](int c) {
        const int k0 = c * 64, nv = min(64, T_ - k0);
        const uint32_t st = lds0 + (c & 1) * STAGE;
        ts_load(base + (int64_t)k0 * ld + C + h * HS, ld, nv, offkv, st, wave, lane);
        ts_load(base + (int64_t)k0 * ld + 2 * C + h * HS, ld, nv, offkv, st + TS_BYTES, wave, lane);
    };
    if (nchunk > 0) issue(0);
    for (int c = 0; c < nchunk; ++c) {
        dma_wait_barrier();
        if (c + 1 < nchunk) issue(c + 1);
        const int k0 = c * 64;
        if constexpr (QBW > 1) {   // see the forward
            if (!wave_live || k0 > qw0 + QW - 1) continue;
        }
        const char* sK = smem + (c & 1) * STAGE;
        const char* sV = sK + TS_BYTES;
        // fragments read one k step ahead of their products, k step outermost, so that the two
        // products into one accumulator are eight apart (and at most one k step's fragments
        // are held: the registers decide how many waves share a SIMD)
        bf16x8 ka[4], va[4], kat[2][4];
        // s = scale * score - L (base 2), dp = dP - D: the offsets start the accumulators
        floatx4 s[4][QBW], dp[4][QBW];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int qb = 0; qb < QBW; ++qb) {
                s[kb][qb] = splat4(-L[qb]);
                dp[kb][qb] = splat4(-Dq[qb]);
            }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                ka[kb] = ts_nat(sK, kb * 16, ks, lane);
                va[kb] = ts_nat(sV, kb * 16, ks, lane);
            }
            __builtin_amdgcn_s_setprio(1);  // MFMA phases at raised priority (see the forward)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int qb = 0; qb < QBW; ++qb) {
                    mma8(s[kb][qb], ka[kb], qf[qb][ks]);
                    mma8(dp[kb][qb], va[kb], of[qb][ks]);
                }
            __builtin_amdgcn_s_setprio(0);
        }

        // rows key = k0 + 16kb + 4g + i, column q = qw0 + 16qb + col; masked and unmasked forms
        // compiled separately, as in the dK/dV kernel
        auto ds = [&](auto masked) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int qb = 0; qb < QBW; ++qb) {
                    const int q = qw0 + qb * 16 + col;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = k0 + kb * 16 + g * 4 + i;
                        float a = s[kb][qb][i];
                        if constexpr (decltype(masked)::value) a += ((key <= q) & (key < T_)) ? 0.f : -INFINITY;  // as in dK/dV
                        const float p = exp2_raw(a);
                        dp[kb][qb][i] *= p;
                    }
                }
        };
        if ((k0 + 63 > qw0) || (k0 + 64 > T_)) ds(std::true_type{});
        else ds(std::false_type{});
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int d = 0; d < 4; ++d) kat[st][d] = ts_tr(sK, d * 16, 32 * st, 32 * st + 16, lane);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            bf16x8 dfr[QBW];
#pragma unroll
            for (int qb = 0; qb < QBW; ++qb) dfr[qb] = frag_from_acc<bf16>(dp[2 * st][qb], dp[2 * st + 1][qb]);
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int qb = 0; qb < QBW; ++qb) mma8(dq[d][qb], kat[st][d], dfr[qb]);
        }
        __builtin_amdgcn_s_setprio(0);
    }
    if (!wave_live) return;
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
        const int q = qw0 + qb * 16 + col;
        if (q >= T_) continue;
        bf16* r = dqkv + ((int64_t)b * T_ + q) * ld + h * HS;
#pragma unroll
        for (int d = 0; d < 4; ++d) store4v<bf16>(r + d * 16 + g * 4, dq[d][qb], scale);
    }
}

constexpr size_t ts_fwd_lds() { return 2 * 2 * TS_BYTES; }
#ifndef ATT_FWD_QB
#define ATT_FWD_QB 1
#endif
#ifndef ATT_DKV_KB
#define ATT_DKV_KB 1
#endif
#ifndef ATT_DQ_QB
#define ATT_DQ_QB 1
#endif
constexpr size_t ts_dkv_lds() { return 2 * (2 * TS_BYTES + 512); }

template <typename T, int HS> constexpr size_t fwd_lds() { return Tile<T, HS>::BYTES + Tile<T, 64>::BYTES; }
template <typename T, int HS> constexpr size_t dkv_lds() { return 2 * (Tile<T, HS>::BYTES + Tile<T, 64>::BYTES) + 128 * sizeof(float); }
template <typename T, int HS> constexpr size_t dq_lds() { return 2 * Tile<T, HS>::BYTES + Tile<T, 64>::BYTES; }

template <typename T, int HS>
static hipError_t fwd_launch(const void* qkv, void* y, float* lse, int B, int T_, int H, hipStream_t s) {
    const float sc = kLog2e / sqrtf((float)HS);
    dim3 grid((T_ + 127) / 128, B * H);
    if constexpr (sizeof(T) == 2 && HS == 64) {
        dim3 g4((T_ + 4 * 16 * ATT_FWD_QB - 1) / (4 * 16 * ATT_FWD_QB), B * H);
        attn_fwd_ts_kernel<ATT_FWD_QB><<<g4, dim3(A_THREADS), ts_fwd_lds(), s>>>((const bf16*)qkv, (bf16*)y, lse, T_, H, sc);
    } else {
        attn_fwd_kernel<T, HS><<<grid, dim3(A_THREADS), fwd_lds<T, HS>(), s>>>((const T*)qkv, (T*)y, lse, T_, H, sc);
    }
    return hipGetLastError();
}

template <typename T, int HS>
static hipError_t bwd_launch(const void* qkv, const void* y, const void* dy, const float* lse, float* D, void* dqkv,
                             int B, int T_, int H, hipStream_t s) {
    const float sc = kLog2e / sqrtf((float)HS);
    const float scale = 1.0f / sqrtf((float)HS);
    const int64_t n = (int64_t)B * T_ * H;
    dim3 grid((T_ + 127) / 128, B * H);
    hipError_t e;
    if constexpr (sizeof(T) == 2 && HS == 64) {
        // the dQ kernel forms D itself (from the dO and O rows it loads) and stores it for the
        // dK/dV kernel, so it runs first and no separate pass over O and dO is needed
        const dim3 gq((T_ + 64 * ATT_DQ_QB - 1) / (64 * ATT_DQ_QB), B * H);
        attn_bwd_dq_ts_kernel<ATT_DQ_QB><<<gq, dim3(A_THREADS), ts_fwd_lds(), s>>>(
            (const bf16*)qkv, (const bf16*)y, (const bf16*)dy, lse, D, (bf16*)dqkv, T_, H, sc, scale);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const dim3 gk((T_ + 64 * ATT_DKV_KB - 1) / (64 * ATT_DKV_KB), B * H);
        attn_bwd_dkv_ts_kernel<ATT_DKV_KB><<<gk, dim3(A_THREADS), ts_dkv_lds(), s>>>(
            (const bf16*)qkv, (const bf16*)dy, D + n, (const float*)D, (bf16*)dqkv, T_, H, sc, scale);
        return hipGetLastError();
    }
    attn_bwd_pre_kernel<T, HS><<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>((const T*)y, (const T*)dy, D,
                                                                                      B * T_, T_, H);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_bwd_dkv_kernel<T, HS><<<grid, dim3(A_THREADS), dkv_lds<T, HS>(), s>>>((const T*)qkv, (const T*)dy, lse,
                                                                              (const float*)D, (T*)dqkv, T_, H, sc, scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_bwd_dq_kernel<T, HS><<<grid, dim3(A_THREADS), dq_lds<T, HS>(), s>>>((const T*)qkv, (const T*)dy, lse,
                                                                            (const float*)D, (T*)dqkv, T_, H, sc, scale);
    return hipGetLastError();
}

hipError_t attention_forward(const void* qkv, void* y, float* lse, int B, int T_, int H, int hs, int is_bf16,
                             hipStream_t s) {
    if (hs == 64) return is_bf16 ? fwd_launch<bf16, 64>(qkv, y, lse, B, T_, H, s) : fwd_launch<float, 64>(qkv, y, lse, B, T_, H, s);
    if (hs == 32) return is_bf16 ? fwd_launch<bf16, 32>(qkv, y, lse, B, T_, H, s) : fwd_launch<float, 32>(qkv, y, lse, B, T_, H, s);
    return hipErrorInvalidValue;
}

hipError_t attention_backward(const void* qkv, const void* y, const void* dy, const float* lse, float* D, void* dqkv,
                              int B, int T_, int H, int hs, int is_bf16, hipStream_t s) {
    if (hs == 64)
        return is_bf16 ? bwd_launch<bf16, 64>(qkv, y, dy, lse, D, dqkv, B, T_, H, s)
                       : bwd_launch<float, 64>(qkv, y, dy, lse, D, dqkv, B, T_, H, s);
    if (hs == 32)
        return is_bf16 ? bwd_launch<bf16, 32>(qkv, y, dy, lse, D, dqkv, B, T_, H, s)
                       : bwd_launch<float, 32>(qkv, y, dy, lse, D, dqkv, B, T_, H, s);
    return hipErrorInvalidValue;
}

void attention_setup() {
#define ASET(T, HS)                                                                                                  \
    (void)hipFuncSetAttribute((const void*)attn_fwd_kernel<T, HS>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)fwd_lds<T, HS>()); \
    (void)hipFuncSetAttribute((const void*)attn_bwd_dkv_kernel<T, HS>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dkv_lds<T, HS>()); \
    (void)hipFuncSetAttribute((const void*)attn_bwd_dq_kernel<T, HS>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dq_lds<T, HS>());
    ASET(bf16, 64) ASET(bf16, 32) ASET(float, 64) ASET(float, 32)
#undef ASET
    (void)hipFuncSetAttribute((const void*)attn_fwd_ts_kernel<ATT_FWD_QB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ts_fwd_lds());
    (void)hipFuncSetAttribute((const void*)attn_bwd_dq_ts_kernel<ATT_DQ_QB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ts_fwd_lds());
    (void)hipFuncSetAttribute((const void*)attn_bwd_dkv_ts_kernel<ATT_DKV_KB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ts_dkv_lds());
}

}  // namespace gpt2k
