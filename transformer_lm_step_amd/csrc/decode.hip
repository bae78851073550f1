// Incremental decoding: attention of one new position over a key/value cache, and top-k
// sampling of the next token.
//
// The sampling loop of "Karpathy's Zero to Hero, Lecture 9" (notes, chapter 0:28:07-0:41:44,
// and the sampling code of chapter 3:22:33-3:28:16) takes the logits at the last position,
// applies the softmax, keeps the 50 most probable tokens, and draws one of them in proportion
// to its probability. Keeping the keys and values of the earlier positions (the cache) makes
// each new position one row of every product instead of a forward over the whole prefix.
#include "common.h"
#include "kernels.h"

namespace gpt2k {

// ---------------------------------------------------------------- attention of one position
// Causal self-attention ("Code you'll write", causal self-attention) of the query at position
// pos of every sequence: softmax over its scaled dot products with the keys at positions
// 0..pos, then the probability-weighted sum of their values. qkv rows are (b, t) ->
// b * Tmax + t, 3C wide (q | k | v, head h in columns h*hs ..). One workgroup per (sequence,
// head); every sum runs in a fixed order.
constexpr int DEC_THREADS = 256;

template <typename T, int HS>
__global__ void __launch_bounds__(DEC_THREADS) attn_decode_kernel(const T* __restrict__ qkv, int Tmax, int pos, int H,
                                                                  float sc, T* __restrict__ y,
                                                                  const int32_t* __restrict__ d_pos) {
    if (d_pos) pos = min(max(*d_pos, 0), Tmax - 1);   // the position from device memory (LDS sized for Tmax)
    constexpr int G = DEC_THREADS / HS;    // key groups of the value sum
    extern __shared__ float dsm[];         // q [HS], partial sums [G][HS], scores [pos + 1]
    __shared__ float red[DEC_THREADS / 64];
    const int b = blockIdx.x / H, h = blockIdx.x - b * H, tid = threadIdx.x;
    const int C = H * HS;
    const int64_t ld = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * Tmax * ld;
    float* sq = dsm;
    float* part = dsm + HS;
    float* ss = part + G * HS;
    if (tid < HS) sq[tid] = to_f<T>(base[(int64_t)pos * ld + h * HS + tid]);
    __syncthreads();
    const int n = pos + 1;
    float mx = -INFINITY;
    for (int t = tid; t < n; t += DEC_THREADS) {
        const T* k = base + (int64_t)t * ld + C + h * HS;
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < HS; i += 16 / (int)sizeof(T)) {
            const uint4 raw = ld16(k + i);
            const T* e = (const T*)&raw;
#pragma unroll
            for (int q = 0; q < 16 / (int)sizeof(T); ++q) d += sq[i + q] * to_f<T>(e[q]);
        }
        d *= sc;                           // log2(e) / sqrt(hs): exp2 below is exp of the scaled score
        ss[t] = d;
        mx = fmaxf(mx, d);
    }
    mx = wave_max(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < DEC_THREADS / 64; ++w) mx = fmaxf(mx, red[w]);
    __syncthreads();
    float sum = 0.f;
    for (int t = tid; t < n; t += DEC_THREADS) {
        const float p = exp2f(ss[t] - mx);
        ss[t] = p;
        sum += p;
    }
    sum = wave_sum(sum);
    if ((tid & 63) == 0) red[tid >> 6] = sum;
    __syncthreads();                       // also: every score is final
    sum = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_THREADS / 64; ++w) sum += red[w];
    const int d = tid % HS, g = tid / HS;
    float acc = 0.f;
    for (int t = g; t < n; t += G) acc += ss[t] * to_f<T>(base[(int64_t)t * ld + 2 * C + h * HS + d]);
    part[g * HS + d] = acc;
    __syncthreads();
    if (tid < HS) {
        float o = 0.f;
#pragma unroll
        for (int j = 0; j < G; ++j) o += part[j * HS + tid];
        y[(int64_t)b * C + h * HS + tid] = from_f<T>(o / sum);
    }
}

size_t attention_decode_lds(int hs, int Tmax) { return (size_t)(hs + DEC_THREADS + Tmax) * 4; }

// With d_pos the position is read on the device (clamped to Tmax - 1) and `pos` is ignored.
hipError_t attention_decode(const void* qkv, void* y, int B, int Tmax, int pos, int H, int hs, int is_bf16,
                            hipStream_t s, const int32_t* d_pos) {
    if ((!d_pos && (pos < 0 || pos >= Tmax)) || (hs != 64 && hs != 32)) return hipErrorInvalidValue;
    const float sc = 1.4426950408889634f / sqrtf((float)hs);
    const size_t lds = attention_decode_lds(hs, d_pos ? Tmax : pos + 1);
    const dim3 grid(B * H), blk(DEC_THREADS);
    if (is_bf16) {
        if (hs == 64) attn_decode_kernel<bf16, 64><<<grid, blk, lds, s>>>((const bf16*)qkv, Tmax, pos, H, sc, (bf16*)y, d_pos);
        else attn_decode_kernel<bf16, 32><<<grid, blk, lds, s>>>((const bf16*)qkv, Tmax, pos, H, sc, (bf16*)y, d_pos);
    } else {
        if (hs == 64)
            attn_decode_kernel<float, 64><<<grid, blk, lds, s>>>((const float*)qkv, Tmax, pos, H, sc, (float*)y, d_pos);
        else
            attn_decode_kernel<float, 32><<<grid, blk, lds, s>>>((const float*)qkv, Tmax, pos, H, sc, (float*)y, d_pos);
    }
    return hipGetLastError();
}

__global__ void decode_advance_kernel(int32_t* __restrict__ d_pos, int pos_end) {
    if (threadIdx.x == 0) *d_pos = min(*d_pos + 1, pos_end);
}
hipError_t decode_advance(int32_t* d_pos, int pos_end, hipStream_t s) {
    hipLaunchKernelGGL(decode_advance_kernel, dim3(1), dim3(64), 0, s, d_pos, pos_end);
    return hipGetLastError();
}

// ---------------------------------------------------------------- top-k sampling
// Per sequence b, over all Vp logits of its row (padded columns included, as in the softmax
// of the pages' sampling code): the k largest logits, larger first and equal ones by lower
// token id (the k most probable tokens, since the softmax preserves order), their softmax
// (the top-k probabilities renormalized), and the draw: the first of them whose cumulative
// probability exceeds u[b] (inverse CDF of the caller's uniform number in [0, 1); the last
// one if rounding leaves every cumulative sum at or below u).
//
// Selection: radix select of the k-th largest order-preserving 32-bit key in four 8-bit passes
// (LDS histograms; two for bf16 rows, whose keys' low 16 bits are set by the sign alone), then an ordered compaction (block scans in
// token order) of the keys above it plus the lowest-id keys equal to it, then one wave sorts
// the k entries.
constexpr int TK_THREADS = 1024;

DEV uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive prefix sum of v over the workgroup (fixed order); *total receives the sum
DEV int block_excl_scan(int v, int* total, int* wsum) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int x = __shfl_up(inc, o);
        if (lane >= o) inc += x;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    int before = 0, all = 0;
    for (int i = 0; i < TK_THREADS / 64; ++i) {
        if (i < w) before += wsum[i];
        all += wsum[i];
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

// Thread t owns the contiguous ids [per t, per t + per), so the compaction keeps token order.
// IN_REG (bf16 rows of at most TK_REG_MAX ids): per is a multiple of 8, and each thread loads
// its ids once with 16-byte loads into registers (up to TK_REG_CHUNKS x 8 values), which every
// pass below then reads; otherwise the passes read the row from global memory.
constexpr int TK_REG_CHUNKS = 8;
constexpr int TK_REG_MAX = TK_THREADS * 8 * TK_REG_CHUNKS;

// the order key of element e (0..7) of a 16-byte chunk of bf16 values
DEV uint32_t chunk_key(const uint4& q, int e) {
    const uint32_t w = e < 2 ? q.x : e < 4 ? q.y : e < 6 ? q.z : q.w;
    return order_key(__uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16)));
}
// the float whose order key is `key`
DEV float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

template <typename T, bool IN_REG>
__global__ void __launch_bounds__(TK_THREADS) topk_sample_kernel(const T* __restrict__ logits, int Vp, int k,
                                                                 const float* __restrict__ u,
                                                                 int32_t* __restrict__ next,
                                                                 int32_t* __restrict__ topk_idx,
                                                                 float* __restrict__ topk_prob) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_state[3];
    __shared__ int wsum[TK_THREADS / 64];
    __shared__ int sel_idx[TOPK_MAX];
    __shared__ uint32_t sel_key[TOPK_MAX];
    const int b = blockIdx.x, tid = threadIdx.x;
    const T* z = logits + (int64_t)b * Vp;
    int per = (Vp + TK_THREADS - 1) / TK_THREADS;
    if constexpr (IN_REG) per = (per + 7) & ~7;
    const int j0 = min(Vp, tid * per), j1 = min(Vp, j0 + per);
    uint4 rowc[IN_REG ? TK_REG_CHUNKS : 1];
    if constexpr (IN_REG) {
#pragma unroll
        for (int c = 0; c < TK_REG_CHUNKS; ++c)
            if (j0 + 8 * c < j1) rowc[c] = ld16(z + j0 + 8 * c);
    }
    // f(j, key) over the thread's ids in ascending order
    auto for_keys = [&](auto f) {
        if constexpr (IN_REG) {
#pragma unroll
            for (int c = 0; c < TK_REG_CHUNKS; ++c)
                if (j0 + 8 * c < j1) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) f(j0 + 8 * c + e, chunk_key(rowc[c], e));
                }
        } else {
            for (int j = j0; j < j1; ++j) f(j, order_key(to_f<T>(z[j])));
        }
    };

    uint32_t prefix = 0, mask = 0;
    int need = k;
    // a bf16 value widens to a float with 16 zero low bits, so its key's low 16 bits are 0000
    // (positive: key = bits | sign bit) or ffff (negative: key = ~bits); passes over them would
    // put every remaining key in one bin and leave `need` as it is
    constexpr int LAST_SHIFT = sizeof(T) == 2 ? 16 : 0;
    for (int shift = 24; shift >= LAST_SHIFT; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for_keys([&](int, uint32_t key) {
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        });
        __syncthreads();
        if (tid == 0) {
            int cum = 0, dgt = 255;
            for (; dgt > 0; --dgt) {
                if (cum + (int)hist[dgt] >= need) break;
                cum += (int)hist[dgt];
            }
            s_state[0] = prefix | ((uint32_t)dgt << shift);
            s_state[1] = mask | (255u << shift);
            s_state[2] = (uint32_t)(need - cum);
        }
        __syncthreads();
        prefix = s_state[0];
        mask = s_state[1];
        need = (int)s_state[2];
        __syncthreads();
    }
    if constexpr (LAST_SHIFT == 16) prefix |= (prefix & 0x80000000u) ? 0u : 0xffffu;
    // prefix is now the k-th largest key; the keys above it and the `need` lowest-id keys equal
    // to it are the selection
    int n_gt = 0, n_eq = 0;
    for_keys([&](int, uint32_t key) {
        n_gt += key > prefix;
        n_eq += key == prefix;
    });
    int tot;
    const int eq_before = block_excl_scan(n_eq, &tot, wsum);
    const int eq_take = max(0, min(n_eq, need - eq_before));
    const int pos0 = block_excl_scan(n_gt + eq_take, &tot, wsum);
    int p = pos0, eq_seen = 0;
    for_keys([&](int j, uint32_t key) {
        bool take = key > prefix;
        if (key == prefix) take = eq_seen++ < eq_take;
        if (take) {
            sel_idx[p] = j;
            sel_key[p] = key;
            ++p;
        }
    });
    __syncthreads();
    if (tid >= 64) return;
    // one wave: bitonic sort of the k entries (padding sorts last) by larger value, then lower id
    const int lane = tid;
    uint64_t e = lane < k ? ((uint64_t)(~sel_key[lane]) << 32) | (uint32_t)sel_idx[lane] : ~(uint64_t)0;
    for (int sz = 2; sz <= 64; sz <<= 1) {
        for (int st = sz >> 1; st > 0; st >>= 1) {
            const uint64_t o = ((uint64_t)__shfl_xor((int)(e >> 32), st) << 32) | (uint32_t)__shfl_xor((int)(uint32_t)e, st);
            const bool lower = (lane & st) == 0, asc = (lane & sz) == 0;
            e = (lower == asc) ? (e < o ? e : o) : (e > o ? e : o);
        }
    }
    const int id = (int)(uint32_t)e;
    // the logit back from its key (exact)
    const float zv = lane < k ? key_value(~(uint32_t)(e >> 32)) : -INFINITY;
    const float zmax = __shfl(zv, 0);
    const float pr = lane < k ? expf(zv - zmax) : 0.f;
    float cdf = pr;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float x = __shfl_up(cdf, o);
        if (lane >= o) cdf += x;
    }
    const float total = __shfl(cdf, k - 1);
    if (topk_idx && lane < k) topk_idx[(int64_t)b * k + lane] = id;
    if (topk_prob && lane < k) topk_prob[(int64_t)b * k + lane] = pr / total;
    if (next) {
        const float thr = u[b] * total;
        const uint64_t hit = __ballot(lane < k && cdf > thr);
        const int pick = hit ? __builtin_ctzll(hit) : k - 1;
        const int chosen = __shfl(id, pick);
        if (lane == 0) next[b] = chosen;
    }
}

hipError_t topk_sample(const void* logits, int B, int Vp, int k, const float* u, int32_t* next, int32_t* topk_idx,
                       float* topk_prob, int is_bf16, hipStream_t s) {
    if (k < 1 || k > TOPK_MAX || k > Vp || Vp % 8) return hipErrorInvalidValue;
    const dim3 grid(B), blk(TK_THREADS);
    if (is_bf16 && Vp <= TK_REG_MAX)
        topk_sample_kernel<bf16, true><<<grid, blk, 0, s>>>((const bf16*)logits, Vp, k, u, next, topk_idx, topk_prob);
    else if (is_bf16)
        topk_sample_kernel<bf16, false><<<grid, blk, 0, s>>>((const bf16*)logits, Vp, k, u, next, topk_idx, topk_prob);
    else
        topk_sample_kernel<float, false><<<grid, blk, 0, s>>>((const float*)logits, Vp, k, u, next, topk_idx, topk_prob);
    return hipGetLastError();
}

}  // namespace gpt2k
