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
// (LDS histograms), then an ordered compaction (block scans in
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

// IN_LDS (bf16 rows of at most TK_LDS_MAX ids): the row is first copied into LDS with 16-byte
// loads, so the five passes below read LDS; otherwise they read the row from global memory.
// Thread t owns the contiguous ids [per t, per t + per), so the compaction keeps token order.
constexpr int TK_LDS_MAX = 65536;

template <typename T, bool IN_LDS>
__global__ void __launch_bounds__(TK_THREADS) topk_sample_kernel(const T* __restrict__ logits, int Vp, int k,
                                                                 const float* __restrict__ u,
                                                                 int32_t* __restrict__ next,
                                                                 int32_t* __restrict__ topk_idx,
                                                                 float* __restrict__ topk_prob) {
    constexpr int E = 16 / sizeof(T);
    extern __shared__ __attribute__((aligned(16))) char tk_row[];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_state[3];
    __shared__ int wsum[TK_THREADS / 64];
    __shared__ int sel_idx[TOPK_MAX];
    __shared__ float sel_val[TOPK_MAX];
    const int b = blockIdx.x, tid = threadIdx.x;
    const T* z = logits + (int64_t)b * Vp;
    const T* src = z;
    if constexpr (IN_LDS) {
        T* row = (T*)tk_row;
#pragma unroll 8
        for (int c = tid; c < Vp / E; c += TK_THREADS) *(uint4*)(row + c * E) = ld16(z + c * E);
        __syncthreads();
        src = row;
    }
    const int per = (Vp + TK_THREADS - 1) / TK_THREADS;
    const int j0 = min(Vp, tid * per), j1 = min(Vp, j0 + per);
    auto key_at = [&](int j) { return order_key(to_f<T>(src[j])); };

    uint32_t prefix = 0, mask = 0;
    int need = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int j = j0; j < j1; ++j) {
            const uint32_t key = key_at(j);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
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
    // prefix is now the k-th largest key; the keys above it and the `need` lowest-id keys equal
    // to it are the selection
    int n_gt = 0, n_eq = 0;
    for (int j = j0; j < j1; ++j) {
        const uint32_t key = key_at(j);
        n_gt += key > prefix;
        n_eq += key == prefix;
    }
    int tot;
    const int eq_before = block_excl_scan(n_eq, &tot, wsum);
    const int eq_take = max(0, min(n_eq, need - eq_before));
    const int pos0 = block_excl_scan(n_gt + eq_take, &tot, wsum);
    int p = pos0, eq_seen = 0;
    for (int j = j0; j < j1; ++j) {
        const uint32_t key = key_at(j);
        bool take = key > prefix;
        if (key == prefix) take = eq_seen++ < eq_take;
        if (take) {
            sel_idx[p] = j;
            sel_val[p] = to_f<T>(src[j]);
            ++p;
        }
    }
    __syncthreads();
    if (tid >= 64) return;
    // one wave: bitonic sort of the k entries (padding sorts last) by larger value, then lower id
    const int lane = tid;
    uint64_t e = lane < k ? ((uint64_t)(~order_key(sel_val[lane])) << 32) | (uint32_t)sel_idx[lane] : ~(uint64_t)0;
    for (int sz = 2; sz <= 64; sz <<= 1) {
        for (int st = sz >> 1; st > 0; st >>= 1) {
            const uint64_t o = ((uint64_t)__shfl_xor((int)(e >> 32), st) << 32) | (uint32_t)__shfl_xor((int)(uint32_t)e, st);
            const bool lower = (lane & st) == 0, asc = (lane & sz) == 0;
            e = (lower == asc) ? (e < o ? e : o) : (e > o ? e : o);
        }
    }
    const int id = (int)(uint32_t)e;
    // the value again from the row (exact: the row is unchanged)
    const float zv = lane < k ? to_f<T>(src[id]) : -INFINITY;
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
    if (is_bf16 && Vp <= TK_LDS_MAX)
        topk_sample_kernel<bf16, true><<<grid, blk, (size_t)Vp * 2, s>>>((const bf16*)logits, Vp, k, u, next, topk_idx,
                                                                         topk_prob);
    else if (is_bf16)
        topk_sample_kernel<bf16, false><<<grid, blk, 0, s>>>((const bf16*)logits, Vp, k, u, next, topk_idx, topk_prob);
    else
        topk_sample_kernel<float, false><<<grid, blk, 0, s>>>((const float*)logits, Vp, k, u, next, topk_idx, topk_prob);
    return hipGetLastError();
}

void decode_setup() {
    (void)hipFuncSetAttribute((const void*)topk_sample_kernel<bf16, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              TK_LDS_MAX * 2);
}

}  // namespace gpt2k
