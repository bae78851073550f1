// Device-side building blocks shared by the kernels of the GPT-2 step (gfx950 / CDNA4).
//
// Storage types: `float` (fp32 check mode) and `bf16` (= __bf16, the bf16 mode). Every
// conversion float -> bf16 rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
//
// Matrix products use 16x16 MFMA tiles on wave64. Operand fragments are "8 consecutive
// k values per lane": lane l covers row/column (l & 15) and the k sub-range owned by lane
// group g = l >> 4. For bf16 one v_mfma_f32_16x16x32_bf16 consumes the 8 values; for fp32
// eight v_mfma_f32_16x16x4f32 consume them one at a time. Because the sum over k is
// order-free, it only matters that the A and B fragments of a product assign k the same way.
// The 16x16 fp32 accumulator holds, in lane l, rows 4*(l>>4)+i (i = 0..3) of column (l & 15).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

#define DEV __device__ __forceinline__

// ------------------------------------------------------------------ conversions
template <typename T> DEV float to_f(T x);
template <> DEV float to_f<float>(float x) { return x; }
template <> DEV float to_f<bf16>(bf16 x) { return (float)x; }

template <typename T> DEV T from_f(float x);
template <> DEV float from_f<float>(float x) { return x; }
template <> DEV bf16 from_f<bf16>(float x) { return (bf16)x; }

// 4 consecutive values of a storage-type row as fp32, and back
template <typename T> DEV void store4(T* p, float a, float b, float c, float d);
template <> DEV void store4<float>(float* p, float a, float b, float c, float d) { *(float4*)p = make_float4(a, b, c, d); }
template <> DEV void store4<bf16>(bf16* p, float a, float b, float c, float d) {
    bf16x4 v;
    v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
    *(bf16x4*)p = v;
}
// 4 fp32 values as they read back after a store in type T (rounded to bf16 for bf16)
template <typename T> DEV float4 load4_rounded(float a, float b, float c, float d);
template <> DEV float4 load4_rounded<float>(float a, float b, float c, float d) { return make_float4(a, b, c, d); }
template <> DEV float4 load4_rounded<bf16>(float a, float b, float c, float d) {
    return make_float4((float)(bf16)a, (float)(bf16)b, (float)(bf16)c, (float)(bf16)d);
}
template <typename T> DEV float4 load4(const T* p);
template <> DEV float4 load4<float>(const float* p) { return *(const float4*)p; }
template <> DEV float4 load4<bf16>(const bf16* p) {
    const bf16x4 v = *(const bf16x4*)p;
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

// nn.LayerNorm epsilon
constexpr float LN_EPS = 1e-5f;

// 8-value fragment type of a storage type
template <typename T> struct FragT;
template <> struct FragT<bf16> { typedef bf16x8 type; };
template <> struct FragT<float> { typedef floatx8 type; };

DEV void mma8(floatx4& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
DEV void mma8(floatx4& acc, const floatx8& a, const floatx8& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
}

// Build a fragment from two 4-element halves (used where a lane's 8 k values are two
// separate runs of 4).
DEV bf16x8 frag_from_halves(const uint2& lo, const uint2& hi) {
    uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
    return __builtin_bit_cast(bf16x8, u);
}
DEV floatx8 frag_from_halves(const float4& lo, const float4& hi) {
    floatx8 r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

// 16-byte vector of a storage type
template <typename T> struct Vec16 { typedef uint4 type; static constexpr int N = 16 / sizeof(T); };

// ------------------------------------------------------------------ reductions
DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
// reduce over the 4 lane groups (lanes l, l^16, l^32, l^48) that share a 16x16 column
DEV float group4_sum(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}
DEV float group4_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
// The same maximum from the gfx950 lane-swap instructions, without the LDS crossbar: the swap
// of the upper half-wave of one copy with the lower half-wave of another leaves, in the two
// results, the values of lanes l & ~32 and l | 32 (then l & ~16 and l | 16 for the swap of
// odd with even 16-lane rows).
DEV float group4_max_swap(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Block-wide sum for a block of NT threads (NT multiple of 64); every thread gets the result.
template <int NT>
DEV float block_sum(float v, float* red /* >= NT/64 floats of shared memory */) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) s += red[i];
    return s;
}

// ------------------------------------------------------------------ 16-byte transposes
// Transpose an E x E block of storage elements held as E rows of 16 bytes (E = 8 for bf16,
// 4 for fp32): out[j] holds column j (element r of out[j] = element j of in[r]).
DEV void transpose_block(const uint4 (&in)[8], uint4 (&out)[8], bf16*) {
    // element (r, j) of the input lives in word j/2 of in[r], half j&1
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int w = j >> 1;
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t a = ((const uint32_t*)&in[2 * p])[w];
            const uint32_t b = ((const uint32_t*)&in[2 * p + 1])[w];
            o[p] = __builtin_amdgcn_perm(b, a, sel);
        }
        out[j] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}
DEV void transpose_block(const uint4 (&in)[8], uint4 (&out)[8], float*) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = ((const uint32_t*)&in[r])[j];
        out[j] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

DEV uint4 ld16(const void* p) { return *(const uint4*)p; }
DEV void st16(void* p, const uint4& v) { *(uint4*)p = v; }

// ------------------------------------------------------------------ GELU (tanh form)
// 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))) and its derivative.
constexpr float kGeluC = 0.7978845608028654f;  // sqrt(2/pi)
constexpr float kGeluA = 0.044715f;
// GELU-tanh through the logistic function: with w = c (u + a u^3) and s = 1 / (1 + e^{-2w}),
//   0.5 (1 + tanh w) = s   and   1 - tanh^2 w = 4 s (1 - s), so
//   gelu(u) = u s,   gelu'(u) = s + 2 u s (1 - s) c (1 + 3 a u^2).
// One v_exp_f32 and one v_rcp_f32 (about 1 ulp each); saturates cleanly for large |u|.
DEV float gelu_sigmoid(float u) {
    const float w2 = -2.0f * 1.4426950408889634f * kGeluC * (u + kGeluA * u * u * u);   // -2w log2(e)
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(w2));
}
DEV float gelu_f(float u) { return u * gelu_sigmoid(u); }
DEV float gelu_grad_f(float u) {
    const float sg = gelu_sigmoid(u);
    return sg + 2.0f * u * sg * (1.0f - sg) * kGeluC * (1.0f + 3.0f * kGeluA * u * u);
}

// ------------------------------------------------------------------ direct global->LDS loads
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_t;
typedef __attribute__((address_space(3))) char* lds_char_t;

// s_waitcnt immediates: vmcnt == 0 only (expcnt, lgkmcnt at their maxima); lgkmcnt == 0 only
// (vmcnt, expcnt at their maxima); both. Waits issued through the builtin are seen by the
// compiler's own wait tracking: one in inline asm is not, and a kernel whose scalar argument
// loads are first used after a loop then gets lgkmcnt(0) before every LDS-fed instruction in
// it (the compiler cannot order LDS returns against scalar loads it believes in flight). The
// barriers below issue both: the builtin for the tracking, the asm copy next to s_barrier so
// that nothing the compiler moves in between escapes the wait.
constexpr int kWaitVm0 = (0x7 << 4) | (0xF << 8);
constexpr int kWaitLgkm0 = 0xF | (0x7 << 4) | (0x3 << 14);
constexpr int kWaitVm0Lgkm0 = 0x7 << 4;

// LDS byte address of a shared-memory pointer
DEV uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_char_t)(p); }

// A wave-uniform pointer held in scalar registers: the compiler can leave a uniform value that
// it computed with vector instructions (an integer division, say) in vector registers, which
// the scalar operand of the direct loads below cannot take; readfirstlane of a value already in
// scalar registers costs nothing.
DEV const void* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// One direct load: the wave's 64 lanes each move 16 bytes from base + voff to LDS address
// lds + 16 * lane (global_load_lds_dwordx4; base and lds wave-uniform). Inline asm (M0 and
// the load in one block, no register results), so the compiler does not make later LDS reads
// wait for it; kernels order these loads with explicit vmcnt waits and barriers. Loads the
// compiler does not track only make its own vmcnt waits stricter (the counter drains in order).
DEV void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(uniform_ptr(base))
                 : "memory");
}
// the same with 4 bytes per lane (LDS address lds + 4 * lane)
DEV void dma4(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(uniform_ptr(base))
                 : "memory");
}
// wait for this wave's direct loads, then a bare barrier (no fence: a fence would also drain
// loads issued for later tiles). Afterwards every wave's loads issued before it have landed
// and every wave's earlier LDS reads have completed.
DEV void dma_wait_barrier() {
    __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Barrier for LDS traffic only: this wave's LDS accesses are complete, then every wave meets.
// Unlike __syncthreads() it does not wait for the wave's global stores to complete, so a
// workgroup can stage the next part of its output in LDS while earlier stores drain.
DEV void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Two transposing LDS reads (ds_read_b64_tr_b16) joined into one 8-value fragment. Within
// each 16-lane group the instruction gives lane i, as its j-th value, element (i % 4) of the
// 8 bytes addressed by lane 4j + i/4 of the group. When the group's lanes address 4 rows
// (lane >> 2) x 4 consecutive 4-element column pieces (lane & 3) of a row-major tile, lane i
// receives column i of those 4 rows: the first read gives values 0..3, the second 4..7.
DEV bf16x8 read_tr_pair(const char* p0, const char* p1) {
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t)(lds_char_t)p0);
    const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t)(lds_char_t)p1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
