// Memory-bound kernels of the GPT-2 step: embedding forward/backward, LayerNorm
// forward/backward, bias (column) sums, softmax cross-entropy, gradient norm, AdamW and
// parameter initialization. Every reduction runs in a fixed order, so results are bitwise
// reproducible run to run.
#include <algorithm>
#include "common.h"
#include "kernels.h"

namespace gpt2k {


// ================================================================== embedding forward
// x[b,t,:] = wte[idx[b,t],:] + wpe[t,:] ("Code you'll write", forward pass: token and
// position embeddings are added), stored in the storage type. One wave per token row.
// With d_pos (one new position per sequence, T_ = 1) the position is read from device memory,
// clamped to pos_max.
template <typename T>
__global__ void embed_forward_kernel(const int32_t* __restrict__ idx, const float* __restrict__ wte,
                                     const float* __restrict__ wpe, T* __restrict__ x, int rows,
                                     int T_, int C, const int32_t* __restrict__ d_pos, int pos_max) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int t = d_pos ? min(max(*d_pos, 0), pos_max) : row % T_;
    const int64_t id = idx[row];
    const int nv = C >> 2;
    const float4* e = (const float4*)(wte + id * C);
    const float4* p = (const float4*)(wpe + (int64_t)t * C);
    T* o = x + (int64_t)row * C;
    for (int c = lane; c < nv; c += 64) {
        const float4 a = e[c], b = p[c];
        store4<T>(o + 4 * c, a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    }
}

hipError_t embed_forward(const int32_t* idx, const float* wte, const float* wpe, void* x, int B, int T,
                         int C, int is_bf16, hipStream_t s, const int32_t* d_pos, int pos_max) {
    const int rows = B * T;
    if (d_pos && T != 1) return hipErrorInvalidValue;
    if (is_bf16)
        hipLaunchKernelGGL(embed_forward_kernel<bf16>, dim3((rows + 3) / 4), dim3(256), 0, s, idx, wte, wpe, (bf16*)x,
                           rows, T, C, d_pos, pos_max);
    else
        hipLaunchKernelGGL(embed_forward_kernel<float>, dim3((rows + 3) / 4), dim3(256), 0, s, idx, wte, wpe,
                           (float*)x, rows, T, C, d_pos, pos_max);
    return hipGetLastError();
}

// ================================================================== LayerNorm
// nn.LayerNorm(C) with eps 1e-5 and the biased variance. One wave per row; the row stays in
// registers (up to 8 float4 per lane: C <= 2048); mean, then centered variance.
constexpr int LN_NV = 8;

// NV = float4 per lane needed for C (C <= 256 * NV): the row is held in registers sized to C.
// TX: type of the residual stream x (fp32, or bf16 in the bf16-residual mode); TO: type of the
// normalized output (the operand type of the product that follows).
template <typename TX, typename TO, int NV>
__global__ void __launch_bounds__(256) layernorm_forward_kernel(const TX* __restrict__ x, const float* __restrict__ w,
                                                                const float* __restrict__ b, TO* __restrict__ out,
                                                                float* __restrict__ mean, float* __restrict__ rstd,
                                                                int rows, int C) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int nv = C >> 2;
    const TX* xr = x + (int64_t)row * C;
    float4 v[NV];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = lane + 64 * j;
        v[j] = c < nv ? load4<TX>(xr + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
        s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
    }
    const float mu = wave_sum(s) / (float)C;
    float s2 = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = lane + 64 * j;
        if (c < nv) {
            const float a = v[j].x - mu, bb = v[j].y - mu, cc = v[j].z - mu, d = v[j].w - mu;
            s2 += (a * a + bb * bb) + (cc * cc + d * d);
        }
    }
    const float var = wave_sum(s2) / (float)C;
    const float r = 1.0f / sqrtf(var + LN_EPS);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = lane + 64 * j;
        if (c < nv) {
            const float4 ww = ((const float4*)w)[c], bb = ((const float4*)b)[c];
            store4<TO>(out + (int64_t)row * C + 4 * c, (v[j].x - mu) * r * ww.x + bb.x, (v[j].y - mu) * r * ww.y + bb.y,
                       (v[j].z - mu) * r * ww.z + bb.z, (v[j].w - mu) * r * ww.w + bb.w);
        }
    }
    if (lane == 0) { mean[row] = mu; rstd[row] = r; }
}

template <typename TX, typename TO>
static hipError_t ln_fwd_launch(int nv4, dim3 g, hipStream_t s, const TX* x, const float* w, const float* b, TO* out,
                                float* mean, float* rstd, int rows, int C) {
#define LNF(NV) hipLaunchKernelGGL((layernorm_forward_kernel<TX, TO, NV>), g, dim3(256), 0, s, x, w, b, out, mean, rstd, rows, C)
    if (nv4 <= 64) LNF(1);
    else if (nv4 <= 128) LNF(2);
    else if (nv4 <= 192) LNF(3);
    else if (nv4 <= 256) LNF(4);
    else if (nv4 <= 320) LNF(5);
    else if (nv4 <= 384) LNF(6);
    else if (nv4 <= 448) LNF(7);
    else LNF(8);
#undef LNF
    return hipGetLastError();
}

// Residual add fused with the LayerNorm that follows it: x_new = x_old + y, then the LayerNorm of
// x_new. y is the projection's output with its bias (bf16 in the bf16 modes: the autocast recipe
// rounds a product's output to bf16 before the fp32 residual add); the add is done in fp32 and
// x_new is stored in the residual stream's type TX, and the statistics are taken on the stored
// value. One wave per row, the row in registers.
template <typename TX, typename TY, typename TO, int NV>
__global__ void __launch_bounds__(256) add_layernorm_forward_kernel(
    const TX* __restrict__ x_old, const TY* __restrict__ y, TX* __restrict__ x_new, const float* __restrict__ w,
    const float* __restrict__ b, TO* __restrict__ out, float* __restrict__ mean, float* __restrict__ rstd, int rows,
    int C) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int nv = C >> 2;
    const int64_t ro = (int64_t)row * C;
    float4 v[NV];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = lane + 64 * j;
        v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c < nv) {
            const float4 a = load4<TX>(x_old + ro + 4 * c), d = load4<TY>(y + ro + 4 * c);
            store4<TX>(x_new + ro + 4 * c, a.x + d.x, a.y + d.y, a.z + d.z, a.w + d.w);
            v[j] = load4_rounded<TX>(a.x + d.x, a.y + d.y, a.z + d.z, a.w + d.w);
        }
        s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
    }
    const float mu = wave_sum(s) / (float)C;
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
            const float4 ww = ((const float4*)w)[c], bb = ((const float4*)b)[c];
            store4<TO>(out + ro + 4 * c, (v[j].x - mu) * r * ww.x + bb.x, (v[j].y - mu) * r * ww.y + bb.y,
                       (v[j].z - mu) * r * ww.z + bb.z, (v[j].w - mu) * r * ww.w + bb.w);
        }
    }
    if (lane == 0) { mean[row] = mu; rstd[row] = r; }
}

template <typename TX, typename TY, typename TO>
static hipError_t add_ln_launch(int nv4, dim3 g, hipStream_t s, const TX* xo, const TY* y, TX* xn, const float* w,
                                const float* b, TO* out, float* mean, float* rstd, int rows, int C) {
#define ALN(NV) hipLaunchKernelGGL((add_layernorm_forward_kernel<TX, TY, TO, NV>), g, dim3(256), 0, s, xo, y, xn, w, b, \
                                   out, mean, rstd, rows, C)
    if (nv4 <= 64) ALN(1);
    else if (nv4 <= 128) ALN(2);
    else if (nv4 <= 192) ALN(3);
    else if (nv4 <= 256) ALN(4);
    else if (nv4 <= 320) ALN(5);
    else if (nv4 <= 384) ALN(6);
    else if (nv4 <= 448) ALN(7);
    else ALN(8);
#undef ALN
    return hipGetLastError();
}

hipError_t add_layernorm_forward(const void* x_old, const void* y, void* x_new, const float* w, const float* b,
                                 void* out, float* mean, float* rstd, int rows, int C, int x_bf16, int op_bf16,
                                 hipStream_t s) {
    if (C > 4 * 64 * LN_NV || (C & 3)) return hipErrorInvalidValue;
    if (x_bf16 && !op_bf16) return hipErrorInvalidValue;
    const dim3 g((rows + 3) / 4);
    if (x_bf16)
        return add_ln_launch<bf16, bf16, bf16>(C / 4, g, s, (const bf16*)x_old, (const bf16*)y, (bf16*)x_new, w, b,
                                               (bf16*)out, mean, rstd, rows, C);
    if (op_bf16)
        return add_ln_launch<float, bf16, bf16>(C / 4, g, s, (const float*)x_old, (const bf16*)y, (float*)x_new, w, b,
                                                (bf16*)out, mean, rstd, rows, C);
    return add_ln_launch<float, float, float>(C / 4, g, s, (const float*)x_old, (const float*)y, (float*)x_new, w, b,
                                              (float*)out, mean, rstd, rows, C);
}

// bf16 rows of C = 256 * NC: one half-wave (32 lanes) per row, NC 16-byte chunks per lane, so
// a wave keeps two rows' loads in flight with half the load instructions. Same arithmetic as
// the kernel above (mean, then the centered variance, each summed over the row in fp32).
template <int NC>
__global__ void __launch_bounds__(256) layernorm_forward_half_kernel(const bf16* __restrict__ x,
                                                                     const float* __restrict__ w,
                                                                     const float* __restrict__ b,
                                                                     bf16* __restrict__ out, float* __restrict__ mean,
                                                                     float* __restrict__ rstd, int rows, int C) {
    const int l = threadIdx.x & 31;
    const int row = blockIdx.x * 8 + (threadIdx.x >> 5);
    const bool live = row < rows;
    const bf16* xr = x + (int64_t)(live ? row : rows - 1) * C;
    float v[NC][8];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const uint4 raw = ld16(xr + 8 * (l + 32 * j));
        const bf16* e = (const bf16*)&raw;
#pragma unroll
        for (int q = 0; q < 8; ++q) { v[j][q] = (float)e[q]; s += v[j][q]; }
    }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) s += __shfl_xor(s, o);
    const float mu = s / (float)C;
    float s2 = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) { const float d = v[j][q] - mu; s2 += d * d; }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) s2 += __shfl_xor(s2, o);
    const float r = 1.0f / sqrtf(s2 / (float)C + LN_EPS);
    if (!live) return;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = 8 * (l + 32 * j);
        const float4 w0 = *(const float4*)(w + c), w1 = *(const float4*)(w + c + 4);
        const float4 b0 = *(const float4*)(b + c), b1 = *(const float4*)(b + c + 4);
        const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        bf16x8 o;
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = (bf16)((v[j][q] - mu) * r * ww[q] + bb[q]);
        *(bf16x8*)(out + (int64_t)row * C + c) = o;
    }
    if (l == 0) { mean[row] = mu; rstd[row] = r; }
}

hipError_t layernorm_forward(const void* x, const float* w, const float* b, void* out, float* mean,
                             float* rstd, int rows, int C, int x_bf16, int out_bf16, hipStream_t s) {
    if (C > 4 * 64 * LN_NV || (C & 3)) return hipErrorInvalidValue;
    if (x_bf16 && !out_bf16) return hipErrorInvalidValue;
    dim3 g((rows + 3) / 4);
    if (x_bf16 && (C == 512 || C == 768 || C == 1024) && ((uintptr_t)x & 15) == 0 && ((uintptr_t)out & 15) == 0) {
        const dim3 g8((rows + 7) / 8);
        if (C == 512) hipLaunchKernelGGL(layernorm_forward_half_kernel<2>, g8, dim3(256), 0, s, (const bf16*)x, w, b, (bf16*)out, mean, rstd, rows, C);
        else if (C == 768) hipLaunchKernelGGL(layernorm_forward_half_kernel<3>, g8, dim3(256), 0, s, (const bf16*)x, w, b, (bf16*)out, mean, rstd, rows, C);
        else hipLaunchKernelGGL(layernorm_forward_half_kernel<4>, g8, dim3(256), 0, s, (const bf16*)x, w, b, (bf16*)out, mean, rstd, rows, C);
        return hipGetLastError();
    }
    if (x_bf16) return ln_fwd_launch<bf16, bf16>(C / 4, g, s, (const bf16*)x, w, b, (bf16*)out, mean, rstd, rows, C);
    if (out_bf16) return ln_fwd_launch<float, bf16>(C / 4, g, s, (const float*)x, w, b, (bf16*)out, mean, rstd, rows, C);
    return ln_fwd_launch<float, float>(C / 4, g, s, (const float*)x, w, b, (float*)out, mean, rstd, rows, C);
}

// Backward through y = xhat*w + b, xhat = (x - mean)*rstd:
//   dxhat = dh*w;  dx = rstd*(dxhat - mean(dxhat) - xhat*mean(dxhat*xhat))
//   dw += sum_rows dh*xhat;  db += sum_rows dh
// and dres = (accumulate ? dres : 0) + dx. With accumulate, the incoming dres is the
// gradient at the output of the residual add that produced x, so its column sum is the bias
// gradient of that add's projection; it is collected as a third partial.
// Each wave takes lnb_rows(rows) consecutive rows; the block's 4 wave partials are combined in a
// fixed order into partial[blk][0:3C] = (dw, db, colsum(dres_in)), finished by sum_partials.
constexpr int LNB_ROWS = 4;
// Rows per wave: LNB_ROWS, or 2 for batches of at most 8192 rows, so that a batch of 4096 rows
// (the 1558M-shaped step at B=4, C = 1600: 7 float4 per lane, whose registers and LDS allow two
// workgroups per CU) fills all 512 workgroup slots in one round instead of half of them (3.84
// -> 2.72 ms per step at that shape; 16,384 rows at C = 768 measured slower with 2).
static int lnb_rows(int rows) { return rows <= 8192 ? 2 : LNB_ROWS; }
int layernorm_backward_blocks(int rows) { const int k = lnb_rows(rows); return (rows + 4 * k - 1) / (4 * k); }
// The most blocks any batch of at most max_rows rows takes (the count is not monotonic across
// the 8192-row switch of lnb_rows): what the partial sets are sized for.
int layernorm_backward_max_blocks(int max_rows) {
    const int a = layernorm_backward_blocks(max_rows), b = layernorm_backward_blocks(max_rows < 8192 ? max_rows : 8192);
    return a > b ? a : b;
}

// NV = float4 per lane needed for C (C <= 256 * NV); sized to C so the row lives in registers.
// TD: type of dh (the operand type); TX: type of x and of the residual gradient dres (fp32, or
// bf16 in the bf16-residual mode). With dres16 non-null, the new dres is also stored as bf16
// (the A operand of the products that take the residual gradient).
template <typename TD, typename TX, int NV>
__global__ void __launch_bounds__(256) layernorm_backward_kernel(
    const TD* __restrict__ dh, const TX* __restrict__ x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const float* __restrict__ w, TX* __restrict__ dres, bf16* __restrict__ dres16,
    int accumulate, float* __restrict__ partial, int rows, int C, int nrw) {
    extern __shared__ float sred[];  // [4][3C]
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nv = C >> 2;
    float4 dw[NV], db[NV], cs[NV], wv[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        dw[j] = db[j] = cs[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        const int c = lane + 64 * j;
        wv[j] = c < nv ? ((const float4*)w)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int r0 = (blockIdx.x * 4 + wave) * nrw;
    for (int row = r0; row < r0 + nrw && row < rows; ++row) {
        const float mu = mean[row], r = rstd[row];
        const TD* dr = dh + (int64_t)row * C;
        const TX* xr = x + (int64_t)row * C;
        TX* o = dres + (int64_t)row * C;
        float4 xh[NV], dxh[NV], old[NV];
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = lane + 64 * j;
            xh[j] = dxh[j] = old[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < nv) {
                const float4 d = load4<TD>(dr + 4 * c), xx = load4<TX>(xr + 4 * c);
                if (accumulate) old[j] = load4<TX>(o + 4 * c);
                xh[j] = make_float4((xx.x - mu) * r, (xx.y - mu) * r, (xx.z - mu) * r, (xx.w - mu) * r);
                dxh[j] = make_float4(d.x * wv[j].x, d.y * wv[j].y, d.z * wv[j].z, d.w * wv[j].w);
                s1 += (dxh[j].x + dxh[j].y) + (dxh[j].z + dxh[j].w);
                s2 += (dxh[j].x * xh[j].x + dxh[j].y * xh[j].y) + (dxh[j].z * xh[j].z + dxh[j].w * xh[j].w);
                dw[j].x += d.x * xh[j].x; dw[j].y += d.y * xh[j].y; dw[j].z += d.z * xh[j].z; dw[j].w += d.w * xh[j].w;
                db[j].x += d.x; db[j].y += d.y; db[j].z += d.z; db[j].w += d.w;
                cs[j].x += old[j].x; cs[j].y += old[j].y; cs[j].z += old[j].z; cs[j].w += old[j].w;
            }
        }
        const float m1 = wave_sum(s1) / (float)C, m2 = wave_sum(s2) / (float)C;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = lane + 64 * j;
            if (c < nv) {
                const float4 g = make_float4(old[j].x + r * (dxh[j].x - m1 - xh[j].x * m2),
                                             old[j].y + r * (dxh[j].y - m1 - xh[j].y * m2),
                                             old[j].z + r * (dxh[j].z - m1 - xh[j].z * m2),
                                             old[j].w + r * (dxh[j].w - m1 - xh[j].w * m2));
                store4<TX>(o + 4 * c, g.x, g.y, g.z, g.w);
                if (dres16) store4<bf16>(dres16 + (int64_t)row * C + 4 * c, g.x, g.y, g.z, g.w);
            }
        }
    }
    // combine the 4 waves' partials in a fixed order
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = lane + 64 * j;
        if (c < nv) {
            *(float4*)(sred + wave * 3 * C + 4 * c) = dw[j];
            *(float4*)(sred + wave * 3 * C + C + 4 * c) = db[j];
            *(float4*)(sred + wave * 3 * C + 2 * C + 4 * c) = cs[j];
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < 3 * C; c += blockDim.x) {
        const float v = ((sred[c] + sred[3 * C + c]) + sred[6 * C + c]) + sred[9 * C + c];
        partial[(int64_t)blockIdx.x * 3 * C + c] = v;
    }
}

template <typename TD, typename TX>
static hipError_t ln_bwd_launch(int nv4, dim3 g, size_t lds, hipStream_t s, const TD* dh, const TX* x,
                                const float* mean, const float* rstd, const float* w, TX* dres, bf16* dres16, int acc,
                                float* partial, int rows, int C) {
#define LNB(NV) hipLaunchKernelGGL((layernorm_backward_kernel<TD, TX, NV>), g, dim3(256), lds, s, dh, x, mean, rstd, w, \
                                   dres, dres16, acc, partial, rows, C, lnb_rows(rows))
    if (nv4 <= 64) LNB(1);
    else if (nv4 <= 128) LNB(2);
    else if (nv4 <= 192) LNB(3);
    else if (nv4 <= 256) LNB(4);
    else if (nv4 <= 320) LNB(5);
    else if (nv4 <= 384) LNB(6);
    else if (nv4 <= 448) LNB(7);
    else LNB(8);
#undef LNB
    return hipGetLastError();
}

hipError_t layernorm_backward(const void* dh, const void* x, const float* mean, const float* rstd,
                              const float* w, void* dres, void* dres16, int accumulate_dres, float* partial,
                              int nblk, int rows, int C, int dh_bf16, int res_bf16, hipStream_t s) {
    if (C > 4 * 64 * LN_NV || (C & 3)) return hipErrorInvalidValue;
    if (res_bf16 && !dh_bf16) return hipErrorInvalidValue;
    const size_t lds = 12 * (size_t)C * sizeof(float);
    if (res_bf16)
        return ln_bwd_launch<bf16, bf16>(C / 4, dim3(nblk), lds, s, (const bf16*)dh, (const bf16*)x, mean, rstd, w,
                                         (bf16*)dres, (bf16*)dres16, accumulate_dres, partial, rows, C);
    if (dh_bf16)
        return ln_bwd_launch<bf16, float>(C / 4, dim3(nblk), lds, s, (const bf16*)dh, (const float*)x, mean, rstd, w,
                                          (float*)dres, (bf16*)dres16, accumulate_dres, partial, rows, C);
    return ln_bwd_launch<float, float>(C / 4, dim3(nblk), lds, s, (const float*)dh, (const float*)x, mean, rstd, w,
                                       (float*)dres, (bf16*)dres16, accumulate_dres, partial, rows, C);
}

// Column sums of partial [np, n] (row stride `stride`), deterministic, in two launches:
//  1. slice z of SUM_SLICES takes partial rows [z*per, (z+1)*per); a workgroup covers 64
//     columns, its 4 waves take every 4th row (two running sums each) and are combined in a
//     fixed order into scratch[z][col];
//  2. out[col] (+)= sum_z scratch[z][col], z ascending.
constexpr int SUM_SLICES = 16;
int sum_scratch_floats(int n) { return SUM_SLICES * n; }

// blockIdx.z selects one of several partial sets of the same shape (set_stride floats apart),
// each with its own SUM_SLICES x n block of scratch
__global__ void __launch_bounds__(256) colred1_kernel(const float* __restrict__ partial, int np, int n,
                                                      int64_t stride, float* __restrict__ scratch,
                                                      int64_t set_stride) {
    __shared__ float red[4][64];
    partial += (int64_t)blockIdx.z * set_stride;
    scratch += (int64_t)blockIdx.z * SUM_SLICES * n;
    const int col = blockIdx.x * 64 + (threadIdx.x & 63), grp = threadIdx.x >> 6;
    const int per = (np + SUM_SLICES - 1) / SUM_SLICES;
    const int p0 = blockIdx.y * per;
    const int p1 = min(p0 + per, np);
    float a0 = 0.f, a1 = 0.f;
    if (col < n) {
        int p = p0 + grp;
        for (; p + 4 < p1; p += 8) {
            a0 += partial[(int64_t)p * stride + col];
            a1 += partial[(int64_t)(p + 4) * stride + col];
        }
        if (p < p1) a0 += partial[(int64_t)p * stride + col];
    }
    red[grp][threadIdx.x & 63] = a0 + a1;
    __syncthreads();
    if (grp == 0 && col < n) {
        const int c = threadIdx.x & 63;
        scratch[(int64_t)blockIdx.y * n + col] = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
    }
}

// columns [0, n1) go to out1[col], columns [n1, n) to out2[col - n1]
__global__ void __launch_bounds__(256) colred2_kernel(const float* __restrict__ scratch, int n, float* __restrict__ out1,
                                                      int n1, float* __restrict__ out2, int accumulate) {
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= n) return;
    float v = 0.f;
#pragma unroll
    for (int z = 0; z < SUM_SLICES; ++z) v += scratch[(int64_t)z * n + col];
    float* o = col < n1 ? out1 + col : out2 + (col - n1);
    *o = accumulate ? *o + v : v;
}

hipError_t sum_partials2(const float* partial, int np, int n, int64_t stride, float* out1, int n1, float* out2,
                         int accumulate, float* scratch, hipStream_t s) {
    hipLaunchKernelGGL(colred1_kernel, dim3((n + 63) / 64, SUM_SLICES), dim3(256), 0, s, partial, np, n, stride,
                       scratch, (int64_t)0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(colred2_kernel, dim3((n + 255) / 256), dim3(256), 0, s, scratch, n, out1, n1, out2, accumulate);
    return hipGetLastError();
}

hipError_t sum_partials(const float* partial, int np, int n, int64_t stride, float* out, int accumulate,
                        float* scratch, hipStream_t s) {
    return sum_partials2(partial, np, n, stride, out, n, nullptr, accumulate, scratch, s);
}

// Second stage for several sets at once (blockIdx.y = set): columns [0, n1) go to
// base[off1[set] + col], columns [n1, n) to base[off2[set] + col - n1], or nowhere when
// off2[set] < 0.
__global__ void __launch_bounds__(256) colred2_sets_kernel(const float* __restrict__ scratch, int n,
                                                           float* __restrict__ base, const int64_t* __restrict__ off1,
                                                           int n1, const int64_t* __restrict__ off2, int accumulate) {
    const int col = blockIdx.x * 256 + threadIdx.x, set = blockIdx.y;
    if (col >= n) return;
    if (col >= n1 && off2[set] < 0) return;
    const float* sc = scratch + (int64_t)set * SUM_SLICES * n;
    float v = 0.f;
#pragma unroll
    for (int z = 0; z < SUM_SLICES; ++z) v += sc[(int64_t)z * n + col];
    float* o = col < n1 ? base + off1[set] + col : base + off2[set] + (col - n1);
    *o = accumulate ? *o + v : v;
}

int sum_sets_scratch_floats(int nset, int n) { return nset * SUM_SLICES * n; }

hipError_t sum_partials_sets(const float* partial, int nset, int64_t set_stride, int np, int n, int64_t stride,
                             float* base, const int64_t* off1, int n1, const int64_t* off2, int accumulate,
                             float* scratch, hipStream_t s) {
    if (nset < 1) return hipSuccess;
    hipLaunchKernelGGL(colred1_kernel, dim3((n + 63) / 64, SUM_SLICES, nset), dim3(256), 0, s, partial, np, n, stride,
                       scratch, set_stride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(colred2_sets_kernel, dim3((n + 255) / 256, nset), dim3(256), 0, s, scratch, n, base, off1, n1,
                       off2, accumulate);
    return hipGetLastError();
}

// column sums of x [rows, n]: stage 1 writes one partial row per row-slice, stage 2 is
// sum_partials. Slices are fixed for a given (rows, n).
constexpr int CS_SLICE_ROWS = 64;
int colsum_partial_floats(int rows, int n) { return ((rows + CS_SLICE_ROWS - 1) / CS_SLICE_ROWS) * n; }

template <typename X>
__global__ void colsum_kernel(const X* __restrict__ x, int rows, int n, float* __restrict__ partial) {
    const int col = blockIdx.x * 256 + threadIdx.x;
    const int slice = blockIdx.y;
    if (col >= n) return;
    const int r0 = slice * CS_SLICE_ROWS;
    int r1 = r0 + CS_SLICE_ROWS;
    if (r1 > rows) r1 = rows;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    int r = r0;
    for (; r + 4 <= r1; r += 4) {
        a0 += to_f<X>(x[(int64_t)r * n + col]);
        a1 += to_f<X>(x[(int64_t)(r + 1) * n + col]);
        a2 += to_f<X>(x[(int64_t)(r + 2) * n + col]);
        a3 += to_f<X>(x[(int64_t)(r + 3) * n + col]);
    }
    for (; r < r1; ++r) a0 += to_f<X>(x[(int64_t)r * n + col]);
    partial[(int64_t)slice * n + col] = (a0 + a1) + (a2 + a3);
}

hipError_t colsum(const void* x, int x_is_f32, int is_bf16, int rows, int n, float* partial, float* out,
                  int accumulate, float* scratch, hipStream_t s) {
    const int ns = (rows + CS_SLICE_ROWS - 1) / CS_SLICE_ROWS;
    dim3 g((n + 255) / 256, ns);
    if (x_is_f32 || !is_bf16) hipLaunchKernelGGL(colsum_kernel<float>, g, dim3(256), 0, s, (const float*)x, rows, n, partial);
    else hipLaunchKernelGGL(colsum_kernel<bf16>, g, dim3(256), 0, s, (const bf16*)x, rows, n, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return sum_partials(partial, ns, n, n, out, accumulate, scratch, s);
}

// ================================================================== cross-entropy
// Per row n of z [rows, Vp]: lse = log sum_j exp z_j (all Vp columns), loss_n = lse - z_{y_n},
// then (write_grad) z is overwritten by dz = (softmax(z) - onehot(y)) / rows (F.cross_entropy
// with mean reduction on the flattened logits). One workgroup per row, two passes (the second
// re-reads the row from cache; evaluation skips it). The (max, sum) pairs are merged in a fixed
// order.
template <typename T>
__global__ void cross_entropy_kernel(T* __restrict__ z, const int32_t* __restrict__ targets,
                                     float* __restrict__ loss_rows, float* __restrict__ z_f32, int rows, int Vp,
                                     int write_grad) {
    constexpr int E = 16 / sizeof(T);
    __shared__ float smax[256 / 64], ssum[256 / 64];
    const int row = blockIdx.x;
    T* zr = z + (int64_t)row * Vp;
    const int nvec = Vp / E;
    float mx = -INFINITY, sm = 0.f;
    for (int v = threadIdx.x; v < nvec; v += 256) {
        const uint4 raw = ld16(zr + v * E);
        const T* e = (const T*)&raw;
        float vals[E];
        float lm = -INFINITY;
#pragma unroll
        for (int q = 0; q < E; ++q) { vals[q] = to_f<T>(e[q]); lm = fmaxf(lm, vals[q]); }
        if (z_f32) {
#pragma unroll
            for (int q = 0; q < E; q += 4)
                *(float4*)(z_f32 + (int64_t)row * Vp + v * E + q) = make_float4(vals[q], vals[q + 1], vals[q + 2], vals[q + 3]);
        }
        const float nm = fmaxf(mx, lm);
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < E; ++q) s += __expf(vals[q] - nm);
        sm = sm * __expf(mx - nm) + s;
        mx = nm;
    }
    // merge (mx, sm) across the wave, then across the 4 waves in order
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float om = __shfl_xor(mx, o), os = __shfl_xor(sm, o);
        const float nm = fmaxf(mx, om);
        sm = (mx == -INFINITY ? 0.f : sm * __expf(mx - nm)) + (om == -INFINITY ? 0.f : os * __expf(om - nm));
        mx = nm;
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { smax[w] = mx; ssum[w] = sm; }
    __syncthreads();
    float M = smax[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) M = fmaxf(M, smax[i]);
    float S = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) S += ssum[i] * __expf(smax[i] - M);
    const float lse = M + __logf(S);
    const int y = targets[row];
    if (threadIdx.x == 0) loss_rows[row] = lse - to_f<T>(zr[y]);
    if (!write_grad) return;
    __syncthreads();  // zr[y] read before any overwrite
    const float inv_n = 1.0f / (float)rows;
    for (int v = threadIdx.x; v < nvec; v += 256) {
        uint4 raw = ld16(zr + v * E);
        T* e = (T*)&raw;
#pragma unroll
        for (int q = 0; q < E; ++q) {
            const int j = v * E + q;
            const float p = __expf(to_f<T>(e[q]) - lse);
            e[q] = from_f<T>((p - (j == y ? 1.f : 0.f)) * inv_n);
        }
        st16(zr + v * E, raw);
    }
}

hipError_t cross_entropy(void* logits, const int32_t* targets, float* loss_rows, float* logits_f32, int n_rows,
                         int Vp, int is_bf16, hipStream_t s, int write_grad) {
    if (Vp % 8) return hipErrorInvalidValue;
    if (is_bf16) hipLaunchKernelGGL(cross_entropy_kernel<bf16>, dim3(n_rows), dim3(256), 0, s, (bf16*)logits, targets, loss_rows, logits_f32, n_rows, Vp, write_grad);
    else hipLaunchKernelGGL(cross_entropy_kernel<float>, dim3(n_rows), dim3(256), 0, s, (float*)logits, targets, loss_rows, logits_f32, n_rows, Vp, write_grad);
    return hipGetLastError();
}

// The same loss and gradient when the logits product has already stored, for every row and every
// 192-column tile of it, the tile's (max, sum exp(z - max)) over the stored values: the row's
// log-sum-exp comes from merging its `tiles` pairs (in a fixed order), so the logits are read
// once (only to write the gradient over them, or to copy them to fp32) instead of twice.
// Two kernels: a row pass (one wave per row) that merges the pairs, writes the row's loss and
// keeps lse * log2(e), then a gradient pass over the logits as one flat array of 8-element
// chunks, one chunk per thread. (One workgroup per row doing both ran at 5.3 TB/s: each row's
// merge stalled its stream, and the row's last trip over the columns left most threads idle. A
// probe of the flat in-place shape with non-temporal accesses measured 6.5 TB/s.)
__global__ void __launch_bounds__(256) ce_rows_kernel(const bf16* __restrict__ z, const float2* __restrict__ stats,
                                                      int tiles, const int32_t* __restrict__ targets,
                                                      float* __restrict__ loss_rows, float* __restrict__ lse2_rows,
                                                      int rows, int Vp) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= rows) return;
    const float2* sr = stats + (int64_t)row * tiles;
    float mx = -INFINITY, sm = 0.f;
    for (int t = lane; t < tiles; t += 64) {
        const float2 v = sr[t];
        const float nm = fmaxf(mx, v.x);
        sm = (mx == -INFINITY ? 0.f : sm * __expf(mx - nm)) + v.y * __expf(v.x - nm);
        mx = nm;
    }
    // butterfly merge: both lanes of a pair form the same (commutative) combination, so every
    // lane ends with the same pair
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float om = __shfl_xor(mx, o), os = __shfl_xor(sm, o);
        const float nm = fmaxf(mx, om);
        sm = (mx == -INFINITY ? 0.f : sm * __expf(mx - nm)) + (om == -INFINITY ? 0.f : os * __expf(om - nm));
        mx = nm;
    }
    if (lane == 0) {
        const float lse = mx + __logf(sm);
        loss_rows[row] = lse - (float)z[(int64_t)row * Vp + targets[row]];
        lse2_rows[row] = lse * 1.4426950408889634f;
    }
}

// dz = (softmax(z) - onehot(y)) / rows over chunks [0, nchunks) of rows row0.. (nvec chunks per
// row), written over the logits; the fp32 copy of the logits first where one is asked for. The
// logits are read once and dz is read next by the products, from HBM either way (1.6 GB at
// B=16): non-temporal accesses keep both out of the caches.
__global__ void __launch_bounds__(256) ce_grad_kernel(bf16* __restrict__ z, const float* __restrict__ lse2_rows,
                                                      const int32_t* __restrict__ targets, float* __restrict__ z_f32,
                                                      uint32_t nvec, uint32_t nchunks, int rows_total, int write_grad) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const uint32_t c = blockIdx.x * 256u + threadIdx.x;
    if (c >= nchunks) return;
    const uint32_t row = c / nvec, v = c - row * nvec;
    bf16* zc = z + (int64_t)row * nvec * 8 + v * 8;
    uint4 raw = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)zc));
    bf16* e = (bf16*)&raw;
    float vals[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) vals[q] = (float)e[q];
    if (z_f32) {
        float* f = z_f32 + (int64_t)row * nvec * 8 + v * 8;
        *(float4*)f = make_float4(vals[0], vals[1], vals[2], vals[3]);
        *(float4*)(f + 4) = make_float4(vals[4], vals[5], vals[6], vals[7]);
    }
    if (!write_grad) return;
    const float inv_n = 1.0f / (float)rows_total;
    const float lse2 = lse2_rows[row];
    const int y = targets[row] - (int)(v * 8);   // the target's position within this chunk
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float p = __builtin_amdgcn_exp2f(vals[q] * 1.4426950408889634f - lse2);
        e[q] = (bf16)((p - (q == y ? 1.f : 0.f)) * inv_n);
    }
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, raw), (u32x4*)zc);
}

hipError_t cross_entropy_tiled(void* logits, const float* stats, int tiles, const int32_t* targets, float* loss_rows,
                               float* lse2_rows, float* logits_f32, int n_rows, int Vp, hipStream_t s,
                               int write_grad) {
    if (Vp % 8 || tiles < 1 || n_rows < 0) return hipErrorInvalidValue;
    if (n_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(ce_rows_kernel, dim3((n_rows + 3) / 4), dim3(256), 0, s, (const bf16*)logits,
                       (const float2*)stats, tiles, targets, loss_rows, lse2_rows, n_rows, Vp);
    if (!write_grad && !logits_f32) return hipGetLastError();
    // row slices whose chunk count stays below 2^31 (32-bit chunk indices)
    const int64_t nvec = Vp / 8;
    const int slice = (int)std::min<int64_t>(n_rows, ((int64_t)1 << 31) / nvec);
    for (int r0 = 0; r0 < n_rows; r0 += slice) {
        const int nr = std::min(slice, n_rows - r0);
        const uint32_t nchunks = (uint32_t)(nr * nvec);
        hipLaunchKernelGGL(ce_grad_kernel, dim3((nchunks + 255) / 256), dim3(256), 0, s,
                           (bf16*)logits + (int64_t)r0 * Vp, lse2_rows + r0, targets + r0,
                           logits_f32 ? logits_f32 + (int64_t)r0 * Vp : nullptr, (uint32_t)nvec, nchunks, n_rows,
                           write_grad);
    }
    return hipGetLastError();
}

// ================================================================== evaluation reductions
// Completion scoring ([LVN] chapter 3:28:16-3:41:50): every sequence b is scored by the
// cross-entropy of the positions its mask selects (the ending's tokens): their sum, their
// count and their mean (0 when the mask selects nothing). One workgroup per sequence; each
// thread sums a strided set of positions in double, then a fixed tree. rowd keeps the double
// sum and count per sequence for the batch total.
constexpr int EVAL_THREADS = 256;
__global__ void __launch_bounds__(EVAL_THREADS) masked_row_loss_kernel(
    const float* __restrict__ loss, const uint8_t* __restrict__ mask, int T, double* __restrict__ rowd,
    float* __restrict__ row_sum, float* __restrict__ row_mean) {
    __shared__ double ss[EVAL_THREADS], sc[EVAL_THREADS];
    const int b = blockIdx.x, tid = threadIdx.x;
    double sum = 0.0, cnt = 0.0;
    for (int t = tid; t < T; t += EVAL_THREADS) {
        const int64_t i = (int64_t)b * T + t;
        if (!mask || mask[i]) {
            sum += (double)loss[i];
            cnt += 1.0;
        }
    }
    ss[tid] = sum;
    sc[tid] = cnt;
    __syncthreads();
    for (int o = EVAL_THREADS / 2; o > 0; o >>= 1) {
        if (tid < o) {
            ss[tid] += ss[tid + o];
            sc[tid] += sc[tid + o];
        }
        __syncthreads();
    }
    if (tid == 0) {
        rowd[2 * b] = ss[0];
        rowd[2 * b + 1] = sc[0];
        if (row_sum) row_sum[b] = (float)ss[0];
        if (row_mean) row_mean[b] = sc[0] > 0.0 ? (float)(ss[0] / sc[0]) : 0.f;
    }
}
// mean over every selected position of the batch: sum_b sum_b / sum_b count_b (0 if none)
__global__ void __launch_bounds__(EVAL_THREADS) masked_total_kernel(const double* __restrict__ rowd, int B,
                                                                    float* __restrict__ out) {
    __shared__ double ss[EVAL_THREADS], sc[EVAL_THREADS];
    const int tid = threadIdx.x;
    double sum = 0.0, cnt = 0.0;
    for (int b = tid; b < B; b += EVAL_THREADS) {
        sum += rowd[2 * b];
        cnt += rowd[2 * b + 1];
    }
    ss[tid] = sum;
    sc[tid] = cnt;
    __syncthreads();
    for (int o = EVAL_THREADS / 2; o > 0; o >>= 1) {
        if (tid < o) {
            ss[tid] += ss[tid + o];
            sc[tid] += sc[tid + o];
        }
        __syncthreads();
    }
    if (tid == 0) *out = sc[0] > 0.0 ? (float)(ss[0] / sc[0]) : 0.f;
}
hipError_t masked_row_loss(const float* loss_rows, const uint8_t* mask, int B, int T, double* rowd, float* row_sum,
                           float* row_mean, float* total, hipStream_t s) {
    hipLaunchKernelGGL(masked_row_loss_kernel, dim3(B), dim3(EVAL_THREADS), 0, s, loss_rows, mask, T, rowd, row_sum,
                       row_mean);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !total) return e;
    hipLaunchKernelGGL(masked_total_kernel, dim3(1), dim3(EVAL_THREADS), 0, s, rowd, B, total);
    return hipGetLastError();
}

template <typename T>
__global__ void convert_kernel(const T* __restrict__ src, float* __restrict__ dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = to_f<T>(src[i]);
}
hipError_t convert_to_f32(const void* src, float* dst, int64_t n, int is_bf16, hipStream_t s) {
    if (is_bf16) hipLaunchKernelGGL(convert_kernel<bf16>, dim3(2048), dim3(256), 0, s, (const bf16*)src, dst, n);
    else hipLaunchKernelGGL(convert_kernel<float>, dim3(2048), dim3(256), 0, s, (const float*)src, dst, n);
    return hipGetLastError();
}

// mean of v[0..n): one block, each thread sums a contiguous slice, fixed tree across threads
__global__ void mean_reduce_kernel(const float* __restrict__ v, int n, float* __restrict__ out) {
    __shared__ double red[1024];
    const int per = (n + 1023) / 1024;
    const int i0 = threadIdx.x * per;
    double s = 0.0;
    for (int i = i0; i < i0 + per && i < n; ++i) s += v[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = (float)(red[0] / (double)n);
}
hipError_t mean_reduce(const float* v, int n, float* d_out, hipStream_t s) {
    hipLaunchKernelGGL(mean_reduce_kernel, dim3(1), dim3(1024), 0, s, v, n, d_out);
    return hipGetLastError();
}

// ================================================================== embedding backward
// dwte[idx[r]] += dx[r] summed in ascending r per id, dwpe[t] (+)= sum_b dx[b,t].
// The gradients of repeated ids add ("Code you'll write" ties wte to lm_head; chapter
// 1:06:18-1:13:27: the two uses' gradients add up on the one tensor).
// 1) one workgroup sorts the (id, row) keys of a chunk of <= 16384 rows (bitonic),
//    cuts the sorted list into segments (same id, <= SEG rows, aligned to SEG) and runs
//    (same id), 2) every segment's rows are summed in order into a partial row,
// 3) every run adds its segments' partials in order to its wte row.
constexpr int EB_CHUNK = 16384;  // rows per sort (keys: id << 14 | row, ids < 2^18)
constexpr int EB_SEG = 32;
constexpr int EB_THREADS = 1024;

struct EbMeta {
    int nseg, nrun;
};

size_t embed_backward_scratch_bytes(int rows, int C) {
    const int n = rows < EB_CHUNK ? rows : EB_CHUNK;
    const int maxseg = n;  // at most one segment per row
    size_t b = 0;
    b += 256;                                   // meta
    b += (size_t)n * 4;                         // sorted rows
    b += (size_t)(maxseg + 1) * 4;              // segment begin
    b += (size_t)(n + 1) * 4 * 2;               // run id, run first segment
    b = (b + 255) & ~(size_t)255;
    b += (size_t)maxseg * C * 4;                // segment partial sums
    return b;
}

constexpr int EB_PER = EB_CHUNK / EB_THREADS;  // keys per thread (16)

// Exclusive prefix sums of two per-thread counts over the workgroup; also returns the totals.
DEV void eb_block_scan(int& a, int& b, int& ta, int& tb, int* wa, int* wb) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int ia = a, ib = b;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int xa = __shfl_up(ia, o), xb = __shfl_up(ib, o);
        if (lane >= o) { ia += xa; ib += xb; }
    }
    if (lane == 63) { wa[wave] = ia; wb[wave] = ib; }
    __syncthreads();
    int pa = 0, pb = 0;
    ta = 0; tb = 0;
    for (int w = 0; w < EB_THREADS / 64; ++w) {
        if (w < wave) { pa += wa[w]; pb += wb[w]; }
        ta += wa[w]; tb += wb[w];
    }
    a = pa + ia - a;
    b = pb + ib - b;
}

// Bitonic sort of EB_CHUNK keys (id << 14 | row; padding keys are all ones) held 16 per
// thread in registers: partners closer than 16 positions are in the same thread, closer than
// 1024 in the same wave (exchanged with lane shuffles); only the passes with partners in other
// waves go through LDS (double-buffered, one barrier each).
__global__ void __launch_bounds__(EB_THREADS) eb_sort_kernel(const int32_t* __restrict__ idx, int n,
                                                             EbMeta* meta, int32_t* __restrict__ srow,
                                                             int32_t* __restrict__ seg_begin, int32_t* __restrict__ run_id,
                                                             int32_t* __restrict__ run_seg) {
    extern __shared__ uint32_t keys[];  // [2][EB_CHUNK]
    __shared__ int wa[EB_THREADS / 64], wb[EB_THREADS / 64];
    const int tid = threadIdx.x, base = tid * EB_PER;
    uint32_t v[EB_PER];
#pragma unroll
    for (int e = 0; e < EB_PER; ++e) {
        const int i = base + e;
        v[e] = i < n ? ((uint32_t)idx[i] << 14) | (uint32_t)i : 0xFFFFFFFFu;
    }
    int buf = 0;
    for (int k = 2; k <= EB_CHUNK; k <<= 1) {
        // partners 16 or more positions away: the thread's 16 keys move as one block
        const bool up = (base & k) == 0;
        for (int j = k >> 1; j >= EB_PER; j >>= 1) {
            const bool keep_min = ((base & j) == 0) == up;
            uint32_t w[EB_PER];
            if (j < EB_PER * 64) {
                const int lm = j / EB_PER;
#pragma unroll
                for (int e = 0; e < EB_PER; ++e) w[e] = (uint32_t)__shfl_xor((int)v[e], lm);
            } else {
                uint32_t* kb = keys + buf * EB_CHUNK;
#pragma unroll
                for (int e = 0; e < EB_PER; e += 4)
                    *(uint4*)(kb + base + e) = make_uint4(v[e], v[e + 1], v[e + 2], v[e + 3]);
                __syncthreads();
                const int pb = base ^ j;
#pragma unroll
                for (int e = 0; e < EB_PER; e += 4) {
                    const uint4 q = *(const uint4*)(kb + pb + e);
                    w[e] = q.x; w[e + 1] = q.y; w[e + 2] = q.z; w[e + 3] = q.w;
                }
                buf ^= 1;
            }
#pragma unroll
            for (int e = 0; e < EB_PER; ++e) v[e] = keep_min ? min(v[e], w[e]) : max(v[e], w[e]);
        }
        // partners inside the thread (distances 8, 4, 2, 1, those below k)
#pragma unroll
        for (int j = EB_PER / 2; j > 0; j >>= 1) {
            if (j < k) {
#pragma unroll
                for (int e = 0; e < EB_PER; ++e) {
                    if ((e & j) == 0) {
                        const bool asc = ((base + e) & k) == 0;
                        const uint32_t a = v[e], b = v[e | j];
                        if ((a > b) == asc) { v[e] = b; v[e | j] = a; }
                    }
                }
            }
        }
    }
    // the key before this thread's first position (the sorted order is now v of thread t at
    // positions 16t + e)
    uint32_t* kb = keys + buf * EB_CHUNK;
    kb[base + EB_PER - 1] = v[EB_PER - 1];
    __syncthreads();
    const uint32_t before = tid > 0 ? kb[base - 1] : 0xFFFFFFFFu;
    int cs = 0, cr = 0;
    uint32_t prev = before;
#pragma unroll
    for (int e = 0; e < EB_PER; ++e) {
        const int i = base + e;
        if (i < n) {
            const bool run = i == 0 || (prev >> 14) != (v[e] >> 14);
            const bool seg = run || (i % EB_SEG) == 0;
            cs += seg;
            cr += run;
        }
        prev = v[e];
    }
    int ts, tr;
    eb_block_scan(cs, cr, ts, tr, wa, wb);
    if (tid == 0) {
        meta->nseg = ts;
        meta->nrun = tr;
        seg_begin[ts] = n;
        run_seg[tr] = ts;
    }
    int sg = cs - 1, r = cr - 1;
    prev = before;
#pragma unroll
    for (int e = 0; e < EB_PER; ++e) {
        const int i = base + e;
        if (i < n) {
            const uint32_t id = v[e] >> 14;
            const bool run = i == 0 || (prev >> 14) != id;
            const bool seg = run || (i % EB_SEG) == 0;
            if (seg) { ++sg; seg_begin[sg] = i; }
            if (run) { ++r; run_id[r] = (int32_t)id; run_seg[r] = sg; }
            srow[i] = (int32_t)(v[e] & 0x3FFF);
        }
        prev = v[e];
    }
}

template <typename T>
__global__ void eb_segment_kernel(const EbMeta* meta, const int32_t* __restrict__ srow,
                                  const int32_t* __restrict__ seg_begin, const T* __restrict__ dx, int row0,
                                  int C, float* __restrict__ part) {
    const int nseg = meta->nseg;
    const int nv = C >> 2;
    for (int sg = blockIdx.x; sg < nseg; sg += gridDim.x) {
        const int b = seg_begin[sg], e = seg_begin[sg + 1];
        for (int c = threadIdx.x; c < nv; c += blockDim.x) {
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int i = b; i < e; ++i) {
                const float4 v = load4<T>(dx + (int64_t)(row0 + srow[i]) * C + 4 * c);
                acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
            }
            ((float4*)(part + (int64_t)sg * C))[c] = acc;
        }
    }
}

__global__ void eb_run_kernel(const EbMeta* meta, const int32_t* __restrict__ run_id,
                              const int32_t* __restrict__ run_seg, const float* __restrict__ part, int C,
                              float* __restrict__ dwte) {
    const int nrun = meta->nrun;
    const int nv = C >> 2;
    for (int r = blockIdx.x; r < nrun; r += gridDim.x) {
        const int s0 = run_seg[r], s1 = run_seg[r + 1];
        float4* dst = (float4*)(dwte + (int64_t)run_id[r] * C);
        for (int c = threadIdx.x; c < nv; c += blockDim.x) {
            float4 acc = dst[c];
            for (int s = s0; s < s1; ++s) {
                const float4 v = ((const float4*)(part + (int64_t)s * C))[c];
                acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
            }
            dst[c] = acc;
        }
    }
}

template <typename S>
__global__ void dwpe_kernel(const S* __restrict__ dx, float* __restrict__ dwpe, int B, int T, int C, int accumulate) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over T*C
    if (i >= (int64_t)T * C) return;
    float s = 0.f;
    for (int b = 0; b < B; ++b) s += to_f<S>(dx[(int64_t)b * T * C + i]);
    dwpe[i] = accumulate ? dwpe[i] + s : s;
}

// the scratch's parts (layout as sized by embed_backward_scratch_bytes)
struct EbScratch {
    EbMeta* meta;
    int32_t *srow, *seg_begin, *run_id, *run_seg;
    float* part;
};
static EbScratch eb_scratch(void* scratch, int rows) {
    EbScratch e;
    char* p = (char*)scratch;
    e.meta = (EbMeta*)p;
    p += 256;
    const int n_max = rows < EB_CHUNK ? rows : EB_CHUNK;
    e.srow = (int32_t*)p; p += (size_t)n_max * 4;
    e.seg_begin = (int32_t*)p; p += (size_t)(n_max + 1) * 4;
    e.run_id = (int32_t*)p; p += (size_t)(n_max + 1) * 4;
    e.run_seg = (int32_t*)p; p += (size_t)(n_max + 1) * 4;
    size_t off = (size_t)(p - (char*)scratch);
    off = (off + 255) & ~(size_t)255;
    e.part = (float*)((char*)scratch + off);
    return e;
}
static hipError_t eb_sort_launch(const int32_t* idx, int n, const EbScratch& e, hipStream_t s) {
    hipLaunchKernelGGL(eb_sort_kernel, dim3(1), dim3(EB_THREADS), (size_t)2 * EB_CHUNK * 4, s, idx, n, e.meta, e.srow,
                       e.seg_begin, e.run_id, e.run_seg);
    return hipGetLastError();
}
bool embed_backward_presortable(int rows) { return rows > 0 && rows <= EB_CHUNK; }
hipError_t embed_backward_sort(const int32_t* idx, int rows, void* scratch, hipStream_t s) {
    if (!embed_backward_presortable(rows)) return hipErrorInvalidValue;
    return eb_sort_launch(idx, rows, eb_scratch(scratch, rows), s);
}

template <typename S>
static hipError_t embed_backward_t(const int32_t* idx, const S* dx, float* dwte, float* dwpe, int B, int T, int C,
                                   int accumulate_wpe, void* scratch, int presorted, hipStream_t s) {
    const int rows = B * T;
    const EbScratch es = eb_scratch(scratch, rows);
    EbMeta* meta = es.meta;
    int32_t *srow = es.srow, *seg_begin = es.seg_begin, *run_id = es.run_id, *run_seg = es.run_seg;
    float* part = es.part;
    if (presorted && !embed_backward_presortable(rows)) return hipErrorInvalidValue;
    for (int r0 = 0; r0 < rows; r0 += EB_CHUNK) {
        const int n = rows - r0 < EB_CHUNK ? rows - r0 : EB_CHUNK;
        hipError_t e = hipSuccess;
        if (!presorted && (e = eb_sort_launch(idx + r0, n, es, s)) != hipSuccess) return e;
        hipLaunchKernelGGL(eb_segment_kernel<S>, dim3(2048), dim3(C / 4 < 256 ? ((C / 4 + 63) / 64) * 64 : 256), 0, s,
                           meta, srow, seg_begin, dx, r0, C, part);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(eb_run_kernel, dim3(2048), dim3(C / 4 < 256 ? ((C / 4 + 63) / 64) * 64 : 256), 0, s,
                           meta, run_id, run_seg, part, C, dwte);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t tc = (int64_t)T * C;
    hipLaunchKernelGGL(dwpe_kernel<S>, dim3((unsigned)((tc + 255) / 256)), dim3(256), 0, s, dx, dwpe, B, T, C,
                       accumulate_wpe);
    return hipGetLastError();
}
hipError_t embed_backward(const int32_t* idx, const void* dx, float* dwte, float* dwpe, int B, int T, int C,
                          int accumulate_wpe, int is_bf16, void* scratch, int presorted, hipStream_t s) {
    if (is_bf16)
        return embed_backward_t(idx, (const bf16*)dx, dwte, dwpe, B, T, C, accumulate_wpe, scratch, presorted, s);
    return embed_backward_t(idx, (const float*)dx, dwte, dwpe, B, T, C, accumulate_wpe, scratch, presorted, s);
}

void rows_setup() {
    // the id sort exchanges keys through two LDS buffers of EB_CHUNK 4-byte keys
    (void)hipFuncSetAttribute((const void*)eb_sort_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              2 * EB_CHUNK * 4);
}

// ================================================================== gradient norm + AdamW
// norm = sqrt(sum g^2) over the whole gradient arena (wte once), clip coefficient
// c = min(1, max_norm/(norm + 1e-6)) as clip_grad_norm_ computes it (chapter 2:14:58-2:25:57).
constexpr int NORM_BLOCKS = 1024;
int norm_blocks() { return NORM_BLOCKS; }

__global__ void norm_partial_kernel(const float* __restrict__ g, int64_t n4, float* __restrict__ partial) {
    __shared__ float red[4];
    float s = 0.f;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        const float4 v = ((const float4*)g)[i];
        s += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
    }
    s = block_sum<256>(s, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

__global__ void norm_final_kernel(const float* __restrict__ partial, int np, const float* __restrict__ tail,
                                  int ntail, float* __restrict__ out, float max_norm) {
    __shared__ double red[1024];
    double s = 0.0;
    for (int i = threadIdx.x; i < np; i += 1024) s += partial[i];
    if (threadIdx.x == 0)
        for (int i = 0; i < ntail; ++i) s += (double)tail[i] * tail[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double norm = sqrt(red[0]);
        double c = (double)max_norm / (norm + 1e-6);
        if (c > 1.0) c = 1.0;
        out[0] = (float)norm;
        out[1] = (float)c;
    }
}

hipError_t grad_norm(const float* g, int64_t n, float* partial, float* d_norm_coef, float max_norm, hipStream_t s) {
    const int64_t n4 = n / 4;
    hipLaunchKernelGGL(norm_partial_kernel, dim3(NORM_BLOCKS), dim3(256), 0, s, g, n4, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(norm_final_kernel, dim3(1), dim3(1024), 0, s, partial, NORM_BLOCKS, g + n4 * 4, (int)(n - n4 * 4),
                       d_norm_coef, max_norm);
    return hipGetLastError();
}

// AdamW, PyTorch form (chapter 52:38-1:06:18 shows its documentation; weight decay only on
// the 2-D tensors, chapter 2:25:57-2:34:49): p *= 1 - lr*wd; m = b1 m + (1-b1) g;
// v = b2 v + (1-b2) g^2; p -= (lr/bc1) * m / (sqrt(v)/sqrt(bc2) + eps), g = c * grad.
// The bf16 copy of the 2-D weights used by the products is refreshed in the same pass.
DEV void adamw4(float4& pp, const float4& gg, float4& mm, float4& vv, float keep, float c, float beta1,
                float beta2, float eps, float step, float inv_bc2_sqrt) {
    float* pa = (float*)&pp;
    const float* ga = (const float*)&gg;
    float* ma = (float*)&mm;
    float* va = (float*)&vv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float gq = c * ga[q];
        pa[q] *= keep;
        ma[q] = beta1 * ma[q] + (1.0f - beta1) * gq;
        va[q] = beta2 * va[q] + (1.0f - beta2) * gq * gq;
        const float den = sqrtf(va[q]) * inv_bc2_sqrt + eps;
        pa[q] -= step * (ma[q] / den);
    }
}
DEV void store_shadow4(bf16* sh, int64_t i, const float4& pp) {
    bf16x4 b;
    b[0] = (bf16)pp.x; b[1] = (bf16)pp.y; b[2] = (bf16)pp.z; b[3] = (bf16)pp.w;
    ((bf16x4*)sh)[i] = b;
}
// Each workgroup updates AW_UNROLL * 256 consecutive float4 groups of every array, one pass
// (no grid-stride loop): thread t takes groups t, t + 256, ... of them, every load issued before
// any arithmetic so their memory latency overlaps. Every array is touched once, so the accesses
// are non-temporal (no cache lines kept for them). A probe of this access mix (four fp32 streams
// read, three fp32 and one bf16 written) measured 5.7 TB/s in this shape against 4.4-4.5 TB/s
// with a fixed grid striding over the arrays.
constexpr int AW_UNROLL = 4;
typedef float f32x4 __attribute__((ext_vector_type(4)));
DEV float4 ntload(const float* p, int64_t i) {
    const f32x4 v = __builtin_nontemporal_load((const f32x4*)p + i);
    return make_float4(v[0], v[1], v[2], v[3]);
}
DEV void ntstore(float* p, int64_t i, const float4& v) {
    const f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (f32x4*)p + i);
}
__global__ void __launch_bounds__(256) adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    bf16* __restrict__ shadow, int64_t n4, int64_t n_decay4,
                                                    const float* __restrict__ norm_coef, float lr, float beta1,
                                                    float beta2, float eps, float wd, float bc1, float bc2_sqrt,
                                                    const float* __restrict__ hp) {
    const float c = norm_coef[1];
    if (hp) {   // (lr, bc1, sqrt(bc2)) from device memory, as the schedule left them
        lr = hp[0];
        bc1 = hp[1];
        bc2_sqrt = hp[2];
    }
    const float step = lr / bc1, inv_bc2_sqrt = 1.0f / bc2_sqrt, kd = 1.0f - lr * wd;
    const int64_t i0 = (int64_t)blockIdx.x * (AW_UNROLL * 256) + threadIdx.x;
    float4 pp[AW_UNROLL], gg[AW_UNROLL], mm[AW_UNROLL], vv[AW_UNROLL];
#pragma unroll
    for (int u = 0; u < AW_UNROLL; ++u) {
        const int64_t i = i0 + u * 256;
        if (i < n4) {
            pp[u] = ntload(p, i); mm[u] = ntload(m, i); vv[u] = ntload(v, i); gg[u] = ntload(g, i);
        }
    }
#pragma unroll
    for (int u = 0; u < AW_UNROLL; ++u) {
        const int64_t i = i0 + u * 256;
        if (i < n4) {
            adamw4(pp[u], gg[u], mm[u], vv[u], i < n_decay4 ? kd : 1.0f, c, beta1, beta2, eps, step, inv_bc2_sqrt);
            ntstore(p, i, pp[u]); ntstore(m, i, mm[u]); ntstore(v, i, vv[u]);
            if (shadow && i < n_decay4) store_shadow4(shadow, i, pp[u]);
        }
    }
}

hipError_t adamw(float* p, const float* g, float* m, float* v, void* shadow, int64_t n, int64_t n_decay,
                 const float* d_norm_coef, float lr, float beta1, float beta2, float eps, float wd, float bc1,
                 float bc2_sqrt, const float* d_hp, hipStream_t s) {
    if ((n & 3) || (n_decay & 3)) return hipErrorInvalidValue;
    const int64_t nblk = (n / 4 + AW_UNROLL * 256 - 1) / (AW_UNROLL * 256);
    if (nblk < 1) return hipSuccess;
    if (nblk > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)nblk), dim3(256), 0, s, p, g, m, v, (bf16*)shadow, n / 4, n_decay / 4,
                       d_norm_coef, lr, beta1, beta2, eps, wd, bc1, bc2_sqrt, d_hp);
    return hipGetLastError();
}

// AdamW's per-step scalars from a learning rate and step count in device memory: hp = (lr,
// 1 - beta1^t, sqrt(1 - beta2^t)), computed in double and rounded once, as the host path does.
__global__ void adamw_hparams_kernel(const float* __restrict__ d_lr, const int32_t* __restrict__ d_t, double beta1,
                                     double beta2, float* __restrict__ hp) {
    if (threadIdx.x != 0) return;
    const double t = (double)*d_t;
    hp[0] = *d_lr;
    hp[1] = (float)(1.0 - pow(beta1, t));
    hp[2] = (float)sqrt(1.0 - pow(beta2, t));
}
hipError_t adamw_hparams(const float* d_lr, const int32_t* d_t, float beta1, float beta2, float* d_hp, hipStream_t s) {
    hipLaunchKernelGGL(adamw_hparams_kernel, dim3(1), dim3(64), 0, s, d_lr, d_t, (double)beta1, (double)beta2, d_hp);
    return hipGetLastError();
}

// One step of the learning-rate schedule in device memory: with it = *d_step, *d_lr = the
// schedule's rate at it (linear warmup, cosine decay to min_lr, min_lr after max_steps; the
// same double arithmetic as the host function), *d_t = it + 1 (AdamW's step count), and
// *d_step = it + 1.
__global__ void schedule_step_kernel(int32_t* __restrict__ d_step, float* __restrict__ d_lr, int32_t* __restrict__ d_t,
                                     double max_lr, double min_lr, int64_t warmup, int64_t max_steps) {
    if (threadIdx.x != 0) return;
    const int64_t it = *d_step;
    double lr;
    if (it < warmup) {
        lr = max_lr * (double)(it + 1) / (double)warmup;
    } else if (it > max_steps) {
        lr = min_lr;
    } else {
        const double ratio = (double)(it - warmup) / (double)(max_steps - warmup);
        lr = min_lr + 0.5 * (1.0 + cos(3.14159265358979323846 * ratio)) * (max_lr - min_lr);
    }
    *d_lr = (float)lr;
    *d_t = (int32_t)(it + 1);
    *d_step = (int32_t)(it + 1);
}
hipError_t schedule_step(int32_t* d_step, float* d_lr, int32_t* d_t, double max_lr, double min_lr, int64_t warmup,
                         int64_t max_steps, hipStream_t s) {
    hipLaunchKernelGGL(schedule_step_kernel, dim3(1), dim3(64), 0, s, d_step, d_lr, d_t, max_lr, min_lr, warmup,
                       max_steps);
    return hipGetLastError();
}

__global__ void shadow_kernel(const float* __restrict__ p, bf16* __restrict__ sh, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        sh[i] = (bf16)p[i];
}
hipError_t refresh_shadow(const float* p, void* shadow, int64_t n, hipStream_t s) {
    hipLaunchKernelGGL(shadow_kernel, dim3(4096), dim3(256), 0, s, p, (bf16*)shadow, n);
    return hipGetLastError();
}

// ================================================================== initialization
// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC'11): 10 rounds of two 32x32->64 multiplies with the published multipliers and Weyl
// key increments. Uniforms from the 4 outputs feed two Box-Muller transforms.
DEV void philox_round(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
}

__global__ void init_normal_kernel(float* __restrict__ p, int64_t n, float stdv, uint64_t seed, uint64_t offset) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i * 4 < n; i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t ctr = offset + (uint64_t)i;
        uint32_t c[4] = {(uint32_t)ctr, (uint32_t)(ctr >> 32), 0u, 0u};
        uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
        for (int r = 0; r < 10; ++r) {
            philox_round(c, k0, k1);
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        float z[4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const float u1 = ((float)(c[2 * q] >> 8) + 0.5f) * (1.0f / 16777216.0f);
            const float u2 = ((float)(c[2 * q + 1] >> 8) + 0.5f) * (1.0f / 16777216.0f);
            const float rad = sqrtf(-2.0f * logf(u1));
            float sn, cs;
            sincosf(6.283185307179586f * u2, &sn, &cs);
            z[2 * q] = rad * cs;
            z[2 * q + 1] = rad * sn;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (i * 4 + q < n) p[i * 4 + q] = stdv * z[q];
    }
}
hipError_t init_normal(float* p, int64_t n, float stdv, uint64_t seed, uint64_t offset, hipStream_t s) {
    hipLaunchKernelGGL(init_normal_kernel, dim3(2048), dim3(256), 0, s, p, n, stdv, seed, offset);
    return hipGetLastError();
}

__global__ void fill_kernel(float* __restrict__ p, int64_t n, float v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}
hipError_t fill(float* p, int64_t n, float v, hipStream_t s) {
    hipLaunchKernelGGL(fill_kernel, dim3(2048), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

}  // namespace gpt2k
