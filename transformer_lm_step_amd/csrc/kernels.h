// Host-side launchers of the GPT-2 step kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt2k {

// ------------------------------------------------------------------ GEMM
enum Epi {
    EPI_BIAS_T = 0,          // C(T)   = alpha*acc + bias[n]           (bias may be null)
    EPI_BIAS_GELU = 2,       // C(T)   = u = acc + bias[n];  C2(T) = gelu_tanh(u)
    EPI_GELU_BWD = 3,        // C(T)   = acc * gelu_tanh'(aux[m][n])
    EPI_F32 = 4,             // C(f32) = (beta ? C : 0) + alpha*acc
    EPI_PARTIAL = 5,         // internal: split-K partials
    EPI_LOGITS = 6,          // C(bf16) = alpha*acc + bias[n], and C2 (fp32 pairs) = for every row m
                             // and 192-column tile t: (max, sum exp(z - max)) of that row's
                             // bf16-rounded outputs in the tile, at C2[2 * (m * tiles + t)]
};

struct GemmDesc {
    const void* A = nullptr; int64_t lda = 0; int a_layout = 0;  // 0: A[m*lda+k], 1: A[k*lda+m]
    const void* B = nullptr; int64_t ldb = 0; int b_layout = 0;  // 0: B[n*ldb+k], 1: B[k*ldb+n]
    int M = 0, N = 0, K = 0;
    int epi = EPI_BIAS_T;
    void* C = nullptr; int64_t ldc = 0;
    void* C2 = nullptr;
    const float* bias = nullptr;
    const void* aux = nullptr; int64_t ldaux = 0;
    float alpha = 1.f;
    int beta = 0;
    int nsplit = 1;          // split K into this many parts (EPI_F32 with ldc == N only)
    void* partial = nullptr; // fp32 scratch of nsplit*M*N floats when nsplit > 1
    int bm = 0, bn = 0;      // block tile (0: chosen from the shape)
    int no_dl = 0;           // 1: never use the direct global->LDS load path
    // optional with a_layout 1 (A[k*lda + m]): rowsum[m] (+= if beta) sum_k A(m, k), i.e. the
    // bias gradient of a weight-gradient product; rowsum_part holds nsplit*M floats
    float* rowsum = nullptr;
    float* rowsum_part = nullptr;
    // few-row products only (decoding): the output starts min(*c_row_dev, c_row_max) * c_row_bytes
    // bytes past C, a row offset read from device memory when the kernel runs
    const int32_t* c_row_dev = nullptr;
    int64_t c_row_bytes = 0;
    int c_row_max = 0;
};

hipError_t gemm(const GemmDesc& d, int is_bf16, hipStream_t s);
// Decoding: a few-row bf16 product (EPI_BIAS_T or EPI_BIAS_GELU, A contiguous [M, K]) whose A
// rows are LayerNorm(x + y) of the residual stream, computed inside the product; x_out (if
// not null) receives x + y. y may be null (no add). gemm_skinny_ln_ok says whether d qualifies.
struct SkinnyLn {
    const void* x;      // residual stream rows [M, K] (fp32, or bf16 with x_bf16)
    const void* y;      // projection output rows [M, K] bf16, or null
    void* x_out;        // x + y (the stream's type), or null
    const float* w;     // LayerNorm weight and bias [K]
    const float* b;
};
int gemm_skinny_ln_ok(const GemmDesc& d, int is_bf16);
hipError_t gemm_skinny_ln(const GemmDesc& d, const SkinnyLn& ln, int x_bf16, hipStream_t s);
// per-kernel timing of the products: hand over an event pair before a product call; after it,
// gemm_time_taken() says whether the product was a single kernel that recorded the pair at its
// own start and end (and forgets the pair either way)
void gemm_time_next(hipEvent_t start, hipEvent_t stop);
bool gemm_time_taken();
// number of 192-column tiles (the C2 row length of EPI_LOGITS) if gemm() can run d with
// EPI_LOGITS (bf16, both operands k-contiguous, whole 128 x 192 tiles), else 0
int gemm_logits_tiles(const GemmDesc& d, int is_bf16);
// 1 if gemm() computes d.rowsum itself (LDS-streamed bf16 path), 0 if the caller must
int gemm_fuses_rowsum(const GemmDesc& d, int is_bf16);
void gemm_pick_tile(int M, int N, int nsplit, int is_bf16, int* bm, int* bn);

// Grouped weight-gradient products (bf16 operands, LDS-streamed path): product i computes
//   C_i[m][n] = (beta ? C_i : 0) + alpha * sum_k A_i[k*lda_i + m] * B_i[k*ldb_i + n]
// over the shared K (dW = dY^T X with K = tokens), and with rowsum_i non-null also
//   rowsum_i[m] = (beta ? rowsum_i : 0) + sum_k A_i[k*lda_i + m]      (the bias gradient).
// One launch of 128 x bn tiles; the products' tile ranges [tile0, tile0 + ntiles) are
// consecutive and ascending (ntiles = gemm_group_tiles(M, N, bn)). Every output element is
// one workgroup's fixed-order sum over K (deterministic, no split-K).
struct GroupProb {
    const void* A; const void* B; float* C; float* rowsum;
    int64_t lda, ldb, ldc;
    int M, N;
    int tile0, ntiles;
};
int gemm_group_tiles(int M, int N, int bn);
bool gemm_group_ok(const GroupProb& g, int K);   // the LDS-streamed path's shape rules hold
hipError_t gemm_grouped(const GroupProb* d_probs, int nprob, int total_tiles, int K, float alpha, int beta, int bn,
                        hipStream_t s);
void gemm_setup();
size_t gemm_lds_bytes();

// ------------------------------------------------------------------ elementwise / rows
// x [B*T, C] = wte[idx] + wpe[t], x in bf16 if x_bf16 else fp32 (the residual stream's type)
hipError_t embed_forward(const int32_t* idx, const float* wte, const float* wpe, void* x, int B, int T,
                         int C, int x_bf16, hipStream_t s, const int32_t* d_pos = nullptr,
                         int pos_max = 0);
// LayerNorm forward: out = (x - mean) * rstd * w + b ; saves mean, rstd (fp32). x is bf16 if
// x_bf16 (the bf16 residual stream) else fp32; out is bf16 if out_bf16 else fp32.
hipError_t layernorm_forward(const void* x, const float* w, const float* b, void* out, float* mean,
                             float* rstd, int rows, int C, int x_bf16, int out_bf16, hipStream_t s);
// Residual add and LayerNorm: x_new = x_old + y (fp32 add, stored in the residual type: bf16
// if x_bf16 else fp32), out = LayerNorm(x_new) with mean, rstd saved; y and out in the operand
// type (bf16 if op_bf16 else fp32).
hipError_t add_layernorm_forward(const void* x_old, const void* y, void* x_new, const float* w, const float* b,
                                 void* out, float* mean, float* rstd, int rows, int C, int x_bf16, int op_bf16,
                                 hipStream_t s);
// LayerNorm backward: dres = (accumulate ? dres : 0) + dx ; partial[blk][0:C] = sum dh*xhat,
// [C:2C] = sum dh, [2C:3C] = sum of the incoming dres (zero without accumulate) over the
// block's rows. dh is bf16 if dh_bf16 else fp32; x and dres are bf16 if res_bf16 else fp32;
// dres16 (nullable) receives a bf16 copy of the new dres.
hipError_t layernorm_backward(const void* dh, const void* x, const float* mean, const float* rstd,
                              const float* w, void* dres, void* dres16, int accumulate_dres,
                              float* partial, int nblk, int rows, int C, int dh_bf16, int res_bf16, hipStream_t s);
int layernorm_backward_blocks(int rows);
int layernorm_backward_max_blocks(int max_rows);
// out[c] (+)= sum_blk partial[blk*stride + c] for c < n (fixed order); scratch holds
// sum_scratch_floats(n) floats
hipError_t sum_partials(const float* partial, int nblk, int n, int64_t stride, float* out, int accumulate,
                        float* scratch, hipStream_t s);
int sum_scratch_floats(int n);
// the same with two destinations: columns [0, n1) into out1, [n1, n) into out2
hipError_t sum_partials2(const float* partial, int nblk, int n, int64_t stride, float* out1, int n1, float* out2,
                         int accumulate, float* scratch, hipStream_t s);
// sum_partials2 over nset partial sets of the same shape in one pass (set i at partial +
// i*set_stride): columns [0, n1) of set i into base + off1[i], [n1, n) into base + off2[i]
// (skipped when off2[i] < 0); off1, off2 are device arrays of nset offsets (floats); the
// per-column order, and so every result, is sum_partials2's. scratch holds
// sum_sets_scratch_floats(nset, n) floats.
hipError_t sum_partials_sets(const float* partial, int nset, int64_t set_stride, int nblk, int n, int64_t stride,
                             float* base, const int64_t* off1, int n1, const int64_t* off2, int accumulate,
                             float* scratch, hipStream_t s);
int sum_sets_scratch_floats(int nset, int n);
// column sums of a [rows, n] matrix (storage T or f32) into out[n] (+)=, deterministic
hipError_t colsum(const void* x, int x_is_f32, int is_bf16, int rows, int n, float* partial,
                  float* out, int accumulate, float* scratch, hipStream_t s);
int colsum_partial_floats(int rows, int n);

// cross-entropy over rows of logits(T) [n_rows, Vp]: loss_rows[r] = lse - z[y]; with
// write_grad the logits are overwritten by dz = (softmax - onehot) / n_rows; optional fp32
// copy of the logits.
hipError_t cross_entropy(void* logits, const int32_t* targets, float* loss_rows, float* logits_f32,
                         int n_rows, int Vp, int is_bf16, hipStream_t s, int write_grad = 1);
// the same for bf16 logits whose per-tile softmax statistics the lm_head product produced
// (EPI_LOGITS: `tiles` (max, sum) pairs per row): one pass over each row instead of two, and
// none without write_grad or logits_f32; lse2_rows [n_rows] receives each row's log-sum-exp
// times log2(e) (scratch of the gradient pass)
hipError_t cross_entropy_tiled(void* logits, const float* stats, int tiles, const int32_t* targets,
                               float* loss_rows, float* lse2_rows, float* logits_f32, int n_rows, int Vp,
                               hipStream_t s, int write_grad = 1);
// per sequence b of B (T positions): sum, count and mean of loss_rows over the positions the
// mask selects (mask null: all); rowd [2B] doubles (sum, count); row_sum / row_mean / total
// may be null; total = mean over every selected position of the batch
hipError_t masked_row_loss(const float* loss_rows, const uint8_t* mask, int B, int T, double* rowd,
                           float* row_sum, float* row_mean, float* total, hipStream_t s);
hipError_t convert_to_f32(const void* src, float* dst, int64_t n, int is_bf16, hipStream_t s);
// mean of loss_rows -> *d_loss (single block, fixed order)
hipError_t mean_reduce(const float* v, int n, float* d_out, hipStream_t s);

// embedding backward (deterministic): dwte[idx[r]] += dx[r] in ascending r, dwpe[t] (+)= sum_b dx[b,t];
// dx (the residual stream's gradient) is bf16 if is_bf16, else fp32
size_t embed_backward_scratch_bytes(int rows, int C);
void rows_setup();
// With presorted, the id sort of the rows was already issued by embed_backward_sort (on a
// stream ordered before s): possible when embed_backward_presortable(rows), one sort chunk.
hipError_t embed_backward(const int32_t* idx, const void* dx, float* dwte, float* dwpe, int B, int T,
                          int C, int accumulate_wpe, int is_bf16, void* scratch, int presorted, hipStream_t s);
bool embed_backward_presortable(int rows);
// the id sort alone (it depends only on idx), into the same scratch
hipError_t embed_backward_sort(const int32_t* idx, int rows, void* scratch, hipStream_t s);

// global grad norm + clip coefficient, AdamW
int norm_blocks();
hipError_t grad_norm(const float* g, int64_t n, float* partial, float* d_norm_coef /* [2] */,
                     float max_norm, hipStream_t s);
// (d_hp, when not null: device (lr, bc1, bc2_sqrt) that replace the three scalars)
hipError_t adamw(float* p, const float* g, float* m, float* v, void* shadow_bf16, int64_t n,
                 int64_t n_decay, const float* d_norm_coef, float lr, float beta1, float beta2,
                 float eps, float wd, float bc1, float bc2_sqrt, const float* d_hp, hipStream_t s);
// d_hp = (*d_lr, 1 - beta1^*d_t, sqrt(1 - beta2^*d_t)) in device memory
hipError_t adamw_hparams(const float* d_lr, const int32_t* d_t, float beta1, float beta2, float* d_hp, hipStream_t s);
// the learning-rate schedule advanced in device memory (see the kernel)
hipError_t schedule_step(int32_t* d_step, float* d_lr, int32_t* d_t, double max_lr, double min_lr, int64_t warmup,
                         int64_t max_steps, hipStream_t s);
hipError_t refresh_shadow(const float* p, void* shadow_bf16, int64_t n, hipStream_t s);

// device init: counter-based normals (Philox-4x32-10 + Box-Muller) times std, or constants
hipError_t init_normal(float* p, int64_t n, float stdv, uint64_t seed, uint64_t offset, hipStream_t s);
hipError_t fill(float* p, int64_t n, float v, hipStream_t s);

// ------------------------------------------------------------------ attention
// qkv(T) [B*T, 3C] (q | k | v, head h = columns h*hs..), y(T) [B*T, C], lse fp32 [B*H*T]
hipError_t attention_forward(const void* qkv, void* y, float* lse, int B, int T, int H, int hs,
                             int is_bf16, hipStream_t s);
// dy(T) [B*T, C], D scratch fp32 [2*B*H*T] (the softmax-gradient term per query, then the
// log-sum-exp in base 2 for the key-block kernel), dqkv(T) [B*T, 3C]
hipError_t attention_backward(const void* qkv, const void* y, const void* dy, const float* lse,
                              float* D, void* dqkv, int B, int T, int H, int hs, int is_bf16,
                              hipStream_t s);
void attention_setup();

// ------------------------------------------------------------------ incremental decoding
// attention of the query at position pos of each of B sequences over the cached keys/values
// at 0..pos; qkv rows (b, t) -> b*Tmax + t (3C wide), y(T) [B, C]
hipError_t attention_decode(const void* qkv, void* y, int B, int Tmax, int pos, int H, int hs, int is_bf16,
                            hipStream_t s, const int32_t* d_pos = nullptr);
// *d_pos = min(*d_pos + 1, pos_end): the next decoding position, advanced on the device
hipError_t decode_advance(int32_t* d_pos, int pos_end, hipStream_t s);
size_t attention_decode_lds(int hs, int Tmax);
// top-k of each logits row (T) [B, Vp] (larger first, ties by lower id), their renormalized
// softmax, and the inverse-CDF draw with u[b] in [0, 1); every output pointer may be null
// except u when next is set
constexpr int TOPK_MAX = 64;
hipError_t topk_sample(const void* logits, int B, int Vp, int k, const float* u, int32_t* next, int32_t* topk_idx,
                       float* topk_prob, int is_bf16, hipStream_t s);

}  // namespace gpt2k
