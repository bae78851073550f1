// C ABI of the GPT-2 training-step library: configuration, canonical parameter layout,
// workspace carving, and the launch sequences of forward, backward and the optimizer.
// Everything here is host code; every operation of the step runs in the kernels of
// gemm.hip, attention.hip and rows.hip on the handle's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gpt2.h"
#include "kernels.h"

using namespace gpt2k;

namespace {

thread_local std::string g_last_error;

int set_error(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

// strict: also the shape requirements of the kernels (needed to size or create a handle);
// otherwise only what the parameter layout needs (counting functions)
bool config_ok(const gpt2_config* c, std::string* why, bool strict = true) {
    auto bad = [&](const char* m) { if (why) *why = m; return false; };
    if (!c) return bad("config is null");
    if (c->n_layer < 1 || c->n_head < 1 || c->n_embd < 1 || c->mlp_hidden < 1 || c->block_size < 1 ||
        c->vocab_size < 1 || c->max_batch < 1)
        return bad("config fields must be positive");
    if (c->n_embd % c->n_head) return bad("n_embd must be a multiple of n_head");
    if (c->padded_vocab_size < c->vocab_size) return bad("padded_vocab_size must be >= vocab_size");
    if (c->dtype != GPT2_FP32 && c->dtype != GPT2_BF16 && c->dtype != GPT2_BF16_RES16)
        return bad("dtype must be GPT2_FP32, GPT2_BF16 or GPT2_BF16_RES16");
    if (!strict) return true;
    const int hs = c->n_embd / c->n_head;
    if (hs != 64 && hs != 32) return bad("head size n_embd/n_head must be 32 or 64");
    if (c->n_embd % 8 || c->mlp_hidden % 8) return bad("n_embd and mlp_hidden must be multiples of 8");
    if (c->n_embd > 2048) return bad("n_embd above 2048 is not supported by the LayerNorm kernels");
    if (c->padded_vocab_size % 8) return bad("padded_vocab_size must be a multiple of 8");
    if (c->padded_vocab_size >= (1 << 18)) return bad("padded_vocab_size must be below 262144");
    if ((int64_t)c->max_batch * c->block_size > (1 << 30)) return bad("max_batch*block_size too large");
    return true;
}

struct Layout {
    // parameter arena
    int64_t n_params = 0, decay_end = 0;
    int64_t wte = 0, wpe = 0, lnf_w = 0, lnf_b = 0;
    std::vector<int64_t> w_qkv, w_o, w_fc, w_pr, ln1_w, ln1_b, b_qkv, b_o, ln2_w, ln2_b, b_fc, b_pr;
};

Layout make_layout(const gpt2_config* c) {
    Layout L;
    const int64_t C = c->n_embd, F = c->mlp_hidden, Vp = c->padded_vocab_size;
    int64_t o = 0;
    L.wte = o; o += Vp * C;
    L.wpe = o; o += (int64_t)c->block_size * C;
    for (int l = 0; l < c->n_layer; ++l) {
        L.w_qkv.push_back(o); o += 3 * C * C;
        L.w_o.push_back(o); o += C * C;
        L.w_fc.push_back(o); o += F * C;
        L.w_pr.push_back(o); o += C * F;
    }
    L.decay_end = o;
    for (int l = 0; l < c->n_layer; ++l) {
        L.ln1_w.push_back(o); o += C;
        L.ln1_b.push_back(o); o += C;
        L.b_qkv.push_back(o); o += 3 * C;
        L.b_o.push_back(o); o += C;
        L.ln2_w.push_back(o); o += C;
        L.ln2_b.push_back(o); o += C;
        L.b_fc.push_back(o); o += F;
        L.b_pr.push_back(o); o += C;
    }
    L.lnf_w = o; o += C;
    L.lnf_b = o; o += C;
    L.n_params = o;
    return L;
}

// name/offset/shape of tensor i of the canonical arena
bool tensor_info(const gpt2_config* c, int i, std::string* name, int64_t* off, int64_t* r, int64_t* cc) {
    const Layout L = make_layout(c);
    const int64_t C = c->n_embd, F = c->mlp_hidden;
    const int nl = c->n_layer;
    char buf[96];
    if (i < 0) return false;
    if (i == 0) { *name = "wte"; *off = L.wte; *r = c->padded_vocab_size; *cc = C; return true; }
    if (i == 1) { *name = "wpe"; *off = L.wpe; *r = c->block_size; *cc = C; return true; }
    i -= 2;
    if (i < 4 * nl) {
        const int l = i / 4, j = i % 4;
        static const char* nm[4] = {"attn.c_attn.weight", "attn.c_proj.weight", "mlp.c_fc.weight", "mlp.c_proj.weight"};
        snprintf(buf, sizeof(buf), "h.%d.%s", l, nm[j]);
        *name = buf;
        const int64_t offs[4] = {L.w_qkv[l], L.w_o[l], L.w_fc[l], L.w_pr[l]};
        const int64_t rows[4] = {3 * C, C, F, C}, cols[4] = {C, C, C, F};
        *off = offs[j]; *r = rows[j]; *cc = cols[j];
        return true;
    }
    i -= 4 * nl;
    if (i < 8 * nl) {
        const int l = i / 8, j = i % 8;
        static const char* nm[8] = {"ln_1.weight", "ln_1.bias", "attn.c_attn.bias", "attn.c_proj.bias",
                                    "ln_2.weight", "ln_2.bias", "mlp.c_fc.bias", "mlp.c_proj.bias"};
        snprintf(buf, sizeof(buf), "h.%d.%s", l, nm[j]);
        *name = buf;
        const int64_t offs[8] = {L.ln1_w[l], L.ln1_b[l], L.b_qkv[l], L.b_o[l], L.ln2_w[l], L.ln2_b[l], L.b_fc[l], L.b_pr[l]};
        const int64_t len[8] = {C, C, 3 * C, C, C, C, F, C};
        *off = offs[j]; *r = len[j]; *cc = 0;
        return true;
    }
    i -= 8 * nl;
    if (i == 0) { *name = "ln_f.weight"; *off = L.lnf_w; *r = C; *cc = 0; return true; }
    if (i == 1) { *name = "ln_f.bias"; *off = L.lnf_b; *r = C; *cc = 0; return true; }
    return false;
}

// Split-K factor and tile width of a weight-gradient product (M x N, K = tokens): as many
// splits as fit in one round of 512 workgroups (two per CU; a partial second round would take
// as long as the first, and every split adds M*N*4 bytes of partials), at least 4 K-tiles per
// split, at most 16 splits. 128x192 tiles are taken when they fill the round better.
struct Split {
    int ns = 1, bn = 128;
};
Split choose_split(int M, int N, int K, bool bf16) {
    const int BK = bf16 ? 64 : 32;
    const int ktiles = (K + BK - 1) / BK;
    auto pick = [&](int bn, double* fill) {
        const int tiles = ((M + 127) / 128) * ((N + bn - 1) / bn);
        int s = 512 / tiles;
        if (s > 16) s = 16;
        if (s > ktiles / 4) s = ktiles / 4;
        if (s < 1) s = 1;
        const int64_t blocks = (int64_t)tiles * s, rounds = (blocks + 511) / 512;
        *fill = (double)blocks / (double)(rounds * 512);
        return s;
    };
    Split r;
    double f128 = 0.0, f192 = 0.0;
    r.ns = pick(128, &f128);
    if (bf16 && N % 192 == 0) {
        const int s192 = pick(192, &f192);
        if (f192 > f128 + 0.01) {
            r.ns = s192;
            r.bn = 192;
        }
    }
    return r;
}

struct Plan {
    size_t total = 0;
    // offsets in bytes
    size_t params, grads, m, v, shadow, idx, tgt;
    std::vector<size_t> x_in, x_mid, h1, mean1, rstd1, qkv, att, lse, h2, mean2, rstd2, u, a;
    size_t hf, meanf, rstdf, logits, lstats, lse2rows, loss_rows, loss, dres, dln, datt, Dbuf;
    size_t yproj;          // a projection's output with its bias, before the residual add
    // output gradients that feed products: per layer in the bf16 modes (kept for the grouped
    // weight-gradient launch at the end of the backward), one shared buffer in fp32 mode
    std::vector<size_t> du, dqkv;
    // bf16 copies of the residual gradient at each layer's output and after its attention
    std::vector<size_t> d16o, d16m;
    size_t gprob;          // GroupProb table of the grouped weight-gradient launch (4 per layer)
    size_t splitk, rspart, lnpart, cspart, sumscr, normpart, normcoef, ebscratch;
    // LayerNorm backward partials: one set per LayerNorm (ln_f, then ln_2 and ln_1 of each layer
    // from the last), reduced together after the backward; the sets' gradient offsets
    size_t lnset_stride, lnscr, lnoff;
    size_t mask, rowd;   // evaluation: copied mask, per-sequence double sums and counts
};

Plan make_plan(const gpt2_config* c) {
    Plan P;
    const Layout L = make_layout(c);
    const bool bf = c->dtype != GPT2_FP32;
    const size_t es = bf ? 2 : 4;                                  // operands and activations
    const size_t er = c->dtype == GPT2_BF16_RES16 ? 2 : 4;         // residual stream and its gradient
    const int64_t BT = (int64_t)c->max_batch * c->block_size;
    const int64_t C = c->n_embd, F = c->mlp_hidden, Vp = c->padded_vocab_size, H = c->n_head;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 255) & ~(size_t)255; return r; };
    P.params = take(L.n_params * 4);
    P.grads = take(L.n_params * 4);
    P.m = take(L.n_params * 4);
    P.v = take(L.n_params * 4);
    P.shadow = bf ? take(L.decay_end * 2) : 0;
    P.idx = take(BT * 4);
    P.tgt = take(BT * 4);
    for (int l = 0; l <= c->n_layer; ++l) P.x_in.push_back(take(BT * C * er));
    for (int l = 0; l < c->n_layer; ++l) {
        P.x_mid.push_back(take(BT * C * er));
        P.h1.push_back(take(BT * C * es));
        P.mean1.push_back(take(BT * 4));
        P.rstd1.push_back(take(BT * 4));
        P.qkv.push_back(take(BT * 3 * C * es));
        P.att.push_back(take(BT * C * es));
        P.lse.push_back(take(BT * H * 4));
        P.h2.push_back(take(BT * C * es));
        P.mean2.push_back(take(BT * 4));
        P.rstd2.push_back(take(BT * 4));
        P.u.push_back(take(BT * F * es));
        P.a.push_back(take(BT * F * es));
    }
    P.yproj = take(BT * C * es);
    P.hf = take(BT * C * es);
    P.meanf = take(BT * 4);
    P.rstdf = take(BT * 4);
    P.logits = take(BT * Vp * es);
    P.lstats = take(BT * ((Vp + 191) / 192) * 8);   // per row and 192-column tile: (max, sum)
    P.lse2rows = take(BT * 4);                        // per row: log-sum-exp * log2(e)
    P.loss_rows = take(BT * 4);
    P.loss = take(256);
    P.mask = take(BT);
    P.rowd = take((size_t)c->max_batch * 2 * 8);
    P.dres = take(BT * C * er);
    P.dln = take(BT * C * es);
    P.datt = take(BT * C * es);
    for (int l = 0; l < (bf ? c->n_layer : 1); ++l) {
        P.dqkv.push_back(take(BT * 3 * C * es));
        P.du.push_back(take(BT * F * es));
    }
    if (bf)
        for (int l = 0; l < c->n_layer; ++l) {
            P.d16o.push_back(take(BT * C * 2));
            P.d16m.push_back(take(BT * C * 2));
        }
    P.gprob = take((size_t)4 * c->n_layer * sizeof(GroupProb));
    P.Dbuf = take(2 * BT * H * 4);   // attention backward: D, then the base-2 log-sum-exp
    size_t sk = 0;
    const int shapes[4][2] = {{(int)(3 * C), (int)C}, {(int)C, (int)C}, {(int)F, (int)C}, {(int)C, (int)F}};
    for (auto& s : shapes) {
        const int ns = choose_split(s[0], s[1], (int)BT, bf).ns;
        if (ns > 1) sk = std::max(sk, (size_t)ns * s[0] * s[1] * 4);
    }
    P.splitk = take(sk ? sk : 256);
    P.rspart = take((size_t)16 * std::max(3 * C, F) * 4);   // <= 16 splits x the widest bias
    const int nln = 2 * c->n_layer + 1;
    P.lnset_stride = (size_t)layernorm_backward_max_blocks((int)BT) * 3 * C;
    P.lnpart = take(nln * P.lnset_stride * 4);
    P.lnscr = take((size_t)sum_sets_scratch_floats(nln, (int)(3 * C)) * 4);
    P.lnoff = take((size_t)2 * nln * 8);
    P.cspart = take((size_t)colsum_partial_floats((int)BT, (int)std::max(3 * C, F)) * 4);
    P.sumscr = take((size_t)sum_scratch_floats((int)std::max(3 * C, F)) * 4);
    P.normpart = take((size_t)norm_blocks() * 4);
    P.normcoef = take(256);
    P.ebscratch = take(embed_backward_scratch_bytes((int)BT, (int)C));
    P.total = o;
    return P;
}

const char* kClasses[] = {"embed_fwd", "layernorm_fwd", "gemm_qkv", "attn_fwd", "gemm_attn_proj", "gemm_fc",
                          "gemm_mlp_proj", "gemm_lm_head", "cross_entropy", "loss_mean", "gemm_lm_head_dx",
                          "gemm_lm_head_dw", "layernorm_bwd", "ln_param_grad", "gemm_dw", "bias_grad", "gemm_dx",
                          "attn_bwd", "embed_bwd", "grad_norm", "adamw", "eval_rows", "attn_decode", "topk_sample", nullptr};

}  // namespace

struct gpt2 {
    gpt2_config cfg;
    Layout L;
    Plan P;
    char* ws = nullptr;
    hipStream_t stream = nullptr;
    // a second stream (default priority) for work that depends only on the inputs: the
    // embedding backward's id sort runs on it under the rest of the backward; it forks from
    // and joins `stream` through the two events (edges in a graph capture of `stream`)
    hipStream_t side = nullptr;
    hipEvent_t side_fork = nullptr, side_join = nullptr;
    ~gpt2() {
        if (side_fork) (void)hipEventDestroy(side_fork);
        if (side_join) (void)hipEventDestroy(side_join);
        if (side) (void)hipStreamDestroy(side);
    }
    int dev = 0;
    bool bf16 = false;    // product and attention operands, activations: bf16 (else fp32)
    bool res16 = false;   // residual stream and its gradient: bf16 (else fp32)
    // state of the last forward
    bool have_fwd = false;
    int B = 0, T = 0;
    int lm_tiles = 0;   // > 0: the logits product also stored per-tile softmax statistics
    // incremental decoding: sequences in the key/value cache (0: no cache) and their length
    int dec_B = 0, dec_pos = 0;
    // device address of this GPU's allocation-free evaluation scratch (the static array below)
    char* na_scratch = nullptr;
    // grouped weight-gradient launch: usable (bf16, shapes the LDS-streamed path takes), its
    // tile width and total workgroups
    bool group_ok = false;
    int group_bn = 128, group_tiles = 0;
    // timing
    bool timing = false;
    std::string filter;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
    // a second pair per slot, handed to a product that is a single kernel (recorded at that
    // kernel's own start and end); ev_kern[i]: slot i's product used it
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev_k;
    std::vector<char> ev_kern;
    std::vector<int> ev_cls;
    size_t ev_used = 0;
    std::map<std::string, std::pair<double, int64_t>> times;

    template <typename X> X* at(size_t off) const { return (X*)(ws + off); }
    float* params() const { return at<float>(P.params); }
    float* grads() const { return at<float>(P.grads); }
    // weight operand of a product: the bf16 copy in bf16 mode, the fp32 master otherwise
    const void* wop(int64_t off) const {
        return bf16 ? (const void*)(at<uint16_t>(P.shadow) + off) : (const void*)(params() + off);
    }
};

namespace {

int class_index(const char* name) {
    for (int i = 0; kClasses[i]; ++i)
        if (!strcmp(kClasses[i], name)) return i;
    return -1;
}

// run one launcher under the timing hook
template <class Fn>
int run(gpt2_t* h, const char* cls, Fn&& fn) {
    const bool rec = h->timing && (h->filter.empty() || h->filter == cls);
    size_t slot = 0;
    if (rec) {
        if (h->ev_used == h->ev.size()) {
            hipEvent_t a, b, c, d;
            if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess ||
                hipEventCreate(&c) != hipSuccess || hipEventCreate(&d) != hipSuccess)
                return set_error(GPT2_EHIP, "hipEventCreate failed");
            h->ev.push_back({a, b});
            h->ev_k.push_back({c, d});
            h->ev_kern.push_back(0);
            h->ev_cls.push_back(0);
        }
        slot = h->ev_used++;
        (void)hipEventRecord(h->ev[slot].first, h->stream);
        gemm_time_next(h->ev_k[slot].first, h->ev_k[slot].second);
    }
    const hipError_t e = fn();
    if (rec) {
        h->ev_kern[slot] = gemm_time_taken() ? 1 : 0;
        (void)hipEventRecord(h->ev[slot].second, h->stream);
        h->ev_cls[slot] = class_index(cls);
    }
    if (e != hipSuccess) return set_error(GPT2_EHIP, "%s: %s", cls, hipGetErrorString(e));
    return GPT2_OK;
}

#define TRY(x)                     \
    do {                           \
        const int _r = (x);        \
        if (_r != GPT2_OK) return _r; \
    } while (0)

#define HIPTRY(x, what)                                                                   \
    do {                                                                                  \
        const hipError_t _e = (x);                                                        \
        if (_e != hipSuccess) return set_error(GPT2_EHIP, "%s: %s", what, hipGetErrorString(_e)); \
    } while (0)

bool g_setup_done = false;

}  // namespace

// =================================================================== allocation-free scratch
// The scratch of gpt2_evaluate_noalloc: per-sequence double sums and counts, the per-position
// losses and the mask copy, in one file-scope device array that each GPU holds for the life of
// the process. In host code `scratch` names a host-side stand-in, so kernels and copies take
// the device address hipGetSymbolAddress returns for it, looked up once per device.
constexpr size_t NA_ROWD_BYTES = (size_t)GPT2_NOALLOC_MAX_SEQ * 2 * sizeof(double);
constexpr size_t NA_LOSS_BYTES = (size_t)GPT2_NOALLOC_MAX_ROWS * sizeof(float);
constexpr size_t NA_MASK_BYTES = (size_t)GPT2_NOALLOC_MAX_ROWS;
constexpr size_t NA_BYTES = NA_ROWD_BYTES + NA_LOSS_BYTES + NA_MASK_BYTES;
static_assert(NA_ROWD_BYTES % 256 == 0 && NA_LOSS_BYTES % 256 == 0, "aligned sub-buffers");
static __device__ __align__(256) char scratch[NA_BYTES];

namespace {
std::mutex g_na_mu;
std::map<int, char*> g_na_ptr;   // device -> address of its copy of `scratch`

// the device address of `scratch` on device `dev` (which must be the current device)
int noalloc_scratch(int dev, char** out) {
    std::lock_guard<std::mutex> lk(g_na_mu);
    auto it = g_na_ptr.find(dev);
    if (it != g_na_ptr.end()) { *out = it->second; return GPT2_OK; }
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
        return set_error(GPT2_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_na_ptr[dev] = (char*)p;
    *out = (char*)p;
    return GPT2_OK;
}
}  // namespace

// =================================================================== sizing
extern "C" size_t gpt2_workspace_bytes(const gpt2_config* cfg) {
    std::string why;
    if (!config_ok(cfg, &why)) { set_error(GPT2_EINVAL, "%s", why.c_str()); return 0; }
    return make_plan(cfg).total;
}

extern "C" int64_t gpt2_num_params(const gpt2_config* cfg) {
    std::string why;
    if (!config_ok(cfg, &why, false)) { set_error(GPT2_EINVAL, "%s", why.c_str()); return -1; }
    return make_layout(cfg).n_params;
}

extern "C" int64_t gpt2_decay_end(const gpt2_config* cfg) {
    std::string why;
    if (!config_ok(cfg, &why, false)) { set_error(GPT2_EINVAL, "%s", why.c_str()); return -1; }
    return make_layout(cfg).decay_end;
}

extern "C" int32_t gpt2_num_tensors(const gpt2_config* cfg) {
    if (!config_ok(cfg, nullptr, false)) return -1;
    return 12 * cfg->n_layer + 4;
}

extern "C" int32_t gpt2_num_decay_tensors(const gpt2_config* cfg) {
    if (!config_ok(cfg, nullptr, false)) return -1;
    return 4 * cfg->n_layer + 2;
}

extern "C" int gpt2_param_info(const gpt2_config* cfg, int32_t i, const char** name, int64_t* offset, int64_t shape[2]) {
    std::string why;
    if (!config_ok(cfg, &why, false)) return set_error(GPT2_EINVAL, "%s", why.c_str());
    static thread_local std::map<std::string, std::string> names;  // stable storage for returned names
    std::string nm;
    int64_t off, r, c;
    if (!tensor_info(cfg, i, &nm, &off, &r, &c)) return set_error(GPT2_EINVAL, "tensor index %d out of range", i);
    auto it = names.emplace(nm, nm).first;
    if (name) *name = it->second.c_str();
    if (offset) *offset = off;
    if (shape) { shape[0] = r; shape[1] = c; }
    return GPT2_OK;
}

extern "C" double gpt2_cosine_lr(int64_t it, double max_lr, double min_lr, int64_t warmup_steps, int64_t max_steps) {
    if (it < warmup_steps) return max_lr * (double)(it + 1) / (double)warmup_steps;
    if (it > max_steps) return min_lr;
    const double ratio = (double)(it - warmup_steps) / (double)(max_steps - warmup_steps);
    const double coeff = 0.5 * (1.0 + std::cos(M_PI * ratio));
    return min_lr + coeff * (max_lr - min_lr);
}

extern "C" const char* gpt2_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* gpt2_kernel_class(int32_t i) {
    const int n = (int)(sizeof(kClasses) / sizeof(kClasses[0])) - 1;
    return (i >= 0 && i < n) ? kClasses[i] : nullptr;
}

// =================================================================== lifetime
extern "C" int gpt2_create(const gpt2_config* cfg, void* d_ws, size_t ws_bytes, uint64_t seed, void* stream, gpt2_t** out) {
    std::string why;
    if (!out) return set_error(GPT2_EINVAL, "out is null");
    *out = nullptr;
    if (!config_ok(cfg, &why)) return set_error(GPT2_EINVAL, "%s", why.c_str());
    if (!d_ws) return set_error(GPT2_EINVAL, "workspace is null");
    if ((uintptr_t)d_ws & 255) return set_error(GPT2_EINVAL, "workspace must be 256-byte aligned");
    gpt2_t* h = new gpt2_t();
    h->cfg = *cfg;
    h->L = make_layout(cfg);
    h->P = make_plan(cfg);
    if (ws_bytes < h->P.total) {
        const size_t need = h->P.total;
        delete h;
        return set_error(GPT2_EINVAL, "workspace too small: %zu bytes given, %zu needed", ws_bytes, need);
    }
    h->ws = (char*)d_ws;
    h->stream = (hipStream_t)stream;
    h->bf16 = cfg->dtype != GPT2_FP32;
    h->res16 = cfg->dtype == GPT2_BF16_RES16;
    (void)hipGetDevice(&h->dev);
    if (hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&h->side_fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&h->side_join, hipEventDisableTiming) != hipSuccess) {
        // without them everything runs on the caller's stream
        if (h->side_fork) (void)hipEventDestroy(h->side_fork);
        if (h->side) (void)hipStreamDestroy(h->side);
        h->side = nullptr;
        h->side_fork = h->side_join = nullptr;
        (void)hipGetLastError();
    }
    if (!g_setup_done) {
        gemm_setup();
        attention_setup();
        rows_setup();
        g_setup_done = true;
    }
    {
        // this device's allocation-free scratch (the handle's device is current here)
        const int r = noalloc_scratch(h->dev, &h->na_scratch);
        if (r != GPT2_OK) { delete h; return r; }
    }
    // parameters per the GPT-2 initialization, gradients and moments zero
    const int n = gpt2_num_tensors(cfg);
    const float resid_std = 0.02f / std::sqrt(2.0f * cfg->n_layer);
    for (int i = 0; i < n; ++i) {
        std::string nm;
        int64_t off, r, c;
        tensor_info(cfg, i, &nm, &off, &r, &c);
        const int64_t cnt = c ? r * c : r;
        float* p = h->params() + off;
        hipError_t e;
        if (c) {
            const bool resid = nm.find("c_proj.weight") != std::string::npos;
            e = init_normal(p, cnt, resid ? resid_std : 0.02f, seed, (uint64_t)off / 4, h->stream);
        } else {
            const bool gain = nm.find("ln_") != std::string::npos && nm.find(".weight") != std::string::npos;
            e = fill(p, cnt, gain ? 1.0f : 0.0f, h->stream);
        }
        if (e != hipSuccess) { delete h; return set_error(GPT2_EHIP, "init: %s", hipGetErrorString(e)); }
    }
    const int64_t N = h->L.n_params;
    hipError_t e = hipMemsetAsync(h->grads(), 0, N * 4, h->stream);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<float>(h->P.m), 0, N * 4, h->stream);
    if (e == hipSuccess) e = hipMemsetAsync(h->at<float>(h->P.v), 0, N * 4, h->stream);
    if (e == hipSuccess && h->bf16) e = refresh_shadow(h->params(), h->at<char>(h->P.shadow), h->L.decay_end, h->stream);
    if (e == hipSuccess) {
        // gradient offsets of the LayerNorm partial sets, in the order the backward fills them:
        // weight and bias (adjacent in the arena), then the bias of the projection whose residual
        // add feeds the LayerNorm (none for ln_f)
        const int nl = cfg->n_layer, nln = 2 * nl + 1;
        std::vector<int64_t> off(2 * nln);
        off[0] = h->L.lnf_w;
        off[nln] = -1;
        for (int l = nl - 1, i = 1; l >= 0; --l, i += 2) {
            off[i] = h->L.ln2_w[l];
            off[nln + i] = h->L.b_pr[l];
            off[i + 1] = h->L.ln1_w[l];
            off[nln + i + 1] = h->L.b_o[l];
        }
        e = hipMemcpy(h->at<int64_t>(h->P.lnoff), off.data(), off.size() * 8, hipMemcpyHostToDevice);
    }
    if (e == hipSuccess && h->bf16) {
        // the weight-gradient products of every layer, for one grouped launch after the backward:
        // mlp.c_proj (A = residual gradient at the layer output, B = a), mlp.c_fc (du, h2; bias
        // = row sums of du), attn.c_proj (residual gradient after attention, y), attn.c_attn
        // (dqkv, h1; bias = row sums of dqkv)
        const Layout& L = h->L;
        const Plan& P = h->P;
        float* grd = h->grads();
        const int C = cfg->n_embd, F = cfg->mlp_hidden;
        // 128x192 tiles (wave tile 64x96) also where C or F is not a multiple of 192: at C = 1600
        // (1558M-shaped step) the ragged last column tile wastes 3% more area than 128x128 tiles
        // and the launch still gains 9% (14.0 -> 12.7 ms per step) from the wider tile's fewer LDS
        // bytes per MFMA
        const int bn = 192;
        std::vector<GroupProb> pr;
        bool ok = true;
        int tile0 = 0;
        for (int l = cfg->n_layer - 1; l >= 0; --l) {
            auto add = [&](const void* A, int64_t lda, const void* B, int64_t ldb, int64_t woff, int M, int N,
                           int64_t boff) {
                GroupProb g{};
                g.A = A; g.lda = lda; g.B = B; g.ldb = ldb;
                g.C = grd + woff; g.ldc = N; g.M = M; g.N = N;
                g.rowsum = boff >= 0 ? grd + boff : nullptr;
                g.tile0 = tile0;
                g.ntiles = gemm_group_tiles(M, N, bn);
                tile0 += g.ntiles;
                ok = ok && gemm_group_ok(g, 64);
                pr.push_back(g);
            };
            add(h->at<char>(P.d16o[l]), C, h->at<char>(P.a[l]), F, L.w_pr[l], C, F, -1);
            add(h->at<char>(P.du[l]), F, h->at<char>(P.h2[l]), C, L.w_fc[l], F, C, L.b_fc[l]);
            add(h->at<char>(P.d16m[l]), C, h->at<char>(P.att[l]), C, L.w_o[l], C, C, -1);
            add(h->at<char>(P.dqkv[l]), 3 * C, h->at<char>(P.h1[l]), C, L.w_qkv[l], 3 * C, C, L.b_qkv[l]);
        }
        h->group_ok = ok;
        h->group_bn = bn;
        h->group_tiles = tile0;
        e = hipMemcpy(h->at<GroupProb>(P.gprob), pr.data(), pr.size() * sizeof(GroupProb), hipMemcpyHostToDevice);
    }
    if (e != hipSuccess) { delete h; return set_error(GPT2_EHIP, "init: %s", hipGetErrorString(e)); }
    *out = h;
    return GPT2_OK;
}

extern "C" int gpt2_destroy(gpt2_t* h) {
    if (!h) return set_error(GPT2_EINVAL, "handle is null");
    for (auto& p : h->ev) { (void)hipEventDestroy(p.first); (void)hipEventDestroy(p.second); }
    for (auto& p : h->ev_k) { (void)hipEventDestroy(p.first); (void)hipEventDestroy(p.second); }
    delete h;
    return GPT2_OK;
}

extern "C" int gpt2_set_stream(gpt2_t* h, void* stream) {
    if (!h) return set_error(GPT2_EINVAL, "handle is null");
    h->stream = (hipStream_t)stream;
    return GPT2_OK;
}

// =================================================================== parameter I/O
static int copy_arena(gpt2_t* h, void* dst, const void* src, size_t bytes, bool to_dev, int on_device) {
    const hipMemcpyKind k = on_device ? hipMemcpyDeviceToDevice : (to_dev ? hipMemcpyHostToDevice : hipMemcpyDeviceToHost);
    HIPTRY(hipMemcpyAsync(dst, src, bytes, k, h->stream), "copy");
    if (!on_device) HIPTRY(hipStreamSynchronize(h->stream), "synchronize");
    return GPT2_OK;
}

extern "C" int gpt2_set_params(gpt2_t* h, const float* src, int on_device) {
    if (!h || !src) return set_error(GPT2_EINVAL, "null argument");
    TRY(copy_arena(h, h->params(), src, h->L.n_params * 4, true, on_device));
    if (h->bf16) HIPTRY(refresh_shadow(h->params(), h->at<char>(h->P.shadow), h->L.decay_end, h->stream), "shadow");
    return GPT2_OK;
}
extern "C" int gpt2_get_params(gpt2_t* h, float* dst, int on_device) {
    if (!h || !dst) return set_error(GPT2_EINVAL, "null argument");
    return copy_arena(h, dst, h->params(), h->L.n_params * 4, false, on_device);
}
extern "C" int gpt2_get_grads(gpt2_t* h, float* dst, int on_device) {
    if (!h || !dst) return set_error(GPT2_EINVAL, "null argument");
    return copy_arena(h, dst, h->grads(), h->L.n_params * 4, false, on_device);
}
extern "C" int gpt2_set_grads(gpt2_t* h, const float* src, int on_device) {
    if (!h || !src) return set_error(GPT2_EINVAL, "null argument");
    return copy_arena(h, h->grads(), src, h->L.n_params * 4, true, on_device);
}
extern "C" int gpt2_get_moments(gpt2_t* h, float* m, float* v, int on_device) {
    if (!h) return set_error(GPT2_EINVAL, "handle is null");
    if (m) TRY(copy_arena(h, m, h->at<float>(h->P.m), h->L.n_params * 4, false, on_device));
    if (v) TRY(copy_arena(h, v, h->at<float>(h->P.v), h->L.n_params * 4, false, on_device));
    return GPT2_OK;
}
extern "C" int gpt2_set_moments(gpt2_t* h, const float* m, const float* v, int on_device) {
    if (!h) return set_error(GPT2_EINVAL, "handle is null");
    if (m) TRY(copy_arena(h, h->at<float>(h->P.m), m, h->L.n_params * 4, true, on_device));
    if (v) TRY(copy_arena(h, h->at<float>(h->P.v), v, h->L.n_params * 4, true, on_device));
    return GPT2_OK;
}
extern "C" float* gpt2_params_device(gpt2_t* h) { return h ? h->params() : nullptr; }
extern "C" float* gpt2_grads_device(gpt2_t* h) { return h ? h->grads() : nullptr; }

// =================================================================== forward
// Embedding, the blocks, ln_f and the tied lm_head over B x T tokens whose ids are already in
// the workspace; leaves the logits (storage type) in P.logits and every activation the
// backward pass reads.
static int forward_trunk(gpt2_t* h, int B, int T) {
    const gpt2_config& c = h->cfg;
    const int BT = B * T, C = c.n_embd, F = c.mlp_hidden, Vp = c.padded_vocab_size, H = c.n_head, hs = C / H;
    const int bf = h->bf16, r16 = h->res16;
    const Layout& L = h->L;
    const Plan& P = h->P;
    float* prm = h->params();
    hipStream_t s = h->stream;
    int32_t* idx = h->at<int32_t>(P.idx);
    char* y = h->at<char>(P.yproj);
    TRY(run(h, "embed_fwd", [&] { return embed_forward(idx, prm + L.wte, prm + L.wpe, h->at<char>(P.x_in[0]), B, T, C, r16, s); }));
    TRY(run(h, "layernorm_fwd", [&] {
        return layernorm_forward(h->at<char>(P.x_in[0]), prm + L.ln1_w[0], prm + L.ln1_b[0], h->at<char>(P.h1[0]),
                                 h->at<float>(P.mean1[0]), h->at<float>(P.rstd1[0]), BT, C, r16, bf, s);
    }));
    for (int l = 0; l < c.n_layer; ++l) {
        GemmDesc g;
        g.A = h->at<char>(P.h1[l]); g.lda = C; g.a_layout = 0;
        g.B = h->wop(L.w_qkv[l]); g.ldb = C; g.b_layout = 0;
        g.M = BT; g.N = 3 * C; g.K = C;
        g.epi = EPI_BIAS_T; g.C = h->at<char>(P.qkv[l]); g.ldc = 3 * C; g.bias = prm + L.b_qkv[l];
        TRY(run(h, "gemm_qkv", [&] { return gemm(g, bf, s); }));
        TRY(run(h, "attn_fwd", [&] {
            return attention_forward(h->at<char>(P.qkv[l]), h->at<char>(P.att[l]), h->at<float>(P.lse[l]), B, T, H, hs, bf, s);
        }));
        // x_mid = x_in + (y Wo^T + bo), then ln_2
        g = GemmDesc();
        g.A = h->at<char>(P.att[l]); g.lda = C;
        g.B = h->wop(L.w_o[l]); g.ldb = C;
        g.M = BT; g.N = C; g.K = C;
        g.epi = EPI_BIAS_T; g.C = y; g.ldc = C; g.bias = prm + L.b_o[l];
        TRY(run(h, "gemm_attn_proj", [&] { return gemm(g, bf, s); }));
        TRY(run(h, "layernorm_fwd", [&] {
            return add_layernorm_forward(h->at<char>(P.x_in[l]), y, h->at<char>(P.x_mid[l]), prm + L.ln2_w[l],
                                         prm + L.ln2_b[l], h->at<char>(P.h2[l]), h->at<float>(P.mean2[l]),
                                         h->at<float>(P.rstd2[l]), BT, C, r16, bf, s);
        }));
        g = GemmDesc();
        g.A = h->at<char>(P.h2[l]); g.lda = C;
        g.B = h->wop(L.w_fc[l]); g.ldb = C;
        g.M = BT; g.N = F; g.K = C;
        g.epi = EPI_BIAS_GELU; g.C = h->at<char>(P.u[l]); g.C2 = h->at<char>(P.a[l]); g.ldc = F; g.bias = prm + L.b_fc[l];
        TRY(run(h, "gemm_fc", [&] { return gemm(g, bf, s); }));
        // x_out = x_mid + (a Wpr^T + bpr), then the next layer's ln_1 (or ln_f)
        g = GemmDesc();
        g.A = h->at<char>(P.a[l]); g.lda = F;
        g.B = h->wop(L.w_pr[l]); g.ldb = F;
        g.M = BT; g.N = C; g.K = F;
        g.epi = EPI_BIAS_T; g.C = y; g.ldc = C; g.bias = prm + L.b_pr[l];
        TRY(run(h, "gemm_mlp_proj", [&] { return gemm(g, bf, s); }));
        const bool last = l + 1 == c.n_layer;
        TRY(run(h, "layernorm_fwd", [&] {
            return add_layernorm_forward(h->at<char>(P.x_mid[l]), y, h->at<char>(P.x_in[l + 1]),
                                         prm + (last ? L.lnf_w : L.ln1_w[l + 1]), prm + (last ? L.lnf_b : L.ln1_b[l + 1]),
                                         h->at<char>(last ? P.hf : P.h1[l + 1]),
                                         h->at<float>(last ? P.meanf : P.mean1[l + 1]),
                                         h->at<float>(last ? P.rstdf : P.rstd1[l + 1]), BT, C, r16, bf, s);
        }));
    }
    {
        GemmDesc g;
        g.A = h->at<char>(P.hf); g.lda = C;
        g.B = h->wop(L.wte); g.ldb = C;  // tied lm_head: logits = hf wte^T, no bias
        g.M = BT; g.N = Vp; g.K = C;
        g.epi = EPI_LOGITS; g.C = h->at<char>(P.logits); g.ldc = Vp; g.C2 = h->at<char>(P.lstats);
        h->lm_tiles = gemm_logits_tiles(g, bf);
        if (!h->lm_tiles) { g.epi = EPI_BIAS_T; g.C2 = nullptr; }
        TRY(run(h, "gemm_lm_head", [&] { return gemm(g, bf, s); }));
    }
    return GPT2_OK;
}

// Per-row loss (and, with write_grad, the logits overwritten by their gradient) after
// forward_trunk: from the statistics the logits product stored when it could, else two passes.
static int loss_rows_after_trunk(gpt2_t* h, int BT, float* loss_rows, float* d_logits, int write_grad) {
    const Plan& P = h->P;
    const int Vp = h->cfg.padded_vocab_size;
    int32_t* tgt = h->at<int32_t>(P.tgt);
    return run(h, "cross_entropy", [&] {
        if (h->lm_tiles)
            return cross_entropy_tiled(h->at<char>(P.logits), h->at<float>(P.lstats), h->lm_tiles, tgt, loss_rows,
                                       h->at<float>(P.lse2rows), d_logits, BT, Vp, h->stream, write_grad);
        return cross_entropy(h->at<char>(P.logits), tgt, loss_rows, d_logits, BT, Vp, h->bf16, h->stream, write_grad);
    });
}

extern "C" int gpt2_forward(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, int32_t B, int32_t T,
                            float* d_logits, float* d_loss, float* h_loss) {
    if (!h || !d_idx) return set_error(GPT2_EINVAL, "null argument");
    const gpt2_config& c = h->cfg;
    if (B < 1 || B > c.max_batch) return set_error(GPT2_EINVAL, "B=%d outside [1, max_batch=%d]", B, c.max_batch);
    if (T < 1 || T > c.block_size) return set_error(GPT2_EINVAL, "T=%d outside [1, block_size=%d]", T, c.block_size);
    if (!d_targets && (d_loss || h_loss)) return set_error(GPT2_EINVAL, "a loss needs targets");
    if (!d_targets && !d_logits) return set_error(GPT2_EINVAL, "without targets, d_logits is required");
    h->have_fwd = false;
    h->dec_B = 0;   // the forward overwrites the key/value cache
    const int BT = B * T, Vp = c.padded_vocab_size;
    const int bf = h->bf16;
    const Plan& P = h->P;
    hipStream_t s = h->stream;
    int32_t* idx = h->at<int32_t>(P.idx);
    int32_t* tgt = h->at<int32_t>(P.tgt);
    HIPTRY(hipMemcpyAsync(idx, d_idx, (size_t)BT * 4, hipMemcpyDeviceToDevice, s), "copy idx");
    if (d_targets) HIPTRY(hipMemcpyAsync(tgt, d_targets, (size_t)BT * 4, hipMemcpyDeviceToDevice, s), "copy targets");

    TRY(forward_trunk(h, B, T));
    if (d_targets) {
        TRY(loss_rows_after_trunk(h, BT, h->at<float>(P.loss_rows), d_logits, 1));
        float* dl = h->at<float>(P.loss);
        TRY(run(h, "loss_mean", [&] { return mean_reduce(h->at<float>(P.loss_rows), BT, dl, s); }));
        if (d_loss) HIPTRY(hipMemcpyAsync(d_loss, dl, 4, hipMemcpyDeviceToDevice, s), "copy loss");
        if (h_loss) {
            HIPTRY(hipMemcpyAsync(h_loss, dl, 4, hipMemcpyDeviceToHost, s), "copy loss");
            HIPTRY(hipStreamSynchronize(s), "synchronize");
        }
        h->have_fwd = true;
        h->B = B;
        h->T = T;
    } else {
        HIPTRY(convert_to_f32(h->at<char>(P.logits), d_logits, (int64_t)BT * Vp, bf, s), "logits");
    }
    return GPT2_OK;
}

// =================================================================== evaluation
// Forward-only scoring with its scratch (per-position losses, mask copy, per-sequence double
// sums and counts) at the given device addresses.
static int evaluate_impl(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, const uint8_t* d_mask, int32_t B,
                         int32_t T, float* d_row_sum, float* d_row_mean, float* d_loss, float* loss_rows,
                         uint8_t* mask_copy, double* rowd) {
    h->have_fwd = false;   // the activations are overwritten and no gradient of the loss is formed
    h->dec_B = 0;
    const int BT = B * T;
    const Plan& P = h->P;
    hipStream_t s = h->stream;
    int32_t* idx = h->at<int32_t>(P.idx);
    int32_t* tgt = h->at<int32_t>(P.tgt);
    uint8_t* mask = d_mask ? mask_copy : nullptr;
    HIPTRY(hipMemcpyAsync(idx, d_idx, (size_t)BT * 4, hipMemcpyDeviceToDevice, s), "copy idx");
    HIPTRY(hipMemcpyAsync(tgt, d_targets, (size_t)BT * 4, hipMemcpyDeviceToDevice, s), "copy targets");
    if (d_mask) HIPTRY(hipMemcpyAsync(mask, d_mask, (size_t)BT, hipMemcpyDeviceToDevice, s), "copy mask");
    TRY(forward_trunk(h, B, T));
    TRY(loss_rows_after_trunk(h, BT, loss_rows, nullptr, /*write_grad=*/0));
    // without a mask the batch mean is the training forward's loss, reduced the same way
    TRY(run(h, "eval_rows", [&] {
        return masked_row_loss(loss_rows, mask, B, T, rowd, d_row_sum, d_row_mean, mask ? d_loss : nullptr, s);
    }));
    if (d_loss && !mask) TRY(run(h, "loss_mean", [&] { return mean_reduce(loss_rows, BT, d_loss, s); }));
    return GPT2_OK;
}

static int evaluate_args_ok(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, int32_t B, int32_t T) {
    if (!h || !d_idx || !d_targets) return set_error(GPT2_EINVAL, "null argument");
    const gpt2_config& c = h->cfg;
    if (B < 1 || B > c.max_batch) return set_error(GPT2_EINVAL, "B=%d outside [1, max_batch=%d]", B, c.max_batch);
    if (T < 1 || T > c.block_size) return set_error(GPT2_EINVAL, "T=%d outside [1, block_size=%d]", T, c.block_size);
    return GPT2_OK;
}

extern "C" int gpt2_evaluate(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, const uint8_t* d_mask,
                             int32_t B, int32_t T, float* d_row_sum, float* d_row_mean, float* d_loss) {
    TRY(evaluate_args_ok(h, d_idx, d_targets, B, T));
    const Plan& P = h->P;
    return evaluate_impl(h, d_idx, d_targets, d_mask, B, T, d_row_sum, d_row_mean, d_loss, h->at<float>(P.loss_rows),
                         h->at<uint8_t>(P.mask), h->at<double>(P.rowd));
}

extern "C" int gpt2_evaluate_noalloc(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, const uint8_t* d_mask,
                                     int32_t B, int32_t T, float* d_row_sum, float* d_row_mean, float* d_loss) {
    TRY(evaluate_args_ok(h, d_idx, d_targets, B, T));
    if (B > GPT2_NOALLOC_MAX_SEQ)
        return set_error(GPT2_EINVAL, "B=%d exceeds the allocation-free scratch (at most %d sequences)", B,
                         GPT2_NOALLOC_MAX_SEQ);
    if ((int64_t)B * T > GPT2_NOALLOC_MAX_ROWS)
        return set_error(GPT2_EINVAL, "B*T=%lld exceeds the allocation-free scratch (at most %d positions)",
                         (long long)B * T, GPT2_NOALLOC_MAX_ROWS);
    if (!h->na_scratch) return set_error(GPT2_ESTATE, "no allocation-free scratch on this handle's device");
    char* base = h->na_scratch;
    return evaluate_impl(h, d_idx, d_targets, d_mask, B, T, d_row_sum, d_row_mean, d_loss,
                         (float*)(base + NA_ROWD_BYTES), (uint8_t*)(base + NA_ROWD_BYTES + NA_LOSS_BYTES),
                         (double*)base);
}

// =================================================================== incremental decoding
extern "C" int gpt2_decode_reset(gpt2_t* h, int32_t B) {
    if (!h) return set_error(GPT2_EINVAL, "handle is null");
    const gpt2_config& c = h->cfg;
    if (B < 1 || B > c.max_batch) return set_error(GPT2_EINVAL, "B=%d outside [1, max_batch=%d]", B, c.max_batch);
    if (c.block_size > GPT2_DECODE_MAX_T)
        return set_error(GPT2_EINVAL, "decoding supports block_size <= %d", GPT2_DECODE_MAX_T);
    h->have_fwd = false;
    h->dec_B = B;
    h->dec_pos = 0;
    return GPT2_OK;
}

// One new position of every cached sequence: the blocks run on B rows (one per sequence),
// the qkv product writes its rows straight into the cache (row b*block_size + pos of the
// layer's qkv buffer), and the attention reads the cache.
// One decoding step at the host's position (d_pos null) or at the position in device memory
// *d_pos (clamped to block_size - 1 by the kernels, then advanced on the device).
static int decode_impl(gpt2_t* h, const int32_t* d_tokens, int32_t* d_pos, float* d_logits, int32_t top_k,
                       const float* d_uniform, int32_t* d_next, int32_t* d_topk_idx, float* d_topk_prob) {
    if (!h || !d_tokens) return set_error(GPT2_EINVAL, "null argument");
    if (!h->dec_B) return set_error(GPT2_ESTATE, "decoding needs gpt2_decode_reset first");
    const gpt2_config& c = h->cfg;
    const int B = h->dec_B, pos = d_pos ? 0 : h->dec_pos, Tmax = c.block_size;
    if (!d_pos && pos >= Tmax) return set_error(GPT2_EINVAL, "the cache is full (block_size=%d positions)", Tmax);
    const bool sample = d_next || d_topk_idx || d_topk_prob;
    if (sample && (top_k < 1 || top_k > GPT2_TOPK_MAX || top_k > c.padded_vocab_size))
        return set_error(GPT2_EINVAL, "top_k=%d outside [1, %d]", top_k, GPT2_TOPK_MAX);
    if (d_next && !d_uniform) return set_error(GPT2_EINVAL, "drawing the next token needs d_uniform");
    const int C = c.n_embd, F = c.mlp_hidden, Vp = c.padded_vocab_size, H = c.n_head, hs = C / H;
    const int bf = h->bf16, r16 = h->res16;
    const size_t es = bf ? 2 : 4;
    const Layout& L = h->L;
    const Plan& P = h->P;
    float* prm = h->params();
    hipStream_t s = h->stream;
    int32_t* idx = h->at<int32_t>(P.idx);
    char* y = h->at<char>(P.yproj);
    HIPTRY(hipMemcpyAsync(idx, d_tokens, (size_t)B * 4, hipMemcpyDeviceToDevice, s), "copy tokens");
    h->dec_B = 0;   // until this step has been enqueued completely
    TRY(run(h, "embed_fwd", [&] {
        return embed_forward(idx, prm + L.wte, prm + L.wpe + (int64_t)pos * C, h->at<char>(P.x_in[0]), B, 1, C, r16, s,
                             d_pos, Tmax - 1);
    }));
    TRY(run(h, "layernorm_fwd", [&] {
        return layernorm_forward(h->at<char>(P.x_in[0]), prm + L.ln1_w[0], prm + L.ln1_b[0], h->at<char>(P.h1[0]),
                                 h->at<float>(P.mean1[0]), h->at<float>(P.rstd1[0]), B, C, r16, bf, s);
    }));
    // the descriptors of one layer's products (the fused forms take the LayerNorm in their A rows)
    auto qkv_desc = [&](int l) {
        GemmDesc g;
        g.A = h->at<char>(P.h1[l]); g.lda = C; g.a_layout = 0;
        g.B = h->wop(L.w_qkv[l]); g.ldb = C; g.b_layout = 0;
        g.M = B; g.N = 3 * C; g.K = C;
        g.epi = EPI_BIAS_T; g.C = h->at<char>(P.qkv[l]) + (size_t)pos * 3 * C * es; g.ldc = (int64_t)Tmax * 3 * C;
        g.bias = prm + L.b_qkv[l];
        if (d_pos) { g.c_row_dev = d_pos; g.c_row_bytes = (int64_t)3 * C * es; g.c_row_max = Tmax - 1; }
        return g;
    };
    auto fc_desc = [&](int l) {
        GemmDesc g;
        g.A = h->at<char>(P.h2[l]); g.lda = C;
        g.B = h->wop(L.w_fc[l]); g.ldb = C;
        g.M = B; g.N = F; g.K = C;
        g.epi = EPI_BIAS_GELU; g.C = h->at<char>(P.u[l]); g.C2 = h->at<char>(P.a[l]); g.ldc = F; g.bias = prm + L.b_fc[l];
        return g;
    };
    // residual add + LayerNorm inside the following product (bf16, few rows), else separate
    const bool fuse = gemm_skinny_ln_ok(qkv_desc(0), bf) && gemm_skinny_ln_ok(fc_desc(0), bf);
    for (int l = 0; l < c.n_layer; ++l) {
        {
            const GemmDesc g = qkv_desc(l);
            if (fuse && l > 0) {
                const SkinnyLn ln{h->at<char>(P.x_mid[l - 1]), y, h->at<char>(P.x_in[l]), prm + L.ln1_w[l],
                                  prm + L.ln1_b[l]};
                TRY(run(h, "gemm_qkv", [&] { return gemm_skinny_ln(g, ln, r16, s); }));
            } else {
                TRY(run(h, "gemm_qkv", [&] { return gemm(g, bf, s); }));
            }
        }
        TRY(run(h, "attn_decode", [&] {
            return attention_decode(h->at<char>(P.qkv[l]), h->at<char>(P.att[l]), B, Tmax, pos, H, hs, bf, s, d_pos);
        }));
        {
            GemmDesc g;
            g.A = h->at<char>(P.att[l]); g.lda = C;
            g.B = h->wop(L.w_o[l]); g.ldb = C;
            g.M = B; g.N = C; g.K = C;
            g.epi = EPI_BIAS_T; g.C = y; g.ldc = C; g.bias = prm + L.b_o[l];
            TRY(run(h, "gemm_attn_proj", [&] { return gemm(g, bf, s); }));
        }
        if (fuse) {
            const SkinnyLn ln{h->at<char>(P.x_in[l]), y, h->at<char>(P.x_mid[l]), prm + L.ln2_w[l], prm + L.ln2_b[l]};
            const GemmDesc g = fc_desc(l);
            TRY(run(h, "gemm_fc", [&] { return gemm_skinny_ln(g, ln, r16, s); }));
        } else {
            TRY(run(h, "layernorm_fwd", [&] {
                return add_layernorm_forward(h->at<char>(P.x_in[l]), y, h->at<char>(P.x_mid[l]), prm + L.ln2_w[l],
                                             prm + L.ln2_b[l], h->at<char>(P.h2[l]), h->at<float>(P.mean2[l]),
                                             h->at<float>(P.rstd2[l]), B, C, r16, bf, s);
            }));
            const GemmDesc g = fc_desc(l);
            TRY(run(h, "gemm_fc", [&] { return gemm(g, bf, s); }));
        }
        {
            GemmDesc g;
            g.A = h->at<char>(P.a[l]); g.lda = F;
            g.B = h->wop(L.w_pr[l]); g.ldb = F;
            g.M = B; g.N = C; g.K = F;
            g.epi = EPI_BIAS_T; g.C = y; g.ldc = C; g.bias = prm + L.b_pr[l];
            TRY(run(h, "gemm_mlp_proj", [&] { return gemm(g, bf, s); }));
        }
        const bool last = l + 1 == c.n_layer;
        if (last || !fuse)
            TRY(run(h, "layernorm_fwd", [&] {
                return add_layernorm_forward(h->at<char>(P.x_mid[l]), y, h->at<char>(P.x_in[l + 1]),
                                             prm + (last ? L.lnf_w : L.ln1_w[l + 1]), prm + (last ? L.lnf_b : L.ln1_b[l + 1]),
                                             h->at<char>(last ? P.hf : P.h1[l + 1]),
                                             h->at<float>(last ? P.meanf : P.mean1[l + 1]),
                                             h->at<float>(last ? P.rstdf : P.rstd1[l + 1]), B, C, r16, bf, s);
            }));
    }
    {
        GemmDesc g;
        g.A = h->at<char>(P.hf); g.lda = C;
        g.B = h->wop(L.wte); g.ldb = C;
        g.M = B; g.N = Vp; g.K = C;
        g.epi = EPI_BIAS_T; g.C = h->at<char>(P.logits); g.ldc = Vp;
        TRY(run(h, "gemm_lm_head", [&] { return gemm(g, bf, s); }));
    }
    if (d_logits) HIPTRY(convert_to_f32(h->at<char>(P.logits), d_logits, (int64_t)B * Vp, bf, s), "logits");
    if (sample)
        TRY(run(h, "topk_sample", [&] {
            return topk_sample(h->at<char>(P.logits), B, Vp, top_k, d_uniform, d_next, d_topk_idx, d_topk_prob, bf, s);
        }));
    if (d_pos) HIPTRY(decode_advance(d_pos, Tmax, s), "advance position");
    h->dec_B = B;
    if (!d_pos) h->dec_pos = pos + 1;
    return GPT2_OK;
}

extern "C" int gpt2_decode_step(gpt2_t* h, const int32_t* d_tokens, float* d_logits, int32_t top_k,
                                const float* d_uniform, int32_t* d_next, int32_t* d_topk_idx, float* d_topk_prob) {
    return decode_impl(h, d_tokens, nullptr, d_logits, top_k, d_uniform, d_next, d_topk_idx, d_topk_prob);
}

extern "C" int gpt2_decode_step_device(gpt2_t* h, const int32_t* d_tokens, int32_t* d_pos, float* d_logits,
                                       int32_t top_k, const float* d_uniform, int32_t* d_next, int32_t* d_topk_idx,
                                       float* d_topk_prob) {
    if (!d_pos) return set_error(GPT2_EINVAL, "d_pos is null");
    return decode_impl(h, d_tokens, d_pos, d_logits, top_k, d_uniform, d_next, d_topk_idx, d_topk_prob);
}

extern "C" int32_t gpt2_decode_position(const gpt2_t* h) { return h && h->dec_B ? h->dec_pos : -1; }

// =================================================================== backward
extern "C" int gpt2_backward(gpt2_t* h, float grad_scale, int32_t accumulate) {
    if (!h) return set_error(GPT2_EINVAL, "handle is null");
    if (!h->have_fwd) return set_error(GPT2_ESTATE, "backward needs a preceding forward with targets");
    const gpt2_config& c = h->cfg;
    const int B = h->B, T = h->T, BT = B * T, C = c.n_embd, F = c.mlp_hidden, Vp = c.padded_vocab_size;
    const int H = c.n_head, hs = C / H;
    const int bf = h->bf16, r16 = h->res16;
    const int acc = accumulate ? 1 : 0;
    const Layout& L = h->L;
    const Plan& P = h->P;
    float* grd = h->grads();
    float* prm = h->params();
    hipStream_t s = h->stream;
    // gradient of the residual stream, in the residual stream's type; the products take it as
    // bf16 (under the autocast recipe the gradient reaching a bf16 product output is cast down)
    char* dres = h->at<char>(P.dres);
    // bf16 copies of the residual gradient, one per point where a product takes it (fp32 mode:
    // the products take the fp32 gradient itself)
    auto d16_out = [&](int l) -> char* { return bf ? h->at<char>(P.d16o[l]) : dres; };
    auto d16_mid = [&](int l) -> char* { return bf ? h->at<char>(P.d16m[l]) : dres; };
    auto du_of = [&](int l) -> char* { return h->at<char>(P.du[bf ? l : 0]); };
    auto dqkv_of = [&](int l) -> char* { return h->at<char>(P.dqkv[bf ? l : 0]); };
    // every weight gradient of the blocks in one grouped launch after the layer loop (whole-K
    // products, no split-K), where the shapes allow it; otherwise per layer with split-K
    const bool grouped = h->group_ok && BT % 64 == 0;
    // gradient of a LayerNorm's output, in the storage type: under the autocast recipe it is the
    // bf16 input gradient of the following product, cast to fp32 where LayerNorm runs
    char* dln = h->at<char>(P.dln);
    float* lnpart = h->at<float>(P.lnpart);
    int lnset = 0;   // the next LayerNorm partial set
    float* cspart = h->at<float>(P.cspart);
    float* sumscr = h->at<float>(P.sumscr);
    void* skpart = h->at<char>(P.splitk);
    const int lnblk = layernorm_backward_blocks(BT);
    // the embedding backward's id sort depends only on the token ids: it runs on the side stream,
    // under the products below, instead of alone at the end (issued after the lm_head input
    // gradient, see there)
    const bool presorted = h->side && embed_backward_presortable(BT);

    // LayerNorm backward; with bias_off >= 0 the incoming residual gradient's column sum
    // (gathered by the same kernel) is the bias gradient of the projection at that offset
    // (the weight, bias and projection-bias gradients come from the partial sets after the last
    // LayerNorm, in one reduction; the sets' order is the one the offsets table was built in)
    // (copy16: where the bf16 copy of the new residual gradient goes, or null)
    auto ln_bwd = [&](const void* x, const float* mean, const float* rstd, int64_t w_off, int accum_dres,
                      char* copy16) -> int {
        float* part = lnpart + (size_t)lnset++ * P.lnset_stride;
        return run(h, "layernorm_bwd", [&] {
            return layernorm_backward(dln, x, mean, rstd, prm + w_off, dres, copy16, accum_dres, part, lnblk, BT, C, bf,
                                      r16, s);
        });
    };
    // weight gradient dW (+)= dy^T x; with bias_off >= 0 also the bias gradient db (+)= colsum(dy),
    // fused into the product when the LDS-streamed path runs it
    auto dw = [&](const void* dy, int ldy, const void* x, int ldx, int M, int N, int64_t off,
                  int64_t bias_off = -1) -> int {
        GemmDesc g;
        g.A = dy; g.lda = ldy; g.a_layout = 1;
        g.B = x; g.ldb = ldx; g.b_layout = 1;
        g.M = M; g.N = N; g.K = BT;
        g.epi = EPI_F32; g.C = grd + off; g.ldc = N; g.alpha = 1.f; g.beta = acc;
        const Split sp = choose_split(M, N, BT, bf);
        g.nsplit = sp.ns; g.bn = sp.bn; g.partial = skpart;
        const bool fused = bias_off >= 0 && gemm_fuses_rowsum(g, bf);
        if (fused) { g.rowsum = grd + bias_off; g.rowsum_part = h->at<float>(P.rspart); }
        TRY(run(h, "gemm_dw", [&] { return gemm(g, bf, s); }));
        if (bias_off >= 0 && !fused)
            return run(h, "bias_grad", [&] { return colsum(dy, 0, bf, BT, M, cspart, grd + bias_off, acc, sumscr, s); });
        return GPT2_OK;
    };
    // lm_head: dhf = s dz wte ; dwte (+)= s dz^T hf   (dz = (softmax - onehot)/BT from the forward)
    {
        GemmDesc g;
        g.A = h->at<char>(P.logits); g.lda = Vp; g.a_layout = 0;
        g.B = h->wop(L.wte); g.ldb = C; g.b_layout = 1;
        g.M = BT; g.N = C; g.K = Vp;
        g.epi = EPI_BIAS_T; g.C = dln; g.ldc = C; g.alpha = grad_scale;
        TRY(run(h, "gemm_lm_head_dx", [&] { return gemm(g, bf, s); }));
        // The sort's one workgroup holds 128 KB of LDS, which leaves no room on its CU for a
        // product workgroup. Issued before this product (one round of tiles that each run the
        // whole vocabulary), it could hold back that CU's tiles; issued after it, the sort takes
        // the first CU that frees up and runs beside the weight-gradient product, whose many
        // tiles flow around it (measured: input gradient 1.14 -> 1.09 ms per step).
        if (presorted) {
            HIPTRY(hipEventRecord(h->side_fork, s), "fork side stream");
            HIPTRY(hipStreamWaitEvent(h->side, h->side_fork, 0), "fork side stream");
            HIPTRY(embed_backward_sort(h->at<int32_t>(P.idx), BT, h->at<char>(P.ebscratch), h->side),
                   "embedding id sort");
            HIPTRY(hipEventRecord(h->side_join, h->side), "join side stream");
        }
        g = GemmDesc();
        g.A = h->at<char>(P.logits); g.lda = Vp; g.a_layout = 1;
        g.B = h->at<char>(P.hf); g.ldb = C; g.b_layout = 1;
        g.M = Vp; g.N = C; g.K = BT;
        g.epi = EPI_F32; g.C = grd + L.wte; g.ldc = C; g.alpha = grad_scale; g.beta = acc;
        TRY(run(h, "gemm_lm_head_dw", [&] { return gemm(g, bf, s); }));
    }
    TRY(ln_bwd(h->at<char>(P.x_in[c.n_layer]), h->at<float>(P.meanf), h->at<float>(P.rstdf), L.lnf_w, 0,
               bf ? d16_out(c.n_layer - 1) : nullptr));

    for (int l = c.n_layer - 1; l >= 0; --l) {
        // x_out = x_mid + a Wpr^T + bpr
        char* g_out = d16_out(l);
        if (!grouped) TRY(dw(g_out, C, h->at<char>(P.a[l]), F, C, F, L.w_pr[l]));
        {
            GemmDesc g;
            g.A = g_out; g.lda = C; g.a_layout = 0;
            g.B = h->wop(L.w_pr[l]); g.ldb = F; g.b_layout = 1;
            g.M = BT; g.N = F; g.K = C;
            g.epi = EPI_GELU_BWD; g.C = du_of(l); g.ldc = F; g.aux = h->at<char>(P.u[l]); g.ldaux = F;
            TRY(run(h, "gemm_dx", [&] { return gemm(g, bf, s); }));
        }
        if (!grouped) TRY(dw(du_of(l), F, h->at<char>(P.h2[l]), C, F, C, L.w_fc[l], L.b_fc[l]));
        {
            GemmDesc g;
            g.A = du_of(l); g.lda = F; g.a_layout = 0;
            g.B = h->wop(L.w_fc[l]); g.ldb = C; g.b_layout = 1;
            g.M = BT; g.N = C; g.K = F;
            g.epi = EPI_BIAS_T; g.C = dln; g.ldc = C; g.alpha = 1.f;
            TRY(run(h, "gemm_dx", [&] { return gemm(g, bf, s); }));
        }
        // (the column sum of the incoming dres is the mlp.c_proj bias gradient)
        TRY(ln_bwd(h->at<char>(P.x_mid[l]), h->at<float>(P.mean2[l]), h->at<float>(P.rstd2[l]), L.ln2_w[l], 1,
                   bf ? d16_mid(l) : nullptr));
        // x_mid = x_in + y Wo^T + bo
        char* g_mid = d16_mid(l);
        if (!grouped) TRY(dw(g_mid, C, h->at<char>(P.att[l]), C, C, C, L.w_o[l]));
        {
            GemmDesc g;
            g.A = g_mid; g.lda = C; g.a_layout = 0;
            g.B = h->wop(L.w_o[l]); g.ldb = C; g.b_layout = 1;
            g.M = BT; g.N = C; g.K = C;
            g.epi = EPI_BIAS_T; g.C = h->at<char>(P.datt); g.ldc = C; g.alpha = 1.f;
            TRY(run(h, "gemm_dx", [&] { return gemm(g, bf, s); }));
        }
        TRY(run(h, "attn_bwd", [&] {
            return attention_backward(h->at<char>(P.qkv[l]), h->at<char>(P.att[l]), h->at<char>(P.datt),
                                      h->at<float>(P.lse[l]), h->at<float>(P.Dbuf), dqkv_of(l), B, T, H, hs, bf, s);
        }));
        if (!grouped) TRY(dw(dqkv_of(l), 3 * C, h->at<char>(P.h1[l]), C, 3 * C, C, L.w_qkv[l], L.b_qkv[l]));
        {
            GemmDesc g;
            g.A = dqkv_of(l); g.lda = 3 * C; g.a_layout = 0;
            g.B = h->wop(L.w_qkv[l]); g.ldb = C; g.b_layout = 1;
            g.M = BT; g.N = C; g.K = 3 * C;
            g.epi = EPI_BIAS_T; g.C = dln; g.ldc = C; g.alpha = 1.f;
            TRY(run(h, "gemm_dx", [&] { return gemm(g, bf, s); }));
        }
        // (the column sum of the incoming dres is the attn.c_proj bias gradient)
        TRY(ln_bwd(h->at<char>(P.x_in[l]), h->at<float>(P.mean1[l]), h->at<float>(P.rstd1[l]), L.ln1_w[l], 1,
                   (bf && l > 0) ? d16_out(l - 1) : nullptr));
    }
    if (grouped)
        TRY(run(h, "gemm_dw", [&] {
            return gemm_grouped(h->at<GroupProb>(P.gprob), 4 * c.n_layer, h->group_tiles, BT, 1.f, acc, h->group_bn, s);
        }));
    // LayerNorm weight and bias gradients, and the projection bias gradients (column sums of the
    // residual gradient entering each ln_2 / ln_1), from every set at once
    TRY(run(h, "ln_param_grad", [&] {
        const int64_t* off = h->at<int64_t>(P.lnoff);
        return sum_partials_sets(lnpart, lnset, (int64_t)P.lnset_stride, lnblk, 3 * C, 3 * C, grd, off, 2 * C,
                                 off + (2 * c.n_layer + 1), acc, h->at<float>(P.lnscr), s);
    }));
    // embeddings: token rows scatter-add on top of the lm_head gradient, position rows
    if (!acc && T < c.block_size)
        HIPTRY(fill(grd + L.wpe + (int64_t)T * C, (int64_t)(c.block_size - T) * C, 0.f, s), "zero wpe tail");
    if (presorted) HIPTRY(hipStreamWaitEvent(s, h->side_join, 0), "join side stream");
    TRY(run(h, "embed_bwd", [&] {
        return embed_backward(h->at<int32_t>(P.idx), dres, grd + L.wte, grd + L.wpe, B, T, C, acc, r16,
                              h->at<char>(P.ebscratch), presorted ? 1 : 0, s);
    }));
    return GPT2_OK;
}

// =================================================================== optimizer
extern "C" int gpt2_adamw_step(gpt2_t* h, float lr, float beta1, float beta2, float eps, float weight_decay,
                               float max_grad_norm, int32_t t, float* d_grad_norm, float* h_grad_norm) {
    if (!h) return set_error(GPT2_EINVAL, "handle is null");
    if (t < 1) return set_error(GPT2_EINVAL, "AdamW step t must be >= 1");
    const Plan& P = h->P;
    hipStream_t s = h->stream;
    float* coef = h->at<float>(P.normcoef);
    const int64_t N = h->L.n_params;
    TRY(run(h, "grad_norm", [&] { return grad_norm(h->grads(), N, h->at<float>(P.normpart), coef, max_grad_norm, s); }));
    const double bc1 = 1.0 - std::pow((double)beta1, (double)t);
    const double bc2 = 1.0 - std::pow((double)beta2, (double)t);
    TRY(run(h, "adamw", [&] {
        return adamw(h->params(), h->grads(), h->at<float>(P.m), h->at<float>(P.v), h->bf16 ? h->at<char>(P.shadow) : nullptr,
                     N, h->L.decay_end, coef, lr, beta1, beta2, eps, weight_decay, (float)bc1, (float)std::sqrt(bc2),
                     nullptr, s);
    }));
    if (d_grad_norm) HIPTRY(hipMemcpyAsync(d_grad_norm, coef, 4, hipMemcpyDeviceToDevice, s), "copy norm");
    if (h_grad_norm) {
        HIPTRY(hipMemcpyAsync(h_grad_norm, coef, 4, hipMemcpyDeviceToHost, s), "copy norm");
        HIPTRY(hipStreamSynchronize(s), "synchronize");
    }
    return GPT2_OK;
}

// The same AdamW step with its learning rate and step count read from device memory when it
// runs, so that a step captured once in a graph keeps following the schedule on every replay.
extern "C" int gpt2_adamw_step_device(gpt2_t* h, const float* d_lr, const int32_t* d_t, float beta1, float beta2,
                                      float eps, float weight_decay, float max_grad_norm, float* d_grad_norm) {
    if (!h || !d_lr || !d_t) return set_error(GPT2_EINVAL, "null argument");
    const Plan& P = h->P;
    hipStream_t s = h->stream;
    float* coef = h->at<float>(P.normcoef);
    float* hp = coef + 16;   // (lr, bc1, sqrt(bc2)) in the same 256-byte block
    const int64_t N = h->L.n_params;
    TRY(run(h, "grad_norm", [&] { return grad_norm(h->grads(), N, h->at<float>(P.normpart), coef, max_grad_norm, s); }));
    HIPTRY(adamw_hparams(d_lr, d_t, beta1, beta2, hp, s), "adamw scalars");
    TRY(run(h, "adamw", [&] {
        return adamw(h->params(), h->grads(), h->at<float>(P.m), h->at<float>(P.v), h->bf16 ? h->at<char>(P.shadow) : nullptr,
                     N, h->L.decay_end, coef, 0.f, beta1, beta2, eps, weight_decay, 1.f, 1.f, hp, s);
    }));
    if (d_grad_norm) HIPTRY(hipMemcpyAsync(d_grad_norm, coef, 4, hipMemcpyDeviceToDevice, s), "copy norm");
    return GPT2_OK;
}

extern "C" int gpt2_schedule_step_device(gpt2_t* h, int32_t* d_step, float* d_lr, int32_t* d_t, double max_lr,
                                         double min_lr, int64_t warmup_steps, int64_t max_steps) {
    if (!h || !d_step || !d_lr || !d_t) return set_error(GPT2_EINVAL, "null argument");
    if (warmup_steps < 1 || max_steps <= warmup_steps) return set_error(GPT2_EINVAL, "need 1 <= warmup_steps < max_steps");
    HIPTRY(schedule_step(d_step, d_lr, d_t, max_lr, min_lr, warmup_steps, max_steps, h->stream), "schedule");
    return GPT2_OK;
}

// =================================================================== diagnostics
extern "C" int gpt2_timing_begin(gpt2_t* h, const char* name) {
    if (!h) return set_error(GPT2_EINVAL, "handle is null");
    if (name && class_index(name) < 0) return set_error(GPT2_EINVAL, "unknown kernel class %s", name);
    h->timing = true;
    h->filter = name ? name : "";
    h->ev_used = 0;
    h->times.clear();
    return GPT2_OK;
}

extern "C" int gpt2_timing_end(gpt2_t* h) {
    if (!h) return set_error(GPT2_EINVAL, "handle is null");
    h->timing = false;
    HIPTRY(hipStreamSynchronize(h->stream), "synchronize");
    for (size_t i = 0; i < h->ev_used; ++i) {
        float ms = 0.f;
        // a single-kernel product: its kernel's own interval; else the bracket of the call
        const auto& pr = h->ev_kern[i] ? h->ev_k[i] : h->ev[i];
        HIPTRY(hipEventElapsedTime(&ms, pr.first, pr.second), "event time");
        auto& t = h->times[kClasses[h->ev_cls[i]]];
        t.first += ms;
        t.second += 1;
    }
    h->ev_used = 0;
    return GPT2_OK;
}

extern "C" int gpt2_timing_get(gpt2_t* h, const char* name, double* total_ms, int64_t* launches) {
    if (!h || !name) return set_error(GPT2_EINVAL, "null argument");
    auto it = h->times.find(name);
    if (total_ms) *total_ms = it == h->times.end() ? 0.0 : it->second.first;
    if (launches) *launches = it == h->times.end() ? 0 : it->second.second;
    return GPT2_OK;
}

extern "C" int gpt2_debug_tensor(gpt2_t* h, const char* which, int32_t layer, float* d_dst, int64_t* count) {
    if (!h || !which || !count) return set_error(GPT2_EINVAL, "null argument");
    const gpt2_config& c = h->cfg;
    const int64_t BT = (int64_t)h->B * h->T;
    if (BT == 0) return set_error(GPT2_ESTATE, "no forward yet");
    const int64_t C = c.n_embd, F = c.mlp_hidden;
    const Plan& P = h->P;
    const bool lay = layer >= 0 && layer < c.n_layer;
    size_t off = 0;
    int64_t n = 0;
    bool f32 = false;
    std::string w = which;
    if (w == "x_in" && layer >= 0 && layer <= c.n_layer) { off = P.x_in[layer]; n = BT * C; f32 = !h->res16; }
    else if (w == "x_out") { off = P.x_in[c.n_layer]; n = BT * C; f32 = !h->res16; }
    else if (w == "hf") { off = P.hf; n = BT * C; }
    else if (w == "dz") { off = P.logits; n = BT * c.padded_vocab_size; }
    else if (lay && w == "h1") { off = P.h1[layer]; n = BT * C; }
    else if (lay && w == "qkv") { off = P.qkv[layer]; n = BT * 3 * C; }
    else if (lay && w == "att") { off = P.att[layer]; n = BT * C; }
    else if (lay && w == "lse") { off = P.lse[layer]; n = BT * c.n_head; f32 = true; }
    else if (lay && w == "h2") { off = P.h2[layer]; n = BT * C; }
    else if (lay && w == "u") { off = P.u[layer]; n = BT * F; }
    else if (lay && w == "a") { off = P.a[layer]; n = BT * F; }
    else return set_error(GPT2_EINVAL, "unknown tensor %s / layer %d", which, layer);
    *count = n;
    if (!d_dst) return GPT2_OK;
    HIPTRY(convert_to_f32(h->ws + off, d_dst, n, f32 ? 0 : h->bf16, h->stream), "convert");
    return GPT2_OK;
}
