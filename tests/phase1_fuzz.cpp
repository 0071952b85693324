// Host fuzz of phase 1 (no GPU): random, mostly invalid, tensor descriptors,
// parameters and length arrays go through fia_get_workspace_size and
// bsa_get_workspace_size, and every accepted plan through fia_run / bsa_run /
// fia_run_noalloc with the device hooks replaced by stand-ins.  Built with
// AddressSanitizer and UndefinedBehaviorSanitizer, so an out-of-bounds read of
// a descriptor, a signed overflow on huge dims or a leaked plan stops the run.
// Checked here: every call returns a defined status; a failed phase 1 leaves
// *plan NULL; an accepted plan is non-NULL and runs or fails with a defined
// status.  Tensor data pointers are never dereferenced by phase 1 (they are
// device pointers), so the descriptors point at nothing.
//
// Cases start from valid configurations of each path (prefill, paged prefill,
// decode, paged decode, int8 KV, MLA, block-sparse, FP8 block-sparse) and
// mutate a few fields with values from a pool of edge values (0, negatives,
// 2^31, 2^62, INT64 extremes, NaN scales, ranks 0 and 9, unknown dtypes and
// layouts), so the validation is exercised past its first checks.
//
// Usage: phase1_fuzz <iterations> <seed>; prints "all ok" and exits 0.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "fia.h"
#include "fia_internal.h"

namespace fia {
int launch_prefill(const fia_plan&, const AttnArgs&, void*) { return 0; }
int launch_decode(const fia_plan&, const DecodeArgs&, void*) { return 0; }
int launch_bsa(const fia_plan&, const AttnArgs&, void*) { return 0; }
static unsigned char g_dev_tables[1];
void* upload_tables(const void*, uint64_t) { return g_dev_tables; }
static unsigned char g_scratch[1];
void* noalloc_scratch() { return g_scratch; }
void free_tables(void*) {}
}  // namespace fia

static std::mt19937_64 rng;

static uint64_t pick(uint64_t n) { return n ? rng() % n : 0; }
static bool coin(double p) { return std::uniform_real_distribution<double>(0, 1)(rng) < p; }

static const int64_t kEdge[] = {0, 1, -1, 2, 3, 7, 15, 16, 17, 31, 32, 63, 64, 65, 127, 128, 129,
                                192, 256, 511, 512, 576, 1024, 2047, 2048, 4096, 65536,
                                (int64_t)1 << 29, (int64_t)1 << 31, ((int64_t)1 << 31) - 1,
                                (int64_t)1 << 40, (int64_t)1 << 62,
                                std::numeric_limits<int64_t>::max(),
                                std::numeric_limits<int64_t>::min()};

static int64_t edge() { return kEdge[pick(sizeof(kEdge) / sizeof(kEdge[0]))]; }

static char g_dummy[64];   // descriptors point here; phase 1 never reads it

static fia_tensor T(int dt, std::initializer_list<int64_t> d)
{
    fia_tensor t{};
    t.data = g_dummy;
    t.dtype = dt;
    t.ndim = (int)d.size();
    int i = 0;
    for (int64_t x : d) t.dims[i++] = x;
    return t;
}

static void mutate(fia_tensor& t)
{
    switch (pick(6)) {
    case 0: t.dims[pick(8)] = edge(); break;
    case 1: t.ndim = (int32_t)pick(11) - 1; break;          // -1 .. 9
    case 2: t.dtype = (int32_t)pick(12) - 1; break;         // -1 .. 10
    case 3: t.data = nullptr; break;
    case 4: if (t.ndim >= 1 && t.ndim <= 8) t.dims[pick((uint64_t)t.ndim)] = edge(); break;
    default:   // a small step, wrapping like the unsigned value it is
        if (t.ndim >= 1 && t.ndim <= 8) {
            int64_t& d = t.dims[pick((uint64_t)t.ndim)];
            d = (int64_t)((uint64_t)d + pick(5) - 2u);
        }
        break;
    }
}

// One case: the tensors and parameters of a phase-1 call, owned here.
struct Case {
    fia_tensor q{}, k{}, v{}, mask{}, bt{}, out{}, lse{}, ks{}, vs{}, ko{}, vo{}, qr{}, kr{};
    bool has_mask = false, has_bt = false, has_lse = false, has_ks = false, has_vs = false;
    bool has_ko = false, has_vo = false, has_qr = false, has_kr = false;
    std::vector<int64_t> lq, lkv;
    bool has_lq = false, has_lkv = false;
    fia_params p{};
    const char* layouts[9] = {"BSH", "BSND", "BNSD", "TND", "BNSD_BSND", "TND_NTD", "", "bsnd", nullptr};
};

static void base_case(Case& c)
{
    fia_params_init(&c.p);
    const int kind = (int)pick(10);
    const int B = 1 + (int)pick(4), QN = 8, KVN = 2, S = 1 + (int)pick(300), D = coin(0.5) ? 64 : 128;
    const int dt = coin(0.5) ? FIA_BF16 : FIA_F16;
    c.p.num_heads = QN;
    c.p.num_key_value_heads = KVN;
    c.p.scale_value = 0.125;
    c.p.return_softmax_lse = 1;
    c.has_lse = true;
    switch (kind) {
    case 0: {   // prefill BNSD / BSND / BSH, mode 0..4
        c.p.input_layout = "BNSD";
        c.q = T(dt, {B, QN, S, D});
        c.k = c.v = T(dt, {B, KVN, S + 7, D});
        c.out = c.q;
        c.lse = T(FIA_F32, {B, QN, S, 1});
        c.p.sparse_mode = (int64_t)pick(5);
        if (c.p.sparse_mode >= 2) { c.mask = T(FIA_U8, {2048, 2048}); c.has_mask = true; }
        if (c.p.sparse_mode == 1 || (c.p.sparse_mode == 0 && coin(0.5))) {
            c.mask = T(FIA_BOOL, {B, 1, S, S + 7});
            c.has_mask = true;
        }
        c.lq.assign((size_t)B, S);
        c.lkv.assign((size_t)B, S + 7);
        c.has_lq = c.has_lkv = coin(0.7);
        break;
    }
    case 1: {   // TND prefill, cumulative lengths
        c.p.input_layout = "TND";
        int64_t t = 0;
        for (int b = 0; b < B; ++b) { t += 1 + (int64_t)pick(100); c.lq.push_back(t); }
        c.lkv = c.lq;
        c.has_lq = c.has_lkv = true;
        c.q = T(dt, {t, QN, D});
        c.k = c.v = T(dt, {t, KVN, D});
        c.out = c.q;
        c.lse = T(FIA_F32, {t, QN, 1});
        c.p.sparse_mode = 3;
        c.mask = T(FIA_U8, {2048, 2048});
        c.has_mask = true;
        if (coin(0.5)) {   // paged
            c.p.block_size = 128;
            c.k = c.v = T(dt, {64, KVN, 128, D});
            c.bt = T(FIA_I32, {B, 16});
            c.has_bt = true;
        }
        break;
    }
    case 2: {   // decode, contiguous or paged, optional mask
        c.p.input_layout = "BSND";
        c.q = T(dt, {B, 1, QN, D});
        c.out = c.q;
        c.lse = T(FIA_F32, {B, QN, 1, 1});
        c.lkv.assign((size_t)B, 1 + (int64_t)pick(4000));
        c.has_lkv = true;
        if (coin(0.5)) {
            c.p.block_size = 128;
            c.k = c.v = T(dt, {256, 128, KVN * D});
            c.bt = T(FIA_I32, {B, 32});
            c.has_bt = true;
        } else {
            c.k = c.v = T(dt, {B, 4096, KVN, D});
        }
        if (coin(0.3)) { c.mask = T(FIA_U8, {B, 4096}); c.has_mask = true; }
        break;
    }
    case 3: {   // int8 KV decode
        c.p.input_layout = "BNSD";
        c.q = T(FIA_BF16, {B, QN, 1, D});
        c.out = c.q;
        c.lse = T(FIA_F32, {B, QN, 1, 1});
        c.k = c.v = T(FIA_I8, {B, KVN, 2048, D});
        c.p.key_quant_mode = c.p.value_quant_mode = (int64_t)pick(2);
        if (c.p.key_quant_mode == 0) c.ks = c.vs = T(FIA_BF16, {KVN, D});
        else c.ks = c.vs = T(FIA_F32, {B, 2048});
        if (coin(0.4)) {   // paged pool, query S 1
            c.p.block_size = 64;
            c.k = c.v = T(FIA_I8, {128, KVN, 64, D});
            c.bt = T(FIA_I32, {B, 32});
            c.has_bt = true;
        } else if (coin(0.4)) {   // multi-token, G * S <= 16, bottom-right causal
            const int Sq = 1 + (int)pick(4);
            c.q = T(FIA_BF16, {B, QN, Sq, D});
            c.out = c.q;
            c.lse = T(FIA_F32, {B, QN, Sq, 1});
            c.p.sparse_mode = 3;
            c.mask = T(FIA_U8, {2048, 2048});
            c.has_mask = Sq > 1;
        }
        c.ko = c.vo = c.ks;
        c.has_ks = c.has_vs = true;
        c.has_ko = c.has_vo = coin(0.5);
        c.lkv.assign((size_t)B, 1 + (int64_t)pick(2048));
        c.has_lkv = true;
        break;
    }
    case 4: {   // MLA decode
        const int MQN = 1 << pick(8);
        c.p.input_layout = "BSND";
        c.p.num_heads = MQN;
        c.p.num_key_value_heads = 1;
        const int Sq = coin(0.5) ? 1 : 1 + (int)pick(16);
        c.q = T(dt, {B, Sq, MQN, 512});
        c.qr = T(dt, {B, Sq, MQN, 64});
        c.out = c.q;
        c.lse = T(FIA_F32, {B, MQN, Sq, 1});
        c.k = c.v = T(dt, {128, 128, 512});
        c.kr = T(dt, {128, 128, 64});
        c.has_qr = c.has_kr = true;
        c.p.block_size = 128;
        c.bt = T(FIA_I32, {B, 32});
        c.has_bt = true;
        c.lkv.assign((size_t)B, (int64_t)pick(4096));
        c.has_lkv = true;
        if (Sq > 1) { c.p.sparse_mode = 3; c.mask = T(FIA_U8, {2048, 2048}); c.has_mask = true; }
        if (coin(0.4)) {   // bottom-right band, also at query S 1
            c.p.sparse_mode = 4;
            c.p.pre_tokens = (int64_t)pick(3000);
            c.p.next_tokens = (int64_t)pick(3);
            c.mask = T(FIA_U8, {2048, 2048});
            c.has_mask = coin(0.7);
        }
        break;
    }
    case 6: {   // MLA decode with a TND query: 1..16 tokens per batch
        const int MQN = 1 << pick(8);
        c.p.input_layout = "TND";
        c.p.num_heads = MQN;
        c.p.num_key_value_heads = 1;
        int64_t t = 0;
        for (int b = 0; b < B; ++b) {
            t += 1 + (int64_t)pick(16);
            c.lq.push_back(t);
            c.lkv.push_back((int64_t)pick(4096));
        }
        c.has_lq = c.has_lkv = true;
        c.q = T(dt, {t, MQN, 512});
        c.qr = T(dt, {t, MQN, 64});
        c.out = c.q;
        c.lse = T(FIA_F32, {t, MQN, 1});
        c.k = c.v = T(dt, {128, 128, 512});
        c.kr = T(dt, {128, 128, 64});
        c.has_qr = c.has_kr = true;
        c.p.block_size = 128;
        c.bt = T(FIA_I32, {B, 32});
        c.has_bt = true;
        c.p.sparse_mode = coin(0.5) ? 3 : 0;
        if (c.p.sparse_mode == 3) { c.mask = T(FIA_U8, {2048, 2048}); c.has_mask = true; }
        break;
    }
    case 7: {   // TND prefill with D_qk 192, D_v 128
        c.p.input_layout = "TND";
        int64_t t = 0;
        for (int b = 0; b < B; ++b) { t += 1 + (int64_t)pick(200); c.lq.push_back(t); }
        c.lkv = c.lq;
        c.has_lq = c.has_lkv = true;
        c.q = T(dt, {t, QN, 192});
        c.k = T(dt, {t, KVN, 192});
        c.v = T(dt, {t, KVN, 128});
        c.out = T(dt, {t, QN, 128});
        c.lse = T(FIA_F32, {t, QN, 1});
        c.p.sparse_mode = (int64_t)pick(5);
        c.mask = T(FIA_U8, {2048, 2048});
        c.has_mask = c.p.sparse_mode >= 2;
        c.p.pre_tokens = (int64_t)pick(300);
        c.p.next_tokens = (int64_t)pick(300);
        break;
    }
    default: {  // multi-token decode / prefill against a paged cache
        c.p.input_layout = "BSH";
        const int Sq = 1 + (int)pick(16);
        c.q = T(dt, {B, Sq, QN * D});
        c.out = c.q;
        c.lse = T(FIA_F32, {B, QN, Sq, 1});
        c.k = c.v = T(dt, {64, KVN, 256, D});
        c.p.block_size = 256;
        c.bt = T(FIA_I32, {B, 16});
        c.has_bt = true;
        c.p.sparse_mode = 3;
        c.mask = T(FIA_U8, {2048, 2048});
        c.has_mask = true;
        c.lkv.assign((size_t)B, Sq + (int64_t)pick(4000));
        c.has_lkv = true;
        break;
    }
    }
}

static void mutate_params(Case& c)
{
    fia_params& p = c.p;
    switch (pick(16)) {
    case 0: p.input_layout = c.layouts[pick(9)]; break;
    case 1: p.num_heads = edge(); break;
    case 2: p.num_key_value_heads = edge(); break;
    case 3: {
        const double s[] = {0.0, -1.0, 1e30, -1e-30, std::nan(""), INFINITY, -INFINITY, 1e-300};
        p.scale_value = s[pick(8)];
        break;
    }
    case 4: p.pre_tokens = edge(); break;
    case 5: p.next_tokens = edge(); break;
    case 6: p.sparse_mode = (int64_t)pick(11) - 1; break;
    case 7: p.block_size = edge(); break;
    case 8: p.inner_precise = (int64_t)pick(7) - 1; break;
    case 9: p.return_softmax_lse = (int32_t)pick(3); break;
    case 10: p.key_quant_mode = (int64_t)pick(8) - 1; break;
    case 11: p.value_quant_mode = (int64_t)pick(8) - 1; break;
    case 12: {   // a length entry
        std::vector<int64_t>& L = coin(0.5) ? c.lq : c.lkv;
        if (!L.empty()) L[pick(L.size())] = edge();
        break;
    }
    case 13: {   // the count of a length array
        std::vector<int64_t>& L = coin(0.5) ? c.lq : c.lkv;
        L.resize(pick(8));
        for (auto& x : L) x = coin(0.5) ? edge() : (int64_t)pick(300);
        break;
    }
    case 14: if (coin(0.5)) c.has_lq = !c.has_lq; else c.has_lkv = !c.has_lkv; break;
    default: {   // drop or add an optional tensor
        bool* flags[] = {&c.has_mask, &c.has_bt, &c.has_lse, &c.has_ks, &c.has_vs, &c.has_ko,
                         &c.has_vo, &c.has_qr, &c.has_kr};
        bool* f = flags[pick(9)];
        *f = !*f;
        break;
    }
    }
}

static void mutate_tensor(Case& c)
{
    fia_tensor* ts[] = {&c.q, &c.k, &c.v, &c.mask, &c.bt, &c.out, &c.lse, &c.ks, &c.vs, &c.ko, &c.vo,
                        &c.qr, &c.kr};
    mutate(*ts[pick(13)]);
}

// A heap copy of a descriptor: a read past its dims then lands in the
// allocator's red zone, where AddressSanitizer reports it.
struct Heap {
    std::vector<fia_tensor*> all;
    const fia_tensor* operator()(const fia_tensor& t)
    {
        all.push_back(new fia_tensor(t));
        return all.back();
    }
    ~Heap()
    {
        for (fia_tensor* t : all) delete t;
    }
};

static long n_ok = 0, n_err = 0, n_run_ok = 0;
static int failures = 0;

static void expect(bool cond, const char* what, long it)
{
    if (!cond) {
        std::printf("FAIL iteration %ld: %s\n", it, what);
        ++failures;
    }
}

static bool status_ok(int s) { return s >= FIA_OK && s <= FIA_ERR_HIP; }

static void run_plan(fia_plan* plan, uint64_t ws, bool bsa, long it)
{
    // the workspace is a device pointer the host side never dereferences
    void* w = ws ? (void*)g_dummy : nullptr;
    const int s1 = bsa ? bsa_run(w, ws, plan, nullptr) : fia_run(w, ws, plan, nullptr);
    expect(status_ok(s1), "run status out of range", it);
    if (s1 == FIA_OK) ++n_run_ok;
    if (ws) {
        const int s2 = bsa ? bsa_run(w, ws - 1, plan, nullptr) : fia_run(w, ws - 1, plan, nullptr);
        expect(s2 == FIA_ERR_WORKSPACE, "a workspace one byte short was accepted", it);
    }
    const int s3 = fia_run_noalloc(plan, nullptr);
    expect(status_ok(s3), "no-alloc run status out of range", it);
    if (bsa && s1 == FIA_OK) {
        uint64_t co = 0, io = 0;
        int64_t nqb = 0, nkb = 0;
        expect(status_ok(bsa_schedule_layout(plan, &co, &io, &nqb, &nkb)), "schedule layout status", it);
    }
}

static void fia_case(long it)
{
    Case c;
    base_case(c);
    const int muts = (int)pick(4);   // 0 .. 3 mutations (0 keeps the valid base case)
    for (int m = 0; m < muts; ++m) {
        if (coin(0.5)) mutate_params(c);
        else mutate_tensor(c);
    }
    Heap h;
    c.p.actual_seq_qlen = c.has_lq ? c.lq.data() : nullptr;
    c.p.n_actual_seq_qlen = c.has_lq ? (int64_t)c.lq.size() : 0;
    c.p.actual_seq_kvlen = c.has_lkv ? c.lkv.data() : nullptr;
    c.p.n_actual_seq_kvlen = c.has_lkv ? (int64_t)c.lkv.size() : 0;
    c.p.dequant_scale_key = c.has_ks ? h(c.ks) : nullptr;
    c.p.dequant_scale_value = c.has_vs ? h(c.vs) : nullptr;
    c.p.dequant_offset_key = c.has_ko ? h(c.ko) : nullptr;
    c.p.dequant_offset_value = c.has_vo ? h(c.vo) : nullptr;
    c.p.query_rope = c.has_qr ? h(c.qr) : nullptr;
    c.p.key_rope = c.has_kr ? h(c.kr) : nullptr;
    uint64_t ws = 12345;
    fia_plan* plan = (fia_plan*)&ws;   // must be overwritten
    const int s = fia_get_workspace_size(h(c.q), h(c.k), coin(0.05) ? nullptr : h(c.v),
                                         c.has_mask ? h(c.mask) : nullptr, c.has_bt ? h(c.bt) : nullptr,
                                         &c.p, h(c.out), c.has_lse ? h(c.lse) : nullptr, &ws, &plan);
    expect(status_ok(s), "phase-1 status out of range", it);
    if (s != FIA_OK) {
        expect(plan == nullptr, "failed phase 1 left a plan", it);
        ++n_err;
        return;
    }
    ++n_ok;
    expect(plan != nullptr, "accepted phase 1 without a plan", it);
    if (plan) run_plan(plan, ws, false, it);
    fia_plan_destroy(plan);
}

static void bsa_case(long it)
{
    bsa_params p;
    bsa_params_init(&p);
    const int B = 1 + (int)pick(3), N1 = 4, N2 = 2, S = 1 + (int)pick(1000), D = coin(0.5) ? 64 : 128;
    const bool fp8 = coin(0.3);
    const int dt = fp8 ? FIA_F8E4M3 : (coin(0.5) ? FIA_BF16 : FIA_F16);
    const int Dd = fp8 ? 128 : D;
    p.num_heads = N1;
    p.num_key_value_heads = N2;
    p.softmax_lse_flag = 1;
    int64_t X = 128, Y = fp8 ? (coin(0.5) ? 256 : 512) : 128;
    p.block_shape[0] = X;
    p.block_shape[1] = Y;
    const int lay = (int)pick(3);   // BNSD, BSND, TND
    const int64_t T_ = (int64_t)B * S;
    fia_tensor q = lay == 0 ? T(dt, {B, N1, S, Dd}) : lay == 1 ? T(dt, {B, S, N1, Dd}) : T(dt, {T_, N1, Dd});
    fia_tensor k = lay == 0 ? T(dt, {B, N2, S, Dd}) : lay == 1 ? T(dt, {B, S, N2, Dd}) : T(dt, {T_, N2, Dd});
    fia_tensor v = k;
    fia_tensor m = T(FIA_U8, {B, N1, (S + X - 1) / X, (S + Y - 1) / Y});
    fia_tensor out = q;
    out.dtype = fp8 ? FIA_BF16 : dt;
    fia_tensor lse = lay == 2 ? T(FIA_F32, {T_, N1, 1}) : T(FIA_F32, {B, N1, S, 1});
    fia_tensor sq = T(FIA_F32, {B, N1, (S + 127) / 128, 1});
    fia_tensor sk = T(FIA_F32, {B, N2, (S + Y - 1) / Y, 1});
    fia_tensor am = T(FIA_U8, {2048, 2048}), bt = T(FIA_I32, {B, 8});
    std::vector<int64_t> lq((size_t)B, S), lkv((size_t)B, S);
    if (lay == 2)   // TND: cumulative
        for (int b = 0; b < B; ++b) lq[(size_t)b] = lkv[(size_t)b] = (int64_t)(b + 1) * S;
    const char* lname = lay == 0 ? "BNSD" : lay == 1 ? "BSND" : "TND";
    p.q_input_layout = p.kv_input_layout = lname;
    bool has_len = lay == 2 || coin(0.5), has_am = false, has_bt = false, has_lse = true;
    bool has_sq = fp8, has_sk = fp8, has_sv = fp8;
    const char* layouts[] = {"BNSD", "BSND", "TND", "BSH", "", nullptr};
    const int muts = (int)pick(4);
    for (int i = 0; i < muts; ++i) {
        switch (pick(12)) {
        case 0: p.q_input_layout = layouts[pick(6)]; break;
        case 1: p.kv_input_layout = layouts[pick(6)]; break;
        case 2: p.num_heads = edge(); break;
        case 3: p.num_key_value_heads = edge(); break;
        case 4: p.block_shape[pick(2)] = edge(); break;
        case 5: p.mask_type = edge(); p.block_size = coin(0.5) ? edge() : 0; break;
        case 6: p.inner_precise = (int64_t)pick(7) - 1; p.pre_tokens = coin(0.5) ? edge() : p.pre_tokens; break;
        case 7: { std::vector<int64_t>& L = coin(0.5) ? lq : lkv;
                  if (coin(0.5)) L.resize(pick(6)); if (!L.empty()) L[pick(L.size())] = edge(); has_len = true; break; }
        case 8: { fia_tensor* ts[] = {&q, &k, &v, &m, &out, &lse, &sq, &sk};
                  mutate(*ts[pick(8)]); break; }
        case 9: has_am = !has_am; break;
        case 10: has_bt = !has_bt; break;
        default: { bool* f[] = {&has_lse, &has_sq, &has_sk, &has_sv}; bool* x = f[pick(4)]; *x = !*x; break; }
        }
    }
    p.actual_seq_lengths = has_len ? lq.data() : nullptr;
    p.n_actual_seq_lengths = has_len ? (int64_t)lq.size() : 0;
    p.actual_seq_lengths_kv = has_len ? lkv.data() : nullptr;
    p.n_actual_seq_lengths_kv = has_len ? (int64_t)lkv.size() : 0;
    Heap h;
    p.dequant_scale_query = has_sq ? h(sq) : nullptr;
    p.dequant_scale_key = has_sk ? h(sk) : nullptr;
    p.dequant_scale_value = has_sv ? h(sk) : nullptr;
    uint64_t ws = 777;
    fia_plan* plan = (fia_plan*)&ws;
    const int s = bsa_get_workspace_size(h(q), h(k), h(v), h(m), has_am ? h(am) : nullptr,
                                         has_bt ? h(bt) : nullptr, &p, h(out), has_lse ? h(lse) : nullptr,
                                         &ws, &plan);
    expect(status_ok(s), "block-sparse phase-1 status out of range", it);
    if (s != FIA_OK) {
        expect(plan == nullptr, "failed block-sparse phase 1 left a plan", it);
        ++n_err;
        return;
    }
    ++n_ok;
    expect(plan != nullptr, "accepted block-sparse phase 1 without a plan", it);
    if (plan) run_plan(plan, ws, true, it);
    fia_plan_destroy(plan);
}

int main(int argc, char** argv)
{
    const long iters = argc > 1 ? std::atol(argv[1]) : 20000;
    rng.seed(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1);
    // NULL arguments
    uint64_t ws;
    fia_plan* plan;
    fia_params p;
    fia_params_init(&p);
    fia_tensor t = T(FIA_BF16, {1, 1, 1, 64});
    expect(fia_get_workspace_size(nullptr, &t, &t, nullptr, nullptr, &p, &t, nullptr, &ws, &plan) ==
               FIA_ERR_NULLPTR, "NULL query", -1);
    expect(fia_get_workspace_size(&t, &t, &t, nullptr, nullptr, nullptr, &t, nullptr, &ws, &plan) ==
               FIA_ERR_NULLPTR, "NULL params", -1);
    expect(fia_run(nullptr, 0, nullptr, nullptr) != FIA_OK, "run of a NULL plan", -1);
    expect(fia_run_noalloc(nullptr, nullptr) != FIA_OK, "no-alloc run of a NULL plan", -1);
    fia_plan_destroy(nullptr);
    for (int s = -2; s < 12; ++s) expect(fia_status_string((fia_status)s) != nullptr, "status string", -1);
    for (long it = 0; it < iters; ++it) {
        if (coin(0.8)) fia_case(it);
        else bsa_case(it);
    }
    std::printf("%ld accepted (%ld ran), %ld rejected, %d failures\n", n_ok, n_run_ok, n_err, failures);
    if (!failures) std::printf("all ok\n");
    return failures ? 1 : 0;
}
