// Host check of the schedule tables that phase 1 builds (no GPU): the planner
// is linked with stand-ins for its device hooks, the table image it would
// upload is captured, and its invariants are checked.
//   prefill: every (batch, head group, row block) holding a valid query row is
//            one workgroup; zero-fill workgroups come first and cover exactly
//            the padding rows of every batch; the workgroups of one XCD bucket
//            (kv head mod 8) appear in non-increasing kv-tile order;
//   block-sparse: every (batch, head, 128-row slice of a q block) is one
//            workgroup and no workgroup straddles two q blocks;
//   decode:  the pieces of each segment are contiguous, 16-aligned at their
//            start, and cover exactly the segment's kv range (for the MLA
//            sliding band from the first key any row can see); the waves' piece
//            ranges are monotone and cover every piece; no wave's token load
//            exceeds the common quota.
// Prints one line per failure and "all ok" at the end; the exit status is the
// number of failing cases.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <map>
#include <random>
#include <tuple>
#include <vector>

#include "fia.h"
#include "fia_internal.h"

static std::vector<unsigned char> g_tables;

namespace fia {
int launch_prefill(const fia_plan&, const AttnArgs&, void*) { return 0; }
int launch_decode(const fia_plan&, const DecodeArgs&, void*) { return 0; }
int launch_bsa(const fia_plan&, const AttnArgs&, void*) { return 0; }
void* upload_tables(const void* src, uint64_t bytes)
{
    g_tables.assign((const unsigned char*)src, (const unsigned char*)src + bytes);
    return &g_tables;   // a non-null stand-in: phase 1 then records a runnable plan
}
void* noalloc_scratch() { return nullptr; }
void free_tables(void*) {}
}  // namespace fia

static int failures = 0;
#define EXPECT(cond, ...)                            \
    do {                                             \
        if (!(cond)) {                               \
            std::printf("FAIL %s: ", name);          \
            std::printf(__VA_ARGS__);                \
            std::printf("\n");                       \
            ++failures;                              \
            return;                                  \
        }                                            \
    } while (0)

static fia_tensor T(int dt, std::vector<int64_t> d)
{
    fia_tensor t{};
    t.data = (void*)0x1000;
    t.dtype = dt;
    t.ndim = (int)d.size();
    for (size_t i = 0; i < d.size(); ++i) t.dims[i] = d[i];
    return t;
}

// kv tiles (64 keys) a row block [q0, q1) of a batch reads under the mode's band
static int64_t kv_tiles(int mode, int64_t lq, int64_t lkv, int64_t q0, int64_t q1)
{
    const int64_t qend = std::min(q1, lq);
    if (qend <= q0 || lkv <= 0) return 0;
    int64_t hi = lkv;
    if (mode == 2) hi = std::min<int64_t>(lkv, qend);
    if (mode == 3) hi = std::min<int64_t>(lkv, qend + lkv - lq);
    if (hi <= 0) return 0;
    return (hi + 63) / 64;
}

// BSND prefill, modes 0 (no mask), 2 or 3, with per-batch lengths L
static void check_prefill(const char* name, int B, int QN, int KVN, int S, int mode, const std::vector<int64_t>& L)
{
    const int D = 128;
    fia_tensor q = T(FIA_BF16, {B, S, QN, D}), k = T(FIA_BF16, {B, S, KVN, D}), o = q;
    fia_tensor lse = T(FIA_F32, {B, QN, S, 1});
    fia_params p;
    fia_params_init(&p);
    p.input_layout = "BSND";
    p.num_heads = QN;
    p.num_key_value_heads = KVN;
    p.sparse_mode = mode;
    p.scale_value = 0.1;
    p.return_softmax_lse = 1;
    p.actual_seq_qlen = L.data();
    p.n_actual_seq_qlen = B;
    p.actual_seq_kvlen = L.data();
    p.n_actual_seq_kvlen = B;
    uint64_t ws = 0;
    fia_plan* plan = nullptr;
    g_tables.clear();
    const fia_status st = fia_get_workspace_size(&q, &k, &k, nullptr, nullptr, &p, &o, &lse, &ws, &plan);
    EXPECT(st == FIA_OK, "phase 1 status %d", (int)st);
    const int n = (int)plan->n_tiles;
    const int hg = plan->attn.hg, G = QN / KVN, rows_per = 32 * 4 / hg;
    EXPECT(n == 0 || g_tables.size() >= plan->off_tiles + (size_t)n * sizeof(fia::Tile), "table image too small");
    const fia::Tile* t = n ? (const fia::Tile*)(g_tables.data() + plan->off_tiles) : nullptr;
    std::map<std::tuple<int, int, int>, int> seen;
    std::vector<std::vector<std::pair<int, int>>> zero(B);
    bool attention_started = false;
    int last_work[8];
    std::fill(last_work, last_work + 8, 1 << 30);
    for (int i = 0; i < n; ++i) {
        if (t[i].h < 0) {
            EXPECT(!attention_started, "zero-fill entry %d after attention entries", i);
            zero[t[i].b].push_back({t[i].q0, t[i].q1});
            continue;
        }
        attention_started = true;
        EXPECT(t[i].h % hg == 0 && t[i].q0 % rows_per == 0, "entry %d misaligned", i);
        ++seen[{t[i].b, t[i].h, t[i].q0}];
        const int x = (t[i].h / G) % 8;
        const int w = (int)kv_tiles(mode, L[t[i].b], L[t[i].b], t[i].q0, t[i].q1);
        EXPECT(w <= last_work[x], "XCD bucket %d out of longest-first order at entry %d", x, i);
        last_work[x] = w;
    }
    for (int b = 0; b < B; ++b) {
        const int zfrom = (int)std::min<int64_t>(S, (L[b] + rows_per - 1) / rows_per * rows_per);
        for (int q0 = 0; q0 < zfrom; q0 += rows_per)
            for (int h = 0; h < QN; h += hg) {
                const int times = seen[std::make_tuple(b, h, q0)];
                EXPECT(times == 1, "batch %d head %d rows %d scheduled %d times", b, h, q0, times);
            }
        std::sort(zero[b].begin(), zero[b].end());
        int at = zfrom;
        for (auto& z : zero[b]) {
            EXPECT(z.first == at && z.second > z.first, "batch %d zero-fill gap or overlap at row %d", b, at);
            at = z.second;
        }
        EXPECT(at == S || (zero[b].empty() && zfrom == S), "batch %d padding rows [%d, %d) not covered", b, at, S);
    }
    EXPECT(seen.size() == (size_t)(n - std::count_if(t, t + n, [](const fia::Tile& e) { return e.h < 0; })),
           "duplicate workgroups");
    fia_plan_destroy(plan);
}

// paged GQA decode (query S 1) with kv lengths L, page size bs
static void check_decode(const char* name, int B, int QN, int KVN, const std::vector<int64_t>& L, int bs)
{
    const int D = 128;
    int64_t maxb = 1;
    for (int64_t x : L) maxb = std::max<int64_t>(maxb, (x + bs - 1) / bs);
    int64_t nb = 0;
    for (int64_t x : L) nb += (x + bs - 1) / bs;
    fia_tensor q = T(FIA_BF16, {B, QN, 1, D}), o = q;
    fia_tensor k = T(FIA_BF16, {std::max<int64_t>(nb, 1), KVN, bs, D});
    fia_tensor lse = T(FIA_F32, {B, QN, 1, 1});
    fia_tensor bt = T(FIA_I32, {B, maxb});
    fia_params p;
    fia_params_init(&p);
    p.input_layout = "BNSD";
    p.num_heads = QN;
    p.num_key_value_heads = KVN;
    p.scale_value = 0.1;
    p.block_size = bs;
    p.return_softmax_lse = 1;
    p.actual_seq_kvlen = L.data();
    p.n_actual_seq_kvlen = B;
    uint64_t ws = 0;
    fia_plan* plan = nullptr;
    g_tables.clear();
    const fia_status st = fia_get_workspace_size(&q, &k, &k, nullptr, &bt, &p, &o, &lse, &ws, &plan);
    EXPECT(st == FIA_OK, "phase 1 status %d", (int)st);
    const fia::DecodeArgs& d = plan->dec;
    const int nseg = B * KVN * d.nhc, np = (int)plan->n_pieces, nw = (int)plan->n_waves;
    const fia::DecSeg* seg = (const fia::DecSeg*)(g_tables.data() + plan->off_batch);
    const fia::DecPiece* pc = (const fia::DecPiece*)(g_tables.data() + plan->off_pieces);
    const int32_t* wf = (const int32_t*)(g_tables.data() + plan->off_waves);
    int64_t total = 0;
    for (int s = 0; s < nseg; ++s) {
        const int b = s / (KVN * d.nhc);
        EXPECT(seg[s].b == b && seg[s].lkv == (int)L[b], "segment %d header", s);
        total += L[b];
        if (L[b] == 0) {
            EXPECT(seg[s].count == 0, "empty segment %d has pieces", s);
            continue;
        }
        EXPECT(seg[s].count > 0 && seg[s].first >= 0 && seg[s].first + seg[s].count <= np, "segment %d range", s);
        int at = 0;
        for (int i = seg[s].first; i < seg[s].first + seg[s].count; ++i) {
            EXPECT(pc[i].seg == s && pc[i].t0 == at && pc[i].t1 > pc[i].t0 && pc[i].t0 % 16 == 0,
                   "segment %d piece %d [%d, %d) at %d", s, i, pc[i].t0, pc[i].t1, at);
            EXPECT((pc[i].t1 - 1) / bs - pc[i].t0 / bs < 64, "piece %d spans more than 64 pages", i);
            at = pc[i].t1;
        }
        EXPECT(at == (int)L[b], "segment %d covers [0, %d) of %d", s, at, (int)L[b]);
    }
    EXPECT(np == 0 || (wf[0] == 0 && wf[nw] == np), "wave ranges do not cover the pieces");
    // total counts every segment's tokens; the planner's quota uses at least as
    // many waves as it fills, so this bound is not tighter than its own
    const int64_t quota = nw > 0 ? ((total + nw - 1) / nw + 31) / 32 * 32 : 0;
    for (int w = 0; w < nw; ++w) {
        EXPECT(wf[w] < wf[w + 1], "wave %d has no piece", w);
        int64_t load = 0;
        for (int i = wf[w]; i < wf[w + 1]; ++i) load += pc[i].t1 - pc[i].t0;
        EXPECT(load <= quota, "wave %d load %lld over the quota %lld", w, (long long)load, (long long)quota);
    }
    fia_plan_destroy(plan);
}

// MLA decode (query D 512 + rope 64, one kv head, paged), BNSD query of S
// tokens; sparse_mode 0 (S 1), 3, or 4 with pre_tokens `pre` (keys below
// Lkv - S - pre are outside every row's band and are not scheduled)
static void check_mla(const char* name, int B, int QN, int S, const std::vector<int64_t>& L, int bs, int mode,
                      int64_t pre)
{
    int64_t maxb = 1, nb = 0;
    for (int64_t x : L) {
        maxb = std::max<int64_t>(maxb, (x + bs - 1) / bs);
        nb += (x + bs - 1) / bs;
    }
    fia_tensor q = T(FIA_BF16, {B, QN, S, 512}), o = q, qr = T(FIA_BF16, {B, QN, S, 64});
    fia_tensor k = T(FIA_BF16, {std::max<int64_t>(nb, 1), bs, 512}), kr = T(FIA_BF16, {std::max<int64_t>(nb, 1), bs, 64});
    fia_tensor lse = T(FIA_F32, {B, QN, S, 1}), bt = T(FIA_I32, {B, maxb});
    fia_tensor tmpl = T(FIA_U8, {2048, 2048});
    fia_params p;
    fia_params_init(&p);
    p.input_layout = "BNSD";
    p.num_heads = QN;
    p.num_key_value_heads = 1;
    p.scale_value = 0.04;
    p.block_size = bs;
    p.sparse_mode = mode;
    if (mode == 4) {
        p.pre_tokens = pre;
        p.next_tokens = 0;
    }
    p.return_softmax_lse = 1;
    p.actual_seq_kvlen = L.data();
    p.n_actual_seq_kvlen = B;
    p.query_rope = &qr;
    p.key_rope = &kr;
    uint64_t ws = 0;
    fia_plan* plan = nullptr;
    g_tables.clear();
    const fia_status st = fia_get_workspace_size(&q, &k, &k, mode >= 3 ? &tmpl : nullptr, &bt, &p, &o, &lse, &ws,
                                                 &plan);
    EXPECT(st == FIA_OK, "phase 1 status %d", (int)st);
    const fia::DecodeArgs& d = plan->dec;
    const int nseg = B * d.nhc, np = (int)plan->n_pieces, nw = (int)plan->n_waves;
    EXPECT(d.mla_nw >= 2 && 16 * d.mla_nw >= d.Gc && d.Gc * d.nhc >= QN * S, "MLA chunking");
    const fia::DecSeg* seg = (const fia::DecSeg*)(g_tables.data() + plan->off_batch);
    const fia::DecPiece* pc = (const fia::DecPiece*)(g_tables.data() + plan->off_pieces);
    const int32_t* wf = (const int32_t*)(g_tables.data() + plan->off_waves);
    for (int sidx = 0; sidx < nseg; ++sidx) {
        const int b = sidx / d.nhc;
        const int64_t first =
            mode == 4 ? std::min<int64_t>(L[b], std::max<int64_t>(0, L[b] - S - pre)) / 16 * 16 : 0;
        if (first >= L[b]) {
            EXPECT(seg[sidx].count == 0, "segment %d with no visible key has pieces", sidx);
            continue;
        }
        int64_t at = first;
        for (int i = seg[sidx].first; i < seg[sidx].first + seg[sidx].count; ++i) {
            EXPECT(pc[i].seg == sidx && pc[i].t0 == at && pc[i].t1 > pc[i].t0 && pc[i].t0 % 16 == 0,
                   "segment %d piece %d [%d, %d) at %lld", sidx, i, pc[i].t0, pc[i].t1, (long long)at);
            EXPECT((pc[i].t1 - 1) / bs - pc[i].t0 / bs < 64, "piece %d spans more than 64 pages", i);
            at = pc[i].t1;
        }
        EXPECT(at == L[b], "segment %d covers [%lld, %lld) of %lld", sidx, (long long)first, (long long)at,
               (long long)L[b]);
    }
    EXPECT(np == 0 || (wf[0] == 0 && wf[nw] == np), "wave ranges do not cover the pieces");
    EXPECT(nw <= 256, "more MLA workgroups (%d) than CUs", nw);
    fia_plan_destroy(plan);
}

// block-sparse prefill, BNSD, block shape [X, Y], lengths L (query = kv)
static void check_bsa(const char* name, int B, int N1, int N2, int S, int X, int Y, const std::vector<int64_t>& L)
{
    const int D = 128;
    fia_tensor q = T(FIA_BF16, {B, N1, S, D}), k = T(FIA_BF16, {B, N2, S, D}), o = q;
    fia_tensor lse = T(FIA_F32, {B, N1, S, 1});
    fia_tensor mask = T(FIA_U8, {B, N1, (S + X - 1) / X, (S + Y - 1) / Y});
    bsa_params p;
    bsa_params_init(&p);
    p.q_input_layout = "BNSD";
    p.kv_input_layout = "BNSD";
    p.num_heads = N1;
    p.num_key_value_heads = N2;
    p.scale_value = 0.1;
    p.block_shape[0] = X;
    p.block_shape[1] = Y;
    p.actual_seq_lengths = L.data();
    p.n_actual_seq_lengths = B;
    p.actual_seq_lengths_kv = L.data();
    p.n_actual_seq_lengths_kv = B;
    p.softmax_lse_flag = 1;
    uint64_t ws = 0;
    fia_plan* plan = nullptr;
    g_tables.clear();
    const fia_status st = bsa_get_workspace_size(&q, &k, &k, &mask, nullptr, nullptr, &p, &o, &lse, &ws, &plan);
    EXPECT(st == FIA_OK, "phase 1 status %d", (int)st);
    const int n = (int)plan->n_tiles;
    const fia::Tile* t = n ? (const fia::Tile*)(g_tables.data() + plan->off_tiles) : nullptr;
    std::map<std::tuple<int, int, int>, int> seen;
    for (int i = 0; i < n; ++i) {
        EXPECT(t[i].h >= 0 && t[i].q1 > t[i].q0 && t[i].q1 - t[i].q0 <= 128 && t[i].q0 / X == (t[i].q1 - 1) / X,
               "entry %d rows [%d, %d) straddle a q block or exceed 128 rows", i, t[i].q0, t[i].q1);
        ++seen[{t[i].b, t[i].h, t[i].q0}];
    }
    int expect = 0;
    for (int b = 0; b < B; ++b)
        for (int qb = 0; qb * X < S; ++qb)
            for (int q0 = qb * X; q0 < std::min(S, (qb + 1) * X); q0 += 128)
                for (int h = 0; h < N1; ++h) {
                    ++expect;
                    const int times = seen[std::make_tuple(b, h, q0)];
                    EXPECT(times == 1, "batch %d head %d rows %d scheduled %d times", b, h, q0, times);
                }
    EXPECT(expect == n, "%d entries for %d (batch, head, row slice) items", n, expect);
    fia_plan_destroy(plan);
}

int main()
{
    check_prefill("causal GQA, padded", 4, 32, 8, 4096, 3, {2700, 2151, 1117, 2011});
    check_prefill("tiny dense", 1, 2, 2, 128, 3, {128});
    check_prefill("top-left causal, short batch", 3, 8, 2, 700, 2, {700, 1, 333});
    check_prefill("no mask, empty batch", 2, 12, 4, 1000, 0, {999, 0});
    check_prefill("GQA 64", 1, 64, 1, 5000, 3, {5000});
    std::mt19937 g(5);
    char nm[64];
    for (int r = 0; r < 30; ++r) {
        const int B = 1 + g() % 5, KVN = 1 << (g() % 4), G = 1 + g() % 8, S = 1 + g() % 3000;
        std::vector<int64_t> L(B);
        for (auto& x : L) x = g() % (S + 1);
        const int modes[3] = {0, 2, 3};
        std::snprintf(nm, sizeof nm, "random prefill %d", r);
        check_prefill(nm, B, KVN * G, KVN, S, modes[g() % 3], L);
    }
    check_decode("paged decode", 8, 32, 8, {512, 32768, 7000, 1, 0, 4096, 100, 20000}, 128);
    check_decode("paged decode, 16-token pages", 3, 8, 2, {5000, 17, 900}, 16);
    for (int r = 0; r < 10; ++r) {
        const int B = 1 + g() % 9, KVN = 1 << (g() % 3), G = 1 + g() % 6;
        std::vector<int64_t> L(B);
        for (auto& x : L) x = g() % 40000;
        const int bss[3] = {16, 64, 128};
        std::snprintf(nm, sizeof nm, "random decode %d", r);
        check_decode(nm, B, KVN * G, KVN, L, bss[g() % 3]);
    }
    check_mla("MLA decode, 128 heads", 6, 128, 1, {8192, 600, 16384, 17, 0, 3000}, 128, 0, 0);
    check_mla("MLA, 4 tokens causal, 16-token pages", 3, 32, 4, {2000, 90, 5000}, 16, 3, 0);
    check_mla("MLA sliding band", 4, 64, 2, {5000, 100, 4097, 1}, 128, 4, 1000);
    check_mla("MLA band wider than the cache", 2, 16, 1, {700, 3000}, 64, 4, 100000);
    check_bsa("block-sparse [128, 128]", 2, 8, 2, 1000, 128, 128, {1000, 333});
    check_bsa("block-sparse [256, 512]", 1, 4, 4, 3000, 256, 512, {2999});
    check_bsa("block-sparse [64, 128]", 3, 6, 3, 700, 64, 128, {700, 1, 650});
    if (!failures) std::printf("all ok\n");
    return failures;
}
