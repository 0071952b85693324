// Phase 1 of the fused inference attention and the block-sparse attention:
// input validation, dispatch, schedule tables and workspace sizing.  Host
// code; its only HIP calls allocate and fill the plan's device copy of the
// schedule tables (skipped when no device is visible).
//
// Validation follows the parameter descriptions and constraints of pages
// "torch_npu.npu_fused_infer_attention_score_v2", "torch_npu.npu_prompt_flash_
// attention", "aclnnFusedInferAttentionScoreV5" and "aclnnBlockSparse
// AttentionV2"; the reading taken where they are silent is stated inline.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <memory>
#include <numeric>
#include <string>

#include "fia_internal.h"

using namespace fia;

namespace {

constexpr int64_t kIntMax = 2147483647;
constexpr double kLog2e = 1.4426950408889634;

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

int64_t numel(const fia_tensor* t)
{
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i) n *= t->dims[i];
    return n;
}

// A descriptor the planner can do arithmetic on: rank 1..8, every dim in
// [0, 2^31), and the product of its non-zero dims at most 2^48 elements, so
// no product of its dims overflows int64.
bool valid_rank(const fia_tensor* t)
{
    if (t->ndim < 1 || t->ndim > 8) return false;
    int64_t vol = 1;
    for (int i = 0; i < t->ndim; ++i) {
        const int64_t d = t->dims[i];
        if (d < 0 || d > kIntMax) return false;
        if (d == 0) continue;
        if (vol > (((int64_t)1 << 48) / d)) return false;
        vol *= d;
    }
    return true;
}

// Every optional descriptor that is given passes valid_rank.
bool valid_optional(std::initializer_list<const fia_tensor*> ts)
{
    for (const fia_tensor* t : ts)
        if (t && !valid_rank(t)) return false;
    return true;
}

bool is_half(int32_t d) { return d == FIA_F16 || d == FIA_BF16; }

bool dims_are(const fia_tensor* t, std::initializer_list<int64_t> d)
{
    if (t->ndim != (int32_t)d.size()) return false;
    int i = 0;
    for (int64_t x : d)
        if (t->dims[i++] != x) return false;
    return true;
}

// Parses an input layout string.  Output-layout variants the pages list
// (e.g. "BNSD_BSND") are recognised and reported as unsupported.
fia_status parse_layout(const char* s, int32_t* layout, bool* bsh)
{
    if (!s) return FIA_ERR_NULLPTR;
    std::string v(s);
    *bsh = false;
    if (v == "BNSD") { *layout = LAYOUT_BNSD; return FIA_OK; }
    if (v == "BSND") { *layout = LAYOUT_BSND; return FIA_OK; }
    if (v == "BSH") { *layout = LAYOUT_BSND; *bsh = true; return FIA_OK; }
    if (v == "TND") { *layout = LAYOUT_TND; return FIA_OK; }
    static const char* variants[] = {"BNSD_BSND", "BSH_NBSD", "BSND_NBSD", "BNSD_NBSD", "TND_NTD",
                                     "NTD_TND", "NTD", "BSH_BNSD", "BSND_BNSD"};
    for (const char* x : variants)
        if (v == x) return FIA_ERR_UNSUPPORTED;
    return FIA_ERR_LAYOUT;
}

// Query/key/value geometry of one tensor under a layout: batch, heads, S, D.
struct Geo {
    int64_t B = 0, N = 0, S = 0, D = 0;
};

fia_status geometry(const fia_tensor* t, int32_t layout, bool bsh, int64_t heads, Geo* g)
{
    if (!valid_rank(t)) return FIA_ERR_SHAPE;
    if (bsh) {
        if (t->ndim != 3 || heads <= 0 || t->dims[2] % heads) return FIA_ERR_SHAPE;
        *g = {t->dims[0], heads, t->dims[1], t->dims[2] / heads};
        return FIA_OK;
    }
    if (layout == LAYOUT_TND) {
        if (t->ndim != 3) return FIA_ERR_SHAPE;
        *g = {0, t->dims[1], t->dims[0], t->dims[2]};
        return FIA_OK;
    }
    if (t->ndim != 4) return FIA_ERR_SHAPE;
    if (layout == LAYOUT_BNSD)
        *g = {t->dims[0], t->dims[1], t->dims[2], t->dims[3]};
    else
        *g = {t->dims[0], t->dims[2], t->dims[1], t->dims[3]};
    return FIA_OK;
}

// actual_seq lengths for padded layouts: count 1 broadcasts, count >= B takes
// the first B, other counts are rejected; NULL = the tensor's S.
fia_status resolve_lengths(const int64_t* arr, int64_t n, int64_t B, int64_t S,
                           std::vector<int64_t>* out)
{
    out->assign((size_t)B, S);
    if (!arr) return FIA_OK;
    if (n != 1 && n < B) return FIA_ERR_PARAM;
    for (int64_t b = 0; b < B; ++b) {
        int64_t v = arr[n == 1 ? 0 : b];
        if (v < 0 || v > S) return FIA_ERR_SHAPE;
        (*out)[(size_t)b] = v;
    }
    return FIA_OK;
}

// TND cumulative lengths: non-decreasing, non-negative, last <= T.
fia_status resolve_cumulative(const int64_t* arr, int64_t n, int64_t T,
                              std::vector<int64_t>* len, std::vector<int64_t>* start)
{
    if (!arr || n <= 0) return FIA_ERR_PARAM;
    len->resize((size_t)n);
    start->resize((size_t)n);
    int64_t prev = 0;
    for (int64_t b = 0; b < n; ++b) {
        if (arr[b] < prev) return FIA_ERR_SHAPE;
        (*start)[(size_t)b] = prev;
        (*len)[(size_t)b] = arr[b] - prev;
        prev = arr[b];
    }
    if (prev > T) return FIA_ERR_SHAPE;
    return FIA_OK;
}

bool mask_dtype_ok(int32_t d) { return d == FIA_BOOL || d == FIA_I8 || d == FIA_U8; }

bool is_template_2048(const fia_tensor* m)
{
    return dims_are(m, {2048, 2048}) || dims_are(m, {1, 2048, 2048}) ||
           dims_are(m, {1, 1, 2048, 2048});
}

// Scheduling weight of a prefill tile: number of kv tiles it visits.
int64_t kv_tiles_of(int32_t mode, bool has_mask, int64_t pre, int64_t next, int64_t lq,
                    int64_t lkv, int64_t q0, int64_t q1)
{
    const int64_t last = std::min(q1, lq) - 1;
    if (last < q0 || lkv <= 0) return 0;
    const int64_t delta = lkv - lq;
    int64_t lo = 0, hi = lkv;
    switch (mode) {
    case 0:
        if (has_mask) {
            lo = std::max<int64_t>(0, q0 - pre);
            hi = std::min<int64_t>(lkv, last + next + 1);
        }
        break;
    case 2: hi = std::min<int64_t>(lkv, last + 1); break;
    case 3: hi = std::min<int64_t>(lkv, last + delta + 1); break;
    case 4:
        lo = std::max<int64_t>(0, q0 + delta - pre);
        hi = std::min<int64_t>(lkv, last + delta + next + 1);
        break;
    default: break;
    }
    if (hi <= lo) return 0;
    const int64_t start = lo / kBlockN * kBlockN;
    return (hi - start + kBlockN - 1) / kBlockN;
}

// Phase-1 temporaries, kept per thread across calls: a caller that plans
// every step then reuses their memory instead of taking fresh pages from the
// allocator each time (the planner's buffers of a few hundred KB otherwise
// cost more than the planning itself).
struct WorkTile {
    int64_t work;                          // kv tiles the tile visits
    Tile t;
};
struct PlanScratch {
    std::vector<unsigned char> tables;     // host image of the schedule tables
    std::vector<Tile> tiles;
    std::vector<WorkTile> wt, wt2;
    std::vector<size_t> idx, pos;
    std::vector<int32_t> pref;
};
PlanScratch& plan_scratch()
{
    thread_local PlanScratch s;
    return s;
}
// Buffers grown past 64 MB by one huge plan are released after it.
void trim_scratch(PlanScratch& s)
{
    constexpr size_t kKeep = (size_t)64 << 20;
    auto trim = [](auto& v) {
        if (v.capacity() * sizeof(v[0]) > kKeep) std::remove_reference_t<decltype(v)>().swap(v);
    };
    trim(s.tables); trim(s.tiles); trim(s.wt); trim(s.wt2);
    trim(s.idx); trim(s.pos); trim(s.pref);
}

// Launch order for n tiles given in priority order: position i runs on XCD
// i % kNumXcds, so position i takes the first remaining tile that prefers
// that XCD; when none is left, the first remaining tile of any XCD.  The
// tiles are written to out[0, n).
template <class Get, class Pref>
void xcd_order(size_t n, Get get, Pref pref, Tile* out, size_t first_pos = 0)
{
    PlanScratch& S = plan_scratch();
    // tile indices bucketed by preferred XCD, each bucket in priority order
    size_t start[kNumXcds + 1] = {};
    S.pref.resize(n);
    for (size_t i = 0; i < n; ++i) {
        S.pref[i] = (int32_t)pref(i);
        ++start[S.pref[i] + 1];
    }
    for (int x = 0; x < kNumXcds; ++x) start[x + 1] += start[x];
    size_t head[kNumXcds], fill[kNumXcds];
    for (int x = 0; x < kNumXcds; ++x) head[x] = fill[x] = start[x];
    S.idx.resize(n);
    for (size_t i = 0; i < n; ++i) S.idx[fill[S.pref[i]]++] = i;
    for (size_t pos = 0; pos < n; ++pos) {
        size_t x = (first_pos + pos) % (size_t)kNumXcds;
        if (head[x] == start[x + 1]) {
            size_t best = n;
            for (size_t y = 0; y < (size_t)kNumXcds; ++y)
                if (head[y] < start[y + 1] && S.idx[head[y]] < best) {
                    best = S.idx[head[y]];
                    x = y;
                }
        }
        out[pos] = get(S.idx[head[x]++]);
    }
}

// The table image gets `n` tiles at byte offset `off` (256-aligned); returns
// where they go.
Tile* tile_slots(std::vector<unsigned char>& buf, uint64_t off, size_t n)
{
    buf.resize(off + n * sizeof(Tile));
    return reinterpret_cast<Tile*>(buf.data() + off);
}

// Stable sort of the work tiles by work, largest first (a counting sort;
// std::stable_sort when the counts are large).
void sort_longest_first(std::vector<WorkTile>& v)
{
    if (v.size() < 2) return;
    int64_t kmax = 0;
    for (const WorkTile& e : v) kmax = std::max<int64_t>(kmax, e.work);
    if (kmax > ((int64_t)1 << 20)) {
        std::stable_sort(v.begin(), v.end(), [](const WorkTile& x, const WorkTile& y) { return x.work > y.work; });
        return;
    }
    PlanScratch& S = plan_scratch();
    S.pos.assign((size_t)kmax + 2, 0);
    for (const WorkTile& e : v) ++S.pos[(size_t)(kmax - e.work) + 1];
    for (size_t k = 1; k < S.pos.size(); ++k) S.pos[k] += S.pos[k - 1];
    S.wt2.resize(v.size());
    for (const WorkTile& e : v) S.wt2[S.pos[(size_t)(kmax - e.work)]++] = e;
    v.swap(S.wt2);
}

template <class T>
uint64_t put(std::vector<unsigned char>& buf, uint64_t off, const std::vector<T>& v)
{
    const uint64_t bytes = v.size() * sizeof(T);
    if (buf.size() < off + bytes) buf.resize(off + bytes);
    if (bytes) std::memcpy(buf.data() + off, v.data(), bytes);
    return off + bytes;
}

// Uploads the host image of the tables (the thread's scratch) into device
// memory the plan owns.
void finish_tables(fia_plan* p)
{
    PlanScratch& S = plan_scratch();
    p->tables_bytes = align_up(S.tables.size(), 256);
    S.tables.resize(p->tables_bytes);
    if (p->tables_bytes) p->dev_tables = upload_tables(S.tables.data(), p->tables_bytes);
    // set-up of the allocation-free run: resolve this device's scratch
    // address now (once per device), not inside a caller's capture
    if (p->dev_tables) (void)noalloc_scratch();
    trim_scratch(S);
}

}  // namespace

extern "C" {

void fia_params_init(fia_params* p)
{
    if (!p) return;
    std::memset(p, 0, sizeof(*p));
    p->input_layout = "BSH";
    p->scale_value = 1.0;
    p->pre_tokens = kIntMax;
    p->next_tokens = kIntMax;
}

void bsa_params_init(bsa_params* p)
{
    if (!p) return;
    std::memset(p, 0, sizeof(*p));
    p->q_input_layout = "BNSD";
    p->kv_input_layout = "BNSD";
    p->scale_value = 1.0;
    p->block_shape[0] = 128;
    p->block_shape[1] = 128;
    p->inner_precise = 4;
    p->pre_tokens = kIntMax;
    p->next_tokens = kIntMax;
}

const char* fia_status_string(fia_status s)
{
    switch (s) {
    case FIA_OK: return "FIA_OK";
    case FIA_ERR_NULLPTR: return "FIA_ERR_NULLPTR: a required tensor or pointer is missing";
    case FIA_ERR_DTYPE: return "FIA_ERR_DTYPE: dtype not allowed or q/k/v dtypes differ";
    case FIA_ERR_SHAPE: return "FIA_ERR_SHAPE: shape inconsistent with layout, heads or lengths";
    case FIA_ERR_LAYOUT: return "FIA_ERR_LAYOUT: unknown or mismatched layout";
    case FIA_ERR_PARAM: return "FIA_ERR_PARAM: parameter outside its allowed range";
    case FIA_ERR_UNSUPPORTED: return "FIA_ERR_UNSUPPORTED: legal on the pages but not provided";
    case FIA_ERR_WORKSPACE: return "FIA_ERR_WORKSPACE: workspace missing or too small";
    case FIA_ERR_HIP: return "FIA_ERR_HIP: a HIP copy or launch failed";
    }
    return "unknown fia_status";
}

void fia_plan_destroy(fia_plan* plan)
{
    if (!plan) return;
    if (plan->dev_tables) free_tables(plan->dev_tables);
    delete plan;
}

fia_status fia_get_workspace_size(const fia_tensor* query, const fia_tensor* key,
                                  const fia_tensor* value, const fia_tensor* atten_mask,
                                  const fia_tensor* block_table, const fia_params* prm,
                                  const fia_tensor* attention_out,
                                  const fia_tensor* softmax_lse, uint64_t* workspace_size,
                                  fia_plan** plan_out)
{
    if (plan_out) *plan_out = nullptr;
    if (workspace_size) *workspace_size = 0;
    if (!query || !key || !value || !prm || !attention_out || !workspace_size || !plan_out)
        return FIA_ERR_NULLPTR;
    if (!valid_rank(query) || !valid_rank(key) || !valid_rank(value) || !valid_rank(attention_out))
        return FIA_ERR_SHAPE;
    if (!valid_optional({atten_mask, block_table, softmax_lse, prm->dequant_scale_key,
                         prm->dequant_scale_value, prm->dequant_offset_key, prm->dequant_offset_value,
                         prm->query_rope, prm->key_rope}))
        return FIA_ERR_SHAPE;

    std::unique_ptr<fia_plan> p(new fia_plan());

    // Empty query or empty output: nothing to compute (constraints: empty
    // input handling).
    if (numel(query) == 0 || numel(attention_out) == 0) {
        p->kind = KIND_EMPTY;
        *plan_out = p.release();
        return FIA_OK;
    }
    if (!query->data || !key->data || !value->data || !attention_out->data) return FIA_ERR_NULLPTR;

    // dtypes: q/k/v fp16 or bf16 and equal; output in the query dtype.  KV
    // pseudo-quantization: int8 key/value with a bf16 query and output, both
    // dequant scales given (kv pseudo-quant constraints).
    const bool kv_i8 = key->dtype == FIA_I8;
    const bool any_quant = prm->dequant_scale_key || prm->dequant_scale_value ||
                           prm->dequant_offset_key || prm->dequant_offset_value;
    if (!is_half(query->dtype)) return FIA_ERR_DTYPE;
    if (attention_out->dtype != query->dtype) return FIA_ERR_DTYPE;
    if (kv_i8) {
        if (value->dtype != FIA_I8 || query->dtype != FIA_BF16) return FIA_ERR_DTYPE;
        if (!prm->dequant_scale_key || !prm->dequant_scale_value) return FIA_ERR_NULLPTR;
    } else {
        if (key->dtype != query->dtype || value->dtype != query->dtype) return FIA_ERR_DTYPE;
        if (any_quant) return FIA_ERR_PARAM;
    }

    // MLA: query_rope and key_rope both given or both absent (v2 page,
    // query_rope / key_rope constraints), in the query's dtype
    const bool mla = prm->query_rope || prm->key_rope;
    if (mla) {
        if (!prm->query_rope || !prm->key_rope) return FIA_ERR_PARAM;
        if (!prm->query_rope->data || !prm->key_rope->data) return FIA_ERR_NULLPTR;
        if (kv_i8) return FIA_ERR_UNSUPPORTED;
        if (prm->query_rope->dtype != query->dtype || prm->key_rope->dtype != query->dtype)
            return FIA_ERR_DTYPE;
        if (!valid_rank(prm->query_rope) || !valid_rank(prm->key_rope)) return FIA_ERR_SHAPE;
    }

    int32_t layout;
    bool bsh;
    fia_status st = parse_layout(prm->input_layout, &layout, &bsh);
    if (st != FIA_OK) return st;

    const int64_t QN = prm->num_heads;
    if (QN <= 0 || QN > 256) return FIA_ERR_PARAM;
    const int64_t KVN = prm->num_key_value_heads == 0 ? QN : prm->num_key_value_heads;
    // GQA ratio <= 64; MLA allows 128 query heads on its single kv head
    if (KVN <= 0 || QN % KVN != 0 || QN / KVN > (mla ? 128 : 64)) return FIA_ERR_PARAM;
    if (prm->sparse_mode < 0 || prm->sparse_mode > 4) return FIA_ERR_PARAM;
    if (prm->inner_precise < 0 || prm->inner_precise > 3) return FIA_ERR_PARAM;
    if (!(std::isfinite(prm->scale_value))) return FIA_ERR_PARAM;

    Geo gq;
    if ((st = geometry(query, layout, bsh, QN, &gq)) != FIA_OK) return st;
    if (gq.N != QN) return FIA_ERR_SHAPE;
    const bool decode = layout != LAYOUT_TND && gq.S == 1;
    const bool paged = block_table != nullptr;

    p->dtype = query->dtype;
    p->layout = layout;
    p->QN = QN;
    p->KVN = KVN;
    p->G = QN / KVN;
    p->Dqk = gq.D;
    p->Sq = gq.S;

    // ----- key / value -----
    Geo gk, gv;
    int64_t B = 0, Skv = 0, Dv = 0;
    int64_t pool_blocks = 0;
    int32_t pool_layout = 0;
    if (paged) {
        // PageAttention (constraints, page attention scenario).  Query S == 1:
        // block_size a multiple of 16; query S > 1: a multiple of 128 in
        // [128, 512]; a TND query (TND constraints): 128, 512 or 1024, the
        // batch being the count of actual_seq_qlen (checked against the
        // table below).
        if (!block_table->data) return FIA_ERR_NULLPTR;
        if (block_table->dtype != FIA_I32) return FIA_ERR_DTYPE;
        if (block_table->ndim != 2) return FIA_ERR_SHAPE;
        if (layout != LAYOUT_TND && block_table->dims[0] != gq.B) return FIA_ERR_SHAPE;
        if (prm->block_size <= 0 || prm->block_size % 16 != 0) return FIA_ERR_PARAM;
        if (mla) {
            // MLA with a query D of 512: block_size 16 or 128 (64 or 128 with
            // sparse_mode 4)
            if (prm->block_size != 16 && prm->block_size != 64 && prm->block_size != 128)
                return FIA_ERR_PARAM;
        } else if (layout == LAYOUT_TND) {
            if (prm->block_size != 128 && prm->block_size != 512 && prm->block_size != 1024)
                return FIA_ERR_PARAM;
        } else if (!decode && (prm->block_size % 128 != 0 || prm->block_size > 512)) {
            return FIA_ERR_PARAM;
        }
        if (!prm->actual_seq_kvlen) return FIA_ERR_PARAM;
        if (key->ndim != value->ndim) return FIA_ERR_SHAPE;
        for (int i = 0; i < key->ndim; ++i)
            if (key->dims[i] != value->dims[i]) return FIA_ERR_SHAPE;
        const int64_t bs = prm->block_size;
        if (key->ndim == 4) {          // (blocknum, KV_N, block_size, D)
            if (key->dims[1] != KVN || key->dims[2] != bs) return FIA_ERR_SHAPE;
            gk.D = key->dims[3];
            pool_layout = 0;
        } else if (key->ndim == 3) {   // (blocknum, block_size, KV_N*D)
            if (key->dims[1] != bs || key->dims[2] % KVN) return FIA_ERR_SHAPE;
            gk.D = key->dims[2] / KVN;
            pool_layout = 1;
        } else {
            return FIA_ERR_SHAPE;
        }
        pool_blocks = key->dims[0];
        B = gq.B;
        Skv = block_table->dims[1] * bs;
        Dv = gk.D;
    } else {
        if ((st = geometry(key, layout, bsh, KVN, &gk)) != FIA_OK) return st;
        if ((st = geometry(value, layout, bsh, KVN, &gv)) != FIA_OK) return st;
        if (gk.N != KVN || gv.N != KVN) return FIA_ERR_SHAPE;
        if (layout != LAYOUT_TND && (gk.B != gq.B || gv.B != gq.B)) return FIA_ERR_SHAPE;
        if (gk.S != gv.S) return FIA_ERR_SHAPE;
        B = gq.B;
        Skv = gk.S;
        Dv = gv.D;
    }
    if (gk.D != gq.D) return FIA_ERR_SHAPE;
    p->Dv = Dv;
    p->Skv = Skv;

    // ----- lengths -----
    std::vector<int64_t> lq, lkv, qstart, kvstart;
    if (layout == LAYOUT_TND) {
        if (!prm->actual_seq_qlen || !prm->actual_seq_kvlen) return FIA_ERR_PARAM;
        if (prm->n_actual_seq_qlen != prm->n_actual_seq_kvlen) return FIA_ERR_PARAM;
        if ((st = resolve_cumulative(prm->actual_seq_qlen, prm->n_actual_seq_qlen, gq.S, &lq,
                                     &qstart)) != FIA_OK)
            return st;
        if (paged && mla) {
            // MLA TND with page attention: actual_seq_kvlen holds each batch's
            // own length (D 512 TND constraints), not cumulative sums
            if ((st = resolve_lengths(prm->actual_seq_kvlen, prm->n_actual_seq_kvlen,
                                      prm->n_actual_seq_qlen, Skv, &lkv)) != FIA_OK)
                return st;
            if (block_table->dims[0] != prm->n_actual_seq_qlen) return FIA_ERR_SHAPE;
        } else if (paged) {
            // other head dims: cumulative as for every TND call; each batch's
            // pages must fit the table's row (checked with the pool below)
            if ((st = resolve_cumulative(prm->actual_seq_kvlen, prm->n_actual_seq_kvlen,
                                         ((int64_t)1 << 40), &lkv, &kvstart)) != FIA_OK)
                return st;
            if (block_table->dims[0] != prm->n_actual_seq_qlen) return FIA_ERR_SHAPE;
        } else if ((st = resolve_cumulative(prm->actual_seq_kvlen, prm->n_actual_seq_kvlen, Skv, &lkv,
                                            &kvstart)) != FIA_OK) {
            return st;
        }
        B = prm->n_actual_seq_qlen;
    } else {
        if (decode)
            lq.assign((size_t)B, 1);   // actual_seq_qlen has no effect at S == 1
        else if ((st = resolve_lengths(prm->actual_seq_qlen, prm->n_actual_seq_qlen, B, gq.S,
                                       &lq)) != FIA_OK)
            return st;
        if ((st = resolve_lengths(prm->actual_seq_kvlen, prm->n_actual_seq_kvlen, B, Skv,
                                  &lkv)) != FIA_OK)
            return st;
    }
    p->B = B;
    // sequence axes up to 2^29 rows (the pages' limit is 20M); kernels index
    // rows in int32
    if (gq.S >= ((int64_t)1 << 29) || Skv >= ((int64_t)1 << 29)) return FIA_ERR_UNSUPPORTED;

    int64_t max_blocks = 0;
    if (paged) {
        const int64_t bs = prm->block_size;
        int64_t need = 0;
        for (int64_t b = 0; b < B; ++b) {
            const int64_t nb = (lkv[(size_t)b] + bs - 1) / bs;
            max_blocks = std::max(max_blocks, nb);
            need += nb;
        }
        if (block_table->dims[1] < max_blocks) return FIA_ERR_SHAPE;
        if (pool_blocks < need) return FIA_ERR_SHAPE;
    }

    // ----- output / lse shapes -----
    {
        Geo go;
        if ((st = geometry(attention_out, layout, bsh, QN, &go)) != FIA_OK) return st;
        if (go.N != QN || go.S != gq.S || go.D != Dv) return FIA_ERR_SHAPE;
        if (layout != LAYOUT_TND && go.B != gq.B) return FIA_ERR_SHAPE;
    }
    const bool want_lse = prm->return_softmax_lse != 0;
    if (want_lse) {
        if (!softmax_lse || !softmax_lse->data) return FIA_ERR_NULLPTR;
        if (softmax_lse->dtype != FIA_F32) return FIA_ERR_DTYPE;
        bool ok = layout == LAYOUT_TND ? dims_are(softmax_lse, {gq.S, QN, 1})
                                       : dims_are(softmax_lse, {gq.B, QN, gq.S, 1});
        if (!ok) return FIA_ERR_SHAPE;
    }

    // ----- mask -----
    const int32_t mode = (int32_t)prm->sparse_mode;
    // pre/next as band bounds: with sequence axes below 2^29, a bound past
    // +-2^30 is the same as an infinite one, so both are clamped there once
    // (no arithmetic below sees the int64 extremes)
    const int64_t pre_c = std::max<int64_t>(-((int64_t)1 << 30), std::min<int64_t>((int64_t)1 << 30, prm->pre_tokens));
    const int64_t next_c = std::max<int64_t>(-((int64_t)1 << 30), std::min<int64_t>((int64_t)1 << 30, prm->next_tokens));
    const uint8_t* mask = nullptr;
    int64_t mask_bstride = 0, mask_rstride = 0;
    if (!decode) {
        if (layout == LAYOUT_TND && (mode == 1 || (mode == 0 && atten_mask)))
            return FIA_ERR_PARAM;      // TND: mode 0 without mask, or modes 2/3/4
        if (mode == 1 && !atten_mask) return FIA_ERR_NULLPTR;
        if (atten_mask) {
            if (!mask_dtype_ok(atten_mask->dtype)) return FIA_ERR_DTYPE;
            if (mode >= 2) {
                if (!is_template_2048(atten_mask)) return FIA_ERR_SHAPE;
            } else {
                if (!atten_mask->data) return FIA_ERR_NULLPTR;
                const fia_tensor* m = atten_mask;
                const int64_t rows = m->dims[m->ndim - 2 < 0 ? 0 : m->ndim - 2];
                const int64_t cols = m->dims[m->ndim - 1];
                int64_t mb = 1;
                if (m->ndim == 2) {
                    mb = 1;
                } else if (m->ndim == 3) {
                    mb = m->dims[0];
                } else if (m->ndim == 4) {
                    if (m->dims[1] != 1) return FIA_ERR_SHAPE;
                    mb = m->dims[0];
                } else {
                    return FIA_ERR_SHAPE;
                }
                // paged: the mask's KV_S covers maxBlockNumPerSeq * block_size
                const int64_t need_cols = paged ? max_blocks * prm->block_size : Skv;
                if (m->ndim < 2 || rows < gq.S || cols < need_cols) return FIA_ERR_SHAPE;
                if (mb != 1 && mb != B) return FIA_ERR_SHAPE;
                mask = (const uint8_t*)m->data;
                mask_rstride = cols;
                mask_bstride = mb == 1 ? 0 : rows * cols;
            }
        }
    } else {
        if (prm->inner_precise > 1) return FIA_ERR_PARAM;   // Q_S == 1: inner_precise 0 or 1 only
        // Q_S == 1: an atten_mask masks kv tokens per batch, shapes (B, KV_S),
        // (B, 1, KV_S) or (B, 1, 1, KV_S) (atten_mask parameter description;
        // a leading 1 broadcasts); with a paged cache KV_S covers
        // maxBlockNumPerSeq * block_size
        if (atten_mask && mla && mode == 4) {
            // MLA sparse_mode 4 at query S 1: the band's 2048 template, not
            // a per-token mask (its contents are not read)
            if (!mask_dtype_ok(atten_mask->dtype)) return FIA_ERR_DTYPE;
            if (!is_template_2048(atten_mask)) return FIA_ERR_SHAPE;
        } else if (atten_mask) {
            const fia_tensor* m = atten_mask;
            if (!mask_dtype_ok(m->dtype)) return FIA_ERR_DTYPE;
            if (!m->data) return FIA_ERR_NULLPTR;
            if (m->ndim < 2 || m->ndim > 4) return FIA_ERR_SHAPE;
            for (int i = 1; i + 1 < m->ndim; ++i)
                if (m->dims[i] != 1) return FIA_ERR_SHAPE;
            const int64_t mb = m->dims[0], cols = m->dims[m->ndim - 1];
            const int64_t need_cols = paged ? max_blocks * prm->block_size : Skv;
            if ((mb != 1 && mb != B) || cols < need_cols) return FIA_ERR_SHAPE;
            mask = (const uint8_t*)m->data;
            mask_bstride = mb == 1 ? 0 : cols;
        }
    }

    // ----- MLA (query D 512, rope D 64, one kv head, paged) -----
    const void* qr_data = nullptr;
    int64_t qr_sB = 0, qr_sH = 0, qr_sS = 0;
    int64_t mla_S = gq.S;               // query tokens per batch (TND: the largest)
    if (mla) {
        if (!paged) return FIA_ERR_UNSUPPORTED;
        if (gq.D != 512 || Dv != 512) return FIA_ERR_UNSUPPORTED;
        if (KVN != 1 || QN > 128 || (QN & (QN - 1)) != 0) return FIA_ERR_UNSUPPORTED;
        if (layout == LAYOUT_TND) {
            mla_S = 1;
            for (int64_t x : lq) mla_S = std::max(mla_S, x);
            // TND: sparse_mode 0 without a mask or 3 (checked with the mask above)
            if (mode != 0 && mode != 3) return FIA_ERR_UNSUPPORTED;
        } else if (mask || (gq.S == 1 && mode != 4 && atten_mask) ||
                   (gq.S == 1 && mode != 0 && mode != 4) || (gq.S > 1 && mode != 3 && mode != 4)) {
            // S == 1: sparse_mode 0 without a mask, or 4; S > 1: sparse_mode 3 or 4
            return FIA_ERR_UNSUPPORTED;
        }
        if (mla_S > kDecodeHeads) return FIA_ERR_UNSUPPORTED;
        Geo gr;
        if ((st = geometry(prm->query_rope, layout, bsh, QN, &gr)) != FIA_OK) return st;
        if (gr.N != QN || gr.B != gq.B || gr.S != gq.S || gr.D != 64) return FIA_ERR_SHAPE;
        const fia_tensor* kr = prm->key_rope;
        const int64_t bs = prm->block_size;
        const bool ok = (kr->ndim == 4 && kr->dims[1] == 1 && kr->dims[2] == bs && kr->dims[3] == 64) ||
                        (kr->ndim == 3 && kr->dims[1] == bs && kr->dims[2] == 64);
        if (!ok || kr->dims[0] != pool_blocks) return FIA_ERR_SHAPE;
        qr_data = prm->query_rope->data;
        if (layout == LAYOUT_BNSD) {
            qr_sB = QN * gq.S * 64; qr_sH = gq.S * 64; qr_sS = 64;
        } else if (layout == LAYOUT_TND) {
            qr_sB = 0; qr_sH = 64; qr_sS = QN * 64;     // row = first row of the batch + token
        } else {
            qr_sB = gq.S * QN * 64; qr_sH = 64; qr_sS = QN * 64;
        }
    }

    // ----- supported head dims -----
    if (mla) {
        // checked above
    } else if (decode) {
        if (!((gq.D == 64 || gq.D == 128) && Dv == gq.D)) return FIA_ERR_UNSUPPORTED;
    } else {
        const bool ok = (gq.D == 64 && Dv == 64) || (gq.D == 128 && Dv == 128) ||
                        (gq.D == 192 && Dv == 128);
        if (!ok) return FIA_ERR_UNSUPPORTED;
    }

    const double scale_log2 = prm->scale_value * kLog2e;

    // Kernel choice.  Query S == 1, and multi-token decode (S <= 16 with all
    // G x S (head, token) rows of a kv head in one 16-column chunk, sparse_mode
    // 3 or 0 without a mask), run on the split-KV decode kernel: each K/V
    // byte is read once for all those rows and the kv range is spread over
    // the whole GPU.  Everything else runs on the prefill kernel.
    const bool dec_kernel =
        mla || decode || (layout != LAYOUT_TND && gq.S <= kDecodeHeads && p->G * gq.S <= kDecodeHeads &&
                   mask == nullptr && (mode == 3 || mode == 0) && Dv == gq.D &&
                   (gq.D == 64 || gq.D == 128));

    // ----- KV pseudo-quantization parameters -----
    const void *k_scale = nullptr, *k_off = nullptr, *v_scale = nullptr, *v_off = nullptr;
    int64_t tok_stride = 0;
    if (kv_i8) {
        if (layout == LAYOUT_TND || gq.S > kDecodeHeads) return FIA_ERR_PARAM;   // query S <= 16
        // key_quant_mode / value_quant_mode (v2 parameter description and the
        // kv pseudo-quant constraints): 0..5 at query S 1, where the two modes
        // are equal except key 0 with value 1; only 0 and 1, and equal, at
        // query S > 1, where page attention is not allowed either.  Block size
        // with an int8 cache: a multiple of 32 (page attention scenario).
        const int64_t km = prm->key_quant_mode, vm = prm->value_quant_mode;
        if (km < 0 || km > 5 || vm < 0 || vm > 5) return FIA_ERR_PARAM;
        if (decode) {
            if (km != vm && !(km == 0 && vm == 1)) return FIA_ERR_PARAM;
            if (paged && prm->block_size % 32 != 0) return FIA_ERR_PARAM;
        } else {
            if (km > 1 || km != vm || paged) return FIA_ERR_PARAM;
        }
        // per-tensor / per-head modes and scales managed by page attention
        if (km > 1) return FIA_ERR_UNSUPPORTED;
        if (!dec_kernel || mask) return FIA_ERR_UNSUPPORTED;
        // per channel: bf16 [KV_N, D] or [KV_N * D]; per token: fp32 [B, KV_S'],
        // KV_S' >= the key's S (paged: the longest kv length), indexed by the
        // logical kv position
        int64_t tok_need = Skv;
        if (paged) {
            tok_need = 0;
            for (int64_t x : lkv) tok_need = std::max(tok_need, x);
        }
        auto check = [&](const fia_tensor* t, int64_t md, int64_t* stride) -> fia_status {
            if (!t->data) return FIA_ERR_NULLPTR;
            if (md == 0) {
                if (t->dtype != FIA_BF16) return FIA_ERR_DTYPE;
                if (!dims_are(t, {KVN, gq.D}) && !dims_are(t, {KVN * gq.D})) return FIA_ERR_SHAPE;
            } else {
                if (t->dtype != FIA_F32) return FIA_ERR_DTYPE;
                if (t->ndim != 2 || t->dims[0] != B || t->dims[1] < tok_need) return FIA_ERR_SHAPE;
                *stride = t->dims[1];
            }
            return FIA_OK;
        };
        auto same = [](const fia_tensor* x, const fia_tensor* y) {
            if (x->dtype != y->dtype || x->ndim != y->ndim) return false;
            for (int i = 0; i < x->ndim; ++i)
                if (x->dims[i] != y->dims[i]) return false;
            return true;
        };
        int64_t ks = 0, vs = 0;
        if ((st = check(prm->dequant_scale_key, km, &ks)) != FIA_OK) return st;
        if ((st = check(prm->dequant_scale_value, vm, &vs)) != FIA_OK) return st;
        if (km == 1 && vm == 1 && ks != vs) return FIA_ERR_SHAPE;
        // equal modes: the two scales (and the two offsets) take one shape
        if (km == vm && !same(prm->dequant_scale_key, prm->dequant_scale_value)) return FIA_ERR_SHAPE;
        if (km == vm && prm->dequant_offset_key && prm->dequant_offset_value &&
            !same(prm->dequant_offset_key, prm->dequant_offset_value))
            return FIA_ERR_SHAPE;
        if (prm->dequant_offset_key) {
            if (!prm->dequant_offset_key->data) return FIA_ERR_NULLPTR;
            if (!same(prm->dequant_offset_key, prm->dequant_scale_key)) return FIA_ERR_SHAPE;
        }
        if (prm->dequant_offset_value) {
            if (!prm->dequant_offset_value->data) return FIA_ERR_NULLPTR;
            if (!same(prm->dequant_offset_value, prm->dequant_scale_value)) return FIA_ERR_SHAPE;
        }
        k_scale = prm->dequant_scale_key->data;
        v_scale = prm->dequant_scale_value->data;
        k_off = prm->dequant_offset_key ? prm->dequant_offset_key->data : nullptr;
        v_off = prm->dequant_offset_value ? prm->dequant_offset_value->data : nullptr;
        tok_stride = km == 1 ? ks : vs;
    }

    if (dec_kernel) {
        p->kind = KIND_DECODE;
        DecodeArgs& d = p->dec;
        d.q = query->data;
        d.k = key->data;
        d.v = value->data;
        d.o = attention_out->data;
        d.lse = want_lse ? (float*)softmax_lse->data : nullptr;
        d.return_lse = want_lse;
        d.paged = paged;
        const int64_t D = gq.D;
        const int64_t S = mla_S;
        d.S = (int32_t)S;
        d.tnd = layout == LAYOUT_TND;
        d.causal = !decode && mode == 3;
        d.mask = decode ? mask : nullptr;     // S > 1 reaches here only without one
        d.mask_bstride = mask_bstride;
        d.kv_i8 = kv_i8;
        d.kmode = (int32_t)prm->key_quant_mode;
        d.vmode = (int32_t)prm->value_quant_mode;
        d.k_scale = k_scale;
        d.k_off = k_off;
        d.v_scale = v_scale;
        d.v_off = v_off;
        d.tok_stride = tok_stride;
        if (layout == LAYOUT_BNSD) {
            d.q_sB = QN * S * D; d.q_sH = S * D; d.q_sS = D;
        } else if (layout == LAYOUT_TND) {
            d.q_sB = 0; d.q_sH = D; d.q_sS = QN * D;        // row = first row of the batch + token
        } else {
            d.q_sB = S * QN * D; d.q_sH = D; d.q_sS = QN * D;
        }
        d.o_sB = d.q_sB; d.o_sH = d.q_sH; d.o_sS = d.q_sS;   // D_v == D
        if (paged) {
            const int64_t bs = prm->block_size;
            d.block_table = (const int32_t*)block_table->data;
            d.bt_stride = block_table->dims[1];
            d.block_size = (int32_t)bs;
            d.p_blk = bs * KVN * D;
            d.p_head = pool_layout == 0 ? bs * D : D;
            d.p_tok = pool_layout == 0 ? D : KVN * D;
        } else {
            d.c_rowmul = KVN * D;
            d.c_head = layout == LAYOUT_BNSD ? Skv * D : D;
            d.c_tok = layout == LAYOUT_BNSD ? D : KVN * D;
        }
        const int64_t G = QN / KVN;
        const int64_t R = G * S;       // (head, token) rows of one kv head
        // rows per chunk: 16 (one wave), or for MLA up to 16 x 8 (one
        // workgroup of nw waves)
        int64_t nw = 0;
        if (mla) {
            const int64_t need = (std::min<int64_t>(R, 16 * kMlaMaxWaves) + 15) / 16;
            nw = 2;                    // the MLA kernel runs 2, 4 or 8 waves
            while (nw < need) nw *= 2;
        }
        const int64_t rows_per_chunk = mla ? 16 * nw : kDecodeHeads;
        const int64_t Gc = std::min<int64_t>(R, rows_per_chunk);
        const int64_t nhc = (R + rows_per_chunk - 1) / rows_per_chunk;
        // Balanced schedule: one wave per resident slot, each with an equal
        // quota of the concatenated token stream (a multiple of 16 tokens, so
        // a 16-token sub-tile never crosses a page).
        const int64_t nseg = B * KVN * nhc;
        // first kv token a batch's rows can see (MLA sparse_mode 4: keys below
        // Lkv - Lq - pre are outside every row's band), 16-aligned
        auto first_token = [&](int64_t b) -> int64_t {
            if (!(mla && mode == 4)) return 0;
            const int64_t lo = lkv[(size_t)b] - lq[(size_t)b] - pre_c;
            return std::min(lkv[(size_t)b], std::max<int64_t>(0, lo)) / 16 * 16;
        };
        int64_t total = 0;
        for (int64_t b = 0; b < B; ++b) total += (lkv[(size_t)b] - first_token(b)) * KVN * nhc;
        const int64_t steps = (total + kDecodeStep - 1) / kDecodeStep;
        // one MLA workgroup per CU (its two stages fill most of the LDS)
        const int64_t W = std::min<int64_t>((int64_t)kNumCUs * (mla ? 1 : kDecodeWavesPerCU), steps);
        int64_t quota = W > 0 ? (total + W - 1) / W : 0;
        quota = (quota + kDecodeStep - 1) / kDecodeStep * kDecodeStep;
        // a piece touches at most 64 pages (one block-table entry per lane)
        const int64_t piece_cap = paged ? std::max<int64_t>(16, 63 * prm->block_size / 16 * 16)
                                        : ((int64_t)1 << 40);
        std::vector<DecSeg> segs((size_t)nseg);
        std::vector<DecPiece> pieces;
        std::vector<int32_t> wave_first;
        wave_first.push_back(0);
        int64_t remaining = quota;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t g = 0; g < KVN * nhc; ++g) {
                const int64_t si = b * KVN * nhc + g;
                const int64_t L = lkv[(size_t)b];
                DecSeg& sg = segs[(size_t)si];
                sg.kv_row0 = paged ? 0 : b * Skv;
                sg.b = (int32_t)b;
                sg.lkv = (int32_t)L;
                sg.lq = (int32_t)lq[(size_t)b];
                sg.q_row0 = layout == LAYOUT_TND ? (int32_t)qstart[(size_t)b] : 0;
                sg.first = (int32_t)pieces.size();
                for (int64_t t = first_token(b); t < L;) {
                    if (remaining < 16) {                  // next wave
                        wave_first.push_back((int32_t)pieces.size());
                        remaining = quota;
                    }
                    const int64_t take = std::min(std::min(L - t, remaining / 16 * 16), piece_cap);
                    pieces.push_back(DecPiece{(int32_t)si, (int32_t)t, (int32_t)(t + take), 0});
                    t += take;
                    remaining -= take;
                    remaining = remaining / 16 * 16;       // keep pieces 16-aligned
                }
                sg.count = (int32_t)pieces.size() - sg.first;
            }
        if (!pieces.empty()) wave_first.push_back((int32_t)pieces.size());
        if (pieces.size() > (size_t)INT32_MAX / 2) return FIA_ERR_UNSUPPORTED;
        d.B = (int32_t)B;
        d.QN = (int32_t)QN;
        d.KVN = (int32_t)KVN;
        d.G = (int32_t)G;
        d.Gc = (int32_t)Gc;
        d.nhc = (int32_t)nhc;
        d.n_waves = (int32_t)(wave_first.size() - 1);
        d.n_pieces = (int32_t)pieces.size();
        d.scale_log2 = (float)scale_log2;
        d.mla_nw = (int32_t)nw;
        // MLA band (bottom-right, relative to Lkv - Lq + t): mode 3 (-2^30, 0],
        // mode 4 [-pre, next] (clamped to +-2^30), otherwise open
        const int64_t band_lim = (int64_t)1 << 30;
        int64_t blo = -band_lim, bhi = band_lim;
        if (mla && mode == 3) bhi = 0;
        if (mla && mode == 4) {
            blo = -pre_c;
            bhi = next_c;
        }
        d.band_lo = (int32_t)blo;
        d.band_hi = (int32_t)bhi;
        if (mla) {
            d.qr = qr_data;
            d.kr = prm->key_rope->data;
            d.qr_sB = qr_sB; d.qr_sH = qr_sH; d.qr_sS = qr_sS;
            d.pr_blk = prm->block_size * 64;
            // value passed as the key tensor itself (same pointer; the shapes
            // are equal): V is read from the K tiles
            d.v_is_k = value->data == key->data;
        }
        p->n_waves = d.n_waves;
        p->n_pieces = d.n_pieces;
        p->off_batch = 0;
        std::vector<unsigned char>& tb = plan_scratch().tables;
        tb.clear();
        uint64_t end = put(tb, 0, segs);
        p->off_pieces = align_up(end, 256);
        end = put(tb, p->off_pieces, pieces);
        p->off_waves = align_up(end, 256);
        put(tb, p->off_waves, wave_first);
        finish_tables(p.get());
        const uint64_t np = std::max<uint64_t>(1, pieces.size());
        p->off_part_o = 0;
        p->off_part_lse = align_up(p->off_part_o + np * Gc * Dv * 4, 256);
        p->workspace_bytes = align_up(p->off_part_lse + np * Gc * 4, 256);
        *workspace_size = p->workspace_bytes;
        *plan_out = p.release();
        return FIA_OK;
    }

    // ----- prefill -----
    p->kind = KIND_PREFILL;
    AttnArgs& a = p->attn;
    a.q = query->data;
    a.k = key->data;
    a.v = value->data;
    a.o = attention_out->data;
    a.lse = want_lse ? (float*)softmax_lse->data : nullptr;
    a.return_lse = want_lse;
    a.mask = mask;
    a.mask_bstride = mask_bstride;
    a.mask_rstride = mask_rstride;
    a.has_mask = mask != nullptr;
    a.mode = mode;
    // Modes 1, 2 and 3 ignore pre/next; mode 0 without a mask ignores them
    // (sparse_mode parameter description).  With S < 2^29 a band bound past
    // +-2^30 is the same as an infinite one, so the kernel works in int32.
    a.pre = (mode == 4 || (mode == 0 && mask)) ? pre_c : (int64_t)1 << 30;
    a.next = (mode == 4 || (mode == 0 && mask)) ? next_c : (int64_t)1 << 30;
    a.QN = (int32_t)QN;
    a.KVN = (int32_t)KVN;
    a.G = (int32_t)(QN / KVN);
    a.scale_log2 = (float)scale_log2;
    const int64_t Dq = gq.D;
    if (layout == LAYOUT_BNSD) {
        a.q_sH = gq.S * Dq;  a.q_sS = Dq;
        a.k_sH = Skv * Dq;   a.k_sS = Dq;
        a.v_sH = Skv * Dv;   a.v_sS = Dv;
        a.o_sH = gq.S * Dv;  a.o_sS = Dv;
        a.lse_sH = gq.S;     a.lse_sS = 1;
    } else {
        a.q_sH = Dq;  a.q_sS = QN * Dq;
        a.k_sH = Dq;  a.k_sS = KVN * Dq;
        a.v_sH = Dv;  a.v_sS = KVN * Dv;
        a.o_sH = Dv;  a.o_sS = QN * Dv;
        if (layout == LAYOUT_TND) { a.lse_sH = 1; a.lse_sS = QN; }
        else { a.lse_sH = gq.S; a.lse_sS = 1; }
    }
    a.q_rowmul = QN * Dq;
    a.k_rowmul = KVN * Dq;
    a.v_rowmul = KVN * Dv;
    a.paged = paged;
    if (paged) {
        // pool (blocknum, KV_N, block_size, D) or (blocknum, block_size, KV_N * D)
        const int64_t bs = prm->block_size;
        a.block_table = (const int32_t*)block_table->data;
        a.bt_stride = block_table->dims[1];
        a.block_size = (int32_t)bs;
        a.p_blk = bs * KVN * Dq;
        a.k_sH = a.v_sH = pool_layout == 0 ? bs * Dq : Dq;
        a.k_sS = a.v_sS = pool_layout == 0 ? Dq : KVN * Dq;
        a.k_rowmul = a.v_rowmul = 0;
    }
    a.o_rowmul = QN * Dv;
    a.lse_rowmul = QN;

    std::vector<BatchInfo> bi((size_t)B);
    for (int64_t b = 0; b < B; ++b) {
        bi[(size_t)b].q_row0 = layout == LAYOUT_TND ? qstart[(size_t)b] : b * gq.S;
        bi[(size_t)b].kv_row0 = paged ? 0 : layout == LAYOUT_TND ? kvstart[(size_t)b] : b * Skv;
        bi[(size_t)b].lq = (int32_t)lq[(size_t)b];
        bi[(size_t)b].lkv = (int32_t)lkv[(size_t)b];
    }
    // A workgroup covers hg heads of one GQA group (hg the largest power of
    // two dividing G, at most kDenseWaves) and 32 kDenseWaves / hg query
    // rows: the heads share every K/V tile.  Longest-first order, with the
    // tiles of one kv head kept on one XCD so that they share its L2.
    // Padded layouts: the rows past the last row block that holds a valid
    // query row are written (out = 0, lse = +inf) by zero-fill workgroups of
    // about 256 KB of output each over all heads (h = -1 marks them); they
    // go first, where their stores overlap the MFMA-bound workgroups.
    const int64_t G = QN / KVN;
    int64_t hg = 1;
    while (hg < kDenseWaves && G % (2 * hg) == 0) hg *= 2;
    a.hg = (int32_t)hg;
    const int64_t rows_per = 32 * kDenseWaves / hg;
    PlanScratch& S = plan_scratch();
    std::vector<WorkTile>& tl = S.wt;
    tl.clear();
    std::vector<Tile>& tiles = S.tiles;    // the zero-fill workgroups (launched first)
    tiles.clear();
    const int64_t zrows = std::max<int64_t>(1, ((int64_t)256 << 10) / (QN * Dv * 2));
    {
        size_t n = 0;
        for (int64_t b = 0; b < B; ++b)
            n += (size_t)((std::min<int64_t>(lq[(size_t)b], layout == LAYOUT_TND ? lq[(size_t)b] : gq.S) +
                           rows_per - 1) / rows_per);
        tl.reserve(n * (size_t)(QN / hg));
    }
    for (int64_t b = 0; b < B; ++b) {
        const int64_t rows = layout == LAYOUT_TND ? lq[(size_t)b] : gq.S;
        const int64_t zfrom = std::min(rows, (lq[(size_t)b] + rows_per - 1) / rows_per * rows_per);
        for (int64_t z0 = zfrom; z0 < rows; z0 += zrows)
            tiles.push_back(Tile{(int32_t)b, -1, (int32_t)z0, (int32_t)std::min(z0 + zrows, rows),
                                 bi[(size_t)b]});
        for (int64_t q0 = 0; q0 < zfrom; q0 += rows_per) {
            const int64_t q1 = std::min<int64_t>(q0 + rows_per, rows);
            const int64_t w = kv_tiles_of(mode, mask != nullptr, a.pre, a.next, lq[(size_t)b],
                                          lkv[(size_t)b], q0, q1);
            for (int64_t h = 0; h < QN; h += hg)
                tl.push_back({w, Tile{(int32_t)b, (int32_t)h, (int32_t)q0, (int32_t)q1, bi[(size_t)b]}});
        }
    }
    sort_longest_first(tl);
    const size_t n_zero = tiles.size(), n_all = n_zero + tl.size();
    if (n_all > (size_t)INT32_MAX) return FIA_ERR_UNSUPPORTED;
    p->n_tiles = (int64_t)n_all;
    a.n_tiles = (int32_t)n_all;
    p->off_batch = 0;
    S.tables.clear();
    uint64_t end = put(S.tables, 0, bi);
    p->off_tiles = align_up(end, 256);
    Tile* slots = tile_slots(S.tables, p->off_tiles, n_all);
    std::copy(tiles.begin(), tiles.end(), slots);
    xcd_order(tl.size(), [&](size_t i) { return tl[i].t; },
              [&](size_t i) { return (int)((tl[i].t.h / (QN / KVN)) % kNumXcds); }, slots + n_zero, n_zero);
    finish_tables(p.get());
    p->workspace_bytes = 0;                  // prefill needs no scratch
    *workspace_size = p->workspace_bytes;
    *plan_out = p.release();
    return FIA_OK;
}

fia_status bsa_get_workspace_size(const fia_tensor* query, const fia_tensor* key,
                                  const fia_tensor* value, const fia_tensor* block_sparse_mask,
                                  const fia_tensor* atten_mask, const fia_tensor* block_table,
                                  const bsa_params* prm, const fia_tensor* attention_out,
                                  const fia_tensor* softmax_lse, uint64_t* workspace_size,
                                  fia_plan** plan_out)
{
    if (plan_out) *plan_out = nullptr;
    if (workspace_size) *workspace_size = 0;
    if (!query || !key || !value || !prm || !attention_out || !workspace_size || !plan_out)
        return FIA_ERR_NULLPTR;
    if (!block_sparse_mask) return FIA_ERR_NULLPTR;
    if (!valid_rank(query) || !valid_rank(key) || !valid_rank(value) ||
        !valid_rank(attention_out) || !valid_rank(block_sparse_mask))
        return FIA_ERR_SHAPE;
    if (!valid_optional({softmax_lse, prm->dequant_scale_query, prm->dequant_scale_key,
                         prm->dequant_scale_value}))
        return FIA_ERR_SHAPE;
    // Constraints of the block-sparse page: no atten_mask, no paged cache,
    // fixed mask_type / inner_precise / pre / next.
    if (atten_mask || block_table) return FIA_ERR_PARAM;
    if (prm->mask_type != 0 || prm->block_size != 0 || prm->inner_precise != 4) return FIA_ERR_PARAM;
    if (prm->pre_tokens != kIntMax || prm->next_tokens != kIntMax) return FIA_ERR_PARAM;
    if (prm->softmax_lse_flag != 0 && prm->softmax_lse_flag != 1) return FIA_ERR_PARAM;
    if (!std::isfinite(prm->scale_value)) return FIA_ERR_PARAM;

    std::unique_ptr<fia_plan> p(new fia_plan());
    if (numel(query) == 0 || numel(attention_out) == 0) {
        p->kind = KIND_EMPTY;
        *plan_out = p.release();
        return FIA_OK;
    }
    if (!query->data || !key->data || !value->data || !attention_out->data ||
        !block_sparse_mask->data)
        return FIA_ERR_NULLPTR;
    // FP8 feature: query, key and value all E4M3FN with the three dequant
    // scales, a bf16 output; otherwise fp16/bf16 throughout and no scales.
    const bool fp8 = query->dtype == FIA_F8E4M3;
    if (fp8) {
        if (key->dtype != FIA_F8E4M3 || value->dtype != FIA_F8E4M3 || attention_out->dtype != FIA_BF16)
            return FIA_ERR_DTYPE;
        if (!prm->dequant_scale_query || !prm->dequant_scale_key || !prm->dequant_scale_value)
            return FIA_ERR_NULLPTR;
    } else {
        if (!is_half(query->dtype) || key->dtype != query->dtype || value->dtype != query->dtype ||
            attention_out->dtype != query->dtype)
            return FIA_ERR_DTYPE;
        if (prm->dequant_scale_query || prm->dequant_scale_key || prm->dequant_scale_value)
            return FIA_ERR_PARAM;
    }
    if (block_sparse_mask->dtype != FIA_U8 && block_sparse_mask->dtype != FIA_BOOL)
        return FIA_ERR_DTYPE;

    int32_t layout, kvlayout;
    bool bsh, kvbsh;
    fia_status st;
    if (!prm->q_input_layout || !prm->kv_input_layout) return FIA_ERR_NULLPTR;
    if ((st = parse_layout(prm->q_input_layout, &layout, &bsh)) != FIA_OK)
        return st == FIA_ERR_UNSUPPORTED ? FIA_ERR_LAYOUT : st;
    if ((st = parse_layout(prm->kv_input_layout, &kvlayout, &kvbsh)) != FIA_OK)
        return st == FIA_ERR_UNSUPPORTED ? FIA_ERR_LAYOUT : st;
    if (bsh || kvbsh) return FIA_ERR_LAYOUT;          // TND, BNSD, BSND only
    if (std::strcmp(prm->q_input_layout, prm->kv_input_layout) != 0) return FIA_ERR_LAYOUT;

    const int64_t N1 = prm->num_heads;
    const int64_t N2 = prm->num_key_value_heads == 0 ? N1 : prm->num_key_value_heads;
    if (N1 <= 0 || N2 <= 0 || N1 < N2 || N1 % N2 != 0) return FIA_ERR_PARAM;
    const int64_t X = prm->block_shape[0], Y = prm->block_shape[1];
    if (X <= 0 || Y <= 0 || X > kIntMax || Y > kIntMax || Y % 128 != 0) return FIA_ERR_PARAM;
    const bool have_q = prm->actual_seq_lengths != nullptr;
    const bool have_kv = prm->actual_seq_lengths_kv != nullptr;
    if (have_q != have_kv) return FIA_ERR_PARAM;
    if (layout == LAYOUT_TND && !have_q) return FIA_ERR_PARAM;

    Geo gq, gk, gv, go;
    if ((st = geometry(query, layout, false, N1, &gq)) != FIA_OK) return st;
    if ((st = geometry(key, layout, false, N2, &gk)) != FIA_OK) return st;
    if ((st = geometry(value, layout, false, N2, &gv)) != FIA_OK) return st;
    if ((st = geometry(attention_out, layout, false, N1, &go)) != FIA_OK) return st;
    if (gq.N != N1 || gk.N != N2 || gv.N != N2 || go.N != N1) return FIA_ERR_SHAPE;
    if (gk.S != gv.S || go.S != gq.S) return FIA_ERR_SHAPE;
    if (gq.D != gk.D || gq.D != gv.D || go.D != gq.D) return FIA_ERR_SHAPE;
    if (layout != LAYOUT_TND && (gk.B != gq.B || gv.B != gq.B || go.B != gq.B)) return FIA_ERR_SHAPE;
    if (gq.D != 64 && gq.D != 128) return FIA_ERR_UNSUPPORTED;   // D of 64 or 128

    std::vector<int64_t> lq, lkv, qstart, kvstart;
    int64_t B;
    if (layout == LAYOUT_TND) {
        if (prm->n_actual_seq_lengths != prm->n_actual_seq_lengths_kv) return FIA_ERR_PARAM;
        if ((st = resolve_cumulative(prm->actual_seq_lengths, prm->n_actual_seq_lengths, gq.S, &lq,
                                     &qstart)) != FIA_OK)
            return st;
        if ((st = resolve_cumulative(prm->actual_seq_lengths_kv, prm->n_actual_seq_lengths_kv,
                                     gk.S, &lkv, &kvstart)) != FIA_OK)
            return st;
        B = prm->n_actual_seq_lengths;
    } else {
        B = gq.B;
        if ((st = resolve_lengths(prm->actual_seq_lengths, prm->n_actual_seq_lengths, B, gq.S,
                                  &lq)) != FIA_OK)
            return st;
        if ((st = resolve_lengths(prm->actual_seq_lengths_kv, prm->n_actual_seq_lengths_kv, B,
                                  gk.S, &lkv)) != FIA_OK)
            return st;
    }
    // Mask shape [B, N1, ceil(maxQS / X), ceil(maxKVS / Y)], maxQS/maxKVS the
    // tensors' S for BNSD/BSND and the longest sequence for TND.
    int64_t maxq = gq.S, maxkv = gk.S;
    if (layout == LAYOUT_TND) {
        maxq = *std::max_element(lq.begin(), lq.end());
        maxkv = *std::max_element(lkv.begin(), lkv.end());
    }
    const int64_t nqb = (maxq + X - 1) / X, nkb = (maxkv + Y - 1) / Y;
    if (!dims_are(block_sparse_mask, {B, N1, nqb, nkb})) return FIA_ERR_SHAPE;
    // FP8: the quantization blocks are the sparse blocks, [128, 256] or
    // [128, 512]; scales fp32 [B, N1, nqb, 1] and [B, N2, nkb, 1]
    if (fp8) {
        if (X != 128 || (Y != 256 && Y != 512)) return FIA_ERR_PARAM;
        if (gq.D != 128) return FIA_ERR_UNSUPPORTED;
        const fia_tensor* sq = prm->dequant_scale_query;
        const fia_tensor* sk = prm->dequant_scale_key;
        const fia_tensor* sv = prm->dequant_scale_value;
        if (!sq->data || !sk->data || !sv->data) return FIA_ERR_NULLPTR;
        if (sq->dtype != FIA_F32 || sk->dtype != FIA_F32 || sv->dtype != FIA_F32) return FIA_ERR_DTYPE;
        if (!dims_are(sq, {B, N1, nqb, 1}) || !dims_are(sk, {B, N2, nkb, 1}) || !dims_are(sv, {B, N2, nkb, 1}))
            return FIA_ERR_SHAPE;
    }
    const bool want_lse = prm->softmax_lse_flag != 0;
    if (want_lse) {
        if (!softmax_lse || !softmax_lse->data) return FIA_ERR_NULLPTR;
        if (softmax_lse->dtype != FIA_F32) return FIA_ERR_DTYPE;
        bool ok = layout == LAYOUT_TND ? dims_are(softmax_lse, {gq.S, N1, 1})
                                       : dims_are(softmax_lse, {B, N1, gq.S, 1});
        if (!ok) return FIA_ERR_SHAPE;
    }

    p->kind = KIND_BSA;
    p->dtype = query->dtype;
    p->layout = layout;
    p->B = B;
    p->QN = N1;
    p->KVN = N2;
    p->G = N1 / N2;
    p->Sq = gq.S;
    p->Skv = gk.S;
    p->Dqk = p->Dv = gq.D;
    p->bsa_mask = (const uint8_t*)block_sparse_mask->data;
    p->bsa_nqb = nqb;
    p->bsa_nkb = nkb;
    p->n_rows = B * N1 * nqb;

    AttnArgs& a = p->attn;
    a.q = query->data;
    a.k = key->data;
    a.v = value->data;
    a.o = attention_out->data;
    a.lse = want_lse ? (float*)softmax_lse->data : nullptr;
    a.return_lse = want_lse;
    a.mode = 0;
    a.has_mask = 0;
    a.pre = a.next = kIntMax;
    a.QN = (int32_t)N1;
    a.KVN = (int32_t)N2;
    a.G = (int32_t)(N1 / N2);
    a.hg = 1;
    a.scale_log2 = (float)(prm->scale_value * kLog2e);
    a.nqb = (int32_t)nqb;
    a.nkb = (int32_t)nkb;
    a.bx = (int32_t)X;
    a.by = (int32_t)Y;
    a.fp8 = fp8;
    if (fp8) {
        a.q_scale = (const float*)prm->dequant_scale_query->data;
        a.k_scale = (const float*)prm->dequant_scale_key->data;
        a.v_scale = (const float*)prm->dequant_scale_value->data;
    }
    const int64_t D = gq.D;
    if (layout == LAYOUT_BNSD) {
        a.q_sH = gq.S * D; a.q_sS = D;
        a.k_sH = gk.S * D; a.k_sS = D;
        a.v_sH = gk.S * D; a.v_sS = D;
        a.o_sH = gq.S * D; a.o_sS = D;
        a.lse_sH = gq.S;   a.lse_sS = 1;
    } else {
        a.q_sH = D; a.q_sS = N1 * D;
        a.k_sH = D; a.k_sS = N2 * D;
        a.v_sH = D; a.v_sS = N2 * D;
        a.o_sH = D; a.o_sS = N1 * D;
        if (layout == LAYOUT_TND) { a.lse_sH = 1; a.lse_sS = N1; }
        else { a.lse_sH = gq.S; a.lse_sS = 1; }
    }
    a.q_rowmul = N1 * D;
    a.k_rowmul = N2 * D;
    a.v_rowmul = N2 * D;
    a.o_rowmul = N1 * D;
    a.lse_rowmul = N1;

    std::vector<BatchInfo> bi((size_t)B);
    for (int64_t b = 0; b < B; ++b) {
        bi[(size_t)b].q_row0 = layout == LAYOUT_TND ? qstart[(size_t)b] : b * gq.S;
        bi[(size_t)b].kv_row0 = layout == LAYOUT_TND ? kvstart[(size_t)b] : b * gk.S;
        bi[(size_t)b].lq = (int32_t)lq[(size_t)b];
        bi[(size_t)b].lkv = (int32_t)lkv[(size_t)b];
    }
    // One tile per (batch, q block, 128-row slice of the block, head); a tile
    // never straddles two q blocks.  Padded layouts also cover padding rows.
    PlanScratch& S = plan_scratch();
    std::vector<Tile>& tiles = S.tiles;
    tiles.clear();
    for (int64_t b = 0; b < B; ++b) {
        const int64_t rows = layout == LAYOUT_TND ? lq[(size_t)b] : gq.S;
        for (int64_t qb = 0; qb * X < rows; ++qb) {
            const int64_t bend = std::min<int64_t>((qb + 1) * X, rows);
            for (int64_t q0 = qb * X; q0 < bend; q0 += kBlockMSparse) {
                const int64_t q1 = std::min<int64_t>(q0 + kBlockMSparse, bend);
                for (int64_t h = 0; h < N1; ++h)
                    tiles.push_back(Tile{(int32_t)b, (int32_t)h, (int32_t)q0, (int32_t)q1, bi[(size_t)b]});
            }
        }
    }
    if (tiles.size() > (size_t)INT32_MAX) return FIA_ERR_UNSUPPORTED;
    // The workgroups of one kv head go to launch positions on one XCD (the
    // tiles of a kv head's GQA group then share that XCD's L2).
    p->n_tiles = (int64_t)tiles.size();
    a.n_tiles = (int32_t)tiles.size();
    p->off_batch = 0;
    S.tables.clear();
    uint64_t end = put(S.tables, 0, bi);
    p->off_tiles = align_up(end, 256);
    xcd_order(tiles.size(), [&](size_t i) { return tiles[i]; },
              [&](size_t i) { return (int)((tiles[i].h / (N1 / N2)) % kNumXcds); },
              tile_slots(S.tables, p->off_tiles, tiles.size()));
    finish_tables(p.get());
    p->off_cnt = 0;
    p->off_idx = align_up(p->off_cnt + (uint64_t)p->n_rows * 4, 256);
    p->workspace_bytes = align_up(p->off_idx + (uint64_t)p->n_rows * nkb * 4, 256);
    *workspace_size = p->workspace_bytes;
    *plan_out = p.release();
    return FIA_OK;
}

fia_status bsa_schedule_layout(const fia_plan* plan, uint64_t* cnt_offset, uint64_t* idx_offset,
                               int64_t* nqb, int64_t* nkb)
{
    if (!plan || !cnt_offset || !idx_offset || !nqb || !nkb) return FIA_ERR_NULLPTR;
    if (plan->kind != KIND_BSA) return FIA_ERR_PARAM;
    *cnt_offset = plan->off_cnt;
    *idx_offset = plan->off_idx;
    *nqb = plan->bsa_nqb;
    *nkb = plan->bsa_nkb;
    return FIA_OK;
}

static fia_status run_common(void* ws, uint64_t ws_size, fia_plan* p, void* stream, bool bsa)
{
    if (!p) return FIA_ERR_NULLPTR;
    if (bsa != (p->kind == KIND_BSA) && p->kind != KIND_EMPTY) return FIA_ERR_PARAM;
    if (p->kind == KIND_EMPTY) return FIA_OK;
    if (ws_size < p->workspace_bytes || (!ws && p->workspace_bytes)) return FIA_ERR_WORKSPACE;
    // phase 1 ran where no device was visible: there is no schedule on a
    // device, and phase 2 neither allocates nor copies
    if (p->tables_bytes && !p->dev_tables) return FIA_ERR_HIP;
    unsigned char* w = (unsigned char*)ws;
    const unsigned char* tb = (const unsigned char*)p->dev_tables;
    int rc = 0;
    if (p->kind == KIND_DECODE) {
        DecodeArgs d = p->dec;
        d.segs = (const DecSeg*)(tb + p->off_batch);
        d.pieces = (const DecPiece*)(tb + p->off_pieces);
        d.wave_first = (const int32_t*)(tb + p->off_waves);
        d.part_o = (float*)(w + p->off_part_o);
        d.part_lse = (float*)(w + p->off_part_lse);
        rc = launch_decode(*p, d, stream);
    } else {
        AttnArgs a = p->attn;
        a.batch = (const BatchInfo*)(tb + p->off_batch);
        a.tiles = (const Tile*)(tb + p->off_tiles);
        if (p->kind == KIND_BSA) {
            a.bsa_cnt = (const int32_t*)(w + p->off_cnt);
            a.bsa_idx = (const int32_t*)(w + p->off_idx);
            rc = launch_bsa(*p, a, stream);
        } else {
            rc = launch_prefill(*p, a, stream);
        }
    }
    return rc ? FIA_ERR_HIP : FIA_OK;
}

fia_status fia_run(void* workspace, uint64_t workspace_size, fia_plan* plan, void* stream)
{
    return run_common(workspace, workspace_size, plan, stream, false);
}

fia_status bsa_run(void* workspace, uint64_t workspace_size, fia_plan* plan, void* stream)
{
    return run_common(workspace, workspace_size, plan, stream, true);
}

fia_status fia_run_noalloc(fia_plan* plan, void* stream)
{
    if (!plan) return FIA_ERR_NULLPTR;
    if (plan->kind == KIND_EMPTY) return FIA_OK;
    static_assert(kNoAllocScratchBytes == FIA_NOALLOC_MAX_WORKSPACE, "scratch size");
    if (plan->workspace_bytes > kNoAllocScratchBytes) return FIA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (plan->workspace_bytes) {
        ws = noalloc_scratch();
        if (!ws) return FIA_ERR_HIP;
    }
    return run_common(ws, kNoAllocScratchBytes, plan, stream, plan->kind == KIND_BSA);
}

}  // extern "C"
