// gfx950 (CDNA4) kernels of the fused inference attention forward.
//
//   attn_fwd        prefill and block-sparse prefill: one workgroup of 4
//                   waves per 32-row block of up to 4 query heads of one GQA
//                   group (block-sparse: 128 rows of one head); K and V tiles
//                   of 64 tokens staged through LDS (double buffered); S^T = K Q^T
//                   and O^T = V^T P^T on v_mfma_f32_32x32x16_{bf16,f16}; fp32
//                   online softmax in registers; optional LSE.
//   decode_split    decode: one wave per resident slot, each with an equal
//                   share of all (batch, kv head, head chunk) token streams;
//                   the GQA heads sharing a kv head are the 16 columns of
//                   v_mfma_f32_16x16x32, so every K/V byte is read once;
//                   pages are gathered through the block table.  The
//                   decode kernels read the cache with the streaming (nt)
//                   cache policy: each byte is read once per run.
//   decode_split_i8 decode against an int8 KV cache (per-channel or
//                   per-token scale and offset), the same column layout.
//   decode_combine  merges the pieces of one (batch, head) by their LSE.
//   bsa_compact     compacts the block-sparse mask into ascending kv-block
//                   lists per (batch, head, q block).
//   bsa_fp8         block-sparse prefill with E4M3FN inputs and per-block
//                   scales: S^T on v_mfma_f32_32x32x64_f8f6f4, P V on bf16.
//   mla_decode      MLA decode (query D 512 + rope 64, one kv head): a
//                   workgroup of up to 8 waves shares DMA-staged K / K_rope /
//                   V tiles across up to 128 (head, token) rows.
//
// The method: pages "torch_npu.npu_prompt_flash_attention" (formula),
// "torch_npu.npu_fused_infer_attention_score_v2" (formula, sparse_mode,
// softmax_lse, kv pseudo-quant and query_rope / key_rope parameters),
// "aclnnBlockSparseAttentionV2" (formula, constraints, FP8 feature).  The
// online-softmax rescaling and the split-KV merge by LSE rest on the identity
// the softmax_lse output description gives: a row's log-sum-exp lets partial
// results over disjoint key sets be merged exactly.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "fia_internal.h"

namespace fia {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef _Float16 f16x2 __attribute__((__vector_size__(2 * sizeof(_Float16))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr float kLn2 = 0.69314718055994530942f;

// Per-dtype MFMA and conversions (round to nearest even).
template <int DT>
struct Ops;

template <>
struct Ops<FIA_BF16> {
    static __device__ __forceinline__ f32x16 mma32(uint4 a, uint4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(uint4 a, uint4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float x, float y)
    {
        f32x2 v = {x, y};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    }
};

template <>
struct Ops<FIA_F16> {
    static __device__ __forceinline__ f32x16 mma32(uint4 a, uint4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(uint4 a, uint4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float x, float y)
    {
        f32x2 v = {x, y};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Helpers of the prefill, block-sparse and decode kernels.
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane j supplies row j/4, columns 4(j%4)..+3 of a 4 x 16 block; lane i
// receives column i of the 4 rows.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p)
{
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(uint2, v);
}

// Value of x in the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float other_half_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float other_half_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Rows whose running max grows by less than 2^kLazy (in exp2 units) keep
// their old max: p stays below 2^kLazy and no O rescale is needed.
constexpr float kLazy = 8.f;
// Smallest scale used in exp2(s * c - m * c): keeps masked (-inf) scores at
// exactly 0 when the scale is 0, while every finite score gives exp2(0) = 1.
constexpr float kMinScale = 1e-30f;

// waitcnt immediates (gfx9 encoding): vmcnt(n) alone, lgkmcnt(0) alone
#define FIA_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x70 | 0xF00)
#define FIA_LGKMCNT0 0xC07F

typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource (V#) over `bytes` bytes at `base`: stride 0, raw 32-bit
// dword format; offsets at or past `bytes` read as zero.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes)
{
    const uint64_t addr = (uint64_t)(uintptr_t)base;
    // the values are wave-uniform; readfirstlane places them in SGPRs
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(addr >> 32) & 0xffffu));
    r.z = __builtin_amdgcn_readfirstlane((int)min(max(bytes, (int64_t)0), (int64_t)0x7fffffff));
    r.w = 0x00020000;
    return r;
}

// 16 bytes per lane from a buffer resource straight into LDS: lane i of the
// wave writes LDS byte address lds_wave + 16 i.  Issued as inline assembly on purpose: the
// compiler cannot prove that LDS reads of the other pipeline buffer do not
// alias these writes and would otherwise wait for the prefetch to finish
// before every read.  The kernels order the data themselves: vmcnt wait +
// barrier before a buffer is read, and no prefetch into a buffer before its
// last reads are complete.
__device__ __forceinline__ void dma16(i32x4 rs, uint32_t lds_wave, uint32_t voff)
{
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_wave);
    // m0 is reserved by the compiler: save and restore it around the load
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(m0v), "v"(voff), "s"(rs) : "memory");
}

// N (2 or 4) such loads with one M0 value: load u writes LDS lds_base +
// 1024 u + 16 lane and reads voff[u] + 1024 u (the instruction offset
// applies to both addresses), so the callers pass offsets reduced by 1024 u.
// Fewer M0 writes between queued LDS loads stall the issuing wave less.
template <int N>
__device__ __forceinline__ void dma16_burst(i32x4 rs, uint32_t lds_base, const uint32_t* voff)
{
    static_assert(N == 2 || N == 4, "burst of 2 or 4");
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
    uint32_t keep;
    if (N == 2)
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                     "buffer_load_dwordx4 %2, %4, 0 offen lds\n\t"
                     "buffer_load_dwordx4 %3, %4, 0 offen offset:1024 lds\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(keep) : "s"(m0v), "v"(voff[0]), "v"(voff[1]), "s"(rs) : "memory");
    else
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                     "buffer_load_dwordx4 %2, %6, 0 offen lds\n\t"
                     "buffer_load_dwordx4 %3, %6, 0 offen offset:1024 lds\n\t"
                     "buffer_load_dwordx4 %4, %6, 0 offen offset:2048 lds\n\t"
                     "buffer_load_dwordx4 %5, %6, 0 offen offset:3072 lds\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(keep)
                     : "s"(m0v), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(rs) : "memory");
}

// Cache policy of the decode kernels' KV-cache loads: nt (streaming).  Each
// cached K / V byte is read once per run, and with the nt bit a plain
// 16-byte read of a 4 GiB buffer moves 6.97 TB/s against 6.2 TB/s without
// it (MI355X).
constexpr int kStream = 2;

// The same load through the compiler-visible intrinsic (the compiler then
// orders the LDS reads after it conservatively); AUX is the cache policy.
template <int AUX = 0>
__device__ __forceinline__ void dma16_tracked(__amdgpu_buffer_rsrc_t rs, uint16_t* lds_wave, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds_wave, 16, voff, 0, 0, AUX);
}

// dma16 with the streaming (nt) cache policy, and its 4-byte form (lane i
// writes lds_wave + 4 i).
__device__ __forceinline__ void dma16_nt(i32x4 rs, uint32_t lds_wave, uint32_t voff)
{
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_wave);
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(m0v), "v"(voff), "s"(rs) : "memory");
}
__device__ __forceinline__ void dma4_nt(i32x4 rs, uint32_t lds_wave, uint32_t voff)
{
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_wave);
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dword %2, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(m0v), "v"(voff), "s"(rs) : "memory");
}

// Buffer resource over rows [row0, lkv) of a row-strided tensor (rows of
// `rowlen` elements every `stride` elements); 0 valid bytes when none.
__device__ __forceinline__ i32x4 rows_rsrc(const uint16_t* base, int64_t row0, int64_t lkv,
                                           int64_t stride, int rowlen)
{
    const int64_t n = lkv - row0;
    const int64_t bytes = n > 0 ? ((n - 1) * stride + rowlen) * 2 : 0;
    return make_rsrc(base + row0 * stride, bytes);
}

// Kinds of the prefill kernel: masks from lengths and sparse_mode bands only;
// plus an explicit byte mask (sparse_mode 0/1); block-sparse tile lists.
enum { kDense = 0, kMasked = 1, kSparse = 2 };

// Running max over values that may be -inf (no NaN quieting needed).
__device__ __forceinline__ float vmax(float x, float y) { return __builtin_elementwise_maximum(x, y); }

// ---------------------------------------------------------------------------
// Prefill / block-sparse attention.
//
// Workgroup: 4 waves of 32 query rows each, over hg heads of one GQA group
// (block-sparse: hg = 1, 128 rows of one head; a tile never straddles two q
// blocks).  Per 64-token kv tile (the q block's list for block-sparse):
//   S^T (64 x 32 per wave) = K Q^T   two 32x32 MFMA tiles, Q in registers,
//                                    K read from LDS (16-byte chunks
//                                    XOR-swizzled by row)
//   online softmax on the S^T accumulators: lane (row, half) holds 32 of the
//   row's 64 scores; the two halves exchange max and sum once.
//   O^T (D_v x 32) += V^T P^T         P straight from the S^T registers as the
//                                    B operand; V read from a row-major LDS
//                                    tile with the gfx950 transpose read.
// The kv index set of the B operand slots (from the S^T accumulator layout)
// and of the A operand slots (from the transposed V reads) is the same, so
// the contraction pairs each P value with its V row.  K and V tiles are
// double buffered; the next tile's loads go out at the top of an iteration.
// ---------------------------------------------------------------------------
template <int DT, int DQK, int DV, int KIND, int NW, int NS, bool PG>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_fwd(AttnArgs a)
{
    constexpr bool BSA = KIND == kSparse;
    constexpr int BN = kBlockN;            // 64 kv tokens per tile
    constexpr int VCH = DV / 8;            // 16-byte chunks per V row
    constexpr int VSW = VCH >= 16 ? 4 : 2; // V chunk swizzle step
    constexpr bool KROWS = DQK == 128;     // K layout: swizzled rows or panels
    constexpr int KT = BN * DQK;           // K tile elements (rows not padded)
    constexpr int STAGE = KT + BN * DV;
    constexpr int NQ = DQK / 16;           // k-steps of S^T = K Q^T
    constexpr int NO = DV / 32;            // 32-row d tiles of O^T
    constexpr int NKI = BN * DQK / 8 / (64 * NW); // K load instructions per wave per tile
    constexpr int NVI = BN * VCH / (64 * NW);     // V load instructions per wave per tile
    static_assert(NKI * 64 * NW * 8 == BN * DQK && NVI * 64 * NW == BN * VCH, "tile split");
    static_assert(NS >= 2 && NS <= 4, "stages");
    using O = Ops<DT>;

    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_void*)smem;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // A workgroup covers hg heads of one GQA group (t.h ..) and 32 NW / hg
    // rows (t.q0 .. t.q1); wave w takes head t.h + w % hg, rows
    // t.q0 + 32 (w / hg) + (0..31).
    const int hg = BSA ? 1 : a.hg;
    const Tile t = a.tiles[blockIdx.x];
    const BatchInfo bi = t.bi;
    if (!BSA && t.h < 0) {
        // zero fill: padding rows [t.q0, t.q1) of batch t.b, every head
        const BatchInfo& zb = bi;
        constexpr int CH = DV / 8;         // 16-byte chunks per (row, head)
        const int nrow = t.q1 - t.q0, QN = a.QN;
        const bool head_inner = a.o_sH == DV;   // heads adjacent in memory (BSND, BSH)
        uint16_t* ob = (uint16_t*)a.o + zb.q_row0 * a.o_rowmul;
        for (int e = tid; e < nrow * QN * CH; e += NW * 64) {
            const int ch = e % CH, rest = e / CH;
            const int r = head_inner ? rest / QN : rest % nrow;
            const int hd = head_inner ? rest % QN : rest / nrow;
            *(uint4*)(ob + (int64_t)hd * a.o_sH + (int64_t)(t.q0 + r) * a.o_sS + 8 * ch) = make_uint4(0, 0, 0, 0);
        }
        if (a.return_lse) {
            float* lb = a.lse + zb.q_row0 * a.lse_rowmul;
            for (int e = tid; e < nrow * QN; e += NW * 64) {
                const int r = e % nrow, hd = e / nrow;
                lb[(int64_t)hd * a.lse_sH + (int64_t)(t.q0 + r) * a.lse_sS] = INFINITY;
            }
        }
        return;
    }
    const int h = t.h + w % hg;
    const int q0 = t.q0, q1 = t.q1;
    const int Lq = bi.lq, Lkv = bi.lkv;
    const int g = h / a.G;
    const int qend = min(q1, Lq);
    const int delta = Lkv - Lq;
    const int mode = a.mode;
    const int pre = (int)a.pre, next = (int)a.next;

    const uint16_t* qp = (const uint16_t*)a.q + bi.q_row0 * a.q_rowmul + (int64_t)h * a.q_sH;
    const uint16_t* kp = (const uint16_t*)a.k + bi.kv_row0 * a.k_rowmul + (int64_t)g * a.k_sH;
    const uint16_t* vp = (const uint16_t*)a.v + bi.kv_row0 * a.v_rowmul + (int64_t)g * a.v_sH;
    // the explicit mask exists only in the kMasked instantiation
    const uint8_t* mbase = KIND == kMasked ? a.mask + (int64_t)t.b * a.mask_bstride : nullptr;

    const int wr0 = q0 + 32 * (w / hg);    // first row of this wave
    const int row = wr0 + l32;             // this lane's query row
    const int wend = min(wr0 + 32, qend);  // rows < wend are computed

    // A negative scale is moved onto Q (exact sign flip) so that c > 0.
    const float c = fmaxf(fabsf(a.scale_log2), kMinScale);
    const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;

    // Q as the B operand of S^T = K Q^T: lane (row, hh) holds d = 16s + 8hh.
    uint4 qf[NQ];
    if (row < qend) {
        const uint16_t* src = qp + (int64_t)row * a.q_sS + 8 * hh;
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
            uint4 v = *(const uint4*)(src + 16 * s);
            v.x ^= qflip; v.y ^= qflip; v.z ^= qflip; v.w ^= qflip;
            qf[s] = v;
        }
    } else {
#pragma unroll
        for (int s = 0; s < NQ; ++s) qf[s] = make_uint4(0, 0, 0, 0);
    }

    // kv tiles of this workgroup
    int ntiles = 0;
    int kv_lo = 0;
    const int32_t* blist = nullptr;
    int per = 1;
    if (BSA) {
        const int qb = q0 / a.bx;
        const int64_t rowi = ((int64_t)t.b * a.QN + h) * a.nqb + qb;
        per = a.by / BN;
        ntiles = qend > q0 ? a.bsa_cnt[rowi] * per : 0;
        blist = a.bsa_idx + rowi * a.nkb;
    } else if (qend > q0 && Lkv > 0) {
        const int last = qend - 1;
        int lo = 0, hi = Lkv;
        if (mode == 0 && mbase) {
            lo = max(0, q0 - pre);
            hi = min(Lkv, last + next + 1);
        } else if (mode == 2) {
            hi = min(Lkv, last + 1);
        } else if (mode == 3) {
            hi = min(Lkv, last + delta + 1);
        } else if (mode == 4) {
            lo = max(0, q0 + delta - pre);
            hi = min(Lkv, last + delta + next + 1);
        }
        if (hi > lo) {
            kv_lo = lo / BN * BN;
            ntiles = (hi - kv_lo + BN - 1) / BN;
        }
    }
    // Block-sparse: 64 entries of the row's block list live in one register
    // per lane (lane l: entry bsa_cb + l) and each tile's block comes from
    // v_readlane, so no scalar load sits between a tile and its loads.  The
    // window is reloaded when an index passes its end; it starts NS entries
    // behind the index that moved it (the current tile is asked for after
    // the next one).
    int bsa_cb = 0, bsa_bc = 0;
    if (BSA && ntiles > 0) bsa_bc = lane < a.nkb ? blist[lane] : 0;
    auto tile_c0 = [&](int it) -> int {
        if (BSA) {
            const int idx = it / per;
            if (idx >= bsa_cb + 64) {
                bsa_cb = idx - NS;
                bsa_bc = bsa_cb + lane < a.nkb ? blist[bsa_cb + lane] : 0;
            }
            return __builtin_amdgcn_readlane(bsa_bc, idx - bsa_cb) * a.by + BN * (it % per);
        }
        return kv_lo + BN * it;
    };

    // Direct-to-LDS loads; instruction u of wave w fills 16-byte slots
    // 64 (4u + w) + lane of the tile.  LDS layouts (64 banks of 4 bytes):
    //   K, D_qk = 128: row-major 256-byte rows; chunk c of row r sits at
    //      c ^ (r & 15).  Other D_qk: column panels of 64 rows x 64 d
    //      (128-byte rows); chunk c of row r sits at c ^ ((r >> 1) & 7).
    //      Either way each 16-row group of the MFMA operand reads hits 16
    //      distinct 16-byte bank groups.
    //   V: row-major rows of DV; chunk c of row r sits at c ^ VSW (r & 3): the
    //      4-row groups of the transposed reads hit distinct bank groups.
    // Instruction u of wave w fills slots 64 u' + lane, u' = NW u + w; the
    // lane offsets do not depend on the tile (computed once).
    auto k_off = [&](int up, int ln) -> int {   // element offset of K slot 64 u' + ln
        const int sl = 64 * up + ln;
        if (KROWS) {
            const int r = sl >> 4;
            return r * a.k_sS + 8 * ((sl & 15) ^ (r & 15));
        }
        const int r = (sl >> 3) & 63;
        return r * a.k_sS + 64 * (sl >> 9) + 8 * ((sl & 7) ^ ((r >> 1) & 7));
    };
    auto v_off = [&](int up, int ln) -> int {   // element offset of V slot 64 u' + ln
        const int sl = 64 * up + ln;
        const int r = sl / VCH;
        return r * a.v_sS + 8 * ((sl % VCH) ^ (VSW * (r & 3)));
    };
    // Load bursts: wave w fills the consecutive slots NKI w .. NKI w + NKI - 1
    // (NVI w .. for V) with one M0 value per burst.  The reduced offsets
    // off(slot) - 1024 u stay >= 0: slot NKI w + u starts at least 4u rows
    // into the tile (rows of >= 128 elements apart) for D = 64, 128 and for
    // V; the D_qk = 192 panels do not guarantee that, so K there takes one
    // M0 per load (slot NW u + w).
    constexpr bool KB = DQK != 192 && (NKI == 2 || NKI == 4);
    constexpr bool VB = NVI == 2 || NVI == 4;
    uint32_t koff[NKI], voff[NVI];
#pragma unroll
    for (int u = 0; u < NKI; ++u)
        koff[u] = KB ? (uint32_t)k_off(NKI * w + u, lane) * 2u - 1024u * u : (uint32_t)k_off(NW * u + w, lane) * 2u;
#pragma unroll
    for (int u = 0; u < NVI; ++u)
        voff[u] = VB ? (uint32_t)v_off(NVI * w + u, lane) * 2u - 1024u * u : (uint32_t)v_off(NW * u + w, lane) * 2u;
    // Paged K/V: a tile lies inside one pool block (block_size % 64 == 0).
    // 64 consecutive block-table entries of the batch live in one register
    // per lane (lane l: entry pg_cb + l) and each tile's block id comes from
    // v_readlane; tiles are loaded in ascending order, so the window only
    // moves forward.  Entries at or past ceil(Lkv / block_size) are never
    // read.
    const int32_t* bt = PG ? a.block_table + (int64_t)t.b * a.bt_stride : nullptr;
    const int npages = PG ? (Lkv + a.block_size - 1) / a.block_size : 0;
    int pg_cb = PG ? kv_lo / a.block_size : 0;
    int pg_bc = 0;
    if (PG && ntiles > 0) pg_bc = pg_cb + lane < npages ? bt[pg_cb + lane] : 0;
    auto load_tile = [&](int c0, int buf) {
        const uint32_t ks = smem_lds + 2u * (uint32_t)(buf * STAGE);
        const uint32_t vs = ks + 2u * KT;
        i32x4 kr, vr;
        if constexpr (PG) {
            const int pi = c0 / a.block_size;
            if (pi >= pg_cb + 64) {
                pg_cb = pi;
                pg_bc = pg_cb + lane < npages ? bt[pg_cb + lane] : 0;
            }
            const int64_t blk = __builtin_amdgcn_readlane(pg_bc, pi - pg_cb);
            const int r0 = c0 - pi * a.block_size;          // row of the tile in its block
            const int r1 = r0 + min(Lkv - c0, BN);           // rows past Lkv read as zero
            kr = rows_rsrc(kp + blk * a.p_blk, r0, r1, a.k_sS, DQK);
            vr = rows_rsrc(vp + blk * a.p_blk, r0, r1, a.v_sS, DV);
        } else {
            kr = rows_rsrc(kp, c0, Lkv, a.k_sS, DQK);
            vr = rows_rsrc(vp, c0, Lkv, a.v_sS, DV);
        }
        if constexpr (KB) {
            dma16_burst<NKI>(kr, ks + 1024u * (NKI * w), koff);
        } else {
#pragma unroll
            for (int u = 0; u < NKI; ++u) dma16(kr, ks + 1024u * (NW * u + w), koff[u]);
        }
        if constexpr (VB) {
            dma16_burst<NVI>(vr, vs + 1024u * (NVI * w), voff);
        } else {
#pragma unroll
            for (int u = 0; u < NVI; ++u) dma16(vr, vs + 1024u * (NW * u + w), voff[u]);
        }
    };

    // per-lane LDS offsets of the MFMA operand reads
    const int krow0 = l32, krow1 = 32 + l32;
    const int kx0 = KROWS ? (krow0 & 15) : ((krow0 >> 1) & 7);
    const int kx1 = KROWS ? (krow1 & 15) : ((krow1 >> 1) & 7);
    // V transposed reads: group gi = lane/16 covers d 16 (gi & 1) of a 32-row
    // d tile and kv rows 4 hh + (i >> 2) (+8 for the second read), i = lane & 15
    const int vi = lane & 15;
    const int vrow = 4 * hh + (vi >> 2);
    const int vswz = VSW * (vi >> 2);      // = VSW * (vrow & 3)
    const int vcol_lo = 2 * ((lane >> 4) & 1) + ((vi & 3) >> 1);
    const int vsub = 4 * (vi & 1);

    f32x16 acc[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[o][r] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float lazy_raw = kLazy / c;

    // NS stages: tiles it + 1 .. it + NS - 2 stay in flight while tile it is
    // computed; tile it + NS - 1 goes into the stage of tile it - 1.
    constexpr int PER = NKI + NVI;         // load instructions per wave and tile
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
        if (j < ntiles) load_tile(tile_c0(j), j);
    // Allowed keys of row r form the band r + lo_off <= j <= r + hi_off
    // (besides j < Lkv and the explicit mask), with +-2^30 for an open side;
    // fixed per wave, so each tile is classified with a few comparisons.
    int lo_off = -(1 << 30), hi_off = 1 << 30;
    bool allow_full = true;                // false: every tile takes the element mask
    if (!BSA) {
        int64_t lo = lo_off, hi = hi_off;
        switch (mode) {
        case 0:
            if (mbase) { lo = -(int64_t)pre; hi = next; allow_full = false; }
            break;
        case 1: allow_full = false; break;
        case 2: hi = 0; break;
        case 3: hi = delta; break;
        case 4: lo = (int64_t)delta - pre; hi = (int64_t)delta + next; break;
        default: break;
        }
        lo_off = (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, lo));
        hi_off = (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, hi));
    }
    // The same conditions as thresholds on the tile start c0 (last key
    // cl = c0 + BN - 1) for the wave's rows [wr0, wend - 1]:
    //   skip <=> c0 < tlo_skip (cl < wr0 + lo_off)  or  c0 > thi_skip
    //            (c0 > wend - 1 + hi_off, or c0 >= Lkv), or no rows;
    //   full <=> tlo_full <= c0 <= thi_full (c0 >= wend - 1 + lo_off,
    //            cl <= wr0 + hi_off, c0 + BN <= Lkv, 32 rows, no mask).
    auto clamp32 = [](int64_t x) -> int { return (int)max<int64_t>(INT32_MIN, min<int64_t>(INT32_MAX, x)); };
    const int tlo_skip = wend <= wr0 ? INT32_MAX : clamp32((int64_t)wr0 + lo_off - BN + 1);
    const int thi_skip = clamp32(min<int64_t>(Lkv - 1, (int64_t)wend - 1 + hi_off));
    const int tlo_full = allow_full && wend - wr0 == 32 ? clamp32((int64_t)wend - 1 + lo_off) : INT32_MAX;
    const int thi_full = clamp32(min<int64_t>((int64_t)Lkv - BN, (int64_t)wr0 + hi_off - BN + 1));

    for (int it = 0; it < ntiles; ++it) {
        const int buf = it % NS;
        // this wave's loads of tile `it` landed: later tiles may be pending
        const int later = min(NS - 2, ntiles - 1 - it);
        if (NS >= 4 && later >= 2) __builtin_amdgcn_s_waitcnt(FIA_VMCNT(2 * PER));
        else if (NS >= 3 && later >= 1) __builtin_amdgcn_s_waitcnt(FIA_VMCNT(PER));
        else __builtin_amdgcn_s_waitcnt(FIA_VMCNT(0));
        __syncthreads();                   // everyone's did; stage of tile it - 1 is free
        const int c0 = tile_c0(it);
        if (it + NS - 1 < ntiles) load_tile(tile_c0(it + NS - 1), (it + NS - 1) % NS);

        // Which part of this tile the wave's rows may see: none (skip), all
        // (full), or some (element mask).
        const bool skip = c0 < tlo_skip || c0 > thi_skip;
        const bool full = c0 >= tlo_full && c0 <= thi_full;
        if (skip) continue;

        const uint16_t* ks = smem + buf * STAGE;
        const uint16_t* vs = ks + KT;
        f32x16 s0, s1;
#pragma unroll
        for (int r = 0; r < 16; ++r) s0[r] = s1[r] = 0.f;
        // The K operands are read two k-steps ahead of the MFMAs that use
        // them; the scheduling barriers keep the compiler from moving each
        // read back next to its MFMA, which would expose the LDS latency at
        // every k-step.
        constexpr int KPD = NQ < 2 ? NQ : 2;
        uint4 ka0[NQ], ka1[NQ];
        auto read_k = [&](int s) {
            if (KROWS) {
                const int ch = 2 * s + hh;
                ka0[s] = *(const uint4*)(ks + krow0 * DQK + 8 * (ch ^ kx0));
                ka1[s] = *(const uint4*)(ks + krow1 * DQK + 8 * (ch ^ kx1));
            } else {
                const int ch = 2 * (s & 3) + hh;
                const uint16_t* pn = ks + (s >> 2) * (BN * 64);
                ka0[s] = *(const uint4*)(pn + krow0 * 64 + 8 * (ch ^ kx0));
                ka1[s] = *(const uint4*)(pn + krow1 * 64 + 8 * (ch ^ kx1));
            }
        };
#pragma unroll
        for (int s = 0; s < KPD; ++s) read_k(s);
        // D_qk = 192: the wave in a matrix phase wins issue over the other
        // wave's softmax (measured 3 % faster there; slower for the
        // block-sparse D = 128 kernel, neutral for dense D = 128)
        constexpr bool PRIO = DQK == 192;
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
            if (s + KPD < NQ) read_k(s + KPD);
            s0 = O::mma32(ka0[s], qf[s], s0);
            s1 = O::mma32(ka1[s], qf[s], s1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);

        // element mask (boundary tiles only): accumulator r holds kv index
        // c0 + 4 hh + kofs(r), kofs(r) = 32 (r/16) + 8 ((r%16)/4) + r%4; the
        // row's allowed keys are [jlo, jhi] relative to c0 + 4 hh, plus the
        // explicit mask in modes 0/1.
        if (!full) {
            const int base = c0 + 4 * hh;
            const int jlo = (int)max<int64_t>(-base, (int64_t)row + lo_off - base);
            const int jhi = row >= qend ? -1 : (int)min<int64_t>(Lkv - 1 - base, (int64_t)row + hi_off - base);
            const uint8_t* mrow =
                (!BSA && mbase && row < qend) ? mbase + (int64_t)row * a.mask_rstride + base : nullptr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int k0 = 8 * (r >> 2) + (r & 3), k1 = 32 + k0;
                bool ok0 = k0 >= jlo && k0 <= jhi, ok1 = k1 >= jlo && k1 <= jhi;
                if (mrow) {
                    ok0 = ok0 && mrow[k0] == 0;
                    ok1 = ok1 && mrow[k1] == 0;
                }
                s0[r] = ok0 ? s0[r] : -INFINITY;
                s1[r] = ok1 ? s1[r] : -INFINITY;
            }
        }

        // row max over the tile (raw score units; c > 0): four independent
        // three-input chains, then their combination (short dependency path)
        float mq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            mq[q] = vmax(s0[4 * q], vmax(s0[4 * q + 1], s1[4 * q]));
            mq[q] = vmax(mq[q], vmax(s0[4 * q + 2], s1[4 * q + 1]));
            mq[q] = vmax(mq[q], vmax(s0[4 * q + 3], s1[4 * q + 2]));
            mq[q] = vmax(mq[q], s1[4 * q + 3]);
        }
        float mt = vmax(vmax(mq[0], vmax(mq[1], mq[2])), mq[3]);
        mt = other_half_max(mt);
        const float mn = fmaxf(m, mt);
        const bool grow = (m == -INFINITY) ? (mn > -INFINITY) : (mn > m + lazy_raw);
        if (__ballot(grow)) {
            // adopt the new max in every row of the wave; rescale O and l
            float alpha = 1.f;
            if (m == -INFINITY) alpha = 0.f;
            else if (mn != -INFINITY) alpha = fast_exp2((m - mn) * c);
            m = mn;
            l *= alpha;
#pragma unroll
            for (int o = 0; o < NO; ++o)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[o][r] *= alpha;
        }
        const float mc = (m == -INFINITY) ? 0.f : m * c;
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s0[r] = fast_exp2(__builtin_fmaf(s0[r], c, -mc));
            s1[r] = fast_exp2(__builtin_fmaf(s1[r], c, -mc));
            ps += s0[r] + s1[r];
        }
        l += ps;

        // P^T as the B operand: k-step k holds accumulators 8k..8k+7 of the
        // 32 (s0 then s1); the matching V rows come from two transposed reads.
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const f32x16& src = (k < 2) ? s0 : s1;
            const int b8 = 8 * (k & 1);
            uint4 pb;
            pb.x = O::pack2(src[b8 + 0], src[b8 + 1]);
            pb.y = O::pack2(src[b8 + 2], src[b8 + 3]);
            pb.z = O::pack2(src[b8 + 4], src[b8 + 5]);
            pb.w = O::pack2(src[b8 + 6], src[b8 + 7]);
            const uint16_t* vk = vs + (16 * k + vrow) * DV + vsub;
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                const int pc = (4 * o + vcol_lo) ^ vswz;
                const uint2 lo = lds_read_tr16(vk + 8 * pc);
                const uint2 hi = lds_read_tr16(vk + 8 * DV + 8 * pc);
                const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
                acc[o] = O::mma32(va, pb, acc[o]);
            }
        }
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    }

    // epilogue: rows < q1 are written; rows in [qend, q1) and rows with no
    // allowed key get out = 0 and lse = +inf.
    const float lt = other_half_sum(l);
    if (row < q1) {
        const bool valid = row < qend && lt > 0.f;
        const float inv = valid ? 1.f / lt : 0.f;
        uint16_t* op = (uint16_t*)a.o + bi.q_row0 * a.o_rowmul + (int64_t)h * a.o_sH +
                       (int64_t)row * a.o_sS;
#pragma unroll
        for (int o = 0; o < NO; ++o)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                uint2 v;
                v.x = O::pack2(acc[o][4 * g4 + 0] * inv, acc[o][4 * g4 + 1] * inv);
                v.y = O::pack2(acc[o][4 * g4 + 2] * inv, acc[o][4 * g4 + 3] * inv);
                *(uint2*)(op + 32 * o + 8 * g4 + 4 * hh) = v;
            }
        if (a.return_lse && hh == 0) {
            float* lp = a.lse + bi.q_row0 * a.lse_rowmul + (int64_t)h * a.lse_sH +
                        (int64_t)row * a.lse_sS;
            *lp = valid ? (m * c + __log2f(lt)) * kLn2 : INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// Block-sparse attention with FP8 (E4M3FN) query, key and value (FP8 feature
// of the block-sparse page): each element stands for its value times the
// fp32 scale of its block (query: 128-row blocks; key / value: the Y-token kv
// blocks of the sparse mask, Y = 256 or 512).  A workgroup is the 128 rows of
// one (batch, head, q block), as in the 16-bit kernel.  Per 64-token tile of
// the compacted block list:
//   S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4 (both operands E4M3FN; K from
//     LDS, Q in registers); lane (row, hh) holds d = 64 s + 32 hh + (0..31)
//     of k-step s in both operands, so every d meets its partner; the
//     scores are then multiplied by qs * ks of the tile's blocks;
//   online softmax as in the 16-bit kernel;
//   O^T += V^T P^T on bf16 MFMAs: P times the tile's vs, rounded to bf16;
//     V widened exactly from E4M3FN to bf16 in LDS (E4M3FN values are bf16
//     values), into the swizzled layout of the 16-bit kernel's V tiles.
// K and V bytes of tile it + 1 go direct-to-LDS at the top of iteration it;
// its V bytes are widened at the end of iteration it, after a barrier that
// frees the one bf16 V tile, by the lanes whose loads brought them, so the
// next per-tile barrier also publishes them.  48 KB of LDS and at most 168
// VGPRs give three workgroups per CU (14 % faster than two with a second bf16
// V tile and one barrier per tile).
// ---------------------------------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x4 rows_rsrc8(const uint8_t* base, int64_t row0, int64_t lkv, int64_t stride,
                                            int rowlen)
{
    const int64_t n = lkv - row0;
    const int64_t bytes = n > 0 ? (n - 1) * stride + rowlen : 0;
    return make_rsrc(base + row0 * stride, bytes);
}

__global__ __launch_bounds__(256, 3) void bsa_fp8(AttnArgs a)
{
    constexpr int NW = 4, BN = kBlockN, D = 128;
    constexpr int K8 = BN * D;               // K tile bytes
    constexpr int STAGE = K8 + K8;           // K bytes, V bytes
    constexpr int VBF = 2 * STAGE;           // offset of the one bf16 V tile
    constexpr int NO = D / 32;
    using O = Ops<FIA_BF16>;

    extern __shared__ __attribute__((aligned(16))) uint8_t smem8[];
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_void*)smem8;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const Tile t = a.tiles[blockIdx.x];
    const BatchInfo bi = t.bi;
    const int h = t.h, q0 = t.q0, q1 = t.q1;
    const int Lq = bi.lq, Lkv = bi.lkv;
    const int g = h / a.G;
    const int qend = min(q1, Lq);
    const uint8_t* qp = (const uint8_t*)a.q + bi.q_row0 * a.q_rowmul + (int64_t)h * a.q_sH;
    const uint8_t* kp = (const uint8_t*)a.k + bi.kv_row0 * a.k_rowmul + (int64_t)g * a.k_sH;
    const uint8_t* vp = (const uint8_t*)a.v + bi.kv_row0 * a.v_rowmul + (int64_t)g * a.v_sH;
    const int wr0 = q0 + 32 * w;
    const int row = wr0 + l32;
    const int wend = min(wr0 + 32, qend);
    const float c = fmaxf(fabsf(a.scale_log2), kMinScale);
    const uint32_t qflip = a.scale_log2 < 0.f ? 0x80808080u : 0u;   // E4M3FN sign bits

    // the workgroup's q block, its scale and its compacted kv-block list
    const int qb = q0 / a.bx;
    const int64_t rowi = ((int64_t)t.b * a.QN + h) * a.nqb + qb;
    const float qs = a.q_scale[rowi];
    const int per = a.by / BN;
    const int ntiles = qend > q0 ? a.bsa_cnt[rowi] * per : 0;
    const int32_t* blist = a.bsa_idx + rowi * a.nkb;
    const float* ksb = a.k_scale + ((int64_t)t.b * a.KVN + g) * a.nkb;
    const float* vsb = a.v_scale + ((int64_t)t.b * a.KVN + g) * a.nkb;

    // Q as the B operand of S^T = K Q^T: lane (row, hh), k-step s: 32 bytes
    // at d = 64 s + 32 hh
    uint4 qf[2][2];
    if (row < qend) {
        const uint8_t* src = qp + (int64_t)row * a.q_sS + 32 * hh;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                uint4 v = *(const uint4*)(src + 64 * s + 16 * e);
                v.x ^= qflip; v.y ^= qflip; v.z ^= qflip; v.w ^= qflip;
                qf[s][e] = v;
            }
    } else {
#pragma unroll
        for (int s = 0; s < 2; ++s) qf[s][0] = qf[s][1] = make_uint4(0, 0, 0, 0);
    }

    // 64 entries of the block list (and their kv scales) in one register per
    // lane each; the window moves forward as in the 16-bit kernel
    int bsa_cb = 0, bsa_bc = 0;
    float ks_w = 0.f, vs_w = 0.f;
    auto reload = [&](int base) {
        bsa_cb = base;
        const int e = base + lane;
        const int kb = e < a.nkb ? blist[e] : -1;
        bsa_bc = kb < 0 ? 0 : kb;
        ks_w = kb >= 0 ? ksb[kb] : 0.f;
        vs_w = kb >= 0 ? vsb[kb] : 0.f;
    };
    if (ntiles > 0) reload(0);
    auto entry = [&](int it) -> int {      // window slot of tile it
        const int idx = it / per;
        if (idx >= bsa_cb + 64) reload(idx - 2);
        return idx - bsa_cb;
    };
    auto tile_c0 = [&](int it) -> int {
        const int sl = entry(it);
        return __builtin_amdgcn_readlane(bsa_bc, sl) * a.by + BN * (it % per);
    };

    // K: row r, 16-byte chunk c at position c ^ ((r >> 1) & 7) (the 16 rows of
    // a quarter-wave operand read hit 16 distinct bank groups); V bytes: plain
    // rows.  Instruction u of wave w fills slots 64 (NW u + w) + lane.
    uint32_t koff[2], voff[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int sl = 64 * (NW * u + w) + lane;
        const int r = sl >> 3, pos = sl & 7;
        koff[u] = (uint32_t)(r * a.k_sS + 16 * (pos ^ ((r >> 1) & 7)));
        voff[u] = (uint32_t)(r * a.v_sS + 16 * pos);
    }
    auto load_tile = [&](int c0, int st) {
        const uint32_t kb = smem_lds + (uint32_t)(st * STAGE);
        const i32x4 kr = rows_rsrc8(kp, c0, Lkv, a.k_sS, D);
        const i32x4 vr = rows_rsrc8(vp, c0, Lkv, a.v_sS, D);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            dma16(kr, kb + 1024u * (NW * u + w), koff[u]);
            dma16(vr, kb + K8 + 1024u * (NW * u + w), voff[u]);
        }
    };
    // widen the V bytes this lane's loads brought into the bf16 tile
    auto widen = [&](int st) {
        uint8_t* base = smem8 + st * STAGE;
        uint16_t* vbf = (uint16_t*)(smem8 + VBF);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int sl = 64 * (NW * u + w) + lane;
            const int r = sl >> 3, cc = sl & 7;
            const uint4 raw = *(const uint4*)(base + K8 + 16 * sl);
            const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
            uint32_t pk[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pk[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w4[e], 1.0f, false));
                pk[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w4[e], 1.0f, true));
            }
            const int sw = 4 * (r & 3);
            *(uint4*)(vbf + r * D + 8 * ((2 * cc) ^ sw)) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
            *(uint4*)(vbf + r * D + 8 * ((2 * cc + 1) ^ sw)) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
        }
    };

    // per-lane LDS offsets of the operand reads (as in the 16-bit kernel for V)
    const int kx = (l32 >> 1) & 7;          // same for rows l32 and 32 + l32
    const int vi = lane & 15;
    const int vrow = 4 * hh + (vi >> 2);
    const int vswz = 4 * (vi >> 2);
    const int vcol_lo = 2 * ((lane >> 4) & 1) + ((vi & 3) >> 1);
    const int vsub = 4 * (vi & 1);

    f32x16 acc[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[o][r] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float lazy_real = kLazy / c;      // in score units

    if (ntiles > 0) {
        load_tile(tile_c0(0), 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        widen(0);
    }
    for (int it = 0; it < ntiles; ++it) {
        const int st = it & 1;
        __syncthreads();                   // tile it (K bytes, widened V) ready; stage st ^ 1 free
        if (it + 1 < ntiles) load_tile(tile_c0(it + 1), st ^ 1);
        const int sl = entry(it);
        const int c0 = __builtin_amdgcn_readlane(bsa_bc, sl) * a.by + BN * (it % per);
        const float f = qs * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ks_w), sl));
        const float vsc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vs_w), sl));

        if (wend > wr0) {
            const uint8_t* kt = smem8 + st * STAGE;
            const uint16_t* vs = (const uint16_t*)(smem8 + VBF);
            f32x16 s0, s1;
#pragma unroll
            for (int r = 0; r < 16; ++r) s0[r] = s1[r] = 0.f;
            // raised wave priority over the two matrix phases: the wave in a
            // matrix phase wins issue over the other waves' softmax (1 %
            // faster at three workgroups per CU)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int ch = 4 * s + 2 * hh;
                const uint8_t* r0p = kt + l32 * D;
                const uint8_t* r1p = kt + (32 + l32) * D;
                const uint4 a00 = *(const uint4*)(r0p + 16 * (ch ^ kx));
                const uint4 a01 = *(const uint4*)(r0p + 16 * ((ch + 1) ^ kx));
                const uint4 a10 = *(const uint4*)(r1p + 16 * (ch ^ kx));
                const uint4 a11 = *(const uint4*)(r1p + 16 * ((ch + 1) ^ kx));
                const i32x8 bq = {(int)qf[s][0].x, (int)qf[s][0].y, (int)qf[s][0].z, (int)qf[s][0].w,
                                  (int)qf[s][1].x, (int)qf[s][1].y, (int)qf[s][1].z, (int)qf[s][1].w};
                const i32x8 ka0 = {(int)a00.x, (int)a00.y, (int)a00.z, (int)a00.w,
                                   (int)a01.x, (int)a01.y, (int)a01.z, (int)a01.w};
                const i32x8 ka1 = {(int)a10.x, (int)a10.y, (int)a10.z, (int)a10.w,
                                   (int)a11.x, (int)a11.y, (int)a11.z, (int)a11.w};
                s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka0, bq, s0, 0, 0, 0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka1, bq, s1, 0, 0, 0, 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
            // scores in dequantized units: raw * f.  For f > 0 (dequant scales
            // are positive factors) the factor rides in the exp2 FMA below and
            // the row max is taken on the raw scores; otherwise it is applied
            // here.
            const bool fpos = f > 0.f;
            if (!fpos) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s0[r] *= f;
                    s1[r] *= f;
                }
            }
            const float fm = fpos ? f : 1.f;
            // keys past the length and rows past the query length
            if (c0 + BN > Lkv || wend - wr0 < 32) {
                const int base = c0 + 4 * hh;
                const int jhi = row >= qend ? -1 : Lkv - 1 - base;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int k0 = 8 * (r >> 2) + (r & 3), k1 = 32 + k0;
                    if (k0 > jhi) s0[r] = -INFINITY;
                    if (k1 > jhi) s1[r] = -INFINITY;
                }
            }
            float mq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                mq[q] = vmax(s0[4 * q], vmax(s0[4 * q + 1], s1[4 * q]));
                mq[q] = vmax(mq[q], vmax(s0[4 * q + 2], s1[4 * q + 1]));
                mq[q] = vmax(mq[q], vmax(s0[4 * q + 3], s1[4 * q + 2]));
                mq[q] = vmax(mq[q], s1[4 * q + 3]);
            }
            float mt = vmax(vmax(mq[0], vmax(mq[1], mq[2])), mq[3]);
            mt = other_half_max(mt) * fm;   // -inf stays -inf (fm > 0)
            const float mn = fmaxf(m, mt);
            const bool grow = (m == -INFINITY) ? (mn > -INFINITY) : (mn > m + lazy_real);
            if (__ballot(grow)) {
                float alpha = 1.f;
                if (m == -INFINITY) alpha = 0.f;
                else if (mn != -INFINITY) alpha = fast_exp2((m - mn) * c);
                m = mn;
                l *= alpha;
#pragma unroll
                for (int o = 0; o < NO; ++o)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[o][r] *= alpha;
            }
            // p = exp2(raw f c - m c); the P fed to the P V MFMAs also carries
            // the tile's value scale: exp2(... + log2 vs) when vs > 0
            const bool vpos = vsc > 0.f;
            const float mc = (m == -INFINITY) ? 0.f : m * c;
            const float cf = c * fm;
            const float lv = vpos ? __log2f(vsc) : 0.f;
            const float pm = vpos ? 1.f : vsc;  // P multiplier left for the pack
            const float ls = vpos ? 1.f / vsc : 1.f;
            float ps = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s0[r] = fast_exp2(__builtin_fmaf(s0[r], cf, lv - mc));
                s1[r] = fast_exp2(__builtin_fmaf(s1[r], cf, lv - mc));
                ps += s0[r] + s1[r];
            }
            l += ps * ls;
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const f32x16& src = (k < 2) ? s0 : s1;
                const int b8 = 8 * (k & 1);
                uint4 pb;
                if (vpos) {
                    pb.x = O::pack2(src[b8 + 0], src[b8 + 1]);
                    pb.y = O::pack2(src[b8 + 2], src[b8 + 3]);
                    pb.z = O::pack2(src[b8 + 4], src[b8 + 5]);
                    pb.w = O::pack2(src[b8 + 6], src[b8 + 7]);
                } else {
                    pb.x = O::pack2(src[b8 + 0] * pm, src[b8 + 1] * pm);
                    pb.y = O::pack2(src[b8 + 2] * pm, src[b8 + 3] * pm);
                    pb.z = O::pack2(src[b8 + 4] * pm, src[b8 + 5] * pm);
                    pb.w = O::pack2(src[b8 + 6] * pm, src[b8 + 7] * pm);
                }
                const uint16_t* vk = vs + (16 * k + vrow) * D + vsub;
#pragma unroll
                for (int o = 0; o < NO; ++o) {
                    const int pc = (4 * o + vcol_lo) ^ vswz;
                    const uint2 lo = lds_read_tr16(vk + 8 * pc);
                    const uint2 hi = lds_read_tr16(vk + 8 * D + 8 * pc);
                    acc[o] = O::mma32(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, acc[o]);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
        if (it + 1 < ntiles) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();               // every wave is done with the bf16 V tile
            widen(st ^ 1);
        }
    }

    // epilogue: rows < q1 are written; rows in [qend, q1) and rows with no
    // allowed key get out = 0 and lse = +inf
    const float lt = other_half_sum(l);
    if (row < q1) {
        const bool valid = row < qend && lt > 0.f;
        const float inv = valid ? 1.f / lt : 0.f;
        uint16_t* op = (uint16_t*)a.o + bi.q_row0 * a.o_rowmul + (int64_t)h * a.o_sH + (int64_t)row * a.o_sS;
#pragma unroll
        for (int o = 0; o < NO; ++o)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                uint2 v;
                v.x = O::pack2(acc[o][4 * g4 + 0] * inv, acc[o][4 * g4 + 1] * inv);
                v.y = O::pack2(acc[o][4 * g4 + 2] * inv, acc[o][4 * g4 + 3] * inv);
                *(uint2*)(op + 32 * o + 8 * g4 + 4 * hh) = v;
            }
        if (a.return_lse && hh == 0) {
            float* lp = a.lse + bi.q_row0 * a.lse_rowmul + (int64_t)h * a.lse_sH + (int64_t)row * a.lse_sS;
            *lp = valid ? (m * c + __log2f(lt)) * kLn2 : INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// Decode: split-KV attention over (optionally paged) K/V.
//
// One wave per resident slot; it walks its pieces, each a token range of one
// segment (batch b, kv head, chunk of <= 16 query heads of its GQA group),
// and writes one partial result per piece.  Per step of 32 tokens (two 16-token sub-tiles;
// a sub-tile never crosses a page because block_size % 16 == 0):
//   S^T (32 tokens x 16 heads) = K Q^T on v_mfma_f32_16x16x32: K comes
//       straight from HBM into the A operand (each lane one token row, four
//       16-byte chunks), the query heads are the 16 B-operand columns, so a
//       K/V byte is read once for the whole GQA group;
//   V rows stream direct-to-LDS and feed O^T += V^T P^T through transposed
//       LDS reads; P stays in registers.
// Page / offset of each sub-tile are tracked as wave-uniform scalars, so the
// per-lane address work is one multiply-add per sub-tile.  The next step's
// K registers and V rows are in flight while the current step computes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float quad_max(float x)
{
    // max over lanes l, l^16, l^32, l^48 (the four quarters of the wave)
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    return other_half_max(x);
}
__device__ __forceinline__ float quad_sum(float x)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    return other_half_sum(x);
}


template <int DT, int D, bool MASK>
__global__ __launch_bounds__(64) void decode_split(DecodeArgs a)
{
    constexpr int ST = kDecodeStep;       // 32 tokens per step
    constexpr int NK = D / 32;            // k-steps of S^T = K Q^T
    constexpr int NO = D / 16;            // 16-row d tiles of O^T
    constexpr int VCH = D / 8;            // 16-byte chunks per V row
    constexpr int RPI = 64 / VCH;         // V rows per DMA instruction
    constexpr int NVI = 16 / RPI;         // DMA instructions per sub-tile
    using O = Ops<DT>;
    __shared__ __attribute__((aligned(16))) uint16_t vbuf0[ST * D];
    __shared__ __attribute__((aligned(16))) uint16_t vbuf1[ST * D];

    const int lane = threadIdx.x;
    const int n = lane & 15, qd = lane >> 4;
    const int wv = blockIdx.x;
    const int p_end = a.wave_first[wv + 1];
    for (int item = a.wave_first[wv]; item < p_end; ++item) {
        const DecPiece pc_ = a.pieces[item];
        const DecSeg db = a.segs[pc_.seg];
        const int b = db.b;
        const int hc = pc_.seg % a.nhc;
        const int kvh = (pc_.seg / a.nhc) % a.KVN;
        const int t0 = pc_.t0;
        const int t1 = pc_.t1;
        // column n is query row r = 16 hc + n of the kv head: head r / S of
        // the GQA group, query token r % S
        const int S = a.S;
        const int r0 = kDecodeHeads * hc;
        const int nh = min(kDecodeHeads, a.G * S - r0);
        const int rq = r0 + n;
        const int tq = rq % S;
        const int hq = kvh * a.G + rq / S;
        const float c = fmaxf(fabsf(a.scale_log2), kMinScale);
        const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
        // sparse_mode 3 (S > 1): token tq sees keys j <= Lkv - Lq + tq; jmin is
        // the smallest such bound over the chunk's columns (wave-uniform), so
        // only the steps that reach past it evaluate the per-column bound
        const int jbase = db.lkv - db.lq;
        const int tq_min = (r0 % S) + nh > S ? 0 : r0 % S;
        const int jmax = a.causal ? jbase + tq : INT32_MAX;
        const int jmin = a.causal ? jbase + tq_min : INT32_MAX;

        // Q^T as the B operand: column n = (head hq, token tq), d = 32s + 8qd.
        uint4 qf[NK];
        if (n < nh) {
            const uint16_t* src = (const uint16_t*)a.q + (int64_t)b * a.q_sB + (int64_t)hq * a.q_sH +
                                  (int64_t)tq * a.q_sS + 8 * qd;
#pragma unroll
            for (int s = 0; s < NK; ++s) {
                uint4 v = *(const uint4*)(src + 32 * s);
                v.x ^= qflip; v.y ^= qflip; v.z ^= qflip; v.w ^= qflip;
                qf[s] = v;
            }
        } else {
#pragma unroll
            for (int s = 0; s < NK; ++s) qf[s] = make_uint4(0, 0, 0, 0);
        }

        // Sub-tile addressing: the page (block) and the token offset inside it.
        const int bs = a.paged ? a.block_size : 0x40000000;
        const int32_t* bt = a.paged ? a.block_table + (int64_t)b * a.bt_stride : nullptr;
        const int64_t tokstride = a.paged ? a.p_tok : a.c_tok;
        const uint16_t* kbase = (const uint16_t*)a.k;
        const uint16_t* vbase = (const uint16_t*)a.v;
        const int64_t hoff = a.paged ? (int64_t)kvh * a.p_head
                                     : db.kv_row0 * a.c_rowmul + (int64_t)kvh * a.c_head;
        // The piece's block-table entries (at most 64 pages; the planner caps
        // piece lengths): lane i holds the id of page pg_first + i, so a
        // sub-tile's page id comes from v_readlane without a memory access.
        const int pg_first = t0 / bs;
        const int pg_last = t1 > t0 ? (t1 - 1) / bs : pg_first;
        const int my_page = (a.paged && pg_first + lane <= pg_last) ? bt[pg_first + lane] : 0;
        // settle the table load here: a wait for it inside the step loop
        // would also drain the prefetch in flight
        __builtin_amdgcn_s_waitcnt(FIA_VMCNT(0));
        auto sub_rsrc = [&](const uint16_t* base, int pg, int off, int tb) {
            // rows [off, off + nvalid) of page pg; rows past t1 read as zero
            const int nvalid = min(16, t1 - tb);
            // a sub-tile past the end reads nothing, not even its table entry
            const int64_t pbase =
                (a.paged && nvalid > 0) ? (int64_t)__builtin_amdgcn_readlane(my_page, pg - pg_first) * a.p_blk : 0;
            const int64_t bytes = nvalid > 0 ? ((int64_t)(nvalid - 1) * tokstride + D) * 2 : 0;
            return __builtin_amdgcn_make_buffer_rsrc((void*)(base + pbase + hoff + (int64_t)off * tokstride),
                                                         (short)0, (int)min(bytes, (int64_t)0x7fffffff),
                                                         0x00020000);
        };

        // K rows into registers: lane (token n, quarter qd) reads d = 32s + 8qd.
        const uint32_t k_voff = (uint32_t)((n * tokstride + 8 * qd) * 2);
        // V rows via DMA: instruction u of sub-tile c fills rows 16c + RPI u + lane / VCH.
        const int vr_in = lane / VCH, vpc = lane % VCH;
        auto vswz = [](int r) { return VCH >= 16 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); };

        // atten_mask (query S == 1): lane l (and l + 32) loads the byte of
        // token tt0 + l of each step, issued with the step's K/V loads; the
        // step turns the 32 bytes into one wave-uniform bit mask by a ballot.
        const uint8_t* mrow = MASK ? a.mask + (int64_t)b * a.mask_bstride : nullptr;
        const int l32 = lane & 31;
        auto issue = [&](int tt0, int pg0, int off0, int pg1, int off1, uint4 (&kf)[2][NK], uint16_t* vb,
                         uint32_t& mbyte) {
            if constexpr (MASK) mbyte = tt0 + l32 < t1 ? mrow[tt0 + l32] : 0u;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int pg = cc ? pg1 : pg0, off = cc ? off1 : off0, tb = tt0 + 16 * cc;
                const __amdgpu_buffer_rsrc_t kr = sub_rsrc(kbase, pg, off, tb);
#pragma unroll
                for (int s = 0; s < NK; ++s)
                    kf[cc][s] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, k_voff + 64 * s, 0, kStream));
                const __amdgpu_buffer_rsrc_t vr = sub_rsrc(vbase, pg, off, tb);
#pragma unroll
                for (int u = 0; u < NVI; ++u) {
                    const int r = RPI * u + vr_in;                 // row inside the sub-tile
                    const int R = 16 * cc + r;                     // row inside the step
                    const int chunk = vpc ^ vswz(R);
                    dma16_tracked<kStream>(vr, vb + (16 * cc + RPI * u) * D, (uint32_t)((r * tokstride + 8 * chunk) * 2));
                }
            }
        };

        // V^T A operand: lane (d = 16 dt + (lane & 15), quarter qd) needs tokens
        // 4 qd + 0..3 and 16 + 4 qd + 0..3; each group of 16 lanes reads its 4-row
        // block with one transposed read (row 4 qd + vi / 4, columns 4 (vi % 4)).
        const int vi = lane & 15;
        const int trow = 4 * qd + (vi >> 2);
        const int tsw = vswz(trow);                          // same for trow + 16
        const int tcol_lo = (vi & 3) >> 1, tsub = 4 * (vi & 1);

        f32x4 acc[NO];
#pragma unroll
        for (int o = 0; o < NO; ++o) acc[o] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY, l = 0.f;
        const float lazy_raw = kLazy / c;

        const int nsteps = (t1 - t0 + ST - 1) / ST;
        int pg = t0 / bs, off = t0 % bs;
        auto advance16 = [&](int& p, int& o) {
            o += 16;
            if (o >= bs) { o -= bs; ++p; }
        };

        uint4 kfa[2][NK], kfb[2][NK];
        uint32_t mba = 0, mbb = 0;
        auto step = [&](int st, uint4 (&kcur)[2][NK], uint4 (&knext)[2][NK], uint16_t* vcur, uint16_t* vnext,
                        uint32_t mcur, uint32_t& mnext) {
            const int tt0 = t0 + ST * st;
            // pg/off point at the first sub-tile of step st + 1 here
            if (st + 1 < nsteps) {
                int pg1 = pg, off1 = off;
                advance16(pg1, off1);
                __builtin_amdgcn_s_waitcnt(FIA_LGKMCNT0);   // reads of the other V buffer done
                issue(tt0 + ST, pg, off, pg1, off1, knext, vnext, mnext);
                pg = pg1; off = off1;
                advance16(pg, off);
                // step st landed (step st + 1's loads, mask byte first, stay in flight)
                __builtin_amdgcn_s_waitcnt(FIA_VMCNT(2 * (NK + NVI) + (MASK ? 1 : 0)));
            } else {
                __builtin_amdgcn_s_waitcnt(FIA_VMCNT(0));
            }
            __syncthreads();

            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NK; ++s) {
                s0 = O::mma16(kcur[0][s], qf[s], s0);
                s1 = O::mma16(kcur[1][s], qf[s], s1);
            }
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = s0[i];
                x[4 + i] = s1[i];
            }
            if (tt0 + ST > t1 || tt0 + ST - 1 > jmin) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int tk = tt0 + 16 * (r >> 2) + 4 * qd + (r & 3);
                    if (tk >= t1 || tk > jmax) x[r] = -INFINITY;
                }
            }
            if constexpr (MASK) {
                // bit i: token tt0 + i is masked
                const uint32_t mm = (uint32_t)__ballot(mcur != 0u);
                if (mm) {
#pragma unroll
                    for (int r = 0; r < 8; ++r)
                        if ((mm >> (16 * (r >> 2) + 4 * qd + (r & 3))) & 1u) x[r] = -INFINITY;
                }
            }
            float mt = x[0];
#pragma unroll
            for (int r = 1; r < 8; ++r) mt = fmaxf(mt, x[r]);
            mt = quad_max(mt);
            const float mn = fmaxf(m, mt);
            const bool grow = (m == -INFINITY) ? (mn > -INFINITY) : (mn > m + lazy_raw);
            if (__ballot(grow)) {
                float alpha = 1.f;
                if (m == -INFINITY) alpha = 0.f;
                else if (mn != -INFINITY) alpha = fast_exp2((m - mn) * c);
                m = mn;
                l *= alpha;
#pragma unroll
                for (int o = 0; o < NO; ++o) acc[o] *= alpha;
            }
            const float mc = (m == -INFINITY) ? 0.f : m * c;
            float ps = 0.f;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                x[r] = fast_exp2(__builtin_fmaf(x[r], c, -mc));
                ps += x[r];
            }
            l += ps;
            uint4 pb;
            pb.x = O::pack2(x[0], x[1]);
            pb.y = O::pack2(x[2], x[3]);
            pb.z = O::pack2(x[4], x[5]);
            pb.w = O::pack2(x[6], x[7]);
            const uint16_t* vb = vcur;
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                const int pc = (2 * o + tcol_lo) ^ tsw;
                const uint2 lo = lds_read_tr16(vb + trow * D + 8 * pc + tsub);
                const uint2 hi = lds_read_tr16(vb + (trow + 16) * D + 8 * pc + tsub);
                acc[o] = O::mma16(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, acc[o]);
            }
        };

        if (nsteps > 0) {
            int pg1 = pg, off1 = off;
            advance16(pg1, off1);
            issue(t0, pg, off, pg1, off1, kfa, vbuf0, mba);
            pg = pg1; off = off1;
            advance16(pg, off);
        }
        for (int st = 0; st < nsteps; st += 2) {
            step(st, kfa, kfb, vbuf0, vbuf1, mba, mbb);
            if (st + 1 < nsteps) step(st + 1, kfb, kfa, vbuf1, vbuf0, mbb, mba);
        }

        // partial: normalised O and natural-log LSE of this split
        const float lt = quad_sum(l);
        if (n < nh) {
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            float* po = a.part_o + ((int64_t)item * a.Gc + n) * D;
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                f32x4 v = acc[o] * inv;
                *(f32x4*)(po + 16 * o + 4 * qd) = v;
            }
            if (qd == 0)
                a.part_lse[(int64_t)item * a.Gc + n] = lt > 0.f ? (m * c + __log2f(lt)) * kLn2 : -INFINITY;
        }
        __syncthreads();     // the LDS buffers are reused by the next piece
    }
}

// ---------------------------------------------------------------------------
// Decode against an int8 KV cache (kv pseudo-quantization), contiguous or
// (query S 1) paged through the block table.  A cached value x stands
// for scale * (x + offset), per channel (bf16 scale/offset [KV_N * D]) or per
// token (fp32 [B, KV_S]), K and V each with their own mode.  K bytes are read
// as u = x + 128 (0..255, exact in bf16) for the bf16 QK MFMAs; V bytes as the
// signed x (exact in fp16) for fp16 P V MFMAs, whose 11-bit P rounding keeps
// the output error below that of the 16-bit path.  Each affine part goes
// where it is cheapest:
//   K per channel: s_j = sum_d q'_d u_jd + C, q'_d = q_d sk_d held as two bf16
//                  parts hi + lo (two MFMAs per k-step, so q' keeps ~16 bits),
//                  C = sum_d q'_d (ok_d - 128) per column;
//   K per token:   s_j = sk_j (sum_d q_d u_jd + (ok_j - 128) sum_d q_d);
//   V per token:   p_j sv_j feeds the P V MFMA and T = sum_j p_j sv_j ov_j per
//                  column; partial O = (P' X + T) / l;
//   V per channel: partial O = P X / l in raw units; the combine writes
//                  sv_d (O_d + ov_d).
// K comes straight into registers (lane (token n, quarter qd) holds the
// contiguous d range [KB qd, KB qd + KB) of its row; Q uses the same d order);
// V rows go direct-to-LDS as bytes and are widened to fp16 into the swizzled
// 16-bit layout the transposed reads of the 16-bit decode kernel use.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

template <int D, int KM, int VM>
__global__ __launch_bounds__(64, 2) void decode_split_i8(DecodeArgs a)
{
    constexpr int ST = kDecodeStep;       // 32 tokens per step
    constexpr int NK = D / 32;            // k-steps of S^T = K Q^T
    constexpr int NO = D / 16;            // 16-row d tiles of O^T
    constexpr int VCH = D / 8;            // 16-byte bf16 chunks per V row
    constexpr int KB = NK * 8;            // K bytes per lane and token row
    constexpr int NKL = KB / 16;          // 16-byte K loads per lane and sub-tile
    constexpr int VCH8 = D / 16;          // 16-byte int8 chunks per V row
    constexpr int RPI8 = 64 / VCH8;       // V rows per DMA instruction
    constexpr int NVI8 = 16 / RPI8;       // DMA instructions per sub-tile
    constexpr int NCV = ST * VCH8 / 64;   // int8 chunks each lane widens per step
    static_assert(NKL >= 1 && NKL * 16 == KB && NVI8 >= 1 && NCV >= 1, "shape");
    using O = Ops<FIA_BF16>;                 // Q K^T
    using OV = Ops<FIA_F16>;                 // P V
    __shared__ __attribute__((aligned(16))) uint16_t vbuf[ST * D];   // widened x (fp16), swizzled
    __shared__ __attribute__((aligned(16))) uint8_t vst0[ST * D];    // bytes as loaded (three steps)
    __shared__ __attribute__((aligned(16))) uint8_t vst1[ST * D];
    __shared__ __attribute__((aligned(16))) uint8_t vst2[ST * D];

    const int lane = threadIdx.x;
    const int n = lane & 15, qd = lane >> 4;
    const int wv = blockIdx.x;
    const int p_end = a.wave_first[wv + 1];
    auto vswz = [](int r) { return VCH >= 16 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); };
    for (int item = a.wave_first[wv]; item < p_end; ++item) {
        const DecPiece pc_ = a.pieces[item];
        const DecSeg db = a.segs[pc_.seg];
        const int b = db.b;
        const int hc = pc_.seg % a.nhc;
        const int kvh = (pc_.seg / a.nhc) % a.KVN;
        const int t0 = pc_.t0;
        const int t1 = pc_.t1;
        const int S = a.S;
        const int r0 = kDecodeHeads * hc;
        const int nh = min(kDecodeHeads, a.G * S - r0);
        const int rq = r0 + n;
        const int tq = rq % S;
        const int hq = kvh * a.G + rq / S;
        const float c = fmaxf(fabsf(a.scale_log2), kMinScale);
        const float qsign = a.scale_log2 < 0.f ? -1.f : 1.f;
        const int jbase = db.lkv - db.lq;
        const int tq_min = (r0 % S) + nh > S ? 0 : r0 % S;
        const int jmax = a.causal ? jbase + tq : INT32_MAX;
        const int jmin = a.causal ? jbase + tq_min : INT32_MAX;

        // Q^T as the B operand: column n, k-step s covers d = KB qd + 8 s + (0..7)
        uint4 qf[NK], ql[NK];             // ql: low part of q' (K per channel)
        float cpart = 0.f, qpart = 0.f;
        if (n < nh) {
            const uint16_t* src = (const uint16_t*)a.q + (int64_t)b * a.q_sB + (int64_t)hq * a.q_sH +
                                  (int64_t)tq * a.q_sS + KB * qd;
            const int64_t ch0 = (int64_t)kvh * D + KB * qd;
#pragma unroll
            for (int s = 0; s < NK; ++s) {
                const uint4 v = *(const uint4*)(src + 8 * s);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                float qv[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    qv[2 * e] = qsign * bf16_to_f32(w4[e] & 0xffffu);
                    qv[2 * e + 1] = qsign * bf16_to_f32(w4[e] >> 16);
                }
                if constexpr (KM == 0) {
                    const uint4 sv = *(const uint4*)((const uint16_t*)a.k_scale + ch0 + 8 * s);
                    const uint4 ov = a.k_off ? *(const uint4*)((const uint16_t*)a.k_off + ch0 + 8 * s)
                                             : make_uint4(0, 0, 0, 0);
                    const uint32_t s4[4] = {sv.x, sv.y, sv.z, sv.w};
                    const uint32_t o4[4] = {ov.x, ov.y, ov.z, ov.w};
                    uint32_t pk[4], pl[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x0 = qv[2 * e] * bf16_to_f32(s4[e] & 0xffffu);
                        const float x1 = qv[2 * e + 1] * bf16_to_f32(s4[e] >> 16);
                        pk[e] = O::pack2(x0, x1);
                        const float h0 = bf16_to_f32(pk[e] & 0xffffu), h1 = bf16_to_f32(pk[e] >> 16);
                        pl[e] = O::pack2(x0 - h0, x1 - h1);
                        // C uses the q' = hi + lo that the MFMAs see
                        const float y0 = h0 + bf16_to_f32(pl[e] & 0xffffu);
                        const float y1 = h1 + bf16_to_f32(pl[e] >> 16);
                        cpart += y0 * (bf16_to_f32(o4[e] & 0xffffu) - 128.f);
                        cpart += y1 * (bf16_to_f32(o4[e] >> 16) - 128.f);
                    }
                    qf[s] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
                    ql[s] = make_uint4(pl[0], pl[1], pl[2], pl[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) qpart += qv[e];
                    uint32_t pk[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) pk[e] = O::pack2(qv[2 * e], qv[2 * e + 1]);
                    qf[s] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < NK; ++s) qf[s] = ql[s] = make_uint4(0, 0, 0, 0);
        }
        const float Cn = quad_sum(cpart);     // K per channel: constant of column n
        const float Qs = quad_sum(qpart);     // K per token: sum_d q_d of column n

        // Contiguous cache, or a paged pool (int8 elements are bytes, so the
        // pool strides are byte strides); a 16-token sub-tile never crosses a
        // page (block_size % 32 == 0, pieces 16-aligned).
        const int64_t tokstride = a.paged ? a.p_tok : a.c_tok;
        const int64_t hoff = a.paged ? (int64_t)kvh * a.p_head
                                     : db.kv_row0 * a.c_rowmul + (int64_t)kvh * a.c_head;
        const uint8_t* kbase = (const uint8_t*)a.k + hoff;
        const uint8_t* vbase = (const uint8_t*)a.v + hoff;
        // the piece's block-table entries (at most 64 pages): lane i holds the
        // id of page pg_first + i; a sub-tile takes its page id by v_readlane
        const int bs = a.paged ? a.block_size : 0x40000000;
        const int32_t* bt = a.paged ? a.block_table + (int64_t)b * a.bt_stride : nullptr;
        const int pg_first = t0 / bs;
        const int pg_last = t1 > t0 ? (t1 - 1) / bs : pg_first;
        const int my_page = (a.paged && pg_first + lane <= pg_last) ? bt[pg_first + lane] : 0;
        // settle the table load here, not inside the prefetching step loop
        __builtin_amdgcn_s_waitcnt(FIA_VMCNT(0));
        // rows [tb, t1) (at most 16) of the piece, which start at row off of
        // page pg (pg 0 and off = tb for a contiguous cache); rows past t1
        // read as zero
        auto sub_rsrc = [&](const uint8_t* base, int pg, int off, int tb) {
            const int nvalid = min(16, t1 - tb);
            // a sub-tile past the end reads nothing, not even its table entry
            const int64_t pbase =
                (a.paged && nvalid > 0) ? (int64_t)__builtin_amdgcn_readlane(my_page, pg - pg_first) * a.p_blk : 0;
            const int64_t bytes = nvalid > 0 ? (int64_t)(nvalid - 1) * tokstride + D : 0;
            return __builtin_amdgcn_make_buffer_rsrc((void*)(base + pbase + (int64_t)off * tokstride), (short)0,
                                                     (int)min(bytes, (int64_t)0x7fffffff), 0x00020000);
        };
        const float* ksrow = KM == 1 ? (const float*)a.k_scale + (int64_t)b * a.tok_stride : nullptr;
        const float* korow = KM == 1 && a.k_off ? (const float*)a.k_off + (int64_t)b * a.tok_stride : nullptr;
        const float* vsrow = VM == 1 ? (const float*)a.v_scale + (int64_t)b * a.tok_stride : nullptr;
        const float* vorow = VM == 1 && a.v_off ? (const float*)a.v_off + (int64_t)b * a.tok_stride : nullptr;
        // per-token values of the lane's 8 tokens of a step (0 past t1)
        auto tok8 = [&](const float* row, int tt0, float (&out)[8]) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int tk = tt0 + 16 * (r >> 2) + 4 * qd + (r & 3);
                out[r] = (row && tk < t1) ? row[tk] : 0.f;
            }
        };

        const uint32_t k_voff = (uint32_t)(n * tokstride + KB * qd);
        const int vr_in = lane / VCH8, vpc = lane % VCH8;
        struct Tok { float ks[8], ko[8], vs[8], vo[8]; };
        auto issue = [&](int tt0, int pg0, int off0, int pg1, int off1, uint4 (&kf)[2][NKL], uint8_t* vb, Tok& tk) {
            if constexpr (KM == 1) { tok8(ksrow, tt0, tk.ks); tok8(korow, tt0, tk.ko); }
            if constexpr (VM == 1) { tok8(vsrow, tt0, tk.vs); tok8(vorow, tt0, tk.vo); }
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int tb = tt0 + 16 * cc;
                const int pg = cc ? pg1 : pg0, off = cc ? off1 : off0;
                const __amdgpu_buffer_rsrc_t kr = sub_rsrc(kbase, pg, off, tb);
#pragma unroll
                for (int l = 0; l < NKL; ++l)
                    kf[cc][l] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, k_voff + 16 * l, 0, kStream));
                const __amdgpu_buffer_rsrc_t vr = sub_rsrc(vbase, pg, off, tb);
#pragma unroll
                for (int u = 0; u < NVI8; ++u) {
                    const int r = RPI8 * u + vr_in;
                    dma16_tracked<kStream>(vr, (uint16_t*)(vb + (16 * cc + RPI8 * u) * D), (uint32_t)(r * tokstride + 16 * vpc));
                }
            }
        };
        // bytes 8s .. 8s + 7 of the lane's K row part as 8 bf16 values u = x + 128
        auto kop = [&](const uint4 (&raw)[NKL], int s) -> uint4 {
            const uint4 q4 = raw[s / 2];
            uint32_t w0 = (s & 1) ? q4.z : q4.x, w1 = (s & 1) ? q4.w : q4.y;
            w0 ^= 0x80808080u;
            w1 ^= 0x80808080u;
            uint4 o;
            o.x = O::pack2((float)(w0 & 0xffu), (float)((w0 >> 8) & 0xffu));
            o.y = O::pack2((float)((w0 >> 16) & 0xffu), (float)(w0 >> 24));
            o.z = O::pack2((float)(w1 & 0xffu), (float)((w1 >> 8) & 0xffu));
            o.w = O::pack2((float)((w1 >> 16) & 0xffu), (float)(w1 >> 24));
            return o;
        };

        // V^T A operand reads (as in the 16-bit kernel)
        const int vi = lane & 15;
        const int trow = 4 * qd + (vi >> 2);
        const int tsw = vswz(trow);
        const int tcol_lo = (vi & 3) >> 1, tsub = 4 * (vi & 1);

        f32x4 acc[NO];
#pragma unroll
        for (int o = 0; o < NO; ++o) acc[o] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY, l = 0.f, tpart = 0.f;
        const float lazy_raw = kLazy / c;
        const int nsteps = (t1 - t0 + ST - 1) / ST;

        // page and row of the next sub-tile to issue (bs % 32 == 0 and
        // t0 % 16 == 0, so a 16-token sub-tile never crosses a page)
        int pg = t0 / bs, off = t0 % bs;
        auto advance16 = [&](int& p, int& o) {
            o += 16;
            if (o >= bs) { o -= bs; ++p; }
        };
        // AHEAD steps in flight (two, or one with per-token K values, whose
        // registers would not fit a third set): AHEAD + 1 K register sets and
        // byte buffers in rotation; step st issues step st + AHEAD into the
        // set step st - 1 used.
        constexpr int AHEAD = KM == 1 ? 1 : 2;
        uint4 kfa[2][NKL], kfb[2][NKL], kfc[2][NKL];
        Tok ta, tb_, tc;
        auto issue_next = [&](int tt0, uint4 (&kf)[2][NKL], uint8_t* vb, Tok& tk) {
            int pg1 = pg, off1 = off;
            advance16(pg1, off1);
            issue(tt0, pg, off, pg1, off1, kf, vb, tk);
            pg = pg1; off = off1;
            advance16(pg, off);
        };
        auto step = [&](int st, uint4 (&kcur)[2][NKL], uint4 (&knn)[2][NKL], uint8_t* vcur, uint8_t* vnn,
                        const Tok& tcur, Tok& tnn) {
            const int tt0 = t0 + ST * st;
            // pg/off point at the first sub-tile of step st + AHEAD here
            if (st + AHEAD < nsteps) {
                __builtin_amdgcn_s_waitcnt(FIA_LGKMCNT0);   // widening reads of step st - 1's bytes done
                issue_next(tt0 + AHEAD * ST, knn, vnn, tnn);
            }
            // step st landed; the K and V loads of the (at most AHEAD) later
            // steps stay in flight (per-token values are loaded before each
            // step's K and V, so with them this waits for some of those too)
            if (AHEAD == 2 && st + 2 < nsteps) __builtin_amdgcn_s_waitcnt(FIA_VMCNT(4 * (NKL + NVI8)));
            else if (st + 1 < nsteps) __builtin_amdgcn_s_waitcnt(FIA_VMCNT(2 * (NKL + NVI8)));
            else __builtin_amdgcn_s_waitcnt(FIA_VMCNT(0));
            __syncthreads();
            // widen this step's V bytes (signed) into the fp16 layout
#pragma unroll
            for (int i = 0; i < NCV; ++i) {
                const int e = lane + 64 * i;
                const int r = e / VCH8, c8 = e % VCH8;
                const uint4 raw = *(const uint4*)(vcur + r * D + 16 * c8);
                const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
                uint32_t pk[8];
                // x = u - 128 with u = x ^ 0x80: the fp16 bit pattern 0x6400 | u
                // is 1024 + u exactly, and one packed fp16 add of -1152 leaves x
                // (integers below 2048 are exact in fp16)
                const f16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const uint32_t u = w4[e4] ^ 0x80808080u;
                    // v_perm_b32 byte selectors: 0..3 take bytes of u (second
                    // source), 4 takes 0x64 (first source); result bytes high to
                    // low: 0x64, u1, 0x64, u0 (and u3, u2)
                    const uint32_t lo2 = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
                    const uint32_t hi2 = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
                    pk[2 * e4] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, lo2) + bias);
                    pk[2 * e4 + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, hi2) + bias);
                }
                *(uint4*)(vbuf + r * D + 8 * ((2 * c8) ^ vswz(r))) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
                *(uint4*)(vbuf + r * D + 8 * ((2 * c8 + 1) ^ vswz(r))) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
            }

            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NK; ++s) {
                const uint4 k0 = kop(kcur[0], s), k1 = kop(kcur[1], s);
                s0 = O::mma16(k0, qf[s], s0);
                s1 = O::mma16(k1, qf[s], s1);
                if constexpr (KM == 0) {
                    s0 = O::mma16(k0, ql[s], s0);
                    s1 = O::mma16(k1, ql[s], s1);
                }
            }
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = s0[i];
                x[4 + i] = s1[i];
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if constexpr (KM == 0) x[r] += Cn;
                else x[r] = tcur.ks[r] * (x[r] + (tcur.ko[r] - 128.f) * Qs);
            }
            if (tt0 + ST > t1 || tt0 + ST - 1 > jmin) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int tk = tt0 + 16 * (r >> 2) + 4 * qd + (r & 3);
                    if (tk >= t1 || tk > jmax) x[r] = -INFINITY;
                }
            }
            float mt = x[0];
#pragma unroll
            for (int r = 1; r < 8; ++r) mt = fmaxf(mt, x[r]);
            mt = quad_max(mt);
            const float mn = fmaxf(m, mt);
            const bool grow = (m == -INFINITY) ? (mn > -INFINITY) : (mn > m + lazy_raw);
            if (__ballot(grow)) {
                float alpha = 1.f;
                if (m == -INFINITY) alpha = 0.f;
                else if (mn != -INFINITY) alpha = fast_exp2((m - mn) * c);
                m = mn;
                l *= alpha;
                tpart *= alpha;
#pragma unroll
                for (int o = 0; o < NO; ++o) acc[o] *= alpha;
            }
            const float mc = (m == -INFINITY) ? 0.f : m * c;
            float ps = 0.f;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                x[r] = fast_exp2(__builtin_fmaf(x[r], c, -mc));
                ps += x[r];
                if constexpr (VM == 1) {
                    tpart += x[r] * tcur.vs[r] * tcur.vo[r];
                    x[r] *= tcur.vs[r];
                }
            }
            l += ps;
            uint4 pb;
            pb.x = OV::pack2(x[0], x[1]);
            pb.y = OV::pack2(x[2], x[3]);
            pb.z = OV::pack2(x[4], x[5]);
            pb.w = OV::pack2(x[6], x[7]);
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                const int pc = (2 * o + tcol_lo) ^ tsw;
                const uint2 lo = lds_read_tr16(vbuf + trow * D + 8 * pc + tsub);
                const uint2 hi = lds_read_tr16(vbuf + (trow + 16) * D + 8 * pc + tsub);
                acc[o] = OV::mma16(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, acc[o]);
            }
        };

        if (nsteps > 0) issue_next(t0, kfa, vst0, ta);
        if constexpr (AHEAD == 2) {
            if (nsteps > 1) issue_next(t0 + ST, kfb, vst1, tb_);
            for (int st = 0; st < nsteps; st += 3) {
                step(st, kfa, kfc, vst0, vst2, ta, tc);
                if (st + 1 < nsteps) step(st + 1, kfb, kfa, vst1, vst0, tb_, ta);
                if (st + 2 < nsteps) step(st + 2, kfc, kfb, vst2, vst1, tc, tb_);
            }
        } else {
            for (int st = 0; st < nsteps; st += 2) {
                step(st, kfa, kfb, vst0, vst1, ta, tb_);
                if (st + 1 < nsteps) step(st + 1, kfb, kfa, vst1, vst0, tb_, ta);
            }
        }

        const float lt = quad_sum(l);
        const float tt = quad_sum(tpart);
        if (n < nh) {
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            float* po = a.part_o + ((int64_t)item * a.Gc + n) * D;
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                f32x4 v = (acc[o] + tt) * inv;
                *(f32x4*)(po + 16 * o + 4 * qd) = v;
            }
            if (qd == 0)
                a.part_lse[(int64_t)item * a.Gc + n] = lt > 0.f ? (m * c + __log2f(lt)) * kLn2 : -INFINITY;
        }
        __syncthreads();     // the LDS buffers are reused by the next piece
    }
}

// ---------------------------------------------------------------------------
// MLA decode (query D 512 + rope 64, one kv head, paged K / V / K-rope pools).
//
// The Q_N x S (head, token) rows of a batch share every K/V byte, so a
// workgroup of NW (2..8) waves serves Gc <= 16 NW rows, wave w the 16
// columns 16 w .. 16 w + 15 of v_mfma_f32_16x16x32 (the decode kernel's
// layout):
//   S^T (32 tokens x 16 rows) = [K | K_rope] [Q | Q_rope]^T, 18 k-steps,
//       Q and Q_rope in registers (B operand), K rows read from LDS;
//   O^T (512 x 16) += V^T P^T, 32 tiles, V through transposed LDS reads.
// Per 32-token step the workgroup moves K (32 x 512) and K_rope (32 x 64)
// into one of two K slots and V (32 x 512) into one of two V slots, straight
// from the pools into LDS (K / V rows as 1 KB loads, K_rope rows as 4-byte
// loads so every wave issues the same number of loads).  The rings are
// decoupled so K runs two steps ahead: at the top of step st (after its K
// landed and every wave left P V of step st - 1) V of step st + 1 goes out;
// after S of step st (its V landed, every wave done with its K slot) K of
// step st + 2 goes out into that slot.  16-byte chunks are XOR-swizzled per
// row so the 16 rows a quarter-wave reads hit distinct banks.
// VK (value is the key tensor itself): V^T is read from the K slot, nothing
// else is loaded, and three K slots keep two steps in flight with one
// barrier per step.
// ---------------------------------------------------------------------------
constexpr int kMlaD = 512, kMlaDR = 64;
constexpr int kMlaKSlot = kDecodeStep * (kMlaD + kMlaDR);   // halves
constexpr int kMlaVSlot = kDecodeStep * kMlaD;
constexpr int kMlaLdsBytes = 2 * 2 * (kMlaKSlot + kMlaVSlot);
constexpr int kMlaLdsBytesVK = 3 * 2 * kMlaKSlot;

template <int DT, int NW, bool VK>
__global__ __launch_bounds__(NW * 64, 1) void mla_decode(DecodeArgs a)
{
    static_assert(NW == 2 || NW == 4 || NW == 8, "2, 4 or 8 waves");
    constexpr int D = kMlaD, DR = kMlaDR;
    constexpr int ST = kDecodeStep;                 // 32 tokens per step
    constexpr int NKM = D / 32, NKR = DR / 32;      // k-steps: latent, rope
    constexpr int NO = D / 16;                      // O^T tiles
    constexpr int NLK = ST / NW + 16 / NW;          // loads per wave: K + K_rope of a step
    constexpr int NLV = ST / NW;                    // V of a step
    constexpr int NSLOT = VK ? 3 : 2;               // K slots
    using O = Ops<DT>;
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_void*)smem;
    // byte addresses: K slots (K rows, then K_rope rows), then V slots
    auto kslot = [&](int st) { return smem_lds + 2u * (uint32_t)(kMlaKSlot * (st % NSLOT)); };
    auto vslot = [&](int st) { return smem_lds + 2u * (uint32_t)(2 * kMlaKSlot + kMlaVSlot * (st & 1)); };

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, qd = lane >> 4;
    const int R = a.G * a.S;                        // rows of the (single) kv head
    const int p_end = a.wave_first[blockIdx.x + 1];
    for (int item = a.wave_first[blockIdx.x]; item < p_end; ++item) {
        const DecPiece pc_ = a.pieces[item];
        const DecSeg db = a.segs[pc_.seg];
        const int b = db.b;
        const int hc = pc_.seg % a.nhc;
        const int t0 = pc_.t0, t1 = pc_.t1;
        const int S = a.S;
        const int c0 = a.Gc * hc + 16 * wid;        // first row of this wave
        const int nh = max(0, min(16, min(a.Gc * (hc + 1), R) - c0));
        const int rq = c0 + n;
        const int tq = rq % S, hq = rq / S;
        const float c = fmaxf(fabsf(a.scale_log2), kMinScale);
        const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
        // allowed keys of query token tq: jbase + tq + band_lo <= j <=
        // jbase + tq + band_hi (sparse_mode 3: (-2^30, 0]; 4: [-pre, next];
        // 0: open); wave-uniform extremes over the wave's columns decide
        // which steps evaluate the per-column bounds
        const int jbase = db.lkv - db.lq;
        const int tq_min = (c0 % S) + nh > S ? 0 : c0 % S;
        const int tq_max = (c0 % S) + nh > S ? S - 1 : c0 % S + max(nh, 1) - 1;
        const int jhi = jbase + tq + a.band_hi, jlo = jbase + tq + a.band_lo;
        const int jhi_min = jbase + tq_min + a.band_hi, jlo_max = jbase + tq_max + a.band_lo;

        // [Q | Q_rope]^T as the B operand: column n, d = 32 s + 8 qd (query
        // tokens at or past the batch's length are not read: in TND they are
        // the next batch's rows)
        uint4 qf[NKM + NKR];
        if (n < nh && tq < db.lq) {
            const int64_t qrow = (int64_t)db.q_row0 + tq;
            const uint16_t* src = (const uint16_t*)a.q + (int64_t)b * a.q_sB + (int64_t)hq * a.q_sH +
                                  qrow * a.q_sS + 8 * qd;
            const uint16_t* srr = (const uint16_t*)a.qr + (int64_t)b * a.qr_sB + (int64_t)hq * a.qr_sH +
                                  qrow * a.qr_sS + 8 * qd;
#pragma unroll
            for (int s = 0; s < NKM + NKR; ++s) {
                uint4 v = s < NKM ? *(const uint4*)(src + 32 * s) : *(const uint4*)(srr + 32 * (s - NKM));
                v.x ^= qflip; v.y ^= qflip; v.z ^= qflip; v.w ^= qflip;
                qf[s] = v;
            }
        } else {
#pragma unroll
            for (int s = 0; s < NKM + NKR; ++s) qf[s] = make_uint4(0, 0, 0, 0);
        }

        // pages of the piece: lane i holds the id of page pg_first + i
        const int bs = a.block_size;
        const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
        const int pg_first = t0 / bs;
        const int pg_last = t1 > t0 ? (t1 - 1) / bs : pg_first;
        const int my_page = pg_first + lane <= pg_last ? bt[pg_first + lane] : 0;
        const uint16_t* kbase = (const uint16_t*)a.k;
        const uint16_t* vbase = (const uint16_t*)a.v;
        const uint16_t* rbase = (const uint16_t*)a.kr;
        // settle the query and page-table loads: the step loop counts only
        // its own loads
        __builtin_amdgcn_s_waitcnt(FIA_VMCNT(0));

        auto advance16 = [&](int& p, int& o) {
            o += 16;
            if (o >= bs) { o -= bs; ++p; }
        };
        // resource over rows [off, off + nvalid) of page pg of a pool; rows
        // of the sub-tile starting at token tb past t1 read as zero
        auto sub_rsrc = [&](const uint16_t* base, int64_t blk, int rowlen, int pg, int off, int tb) {
            const int nvalid = max(0, min(16, t1 - tb));
            const int64_t page = nvalid > 0 ? (int64_t)__builtin_amdgcn_readlane(my_page, pg - pg_first) : 0;
            return make_rsrc(base + page * blk + (int64_t)off * rowlen, (int64_t)nvalid * rowlen * 2);
        };
        // K and K_rope of the step starting at token tt0 (first sub-tile at
        // page pg, offset off) into K slot `dst`
        auto issue_k = [&](int tt0, int pg, int off, uint32_t dst) {
            int ln = lane;
            asm volatile("" : "+v"(ln));              // per-step offsets, not held in registers
            int pg1 = pg, off1 = off;
            advance16(pg1, off1);
            const i32x4 rk0 = sub_rsrc(kbase, a.p_blk, D, pg, off, tt0);
            const i32x4 rk1 = sub_rsrc(kbase, a.p_blk, D, pg1, off1, tt0 + 16);
            const i32x4 rr0 = sub_rsrc(rbase, a.pr_blk, DR, pg, off, tt0);
            const i32x4 rr1 = sub_rsrc(rbase, a.pr_blk, DR, pg1, off1, tt0 + 16);
#pragma unroll
            for (int i = 0; i < ST / NW; ++i) {
                const int r = NW * i + wid;
                dma16_nt(r < 16 ? rk0 : rk1, dst + 2u * (uint32_t)(r * D),
                      ((uint32_t)((r & 15) * D) + 8u * (uint32_t)(ln ^ (r & 15))) * 2u);
            }
            // K_rope: 16 loads of 4 bytes per lane, two 128-byte rows each
#pragma unroll
            for (int i = 0; i < 16 / NW; ++i) {
                const int u = NW * i + wid;
                const int r = 2 * u + (ln >> 5);
                const int pch = (ln & 31) >> 2;      // 16-byte position in the row
                const uint32_t e = (uint32_t)(8 * (pch ^ ((r >> 1) & 7)) + 2 * (ln & 3));
                dma4_nt(u < 8 ? rr0 : rr1, dst + 2u * (uint32_t)(ST * D) + 256u * (uint32_t)u,
                     ((uint32_t)((r & 15) * DR) + e) * 2u);
            }
        };
        auto issue_v = [&](int tt0, int pg, int off, uint32_t dst) {
            int ln = lane;
            asm volatile("" : "+v"(ln));
            int pg1 = pg, off1 = off;
            advance16(pg1, off1);
            const i32x4 rv0 = sub_rsrc(vbase, a.p_blk, D, pg, off, tt0);
            const i32x4 rv1 = sub_rsrc(vbase, a.p_blk, D, pg1, off1, tt0 + 16);
#pragma unroll
            for (int i = 0; i < ST / NW; ++i) {
                const int r = NW * i + wid;
                dma16_nt(r < 16 ? rv0 : rv1, dst + 2u * (uint32_t)(r * D),
                      ((uint32_t)((r & 15) * D) + 8u * (uint32_t)(ln ^ (2 * (r & 7)))) * 2u);
            }
        };

        // LDS read offsets (halves) as per-lane bases plus constants:
        // K row n, chunk (4 s + qd) ^ n = 16 (s / 4) + 4 ((s % 4) ^ (n / 4)) + (qd ^ n % 4);
        // K_rope row n, chunk (4 s + qd) ^ ((n / 2) % 8) (the same for row 16 + n);
        // V^T (transposed reads as in the decode kernel): tile o = 8 og + oi
        // reads chunk pair 2 (o ^ (trow % 8)) = 16 og + 2 (oi ^ (trow % 8)).
        int koff[4], roff[NKR];
#pragma unroll
        for (int si = 0; si < 4; ++si) koff[si] = n * D + 8 * (4 * (si ^ (n >> 2)) + (qd ^ (n & 3)));
#pragma unroll
        for (int sr = 0; sr < NKR; ++sr) roff[sr] = ST * D + n * DR + 8 * ((4 * sr + qd) ^ ((n >> 1) & 7));
        // V^T reads (offsets computed per read: fewer registers held for the
        // read-ahead); V in the K slot uses K's swizzle
        const int vi = lane & 15;
        const int trow = 4 * qd + (vi >> 2);
        const int tcol_lo = (vi & 3) >> 1, tsub = 4 * (vi & 1);
        const int vrb = trow * D + tsub + 8 * tcol_lo, vsw = trow & 7;
        auto vofs = [&](int o) {
            if (VK) return trow * D + tsub + 8 * ((2 * (o & 7) + tcol_lo) ^ (trow & 15)) + 128 * (o >> 3);
            return vrb + 16 * ((o & 7) ^ vsw) + 128 * (o >> 3);
        };


        f32x4 acc[NO];
#pragma unroll
        for (int o = 0; o < NO; ++o) acc[o] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY, l = 0.f;
        const float lazy_raw = kLazy / c;

        const int nsteps = (t1 - t0 + ST - 1) / ST;
        // next K step to issue and next V step to issue: first sub-tile's page / offset
        int kpg = t0 / bs, koffs = t0 % bs;
        int vpg = kpg, voffp = koffs;
        auto skip32 = [&](int& p, int& o) { advance16(p, o); advance16(p, o); };
        if (nsteps > 0) {
            issue_k(t0, kpg, koffs, kslot(0));
            skip32(kpg, koffs);
            if constexpr (!VK) {
                issue_v(t0, vpg, voffp, vslot(0));
                skip32(vpg, voffp);
            }
            if (nsteps > 1) {
                issue_k(t0 + ST, kpg, koffs, kslot(1));
                skip32(kpg, koffs);
            }
        }
        for (int st = 0; st < nsteps; ++st) {
            const int tt0 = t0 + ST * st;
            const bool more = st + 1 < nsteps;
            if constexpr (VK) {
                // K of step st landed (K of st + 1 may still fly); every wave
                // is done with step st - 1, whose slot takes K of st + 2
                if (more) __builtin_amdgcn_s_waitcnt(FIA_VMCNT(NLK));
                else __builtin_amdgcn_s_waitcnt(FIA_VMCNT(0));
                __syncthreads();
                if (st + 2 < nsteps) {
                    issue_k(tt0 + 2 * ST, kpg, koffs, kslot(st + 2));
                    skip32(kpg, koffs);
                }
            } else {
                // K of step st landed (V of st and K of st + 1 may still fly)
                if (more) __builtin_amdgcn_s_waitcnt(FIA_VMCNT(NLV + NLK));
                else __builtin_amdgcn_s_waitcnt(FIA_VMCNT(NLV));
                __syncthreads();
                if (more) {
                    issue_v(tt0 + ST, vpg, voffp, vslot(st + 1));
                    skip32(vpg, voffp);
                }
            }
            uint4 pb = make_uint4(0, 0, 0, 0);
            if (nh > 0) {
                const uint16_t* kb = smem + kMlaKSlot * (st % NSLOT);
                f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
                if constexpr (!VK) {
                    // K operands one k-step ahead of their MFMAs (the scheduling
                    // barrier keeps each read ahead of the previous step's
                    // MFMAs; measured 3 % faster; with V read from the K slot
                    // the extra registers spill, so that path reads in place)
                    auto rdk = [&](int s, uint4& x0, uint4& x1) {
                        const uint16_t* kp = s < NKM ? kb + koff[s & 3] + 128 * (s >> 2) : kb + roff[s - NKM];
                        const int r16 = s < NKM ? 16 * D : 16 * DR;
                        x0 = *(const uint4*)(kp);
                        x1 = *(const uint4*)(kp + r16);
                    };
                    uint4 c0, c1, n0, n1;
                    rdk(0, c0, c1);
#pragma unroll
                    for (int s = 0; s < NKM + NKR; ++s) {
                        if (s + 1 < NKM + NKR) rdk(s + 1, n0, n1);
                        s0 = O::mma16(c0, qf[s], s0);
                        s1 = O::mma16(c1, qf[s], s1);
                        __builtin_amdgcn_sched_barrier(0);
                        c0 = n0; c1 = n1;
                    }
                } else {
#pragma unroll
                    for (int s = 0; s < NKM; ++s) {
                        const uint16_t* kp = kb + koff[s & 3] + 128 * (s >> 2);
                        const uint4 a0 = *(const uint4*)(kp);
                        const uint4 a1 = *(const uint4*)(kp + 16 * D);
                        s0 = O::mma16(a0, qf[s], s0);
                        s1 = O::mma16(a1, qf[s], s1);
                    }
#pragma unroll
                    for (int s = 0; s < NKR; ++s) {
                        const uint4 a0 = *(const uint4*)(kb + roff[s]);
                        const uint4 a1 = *(const uint4*)(kb + roff[s] + 16 * DR);
                        s0 = O::mma16(a0, qf[NKM + s], s0);
                        s1 = O::mma16(a1, qf[NKM + s], s1);
                    }
                }
                float x[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] = s0[i];
                    x[4 + i] = s1[i];
                }
                if (tt0 + ST > t1 || tt0 + ST - 1 > jhi_min || tt0 < jlo_max) {
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const int tk = tt0 + 16 * (r >> 2) + 4 * qd + (r & 3);
                        if (tk >= t1 || tk > jhi || tk < jlo) x[r] = -INFINITY;
                    }
                }
                float mt = x[0];
#pragma unroll
                for (int r = 1; r < 8; ++r) mt = fmaxf(mt, x[r]);
                mt = quad_max(mt);
                const float mn = fmaxf(m, mt);
                const bool grow = (m == -INFINITY) ? (mn > -INFINITY) : (mn > m + lazy_raw);
                if (__ballot(grow)) {
                    float alpha = 1.f;
                    if (m == -INFINITY) alpha = 0.f;
                    else if (mn != -INFINITY) alpha = fast_exp2((m - mn) * c);
                    m = mn;
                    l *= alpha;
#pragma unroll
                    for (int o = 0; o < NO; ++o) acc[o] *= alpha;
                }
                const float mc = (m == -INFINITY) ? 0.f : m * c;
                float ps = 0.f;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    x[r] = fast_exp2(__builtin_fmaf(x[r], c, -mc));
                    ps += x[r];
                }
                l += ps;
                pb.x = O::pack2(x[0], x[1]);
                pb.y = O::pack2(x[2], x[3]);
                pb.z = O::pack2(x[4], x[5]);
                pb.w = O::pack2(x[6], x[7]);
            }
            if constexpr (!VK) {
                // V of step st landed (K of st + 1 and V of st + 1 may still fly)
                if (more) __builtin_amdgcn_s_waitcnt(FIA_VMCNT(NLK + NLV));
                else __builtin_amdgcn_s_waitcnt(FIA_VMCNT(0));
                __syncthreads();
                if (st + 2 < nsteps) {
                    issue_k(tt0 + 2 * ST, kpg, koffs, kslot(st));
                    skip32(kpg, koffs);
                }
            }
            if (nh > 0) {
                const uint16_t* vb = VK ? smem + kMlaKSlot * (st % NSLOT) : smem + 2 * kMlaKSlot + kMlaVSlot * (st & 1);
                {
                    // V^T operands one tile ahead of their MFMAs
                    uint2 cl, ch, nl, nh2;
                    cl = lds_read_tr16(vb + vofs(0));
                    ch = lds_read_tr16(vb + vofs(0) + 16 * D);
#pragma unroll
                    for (int o = 0; o < NO; ++o) {
                        if (o + 1 < NO) {
                            const uint16_t* vp = vb + vofs(o + 1);
                            nl = lds_read_tr16(vp);
                            nh2 = lds_read_tr16(vp + 16 * D);
                        }
                        acc[o] = O::mma16(make_uint4(cl.x, cl.y, ch.x, ch.y), pb, acc[o]);
                        __builtin_amdgcn_sched_barrier(0);
                        cl = nl; ch = nh2;
                    }
                }
            }
        }

        // partial: normalised O and natural-log LSE of this split
        const float lt = quad_sum(l);
        if (n < nh) {
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            float* po = a.part_o + ((int64_t)item * a.Gc + 16 * wid + n) * D;
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                f32x4 v = acc[o] * inv;
                *(f32x4*)(po + 16 * o + 4 * qd) = v;
            }
            if (qd == 0)
                a.part_lse[(int64_t)item * a.Gc + 16 * wid + n] =
                    lt > 0.f ? (m * c + __log2f(lt)) * kLn2 : -INFINITY;
        }
        __syncthreads();     // the slots are reused by the next piece
    }
}

// Merge the kv splits of one (batch, head, query token): weights
// exp(lse_s - max lse).  Tokens at or past the batch's query length are
// written as out = 0, lse = +inf.
template <int DT, int D>
__global__ __launch_bounds__(64) void decode_combine(DecodeArgs a)
{
    using O = Ops<DT>;
    const int bht = blockIdx.x;
    const int S = a.S;
    const int t = bht % S;
    const int b = bht / (a.QN * S), h = (bht / S) % a.QN;
    const int kvh = h / a.G, r = (h % a.G) * S + t;
    const int hc = r / a.Gc, n = r % a.Gc;
    const DecSeg sg = a.segs[((int64_t)b * a.KVN + kvh) * a.nhc + hc];
    if (a.tnd && t >= sg.lq) return;        // TND: the row does not exist
    const int ns = t < sg.lq ? sg.count : 0;
    const int64_t slot0 = sg.first;
    const int lane = threadIdx.x;
    const int64_t orow = (int64_t)sg.q_row0 + t;
    uint16_t* op = (uint16_t*)a.o + (int64_t)b * a.o_sB + (int64_t)h * a.o_sH + orow * a.o_sS;

    // the pieces' LSEs 64 at a time (lane i: piece s0 + i), their max by a
    // wave reduction; the merge itself runs over the pieces in order
    auto lse_of = [&](int s0) {
        return s0 + lane < ns ? a.part_lse[(slot0 + s0 + lane) * a.Gc + n] : -INFINITY;
    };
    float lv = lse_of(0);
    float M = lv;
    for (int s0 = 64; s0 < ns; s0 += 64) M = fmaxf(M, lse_of(s0));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float wsum = 0.f;
    constexpr int PER = D / 64;
    float accv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) accv[e] = 0.f;
    if (M != -INFINITY) {
        for (int s0 = 0; s0 < ns; s0 += 64) {
            if (s0 > 0) lv = lse_of(s0);
            const float wl = __expf(lv - M);
            const int cnt = min(64, ns - s0);
            // four pieces' partials loaded together, then merged in order
            int s = 0;
            for (; s + 4 <= cnt; s += 4) {
                float v[4][PER];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float* po = a.part_o + ((slot0 + s0 + s + u) * a.Gc + n) * D + PER * lane;
#pragma unroll
                    for (int e = 0; e < PER; ++e) v[u][e] = po[e];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s + u));
                    wsum += ws;
#pragma unroll
                    for (int e = 0; e < PER; ++e) accv[e] += ws * v[u][e];
                }
            }
            for (; s < cnt; ++s) {
                const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s));
                wsum += ws;
                const float* po = a.part_o + ((slot0 + s0 + s) * a.Gc + n) * D + PER * lane;
#pragma unroll
                for (int e = 0; e < PER; ++e) accv[e] += ws * po[e];
            }
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    float vals[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        float val = accv[e] * inv;
        if (a.kv_i8 && a.vmode == 0 && wsum > 0.f) {
            // int8 V per channel: the partials are in raw int8 units
            const int64_t ch = (int64_t)kvh * D + PER * lane + e;
            const float sv = __uint_as_float((uint32_t)((const uint16_t*)a.v_scale)[ch] << 16);
            const float ov = a.v_off ? __uint_as_float((uint32_t)((const uint16_t*)a.v_off)[ch] << 16) : 0.f;
            val = sv * (val + ov);
        }
        vals[e] = val;
    }
    if constexpr (PER % 2 == 0) {
        // lane's PER consecutive outputs as bf16 / fp16 pairs
        uint32_t* op2 = (uint32_t*)(op + PER * lane);
#pragma unroll
        for (int e = 0; e < PER / 2; ++e) op2[e] = O::pack2(vals[2 * e], vals[2 * e + 1]);
    } else {
#pragma unroll
        for (int e = 0; e < PER; ++e) op[PER * lane + e] = (uint16_t)(O::pack2(vals[e], 0.f) & 0xffffu);
    }
    if (a.return_lse && lane == 0) {
        const int64_t li = a.tnd ? orow * a.QN + h : ((int64_t)b * a.QN + h) * S + t;
        a.lse[li] = wsum > 0.f ? M + __logf(wsum) : INFINITY;
    }
}

// ---------------------------------------------------------------------------
// Block-sparse schedule compaction: one wave per (batch, head, q block).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bsa_compact(const uint8_t* mask, const BatchInfo* batch,
                                                   int32_t* cnt, int32_t* idx, int N1, int nqb,
                                                   int nkb, int X, int Y, int64_t n_rows)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int64_t b = row / ((int64_t)N1 * nqb);
    const int qb = (int)(row % nqb);
    const BatchInfo bi = batch[b];
    const int64_t klim = ((int64_t)bi.lkv + Y - 1) / Y;
    const bool qok = (int64_t)qb * X < bi.lq;
    const uint8_t* mrow = mask + row * nkb;
    int32_t* irow = idx + row * nkb;
    int base = 0;
    for (int c0 = 0; c0 < nkb; c0 += 64) {
        const int kb = c0 + lane;
        const bool sel = kb < nkb && qok && kb < klim && mrow[kb] != 0;
        const unsigned long long bal = __ballot(sel);
        const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
        if (sel) irow[pos] = kb;
        base += __popcll(bal);
    }
    for (int kb = base + lane; kb < nkb; kb += 64) irow[kb] = -1;
    if (lane == 0) cnt[row] = base;
}

template <typename K>
void raise_lds_limit(K kernel, size_t lds, bool& configured)
{
    if (!configured) {
        // raise the dynamic LDS limit past the 64 KB default (gfx950: 160 KB)
        (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        (void)hipGetLastError();
        configured = true;
    }
}

template <int DT, int DQK, int DV, int KIND, bool PG = false>
int launch_attn(const fia_plan& p, const AttnArgs& a, hipStream_t stream)
{
    // 4 waves, two workgroups per CU, K/V double buffered (measured faster
    // than 8-wave workgroups with deeper LDS pipelines)
    constexpr int NW = kDenseWaves;
    constexpr int NS = 2;
    const size_t lds = (size_t)NS * kBlockN * (DQK + DV) * sizeof(uint16_t);
    static bool configured = false;
    raise_lds_limit(attn_fwd<DT, DQK, DV, KIND, NW, NS, PG>, lds, configured);
    if (p.n_tiles == 0) return 0;
    hipLaunchKernelGGL((attn_fwd<DT, DQK, DV, KIND, NW, NS, PG>), dim3((unsigned)p.n_tiles), dim3(NW * 64),
                       lds, stream, a);
    return (int)hipGetLastError();
}

template <int D>
void launch_split_i8(const fia_plan& p, const DecodeArgs& a, hipStream_t stream)
{
    const dim3 g((unsigned)p.n_waves), blk(64);
    // the mode pairs phase 1 accepts: equal, or key per channel with value per token
    if (a.kmode == 0 && a.vmode == 0) hipLaunchKernelGGL((decode_split_i8<D, 0, 0>), g, blk, 0, stream, a);
    else if (a.kmode == 0) hipLaunchKernelGGL((decode_split_i8<D, 0, 1>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((decode_split_i8<D, 1, 1>), g, blk, 0, stream, a);
}

template <int DT, int D>
int launch_dec(const fia_plan& p, const DecodeArgs& a, hipStream_t stream)
{
    if (p.n_waves > 0 && a.kv_i8)
        launch_split_i8<D>(p, a, stream);
    else if (p.n_waves > 0 && a.mask)
        hipLaunchKernelGGL((decode_split<DT, D, true>), dim3((unsigned)p.n_waves), dim3(64), 0, stream, a);
    else if (p.n_waves > 0)
        hipLaunchKernelGGL((decode_split<DT, D, false>), dim3((unsigned)p.n_waves), dim3(64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL((decode_combine<DT, D>), dim3((unsigned)(p.B * p.QN * a.S)), dim3(64), 0, stream, a);
    return (int)hipGetLastError();
}

}  // namespace

template <int DT, int DQK, int DV>
int launch_prefill_kind(const fia_plan& p, const AttnArgs& a, hipStream_t s)
{
    if (a.paged)
        return a.has_mask ? launch_attn<DT, DQK, DV, kMasked, true>(p, a, s)
                          : launch_attn<DT, DQK, DV, kDense, true>(p, a, s);
    return a.has_mask ? launch_attn<DT, DQK, DV, kMasked>(p, a, s) : launch_attn<DT, DQK, DV, kDense>(p, a, s);
}

int launch_prefill(const fia_plan& p, const AttnArgs& a, void* stream)
{
    hipStream_t s = (hipStream_t)stream;
    const bool bf = p.dtype == FIA_BF16;
    if (p.Dqk == 64 && p.Dv == 64)
        return bf ? launch_prefill_kind<FIA_BF16, 64, 64>(p, a, s) : launch_prefill_kind<FIA_F16, 64, 64>(p, a, s);
    if (p.Dqk == 128 && p.Dv == 128)
        return bf ? launch_prefill_kind<FIA_BF16, 128, 128>(p, a, s) : launch_prefill_kind<FIA_F16, 128, 128>(p, a, s);
    if (p.Dqk == 192 && p.Dv == 128)
        return bf ? launch_prefill_kind<FIA_BF16, 192, 128>(p, a, s) : launch_prefill_kind<FIA_F16, 192, 128>(p, a, s);
    return (int)hipErrorInvalidValue;
}

int launch_bsa(const fia_plan& p, const AttnArgs& a, void* stream)
{
    hipStream_t s = (hipStream_t)stream;
    if (p.n_rows > 0) {
        hipLaunchKernelGGL(bsa_compact, dim3((unsigned)((p.n_rows + 3) / 4)), dim3(256), 0, s,
                           p.bsa_mask, a.batch, (int32_t*)a.bsa_cnt, (int32_t*)a.bsa_idx,
                           (int)p.QN, (int)p.bsa_nqb, (int)p.bsa_nkb, a.bx, a.by, p.n_rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    if (a.fp8) {
        const size_t lds = 2u * (2u * kBlockN * 128u) + 2u * kBlockN * 128u;   // 2 x 16 KB + 16 KB
        static bool configured = false;
        raise_lds_limit(bsa_fp8, lds, configured);
        if (p.n_tiles == 0) return 0;
        hipLaunchKernelGGL(bsa_fp8, dim3((unsigned)p.n_tiles), dim3(256), lds, s, a);
        return (int)hipGetLastError();
    }
    const bool bf = p.dtype == FIA_BF16;
    if (p.Dqk == 64)
        return bf ? launch_attn<FIA_BF16, 64, 64, kSparse>(p, a, s) : launch_attn<FIA_F16, 64, 64, kSparse>(p, a, s);
    if (p.Dqk == 128)
        return bf ? launch_attn<FIA_BF16, 128, 128, kSparse>(p, a, s) : launch_attn<FIA_F16, 128, 128, kSparse>(p, a, s);
    return (int)hipErrorInvalidValue;
}

template <int DT, int NW, bool VK>
int launch_mla_nw(const fia_plan& p, const DecodeArgs& a, hipStream_t stream)
{
    // 2 K slots of 36 KB and 2 V slots of 32 KB, or 3 K slots when V is K
    const size_t lds = VK ? kMlaLdsBytesVK : kMlaLdsBytes;
    static bool configured = false;
    raise_lds_limit(mla_decode<DT, NW, VK>, lds, configured);
    if (p.n_waves > 0)
        hipLaunchKernelGGL((mla_decode<DT, NW, VK>), dim3((unsigned)p.n_waves), dim3(NW * 64), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL((decode_combine<DT, kMlaD>), dim3((unsigned)(p.B * p.QN * a.S)), dim3(64), 0, stream, a);
    return (int)hipGetLastError();
}

template <int DT>
int launch_mla(const fia_plan& p, const DecodeArgs& a, hipStream_t s)
{
    if (a.v_is_k) {
        switch (a.mla_nw) {
        case 2: return launch_mla_nw<DT, 2, true>(p, a, s);
        case 4: return launch_mla_nw<DT, 4, true>(p, a, s);
        case 8: return launch_mla_nw<DT, 8, true>(p, a, s);
        }
    } else {
        switch (a.mla_nw) {
        case 2: return launch_mla_nw<DT, 2, false>(p, a, s);
        case 4: return launch_mla_nw<DT, 4, false>(p, a, s);
        case 8: return launch_mla_nw<DT, 8, false>(p, a, s);
        }
    }
    return (int)hipErrorInvalidValue;
}

int launch_decode(const fia_plan& p, const DecodeArgs& a, void* stream)
{
    hipStream_t s = (hipStream_t)stream;
    if (a.mla_nw) return p.dtype == FIA_BF16 ? launch_mla<FIA_BF16>(p, a, s) : launch_mla<FIA_F16>(p, a, s);
    const bool bf = p.dtype == FIA_BF16;
    if (p.Dqk == 64) return bf ? launch_dec<FIA_BF16, 64>(p, a, s) : launch_dec<FIA_F16, 64>(p, a, s);
    if (p.Dqk == 128) return bf ? launch_dec<FIA_BF16, 128>(p, a, s) : launch_dec<FIA_F16, 128>(p, a, s);
    return (int)hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free run: one static device array per GPU the
// library runs on (it lives until the process ends).  In host code the
// array's name is only a host-side stand-in; its device address comes from
// hipGetSymbolAddress, resolved once per device with that device current,
// and only that address is ever handed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};
}  // namespace

void* noalloc_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        scratch_ptr[dev] = ptr;
    }
    return scratch_ptr[dev];
}

void* upload_tables(const void* src, uint64_t bytes)
{
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n == 0) {
        (void)hipGetLastError();
        return nullptr;
    }
    void* dev = nullptr;
    if (hipMalloc(&dev, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (hipMemcpy(dev, src, bytes, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipFree(dev);
        return nullptr;
    }
    return dev;
}

void free_tables(void* dev)
{
    if (dev) (void)hipFree(dev);
}

}  // namespace fia
