// Sparse MLA decode for AMD CDNA4 (gfx950): split-K decode kernel, log-sum-exp
// combine kernel, and the C ABI declared in include/smla.h.
//
// What is computed ("The Moment of Compilation", section "The Context: A Kernel
// Optimization Campaign"; "The Power-of-Two Trap", sections "The Scene" and
// "The Scale Indexing Complication"; "The 80KB Mystery", section "The Context:
// Optimizing Attention on Blackwell"): each query token attends, with all heads
// of this GPU, over the latent rows its top-k list selects; each row is read
// from HBM once per group of 16 heads and shared by those heads in one matrix
// product; the selected list is split across workgroups (split-K) when there
// are too few (sequence, head group) pairs to fill the chip, and the partial
// results are merged with a log-sum-exp combine.
//
// Design on gfx950 (differs from the Triton kernel of the pages, which pads
// 448 to 512 because its tile ranges must be powers of two, and which stages
// one tile per thread block through shared memory):
//  * 448 = 7 groups x 64 columns = 14 MFMA K-steps of 32: no padding at all.
//  * Every wave is an independent decoder for 16 heads over the full 512-wide
//    latent: it owns two 32-token LDS slots, gathers its next tile straight
//    into one (global_load_lds, 16 bytes per lane, coalesced along the row)
//    while it computes the current one from the other, and never waits for
//    another wave until the end.  A workgroup is four such waves (one per
//    SIMD, the whole 160 KB LDS) on the same (sequence, head group, split);
//    they take the split's tiles round robin and merge their online-softmax
//    states once, through LDS, at the end.
//  * QK^T runs as S^T = K . Q^T on v_mfma_f32_16x16x32_bf16: the fp8 codes are
//    converted exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8 with unit scale),
//    q is used as stored, and each 64-column group's fp32 scale multiplies that
//    group's fp32 partial logits after the MFMA.  Logits are therefore as
//    accurate as fp32 accumulation allows.
//  * Online softmax in the log2 domain with lazy rescaling: the running base
//    only moves when the tile maximum exceeds it by more than 8 (so weights
//    stay below 2^8), which keeps the 128-register accumulator rescale rare.
//    Cross-lane maxima use v_permlane16_swap / v_permlane32_swap (no LDS).
//  * PV runs as O^T = V^T . P^T on v_mfma_f32_16x16x32_f16.  The S^T
//    accumulator layout already is the P^T operand layout, so no data moves
//    between lanes.  The group scale is folded into the weights
//    (fp16(p * scale_g)), the value codes enter exactly (fp8 -> fp16), and the
//    V^T operand is read from the row-major LDS tile with ds_read_b64_tr_b8
//    (rope: ds_read_b64_tr_b16, bf16 values with the weight split into bf16
//    high and low parts).
//  * fp16 weights keep 11 significant bits, which bounds the value-product
//    error by 2^-11 relative; bf16 weights (8 bits) would not meet 1e-2
//    absolute on outputs near 4 once the bf16 output rounding is added.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/smla.h"

namespace {

constexpr int kRowBytes = SMLA_ROW_BYTES;   // 640
constexpr int kNope = SMLA_NOPE_DIM;        // 448
constexpr int kLatent = SMLA_LATENT_DIM;    // 512
constexpr int kTile = 32;                   // tokens per tile
constexpr float kTau = 8.0f;                // lazy-rescale threshold (log2 units)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const u32x4 lds_cu32x4;
typedef __attribute__((address_space(3))) const f32x4 lds_cf32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) const float lds_cf32;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) int32_t lds_i32;
typedef __attribute__((address_space(3))) const int32_t lds_ci32;

// LDS tile slot: 32 rows of codes and rope, row-major, kRowLds bytes apart,
// followed by the tile's group scales transposed to [group][token].
// LDS row: bytes 0..447 the fp8 codes, 448..575 the rope, 576..591 unused.
// The pitch of 37 16-byte pieces makes the 16 rows read by one 16-lane group
// start in 16 distinct 4-bank sets.  The scales arrive by a separate 4-byte
// gather per (token, group), which writes the transposed table directly.
constexpr int kPieces = 37;                         // LDS row pitch in 16-byte pieces
constexpr int kCodePieces = 28;                     // pieces 0..27: codes; 28..35: rope
constexpr int kRowLds = kPieces * 16;               // 592
constexpr int kLdsRope = kNope;                     // rope offset inside an LDS row (448)
constexpr int kScaleTable = kTile * kRowLds;        // scale table offset in a slot (18944)
constexpr int kSlot = kScaleTable + 8 * kTile * 4;  // 19968 bytes per tile slot
constexpr int kRowGathers = (kTile * kPieces + 63) / 64;   // 19 row gathers of 64 lanes
constexpr int kScaleGathers = 4;                    // 4-byte gathers of the scale table
constexpr int kWaves = 4;                           // waves per workgroup (one per SIMD)
constexpr int kMaxChunk = 2048;                     // list entries of a shared-tile workgroup
constexpr int kAccBytes = 32 * 64 * 16;             // one wave's output accumulator (32 KB)

// Workgroup geometry for G head groups of 16 heads per workgroup (G = 1, 2, 4).
// The four waves form T = 4 / G tile streams; stream s takes tiles s, s + T,
// ... of the workgroup's chunk, and its G waves (one per head group) share
// each of its tiles.  A stream owns a ring of NS tile slots.
//  * G = 1: every wave is its own stream with two slots; it loads the rows of
//    its next tile into registers one tile ahead and issues all gathers of a
//    tile itself; no wave ever waits for another before the merge.
//  * G = 2, 4: the chunk's (sanitised) list entries sit in an LDS table, every
//    wave issues L of the tile's 23 gathers (one more, a no-op load, pads the
//    count so that all waves count the same loads per tile), NS - 1 tiles are
//    in flight, and a workgroup barrier per tile step recycles the slot of the
//    previous step.
template <int G>
struct Geo {
    static constexpr int T = kWaves / G;
    static constexpr int NS = G == 1 ? 2 : G == 2 ? 3 : 4;
    static constexpr int L = (kRowGathers + kScaleGathers + G - 1) / G;   // shared modes
    static constexpr int kRing = T * NS * kSlot;
    static constexpr int kIdx = kRing;                                   // index table
    static constexpr int kDummy = kIdx + (G > 1 ? kMaxChunk * 4 : 0);    // no-op gather target
    static constexpr int kEnd = kDummy + (G > 1 ? 1024 : 0);
    static constexpr int kMerge = T > 1 ? kWaves * kAccBytes : 0;        // reuses the ring
    static constexpr int kStat = kEnd > kMerge ? kEnd : kMerge;          // per-wave (max, sum)
    static constexpr int kLds = kStat + kWaves * 32 * 4;
    static_assert(kLds <= 160 * 1024, "LDS budget of one gfx950 workgroup");
    static_assert(G == 1 || L * G <= kRowGathers + kScaleGathers + 1, "at most one no-op gather per tile");
};

__device__ __forceinline__ bf16x8 codes_to_bf16(uint32_t lo, uint32_t hi) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ f16x8 codes_to_f16(uint32_t lo, uint32_t hi) {
    f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
    f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
    f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
    f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    bf16x8 r;
    memcpy(&r, &v, 16);
    return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32: round to nearest even
    uint32_t u;
    memcpy(&u, &v, 4);
    return u;
}

// Maximum / sum over the four 16-lane groups (lanes l, l^16, l^32, l^48),
// returned to every lane.  v_permlane16_swap with both operands equal leaves
// rows (0,0,2,2) in one result and (1,1,3,3) in the other; v_permlane32_swap
// leaves (0,1,0,1) and (2,3,2,3).  Both orders of each pair give the same sum.
__device__ __forceinline__ float lanegroup_max(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(x);
    const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ float lanegroup_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t v = __float_as_uint(x);
    const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// An LDS address the compiler must treat as opaque: every read of a tile then
// uses one base register plus immediate offsets, instead of loop-invariant
// per-offset address registers.
__device__ __forceinline__ const lds_u8* opaque(const lds_u8* p) {
    asm volatile("" : "+v"(p));
    return p;
}

// Token held in MFMA k-slot `slot` (0..31) of a 32-token tile.  The S^T
// accumulator of lane group q holds tokens 4q..4q+3 (first 16-token half) and
// 16+4q..16+4q+3 (second half); the PV product uses k-slots 8q..8q+7 for them.
__device__ __forceinline__ int slot_token(int slot) {
    int q = slot >> 3, r = slot & 7;
    return r < 4 ? 4 * q + r : 16 + 4 * q + (r - 4);
}

// Buffer resource over one sequence's cache rows (gfx9 raw buffer, stride 0):
// a gather addresses a row by a 32-bit byte offset, and the hardware range
// check turns every offset at or past `bytes` into a load of zeros.  A masked
// list entry therefore uses row -1: its offset is negative, i.e. above 2^32 -
// 640 as an unsigned number, and it stages zeros (finite, contributes nothing).
__device__ __forceinline__ i32x4 row_rsrc(const uint8_t* base, uint32_t bytes) {
    const uint64_t p = (uint64_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(p >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
    r[3] = 0x00020000;
    return r;
}

// Byte offset of 16-byte piece `off` of cache row `row` (row in [-1, 2^23)).
__device__ __forceinline__ uint32_t row_offset(int row, int off) {
    return (uint32_t)(__mul24(row, kRowBytes) + off);
}

// 16-byte (4-byte) gather of one lane straight into LDS at lds_base + 16 *
// lane (+ 4 * lane): buffer_load_dwordx4 / _dword with the lds bit; the LDS
// base goes through M0 and must be wave-uniform.  Written as inline assembly
// so that the compiler does not treat every later LDS read as dependent on
// every gather in flight; the ordering is explicit instead (s_waitcnt vmcnt
// before a slot is read, and a workgroup barrier where slots are shared).
__device__ __forceinline__ void gather16(uint32_t voff, i32x4 rsrc, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}

__device__ __forceinline__ void gather4(uint32_t voff, i32x4 rsrc, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without a memory fence: only this wave's LDS operations are
// waited for, so gathers still in flight into other ring slots stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct DecodeArgs {
    const uint16_t* q;
    const uint8_t* kv;
    const int32_t* idx;
    const int32_t* seqlens;
    uint16_t* out;
    float* lse;
    float* o_part;
    float* lse_part;
    int64_t kv_seq_stride;
    uint32_t seq_bytes;   // kv_seq_stride * 640 (< 2^31): the range of a sequence's rows
    float logit_factor;   // scale * log2(e)
    int32_t batch, heads, topk, nsplit, chunk, n_hb;
    int32_t force_partials;   // write split partials even when nsplit == 1
    int32_t xcd_remap;        // grid is a multiple of 8: keep a sequence's blocks on one XCD
};

// Source byte offset inside a cache row of LDS piece p: pieces 0..27 are the
// codes, 28..35 the rope (cache pieces 30..37), 36 the unused pitch padding
// (cache piece 38).
__device__ __forceinline__ int piece_src(int p) { return 16 * (p < kCodePieces ? p : p + 2); }

// G = 1: gather one whole 32-token tile into the LDS slot at slot_lds.  Every
// lane holds the (sanitised) row of token (lane & 31).  Row gather k covers
// the slot's bytes [1024k, 1024k + 1024): lane l loads LDS piece p = c % 37 of
// token r = c / 37 (c = 64k + l), whose row comes from lane r by ds_bpermute.
// Scale gather k' loads scale 2k' + (l >> 5) of token l & 31 into the table.
__device__ __forceinline__ void issue_tile_own(int row_of_lane, i32x4 rsrc, uint32_t slot_lds, int lane_in) {
    int lane = lane_in;
    asm volatile("" : "+v"(lane));   // keep the per-lane piece walk inside the loop (registers)
    int r = 0;
    int p = lane;
    if (p >= kPieces) {
        p -= kPieces;
        r = 1;
    }
    int rows[kRowGathers];
    int offs[kRowGathers];
#pragma unroll
    for (int k = 0; k < kRowGathers; k++) {
        rows[k] = __builtin_amdgcn_ds_bpermute(4 * (r & 31), row_of_lane);
        offs[k] = piece_src(p);
        // next piece: c + 64 = c + 37 + 27
        p += 27;
        r += 1;
        if (p >= kPieces) {
            p -= kPieces;
            r += 1;
        }
    }
    // all lookups are issued before the first one is used
#pragma unroll
    for (int k = 0; k < kRowGathers; k++) asm volatile("" : "+v"(rows[k]));
#pragma unroll
    for (int k = 0; k < kScaleGathers; k++)
        gather4(row_offset(row_of_lane, SMLA_SCALE_OFFSET + 4 * (2 * k + (lane >> 5))), rsrc,
                slot_lds + kScaleTable + 256 * k);
#pragma unroll
    for (int k = 0; k < kRowGathers; k++)
        if (k + 1 < kRowGathers || lane < kTile * kPieces - 64 * (kRowGathers - 1))
            gather16(row_offset(rows[k], offs[k]), rsrc, slot_lds + 1024 * k);
}

// G = 2, 4: this wave's gathers of a tile are ids hgl, hgl + G, ... (L of
// them): 0..18 row gathers, 19..22 scale gathers, anything else a no-op load
// of zeros into the dummy area.  rows points at the tile's 32 entries of the
// LDS index table; live = false gathers zeros.  The table lookups are all
// issued before the first gather.
template <int G, int L>
__device__ __forceinline__ void issue_tile_shared(lds_ci32* rows, bool live, i32x4 rsrc, uint32_t slot_lds,
                                                  uint32_t dummy_lds, int hgl, int lane) {
    int row[L];
#pragma unroll
    for (int u = 0; u < L; u++) {
        const int id = hgl + G * u;
        const int c = 64 * id + lane;
        const int r = id < kRowGathers ? (c * 1772) >> 16 : lane;   // c / 37 for c < 1216
        row[u] = rows[r & 31];
    }
#pragma unroll
    for (int u = 0; u < L; u++) asm volatile("" : "+v"(row[u]));
#pragma unroll
    for (int u = 0; u < L; u++) {
        const int id = hgl + G * u;
        const int rw = live ? row[u] : -1;
        if (id < kRowGathers) {
            const int c = 64 * id + lane;
            const int p = c - kPieces * ((c * 1772) >> 16);
            if (c < kTile * kPieces) gather16(row_offset(rw, piece_src(p)), rsrc, slot_lds + 1024 * id);
        } else if (id < kRowGathers + kScaleGathers) {
            const int k = id - kRowGathers;
            gather4(row_offset(rw, SMLA_SCALE_OFFSET + 4 * (2 * k + (lane >> 5))), rsrc,
                    slot_lds + kScaleTable + 256 * k);
        } else {
            gather4(0x80000000u, rsrc, dummy_lds);
        }
    }
}

// One 32-token tile for one wave: 16 heads x the full latent.  st is the
// tile's LDS slot; vmask marks the kept tokens.
__device__ __forceinline__ void compute_tile(const lds_u8* st, uint64_t vmask, const bf16x8 (&qop)[16],
                                             f32x4 (&acc_o)[32], float& m_run, float& l_run, int lane,
                                             float logit_factor) {
    const int qg = lane >> 4, ln = lane & 15;

    // group scales, transposed: sT[g * 32 + t] = scale g of token t
    lds_cf32* sT = (lds_cf32*)(st + kScaleTable);

    // ---------------- S^T = K . Q^T per 16-token half; lane group q takes
    // columns 16q..16q+15 of every 64-column group (two K-steps of 8), and rope
    // columns 16q..16q+15.  The K rows of the second half are read before the
    // first half is converted.
    u32x4 raw[2][7];
    u32x4 rr[2][2];
    auto load_half = [&](int tt) {
        const lds_u8* krow = st + (16 * tt + ln) * kRowLds;
#pragma unroll
        for (int g = 0; g < 7; g++) raw[tt][g] = *(lds_cu32x4*)(krow + 64 * g + 16 * qg);
        rr[tt][0] = *(lds_cu32x4*)(krow + kLdsRope + 32 * qg);
        rr[tt][1] = *(lds_cu32x4*)(krow + kLdsRope + 32 * qg + 16);
    };
    load_half(0);
    load_half(1);
    f32x4 s[2];
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
        f32x4 acc[8];
#pragma unroll
        for (int g = 0; g < 7; g++)
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw[tt][g][0], raw[tt][g][1]),
                                                             qop[2 * g], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        acc[7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rr[tt][0]), qop[14], f32x4{0.f, 0.f, 0.f, 0.f},
                                                         0, 0, 0);
#pragma unroll
        for (int g = 0; g < 7; g++)
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw[tt][g][2], raw[tt][g][3]),
                                                             qop[2 * g + 1], acc[g], 0, 0, 0);
        acc[7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rr[tt][1]), qop[15], acc[7], 0, 0, 0);
        f32x4 v = acc[7];
#pragma unroll
        for (int g = 0; g < 7; g++)
            v += *(lds_cf32x4*)(sT + g * kTile + 16 * tt + 4 * qg) * acc[g];
        s[tt] = v;
    }
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float z = s[tt][j] * logit_factor;
            s[tt][j] = ((vmask >> (16 * tt + 4 * qg + j)) & 1) ? z : -INFINITY;
        }

    // ---------------- online softmax (log2 domain), lazy rescale
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = lanegroup_max(mx);
    const bool need = mx > m_run + kTau;
    if (__any(need)) {
        const float m_new = need ? mx : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        // the first kept tokens only set the base: the accumulators are still zero
        if (__any(m_run != -INFINITY)) {
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 32; i++) acc_o[i] *= alpha;
        }
        m_run = m_new;
    }
    const float base = m_run == -INFINITY ? 0.f : m_run;
    float p[8];   // k-slot order: tokens 4q+j (j < 4), then 16+4q+(j-4)
#pragma unroll
    for (int j = 0; j < 8; j++) {
        p[j] = __builtin_amdgcn_exp2f(s[j >> 2][j & 3] - base);
        l_run += p[j];
    }

    // ---------------- O^T += V^T . P^T
    // V^T operands: tr8 source rows, lane 16q + j supplies token slot_token(8q + j/2),
    // byte half j%2; rope V^T via tr16, lane 16q + 4r + c supplies
    // slot_token(8q + r), then slot_token(8q + 4 + r), columns 4c..4c+3 of each
    // 16-column block.  The reads of group g + 1 are issued before group g is
    // converted (one wave per SIMD has no other wave to hide LDS latency).
    const lds_u8* tr_row = st + slot_token(8 * qg + (ln >> 1)) * kRowLds + 8 * (ln & 1);
    const int col = 8 * (ln & 3);
    const lds_u8* r0 = st + slot_token(8 * qg + (ln >> 2)) * kRowLds + kLdsRope + col;
    const lds_u8* r1 = st + slot_token(8 * qg + 4 + (ln >> 2)) * kRowLds + kLdsRope + col;
    i32x2 vraw[2][4];
    f32x4 svv[2][2];
    auto load_group = [&](int g, int buf) {
#pragma unroll
        for (int cb = 0; cb < 4; cb++)
            vraw[buf][cb] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(tr_row + 64 * g + 16 * cb));
        svv[buf][0] = *(lds_cf32x4*)(sT + g * kTile + 4 * qg);
        svv[buf][1] = *(lds_cf32x4*)(sT + g * kTile + 16 + 4 * qg);
    };
    load_group(0, 0);
    s16x4 rv[4][2];
#pragma unroll
    for (int g = 0; g < 7; g++) {
        const int cur = g & 1;
        if (g + 1 < 7) load_group(g + 1, cur ^ 1);
        if (g == 1) {
#pragma unroll
            for (int dt = 0; dt < 4; dt++) {
                rv[dt][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(r0 + 32 * dt));
                rv[dt][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(r1 + 32 * dt));
            }
        }
        // weights fp16(p * scale_g); exact fp8 -> fp16 value codes
        f16x8 bop;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            bop[j] = (_Float16)(p[j] * svv[cur][0][j]);
            bop[4 + j] = (_Float16)(p[4 + j] * svv[cur][1][j]);
        }
#pragma unroll
        for (int cb = 0; cb < 4; cb++)
            acc_o[4 * g + cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                codes_to_f16((uint32_t)vraw[cur][cb][0], (uint32_t)vraw[cur][cb][1]), bop, acc_o[4 * g + cb],
                0, 0, 0);
    }
    {
        // rope: bf16 values as stored; weights split into bf16 high and low parts
        bf16x8 phi, plo;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const __bf16 h = (__bf16)p[j];
            phi[j] = h;
            plo[j] = (__bf16)(p[j] - (float)h);
        }
#pragma unroll
        for (int dt = 0; dt < 4; dt++) {
            bf16x8 aop;
            memcpy(&aop, rv[dt], 16);
            f32x4 c = acc_o[28 + dt];
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, phi, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, plo, c, 0, 0, 0);
            acc_o[28 + dt] = c;
        }
    }
}

// The query and the output accumulator stay in AGPRs across tiles (the MFMAs
// read and write them there); VGPRs hold the per-tile work.
__device__ __forceinline__ void pin_state(bf16x8 (&qop)[16], f32x4 (&acc_o)[32]) {
#pragma unroll
    for (int k = 0; k < 16; k++) asm volatile("" : "+a"(qop[k]));
#pragma unroll
    for (int k = 0; k < 32; k++) asm volatile("" : "+a"(acc_o[k]));
}

// One workgroup = (sequence b, head block hb of G x 16 heads, split); see Geo
// for how its four waves share the split's tiles.  At the end the T streams'
// states of each head group are merged through LDS and the workgroup writes
// the split's normalised output and log-sum-exp (or the final bf16 result).
template <int G>
__global__ __launch_bounds__(64 * kWaves, 1) void smla_decode_kernel(DecodeArgs a) {
    using Ge = Geo<G>;
    constexpr int T = Ge::T, NS = Ge::NS;
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[Ge::kLds];
    lds_u8* const lds = (lds_u8*)lds_raw;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qg = lane >> 4;                  // lane group 0..3
    const int ln = lane & 15;                  // head column of the 16x16 tiles
    const int strm = wave / G;                 // tile stream
    const int hgl = wave % G;                  // head group within the workgroup

    int bid = blockIdx.x;
    if (a.xcd_remap) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
    const int split = bid % a.nsplit;
    bid /= a.nsplit;
    const int hb = bid % a.n_hb;
    const int b = bid / a.n_hb;

    const int head = 16 * (G * hb + hgl) + ln;
    const int t_begin = split * a.chunk;
    const int n_ent = max(min(a.topk, t_begin + a.chunk) - t_begin, 0);
    const int ntiles = (n_ent + kTile - 1) / kTile;
    const int seqlen = a.seqlens[b];
    const i32x4 rsrc = row_rsrc(a.kv + (int64_t)b * a.kv_seq_stride * kRowBytes, a.seq_bytes);
    const int32_t* idx_b = a.idx + (int64_t)b * a.topk + t_begin;

    // ---- the query of this lane's head as the B operand of S^T = K . Q^T
    // (k-slot order matches the K reads: lane group q takes columns 16q..16q+15
    // of every 64-column group, 8 per K-step, and rope columns 16q..16q+15).
    // Loaded after the first tile's gathers are issued; pin_state then makes
    // the compiler wait for it once, before the tile loop.
    bf16x8 qop[16];
    auto load_query = [&]() {
        const uint16_t* qh = a.q + ((int64_t)b * a.heads + head) * kLatent;
#pragma unroll
        for (int g = 0; g < 7; g++)
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
                qop[2 * g + ks] = as_bf16x8(*(const u32x4*)(qh + 64 * g + 16 * qg + 8 * ks));
        qop[14] = as_bf16x8(*(const u32x4*)(qh + kNope + 16 * qg));
        qop[15] = as_bf16x8(*(const u32x4*)(qh + kNope + 16 * qg + 8));
    };

    f32x4 acc_o[32];
#pragma unroll
    for (int i = 0; i < 32; i++) acc_o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // base of the exponentials for this lane's head (log2 units)
    float l_run = 0.f;         // partial sum of weights over this lane's tokens

    if constexpr (G == 1) {
        // ---- independent waves: tiles wave, wave + 4, ...; rows one tile ahead
        const int my_n = wave < ntiles ? (ntiles - 1 - wave) / kWaves + 1 : 0;
        lds_u8* my_lds = lds + wave * NS * kSlot;
        const uint32_t my_lds_addr = (uint32_t)(uintptr_t)my_lds;
        auto tile_row = [&](int i) -> int {   // sanitised row of token (lane & 31) of tile i
            const int e = (wave + kWaves * i) * kTile + (lane & 31);
            int row = -1;
            if (e < n_ent) {
                row = idx_b[e];
                if (row < 0 || row >= seqlen) row = -1;
            }
            return row;
        };
        int row_cur = -1, row_next = -1;
        if (my_n > 0) {
            row_cur = tile_row(0);
            issue_tile_own(row_cur, rsrc, my_lds_addr, lane);
        }
        load_query();
        pin_state(qop, acc_o);
        if (my_n > 1) row_next = tile_row(1);
        for (int i = 0; i < my_n; i++) {
            pin_state(qop, acc_o);
            wait_vmcnt<0>();   // tile i is in its slot; the rows of tile i + 1 are in registers
            if (i + 1 < my_n) issue_tile_own(row_next, rsrc, my_lds_addr + ((i + 1) & 1) * kSlot, lane);
            const int row_after = i + 2 < my_n ? tile_row(i + 2) : -1;
            const uint64_t vmask = __ballot(lane < kTile && row_cur >= 0);
            compute_tile(my_lds + (i & 1) * kSlot, vmask, qop, acc_o, m_run, l_run, lane, a.logit_factor);
            row_cur = row_next;
            row_next = row_after;
        }
        wait_vmcnt<0>();
    } else {
        // ---- shared tiles: sanitised index table, NS-slot ring per stream
        lds_i32* idx_s = (lds_i32*)(lds + Ge::kIdx);
        for (int i = threadIdx.x; i < ntiles * kTile; i += 64 * kWaves) {
            int row = -1;
            if (i < n_ent) {
                row = idx_b[i];
                if (row < 0 || row >= seqlen) row = -1;
            }
            idx_s[i] = row;
        }
        __syncthreads();
        const int nsteps = (ntiles + T - 1) / T;
        lds_u8* ring = lds + strm * NS * kSlot;
        const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
        const uint32_t dummy_addr = (uint32_t)(uintptr_t)(lds + Ge::kDummy);
        auto issue_step = [&](int step) {
            const int tile = strm + T * step;
            const bool live = tile < ntiles;
            lds_ci32* rows = idx_s + (live ? tile : 0) * kTile;
            const uint32_t slot = ring_addr + (step % NS) * kSlot;
            issue_tile_shared<G, Ge::L>(rows, live, rsrc, slot, dummy_addr, hgl, lane);
        };
        issue_step(0);
        load_query();
        pin_state(qop, acc_o);
#pragma unroll
        for (int st = 1; st < NS - 1; st++) issue_step(st);
        // at least one step even for an empty split (it computes a zero-filled
        // slot with no kept token), so the accumulators have a single path
        int step = 0;
        do {
            pin_state(qop, acc_o);
            wait_vmcnt<(NS - 2) * Ge::L>();   // this wave's gathers of this step's tile have landed
            lds_barrier();                    // ... and everyone's; the previous step's slot is free
            issue_step(step + NS - 1);
            // a stream past the end of the chunk (G = 2, last step) computes its
            // zero-filled slot with no kept token, which changes nothing
            const int tile = strm + T * step;
            const bool live = tile < ntiles;
            const uint64_t vmask = __ballot(live && lane < kTile && idx_s[(live ? tile : 0) * kTile + (lane & 31)] >= 0);
            compute_tile(ring + (step % NS) * kSlot, vmask, qop, acc_o, m_run, l_run, lane, a.logit_factor);
        } while (++step < nsteps);
        wait_vmcnt<0>();   // trailing no-op loads of the ring
    }

    // ---------------- merge of the T streams of each head group
    const float l_tot = lanegroup_sum(l_run);
    float M = m_run, L = l_tot;
    if constexpr (T > 1) {
        __syncthreads();   // every wave is done with the ring (the merge reuses it)
        lds_f32* stat = (lds_f32*)(lds + Ge::kStat);   // [wave][max 16 | sum 16]
        if (lane < 16) {
            stat[wave * 32 + lane] = m_run;
            stat[wave * 32 + 16 + lane] = l_tot;
        }
        __syncthreads();
        M = -INFINITY;
#pragma unroll
        for (int s2 = 0; s2 < T; s2++) M = fmaxf(M, stat[(s2 * G + hgl) * 32 + ln]);
        const float Ms0 = M == -INFINITY ? 0.f : M;
        L = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < T; s2++)
            L += __builtin_amdgcn_exp2f(stat[(s2 * G + hgl) * 32 + ln] - Ms0) * stat[(s2 * G + hgl) * 32 + 16 + ln];
        const float aw = __builtin_amdgcn_exp2f(m_run - Ms0);
        lds_f32x4* part = (lds_f32x4*)(lds + wave * kAccBytes);
#pragma unroll
        for (int i = 0; i < 32; i++) part[i * 64 + lane] = acc_o[i] * aw;
        __syncthreads();
    }

    // stream s finishes accumulator blocks [s * 32 / T, (s + 1) * 32 / T) of its
    // head group; block i holds columns 16i + 4qg + j for head ln
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const float lse2 = L > 0.f ? M + log2f(L) : -INFINITY;
    const int64_t bh = (int64_t)b * a.heads + head;
    const bool final_out = a.nsplit == 1 && !a.force_partials;
    auto block_sum = [&](int i) -> f32x4 {
        if constexpr (T > 1) {
            f32x4 v = ((lds_cf32x4*)(lds + hgl * kAccBytes))[i * 64 + lane];
#pragma unroll
            for (int s2 = 1; s2 < T; s2++) v += ((lds_cf32x4*)(lds + (s2 * G + hgl) * kAccBytes))[i * 64 + lane];
            return v;
        } else {
            return acc_o[i];
        }
    };
    const int i0 = T == 1 ? 0 : strm * (32 / T);   // static index when T == 1
    if (final_out) {
        uint16_t* o = a.out + bh * kLatent + 4 * qg;
#pragma unroll
        for (int ii = 0; ii < 32 / T; ii++) {
            const f32x4 v = block_sum(i0 + ii);
            u32x2 w;
            w[0] = pack_bf16x2(v[0] * inv, v[1] * inv);
            w[1] = pack_bf16x2(v[2] * inv, v[3] * inv);
            *(u32x2*)(o + 16 * (i0 + ii)) = w;
        }
    } else {
        float* o = a.o_part + (bh * a.nsplit + split) * kLatent + 4 * qg;
#pragma unroll
        for (int ii = 0; ii < 32 / T; ii++) *(f32x4*)(o + 16 * (i0 + ii)) = block_sum(i0 + ii) * inv;
    }
    if (strm == 0 && qg == 0) {
        if (final_out) a.lse[bh] = lse2 * kLn2;
        else a.lse_part[bh * a.nsplit + split] = lse2 * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Shared tiles with the latent split across wave pairs: G = 2 or 4 head
// groups of 16 heads per workgroup and 2G waves.  Wave 2h + d serves head
// group h for half d of the latent: d = 0 takes nope groups 0..3 (columns
// 0..255), d = 1 nope groups 4..6 and the rope (columns 256..511).  Each wave
// therefore holds half of its heads' query (32 registers) and half of their
// output accumulator (64 registers), so that two waves share a SIMD and hide
// each other's latencies.  The two halves of a pair exchange their partial
// logits through LDS; the loop is software-pipelined so that one workgroup
// barrier per tile suffices: iteration j finishes tile j - 1 (partner's
// partial logits, softmax, PV) and starts tile j (QK partial), and the tile
// slot is refilled two iterations after its QK.
template <int G>
struct SplitGeo {
    static constexpr int W = 2 * G;                                           // waves
    static constexpr int NS = G == 4 ? 5 : 6;                                 // ring slots
    static constexpr int L = (kRowGathers + kScaleGathers + W - 1) / W;      // gathers per wave per tile
    static constexpr int kIdx = NS * kSlot;                                   // index table
    static constexpr int kDummy = kIdx + kMaxChunk * 4;                       // no-op gather target
    static constexpr int kXs = kDummy + 1024;                                 // [2][W][64 lanes][8] partial logits
    static constexpr int kLds = kXs + 2 * W * 64 * 8 * 4;
    static_assert(kLds <= 160 * 1024, "LDS budget of one gfx950 workgroup");
    static_assert(L * W <= kRowGathers + kScaleGathers + 1, "at most one no-op gather per tile");
    static_assert(NS >= 3, "a slot is read by the QK of one iteration and the PV of the next");
};

// Partial logits S^T of latent half dh for the 32 tokens of a tile: sp[tt]
// holds tokens 16tt + 4q + j (j = 0..3) for head ln, summed over the half's
// units with the group scales applied.  Units 0..2 are nope groups 4dh + u;
// unit 3 is nope group 3 (dh = 0) or the rope (dh = 1, unscaled).  Both
// halves run the same instruction stream apart from unit 3.  qh[2u + ks]: the
// query columns of unit u for K-step ks (8 columns per lane group q:
// 16q + 8ks.. of the unit's 64 columns).
__device__ __forceinline__ void qk_half(const lds_u8* st, int dh, const bf16x8 (&qh)[8], int lane, f32x4 (&sp)[2]) {
    const int qg = lane >> 4, ln = lane & 15;
    const lds_u8* kbase = opaque(st + ln * kRowLds + 16 * qg + 256 * dh);                // K rows, this half
    lds_cf32* sT = (lds_cf32*)opaque(st + kScaleTable + 16 * qg + 512 * dh);            // scales of groups 4dh..
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
        const lds_u8* krow = kbase + 16 * tt * kRowLds;
        u32x4 raw[4];
        u32x4 rr[2];
#pragma unroll
        for (int u = 0; u < 3; u++) raw[u] = *(lds_cu32x4*)(krow + 64 * u);
        if (dh == 0) {
            raw[3] = *(lds_cu32x4*)(krow + 64 * 3);
        } else {
            // rope columns 16q..16q+15 sit at LDS bytes 448 + 32q of the row (krow is 256 + 16q)
            rr[0] = *(lds_cu32x4*)(krow + kLdsRope - 256 + 16 * qg);
            rr[1] = *(lds_cu32x4*)(krow + kLdsRope - 256 + 16 * qg + 16);
        }
        f32x4 acc[4];
#pragma unroll
        for (int u = 0; u < 3; u++)
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw[u][0], raw[u][1]), qh[2 * u],
                                                             f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 3; u++)
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw[u][2], raw[u][3]), qh[2 * u + 1],
                                                             acc[u], 0, 0, 0);
        f32x4 v;
        if (dh == 0) {
            acc[3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw[3][0], raw[3][1]), qh[6],
                                                             f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            acc[3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw[3][2], raw[3][3]), qh[7], acc[3],
                                                             0, 0, 0);
            v = *(lds_cf32x4*)(sT + 3 * kTile + 16 * tt) * acc[3];
        } else {
            v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rr[0]), qh[6], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rr[1]), qh[7], v, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 3; u++) v += *(lds_cf32x4*)(sT + u * kTile + 16 * tt) * acc[u];
        sp[tt] = v;
    }
}

// Online softmax (log2 domain, lazy rescale) of one tile's logits s (tokens
// 16tt + 4q + j for head ln); masked tokens get -inf.  Returns the weights in
// k-slot order (tokens 4q+j, then 16+4q+j) and rescales acc when the base moves.
template <int NACC>
__device__ __forceinline__ void softmax_tile(f32x4 (&s)[2], uint64_t vmask, float logit_factor, int lane,
                                             f32x4 (&acc)[NACC], float& m_run, float& l_run, float (&p)[8]) {
    const int qg = lane >> 4;
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float z = s[tt][j] * logit_factor;
            s[tt][j] = ((vmask >> (16 * tt + 4 * qg + j)) & 1) ? z : -INFINITY;
        }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = lanegroup_max(mx);
    const bool need = mx > m_run + kTau;
    if (__any(need)) {
        const float m_new = need ? mx : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        // the first kept tokens only set the base: the accumulators are still zero
        if (__any(m_run != -INFINITY)) {
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < NACC; i++) acc[i] *= alpha;
        }
        m_run = m_new;
    }
    const float base = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        p[j] = __builtin_amdgcn_exp2f(s[j >> 2][j & 3] - base);
        l_run += p[j];
    }
}

// O^T += V^T . P^T over latent half dh's columns: acc[4u + cb] holds unit u,
// column block cb (units as in qk_half: nope groups 4dh + u, and unit 3 =
// nope group 3 or the rope).
__device__ __forceinline__ void pv_half(const lds_u8* st, int dh, const float (&p)[8], int lane, f32x4 (&acc)[16]) {
    const int qg = lane >> 4, ln = lane & 15;
    lds_cf32* sT = (lds_cf32*)opaque(st + kScaleTable + 16 * qg + 512 * dh);
    // V^T operands: tr8 source rows, lane 16q + j supplies token slot_token(8q + j/2),
    // byte half j%2; the reads of unit u + 1 are issued before unit u is converted
    const lds_u8* tr_row = opaque(st + slot_token(8 * qg + (ln >> 1)) * kRowLds + 8 * (ln & 1) + 256 * dh);
    const int nnope = dh == 0 ? 4 : 3;   // nope units of this half
    i32x2 vraw[2][4];
    f32x4 sv[2][2];
    auto load_unit = [&](int u, int buf) {
#pragma unroll
        for (int cb = 0; cb < 4; cb++)
            vraw[buf][cb] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(tr_row + 64 * u + 16 * cb));
        sv[buf][0] = *(lds_cf32x4*)(sT + u * kTile);
        sv[buf][1] = *(lds_cf32x4*)(sT + u * kTile + 16);
    };
    load_unit(0, 0);
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int cur = u & 1;
        if (u == 3 && nnope == 3) break;
        if (u + 1 < 3 || (u + 1 == 3 && nnope == 4)) load_unit(u + 1, cur ^ 1);
        // weights fp16(p * scale_g); exact fp8 -> fp16 value codes
        f16x8 bop;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            bop[j] = (_Float16)(p[j] * sv[cur][0][j]);
            bop[4 + j] = (_Float16)(p[4 + j] * sv[cur][1][j]);
        }
#pragma unroll
        for (int cb = 0; cb < 4; cb++)
            acc[4 * u + cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                codes_to_f16((uint32_t)vraw[cur][cb][0], (uint32_t)vraw[cur][cb][1]), bop, acc[4 * u + cb], 0, 0, 0);
    }
    if (dh == 1) {
        // rope V^T via tr16: lane 16q + 4r + c supplies slot_token(8q + r), then
        // slot_token(8q + 4 + r), columns 4c..4c+3 of each 16-column block; bf16
        // values as stored, weights split into bf16 high and low parts
        const int col = 8 * (ln & 3);
        const lds_u8* r0 = opaque(st + slot_token(8 * qg + (ln >> 2)) * kRowLds + kLdsRope + col);
        const lds_u8* r1 = opaque(st + slot_token(8 * qg + 4 + (ln >> 2)) * kRowLds + kLdsRope + col);
        bf16x8 phi, plo;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const __bf16 h = (__bf16)p[j];
            phi[j] = h;
            plo[j] = (__bf16)(p[j] - (float)h);
        }
#pragma unroll
        for (int dt = 0; dt < 4; dt++) {
            s16x4 rv[2];
            rv[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(r0 + 32 * dt));
            rv[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(r1 + 32 * dt));
            bf16x8 aop;
            memcpy(&aop, rv, 16);
            f32x4 c = acc[12 + dt];
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, phi, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, plo, c, 0, 0, 0);
            acc[12 + dt] = c;
        }
    }
}

template <int G>
__device__ __forceinline__ void split_loop(const DecodeArgs& a, lds_u8* lds, int wave, int dh, int lane, int ntiles,
                                           lds_ci32* idx_s, i32x4 rsrc, const bf16x8 (&qh_in)[8],
                                           f32x4 (&acc)[16], float& m_run, float& l_run) {
    using Ge = SplitGeo<G>;
    constexpr int W = Ge::W, NS = Ge::NS, L = Ge::L;
    bf16x8 qh[8];
#pragma unroll
    for (int k = 0; k < 8; k++) qh[k] = qh_in[k];
    const uint32_t ring_addr = (uint32_t)(uintptr_t)lds;
    const uint32_t dummy_addr = (uint32_t)(uintptr_t)(lds + Ge::kDummy);
    lds_f32* xs = (lds_f32*)(lds + Ge::kXs);   // [buf][wave][lane][8]
    const int partner = wave ^ 1;
    auto issue = [&](int t) {
        const bool live = t < ntiles;
        issue_tile_shared<W, L>(idx_s + (live ? t : 0) * kTile, live, rsrc, ring_addr + (t % NS) * kSlot,
                                dummy_addr, wave, lane);
    };
#pragma unroll
    for (int t = 1; t < NS - 2; t++) issue(t);
    f32x4 sp[2];
    for (int j = 0; j <= ntiles; j++) {
        wait_vmcnt<(NS - 3) * L>();   // this wave's gathers of tile j have landed
        lds_barrier();                // ... and everyone's; tile j - 2's slot and xs[j & 1] are free
        issue(j + NS - 2);
        float p[8];
        if (j >= 1) {
            // logits of tile j - 1: both halves, summed in the same order in both waves
            lds_cf32* xo = xs + (((j - 1) & 1) * W + partner) * 512 + 8 * lane;
            const f32x4 o0 = *(lds_cf32x4*)xo;
            const f32x4 o1 = *(lds_cf32x4*)(xo + 4);
            f32x4 s[2];
            s[0] = dh == 0 ? sp[0] + o0 : o0 + sp[0];
            s[1] = dh == 0 ? sp[1] + o1 : o1 + sp[1];
            const uint64_t vmask = __ballot(lane < kTile && idx_s[(j - 1) * kTile + (lane & 31)] >= 0);
            softmax_tile<16>(s, vmask, a.logit_factor, lane, acc, m_run, l_run, p);
        }
        if (j >= 1) pv_half(lds + ((j - 1) % NS) * kSlot, dh, p, lane, acc);
        __builtin_amdgcn_sched_barrier(0);   // register budget: PV's operands die before QK's are read
        if (j < ntiles) {
            qk_half(lds + (j % NS) * kSlot, dh, qh, lane, sp);
            lds_f32* xm = xs + ((j & 1) * W + wave) * 512 + 8 * lane;
            *(lds_f32x4*)xm = sp[0];
            *(lds_f32x4*)(xm + 4) = sp[1];
        }
    }
    wait_vmcnt<0>();   // trailing no-op loads of the ring
}

template <int G>
__global__ __launch_bounds__(128 * G, 1) void smla_decode_split_kernel(DecodeArgs a) {
    using Ge = SplitGeo<G>;
    constexpr int W = Ge::W;
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[Ge::kLds];
    lds_u8* const lds = (lds_u8*)lds_raw;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qg = lane >> 4;
    const int ln = lane & 15;
    const int dh = wave & 1;                   // latent half
    const int hgl = wave >> 1;                 // head group within the workgroup

    int bid = blockIdx.x;
    if (a.xcd_remap) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
    const int split = bid % a.nsplit;
    bid /= a.nsplit;
    const int hb = bid % a.n_hb;
    const int b = bid / a.n_hb;

    const int head = 16 * (G * hb + hgl) + ln;
    const int t_begin = split * a.chunk;
    const int n_ent = max(min(a.topk, t_begin + a.chunk) - t_begin, 0);
    const int ntiles = (n_ent + kTile - 1) / kTile;
    const int seqlen = a.seqlens[b];
    const i32x4 rsrc = row_rsrc(a.kv + (int64_t)b * a.kv_seq_stride * kRowBytes, a.seq_bytes);
    const int32_t* idx_b = a.idx + (int64_t)b * a.topk + t_begin;

    // ---- sanitised index table of the split's chunk
    lds_i32* idx_s = (lds_i32*)(lds + Ge::kIdx);
    for (int i = threadIdx.x; i < ntiles * kTile; i += 64 * W) {
        int row = -1;
        if (i < n_ent) {
            row = idx_b[i];
            if (row < 0 || row >= seqlen) row = -1;
        }
        idx_s[i] = row;
    }
    __syncthreads();
    {
        const bool live = ntiles > 0;
        issue_tile_shared<W, Ge::L>(idx_s, live, rsrc, (uint32_t)(uintptr_t)lds,
                                    (uint32_t)(uintptr_t)(lds + Ge::kDummy), wave, lane);
    }

    // ---- this half of the query as the B operand of S^T = K . Q^T (k-slot
    // order matches the K reads: lane group q takes columns 16q..16q+15 of
    // every 64-column group, 8 per K-step, and rope columns 16q..16q+15)
    bf16x8 qh[8];
    {
        // units 0..2: nope groups 4dh + u; unit 3: nope group 3 (dh = 0) or the rope
        const uint16_t* qrow = a.q + ((int64_t)b * a.heads + head) * kLatent;
        const uint16_t* qhalf = qrow + 256 * dh;
#pragma unroll
        for (int u = 0; u < 3; u++)
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
                qh[2 * u + ks] = as_bf16x8(*(const u32x4*)(qhalf + 64 * u + 16 * qg + 8 * ks));
        const uint16_t* q3 = dh == 0 ? qrow + 64 * 3 : qrow + kNope;
        qh[6] = as_bf16x8(*(const u32x4*)(q3 + 16 * qg));
        qh[7] = as_bf16x8(*(const u32x4*)(q3 + 16 * qg + 8));
    }
    f32x4 acc[16];
#pragma unroll
    for (int i = 0; i < 16; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the query must have landed before the tile loop (one wait, here)
#pragma unroll
    for (int k = 0; k < 8; k++) asm volatile("" : "+v"(qh[k]));
    float m_run = -INFINITY, l_run = 0.f;
    split_loop<G>(a, lds, wave, dh, lane, ntiles, idx_s, rsrc, qh, acc, m_run, l_run);

    // ---- this half of the split's output: block i holds columns 256 dh + 16i + 4qg + j
    const float L = lanegroup_sum(l_run);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const float lse2 = L > 0.f ? m_run + log2f(L) : -INFINITY;
    const int64_t bh = (int64_t)b * a.heads + head;
    if (a.nsplit == 1 && !a.force_partials) {
        uint16_t* o = a.out + bh * kLatent + 256 * dh + 4 * qg;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[i][0] * inv, acc[i][1] * inv);
            w[1] = pack_bf16x2(acc[i][2] * inv, acc[i][3] * inv);
            *(u32x2*)(o + 16 * i) = w;
        }
        if (dh == 0 && qg == 0) a.lse[bh] = lse2 * kLn2;
    } else {
        float* o = a.o_part + (bh * a.nsplit + split) * kLatent + 256 * dh + 4 * qg;
#pragma unroll
        for (int i = 0; i < 16; i++) *(f32x4*)(o + 16 * i) = acc[i] * inv;
        if (dh == 0 && qg == 0) a.lse_part[bh * a.nsplit + split] = lse2 * kLn2;
    }
}

// Log-sum-exp merge: one wave per (b, h), 8 columns per lane.  The split
// log-sum-exps are wave-uniform (scalar loads); the partial outputs are read
// four splits at a time with all loads issued before they are used, so every
// wave keeps eight 16-byte loads in flight.  An empty split (lse = -inf) has
// weight exp(-inf) = 0 and a zero partial.
__global__ __launch_bounds__(256) void smla_combine_kernel(const float* o_part, const float* lse_part,
                                                           int32_t rows, int32_t nsplit,
                                                           uint16_t* out, float* lse) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const float* lp = lse_part + (int64_t)row * nsplit;
    float M = -INFINITY;
    for (int i = 0; i < nsplit; i++) M = fmaxf(M, lp[i]);
    const float Ms = M == -INFINITY ? 0.f : M;
    const float* src = o_part + (int64_t)row * nsplit * kLatent + 8 * lane;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    float W = 0.f;
    int i = 0;
    for (; i + 4 <= nsplit; i += 4) {
        f32x4 lo[4], hi[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            lo[k] = *(const f32x4*)(src + (i + k) * kLatent);
            hi[k] = *(const f32x4*)(src + (i + k) * kLatent + 4);
        }
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const float w = __expf(lp[i + k] - Ms);
            W += w;
            acc0 += w * lo[k];
            acc1 += w * hi[k];
        }
    }
    for (; i < nsplit; i++) {
        const f32x4 lo = *(const f32x4*)(src + i * kLatent);
        const f32x4 hi = *(const f32x4*)(src + i * kLatent + 4);
        const float w = __expf(lp[i] - Ms);
        W += w;
        acc0 += w * lo;
        acc1 += w * hi;
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    u32x4 pk;
    pk[0] = pack_bf16x2(acc0[0] * inv, acc0[1] * inv);
    pk[1] = pack_bf16x2(acc0[2] * inv, acc0[3] * inv);
    pk[2] = pack_bf16x2(acc1[0] * inv, acc1[1] * inv);
    pk[3] = pack_bf16x2(acc1[2] * inv, acc1[3] * inv);
    *(u32x4*)(out + (int64_t)row * kLatent + 8 * lane) = pk;
    if (lane == 0) lse[row] = W > 0.f ? M + logf(W) : -INFINITY;
}

// ---------------------------------------------------------------------------
// host side

struct Plan {
    int g;        // 16-head groups per workgroup (1, 2 or 4)
    int n_hb;     // head blocks (workgroups per sequence and split)
    int nsplit;
    int chunk;    // list entries per split (multiple of kTile)
};

// Rows of one sequence are addressed by 32-bit byte offsets below 2^31.
constexpr int64_t kMaxSeqStride = ((int64_t)1 << 31) / kRowBytes;

bool shape_ok(const smla_shape* s) {
    return s && s->batch >= 0 && s->num_heads >= 0 && s->num_heads % 16 == 0 &&
           s->num_heads <= 256 && s->topk >= 0 && s->num_splits >= 0 && s->kv_seq_stride >= 1 &&
           s->kv_seq_stride <= kMaxSeqStride;
}

constexpr int kComputeUnits = 256;   // MI355X; one workgroup per compute unit

// Split count when the caller leaves it to the library.  A workgroup's time is
// taken as (tile steps + 1) tile times, where a step is T tiles of the split
// (T = 4 / g), a launch as that times the number of rounds of kComputeUnits
// workgroups, and any split adds one tile time for the partials and the
// combine.  Ties go to fewer splits.  min_ns bounds the split size from below.
int choose_splits(int base, int tiles, int t_streams, int min_ns) {
    if (base <= 0 || tiles <= 1) return 1;
    int best = 1;
    long best_cost = -1;
    for (int ns = min_ns; ns <= tiles; ns++) {
        const int per_block = (tiles + ns - 1) / ns;
        if (ns > min_ns && (tiles + per_block - 1) / per_block < ns) continue;   // same chunks as fewer splits
        const long rounds = ((long)base * ns + kComputeUnits - 1) / kComputeUnits;
        const long cost = rounds * ((per_block + t_streams - 1) / t_streams + 1) + (ns > 1 ? 1 : 0);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = ns;
        }
    }
    return best;
}

Plan make_plan(const smla_shape* s) {
    Plan p;
    const int n_hg = s->num_heads / 16;
    // shared tiles pay for themselves once there are enough (sequence, head
    // block) pairs that few splits fill the chip; otherwise the per-wave mode
    // keeps the split partials (and the combine) small
    const int64_t pairs4 = (int64_t)s->batch * (n_hg / 4), pairs2 = (int64_t)s->batch * (n_hg / 2);
    p.g = n_hg % 4 == 0 && pairs4 >= 64 ? 4 : n_hg % 2 == 0 && pairs2 >= 64 ? 2 : 1;
    p.n_hb = n_hg / p.g;
    const int tiles = (s->topk + kTile - 1) / kTile;
    // shared-tile workgroups keep their chunk's list entries in LDS
    const int min_ns = p.g > 1 ? (s->topk + kMaxChunk - 1) / kMaxChunk : 1;
    int ns = s->num_splits;
    if (ns == 0) ns = choose_splits(s->batch * p.n_hb, tiles, kWaves / p.g, min_ns > 0 ? min_ns : 1);
    if (ns < min_ns) ns = min_ns;
    if (ns > tiles) ns = tiles;
    if (ns < 1) ns = 1;
    const int per = (s->topk + ns - 1) / ns;
    p.chunk = ((per + kTile - 1) / kTile) * kTile;
    if (p.chunk == 0) p.chunk = kTile;
    p.nsplit = (s->topk + p.chunk - 1) / p.chunk;
    if (p.nsplit < 1) p.nsplit = 1;
    return p;
}

size_t workspace_for(const smla_shape* s, const Plan& p) {
    if (p.nsplit <= 1) return 0;
    const size_t rows = (size_t)s->batch * s->num_heads * p.nsplit;
    size_t o_bytes = rows * kLatent * sizeof(float);
    o_bytes = (o_bytes + 255) & ~(size_t)255;
    return o_bytes + ((rows * sizeof(float) + 255) & ~(size_t)255);
}

smla_status device_check() {
    int dev = -1;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return SMLA_ERR_NO_DEVICE;
    }
    if (hipGetDevice(&dev) != hipSuccess) return SMLA_ERR_HIP;
    static int checked[64] = {0};   // 0 unknown, 1 ok, 2 unsupported
    if (dev < 0 || dev >= 64) return SMLA_ERR_HIP;
    if (checked[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SMLA_ERR_HIP;
        checked[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    return checked[dev] == 1 ? SMLA_OK : SMLA_ERR_UNSUPPORTED;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace

extern "C" {

int32_t smla_num_splits(const smla_shape* shape) {
    if (!shape_ok(shape)) return -1;
    return make_plan(shape).nsplit;
}

size_t smla_workspace_bytes(const smla_shape* shape) {
    if (!shape_ok(shape)) return 0;
    return workspace_for(shape, make_plan(shape));
}

const char* smla_status_str(smla_status s) {
    switch (s) {
        case SMLA_OK: return "ok";
        case SMLA_ERR_NULL: return "required pointer is NULL";
        case SMLA_ERR_SHAPE: return "invalid shape";
        case SMLA_ERR_UNSUPPORTED: return "device is not gfx950";
        case SMLA_ERR_WORKSPACE: return "workspace missing or too small";
        case SMLA_ERR_HIP: return "HIP runtime error";
        case SMLA_ERR_ALIGN: return "pointer misaligned";
        case SMLA_ERR_NO_DEVICE: return "no HIP device";
    }
    return "unknown status";
}

smla_status sparse_mla_combine(const float* o_part, const float* lse_part, int32_t batch,
                               int32_t num_heads, int32_t num_splits, void* out, float* lse,
                               void* stream) {
    if (!o_part || !lse_part || !out || !lse) return SMLA_ERR_NULL;
    if (batch < 0 || num_heads < 0 || num_splits < 1) return SMLA_ERR_SHAPE;
    if (!aligned(o_part, 16) || !aligned(out, 16) || !aligned(lse_part, 4) || !aligned(lse, 4))
        return SMLA_ERR_ALIGN;
    smla_status st = device_check();
    if (st != SMLA_OK) return st;
    const int rows = batch * num_heads;
    if (rows == 0) return SMLA_OK;
    hipLaunchKernelGGL(smla_combine_kernel, dim3((rows + 3) / 4), dim3(256), 0, (hipStream_t)stream,
                       o_part, lse_part, rows, num_splits, (uint16_t*)out, lse);
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

static smla_status prepare(const void* q, const void* kv_cache, const int32_t* topk_idx,
                           const int32_t* seqlens, float scale, const smla_shape* shape,
                           DecodeArgs* a, Plan* p, bool* nothing) {
    *nothing = false;
    if (!shape) return SMLA_ERR_NULL;
    if (!shape_ok(shape)) return SMLA_ERR_SHAPE;
    if (shape->batch == 0 || shape->num_heads == 0) {   // nothing to touch
        *nothing = true;
        return SMLA_OK;
    }
    if (!q || !seqlens) return SMLA_ERR_NULL;
    if (shape->topk > 0 && (!kv_cache || !topk_idx)) return SMLA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(topk_idx, 4) || !aligned(seqlens, 4))
        return SMLA_ERR_ALIGN;
    *p = make_plan(shape);
    memset(a, 0, sizeof(*a));
    a->q = (const uint16_t*)q;
    a->kv = (const uint8_t*)kv_cache;
    a->idx = topk_idx;
    a->seqlens = seqlens;
    a->kv_seq_stride = shape->kv_seq_stride;
    a->logit_factor = scale * kLog2e;
    a->batch = shape->batch;
    a->heads = shape->num_heads;
    a->topk = shape->topk;
    a->nsplit = p->nsplit;
    a->chunk = p->chunk;
    a->n_hb = p->n_hb;
    a->seq_bytes = (uint32_t)(shape->kv_seq_stride * kRowBytes);
    return SMLA_OK;
}

static smla_status launch(const DecodeArgs& a, const Plan& p, hipStream_t hs) {
    const int grid = a.batch * p.n_hb * p.nsplit;
    DecodeArgs args = a;
    args.xcd_remap = (grid % 8 == 0) ? 1 : 0;
    switch (p.g) {
        case 4: hipLaunchKernelGGL(smla_decode_split_kernel<4>, dim3(grid), dim3(128 * 4), 0, hs, args); break;
        case 2: hipLaunchKernelGGL(smla_decode_split_kernel<2>, dim3(grid), dim3(128 * 2), 0, hs, args); break;
        default: hipLaunchKernelGGL(smla_decode_kernel<1>, dim3(grid), dim3(64 * kWaves), 0, hs, args); break;
    }
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

smla_status sparse_mla_decode(const void* q, const void* kv_cache, const int32_t* topk_idx,
                              const int32_t* seqlens, float scale, void* out, float* lse,
                              const smla_shape* shape, void* workspace, size_t workspace_bytes,
                              void* stream) {
    DecodeArgs a;
    Plan p;
    bool nothing;
    smla_status st = prepare(q, kv_cache, topk_idx, seqlens, scale, shape, &a, &p, &nothing);
    if (st != SMLA_OK || nothing) return st;
    if (!out || !lse) return SMLA_ERR_NULL;
    if (!aligned(out, 16) || !aligned(lse, 4)) return SMLA_ERR_ALIGN;
    const size_t need = workspace_for(shape, p);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return SMLA_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return SMLA_ERR_ALIGN;
    }
    st = device_check();
    if (st != SMLA_OK) return st;
    a.out = (uint16_t*)out;
    a.lse = lse;
    if (p.nsplit > 1) {
        const size_t rows = (size_t)shape->batch * shape->num_heads * p.nsplit;
        a.o_part = (float*)workspace;
        a.lse_part = (float*)((char*)workspace + ((rows * kLatent * sizeof(float) + 255) & ~(size_t)255));
    }
    hipStream_t hs = (hipStream_t)stream;
    st = launch(a, p, hs);
    if (st != SMLA_OK) return st;
    if (p.nsplit > 1) {
        const int rws = shape->batch * shape->num_heads;
        hipLaunchKernelGGL(smla_combine_kernel, dim3((rws + 3) / 4), dim3(256), 0, hs, a.o_part,
                           a.lse_part, rws, p.nsplit, (uint16_t*)out, lse);
        if (hipGetLastError() != hipSuccess) return SMLA_ERR_HIP;
    }
    return SMLA_OK;
}

smla_status sparse_mla_decode_partials(const void* q, const void* kv_cache, const int32_t* topk_idx,
                                       const int32_t* seqlens, float scale, const smla_shape* shape,
                                       float* o_part, float* lse_part, void* stream) {
    DecodeArgs a;
    Plan p;
    bool nothing;
    smla_status st = prepare(q, kv_cache, topk_idx, seqlens, scale, shape, &a, &p, &nothing);
    if (st != SMLA_OK || nothing) return st;
    if (!o_part || !lse_part) return SMLA_ERR_NULL;
    if (!aligned(o_part, 16) || !aligned(lse_part, 4)) return SMLA_ERR_ALIGN;
    st = device_check();
    if (st != SMLA_OK) return st;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.force_partials = 1;
    return launch(a, p, (hipStream_t)stream);
}

int32_t smla_split_size(const smla_shape* shape) {
    if (!shape_ok(shape)) return -1;
    return make_plan(shape).chunk;
}

}  // extern "C"
