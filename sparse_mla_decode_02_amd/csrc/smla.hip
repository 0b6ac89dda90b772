// Sparse MLA decode for AMD CDNA4 (gfx950): split-K decode kernel, log-sum-exp
// combine kernel, the per-head ablation kernel, and the C ABI declared in
// include/smla.h.
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
//    into one (buffer_load_dwordx4 with the lds bit, 16 bytes per lane,
//    coalesced along the row) while it computes the current one from the
//    other, and never waits for another wave until the end.  A workgroup is
//    four such waves (one per SIMD, 152 KB of the 160 KB LDS) on the same
//    (sequence, head group, split); they take the split's tiles round robin
//    and merge their online-softmax states once, through LDS, at the end.
//  * Rows come from a cache contiguous per sequence (a buffer resource per
//    sequence, 32-bit row offsets, the range check zero-filling masked rows)
//    or from a paged pool of any size through a block table (64-bit
//    global_load_lds gathers, masked rows from a zero row); in either row
//    format, fp32 group scales (640-byte rows) or UE8M0 exponent bytes
//    (584-byte rows, expanded to the same fp32 scale table in LDS).
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
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <type_traits>


#include "../../include/smla.h"

namespace {

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
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
typedef __attribute__((address_space(3))) f32x2 lds_f32x2;
typedef __attribute__((address_space(3))) const f32x2 lds_cf32x2;
typedef __attribute__((address_space(3))) int32_t lds_i32;
typedef __attribute__((address_space(3))) const int32_t lds_ci32;
typedef __attribute__((address_space(3))) const uint32_t lds_cu32;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

// LDS tile slot.  The 36 16-byte pieces of a row (0..27 the fp8 codes, 28..35
// the rope) are stored in 18 blocks of 1 KB: block 2j + hh holds pieces
// 4j..4j+3 of the 16 rows in LDS positions 16hh..16hh+15, 64 bytes per row,
// piece 4j + c of position 16hh + ss at chunk c ^ ((ss >> 2) & 3).  One gather
// of 64 lanes x 16 bytes fills one block, i.e. 64 contiguous bytes of each of
// 16 rows (4 rows per quarter-wave: full 64-byte granules), with per-lane
// source offsets that differ between blocks only by an instruction immediate.
// The chunk swizzle puts the 16 rows read by one 16-lane group in distinct
// banks; the position of MFMA token t is lds_pos(t), which does the same for
// the 8 tokens of one transposed value read.  Then the tile's group scales,
// transposed to [group][position] (4 bytes each).
constexpr int kPiecesUsed = 36;                       // 28 code pieces + 8 rope pieces
constexpr int kCodePieces = 28;
constexpr int kScaleTable = kPiecesUsed * kTile * 16;  // scale table offset in a slot (18432)
constexpr int kSlot = kScaleTable + 8 * kTile * 4;    // 19456 bytes per tile slot
constexpr int kRowGathers = kPiecesUsed / 2;          // 18 row gathers of 64 lanes (one block each)
constexpr int kScaleGathers = 4;                      // 4-byte gathers of the scale table
constexpr int kWaves = 4;                             // waves per workgroup (one per SIMD)
constexpr int kAccBytes = 32 * 64 * 16;               // one wave's output accumulator (32 KB)
constexpr int kWaveLds = 2 * kSlot;                   // two tile slots per wave
constexpr int kLdsBytes = kWaves * kWaveLds;          // 152 KB

// Byte layout of a cache row in each format (include/smla.h).  Both keep the
// codes at 0..447 and the scales at 448; the rope follows the scales.
template <int F>
struct RowFormat;
template <>
struct RowFormat<SMLA_ROW_FP32_SCALES> {
    static constexpr int kBytes = SMLA_ROW_BYTES;        // 640
    static constexpr int kRopeOff = SMLA_ROPE_OFFSET;    // 480
};
template <>
struct RowFormat<SMLA_ROW_UE8M0_SCALES> {
    static constexpr int kBytes = SMLA_ROW_BYTES_UE8M0;      // 584
    static constexpr int kRopeOff = SMLA_ROPE_OFFSET_UE8M0;  // 456
};

// UE8M0 rows: the tile's 7 scale bytes per row are first gathered as two
// dwords per position (lane l: bytes 448 + 4 (l >> 5) .. + 3 of the row in
// position l & 31) into rows 4 and 5 of the scale table, then expanded in place
// into the fp32 table rows 0..6 before the tile is computed.
constexpr int kScaleRaw = kScaleTable + 4 * kTile * 4;

static_assert(kAccBytes + 32 * 4 <= kWaveLds, "a wave's accumulator and statistics fit in its own slots");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");

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

// LDS position of MFMA token t (an involution).  Tokens 4q..4q+3 and
// 16+4q..16+4q+3 (one transposed value read) then sit in positions whose
// 16-byte chunks fall in distinct banks, and each 16-token half still covers
// 16 positions with distinct banks.
__device__ __forceinline__ int lds_pos(int t) { return t ^ ((t & 16) >> 2); }

// Byte offset in a slot of bytes 8h..8h+7 (h = 0, 1) of piece p of the row in
// LDS position s (see the slot layout above).
__device__ __forceinline__ int piece_addr(int p, int s, int h = 0) {
    const int ss = s & 15;
    return 1024 * (2 * (p >> 2) + (s >> 4)) + 64 * ss + 16 * ((p & 3) ^ ((ss >> 2) & 3)) + 8 * h;
}

// Valid-token mask in MFMA token order from one in LDS-position order.
__device__ __forceinline__ uint64_t mask_by_token(uint64_t by_pos) {
    return (by_pos & 0xFFFFull) | ((by_pos & 0x0F0F0000ull) << 4) | ((by_pos & 0xF0F00000ull) >> 4);
}

// Buffer resource over one sequence's cache rows (gfx9 raw buffer, stride 0):
// a gather addresses a row by a 32-bit byte offset, and the hardware range
// check turns every offset at or past `bytes` into a load of zeros.  A masked
// list entry therefore uses row -1: its offset is negative, i.e. above 2^32
// minus the row bytes as an unsigned number, and it stages zeros (finite,
// contributes nothing).
__device__ __forceinline__ i32x4 row_rsrc(const uint8_t* base, uint32_t bytes) {
    const uint64_t p = (uint64_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(p >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
    r[3] = 0x00020000;
    return r;
}

// Byte offset of byte `off` (< row bytes) of cache row `row` (row in
// [-1, 2^23)) in format F, modulo 2^32.  Row -1 gives an offset above 2^32 minus
// the row bytes, out of range for every sequence.
template <int F>
__device__ __forceinline__ uint32_t row_offset(int row, uint32_t off) {
    return (uint32_t)__mul24(row, RowFormat<F>::kBytes) + off;
}

// 4-byte gather of one lane straight into LDS at lds_base + 4 * lane:
// buffer_load_dword with the lds bit; the LDS base goes through M0 and must be
// wave-uniform.  Written as inline assembly so that the compiler does not
// treat every later LDS read as dependent on every gather in flight: the
// ordering is explicit instead (wait_vmcnt before the destination is read).
// No memory clobber, for the same reason as the gathers below.
__device__ __forceinline__ void gather4(uint32_t voff, i32x4 rsrc, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "m0");
}

// 16-byte (4-byte) gathers with a constant byte offset kOff (< 4096) in the
// instruction; lane l writes lds_base + 16 l (+ 4 l).  The
// instruction offset moves the LDS destination as well as the source (checked
// on gfx950), so M0 is set kOff bytes lower to keep the destination at
// lds_base (which is at least kOff).  These carry no memory clobber, so that
// the compiler may schedule the compute's LDS reads of the other slot around
// them: the gathers only write a slot that nothing reads until the next
// wait_vmcnt, which is a compiler barrier.
template <int kOff>
__device__ __forceinline__ void gather16_at(uint32_t voff, i32x4 rsrc, uint32_t lds_base) {
    static_assert(kOff >= 0 && kOff < 4096, "buffer instruction offset");
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen offset:%3 lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base - kOff)), "n"(kOff)
                 : "m0");
}

template <int kOff>
__device__ __forceinline__ void gather4_at(uint32_t voff, i32x4 rsrc, uint32_t lds_base) {
    static_assert(kOff >= 0 && kOff < 4096, "buffer instruction offset");
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen offset:%3 lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base - kOff)), "n"(kOff)
                 : "m0");
}

// The same gathers from 64-bit per-lane addresses (paged pool, which may
// exceed the 4 GB that a buffer instruction's 32-bit offset reaches):
// global_load_lds_dword{,x4}; the LDS destination follows the same rule
// (M0 + instruction offset + 4 or 16 * lane, checked on gfx950).  There is no
// range check: a masked lane reads the zero row below instead.
template <int kOff>
__device__ __forceinline__ void gather16_global_at(const uint8_t* a, uint32_t lds_base) {
    static_assert(kOff >= 0 && kOff < 4096, "global instruction offset");
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off offset:%2"
                 :
                 : "v"(a), "s"(__builtin_amdgcn_readfirstlane(lds_base - kOff)), "n"(kOff)
                 : "m0");
}

template <int kOff>
__device__ __forceinline__ void gather4_global_at(const uint8_t* a, uint32_t lds_base) {
    static_assert(kOff >= 0 && kOff < 4096, "global instruction offset");
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off offset:%2"
                 :
                 : "v"(a), "s"(__builtin_amdgcn_readfirstlane(lds_base - kOff)), "n"(kOff)
                 : "m0");
}

// Source of the masked rows of a paged gather: a row of zeros (finite, adds
// nothing), as long as the largest row format.
__device__ __attribute__((aligned(64))) const uint8_t kZeroRow[SMLA_ROW_BYTES] = {0};

template <int K, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (K < N) {
        f(std::integral_constant<int, K>{});
        static_for<K + 1, N>(f);
    }
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
// It is also a compiler barrier for memory accesses: LDS reads of a slot that
// the gathers fill must not be moved above the wait for them.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}

// Workgroup barrier without a memory fence: only this wave's LDS operations are
// waited for, so gathers still in flight into other ring slots stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Block (sequence b, head block hb, split) of a decode workgroup: the XCD remap
// (remap_stride = gridDim.x / 8, or 0) gives consecutive logical blocks the
// same XCD, then the logical index splits as ((b * n_hb) + hb) * nsplit +
// split.  Split and head-block counts that are powers of two (the usual ones)
// take shifts and masks instead of the scalar division sequence (~50 scalar
// instructions per wave, issued before the first memory request).
__device__ __forceinline__ void block_coords(uint32_t bid, uint32_t remap_stride, int32_t nsplit, int32_t n_hb,
                                             int& split, int& hb, int& b) {
    if (remap_stride) bid = (bid & 7u) * remap_stride + (bid >> 3);
    const uint32_t ns = (uint32_t)nsplit, nh = (uint32_t)n_hb;
    uint32_t q;
    if ((ns & (ns - 1u)) == 0u) {
        split = (int)(bid & (ns - 1u));
        q = bid >> __builtin_ctz(ns);
    } else {
        split = (int)(bid % ns);
        q = bid / ns;
    }
    if ((nh & (nh - 1u)) == 0u) {
        hb = (int)(q & (nh - 1u));
        b = (int)(q >> __builtin_ctz(nh));
    } else {
        hb = (int)(q % nh);
        b = (int)(q / nh);
    }
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
    uint32_t seq_bytes;   // kv_seq_stride * row bytes (< 2^31): the range of a sequence's rows
    float logit_factor;   // scale * log2(e)
    int32_t batch, heads, topk, nsplit, chunk, n_hb;
    int32_t force_partials;   // write split partials even when nsplit == 1
    int32_t xcd_remap;        // host only: grid is a multiple of 8, keep a sequence's blocks on one XCD
    int32_t row_format;       // host only: selects the kernel instance
    // paged pool (kv is the pool): block_table [batch][pages_per_seq]
    const int32_t* block_table;
    int32_t page_shift;       // log2 rows per page
    int32_t pages_per_seq;
    uint32_t pool_rows;       // num_pages << page_shift (< 2^32)
    // single-launch merge: one arrival counter per (sequence, head block),
    // zero between launches (nullptr: the combine runs as its own kernel)
    uint32_t* arrive;
};

// Gather one whole 32-token tile into the LDS slot at slot_lds.  Lane l holds
// the (sanitised) row of LDS position l & 31.  Block gather 2j + hh: lane l
// loads the 16 bytes that belong at chunk l & 3 of position 16hh + (l >> 2),
// i.e. piece 4j + ((l & 3) ^ ((l >> 4) & 3)) of that position's row, from
// source byte 16 * piece (codes) or 16 * piece + rope offset - 448 (rope; the
// scales sit between them in the cache row).  The two rows each lane needs come
// from the lanes holding them (2 ds_bpermute per tile), and the 18 gathers share
// two offset registers.  fp32 scales: scale gather k loads scale 2k + (l >> 5) of
// position l & 31 into row 2k + (l >> 5) of the table; the last one leaves out
// group 7 (padding), whose row holds list entries instead (see
// load_entries_lds).  UE8M0 scales: one gather of 4 bytes per lane (see
// kScaleRaw).
// Source addresses: a byte offset from the sequence's first row (contiguous
// cache, through the buffer resource), or a 64-bit address (paged pool; a
// masked row reads kZeroRow).
template <bool P>
struct TileGather {
    using Addr = std::conditional_t<P, const uint8_t*, uint32_t>;
    Addr v0, v1;         // blocks of positions 0..15 and 16..31
    Addr vscale;         // this lane's scale pair
    uint32_t slot;       // LDS slot address
};

template <int F, bool P>
__device__ __forceinline__ typename TileGather<P>::Addr source(int row, uint32_t off, const uint8_t* pool) {
    if constexpr (P)
        return (row == -1 ? kZeroRow : pool + (uint64_t)(uint32_t)row * RowFormat<F>::kBytes) + off;
    else return row_offset<F>(row, off);
}

template <int F, bool P>
__device__ __forceinline__ TileGather<P> plan_tile(int row, uint32_t slot_lds, int lane, const uint8_t* pool) {
    const int row0 = __builtin_amdgcn_ds_bpermute(4 * (lane >> 2), row);
    const int row1 = __builtin_amdgcn_ds_bpermute(4 * (16 + (lane >> 2)), row);
    const uint32_t pp = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    TileGather<P> g;
    g.v0 = source<F, P>(row0, 16u * pp, pool);
    g.v1 = source<F, P>(row1, 16u * pp, pool);
    g.vscale = source<F, P>(row, SMLA_SCALE_OFFSET + 4u * ((uint32_t)lane >> 5), pool);
    g.slot = slot_lds;
    return g;
}

template <int kOff, bool P>
__device__ __forceinline__ void gather16(const typename TileGather<P>::Addr& v, i32x4 rsrc, uint32_t lds_base) {
    if constexpr (P) gather16_global_at<kOff>(v, lds_base);
    else gather16_at<kOff>(v, rsrc, lds_base);
}

template <int kOff, bool P>
__device__ __forceinline__ void gather4s(const typename TileGather<P>::Addr& v, i32x4 rsrc, uint32_t lds_base) {
    if constexpr (P) gather4_global_at<kOff>(v, lds_base);
    else gather4_at<kOff>(v, rsrc, lds_base);
}

template <int F, bool P>
__device__ __forceinline__ void issue_scales(const TileGather<P>& g, i32x4 rsrc, int lane) {
    if constexpr (F == SMLA_ROW_UE8M0_SCALES) {
        gather4s<0, P>(g.vscale, rsrc, g.slot + kScaleRaw);
    } else {
        static_for<0, kScaleGathers - 1>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            gather4s<8 * k, P>(g.vscale, rsrc, g.slot + kScaleTable + 256 * k);
        });
        if (lane < 32)
            gather4s<8 * (kScaleGathers - 1), P>(g.vscale, rsrc, g.slot + kScaleTable + 256 * (kScaleGathers - 1));
    }
}

// Blocks 2j and 2j + 1 for j in [J0, J1).
template <int F, int J0, int J1, bool P>
__device__ __forceinline__ void issue_blocks(const TileGather<P>& g, i32x4 rsrc) {
    static_for<J0, J1>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int off = 64 * j + (4 * j >= kCodePieces ? RowFormat<F>::kRopeOff - SMLA_SCALE_OFFSET : 0);
        gather16<off, P>(g.v0, rsrc, g.slot + 1024 * (2 * j));
        gather16<off, P>(g.v1, rsrc, g.slot + 1024 * (2 * j + 1));
    });
}

template <int F, bool P>
__device__ __forceinline__ void issue_tile(int row, i32x4 rsrc, uint32_t slot_lds, int lane, const uint8_t* pool) {
    const TileGather<P> g = plan_tile<F, P>(row, slot_lds, lane, pool);
    issue_scales<F, P>(g, rsrc, lane);
    issue_blocks<F, 0, kRowGathers / 2, P>(g, rsrc);
}

// Value 2^(e - 127) of a UE8M0 scale byte as fp32: the exponent field alone,
// except 0 (2^-127, a subnormal) and 255 (NaN).
__device__ __forceinline__ float ue8m0_value(uint32_t e) {
    const uint32_t bits = e == 0 ? 0x00400000u : e == 255 ? 0x7FC00000u : e << 23;
    return __uint_as_float(bits);
}

// Expands the gathered UE8M0 bytes of a landed tile into its fp32 scale table
// (rows 0..6; row 7 holds list entries).  Lane l holds bytes of groups
// 4 (l >> 5) .. + 3 of position l & 31; its one LDS read precedes the writes,
// which overwrite the raw dwords.
__device__ __forceinline__ void expand_ue8m0_scales(lds_u8* st, int lane) {
    const uint32_t d = ((lds_cu32*)(st + kScaleRaw))[lane];
    lds_f32* sT = (lds_f32*)(st + kScaleTable) + 4 * kTile * (lane >> 5) + (lane & 31);
#pragma unroll
    for (int k = 0; k < 3; k++) sT[k * kTile] = ue8m0_value((d >> (8 * k)) & 0xFFu);
    if (lane < 32) sT[3 * kTile] = ue8m0_value(d >> 24);
}

// Position of the list entries of a tile in an LDS slot: the unused group-7
// row of its scale table.
constexpr int kEntryTable = kScaleTable + 7 * kTile * 4;

// List entries of one tile (token t = lane & 31 at byte 4t of the table, for
// lanes 0..31) straight into LDS.  The buffer resource covers the chunk's
// entries, so an entry past the chunk reads 0 (and is masked by its index).
__device__ __forceinline__ void load_entries_lds(uint32_t first_entry, i32x4 idx_rsrc, uint32_t slot_lds,
                                                 int lane) {
    if (lane < 32) gather4(4u * (first_entry + lane), idx_rsrc, slot_lds + kEntryTable);
}

// One 32-token tile for one wave: 16 heads x the full latent.  st is the
// tile's LDS slot; vmask marks the kept tokens.
// issue_part(stage) is called at four points (stages 0..3) to spread the next
// tile's gathers over the compute: a run of gather instructions stalls the
// wave while the address unit drains them.
template <typename IssuePart>
__device__ __forceinline__ void compute_tile(const lds_u8* st, uint64_t vmask, const bf16x8 (&qop)[16],
                                             f32x4 (&acc_o)[32], float& m_run, float& l_run, int lane,
                                             float logit_factor, IssuePart&& issue_part) {
    const int qg = lane >> 4, ln = lane & 15;

    // group scales, transposed: sT[g * 32 + s] = scale g of the row in LDS position s
    lds_cf32* sT = (lds_cf32*)(st + kScaleTable);

    // ---------------- S^T = K . Q^T per 16-token half; lane group q takes
    // columns 16q..16q+15 of every 64-column group (two K-steps of 8), and rope
    // columns 16q..16q+15.  The K rows of the second half are read before the
    // first half is converted.
    u32x4 raw[2][7];
    u32x4 rr[2][2];
    auto load_half = [&](int tt) {
        // pieces 4g + qg (codes) and rope pieces 2qg, 2qg + 1 of token 16tt + ln;
        // piece 4g + qg sits 2048 g bytes after piece qg
        const int pos = lds_pos(16 * tt + ln);
        const lds_u8* kb = st + piece_addr(qg, pos);
#pragma unroll
        for (int g = 0; g < 7; g++) raw[tt][g] = *(lds_cu32x4*)(kb + 2048 * g);
        rr[tt][0] = *(lds_cu32x4*)(st + piece_addr(kCodePieces + 2 * qg, pos));
        rr[tt][1] = *(lds_cu32x4*)(st + piece_addr(kCodePieces + 2 * qg + 1, pos));
    };
    load_half(0);
    load_half(1);
    issue_part(std::integral_constant<int, 0>{});
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
            v += *(lds_cf32x4*)(sT + g * kTile + lds_pos(16 * tt + 4 * qg)) * acc[g];
        s[tt] = v;
    }
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float z = s[tt][j] * logit_factor;
            s[tt][j] = ((vmask >> (16 * tt + 4 * qg + j)) & 1) ? z : -INFINITY;
        }

    issue_part(std::integral_constant<int, 1>{});

    // ---------------- O^T += V^T . P^T: operand addresses, first groups' reads
    // V^T operands: tr8 source rows, lane 16q + j supplies token slot_token(8q + j/2),
    // byte half j%2; rope V^T via tr16, lane 16q + 4r + c supplies
    // slot_token(8q + r), then slot_token(8q + 4 + r), columns 4c..4c+3 of each
    // 16-column block.  The reads of group g + 1 are issued before group g is
    // converted (one wave per SIMD has no other wave to hide LDS latency),
    // and the first two groups' reads before the softmax, whose cross-lane
    // reductions and exponentials then cover their latency.
    // value pieces 4g + cb of this lane's token: piece cb plus 2048 g bytes
    const int vpos = lds_pos(slot_token(8 * qg + (ln >> 1)));
    const lds_u8* tr_cb[4];
#pragma unroll
    for (int cb = 0; cb < 4; cb++) tr_cb[cb] = st + piece_addr(cb, vpos, ln & 1);
    // rope bytes 32 dt + 8 (ln & 3): piece 28 + 2 dt + ((ln & 3) >> 1), half
    // ln & 1; dt and dt + 2 are 2048 bytes apart
    const int rpos0 = lds_pos(slot_token(8 * qg + (ln >> 2)));
    const int rpos1 = lds_pos(slot_token(8 * qg + 4 + (ln >> 2)));
    const int rp = kCodePieces + ((ln & 3) >> 1);
    const lds_u8* r0[2] = {st + piece_addr(rp, rpos0, ln & 1), st + piece_addr(rp + 2, rpos0, ln & 1)};
    const lds_u8* r1[2] = {st + piece_addr(rp, rpos1, ln & 1), st + piece_addr(rp + 2, rpos1, ln & 1)};
    i32x2 vraw[2][4];
    f32x4 svv[2][2];
    auto load_group = [&](int g, int buf) {
#pragma unroll
        for (int cb = 0; cb < 4; cb++)
            vraw[buf][cb] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(tr_cb[cb] + 2048 * g));
        svv[buf][0] = *(lds_cf32x4*)(sT + g * kTile + lds_pos(4 * qg));
        svv[buf][1] = *(lds_cf32x4*)(sT + g * kTile + lds_pos(16 + 4 * qg));
    };
    load_group(0, 0);
    load_group(1, 1);

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
            // the accumulator lives in AGPRs; this keeps its copy to VGPRs (for
            // the multiply) inside this rarely taken branch
#pragma unroll
            for (int i = 0; i < 32; i++) asm volatile("" : "+a"(acc_o[i]));
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

    issue_part(std::integral_constant<int, 2>{});

    // ---------------- O^T += V^T . P^T, group by group
    s16x4 rv[4][2];
#pragma unroll
    for (int g = 0; g < 7; g++) {
        const int cur = g & 1;
        if (g >= 1 && g + 1 < 7) load_group(g + 1, cur ^ 1);
        if (g == 1) {
#pragma unroll
            for (int dt = 0; dt < 4; dt++) {
                rv[dt][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(r0[dt & 1] + 2048 * (dt >> 1)));
                rv[dt][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(r1[dt & 1] + 2048 * (dt >> 1)));
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
        if (g == 3) issue_part(std::integral_constant<int, 3>{});
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

// Log-sum-exp merge of the split partials of R (b, h) rows (row0 + k * rstep)
// by one wave, 8 columns per lane.  Splits are taken four at a time: the four
// log-sum-exps (scalar loads) and partial outputs (vector loads) of a group
// are issued for all R rows before any is used, so R rows with at most four
// splits cost one round trip to memory; later groups are folded in with a
// running-maximum rescale.  Each row's arithmetic is the same for every R.
// (Issuing the next group's loads before folding in this one measured slower,
// in the combine kernel and in the single-launch merge.)
// Split indices past the end are clamped and given weight 0.  An empty split
// (lse = -inf) has weight exp(-inf) = 0 and a zero partial.
template <int R>
__device__ __forceinline__ void combine_rows(const float* o_part, const float* lse_part, int64_t row0,
                                             int64_t rstep, int nsplit, uint16_t* out, float* lse, int lane) {
    float M[R], W[R];
    f32x4 acc0[R], acc1[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        M[r] = -INFINITY;
        W[r] = 0.f;
        acc0[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc1[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int s0 = 0; s0 < nsplit; s0 += 4) {
        float l[R][4];
        f32x4 lo[R][4], hi[R][4];
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int64_t row = row0 + r * rstep;
            const float* lp = lse_part + row * nsplit;
            const float* src = o_part + row * nsplit * kLatent + 8 * lane;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const int sk = min(s0 + k, nsplit - 1);
                l[r][k] = lp[sk];
                lo[r][k] = *(const f32x4*)(src + sk * kLatent);
                hi[r][k] = *(const f32x4*)(src + sk * kLatent + 4);
            }
        }
#pragma unroll
        for (int r = 0; r < R; r++) {
            float m = M[r];
#pragma unroll
            for (int k = 0; k < 4; k++)
                if (s0 + k < nsplit) m = fmaxf(m, l[r][k]);
            const float ms = m == -INFINITY ? 0.f : m;
            const float f = __expf(M[r] - ms);   // 0 while nothing was folded in
            W[r] *= f;
            acc0[r] *= f;
            acc1[r] *= f;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const float w = s0 + k < nsplit ? __expf(l[r][k] - ms) : 0.f;
                W[r] += w;
                acc0[r] += w * lo[r][k];
                acc1[r] += w * hi[r][k];
            }
            M[r] = m;
        }
    }
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int64_t row = row0 + r * rstep;
        const float inv = W[r] > 0.f ? 1.f / W[r] : 0.f;
        u32x4 pk;
        pk[0] = pack_bf16x2(acc0[r][0] * inv, acc0[r][1] * inv);
        pk[1] = pack_bf16x2(acc0[r][2] * inv, acc0[r][3] * inv);
        pk[2] = pack_bf16x2(acc1[r][0] * inv, acc1[r][1] * inv);
        pk[3] = pack_bf16x2(acc1[r][2] * inv, acc1[r][3] * inv);
        *(u32x4*)(out + row * kLatent + 8 * lane) = pk;
        if (lane == 0) lse[row] = W[r] > 0.f ? M[r] + logf(W[r]) : -INFINITY;
    }
}

// Single-launch merge.  The split partials go out as device-scope stores
// (store16_device / store4_device: written through the XCD's L2, which keeps no
// dirty copy of them), so that the one agent-scope release fence below has
// nothing of theirs to write back.  After its partial stores every wave waits
// for them to complete; then wave 0 takes the release fence and counts the
// workgroup in at its (sequence, head block) counter.  In the last of the
// nsplit workgroups to arrive, wave 0 takes an agent-scope acquire fence and a
// workgroup barrier orders every wave's loads after it (the fence invalidates
// the XCD's L2, so once per workgroup: once per wave cost the other
// workgroups on the XCD their cached rows, ~4.5 us per step at 32 x 64 heads);
// then the workgroup merges the 16 heads' partials of every split
// (combine_rows: each wave its 16 / NWAVES rows together) into the output
// rows and lse, and puts the counter back to zero for the next launch.  No workgroup waits for another, so the grid drains in
// any dispatch order.  flag: an LDS word no wave reads or writes after its
// partial stores.
__device__ __forceinline__ void store16_device(float* base, uint32_t range, uint32_t off, f32x4 v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)range, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off, 0, 16 /* sc1 */);
}

__device__ __forceinline__ void store4_device(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int NWAVES>
__device__ __forceinline__ void merge_if_last(const DecodeArgs& a, int b, int hb, int wave, int lane, lds_u32* flag) {
    wait_vmcnt<0>();
    __syncthreads();
    uint32_t* const ctr = a.arrive + (int64_t)b * a.n_hb + hb;
    if (wave == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        if (lane == 0)
            *flag = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    (uint32_t)(a.nsplit - 1);
    }
    __syncthreads();
    if (!*flag) return;
    if (wave == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
    const int64_t bh0 = (int64_t)b * a.heads + 16 * hb;
    combine_rows<16 / NWAVES>(a.o_part, a.lse_part, bh0 + wave, NWAVES, a.nsplit, a.out, a.lse, lane);
    if (wave == 0 && lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

#if !defined(SMLA_PAGED_TU) && !defined(SMLA_FOURWAVE_TU)
// The combine as its own kernel: one wave per (b, h), four rows per
// workgroup.  When the grid is a multiple of 8, workgroup ids are remapped like
// the decode kernel's, so that XCD x merges the rows of the same contiguous
// range of sequences whose partials its L2 received from the decode kernel
// (exactly so when the batch is a multiple of 8).
__global__ __launch_bounds__(256) void smla_combine_kernel(const float* o_part, const float* lse_part,
                                                           int32_t rows, int32_t nsplit,
                                                           uint16_t* out, float* lse) {
    int bid = blockIdx.x;
    if ((gridDim.x & 7) == 0) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
    const int row = bid * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    combine_rows<1>(o_part, lse_part, row, 0, nsplit, out, lse, threadIdx.x & 63);
}

// Debug scan of the device-resident inputs, launched ahead of the decode
// kernel when SMLA_DEBUG_VALIDATE is set: the conditions it finds (SMLA_DBG_*)
// are OR-ed into g_debug_flags, which smla_debug_flags reads.  The results of
// the decode do not depend on it.
__device__ uint32_t g_debug_flags;

struct ValidateArgs {
    const int32_t* idx;
    const int32_t* seqlens;
    const int32_t* block_table;   // NULL for a contiguous cache
    int64_t reach;                // rows a sequence can address: kv_seq_stride, or pages_per_seq << page_shift
    int32_t topk, page_shift, pages_per_seq;
    uint32_t num_pages;
};

// One workgroup per sequence.  Repeated entries are found by comparing every
// kept entry with the later ones, 1024 at a time staged in LDS: O(topk^2) per
// list, which is why this is a debug path.
__global__ __launch_bounds__(256) void smla_validate_kernel(ValidateArgs a) {
    __shared__ int32_t part[1024];
    const int b = blockIdx.x;
    const int32_t* row = a.idx + (int64_t)b * a.topk;
    const int32_t sl = a.seqlens[b];
    const int64_t kept_below = sl < 0 ? 0 : (sl < a.reach ? (int64_t)sl : a.reach);
    uint32_t f = (threadIdx.x == 0 && (sl < 0 || (int64_t)sl > a.reach)) ? SMLA_DBG_SEQLEN : 0u;
    for (int j = threadIdx.x; j < a.topk; j += blockDim.x) {
        const int32_t e = row[j];
        if (e < -1 || (e >= 0 && e >= sl)) f |= SMLA_DBG_INDEX;
        if (a.block_table != nullptr && e >= 0 && e < kept_below) {
            const int32_t pg = a.block_table[(int64_t)b * a.pages_per_seq + (e >> a.page_shift)];
            if (pg < 0 || (uint32_t)pg >= a.num_pages) f |= SMLA_DBG_PAGE;
        }
    }
    for (int c0 = 0; c0 < a.topk; c0 += 1024) {
        const int n = min(1024, a.topk - c0);
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += blockDim.x) part[i] = row[c0 + i];
        __syncthreads();
        for (int j = threadIdx.x; j < c0 + n; j += blockDim.x) {
            const int32_t e = row[j];
            if (e < 0 || e >= kept_below) continue;
            for (int i = max(j + 1 - c0, 0); i < n; i++)
                if (part[i] == e) {
                    f |= SMLA_DBG_DUPLICATE;
                    break;
                }
        }
    }
    if (f != 0u) atomicOr(&g_debug_flags, f);
}
#endif

// Paged pool: the page ids of a tile's entries, 32 per wave and slot, after
// the tile slots.
constexpr int kPageIds = kLdsBytes;
constexpr int kPagedLdsBytes = kLdsBytes + kWaves * 2 * kTile * 4;
static_assert(kPagedLdsBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");

// One workgroup = (sequence b, block hb of 16 heads, split).  Its four waves
// decode the split's tiles independently (wave w takes tiles w, w + 4, ...,
// each gathered into the wave's own two LDS slots one tile ahead), then merge
// their online-softmax states once, through LDS, and write the split's
// normalised output and log-sum-exp (or the final bf16 result).
// F: row format; P: rows in a paged pool found through the block table.
// The values the first list entries and rows wait for come as leading scalar
// arguments, which the build preloads into SGPRs (kernarg preload, gfx950):
// no kernel-argument load before the first memory requests (~0.8 us per
// launch at the default workload).  remap_stride is gridDim.x / 8 when the
// XCD remap applies, else 0; the rest of DecodeArgs is read as usual.
template <int F, bool P>
__global__ __launch_bounds__(64 * kWaves, 1) void smla_decode_kernel(const uint8_t* kv, const int32_t* idx,
                                                                    const int32_t* seqlens, int64_t kv_seq_stride,
                                                                    int32_t topk, int32_t nsplit, int32_t chunk,
                                                                    int32_t n_hb, int32_t heads,
                                                                    int32_t remap_stride, DecodeArgs a) {
    a.kv = kv;
    a.idx = idx;
    a.seqlens = seqlens;
    a.kv_seq_stride = kv_seq_stride;
    a.seq_bytes = (uint32_t)kv_seq_stride * (uint32_t)RowFormat<F>::kBytes;
    a.topk = topk;
    a.nsplit = nsplit;
    a.chunk = chunk;
    a.n_hb = n_hb;
    a.heads = heads;
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[P ? kPagedLdsBytes : kLdsBytes];
    lds_u8* const lds = (lds_u8*)lds_raw;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qg = lane >> 4;                  // lane group 0..3
    const int ln = lane & 15;                  // head column of the 16x16 tiles

    int split, hb, b;
    block_coords(blockIdx.x, remap_stride, a.nsplit, a.n_hb, split, hb, b);

    const int head = 16 * hb + ln;
    const int t_begin = split * a.chunk;
    const int n_ent = max(min(a.topk, t_begin + a.chunk) - t_begin, 0);
    const int ntiles = (n_ent + kTile - 1) / kTile;
    // contiguous cache: entries at or past the sequence stride are skipped too,
    // so that a sequence never reaches another's rows
    const int seqlen = P ? a.seqlens[b] : (int)min((int64_t)a.seqlens[b], a.kv_seq_stride);
    // contiguous cache: a buffer resource over the sequence's rows
    const i32x4 rsrc = P ? i32x4{0, 0, 0, 0}
                         : row_rsrc(a.kv + (int64_t)b * a.kv_seq_stride * RowFormat<F>::kBytes, a.seq_bytes);
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

    // ---- tiles wave, wave + 4, ...  The gather of tile i + 1 is issued when
    // tile i has landed and overlaps its compute.  (Gathering the first two
    // tiles together measured no faster: the first one then lands later.)
    // The first three tiles' list entries are loaded before any gather (the
    // query after the first gather); the entries of tile i + 2 go straight into LDS with the gathers
    // of tile i + 1 and are read after the next wait.  An entry loaded into
    // registers while gathers are in flight would make the compiler's own wait
    // for it cover those gathers.
    const int my_n = wave < ntiles ? (ntiles - 1 - wave) / kWaves + 1 : 0;
    lds_u8* my_lds = lds + wave * kWaveLds;
    const uint32_t my_lds_addr = (uint32_t)(uintptr_t)my_lds;
    const i32x4 idx_rsrc = row_rsrc((const uint8_t*)idx_b, 4u * (uint32_t)n_ent);
    auto first_entry = [&](int i) { return (wave + kWaves * i) * kTile; };
    // list entry of token (lane & 31) of tile i < my_n
    auto load_entry = [&](int i) -> int { return idx_b[min(first_entry(i) + (lane & 31), n_ent - 1)]; };
    // the row it selects, or -1 for a masked entry (past the list, negative,
    // or not below the sequence length)
    auto sanitise = [&](int i, int v) -> int {
        return first_entry(i) + (lane & 31) < n_ent && v >= 0 && v < seqlen ? v : -1;
    };
    int row_cur = -1, row_1 = -1, row_2 = -1;
    // Paged pool: a kept entry e of the sequence is at pool row
    // (block_table[b][e >> page_shift] << page_shift) + (e & (page - 1)).  The
    // page ids take one more memory round trip, so the pipeline runs one tile
    // further ahead: the entries of tile i + 3 (into LDS) and the page ids of
    // tile i + 2 (into LDS, from the entries read at the top of tile i) are
    // loaded during tile i, and tile i + 1's rows are formed at its top.
    const int32_t* bt_b = P ? a.block_table + (int64_t)b * a.pages_per_seq : nullptr;
    const uint32_t page_mask = (1u << a.page_shift) - 1u;
    // sanitised entry -> pool row, or -1 (no page, or past the table row)
    auto to_pool_row = [&](int e, int page) -> int {
        return e >= 0 && (e >> a.page_shift) < a.pages_per_seq && page >= 0 &&
                       (uint32_t)page < (a.pool_rows >> a.page_shift)
                   ? (int)(((uint32_t)page << a.page_shift) | ((uint32_t)e & page_mask))
                   : -1;
    };
    auto page_of = [&](int e) -> int { return bt_b[e >= 0 ? min(e >> a.page_shift, a.pages_per_seq - 1) : 0]; };
    const i32x4 bt_rsrc = P ? row_rsrc((const uint8_t*)bt_b, 4u * (uint32_t)a.pages_per_seq) : i32x4{0, 0, 0, 0};
    lds_u8* const my_page_ids = lds + kPageIds + wave * 2 * kTile * 4;   // two tiles' page ids
    const uint32_t my_pages = (uint32_t)(uintptr_t)my_page_ids;
    int e_n1 = -1, e_n2 = -1;   // sanitised entries of tiles i + 1 and i + 2 (paged)
    if (my_n > 0) {
        const int e0 = load_entry(0);
        const int e1 = load_entry(min(1, my_n - 1));
        const int e2 = load_entry(min(2, my_n - 1));
        row_cur = sanitise(0, e0);
        row_1 = sanitise(1, e1);
        row_2 = sanitise(2, e2);
        if constexpr (P) {
            e_n1 = row_1;
            e_n2 = row_2;
            const int pg0 = page_of(row_cur), pg1 = page_of(row_1);
            row_cur = to_pool_row(row_cur, pg0);
            row_1 = to_pool_row(row_1, pg1);
        }
        issue_tile<F, P>(row_cur, rsrc, my_lds_addr, lane, a.kv);
    }
    // the query lands while the first tile is gathered
    load_query();
    pin_state(qop, acc_o);
    for (int i = 0; i < my_n; i++) {
        pin_state(qop, acc_o);
        wait_vmcnt<0>();   // tile i has landed, and the entries (and page ids) loaded with it
        const int slot1 = (i + 1) & 1;
        int row_next;
        if constexpr (P) {
            row_next = i == 0 ? row_1
                              : to_pool_row(e_n1, ((lds_ci32*)(my_page_ids + slot1 * kTile * 4))[lane & 31]);
            if (i >= 1 && i + 2 < my_n)
                e_n2 = sanitise(i + 2, ((lds_ci32*)(my_lds + (i & 1) * kSlot + kEntryTable))[lane & 31]);
        } else {
            row_next = i == 0   ? row_1
                       : i == 1 ? row_2
                                : sanitise(i + 1, ((lds_ci32*)(my_lds + slot1 * kSlot + kEntryTable))[lane & 31]);
        }
        // the gathers of tile i + 1: the scales and two blocks now, the rest
        // within the logit product of tile i (early enough for the memory-bound
        // lists); then the entries of tile i + 2, into the slot being computed
        // (its entry table is not read by the compute)
        const bool more = i + 1 < my_n;
        TileGather<P> tg = {};
        if (more) {
            tg = plan_tile<F, P>(row_next, my_lds_addr + slot1 * kSlot, lane, a.kv);
            issue_scales<F, P>(tg, rsrc, lane);
            issue_blocks<F, 0, 2, P>(tg, rsrc);
        }
        auto issue_part = [&](auto stage) {
            if (!more) return;
            constexpr int k = decltype(stage)::value;
            if constexpr (k == 0) {
                issue_blocks<F, 2, 6, P>(tg, rsrc);
            } else if constexpr (k == 1) {
                issue_blocks<F, 6, kRowGathers / 2, P>(tg, rsrc);
                if constexpr (P) {
                    // page ids of tile i + 2 (into page slot i & 1), entries of
                    // tile i + 3 (into the entry table of slot (i + 1) & 1)
                    if (i + 2 < my_n && lane < 32)
                        gather4(e_n2 >= 0 ? 4u * (uint32_t)(e_n2 >> a.page_shift) : 0x80000000u, bt_rsrc,
                                my_pages + (i & 1) * kTile * 4);
                    if (i + 3 < my_n)
                        load_entries_lds(first_entry(i + 3), idx_rsrc, my_lds_addr + slot1 * kSlot, lane);
                } else {
                    if (i >= 1 && i + 2 < my_n)
                        load_entries_lds(first_entry(i + 2), idx_rsrc, my_lds_addr + (i & 1) * kSlot, lane);
                }
            }
        };
        const uint64_t vmask = mask_by_token(__ballot(lane < kTile && row_cur != -1));
        if constexpr (F == SMLA_ROW_UE8M0_SCALES) expand_ue8m0_scales(my_lds + (i & 1) * kSlot, lane);
        compute_tile(my_lds + (i & 1) * kSlot, vmask, qop, acc_o, m_run, l_run, lane, a.logit_factor, issue_part);
        row_cur = row_next;
        if constexpr (P) e_n1 = e_n2;
    }
    wait_vmcnt<0>();

    // ---------------- merge of the four waves' states.  Each wave stores its
    // accumulator (unscaled, straight from its AGPRs) and its statistics into
    // its own two tile slots, which no other wave touches, as soon as its last
    // tile is done; one barrier then makes the four visible to all.
    const float l_tot = lanegroup_sum(l_run);
    {
        lds_u8* const mine = lds + wave * kWaveLds;
        lds_f32x4* part = (lds_f32x4*)mine;
#pragma unroll
        for (int i = 0; i < 32; i++) part[i * 64 + lane] = acc_o[i];
        lds_f32* stat = (lds_f32*)(mine + kAccBytes);   // [max 16 | sum 16]
        if (lane < 16) {
            stat[lane] = m_run;
            stat[16 + lane] = l_tot;
        }
    }
    __syncthreads();
    auto stat_of = [&](int w) { return (lds_cf32*)(lds + w * kWaveLds + kAccBytes); };
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; w++) M = fmaxf(M, stat_of(w)[ln]);
    const float Ms0 = M == -INFINITY ? 0.f : M;
    // weight of wave w's accumulator for head ln: 2^(m_w - M)
    float wgt[kWaves];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
        wgt[w] = __builtin_amdgcn_exp2f(stat_of(w)[ln] - Ms0);
        L += wgt[w] * stat_of(w)[16 + ln];
    }

    // wave w finishes accumulator blocks 8w..8w+7; block i holds columns
    // 16i + 4qg + j for head ln
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const float lse2 = L > 0.f ? M + log2f(L) : -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; w++) wgt[w] *= inv;
    const int64_t bh = (int64_t)b * a.heads + head;
    const bool final_out = a.nsplit == 1 && !a.force_partials;
    auto block_sum = [&](int i) -> f32x4 {   // the normalised output block
        f32x4 v = wgt[0] * ((lds_cf32x4*)lds)[i * 64 + lane];
#pragma unroll
        for (int w = 1; w < kWaves; w++) v += wgt[w] * ((lds_cf32x4*)(lds + w * kWaveLds))[i * 64 + lane];
        return v;
    };
    const int i0 = wave * (32 / kWaves);
    if (final_out) {
        uint16_t* o = a.out + bh * kLatent + 4 * qg;
#pragma unroll
        for (int ii = 0; ii < 32 / kWaves; ii++) {
            const f32x4 v = block_sum(i0 + ii);
            u32x2 w;
            w[0] = pack_bf16x2(v[0], v[1]);
            w[1] = pack_bf16x2(v[2], v[3]);
            *(u32x2*)(o + 16 * (i0 + ii)) = w;
        }
    } else if (a.arrive) {
        // single launch: device-scope stores from the workgroup's first row
        const int64_t bh0 = (int64_t)b * a.heads + 16 * hb;
        float* const base = a.o_part + (bh0 * a.nsplit + split) * kLatent;
        const uint32_t row_off = (uint32_t)(ln * a.nsplit) * (kLatent * 4) + 16 * qg;
#pragma unroll
        for (int ii = 0; ii < 32 / kWaves; ii++)
            store16_device(base, 16u * (uint32_t)a.nsplit * (kLatent * 4), row_off + 64 * (i0 + ii),
                           block_sum(i0 + ii));
    } else {
        float* o = a.o_part + (bh * a.nsplit + split) * kLatent + 4 * qg;
#pragma unroll
        for (int ii = 0; ii < 32 / kWaves; ii++) *(f32x4*)(o + 16 * (i0 + ii)) = block_sum(i0 + ii);
    }
    if (wave == 0 && qg == 0) {
        if (final_out) a.lse[bh] = lse2 * kLn2;
        else if (a.arrive) store4_device(a.lse_part + bh * a.nsplit + split, lse2 * kLn2);
        else a.lse_part[bh * a.nsplit + split] = lse2 * kLn2;
    }
    if (a.arrive) merge_if_last<kWaves>(a, b, hb, wave, lane, (lds_u32*)lds);
}

// ---------------------------------------------------------------------------
// Pipelined decode kernel (contiguous cache): one workgroup = (sequence b,
// block hb of 16 heads, split), eight waves in two roles, one of each per
// SIMD (waves w and w + 4 share one).  The split's list is taken in batches of
// two 32-token tiles, which move through a ring of four batch buffers in LDS.
// In step s:
//   - the logit waves (0..3) compute S^T for 16-token half (w & 1) of tile
//     (w >> 1) of batch s against the 16 heads (the bf16 MFMA product of the
//     four-wave kernel), mask it, take as its base the running maximum, or its
//     own maximum when that exceeds the running one by more than kTau, and
//     write its weights p = 2^(z - base) to a weight table and its base per
//     head to a statistics row; between those parts each issues, in three
//     stages, its half of the gathers of one tile of batch s + 2 (wave 0 first
//     copies the list entries of batch s + 3), and at the end waits for its
//     gathers of batch s + 1;
//   - the value waves (4..7) accumulate O^T += V^T . P^T for batch s - 1 over
//     their own output columns (value wave i: nope groups 2i, 2i + 1, or group
//     6 and the rope for i = 3), each half's weights scaled by 2^(base - M)
//     (skipped when every factor is 1); they read no memory, only LDS, and the
//     rope wave also forms the weight sum as the product with a column of ones;
// and one barrier ends the step.  At its top all eight waves form the same
// new running maximum M from the four bases of batch s - 1.  The two roles
// share each SIMD, so one role's waits and dependency stalls are filled by
// the other's work; the weights, not accumulators, cross between waves, and
// no wave's registers exceed the 256 that two waves per SIMD allow.
// Every tile of every batch is gathered (list entries past the split or
// masked read row -1, i.e. zeros), so no wave ever reads stale bytes and the
// tile loops carry no branches.
// LDS: four batch buffers of two tile slots (the slot layout above) and two
// weight tables (batch parity), 160 KB.  Row 7 of each slot, which the gathers
// never write, holds the list entries of the batch after next (slots 0..3, by
// batch parity, copied from memory by the DMA path like the rows) and the
// bases (slots 4..7).  Every asynchronous memory read of the loop is such a
// DMA into LDS, so each wave's waits count only its own DMAs.  At the start
// the fourth buffer stages the workgroup's query (16 rows of 1 KB, read once
// from memory instead of once per wave) and all eight waves gather batches 0
// and 1.
constexpr int kPlWaves = 8;
constexpr int kPlPagedBatches = 8;                        // batches of a split on a paged pool (512 entries)
constexpr int kPlBtLds = 8192;                            // block-table slots copied into LDS (32 KB)
constexpr int kPlTiles = 2;                               // tiles per batch
constexpr int kPlRing = 4;                                // batch buffers
constexpr int kPlBatch = kPlTiles * kSlot;                // 38912 bytes per batch buffer
constexpr int kPlPTable = kPlRing * kPlBatch;             // weight tables offset
constexpr int kPlPTile = 16 * kTile * 4;                  // one tile's weights: [16 heads][32 tokens] fp32
constexpr int kPlLdsBytes = kPlPTable + 2 * kPlTiles * kPlPTile;
static_assert(kPlLdsBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
static_assert(16 * 1024 <= kScaleTable, "the staged query stays clear of its slot's scale table");
static_assert(kPlBatch == 2 * kSlot, "slot k of the ring is slot k & 1 of buffer k >> 1");
// the output rows of a workgroup's 16 heads (fp32, not yet normalised), staged
// at the end in the first batch buffer (free by then): row pitch 16 bytes above
// the row, so that the sixteen rows start on sixteen different groups of four
// banks
constexpr int kPlStagePitchF32 = 4 * kLatent + 16;
static_assert(16 * kPlStagePitchF32 <= kPlBatch, "staged rows within the first batch buffer");
static_assert(4 * kPlBtLds <= kPlBatch, "a paged prologue's block-table row fits the third batch buffer");

// Byte offset in a weight table of tokens 4c..4c+3 of head h in a tile:
// 16-byte chunks XOR-swizzled by head so that the 16 heads read by one
// quarter-wave fall in distinct banks.
__device__ __forceinline__ int ptable_chunk(int h, int c) { return 128 * h + 16 * (c ^ ((h >> 1) & 7)); }

// Staged query: byte offset of 16-byte chunk c (columns 8c..8c+7) of head h,
// chunks XOR-swizzled by h so that 16 heads read at one column fall in
// distinct banks.
__device__ __forceinline__ int qstage_addr(int h, int c) { return 1024 * h + 16 * (c ^ (h & 15)); }

// fp16 weights fp16(p * s) of eight tokens (p0, p1 and s0, s1 hold tokens
// 0..3 and 4..7): the fp32 product, rounded to fp16 (v_cvt_pk_f16_f32, round
// to nearest even).  Plain arithmetic, not inline assembly, so that the
// compiler sees these vector writes and keeps the wait states the matrix
// instructions reading them require.
__device__ __forceinline__ f16x8 weights_f16(f32x4 p0, f32x4 p1, f32x4 s0, f32x4 s1) {
    const f32x4 w0 = p0 * s0, w1 = p1 * s1;
    return f16x8{(_Float16)w0[0], (_Float16)w0[1], (_Float16)w0[2], (_Float16)w0[3],
                 (_Float16)w1[0], (_Float16)w1[1], (_Float16)w1[2], (_Float16)w1[3]};
}

template <int F, bool P>
__global__ __launch_bounds__(64 * kPlWaves) void smla_decode_pipelined_kernel(const uint8_t* kv, const int32_t* idx,
                                                                      const int32_t* seqlens, int64_t kv_seq_stride,
                                                                      int32_t topk, int32_t nsplit, int32_t chunk,
                                                                      int32_t n_hb, int32_t heads,
                                                                      int32_t remap_stride, DecodeArgs a) {
    a.kv = kv;
    a.idx = idx;
    a.seqlens = seqlens;
    a.kv_seq_stride = kv_seq_stride;
    a.seq_bytes = (uint32_t)kv_seq_stride * (uint32_t)RowFormat<F>::kBytes;
    a.topk = topk;
    a.nsplit = nsplit;
    a.chunk = chunk;
    a.n_hb = n_hb;
    a.heads = heads;
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[kPlLdsBytes];
    lds_u8* const lds = (lds_u8*)lds_raw;
    const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qg = lane >> 4;                  // lane group 0..3
    const int ln = lane & 15;                  // head column of the 16x16 tiles

    int split, hb, b;
    block_coords(blockIdx.x, remap_stride, a.nsplit, a.n_hb, split, hb, b);

    const int head = 16 * hb + ln;
    const int t_begin = split * a.chunk;
    const int n_ent = max(min(a.topk, t_begin + a.chunk) - t_begin, 0);
    const int nb = (n_ent + kPlTiles * kTile - 1) / (kPlTiles * kTile);
    const int seqlen = P ? a.seqlens[b] : (int)min((int64_t)a.seqlens[b], a.kv_seq_stride);
    // rows through one buffer resource: the sequence's rows, or (paged) the
    // whole pool, below 2^31 bytes (pool rows then fit the 24-bit multiply of
    // row_offset)
    const i32x4 rsrc = P ? row_rsrc(a.kv, a.pool_rows * (uint32_t)RowFormat<F>::kBytes)
                         : row_rsrc(a.kv + (int64_t)b * a.kv_seq_stride * RowFormat<F>::kBytes, a.seq_bytes);
    const int32_t* idx_b = a.idx + (int64_t)b * a.topk + t_begin;

    // In the loop, logit wave w issues the gathers of tile w & 1 of each batch:
    // half 0 (waves 0, 1) the scale table and block pairs 0..3, half 1 pairs
    // 4..8.  In the prologue all eight waves gather batches 0 and 1: wave w
    // part w >> 1 of tile w & 1 (part 0 the scale table and pairs 0, 1, part 1
    // pairs 2, 3, part 2 pairs 4, 5, part 3 pairs 6..8).
    const int gtile = wave & 1;
    const int ghalf = (wave >> 1) & 1;
    const int ppart = wave >> 1;
    constexpr int kScaleInstr = F == SMLA_ROW_UE8M0_SCALES ? 1 : kScaleGathers;

    // sanitised list entry of batch bt for lane l: tile l >> 5, position l & 31
    // (row -1 past the split, past the sequence or masked)
    auto sanitise = [&](int bt, int v) -> int {
        return bt * (kPlTiles * kTile) + lane < n_ent && v >= 0 && v < seqlen ? v : -1;
    };
    // the entries of batch bt in row 7 of slots 2 (bt & 1) and 2 (bt & 1) + 1:
    // copied there by wave 0 (lanes past the split read zeros through the
    // buffer range check), read back by the logit waves
    const i32x4 irsrc = row_rsrc((const uint8_t*)idx_b, 4u * (uint32_t)n_ent);
    auto stage_entries = [&](int bt) {
        const uint32_t voff = 4u * (uint32_t)(bt * (kPlTiles * kTile) + lane);
        const uint32_t row7 = lds_addr + 2 * (bt & 1) * kSlot + kEntryTable;
        if (lane < 32) gather4(voff, irsrc, row7);
        else gather4(voff, irsrc, row7 + kSlot - 4 * 32);
    };
    auto read_entries = [&](int bt) -> int {
        return sanitise(bt, ((lds_ci32*)(lds + (2 * (bt & 1) + (lane >> 5)) * kSlot + kEntryTable))[lane & 31]);
    };
    // bases of half j of the batch of parity p: row 7 of slot 4 + 2p + (j >> 1)
    auto stats_row = [&](int parity, int j) -> lds_u8* {
        return lds + (4 + 2 * parity + (j >> 1)) * kSlot + kEntryTable + 64 * (j & 1);
    };
    auto plan_batch = [&](int bt, int e) {
        const int row = __builtin_amdgcn_ds_bpermute(4 * (32 * gtile + (lane & 31)), e);
        return plan_tile<F, false>(row, lds_addr + (bt % kPlRing) * kPlBatch + gtile * kSlot, lane, nullptr);
    };
    // a logit wave's half of the gathers of one batch, in three stages: half 0
    // the scale table and pair 0, pairs 1, 2, pair 3; half 1 pairs 4, 5,
    // pairs 6, 7, pair 8
    auto issue_stage = [&](const TileGather<false>& g, auto stage) {
        constexpr int k = decltype(stage)::value;
        if (ghalf == 0) {
            if constexpr (k == 0) {
                issue_scales<F, false>(g, rsrc, lane);
                issue_blocks<F, 0, 1, false>(g, rsrc);
            } else if constexpr (k == 1) {
                issue_blocks<F, 1, 3, false>(g, rsrc);
            } else {
                issue_blocks<F, 3, 4, false>(g, rsrc);
            }
        } else {
            if constexpr (k == 0) issue_blocks<F, 4, 6, false>(g, rsrc);
            else if constexpr (k == 1) issue_blocks<F, 6, 8, false>(g, rsrc);
            else issue_blocks<F, 8, kRowGathers / 2, false>(g, rsrc);
        }
    };
    // wait until at most this logit wave's gathers of one batch are in flight
    auto wait_but_one_batch = [&]() {
        if (ghalf == 0) wait_vmcnt<kScaleInstr + 8>();
        else wait_vmcnt<10>();
    };
    // the prologue part of wave w
    auto issue_part = [&](int bt, int e) {
        const TileGather<false> g = plan_batch(bt, e);
        if (ppart == 0) {
            issue_scales<F, false>(g, rsrc, lane);
            issue_blocks<F, 0, 2, false>(g, rsrc);
        } else if (ppart == 1) {
            issue_blocks<F, 2, 4, false>(g, rsrc);
        } else if (ppart == 2) {
            issue_blocks<F, 4, 6, false>(g, rsrc);
        } else {
            issue_blocks<F, 6, kRowGathers / 2, false>(g, rsrc);
        }
    };

    // ---- prologue.  Wave 0 copies the entries of batches 0 and 1 into the
    // free slot 7 and those of batch 2 into its ring rows, then every wave
    // stages two query rows into the fourth buffer (slot 6).  Once the
    // entries are visible, all eight waves issue the gathers of batches 0 and 1
    // (wave w: tile w & 1, part w >> 1 of its gathers), so that no wave waits
    // for the query before the first rows are requested.
    const uint32_t pro_entries = lds_addr + 7 * kSlot;
    if (!P && wave == 0) {
        if (nb > 0) gather4(4u * (uint32_t)lane, irsrc, pro_entries);
        if (nb > 1) gather4(4u * (uint32_t)(kPlTiles * kTile + lane), irsrc, pro_entries + 256);
        if (nb > 2) stage_entries(2);
    }
    auto stage_query = [&]() {
        const uint8_t* qblk = (const uint8_t*)(a.q + ((int64_t)b * a.heads + 16 * hb) * kLatent);
#pragma unroll
        for (int r = 0; r < 2; r++) {
            const int h = 2 * wave + r;
            gather16_global_at<0>(qblk + 1024 * h + 16 * (lane ^ (h & 15)), lds_addr + 3 * kPlBatch + 1024 * h);
        }
    };
    if (!P) stage_query();
    // Paged pool: a kept entry e of the sequence is at pool row
    // (block_table[b][e >> page_shift] << page_shift) + (e & (page - 1)).  A
    // split of this kernel holds at most kPlPagedBatches batches: wave k
    // translates the entries of batch k here, once, and every wave then keeps
    // the pool rows of every batch in registers: lane l, batch k: tile l >> 5,
    // position l & 31; -1 for a masked entry, a page past the table row or a
    // slot outside the pool.  The sequence's block-table row does not depend
    // on the entries: up to kPlBtLds pages it is copied into the third batch
    // buffer (free until step 0) while the entries load, so the translation
    // costs no second memory round trip; a longer row is read entry by entry
    // after the entries.
    int prow[P ? kPlPagedBatches : 1];
    const int32_t* const bt_b = P ? a.block_table + (int64_t)b * a.pages_per_seq : nullptr;
    const bool bt_in_lds = P && a.pages_per_seq <= kPlBtLds;
    if constexpr (P) {
        if (bt_in_lds) {
            const i32x4 btrsrc = row_rsrc((const uint8_t*)bt_b, 4u * (uint32_t)a.pages_per_seq);
            const int n_copy = (a.pages_per_seq + 63) / 64;   // 64 slots per copy; lanes past the row read zeros
            for (int k = wave; k < n_copy; k += kPlWaves)
                gather4(4u * (uint32_t)(64 * k + lane), btrsrc, lds_addr + 2 * kPlBatch + 256 * k);
        }
        // the entries of batch w into slot 7 by wave w (one copy per wave:
        // the CU's address unit takes each request in turn, so few wide ones
        // are issued sooner than one register load per batch and wave)
        static_assert(kPlPagedBatches <= kPlWaves, "one entry copy per wave");
        static_assert(kPlPagedBatches * kPlTiles * kTile * 4 <= kSlot, "the entries fit in slot 7");
        if (wave < nb) gather4(4u * (uint32_t)(wave * kPlTiles * kTile + lane), irsrc, lds_addr + 7 * kSlot + 256 * wave);
        stage_query();
        wait_vmcnt<2>();   // the entries and this wave's share of the block-table row (the query may be in flight)
    }
    // the pool rows of batch bt (a uniform index)
    auto prow_of = [&](int bt) -> int {
        int r = prow[0];
#pragma unroll
        for (int k = 1; k < (P ? kPlPagedBatches : 1); k++) r = bt == k ? prow[k] : r;
        return r;
    };
    if (!P && wave == 0) wait_vmcnt<2>();   // the entries (the two query rows may still be in flight)
    if (wave == 4) ((lds_f32*)stats_row(1, lane >> 4))[ln] = -INFINITY;   // bases of "batch -1"
    lds_barrier();     // the entries of batches 0..2 (paged: the block-table row) are visible
    int e0 = -1, e1 = -1;
    if constexpr (P) {
        // wave w translates batch w (its entries in slot 7, one per lane) and
        // writes the pool rows back in place; after a barrier every wave keeps
        // every batch's pool rows in registers (slot 7 is gathered into from
        // step 1 on)
        lds_i32* const etab = (lds_i32*)(lds + 7 * kSlot);
        {
            const int k = wave;
            const int e = k < nb ? sanitise(k, etab[64 * k + lane]) : -1;
            const int sl = e >= 0 ? min(e >> a.page_shift, a.pages_per_seq - 1) : 0;
            const int pg = bt_in_lds ? ((lds_ci32*)(lds + 2 * kPlBatch))[sl] : bt_b[sl];
            const uint32_t page_mask = (1u << a.page_shift) - 1u;
            etab[64 * k + lane] = k < nb && e >= 0 && (e >> a.page_shift) < a.pages_per_seq && pg >= 0 &&
                                          (uint32_t)pg < (a.pool_rows >> a.page_shift)
                                      ? (int)(((uint32_t)pg << a.page_shift) | ((uint32_t)e & page_mask))
                                      : -1;
        }
        lds_barrier();   // every batch's pool rows are in slot 7
#pragma unroll
        for (int k = 0; k < kPlPagedBatches; k++) prow[k] = etab[64 * k + lane];
        e0 = prow[0];
        e1 = prow_of(1);
    } else {
        if (nb > 0) e0 = sanitise(0, ((lds_ci32*)(lds + 7 * kSlot))[lane]);
        if (nb > 1) e1 = sanitise(1, ((lds_ci32*)(lds + 7 * kSlot + 256))[lane]);
    }
    if (nb > 0) issue_part(0, e0);
    // contiguous cache: every wave's gathers of batch 0 are issued before any
    // of batch 1, so that the CU's address unit takes batch 0 first and it
    // lands sooner (measured -0.45 us per step at 32 x 64 heads x top-512; on a
    // paged pool, where the waves reach this point less evenly, +0.9 us)
    if (!P && nb > 1) __builtin_amdgcn_s_barrier();
    if (nb > 1) issue_part(1, e1);
    if (nb > 1) {
        // at most this wave's gathers of batch 1 in flight
        if (ppart == 0) wait_vmcnt<kScaleInstr + 4>();
        else if (ppart == 3) wait_vmcnt<6>();
        else wait_vmcnt<4>();
    } else {
        wait_vmcnt<0>();
    }
    if constexpr (F == SMLA_ROW_UE8M0_SCALES)
        if (ppart == 0 && nb > 0) expand_ue8m0_scales(lds + gtile * kSlot, lane);
    lds_barrier();     // batch 0 and the query rows are in LDS

    // Each role runs its own loop over the steps (the same barriers: one per
    // step, then one for the weight sum), and each kind of value wave its own
    // copy of the value loop, so that a wave's registers keep their values
    // across the steps instead of being merged (copied) between code paths.
    // ---- the end: the value waves stage their columns in LDS (and the rope
    // wave the weight sums), then after one barrier all eight waves normalise
    // and write the 16 rows in whole 1 KB pieces, 16 bytes per lane (a store
    // instruction costs a wave about the same time whatever its width or
    // address pattern, so few wide contiguous ones end the workgroup sooner)
    const bool final_out = a.nsplit == 1 && !a.force_partials;
    auto inv_sum = [&](int h) {   // 1 / (weight sum of row h), 0 for a row that kept nothing
        const float l = ((lds_cf32*)stats_row(0, 0))[h];
        return l > 0.f ? 1.f / l : 0.f;
    };
    auto store_rows = [&]() {
        const int64_t bh0 = (int64_t)b * a.heads + 16 * hb;
        if (final_out) {
            // rows 2w, 2w + 1; lane l: columns 8l..8l+7
            f32x4 v[2][2];
#pragma unroll
            for (int p = 0; p < 2; p++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    v[p][j] = *(lds_cf32x4*)(lds + (2 * wave + p) * kPlStagePitchF32 + 32 * lane + 16 * j);
#pragma unroll
            for (int p = 0; p < 2; p++) {
                const float inv = inv_sum(2 * wave + p);
                const f32x4 x = v[p][0] * inv, y = v[p][1] * inv;
                const u32x4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]),
                                 pack_bf16x2(y[2], y[3])};
                *(u32x4*)((uint8_t*)(a.out + (bh0 + 2 * wave + p) * kLatent) + 16 * lane) = w;
            }
        } else {
            // pieces 4w..4w+3: head k >> 1, half k & 1 of its row
            f32x4 v[4];
#pragma unroll
            for (int p = 0; p < 4; p++) {
                const int k = 4 * wave + p;
                v[p] = *(lds_cf32x4*)(lds + (k >> 1) * kPlStagePitchF32 + 1024 * (k & 1) + 16 * lane);
            }
            const float inv0 = inv_sum(2 * wave), inv1 = inv_sum(2 * wave + 1);
            if (a.arrive) {
                // single launch: device-scope stores from the workgroup's first row
                float* const base = a.o_part + (bh0 * a.nsplit + split) * kLatent;
#pragma unroll
                for (int p = 0; p < 4; p++) {
                    const int k = 4 * wave + p;
                    store16_device(base, 16u * (uint32_t)a.nsplit * (kLatent * 4),
                                   (uint32_t)((k >> 1) * a.nsplit) * (kLatent * 4) + 1024 * (k & 1) + 16 * lane,
                                   v[p] * (p < 2 ? inv0 : inv1));
                }
            } else {
#pragma unroll
                for (int p = 0; p < 4; p++) {
                    const int k = 4 * wave + p;
                    *(f32x4*)((uint8_t*)(a.o_part + ((bh0 + (k >> 1)) * a.nsplit + split) * kLatent) +
                              1024 * (k & 1) + 16 * lane) = v[p] * (p < 2 ? inv0 : inv1);
                }
            }
        }
    };

    const int vi = wave - 4;   // value waves: output columns 128 vi + 16 c + 4 qg .. + 3 of head ln in
                               // block c (nope groups 2vi, 2vi + 1; group 6 and the rope for vi = 3)
    lds_f32* const lsum = (lds_f32*)stats_row(0, 0);   // the weight sum (after the loop)
    if (wave < 4) {
        // ---- logit wave: the query operands (16 x 8 bf16: the B operand of
        // S^T = K . Q^T, lane group q taking columns 16q..16q+15 of every
        // 64-column group, 8 per K-step, and rope columns 16q..16q+15)
        bf16x8 qop[16];
        {
            const lds_u8* qs = lds + 3 * kPlBatch;
#pragma unroll
            for (int g = 0; g < 7; g++)
#pragma unroll
                for (int ks = 0; ks < 2; ks++)
                    qop[2 * g + ks] = as_bf16x8(*(lds_cu32x4*)(qs + qstage_addr(ln, 8 * g + 2 * qg + ks)));
            qop[14] = as_bf16x8(*(lds_cu32x4*)(qs + qstage_addr(ln, 56 + 2 * qg)));
            qop[15] = as_bf16x8(*(lds_cu32x4*)(qs + qstage_addr(ln, 56 + 2 * qg + 1)));
        }
        float m_run = -INFINITY;   // running base of head ln (log2 units), the same in every wave
        for (int s = 0; s <= nb; s++) {
            // the bases of batch s - 1 (-inf for s = 0)
            float bk[4];
#pragma unroll
            for (int j = 0; j < 4; j++) bk[j] = ((lds_cf32*)stats_row((s - 1) & 1, j))[ln];
            const float M = fmaxf(fmaxf(m_run, fmaxf(bk[0], bk[1])), fmaxf(bk[2], bk[3]));
            // ---- logits of half (wave & 1) of tile (wave >> 1) of batch s, with
            // this wave's gathers of batch s + 2 issued in three stages between
            // its parts (and before them wave 0's copy of the entries of batch
            // s + 3)
            const int qtile = wave >> 1, qhalf = wave & 1;
            const bool issuing = s + 2 < nb;
            int e2 = -1;
            if (issuing) e2 = P ? prow_of(s + 2) : read_entries(s + 2);
            TileGather<false> tg = {};
            if (issuing) {
                tg = plan_batch(s + 2, e2);
                if (!P && wave == 0 && s + 3 < nb) stage_entries(s + 3);
                issue_stage(tg, std::integral_constant<int, 0>{});
            }
            __builtin_amdgcn_sched_barrier(0);
            if (s < nb) {
                const lds_u8* st = opaque(lds + (s % kPlRing) * kPlBatch + qtile * kSlot);
                lds_cf32* sT = (lds_cf32*)(st + kScaleTable);
                const int pos = lds_pos(16 * qhalf + ln);
                const lds_u8* kb = st + piece_addr(qg, pos);
                u32x4 raw[7], rr[2];
#pragma unroll
                for (int g = 0; g < 7; g++) raw[g] = *(lds_cu32x4*)(kb + 2048 * g);
                rr[0] = *(lds_cu32x4*)(st + piece_addr(kCodePieces + 2 * qg, pos));
                rr[1] = *(lds_cu32x4*)(st + piece_addr(kCodePieces + 2 * qg + 1, pos));
                f32x4 acc[8];
#pragma unroll
                for (int g = 0; g < 7; g++)
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw[g][0], raw[g][1]), qop[2 * g],
                                                                     f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                acc[7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rr[0]), qop[14],
                                                                 f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (issuing) issue_stage(tg, std::integral_constant<int, 1>{});
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < 7; g++)
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw[g][2], raw[g][3]),
                                                                     qop[2 * g + 1], acc[g], 0, 0, 0);
                acc[7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rr[1]), qop[15], acc[7], 0, 0, 0);
                f32x4 v = acc[7];
#pragma unroll
                for (int g = 0; g < 7; g++)
                    v += *(lds_cf32x4*)(sT + g * kTile + lds_pos(16 * qhalf + 4 * qg)) * acc[g];
                // kept tokens of the tile, by MFMA token
                const uint64_t vmask =
                    mask_by_token((__ballot(e0 != -1) >> (32 * qtile)) & 0xFFFFFFFFull) >> (16 * qhalf + 4 * qg);
                f32x4 z;
#pragma unroll
                for (int j = 0; j < 4; j++) z[j] = ((vmask >> j) & 1) ? v[j] * a.logit_factor : -INFINITY;
                const float mh = lanegroup_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
                // base of this half: the running maximum, or its own maximum when
                // that is more than kTau above it (weights then stay at most 2^kTau)
                const float bw = mh > M + kTau ? mh : M;
                const float be = bw == -INFINITY ? 0.f : bw;
                f32x4 pw;
#pragma unroll
                for (int j = 0; j < 4; j++) pw[j] = __builtin_amdgcn_exp2f(z[j] - be);
                *(lds_f32x4*)(lds + kPlPTable + (2 * (s & 1) + qtile) * kPlPTile +
                              ptable_chunk(ln, 4 * qhalf + qg)) = pw;
                if (qg == 0) ((lds_f32*)stats_row(s & 1, wave))[ln] = bw;
            } else if (issuing) {
                issue_stage(tg, std::integral_constant<int, 1>{});
            }
            m_run = M;
            __builtin_amdgcn_sched_barrier(0);

            // ---- the last stage; then this wave's gathers of batch s + 1 have landed
            if (issuing) {
                issue_stage(tg, std::integral_constant<int, 2>{});
                wait_but_one_batch();
            } else {
                wait_vmcnt<0>();
            }
            if constexpr (F == SMLA_ROW_UE8M0_SCALES)
                if (ghalf == 0 && s + 1 < nb)
                    expand_ue8m0_scales(lds + ((s + 1) % kPlRing) * kPlBatch + gtile * kSlot, lane);
            e0 = e1;
            e1 = e2;
            lds_barrier();   // ends the step
        }
        lds_barrier();   // the weight sums and the output rows are staged
        store_rows();
        if (a.arrive) merge_if_last<kPlWaves>(a, b, hb, wave, lane, (lds_u32*)(lds + kPlPTable));
        return;
    }

    auto value_loop = [&](auto rope_c) {
        constexpr bool kRope = decltype(rope_c)::value;   // second group is the rope
        constexpr int kNope = kRope ? 1 : 2;               // nope groups of this wave
        // the accumulators (and the rope wave's weight sum in the ninth)
        f32x4 acc[kRope ? 9 : 8];
#pragma unroll
        for (int i = 0; i < (kRope ? 9 : 8); i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY;
        wait_vmcnt<0>();   // step 0: this wave's gathers of batch 1 (prologue)
        lds_barrier();
        for (int s = 1; s <= nb; s++) {
            // the bases of batch s - 1
            float bk[4];
#pragma unroll
            for (int j = 0; j < 4; j++) bk[j] = ((lds_cf32*)stats_row((s - 1) & 1, j))[ln];
            const float M = fmaxf(fmaxf(m_run, fmaxf(bk[0], bk[1])), fmaxf(bk[2], bk[3]));
            // ---- value product of batch s - 1 over this wave's columns: every
            // operand of both tiles is read first, then the factors 2^(base - M)
            // of the four halves are formed, then the products run
            const lds_u8* const st0 = opaque(lds + ((s - 1) % kPlRing) * kPlBatch);
            const lds_u8* const pt0 = lds + kPlPTable + 2 * ((s - 1) & 1) * kPlPTile;
            const int vpos = lds_pos(8 * qg + (ln >> 1));
            const int r4 = ln >> 2, c4 = ln & 3;
            const int rpos0 = lds_pos(8 * qg + r4), rpos1 = lds_pos(8 * qg + 4 + r4);
            f32x4 Pw[kPlTiles][2], S[kPlTiles][kNope][2];
            i32x2 V[kPlTiles][kNope][4];
            s16x4 R[kPlTiles][kRope ? 4 : 1][2];
#pragma unroll
            for (int tt = 0; tt < kPlTiles; tt++) {
                const lds_u8* st = st0 + tt * kSlot;
                const lds_u8* pt = pt0 + tt * kPlPTile;
                Pw[tt][0] = *(lds_cf32x4*)(pt + ptable_chunk(ln, 2 * qg));
                Pw[tt][1] = *(lds_cf32x4*)(pt + ptable_chunk(ln, 2 * qg + 1));
#pragma unroll
                for (int gi = 0; gi < kNope; gi++) {
                    const int g = 2 * vi + gi;
                    lds_cf32* sT = (lds_cf32*)(st + kScaleTable) + g * kTile;
                    S[tt][gi][0] = *(lds_cf32x4*)(sT + lds_pos(8 * qg));
                    S[tt][gi][1] = *(lds_cf32x4*)(sT + lds_pos(8 * qg + 4));
#pragma unroll
                    for (int cb = 0; cb < 4; cb++)
                        V[tt][gi][cb] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                            (lds_i32x2*)(st + piece_addr(4 * g + cb, vpos, ln & 1)));
                }
                if constexpr (kRope) {
#pragma unroll
                    for (int dt = 0; dt < 4; dt++) {
                        const int piece = kCodePieces + 2 * dt + (c4 >> 1);
                        R[tt][dt][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_s16x4*)(st + piece_addr(piece, rpos0, c4 & 1)));
                        R[tt][dt][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_s16x4*)(st + piece_addr(piece, rpos1, c4 & 1)));
                    }
                }
            }

            // factors of the halves (0 for a half that kept nothing) and the
            // rescale of the accumulators when the running maximum rose
            float fh[4];
#pragma unroll
            for (int j = 0; j < 4; j++) fh[j] = bk[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(bk[j] - M);
            const float alpha = M > m_run ? __builtin_amdgcn_exp2f(m_run - M) : 1.f;   // 0 while nothing was kept
            m_run = M;
            if (!__all(alpha == 1.f)) {
#pragma unroll
                for (int i = 0; i < (kRope ? 9 : 8); i++) acc[i] *= alpha;
            }
            // (unconditional: a branch here would split the value
            // product's instruction stream, and p * 1 is exact)
#pragma unroll
            for (int tt = 0; tt < kPlTiles; tt++) {
                const float f = (qg >> 1) ? fh[2 * tt + 1] : fh[2 * tt];
                Pw[tt][0] *= f;
                Pw[tt][1] *= f;
            }
#pragma unroll
            for (int tt = 0; tt < kPlTiles; tt++) {
                const f32x4 p0 = Pw[tt][0], p1 = Pw[tt][1];
#pragma unroll
                for (int gi = 0; gi < kNope; gi++) {
                    // weights fp16(p * scale), exact fp8 -> fp16 value codes
                    const f16x8 bop = weights_f16(p0, p1, S[tt][gi][0], S[tt][gi][1]);
#pragma unroll
                    for (int cb = 0; cb < 4; cb++)
                        acc[4 * gi + cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            codes_to_f16((uint32_t)V[tt][gi][cb][0], (uint32_t)V[tt][gi][cb][1]), bop,
                            acc[4 * gi + cb], 0, 0, 0);
                }
                if constexpr (kRope) {
                    // rope: bf16 values as stored; weights split into bf16
                    // high parts and the bf16 of the remainders
                    u32x4 hi, lo;
                    hi[0] = pack_bf16x2(p0[0], p0[1]);
                    hi[1] = pack_bf16x2(p0[2], p0[3]);
                    hi[2] = pack_bf16x2(p1[0], p1[1]);
                    hi[3] = pack_bf16x2(p1[2], p1[3]);
                    lo[0] = pack_bf16x2(p0[0] - __uint_as_float(hi[0] << 16), p0[1] - __uint_as_float(hi[0] & 0xFFFF0000u));
                    lo[1] = pack_bf16x2(p0[2] - __uint_as_float(hi[1] << 16), p0[3] - __uint_as_float(hi[1] & 0xFFFF0000u));
                    lo[2] = pack_bf16x2(p1[0] - __uint_as_float(hi[2] << 16), p1[1] - __uint_as_float(hi[2] & 0xFFFF0000u));
                    lo[3] = pack_bf16x2(p1[2] - __uint_as_float(hi[3] << 16), p1[3] - __uint_as_float(hi[3] & 0xFFFF0000u));
                    const bf16x8 phi = __builtin_bit_cast(bf16x8, hi), plo = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
                    for (int dt = 0; dt < 4; dt++) {
                        const bf16x8 aop = __builtin_bit_cast(
                            bf16x8, __builtin_shufflevector(R[tt][dt][0], R[tt][dt][1], 0, 1, 2, 3, 4, 5, 6, 7));
                        f32x4 cc = acc[4 + dt];
                        cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, phi, cc, 0, 0, 0);
                        cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, plo, cc, 0, 0, 0);
                        acc[4 + dt] = cc;
                    }
                    // the weight sum of head ln as the product with a
                    // column of ones (every element of block 8 holds it)
                    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
                    f32x4 cl = acc[8];
                    cl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, phi, cl, 0, 0, 0);
                    cl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, plo, cl, 0, 0, 0);
                    acc[8] = cl;
                }
            }
            lds_barrier();   // ends the step
        }
        // ---- the weight sum of head ln, from the rope wave's product with a
        // column of ones (through a row that no gather writes), and this
        // wave's columns, not yet normalised, into the staged rows
        if constexpr (kRope)
            if (qg == 0) lsum[ln] = acc[8][0];
        {
            lds_u8* const o = lds + ln * kPlStagePitchF32 + 4 * (128 * vi + 4 * qg);
#pragma unroll
            for (int c = 0; c < 8; c++) *(lds_f32x4*)(o + 64 * c) = acc[c];
        }
        lds_barrier();   // the weight sums and the output rows are staged
        if (vi == 0 && qg == 0) {
            const float l_run = ((lds_cf32*)lsum)[ln];
            const float lse = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
            const int64_t bh = (int64_t)b * a.heads + head;
            if (final_out) a.lse[bh] = lse;
            else if (a.arrive) store4_device(a.lse_part + bh * a.nsplit + split, lse);
            else a.lse_part[bh * a.nsplit + split] = lse;
        }
        store_rows();
        if (a.arrive) merge_if_last<kPlWaves>(a, b, hb, wave, lane, (lds_u32*)(lds + kPlPTable));
    };
    if (vi < 3) value_loop(std::false_type{});
    else value_loop(std::true_type{});
}

// ---------------------------------------------------------------------------
// Per-head SIMT decode: the ablation baseline.  The production kernel that the
// shared-read rewrite replaced ("The Moment of Compilation", section "The
// Context: A Kernel Optimization Campaign"; "The Power-of-Two Trap", section
// "The Scene") ran one program per head in f32 on the vector units and read
// every selected row again for every head.  This is that design on gfx950: one
// wave per (sequence, head), lane l holding latent columns 8l..8l+7 (l < 56:
// fp8 codes of group l / 8 with its scale; l >= 56: rope), one row at a time
// through global loads, q . K reduced across the wave, an online softmax in
// fp32, no split of the list.  Same results as the main path (fp32 logits from
// exact operands), different cost: each row is read H times.
struct PerHeadArgs {
    const uint16_t* q;
    const uint8_t* kv;
    const int32_t* idx;
    const int32_t* seqlens;
    uint16_t* out;
    float* lse;
    int64_t kv_seq_stride;
    float logit_factor;   // scale * log2(e)
    int32_t batch, heads, topk;
    int32_t row_format;   // host only
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
    return x;
}

template <int F>
__global__ __launch_bounds__(256) void smla_per_head_kernel(PerHeadArgs a) {
    constexpr int RB = RowFormat<F>::kBytes;
    const int lane = threadIdx.x & 63;
    const int bh = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
    if (bh >= a.batch * a.heads) return;
    const int b = bh / a.heads;
    const bool rope = lane >= 56;

    float qv[8];
    {
        const u32x4 qq = *(const u32x4*)(a.q + (int64_t)bh * kLatent + 8 * lane);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            qv[2 * k] = __uint_as_float(qq[k] << 16);
            qv[2 * k + 1] = __uint_as_float(qq[k] & 0xFFFF0000u);
        }
    }
    const uint8_t* seq = a.kv + (int64_t)b * a.kv_seq_stride * RB;
    const int32_t* list = a.idx + (int64_t)b * a.topk;
    const int seqlen = (int)min((int64_t)a.seqlens[b], a.kv_seq_stride);   // never past the stride
    const int off = rope ? RowFormat<F>::kRopeOff + 16 * (lane - 56) : 8 * lane;

    // this lane's bytes of a row: 8 code bytes and the group scale, or 16 rope bytes
    auto load_raw = [&](int t) -> u32x4 {
        const uint8_t* row = seq + (int64_t)t * RB;
        const u32x2 lo = *(const u32x2*)(row + off);
        u32x4 r;
        r[0] = lo[0];
        r[1] = lo[1];
        if (rope) {
            const u32x2 hi = *(const u32x2*)(row + off + 8);
            r[2] = hi[0];
            r[3] = hi[1];
        } else {
            if constexpr (F == SMLA_ROW_UE8M0_SCALES)
                r[2] = __float_as_uint(ue8m0_value(row[SMLA_SCALE_OFFSET + (lane >> 3)]));
            else r[2] = *(const uint32_t*)(row + SMLA_SCALE_OFFSET + 4 * (lane >> 3));
            r[3] = 0;
        }
        return r;
    };
    // its 8 dequantised columns
    auto dequant = [&](const u32x4& r, float (&K)[8]) {
        if (rope) {
#pragma unroll
            for (int k = 0; k < 4; k++) {
                K[2 * k] = __uint_as_float(r[k] << 16);
                K[2 * k + 1] = __uint_as_float(r[k] & 0xFFFF0000u);
            }
        } else {
            const float sc = __uint_as_float(r[2]);
#pragma unroll
            for (int k = 0; k < 2; k++) {
                const f32x2 c0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r[k], 1.0f, false);
                const f32x2 c1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r[k], 1.0f, true);
                K[4 * k] = c0[0] * sc;
                K[4 * k + 1] = c0[1] * sc;
                K[4 * k + 2] = c1[0] * sc;
                K[4 * k + 3] = c1[1] * sc;
            }
        }
    };

    // kU rows in flight per step: their raw bytes are loaded together, the
    // logits reduced together, and each row is dequantised again for the
    // value sum (registers rather than memory traffic)
    float m = -INFINITY, l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    constexpr int kU = 8;
    for (int j0 = 0; j0 < a.topk; j0 += kU) {
        bool ok[kU];
        u32x4 raw[kU];
        float z[kU];
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const int t = j0 + u < a.topk ? list[j0 + u] : -1;
            ok[u] = t >= 0 && t < seqlen;
            raw[u] = ok[u] ? load_raw(t) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kU; u++) {
            float K[8];
            dequant(raw[u], K);
            float d = 0.f;
#pragma unroll
            for (int k = 0; k < 8; k++) d += qv[k] * K[k];
            z[u] = d;
        }
#pragma unroll
        for (int u = 0; u < kU; u++) z[u] = ok[u] ? wave_sum(z[u]) * a.logit_factor : -INFINITY;
        float mx = m;
#pragma unroll
        for (int u = 0; u < kU; u++) mx = fmaxf(mx, z[u]);
        if (mx == -INFINITY) continue;   // nothing kept so far
        const float alpha = __builtin_amdgcn_exp2f(m - mx);
        l *= alpha;
#pragma unroll
        for (int k = 0; k < 8; k++) o[k] *= alpha;
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const float p = __builtin_amdgcn_exp2f(z[u] - mx);
            l += p;
            float K[8];
            dequant(raw[u], K);
#pragma unroll
            for (int k = 0; k < 8; k++) o[k] += p * K[k];
        }
        m = mx;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    u32x4 pk;
#pragma unroll
    for (int k = 0; k < 4; k++) pk[k] = pack_bf16x2(o[2 * k] * inv, o[2 * k + 1] * inv);
    *(u32x4*)(a.out + (int64_t)bh * kLatent + 8 * lane) = pk;
    if (lane == 0) a.lse[bh] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

#if !defined(SMLA_PAGED_TU) && !defined(SMLA_FOURWAVE_TU)
struct Plan {
    int n_hb;     // 16-head blocks (workgroups per sequence and split)
    int nsplit;
    int chunk;    // list entries per split (multiple of kTile)
};

int row_bytes_of(int32_t fmt) {
    return fmt == SMLA_ROW_FP32_SCALES ? SMLA_ROW_BYTES : fmt == SMLA_ROW_UE8M0_SCALES ? SMLA_ROW_BYTES_UE8M0 : 0;
}

// Rows of one sequence are addressed by 32-bit byte offsets below 2^31.  (The
// paged calls do not use the stride but check it the same way.)
bool shape_ok(const smla_shape* s) {
    return s && row_bytes_of(s->row_format) > 0 && s->batch >= 0 && s->num_heads >= 0 &&
           s->num_heads % 16 == 0 && s->num_heads <= 256 && s->topk >= 0 && s->topk <= SMLA_MAX_TOPK &&
           s->num_splits >= 0 &&
           s->kv_seq_stride >= 1 && s->kv_seq_stride <= (((int64_t)1 << 31) - 1) / row_bytes_of(s->row_format);
}

// Paged pool: rows are record indices below 2^32 - 1 (the all-ones index is the
// masked row), the block-table row is a raw buffer below 2^31 bytes.
bool paged_ok(const smla_paged* g) {
    if (!g || g->page_size < 1 || g->page_size > (1 << 20) || (g->page_size & (g->page_size - 1)) != 0)
        return false;
    if (g->pages_per_seq < 1 || g->pages_per_seq > (1 << 29) || g->num_pages < 1) return false;
    return g->num_pages <= (int64_t)(0xFFFFFFFFu / (uint32_t)g->page_size);
}

int log2_exact(int32_t v) {
    int k = 0;
    while ((1 << k) < v) k++;
    return k;
}

constexpr int kComputeUnits = 256;   // MI355X; one workgroup per compute unit
// Longest split list (entries per workgroup) taken by the pipelined kernel for
// UE8M0 rows and on a paged pool; longer splits go to the four-wave kernel.
// Measured on MI355X (steps of the five benchmark workloads, three rounds):
// with fp32 group scales on a contiguous cache the pipelined kernel is ahead
// at every split length (1024 entries: 34.8-35.1 against 36.5-36.8 us; 2048:
// 49.8-50.0 against 50.4-50.9), with UE8M0 rows the four-wave kernel from
// 1024 entries on (39.4-39.5 against 39.9-40.2 us; 51.2-52.4 against
// 53.2-54.0: the pipelined kernel expands the scale bytes in two of its logit
// waves, the four-wave kernel in every wave).
constexpr int kPipelinedMaxChunk = 512;
constexpr int kMaxSplits = 4096;     // bound on the split count

// Environment overrides, read once when the library is loaded:
//   SMLA_NSPLIT=n           split count used when a shape leaves it to the
//                           library (num_splits == 0), 1 <= n <= kMaxSplits
//   SMLA_DEBUG_VALIDATE=1   scan the device-resident inputs before every decode
//   SMLA_KERNEL=four-wave | pipelined
//                           contiguous-cache kernel for every shape, instead of
//                           the choice by row format and split length
//                           (kPipelinedMaxChunk)
struct EnvConfig {
    int nsplit;           // 0: the heuristic
    int debug_validate;
    int kernel;           // 0: by row format and split length, 1: four-wave, 2: pipelined
};

EnvConfig read_env() {
    EnvConfig c = {0, 0, 0};
    if (const char* v = getenv("SMLA_KERNEL")) c.kernel = strcmp(v, "four-wave") == 0 ? 1 : strcmp(v, "pipelined") == 0 ? 2 : 0;
    if (const char* v = getenv("SMLA_NSPLIT")) {
        char* end = nullptr;
        const long n = strtol(v, &end, 10);
        if (end != v && *end == '\0' && n >= 1 && n <= kMaxSplits) c.nsplit = (int)n;
    }
    if (const char* v = getenv("SMLA_DEBUG_VALIDATE")) c.debug_validate = (v[0] != '\0' && strcmp(v, "0") != 0);
    return c;
}

const EnvConfig g_env = read_env();

// Split count when the caller leaves it to the library, from a cost model in
// fortieths of a tile time fitted to measured steps (MI355X; 16- and 64-head
// workloads of 1 to 96 sequences, 64 to 2048 entries, split counts 1 to 16):
// a workgroup costs its tiles per wave plus 3 tile times of fixed cost (its
// start, first entries and gather, and the merge) plus an eighth of a tile
// time per tile it holds (its waves share the compute unit's gather and LDS
// paths); a launch costs that times the number of rounds of kComputeUnits
// workgroups; a split list adds one tile time for the partials and the
// combine plus a fifth per four splits the combine merges.  Ties go to fewer
// splits.  For the single launch (single) a split list adds 3.25 tile times
// plus a fifth per split instead: the in-kernel merge (device-scope stores,
// the fences and the counter, then one workgroup reading every split's
// partial) costs more than the combine kernel, and more per split.  Its
// penalty over the combine's grows with the split count, so it never picks
// more splits than the two-launch model, and the same workspace suffices.
int choose_splits(int base, int tiles, bool single = false) {
    if (base <= 0 || tiles <= 1) return 1;
    int best = 1;
    long best_cost = -1;
    for (int ns = 1; ns <= tiles; ns++) {
        const int per_block = (tiles + ns - 1) / ns;
        if (ns > 1 && (tiles + per_block - 1) / per_block < ns) continue;   // same chunks as fewer splits
        const long rounds = ((long)base * ns + kComputeUnits - 1) / kComputeUnits;
        const long block = 40L * ((per_block + kWaves - 1) / kWaves + 3) + 5L * per_block;
        const long split_cost = single ? 130L + 8L * ns : 40L + 8L * ((ns + 3) / 4);
        const long cost = rounds * block + (ns > 1 ? split_cost : 0L);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = ns;
        }
    }
    return best;
}

Plan make_plan(const smla_shape* s, bool single = false) {
    Plan p;
    p.n_hb = s->num_heads / 16;
    const int tiles = (s->topk + kTile - 1) / kTile;
    int ns = s->num_splits;
    if (ns == 0) ns = g_env.nsplit > 0 ? g_env.nsplit : choose_splits(s->batch * p.n_hb, tiles, single);
    if (ns > tiles) ns = tiles;
    if (ns > kMaxSplits) ns = kMaxSplits;
    if (ns < 1) ns = 1;
    const int per = (s->topk + ns - 1) / ns;
    p.chunk = ((per + kTile - 1) / kTile) * kTile;
    if (p.chunk == 0) p.chunk = kTile;
    p.nsplit = (s->topk + p.chunk - 1) / p.chunk;
    if (p.nsplit < 1) p.nsplit = 1;
    return p;
}

// Workspace of a split launch: o_part fp32 [B][H][S][512], then lse_part fp32
// [B][H][S], each 256-byte aligned.
struct WorkspaceLayout {
    size_t lse_off, bytes;
};

WorkspaceLayout workspace_layout(const smla_shape* s, const Plan& p) {
    WorkspaceLayout w = {0, 0};
    if (p.nsplit <= 1) return w;
    const size_t rows = (size_t)s->batch * s->num_heads * p.nsplit;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    w.lse_off = up(rows * kLatent * sizeof(float));
    w.bytes = w.lse_off + up(rows * sizeof(float));
    return w;
}

size_t workspace_for(const smla_shape* s, const Plan& p) { return workspace_layout(s, p).bytes; }

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

// Fixed split-partial scratch of sparse_mla_decode_noalloc: a device array in
// the code object, one copy per GPU, held until the process ends.  Host code
// never passes its name to a kernel (that is a host-side stand-in, not a device
// address): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept here.
static __device__ __align__(256) uint8_t scratch[SMLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (nullptr on failure).
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}
#endif  // SMLA_PAGED_TU

}  // namespace

// The paged-pool instances of the decode kernel are built in a translation
// unit of their own (smla_paged.hip includes this file with SMLA_PAGED_TU):
// the contiguous instances are compiled with MFMA results in VGPRs (the
// logit accumulators then need no copy out of AGPRs, build.py), which makes
// the paged instances, 15 registers fuller, spill into AGPRs.  This launcher
// is their only entry; it returns false without launching when the two units
// disagree on the argument block.
__attribute__((visibility("hidden"))) bool smla_launch_paged_decode(const void* args, size_t bytes,
                                                                    int row_format, unsigned grid,
                                                                    hipStream_t hs);
// The contiguous-cache instances of the four-wave kernel likewise (included by
// smla_fourwave.hip with SMLA_FOURWAVE_TU): this unit's pipelined kernel is
// scheduled for instruction-level parallelism, which measured faster for it
// (build.py) and slower for the four-wave kernel.
__attribute__((visibility("hidden"))) bool smla_launch_fourwave_decode(const void* args, size_t bytes,
                                                                       int row_format, unsigned grid,
                                                                       hipStream_t hs);

#ifdef SMLA_PAGED_TU
bool smla_launch_paged_decode(const void* args, size_t bytes, int row_format, unsigned grid, hipStream_t hs) {
    DecodeArgs a;
    if (bytes != sizeof(a)) return false;
    memcpy(&a, args, sizeof(a));
    const dim3 g(grid), blk(64 * kWaves);
    if (row_format == SMLA_ROW_UE8M0_SCALES)
        hipLaunchKernelGGL((smla_decode_kernel<SMLA_ROW_UE8M0_SCALES, true>), g, blk, 0, hs, a.kv, a.idx, a.seqlens,
                           a.kv_seq_stride, a.topk, a.nsplit, a.chunk, a.n_hb, a.heads,
                           a.xcd_remap ? (int32_t)(grid / 8) : 0, a);
    else
        hipLaunchKernelGGL((smla_decode_kernel<SMLA_ROW_FP32_SCALES, true>), g, blk, 0, hs, a.kv, a.idx, a.seqlens,
                           a.kv_seq_stride, a.topk, a.nsplit, a.chunk, a.n_hb, a.heads,
                           a.xcd_remap ? (int32_t)(grid / 8) : 0, a);
    return true;
}
#elif defined(SMLA_FOURWAVE_TU)
bool smla_launch_fourwave_decode(const void* args, size_t bytes, int row_format, unsigned grid, hipStream_t hs) {
    DecodeArgs a;
    if (bytes != sizeof(a)) return false;
    memcpy(&a, args, sizeof(a));
    const dim3 g(grid), blk(64 * kWaves);
    const int32_t remap = a.xcd_remap ? (int32_t)(grid / 8) : 0;
    if (row_format == SMLA_ROW_UE8M0_SCALES)
        hipLaunchKernelGGL((smla_decode_kernel<SMLA_ROW_UE8M0_SCALES, false>), g, blk, 0, hs, a.kv, a.idx,
                           a.seqlens, a.kv_seq_stride, a.topk, a.nsplit, a.chunk, a.n_hb, a.heads, remap, a);
    else
        hipLaunchKernelGGL((smla_decode_kernel<SMLA_ROW_FP32_SCALES, false>), g, blk, 0, hs, a.kv, a.idx,
                           a.seqlens, a.kv_seq_stride, a.topk, a.nsplit, a.chunk, a.n_hb, a.heads, remap, a);
    return true;
}
#else

extern "C" {

int32_t smla_num_splits(const smla_shape* shape) {
    if (!shape_ok(shape)) return -1;
    return make_plan(shape).nsplit;
}

int32_t smla_num_splits_single_launch(const smla_shape* shape) {
    if (!shape_ok(shape)) return -1;
    return make_plan(shape, true).nsplit;
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
        case SMLA_ERR_SCRATCH: return "split partials exceed the fixed scratch of sparse_mla_decode_noalloc";
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

// paged: NULL for a contiguous cache; then block_table is not used.
static smla_status prepare(const void* q, const void* kv_cache, const int32_t* topk_idx,
                           const int32_t* seqlens, float scale, const smla_shape* shape,
                           const smla_paged* paged, const int32_t* block_table,
                           DecodeArgs* a, Plan* p, bool* nothing, bool single = false) {
    *nothing = false;
    if (!shape) return SMLA_ERR_NULL;
    if (!shape_ok(shape) || (paged && !paged_ok(paged))) return SMLA_ERR_SHAPE;
    if (shape->batch == 0 || shape->num_heads == 0) {   // nothing to touch
        *nothing = true;
        return SMLA_OK;
    }
    if (!q || !seqlens) return SMLA_ERR_NULL;
    if (shape->topk > 0 && (!kv_cache || !topk_idx)) return SMLA_ERR_NULL;
    if (paged && shape->topk > 0 && !block_table) return SMLA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(topk_idx, 4) || !aligned(seqlens, 4) ||
        !aligned(block_table, 4))
        return SMLA_ERR_ALIGN;
    *p = make_plan(shape, single);
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
    a->row_format = shape->row_format;
    if (paged) {
        a->block_table = block_table;
        a->page_shift = log2_exact(paged->page_size);
        a->pages_per_seq = paged->pages_per_seq;
        a->pool_rows = (uint32_t)(paged->num_pages << a->page_shift);
        if (shape->topk == 0) a->block_table = nullptr;   // nothing is gathered
    } else {
        a->seq_bytes = (uint32_t)(shape->kv_seq_stride * row_bytes_of(shape->row_format));
    }
    return SMLA_OK;
}

// Under SMLA_DEBUG_VALIDATE: the input scan, on the stream of the decode.
static bool launch_validate(const DecodeArgs& a, hipStream_t hs) {
    ValidateArgs v;
    v.idx = a.idx;
    v.seqlens = a.seqlens;
    v.block_table = a.block_table;
    v.reach = a.pages_per_seq > 0 ? ((int64_t)a.pages_per_seq << a.page_shift) : a.kv_seq_stride;   // paged : contiguous
    v.topk = a.topk;
    v.page_shift = a.page_shift;
    v.pages_per_seq = a.pages_per_seq;
    v.num_pages = a.pool_rows >> a.page_shift;
    hipLaunchKernelGGL(smla_validate_kernel, dim3(a.batch), dim3(256), 0, hs, v);
    return hipGetLastError() == hipSuccess;
}

static smla_status launch(const DecodeArgs& a, const Plan& p, hipStream_t hs) {
    const int grid = a.batch * p.n_hb * p.nsplit;
    DecodeArgs args = a;
    args.xcd_remap = (grid % 8 == 0) ? 1 : 0;
    const dim3 g(grid);
    (void)hipGetLastError();   // a launch error reported below is this launch's
    if (g_env.debug_validate && !launch_validate(a, hs)) return SMLA_ERR_HIP;
    // the pipelined kernel for fp32 group scales on a contiguous cache, and for
    // split lists of up to kPipelinedMaxChunk entries otherwise (on a paged
    // pool also at most kPlPagedBatches batches), unless SMLA_KERNEL chooses
    const bool paged = a.block_table != nullptr;
    const bool by_default = p.chunk <= kPipelinedMaxChunk || (!paged && a.row_format == SMLA_ROW_FP32_SCALES);
    const bool pipelined =
        (g_env.kernel == 2 || (g_env.kernel == 0 && by_default)) &&
        (!paged || (p.chunk <= kPlPagedBatches * kPlTiles * kTile &&
                    (uint64_t)a.pool_rows * (uint64_t)row_bytes_of(a.row_format) < (1ull << 31)));
    const int32_t remap = args.xcd_remap ? (int32_t)(grid / 8) : 0;
    if (pipelined) {
        const dim3 blk2(64 * kPlWaves);
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, g, blk2, 0, hs, args.kv, args.idx, args.seqlens, args.kv_seq_stride, args.topk,
                               args.nsplit, args.chunk, args.n_hb, args.heads, remap, args);
        };
        if (a.row_format == SMLA_ROW_UE8M0_SCALES) {
            if (paged) go(smla_decode_pipelined_kernel<SMLA_ROW_UE8M0_SCALES, true>);
            else go(smla_decode_pipelined_kernel<SMLA_ROW_UE8M0_SCALES, false>);
        } else {
            if (paged) go(smla_decode_pipelined_kernel<SMLA_ROW_FP32_SCALES, true>);
            else go(smla_decode_pipelined_kernel<SMLA_ROW_FP32_SCALES, false>);
        }
    } else if (paged) {
        if (!smla_launch_paged_decode(&args, sizeof(args), a.row_format, (unsigned)grid, hs)) return SMLA_ERR_HIP;
    } else {
        if (!smla_launch_fourwave_decode(&args, sizeof(args), a.row_format, (unsigned)grid, hs)) return SMLA_ERR_HIP;
    }
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

// single: a split shape merges its partials in the decode kernel (the last
// split of each head block to finish, counted at counters), with no combine
// launch
static smla_status decode_impl(const void* q, const void* kv_cache, const int32_t* block_table,
                               const int32_t* topk_idx, const int32_t* seqlens, float scale, void* out,
                               float* lse, const smla_shape* shape, const smla_paged* paged,
                               void* workspace, size_t workspace_bytes, void* stream, bool single = false,
                               uint32_t* counters = nullptr) {
    DecodeArgs a;
    Plan p;
    bool nothing;
    smla_status st = prepare(q, kv_cache, topk_idx, seqlens, scale, shape, paged, block_table, &a, &p, &nothing,
                             single);
    if (st != SMLA_OK || nothing) return st;
    if (!out || !lse) return SMLA_ERR_NULL;
    if (!aligned(out, 16) || !aligned(lse, 4)) return SMLA_ERR_ALIGN;
    const size_t need = workspace_for(shape, p);
    if (single && p.nsplit > 1) {
        if (!counters) return SMLA_ERR_NULL;
        if (!aligned(counters, 4)) return SMLA_ERR_ALIGN;
    }
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return SMLA_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return SMLA_ERR_ALIGN;
    }
    st = device_check();
    if (st != SMLA_OK) return st;
    a.out = (uint16_t*)out;
    a.lse = lse;
    if (p.nsplit > 1) {
        const WorkspaceLayout w = workspace_layout(shape, p);
        a.o_part = (float*)workspace;
        a.lse_part = (float*)((char*)workspace + w.lse_off);
        if (single) a.arrive = counters;
    }
    hipStream_t hs = (hipStream_t)stream;
    st = launch(a, p, hs);
    if (st != SMLA_OK) return st;
    if (p.nsplit > 1 && !single) {
        const int rws = shape->batch * shape->num_heads;
        hipLaunchKernelGGL(smla_combine_kernel, dim3((rws + 3) / 4), dim3(256), 0, hs, a.o_part,
                           a.lse_part, rws, p.nsplit, (uint16_t*)out, lse);
        if (hipGetLastError() != hipSuccess) return SMLA_ERR_HIP;
    }
    return SMLA_OK;
}

static smla_status partials_impl(const void* q, const void* kv_cache, const int32_t* block_table,
                                 const int32_t* topk_idx, const int32_t* seqlens, float scale,
                                 const smla_shape* shape, const smla_paged* paged, float* o_part,
                                 float* lse_part, void* stream) {
    DecodeArgs a;
    Plan p;
    bool nothing;
    smla_status st = prepare(q, kv_cache, topk_idx, seqlens, scale, shape, paged, block_table, &a, &p, &nothing);
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

smla_status sparse_mla_decode(const void* q, const void* kv_cache, const int32_t* topk_idx,
                              const int32_t* seqlens, float scale, void* out, float* lse,
                              const smla_shape* shape, void* workspace, size_t workspace_bytes,
                              void* stream) {
    return decode_impl(q, kv_cache, nullptr, topk_idx, seqlens, scale, out, lse, shape, nullptr, workspace,
                       workspace_bytes, stream);
}

smla_status sparse_mla_decode_partials(const void* q, const void* kv_cache, const int32_t* topk_idx,
                                       const int32_t* seqlens, float scale, const smla_shape* shape,
                                       float* o_part, float* lse_part, void* stream) {
    return partials_impl(q, kv_cache, nullptr, topk_idx, seqlens, scale, shape, nullptr, o_part, lse_part,
                         stream);
}

smla_status sparse_mla_decode_paged(const void* q, const void* kv_pool, const int32_t* block_table,
                                    const int32_t* topk_idx, const int32_t* seqlens, float scale, void* out,
                                    float* lse, const smla_shape* shape, const smla_paged* paged,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    if (!paged) return SMLA_ERR_NULL;
    return decode_impl(q, kv_pool, block_table, topk_idx, seqlens, scale, out, lse, shape, paged, workspace,
                       workspace_bytes, stream);
}

smla_status sparse_mla_decode_single_launch(const void* q, const void* kv_cache, const int32_t* block_table,
                                            const int32_t* topk_idx, const int32_t* seqlens, float scale,
                                            void* out, float* lse, const smla_shape* shape,
                                            const smla_paged* paged, void* workspace, size_t workspace_bytes,
                                            uint32_t* counters, void* stream) {
    return decode_impl(q, kv_cache, paged ? block_table : nullptr, topk_idx, seqlens, scale, out, lse, shape,
                       paged, workspace, workspace_bytes, stream, true, counters);
}

smla_status sparse_mla_decode_partials_paged(const void* q, const void* kv_pool, const int32_t* block_table,
                                             const int32_t* topk_idx, const int32_t* seqlens, float scale,
                                             const smla_shape* shape, const smla_paged* paged, float* o_part,
                                             float* lse_part, void* stream) {
    if (!paged) return SMLA_ERR_NULL;
    return partials_impl(q, kv_pool, block_table, topk_idx, seqlens, scale, shape, paged, o_part, lse_part,
                         stream);
}

smla_status sparse_mla_decode_per_head(const void* q, const void* kv_cache, const int32_t* topk_idx,
                                       const int32_t* seqlens, float scale, void* out, float* lse,
                                       const smla_shape* shape, void* stream) {
    DecodeArgs d;
    Plan p;
    bool nothing;
    smla_status st = prepare(q, kv_cache, topk_idx, seqlens, scale, shape, nullptr, nullptr, &d, &p, &nothing);
    if (st != SMLA_OK || nothing) return st;
    if (!out || !lse) return SMLA_ERR_NULL;
    if (!aligned(out, 16) || !aligned(lse, 4)) return SMLA_ERR_ALIGN;
    st = device_check();
    if (st != SMLA_OK) return st;
    PerHeadArgs a;
    memset(&a, 0, sizeof(a));
    a.q = (const uint16_t*)q;
    a.kv = (const uint8_t*)kv_cache;
    a.idx = topk_idx;
    a.seqlens = seqlens;
    a.out = (uint16_t*)out;
    a.lse = lse;
    a.kv_seq_stride = shape->kv_seq_stride;
    a.logit_factor = scale * kLog2e;
    a.batch = shape->batch;
    a.heads = shape->num_heads;
    a.topk = shape->topk;
    const int rows = shape->batch * shape->num_heads;
    const dim3 g((rows + 3) / 4), blk(256);
    (void)hipGetLastError();
    if (g_env.debug_validate && !launch_validate(d, (hipStream_t)stream)) return SMLA_ERR_HIP;
    if (shape->row_format == SMLA_ROW_UE8M0_SCALES)
        hipLaunchKernelGGL(smla_per_head_kernel<SMLA_ROW_UE8M0_SCALES>, g, blk, 0, (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL(smla_per_head_kernel<SMLA_ROW_FP32_SCALES>, g, blk, 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

smla_status sparse_mla_decode_noalloc(const void* q, const void* kv_cache, const int32_t* topk_idx,
                                      const int32_t* seqlens, float scale, void* out, float* lse,
                                      const smla_shape* shape, void* stream) {
    if (!shape) return SMLA_ERR_NULL;
    if (!shape_ok(shape)) return SMLA_ERR_SHAPE;
    const size_t need = workspace_for(shape, make_plan(shape));
    if (need > (size_t)SMLA_NOALLOC_SCRATCH_BYTES) return SMLA_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        const smla_status st = device_check();
        if (st != SMLA_OK) return st;
        ws = scratch_for_current_device();
        if (ws == nullptr) return SMLA_ERR_HIP;
    }
    return decode_impl(q, kv_cache, nullptr, topk_idx, seqlens, scale, out, lse, shape, nullptr, ws,
                       (size_t)SMLA_NOALLOC_SCRATCH_BYTES, stream);
}

int32_t smla_split_size(const smla_shape* shape) {
    if (!shape_ok(shape)) return -1;
    return make_plan(shape).chunk;
}

int32_t smla_debug_validate_enabled(void) { return g_env.debug_validate; }

smla_status smla_debug_flags(uint32_t* flags, int32_t clear) {
    if (!flags) return SMLA_ERR_NULL;
    smla_status st = device_check();
    if (st != SMLA_OK) return st;
    if (hipDeviceSynchronize() != hipSuccess) return SMLA_ERR_HIP;
    uint32_t v = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_flags), sizeof(v), 0, hipMemcpyDeviceToHost) != hipSuccess)
        return SMLA_ERR_HIP;
    if (clear) {
        const uint32_t zero = 0;
        if (hipMemcpyToSymbol(HIP_SYMBOL(g_debug_flags), &zero, sizeof(zero), 0, hipMemcpyHostToDevice) !=
            hipSuccess)
            return SMLA_ERR_HIP;
    }
    *flags = v;
    return SMLA_OK;
}

}  // extern "C"
#endif  // SMLA_PAGED_TU
