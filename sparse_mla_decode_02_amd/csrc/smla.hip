// Sparse MLA decode for AMD CDNA4 (gfx950): split-K decode kernel, log-sum-exp
// combine kernel, and the C ABI declared in include/smla.h.
//
// What is computed ("The Moment of Compilation", section "The Context: A Kernel
// Optimization Campaign"; "The Power-of-Two Trap", sections "The Scene" and
// "The Scale Indexing Complication"; "The 80KB Mystery", section "The Context:
// Optimizing Attention on Blackwell"): each query token attends, with all heads
// of this GPU, over the latent rows its top-k list selects; each row is read
// from HBM once and shared by every head in one matrix product; the selected
// list is split across workgroups (split-K) and the partial results merged
// with a log-sum-exp combine.
//
// Design on gfx950 (differs from the Triton kernel of the pages, which pads
// 448 to 512 because its tile ranges must be powers of two):
//  * 448 = 7 groups x 64 columns = 14 MFMA K-steps of 32: no padding at all.
//  * Workgroup = (sequence, group of up to 64 heads, split); one wave per 16
//    heads.  A 32-token tile of raw cache rows is gathered into LDS once per
//    workgroup with 16-byte loads and shared by all its waves.
//  * QK^T runs as S^T = K . Q^T on v_mfma_f32_16x16x32_bf16: the fp8 codes are
//    converted exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8 with unit scale),
//    q is used as stored, and each 64-column group's fp32 scale multiplies that
//    group's fp32 partial logits after the MFMA.  Logits are therefore as
//    accurate as fp32 accumulation allows.
//  * Online softmax in the log2 domain with lazy rescaling: the running base
//    only moves when the tile maximum exceeds it by more than 8 (so weights
//    stay below 2^8), which keeps the 128-register accumulator rescale rare.
//  * PV runs as O^T = V^T . P^T on v_mfma_f32_16x16x32_f16.  The S^T
//    accumulator layout already is the P^T operand layout, so no data moves
//    between lanes.  The group scale is folded into the weights
//    (fp16(p * scale_g)), the value codes enter exactly (fp8 -> fp16), and the
//    V^T operand is read from the row-major LDS tile with ds_read_b64_tr_b8
//    (rope: ds_read_b64_tr_b16 from an fp16 copy made at gather time).
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
typedef short s16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kPieces = 39;                  // 16-byte pieces staged per row (608 payload + pad)
constexpr int kRowLds = kPieces * 16;        // 624 bytes per token row in LDS
constexpr int kTileBlocks = (kTile * kPieces + 63) / 64;   // 1 KB blocks per tile (20)
constexpr int kMaxChunk = 2048;              // list entries per workgroup (index chunk in LDS)

// A zero row: masked list entries are gathered from here, so every staged byte
// is finite and a masked token contributes exactly zero.
__device__ __attribute__((aligned(256))) uint8_t g_zero_row[kRowBytes];

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

// Token held in MFMA k-slot `slot` (0..31) of a 32-token tile.  The S^T
// accumulator of lane group q holds tokens 4q..4q+3 (first 16-token half) and
// 16+4q..16+4q+3 (second half); the PV product uses k-slots 8q..8q+7 for them.
__device__ __forceinline__ int slot_token(int slot) {
    int q = slot >> 3, r = slot & 7;
    return r < 4 ? 4 * q + r : 16 + 4 * q + (r - 4);
}

// 16-byte gather of one lane straight into LDS at lds_base + 16 * lane
// (global_load_lds_dwordx4; the LDS base goes through M0 and must be
// wave-uniform).  Written as inline assembly so that the compiler does not
// treat every later LDS read as dependent on every gather in flight; the
// ordering is explicit instead: wait_vmcnt<N>() then lds_barrier().
__device__ __forceinline__ void gather16(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}

// Workgroup barrier without a memory fence: only this wave's LDS operations are
// waited for, so gathers still in flight into other ring slots stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
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
    float logit_factor;   // scale * log2(e)
    int32_t batch, heads, topk, nsplit, chunk, n_hg;
    int32_t force_partials;   // write split partials even when nsplit == 1
    int32_t xcd_remap;        // grid is a multiple of 8: keep a sequence's blocks on one XCD
};

// One 32-token tile for one wave: 16 heads x one latent half (DH = 0: nope
// groups 0..3; DH = 1: nope groups 4..6 and the rope).  st is the tile's ring
// slot (32 raw rows, kRowLds apart); vmask marks the kept tokens.  The partial
// logits of the two halves are exchanged through xs_mine / xs_other, and the
// caller's workgroup barrier separates the write from the partner's read.
template <int DH>
__device__ __forceinline__ void compute_tile(const uint8_t* st, uint64_t vmask, const bf16x8 (&qop)[8],
                                             f32x4 (&acc_o)[16], float& m_run, float& l_run,
                                             float* sT, float* xs_mine, const float* xs_other,
                                             int lane, float logit_factor) {
    constexpr int G0 = 4 * DH;           // first nope group
    constexpr int NG = DH == 0 ? 4 : 3;  // nope groups
    const int qg = lane >> 4, ln = lane & 15;

    // group scales of this half, transposed to [group][token] in this wave's
    // own LDS block (a wave's LDS operations complete in order)
#pragma unroll
    for (int k = 0; k < 2; k++) {
        const int e = lane + 64 * k;          // 0..127: token e / 4, group G0 + e % 4
        const int t = e >> 2, g = e & 3;
        if (g < NG) sT[g * kTile + t] = *(const float*)(st + t * kRowLds + SMLA_SCALE_OFFSET + 4 * (G0 + g));
    }

    // ---------------- partial S^T over this half's columns, per 16-token half:
    // operands read first, then one MFMA chain per group (independent chains)
    f32x4 s[2];
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
        const uint8_t* krow = st + (16 * tt + ln) * kRowLds;
        u32x4 raw[NG];
        u32x4 rrope[2];
#pragma unroll
        for (int g = 0; g < NG; g++) raw[g] = *(const u32x4*)(krow + 64 * (G0 + g) + 16 * qg);
        if (DH == 1) {
            rrope[0] = *(const u32x4*)(krow + SMLA_ROPE_OFFSET + 32 * qg);
            rrope[1] = *(const u32x4*)(krow + SMLA_ROPE_OFFSET + 16 + 32 * qg);
        }
        f32x4 acc[NG + 1];
#pragma unroll
        for (int g = 0; g < NG; g++)
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw[g][0], raw[g][1]), qop[2 * g],
                                                             f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        if (DH == 1)
            acc[NG] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rrope[0]), qop[6],
                                                              f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int g = 0; g < NG; g++)
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw[g][2], raw[g][3]), qop[2 * g + 1],
                                                             acc[g], 0, 0, 0);
        if (DH == 1)
            acc[NG] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rrope[1]), qop[7], acc[NG], 0, 0, 0);
        f32x4 v = DH == 1 ? acc[NG] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < NG; g++) v += *(const f32x4*)(sT + g * kTile + 16 * tt + 4 * qg) * acc[g];
        s[tt] = v;
    }

    // exchange with the partner wave; both form S = S_half0 + S_half1 in the
    // same order, so both hold bit-identical logits
    *(f32x4*)(xs_mine + 8 * lane) = s[0];
    *(f32x4*)(xs_mine + 8 * lane + 4) = s[1];
    lds_barrier();
    {
        const f32x4 o0 = *(const f32x4*)(xs_other + 8 * lane);
        const f32x4 o1 = *(const f32x4*)(xs_other + 8 * lane + 4);
        s[0] = DH == 0 ? s[0] + o0 : o0 + s[0];
        s[1] = DH == 0 ? s[1] + o1 : o1 + s[1];
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
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool need = mx > m_run + kTau;
    if (__any(need)) {
        const float m_new = need ? mx : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 16; i++) acc_o[i] *= alpha;
    }
    const float base = m_run == -INFINITY ? 0.f : m_run;
    float p[8];   // k-slot order: tokens 4q+j (j < 4), then 16+4q+(j-4)
#pragma unroll
    for (int j = 0; j < 8; j++) {
        p[j] = __builtin_amdgcn_exp2f(s[j >> 2][j & 3] - base);
        l_run += p[j];
    }

    // ---------------- O^T += V^T . P^T over this half's columns
    // V^T operands: tr8 source rows, lane 16q + j supplies token slot_token(8q + j/2), byte half j%2
    const uint8_t* tr_row = st + slot_token(8 * qg + (ln >> 1)) * kRowLds + 8 * (ln & 1);
    s16x4 rv[4][2];
    if (DH == 1) {
        // rope V^T via tr16: lane 16q + 4r + c supplies slot_token(8q + r), then (8q + 4 + r)
        const int col = 8 * (ln & 3);
        const uint8_t* r0 = st + slot_token(8 * qg + (ln >> 2)) * kRowLds + SMLA_ROPE_OFFSET + col;
        const uint8_t* r1 = st + slot_token(8 * qg + 4 + (ln >> 2)) * kRowLds + SMLA_ROPE_OFFSET + col;
#pragma unroll
        for (int dt = 0; dt < 4; dt++) {
            rv[dt][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(r0 + 32 * dt));
            rv[dt][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(r1 + 32 * dt));
        }
    }
#pragma unroll
    for (int g = 0; g < NG; g++) {
        i32x2 vraw[4];
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
            vraw[dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(tr_row + 64 * (G0 + g) + 16 * dt));
        const f32x4 sv0 = *(const f32x4*)(sT + g * kTile + 4 * qg);
        const f32x4 sv1 = *(const f32x4*)(sT + g * kTile + 16 + 4 * qg);
        // weights fp16(p * scale_g); exact fp8 -> fp16 value codes
        f16x8 bop;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            bop[j] = (_Float16)(p[j] * sv0[j]);
            bop[4 + j] = (_Float16)(p[4 + j] * sv1[j]);
        }
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
            acc_o[4 * g + dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                codes_to_f16((uint32_t)vraw[dt][0], (uint32_t)vraw[dt][1]), bop, acc_o[4 * g + dt], 0, 0, 0);
    }
    if (DH == 1) {
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
            f32x4 c = acc_o[12 + dt];
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, phi, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, plo, c, 0, 0, 0);
            acc_o[12 + dt] = c;
        }
    }
}

// Workgroup geometry.  A workgroup covers NHG groups of 16 heads.  Each head
// group is served by a pair of waves, one per latent half: half 0 holds nope
// groups 0..3 (columns 0..255), half 1 holds nope groups 4..6 and the rope
// (columns 256..511).  TW such sets of pairs take different tiles of the list
// (token-parallel) and are merged at the end.  Each wave thus holds half of
// its heads' query (32 registers) and half of their output accumulator (64
// registers), which lets two waves share a SIMD.
template <int NHG, int TW>
struct Geo {
    static constexpr int NWAVES = NHG * 2 * TW;
    static constexpr int NT = 64 * NWAVES;
    static constexpr int STAGE = kTileBlocks * 1024;              // one tile of raw rows
    static constexpr int NS = TW == 1 ? 5 : 6;                    // ring stages
    static constexpr int PMAX = (kTileBlocks + NWAVES - 1) / NWAVES;   // loads per wave per tile
    static constexpr int XS = NWAVES * 64 * 8 * 4;                // partial-logit exchange
    static constexpr int ST = NWAVES * 4 * kTile * 4;             // per-wave transposed scales
};

// One workgroup = (sequence b, head block hb, split s).  Rows of the split's
// list are gathered straight into an LDS ring of NS tiles (global_load_lds,
// 16 bytes per lane), NS - TW tiles in flight while TW tiles are computed.
template <int NHG, int TW>
__global__ __launch_bounds__(64 * NHG * 2 * TW, 2) void smla_decode_kernel(DecodeArgs a) {
    using G = Geo<NHG, TW>;
    constexpr int NWAVES = G::NWAVES, NT = G::NT, STAGE = G::STAGE, NS = G::NS;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * STAGE];
    __shared__ int32_t idx_s[kMaxChunk + TW * kTile];   // padded to whole rounds
    __shared__ __attribute__((aligned(16))) float xs[NWAVES][64 * 8];
    __shared__ __attribute__((aligned(16))) float sts[NWAVES][4 * kTile];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int dh = wave & 1;                   // latent half
    const int hw = (wave >> 1) % NHG;          // head group within the block
    const int tw = (wave >> 1) / NHG;          // token-parallel set
    const int partner = wave ^ 1;
    const int qg = lane >> 4;                  // lane group 0..3
    const int ln = lane & 15;                  // head column of the 16x16 tiles
    const int g0 = 4 * dh;                     // first nope group of this half
    const int ng = dh == 0 ? 4 : 3;            // nope groups of this half

    int bid = blockIdx.x;
    if (a.xcd_remap) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
    const int hb = bid % a.n_hg;
    bid /= a.n_hg;
    const int split = bid % a.nsplit;
    const int b = bid / a.nsplit;

    const int head = hb * (16 * NHG) + 16 * hw + ln;
    const int t_begin = split * a.chunk;
    const int t_end = min(a.topk, t_begin + a.chunk);
    const int n_ent = max(t_end - t_begin, 0);
    const int ntiles = (n_ent + kTile - 1) / kTile;
    const int nrounds = (ntiles + TW - 1) / TW;
    const int seqlen = a.seqlens[b];
    const uint8_t* kv_b = a.kv + (int64_t)b * a.kv_seq_stride * kRowBytes;

    // ---- index chunk -> LDS: the cache row of each entry, or -1 when masked
    {
        const int32_t* src = a.idx + (int64_t)b * a.topk + t_begin;
        for (int i = tid; i < nrounds * TW * kTile; i += NT) {
            int row = -1;
            if (i < n_ent) {
                row = src[i];
                if (row < 0 || row >= seqlen) row = -1;
            }
            idx_s[i] = row;
        }
    }
    // ---- this half of the query as the B operand of S^T = K . Q^T
    // (k-slot order matches the K reads: lane group q takes columns 16q..16q+15
    // of every 64-column group, 8 per K-step)
    bf16x8 qop[8];
    {
        const uint16_t* qh = a.q + ((int64_t)b * a.heads + head) * kLatent + 256 * dh;
#pragma unroll
        for (int g = 0; g < 4; g++)
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
                qop[2 * g + ks] = as_bf16x8(*(const u32x4*)(qh + 64 * g + 16 * qg + 8 * ks));
    }
    wait_vmcnt<0>();
    __syncthreads();

    // ---- gather of tile t into ring slot t % NS.  The tile is 1248 16-byte
    // pieces (32 rows x 39); piece c is row c/39, piece c%39, placed at byte 16c
    // of the slot.  1 KB block k of the slot is loaded by wave k % NWAVES.
    // Pieces past the tile and tiles past the end load the zero row, so each
    // wave issues the same number of loads for every tile.
    auto issue = [&](int t) {
        uint8_t* base = ring + (t % NS) * STAGE;
#pragma unroll
        for (int k = 0; k < G::PMAX; k++) {
            const int blk = k * NWAVES + wave;
            if (blk < kTileBlocks) {
                const int c = blk * 64 + lane;
                const int r = c / kPieces;
                const int p = c - r * kPieces;
                const uint8_t* src = g_zero_row;
                if (t < ntiles && c < kTile * kPieces) {
                    const int row = idx_s[t * kTile + r];
                    src = (row >= 0 ? kv_b + (int64_t)row * kRowBytes : g_zero_row) + 16 * p;
                }
                gather16(src, (uint32_t)(uintptr_t)(base + blk * 1024));
            }
        }
    };
    // loads this wave issues per tile: blocks wave, wave + NWAVES, ... < 20
    const int my_loads = (kTileBlocks - wave + NWAVES - 1) / NWAVES;

    f32x4 acc_o[16];
#pragma unroll
    for (int i = 0; i < 16; i++) acc_o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // base of the exponentials for this lane's head (log2 units)
    float l_run = 0.f;         // partial sum of weights over this lane's tokens

    float* sT = sts[wave];

    int frontier = 0;
    for (; frontier < NS - TW; frontier++) issue(frontier);

    for (int round = 0; round < nrounds; round++) {
        for (; frontier < round * TW + NS; frontier++) issue(frontier);
        // this wave's pieces of the round's tiles have landed (NS - TW tiles may
        // still be in flight), then everyone else's
        if (my_loads == G::PMAX) wait_vmcnt<(NS - TW) * G::PMAX>();
        else wait_vmcnt<(NS - TW) * (G::PMAX - 1)>();
        lds_barrier();

        const int tile = round * TW + tw;
        const uint8_t* st = ring + (tile % NS) * STAGE;
        const bool my_valid = lane < kTile && idx_s[tile * kTile + lane] >= 0;
        const uint64_t vmask = __ballot(my_valid);

        if (dh == 0)
            compute_tile<0>(st, vmask, qop, acc_o, m_run, l_run, sT, xs[wave], xs[partner], lane,
                            a.logit_factor);
        else
            compute_tile<1>(st, vmask, qop, acc_o, m_run, l_run, sT, xs[wave], xs[partner], lane,
                            a.logit_factor);
        lds_barrier();   // all waves are done with the round's slots before they are refilled
    }
    wait_vmcnt<0>();     // trailing zero-row loads of the ring

    // ---------------- epilogue
    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (TW > 1) {
        // merge the token-parallel sets through LDS (the ring is free now)
        __syncthreads();
        float* mb = (float*)ring;   // [NHG*2][TW-1][64 lanes][16 tiles * 4 + 2]
        constexpr int REC = 16 * 4 + 2;
        const int pair_slot = hw * 2 + dh;
        if (tw > 0) {
            float* dst = mb + ((pair_slot * (TW - 1) + (tw - 1)) * 64 + lane) * REC;
#pragma unroll
            for (int i = 0; i < 16; i++) *(f32x4*)(dst + 4 * i) = acc_o[i];
            dst[64] = m_run;
            dst[65] = l_tot;
        }
        __syncthreads();
        if (tw > 0) return;
        float M = m_run;
        for (int k = 0; k < TW - 1; k++)
            M = fmaxf(M, mb[((pair_slot * (TW - 1) + k) * 64 + lane) * REC + 64]);
        const float Ms = M == -INFINITY ? 0.f : M;
        const float a0 = __builtin_amdgcn_exp2f(m_run - Ms);
        l_tot *= a0;
#pragma unroll
        for (int i = 0; i < 16; i++) acc_o[i] *= a0;
        for (int k = 0; k < TW - 1; k++) {
            const float* src = mb + ((pair_slot * (TW - 1) + k) * 64 + lane) * REC;
            const float ak = __builtin_amdgcn_exp2f(src[64] - Ms);
            l_tot += ak * src[65];
#pragma unroll
            for (int i = 0; i < 16; i++) acc_o[i] += ak * *(const f32x4*)(src + 4 * i);
        }
        m_run = M;
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
    const int64_t bh = (int64_t)b * a.heads + head;
    if (a.nsplit == 1 && !a.force_partials) {
        uint16_t* o = a.out + bh * kLatent + 256 * dh;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int d0 = 16 * i + 4 * qg;
            u32x2 w;
            w[0] = pack_bf16x2(acc_o[i][0] * inv, acc_o[i][1] * inv);
            w[1] = pack_bf16x2(acc_o[i][2] * inv, acc_o[i][3] * inv);
            *(u32x2*)(o + d0) = w;
        }
        if (dh == 0 && qg == 0) a.lse[bh] = lse2 * kLn2;
    } else {
        float* o = a.o_part + (bh * a.nsplit + split) * kLatent + 256 * dh;
#pragma unroll
        for (int i = 0; i < 16; i++) *(f32x4*)(o + 16 * i + 4 * qg) = acc_o[i] * inv;
        if (dh == 0 && qg == 0) a.lse_part[bh * a.nsplit + split] = lse2 * kLn2;
    }
}

// Log-sum-exp merge: one wave per (b, h), 8 columns per lane.
__global__ __launch_bounds__(256) void smla_combine_kernel(const float* o_part, const float* lse_part,
                                                           int32_t rows, int32_t nsplit,
                                                           uint16_t* out, float* lse) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const float* lp = lse_part + (int64_t)row * nsplit;
    float M = -INFINITY;
    for (int i = 0; i < nsplit; i++) M = fmaxf(M, lp[i]);
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    float W = 0.f;
    if (M != -INFINITY) {
        for (int i = 0; i < nsplit; i++) {
            const float li = lp[i];
            if (li == -INFINITY) continue;
            const float w = __expf(li - M);
            W += w;
            const float* src = o_part + ((int64_t)row * nsplit + i) * kLatent + 8 * lane;
            acc0 += w * *(const f32x4*)src;
            acc1 += w * *(const f32x4*)(src + 4);
        }
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
    int nhg;      // 16-head groups per workgroup
    int tw;       // token-parallel wave sets per workgroup
    int n_hg;     // head blocks (workgroups per sequence and split)
    int nsplit;
    int chunk;    // list entries per split (multiple of kTile)
};

bool shape_ok(const smla_shape* s) {
    return s && s->batch >= 0 && s->num_heads >= 0 && s->num_heads % 16 == 0 &&
           s->num_heads <= 256 && s->topk >= 0 && s->num_splits >= 0 && s->kv_seq_stride >= 1;
}

Plan make_plan(const smla_shape* s) {
    Plan p;
    const int k = s->num_heads / 16;
    // head groups per workgroup: 4 when the heads allow it, else 3, 2, 1; the
    // workgroup then has 8 waves (6 for 3 groups) through token-parallel sets
    p.nhg = k % 4 == 0 ? 4 : k % 3 == 0 ? 3 : k % 2 == 0 ? 2 : 1;
    if (k == 0) p.nhg = 1;
    p.tw = p.nhg == 4 || p.nhg == 3 ? 1 : p.nhg == 2 ? 2 : 4;
    p.n_hg = k == 0 ? 0 : k / p.nhg;
    const int tiles = (s->topk + kTile - 1) / kTile;
    int ns = s->num_splits;
    if (ns == 0) {
        // about one workgroup per compute unit
        const int base = s->batch * (p.n_hg > 0 ? p.n_hg : 1);
        ns = base > 0 ? (256 + base - 1) / base : 1;
    }
    // the index chunk of a workgroup lives in LDS: at most kMaxChunk entries
    const int min_ns = (s->topk + kMaxChunk - 1) / kMaxChunk;
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

template <int NHG, int TW>
hipError_t launch_decode(const DecodeArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((smla_decode_kernel<NHG, TW>), dim3(grid), dim3(64 * NHG * 2 * TW), 0, st, a);
    return hipGetLastError();
}

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
    a->n_hg = p->n_hg;
    return SMLA_OK;
}

static smla_status launch(const DecodeArgs& a, const Plan& p, hipStream_t hs) {
    const int grid = a.batch * p.n_hg * p.nsplit;
    DecodeArgs args = a;
    args.xcd_remap = (grid % 8 == 0) ? 1 : 0;
    hipError_t e;
    switch (p.nhg) {
        case 4: e = launch_decode<4, 1>(args, grid, hs); break;
        case 3: e = launch_decode<3, 1>(args, grid, hs); break;
        case 2: e = launch_decode<2, 2>(args, grid, hs); break;
        default: e = launch_decode<1, 4>(args, grid, hs); break;
    }
    return e == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
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
