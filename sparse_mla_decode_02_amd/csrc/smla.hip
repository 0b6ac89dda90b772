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
constexpr int kChunks = 38;                 // 16-byte pieces of a row that are read (0..607)
constexpr int kKrStride = 624;              // LDS bytes per token row (608 + 16 pad)
constexpr int kRopeStride = 144;            // LDS bytes per token of the fp16 rope copy
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

struct __attribute__((aligned(16))) TileLds {
    uint8_t kr[kTile * kKrStride];       // raw row bytes 0..607 of each token
    uint8_t ropeh[kTile * kRopeStride];  // rope as fp16, 64 values per token
    float sq[8][kTile];                  // logit factor per (group, token): scale_g * c (rope: c)
    float sv[8][kTile];                  // value factor per (group, token): scale_g (rope: 1)
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

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    _Float16 ha = (_Float16)a, hb = (_Float16)b;
    uint16_t ua, ub;
    memcpy(&ua, &ha, 2);
    memcpy(&ub, &hb, 2);
    return (uint32_t)ua | ((uint32_t)ub << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
    uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    // round to nearest even; NaN stays NaN (quiet bit set)
    uint32_t ra = (ua & 0x7fffffffu) > 0x7f800000u ? (ua | 0x00400000u) : ua + 0x7fffu + ((ua >> 16) & 1u);
    uint32_t rb = (ub & 0x7fffffffu) > 0x7f800000u ? (ub | 0x00400000u) : ub + 0x7fffu + ((ub >> 16) & 1u);
    return (ra >> 16) | (rb & 0xffff0000u);
}

// Token held in MFMA k-slot `slot` (0..31) of a 32-token tile.  The S^T
// accumulator of lane group q holds tokens 4q..4q+3 (first 16-token half) and
// 16+4q..16+4q+3 (second half); the PV product uses k-slots 8q..8q+7 for them.
__device__ __forceinline__ int slot_token(int slot) {
    int q = slot >> 3, r = slot & 7;
    return r < 4 ? 4 * q + r : 16 + 4 * q + (r - 4);
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
};

// One workgroup = (sequence b, head group hg, split s); NW waves, 16 heads each.
template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void smla_decode_kernel(DecodeArgs a) {
    constexpr int NT = 64 * NW;
    constexpr int KPER = (kTile * kChunks + NT - 1) / NT;   // 16-byte pieces per thread per tile
    __shared__ TileLds lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int qg = lane >> 4;      // lane group 0..3
    const int ln = lane & 15;      // column within the 16x16 tile (head)

    int bid = blockIdx.x;
    const int hg = bid % a.n_hg;
    bid /= a.n_hg;
    const int split = bid % a.nsplit;
    const int b = bid / a.nsplit;

    const int head = hg * (16 * NW) + 16 * wave + ln;
    const int t_begin = split * a.chunk;
    const int t_end = min(a.topk, t_begin + a.chunk);
    const int ntiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;
    const int seqlen = a.seqlens[b];
    const int32_t* idx_b = a.idx + (int64_t)b * a.topk;
    const uint8_t* kv_b = a.kv + (int64_t)b * a.kv_seq_stride * kRowBytes;

    // ---- query as the B operand of S^T = K . Q^T (k-slot order matches the K reads)
    bf16x8 qn[7][2], qr[2];
    {
        const uint16_t* qh = a.q + ((int64_t)b * a.heads + head) * kLatent;
#pragma unroll
        for (int g = 0; g < 7; g++)
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
                qn[g][ks] = as_bf16x8(*(const u32x4*)(qh + 64 * g + 16 * qg + 8 * ks));
#pragma unroll
        for (int ks = 0; ks < 2; ks++)
            qr[ks] = as_bf16x8(*(const u32x4*)(qh + kNope + 16 * qg + 8 * ks));
    }

    f32x4 acc_o[32];
#pragma unroll
    for (int i = 0; i < 32; i++) acc_o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // base of the exponentials for this lane's head
    float l_run = 0.f;         // partial sum of weights over this lane's tokens

    // ---- gather staging: piece c = tid + k*NT of the tile -> (row r, piece p)
    // With 4 waves the next tile is prefetched into registers while the current
    // one is computed; with fewer waves the staging would not fit in registers,
    // so the tile is loaded in batches right before it is used.
    constexpr bool kPrefetch = NW == 4;
    constexpr int KB = kPrefetch ? KPER : 5;           // pieces staged at once
    u32x4 stage[KPER];
    auto issue_loads = [&](int tile, int k0) {
        const int t0 = t_begin + tile * kTile;
#pragma unroll
        for (int k = k0; k < (k0 + KB < KPER ? k0 + KB : KPER); k++) {
            const int c = tid + k * NT;
            const int r = c / kChunks, p = c - r * kChunks;
            const int t = t0 + r;
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (c < kTile * kChunks && t < t_end) {
                const int row = idx_b[t];
                if (row >= 0 && row < seqlen)
                    v = *(const u32x4*)(kv_b + (int64_t)row * kRowBytes + 16 * p);
            }
            stage[k] = v;
        }
    };
    auto store_stage = [&](int k0) {
#pragma unroll
        for (int k = k0; k < (k0 + KB < KPER ? k0 + KB : KPER); k++) {
            const int c = tid + k * NT;
            if (c >= kTile * kChunks) continue;
            const int r = c / kChunks, p = c - r * kChunks;
            const u32x4 v = stage[k];
            if (p < 28) {
                *(u32x4*)(lds.kr + r * kKrStride + 16 * p) = v;
            } else if (p < 30) {
                // group scales, slots 4(p-28)..4(p-28)+3; slot 7 (padding) is never
                // read and becomes the rope factor.  A skipped row is all zeros and
                // its weight is exactly 0, so its factors do not matter.
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int g = 4 * (p - 28) + j;
                    const float s = g == 7 ? 1.f : __uint_as_float(v[j]);
                    lds.sv[g][r] = s;
                    lds.sq[g][r] = s * a.logit_factor;
                }
            } else {
                *(u32x4*)(lds.kr + r * kKrStride + 16 * p) = v;
                u32x4 h;
#pragma unroll
                for (int j = 0; j < 4; j++)
                    h[j] = pack_f16x2(bf16_bits_to_f32(v[j] & 0xffffu), bf16_bits_to_f32(v[j] >> 16));
                *(u32x4*)(lds.ropeh + r * kRopeStride + 16 * (p - 30)) = h;
            }
        }
    };

    if (kPrefetch && ntiles > 0) issue_loads(0, 0);

    for (int tile = 0; tile < ntiles; tile++) {
        // validity of the tile's 32 entries (lanes 0..31 of every wave)
        const int t0 = t_begin + tile * kTile;
        bool my_valid = false;
        if (lane < kTile && t0 + lane < t_end) {
            const int row = idx_b[t0 + lane];
            my_valid = row >= 0 && row < seqlen;
        }
        const uint64_t vmask = __ballot(my_valid);

        if (kPrefetch) {
            store_stage(0);
        } else {
#pragma unroll
            for (int k0 = 0; k0 < KPER; k0 += KB) {
                issue_loads(tile, k0);
                store_stage(k0);
            }
        }
        __syncthreads();
        if (kPrefetch && tile + 1 < ntiles) issue_loads(tile + 1, 0);

        if (vmask != 0) {
            // ---------------- S^T = K . Q^T for two 16-token halves
            f32x4 s[2];
#pragma unroll
            for (int tt = 0; tt < 2; tt++) {
                const uint8_t* krow = lds.kr + (16 * tt + ln) * kKrStride;
                f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int g = 0; g < 7; g++) {
                    const u32x4 raw = *(const u32x4*)(krow + 64 * g + 16 * qg);
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw[0], raw[1]), qn[g][0], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw[2], raw[3]), qn[g][1], acc, 0, 0, 0);
                    const f32x4 f = *(const f32x4*)&lds.sq[g][16 * tt + 4 * qg];
                    sacc += f * acc;
                }
                {
                    const u32x4 r0 = *(const u32x4*)(krow + 480 + 32 * qg);
                    const u32x4 r1 = *(const u32x4*)(krow + 496 + 32 * qg);
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r0), qr[0], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r1), qr[1], acc, 0, 0, 0);
                    const f32x4 f = *(const f32x4*)&lds.sq[7][16 * tt + 4 * qg];
                    sacc += f * acc;
                }
#pragma unroll
                for (int j = 0; j < 4; j++)
                    if (!((vmask >> (16 * tt + 4 * qg + j)) & 1)) sacc[j] = -INFINITY;
                s[tt] = sacc;
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
                for (int i = 0; i < 32; i++) acc_o[i] *= alpha;
            }
            const float base = m_run == -INFINITY ? 0.f : m_run;
            float p[2][4];
#pragma unroll
            for (int tt = 0; tt < 2; tt++)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    p[tt][j] = __builtin_amdgcn_exp2f(s[tt][j] - base);
                    l_run += p[tt][j];
                }

            // ---------------- O^T += V^T . P^T, group by group
            // tr8 source rows: lane 16q + j supplies token slot_token(8q + j/2), byte half j%2
            const int tr_tok = slot_token(8 * qg + (ln >> 1));
            const uint8_t* tr_row = lds.kr + tr_tok * kKrStride + 8 * (ln & 1);
#pragma unroll
            for (int g = 0; g < 8; g++) {
                const f32x4 v0 = *(const f32x4*)&lds.sv[g][4 * qg];
                const f32x4 v1 = *(const f32x4*)&lds.sv[g][16 + 4 * qg];
                u32x4 bw;
                bw[0] = pack_f16x2(p[0][0] * v0[0], p[0][1] * v0[1]);
                bw[1] = pack_f16x2(p[0][2] * v0[2], p[0][3] * v0[3]);
                bw[2] = pack_f16x2(p[1][0] * v1[0], p[1][1] * v1[1]);
                bw[3] = pack_f16x2(p[1][2] * v1[2], p[1][3] * v1[3]);
                f16x8 bop;
                memcpy(&bop, &bw, 16);
#pragma unroll
                for (int dt = 0; dt < 4; dt++) {
                    f16x8 aop;
                    if (g < 7) {
                        const lds_i32x2* src = (const lds_i32x2*)(tr_row + 64 * g + 16 * dt);
                        const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)src);
                        aop = codes_to_f16((uint32_t)raw[0], (uint32_t)raw[1]);
                    } else {
                        // tr16: lane 16q + 4r + c supplies token slot_token(8q + r) (then 8q+4+r), columns 16dt + 4c..+3
                        const int r = ln >> 2, cc = ln & 3;
                        const uint8_t* base0 = lds.ropeh + slot_token(8 * qg + r) * kRopeStride + 2 * (16 * dt + 4 * cc);
                        const uint8_t* base1 = lds.ropeh + slot_token(8 * qg + 4 + r) * kRopeStride + 2 * (16 * dt + 4 * cc);
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)base0);
                        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)base1);
                        s16x4 both[2] = {lo, hi};
                        memcpy(&aop, both, 16);
                    }
                    acc_o[4 * g + dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, acc_o[4 * g + dt], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // ---------------- epilogue: total weight, normalise, write
    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
    const int64_t bh = (int64_t)b * a.heads + head;
    if (a.nsplit == 1 && !a.force_partials) {
        uint16_t* o = a.out + bh * kLatent;
#pragma unroll
        for (int i = 0; i < 32; i++) {
            const int d0 = 16 * i + 4 * qg;
            u32x2 w;
            w[0] = pack_bf16x2_rne(acc_o[i][0] * inv, acc_o[i][1] * inv);
            w[1] = pack_bf16x2_rne(acc_o[i][2] * inv, acc_o[i][3] * inv);
            *(u32x2*)(o + d0) = w;
        }
        if (qg == 0) a.lse[bh] = lse2 * kLn2;
    } else {
        float* o = a.o_part + (bh * a.nsplit + split) * kLatent;
#pragma unroll
        for (int i = 0; i < 32; i++) *(f32x4*)(o + 16 * i + 4 * qg) = acc_o[i] * inv;
        if (qg == 0) a.lse_part[bh * a.nsplit + split] = lse2 * kLn2;
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
    pk[0] = pack_bf16x2_rne(acc0[0] * inv, acc0[1] * inv);
    pk[1] = pack_bf16x2_rne(acc0[2] * inv, acc0[3] * inv);
    pk[2] = pack_bf16x2_rne(acc1[0] * inv, acc1[1] * inv);
    pk[3] = pack_bf16x2_rne(acc1[2] * inv, acc1[3] * inv);
    *(u32x4*)(out + (int64_t)row * kLatent + 8 * lane) = pk;
    if (lane == 0) lse[row] = W > 0.f ? M + logf(W) : -INFINITY;
}

// ---------------------------------------------------------------------------
// host side

struct Plan {
    int nw;       // waves (16 heads each) per workgroup
    int n_hg;     // head groups
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
    p.nw = k % 4 == 0 ? 4 : k % 3 == 0 ? 3 : k % 2 == 0 ? 2 : 1;
    if (k == 0) p.nw = 1;
    p.n_hg = k == 0 ? 0 : k / p.nw;
    const int tiles = (s->topk + kTile - 1) / kTile;
    int ns = s->num_splits;
    if (ns == 0) {
        // fill the machine: about one workgroup per compute unit for 4-wave
        // workgroups, four per compute unit for 1-wave workgroups
        const int target = 256 * (p.nw == 4 ? 1 : p.nw == 1 ? 4 : 2);
        const int base = s->batch * (p.n_hg > 0 ? p.n_hg : 1);
        ns = base > 0 ? (target + base - 1) / base : 1;
    }
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

template <int NW>
hipError_t launch_decode(const DecodeArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL(smla_decode_kernel<NW>, dim3(grid), dim3(64 * NW), 0, st, a);
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
    hipError_t e;
    switch (p.nw) {
        case 4: e = launch_decode<4>(a, grid, hs); break;
        case 3: e = launch_decode<3>(a, grid, hs); break;
        case 2: e = launch_decode<2>(a, grid, hs); break;
        default: e = launch_decode<1>(a, grid, hs); break;
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
