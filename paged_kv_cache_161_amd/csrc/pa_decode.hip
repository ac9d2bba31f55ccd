// pa_decode.hip -- decode-phase paged attention for CDNA4 (gfx950).
//
// What is computed: for each sequence b and q-head h, softmax(q . K^T * scale) . V over
// the sequence's context, with K/V rows found through the block table (token t is row
// t % 16 of physical block table[t / 16]) and q-head h reading kv-head h / group.
// Sources: LLM-101-CN "推理优化", sections "物理块与逻辑块" (logical -> physical blocks
// of 16 tokens) and "PagedAttention 内核实现" (decode: local attention per page, then
// the max / normaliser combine, exact rather than approximate); "Deep dive into vLLM
// 06", Online Softmax section (running max m, sum l, deferred divide) and the
// Flash-Decoding section (split the KV axis, merge the partials with the same rule);
// "大模型推理的三维本质原理解析与工程实践", section 6 GQA (q-head groups share a KV head).
//
// Work decomposition
//   grid  (P partitions, kv-heads x head-chunks, sequences); a workgroup of NW waves
//   owns one (sequence, kv-head, <=16 q-heads of its group, partition); with fp8 pools
//   and a group above 16, <=32 q-heads, as two MFMA column blocks whose products read
//   the same tile registers (groups above 16 with 16-bit pools take the shared-tile
//   kernel further below, which stages each tile in LDS for 32 or 64 q-heads).  Wave w walks
//   the partition's blocks w, w+NW, ...; at the end the NW waves merge their running
//   (m, l, O) in LDS.  A sequence whose context fits one partition is finished by
//   that workgroup; longer ones leave unnormalised partials (o, m, l) that
//   pa_decode_reduce merges in a second launch (the kernel boundary makes every
//   partition's partial visible to it).
//
// Per 16-token block a wave does two MFMA contractions, no LDS:
//   S[t][h]  = sum_e K[t][e] * Q[h][e]      A = K tile rows (token t = lane % 16),
//                                           B = Q rows of the group (head h = lane % 16)
//   O^T[e][h] += sum_t V^T[e][t] * P[t][h]  A = V^T tile (e = lane % 16),
//                                           B = P, which is exactly S's accumulator
//                                           layout (lane: head lane % 16, tokens
//                                           4*(lane/16) .. +3) rounded to 16 bits.
//   Because the V pool stores each block token-minor ([d][16]), the PV A operand
//   (4 consecutive tokens of one e) is a plain 8-byte load, and the K operand (8
//   consecutive e of one token) a 16-byte load; both come straight from HBM into
//   registers, and every q-head of the group shares them inside the MFMA.  Each tile
//   is read once per launch, so the loads carry the non-temporal hint unless the
//   call's block tables share blocks between sequences (then the caches serve the
//   repeats).
//   The softmax statistics of head h live in the 4 lanes {h, h+16, h+32, h+48}; the
//   tile max needs two cross-row exchanges, the O rescale none (O^T's head is lane % 16).
#include <math.h>

#include <type_traits>

#include "pa_common.h"
#include "pa_fp8.h"

namespace pa {

constexpr int kXcds = 8;   // MI355X: workgroup ids go round-robin over its 8 XCDs

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max_rows(float v)
{
    // max over the 4 lanes that share lane % 16 (one per 16-lane row)
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

__device__ __forceinline__ float wave_sum_rows(float v)
{
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// fp32 -> storage element, round to nearest even.
template <int DT>
__device__ __forceinline__ void store_elem(void *base, size_t idx, float v)
{
    if constexpr (DT == DT_F32) {
        static_cast<float *>(base)[idx] = v;
    } else if constexpr (DT == DT_F16) {
        static_cast<_Float16 *>(base)[idx] = static_cast<_Float16>(v);
    } else {
        static_cast<__bf16 *>(base)[idx] = static_cast<__bf16>(v);
    }
}

// ------------------------------------------------------------------ tile fragments

// 16-bit K/V (f16, bf16).  Lane (r = lane % 16, g = lane / 16).
template <int DT, int D>
struct Tile16 {
    static constexpr int NQK = D / 32;   // 16x16x32 MFMAs per block for S
    static constexpr int NPV = D / 16;   // 16x16x16 MFMAs per block for O (one per e-tile)
    u32x4 k[NQK];                        // K[r][32i + 8g .. +7]
    u32x2 v[NPV];                        // V^T[16n + r][4g .. 4g+3]

    // ks: elements from one K row to the next (D in the pool; padded rows in LDS)
    template <bool NT = false>
    __device__ __forceinline__ void load(const uint16_t *kt, const uint16_t *vt, int r, int g,
                                         int ks = D)
    {
#pragma unroll
        for (int i = 0; i < NQK; ++i)
            k[i] = load_kv<NT, u32x4>(kt + r * ks + 32 * i + 8 * g);
        // V^T as 16-byte half rows (half as many load instructions as 8-byte pieces,
        // which sets how fast one CU streams): lane (r, g) loads tokens 8 (g / 2) .. +7
        // of row 16 (2 i + g % 2) + r into v[2 i] (its first 4 tokens) and v[2 i + 1];
        // finish() swaps halves between lanes g and g ^ 1, once the loads have landed
        // (swapping here would make a prefetched tile wait for its own loads).
#pragma unroll
        for (int i = 0; i < NPV / 2; ++i) {
            const u32x4 w =
                load_kv<NT, u32x4>(vt + (16 * (2 * i + (g & 1)) + r) * kBlock + 8 * (g >> 1));
            v[2 * i] = u32x2{w[0], w[1]};
            v[2 * i + 1] = u32x2{w[2], w[3]};
        }
    }

    // After the loads have landed: v[n] = V^T[16 n + r][4 g .. 4 g + 3].
    __device__ __forceinline__ void finish()
    {
#pragma unroll
        for (int i = 0; i < NPV / 2; ++i) {
            auto a = __builtin_amdgcn_permlane16_swap(v[2 * i][0], v[2 * i + 1][0], false, false);
            auto b = __builtin_amdgcn_permlane16_swap(v[2 * i][1], v[2 * i + 1][1], false, false);
            v[2 * i] = u32x2{a[0], b[0]};
            v[2 * i + 1] = u32x2{a[1], b[1]};
        }
    }

    // Write the patched block back: K row `off` and every V^T piece (whole rows, so the
    // stores fill whole sectors; only token off's values differ from the pool's).
    __device__ __forceinline__ void store_row(uint16_t *kt, uint16_t *vt, int off, int r, int g) const
    {
        if (r == off) {
#pragma unroll
            for (int i = 0; i < NQK; ++i)
                *reinterpret_cast<u32x4 *>(kt + r * D + 32 * i + 8 * g) = k[i];
        }
#pragma unroll
        for (int n = 0; n < NPV; ++n)
            *reinterpret_cast<u32x2 *>(vt + (16 * n + r) * kBlock + 4 * g) = v[n];
    }

    // Replace token `off` of this block by a new row (k_row, v_row: D elements).
    __device__ __forceinline__ void patch(const uint16_t *k_row, const uint16_t *v_row, int off,
                                          int r, int g)
    {
        if (r == off) {
#pragma unroll
            for (int i = 0; i < NQK; ++i)
                k[i] = *reinterpret_cast<const u32x4 *>(k_row + 32 * i + 8 * g);
        }
        if (g == off / 4) {
            const int w = (off % 4) / 2, sh = 16 * (off % 2);
#pragma unroll
            for (int n = 0; n < NPV; ++n)
                v[n][w] = (v[n][w] & ~(0xFFFFu << sh)) | ((uint32_t)v_row[16 * n + r] << sh);
        }
    }
};

template <int DT, int D>
struct Q16 {
    u32x4 f[D / 32];                     // Q[h = r][32i + 8g .. +7]
    __device__ __forceinline__ void load(const uint16_t *qrow, bool valid, int g)
    {
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
            f[i] = valid ? *reinterpret_cast<const u32x4 *>(qrow + 32 * i + 8 * g)
                         : u32x4{0u, 0u, 0u, 0u};
    }
};

// fp32 K/V.  QK uses 16x16x4 MFMAs: lane (r, g) covers e in [g*D/4, (g+1)*D/4).
template <int D>
struct Tile32 {
    __device__ __forceinline__ void finish() {}
    static constexpr int NC = D / 16;    // float4 chunks
    f32x4 k[NC];                         // K[r][(D/4)g + 4c .. +3]
    f32x4 v[NC];                         // V^T[16n + r][4g .. 4g+3]

    template <bool NT = false>
    __device__ __forceinline__ void load(const float *kt, const float *vt, int r, int g,
                                         int ks = D)
    {
#pragma unroll
        for (int c = 0; c < NC; ++c)
            k[c] = load_kv<NT, f32x4>(kt + r * ks + (D / 4) * g + 4 * c);
#pragma unroll
        for (int n = 0; n < NC; ++n)
            v[n] = load_kv<NT, f32x4>(vt + (16 * n + r) * kBlock + 4 * g);
    }

    __device__ __forceinline__ void store_row(float *kt, float *vt, int off, int r, int g) const
    {
        if (r == off) {
#pragma unroll
            for (int c = 0; c < NC; ++c)
                *reinterpret_cast<f32x4 *>(kt + r * D + (D / 4) * g + 4 * c) = k[c];
        }
#pragma unroll
        for (int n = 0; n < NC; ++n)
            *reinterpret_cast<f32x4 *>(vt + (16 * n + r) * kBlock + 4 * g) = v[n];
    }

    __device__ __forceinline__ void patch(const float *k_row, const float *v_row, int off, int r,
                                          int g)
    {
        if (r == off) {
#pragma unroll
            for (int c = 0; c < NC; ++c)
                k[c] = *reinterpret_cast<const f32x4 *>(k_row + (D / 4) * g + 4 * c);
        }
        if (g == off / 4) {
#pragma unroll
            for (int n = 0; n < NC; ++n)
                v[n][off % 4] = v_row[16 * n + r];
        }
    }
};

template <int D>
struct Q32 {
    f32x4 f[D / 16];                     // Q[h = r][(D/4)g + 4c .. +3]
    __device__ __forceinline__ void load(const float *qrow, bool valid, int g)
    {
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
            f[c] = valid ? *reinterpret_cast<const f32x4 *>(qrow + (D / 4) * g + 4 * c)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
    }
};

// FP8 (OCP E4M3) K/V with 16-bit q.  The same lane roles as the 16-bit tiles, with
// half the bytes: each code converts exactly to the 16-bit MFMA type in registers
// (every E4M3 value is a bf16 and an f16 value), the per-tensor scales are applied
// in fp32 outside the MFMAs (one pair per pool, or per kv-head).  A lane loads K in 16-byte pieces (16 codes, two MFMAs'
// worth): chunk c = 4j + g of its row, so one load instruction covers 64 contiguous
// bytes of each of the 16 rows, as the 16-bit tile does.  MFMA i = 2j + h uses codes
// 8h .. 8h+7 of piece j, and the q fragments follow the same e mapping.
template <int AT, int D>
struct Tile8 {
    static constexpr int NKL = D / 64;   // 16-byte K pieces per lane
    static constexpr int NPV = D / 16;
    u32x4 k[NKL];                        // 16 codes of K[r][64j + 16g .. +15]
    uint32_t v[NPV];                     // 4 codes of V^T[16n + r][4g .. 4g+3]

    // V^T rows are 16 bytes.  Lane (r, g) loads whole rows 16 (g + 4 i) + r, i < NPV / 4
    // (each load instruction: 64 contiguous rows, 1 KiB), and the four lanes sharing r
    // transpose their 4 x 4 blocks of 4-byte pieces with two rounds of lane swaps
    // (16-lane, then 32-lane), so that v[4 i + j] = V^T[16 (4 i + j) + r][4 g .. 4 g + 3]
    // as the MFMA operand wants: 2 loads per block at d = 128 instead of 8.
    template <bool NT = false>
    __device__ __forceinline__ void load(const uint8_t *kt, const uint8_t *vt, int r, int g,
                                         int ks = D)
    {
#pragma unroll
        for (int j = 0; j < NKL; ++j)
            k[j] = load_kv<NT, u32x4>(kt + r * ks + 64 * j + 16 * g);
#pragma unroll
        for (int i = 0; i < NPV / 4; ++i) {
            const u32x4 w = load_kv<NT, u32x4>(vt + (16 * (g + 4 * i) + r) * kBlock);
            // lane g holds e[g][j] = w[j]; afterwards lane g's register j holds e[j][g]
            auto s01 = __builtin_amdgcn_permlane16_swap(w[0], w[1], false, false);
            auto s23 = __builtin_amdgcn_permlane16_swap(w[2], w[3], false, false);
            auto s02 = __builtin_amdgcn_permlane32_swap(s01[0], s23[0], false, false);
            auto s13 = __builtin_amdgcn_permlane32_swap(s01[1], s23[1], false, false);
            v[4 * i + 0] = s02[0];
            v[4 * i + 1] = s13[0];
            v[4 * i + 2] = s02[1];
            v[4 * i + 3] = s13[1];
        }
    }

    __device__ __forceinline__ void finish() {}

    __device__ __forceinline__ void store_row(uint8_t *kt, uint8_t *vt, int off, int r, int g) const
    {
        if (r == off) {
#pragma unroll
            for (int j = 0; j < NKL; ++j)
                *reinterpret_cast<u32x4 *>(kt + r * D + 64 * j + 16 * g) = k[j];
        }
#pragma unroll
        for (int n = 0; n < NPV; ++n)
            *reinterpret_cast<uint32_t *>(vt + (16 * n + r) * kBlock + 4 * g) = v[n];
    }

    // The new row arrives already as the codes the append stores.
    __device__ __forceinline__ void patch(const uint8_t *k_row, const uint8_t *v_row, int off,
                                          int r, int g)
    {
        if (r == off) {
#pragma unroll
            for (int j = 0; j < NKL; ++j)
                k[j] = *reinterpret_cast<const u32x4 *>(k_row + 64 * j + 16 * g);
        }
        if (g == off / 4) {
            const int sh = 8 * (off % 4);
#pragma unroll
            for (int n = 0; n < NPV; ++n)
                v[n] = (v[n] & ~(0xFFu << sh)) | ((uint32_t)v_row[16 * n + r] << sh);
        }
    }
};

// q fragments in the fp8 tile's e mapping: f[2j + h] = Q[r][64j + 16g + 8h .. +7].
template <int AT, int D>
struct Q8 {
    u32x4 f[D / 32];
    __device__ __forceinline__ void load(const uint16_t *qrow, bool valid, int g)
    {
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
            f[i] = valid ? *reinterpret_cast<const u32x4 *>(qrow + 64 * (i / 2) + 16 * g +
                                                            8 * (i % 2))
                         : u32x4{0u, 0u, 0u, 0u};
    }
};

// Two E4M3 codes (low or high half of w) -> two 16-bit values of type AT, packed.
template <int AT, bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_16(uint32_t w)
{
    if constexpr (AT == DT_BF16)
        return __builtin_bit_cast(uint32_t,
                                  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HIGH));
    else
        return __builtin_bit_cast(uint32_t,
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HIGH));
}

template <int DT, int AT, int D> struct Frags {          // 16-bit K/V, DT == AT
    using Tile = Tile16<DT, D>;
    using Q = Q16<DT, D>;
    using Elem = uint16_t;
    using QElem = uint16_t;
};
template <int D> struct Frags<DT_F32, DT_F32, D> {
    using Tile = Tile32<D>;
    using Q = Q32<D>;
    using Elem = float;
    using QElem = float;
};
template <int AT, int D> struct Frags<DT_FP8, AT, D> {
    using Tile = Tile8<AT, D>;
    using Q = Q8<AT, D>;
    using Elem = uint8_t;
    using QElem = uint16_t;
};

// 16x16x32 MFMA on 16-bit operands of type AT.
template <int AT>
__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (AT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 16x16x16 MFMA on 16-bit operands of type AT.
template <int AT>
__device__ __forceinline__ f32x4 mfma_k16(u32x2 a, u32x2 b, f32x4 c)
{
    if constexpr (AT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                         __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// fp32 weights -> two packed 16-bit words of type AT (RNE), and back to fp32.
template <int AT>
__device__ __forceinline__ u32x2 pack16(f32x4 p, f32x4 &rounded)
{
    if constexpr (AT == DT_BF16) {
        bf16x4 pb = __builtin_convertvector(p, bf16x4);
        rounded = __builtin_convertvector(pb, f32x4);
        return __builtin_bit_cast(u32x2, pb);
    } else {
        f16x4 ph = __builtin_convertvector(p, f16x4);
        rounded = __builtin_convertvector(ph, f32x4);
        return __builtin_bit_cast(u32x2, ph);
    }
}

// S[t][h] for the 16 tokens of a block (lane holds tokens 4g..4g+3 of head r).
template <int DT, int AT, int D>
__device__ __forceinline__ f32x4 scores(const typename Frags<DT, AT, D>::Tile &t,
                                        const typename Frags<DT, AT, D>::Q &q)
{
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s = __builtin_amdgcn_mfma_f32_16x16x4f32(t.k[c][j], q.f[c][j], s, 0, 0, 0);
    } else if constexpr (DT == DT_FP8) {
#pragma unroll
        for (int j = 0; j < D / 64; ++j) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t w0 = t.k[j][2 * h], w1 = t.k[j][2 * h + 1];
                const u32x4 kk = {e4m3x2_to_16<AT, false>(w0), e4m3x2_to_16<AT, true>(w0),
                                  e4m3x2_to_16<AT, false>(w1), e4m3x2_to_16<AT, true>(w1)};
                s = mfma_k32<AT>(kk, q.f[2 * j + h], s);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
            s = mfma_k32<AT>(t.k[i], q.f[i], s);
    }
    return s;
}

// O^T[e][h] += V^T[e][t] P[t][h].  p holds this lane's 4 weights (tokens 4g..4g+3 of
// head r).  Returns the weights as the MFMA consumed them (16-bit rounded for 16-bit
// and fp8 K/V), so the caller's normaliser sums exactly what was multiplied into V.
template <int DT, int AT, int D>
__device__ __forceinline__ f32x4 accumulate_pv(typename Frags<DT, AT, D>::Tile &t, f32x4 p,
                                               f32x4 (&o)[D / 16])
{
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int n = 0; n < D / 16; ++n)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.v[n][j], p[j], o[n], 0, 0, 0);
        return p;
    } else {
        f32x4 used;
        const u32x2 pk = pack16<AT>(p, used);
#pragma unroll
        for (int n = 0; n < D / 16; ++n) {
            if constexpr (DT == DT_FP8) {
                const u32x2 vv = {e4m3x2_to_16<AT, false>(t.v[n]), e4m3x2_to_16<AT, true>(t.v[n])};
                o[n] = mfma_k16<AT>(vv, pk, o[n]);
            } else {
                o[n] = mfma_k16<AT>(t.v[n], pk, o[n]);
            }
        }
        return used;
    }
}

// Zero the V^T entries of tokens >= valid in a partial block.  Rows past the context
// may hold anything (NaN included); a zero weight alone would not cancel them.
template <int DT, int AT, int D>
__device__ __forceinline__ void mask_tail_v(typename Frags<DT, AT, D>::Tile &t, int valid, int g)
{
    const int t0 = 4 * g;
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int n = 0; n < D / 16; ++n)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                t.v[n][j] = (t0 + j < valid) ? t.v[n][j] : 0.f;
    } else if constexpr (DT == DT_FP8) {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            m |= (t0 + j < valid) ? (0xFFu << (8 * j)) : 0u;
#pragma unroll
        for (int n = 0; n < D / 16; ++n)
            t.v[n] &= m;
    } else {
        const uint32_t m0 = (t0 < valid ? 0x0000FFFFu : 0u) | (t0 + 1 < valid ? 0xFFFF0000u : 0u);
        const uint32_t m1 = (t0 + 2 < valid ? 0x0000FFFFu : 0u) | (t0 + 3 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int n = 0; n < D / 16; ++n) {
            t.v[n][0] &= m0;
            t.v[n][1] &= m1;
        }
    }
}

// ------------------------------------------------------------------ partition kernel

// Waves per SIMD the register budget must allow: a tile ring of up to 64 VGPRs (two
// 16-bit tiles, or four fp8 tiles, at d = 128) fits three waves per SIMD with one
// column block of q-heads per wave, two with two.
constexpr int min_waves_per_simd(int dt, int d, int pf, int cb)
{
    return (d > 128 || dt == DT_F32)
               ? 1
               : ((pf + 1) * (dt == DT_FP8 ? 16 : 32) * d / 128 <= 64
                      ? (cb > 1 ? 2 : 3)
                      : ((pf + 1) * (dt == DT_FP8 ? 16 : 32) * d / 128 <= 96 ? 2 : 1));
}

// NT: K/V tiles are read with non-temporal loads (no block is shared between the
// batch's sequences; never for fp32 pools).  CB: 16-head MFMA column blocks per wave
// (the workgroup serves 16 CB q-heads of a group); with two, every K/V tile a wave
// loads feeds both blocks' products from the same registers.
template <int DT, int AT, int D, int NW, int PF, bool FUSE, bool NT, int CB>
__global__ __launch_bounds__(NW *kWave, min_waves_per_simd(DT, D, PF, CB)) void pa_decode_partition(DecodeArgs a)
{
    using F = Frags<DT, AT, D>;
    using Elem = typename F::Elem;        // K/V storage element
    using QElem = typename F::QElem;      // q / out element
    constexpr int DP = D + 4;                       // padded LDS row (floats)
    constexpr int HS = 16 * CB;                     // q-head slots of the workgroup

    extern __shared__ float smem[];
    float *s_m = smem;                              // [NW][HS]
    float *s_l = smem + NW * HS;                    // [NW][HS]
    int *s_bad = reinterpret_cast<int *>(smem + 2 * NW * HS);   // [NW] (16 ints reserved)
    float *s_o = smem + 2 * NW * HS + 16;           // [NW][GS][DP]

    // (partition, kv-head x head chunk, sequence rank).  A group above 16 CB q-heads runs
    // one workgroup per 16 CB heads (a head chunk), each streaming the same K/V: the ids are then
    // regrouped so a (sequence, kv-head, partition) unit's chunks are dispatched back
    // to back on one XCD (ids round-robin over the XCDs, so ids L, L + 8, ... share
    // one L2), where the later chunks find the K/V in that L2.  Units keep the plain
    // order (partition fastest, then kv-head, then sequence rank); the last group of
    // fewer than 8 units is spread without that alignment.
    int px = blockIdx.x, py = blockIdx.y, pz = blockIdx.z;
    if (a.wg_chunks > 1) {
        const int64_t C = a.wg_chunks;
        const int64_t hkv = gridDim.y / C;
        const int64_t L = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
        const int64_t U = (int64_t)gridDim.x * hkv * gridDim.z;
        const int64_t full = U / kXcds * kXcds;
        int64_t u, c;
        if (L < full * C) {
            const int64_t rr = L % (kXcds * C);
            c = rr / kXcds;
            u = L / (kXcds * C) * kXcds + rr % kXcds;
        } else {
            const int64_t rem = U - full, rr = L - full * C;
            c = rr / rem;
            u = full + rr % rem;
        }
        px = (int)(u % gridDim.x);
        const int64_t t = u / gridDim.x;
        py = (int)(t % hkv * C + c);
        pz = (int)(t / hkv);
    }
    const int p = px;
    const int kvh = py / a.wg_chunks;
    const int chunk = py - kvh * a.wg_chunks;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;

    const int gs = min(HS, a.group - chunk * HS);   // q-heads handled here
    const int hq0 = kvh * a.group + chunk * HS;     // first q-head of this workgroup

    // This wave's block ids (one per lane) and the group's q rows, issued before the
    // context length is known so the loads overlap: the table row has max_blocks
    // entries, so every index below that bound is readable.
    const int lb_begin = p * a.part_blocks;
    const int lb_cap = min(lb_begin + a.part_blocks, a.max_blocks);
    const int lb_lane = lb_begin + wave + lane * NW;   // this wave's (lane)-th block
    typename F::Q qf[CB];                            // q rows of the group (0 past gs)
    int bt_lane;
    auto load_seq = [&](int seq) {
        bt_lane = lb_lane < lb_cap ? a.block_tables[(size_t)seq * a.max_blocks + lb_lane] : 0;
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const bool hvalid = 16 * c + r < gs;
            const QElem *qrow = static_cast<const QElem *>(a.q) +
                               ((size_t)seq * a.num_q_heads + hq0 + (hvalid ? 16 * c + r : 0)) * D;
            qf[c].load(qrow, hvalid, g);
        }
    };

    // Workgroups are dispatched in z order, so with longest_first workgroup z takes the
    // sequence whose context length ranks z-th (longest first, ties by index): a ragged
    // batch then starts its longest streams first instead of last.  The loads for
    // sequence z go out first; they are kept when the rank maps z to itself (always,
    // in a batch of equal lengths) and reissued otherwise.
    int b = pz;
    load_seq(b);
    // This kv-head's scales: fp8 pools with per-head arrays read them here (a bad one
    // poisons the head's outputs); otherwise the pool's, folded in on the host.
    float sl_h = a.scale_log2, vs_h = a.v_scale, kq_h = a.k_quant, vq_h = a.v_quant;
    bool bad_scale = false;
    if constexpr (DT == DT_FP8) {
        if (a.k_head_scales) {
            const float s = a.k_head_scales[kvh];
            bad_scale |= !scale_ok(s);
            sl_h *= s;
            kq_h = s;
        }
        if (a.v_head_scales) {
            const float s = a.v_head_scales[kvh];
            bad_scale |= !scale_ok(s);
            vs_h = s;
            vq_h = s;
        }
        if (bad_scale)
            sl_h = 1.f;       // keeps the arithmetic tame; every output is NaN anyway
        // workgroup-uniform: kept in scalar registers, as kernel arguments are
        sl_h = uniform(sl_h);
        vs_h = uniform(vs_h);
        kq_h = uniform(kq_h);
        vq_h = uniform(vq_h);
    }
    int ctx = -1;
    if (a.longest_first) {
        int *s_ctx = reinterpret_cast<int *>(smem + 2 * NW * HS + 16 + NW * min(HS, a.group) * DP);
        const int nseq = gridDim.z;
        for (int t = tid; t < nseq; t += NW * kWave)
            s_ctx[t] = a.context_lens[t];
        __syncthreads();
        for (int t = tid; t < nseq; t += NW * kWave) {
            const int c = s_ctx[t];
            int rank = 0;
            for (int u = 0; u < nseq; ++u) {
                const int cu = s_ctx[u];
                rank += (cu > c || (cu == c && u < t)) ? 1 : 0;
            }
            if (rank == pz)
                s_ctx[nseq] = t;
        }
        __syncthreads();
        b = __builtin_amdgcn_readfirstlane(s_ctx[nseq]);
        ctx = s_ctx[b];
        if (b != pz)
            load_seq(b);
    } else {
        ctx = a.context_lens[b];
    }
    // unsigned: defined for any device value (a negative one is flagged just below)
    const int nblk_seq = ctx > 0 ? (int)(((unsigned)ctx + (kBlock - 1)) / kBlock) : 0;
    const bool bad_ctx = ctx < 0 || ctx > a.max_context_len || nblk_seq > a.max_blocks;
    const int lb_end = min(lb_begin + a.part_blocks, nblk_seq);

    if (bad_ctx || lb_begin >= lb_end) {
        // Nothing to stream.  When no workgroup of this sequence streams at all,
        // partition 0 writes its answer: zeros for an empty context, NaN for an
        // inconsistent length.
        if (p == 0 && (bad_ctx || nblk_seq == 0)) {
            const float fill = (bad_ctx || bad_scale) ? __builtin_nanf("") : 0.f;
            for (int idx = tid; idx < gs * D; idx += NW * kWave)
                store_elem<AT>(a.out, ((size_t)b * a.num_q_heads + hq0) * D + idx, fill);
        }
        return;
    }

    // Fused append: the sequence's new row is token ctx - 1, in logical block lb_new.
    // In every workgroup whose partition holds that block, the wave that computes on
    // it stages the row in LDS and patches it into its registers from there instead of
    // reading it back from the pool; in head chunk 0's workgroup it also writes the row
    // into the pool.  Nothing in this launch depends on the order of that write and
    // the pool reads (the block is private to the sequence).
    const bool fuse = FUSE && ctx >= 1;
    const int lb_new = fuse ? (ctx - 1) / kBlock : -1;
    const int off_new = fuse ? (ctx - 1) % kBlock : 0;
    const bool has_new = fuse && lb_new >= lb_begin && lb_new < lb_end;   // workgroup-uniform
    int ph_new = -1;       // block lb_new's physical id, where this workgroup writes the row
    __shared__ __align__(16) Elem s_newk[FUSE ? D : 16];   // the row as the pool stores it
    __shared__ __align__(16) Elem s_newv[FUSE ? D : 16];

    const int nb = lb_end - lb_begin;
    const int my_n = nb > wave ? (nb - wave + NW - 1) / NW : 0;   // <= 64 (host-checked)

    const Elem *kbase = static_cast<const Elem *>(a.k_pool) + (size_t)kvh * kBlock * D;
    const Elem *vbase = static_cast<const Elem *>(a.v_pool) + (size_t)kvh * kBlock * D;
    const size_t blk_stride = (size_t)a.num_kv_heads * kBlock * D;

    float m_run[CB], l_run[CB];
    f32x4 o[CB][D / 16];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        m_run[c] = -INFINITY;
        l_run[c] = 0.f;
#pragma unroll
        for (int n = 0; n < D / 16; ++n)
            o[c][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bool tbl_bad = bad_scale;   // (workgroup-uniform)

    auto phys_of = [&](int i) -> size_t {
        int ph = __builtin_amdgcn_readlane(bt_lane, i);
        if ((unsigned)ph >= (unsigned)a.num_blocks) {   // never read outside the pool
            tbl_bad = true;
            ph = 0;
        }
        return (size_t)ph * blk_stride;
    };

    // PATCH: this call may hold the block that receives the new row (fused append).
    auto process = [&](auto patch_tag, typename F::Tile &t, int i) {
        constexpr bool PATCH = decltype(patch_tag)::value;
        t.finish();
        const int lb = lb_begin + wave + i * NW;
        const int valid = ctx - lb * kBlock;            // >= 1
        if constexpr (PATCH) {
            if (lb == lb_new) {                         // wave-uniform
                t.patch(s_newk, s_newv, off_new, r, g);
                if (ph_new >= 0) {                      // head chunk 0: into the pool
                    const size_t tile = ((size_t)ph_new * a.num_kv_heads + kvh) * kBlock * D;
                    t.store_row(static_cast<Elem *>(const_cast<void *>(a.k_pool)) + tile,
                                static_cast<Elem *>(const_cast<void *>(a.v_pool)) + tile,
                                off_new, r, g);
                }
            }
        }
        f32x4 x[CB];
#pragma unroll
        for (int c = 0; c < CB; ++c)
            x[c] = scores<DT, AT, D>(t, qf[c]) * sl_h;
        if (valid < kBlock) {
#pragma unroll
            for (int c = 0; c < CB; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    x[c][j] = (4 * g + j < valid) ? x[c][j] : -INFINITY;
            mask_tail_v<DT, AT, D>(t, valid, g);
        }
        // The running max is only a reference point: O and l are both scaled by
        // 2^(-m), which cancels in O / l (and in the merges of waves and partitions).
        // It is moved only when a score exceeds it by more than kRescaleSlack (weights
        // stay <= 256), so the cross-row max, the exp2 and the rescale of O and l run
        // about once per wave instead of whenever a head sees a new maximum.  An empty
        // history (-inf) always takes the first finite max; an all-masked lane never
        // moves it.
        float lmx[CB];
        bool grow = false;
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            lmx[c] = fmaxf(fmaxf(x[c][0], x[c][1]), fmaxf(x[c][2], x[c][3]));
            grow |= lmx[c] - m_run[c] > kRescaleSlack;
        }
        if (__any(grow)) {
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                const float m_new = fmaxf(m_run[c], wave_max_rows(lmx[c]));
                const float alpha = fast_exp2(m_run[c] - m_new);
#pragma unroll
                for (int n = 0; n < D / 16; ++n)
                    o[c][n] *= alpha;
                l_run[c] *= alpha;
                m_run[c] = m_new;
            }
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            f32x4 pw;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                pw[j] = fast_exp2(x[c][j] - m_run[c]);
            const f32x4 pu = accumulate_pv<DT, AT, D>(t, pw, o[c]);
            l_run[c] += (pu[0] + pu[1]) + (pu[2] + pu[3]);
        }
    };

    // Ring of PF + 1 tiles: block i + PF is loaded while block i is computed.  The
    // inner loop is fully unrolled so every ring slot stays a fixed register range.
    auto prologue = [&](typename F::Tile (&ring)[PF + 1]) {
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            if (k < my_n) {
                const size_t off = phys_of(k);
                ring[k].template load<NT>(kbase + off, vbase + off, r, g);
            }
        }
    };
    // The new row of a fused append lands in the sequence's last block, which is the
    // last block of the wave that holds it; with FUSE the loop stops one block short
    // and that block is computed apart, so the loop itself carries no patch test.
    using NoPatch = std::integral_constant<bool, false>;
    using Patch = std::integral_constant<bool, true>;
    auto stream_blocks = [&](typename F::Tile (&ring)[PF + 1]) {
        const int n_loop = FUSE ? my_n - 1 : my_n;
        for (int i = 0; i < n_loop; i += PF + 1) {
#pragma unroll
            for (int u = 0; u <= PF; ++u) {
                const int it = i + u;
                if (it < n_loop) {
                    if (it + PF < my_n) {
                        const size_t off = phys_of(it + PF);
                        ring[(u + PF) % (PF + 1)].template load<NT>(kbase + off, vbase + off, r, g);
                    }
                    process(NoPatch{}, ring[u], it);
                }
            }
        }
        if constexpr (FUSE) {
            const int ul = n_loop % (PF + 1);
#pragma unroll
            for (int u = 0; u <= PF; ++u)
                if (u == ul)
                    process(Patch{}, ring[u], n_loop);
        }
    };
    if constexpr (FUSE) {
        // The new row's block is the last block of wave w_new, and that wave alone
        // stages the row (its table lane already holds the block's id), later patches it
        // into the block's tile from its own LDS copy and, in head chunk 0, writes the
        // patched tile's row back (whole V^T rows, so the stores fill whole sectors), so
        // no other wave waits.  Its loads go out before the first tiles' loads, which
        // are issued for every wave (a wave without blocks loads pool block 0, which
        // always exists, without consulting the table, and never uses it): the count of
        // loads issued after the row's is fixed, and staging waits for the row alone.
        const bool stager = has_new && wave == (lb_new - lb_begin) % NW;    // wave-uniform
        QElem nk[(D + kWave - 1) / kWave], nv[(D + kWave - 1) / kWave];
        if (stager) {
            const QElem *kr = static_cast<const QElem *>(a.k_new) +
                              ((size_t)b * a.num_kv_heads + kvh) * D;
            const QElem *vr = static_cast<const QElem *>(a.v_new) +
                              ((size_t)b * a.num_kv_heads + kvh) * D;
#pragma unroll
            for (int j = 0; j < (D + kWave - 1) / kWave; ++j) {
                nk[j] = kr[min(lane + j * kWave, D - 1)];
                nv[j] = vr[min(lane + j * kWave, D - 1)];
            }
        }
        typename F::Tile ring[PF + 1];
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            const size_t off = my_n > 0 ? phys_of(min(k, my_n - 1)) : 0;
            ring[k].template load<NT>(kbase + off, vbase + off, r, g);
        }
        if (stager) {
            const int ph = __builtin_amdgcn_readlane(bt_lane, (lb_new - lb_begin) / NW);
            ph_new = (chunk == 0 && (unsigned)ph < (unsigned)a.num_blocks) ? ph : -1;
#pragma unroll
            for (int j = 0; j < (D + kWave - 1) / kWave; ++j) {
                const int e = lane + j * kWave;
                if (e < D) {
                    Elem sk, sv;
                    if constexpr (DT == DT_FP8) {
                        sk = (Elem)e4m3_of_16(nk[j], a.act_bf16 != 0, kq_h);
                        sv = (Elem)e4m3_of_16(nv[j], a.act_bf16 != 0, vq_h);
                    } else {
                        sk = nk[j];
                        sv = nv[j];
                    }
                    s_newk[e] = sk;
                    s_newv[e] = sv;
                }
            }
        }
        if (my_n > 0)
            stream_blocks(ring);
    } else if (my_n > 0) {
        typename F::Tile ring[PF + 1];
        prologue(ring);
        stream_blocks(ring);
    }
#pragma unroll
    for (int c = 0; c < CB; ++c)
        l_run[c] = wave_sum_rows(l_run[c]);

    // ---- merge the NW waves' (m, l, O) in LDS
    if (lane == 0)
        s_bad[wave] = tbl_bad ? 1 : 0;
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        const int h = 16 * c + r;
        if (g == 0) {
            s_m[wave * HS + h] = m_run[c];
            s_l[wave * HS + h] = l_run[c];
        }
        if (h < gs) {
#pragma unroll
            for (int n = 0; n < D / 16; ++n)
                *reinterpret_cast<f32x4 *>(s_o + (wave * gs + h) * DP + 16 * n + 4 * g) = o[c][n];
        }
    }
    __syncthreads();

    bool any_bad = false;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        any_bad |= s_bad[w] != 0;
    // A sequence that fits one partition is finished here; longer ones leave
    // unnormalised partials for pa_decode_reduce.
    const bool partial = a.split && nblk_seq > a.part_blocks;
    const float qnan = __builtin_nanf("");
    for (int idx = tid; idx < gs * D; idx += NW * kWave) {
        const int h = idx / D;
        const int e = idx - h * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            M = fmaxf(M, s_m[w * HS + h]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = s_m[w * HS + h];
            const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
            num += f * s_o[(w * gs + h) * DP + e];
            den += f * s_l[w * HS + h];
        }
        const size_t row = (size_t)b * a.num_q_heads + hq0 + h;
        if (!partial) {
            const float val = any_bad ? qnan : (den > 0.f ? num / den * vs_h : 0.f);
            store_elem<AT>(a.out, row * D + e, val);
        } else {
            const size_t slot = row * a.num_parts + p;
            a.ws_o[slot * D + e] = any_bad ? qnan : num * vs_h;
            if (e == 0) {
                a.ws_m[slot] = any_bad ? qnan : M;
                a.ws_l[slot] = any_bad ? qnan : den;
            }
        }
    }
}

// ------------------------------------------------------------------ shared-tile kernel

// Groups above 16 q-heads with 16-bit pools (head_dim <= 128).  One 8-wave workgroup owns (sequence,
// kv-head, up to 16 CH q-heads of its group, partition).  Wave w computes head chunk
// c = w % CH over the blocks of block lane j = w / CH (blocks j, j + NB, ... of the
// partition, NB = 8 / CH).  Each K/V tile is read from HBM once per workgroup: the CH
// waves of a block lane each load a share of it and write it to LDS, and after a
// barrier every one of them reads the whole tile into its MFMA fragments, so one
// stream of K/V serves 16 CH q-heads, each wave holding the registers of one chunk
// (q fragments, O accumulators).  K rows are padded by 16 bytes in LDS so the fragment
// reads of a row group fall on distinct banks.  Groups above 64 q-heads take several
// such workgroups per (sequence, kv-head, partition), regrouped onto one XCD as in
// the per-chunk kernel.
constexpr int kSharedWaves = 8;

template <int DT, int D, int CH>
struct SharedShape {
    static constexpr int EB = DT == DT_F32 ? 4 : (DT == DT_FP8 ? 1 : 2);
    static constexpr int NB = kSharedWaves / CH;       // block lanes
    static constexpr int HS = 16 * CH;                 // q-head slots of the workgroup
    static constexpr int DP = D + 4;
    static constexpr int KROW = D * EB + 16;           // padded K row in LDS (bytes)
    static constexpr int KBYTES = kBlock * KROW;
    static constexpr int VBYTES = D * kBlock * EB;
    static constexpr int TBYTES = KBYTES + VBYTES;     // one tile in LDS
    static constexpr int KP = D * EB;                  // 16-byte pieces of a K tile
    static constexpr int PIECES = KP + VBYTES / 16;
    static constexpr int PPL = (PIECES + CH * kWave - 1) / (CH * kWave);   // per lane
    // Tiles a block lane takes between two barriers (16 KB of K/V at head_dim 128, so
    // the dependent chains of several tiles overlap; an fp32 tile is 16 KB alone), and
    // two groups of them in flight per block lane.  With 4 block lanes (CH = 2) one
    // 16-bit tile per lane and barrier measured 3-4 % faster under non-temporal loads;
    // with 2 lanes (CH = 4) two tiles stay faster.
    static constexpr int TPI = DT == DT_F32 ? 1 : (DT == DT_FP8 ? 4 : (CH == 2 ? 1 : 2));
    static constexpr int RING = 2;
    static constexpr int TILE_AREA = NB * 2 * TPI * TBYTES;
    static constexpr int MERGE_AREA = (2 * NB * HS + NB * HS * DP) * 4 + kSharedWaves * 4;
    static constexpr int AREA = TILE_AREA > MERGE_AREA ? TILE_AREA : MERGE_AREA;
};

template <int DT, int AT, int D, int CH, bool FUSE, bool NT>
__global__ __launch_bounds__(kSharedWaves *kWave, 2) void pa_decode_shared(DecodeArgs a)
{
    using F = Frags<DT, AT, D>;
    using Elem = typename F::Elem;
    using QElem = typename F::QElem;
    using S = SharedShape<DT, D, CH>;
    constexpr int NW = kSharedWaves;
    constexpr int NB = S::NB, HS = S::HS, DP = S::DP, PPL = S::PPL, R = S::RING, TPI = S::TPI;

    // [NB][2][TPI][TBYTES] tile buffers while streaming; after the loop the same bytes
    // hold the merge; the longest-first ranks sit behind both
    extern __shared__ __align__(16) unsigned char s_raw[];
    int *s_ctx = reinterpret_cast<int *>(s_raw + S::AREA);

    int px = blockIdx.x, py = blockIdx.y, pz = blockIdx.z;
    if (a.wg_chunks > 1) {
        const int64_t C = a.wg_chunks;
        const int64_t hkv = gridDim.y / C;
        const int64_t L = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
        const int64_t U = (int64_t)gridDim.x * hkv * gridDim.z;
        const int64_t full = U / kXcds * kXcds;
        int64_t u, cc;
        if (L < full * C) {
            const int64_t rr = L % (kXcds * C);
            cc = rr / kXcds;
            u = L / (kXcds * C) * kXcds + rr % kXcds;
        } else {
            const int64_t rem = U - full, rr = L - full * C;
            cc = rr / rem;
            u = full + rr % rem;
        }
        px = (int)(u % gridDim.x);
        const int64_t t = u / gridDim.x;
        py = (int)(t % hkv * C + cc);
        pz = (int)(t / hkv);
    }
    const int p = px;
    const int kvh = py / a.wg_chunks;
    const int chunk = py - kvh * a.wg_chunks;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const int c = wave % CH;                            // this wave's head chunk
    const int j = wave / CH;                            // its block lane

    const int gs = min(HS, a.group - chunk * HS);       // q-heads handled here
    const int hq0 = kvh * a.group + chunk * HS;         // first q-head of this workgroup
    const bool chunk_live = 16 * c < gs;                // wave-uniform

    const int lb_begin = p * a.part_blocks;
    const int lb_cap = min(lb_begin + a.part_blocks, a.max_blocks);
    const int lb_lane = lb_begin + j + lane * NB;       // this block lane's (lane)-th block
    typename F::Q qf;
    int bt_lane;
    auto load_seq = [&](int seq) {
        bt_lane = lb_lane < lb_cap ? a.block_tables[(size_t)seq * a.max_blocks + lb_lane] : 0;
        const bool hvalid = 16 * c + r < gs;
        const QElem *qrow = static_cast<const QElem *>(a.q) +
                           ((size_t)seq * a.num_q_heads + hq0 + (hvalid ? 16 * c + r : 0)) * D;
        qf.load(qrow, hvalid, g);
    };

    int b = pz;
    load_seq(b);
    float sl_h = a.scale_log2, vs_h = a.v_scale, kq_h = a.k_quant, vq_h = a.v_quant;
    bool bad_scale = false;
    if constexpr (DT == DT_FP8) {
        if (a.k_head_scales) {
            const float s = a.k_head_scales[kvh];
            bad_scale |= !scale_ok(s);
            sl_h *= s;
            kq_h = s;
        }
        if (a.v_head_scales) {
            const float s = a.v_head_scales[kvh];
            bad_scale |= !scale_ok(s);
            vs_h = s;
            vq_h = s;
        }
        if (bad_scale)
            sl_h = 1.f;       // keeps the arithmetic tame; every output is NaN anyway
        sl_h = uniform(sl_h);
        vs_h = uniform(vs_h);
        kq_h = uniform(kq_h);
        vq_h = uniform(vq_h);
    }
    int ctx = -1;
    if (a.longest_first) {
        const int nseq = gridDim.z;
        for (int t = tid; t < nseq; t += NW * kWave)
            s_ctx[t] = a.context_lens[t];
        __syncthreads();
        for (int t = tid; t < nseq; t += NW * kWave) {
            const int cx = s_ctx[t];
            int rank = 0;
            for (int u = 0; u < nseq; ++u) {
                const int cu = s_ctx[u];
                rank += (cu > cx || (cu == cx && u < t)) ? 1 : 0;
            }
            if (rank == pz)
                s_ctx[nseq] = t;
        }
        __syncthreads();
        b = __builtin_amdgcn_readfirstlane(s_ctx[nseq]);
        ctx = s_ctx[b];
        if (b != pz)
            load_seq(b);
    } else {
        ctx = a.context_lens[b];
    }
    const int nblk_seq = ctx > 0 ? (int)(((unsigned)ctx + (kBlock - 1)) / kBlock) : 0;
    const bool bad_ctx = ctx < 0 || ctx > a.max_context_len || nblk_seq > a.max_blocks;
    const int lb_end = min(lb_begin + a.part_blocks, nblk_seq);

    if (bad_ctx || lb_begin >= lb_end) {
        if (p == 0 && (bad_ctx || nblk_seq == 0)) {
            const float fill = (bad_ctx || bad_scale) ? __builtin_nanf("") : 0.f;
            for (int idx = tid; idx < gs * D; idx += NW * kWave)
                store_elem<AT>(a.out, ((size_t)b * a.num_q_heads + hq0) * D + idx, fill);
        }
        return;
    }

    // Fused append: token ctx - 1 (in logical block lb_new) arrives as a new row.  The
    // chunk-0 wave of the block lane holding that block stages the row in LDS (its table
    // register holds the block's id); every wave of that lane patches it into its
    // registers when it reaches the block, and the staging wave, in head chunk 0's
    // workgroup, writes the patched row into the pool.
    const bool fuse = FUSE && ctx >= 1;
    const int lb_new = fuse ? (ctx - 1) / kBlock : -1;
    const int off_new = fuse ? (ctx - 1) % kBlock : 0;
    const bool has_new = fuse && lb_new >= lb_begin && lb_new < lb_end;   // workgroup-uniform
    int ph_new = -1;
    __shared__ __align__(16) Elem s_newk[FUSE ? D : 16];
    __shared__ __align__(16) Elem s_newv[FUSE ? D : 16];
    if constexpr (FUSE) {
        if (has_new && wave == ((lb_new - lb_begin) % NB) * CH) {
            const QElem *kr = static_cast<const QElem *>(a.k_new) +
                              ((size_t)b * a.num_kv_heads + kvh) * D;
            const QElem *vr = static_cast<const QElem *>(a.v_new) +
                              ((size_t)b * a.num_kv_heads + kvh) * D;
            const int ph = __builtin_amdgcn_readlane(bt_lane, (lb_new - lb_begin) / NB);
            ph_new = (chunk == 0 && (unsigned)ph < (unsigned)a.num_blocks) ? ph : -1;
            for (int e = lane; e < D; e += kWave) {
                Elem sk, sv;
                if constexpr (DT == DT_FP8) {
                    sk = (Elem)e4m3_of_16(kr[e], a.act_bf16 != 0, kq_h);
                    sv = (Elem)e4m3_of_16(vr[e], a.act_bf16 != 0, vq_h);
                } else {
                    sk = kr[e];
                    sv = vr[e];
                }
                s_newk[e] = sk;
                s_newv[e] = sv;
            }
        }
    }

    const int nb = lb_end - lb_begin;                           // >= 1
    const int my_n = nb > j ? (nb - j + NB - 1) / NB : 0;       // tiles of this block lane
    const int niter = ((nb + NB - 1) / NB + TPI - 1) / TPI;     // iterations, every wave

    const Elem *kbase = static_cast<const Elem *>(a.k_pool) + (size_t)kvh * kBlock * D;
    const Elem *vbase = static_cast<const Elem *>(a.v_pool) + (size_t)kvh * kBlock * D;
    const size_t blk_stride = (size_t)a.num_kv_heads * kBlock * D;

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x4 o[D / 16];
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
        o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool tbl_bad = bad_scale;

    auto phys_of = [&](int i) -> size_t {
        int ph = __builtin_amdgcn_readlane(bt_lane, i);
        if ((unsigned)ph >= (unsigned)a.num_blocks) {   // never read outside the pool
            tbl_bad = true;
            ph = 0;
        }
        return (size_t)ph * blk_stride;
    };

    // This lane's 16-byte pieces of a tile (piece q = (i CH + c) 64 + lane): where it
    // sits in the pool's K or V tile, and where in the LDS tile.  A lane past the last
    // piece takes the last one again: it loads and stores the same bytes as its owner.
    int g_off[PPL], l_off[PPL];
    bool is_k[PPL];
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
        const int q = min((i * CH + c) * kWave + lane, S::PIECES - 1);
        if (q < S::KP) {
            const int row = q / (D * S::EB / 16), col = q % (D * S::EB / 16);
            g_off[i] = row * D * S::EB + col * 16;
            l_off[i] = row * S::KROW + col * 16;
            is_k[i] = true;
        } else {
            const int qv = q - S::KP;
            g_off[i] = qv * 16;
            l_off[i] = S::KBYTES + qv * 16;
            is_k[i] = false;
        }
    }
    // Every fetch issues the same PPL loads (a tile past the lane's last one reloads
    // that last tile, a lane without tiles reads pool block 0, neither is stored), so
    // the count of loads in flight is fixed and each wait covers exactly its slot.
    u32x4 ring[R][TPI][PPL];
    auto fetch = [&](int grp, int slot) {               // tile group grp -> ring slot
#pragma unroll
        for (int k = 0; k < TPI; ++k) {
            const size_t off = my_n > 0 ? phys_of(min(grp * TPI + k, my_n - 1)) : 0;
            const char *kb = reinterpret_cast<const char *>(kbase + off);
            const char *vb = reinterpret_cast<const char *>(vbase + off);
#pragma unroll
            for (int i = 0; i < PPL; ++i)
                ring[slot][k][i] =
                    load_kv<NT, u32x4>((is_k[i] ? kb : vb) + g_off[i]);
        }
    };
    // Stashes are unconditional too: a tile past the lane's last one lands in a buffer
    // slot that no wave reads before its next stash.
    auto stash = [&](int grp, int slot) {               // ring slot -> LDS buffer grp & 1
#pragma unroll
        for (int k = 0; k < TPI; ++k) {
            unsigned char *dst = s_raw + ((j * 2 + (grp & 1)) * TPI + k) * S::TBYTES;
#pragma unroll
            for (int i = 0; i < PPL; ++i)
                *reinterpret_cast<u32x4 *>(dst + l_off[i]) = ring[slot][k][i];
        }
    };
    auto process = [&](typename F::Tile &t, int i) {
        t.finish();
        const int lb = lb_begin + j + i * NB;
        const int valid = ctx - lb * kBlock;            // >= 1
        if constexpr (FUSE) {
            if (lb == lb_new) {                         // wave-uniform
                t.patch(s_newk, s_newv, off_new, r, g);
                if (ph_new >= 0) {                      // head chunk 0: into the pool
                    const size_t tile = ((size_t)ph_new * a.num_kv_heads + kvh) * kBlock * D;
                    t.store_row(static_cast<Elem *>(const_cast<void *>(a.k_pool)) + tile,
                                static_cast<Elem *>(const_cast<void *>(a.v_pool)) + tile,
                                off_new, r, g);
                }
            }
        }
        f32x4 s = scores<DT, AT, D>(t, qf);
        f32x4 x = s * sl_h;
        if (valid < kBlock) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                x[jj] = (4 * g + jj < valid) ? x[jj] : -INFINITY;
            mask_tail_v<DT, AT, D>(t, valid, g);
        }
        // lazy running max, as in the per-chunk kernel
        const float lmx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        if (__any(lmx - m_run > kRescaleSlack)) {
            const float m_new = fmaxf(m_run, wave_max_rows(lmx));
            const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
            for (int n = 0; n < D / 16; ++n)
                o[n] *= alpha;
            l_run *= alpha;
            m_run = m_new;
        }
        f32x4 pw;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            pw[jj] = fast_exp2(x[jj] - m_run);
        const f32x4 pu = accumulate_pv<DT, AT, D>(t, pw, o);
        l_run += (pu[0] + pu[1]) + (pu[2] + pu[3]);
    };

    // Group g (tiles g TPI .. g TPI + TPI - 1) of a block lane sits in ring slot g % R
    // from its fetch until its stash, and in LDS buffer g & 1 from its stash until the
    // barrier after it is read.  In iteration i each wave stashes group i + 1 (its share
    // of it), refills the freed slot with group i + R, reads group i from LDS and
    // computes its chunk on those tiles; the barrier at the end makes group i + 1
    // visible and frees buffer i & 1 for group i + 2.  The loop runs whole rounds of R
    // iterations with the same loads and stores in each, and no exit but its end, so
    // every wait for a ring slot covers exactly that slot's loads.
#pragma unroll
    for (int k = 0; k < R; ++k)
        fetch(k, k);
    stash(0, 0);
    __syncthreads();                                    // (and the staged new row)
    for (int i0 = 0; i0 < niter; i0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int i = i0 + u;
            stash(i + 1, (u + 1) % R);
            fetch(i + R, u);
#pragma unroll
            for (int k = 0; k < TPI; ++k) {
                const int t_idx = i * TPI + k;          // tile of this block lane
                if (t_idx < my_n && chunk_live) {       // wave-uniform
                    const unsigned char *src = s_raw + ((j * 2 + (i & 1)) * TPI + k) * S::TBYTES;
                    typename F::Tile t;
                    t.load(reinterpret_cast<const Elem *>(src),
                           reinterpret_cast<const Elem *>(src + S::KBYTES), r, g,
                           S::KROW / S::EB);
                    process(t, t_idx);
                }
            }
            __syncthreads();
        }
    }
    l_run = wave_sum_rows(l_run);

    // ---- merge the NB block lanes' (m, l, O) of each head in LDS (tile buffers free)
    float *s_m = reinterpret_cast<float *>(s_raw);      // [NB][HS]
    float *s_l = s_m + NB * HS;                          // [NB][HS]
    float *s_o = s_l + NB * HS;                          // [NB][HS][DP]
    int *s_bad = reinterpret_cast<int *>(s_o + NB * HS * DP);   // [NW]
    if (lane == 0)
        s_bad[wave] = tbl_bad ? 1 : 0;
    if (chunk_live) {
        const int hs = 16 * c + r;
        if (g == 0) {
            s_m[j * HS + hs] = m_run;
            s_l[j * HS + hs] = l_run;
        }
        if (hs < gs) {
#pragma unroll
            for (int n = 0; n < D / 16; ++n)
                *reinterpret_cast<f32x4 *>(s_o + (j * HS + hs) * DP + 16 * n + 4 * g) = o[n];
        }
    }
    __syncthreads();
    bool any_bad = false;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        any_bad |= s_bad[w] != 0;
    const bool partial = a.split && nblk_seq > a.part_blocks;
    const float qnan = __builtin_nanf("");
    for (int idx = tid; idx < gs * D; idx += NW * kWave) {
        const int h = idx / D;
        const int e = idx - h * D;
        // (a block lane without tiles left m = -inf, l = 0, O = 0: weight 0)
        float M = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < NB; ++jj)
            M = fmaxf(M, s_m[jj * HS + h]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
            const float mw = s_m[jj * HS + h];
            const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
            num += f * s_o[(jj * HS + h) * DP + e];
            den += f * s_l[jj * HS + h];
        }
        const size_t row = (size_t)b * a.num_q_heads + hq0 + h;
        if (!partial) {
            const float val = any_bad ? qnan : (den > 0.f ? num / den * vs_h : 0.f);
            store_elem<AT>(a.out, row * D + e, val);
        } else {
            const size_t slot = row * a.num_parts + p;
            a.ws_o[slot * D + e] = any_bad ? qnan : num * vs_h;
            if (e == 0) {
                a.ws_m[slot] = any_bad ? qnan : M;
                a.ws_l[slot] = any_bad ? qnan : den;
            }
        }
    }
}

// ------------------------------------------------------------------ reduce kernel

// Merges the partials of every sequence that spans more than one partition:
//   M = max_p m_p,   out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p
// (the pages' combine rule, in the log2 domain the partition kernel uses).  One
// workgroup per (sequence, kv-head, head chunk); a thread owns 4 consecutive elements
// of one q-head and walks the partials 8 at a time, issuing all 8 partitions' loads
// before using any of them.
template <int AT, int D>
__global__ __launch_bounds__(256) void pa_decode_reduce(DecodeArgs a)
{
    constexpr int QB = 8;
    const int kvh = blockIdx.x / a.head_chunks;
    const int chunk = blockIdx.x - kvh * a.head_chunks;
    const int b = blockIdx.y;
    const int gs = min(16, a.group - chunk * 16);
    const int hq0 = kvh * a.group + chunk * 16;
    const int ctx = a.context_lens[b];
    const int nblk = ctx > 0 ? (int)(((unsigned)ctx + (kBlock - 1)) / kBlock) : 0;
    const bool bad_ctx = ctx < 0 || ctx > a.max_context_len || nblk > a.max_blocks;
    if (bad_ctx || nblk <= a.part_blocks)
        return;                                  // finished by the partition kernel
    const int np = (nblk + a.part_blocks - 1) / a.part_blocks;
    const float qnan = __builtin_nanf("");

    for (int idx = threadIdx.x; idx < gs * (D / 4); idx += blockDim.x) {
        const int h = idx / (D / 4);
        const int c4 = idx - h * (D / 4);
        const size_t row = (size_t)b * a.num_q_heads + hq0 + h;
        const float *mrow = a.ws_m + row * a.num_parts;
        const float *lrow = a.ws_l + row * a.num_parts;
        const f32x4 *orow = reinterpret_cast<const f32x4 *>(a.ws_o + row * a.num_parts * D) + c4;
        float M = -INFINITY, den = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        bool nan_seen = false;
        for (int q0 = 0; q0 < np; q0 += QB) {
            float mq[QB], lq[QB];
            f32x4 oq[QB];
#pragma unroll
            for (int j = 0; j < QB; ++j) {
                const bool in = q0 + j < np;
                mq[j] = in ? mrow[q0 + j] : -INFINITY;
                lq[j] = in ? lrow[q0 + j] : 0.f;
                oq[j] = in ? orow[(size_t)(q0 + j) * (D / 4)] : f32x4{0.f, 0.f, 0.f, 0.f};
            }
            float mc = M;
#pragma unroll
            for (int j = 0; j < QB; ++j) {
                nan_seen |= (mq[j] != mq[j]);
                mc = fmaxf(mc, mq[j]);
            }
            const float sa = (M == -INFINITY) ? 0.f : fast_exp2(M - mc);
            den *= sa;
            acc *= sa;
#pragma unroll
            for (int j = 0; j < QB; ++j) {
                const float f = (mq[j] == -INFINITY) ? 0.f : fast_exp2(mq[j] - mc);
                den += f * lq[j];
                acc += f * oq[j];
            }
            M = mc;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float val = nan_seen ? qnan : (den > 0.f ? acc[j] / den : 0.f);
            store_elem<AT>(a.out, row * D + 4 * c4 + j, val);
        }
    }
}

template <int DT, int AT, int D, int CH>
hipError_t launch_shared_t(const DecodeArgs &a, int num_seqs, hipStream_t stream)
{
    using S = SharedShape<DT, D, CH>;
    const size_t lds = (size_t)S::AREA + (a.longest_first ? sizeof(int) * (num_seqs + 1) : 0);
    auto kern = a.k_new ? (a.stream_kv ? pa_decode_shared<DT, AT, D, CH, true, true>
                                       : pa_decode_shared<DT, AT, D, CH, true, false>)
                        : (a.stream_kv ? pa_decode_shared<DT, AT, D, CH, false, true>
                                       : pa_decode_shared<DT, AT, D, CH, false, false>);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    dim3 grid(a.num_parts, a.num_kv_heads * a.wg_chunks, num_seqs);
    hipLaunchKernelGGL(kern, grid, dim3(kSharedWaves * kWave), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.split)
        return e;
    dim3 rgrid(a.num_kv_heads * a.head_chunks, num_seqs);
    hipLaunchKernelGGL((pa_decode_reduce<AT, D>), rgrid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int DT, int AT, int D, int CB>
hipError_t launch_partition_t(const DecodeArgs &a, int num_seqs, hipStream_t stream)
{
    constexpr int NW = waves_per_group(D);
    // Blocks in flight per wave.  With ordinary loads fp8 tiles (half the bytes) keep
    // the 16-bit tiles' bytes in flight with a deeper ring; with non-temporal loads the
    // 2-tile ring is fastest for them too (4 tiles measured 3-6 % slower).
    constexpr int PF = (D > 128 || DT == DT_F32) ? 1 : kPrefetchMain;
    constexpr int PF_PLAIN = DT == DT_FP8 && D <= 128 ? 2 * kPrefetchMain + 1 : PF;
    constexpr int HS = 16 * CB;
    const int gs_max = min(HS, a.group);
    const size_t lds = sizeof(float) * (2 * NW * HS + 16 + (size_t)NW * gs_max * (D + 4)) +
                       (a.longest_first ? sizeof(int) * (num_seqs + 1) : 0);
    // fp32 tiles stream with ordinary loads (the hint measured slower for them)
    constexpr bool kNt = DT != DT_F32;
    const bool nt = kNt && a.stream_kv;
    auto kern = a.k_new ? (nt ? pa_decode_partition<DT, AT, D, NW, PF, true, kNt, CB>
                              : pa_decode_partition<DT, AT, D, NW, PF_PLAIN, true, false, CB>)
                        : (nt ? pa_decode_partition<DT, AT, D, NW, PF, false, kNt, CB>
                              : pa_decode_partition<DT, AT, D, NW, PF_PLAIN, false, false, CB>);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    dim3 grid(a.num_parts, a.num_kv_heads * a.wg_chunks, num_seqs);
    hipLaunchKernelGGL(kern, grid, dim3(NW * kWave), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.split)
        return e;
    dim3 rgrid(a.num_kv_heads * a.head_chunks, num_seqs);
    hipLaunchKernelGGL((pa_decode_reduce<AT, D>), rgrid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int DT, int AT, int D>
hipError_t launch_decode_t(const DecodeArgs &a, int num_seqs, hipStream_t stream)
{
    // the host sized the grid and the partitions for decode_chunks(D, group) chunks per
    // workgroup; the launch must hold exactly that many
    const int ch = decode_chunks(DT, D, a.group);
    if (a.wg_heads != 16 * ch)
        return hipErrorInvalidValue;
    if constexpr (D <= 128 && (DT == DT_F16 || DT == DT_BF16)) {
        if (decode_shared(DT, D, a.group)) {
            if (ch == 4)
                return launch_shared_t<DT, AT, D, 4>(a, num_seqs, stream);
            if (ch == 2)
                return launch_shared_t<DT, AT, D, 2>(a, num_seqs, stream);
            return hipErrorInvalidValue;
        }
    }
    if constexpr (D <= 128 && DT != DT_F32) {
        if (ch == 2)
            return launch_partition_t<DT, AT, D, 2>(a, num_seqs, stream);
    }
    if (ch != 1)
        return hipErrorInvalidValue;
    return launch_partition_t<DT, AT, D, 1>(a, num_seqs, stream);
}

}  // namespace

hipError_t launch_decode(int dtype, int act_dtype, int head_dim, const DecodeArgs &a,
                         int num_seqs, hipStream_t stream)
{
#define PA_CASE(DT, AT, D)                                                                \
    if (dtype == DT && act_dtype == AT && head_dim == D)                                  \
        return launch_decode_t<DT, AT, D>(a, num_seqs, stream);
    PA_CASE(DT_F32, DT_F32, 64)
    PA_CASE(DT_F32, DT_F32, 128)
    PA_CASE(DT_F16, DT_F16, 64)
    PA_CASE(DT_F16, DT_F16, 128)
    PA_CASE(DT_F16, DT_F16, 256)
    PA_CASE(DT_BF16, DT_BF16, 64)
    PA_CASE(DT_BF16, DT_BF16, 128)
    PA_CASE(DT_BF16, DT_BF16, 256)
    PA_CASE(DT_FP8, DT_F16, 64)
    PA_CASE(DT_FP8, DT_F16, 128)
    PA_CASE(DT_FP8, DT_F16, 256)
    PA_CASE(DT_FP8, DT_BF16, 64)
    PA_CASE(DT_FP8, DT_BF16, 128)
    PA_CASE(DT_FP8, DT_BF16, 256)
#undef PA_CASE
    return hipErrorInvalidValue;
}

}  // namespace pa
