// pa_prefill.hip -- paged prefill (chunked prefill) attention for CDNA4 (gfx950).
//
// What is computed: the query rows of a prompt chunk attend to the paged cache through
// the same block tables as decode.  Sequence b's chunk is rows query_start[b] ..
// query_start[b+1]-1 of q; the chunk's K/V rows were appended first, so its i-th query
// is token ctx - q_len + i and attends, causally, to tokens 0 .. ctx - q_len + i.
// Sources: LLM-101-CN "推理优化", section "Chunked Prefill" (the chunk's queries over
// the earlier chunks' cache joined with the chunk's own K/V, 1/sqrt(d_h) softmax; the
// mixed prefill/decode batch with per-request chunk lengths); "Deep dive into vLLM 06",
// section 4.2 (one forward yields every position from its own prefix: the causal rule);
// the block layout, online softmax and GQA sources are those of the decode kernel.
//
// Work decomposition
//   One workgroup of NW waves owns one (sequence, kv-head, query tile).  Its R =
//   NW * C * 16 rows are (position, q-head of the group) pairs, position-major, so
//   every q-head of a GQA group shares one stream of K/V.  Wave w owns rows
//   [16 C w, 16 C (w + 1)) as C MFMA column blocks.
//   Keys are walked 32 at a time (two pool blocks).  The workgroup stages each step's
//   K and V in LDS, double-buffered, in MFMA fragment order, so every wave's operand
//   read is one conflict-free 16-byte LDS load per lane:
//     S^T[t][row]  = sum_e K[t][e] Q[row][e]        16x16x32, A = K rows, B = Q rows
//     O^T[e][row] += sum_t V^T[e][t] P[t][row]       16x16x32, A = V^T, B = P
//   S^T's accumulator layout (lane: row lane % 16, tokens 4 (lane / 16) .. +3 of each
//   16-token block) is the PV B operand once the 32 keys are ordered as
//   k = 8 g + j -> block j / 4, token 4 g + j % 4; the V^T fragments use the same order.
//   The softmax normaliser is a third product, ones[16][32] . P: it sums exactly the
//   16-bit weights the PV product used, lands already reduced over the wave's four
//   row groups, and keeps that work off the vector ALU, which the exponentials load.
//   Workgroup ids go round-robin over the 8 XCDs; the id -> (pair, tile) map keeps all
//   query tiles of one (sequence, kv-head) on one XCD, so they share its L2.  Batches
//   of up to 256 sequences are taken in order of estimated tile cost (longest first),
//   and where tiles can be partial the grid enumerates only the tiles that exist.
//   A tile whose rows fit one column block (a decode row, a chunk's last position or
//   two) is split over the waves by keys instead of rows: each wave streams its share
//   straight into registers and the partial (m, l, O) sets are merged in LDS.
#include <limits.h>
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "pa_common.h"
#include "pa_prefill.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;                 // MI355X: workgroups go round-robin over 8 XCDs

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float max_over_row_groups(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// Largest of a step's 8 scores in this lane.  IEEE maximum needs no canonicalising of
// the MFMA results (it maps onto three-input v_maximum3); the scores are never NaN
// (finite, or -inf once masked).
__device__ __forceinline__ float max8(const f32x4 (&x)[2])
{
    const float a = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0][0], x[0][1]),
                                                  x[0][2]);
    const float b = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0][3], x[1][0]),
                                                  x[1][1]);
    const float c = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[1][2], x[1][3]), a);
    return __builtin_elementwise_maximum(b, c);
}

template <int AT>
__device__ __forceinline__ f32x4 mma32(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (AT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Eight fp32 weights -> eight 16-bit values (RNE), packed as one MFMA operand.
template <int AT>
__device__ __forceinline__ u32x4 pack8(f32x4 lo, f32x4 hi)
{
    u32x2 a, b;
    if constexpr (AT == DT_BF16) {
        a = __builtin_bit_cast(u32x2, __builtin_convertvector(lo, bf16x4));
        b = __builtin_bit_cast(u32x2, __builtin_convertvector(hi, bf16x4));
    } else {
        a = __builtin_bit_cast(u32x2, __builtin_convertvector(lo, f16x4));
        b = __builtin_bit_cast(u32x2, __builtin_convertvector(hi, f16x4));
    }
    return u32x4{a[0], a[1], b[0], b[1]};
}

// The 16-bit pattern of 1.0, twice.
template <int AT>
constexpr uint32_t one_pair() { return AT == DT_BF16 ? 0x3F803F80u : 0x3C003C00u; }

// Two E4M3 codes (low or high half of w) -> two 16-bit values of type AT (exact).
template <int AT, bool HIGH>
__device__ __forceinline__ uint32_t fp8x2_to_16(uint32_t w)
{
    if constexpr (AT == DT_BF16)
        return __builtin_bit_cast(uint32_t,
                                  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HIGH));
    else
        return __builtin_bit_cast(uint32_t,
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HIGH));
}

// Keep the 16-bit elements of an 8-token V^T piece (tokens t0 .. t0+7) below `valid`.
__device__ __forceinline__ u32x4 keep_tokens16(u32x4 v, int t0, int valid)
{
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t m = (t0 + 2 * w < valid ? 0x0000FFFFu : 0u) |
                           (t0 + 2 * w + 1 < valid ? 0xFFFF0000u : 0u);
        v[w] &= m;
    }
    return v;
}

// The same for 16 fp8 codes (tokens t0 .. t0+15).
__device__ __forceinline__ u32x4 keep_tokens8(u32x4 v, int t0, int valid)
{
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            m |= (t0 + 4 * w + j < valid) ? (0xFFu << (8 * j)) : 0u;
        v[w] &= m;
    }
    return v;
}

// One row's partial result of a key split, for the reduce kernel: the unnormalised
// output (this lane's four elements of each 16-element block, times the V scale), the
// reference max it is relative to (log2 domain; -inf when the split saw no key) and the
// normaliser.  A workgroup with bad input writes NaN, which the merge propagates.
template <int NDB>
__device__ __forceinline__ void store_partial(const PrefillArgs &a, int orow, int split,
                                              int nsplit, const f32x4 (&o)[NDB], float m_raw,
                                              float sl, float l, float vs, bool bad, int g)
{
    constexpr int D = NDB * 16;
    const float qnan = __builtin_nanf("");
    const size_t slot = (size_t)orow * nsplit + split;
#pragma unroll
    for (int n = 0; n < NDB; ++n) {
        const f32x4 v = bad ? f32x4{qnan, qnan, qnan, qnan} : o[n] * vs;
        *reinterpret_cast<f32x4 *>(a.ws_o + slot * D + 16 * n + 4 * g) = v;
    }
    if (g == 0) {
        a.ws_m[slot] = bad ? qnan : (m_raw == -INFINITY ? -INFINITY : m_raw * sl);
        a.ws_l[slot] = bad ? qnan : l;
    }
}

template <int DT, int AT, int D, int NW, int C, bool IDLE, bool SMALLQ, bool SPLIT>
__global__ __launch_bounds__(NW *kWave, C * D <= 256 ? 2 : 1) void pa_prefill_kernel(PrefillArgs a)
{
    using Elem = typename std::conditional<DT == DT_FP8, uint8_t, uint16_t>::type;
    constexpr int NT = NW * kWave;
    constexpr int NKC = D / 32;              // QK MFMAs per 16-token block
    constexpr int NDB = D / 16;              // 16-row blocks of O^T
    constexpr int KSLOTS = 2 * NKC * kWave;  // one step's K fragments (16 bytes each)
    constexpr int VSLOTS = NDB * kWave;      // one step's V^T fragments
    // 16-byte global pieces per step: 16-bit K rows hold 8 elements per piece, fp8 16.
    constexpr int EPP = DT == DT_FP8 ? 16 : 8;
    constexpr int KCH = 2 * kBlock * (D / EPP);
    constexpr int VCH = 2 * D * (kBlock / EPP);
    constexpr int KPT = (KCH + NT - 1) / NT;
    constexpr int VPT = (VCH + NT - 1) / NT;

    __shared__ u32x4 s_k[2][KSLOTS];
    __shared__ u32x4 s_v[2][VSLOTS];

    // ---- which (sequence, kv-head, query tile).  Workgroup ids go round-robin over
    // the XCDs; XCD x takes the (sequence, kv-head) pairs p with p % 8 == x, pair p
    // being kv-head p % Hkv of the (p / Hkv)-th sequence, so all query tiles of a pair
    // share that XCD's L2.  A pair's tiles run last tile (most keys) first.
    const int id = blockIdx.x;
    const int xcd = id % kXcds;
    const int k_x = id / kXcds;                  // this workgroup's rank on its XCD
    int b, kvh, qt;
    if (a.longest_first) {
        // Sequences are taken in order of estimated tile cost, highest first (ties by
        // index), so the tiles that walk the most keys start first instead of behind
        // a batch of short ones.  The estimate is the key count of a sequence's last
        // tile (its whole context), halved for tiles whose keys are split over the
        // waves (measured to take about half as long as a full tile over the same
        // keys).  In the launch that allows partial tiles, the grid is also compact:
        // XCD x's work items are its pairs' tiles in that order, found by a prefix
        // sum over the ranked sequences, so no workgroup is spent on a tile past a
        // short chunk's end.  The scratch sits in the K staging buffer, free until
        // the first staging.
        __shared__ int s_pick[3];
        int *s_cost = reinterpret_cast<int *>(&s_k[0][0]);   // [kLongestFirstMax] each
        int *s_ntl = s_cost + kLongestFirstMax;
        int *s_seq = s_ntl + kLongestFirstMax;
        const int nseq = a.num_seqs;                 // <= kLongestFirstMax (host-checked)
        const int tid0 = threadIdx.x;
        if (tid0 < nseq) {
            const int q0t = a.query_start[tid0];
            const int qlt = a.query_start[tid0 + 1] - q0t;
            const int cx = a.context_lens[tid0];
            const bool valid = q0t >= 0 && qlt >= 0 && qlt <= a.max_query_len &&
                               q0t <= a.num_tokens - qlt;
            int cost = valid && qlt > 0 && cx > 0 ? cx : 0;
            if (IDLE && D <= 128 && qlt * a.group <= (SMALLQ ? 32 : 16))
                cost /= 2;
            s_cost[tid0] = cost;
            s_ntl[tid0] = valid ? (qlt + a.q_tile - 1) / a.q_tile : 0;
        }
        __syncthreads();
        // the plain map's pair, for the full-tile launch (every sequence has the same
        // tile count there)
        const int pair = (k_x / a.num_qtiles) * kXcds + xcd;
        if (tid0 < nseq) {
            const int c = s_cost[tid0];
            int rank = 0;
            for (int u = 0; u < nseq; ++u) {
                const int cu = s_cost[u];
                rank += (cu > c || (cu == c && u < tid0)) ? 1 : 0;
            }
            s_seq[rank] = tid0;
            if (!IDLE && rank == pair / a.num_kv_heads)
                s_pick[0] = tid0;
        }
        __syncthreads();
        if constexpr (IDLE) {
            // rank r's pairs on this XCD: kv-heads h0, h0 + 8, ... below Hkv, with
            // h0 = (x - r Hkv) mod 8; each has the sequence's tile count.  An
            // inclusive prefix over ranks (ranks are thread ids, four waves at most).
            const int hkv = a.num_kv_heads;
            int cnt = 0, h0 = 0, ntl = 0;
            if (tid0 < nseq) {
                h0 = ((xcd - (int)(((int64_t)tid0 * hkv) % kXcds)) % kXcds + kXcds) % kXcds;
                ntl = s_ntl[s_seq[tid0]];
                cnt = h0 < hkv ? ((hkv - 1 - h0) / kXcds + 1) * ntl : 0;
            }
            int incl = cnt;
#pragma unroll
            for (int o = 1; o < kWave; o *= 2) {
                const int v = __shfl_up(incl, o);
                if ((tid0 & (kWave - 1)) >= o)
                    incl += v;
            }
            int *s_wsum = s_seq + kLongestFirstMax;          // [NW]
            if ((tid0 & (kWave - 1)) == kWave - 1)
                s_wsum[tid0 / kWave] = incl;
            __syncthreads();
            for (int w = 0; w < tid0 / kWave; ++w)
                incl += s_wsum[w];
            const int excl = incl - cnt;
            if (tid0 < nseq && excl <= k_x && k_x < incl) {
                const int off = k_x - excl;
                s_pick[0] = s_seq[tid0];
                s_pick[1] = h0 + kXcds * (off / ntl);
                s_pick[2] = ntl - 1 - off % ntl;
            }
            if (tid0 == nseq - 1 && k_x >= incl)
                s_pick[0] = -1;                      // past this XCD's last item
            __syncthreads();
            b = __builtin_amdgcn_readfirstlane(s_pick[0]);
            if (b < 0)
                return;
            kvh = __builtin_amdgcn_readfirstlane(s_pick[1]);
            qt = __builtin_amdgcn_readfirstlane(s_pick[2]);
        } else {
            if (pair >= a.num_seqs * a.num_kv_heads)
                return;
            qt = a.num_qtiles - 1 - k_x % a.num_qtiles;
            kvh = pair % a.num_kv_heads;
            b = __builtin_amdgcn_readfirstlane(s_pick[0]);
        }
    } else {
        const int pair = (k_x / a.num_qtiles) * kXcds + xcd;
        if (pair >= a.num_seqs * a.num_kv_heads)
            return;
        qt = a.num_qtiles - 1 - k_x % a.num_qtiles;
        kvh = pair % a.num_kv_heads;
        b = pair / a.num_kv_heads;
    }
    const int q0 = a.query_start[b];
    const int q_len = a.query_start[b + 1] - q0;
    // A malformed query range has no rows that can be written safely.
    if (q0 < 0 || q_len < 0 || q_len > a.max_query_len || q0 > a.num_tokens - q_len)
        return;
    const int p_lo = qt * a.q_tile;
    if (p_lo >= q_len)
        return;
    const int ctx = a.context_lens[b];
    const bool bad_ctx = ctx < 0 || ctx > a.max_context_len ||
                         (int)(((unsigned)ctx + (kBlock - 1)) / kBlock) > a.max_blocks;
    const int n_here = min(a.q_tile, q_len - p_lo);      // query positions in this tile
    const int first = ctx - q_len + p_lo;                // position of the tile's first
    const int key_end = bad_ctx ? 0 : max(0, first + n_here);   // keys [0, key_end)
    const int nsteps = (key_end + 31) / 32;
    // This workgroup's share of the tile's 32-key steps: all of them, or, in the
    // instance for launches that split keys (SPLIT, gridDim.y splits: a grid too small
    // to fill the chip), the split-th of gridDim.y contiguous ranges, whose partial
    // (m, l, O) the reduce kernel merges with the max/normaliser rule.  Ranges start
    // on even steps, so every range but the tile's last holds whole pairs of steps and
    // the staged loop, which runs pairs, never computes a step outside its range; the
    // last range's padding step lies past every row's position, as without a split.
    const int nsplit = SPLIT ? (int)gridDim.y : 1;
    const int split = SPLIT ? (int)blockIdx.y : 0;
    const int npair_all = (nsteps + 1) / 2;
    const int s_begin = SPLIT ? 2 * (int)(((int64_t)npair_all * split) / nsplit) : 0;
    const int s_end =
        SPLIT ? min(nsteps, 2 * (int)(((int64_t)npair_all * (split + 1)) / nsplit)) : nsteps;

    // This kv-head's scales: fp8 pools with per-head arrays read them here (a bad one
    // poisons the head's rows); otherwise the pool's, folded in on the host.
    float sl_h = a.scale_log2, vs_h = a.v_scale;
    bool bad_scale = false;
    if constexpr (DT == DT_FP8) {
        if (a.k_head_scales) {
            const float s = a.k_head_scales[kvh];
            bad_scale |= !scale_ok(s);
            sl_h *= s;
        }
        if (a.v_head_scales) {
            const float s = a.v_head_scales[kvh];
            bad_scale |= !scale_ok(s);
            vs_h = s;
        }
        if (bad_scale)
            sl_h = 1.f;       // keeps the arithmetic tame; every row is NaN anyway
        // workgroup-uniform: kept in scalar registers, as kernel arguments are
        sl_h = uniform(sl_h);
        vs_h = uniform(vs_h);
    }

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15;
    const int g = lane >> 4;

    // ---- this lane's rows: q fragments, positions, output offsets
    const uint16_t *qp = static_cast<const uint16_t *>(a.q);
    u32x4 qf[C][NKC];
    int pos[C];
    int orow[C];                             // q-row * Hq + head, or -1 for an idle row
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int row = (wave * C + c) * 16 + r16;
        const int lp = row / a.group;
        const int hh = row - lp * a.group;
        const bool ok = lp < n_here;
        orow[c] = ok ? (q0 + p_lo + lp) * a.num_q_heads + kvh * a.group + hh : -1;
        pos[c] = ok ? first + lp : INT_MIN / 2;
        const uint16_t *qrow = qp + (size_t)(ok ? orow[c] : 0) * D;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
            qf[c][kc] = ok ? *reinterpret_cast<const u32x4 *>(qrow + 32 * kc + 8 * g)
                           : u32x4{0u, 0u, 0u, 0u};
    }

    const Elem *kbase = static_cast<const Elem *>(a.k_pool) + (size_t)kvh * kBlock * D;
    const Elem *vbase = static_cast<const Elem *>(a.v_pool) + (size_t)kvh * kBlock * D;
    const size_t blk_stride = (size_t)a.num_kv_heads * kBlock * D;
    const uint32_t blk_stride32 = (uint32_t)blk_stride;     // < 2^32 (host-checked)
    // the table row through the constant address space: uniform reads of it stay
    // scalar loads, whose wait does not hold up the vector loads in flight
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    const_i32 *trow = (const_i32 *)(a.block_tables + (size_t)b * a.max_blocks);
    bool bad = bad_scale;

    // ---- block ids of step s (blocks 2s, 2s+1), read one step before their loads are
    // issued and checked only then, so the scalar loads' latency is hidden.  Entries
    // past key_end may be padding and are never used: such a block, and an id outside
    // the pool, use block 0, whose rows stay in bounds and are zeroed or flagged below.
    auto table = [&](int s, int (&raw)[2]) {
#pragma unroll
        for (int tl = 0; tl < 2; ++tl)
            raw[tl] = trow[min(2 * s + tl, a.max_blocks - 1)];
    };
    auto resolve = [&](int s, const int (&raw)[2], int (&ph)[2]) {
#pragma unroll
        for (int tl = 0; tl < 2; ++tl) {
            const bool need = (2 * s + tl) * kBlock < key_end;
            const bool in_pool = (unsigned)raw[tl] < (unsigned)a.num_blocks;
            bad |= need && !in_pool;                  // never read outside the pool
            ph[tl] = (need && in_pool) ? raw[tl] : 0;
        }
    };

    // ---- a tile whose rows all fit one or two MFMA column blocks (a decode row, a
    // chunk's last few positions): with the usual split, one wave would own every row
    // and the other waves would only stage its keys.  Instead every wave takes those
    // same rows and a contiguous 1/NW of the key steps, loads its K and V fragments
    // straight from the pool into registers (no LDS staging, two steps in flight),
    // and the NW partial (max, sum, O) sets are merged through LDS at the end with the
    // same rescaling rule as the online softmax.  Only in the launch that allows
    // partial tiles, at d <= 128.
    if constexpr (IDLE && D <= 128) {
        const int tile_rows = n_here * a.group;
        if (tile_rows <= 16 || (SMALLQ && tile_rows <= 32)) {
            // Key order inside a 32-key step: QK product t's output row 4 gr + j is
            // key 16 (gr / 2) + 8 (gr % 2) + 4 t + j, so lane group g of the weights
            // holds keys 16 (g / 2) + 8 (g % 2) + 0 .. 7: eight consecutive tokens of
            // one block.  The V^T operand is then one piece per row block (16 bytes,
            // 8 for fp8) and K one 16-byte piece per product (fp8: per two products,
            // whose e ranges are interleaved so a lane's 16 codes are contiguous, q
            // following the same e order): 16 load instructions per step (fp8: 12)
            // instead of 24, which sets how fast one CU streams a long row.
            constexpr int KL = DT == DT_FP8 ? NKC / 2 : NKC;      // K pieces per product row
            using VRaw = typename std::conditional<DT == DT_FP8, u32x2, u32x4>::type;
            struct Frag {
                u32x4 k[KL][2];
                VRaw v[NDB];
            };
            const float sl = sl_h;
            const float grow_thr = fminf(kRescaleSlack / sl, 3.0e38f);
            const u32x4 ones = {one_pair<AT>(), one_pair<AT>(), one_pair<AT>(), one_pair<AT>()};
            const int s_lo = s_begin + (int)(((int64_t)(s_end - s_begin) * wave) / NW);
            const int s_hi = s_begin + (int)(((int64_t)(s_end - s_begin) * (wave + 1)) / NW);
            // this lane's K row (product row r16) and V^T piece, inside a step
            const int k_blk = r16 >> 3;                                    // 0 or 1
            const int k_tok0 = 8 * ((r16 >> 2) & 1) + (r16 & 3);          // + 4 t
            const int v_blk = g >> 1;
            const int v_tok0 = 8 * (g & 1);

            // The wave's block ids, one per lane, for logical blocks ids_base ..
            // ids_base + 63 (32 steps), read with one vector load and picked out with
            // readlane.  Scalar loads of the table would not do here: using any scalar
            // load's result waits for every scalar load in flight, so a step could not
            // start before the table read issued for a later one had come back.
            const int32_t *trow_v = a.block_tables + (size_t)b * a.max_blocks;
            int ids_base = 0, ids = 0;                   // set at the start of each run
            auto load_step = [&](int s, Frag &fr) {
                if (2 * s + 1 >= ids_base + kWave) {              // wave-uniform, rare
                    ids_base = 2 * s;
                    ids = trow_v[min(ids_base + lane, a.max_blocks - 1)];
                }
                int raw[2], ph[2];
                raw[0] = __builtin_amdgcn_readlane(ids, 2 * s - ids_base);
                raw[1] = __builtin_amdgcn_readlane(ids, 2 * s + 1 - ids_base);
                resolve(s, raw, ph);
                const size_t kblk = (uint64_t)(uint32_t)(k_blk ? ph[1] : ph[0]) * blk_stride32;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const Elem *kp = kbase + kblk + (size_t)(k_tok0 + 4 * t) * D;
#pragma unroll
                    for (int i = 0; i < KL; ++i)
                        fr.k[i][t] = *reinterpret_cast<const u32x4 *>(
                            kp + (DT == DT_FP8 ? 64 * i + 16 * g : 32 * i + 8 * g));
                }
                const size_t vblk = (uint64_t)(uint32_t)(v_blk ? ph[1] : ph[0]) * blk_stride32;
                const Elem *vp = vbase + vblk + r16 * kBlock + v_tok0;
#pragma unroll
                for (int n = 0; n < NDB; ++n)
                    fr.v[n] = *reinterpret_cast<const VRaw *>(vp + 16 * kBlock * n);
            };

            __shared__ float s_m[2][NW][16];
            __shared__ float s_l[2][NW][16];

            // CS column blocks (tile rows row0 + 16 c + r16), PF steps in flight
            auto run = [&](auto cs_tag, auto pf_tag, int row0) {
                constexpr int CS = decltype(cs_tag)::value;
                constexpr int PF = decltype(pf_tag)::value;
                ids_base = 2 * s_lo;
                ids = trow_v[min(ids_base + lane, a.max_blocks - 1)];
                int orow1[CS], pos1[CS];
                // q fragment of product kc: e = 32 kc + 8 g .. +7 (16-bit pools), or
                // 64 (kc / 2) + 16 g + 8 (kc % 2) .. +7 (fp8 pools)
                u32x4 q1[CS][NKC];
#pragma unroll
                for (int c = 0; c < CS; ++c) {
                    const int row = row0 + 16 * c + r16;
                    const int lp = row / a.group;
                    const int hh = row - lp * a.group;
                    const bool ok = lp < n_here;
                    orow1[c] = ok ? (q0 + p_lo + lp) * a.num_q_heads + kvh * a.group + hh : -1;
                    pos1[c] = ok ? first + lp : INT_MIN / 2;
                    const uint16_t *qrow = qp + (size_t)(ok ? orow1[c] : 0) * D;
#pragma unroll
                    for (int kc = 0; kc < NKC; ++kc) {
                        const int e0 = DT == DT_FP8 ? 64 * (kc / 2) + 16 * g + 8 * (kc % 2)
                                                    : 32 * kc + 8 * g;
                        q1[c][kc] = ok ? *reinterpret_cast<const u32x4 *>(qrow + e0)
                                       : u32x4{0u, 0u, 0u, 0u};
                    }
                }
                f32x4 o1[CS][NDB], l1[CS];
                float m1[CS], mneg1[CS];
#pragma unroll
                for (int c = 0; c < CS; ++c) {
#pragma unroll
                    for (int n = 0; n < NDB; ++n)
                        o1[c][n] = f32x4{0.f, 0.f, 0.f, 0.f};
                    l1[c] = f32x4{0.f, 0.f, 0.f, 0.f};
                    m1[c] = -INFINITY;
                    mneg1[c] = 0.f;
                }

                auto step = [&](int s, const Frag &fr) {
                    f32x4 sc[CS][2];
#pragma unroll
                    for (int c = 0; c < CS; ++c)
                        sc[c][0] = sc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < KL; ++i)
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            const u32x4 w = fr.k[i][t];
                            if constexpr (DT == DT_FP8) {
                                const u32x4 lo = {fp8x2_to_16<AT, false>(w[0]), fp8x2_to_16<AT, true>(w[0]),
                                                  fp8x2_to_16<AT, false>(w[1]), fp8x2_to_16<AT, true>(w[1])};
                                const u32x4 hi = {fp8x2_to_16<AT, false>(w[2]), fp8x2_to_16<AT, true>(w[2]),
                                                  fp8x2_to_16<AT, false>(w[3]), fp8x2_to_16<AT, true>(w[3])};
#pragma unroll
                                for (int c = 0; c < CS; ++c) {
                                    sc[c][t] = mma32<AT>(lo, q1[c][2 * i], sc[c][t]);
                                    sc[c][t] = mma32<AT>(hi, q1[c][2 * i + 1], sc[c][t]);
                                }
                            } else {
#pragma unroll
                                for (int c = 0; c < CS; ++c)
                                    sc[c][t] = mma32<AT>(w, q1[c][i], sc[c][t]);
                            }
                        }
                    // score (t, j) of lane group g is key 32 s + 16 (g / 2) + 8 (g % 2) + 4 t + j
                    if (32 * s + 31 > first) {
#pragma unroll
                        for (int c = 0; c < CS; ++c)
#pragma unroll
                            for (int t = 0; t < 2; ++t)
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    sc[c][t][j] = (32 * s + 16 * v_blk + v_tok0 + 4 * t + j <= pos1[c])
                                                      ? sc[c][t][j] : -INFINITY;
                    }
                    float lmx[CS];
                    bool grow = false;
#pragma unroll
                    for (int c = 0; c < CS; ++c) {
                        lmx[c] = max8(sc[c]);
                        grow |= lmx[c] - m1[c] > grow_thr;
                    }
                    if (__any(grow)) {
#pragma unroll
                        for (int c = 0; c < CS; ++c) {
                            const float m_new = fmaxf(m1[c], max_over_row_groups(lmx[c]));
                            const float alpha =
                                (m_new == -INFINITY) ? 1.f : exp2_fast((m1[c] - m_new) * sl);
#pragma unroll
                            for (int n = 0; n < NDB; ++n)
                                o1[c][n] *= alpha;
                            l1[c] *= alpha;
                            m1[c] = m_new;
                            mneg1[c] = (m_new == -INFINITY) ? 0.f : -m_new * sl;
                        }
                    }
                    u32x4 pb[CS];                       // weights of keys v_tok0 + 0 .. 7
#pragma unroll
                    for (int c = 0; c < CS; ++c) {
                        f32x4 p0, p1;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            p0[j] = exp2_fast(fmaf(sc[c][0][j], sl, mneg1[c]));
                            p1[j] = exp2_fast(fmaf(sc[c][1][j], sl, mneg1[c]));
                        }
                        pb[c] = pack8<AT>(p0, p1);
                    }
                    // V^T tokens past the context, and whole blocks past key_end (padding
                    // entries read as block 0), may hold anything: zero them.  Only a
                    // step that reaches past key_end (<= ctx) has such tokens.
                    VRaw keep;
                    if constexpr (DT == DT_FP8)
                        keep = VRaw{~0u, ~0u};
                    else
                        keep = VRaw{~0u, ~0u, ~0u, ~0u};
                    if (32 * s + 32 > key_end) {                        // wave-uniform
                        const int blk0 = (2 * s + v_blk) * kBlock;
                        const int valid = blk0 >= key_end ? 0 : ctx - blk0;
                        if constexpr (DT == DT_FP8) {
#pragma unroll
                            for (int w = 0; w < 2; ++w) {
                                uint32_t m = 0;
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    m |= (v_tok0 + 4 * w + j < valid) ? (0xFFu << (8 * j)) : 0u;
                                keep[w] = m;
                            }
                        } else {
#pragma unroll
                            for (int w = 0; w < 4; ++w)
                                keep[w] = (v_tok0 + 2 * w < valid ? 0x0000FFFFu : 0u) |
                                          (v_tok0 + 2 * w + 1 < valid ? 0xFFFF0000u : 0u);
                        }
                    }
#pragma unroll
                    for (int n = 0; n < NDB; ++n) {
                        u32x4 vf;
                        if constexpr (DT == DT_FP8) {
                            const uint32_t w0 = fr.v[n][0] & keep[0];
                            const uint32_t w1 = fr.v[n][1] & keep[1];
                            vf = u32x4{fp8x2_to_16<AT, false>(w0), fp8x2_to_16<AT, true>(w0),
                                       fp8x2_to_16<AT, false>(w1), fp8x2_to_16<AT, true>(w1)};
                        } else {
                            vf = fr.v[n] & keep;
                        }
#pragma unroll
                        for (int c = 0; c < CS; ++c)
                            o1[c][n] = mma32<AT>(vf, pb[c], o1[c][n]);
                    }
#pragma unroll
                    for (int c = 0; c < CS; ++c)
                        l1[c] = mma32<AT>(ones, pb[c], l1[c]);
                };

                // PF = 2: the loads of the step after next are issued before a step's
                // products, and the last step's loads are repeated past the end so every
                // pass issues the same loads; PF = 1: each step's loads, then its products
                if (s_lo < s_hi) {
                    if constexpr (PF == 2) {
                        Frag fa, fb;
                        load_step(s_lo, fa);
                        for (int s = s_lo; s < s_hi; s += 2) {
                            load_step(min(s + 1, s_hi - 1), fb);
                            step(s, fa);
                            load_step(min(s + 2, s_hi - 1), fa);
                            if (s + 1 < s_hi)
                                step(s + 1, fb);
                        }
                    } else {
                        Frag fa;
                        for (int s = s_lo; s < s_hi; ++s) {
                            load_step(s, fa);
                            step(s, fa);
                        }
                    }
                }

                // ---- merge: each row's reference max over the waves, every wave's O
                // and l rescaled to it, then summed (a tree over four LDS slots: the
                // staging buffers, idle here, each hold one column block of one wave's
                // O^T fragments exactly)
                if (g == 0) {
#pragma unroll
                    for (int c = 0; c < CS; ++c)
                        s_m[c][wave][r16] = m1[c];
                }
                const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0 || bad_ctx;
#pragma unroll
                for (int c = 0; c < CS; ++c) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int w = 0; w < NW; ++w)
                        mx = fmaxf(mx, s_m[c][w][r16]);
                    const float f = (m1[c] == -INFINITY) ? 0.f : exp2_fast((m1[c] - mx) * sl);
#pragma unroll
                    for (int n = 0; n < NDB; ++n)
                        o1[c][n] *= f;
                    if (g == 0)
                        s_l[c][wave][r16] = l1[c][0] * f;
                }
#pragma unroll
                for (int c = 0; c < CS; ++c) {
#pragma unroll
                    for (int half = NW / 2; half >= 1; half /= 2) {
                        if (wave >= half && wave < 2 * half) {
                            const int k = wave - half;
                            u32x4 *slot = k < 2 ? s_k[k] : s_v[k - 2];
#pragma unroll
                            for (int n = 0; n < NDB; ++n)
                                slot[n * kWave + lane] = __builtin_bit_cast(u32x4, o1[c][n]);
                        }
                        __syncthreads();
                        if (wave < half) {
                            const u32x4 *slot = wave < 2 ? s_k[wave] : s_v[wave - 2];
#pragma unroll
                            for (int n = 0; n < NDB; ++n)
                                o1[c][n] += __builtin_bit_cast(f32x4, slot[n * kWave + lane]);
                        }
                        __syncthreads();
                    }
                }
                if (wave == 0) {
                    const float qnan = __builtin_nanf("");
#pragma unroll
                    for (int c = 0; c < CS; ++c) {
                        if (orow1[c] < 0)
                            continue;
                        float l = 0.f;
#pragma unroll
                        for (int w = 0; w < NW; ++w)
                            l += s_l[c][w][r16];
                        if constexpr (SPLIT) {
                            float mx = -INFINITY;
#pragma unroll
                            for (int w = 0; w < NW; ++w)
                                mx = fmaxf(mx, s_m[c][w][r16]);
                            store_partial(a, orow1[c], split, nsplit, o1[c], mx, sl, l, vs_h,
                                          any_bad, g);
                            continue;
                        }
                        const float fo = l > 0.f ? vs_h / l : 0.f;
#pragma unroll
                        for (int n = 0; n < NDB; ++n) {
                            f32x4 v = o1[c][n] * fo;
                            if (any_bad)
                                v = f32x4{qnan, qnan, qnan, qnan};
                            uint16_t *dst = static_cast<uint16_t *>(a.out) + (size_t)orow1[c] * D +
                                            16 * n + 4 * g;
                            if constexpr (AT == DT_BF16)
                                *reinterpret_cast<bf16x4 *>(dst) = __builtin_convertvector(v, bf16x4);
                            else
                                *reinterpret_cast<f16x4 *>(dst) = __builtin_convertvector(v, f16x4);
                        }
                    }
                }
            };
            // 17 .. 32 rows: the two column blocks one after the other, each as above
            // (both passes read the same keys; one pass over both blocks would need
            // registers the rest of this kernel instance would then also pay for)
            // Two column blocks (17 .. 32 rows) only in the launch whose tiles are all
            // this small: their registers would otherwise be paid by the whole kernel.
            if (tile_rows <= 16)
                run(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{}, 0);
            else if constexpr (SMALLQ)
                run(std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{}, 0);
            return;
        }
    }

    // Every tile of a small-query launch took the split path above.
    if constexpr (SMALLQ)
        return;

    // ---- each thread's 16-byte pieces of a step, fixed for the whole loop: which of
    // the step's two blocks (the same for a whole wave, kept scalar), the element
    // offset inside that block, and the LDS fragment slot(s) it fills.  Pieces past
    // the step's count repeat the last one (loaded, never staged).
    int k_tl[KPT], k_off[KPT], k_slot[KPT][DT == DT_FP8 ? 2 : 1];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int q = min(tid + i * NT, KCH - 1);
        const int tl = q / (KCH / 2);
        const int rem = q - tl * (KCH / 2);
        const int tok = rem % kBlock;
        const int ch = rem / kBlock;
        k_tl[i] = __builtin_amdgcn_readfirstlane(tl);   // KCH / 2 is a multiple of 64
        k_off[i] = tok * D + ch * EPP;
        if constexpr (DT == DT_FP8) {
            const int c0 = 2 * ch, c1 = 2 * ch + 1;     // 8-element chunks
            k_slot[i][0] = (tl * NKC + c0 / 4) * kWave + tok + 16 * (c0 % 4);
            k_slot[i][1] = (tl * NKC + c1 / 4) * kWave + tok + 16 * (c1 % 4);
        } else {
            k_slot[i][0] = (tl * NKC + ch / 4) * kWave + tok + 16 * (ch % 4);
        }
    }
    constexpr int PPR = kBlock / EPP;                   // pieces per V^T row
    int v_tl[VPT], v_off[VPT], v_t0[VPT], v_slot[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int q = min(tid + i * NT, VCH - 1);
        const int tl = q / (VCH / 2);
        const int rem = q - tl * (VCH / 2);
        const int half = rem % PPR;
        const int d = rem / PPR;
        v_tl[i] = __builtin_amdgcn_readfirstlane(tl);   // VCH / 2 is a multiple of 64
        v_off[i] = d * kBlock + half * EPP;
        v_t0[i] = half * EPP;                           // first token held, in the block
        v_slot[i] = ((d / 16) * kWave + (d % 16) + 16 * (PPR == 2 ? 2 * half : 0)) * 2 + tl;
    }

    // ---- global -> registers: one step's K (or V) pieces into ring slot `slot`, from
    // a scalar block base plus the thread's fixed offset.  Every call issues the same
    // loads, so the number in flight is fixed and each wait covers exactly its slot.
    u32x4 kreg[2][KPT], vreg[2][VPT];
    auto fetch_k = [&](const int (&ph)[2], int slot) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const Elem *blk = kbase + (uint64_t)(uint32_t)(k_tl[i] ? ph[1] : ph[0]) * blk_stride32;
            kreg[slot][i] = *reinterpret_cast<const u32x4 *>(blk + k_off[i]);
        }
    };
    auto fetch_v = [&](const int (&ph)[2], int slot) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const Elem *blk = vbase + (uint64_t)(uint32_t)(v_tl[i] ? ph[1] : ph[0]) * blk_stride32;
            vreg[slot][i] = *reinterpret_cast<const u32x4 *>(blk + v_off[i]);
        }
    };

    // ---- registers -> LDS buffer, in fragment order.  K needs no clean-up: every key
    // of a block past key_end (or past the context) lies after every row's position,
    // so its scores are masked whatever the rows hold.  V^T entries of tokens past the
    // context, and whole blocks past key_end, are zeroed: those rows may hold anything,
    // NaN included, and a zero weight alone would not cancel them.  That happens only
    // in a sequence's last steps, behind a wave-uniform test.
    auto stash_k = [&](int buf, int slot) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            if (KCH % NT == 0 || tid + i * NT < KCH) {
                if constexpr (DT == DT_FP8) {
                    const u32x4 w = kreg[slot][i];
                    s_k[buf][k_slot[i][0]] =
                        u32x4{fp8x2_to_16<AT, false>(w[0]), fp8x2_to_16<AT, true>(w[0]),
                              fp8x2_to_16<AT, false>(w[1]), fp8x2_to_16<AT, true>(w[1])};
                    s_k[buf][k_slot[i][1]] =
                        u32x4{fp8x2_to_16<AT, false>(w[2]), fp8x2_to_16<AT, true>(w[2]),
                              fp8x2_to_16<AT, false>(w[3]), fp8x2_to_16<AT, true>(w[3])};
                } else {
                    s_k[buf][k_slot[i][0]] = kreg[slot][i];
                }
            }
        }
    };
    auto stash_v = [&](int s, int buf, int slot) {
        u32x2 *sv = reinterpret_cast<u32x2 *>(s_v[buf]);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            if (VCH % NT == 0 || tid + i * NT < VCH) {
                u32x4 w = vreg[slot][i];
                const int blk0 = (2 * s + v_tl[i]) * kBlock;    // first token of the block
                if (blk0 + kBlock > ctx || blk0 >= key_end) {   // wave-uniform, rare
                    const int valid = blk0 >= key_end ? 0 : ctx - blk0;
                    w = DT == DT_FP8 ? keep_tokens8(w, v_t0[i], valid)
                                     : keep_tokens16(w, v_t0[i], valid);
                }
                if constexpr (DT == DT_FP8) {
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq)
                        sv[v_slot[i] + 32 * gq] =
                            u32x2{fp8x2_to_16<AT, false>(w[gq]), fp8x2_to_16<AT, true>(w[gq])};
                } else {
                    sv[v_slot[i]] = u32x2{w[0], w[1]};
                    sv[v_slot[i] + 32] = u32x2{w[2], w[3]};
                }
            }
        }
    };

    // ---- running state per column block
    f32x4 o[C][NDB];
    f32x4 lacc[C];
    float m_run[C];
    float mneg[C];                           // -m_run * scale_log2 (0 while m_run = -inf)
#pragma unroll
    for (int c = 0; c < C; ++c) {
#pragma unroll
        for (int n = 0; n < NDB; ++n)
            o[c][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        lacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[c] = -INFINITY;
        mneg[c] = 0.f;
    }
    const float sl = sl_h;                   // > 0 (checked scales): max commutes with it
    // The running max is only a reference point: O and l are both scaled by 2^(-m sl),
    // which cancels in O / l whatever m is.  It is therefore moved only when a score
    // exceeds it by more than 2^kRescaleSlack in the exp2 domain; weights stay at most
    // 2^kRescaleSlack (well inside 16-bit and fp32 range) and the rescale of O, which
    // would otherwise run whenever any row sees a new maximum, runs about once.
    const float grow_thr = fminf(kRescaleSlack / sl, 3.0e38f);
    const u32x4 ones = {one_pair<AT>(), one_pair<AT>(), one_pair<AT>(), one_pair<AT>()};

    // S^T of step s from K buffer kb.  The K fragments are read e-chunk-major, in the
    // order the products use them; the e-chunk is outermost so the 2 C accumulators
    // form independent chains.
    auto qk = [&](int kb, f32x4 (&sc)[C][2]) {
        u32x4 kf[NKC][2];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int tl = 0; tl < 2; ++tl)
                kf[kc][tl] = s_k[kb][(tl * NKC + kc) * kWave + lane];
#pragma unroll
        for (int c = 0; c < C; ++c)
            sc[c][0] = sc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int tl = 0; tl < 2; ++tl)
#pragma unroll
                for (int c = 0; c < C; ++c)
                    sc[c][tl] = mma32<AT>(kf[kc][tl], qf[c][kc], sc[c][tl]);
    };

    // Step s's scores: causal mask, running max, and the rescale of O and l when some
    // score exceeds a row's reference max by more than the slack.  Only steps reaching
    // past the tile's first position can hold keys after a row's position.  An empty
    // history (-inf) always takes the first finite max; an all-masked lane never moves it.
    auto mask_max = [&](int s, f32x4 (&sc)[C][2]) {
        const bool diag = 32 * s + 31 > first;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (diag) {
#pragma unroll
                for (int tl = 0; tl < 2; ++tl)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        sc[c][tl][j] = (32 * s + 16 * tl + 4 * g + j <= pos[c]) ? sc[c][tl][j]
                                                                                : -INFINITY;
            }
        }
        float lmx[C];
        bool grow = false;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            lmx[c] = max8(sc[c]);
            grow |= lmx[c] - m_run[c] > grow_thr;
        }
        if (__any(grow)) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const float m_new = fmaxf(m_run[c], max_over_row_groups(lmx[c]));
                const float alpha =
                    (m_new == -INFINITY) ? 1.f : exp2_fast((m_run[c] - m_new) * sl);
#pragma unroll
                for (int n = 0; n < NDB; ++n)
                    o[c][n] *= alpha;
                lacc[c] *= alpha;
                m_run[c] = m_new;
                mneg[c] = (m_new == -INFINITY) ? 0.f : -m_new * sl;
            }
        }
    };

    // Weights of a masked step against the current max, rounded to 16 bits.
    auto weights = [&](const f32x4 (&sc)[C][2], u32x4 (&pb)[C]) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            f32x4 p0, p1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                p0[j] = exp2_fast(fmaf(sc[c][0][j], sl, mneg[c]));
                p1[j] = exp2_fast(fmaf(sc[c][1][j], sl, mneg[c]));
            }
            pb[c] = pack8<AT>(p0, p1);
        }
    };

    // O += V^T P and l += ones P from V buffer vb.
    auto pv = [&](const u32x4 (&vf)[NDB], const u32x4 (&pb)[C]) {
#pragma unroll
        for (int n = 0; n < NDB; ++n)
#pragma unroll
            for (int c = 0; c < C; ++c)
                o[c][n] = mma32<AT>(vf[n], pb[c], o[c][n]);
#pragma unroll
        for (int c = 0; c < C; ++c)
            lacc[c] = mma32<AT>(ones, pb[c], lacc[c]);
    };

    // Two-stage pipeline over 32-key steps.  K is staged one step ahead of V.  Pass
    // it first stages K of step it+2 and V of step it+1 into the LDS buffers those
    // steps last used and reissues the freed register slots for K of step it+4 and V
    // of step it+3 (two passes ahead of their staging); then, in one branch-free
    // stretch, it issues step it+1's QK products interleaved with step it's weights
    // (its mask and max were settled in the previous pass), then step it's PV
    // products; after the barrier it masks step it+1's scores and updates the running
    // max.  The loop is
    // unrolled by two, so the ring slots and the two score sets are fixed registers,
    // and runs whole pairs of passes with no other exit: every pass issues the same
    // loads and waits, so each wait covers exactly the slot it needs.  Loads past the
    // last step are clamped to it; steps past the tile's last stage zeros, and every
    // key of theirs lies after every row's position, so they are masked out entirely
    // and change nothing.  Steps are counted from the tile's first key; the workgroup
    // walks steps s_begin .. s_end-1.  Every LDS buffer is rewritten only after a
    // barrier that follows all reads of its previous contents.
    if (s_end > s_begin) {
        const int sb = s_begin;
        const int last = s_end - 1;
        int raw[2], ph_a[2], ph_b[2];
        table(sb, raw);
        resolve(sb, raw, ph_a);
        table(min(sb + 1, last), raw);
        resolve(min(sb + 1, last), raw, ph_b);
        fetch_k(ph_a, 0);
        fetch_k(ph_b, 1);
        fetch_v(ph_a, 0);
        stash_k(0, 0);                            // waits for these loads and for q
        stash_k(1, 1);
        stash_v(sb, 0, 0);
        table(min(sb + 2, last), raw);
        resolve(min(sb + 2, last), raw, ph_a);       // step sb+2
        fetch_k(ph_a, 0);
        table(min(sb + 3, last), raw);
        int ph_k[2];                                 // block ids of the last K fetch
        resolve(min(sb + 3, last), raw, ph_k);       // step sb+3
        fetch_k(ph_k, 1);
        fetch_v(ph_b, 1);                            // V of step sb+1
        fetch_v(ph_a, 0);                            // V of step sb+2
        table(min(sb + 4, last), raw);
        __syncthreads();
        // Pass it's staging, first thing after the barrier that ended pass it-1: K of
        // step it+2 and V of step it+1 into the LDS buffers whose contents (steps it and
        // it-1) were last read in pass it-1, then the freed register slots reissued for
        // K of step it+4 and V of step it+3.  Done at the start of the pass, the stores
        // have the whole pass to complete before the next barrier waits on them.
        auto stage = [&](int it, int u) {
            stash_k(u, u);
            stash_v(sb + it + 1, u ^ 1, u ^ 1);
            int ph_n[2];
            resolve(min(sb + it + 4, last), raw, ph_n);
            fetch_k(ph_n, u);                        // K of step sb+it+4
            fetch_v(ph_k, u ^ 1);                    // V of step sb+it+3
            ph_k[0] = ph_n[0];
            ph_k[1] = ph_n[1];
            table(min(sb + it + 5, last), raw);
        };
        const int npairs = (s_end - s_begin + 1) / 2;
        // A wave whose rows are all idle (a short chunk, a decode row in the tile)
        // runs only the staging: the same loads, stores and barriers, no products.
        // Launches where every tile is full (IDLE false) carry no such branch.
        const bool idle = IDLE && wave * C * 16 >= n_here * a.group;   // wave-uniform
        f32x4 sc[2][C][2];
        if (!idle) {
            qk(0, sc[0]);
            mask_max(sb, sc[0]);
        }
        // Pass 0 restages buffer 0 (K of step 2): every wave's reads of step 0's K
        // must be done first.
        __syncthreads();
        if (idle) {
            for (int pr = 0; pr < npairs; ++pr) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    stage(2 * pr + u, u);
                    __syncthreads();
                }
            }
        } else {
            for (int pr = 0; pr < npairs; ++pr) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int it = 2 * pr + u;
                    stage(it, u);
                    qk(u ^ 1, sc[u ^ 1]);                // step it+1's scores
                    u32x4 vf[NDB];
#pragma unroll
                    for (int n = 0; n < NDB; ++n)
                        vf[n] = s_v[u][n * kWave + lane];
                    u32x4 pb[C];
                    weights(sc[u], pb);
                    pv(vf, pb);
                    // Issue order.  All 8 waves leave the barrier together, so fragment
                    // reads issued in one burst keep the LDS busy while the MFMA pipes
                    // wait; instead the reads are spread over the QK products, each one
                    // e-chunk or more ahead of its use: the first two e-chunks' K
                    // fragments, then per e-chunk its QK products (each followed by a
                    // share of step it's weights), with the later K fragments and the V
                    // fragments issued between them; then the PV and normaliser products.
                    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                    for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
                        for (int k = 0; k < 2 * C; ++k) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
                        }
                        if (kc == 0)
                            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                        else if (kc == 1)
                            __builtin_amdgcn_sched_group_barrier(0x100, 2 + NDB / 2, 0);
                        else if (kc == 2)
                            __builtin_amdgcn_sched_group_barrier(0x100, NDB / 2, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, NDB * C + C, 0);
                    __syncthreads();
                    mask_max(sb + it + 1, sc[u ^ 1]);
                }
            }
        }
    }

    const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0 || bad_ctx;
    const float qnan = __builtin_nanf("");
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if (orow[c] < 0)
            continue;
        const float l = lacc[c][0];
        if constexpr (SPLIT) {
            store_partial(a, orow[c], split, nsplit, o[c], m_run[c], sl, l, vs_h, any_bad, g);
            continue;
        }
        const float f = l > 0.f ? vs_h / l : 0.f;
#pragma unroll
        for (int n = 0; n < NDB; ++n) {
            f32x4 v = o[c][n] * f;
            if (any_bad)
                v = f32x4{qnan, qnan, qnan, qnan};
            uint16_t *dst = static_cast<uint16_t *>(a.out) + (size_t)orow[c] * D + 16 * n + 4 * g;
            if constexpr (AT == DT_BF16)
                *reinterpret_cast<bf16x4 *>(dst) = __builtin_convertvector(v, bf16x4);
            else
                *reinterpret_cast<f16x4 *>(dst) = __builtin_convertvector(v, f16x4);
        }
    }
}

// ------------------------------------------------------------------ reduce kernel

// Merges the key splits' partials of every query row with the max/normaliser rule of
// the decode path ("Deep dive into vLLM 06", Flash-Decoding: each split's partial
// result carries its own max and sum):
//   M = max_s m_s,   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
// (splits that saw no key have m = -inf and weigh nothing; a query with no key at all
// gets a zero row; a NaN partial, written by a workgroup with bad input, gives NaN).
// One workgroup per (row chunk, kv-head, sequence): its rows are validated as the main
// kernel does, so a malformed query range stays unwritten.  A thread owns 4
// consecutive elements of one (row, q-head) and issues every split's loads together.
template <int AT, int D>
__global__ __launch_bounds__(256) void pa_prefill_reduce(PrefillArgs a)
{
    const int b = blockIdx.z;
    const int kvh = blockIdx.y;
    const int q0 = a.query_start[b];
    const int q_len = a.query_start[b + 1] - q0;
    if (q0 < 0 || q_len < 0 || q_len > a.max_query_len || q0 > a.num_tokens - q_len)
        return;
    const int rows = prefill_reduce_rows(a.group, D);
    const int p0 = blockIdx.x * rows;
    const int S = a.splits;
    const int items = min(rows, q_len - p0) * a.group * (D / 4);
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
        const int e4 = it % (D / 4);
        const int hr = it / (D / 4);
        const int h = hr % a.group;
        const int p = p0 + hr / a.group;
        const size_t row = (size_t)(q0 + p) * a.num_q_heads + kvh * a.group + h;
        float m[kPrefillMaxSplits], l[kPrefillMaxSplits];
        f32x4 o[kPrefillMaxSplits];
#pragma unroll
        for (int sp = 0; sp < kPrefillMaxSplits; ++sp) {
            if (sp < S) {
                const size_t slot = row * S + sp;
                m[sp] = a.ws_m[slot];
                l[sp] = a.ws_l[slot];
                o[sp] = *reinterpret_cast<const f32x4 *>(a.ws_o + slot * D + 4 * e4);
            }
        }
        float M = -INFINITY;
        bool nan = false;
#pragma unroll
        for (int sp = 0; sp < kPrefillMaxSplits; ++sp)
            if (sp < S) {
                M = fmaxf(M, m[sp]);
                nan |= m[sp] != m[sp];
            }
        f32x4 num = {0.f, 0.f, 0.f, 0.f};
        float den = 0.f;
#pragma unroll
        for (int sp = 0; sp < kPrefillMaxSplits; ++sp)
            if (sp < S) {
                const float f = m[sp] == -INFINITY ? 0.f : exp2_fast(m[sp] - M);
                num += f * o[sp];
                den += f * l[sp];
            }
        f32x4 v = den > 0.f ? num * (1.f / den) : f32x4{0.f, 0.f, 0.f, 0.f};
        if (nan)
            v = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                      __builtin_nanf("")};
        uint16_t *dst = static_cast<uint16_t *>(a.out) + row * D + 4 * e4;
        if constexpr (AT == DT_BF16)
            *reinterpret_cast<bf16x4 *>(dst) = __builtin_convertvector(v, bf16x4);
        else
            *reinterpret_cast<f16x4 *>(dst) = __builtin_convertvector(v, f16x4);
    }
}

template <int DT, int AT, int D>
hipError_t launch_prefill_t(const PrefillArgs &a, int grid, bool idle, bool smallq,
                            hipStream_t stream)
{
    constexpr int C = prefill_cols(D);
    constexpr int NW = kPrefillWaves;
    const dim3 g2(grid, a.splits);
    const dim3 blk(NW * kWave);
    const bool split = a.splits > 1;
    bool launched = false;
    if constexpr (D <= 128) {
        if (smallq) {
            if (split)
                hipLaunchKernelGGL((pa_prefill_kernel<DT, AT, D, NW, C, true, true, true>), g2,
                                   blk, 0, stream, a);
            else
                hipLaunchKernelGGL((pa_prefill_kernel<DT, AT, D, NW, C, true, true, false>), g2,
                                   blk, 0, stream, a);
            launched = true;
        }
    }
    if (!launched) {
        if (idle && split)
            hipLaunchKernelGGL((pa_prefill_kernel<DT, AT, D, NW, C, true, false, true>), g2, blk,
                               0, stream, a);
        else if (idle)
            hipLaunchKernelGGL((pa_prefill_kernel<DT, AT, D, NW, C, true, false, false>), g2, blk,
                               0, stream, a);
        else if (split)
            hipLaunchKernelGGL((pa_prefill_kernel<DT, AT, D, NW, C, false, false, true>), g2, blk,
                               0, stream, a);
        else
            hipLaunchKernelGGL((pa_prefill_kernel<DT, AT, D, NW, C, false, false, false>), g2,
                               blk, 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits <= 1)
        return e;
    const int rows = prefill_reduce_rows(a.group, D);
    const dim3 rgrid((a.max_query_len + rows - 1) / rows, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((pa_prefill_reduce<AT, D>), rgrid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

int prefill_rows_per_group(int head_dim) { return kPrefillWaves * prefill_cols(head_dim) * 16; }

hipError_t launch_prefill(int dtype, int act_dtype, int head_dim, const PrefillArgs &a,
                          hipStream_t stream)
{
    const int pairs = a.num_seqs * a.num_kv_heads;
    const int grid_plain = (pairs + kXcds - 1) / kXcds * kXcds * a.num_qtiles;
    // Every tile is full, and so every wave has rows, when all chunks have the
    // longest length, that length is a whole number of tiles, and a tile's rows reach
    // the last wave; otherwise idle waves may occur and the kernel that lets them
    // skip the products is launched.
    const bool full = (int64_t)a.num_tokens == (int64_t)a.num_seqs * a.max_query_len &&
                      a.max_query_len % a.q_tile == 0 &&
                      a.q_tile * a.group > (kPrefillWaves - 1) * prefill_cols(head_dim) * 16;
    // The compact map (partial tiles possible, ranked batch) needs as many workgroups
    // per XCD as its busiest XCD has tiles: a sequence puts at most ceil(Hkv / 8) of its
    // pairs on one XCD, and the chunks hold at most T / q_tile + B tiles when their
    // query ranges do not overlap (ranges that do are outside the contract and may then
    // lose tiles).  Never more than the plain map's share per XCD.
    // Every tile has at most two column blocks of rows: the instance that holds only
    // the split path (its registers are not shared with the staged loop).
    const bool smallq = head_dim <= 128 && (int64_t)a.max_query_len * a.group <= 32;
    int grid = grid_plain;
    if (!full && a.longest_first) {
        const int64_t tiles = std::min<int64_t>((int64_t)a.num_tokens / a.q_tile + a.num_seqs,
                                                (int64_t)a.num_seqs * a.num_qtiles);
        const int64_t per_xcd = std::min<int64_t>((a.num_kv_heads + kXcds - 1) / kXcds * tiles,
                                                  (int64_t)grid_plain / kXcds);
        grid = (int)(per_xcd * kXcds);
    }
#define PA_PF_CASE(DT, AT, D)                                                      \
    if (dtype == DT && act_dtype == AT && head_dim == D)                          \
        return launch_prefill_t<DT, AT, D>(a, grid, !full, smallq, stream);
    PA_PF_CASE(DT_BF16, DT_BF16, 128)
    PA_PF_CASE(DT_BF16, DT_BF16, 64)
    PA_PF_CASE(DT_BF16, DT_BF16, 256)
    PA_PF_CASE(DT_F16, DT_F16, 128)
    PA_PF_CASE(DT_F16, DT_F16, 64)
    PA_PF_CASE(DT_F16, DT_F16, 256)
    PA_PF_CASE(DT_FP8, DT_BF16, 128)
    PA_PF_CASE(DT_FP8, DT_BF16, 64)
    PA_PF_CASE(DT_FP8, DT_BF16, 256)
    PA_PF_CASE(DT_FP8, DT_F16, 128)
    PA_PF_CASE(DT_FP8, DT_F16, 64)
    PA_PF_CASE(DT_FP8, DT_F16, 256)
#undef PA_PF_CASE
    return hipErrorInvalidValue;
}

}  // namespace pa
