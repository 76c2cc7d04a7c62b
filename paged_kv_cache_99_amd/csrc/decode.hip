// decode.hip -- paged decode attention for gfx950 (HBM-bound; vector ALU, no MFMA).
//
// What it computes: for each sequence s and query head h, softmax(scale * q K^T) V over positions
// 0..L-1 of kv head h / group (lecture 32 "LLM 在线推理两阶段" §3.1 formula and decode step, §3.4
// GQA groups), with position i read from block table[s][i / 16] at offset i % 16
// (openeuler.csdn.net "高并发 AI 服务的内存瓶颈", Attention 计算时的 Block 映射). Blocks are
// consumed one at a time with a running maximum and running sum of exponentials, and partial results
// are combined by rescaling to the common maximum (devpress.csdn.net/amd vLLM overview, §9 (4)
// online softmax; §3 (3) per-block accumulation over the block table).
//
// Work unit: one wavefront per (sequence, kv head, query-head subgroup, partition). A (block,
// kv head) tile is 16 rows x D contiguous 16-bit words (4 KiB at D = 128). Lane l of the wave
// loads 16 bytes at offset 16*l of each 1 KiB piece of the tile, so every load instruction reads
// one contiguous KiB, and lane l then holds 8 dims (l % RL)*8.. of token rows (l / RL) + ROWS*i.
// Scores: each lane dots its 8 dims with the G queries (v_dot2_f32_{f16,bf16}); the RL lanes of a
// row finish the sum with DPP. Softmax and P*V need no cross-lane traffic at all: every lane keeps
// its own running max / sum / 8-dim accumulator for the tokens of its row class, and the ROWS row
// classes are merged once at the end of the unit. The next tile's loads are issued before the
// current tile is consumed.
//
// E4M3 caches (lecture 34 "vLLM 生产级系统架构全景剖析" §4.4): the same kernel with one byte per
// element, so a lane's 16-byte piece holds 16 dims; keys are widened to 16-bit pairs
// (v_cvt_scalef32_pk_*_fp8) for the dot products and values to float32 (v_cvt_pk_f32_fp8), exact
// conversions; k_scale is folded into the score scale and v_scale into the output.
//
// Split-K: with partition_size P > 0 the unit covers tokens [part*P, (part+1)*P) and writes its
// unnormalised accumulator, max and sum (log2 domain) to the workspace; a merge kernel rescales the
// parts of each (sequence, head) to their common maximum and normalises.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

struct DecodeParams {
    const uint16_t *__restrict__ query;
    const uint16_t *__restrict__ k_cache;
    const uint16_t *__restrict__ v_cache;
    const int32_t *__restrict__ block_tables;
    const int32_t *__restrict__ seq_lens;
    uint16_t *__restrict__ out;
    float *__restrict__ ws_acc;
    float *__restrict__ ws_ml;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t num_blocks;
    int32_t max_seq_len;
    int32_t part_tokens;  // tokens per unit (multiple of 16)
    int32_t max_parts;
    int32_t n_sub;        // query-head subgroups per kv head
    int32_t n_units;
    int32_t split;
    float scale_log2;     // scale * log2(e) (* k_scale for E4M3 caches): scores in the log2 domain
    float v_scale;        // E4M3 caches: value scale, applied to the accumulated output
    // Shared-prefix (cascade) support; zero / null for a plain decode.
    const int32_t *__restrict__ seq_starts;   // [num_seqs] first position of a unit's range
    const int32_t *__restrict__ group_starts; // [num_groups + 1] members of prefix group g
    int32_t num_groups;
    int32_t ws_slots;     // partial-result slots per (sequence, head) row of the workspace
    int32_t slot_base;    // first slot these units write
    int32_t pre_slots;    // slots [0, pre_slots) hold shared-prefix parts (merge)
    int32_t n_vsub;       // prefix units: groups of GK (member, head) pairs per kv head
};

// Position range of unit `part` of a sequence: [start + part*P, min(L, start + (part+1)*P)).
__device__ __forceinline__ int unit_start(const DecodeParams &p, int seq, int L)
{
    return p.seq_starts ? min(max(p.seq_starts[seq], 0), L) : 0;
}

// F8: the caches hold E4M3 codes (one byte per element) instead of 16-bit elements.
template <bool BF, bool F8, int D, int GK>
__global__ __launch_bounds__(64) void decode_partition_kernel(DecodeParams p)
{
    constexpr int EPL = F8 ? 16 : 8;     // cache elements per 16-byte piece = dims per lane
    constexpr int RL = D / EPL;          // lanes per token row
    constexpr int ROWS = kWave / RL;     // token rows per 1 KiB load
    constexpr int NCH = kBlock / ROWS;   // loads per (block, kv head) tile
    constexpr int QV = EPL / 8;          // 16-byte query pieces per lane and head
    constexpr int ESZ = F8 ? 1 : 2;      // bytes per cache element
    const int lane = threadIdx.x;
    const int r = lane / RL;

    const int unit = xcd_logical_id(blockIdx.x, gridDim.x);
    if (unit >= p.n_units)
        return;
    const int seq = unit % p.num_seqs;
    int rest = unit / p.num_seqs;
    const int part = rest % p.max_parts;
    rest /= p.max_parts;
    const int sub = rest % p.n_sub;
    const int kvh = rest / p.n_sub;
    const int h0 = (kvh * p.n_sub + sub) * GK;  // first query head of this unit

    const int L = min(max(p.seq_lens[seq], 0), p.max_seq_len);
    const int t0 = unit_start(p, seq, L) + part * p.part_tokens;
    if (p.split && t0 >= L)
        return;  // a part with no tokens: the merge never reads it
    const int t1 = min(L, t0 + p.part_tokens);

    uint4 q[GK][QV];
#pragma unroll
    for (int h = 0; h < GK; ++h)
#pragma unroll
        for (int k = 0; k < QV; ++k)
            q[h][k] = *(const uint4 *)(p.query + ((size_t)seq * p.num_q_heads + h0 + h) * D +
                                       (lane % RL) * EPL + k * 8);

    float m[GK], l[GK], acc[GK][EPL];
#pragma unroll
    for (int h = 0; h < GK; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
            acc[h][j] = 0.0f;
    }

    const int32_t *table = p.block_tables + (size_t)seq * p.max_blocks;
    const uint8_t *kbase = (const uint8_t *)p.k_cache;
    const uint8_t *vbase = (const uint8_t *)p.v_cache;
    // byte offsets: lane l reads piece l % RL of row l / RL of each 1 KiB load
    const size_t block_stride = (size_t)p.num_kv_heads * kBlock * D * ESZ;
    const size_t tile_off = ((size_t)kvh * kBlock * D + lane * EPL) * ESZ;

    for (int bb = t0 / kBlock; bb * kBlock < t1; bb += kWave) {
        const int nb = min(kWave, (t1 - bb * kBlock + kBlock - 1) / kBlock);
        const int my_blk = lane < nb ? table[bb + lane] : 0;

        auto load = [&](int k, uint4(&kk)[NCH], uint4(&vv)[NCH]) {
            int blk = __builtin_amdgcn_readlane(my_blk, k);
            blk = (unsigned)blk < (unsigned)p.num_blocks ? blk : 0;
            const uint8_t *kp = kbase + blk * block_stride + tile_off;
            const uint8_t *vp = vbase + blk * block_stride + tile_off;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                kk[i] = load_nt(kp + i * 1024);
                vv[i] = load_nt(vp + i * 1024);
            }
        };

        auto consume = [&](int k, const uint4(&kk)[NCH], uint4(&vv)[NCH]) {
            const int base = (bb + k) * kBlock;
            const int raw = __builtin_amdgcn_readlane(my_blk, k);
            const bool good_blk = (unsigned)raw < (unsigned)p.num_blocks;
            float s[GK][NCH];
#pragma unroll
            for (int h = 0; h < GK; ++h)
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    float d;
                    if constexpr (F8)
                        d = dot16_e4m3<BF>(q[h], kk[i]);
                    else
                        d = dot8<BF>(q[h][0], kk[i]);
                    s[h][i] = group_sum<RL>(d) * p.scale_log2;
                }
            if (!(good_blk && base >= t0 && base + kBlock <= t1)) {  // an edge block or a bad id
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    const int tok = base + i * ROWS + r;
                    const bool ok = good_blk && tok >= t0 && tok < t1;
#pragma unroll
                    for (int h = 0; h < GK; ++h)
                        s[h][i] = ok ? s[h][i] : -INFINITY;
                    // a masked row may hold any bits (NaN included): zero it before P*V
                    vv[i] = ok ? vv[i] : make_uint4(0, 0, 0, 0);
                }
            }
            float pr[GK][NCH];
#pragma unroll
            for (int h = 0; h < GK; ++h) {
                float mx = s[h][0];
#pragma unroll
                for (int i = 1; i < NCH; ++i)
                    mx = fmaxf(mx, s[h][i]);
                const float mn = fmaxf(m[h], mx);
                const float ms = mn == -INFINITY ? 0.0f : mn;
                const float alpha = fast_exp2(m[h] - ms);
                float psum = 0.0f;
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    pr[h][i] = fast_exp2(s[h][i] - ms);
                    psum += pr[h][i];
                }
                l[h] = l[h] * alpha + psum;
                m[h] = mn;
#pragma unroll
                for (int j = 0; j < EPL; ++j)
                    acc[h][j] *= alpha;
            }
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const uint32_t w[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (F8) {
                        float v[4];
                        e4m3x4_to_f32(w[j], v);
#pragma unroll
                        for (int h = 0; h < GK; ++h)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                acc[h][4 * j + e] += pr[h][i] * v[e];
                    } else {
                        const float v0 = lo_f32<BF>(w[j]), v1 = hi_f32<BF>(w[j]);
#pragma unroll
                        for (int h = 0; h < GK; ++h) {
                            acc[h][2 * j] += pr[h][i] * v0;
                            acc[h][2 * j + 1] += pr[h][i] * v1;
                        }
                    }
                }
            }
        };

        uint4 ka[NCH], va[NCH], kn[NCH], vn[NCH];
        load(0, ka, va);
        for (int k = 0; k < nb; ++k) {
            if (k + 1 < nb)
                load(k + 1, kn, vn);
            consume(k, ka, va);
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                ka[i] = kn[i];
                va[i] = vn[i];
            }
        }
    }

    // merge the ROWS row classes of every head (lanes that differ in their row index)
#pragma unroll
    for (int h = 0; h < GK; ++h) {
        float M = m[h];
#pragma unroll
        for (int off = RL; off < kWave; off <<= 1)
            M = fmaxf(M, xor_shfl(M, off));
        const float f = fast_exp2(m[h] - (M == -INFINITY ? 0.0f : M));
        float lh = l[h] * f;
#pragma unroll
        for (int off = RL; off < kWave; off <<= 1)
            lh += xor_shfl(lh, off);
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            float a = acc[h][j] * f;
#pragma unroll
            for (int off = RL; off < kWave; off <<= 1)
                a += xor_shfl(a, off);
            acc[h][j] = F8 ? a * p.v_scale : a;
        }
        m[h] = M;
        l[h] = lh;
    }

    if (lane < RL) {
#pragma unroll
        for (int h = 0; h < GK; ++h) {
            const size_t row = (size_t)seq * p.num_q_heads + h0 + h;
            if (p.split) {
                const size_t slot = row * p.ws_slots + p.slot_base + part;
                float *wa = p.ws_acc + slot * D + lane * EPL;
#pragma unroll
                for (int j = 0; j < EPL; j += 4)
                    *(float4 *)(wa + j) =
                        make_float4(acc[h][j], acc[h][j + 1], acc[h][j + 2], acc[h][j + 3]);
                if (lane == 0)
                    *(float2 *)(p.ws_ml + slot * 2) = make_float2(m[h], l[h]);
            } else {
                const float inv = l[h] > 0.0f ? 1.0f / l[h] : 0.0f;
#pragma unroll
                for (int j = 0; j < EPL; j += 8) {
                    uint4 o;
                    o.x = pack2<BF>(acc[h][j] * inv, acc[h][j + 1] * inv);
                    o.y = pack2<BF>(acc[h][j + 2] * inv, acc[h][j + 3] * inv);
                    o.z = pack2<BF>(acc[h][j + 4] * inv, acc[h][j + 5] * inv);
                    o.w = pack2<BF>(acc[h][j + 6] * inv, acc[h][j + 7] * inv);
                    *(uint4 *)(p.out + row * D + lane * EPL + j) = o;
                }
            }
        }
    }
}

// ------------------------------------------------------------------ head groups of 4 and 8
// The kernel above computes every score in all 16 lanes of a token row and repeats the softmax
// there, once per query head: for GQA groups that redundancy, not HBM, bounds it. Here each
// (block, kv head) K tile is staged in LDS and re-read in a scoring layout where GK lanes own one
// token (lane j covers dims [j*D/GK, (j+1)*D/GK) for all GK heads). A transpose-reduce over those
// GK lanes leaves lane j with the full score of head j, so the exponential and the running sum are
// computed once per (token, head). The softmax reference point m is wave-uniform per head and
// moves only when a score exceeds it by more than 2^kLazy (then the accumulators are rescaled): all
// tokens of a head share one m, so P*V may use any lane layout. Probabilities reach the P*V lanes
// (the coalesced V layout of the kernel above) through a 16 x GK float buffer in LDS.
constexpr float kLazy = 8.0f;  // log2 units: partial sums stay below 2^8 times their true scale

// Sum the GK values x[0..GK) of each lane over aligned groups of GK lanes, leaving lane j of a
// group with the group's total of x[j]. Stage s pairs lanes that differ in bit s of j (for GK = 8,
// bit 2 via row_half_mirror, which reverses each group of 8): each lane keeps the half of its values
// selected by that bit and adds the partner's copy of the same half.
template <int GK>
__device__ __forceinline__ float transpose_reduce(float (&x)[GK], int j)
{
    if constexpr (GK == 8) {
        const bool b2 = (j >> 2) & 1;
        float y[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float keep = b2 ? x[4 + k] : x[k], send = b2 ? x[k] : x[4 + k];
            y[k] = keep + dpp_f(send, 2);  // row_half_mirror: lane j <-> 7 - j
        }
        const bool b1 = (j >> 1) & 1;
        float z[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const float keep = b1 ? y[2 + k] : y[k], send = b1 ? y[k] : y[2 + k];
            z[k] = keep + dpp_f(send, 1);  // j <-> j ^ 2
        }
        const bool b0 = j & 1;
        const float keep = b0 ? z[1] : z[0], send = b0 ? z[0] : z[1];
        return keep + dpp_f(send, 0);  // j <-> j ^ 1
    } else {
        static_assert(GK == 4, "groups of 4 or 8");
        const bool b1 = (j >> 1) & 1;
        float z[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const float keep = b1 ? x[2 + k] : x[k], send = b1 ? x[k] : x[2 + k];
            z[k] = keep + dpp_f(send, 1);
        }
        const bool b0 = j & 1;
        const float keep = b0 ? z[1] : z[0], send = b0 ? z[0] : z[1];
        return keep + dpp_f(send, 0);
    }
}

// XOR swizzle of the 16-byte pieces of K row `row` in LDS: the coalesced writes fill whole rows;
// the scoring reads (16 lanes = 16/GK*... rows x pieces) then fall on distinct banks.
template <int D, int GK>
__device__ __forceinline__ int kswz(int row)
{
    if constexpr (D == 128)
        return row & (16 / GK - 1);
    else
        return (row >> 1) & (8 / GK - 1);
}

// One unit over positions [t0, t1) of the table `table` and kv head kvh, for GK query rows qrow[h]
// (rows of query / out / workspace; -1 = no query). Split units write slot `slot` of each row.
template <bool BF, int D, int GK>
__device__ __forceinline__ void gqa_unit(const DecodeParams &p, const int (&qrow)[GK],
                                         const int32_t *table, int kvh, int t0, int t1, int slot,
                                         bool split)
{
    constexpr int RL = D / 8;            // P*V layout: lanes per token row
    constexpr int ROWS = kWave / RL;     // token rows per 1 KiB load
    constexpr int NCH = kBlock / ROWS;   // loads per (block, kv head) tile
    constexpr int TPP = kWave / GK;      // tokens scored per pass
    constexpr int NPASS = kBlock / TPP;  // passes per block
    constexpr int CPL = D / GK / 8;      // 16-byte pieces of a K row per scoring lane
    constexpr int ROWB = D * 2;
    __shared__ __align__(16) uint8_t k_lds[kBlock * ROWB];
    __shared__ __align__(16) float p_lds[kBlock * GK];

    const int lane = threadIdx.x;
    const int r = lane / RL, c = lane % RL;  // P*V layout
    const int ts = lane / GK, j = lane % GK; // scoring layout: token slot, dim slice = own head

    // queries in the scoring layout: dims [j*D/GK, (j+1)*D/GK) of every head of the group
    uint4 q[GK][CPL];
#pragma unroll
    for (int h = 0; h < GK; ++h)
#pragma unroll
        for (int k = 0; k < CPL; ++k)
            q[h][k] = qrow[h] >= 0 ? *(const uint4 *)(p.query + (size_t)qrow[h] * D + (j * CPL + k) * 8)
                                   : make_uint4(0, 0, 0, 0);

    float m_own = -INFINITY, l_own = 0.0f;  // reference point and partial sum of head j
    float acc[GK][8];
#pragma unroll
    for (int h = 0; h < GK; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[h][e] = 0.0f;

    const size_t block_stride = (size_t)p.num_kv_heads * kBlock * D;
    const size_t tile_off = (size_t)kvh * kBlock * D + lane * 8;

    for (int bb = t0 / kBlock; bb * kBlock < t1; bb += kWave) {
        const int nb = min(kWave, (t1 - bb * kBlock + kBlock - 1) / kBlock);
        const int my_blk = lane < nb ? table[bb + lane] : 0;

        auto load = [&](int k, uint4(&kk)[NCH], uint4(&vv)[NCH]) {
            int blk = __builtin_amdgcn_readlane(my_blk, k);
            blk = (unsigned)blk < (unsigned)p.num_blocks ? blk : 0;
            const uint16_t *kp = p.k_cache + blk * block_stride + tile_off;
            const uint16_t *vp = p.v_cache + blk * block_stride + tile_off;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                kk[i] = load_nt(kp + i * ROWS * D);
                vv[i] = load_nt(vp + i * ROWS * D);
            }
        };

        auto consume = [&](int k, const uint4(&kk)[NCH], uint4(&vv)[NCH]) {
            const int base = (bb + k) * kBlock;
            const int raw = __builtin_amdgcn_readlane(my_blk, k);
            const bool good_blk = (unsigned)raw < (unsigned)p.num_blocks;
            const bool whole = good_blk && base >= t0 && base + kBlock <= t1;

            // stage the K tile: row ROWS*i + r, piece c (swizzled)
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int row = ROWS * i + r;
                *(uint4 *)(k_lds + row * ROWB + ((c ^ kswz<D, GK>(row)) << 4)) = kk[i];
            }

            // scores of head j for tokens ts + TPP*pass
            float sc[NPASS];
#pragma unroll
            for (int ps = 0; ps < NPASS; ++ps) {
                const int row = ps * TPP + ts;
                uint4 kr[CPL];
#pragma unroll
                for (int k2 = 0; k2 < CPL; ++k2)
                    kr[k2] = *(const uint4 *)(k_lds + row * ROWB +
                                              (((j * CPL + k2) ^ kswz<D, GK>(row)) << 4));
                float part_sum[GK];
#pragma unroll
                for (int h = 0; h < GK; ++h) {
                    float a = 0.0f;
#pragma unroll
                    for (int k2 = 0; k2 < CPL; ++k2)
                        a += dot8<BF>(q[h][k2], kr[k2]);
                    part_sum[h] = a;
                }
                float x = transpose_reduce<GK>(part_sum, j) * p.scale_log2;
                if (!whole && !(good_blk && base + row >= t0 && base + row < t1))
                    x = -INFINITY;
                sc[ps] = x;
            }

            // lazy reference point: move it (and rescale) only when a score passes it by 2^kLazy
            float over = sc[0] - m_own;
#pragma unroll
            for (int ps = 1; ps < NPASS; ++ps)
                over = fmaxf(over, sc[ps] - m_own);
            if (!__all(!(over > kLazy))) {
                float mx = sc[0];
#pragma unroll
                for (int ps = 1; ps < NPASS; ++ps)
                    mx = fmaxf(mx, sc[ps]);
#pragma unroll
                for (int off = GK; off < kWave; off <<= 1)
                    mx = fmaxf(mx, xor_shfl(mx, off));  // max over the token slots of head j
                const float mn = fmaxf(m_own, mx);
                const float alpha = fast_exp2(m_own - mn);  // 0 on the first block
                m_own = mn;
                l_own *= alpha;
#pragma unroll
                for (int h = 0; h < GK; ++h) {
                    const float ah = __int_as_float(
                        __builtin_amdgcn_readlane(__float_as_int(alpha), h));  // lane h has head h
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[h][e] *= ah;
                }
            }

            // probabilities: own head, own tokens; to LDS as p[token][head]
#pragma unroll
            for (int ps = 0; ps < NPASS; ++ps) {
                const float pr = fast_exp2(sc[ps] - m_own);  // masked: exp2(-inf) = 0
                l_own += pr;
                p_lds[(ps * TPP + ts) * GK + j] = pr;
            }

            // P*V in the coalesced layout: lane (r, c) holds tokens ROWS*i + r, dims c*8..c*8+7
            if (!whole) {
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    const int tok = base + ROWS * i + r;
                    const bool ok = good_blk && tok >= t0 && tok < t1;
                    vv[i] = ok ? vv[i] : make_uint4(0, 0, 0, 0);  // masked rows may hold NaN bits
                }
            }
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                float pv[GK];
#pragma unroll
                for (int h4 = 0; h4 < GK; h4 += 4) {
                    const float4 t = *(const float4 *)(p_lds + (ROWS * i + r) * GK + h4);
                    pv[h4] = t.x;
                    pv[h4 + 1] = t.y;
                    pv[h4 + 2] = t.z;
                    pv[h4 + 3] = t.w;
                }
                const uint32_t w[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v0 = lo_f32<BF>(w[e]), v1 = hi_f32<BF>(w[e]);
#pragma unroll
                    for (int h = 0; h < GK; ++h) {
                        acc[h][2 * e] += pv[h] * v0;
                        acc[h][2 * e + 1] += pv[h] * v1;
                    }
                }
            }
        };

        uint4 ka[NCH], va[NCH], kn[NCH], vn[NCH];
        load(0, ka, va);
        for (int k = 0; k < nb; ++k) {
            if (k + 1 < nb)
                load(k + 1, kn, vn);
            consume(k, ka, va);
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                ka[i] = kn[i];
                va[i] = vn[i];
            }
        }
    }

    // totals: l of head j over its token slots; acc over the row classes (one m per head: no
    // rescaling needed)
#pragma unroll
    for (int off = GK; off < kWave; off <<= 1)
        l_own += xor_shfl(l_own, off);
#pragma unroll
    for (int h = 0; h < GK; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a = acc[h][e];
#pragma unroll
            for (int off = RL; off < kWave; off <<= 1)
                a += xor_shfl(a, off);
            acc[h][e] = a;
        }

#pragma unroll
    for (int h = 0; h < GK; ++h) {
        const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_own), h));
        const float lh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_own), h));
        if (lane < RL && qrow[h] >= 0) {
            const size_t row = (size_t)qrow[h];
            if (split) {
                const size_t sl = row * p.ws_slots + slot;
                float *wa = p.ws_acc + sl * D + lane * 8;
                *(float4 *)wa = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
                *(float4 *)(wa + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
                if (lane == 0)
                    *(float2 *)(p.ws_ml + sl * 2) = make_float2(mh, lh);
            } else {
                const float inv = lh > 0.0f ? 1.0f / lh : 0.0f;
                uint4 o;
                o.x = pack2<BF>(acc[h][0] * inv, acc[h][1] * inv);
                o.y = pack2<BF>(acc[h][2] * inv, acc[h][3] * inv);
                o.z = pack2<BF>(acc[h][4] * inv, acc[h][5] * inv);
                o.w = pack2<BF>(acc[h][6] * inv, acc[h][7] * inv);
                *(uint4 *)(p.out + row * D + lane * 8) = o;
            }
        }
    }
}

// Plain decode unit for a head group of GK: (sequence, kv head, subgroup, part).
template <bool BF, int D, int GK>
__global__ __launch_bounds__(64) void decode_gqa_kernel(DecodeParams p)
{
    const int unit = xcd_logical_id(blockIdx.x, gridDim.x);
    if (unit >= p.n_units)
        return;
    const int seq = unit % p.num_seqs;
    int rest = unit / p.num_seqs;
    const int part = rest % p.max_parts;
    rest /= p.max_parts;
    const int sub = rest % p.n_sub;
    const int kvh = rest / p.n_sub;
    const int L = min(max(p.seq_lens[seq], 0), p.max_seq_len);
    const int t0 = unit_start(p, seq, L) + part * p.part_tokens;
    if (p.split && t0 >= L)
        return;
    const int t1 = min(L, t0 + p.part_tokens);
    int qrow[GK];
#pragma unroll
    for (int h = 0; h < GK; ++h)
        qrow[h] = seq * p.num_q_heads + (kvh * p.n_sub + sub) * GK + h;
    gqa_unit<BF, D, GK>(p, qrow, p.block_tables + (size_t)seq * p.max_blocks, kvh, t0, t1,
                        p.slot_base + part, p.split != 0);
}

// Shared-prefix unit: (prefix group g, kv head, subgroup of GK (member, query head) pairs, part).
// The members of group g are sequences group_starts[g] .. group_starts[g+1]-1; they share the
// blocks of positions [0, seq_starts[first member]), read here once through the first member's
// table for all of them (openeuler.csdn.net "高并发 AI 服务的内存瓶颈", 机制 2: shared blocks are
// stored once). Pair v of the group is member v / G, query head kvh*G + v % G.
template <bool BF, int D, int GK>
__global__ __launch_bounds__(64) void decode_prefix_kernel(DecodeParams p)
{
    const int unit = xcd_logical_id(blockIdx.x, gridDim.x);
    if (unit >= p.n_units)
        return;
    int rest = unit;
    const int vsub = rest % p.n_vsub;
    rest /= p.n_vsub;
    const int kvh = rest % p.num_kv_heads;
    rest /= p.num_kv_heads;
    const int part = rest % p.max_parts;
    const int g = rest / p.max_parts;
    const int first = min(max(p.group_starts[g], 0), p.num_seqs);
    const int n_mem = min(max(p.group_starts[g + 1], first), p.num_seqs) - first;
    const int G = p.num_q_heads / p.num_kv_heads;
    const int v0 = vsub * GK;
    if (n_mem == 0 || v0 >= n_mem * G)
        return;
    const int L0 = min(max(p.seq_lens[first], 0), p.max_seq_len);
    const int prefix = min(max(p.seq_starts[first], 0), L0);
    const int t0 = part * p.part_tokens;
    if (t0 >= prefix)
        return;
    const int t1 = min(prefix, t0 + p.part_tokens);
    int qrow[GK];
#pragma unroll
    for (int h = 0; h < GK; ++h) {
        const int v = v0 + h;
        qrow[h] = v < n_mem * G ? (first + v / G) * p.num_q_heads + kvh * G + v % G : -1;
    }
    gqa_unit<BF, D, GK>(p, qrow, p.block_tables + (size_t)first * p.max_blocks, kvh, t0, t1, part,
                        true);
}

// One wave per (sequence, query head): rescale every part to the common maximum M,
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
template <bool BF, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p)
{
    constexpr int DPL = D / kWave;  // dims per lane
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int idx = blockIdx.x * 4 + wave;
    if (idx >= p.num_seqs * p.num_q_heads)
        return;
    const int seq = idx / p.num_q_heads;
    const int L = min(max(p.seq_lens[seq], 0), p.max_seq_len);
    const int start = unit_start(p, seq, L);
    // parts of this row: shared-prefix parts in slots [0, n_pre), own parts after pre_slots
    const int n_pre = p.pre_slots > 0 ? (start + p.part_tokens - 1) / p.part_tokens : 0;
    const int n_own = (L - start + p.part_tokens - 1) / p.part_tokens;
    const int np = n_pre + n_own;
    auto slot_of = [&](int jj) { return jj < n_pre ? jj : p.pre_slots + (jj - n_pre); };
    const float *ml = p.ws_ml + (size_t)idx * p.ws_slots * 2;
    const float *ac = p.ws_acc + (size_t)idx * p.ws_slots * D + lane * DPL;

    float M = -INFINITY;
    for (int jj = lane; jj < np; jj += kWave)
        M = fmaxf(M, ml[2 * slot_of(jj)]);
    M = wave_max(M);
    float W = 0.0f;
    for (int jj = lane; jj < np; jj += kWave)
        W += fast_exp2(ml[2 * slot_of(jj)] - M) * ml[2 * slot_of(jj) + 1];
    W = wave_sum(W);

    float o[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d)
        o[d] = 0.0f;
    for (int jj = 0; jj < np; ++jj) {
        const int sl = slot_of(jj);
        const float w = fast_exp2(ml[2 * sl] - M);
#pragma unroll
        for (int d = 0; d < DPL; ++d)
            o[d] += w * ac[(size_t)sl * D + d];
    }
    const float inv = W > 0.0f ? 1.0f / W : 0.0f;
    uint16_t *dst = p.out + (size_t)idx * D + lane * DPL;
    if constexpr (DPL == 2)
        *(uint32_t *)dst = pack2<BF>(o[0] * inv, o[1] * inv);
    else
        *dst = (uint16_t)to_word<BF>(o[0] * inv);
}

template <bool BF, bool F8, int D, int GK>
hipError_t launch_units(const DecodeParams &p, hipStream_t stream)
{
    const int grid = round_up8(p.n_units);
    if constexpr (GK >= 4 && !F8)
        hipLaunchKernelGGL((decode_gqa_kernel<BF, D, GK>), dim3(grid), dim3(kWave), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_partition_kernel<BF, F8, D, GK>), dim3(grid), dim3(kWave), 0,
                           stream, p);
    return hipGetLastError();
}

template <bool BF, bool F8, int D>
hipError_t launch_units_gk(int gk, const DecodeParams &p, hipStream_t stream)
{
    if constexpr (F8) {  // E4M3 caches: the per-row-class kernel for head groups up to 4
        switch (gk) {
        case 4: return launch_units<BF, true, D, 4>(p, stream);
        case 2: return launch_units<BF, true, D, 2>(p, stream);
        default: return launch_units<BF, true, D, 1>(p, stream);
        }
    } else {
        switch (gk) {
        case 8: return launch_units<BF, false, D, 8>(p, stream);
        case 4: return launch_units<BF, false, D, 4>(p, stream);
        case 2: return launch_units<BF, false, D, 2>(p, stream);
        default: return launch_units<BF, false, D, 1>(p, stream);
        }
    }
}

template <bool BF, bool F8, int D>
hipError_t run_decode(int gk, int gkp, const DecodeParams &p, const DecodeParams *pre,
                      hipStream_t stream)
{
    hipError_t e;
    if constexpr (!F8) {  // shared-prefix units exist for 16-bit caches only
        if (pre) {
            const int grid = round_up8(pre->n_units);
            if (gkp == 8)
                hipLaunchKernelGGL((decode_prefix_kernel<BF, D, 8>), dim3(grid), dim3(kWave), 0,
                                   stream, *pre);
            else
                hipLaunchKernelGGL((decode_prefix_kernel<BF, D, 4>), dim3(grid), dim3(kWave), 0,
                                   stream, *pre);
            if ((e = hipGetLastError()) != hipSuccess)
                return e;
        }
    }
    if ((e = launch_units_gk<BF, F8, D>(gk, p, stream)) != hipSuccess || !p.split)
        return e;
    const int rows = p.num_seqs * p.num_q_heads;
    hipLaunchKernelGGL((decode_merge_kernel<BF, D>), dim3((rows + 3) / 4), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

bool decode_supported(int32_t head_dim, int32_t group)
{
    return (head_dim == 64 || head_dim == 128) && group >= 1;
}

hipError_t launch_decode(const DecodeLaunch &d, hipStream_t stream)
{
    if (d.num_seqs == 0)
        return hipSuccess;
    const int group = d.num_q_heads / d.c.num_kv_heads;
    const int gk = group % 8 == 0 && !d.fp8 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
    const bool cascade = d.group_starts != nullptr && d.num_groups > 0;
    if (d.fp8 && cascade)
        return hipErrorInvalidValue;  // no shared-prefix kernel for E4M3 caches
    DecodeParams p = {};
    p.query = (const uint16_t *)d.query;
    p.k_cache = (const uint16_t *)d.k_cache;
    p.v_cache = (const uint16_t *)d.v_cache;
    p.block_tables = d.block_tables;
    p.seq_lens = d.seq_lens;
    p.out = (uint16_t *)d.out;
    p.ws_acc = d.ws_acc;
    p.ws_ml = d.ws_ml;
    p.max_blocks = d.max_blocks;
    p.num_seqs = d.num_seqs;
    p.num_kv_heads = d.c.num_kv_heads;
    p.num_q_heads = d.num_q_heads;
    p.num_blocks = d.c.num_blocks;
    p.max_seq_len = d.max_seq_len;
    p.scale_log2 = (float)((double)d.scale * (d.fp8 ? (double)d.k_scale : 1.0) * 1.4426950408889634);
    p.v_scale = d.fp8 ? d.v_scale : 1.0f;
    p.n_sub = group / gk;
    p.split = d.max_parts > 0 ? 1 : 0;
    p.part_tokens = p.split ? d.partition_size : ((d.max_seq_len + kBlock - 1) / kBlock) * kBlock;
    if (p.part_tokens < kBlock)
        p.part_tokens = kBlock;
    p.max_parts = p.split ? d.max_parts : 1;
    p.ws_slots = p.max_parts;

    DecodeParams pre;
    int gkp = 8;
    if (cascade) {
        // slots [0, pre_parts) of every row hold shared-prefix parts, the rest its own parts
        const int pre_parts = (d.max_prefix_len + d.partition_size - 1) / d.partition_size;
        p.seq_starts = d.seq_starts;
        p.pre_slots = pre_parts;
        p.slot_base = pre_parts;
        p.ws_slots = pre_parts + p.max_parts;
        pre = p;
        pre.group_starts = d.group_starts;
        pre.num_groups = d.num_groups;
        const int pairs = d.max_group_size * group;  // (member, query head) pairs per kv head
        gkp = pairs >= 8 ? 8 : 4;
        pre.n_vsub = (pairs + gkp - 1) / gkp;
        pre.max_parts = pre_parts;
        const int64_t pre_units = (int64_t)d.num_groups * pre_parts * d.c.num_kv_heads * pre.n_vsub;
        if (pre_units > 0x7ffffff0)
            return hipErrorInvalidValue;
        pre.n_units = (int32_t)pre_units;
    }
    const int64_t units = (int64_t)d.num_seqs * d.c.num_kv_heads * p.n_sub * p.max_parts;
    if (units > 0x7ffffff0)
        return hipErrorInvalidValue;
    p.n_units = (int32_t)units;
    const DecodeParams *pp = cascade ? &pre : nullptr;
    if (d.fp8) {
        if (d.c.bf16)
            return d.c.head_dim == 64 ? run_decode<true, true, 64>(gk, gkp, p, pp, stream)
                                      : run_decode<true, true, 128>(gk, gkp, p, pp, stream);
        return d.c.head_dim == 64 ? run_decode<false, true, 64>(gk, gkp, p, pp, stream)
                                  : run_decode<false, true, 128>(gk, gkp, p, pp, stream);
    }
    if (d.c.bf16)
        return d.c.head_dim == 64 ? run_decode<true, false, 64>(gk, gkp, p, pp, stream)
                                  : run_decode<true, false, 128>(gk, gkp, p, pp, stream);
    return d.c.head_dim == 64 ? run_decode<false, false, 64>(gk, gkp, p, pp, stream)
                              : run_decode<false, false, 128>(gk, gkp, p, pp, stream);
}

}  // namespace pa
