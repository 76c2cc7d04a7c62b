// decode.hip -- paged decode attention for gfx950 (HBM-bound): a vector-ALU kernel for groups of 1
// or 2 query heads per kv head, an MFMA kernel for larger GQA groups and for shared prefixes, and
// the split-K merge.
//
// What it computes: for each sequence s and query head h, softmax(scale * q K^T) V over positions
// 0..L-1 of kv head h / group (lecture 32 "LLM 在线推理两阶段" §3.1 formula and decode step, §3.4
// GQA groups), with position i read from block table[s][i / 16] at offset i % 16
// (openeuler.csdn.net "高并发 AI 服务的内存瓶颈", Attention 计算时的 Block 映射). Blocks are
// consumed one at a time with a running maximum and running sum of exponentials, and partial results
// are combined by rescaling to the common maximum (devpress.csdn.net/amd vLLM overview, §9 (4)
// online softmax; §3 (3) per-block accumulation over the block table).
//
// Vector-ALU kernel. Work unit: one workgroup of UW (4 or 8) wavefronts per (sequence, kv head,
// query-head subgroup, partition); wave w takes blocks w, w + UW, ... of the unit's range,
// and the waves' results are merged through LDS at the end (a unit then takes a quarter of the
// time, which shortens the tail of batches with few, uneven units). A (block, kv head) tile is
// 16 rows x D contiguous 16-bit words (4 KiB at D = 128). Lane l of the wave
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
// unnormalised accumulator, max and sum (log2 domain) to a workspace slot (the MFMA kernel first
// merges four consecutive parts in LDS and writes one slot for them); a merge kernel rescales the
// slots of each (sequence, head) to their common maximum and normalises.
//
// MFMA kernel (GQA groups of 3 or more, and shared prefixes): the query rows that read one
// (kv head, token range) are the 16 columns of v_mfma_f32_16x16x32; see mfma_unit below.
#include <math.h>

#include <mutex>

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
    int32_t ws_rows;      // (sequence, head) rows: num_seqs * num_q_heads
    int32_t wg_parts;     // MFMA kernel: parts merged per workgroup (1 or kMfmaWaves)
    int32_t slot_tokens;  // tokens of a row's own workspace slot: part_tokens * wg_parts
    int32_t pre_slot_tokens;  // tokens of a shared-prefix slot: partition_size * kMfmaWaves
    int32_t slot_base;    // first slot these units write
    int32_t pre_slots;    // slots [0, pre_slots) hold shared-prefix results (merge)
    int32_t n_vsub;       // prefix units: groups of GK (member, head) pairs per kv head
    // shared-prefix decode whose own ranges all fit one part (vector-ALU units): each own unit
    // folds its row's shared-prefix partials in and writes the output, and no merge kernel runs
    int32_t fused_finish;
    // Multi-token decode (mt_rows > 0, MFMA kernel): sequence s has q_len = cu_q[s+1] - cu_q[s]
    // (at most mt_rows) query rows, rows cu_q[s] .. of the [total_q][num_q_heads][D] query and
    // output; row r sits at position L - q_len + r and sees the positions before the rows, and row
    // j <= r of them when bit j of tree_mask[cu_q[s] + r] is set (every such j without a mask).
    // Workspace rows are (sequence, row, head): (s * mt_rows + r) * num_q_heads + head.
    const int32_t *__restrict__ cu_q;
    const uint64_t *__restrict__ tree_mask;
    int32_t mt_rows;
    int32_t total_q;
};

// Position range of unit `part` of a sequence: [start + part*P, min(L, start + (part+1)*P)).
__device__ __forceinline__ int unit_start(const DecodeParams &p, int seq, int L)
{
    return p.seq_starts ? min(max(p.seq_starts[seq], 0), L) : 0;
}

// Lazy reference point of the running softmax: a row's running maximum moves (and its sums are
// rescaled) only when a score passes it by more than 2^kLazy, so probabilities and partial sums
// stay below 2^8 times their true scale and most blocks skip the rescale.
constexpr float kLazy = 8.0f;  // log2 units

// Unit order. Units are numbered sequence fastest, then part (slot), then head subgroup and kv
// head (the slowest index, so that each XCD's contiguous share of the numbering holds whole kv
// heads). In a plain decode the parts of a sequence are taken in descending order: the units
// issued last are then every sequence's first part -- many units of the full part length -- and
// not the last parts that only the longest sequences have, which would leave most CUs idle while
// a few finish (32 sequences of 8K-32K tokens, 64 query / 8 kv heads: 431.8 → 422.9 µs; 64
// sequences of 512-4K tokens, 32 heads: 409.5 → 405.4-407.2 µs). Units that start at a
// per-sequence offset (the own tokens after a shared prefix, mostly under one part) keep the
// ascending order: descending would issue their many empty high parts first (256 sequences in
// groups of 8 sharing a 2040-token prompt: 383 → 388 µs).
__device__ __forceinline__ int unit_part(const DecodeParams &p, int r, int n)
{
    return p.seq_starts ? r : n - 1 - r;
}

// F8: the caches hold E4M3 codes (one byte per element) instead of 16-bit elements.
// UW: waves per unit of the vector-ALU kernel. Four suit units of up to 512 tokens: measured on
// the 7B-shaped layer (512-token parts) and on 256 sequences of U{1..512} tokens, 1 wave per unit
// (two units per workgroup) 76.7 % / 70.5 % of 8 TB/s, 2 waves 77.3 % / 74.3 %, 4 waves 77.5 % /
// 76.7 %. Eight suit 16-bit units of 1024 tokens or more -- each wave still streams eight blocks
// while the units, partials and merge work halve: 7B-shaped layer, 512-token parts with four waves
// 408.8-409.2 µs, 1024-token parts with eight 396.6-398.9 µs. E4M3 units keep four (eight lost,
// 66 %), and so do shared-prefix own ranges (eight: 388 → 419 µs).
constexpr int kUnitWavesMax = 8;

template <bool BF, bool F8, int D, int GK, int UW>
__global__ __launch_bounds__(64 * UW) void decode_partition_kernel(DecodeParams p)
{
    constexpr int kUnitWaves = UW;
    constexpr int EPL = F8 ? 16 : 8;     // cache elements per 16-byte piece = dims per lane
    constexpr int RL = D / EPL;          // lanes per token row
    constexpr int ROWS = kWave / RL;     // token rows per 1 KiB load
    constexpr int NCH = kBlock / ROWS;   // loads per (block, kv head) tile
    constexpr int QV = EPL / 8;          // 16-byte query pieces per lane and head
    constexpr int ESZ = F8 ? 1 : 2;      // bytes per cache element
    const int lane = threadIdx.x & (kWave - 1);
    const int r = lane / RL;
    const int w = threadIdx.x / kWave;  // this wave takes blocks w, w + kUnitWaves, ... of the unit

    const int unit = xcd_logical_id(blockIdx.x, gridDim.x);  // one unit per workgroup
    if (unit >= p.n_units)
        return;  // uniform over the workgroup
    const int seq = unit % p.num_seqs;
    int rest = unit / p.num_seqs;
    const int part = unit_part(p, rest % p.max_parts, p.max_parts);
    rest /= p.max_parts;
    const int sub = rest % p.n_sub;
    const int kvh = rest / p.n_sub;
    const int h0 = (kvh * p.n_sub + sub) * GK;  // first query head of this unit

    const int L = min(max(p.seq_lens[seq], 0), p.max_seq_len);
    const int t0 = unit_start(p, seq, L) + part * p.part_tokens;
    if (p.split && t0 >= L && !p.fused_finish)
        return;  // a part with no tokens: the merge never reads it (uniform)
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
                // the reference m moves only when some lane's scores pass it by more than
                // 2^kLazy (the first valid block always does: m starts at -inf)
                if (!__all(!(mx - m[h] > kLazy))) {
                    const float mn = fmaxf(m[h], mx);
                    const float alpha = fast_exp2(m[h] - (mn == -INFINITY ? 0.0f : mn));
                    l[h] *= alpha;
#pragma unroll
                    for (int j = 0; j < EPL; ++j)
                        acc[h][j] *= alpha;
                    m[h] = mn;
                }
                const float ms = m[h] == -INFINITY ? 0.0f : m[h];
                float psum = 0.0f;
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    pr[h][i] = fast_exp2(s[h][i] - ms);  // masked: exp2(-inf) = 0
                    psum += pr[h][i];
                }
                l[h] += psum;
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
        if (w < nb)
            load(w, ka, va);
        for (int k = w; k < nb; k += kUnitWaves) {
            if (k + kUnitWaves < nb)
                load(k + kUnitWaves, kn, vn);
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

    // merge the waves' results: waves 1.. publish theirs, wave 0 rescales to the common maximum
    __shared__ float xs[kUnitWaves - 1][GK][RL][EPL + 2];
    if (w > 0 && lane < RL) {
#pragma unroll
        for (int h = 0; h < GK; ++h) {
#pragma unroll
            for (int j = 0; j < EPL; ++j)
                xs[w - 1][h][lane][j] = acc[h][j];
            xs[w - 1][h][lane][EPL] = m[h];
            xs[w - 1][h][lane][EPL + 1] = l[h];
        }
    }
    __syncthreads();
    if (w > 0)
        return;
    if (lane < RL) {
#pragma unroll
        for (int h = 0; h < GK; ++h) {
            float M = m[h];
#pragma unroll
            for (int v = 0; v < kUnitWaves - 1; ++v)
                M = fmaxf(M, xs[v][h][lane][EPL]);
            const float Ms = M == -INFINITY ? 0.0f : M;
            const float f0 = fast_exp2(m[h] - Ms);
            float lh = l[h] * f0;
#pragma unroll
            for (int j = 0; j < EPL; ++j)
                acc[h][j] *= f0;
#pragma unroll
            for (int v = 0; v < kUnitWaves - 1; ++v) {
                const float fv = fast_exp2(xs[v][h][lane][EPL] - Ms);
                lh += xs[v][h][lane][EPL + 1] * fv;
#pragma unroll
                for (int j = 0; j < EPL; ++j)
                    acc[h][j] += xs[v][h][lane][j] * fv;
            }
            m[h] = M;
            l[h] = lh;
        }
    }

    if (lane < RL) {
#pragma unroll
        for (int h = 0; h < GK; ++h) {
            const size_t row = (size_t)seq * p.num_q_heads + h0 + h;
            if (p.fused_finish) {
                // the row's own tokens are this unit's range (its only part): fold in the row's
                // shared-prefix partials, written by the prefix kernel that ran before this one
                // on the stream, by rescaling to the common maximum, and write the output
                const int n_pre = min((t0 + p.pre_slot_tokens - 1) / p.pre_slot_tokens, p.pre_slots);
                const float *ml = p.ws_ml + row * p.ws_slots * 2;
                float M = m[h];
                for (int q = 0; q < n_pre; ++q)
                    M = fmaxf(M, ml[2 * q]);
                const float Ms = M == -INFINITY ? 0.0f : M;
                const float f0 = fast_exp2(m[h] - Ms);
                float W = l[h] * f0;
                float o[EPL];
#pragma unroll
                for (int j = 0; j < EPL; ++j)
                    o[j] = acc[h][j] * f0;
                for (int q = 0; q < n_pre; ++q) {
                    const float fq = fast_exp2(ml[2 * q] - Ms);
                    W += ml[2 * q + 1] * fq;
                    const float *wa = p.ws_acc + ((size_t)q * p.ws_rows + row) * D + lane * EPL;
#pragma unroll
                    for (int j = 0; j < EPL; j += 4) {
                        const float4 a = *(const float4 *)(wa + j);
                        o[j] += a.x * fq;
                        o[j + 1] += a.y * fq;
                        o[j + 2] += a.z * fq;
                        o[j + 3] += a.w * fq;
                    }
                }
                const float inv = W > 0.0f ? 1.0f / W : 0.0f;
#pragma unroll
                for (int j = 0; j < EPL; j += 8) {
                    uint4 ov;
                    ov.x = pack2<BF>(o[j] * inv, o[j + 1] * inv);
                    ov.y = pack2<BF>(o[j + 2] * inv, o[j + 3] * inv);
                    ov.z = pack2<BF>(o[j + 4] * inv, o[j + 5] * inv);
                    ov.w = pack2<BF>(o[j + 6] * inv, o[j + 7] * inv);
                    *(uint4 *)(p.out + row * D + lane * EPL + j) = ov;
                }
            } else if (p.split) {
                const size_t slot = row * p.ws_slots + p.slot_base + part;
                float *wa = p.ws_acc + ((size_t)(p.slot_base + part) * p.ws_rows + row) * D +
                            lane * EPL;
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

// ------------------------------------------------------------------ head groups on MFMA
// Up to 16 query rows that read one (kv head, token range) -- the query heads of a GQA group, or the
// (member, query head) pairs of a shared-prefix group -- are the 16 columns of
// v_mfma_f32_16x16x32_{f16,bf16}; a step covers two blocks (32 tokens):
//   S[t][j]  = sum_d K[t][d] Q[j][d]   A = K, 16 tokens x 32 dims, loaded from HBM straight into
//                                       the operand layout (lane l: token l % 16; plain loads, since
//                                       one instruction covers half of each 128-byte line and the
//                                       next the other half); B = Q in registers
//   O[d][j] += sum_t V[t][d] P[t][j]   A = V^T, 16 dims x 32 tokens, read from row-major V in LDS
//                                       with ds_read_b64_tr_b16; B = P, taken from the S accumulators
//                                       where it already sits in the operand layout.
// Lane l owns column j = l % 16 and row group g = l / 16: its S values are tokens 4g..4g+3 of each
// block, its O values dims 16c + 4g..4g+3 of each 16-dim tile c. The score scale and the running
// reference point are per column, kept equal across the 4 row groups; like the kernel above the
// reference moves only when a score passes it by more than 2^kLazy. Token order inside the PV
// contraction: operand slot 8g + e is token 4g + e of the first block (e < 4) or 4g + e - 4 of the
// second, for both operands. bf16 probabilities go in as a hi + lo pair (about 16 significant bits).
// E4M3 caches: K bytes are widened to 16-bit pairs in registers, V bytes on their way into LDS.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kCols = 16;  // query rows per MFMA unit

template <bool BF>
__device__ __forceinline__ f32x4 mfma16(const uint4 &a, const uint4 &b, const f32x4 &c)
{
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// First of the 8 dims that row group g holds in QK k-chunk c. 16-bit caches: chunk c is dims
// 32c..32c+31. E4M3 caches: a lane's 16-byte load holds 16 dims, the halves of which feed chunks
// 2c2 and 2c2+1 (any dim order serves, as long as K and Q agree).
template <bool F8>
__device__ __forceinline__ int qk_dim(int c, int g)
{
    return F8 ? 16 * (g + 4 * (c >> 1)) + 8 * (c & 1) : 32 * c + 8 * g;
}

// XOR swizzle of the 16-byte pieces of V row r in LDS (rows of D 16-bit elements). A transposed
// read serves 32 lanes a cycle: 8 consecutive rows at 2 adjacent pieces, which must fall on
// distinct 16-byte bank groups (64 four-byte banks, one 256-byte line per D = 128 row; two rows per
// line for D = 64). For D = 128, 2 (r & 7) + (r >> 3 & 1) does that; r & 15 sent rows r and r + 1
// to the same pieces (2-way conflicts; measured neutral in time, the kernel waits on HBM).
template <int D>
__device__ __forceinline__ int vswz(int r)
{
    return D == 128 ? ((r & 7) << 1) | ((r >> 3) & 1) : (r & 7);
}

// Bytes of LDS one MFMA unit stages V through: two blocks of 16 rows of D 16-bit elements.
template <int D>
constexpr int kUnitLds = 2 * kBlock * D * 2;

// Orders this wave's LDS accesses on either side of it for the compiler. The LDS unit performs one
// wave's accesses in program order, so lanes reading what other lanes of the same wave wrote need
// no s_barrier: the V staging below is private to its wave.
__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Attention of the query rows in one wave's 16 MFMA columns over tokens [t0, t1) of kv head kvh.
// On return o holds the unnormalised accumulator (lane (j, g): column j, dims 16t + 4g .. +3 of
// tile t), m the running maximum of column j (log2 domain) and l this lane's share of column j's
// running sum (the four row groups g add up to it). v_lds is the wave's own staging area
// (kUnitLds<D> bytes). An empty range leaves o = 0, m = -inf, l = 0.
// NCG column groups of 16 (query rows qrow[cg]) share every K operand and every transposed V
// read: a unit of NCG groups reads the context once for 16 * NCG rows.
// MT (multi-token rows): positions from c0 on are the query rows' own; column j of group cg sees
// position c0 + i only when bit i of its vis[cg] is set (none from c0 + 32 on).
template <bool BF, bool F8, int D, bool MT, int NCG>
__device__ __forceinline__ void mfma_unit_cols(const DecodeParams &p, const int (&qrow)[NCG],
                                               const int32_t *table, int kvh, int t0, int t1,
                                               uint8_t *v_lds, f32x4 (&o)[NCG][D / 16],
                                               float (&m)[NCG], float (&l)[NCG], int c0,
                                               const uint32_t (&vis)[NCG])
{
    constexpr int NC = D / 32;              // QK k-chunks
    constexpr int NT = D / 16;              // PV output tiles
    constexpr int ESZ = F8 ? 1 : 2;
    constexpr int TILE = kBlock * D * ESZ;  // bytes of a (block, kv head) tile
    constexpr int NV = TILE / 1024;         // 1 KiB V loads per block
    constexpr int KL = F8 ? NC / 2 : NC;    // 16-byte K loads per lane per block
    constexpr int ROWB = D * 2;             // bytes of a 16-bit V row in LDS

    const int lane = threadIdx.x & (kWave - 1);
    const int j = lane & 15, g = lane >> 4;

    uint4 q[NCG][NC];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
            q[cg][c] = qrow[cg] >= 0
                           ? *(const uint4 *)(p.query + (size_t)qrow[cg] * D + qk_dim<F8>(c, g))
                           : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            o[cg][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        m[cg] = -INFINITY;
        l[cg] = 0.0f;
    }

    const uint8_t *kbase = (const uint8_t *)p.k_cache + (size_t)kvh * TILE;
    const uint8_t *vbase = (const uint8_t *)p.v_cache + (size_t)kvh * TILE;
    const size_t block_stride = (size_t)p.num_kv_heads * TILE;

    // transposed-read addresses: source lane s = 4k + qd of a row group points at row 4g + k (first
    // block; + 16 for the second), dims 16c + 4qd .. +3
    const int tr_k = (lane & 15) >> 2, tr_q = lane & 3;

    for (int bb = t0 / kBlock; bb * kBlock < t1; bb += kWave) {
        const int nb = min(kWave, (t1 - bb * kBlock + kBlock - 1) / kBlock);
        const int my_blk = lane < nb ? table[bb + lane] : 0;
        const int nsteps = (nb + 1) / 2;

        auto blk_of = [&](int k) {  // block id of the window's k-th block (k < nb), 0 if bad
            const int blk = __builtin_amdgcn_readlane(my_blk, k);
            return (unsigned)blk < (unsigned)p.num_blocks ? blk : 0;
        };
        // a second block past the window's end (odd nb) is not loaded: its operands are zero
        auto load_k = [&](int st, uint4(&kk)[2][KL]) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int k = 2 * st + b;
                if (k < nb) {
                    const uint8_t *kt = kbase + (size_t)blk_of(k) * block_stride;
#pragma unroll
                    for (int c = 0; c < KL; ++c)  // plain loads: each covers half lines
                        kk[b][c] = F8 ? *(const uint4 *)(kt + j * D + 16 * (g + 4 * c))
                                      : *(const uint4 *)(kt + (j * D + 32 * c + 8 * g) * 2);
                } else {
#pragma unroll
                    for (int c = 0; c < KL; ++c)
                        kk[b][c] = make_uint4(0, 0, 0, 0);
                }
            }
        };
        auto load_v = [&](int st, uint4(&vv)[2][NV]) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int k = 2 * st + b;
                if (k < nb) {
                    const uint8_t *vt = vbase + (size_t)blk_of(k) * block_stride;
#pragma unroll
                    for (int i = 0; i < NV; ++i)
                        vv[b][i] = load_nt(vt + 1024 * i + 16 * lane);
                } else {
#pragma unroll
                    for (int i = 0; i < NV; ++i)
                        vv[b][i] = make_uint4(0, 0, 0, 0);
                }
            }
        };

        // validity of the step's 32 tokens: block ids in the pool and positions in [t0, t1)
        auto tok_ok = [&](int st, int b, int r) {
            const int k = 2 * st + b;
            const int raw = __builtin_amdgcn_readlane(my_blk, k < nb ? k : 0);
            const int tok = (bb + k) * kBlock + r;
            return k < nb && (unsigned)raw < (unsigned)p.num_blocks && tok >= t0 && tok < t1;
        };
        auto whole_step = [&](int st) {
            bool w = 2 * st + 1 < nb && (bb + 2 * st) * kBlock >= t0 &&
                     (bb + 2 * st + 2) * kBlock <= (MT ? min(t1, c0) : t1);
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int raw = __builtin_amdgcn_readlane(my_blk, w ? 2 * st + b : 0);
                w = w && (unsigned)raw < (unsigned)p.num_blocks;
            }
            return w;
        };

        // V of a step into LDS as 16-bit rows 0..31 (masked rows zeroed: they may hold any bits)
        auto stage = [&](int st, bool whole, const uint4(&vv)[2][NV]) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    const int byte = 1024 * i + 16 * lane;       // in the tile
                    const int r = byte / (D * ESZ);               // row in the block
                    const int e0 = (byte % (D * ESZ)) / ESZ;      // first element
                    uint4 x = vv[b][i];
                    if (!whole && !tok_ok(st, b, r))
                        x = make_uint4(0, 0, 0, 0);
                    const int R = kBlock * b + r;
                    uint8_t *row = v_lds + R * ROWB;
                    if constexpr (F8) {
                        const uint4 lo = make_uint4(e4m3x2_to_pk16<BF, false>(x.x),
                                                    e4m3x2_to_pk16<BF, true>(x.x),
                                                    e4m3x2_to_pk16<BF, false>(x.y),
                                                    e4m3x2_to_pk16<BF, true>(x.y));
                        const uint4 hi = make_uint4(e4m3x2_to_pk16<BF, false>(x.z),
                                                    e4m3x2_to_pk16<BF, true>(x.z),
                                                    e4m3x2_to_pk16<BF, false>(x.w),
                                                    e4m3x2_to_pk16<BF, true>(x.w));
                        const int pc = e0 / 8;
                        *(uint4 *)(row + ((pc ^ vswz<D>(R)) << 4)) = lo;
                        *(uint4 *)(row + (((pc + 1) ^ vswz<D>(R)) << 4)) = hi;
                    } else {
                        *(uint4 *)(row + (((e0 / 8) ^ vswz<D>(R)) << 4)) = x;
                    }
                }
        };

        auto scores = [&](int st, bool whole, const uint4(&kk)[2][KL], float(&sv)[NCG][8]) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                f32x4 acc[NCG];
#pragma unroll
                for (int cg = 0; cg < NCG; ++cg)
                    acc[cg] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    uint4 a;
                    if constexpr (F8) {
                        const uint4 &raw = kk[b][c >> 1];
                        const uint32_t w0 = (c & 1) ? raw.z : raw.x;
                        const uint32_t w1 = (c & 1) ? raw.w : raw.y;
                        a = make_uint4(e4m3x2_to_pk16<BF, false>(w0), e4m3x2_to_pk16<BF, true>(w0),
                                       e4m3x2_to_pk16<BF, false>(w1), e4m3x2_to_pk16<BF, true>(w1));
                    } else {
                        a = kk[b][c];
                    }
#pragma unroll
                    for (int cg = 0; cg < NCG; ++cg)
                        acc[cg] = mfma16<BF>(a, q[cg][c], acc[cg]);
                }
#pragma unroll
                for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float x = acc[cg][v] * p.scale_log2;
                        if (!whole) {
                            bool ok = tok_ok(st, b, 4 * g + v);
                            if constexpr (MT) {
                                const int tok = (bb + 2 * st + b) * kBlock + 4 * g + v;
                                if (ok && tok >= c0)
                                    ok = tok - c0 < 32 && ((vis[cg] >> (tok - c0)) & 1u);
                            }
                            if (!ok)
                                x = -INFINITY;
                        }
                        sv[cg][4 * b + v] = x;
                    }
            }
        };

        auto accumulate = [&](const float(&sv)[NCG][8]) {
            uint4 pb[NCG], pl[NCG];
#pragma unroll
            for (int cg = 0; cg < NCG; ++cg) {
                float over = sv[cg][0] - m[cg];
#pragma unroll
                for (int e = 1; e < 8; ++e)
                    over = fmaxf(over, sv[cg][e] - m[cg]);
                if (!__all(!(over > kLazy))) {
                    float mx = sv[cg][0];
#pragma unroll
                    for (int e = 1; e < 8; ++e)
                        mx = fmaxf(mx, sv[cg][e]);
                    mx = fmaxf(mx, xor_shfl(mx, 16));
                    mx = fmaxf(mx, xor_shfl(mx, 32));  // column max over the 4 row groups
                    if (mx > m[cg]) {
                        const float alpha = fast_exp2(m[cg] - mx);  // 0 while m = -inf
                        l[cg] *= alpha;
#pragma unroll
                        for (int t = 0; t < NT; ++t)
                            o[cg][t] *= alpha;
                        m[cg] = mx;
                    }
                }
                const float ms = m[cg] == -INFINITY ? 0.0f : m[cg];
                float pr[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pr[e] = fast_exp2(sv[cg][e] - ms);  // masked: exp2(-inf) = 0
                    l[cg] += pr[e];
                }
                uint32_t *hw = &pb[cg].x, *lw = &pl[cg].x;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hw[e] = pack2<BF>(pr[2 * e], pr[2 * e + 1]);
                    if constexpr (BF)
                        lw[e] = pack2<BF>(pr[2 * e] - lo_f32<BF>(hw[e]),
                                          pr[2 * e + 1] - hi_f32<BF>(hw[e]));
                }
            }

#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int pc = 2 * t + (tr_q >> 1), half = (tr_q & 1) * 8;
                const int r1 = 4 * g + tr_k, r2 = r1 + kBlock;
                const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16 *)(v_lds + r1 * ROWB + ((pc ^ vswz<D>(r1)) << 4) + half));
                const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16 *)(v_lds + r2 * ROWB + ((pc ^ vswz<D>(r2)) << 4) + half));
                const uint4 a = make_uint4(__builtin_bit_cast(uint2, lo4).x,
                                           __builtin_bit_cast(uint2, lo4).y,
                                           __builtin_bit_cast(uint2, hi4).x,
                                           __builtin_bit_cast(uint2, hi4).y);
#pragma unroll
                for (int cg = 0; cg < NCG; ++cg) {
                    o[cg][t] = mfma16<BF>(a, pb[cg], o[cg][t]);
                    if constexpr (BF)
                        o[cg][t] = mfma16<BF>(a, pl[cg], o[cg][t]);
                }
            }
        };

        // One set of operand registers: V of step st+1 is loaded as soon as V of step st sits in
        // LDS, K of step st+1 as soon as the scores of step st are out; both then stream in while
        // the rest of step st runs.
        uint4 ka[2][KL], va[2][NV];
        load_k(0, ka);
        load_v(0, va);
        for (int st = 0; st < nsteps; ++st) {
            const bool whole = whole_step(st);
            wave_lds_fence();  // after the previous step's transposed reads
            stage(st, whole, va);
            if (st + 1 < nsteps)
                load_v(st + 1, va);
            wave_lds_fence();
            float sv[NCG][8];
            scores(st, whole, ka, sv);
            if (st + 1 < nsteps)
                load_k(st + 1, ka);
            accumulate(sv);
        }
    }

}

// One column group of query rows, no multi-token view: the plain and shared-prefix decodes.
template <bool BF, bool F8, int D>
__device__ __forceinline__ void mfma_unit(const DecodeParams &p, int qrow, const int32_t *table,
                                          int kvh, int t0, int t1, uint8_t *v_lds,
                                          f32x4 (&o)[D / 16], float &m, float &l)
{
    const int qr[1] = {qrow};
    const uint32_t vis[1] = {0u};
    f32x4 oo[1][D / 16];
    float mm[1], ll[1];
    mfma_unit_cols<BF, F8, D, false, 1>(p, qr, table, kvh, t0, t1, v_lds, oo, mm, ll, 0, vis);
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
        o[t] = oo[0][t];
    m = mm[0];
    l = ll[0];
}

// Column sums of the four row groups' running sums (every lane of column j gets column j's).
__device__ __forceinline__ float column_sum(float l)
{
    l += xor_shfl(l, 16);
    return l + xor_shfl(l, 32);
}

// Partial result of query row qrow into workspace slot `slot`: the accumulator times v_scale, the
// maximum m and the column sum lsum.
template <bool F8, int D>
__device__ __forceinline__ void mfma_write_partial(const DecodeParams &p, int qrow, int slot,
                                                   const f32x4 (&o)[D / 16], float m, float lsum)
{
    if (qrow < 0)
        return;
    const int g = (threadIdx.x & (kWave - 1)) >> 4;
    const float vs = F8 ? p.v_scale : 1.0f;
    float *wa = p.ws_acc + ((size_t)slot * p.ws_rows + qrow) * D + 4 * g;
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
        *(float4 *)(wa + 16 * t) = make_float4(o[t][0] * vs, o[t][1] * vs, o[t][2] * vs,
                                               o[t][3] * vs);
    if (g == 0)
        *(float2 *)(p.ws_ml + ((size_t)qrow * p.ws_slots + slot) * 2) = make_float2(m, lsum);
}

// Normalised output of query row qrow (a range that is the whole context).
template <bool BF, bool F8, int D>
__device__ __forceinline__ void mfma_write_output(const DecodeParams &p, int qrow,
                                                  const f32x4 (&o)[D / 16], float lsum)
{
    if (qrow < 0)
        return;
    const int g = (threadIdx.x & (kWave - 1)) >> 4;
    const float inv = lsum > 0.0f ? (F8 ? p.v_scale : 1.0f) / lsum : 0.0f;
    uint16_t *dst = p.out + (size_t)qrow * D + 4 * g;
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
        *(uint2 *)(dst + 16 * t) = make_uint2(pack2<BF>(o[t][0] * inv, o[t][1] * inv),
                                              pack2<BF>(o[t][2] * inv, o[t][3] * inv));
}

constexpr int kMfmaWaves = kDecodeMfmaWaves;  // MFMA units (waves) per workgroup

// LDS of a workgroup of kMfmaWaves MFMA units: each wave's V staging area, reused by the merge.
template <int D>
struct MfmaLds {
    uint8_t stage[kMfmaWaves * kUnitLds<D>];
    float2 ml[kMfmaWaves][kWave];
};

// Merge the (m, l, acc) results of the workgroup's kMfmaWaves waves (tokens of disjoint ranges of
// the same query rows) by rescaling to their common maximum, and write the result as one partial
// to workspace slot `slot`. Every wave of the workgroup must call it (it holds two barriers); wave w
// combines output tiles w, w + kMfmaWaves, ... A wave with an empty range contributes m = -inf.
template <bool F8, int D>
__device__ __forceinline__ void mfma_workgroup_merge(const DecodeParams &p, int qrow, int slot,
                                                     const f32x4 (&o)[D / 16], float m, float lsum,
                                                     MfmaLds<D> &sm)
{
    constexpr int NT = D / 16;
    static_assert(kMfmaWaves * NT * kWave * 16 <= (int)sizeof(sm.stage), "merge buffer");
    const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    __syncthreads();  // every wave is done with its V staging
    f32x4 *ox = (f32x4 *)sm.stage;  // [wave][tile][lane]
#pragma unroll
    for (int t = 0; t < NT; ++t)
        ox[(w * NT + t) * kWave + lane] = o[t];
    sm.ml[w][lane] = make_float2(m, lsum);
    __syncthreads();
    float2 mls[kMfmaWaves];
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kMfmaWaves; ++v) {
        mls[v] = sm.ml[v][lane];
        M = fmaxf(M, mls[v].x);
    }
    float a[kMfmaWaves], lm = 0.0f;
#pragma unroll
    for (int v = 0; v < kMfmaWaves; ++v) {
        a[v] = mls[v].x == -INFINITY ? 0.0f : fast_exp2(mls[v].x - M);
        lm += a[v] * mls[v].y;
    }
    if (qrow < 0)
        return;
    const int g = lane >> 4;
    const float vs = F8 ? p.v_scale : 1.0f;
    float *wa = p.ws_acc + ((size_t)slot * p.ws_rows + qrow) * D + 4 * g;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t % kMfmaWaves != w)
            continue;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int v = 0; v < kMfmaWaves; ++v)
            acc += a[v] * ox[(v * NT + t) * kWave + lane];
        *(float4 *)(wa + 16 * t) = make_float4(acc[0] * vs, acc[1] * vs, acc[2] * vs, acc[3] * vs);
    }
    if (w == 0 && g == 0)
        *(float2 *)(p.ws_ml + ((size_t)qrow * p.ws_slots + slot) * 2) = make_float2(M, lm);
}

// Wave w's share [t0, t1) of a slot's tokens [s0, s1): the slot split evenly over the kMfmaWaves
// waves in 32-token steps. A sequence's last slot is usually partial, and fixed parts would leave
// waves idle beside one full part (the mixed step's decode, G = 4: 541 -> 537 us; over E4M3
// caches 300 -> 293-296 us).
__device__ __forceinline__ void wave_share(int s0, int s1, int w, int &t0, int &t1)
{
    const int chunk = ((s1 - s0 + kMfmaWaves - 1) / kMfmaWaves + 31) & ~31;
    t0 = min(s1, s0 + w * chunk);
    t1 = min(s1, t0 + chunk);
}

// Plain decode of head groups of 3 or more. A workgroup is kMfmaWaves waves, at most three per SIMD
// (at most 168 registers): each unit holds one step of K and V operands in flight, so the number
// of resident waves sets the bytes in flight per CU.
//  * Split (p.wg_parts == kMfmaWaves): workgroup (sequence, slot q, subgroup of 16 query heads,
//    kv head); wave w computes the w-th quarter of slot q's tokens on its own, then the
//    workgroup merges its parts through LDS by rescaling to their common maximum (the same
//    log-sum-exp merge as the merge kernel's) and writes one partial result per row to slot q. Every part's partial would
//    otherwise be an fp32 write of D floats per query head, and at G = 8 those writes cost several
//    times their share of the HBM traffic.
//  * Otherwise (p.wg_parts == 1): the waves are independent units (sequence, part, subgroup, kv
//    head) that write their own partial result, or the output when the decode is not split.

template <bool BF, bool F8, int D>
__global__ __launch_bounds__(kWave * kMfmaWaves) __attribute__((amdgpu_waves_per_eu(3))) void
decode_mfma_kernel(DecodeParams p)
{
    constexpr int NT = D / 16;
    __shared__ __align__(16) MfmaLds<D> sm;
    const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const bool merged = p.wg_parts == kMfmaWaves;
    const int unit = merged ? wg : wg * kMfmaWaves + w;
    if (unit >= p.n_units)
        return;  // uniform over the workgroup in the merged mode
    const int seq = unit % p.num_seqs;
    int rest = unit / p.num_seqs;
    const int n_slot = merged ? p.ws_slots - p.slot_base : p.max_parts;  // slots (parts) per row
    const int q = unit_part(p, rest % n_slot, n_slot);
    rest /= n_slot;
    const int sub = rest % p.n_sub;
    const int kvh = rest / p.n_sub;
    const int L = min(max(p.seq_lens[seq], 0), p.max_seq_len);
    const int start = unit_start(p, seq, L);
    const int part = merged ? q * kMfmaWaves + w : q;
    if (p.split && start + q * p.slot_tokens >= L)
        return;  // the slot holds no tokens (uniform over the workgroup in the merged mode)
    int t0, t1;
    if (merged) {
        const int s0 = start + q * p.slot_tokens;
        wave_share(s0, min(L, s0 + p.slot_tokens), w, t0, t1);
    } else {
        t0 = min(L, start + part * p.part_tokens);
        t1 = min(L, t0 + p.part_tokens);
    }
    const int G = p.num_q_heads / p.num_kv_heads;
    const int h = sub * kCols + (lane & 15);
    const int qrow = h < G ? seq * p.num_q_heads + kvh * G + h : -1;
    f32x4 o[NT];
    float m, l;
    mfma_unit<BF, F8, D>(p, qrow, p.block_tables + (size_t)seq * p.max_blocks, kvh, t0, t1,
                         sm.stage + w * kUnitLds<D>, o, m, l);
    const float lsum = column_sum(l);
    if (!p.split) {
        mfma_write_output<BF, F8, D>(p, qrow, o, lsum);
        return;
    }
    if (!merged) {
        mfma_write_partial<F8, D>(p, qrow, p.slot_base + part, o, m, lsum);
        return;
    }
    mfma_workgroup_merge<F8, D>(p, qrow, p.slot_base + q, o, m, lsum, sm);
}

// Multi-token decode (p.mt_rows > 0): the MFMA units of decode_mfma_kernel, whose columns are the
// (row, query head) pairs of a kv head, row-major (pair v: row v / G, query head kvh * G + v % G),
// in NCG groups of 16 per wave that share the wave's K and V reads. Workgroups are numbered with
// the subgroups of 16 * NCG pairs fastest, so that the subgroups reading one (sequence, slot,
// kv head) run side by side on one XCD, where the later ones find part of the context in its L2.
// Each column carries its row's view of the rows' own positions (mfma_unit_cols' c0 and vis);
// workspace rows are (sequence, row, head). Two groups take up to 252 registers: two waves per
// SIMD instead of three.
template <bool BF, bool F8, int D, int NCG>
__global__ __launch_bounds__(kWave * kMfmaWaves) __attribute__((amdgpu_waves_per_eu(4 - NCG))) void
decode_multi_kernel(DecodeParams p)
{
    constexpr int NT = D / 16;
    __shared__ __align__(16) MfmaLds<D> sm;
    const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
    const bool merged = p.wg_parts == kMfmaWaves;
    const int unit = merged ? wg : wg * kMfmaWaves + w;
    if (unit >= p.n_units)
        return;  // uniform over the workgroup in the merged mode
    int rest = unit;
    const int sub = rest % p.n_sub;
    rest /= p.n_sub;
    const int seq = rest % p.num_seqs;
    rest /= p.num_seqs;
    const int n_slot = merged ? p.ws_slots : p.max_parts;  // slots (parts) per row
    const int q = unit_part(p, rest % n_slot, n_slot);
    const int kvh = rest / n_slot;
    const int L = min(max(p.seq_lens[seq], 0), p.max_seq_len);
    const int part = merged ? q * kMfmaWaves + w : q;
    if (p.split && q * p.slot_tokens >= L)
        return;  // the slot holds no tokens (uniform over the workgroup in the merged mode)
    int t0, t1;
    if (merged) {
        wave_share(q * p.slot_tokens, min(L, (q + 1) * p.slot_tokens), w, t0, t1);
    } else {
        t0 = min(L, part * p.part_tokens);
        t1 = min(L, t0 + p.part_tokens);
    }
    const int G = p.num_q_heads / p.num_kv_heads;
    // offsets are clamped to [0, total_q] so that no index contents reach outside the arrays; no
    // cu_q: one row per sequence (a plain decode of a head group above kCols)
    const int q0 = p.cu_q ? min(max(p.cu_q[seq], 0), p.total_q) : seq;
    const int q_len = p.cu_q ? min(max(p.cu_q[seq + 1], q0), p.total_q) - q0 : 1;
    const int rows = min(q_len, p.mt_rows);
    if (sub * kCols * NCG >= rows * G)
        return;  // no row of this subgroup (uniform over the workgroup in the merged mode)
    const int c0 = L - q_len;  // position of row 0
    int qrow[NCG], wrow[NCG];  // query / output row and workspace row of each column (-1: none)
    uint32_t vis[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
        const int v = (sub * NCG + cg) * kCols + (lane & 15), r = v / G;
        const bool ok = r < rows;
        const int head = kvh * G + v % G;
        qrow[cg] = ok ? (q0 + r) * p.num_q_heads + head : -1;
        wrow[cg] = ok ? (seq * p.mt_rows + r) * p.num_q_heads + head : -1;
        vis[cg] = ok ? (2u << r) - 1u : 0u;  // rows 0..r (r < mt_rows <= 16)
        if (ok && p.tree_mask)
            vis[cg] &= (uint32_t)p.tree_mask[q0 + r];
    }
    f32x4 o[NCG][NT];
    float m[NCG], l[NCG];
    mfma_unit_cols<BF, F8, D, true, NCG>(p, qrow, p.block_tables + (size_t)seq * p.max_blocks, kvh,
                                         t0, t1, sm.stage + w * kUnitLds<D>, o, m, l, c0, vis);
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
        const float lsum = column_sum(l[cg]);
        if (!p.split)
            mfma_write_output<BF, F8, D>(p, qrow[cg], o[cg], lsum);
        else if (!merged)
            mfma_write_partial<F8, D>(p, wrow[cg], part, o[cg], m[cg], lsum);
        else
            mfma_workgroup_merge<F8, D>(p, wrow[cg], q, o[cg], m[cg], lsum, sm);  // every wave
    }
}

// Shared-prefix units: workgroup (prefix group g, kv head, subgroup of 16 (member, query head)
// pairs, prefix slot q); wave w takes its share of slot q's prefix tokens (wave_share) and the
// workgroup merges its parts into slot q as decode_mfma_kernel does. The members of group g are sequences
// group_starts[g] .. group_starts[g+1]-1; they share the blocks of positions
// [0, seq_starts[first member]), read here once through the first member's table for all of them
// (openeuler.csdn.net "高并发 AI 服务的内存瓶颈", 机制 2: shared blocks are stored once). Pair v of
// the group is member v / G, query head kvh*G + v % G.
template <bool BF, bool F8, int D>
__global__ __launch_bounds__(kWave * kMfmaWaves) __attribute__((amdgpu_waves_per_eu(3))) void
decode_prefix_mfma_kernel(DecodeParams p)
{
    __shared__ __align__(16) MfmaLds<D> sm;
    const int w = threadIdx.x / kWave;
    const int unit = xcd_logical_id(blockIdx.x, gridDim.x);
    if (unit >= p.n_units)
        return;  // uniform over the workgroup
    int rest = unit;
    const int vsub = rest % p.n_vsub;
    rest /= p.n_vsub;
    const int kvh = rest % p.num_kv_heads;
    rest /= p.num_kv_heads;
    const int q = rest % p.pre_slots;
    const int grp = rest / p.pre_slots;
    const int first = min(max(p.group_starts[grp], 0), p.num_seqs);
    const int n_mem = min(max(p.group_starts[grp + 1], first), p.num_seqs) - first;
    const int G = p.num_q_heads / p.num_kv_heads;
    if (n_mem == 0 || vsub * kCols >= n_mem * G)
        return;  // uniform
    const int L0 = min(max(p.seq_lens[first], 0), p.max_seq_len);
    const int prefix = min(max(p.seq_starts[first], 0), L0);
    if (q * p.pre_slot_tokens >= prefix)
        return;  // uniform: the slot holds no prefix tokens
    int t0, t1;
    wave_share(q * p.pre_slot_tokens, min(prefix, (q + 1) * p.pre_slot_tokens), w, t0, t1);
    const int v = vsub * kCols + (threadIdx.x & 15);
    const int qrow = v < n_mem * G ? (first + v / G) * p.num_q_heads + kvh * G + v % G : -1;
    f32x4 o[D / 16];
    float m, l;
    mfma_unit<BF, F8, D>(p, qrow, p.block_tables + (size_t)first * p.max_blocks, kvh, t0, t1,
                         sm.stage + w * kUnitLds<D>, o, m, l);
    mfma_workgroup_merge<F8, D>(p, qrow, q, o, m, column_sum(l), sm);
}

// One wave per (sequence, query head): rescale every part to the common maximum M,
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
// A part's accumulator is read as LPP lanes x 4 floats, so one load instruction covers PPI parts
// (lane group g takes part j + g); U instructions are in flight per wave. The weights of 64 parts
// at a time sit one per lane and are broadcast with readlane.
template <bool BF, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p)
{
    constexpr int LPP = D / 4;          // lanes per part
    constexpr int PPI = kWave / LPP;    // parts per load instruction
    constexpr int U = 8;                // load instructions in flight
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int grp = lane / LPP, sub = lane % LPP;
    const int idx = blockIdx.x * 4 + wave;  // workspace row
    if (idx >= p.ws_rows)
        return;
    int seq, orow;  // sequence and output row
    if (p.mt_rows > 0) {  // workspace rows (sequence, row, head) of a multi-token decode
        const int per_seq = p.mt_rows * p.num_q_heads;
        seq = idx / per_seq;
        const int r = idx % per_seq / p.num_q_heads;
        const int q0 = p.cu_q ? min(max(p.cu_q[seq], 0), p.total_q) : seq;
        const int q_len = p.cu_q ? min(max(p.cu_q[seq + 1], q0), p.total_q) - q0 : 1;
        if (r >= min(q_len, p.mt_rows))
            return;
        orow = (q0 + r) * p.num_q_heads + idx % p.num_q_heads;
    } else {
        seq = idx / p.num_q_heads;
        orow = idx;
    }
    const int L = min(max(p.seq_lens[seq], 0), p.max_seq_len);
    const int start = unit_start(p, seq, L);
    // parts of this row: shared-prefix parts in slots [0, n_pre), own parts after pre_slots.
    // Both counts are clamped to the slots the workspace has, so that prefix lengths breaking the
    // caller's contract (unequal within a group, above max_prefix_len) give unspecified output but
    // never a read outside the workspace.
    const int n_pre = p.pre_slots > 0
                          ? min((start + p.pre_slot_tokens - 1) / p.pre_slot_tokens, p.pre_slots)
                          : 0;
    const int n_own = min((L - start + p.slot_tokens - 1) / p.slot_tokens, p.ws_slots - p.pre_slots);
    const int np = n_pre + n_own;
    auto slot_of = [&](int jj) { return jj < n_pre ? jj : p.pre_slots + (jj - n_pre); };
    const float *ml = p.ws_ml + (size_t)idx * p.ws_slots * 2;
    const float *ac = p.ws_acc + (size_t)idx * D + sub * 4;  // + slot * ws_rows * D

    float M = -INFINITY;
    for (int jj = lane; jj < np; jj += kWave)
        M = fmaxf(M, ml[2 * slot_of(jj)]);
    M = wave_max(M);
    // a row that sees no position (every part at -inf, possible under a multi-token tree mask)
    // gets weights exp2(-inf) = 0 and is written as zeros
    if (M == -INFINITY)
        M = 0.0f;
    float W = 0.0f;
    for (int jj = lane; jj < np; jj += kWave)
        W += fast_exp2(ml[2 * slot_of(jj)] - M) * ml[2 * slot_of(jj) + 1];
    W = wave_sum(W);

    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c0 = 0; c0 < np; c0 += kWave) {
        const int n = min(kWave, np - c0);
        const float wl = lane < n ? fast_exp2(ml[2 * slot_of(c0 + lane)] - M) : 0.0f;
        for (int k = 0; k < n; k += U * PPI) {
            float4 a[U];
            float wk[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j0 = k + u * PPI;  // first part of instruction u (wave-uniform)
                float wv = 0.0f;
#pragma unroll
                for (int g = 0; g < PPI; ++g) {
                    const float x = __int_as_float(
                        __builtin_amdgcn_readlane(__float_as_int(wl), min(j0 + g, kWave - 1)));
                    wv = grp == g ? x : wv;
                }
                const int j = j0 + grp;
                wk[u] = j < n ? wv : 0.0f;
                a[u] = j < n ? *(const float4 *)(ac + (size_t)slot_of(c0 + j) * p.ws_rows * D)
                             : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                o[0] += wk[u] * a[u].x;
                o[1] += wk[u] * a[u].y;
                o[2] += wk[u] * a[u].z;
                o[3] += wk[u] * a[u].w;
            }
        }
    }
#pragma unroll
    for (int off = LPP; off < kWave; off <<= 1)
#pragma unroll
        for (int d = 0; d < 4; ++d)
            o[d] += xor_shfl(o[d], off);
    if (grp == 0) {
        const float inv = W > 0.0f ? 1.0f / W : 0.0f;
        uint2 w2;
        w2.x = pack2<BF>(o[0] * inv, o[1] * inv);
        w2.y = pack2<BF>(o[2] * inv, o[3] * inv);
        *(uint2 *)(p.out + (size_t)orow * D + sub * 4) = w2;
    }
}

template <bool BF, bool F8, int D, int GK>
hipError_t launch_units(const DecodeParams &p, hipStream_t stream)
{
    if constexpr (GK == kCols)
        hipLaunchKernelGGL((decode_mfma_kernel<BF, F8, D>),
                           dim3(round_up8(p.wg_parts == kMfmaWaves
                                              ? p.n_units
                                              : (p.n_units + kMfmaWaves - 1) / kMfmaWaves)),
                           dim3(kWave * kMfmaWaves), 0, stream, p);
    else if (!F8 && p.part_tokens >= 1024)
        hipLaunchKernelGGL((decode_partition_kernel<BF, F8, D, GK, kUnitWavesMax>),
                           dim3(round_up8(p.n_units)), dim3(kWave * kUnitWavesMax), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_partition_kernel<BF, F8, D, GK, 4>), dim3(round_up8(p.n_units)),
                           dim3(kWave * 4), 0, stream, p);
    return hipGetLastError();
}

// gk: query rows per unit -- 1 or 2 (one row class per lane, vector ALU) or kCols (MFMA columns)
template <bool BF, bool F8, int D>
hipError_t run_decode(int gk, const DecodeParams &p, const DecodeParams *pre, hipStream_t stream)
{
    hipError_t e;
    if (pre && pre->n_units > 0) {  // no prefix units when no sequence shares a token
        hipLaunchKernelGGL((decode_prefix_mfma_kernel<BF, F8, D>), dim3(round_up8(pre->n_units)),
                           dim3(kWave * kMfmaWaves), 0, stream, *pre);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    e = gk == kCols ? launch_units<BF, F8, D, kCols>(p, stream)
        : gk == 2   ? launch_units<BF, F8, D, 2>(p, stream)
                    : launch_units<BF, F8, D, 1>(p, stream);
    if (e != hipSuccess || !p.split || p.fused_finish)
        return e;
    hipLaunchKernelGGL((decode_merge_kernel<BF, D>), dim3((p.ws_rows + 3) / 4), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

// Multi-token decode: the MFMA kernel with per-column views of the rows' own positions, then the
// merge of the split parts
template <bool BF, bool F8, int D>
hipError_t run_decode_multi(int ncg, const DecodeParams &p, hipStream_t stream)
{
    const dim3 grid(round_up8(p.wg_parts == kMfmaWaves ? p.n_units
                                                       : (p.n_units + kMfmaWaves - 1) / kMfmaWaves));
    if (ncg == 2)
        hipLaunchKernelGGL((decode_multi_kernel<BF, F8, D, 2>), grid, dim3(kWave * kMfmaWaves), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((decode_multi_kernel<BF, F8, D, 1>), grid, dim3(kWave * kMfmaWaves), 0,
                           stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.split)
        return e;
    hipLaunchKernelGGL((decode_merge_kernel<BF, D>), dim3((p.ws_rows + 3) / 4), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

// Decode scratch for callers that cannot allocate (pa_decode_noalloc): a file-scope device array,
// one copy per GPU at its own address, held from the library's first use on that GPU until the
// process ends. Host code never passes the array's name to a kernel: in host code that name is a
// host-side stand-in. It uses the address hipGetSymbolAddress returns on each device instead.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // per device ordinal; null until looked up
}  // namespace

hipError_t decode_scratch(hipStream_t stream, void **ptr)
{
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        // the lookup needs the stream's device current; the caller's current device is restored
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess)
            return e;
        if (back != hipSuccess)
            return back;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeLaunch &d, hipStream_t stream)
{
    if (d.num_seqs == 0)
        return hipSuccess;
    const int group = d.num_q_heads / d.c.num_kv_heads;
    if (group > kCols && !(d.group_starts != nullptr && d.num_groups > 0)) {
        // head groups above one MFMA column group (MQA-like): the multi-token units with one row
        // per sequence hold 32 query heads per wave, so each context is read once per 32 heads
        // instead of once per 16 (the same workspace rows and slots as the MFMA decode)
        DecodeLaunch m = d;
        m.cu_q_lens = nullptr;
        m.tree_mask = nullptr;
        m.max_q_len = 1;
        m.total_q = d.num_seqs;
        return launch_decode_multi(m, stream);
    }
    // groups of 1 and 2: one unit per query head pair on the vector ALU; larger groups: up to 16
    // query heads per unit on MFMA
    const int gk = group <= 2 ? group : kCols;
    const bool cascade = d.group_starts != nullptr && d.num_groups > 0;
    DecodeParams p = {};
    p.query = (const uint16_t *)d.query;
    p.k_cache = (const uint16_t *)d.k_cache;
    p.v_cache = (const uint16_t *)d.v_cache;
    p.block_tables = d.block_tables;
    p.seq_lens = d.seq_lens;
    p.out = (uint16_t *)d.out;
    p.max_blocks = d.max_blocks;
    p.num_seqs = d.num_seqs;
    p.num_kv_heads = d.c.num_kv_heads;
    p.num_q_heads = d.num_q_heads;
    p.num_blocks = d.c.num_blocks;
    p.max_seq_len = d.max_seq_len;
    p.scale_log2 = (float)((double)d.scale * (d.fp8 ? (double)d.k_scale : 1.0) * 1.4426950408889634);
    p.v_scale = d.fp8 ? d.v_scale : 1.0f;
    p.n_sub = (group + gk - 1) / gk;
    p.split = d.max_parts > 0 ? 1 : 0;
    p.part_tokens = p.split ? d.partition_size : ((d.max_seq_len + kBlock - 1) / kBlock) * kBlock;
    if (p.part_tokens < kBlock)
        p.part_tokens = kBlock;
    p.max_parts = p.split ? d.max_parts : 1;
    // Shared prefixes on the vector-ALU kernel whose own ranges all fit 1024 tokens: one own part
    // per row, as long as the longest own range, so that each own unit can finish its row (below)
    const bool own_one_part = cascade && gk != kCols && d.max_own_len > 0 && d.max_own_len <= 1024;
    if (own_one_part) {
        p.part_tokens = (d.max_own_len + kBlock - 1) / kBlock * kBlock;
        p.max_parts = 1;
    }
    // split MFMA decode: kMfmaWaves consecutive parts per workgroup, merged into one slot
    p.wg_parts = gk == kCols && p.split ? kMfmaWaves : 1;
    p.slot_tokens = p.part_tokens * p.wg_parts;
    const int own_slots = (p.max_parts + p.wg_parts - 1) / p.wg_parts;
    p.ws_slots = own_slots;
    p.ws_rows = d.num_seqs * d.num_q_heads;
    int pre_slots = 0;
    if (cascade) {
        // slots [0, pre_slots) of every row hold shared-prefix results (kMfmaWaves parts each),
        // the rest its own parts
        const int pre_parts = (d.max_prefix_len + d.partition_size - 1) / d.partition_size;
        pre_slots = (pre_parts + kMfmaWaves - 1) / kMfmaWaves;
        p.ws_slots = pre_slots + own_slots;
    }
    // workspace: acc [slots][rows][D], then (m, l) [rows][slots][2]
    p.ws_acc = (float *)d.workspace;
    p.ws_ml = p.split ? p.ws_acc + (size_t)p.ws_rows * p.ws_slots * d.c.head_dim : nullptr;

    // own ranges that all fit one part on the vector-ALU kernel finish their rows themselves
    p.fused_finish = own_one_part ? 1 : 0;

    DecodeParams pre;
    if (cascade) {
        p.seq_starts = d.seq_starts;
        p.pre_slots = pre_slots;
        p.pre_slot_tokens = d.partition_size * kMfmaWaves;
        p.slot_base = pre_slots;
        pre = p;
        pre.group_starts = d.group_starts;
        pre.num_groups = d.num_groups;
        const int pairs = d.max_group_size * group;  // (member, query head) pairs per kv head
        pre.n_vsub = (pairs + kCols - 1) / kCols;
        // workgroups: (group, prefix slot, kv head, pair subgroup)
        const int64_t pre_units = (int64_t)d.num_groups * pre_slots * d.c.num_kv_heads * pre.n_vsub;
        if (pre_units > 0x7ffffff0)
            return hipErrorInvalidValue;
        pre.n_units = (int32_t)pre_units;
    }
    // units: workgroups of merged parts, else waves
    const int64_t units = (int64_t)d.num_seqs * d.c.num_kv_heads * p.n_sub *
                          (p.wg_parts == kMfmaWaves ? own_slots : p.max_parts);
    if (units > 0x7ffffff0)
        return hipErrorInvalidValue;
    p.n_units = (int32_t)units;
    const DecodeParams *pp = cascade ? &pre : nullptr;
    if (d.fp8) {
        if (d.c.bf16)
            return d.c.head_dim == 64 ? run_decode<true, true, 64>(gk, p, pp, stream)
                                      : run_decode<true, true, 128>(gk, p, pp, stream);
        return d.c.head_dim == 64 ? run_decode<false, true, 64>(gk, p, pp, stream)
                                  : run_decode<false, true, 128>(gk, p, pp, stream);
    }
    if (d.c.bf16)
        return d.c.head_dim == 64 ? run_decode<true, false, 64>(gk, p, pp, stream)
                                  : run_decode<true, false, 128>(gk, p, pp, stream);
    return d.c.head_dim == 64 ? run_decode<false, false, 64>(gk, p, pp, stream)
                              : run_decode<false, false, 128>(gk, p, pp, stream);
}

}  // namespace pa

namespace pa {

hipError_t launch_decode_multi(const DecodeLaunch &d, hipStream_t stream)
{
    if (d.num_seqs == 0 || d.total_q == 0 || d.max_q_len == 0)
        return hipSuccess;
    const int group = d.num_q_heads / d.c.num_kv_heads;
    DecodeParams p = {};
    p.query = (const uint16_t *)d.query;
    p.k_cache = (const uint16_t *)d.k_cache;
    p.v_cache = (const uint16_t *)d.v_cache;
    p.block_tables = d.block_tables;
    p.seq_lens = d.seq_lens;
    p.out = (uint16_t *)d.out;
    p.max_blocks = d.max_blocks;
    p.num_seqs = d.num_seqs;
    p.num_kv_heads = d.c.num_kv_heads;
    p.num_q_heads = d.num_q_heads;
    p.num_blocks = d.c.num_blocks;
    p.max_seq_len = d.max_seq_len;
    p.scale_log2 = (float)((double)d.scale * (d.fp8 ? (double)d.k_scale : 1.0) * 1.4426950408889634);
    p.v_scale = d.fp8 ? d.v_scale : 1.0f;
    p.cu_q = d.cu_q_lens;
    p.tree_mask = d.tree_mask;
    p.mt_rows = d.max_q_len;
    p.total_q = d.total_q;
    // the (row, query head) pairs of a kv head: one column group of kCols when they fit it, else
    // subgroups of two column groups per wave
    const int pairs = d.max_q_len * group;
    const int ncg = pairs > kCols ? 2 : 1;
    p.n_sub = (pairs + kCols * ncg - 1) / (kCols * ncg);
    p.split = d.max_parts > 0 ? 1 : 0;
    p.part_tokens = p.split ? d.partition_size : ((d.max_seq_len + kBlock - 1) / kBlock) * kBlock;
    if (p.part_tokens < kBlock)
        p.part_tokens = kBlock;
    p.max_parts = p.split ? d.max_parts : 1;
    p.wg_parts = p.split ? kMfmaWaves : 1;
    p.slot_tokens = p.part_tokens * p.wg_parts;
    p.ws_slots = (p.max_parts + p.wg_parts - 1) / p.wg_parts;
    const int64_t rows = (int64_t)d.num_seqs * d.max_q_len * d.num_q_heads;
    if (rows > 0x7fffffff)
        return hipErrorInvalidValue;
    p.ws_rows = (int32_t)rows;
    // workspace: acc [slots][rows][D], then (m, l) [rows][slots][2]
    p.ws_acc = (float *)d.workspace;
    p.ws_ml = p.split ? p.ws_acc + (size_t)p.ws_rows * p.ws_slots * d.c.head_dim : nullptr;
    const int64_t units = (int64_t)d.num_seqs * d.c.num_kv_heads * p.n_sub *
                          (p.wg_parts == kMfmaWaves ? p.ws_slots : p.max_parts);
    if (units > 0x7ffffff0)
        return hipErrorInvalidValue;
    p.n_units = (int32_t)units;
    if (d.fp8) {
        if (d.c.bf16)
            return d.c.head_dim == 64 ? run_decode_multi<true, true, 64>(ncg, p, stream)
                                      : run_decode_multi<true, true, 128>(ncg, p, stream);
        return d.c.head_dim == 64 ? run_decode_multi<false, true, 64>(ncg, p, stream)
                                  : run_decode_multi<false, true, 128>(ncg, p, stream);
    }
    if (d.c.bf16)
        return d.c.head_dim == 64 ? run_decode_multi<true, false, 64>(ncg, p, stream)
                                  : run_decode_multi<true, false, 128>(ncg, p, stream);
    return d.c.head_dim == 64 ? run_decode_multi<false, false, 64>(ncg, p, stream)
                              : run_decode_multi<false, false, 128>(ncg, p, stream);
}

}  // namespace pa
