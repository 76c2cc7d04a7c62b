// prefill.hip -- paged causal attention of prefill chunks on the gfx950 matrix cores (MFMA).
//
// What it computes: sequence s owns query rows cu_q_lens[s] .. cu_q_lens[s+1]-1, its last q_len
// positions; row i at position p = seq_lens[s] - q_len + i attends keys 0..p (lecture 32
// "LLM 在线推理两阶段" §5.4 chunked prefill: a chunk sees the cached context and the earlier part of
// itself; §1.1 causal order; §3.1 softmax(QK^T/sqrt(d))V; §3.4 GQA groups). Keys are read through
// the block table (openeuler.csdn.net "高并发 AI 服务的内存瓶颈", Attention 计算时的 Block 映射) and
// consumed tile by tile with a running max and sum (devpress.csdn.net/amd vLLM overview §9 (3)(4):
// query and key/value tiling with online softmax).
//
// Tiling. A workgroup of 8 waves owns 256 (query row, query head) pairs of one kv-head group: the
// GK heads that share the kv head, for 256/GK consecutive rows, so each K/V tile staged in LDS serves
// every head of the group. (Short causal contexts use 4 waves and 128 pairs, so that two workgroups
// share a CU; the arithmetic of every pair is the same.) Per 64-key tile (4 paged blocks):
//   - 16-bit K and V rows go to LDS untouched, straight from HBM (global_load_lds_dwordx4: no
//     staging registers), into buffers that are filled while others are computed. Rows are stored
//     without padding; the 16-byte pieces of row r are XOR-swizzled (piece c at c ^ swz(r)) so that
//     the column reads below hit distinct banks. E4M3 rows pass through registers instead, where
//     they are converted exactly to the query's 16-bit type, and land in the same LDS layout.
//   - Each wave computes S^T = K Q^T for its 32 pairs with v_mfma_f32_32x32x16 (A = 32 keys x 16
//     dims, one ds_read_b128 per lane; B = Q^T held in registers for the whole kernel).
//   - Online softmax in the accumulator layout: lane l holds column l%32 (one pair) and 16 keys per
//     32-key tile; the two lanes of a column exchange the maximum once per tile.
//   - O^T += V^T P^T, again 32x32x16 MFMAs. P^T is the softmax tile packed to 16 bits straight from
//     the S^T accumulators, whose layout gives lane half h the keys {4h..4h+3, 8+4h..8+4h+3} of each
//     16-key step. The V^T operand comes from row-major V with ds_read_b64_tr_b16, which hands lane j
//     of a 16-lane group element j%4 of the 8 bytes addressed by lane 4k + j/4 (k = 0..3): each lane
//     addresses 4 dims of one key row, and the key rows are chosen so that key and probability meet on
//     the same MFMA k-slot.
// The causal mask is applied only on tiles that reach past the workgroup's first position. Keys
// beyond the context are never loaded; LDS starts zeroed, so such slots hold finite stale values that
// meet zero probabilities (no NaN reaches an MFMA).
//
// Two tile loops. The main loop is software-pipelined so that the matrix cores and the vector ALUs
// work at once: while the softmax of tile t runs on the VALU, the MFMAs of S^T for tile t+1 and of
// O^T += V^T P^T for tile t-1 are in flight (K and V have four LDS slots each: K runs two tiles
// ahead of V). P is rounded to the 16-bit type in one part there. fp16 queries always take it;
// bfloat16 ones where every row of the workgroup attends at least kOnePartKeys keys. Rows with fewer
// keys -- the first rows of a prompt, where a handful of keys can dominate and cancel -- take the
// plain loop, which splits a bfloat16 P into hi + lo parts.
#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <bool BF>
__device__ __forceinline__ f32x16 mfma32(const uint4 &a, const uint4 &b, const f32x16 &c)
{
    if constexpr (BF) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

struct PrefillParams {
    const uint16_t *__restrict__ query;
    const uint16_t *__restrict__ k_cache;
    const uint16_t *__restrict__ v_cache;
    const int32_t *__restrict__ block_tables;
    const int32_t *__restrict__ seq_lens;
    const int32_t *__restrict__ cu_q_lens;
    const uint64_t *__restrict__ tree_mask;  // null: causal; else one mask per query row
    uint16_t *__restrict__ out;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t num_blocks;
    int32_t n_sub;
    int32_t row_tiles;
    int32_t n_items;
    int32_t total_q;
    float scale_log2;
    float v_scale;  // value scale (E4M3 caches, also widened), applied to the output; k_scale is
                    // in scale_log2
    int32_t identity_blocks;  // block i of sequence s is block s * max_blocks + i (a widened copy)
};

// Causal chunks whose block tables span at most this many tokens run four-wave workgroups (the
// 16-bit and widened instances): measured on whole fresh prompts, 32 query / 8 kv heads of 128,
// 3-12 % faster up to 1024 tokens, even at 2048, and 2-5 % slower at 4096.
constexpr int kFourWaveKeys = 2048;
constexpr int kKeys = 64;  // keys per tile
// A workgroup whose first row attends at least this many keys rounds P to the 16-bit type in one
// part: a bfloat16 probability keeps 8 significant bits, and over L keys of comparable weight the
// rounding errors add up to about 2^-9 |v| / sqrt(L) (below 1e-4 here), far inside the 2e-3 gate.
constexpr int kOnePartKeys = 512;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// XOR swizzle of the 16-byte pieces of LDS row r (D = 128: 16 pieces; D = 64: 8 pieces, two rows
// per 256-byte line of the 64 four-byte banks). Chosen so that both operand reads are free of bank
// conflicts:
//   - K: 16 consecutive rows read at one column (ds_read_b128, 16 lanes a cycle) -- swz over each
//     aligned 16 rows (each row parity, for D = 64) is a permutation;
//   - V: 4 consecutive rows read at 4 adjacent pieces (ds_read_b64_tr_b16, 32 lanes a cycle) --
//     rows r and r + 1 (D = 128), r and r + 2 (D = 64) take different groups of 4 pieces.
// (An earlier swizzle, 2 (r & 7) + (r >> 3 & 1), sent rows r and r + 1 of V to the same pieces:
// 2 conflict cycles per V read, 64 per wave-step; removing them took the 1856-row chunk from
// 249-252 to 246 us, bit-identical.) swz(r + 8) = swz(r) ^ 2 for both.
template <int D>
__device__ __forceinline__ int swz(int r)
{
    if constexpr (D == 128)
        return ((r & 3) << 2) | ((r >> 2) & 3);
    else
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// W waves per workgroup: 8 (one workgroup per CU, 128 KiB of LDS: K and V four tiles each), or 4
// for short causal work (64 KiB: two tiles each), so that two workgroups share a CU and one's set-up
// and drain overlap the other's tile loop. Both compute every (row, head) pair the same way.
template <bool BF, int D, int GK, bool TREE, bool F8, int W>
__global__ __launch_bounds__(W * 64, 8 / W) void prefill_kernel(PrefillParams p)
{
    static_assert(W == 8 || (W == 4 && !F8), "E4M3 staging needs eight waves");
    constexpr int kWavesW = W;
    constexpr int kThreadsW = W * 64;
    constexpr int KS = W == 8 ? 4 : 2;              // LDS tile slots per cache
    constexpr int R = kWavesW * 32 / GK;            // query rows per workgroup
    constexpr int DC = D / 16;                      // k-steps of S^T = K Q^T
    constexpr int DT = D / 32;                      // 32-dim tiles of O^T
    constexpr int ROWB = D * 2;                     // bytes per LDS row (no padding)
    constexpr int CPR = D / 8;                      // 16-byte pieces per row
    constexpr int TILEB = kKeys * ROWB;             // bytes of one K or V tile
    // Four K slots and four V slots of one 64-key tile each: 64-key tile j of the K cache lives in
    // bytes [(j % 4) * TILEB, +TILEB), of the V cache from (4 + j % 4) * TILEB on. The direct-to-LDS loads are
    // issued so that the compiler does not track them (dma16_to_lds): reads of the tiles being
    // computed run while later tiles are in flight, and every wait for a load is explicit below.
    __shared__ __align__(1024) uint8_t lds[2 * KS * TILEB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hh = lane >> 5;

    const int item = xcd_logical_id(blockIdx.x, gridDim.x);
    if (item >= p.n_items)
        return;
    int rest = item;
    const int tile_r = rest % p.row_tiles;
    rest /= p.row_tiles;
    const int sub = rest % p.n_sub;
    rest /= p.n_sub;
    const int kvh = rest % p.num_kv_heads;
    const int seq = rest / p.num_kv_heads;

    // offsets are clamped to [0, total_q] so that no index contents can reach outside the arrays
    const int q0 = min(max(p.cu_q_lens[seq], 0), p.total_q);
    const int q_len = min(max(p.cu_q_lens[seq + 1], q0), p.total_q) - q0;
    const int row_base = tile_r * R;
    if (row_base >= q_len)
        return;
    const int L = p.num_blocks > 0 ? min(max(p.seq_lens[seq], 0), p.max_blocks * kBlock) : 0;
    const int first_pos = L - q_len;  // position of the chunk's row 0

    // this lane's (row, head) pair: column n of the wave's S^T / O^T tiles
    const int pair = wave * 32 + n;
    const int row = row_base + pair / GK;
    const int head = (kvh * p.n_sub + sub) * GK + pair % GK;
    const bool row_ok = row < q_len;
    const int pos = row_ok ? first_pos + row : -1;  // attends keys 0..pos

    uint4 qv[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c)
        qv[c] = row_ok ? *(const uint4 *)(p.query +
                                          ((size_t)(q0 + row) * p.num_q_heads + head) * D +
                                          c * 16 + hh * 8)
                       : make_uint4(0, 0, 0, 0);

    // TREE (drafted-token trees): the row sees chunk row j (position first_pos + j, j <= row) only
    // when bit j of its mask p.tree_mask[row] is set; every position before the chunk stays visible
    constexpr bool tree = TREE;

    const int last_row = min(row_base + R, q_len) - 1;
    const int key_end = max(0, min(L, first_pos + last_row + 1));
    const int n_tiles = (key_end + kKeys - 1) / kKeys;
    // every row of the group sees the keys <= this
    const int unmasked_below = tree ? first_pos - 1 : first_pos + row_base;
    const bool ragged_rows = row_base + R > q_len;
    // visibility bits of the lane's keys in tile t, bit kr for key t*64 + 4*hh + kr (kr < 64)
    auto tree_bits = [&](int t) PA_INLINE -> uint64_t {
        // read where needed (masked tiles only): no register holds it through the tile loop
        const uint64_t tmask = row_ok ? p.tree_mask[q0 + row] : ~0ull;
        const int jb = t * kKeys + 4 * hh - first_pos;  // chunk row of kr = 0
        if (jb >= 64)
            return 0;
        if (jb >= 0)
            return tmask >> jb;
        if (jb > -64)
            return (tmask << -jb) | ((1ull << -jb) - 1);
        return ~0ull;
    };
    // the causal mask of tile t (keys past the row's position), and the tree mask when given
    auto apply_mask = [&](f32x16 (&s)[2], int t, int row_pos) PA_INLINE {
        const int last = row_pos - t * kKeys - 4 * hh;  // key kr must be <= last
        if constexpr (tree) {
            const uint64_t bits = tree_bits(t);
            const uint32_t lo = (uint32_t)bits, hi = (uint32_t)(bits >> 32);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int kr = kt * 32 + 8 * (v >> 2) + (v & 3);
                    const bool seen = ((kr < 32 ? lo >> kr : hi >> (kr - 32)) & 1u) != 0;
                    s[kt][v] = kr <= last && seen ? s[kt][v] : -INFINITY;
                }
        } else {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    s[kt][v] = kt * 32 + 8 * (v >> 2) + (v & 3) <= last ? s[kt][v] : -INFINITY;
        }
    };

    // the sequence's block table, read with scalar loads (it is read-only while the kernel runs)
    typedef const __attribute__((address_space(4))) int32_t *ctable_t;
    const ctable_t table = (ctable_t)(p.block_tables + (size_t)seq * p.max_blocks);
    const size_t blk_stride = (size_t)p.num_kv_heads * kBlock * D;

    // LDS starts zeroed: slots of keys that are never loaded then hold finite values
    for (int i = tid; i < 2 * KS * TILEB / 16; i += kThreadsW)
        ((uint4 *)lds)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();

    // Direct-to-LDS loads of the SPAN * 64 keys from key t * 64 * SPAN of one cache into buf. Wave
    // w loads paged block w of the span (16 rows, one block id, one source base): PER_BLK loads of
    // RPI rows each; lane i of load k writes the 16-byte piece at LDS offset 16*i of rows
    // [16 w + k RPI, +RPI). Its source is row k RPI + i / CPR of the (block, kv head) tile, piece
    // (i % CPR) ^ swz(row) -- the same for every block, so the lane offsets are computed once.
    // Returns how many load instructions this wave issued (the counted waits below rely on it; a
    // block id outside the pool skips its loads but still counts them, so such tables make those
    // waits end early -- unspecified results, never a fault). A load instruction is issued exactly
    // when its first row lies in the context, so at least one of its lanes is active.
    constexpr int RPI = kWave * 16 / ROWB;       // rows per load instruction
    constexpr int PER_BLK = kBlock / RPI;        // load instructions per block
    const int lane_row = lane / CPR;
    const int lane_piece = lane % CPR;
    uint32_t dma_voff[PER_BLK];
#pragma unroll
    for (int k = 0; k < PER_BLK; ++k) {
        const int r = k * RPI + lane_row;
        dma_voff[k] = (uint32_t)((r * D + (lane_piece ^ swz<D>(r)) * 8) * 2);
    }
    const size_t blk_bytes = blk_stride * 2;
    const size_t kvh_bytes = (size_t)kvh * kBlock * D * 2;
    auto issue_span = [&](auto span, const uint16_t *cache, uint8_t *buf, int t) PA_INLINE -> int {
        constexpr int KEYS = kKeys * decltype(span)::value, NBLK = KEYS / kBlock;
        static_assert(NBLK <= kWavesW, "one block per wave");
        const int key0 = t * KEYS + wave * kBlock;  // first key of this wave's block
        if (wave >= NBLK || key0 >= L)
            return 0;
        const int blk =
            p.identity_blocks ? seq * p.max_blocks + key0 / kBlock : table[key0 / kBlock];
        if ((unsigned)blk >= (unsigned)p.num_blocks)
            return PER_BLK;
        const char *sbase = (const char *)cache + kvh_bytes + (size_t)blk * blk_bytes;
        const uint32_t dst0 = lds_address(buf + wave * kBlock * ROWB);
        if (key0 + kBlock <= L) {
#pragma unroll
            for (int k = 0; k < PER_BLK; ++k)
                dma16_to_lds(dma_voff[k], sbase, dst0 + k * RPI * ROWB);
            return PER_BLK;
        }
        // the context's last block: rows past it are not loaded, and a load none of whose rows
        // lies in the context is not issued (nor counted)
        int issued = 0;
#pragma unroll
        for (int k = 0; k < PER_BLK; ++k) {
            if (key0 + k * RPI >= L)
                break;
            ++issued;
            if (key0 + k * RPI + lane_row < L)
                dma16_to_lds(dma_voff[k], sbase, dst0 + k * RPI * ROWB);
        }
        return issued;
    };
    using One = std::integral_constant<int, 1>;
    using Two = std::integral_constant<int, 2>;

    float m_run = -INFINITY, l_run = 0.0f;
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            o[dt][v] = 0.0f;

    // lane-constant parts of the LDS read addresses
    const int k_sw = swz<D>(n);                      // K operand: rows kt*32 + n share swz(n)
    const int g16 = lane >> 4, sl = lane & 15;       // transposed V reads: 16-lane group, source lane
    const int v_k = sl >> 2, v_q = sl & 3;           // source lane 4k + q: key row k, dims 4q..4q+3
    const int v_half = g16 >> 1;                     // lane half h of the destination lanes
    const int v_dim = (g16 & 1) * 16 + 4 * v_q;      // dim within a 32-dim tile

    // E4M3 caches ([V1] §4.4: one byte per element) are staged through registers: thread i loads
    // the 16 codes of piece i % PPR of row i / PPR of a 64-key tile, converts them exactly to the
    // 16-bit type (v_cvt_scalef32_pk_*_fp8) and writes them as the two 16-byte pieces of the same
    // swizzled LDS row the 16-bit path fills. A wave's rows lie in one paged block (8 or 16 rows,
    // block aligned), so its block id is one scalar load. Rows past the context are not written
    // (they keep finite values, as above).
    constexpr int PPR = D / 16;                // 16-code pieces per row
    constexpr int STAGERS = kKeys * PPR;       // threads that stage a tile
    const int r8 = tid / PPR, c8 = tid % PPR;
    const int row0_8 = __builtin_amdgcn_readfirstlane((wave * kWave) / PPR);  // the wave's first row
    // this thread's codes of tile t of one cache; false where its row holds no token
    auto load_codes = [&](const uint16_t *cache, int t, uint4 &dst) PA_INLINE -> bool {
        if (tid >= STAGERS || t * kKeys + row0_8 >= L)
            return false;
        const int blk = table[(t * kKeys + row0_8) / kBlock];
        const int key = t * kKeys + r8;
        if ((unsigned)blk >= (unsigned)p.num_blocks || key >= L)
            return false;
        const size_t off = (((size_t)blk * p.num_kv_heads + kvh) * kBlock + key % kBlock) * D +
                           c8 * 16;
        dst = *(const uint4 *)((const uint8_t *)cache + off);
        return true;
    };
    auto put_codes = [&](uint8_t *tile, const uint4 &w) PA_INLINE {
        const int swr = swz<D>(r8);
        const uint4 lo = make_uint4(e4m3x2_to_pk16<BF, false>(w.x), e4m3x2_to_pk16<BF, true>(w.x),
                                    e4m3x2_to_pk16<BF, false>(w.y), e4m3x2_to_pk16<BF, true>(w.y));
        const uint4 hi = make_uint4(e4m3x2_to_pk16<BF, false>(w.z), e4m3x2_to_pk16<BF, true>(w.z),
                                    e4m3x2_to_pk16<BF, false>(w.w), e4m3x2_to_pk16<BF, true>(w.w));
        *(uint4 *)(tile + r8 * ROWB + (((2 * c8) ^ swr) << 4)) = lo;
        *(uint4 *)(tile + r8 * ROWB + (((2 * c8 + 1) ^ swr) << 4)) = hi;
    };

    // a bfloat16 P needs its hi + lo split only while some row sees few keys (see kOnePartKeys)
    const bool one_part = !BF || unmasked_below + 1 >= kOnePartKeys;
    if (one_part && n_tiles > 0) {
        // ---------------------------------------------------------------- pipelined loop
        // Step t computes PV(t-1), QK(t+1) and the softmax of tile t. Tiles are loaded in pairs:
        // odd steps t = 2u+1 wait for the loads of the two steps before, pass a barrier and issue
        // K tiles 2u+4, 2u+5 (into the slots of K tiles 2u, 2u+1, which QK read in steps 2u-1 and
        // 2u); the even step after it issues V tiles 2u+2, 2u+3 (into the slots of V tiles 2u-2,
        // 2u-1, read by PV in steps 2u-1 and 2u, before that barrier). Spreading the two pairs
        // over both steps keeps the load issue off one step; the K pair has two steps to land,
        // the V pair one (both are waited for at step 2u+3, which first reads them).
        auto kslot = [&](int j) PA_INLINE -> uint8_t * { return lds + (j & (KS - 1)) * TILEB; };
        auto vslot = [&](int j) PA_INLINE -> uint8_t * {
            return lds + (KS + (j & (KS - 1))) * TILEB;
        };
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        // wait until at most n of this wave's loads are in flight (and LDS/scalar reads are done)
        auto wait_loads = [&](int n) PA_INLINE {
            switch (n) {
            case 0: __builtin_amdgcn_s_waitcnt(0x70); break;
            case 1: __builtin_amdgcn_s_waitcnt(0x71); break;
            case 2: __builtin_amdgcn_s_waitcnt(0x72); break;
            case 3: __builtin_amdgcn_s_waitcnt(0x73); break;
            case 4: __builtin_amdgcn_s_waitcnt(0x74); break;
            case 5: __builtin_amdgcn_s_waitcnt(0x75); break;
            case 6: __builtin_amdgcn_s_waitcnt(0x76); break;
            case 7: __builtin_amdgcn_s_waitcnt(0x77); break;
            default: __builtin_amdgcn_s_waitcnt(0x78); break;
            }
        };
        static_assert(2 * PER_BLK <= 8, "wait_loads covers a K pair and a V pair");

        // LDS read addresses, computed per step from one lane base per cache (no per-slot
        // registers). K operand of k-step c, rows kt*32 + n: piece (2c + hh) ^ swz(n) of the row,
        // i.e. byte (32 c) ^ 16 (hh ^ swz(n)). V operand of 32-dim tile dt, key rows r1 = 16 c4 +
        // 4 v_half + v_k and r2 = r1 + 8: piece (dim / 8) ^ swz(r), i.e. byte (64 dt) ^ 16 w for a
        // lane constant w, and swz(r2) = swz(r1) ^ 2, i.e. byte X2 = 32. Slot bases are
        // multiples of 8 KiB and the lane bases stay below 8 KiB, so the XORs and the slot offset
        // never interact.
        const uint32_t lds0 = lds_address(lds);
        const int k_lane = n * ROWB + 16 * (hh ^ k_sw);
        const int r1b = 4 * v_half + v_k;
        const int v_lane = r1b * ROWB + 16 * ((v_dim >> 3) ^ swz<D>(r1b)) + (v_dim & 7) * 2;
        constexpr int X2 = 32;

        // S^T = K Q^T of one tile into s, k-steps [C0, C1) (k-step 0 starts from zero); ka is the
        // lane's K base in the tile's slot
        auto qk = [&](auto c0, auto c1, f32x16 (&s)[2], uint32_t ka) PA_INLINE {
            const f32x16 zero = {};
#pragma unroll
            for (int c = decltype(c0)::value; c < decltype(c1)::value; ++c)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const uint32_t addr = (ka ^ (32 * c)) + kt * 32 * ROWB;
                    const uint4 a = lds_read16(addr);
                    s[kt] = mfma32<BF>(a, qv[c], c == 0 ? zero : s[kt]);
                }
        };
        // O^T += V^T P^T for the 16 keys of step c4 of one tile; va is the lane's V base
        auto pv = [&](auto c4c, const uint4 (&pt)[4], uint32_t va) PA_INLINE {
            constexpr int c4 = decltype(c4c)::value;
            uint4 a[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint32_t a1 = (va ^ (64 * dt)) + c4 * 16 * ROWB;
                const uint32_t a2 = (va ^ (64 * dt) ^ X2) + (c4 * 16 + 8) * ROWB;
                const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)a1);
                const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)a2);
                a[dt].x = __builtin_bit_cast(uint2, lo4).x;
                a[dt].y = __builtin_bit_cast(uint2, lo4).y;
                a[dt].z = __builtin_bit_cast(uint2, hi4).x;
                a[dt].w = __builtin_bit_cast(uint2, hi4).y;
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                o[dt] = mfma32<BF>(a[dt], pt[c4], o[dt]);
        };
        // invalid rows (past the chunk) have zero queries and are never stored: no mask for them
        const int pos_p = row_ok ? pos : 0x3fffffff;
        // Online softmax of the tile in s, in three parts: the maximum (and the mask), the
        // exponentials of values [I0, I1) (value i = s[i / 16][i % 16]), and the packing of P.
        float ms = 0.0f, psum = 0.0f;
        auto sm_max = [&](auto masked, f32x16 (&s)[2], int t) PA_INLINE -> float {
            if constexpr (decltype(masked)::value)
                apply_mask(s, t, pos_p);
            float mx = s[0][0];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    mx = fmaxf(mx, s[kt][v]);
            mx = pair_max(mx) * p.scale_log2;  // scale > 0 keeps the order
            const float mn = fmaxf(m_run, mx);
            ms = mn == -INFINITY ? 0.0f : mn;
            const float alpha = fast_exp2(m_run - ms);
            m_run = mn;
            psum = 0.0f;
            return alpha;
        };
        auto sm_exp = [&](auto i0, auto i1, f32x16 (&s)[2]) PA_INLINE {
#pragma unroll
            for (int i = decltype(i0)::value; i < decltype(i1)::value; ++i) {
                s[i >> 4][i & 15] = fast_exp2(fmaf(s[i >> 4][i & 15], p.scale_log2, -ms));
                psum += s[i >> 4][i & 15];
            }
        };
        auto sm_pack = [&](auto c4c, const f32x16 (&s)[2], uint4 (&pt)[4]) PA_INLINE {
            constexpr int c4 = decltype(c4c)::value, kt = c4 >> 1, b = 8 * (c4 & 1);
            pt[c4].x = pack2<BF>(s[kt][b + 0], s[kt][b + 1]);
            pt[c4].y = pack2<BF>(s[kt][b + 2], s[kt][b + 3]);
            pt[c4].z = pack2<BF>(s[kt][b + 4], s[kt][b + 5]);
            pt[c4].w = pack2<BF>(s[kt][b + 6], s[kt][b + 7]);
        };
        // The work of one iteration in four chunks; the compiler interleaves within a chunk and
        // never moves work across chunk boundaries, which bounds the operands in flight. The wave's
        // issue priority steps down from 3 to 0 over the four chunks (s_setprio: a per-wave issue
        // preference inside the SIMD): of the two waves on a SIMD, the one earlier in its step
        // issues first, which keeps the two out of phase so that one's MFMAs overlap the other's
        // softmax (a 1856-row chunk over 6144 cached tokens, 32 query / 8 kv heads: 227.9 ->
        // 221.3 us, results bit-identical; a strict split of
        // each chunk into an MFMA block at priority 1 and a vector block at 0 was slower). E4M3
        // instances keep one priority: their register staging at odd steps already staggers the
        // waves, and the steps measured 245 -> 247 us there.
        auto region = [&](auto masked, int t, f32x16 (&s_in)[2], f32x16 (&s_out)[2],
                          const uint4 (&p_in)[4], uint4 (&p_out)[4], uint32_t kb,
                          uint32_t vb) PA_INLINE -> float {
            using C = std::integral_constant<int, 0>;
            if constexpr (!F8)
                __builtin_amdgcn_s_setprio(3);
            pv(std::integral_constant<int, 0>{}, p_in, vb);
            qk(C{}, std::integral_constant<int, DC / 4>{}, s_out, kb);
            const float alpha = sm_max(masked, s_in, t);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!F8)
                __builtin_amdgcn_s_setprio(2);
            pv(std::integral_constant<int, 1>{}, p_in, vb);
            qk(std::integral_constant<int, DC / 4>{}, std::integral_constant<int, DC / 2>{}, s_out, kb);
            sm_exp(C{}, std::integral_constant<int, 11>{}, s_in);
            sm_pack(std::integral_constant<int, 0>{}, s_in, p_out);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!F8)
                __builtin_amdgcn_s_setprio(1);
            pv(std::integral_constant<int, 2>{}, p_in, vb);
            qk(std::integral_constant<int, DC / 2>{}, std::integral_constant<int, 3 * DC / 4>{}, s_out, kb);
            sm_exp(std::integral_constant<int, 11>{}, std::integral_constant<int, 22>{}, s_in);
            sm_pack(std::integral_constant<int, 1>{}, s_in, p_out);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!F8)
                __builtin_amdgcn_s_setprio(0);
            pv(std::integral_constant<int, 3>{}, p_in, vb);
            qk(std::integral_constant<int, 3 * DC / 4>{}, std::integral_constant<int, DC>{}, s_out, kb);
            sm_exp(std::integral_constant<int, 22>{}, std::integral_constant<int, 32>{}, s_in);
            sm_pack(std::integral_constant<int, 2>{}, s_in, p_out);
            sm_pack(std::integral_constant<int, 3>{}, s_in, p_out);
            l_run = l_run * alpha + psum;
            // P is complete here: keeps the compiler from sinking the softmax into the next
            // iteration, past its rescale branch, where it would no longer overlap these MFMAs
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                asm volatile("" : "+v"(p_out[c4].x), "+v"(p_out[c4].y), "+v"(p_out[c4].z),
                                  "+v"(p_out[c4].w));
            __builtin_amdgcn_sched_barrier(0);
            return alpha;
        };

        // tiles from t_mask on hold keys that some row of the group does not see
        const int t_mask = min(n_tiles, max(0, (unmasked_below + 1) / kKeys));
        f32x16 sa[2], sb[2];
        uint4 pa[4], pb[4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
            pb[c4] = make_uint4(0, 0, 0, 0);  // "tile -1": zero probabilities
        float alpha_prev = 1.0f;
        bool rescale = false;

        // E4M3: the codes staged at an odd step (K tiles 2v+2, 2v+3, V tiles 2v, 2v+1 for v =
        // (t+1)/2) are converted into their slots at the next odd step, before its barrier: by
        // then no wave reads those slots (their previous tiles were last read two steps before)
        uint4 sk[2], sv[2];
        bool okk[2] = {false, false}, okv[2] = {false, false};
        int staged_v = 0;
        auto stage = [&](int v) PA_INLINE {
            staged_v = v;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                okk[i] = 2 * v + 2 + i < n_tiles && load_codes(p.k_cache, 2 * v + 2 + i, sk[i]);
                okv[i] = 2 * v + i < n_tiles && load_codes(p.v_cache, 2 * v + i, sv[i]);
            }
        };
        auto write_staged = [&]() PA_INLINE {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (okk[i])
                    put_codes(kslot(2 * staged_v + 2 + i), sk[i]);
                if (okv[i])
                    put_codes(vslot(2 * staged_v + i), sv[i]);
            }
        };

        // K tiles 0..3 and V tiles 0, 1 before step 0; QK(0) needs K tiles 0, 1 only
        if constexpr (F8) {
            uint4 c;
            if (load_codes(p.k_cache, 0, c))
                put_codes(kslot(0), c);
            if (n_tiles > 1 && load_codes(p.k_cache, 1, c))
                put_codes(kslot(1), c);
            stage(0);
            __syncthreads();
        } else if constexpr (W == 4) {
            // K tiles 0 and 1; V tile t is issued at step t
            (void)issue_span(One{}, p.k_cache, kslot(0), 0);
            if (n_tiles > 1)
                (void)issue_span(One{}, p.k_cache, kslot(1), 1);
            wait_loads(0);
            __syncthreads();
        } else {
            (void)issue_span(Two{}, p.k_cache, kslot(0), 0);
            const int c1 = n_tiles > 2 ? issue_span(Two{}, p.k_cache, kslot(2), 1) : 0;
            const int c2 = issue_span(Two{}, p.v_cache, vslot(0), 0);
            wait_loads(c1 + c2);
            __syncthreads();
        }
        qk(std::integral_constant<int, 0>{}, std::integral_constant<int, DC>{}, sa,
           lds0 + k_lane);

        // One step, t % 2 == P: s_in holds S of tile t, s_out receives S of tile t+1, p_in is P
        // of tile t-1. After the loads are issued it is straight-line code, so the scheduler can
        // interleave the MFMAs of pv and qk with the vector work of the softmax.
        auto iter = [&](auto par, auto masked, int t, f32x16 (&s_in)[2], f32x16 (&s_out)[2],
                        const uint4 (&p_in)[4], uint4 (&p_out)[4]) PA_INLINE {
            if constexpr (W == 4) {
                // two slots per cache, one step of lead: the loads of step t-1 (K tile t+1, V
                // tile t-1) land; every wave is done with step t-1, which last read the slots
                // of K tile t and V tile t-2
                wait_loads(0);
                __syncthreads();
                if (t + 2 < n_tiles)
                    (void)issue_span(One{}, p.k_cache, kslot(t + 2), t + 2);
                (void)issue_span(One{}, p.v_cache, vslot(t), t);
            } else if constexpr (decltype(par)::value == 1) {
                const int u = t >> 1;  // t = 2u + 1
                if constexpr (F8) {
                    write_staged();    // K tiles 2u+2, 2u+3 and V tiles 2u, 2u+1
                    __syncthreads();
                    stage(u + 1);      // K tiles 2u+4, 2u+5 and V tiles 2u+2, 2u+3
                } else {
                    wait_loads(0);     // K tiles 2u+2, 2u+3 and V tiles 2u, 2u+1 landed
                    __syncthreads();   // for every wave; every wave is done with step t-1
                    if (2 * u + 4 < n_tiles)
                        (void)issue_span(Two{}, p.k_cache, kslot(2 * u + 4), u + 2);
                }
            } else if constexpr (!F8) {
                const int u = (t >> 1) - 1;  // t = 2u + 2: V tiles 2u+2, 2u+3
                if (u >= 0 && 2 * u + 2 < n_tiles)
                    (void)issue_span(Two{}, p.v_cache, vslot(2 * u + 2), u + 1);
            }
            if (rescale) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        o[dt][v] *= alpha_prev;
            }
            // K tile t+1 (past the last tile: stale, finite) and V tile t-1 (before the first:
            // slot 3, still zero)
            const uint32_t kb = lds0 + ((t + 1) & (KS - 1)) * TILEB + k_lane;
            const uint32_t vb = lds0 + (KS + ((t - 1) & (KS - 1))) * TILEB + v_lane;
            const float alpha = region(masked, t, s_in, s_out, p_in, p_out, kb, vb);
            rescale = !__all(alpha == 1.0f);
            alpha_prev = alpha;
        };
        // Steps [t, t_end) with or without the mask, two per trip (even t first) so that S and P
        // alternate between their two register sets without copies. At entry and exit S of tile
        // t is in sa and P of tile t-1 in pb.
        int t = 0;
        auto swap_sets = [&]() PA_INLINE {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                sa[kt] = sb[kt];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                pb[c4] = pa[c4];
        };
        auto run = [&](auto masked, int t_end) PA_INLINE {
            if ((t & 1) && t < t_end) {
                iter(P1{}, masked, t, sa, sb, pb, pa);
                ++t;
                swap_sets();
            }
            for (; t + 1 < t_end; t += 2) {
                iter(P0{}, masked, t, sa, sb, pb, pa);
                iter(P1{}, masked, t + 1, sb, sa, pa, pb);
            }
            if (t < t_end) {
                iter(P0{}, masked, t, sa, sb, pb, pa);
                ++t;
                swap_sets();
            }
        };
        run(std::false_type{}, t_mask);
        run(std::true_type{}, n_tiles);
        if constexpr (F8)
            write_staged();  // V tile n_tiles-1 may be among them
        else
            wait_loads(0);
        __syncthreads();
        if (rescale) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    o[dt][v] *= alpha_prev;
        }
        const uint32_t v_last = lds0 + (KS + ((n_tiles - 1) & (KS - 1))) * TILEB + v_lane;
        pv(std::integral_constant<int, 0>{}, pb, v_last);
        pv(std::integral_constant<int, 1>{}, pb, v_last);
        pv(std::integral_constant<int, 2>{}, pb, v_last);
        pv(std::integral_constant<int, 3>{}, pb, v_last);
    }

    // ---------------------------------------------------------------- plain loop (split P)
    auto issue = [&](int t, int b) PA_INLINE {
        (void)issue_span(One{}, p.k_cache, lds + b * TILEB, t);
        (void)issue_span(One{}, p.v_cache, lds + (KS + b) * TILEB, t);
    };
    // E4M3 staging of the plain loop: this thread's K and V codes of the next tile
    uint4 k8 = make_uint4(0, 0, 0, 0), v8 = k8;
    bool have8 = false;
    auto load8 = [&](int t) PA_INLINE {
        have8 = load_codes(p.k_cache, t, k8);
        if (have8)
            (void)load_codes(p.v_cache, t, v8);
    };
    auto store8 = [&](int b) PA_INLINE {
        if (have8) {
            put_codes(lds + b * TILEB, k8);
            put_codes(lds + (KS + b) * TILEB, v8);
        }
    };
    // bfloat16 P in hi + lo parts: this loop runs only while some row of the group sees fewer
    // than kOnePartKeys keys
    constexpr bool lo_part = BF;
    if (!one_part && n_tiles > 0) {
        if constexpr (F8) {
            load8(0);
            store8(0);
        } else {
            issue(0, 0);
        }
    }
    for (int t = 0; !one_part && t < n_tiles; ++t) {
        if constexpr (!F8)
            __builtin_amdgcn_s_waitcnt(0);  // this thread's loads of tile t have landed in LDS
        __syncthreads();                // everyone's have; everyone is done with tile t-1
        if constexpr (F8) {
            if (t + 1 < n_tiles)
                load8(t + 1);  // registers: converted into the other buffer after tile t
        } else {
            if (t + 1 < n_tiles)
                issue(t + 1, (t + 1) & 1);  // lands in the other buffer while tile t is computed
        }
        const uint8_t *kb = lds + (t & 1) * TILEB;
        const uint8_t *vb = lds + (KS + (t & 1)) * TILEB;
        // the two 32-key halves are independent accumulator chains: interleave them so that no
        // MFMA waits on the one issued just before it
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                s[kt][v] = 0.0f;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const uint4 a = *(const uint4 *)(kb + (kt * 32 + n) * ROWB + (((2 * c + hh) ^ k_sw) * 16));
                s[kt] = mfma32<BF>(a, qv[c], s[kt]);
            }
        }

        const int k0 = t * kKeys;
        const bool need_mask = ragged_rows || k0 + kKeys - 1 > unmasked_below;
        if (need_mask)
            apply_mask(s, t, pos);
        float mx = s[0][0];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                mx = fmaxf(mx, s[kt][v]);
        mx = fmaxf(mx, xor_shfl(mx, 32)) * p.scale_log2;  // scale > 0 keeps the order
        const float mn = fmaxf(m_run, mx);
        const float ms = mn == -INFINITY ? 0.0f : mn;
        const float alpha = fast_exp2(m_run - ms);
        float psum = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                s[kt][v] = fast_exp2(fmaf(s[kt][v], p.scale_log2, -ms));
                psum += s[kt][v];
            }
        l_run = l_run * alpha + psum;
        m_run = mn;
        if (!__all(alpha == 1.0f)) {  // some lane's running max moved: rescale its accumulators
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    o[dt][v] *= alpha;
        }

        // P^T operands. In bfloat16 a probability keeps 8 significant bits, which on a few
        // dominant keys costs up to 2^-9 of the output's spread; bf16 P is therefore split into
        // hi + lo parts (both bf16, hi = round(p), lo = round(p - hi)) and both are multiplied, so
        // P enters the float32 accumulation with ~16 significant bits. fp16 keeps 11 bits: one part.
        uint4 pb[4], pl[4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const int kt = c4 >> 1, b = 8 * (c4 & 1);
            uint32_t *hw = &pb[c4].x, *lw = &pl[c4].x;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = s[kt][b + 2 * e], p1 = s[kt][b + 2 * e + 1];
                hw[e] = pack2<BF>(p0, p1);
                if constexpr (BF)
                    if (lo_part)
                        lw[e] = pack2<BF>(p0 - lo_f32<BF>(hw[e]), p1 - hi_f32<BF>(hw[e]));
            }
        }
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            // destination slots 0..3 hold keys 16*c4 + 4h + (0..3), slots 4..7 keys 16*c4 + 8 + 4h + (0..3)
            const int r1 = c4 * 16 + 4 * v_half + v_k, r2 = r1 + 8;
            uint4 a[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int dim = dt * 32 + v_dim;
                const int off1 = r1 * ROWB + (((dim >> 3) ^ swz<D>(r1)) << 4) + (dim & 7) * 2;
                const int off2 = r2 * ROWB + (((dim >> 3) ^ swz<D>(r2)) << 4) + (dim & 7) * 2;
                const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + off1));
                const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + off2));
                a[dt].x = __builtin_bit_cast(uint2, lo4).x;
                a[dt].y = __builtin_bit_cast(uint2, lo4).y;
                a[dt].z = __builtin_bit_cast(uint2, hi4).x;
                a[dt].w = __builtin_bit_cast(uint2, hi4).y;
            }
            // consecutive MFMAs go to different accumulators (distance DT)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                o[dt] = mfma32<BF>(a[dt], pb[c4], o[dt]);
            if constexpr (BF) {
                if (lo_part) {
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
                        o[dt] = mfma32<BF>(a[dt], pl[c4], o[dt]);
                }
            }
        }
        if constexpr (F8) {
            // the other buffer was last read in step t-1, which every wave finished before the
            // barrier of this step
            if (t + 1 < n_tiles)
                store8((t + 1) & 1);
        }
    }

    l_run = pair_sum(l_run);
    if (!row_ok)
        return;
    const float inv = l_run > 0.0f ? p.v_scale / l_run : 0.0f;
    uint16_t *dst = p.out + ((size_t)(q0 + row) * p.num_q_heads + head) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint2 w;
            w.x = pack2<BF>(o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv);
            w.y = pack2<BF>(o[dt][4 * j + 2] * inv, o[dt][4 * j + 3] * inv);
            *(uint2 *)(dst + dt * 32 + 8 * j + 4 * hh) = w;
        }
}

// E4M3 context widened for the 16-bit kernel: block i < ceil(L_s / 16) of sequence s, both caches,
// every kv head, converted exactly to the query's 16-bit type (the conversion of the register-
// staged E4M3 path) into block s * max_blocks + i of a 16-bit pool of the cache layout
// [block][kv head][16][D]. A block id outside the pool gives zeros. Rows past a sequence's end
// are converted too, but the prefill never loads them.
struct WidenParams {
    const uint8_t *__restrict__ k8;
    const uint8_t *__restrict__ v8;
    uint16_t *__restrict__ k16;
    uint16_t *__restrict__ v16;
    const int32_t *__restrict__ block_tables;
    const int32_t *__restrict__ seq_lens;
    int32_t num_seqs;
    int32_t max_blocks;
    int32_t num_blocks;
    int32_t num_kv_heads;
};

constexpr int kWidenThreads = 256;

template <bool BF, int D>
__global__ __launch_bounds__(kWidenThreads) void widen_e4m3_kernel(WidenParams w)
{
    const int sb = blockIdx.x;  // s * max_blocks + i
    const int s = sb / w.max_blocks, i = sb % w.max_blocks;
    if (s >= w.num_seqs)
        return;
    const int L = min(max(w.seq_lens[s], 0), w.max_blocks * kBlock);
    if (i * kBlock >= L)
        return;
    const int blk = w.block_tables[(size_t)s * w.max_blocks + i];
    const bool ok = (unsigned)blk < (unsigned)w.num_blocks;
    const size_t per_blk = (size_t)w.num_kv_heads * kBlock * D;  // elements of a block, all heads
    const int pieces = (int)(per_blk / 16);                        // 16-code pieces per cache
    for (int j = threadIdx.x; j < 2 * pieces; j += kWidenThreads) {
        const bool v = j >= pieces;
        const int jj = v ? j - pieces : j;
        const uint8_t *src = (v ? w.v8 : w.k8) + (size_t)blk * per_blk + (size_t)jj * 16;
        uint16_t *dst = (v ? w.v16 : w.k16) + (size_t)sb * per_blk + (size_t)jj * 16;
        const uint4 c = ok ? *(const uint4 *)src : make_uint4(0, 0, 0, 0);
        ((uint4 *)dst)[0] = make_uint4(e4m3x2_to_pk16<BF, false>(c.x), e4m3x2_to_pk16<BF, true>(c.x),
                                       e4m3x2_to_pk16<BF, false>(c.y), e4m3x2_to_pk16<BF, true>(c.y));
        ((uint4 *)dst)[1] = make_uint4(e4m3x2_to_pk16<BF, false>(c.z), e4m3x2_to_pk16<BF, true>(c.z),
                                       e4m3x2_to_pk16<BF, false>(c.w), e4m3x2_to_pk16<BF, true>(c.w));
    }
}

template <bool BF, int D, int GK>
hipError_t launch_typed(const PrefillParams &p, bool fp8, bool four, hipStream_t stream)
{
    const dim3 grid(round_up8(p.n_items));
    if (fp8)
        hipLaunchKernelGGL((prefill_kernel<BF, D, GK, false, true, 8>), grid, dim3(8 * 64), 0,
                           stream, p);
    else if (p.tree_mask)
        hipLaunchKernelGGL((prefill_kernel<BF, D, GK, true, false, 8>), grid, dim3(8 * 64), 0,
                           stream, p);
    else if (four)
        hipLaunchKernelGGL((prefill_kernel<BF, D, GK, false, false, 4>), grid, dim3(4 * 64), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((prefill_kernel<BF, D, GK, false, false, 8>), grid, dim3(8 * 64), 0,
                           stream, p);
    return hipGetLastError();
}

template <bool BF, int D>
hipError_t launch_gk(int gk, const PrefillParams &p, bool fp8, bool four, hipStream_t stream)
{
    switch (gk) {
    case 8: return launch_typed<BF, D, 8>(p, fp8, four, stream);
    case 4: return launch_typed<BF, D, 4>(p, fp8, four, stream);
    case 2: return launch_typed<BF, D, 2>(p, fp8, four, stream);
    default: return launch_typed<BF, D, 1>(p, fp8, four, stream);
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillLaunch &d, hipStream_t stream)
{
    if (d.num_seqs == 0 || d.total_q == 0 || d.max_q_len == 0)
        return hipSuccess;
    const int group = d.num_q_heads / d.c.num_kv_heads;
    const int gk = group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
    PrefillParams p;
    p.query = (const uint16_t *)d.query;
    p.k_cache = (const uint16_t *)d.k_cache;
    p.v_cache = (const uint16_t *)d.v_cache;
    p.block_tables = d.block_tables;
    p.seq_lens = d.seq_lens;
    p.cu_q_lens = d.cu_q_lens;
    p.tree_mask = d.tree_mask;
    p.out = (uint16_t *)d.out;
    p.max_blocks = d.max_blocks;
    p.num_seqs = d.num_seqs;
    p.num_kv_heads = d.c.num_kv_heads;
    p.num_q_heads = d.num_q_heads;
    p.num_blocks = d.c.num_blocks;
    p.n_sub = group / gk;
    p.total_q = d.total_q;
    bool fp8 = d.c.fp8;
    if (fp8 && d.tree_mask)
        return hipErrorInvalidValue;  // no tree mask over E4M3 caches
    p.scale_log2 = (float)((double)d.scale * (fp8 ? (double)d.k_scale : 1.0) * 1.4426950408889634);
    p.v_scale = fp8 ? d.v_scale : 1.0f;
    p.identity_blocks = 0;
    if (fp8 && d.widen_k16) {
        // widen the sequences' E4M3 blocks into the workspace, then run the 16-bit kernel on it
        WidenParams w;
        w.k8 = (const uint8_t *)d.k_cache;
        w.v8 = (const uint8_t *)d.v_cache;
        w.k16 = (uint16_t *)d.widen_k16;
        w.v16 = (uint16_t *)d.widen_v16;
        w.block_tables = d.block_tables;
        w.seq_lens = d.seq_lens;
        w.num_seqs = d.num_seqs;
        w.max_blocks = d.max_blocks;
        w.num_blocks = d.c.num_blocks;
        w.num_kv_heads = d.c.num_kv_heads;
        const int64_t n_sb = (int64_t)d.num_seqs * d.max_blocks;
        if (n_sb > 0x7fffffff)
            return hipErrorInvalidValue;
        if (d.c.bf16)
            hipLaunchKernelGGL((d.c.head_dim == 64 ? widen_e4m3_kernel<true, 64>
                                                   : widen_e4m3_kernel<true, 128>),
                               dim3((unsigned)n_sb), dim3(kWidenThreads), 0, stream, w);
        else
            hipLaunchKernelGGL((d.c.head_dim == 64 ? widen_e4m3_kernel<false, 64>
                                                   : widen_e4m3_kernel<false, 128>),
                               dim3((unsigned)n_sb), dim3(kWidenThreads), 0, stream, w);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        p.k_cache = (const uint16_t *)d.widen_k16;
        p.v_cache = (const uint16_t *)d.widen_v16;
        p.num_blocks = (int32_t)n_sb;
        p.identity_blocks = 1;
        fp8 = false;  // the 16-bit kernel, with k_scale in scale_log2 and v_scale on the output
    }
    // short contexts (every sequence's table, so its context, at most kFourWaveKeys tokens): four-
    // wave workgroups, two per CU
    const bool four = !fp8 && !d.tree_mask && (int64_t)kBlock * d.max_blocks <= kFourWaveKeys;
    const int rows_per_wg = (four ? 4 : 8) * 32 / gk;
    p.row_tiles = (d.max_q_len + rows_per_wg - 1) / rows_per_wg;
    const int64_t items = (int64_t)d.num_seqs * d.c.num_kv_heads * p.n_sub * p.row_tiles;
    if (items > 0x7ffffff0)
        return hipErrorInvalidValue;
    p.n_items = (int32_t)items;
    if (d.c.bf16)
        return d.c.head_dim == 64 ? launch_gk<true, 64>(gk, p, fp8, four, stream)
                                  : launch_gk<true, 128>(gk, p, fp8, four, stream);
    return d.c.head_dim == 64 ? launch_gk<false, 64>(gk, p, fp8, four, stream)
                              : launch_gk<false, 128>(gk, p, fp8, four, stream);
}

}  // namespace pa
