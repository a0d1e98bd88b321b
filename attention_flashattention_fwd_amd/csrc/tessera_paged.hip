// tessera_paged.hip -- gfx950 (MI355X) attention decode over a block-paged KV
// cache, and its C ABI (page "Tessera: a from-scratch distillation and
// serving stack in one repository", section "Serving: block-paged KV, batch
// recomposition, speculation": the block-paged cache, and the fused
// paged-attention decode that the pages' Status lists name as not done).
//
// Decode is bound by HBM: each cached K and V row is read once and meets only
// the few query rows of its KV head (Hq / Hkv heads times Tq new tokens, at
// most 32), about 2 flops per byte.  The design therefore aims at keeping
// enough bytes in flight, not at the matrix cores:
//   * Equal shares.  The 32-key tiles of a KV head, over all sequences one
//     after another, are cut into equal contiguous shares, one per wave of a
//     fixed set (1536 one-wave workgroups, six per CU, 2048 at D=32, all
//     resident at once), so every wave streams the same number of bytes and all of them
//     finish together: no wave waits behind a long sequence, and no
//     workgroup is launched for nothing.  A wave computes all query rows of
//     its KV head over each piece of a sequence in its share with an online
//     softmax.  A piece that is a whole sequence writes the result; the
//     others write their normalised partial output and log2-sum-exp to the
//     workspace, and a second kernel merges them:
//     O = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M).
//   * Each wave streams its keys through its own small ring of LDS stages
//     (32 keys of K and of V per stage, one or two stages) with direct
//     non-temporal global->LDS loads, issued as soon as a stage is free, and
//     no barrier: a wave only ever reads what it loaded itself.  The rings
//     are kept small so that many waves share a CU: the bytes in flight come
//     from the number of waves.  The block table is read 64 entries at a time
//     into a register (one entry per lane), a window ahead; the base address
//     of every 16-key half-tile is a scalar taken from it, so a half-tile
//     load is one contiguous 16-row piece of one block.
//   * Both products run on v_mfma_f32_32x32x16_bf16 in the transposed form
//     of the prefill kernel, S^T = K Q^T and O^T = V^T P^T, with the query
//     rows of the KV head as the 32 columns (unused columns hold zero
//     queries and are dropped); the LDS layout, swizzle and operand reads are
//     those of the prefill kernel for a 32-key tile.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "tessera_paged.h"
#include "launch.h"
#include "lds_poison.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLn2 = 0.693147180559945309f;
constexpr double kLog2e = 1.442695040888963407;
constexpr int kTileKeys = 32;          // keys per LDS stage
constexpr int kMaxCols = 32;           // query rows per (sequence, KV head)
constexpr int kWindow = 64;            // table entries held at once: one per lane
// Waves per call: six per CU of 256 (eight at D=32, whose waves are small
// enough to fit more; measured 105 -> 92 us on the serving batch, no gain at
// D=64 or D=128).
constexpr int stream_waves(int D) { return D == 32 ? 2048 : 1536; }
constexpr uint32_t kBadBits = 0x7fc00000u;    // quiet NaN: marks bad table data
constexpr uint16_t kBadBf16 = 0x7fc0u;

// LDS ring stages per wave: one 32-key stage of K and V at D=128 and D=64
// (16 KB and 8 KB), two at D=32 (8 KB).  What sets the decode's bandwidth is
// how many waves stream at once, not how deep one wave's ring is: measured on
// this kernel, one 16 KB stage per wave (eight waves per CU) reads faster
// than two (32 KB, four waves per CU), and at D=64 and D=32 the small rings
// are 12% and 50% faster than 32 KB ones.
template <int D>
constexpr int ring_stages() {
    return D == 32 ? 2 : 1;
}

// The prefill kernel's 16-byte chunk swizzles (they depend on key % 8 and
// key % 16 only, so they hold for any 16-row piece).
template <int D>
__device__ __forceinline__ int swz_k(int key) {
    if constexpr (D == 128) return key & 15;
    else if constexpr (D == 64) return (key >> 1) & 7;
    else return (key >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int swz_v(int key) {
    if constexpr (D == 128) return ((key & 3) << 2) | (((key >> 2) & 1) << 1);
    else if constexpr (D == 64) return ((key >> 1) & 1) << 2;
    else return 0;
}

struct PagedArgs {
    const uint16_t *q, *kc, *vc;
    const int32_t *table, *lens;
    uint16_t *o;
    float *lse;
    float *ws_lse;   // [Hkv, nslot, M] log2-sum-exp of each piece
    float *ws_o;     // [Hkv, nslot, M, D] normalised partial output of each piece
    int *meta;       // [B, Hkv, 2] ranks of a sequence's first and last pieces
    int B, Hq, Hkv, G, Tq, M;    // M = G * Tq query rows per KV head
    int bs, max_blocks, num_blocks;
    int wg;          // waves per KV head
    int nslot;       // piece slots per KV head: wg + B
    int causal;
    int qmode;       // 0: q as given, 1: q negated (scale < 0), 2: q zeroed (scale == 0)
    float c;         // |scale| * log2(e)  (1 when scale == 0)
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// A wave-uniform pointer in scalar registers.  The base of every load below
// is uniform by construction; this states it for the compiler, whose
// divergence analysis does not always see it.
__device__ __forceinline__ const char *uniform_ptr(const char *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const char *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// One 16-byte global->LDS load per lane (base + voff -> lds + 16 * lane),
// untracked by the compiler: the kernel waits for it with an explicit vmcnt.
// The s_nop covers the M0-write hazard before the load.  The load is
// non-temporal: every cached row is read exactly once, and streaming it past
// the caches reads about 10% faster than the default policy.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds) {
    lds_poison_lane16(lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(uniform_ptr((const char *)base)), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Waits until at most N of this wave's vector memory loads are outstanding
// (loads complete in issue order); also a compiler barrier for memory.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// max(x, x of lane l ^ 32): a swap of the wave's halves, without LDS.
__device__ __forceinline__ float max_with_partner(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Row sums on the matrix cores from the bf16 P, as in the prefill kernel: a
// 16x16x32 MFMA of this selector with the P^T operand leaves the sum of query
// n in the even rows of column n and that of query n + 16 in the odd rows, so
// a lane finds its own query's sum in entry (lane / 16) % 2.
__device__ __forceinline__ bf16x8 row_sum_selector(int lane) {
    const __bf16 x = ((lane ^ (lane >> 4)) & 1) == 0 ? (__bf16)1.0f : (__bf16)0.0f;
    return bf16x8{x, x, x, x, x, x, x, x};
}

// Tiles of 32 keys in a sequence of n tokens; none for a length out of range
// (the merge writes NaN for such a sequence).
__device__ __forceinline__ int tiles_of(const PagedArgs &a, int n) {
    return (n >= 0 && n <= a.max_blocks * a.bs) ? (n + kTileKeys - 1) / kTileKeys : 0;
}

// One wave per workgroup, blockIdx.x = rank * Hkv + KV head.  The work of a KV
// head is the list of every sequence's 32-key tiles, sequence after sequence
// (T tiles); wave `rank` of the head takes the contiguous share
// [rank T / W, (rank + 1) T / W) with W = min(wg, T), so every wave has the
// same number of tiles to stream and all of them finish together.  A share
// holds pieces of one or more sequences.  A wave whose piece is a whole
// sequence writes out and lse itself; otherwise it writes the piece's
// normalised partial output and log2-sum-exp to slot rank + sequence of its
// KV head (shares are ordered like the sequences, so no two pieces share a
// slot), and the wave holding the sequence's first tile records the ranks of
// its first and last pieces for the merge.
template <int D>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) paged_decode_kernel(PagedArgs a) {
    constexpr int R = ring_stages<D>();
    constexpr int kRowBytes = 2 * D;
    constexpr int kTileBytes = kTileKeys * kRowBytes;   // one K or V tile
    constexpr int kLoads = kTileBytes / 1024;           // 1 KB loads per tile
    constexpr int kHalfLoads = kLoads / 2;              // ... per 16-key half
    constexpr int kCpr = D / 8;                         // 16-byte chunks per row
    constexpr int kKeysPerLoad = 64 / kCpr;
    static_assert((R - 1) * 2 * kLoads <= 63, "loads in flight exceed the vmcnt range");
    __shared__ __attribute__((aligned(16))) char lds[R][2][kTileBytes];
    lds_poison_all();

    const int lane = threadIdx.x;
    const int col = lane & 31, hi = lane >> 5;
    const int g = (int)(blockIdx.x % (unsigned)a.Hkv);
    const int rank = (int)(blockIdx.x / (unsigned)a.Hkv);

    // Tiles per sequence: lane l adds up sequences [l seg, (l + 1) seg), and a
    // scan over the lanes gives the first tile of each lane's sequences.
    const int seg = (a.B + 63) / 64;
    int mine = 0;
    for (int i = 0; i < seg; ++i) {
        const int bb = lane * seg + i;
        if (bb < a.B) mine += tiles_of(a, a.lens[bb]);
    }
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    const int total = __shfl(incl, 63);
    const int waves = min(a.wg, total);
    if (rank >= waves) return;
    const int t_lo = (int)((int64_t)rank * total / waves);
    const int t_hi = (int)((int64_t)(rank + 1) * total / waves);

    // The sequence holding tile t_lo: first the lane, then among its sequences.
    const int excl = incl - mine;
    const uint64_t own = __builtin_amdgcn_ballot_w64(mine > 0 && excl <= t_lo && t_lo < incl);
    const int owner = (int)__builtin_ctzll(own);
    int b = owner * seg;
    int pos = __builtin_amdgcn_readlane(excl, owner);   // first tile of sequence b
    for (;;) {
        const int nt = tiles_of(a, a.lens[b]);
        if (pos + nt > t_lo) break;
        pos += nt;
        ++b;
    }

    // Per-lane byte offsets of the loads of one 16-key half (rows relative to
    // the half's first row).  Load r of a tile fills LDS slots [64r, 64r + 64)
    // (16 bytes each, slot p by lane p % 64): slot p is row p / kCpr, physical
    // chunk p % kCpr, which holds logical chunk (p % kCpr) ^ swizzle(row).
    uint32_t koff[kHalfLoads], voff[kHalfLoads];
#pragma unroll
    for (int r = 0; r < kHalfLoads; ++r) {
        const int key = r * kKeysPerLoad + lane / kCpr;   // 0 .. 15
        const int c = lane % kCpr;
        koff[r] = key * kRowBytes + ((c ^ swz_k<D>(key)) << 4);
        voff[r] = key * kRowBytes + ((c ^ swz_v<D>(key)) << 4);
    }
    // LDS operand offsets (as in the prefill kernel).  K: lane (col, hi) reads
    // 16 bytes of key row col, dims 16*ks + 8*hi .. +7.  V: transposing 8-byte
    // reads; for 16-key step st and dim block db, lane (grp, s16) reads key
    // rows 16*st + 4*hi + s16/4 and 8 rows further, dims 32*db + 16*(grp&1) +
    // 4*(s16&3) .. +3, which after the transpose are 8 keys of one dim in the
    // order of the lane's S^T rows.
    int kread[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        kread[ks] = col * kRowBytes + (((2 * ks + hi) ^ swz_k<D>(col)) << 4);
    int vread[D / 32];
    {
        const int grp = lane >> 4, s16 = lane & 15;
        const int r = 4 * hi + (s16 >> 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int d = 32 * db + 16 * (grp & 1) + 4 * (s16 & 3);
            vread[db] = r * kRowBytes + (((d >> 3) ^ swz_v<D>(r)) << 4) + (d & 7) * 2;
        }
    }
    const float c = a.c;
    const bf16x8 sumsel = row_sum_selector(lane);
    const int qi = col < a.M ? col % a.Tq : a.Tq - 1;

    int t = t_lo;
    int k0 = t_lo - pos;   // first tile of the piece within sequence b
    while (t < t_hi) {
        const int n = a.lens[b];
        const int nt = tiles_of(a, n);
        if (nt == 0) {   // only between pieces: an empty sequence has no tiles
            ++b;
            continue;
        }
        const int k1 = min(nt, k0 + (t_hi - t));
        const int ntl = k1 - k0;
        const int start = k0 * kTileKeys;
        const int end = min(k1 * kTileKeys, n);

        // Q fragments (B operand of S^T = K Q^T): lane (col, hi) holds dims
        // 16*ks + 8*hi .. +7 of query row col of this KV head, rows >= M zero.
        const int64_t qrow0 = ((int64_t)b * a.Hq + (int64_t)g * a.G) * a.Tq;
        bf16x8 qf[D / 16];
        {
            const uint32_t flip = a.qmode == 1 ? 0x80008000u : 0u;
            const uint32_t keep = (a.qmode == 2 || col >= a.M) ? 0u : 0xffffffffu;
            const uint16_t *src = a.q + (qrow0 + min(col, a.M - 1)) * D + 8 * hi;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const u32x4 raw = *(const u32x4 *)(src + 16 * ks);
                qf[ks] = __builtin_bit_cast(bf16x8, (raw ^ flip) & keep);
            }
            // Take the fragments here: the compiler does not see the K/V loads
            // below, and would otherwise wait for all of them before the first use.
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(qf[ks]));
        }

        // The piece's table entries, 64 at a time (one per lane): the current
        // window and the next one, loaded a window ahead.  An entry out of
        // range marks the piece bad (its output is NaN) and is read as a valid
        // block, so that no load leaves the cache.
        const int blast = (end - 1) / a.bs;   // last block of the piece
        const int64_t trow = (int64_t)b * a.max_blocks;
        int wbase = start / a.bs;
        auto window = [&](int base) __attribute__((always_inline)) {
            return base + lane <= blast ? a.table[trow + base + lane] : 0;
        };
        auto bad_in = [&](int e, int base) __attribute__((always_inline)) {
            return __builtin_amdgcn_ballot_w64(base + lane <= blast &&
                                               (e < 0 || e >= a.num_blocks)) != 0;
        };
        int ent = window(wbase);
        int ent_nx = wbase + kWindow <= blast ? window(wbase + kWindow) : 0;
        bool bad = bad_in(ent, wbase);
        auto block_at = [&](int key) __attribute__((always_inline)) {
            const int rel = key / a.bs - wbase;
            const int e = rel < kWindow ? __builtin_amdgcn_readlane(ent, rel)
                                        : __builtin_amdgcn_readlane(ent_nx, rel - kWindow);
            return min(max(e, 0), a.num_blocks - 1);
        };

        // Loads tile i of the piece into stage `st`.  Each 16-key half lies in
        // one block.  Rows at or past `end` are clamped to the last row that
        // holds a token (a half with none reads the first half's rows): they
        // meet only masked scores, and stay finite so that a zero weight
        // keeps them out.
        auto issue = [&](int i, int st) __attribute__((always_inline)) {
            const int t0 = start + i * kTileKeys;
            if (t0 / a.bs - wbase >= kWindow) {   // the next window becomes current
                wbase += kWindow;
                ent = ent_nx;
                bad |= bad_in(ent, wbase);
                ent_nx = wbase + kWindow <= blast ? window(wbase + kWindow) : 0;
            }
            const char *kb[2], *vb[2];
            int lastrow[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int th = t0 + 16 * h;
                if (h == 0 || th < end) {
                    const int blk = block_at(th);
                    const int64_t e = (((int64_t)blk * a.Hkv + g) * a.bs + th % a.bs) * D;
                    kb[h] = (const char *)(a.kc + e);
                    vb[h] = (const char *)(a.vc + e);
                    lastrow[h] = min(15, end - 1 - th);
                } else {
                    kb[h] = kb[0];
                    vb[h] = vb[0];
                    lastrow[h] = lastrow[0];
                }
            }
            const bool full = t0 + kTileKeys <= end;
            const uint32_t kdst = (uint32_t)(uintptr_t)(LDS_AS char *)lds[st][0];
            const uint32_t vdst = (uint32_t)(uintptr_t)(LDS_AS char *)lds[st][1];
            // The stage's last LDS reads (the previous tile in it) have returned.
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int r = 0; r < kLoads; ++r) {
                const int h = r / kHalfLoads;
                uint32_t ko = koff[r % kHalfLoads], vo = voff[r % kHalfLoads];
                if (!full) {
                    const int key = (int)(ko / kRowBytes);
                    const uint32_t back = (uint32_t)(key - min(key, lastrow[h])) * kRowBytes;
                    ko -= back;
                    vo -= back;
                }
                dma16(kb[h], ko, kdst + 1024 * r);
                dma16(vb[h], vo, vdst + 1024 * r);
            }
        };

        const int pre = min(R, ntl);
        for (int i = 0; i < pre; ++i) issue(i, i);

        // The visible tokens of this lane's query row: 0 .. kend - 1.
        const int kend = a.causal ? n - a.Tq + qi + 1 : n;
        const int mask_from = a.causal ? n - a.Tq + 1 : n;   // smallest kend of the rows

        f32x16 acc[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
        float m_run = -INFINITY;   // running max of c * s (log2 units)
        f32x4 lsum = f32x4{};      // row sums: entry (lane / 16) % 2 is this lane's

        for (int i = 0; i < ntl; ++i) {
            const int st = i % R;
            if (i + R <= ntl) wait_vmcnt<(R - 1) * 2 * kLoads>();
            else wait_vmcnt<0>();
            const LDS_AS char *kt = (const LDS_AS char *)lds[st][0];
            const LDS_AS char *vt = (const LDS_AS char *)lds[st][1];

            f32x16 sc = f32x16{};
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                sc = mfma32(*(const LDS_AS bf16x8 *)(kt + kread[ks]), qf[ks], sc);

            // Row e of this lane's S^T is key t0 + 8*(e/4) + 4*hi + e%4.
            const int t0 = start + i * kTileKeys;
            if (t0 + kTileKeys > mask_from) {
                const int last = kend - 1 - t0 - 4 * hi;
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (8 * (e >> 2) + (e & 3) > last) sc[e] = -INFINITY;
            }

            // Online softmax in log2 units; the accumulators are rescaled only
            // when some row's maximum grew.
            float mt = sc[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) mt = fmaxf(mt, sc[e]);
            const float m_new = fmaxf(m_run, max_with_partner(mt) * c);
            if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
                const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
                lsum[0] *= alpha;
                lsum[1] *= alpha;
                m_run = m_new;
            }
            const float m_use = m_run == -INFINITY ? 0.f : m_run;
            u32x4 pu[2];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * e], c, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * e + 1], c, -m_use));
                const bf16x2 p = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
                pu[e >> 2][e & 3] = __builtin_bit_cast(uint32_t, p);
            }
            lsum = mfma16(sumsel, __builtin_bit_cast(bf16x8, pu[0]), lsum);
            lsum = mfma16(sumsel, __builtin_bit_cast(bf16x8, pu[1]), lsum);
#pragma unroll
            for (int step = 0; step < 2; ++step) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const LDS_AS char *p = vt + vread[db] + step * 16 * kRowBytes;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)p);
                    const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (LDS_AS i16x4 *)(p + 8 * kRowBytes));
                    const bf16x8 vop = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
                    acc[db] = mfma32(vop, __builtin_bit_cast(bf16x8, pu[step]), acc[db]);
                }
            }
            if (i + R < ntl) issue(i + R, st);
        }
        // No load may still write this wave's LDS when the next piece starts.
        wait_vmcnt<0>();
        // The last tile's second half may have used the next window.
        if (wbase + kWindow <= blast) bad |= bad_in(ent_nx, wbase + kWindow);

        const bool whole = k0 == 0 && k1 == nt;
        if (k0 == 0 && lane == 0) {
            const int pe = pos + nt;   // one past the sequence's last tile
            const int last = whole ? rank : min(waves - 1, (int)(((int64_t)pe * waves - 1) / total));
            a.meta[2 * (b * a.Hkv + g)] = rank;
            a.meta[2 * (b * a.Hkv + g) + 1] = last;
        }
        if (col < a.M) {
            const float l = ((lane >> 4) & 1) ? lsum[1] : lsum[0];
            const float inv = l > 0.f ? 1.f / l : 0.f;
            const float lse2 = l > 0.f ? m_run + log2f(l) : -INFINITY;
            const int64_t row = qrow0 + col;
            if (whole) {
                uint16_t *dst = a.o + row * D;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        f32x4 x;
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * g4 + e] * inv;
                        bf16x4 y = __builtin_convertvector(x, bf16x4);
                        if (bad)
                            y = __builtin_bit_cast(bf16x4, u16x4{kBadBf16, kBadBf16, kBadBf16, kBadBf16});
                        *(bf16x4 *)(dst + 32 * db + 8 * g4 + 4 * hi) = y;
                    }
                }
                if (hi == 0) a.lse[row] = bad ? __uint_as_float(kBadBits) : lse2 * kLn2;
            } else {
                const int64_t cell = ((int64_t)g * a.nslot + rank + b) * a.M + col;
                if (!bad) {
                    float *dst = a.ws_o + cell * D;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            f32x4 x;
#pragma unroll
                            for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * g4 + e] * inv;
                            *(f32x4 *)(dst + 32 * db + 8 * g4 + 4 * hi) = x;
                        }
                    }
                }
                if (hi == 0) a.ws_lse[cell] = bad ? __uint_as_float(kBadBits) : lse2;
            }
        }
        t += ntl;
        pos += nt;
        ++b;
        k0 = 0;
    }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

// Merges the pieces of every query row: one wave per row, four rows per
// workgroup.  It also writes the rows no decode wave wrote: an empty sequence
// (out 0, lse -inf) and a length out of range (NaN).  Lane s first takes
// piece s's log2-sum-exp (64 pieces at a time), so the weights cost one load
// per lane; the partial rows are then read eight pieces at a time, all eight
// loads in flight together.  The sums run over the pieces in order, as in
// the formula O = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M).
template <int D>
__global__ void __launch_bounds__(256) paged_combine_kernel(PagedArgs a, int64_t rows) {
    constexpr int kPer = D / 64 > 0 ? D / 64 : 1;   // dims per lane
    constexpr int kUnroll = 8;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int64_t per_seq = (int64_t)a.Hq * a.Tq;
    const int b = (int)(row / per_seq);
    const int hq = (int)((row - b * per_seq) / a.Tq);
    const int g = hq / a.G;
    const int m = (int)(row - b * per_seq) - g * a.M;   // row within the KV head's M
    const int n = a.lens[b];
    uint16_t *dst = a.o + row * D;
    const bool len_ok = n >= 0 && n <= a.max_blocks * a.bs;
    if (!len_ok || n == 0) {
#pragma unroll
        for (int k = 0; k < (D + 63) / 64; ++k)
            if (lane + 64 * k < D) dst[lane + 64 * k] = len_ok ? 0 : kBadBf16;
        if (lane == 0) a.lse[row] = len_ok ? -INFINITY : __uint_as_float(kBadBits);
        return;
    }
    const int first = a.meta[2 * (b * a.Hkv + g)];
    const int last = a.meta[2 * (b * a.Hkv + g) + 1];
    if (first == last) return;   // one piece: its wave wrote the result
    const int np = last - first + 1;
    const int64_t cell0 = ((int64_t)g * a.nslot + first + b) * a.M + m;
    const float *pl = a.ws_lse + cell0;   // piece s at pl[s * M]
    float mx = -INFINITY;
    bool bad = false;
    for (int s = lane; s < np; s += 64) {
        const float x = pl[(int64_t)s * a.M];
        bad |= __float_as_uint(x) == kBadBits;
        mx = fmaxf(mx, x);
    }
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
#pragma unroll
        for (int k = 0; k < (D + 63) / 64; ++k)
            if (lane + 64 * k < D) dst[lane + 64 * k] = kBadBf16;
        if (lane == 0) a.lse[row] = __uint_as_float(kBadBits);
        return;
    }
    mx = wave_max(mx);
    const float m_use = mx == -INFINITY ? 0.f : mx;
    // Lane d0 = kPer * lane holds dims d0 .. d0 + kPer - 1 (at D=32 the upper
    // half of the wave reads dims of its own row again and stores nothing).
    const int d0 = (kPer * lane) % D;
    const int64_t ostride = (int64_t)a.M * D;   // floats from one piece's row to the next's
    const float *src0 = a.ws_o + cell0 * D + d0;
    float o[kPer] = {};
    float wsum = 0.f;
    for (int c0 = 0; c0 < np; c0 += 64) {
        const int cnt = min(64, np - c0);
        const float wl =
            lane < cnt ? __builtin_amdgcn_exp2f(pl[(int64_t)(c0 + lane) * a.M] - m_use) : 0.f;
        int j = 0;
        for (; j + kUnroll <= cnt; j += kUnroll) {
            float x[kUnroll][kPer];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const float *p = src0 + (int64_t)(c0 + j + u) * ostride;
                if constexpr (kPer == 2) {
                    const f32x2 v = *(const f32x2 *)p;
                    x[u][0] = v[0];
                    x[u][1] = v[1];
                } else {
                    x[u][0] = *p;
                }
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const float w = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wl), j + u));
                wsum += w;
#pragma unroll
                for (int k = 0; k < kPer; ++k) o[k] = __builtin_fmaf(w, x[u][k], o[k]);
            }
        }
        for (; j < cnt; ++j) {
            const float *p = src0 + (int64_t)(c0 + j) * ostride;
            const float w = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wl), j));
            wsum += w;
#pragma unroll
            for (int k = 0; k < kPer; ++k) o[k] = __builtin_fmaf(w, p[k], o[k]);
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    if (kPer * lane < D) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const __bf16 y = (__bf16)(o[k] * inv);
            dst[d0 + k] = __builtin_bit_cast(uint16_t, y);
        }
    }
    if (lane == 0) a.lse[row] = wsum > 0.f ? (mx + log2f(wsum)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Waves per KV head: stream_waves(D) in all, at least one per head, and no
// more than the most tiles a head can have (B sequences of max_blocks *
// block_size tokens), so that small calls get a small grid and workspace.
int waves_per_head(int B, int Hkv, int D, int block_size, int max_blocks) {
    const int64_t tiles = (int64_t)B * (((int64_t)max_blocks * block_size + 31) / 32);
    int64_t w = stream_waves(D) / Hkv;
    w = w < tiles ? w : tiles;
    return w > 1 ? (int)w : 1;
}

// The workspace: the log2-sum-exp of every piece slot (fp32, padded to 256
// bytes), the normalised partial outputs (fp32 x D), and two ints per
// (sequence, KV head) for the merge (padded to 256 bytes).
struct Layout {
    int wg, nslot;
    int64_t o_off, meta_off, bytes;
};

Layout layout_for(int B, int Hq, int Hkv, int Tq, int D, int block_size, int max_blocks) {
    Layout l;
    l.wg = waves_per_head(B, Hkv, D, block_size, max_blocks);
    l.nslot = l.wg + B;
    const int64_t cells = (int64_t)Hkv * l.nslot * (Hq / Hkv) * Tq;
    l.o_off = (cells * 4 + 255) / 256 * 256;
    l.meta_off = l.o_off + cells * D * 4;
    l.bytes = l.meta_off + ((int64_t)B * Hkv * 8 + 255) / 256 * 256;
    return l;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

// The size checks shared by both entry points.
int check_sizes(int B, int Hq, int Hkv, int Tq, int D, int block_size, int max_blocks) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || block_size < 1 || max_blocks < 1 ||
        Hq % Hkv != 0)
        return TESSERA_ERR_SHAPE;
    if (D != 32 && D != 64 && D != 128) return TESSERA_ERR_UNSUPPORTED;
    if ((int64_t)(Hq / Hkv) * Tq > kMaxCols || block_size % 16 != 0)
        return TESSERA_ERR_UNSUPPORTED;
    const int64_t cap = (int64_t)max_blocks * block_size;
    if (cap > 0x7fffffff) return TESSERA_ERR_TOO_LARGE;
    // the tiles of one KV head, and the (sequence, KV head) records, count in int
    if ((int64_t)B * ((cap + 31) / 32) > 0x7fffffff || (int64_t)B * Hkv * 2 > 0x7fffffff)
        return TESSERA_ERR_TOO_LARGE;
    return TESSERA_OK;
}

}  // namespace

extern "C" long long tessera_paged_decode_workspace(int B, int Hq, int Hkv, int Tq, int D,
                                                    int block_size, int max_blocks) {
    const int st = check_sizes(B, Hq, Hkv, Tq, D, block_size, max_blocks);
    if (st != TESSERA_OK) return -(long long)st;
    return layout_for(B, Hq, Hkv, Tq, D, block_size, max_blocks).bytes;
}

// ---------------------------------------------------------------------------
// The decode without a caller workspace: the partial results go to `scratch`, a
// fixed buffer of the library in each GPU's memory (every GPU the library runs
// on holds its own copy until the process ends).  In host code the array's
// name is only a stand-in for it; the device address of the current GPU's
// copy is looked up once per device with hipGetSymbolAddress and kept, and
// only that address is ever handed to a kernel.  Calls on one GPU share the
// buffer: two of them that overlap in time (other streams, other threads)
// race on it.  Its contents on entry do not matter (every cell the merge
// reads is written by the decode kernel of the same call), so nothing clears
// it.
// ---------------------------------------------------------------------------
constexpr long long kScratchBytes = 32ll << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// The device address of the current GPU's scratch, looked up on first use.
int scratch_of_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return tessera_launch_result(e);
    if (dev < 0 || dev >= kMaxDevices) return TESSERA_ERR_UNSUPPORTED;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e == hipSuccess && !p) e = hipErrorInvalidSymbol;
            if (e != hipSuccess) return tessera_launch_result(e);
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return TESSERA_OK;
}

// The body of both decode entry points: checks, then the two launches.
// With use_scratch, the library's scratch buffer of the current GPU takes the
// place of the caller's workspace (which is then ignored), looked up only
// once every argument has passed its checks.
int paged_decode(const void *q, const void *k_cache, const void *v_cache, const int *block_table,
                 const int *context_lens, void *out, float *lse, int B, int Hq, int Hkv, int Tq,
                 int D, int num_blocks, int block_size, int max_blocks, int causal, float scale,
                 void *workspace, long long workspace_bytes, bool use_scratch, void *stream) {
    if (use_scratch) {
        workspace = nullptr;
        workspace_bytes = 0;
    }
    if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out || !lse)
        return TESSERA_ERR_NULL;
    if (num_blocks < 1) return TESSERA_ERR_SHAPE;
    int st = check_sizes(B, Hq, Hkv, Tq, D, block_size, max_blocks);
    if (st != TESSERA_OK) return st;
    if (causal != 0 && causal != 1) return TESSERA_ERR_CAUSAL;
    if (!isfinite(scale)) return TESSERA_ERR_SCALE;
    if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out |
         (uintptr_t)workspace) & 15u)
        return TESSERA_ERR_ALIGN;
    if (((uintptr_t)lse | (uintptr_t)block_table | (uintptr_t)context_lens) & 3u)
        return TESSERA_ERR_ALIGN;
    const Layout lay = layout_for(B, Hq, Hkv, Tq, D, block_size, max_blocks);
    const int64_t need = lay.bytes;
    if (use_scratch && need > kScratchBytes) return TESSERA_ERR_SCRATCH;
    if (!use_scratch && (!workspace || workspace_bytes < need)) return TESSERA_ERR_WORKSPACE;
    const size_t rows = (size_t)B * Hq * Tq;
    const size_t qbytes = rows * D * 2, lbytes = rows * 4;
    const size_t cbytes = (size_t)num_blocks * Hkv * block_size * D * 2;
    const size_t tbytes = (size_t)B * max_blocks * 4, nbytes = (size_t)B * 4;
    const size_t wbytes = workspace ? (size_t)need : 0;   // the library scratch: no overlap
    const void *ins[5] = {q, k_cache, v_cache, block_table, context_lens};
    const size_t insz[5] = {qbytes, cbytes, cbytes, tbytes, nbytes};
    for (int i = 0; i < 5; ++i)
        if (overlaps(out, qbytes, ins[i], insz[i]) || overlaps(lse, lbytes, ins[i], insz[i]) ||
            overlaps(workspace, wbytes, ins[i], insz[i]))
            return TESSERA_ERR_ALIAS;
    if (overlaps(out, qbytes, lse, lbytes) || overlaps(out, qbytes, workspace, wbytes) ||
        overlaps(lse, lbytes, workspace, wbytes))
        return TESSERA_ERR_ALIAS;
    if (use_scratch) {
        st = scratch_of_current_device(&workspace);
        if (st != TESSERA_OK) return st;
    }

    PagedArgs a;
    a.q = (const uint16_t *)q;
    a.kc = (const uint16_t *)k_cache;
    a.vc = (const uint16_t *)v_cache;
    a.table = block_table;
    a.lens = context_lens;
    a.o = (uint16_t *)out;
    a.lse = lse;
    a.ws_lse = (float *)workspace;
    a.ws_o = (float *)((char *)workspace + lay.o_off);
    a.meta = (int *)((char *)workspace + lay.meta_off);
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.Tq = Tq;
    a.M = a.G * Tq;
    a.bs = block_size;
    a.max_blocks = max_blocks;
    a.num_blocks = num_blocks;
    a.wg = lay.wg;
    a.nslot = lay.nslot;
    a.causal = causal;
    a.qmode = scale < 0.f ? 1 : (scale == 0.f ? 2 : 0);
    a.c = scale == 0.f ? 1.0f : (float)(fabs((double)scale) * kLog2e);

    hipStream_t sm = (hipStream_t)stream;
    const dim3 grid((unsigned)((int64_t)lay.wg * Hkv)), blk(64);
    if (D == 128) st = tessera_launch(paged_decode_kernel<128>, grid, blk, sm, a);
    else if (D == 64) st = tessera_launch(paged_decode_kernel<64>, grid, blk, sm, a);
    else st = tessera_launch(paged_decode_kernel<32>, grid, blk, sm, a);
    if (st != TESSERA_OK) return st;
    const int64_t nrows = (int64_t)rows;
    const dim3 cgrid((unsigned)((nrows + 3) / 4)), cblk(256);
    if (D == 128) return tessera_launch(paged_combine_kernel<128>, cgrid, cblk, sm, a, nrows);
    if (D == 64) return tessera_launch(paged_combine_kernel<64>, cgrid, cblk, sm, a, nrows);
    return tessera_launch(paged_combine_kernel<32>, cgrid, cblk, sm, a, nrows);
}

}  // namespace

extern "C" int tessera_paged_decode(const void *q, const void *k_cache, const void *v_cache,
                                    const int *block_table, const int *context_lens, void *out,
                                    float *lse, int B, int Hq, int Hkv, int Tq, int D,
                                    int num_blocks, int block_size, int max_blocks, int causal,
                                    float scale, void *workspace, long long workspace_bytes,
                                    void *stream) {
    return paged_decode(q, k_cache, v_cache, block_table, context_lens, out, lse, B, Hq, Hkv, Tq,
                        D, num_blocks, block_size, max_blocks, causal, scale, workspace,
                        workspace_bytes, false, stream);
}

extern "C" long long tessera_paged_decode_scratch_limit(void) { return kScratchBytes; }

extern "C" int tessera_paged_decode_noalloc(const void *q, const void *k_cache,
                                            const void *v_cache, const int *block_table,
                                            const int *context_lens, void *out, float *lse, int B,
                                            int Hq, int Hkv, int Tq, int D, int num_blocks,
                                            int block_size, int max_blocks, int causal,
                                            float scale, void *stream) {
    return paged_decode(q, k_cache, v_cache, block_table, context_lens, out, lse, B, Hq, Hkv, Tq,
                        D, num_blocks, block_size, max_blocks, causal, scale, nullptr, 0, true,
                        stream);
}
