// tessera_attn.hip -- gfx950 (MI355X) kernels and C ABI for the attention
// forward pass with online softmax, causal masking and grouped-query attention
// (page "Tessera: a from-scratch distillation and serving stack in one
// repository", section "The kernel set and its torch fallback").
//
// The kernel:
//   * attn_fwd_bf16_kernel -- the hot path.  Both contractions (Q K^T and P V)
//     run on v_mfma_f32_32x32x16_bf16 in a transposed form, S^T = K Q^T and
//     O^T = V^T P^T, so that every lane owns one query row: the softmax row
//     statistics live in a lane (plus its partner lane 32 away) instead of
//     being spread over the wave.  K/V tiles are staged through a four-deep
//     LDS ring, and one staged tile serves the query heads of a GQA group.
// The fp32 kernel (tessera_attn_fwd_f32) is in tessera_attn_f32.hip.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <utility>

#include "tessera_attn.h"
#include "launch.h"
#include "lds_poison.h"

#define TESSERA_VERSION 10200

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLn2 = 0.693147180559945309f;
constexpr double kLog2e = 1.442695040888963407;

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
constexpr int kWaves = 8;                 // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kKeyTile = 64;              // keys per staged K/V tile
// The running maximum m is lazy: P = 2^(s*c - m) is computed with the m in
// hand, and m is only raised when some p of the tile reaches 2.  A raise sets
// m to the tile max plus kHeadroom, so every p is then at most 2^-kHeadroom and
// the next raise waits until a score exceeds that max by kHeadroom + 1 (log2
// units).  Any stale m gives the same result: it cancels between the
// numerator and the row sum.  No p that reaches the matrix cores exceeds 2,
// so the fp32 sums over up to 2^31 keys cannot overflow, and the row's largest
// p stays at least 2^-(kHeadroom+1), so the sums keep full precision.  The
// test needs no max: p >= 2 exactly when bit 14 of its bf16 code is set, so one
// OR over the packed P words decides it.
constexpr int kHeadroom = 32;

// LDS chunk swizzles (16-byte chunks of a D-wide bf16 row).  K is read as
// 16-byte MFMA operands, one key row per lane; V is read with transposing
// 8-byte reads, eight key rows per quarter-wave.  Each XOR spreads the rows a
// read touches over distinct LDS banks.
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

struct Bf16Args {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int Hq, Hkv, G;
    int Tq, Tk;   // query rows and key rows per head
    int qoff;     // query row i stands at key position i + qoff (qoff = Tk - Tq)
    int hg;       // heads of one GQA group handled by a workgroup
    int nqb;      // 32-row query blocks per workgroup (kWaves / hg)
    int nslots;   // workgroups sharing one (query tile, KV head): G / hg
    int nbh;      // B * Hkv
    int nqt;      // query tiles per head
    int causal;
    int qmode;    // 0: q as given, 1: q negated (scale < 0), 2: q zeroed (scale == 0)
    float c;      // |scale| * log2(e)  (1 when scale == 0)
    int nitems;   // work items: query tiles x (KV head, head slot) pairs
    int xcd_cus;  // compute units per XCD (the workgroup order of paired launches)
    uint32_t *queue;   // work queues of a persistent launch, or null (one item per workgroup)
};

// Persistent launches.  The chip's XCDs do not run at one speed (in one
// measurement the slowest took 6 % longer per tile than the fastest), and a
// plain grid hands each XCD a fixed share of the items (workgroup i runs on
// XCD i mod 8), so the slowest XCD finishes last while the others idle.  A
// persistent launch instead keeps one workgroup per free slot and lets each
// pull items from a queue: queue x holds the items i = x mod 8 in order,
// which is the set and the order (longest causal tile first) that XCD x would
// get from a plain grid, so its K/V rows stay in that XCD's L2.  A workgroup
// starts with the queue of its own XCD; once that queue is empty it takes the
// next item of the other queues, which by then are the shortest ones.  The
// queue heads, a count of items handed out and a count of finished workgroups
// live in a small block of device memory (kQueueWords words, one 128-byte
// line per counter); the last workgroup to finish sets them back to zero for
// the next launch.  A persistent launch pays an atomic round trip per item and
// its workgroups cannot overlap one item's end with the next one's start, so
// it is used only where the tile table's sweep found it faster, and only when
// there are more items than workgroup slots.
constexpr int kQueues = 8;
constexpr int kTicket = kQueues;                       // counter of items handed out
constexpr int kDone = kQueues + 1;                     // counter of finished workgroups
constexpr int kCounters = kQueues + 2;
constexpr int kQueueStride = 32;                       // words between counters
constexpr int kQueueWords = kCounters * kQueueStride;
// The kernel arguments in the kernel-argument (constant) address space, so
// that reads of them stay scalar loads.
typedef const __attribute__((address_space(4))) Bf16Args *ArgsPtr;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One 16-byte global->LDS load per lane: lane l's 16 bytes, read from
// base + voff (base uniform, voff per lane), land at LDS byte address
// lds + 16*l.  Written as inline assembly so that the compiler does not track
// these LDS writes itself: the kernel orders them explicitly (vmcnt wait plus
// barrier before any read of the buffer), and the compiler's own tracking
// would otherwise stall reads of other buffers while a load is in flight.
// The s_nop covers the M0-write hazard before the load.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds) {
    lds_poison_lane16(lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// The LDS ring: four K tiles, then four V tiles, each kKeyTile rows of D bf16
// in swizzled 16-byte chunks.
template <int D>
struct LdsRing {
    static constexpr int kTileBytes = kKeyTile * D * 2;
    __attribute__((aligned(16))) char k[4][kTileBytes];
    __attribute__((aligned(16))) char v[4][kTileBytes];
};

// The loads that copy key rows [j0, j0 + kKeyTile) of one K or V head into an
// LDS tile, split over NW waves (this is wave wi of them).  Load i of the tile
// fills LDS chunk slots [64i, 64i + 64) -- slot p by lane p%64 -- so each lane
// fetches the logical chunk that the swizzle places in its slot.  The per-lane
// byte offsets within a tile are fixed; only the tile's base row moves.  Rows
// past the last key row Tk-1 (last, ragged tile) are clamped to it: they only
// ever meet masked scores.
template <int D, bool IS_V, int NW>
struct TileLoader {
    static constexpr int kRowBytes = D * 2;
    static constexpr int kCpr = D / 8;
    static constexpr int kLoadsPerTile = kKeyTile * kCpr / 64;    // 64-lane loads per tile
    static constexpr int kPerWave = (kLoadsPerTile + NW - 1) / NW;
    uint32_t off[kPerWave];     // key * row bytes + swizzled chunk * 16
    int wi;

    __device__ __forceinline__ TileLoader(int wi_, int lane) : wi(wi_) {
#pragma unroll
        for (int r = 0; r < kPerWave; ++r) {
            const int p = 64 * (wi + NW * r) + lane;
            const int key = p / kCpr;
            const int c = (p % kCpr) ^ (IS_V ? swz_v<D>(key) : swz_k<D>(key));
            off[r] = key * kRowBytes + c * 16;
        }
    }
    __device__ __forceinline__ bool active(int r) const {
        return kLoadsPerTile % NW == 0 || wi + NW * r < kLoadsPerTile;
    }
    // Load r alone, for the tile whose row 0 is at base.  With CLAMP, rows past
    // `last` (Tk - 1 - j0, which may exceed the tile) are clamped to row `last`;
    // without, the caller guarantees that every row of the tile is below Tk.
    template <bool CLAMP>
    __device__ __forceinline__ void load_one(int r, LDS_AS char *dst, const char *base,
                                             int last) const {
        if (!active(r)) return;
        uint32_t o = off[r];
        if constexpr (CLAMP) {
            const int key = (int)(off[r] / kRowBytes);
            o += (uint32_t)(min(key, last) - key) * kRowBytes;
        }
        dma16(base, o, (uint32_t)(uintptr_t)dst + 1024 * (wi + NW * r));
    }
    __device__ __forceinline__ void load(LDS_AS char *dst, const uint16_t *head, int j0,
                                         int Tk) const {
        const char *base = (const char *)(head + (int64_t)j0 * D);
        const uint32_t lds = (uint32_t)(uintptr_t)dst;
        if (j0 + kKeyTile <= Tk) {
#pragma unroll
            for (int r = 0; r < kPerWave; ++r)
                if (active(r)) dma16(base, off[r], lds + 1024 * (wi + NW * r));
        } else {
            const int last = Tk - 1 - j0;   // last valid row of this tile
#pragma unroll
            for (int r = 0; r < kPerWave; ++r) {
                if (!active(r)) continue;
                const int key = (int)(off[r] / kRowBytes);
                const uint32_t o = (uint32_t)(min(key, last) - key) * kRowBytes + off[r];
                dma16(base, o, lds + 1024 * (wi + NW * r));
            }
        }
    }
};

// The K/V loads that ride in one MFMA phase: this wave's share of one K tile
// and one V tile, issued in kSteps single loads spread over the phase.  Step 0
// first waits for the loads this wave issued in its previous MFMA phase.
// RAGGED: Tk is not a multiple of the key tile, so a tile may cross Tk.
template <int D, bool RAGGED>
struct PhaseLoads {
    static constexpr int kPer = TileLoader<D, false, kWaves>::kPerWave;
    static constexpr int kSteps = 2 * kPer;
    const TileLoader<D, false, kWaves> &kl;
    const TileLoader<D, true, kWaves> &vl;
    LDS_AS char *kdst, *vdst;
    const char *ksrc, *vsrc;
    int klast, vlast;
    __device__ __forceinline__ void step(int s) const {
        if (s == 0) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        if (s < kPer) kl.template load_one<RAGGED>(s, kdst, ksrc, klast);
        else vl.template load_one<RAGGED>(s - kPer, vdst, vsrc, vlast);
    }
};
struct NoLoads {
    static constexpr int kSteps = 0;
    __device__ __forceinline__ void step(int) const {}
};

// Workgroup barrier without a memory fence.  __syncthreads() also waits for
// every outstanding memory operation of the wave, including the direct
// global->LDS loads issued for the next tiles, which would serialise them.
// Here every LDS write is such a load and is waited for explicitly (vmcnt)
// before the barrier that publishes it, and every LDS read is consumed within
// its phase.  The empty asm statements stop the compiler from moving memory
// accesses across the barrier, the scheduling barriers any other instruction:
// each phase's MFMA or vector work stays inside its phase.
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Pins a vector phase's result to the end of that phase.  P feeds only later
// code, so without this the compiler may sink its exp2 and convert work past
// the barrier into the wave's own MFMA phase.
template <int NQ>
__device__ __forceinline__ void settle(const u32x4 (&pu)[NQ][4]) {
#pragma unroll
    for (int nb = 0; nb < NQ; ++nb)
        asm volatile("" ::"v"(pu[nb][0]), "v"(pu[nb][1]), "v"(pu[nb][2]), "v"(pu[nb][3]));
}

// The lane index, computed where it is called: the compiler cannot tie it to an
// earlier copy and keep that one live instead.
__device__ __forceinline__ int lane_id_opaque() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// max(x, x of lane l ^ 32): a swap of the wave's halves, without LDS.
__device__ __forceinline__ float max_with_partner(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ void wait_dma_and_barrier() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's LDS loads have landed
    __syncthreads();                      // ... and everyone else's
}

// Per-lane LDS byte offsets of the MFMA operands inside a K or V tile.
//  * K (A operand of S^T = K Q^T): lane (col, hi) reads 16 bytes of key row col
//    (and col + 32 for the second 32-key block, a fixed +32 rows), dims
//    16*ks + 8*hi .. +7, for ks = 0 .. D/16-1.
//  * V (A operand of O^T = V^T P^T): ds_read_b64_tr_b16 hands lane j of a
//    16-lane group element j%4 of the 8-byte pieces read by lanes 4r + j/4,
//    r = 0..3.  For step st and dim block db, lane (grp, s16) reads key row
//    16*st + 4*hi + s16/4 (and +8 rows), dims 32*db + 16*(grp&1) + 4*(s16&3)
//    .. +3; after the transpose it holds 8 keys of one dim.  The keys come in
//    the same order as the lane's rows of S^T, so P needs no data movement.
//    The st and +8-row parts are fixed offsets; only db needs a register.
template <int D>
struct LaneOffsets {
    int k[D / 16];
    uint32_t v[D / 32];       // LDS byte addresses within V buffer 0
    __device__ __forceinline__ LaneOffsets(int lane, const LDS_AS char *v0) {
        constexpr int kRowBytes = D * 2;
        const int col = lane & 31, hi = lane >> 5, grp = lane >> 4, s16 = lane & 15;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            k[ks] = col * kRowBytes + (((2 * ks + hi) ^ swz_k<D>(col)) << 4);
        const int r = 4 * hi + (s16 >> 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int d = 32 * db + 16 * (grp & 1) + 4 * (s16 & 3);
            v[db] = (uint32_t)(uintptr_t)v0 + r * kRowBytes + (((d >> 3) ^ swz_v<D>(r)) << 4) +
                    (d & 7) * 2;
            // Opaque to the compiler: a V read is then this register plus an
            // immediate offset (the buffer and row step, < 64 KB), with no add.
            asm("" : "+v"(v[db]));
        }
    }
};

// The MFMA phase of one tile: S^T(t) = K(t) Q^T (two 32-key blocks, chains
// s0 and s1) and O^T += V(t-1)^T P(t-1)^T (D/32 chains acc[db]), as one
// software pipeline.  The D/8 score MFMAs and D/8 P V MFMAs alternate, and the
// LDS operands are read kPrefetch MFMAs ahead.  MODE: 0 both, 1 scores only
// (first tile), 2 P V only (after the last tile).
constexpr int kPrefetch = 3;

// LDS reads feeding op i of an MFMA phase: one 16-byte read for a score MFMA,
// two transposing 8-byte reads for a P V MFMA.
constexpr int phase_reads(int mode, int i) {
    return (mode == 1 || (mode == 0 && (i & 1) == 0)) ? 1 : 2;
}

// Row sums on the matrix cores, from the same bf16 P that the P V product
// uses, so the weights of a row sum to one however sharply it peaks.  One
// 16x16x32 MFMA per 16-key step takes the P^T operand of the P V MFMAs as its
// B operand.  Read that way, column n of B holds the keys of query n in lane
// groups 0 and 2 and those of query n + 16 in lane groups 1 and 3, so an A
// operand that is one on (row r, lane group g) with r + g even, else zero,
// puts the sum of query n in the even rows of output column n and that of
// query n + 16 in the odd rows.  Each lane then holds both in its entries 0
// and 1 and keeps the one of its own query, (lane / 16) % 2.  Half the cost
// of a 32x32 ones x P^T product, and no vector adds.
__device__ __forceinline__ bf16x8 row_sum_selector(int lane) {
    const __bf16 x = ((lane ^ (lane >> 4)) & 1) == 0 ? (__bf16)1.0f : (__bf16)0.0f;
    return bf16x8{x, x, x, x, x, x, x, x};
}


// Scheduling groups for the MFMA phase: the row-sum MFMAs first (they need no
// LDS operand), then for every op its MFMA followed by the reads of the op
// kPrefetch later (the first kPrefetch ops' operands arrive preloaded).  This
// pins the prefetch distance that the plain schedule would shrink.
template <int MODE, int I, int N, bool SUM, int NQ>
__device__ __forceinline__ void schedule_mfma_phase() {
    if constexpr (I == 0 && SUM) __builtin_amdgcn_sched_group_barrier(0x008, 4 * NQ, 0);
    if constexpr (I < N) {
        __builtin_amdgcn_sched_group_barrier(0x008, NQ, 0);
        if constexpr (I + kPrefetch < N)
            __builtin_amdgcn_sched_group_barrier(0x100, phase_reads(MODE, I + kPrefetch), 0);
        schedule_mfma_phase<MODE, I + 1, N, false, NQ>();
    }
}

// Op i of an MFMA phase: whether it is a score MFMA, and its index among the
// ops of its kind.
template <int MODE>
__device__ __forceinline__ constexpr bool op_is_score(int i) {
    return MODE == 1 || (MODE == 0 && (i & 1) == 0);
}
template <int MODE>
__device__ __forceinline__ constexpr int op_index(int i) {
    return MODE == 0 ? (i >> 1) : i;
}

// The LDS operand of op i: a K row chunk (score MFMA, K tile kt) or two
// transposing reads of V (P V MFMA, V tile at byte offset vrel from V buffer 0).
template <int D, int MODE>
__device__ __forceinline__ u32x4 phase_operand(const LDS_AS char *kt, uint32_t vrel,
                                               const LaneOffsets<D> &off, int i) {
    constexpr int kRowBytes = D * 2;
    const int j = op_index<MODE>(i);
    if (op_is_score<MODE>(i)) {
        const int ks = j >> 1, kb = j & 1;
        return *(const LDS_AS u32x4 *)(kt + off.k[ks] + kb * 32 * kRowBytes);
    }
    const int st = j / (D / 32), db = j % (D / 32);
    const LDS_AS char *p =
        (const LDS_AS char *)(uintptr_t)(off.v[db] + vrel + st * 16 * kRowBytes);
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)p);
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(p + 8 * kRowBytes));
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Reads the operands of the first kPrefetch ops of an MFMA phase, ahead of it.
template <int D, int MODE>
__device__ __forceinline__ void preload(const LDS_AS char *kt, uint32_t vrel,
                                        const LaneOffsets<D> &off, u32x4 (&ring)[kPrefetch]) {
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) ring[i] = phase_operand<D, MODE>(kt, vrel, off, i);
}

// The phase itself; `ring` holds the operands of its first kPrefetch ops.
template <int D, int MODE, int NQ, class Loads>
__device__ __forceinline__ void mfma_phase(const LDS_AS char *kt, uint32_t vrel,
                                           const LaneOffsets<D> &off,
                                           const bf16x8 (&qf)[NQ][D / 16],
                                           const u32x4 (&pu)[NQ][4], f32x16 (&s0)[NQ],
                                           f32x16 (&s1)[NQ], f32x16 (&acc)[NQ][D / 32],
                                           f32x4 (&lsum)[NQ], bf16x8 sumsel, const Loads &loads,
                                           u32x4 (&ring)[kPrefetch]) {
    constexpr int kHalf = D / 8;                         // MFMAs of each kind
    constexpr int kN = MODE == 0 ? 2 * kHalf : kHalf;    // MFMAs in this phase
    static_assert(kN >= kPrefetch, "phase shorter than the prefetch ring");
    if (MODE != 2) {
#pragma unroll
        for (int nb = 0; nb < NQ; ++nb) {
            s0[nb] = f32x16{};
            s1[nb] = f32x16{};
        }
    }
    constexpr bool kSum = MODE != 1;
    if constexpr (kSum) {
#pragma unroll
        for (int nb = 0; nb < NQ; ++nb) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
                lsum[nb] = mfma16(sumsel, __builtin_bit_cast(bf16x8, pu[nb][st]), lsum[nb]);
        }
    }
#pragma unroll
    for (int i = 0; i < kN; ++i) {
        const u32x4 cur = ring[i % kPrefetch];
        if (i + kPrefetch < kN)
            ring[i % kPrefetch] = phase_operand<D, MODE>(kt, vrel, off, i + kPrefetch);
        const int j = op_index<MODE>(i);
        // One LDS operand feeds the MFMA of every query block of the wave.
        if (op_is_score<MODE>(i)) {
            const int ks = j >> 1;
#pragma unroll
            for (int nb = 0; nb < NQ; ++nb) {
                if ((j & 1) == 0) s0[nb] = mfma32(__builtin_bit_cast(bf16x8, cur), qf[nb][ks], s0[nb]);
                else s1[nb] = mfma32(__builtin_bit_cast(bf16x8, cur), qf[nb][ks], s1[nb]);
            }
        } else {
            const int st = j / (D / 32), db = j % (D / 32);
#pragma unroll
            for (int nb = 0; nb < NQ; ++nb)
                acc[nb][db] = mfma32(__builtin_bit_cast(bf16x8, cur),
                                     __builtin_bit_cast(bf16x8, pu[nb][st]), acc[nb][db]);
        }
        // The phase's K/V loads, one after each of kSteps evenly spaced ops.
        if constexpr (Loads::kSteps > 0) {
#pragma unroll
            for (int st = 0; st < Loads::kSteps; ++st)
                if (i == kN * (2 * st + 1) / (2 * Loads::kSteps)) loads.step(st);
        }
    }
    schedule_mfma_phase<MODE, 0, kN, kSum, NQ>();
}

// Work split.  A workgroup owns one query tile of 32*NQ*nqb rows for hg query
// heads of one KV head; wave w takes head (w % hg) and the NQ query blocks
// w / hg (32*NQ consecutive rows; NQ = 2 only at D = 64 without the mask).
// Its waves therefore read the same K/V rows, staged once in LDS.  Workgroup
// ids run over (KV head, slot) fastest so that, with B*Hkv a multiple of the
// 8 XCDs, every tile of one KV head lands on the same XCD and its L2; causal
// query tiles are issued longest first.
//
// Ping-pong.  Each tile is two phases per wave: an MFMA phase (S(t) = K(t)
// Q^T and acc += V(t-1)^T P(t-1)^T) and a vector phase (mask, online softmax,
// P(t) = 2^(S c - m) in bf16), separated by barriers.  Waves 0-3 and 4-7 (one
// of each per SIMD) run the same code one phase apart -- waves 4-7 pass one
// extra barrier first -- so in every phase one wave of a SIMD feeds the matrix
// cores while the other works the vector ALUs.  K/V tiles stream into a
// four-deep LDS ring with direct global->LDS loads issued between the MFMAs;
// the schedule of loads, waits and reads is spelled out at the loop below,
// which is unrolled by four so every LDS buffer is a distinct array.
// RAGGED: Tk % kKeyTile != 0 (the last key tile crosses Tk).
// PAIRED: two workgroups per CU (four waves per SIMD, at most 128 VGPRs each;
// D <= 64 with Tk a multiple of the key tile only: the LDS ring is at most
// 64 KB, and the ragged build would spill in the loop).  The two run independently, so the
// vector phases of one overlap the matrix-core phases of the other on top of
// the ping-pong inside each: the vector work of a single wave is bound by its
// own issue rate, and two waves issuing it side by side go about twice as fast.
//
// attn_fwd_bf16_item is one work item: the query tile, KV head and head slot
// of `item`, from the prologue loads to the stores of out and lse.
template <int D, bool RAGGED, bool PAIRED, int NQ, bool PERSIST, class Args>
__device__ __forceinline__ void attn_fwd_bf16_item(Args &a, LdsRing<D> &lds, int item) {
    // In a persistent workgroup the lane index is opaque, so that nothing
    // derived from it is hoisted out of the loop over items and held across
    // items.
    const int lane = PERSIST ? lane_id_opaque() : (int)(threadIdx.x & 63);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const bool lag = w >= 4;      // the half that runs one phase behind
    const int hi = lane >> 5;     // which half of the wave
    const int col = lane & 31;    // query column of this lane

    const int per_tile = a.nbh * a.nslots;
    const int qt_rev = item / per_tile;
    const int rem = item - qt_rev * per_tile;
    const int qt = a.causal ? (a.nqt - 1 - qt_rev) : qt_rev;
    const int slot = rem / a.nbh;
    const int bh = rem - slot * a.nbh;                // b * Hkv + kv head
    const int b = bh / a.Hkv;
    const int hkv = bh - b * a.Hkv;
    const int head = hkv * a.G + slot * a.hg + (w % a.hg);
    const int rows_wg = 32 * NQ * a.nqb;
    const int q0 = qt * rows_wg;
    const int qw0 = q0 + 32 * NQ * (w / a.hg);   // the wave's first query row
    const int Tq = a.Tq, Tk = a.Tk, qoff = a.qoff;
    const bool causal = a.causal != 0;

    const int64_t q_row0 = ((int64_t)b * a.Hq + head) * Tq;
    const uint16_t *khead = a.k + (int64_t)bh * Tk * D;
    const uint16_t *vhead = a.v + (int64_t)bh * Tk * D;

    // Causal: query row i sees keys 0 .. i + qoff, so the workgroup's last row
    // sees up to key q_end - 1 + qoff (at most Tk - 1).
    const int q_end = min(q0 + rows_wg, Tq);
    const int kv_end = causal ? q_end + qoff : Tk;
    const int ntiles = (kv_end + kKeyTile - 1) / kKeyTile;

    // Prologue loads, shared by all waves: K(0), K(1), K(2), V(0), V(1).
    {
        const TileLoader<D, false, kWaves> kl(w, lane);
        const TileLoader<D, true, kWaves> vl(w, lane);
        kl.load((LDS_AS char *)lds.k[0], khead, 0, Tk);
        if (ntiles > 1) kl.load((LDS_AS char *)lds.k[1], khead, kKeyTile, Tk);
        if (ntiles > 2) kl.load((LDS_AS char *)lds.k[2], khead, 2 * kKeyTile, Tk);
        vl.load((LDS_AS char *)lds.v[0], vhead, 0, Tk);
        if (ntiles > 1) vl.load((LDS_AS char *)lds.v[1], vhead, kKeyTile, Tk);
    }

    // Q fragments (B operand of S^T = K Q^T) of the wave's NQ query blocks:
    // lane holds 8 dims of its query row of block nb, row qw0 + 32 nb + col,
    // per 16-dim step.  Rows past Tq are clamped; their results are dropped.
    bf16x8 qf[NQ][D / 16];
    {
        const uint32_t flip = a.qmode == 1 ? 0x80008000u : 0u;
        const uint32_t keep = a.qmode == 2 ? 0u : 0xffffffffu;
#pragma unroll
        for (int nb = 0; nb < NQ; ++nb) {
            const uint16_t *src =
                a.q + (q_row0 + min(qw0 + 32 * nb + col, Tq - 1)) * D + 8 * hi;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const u32x4 raw = *(const u32x4 *)(src + 16 * ks);
                qf[nb][ks] = __builtin_bit_cast(bf16x8, (raw ^ flip) & keep);
            }
        }
    }

    // Per query block: the accumulators, running max (scale*log2(e)*s, log2
    // units) and row sums (entry (lane / 16) % 2 is this lane's query), the
    // scores of the tile in flight and its probabilities (bf16, per 16-key step).
    f32x16 acc[NQ][D / 32];
    float m_run[NQ];
    f32x4 lsum[NQ];
    f32x16 s0[NQ], s1[NQ];
    u32x4 pu[NQ][4];
#pragma unroll
    for (int nb = 0; nb < NQ; ++nb) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[nb][db] = f32x16{};
        m_run[nb] = -INFINITY;
        lsum[nb] = f32x4{};
        s0[nb] = f32x16{};
        s1[nb] = f32x16{};
    }
    const bf16x8 sumsel = row_sum_selector(lane);
    const float c = a.c;

    const LaneOffsets<D> off(lane, (const LDS_AS char *)lds.v[0]);
    // Every wave issues its share (1/8) of each later K/V tile load.
    const TileLoader<D, false, kWaves> kload(w, lane);
    const TileLoader<D, true, kWaves> vload(w, lane);
    // Vector phase of tile t: mask, online softmax, P(t).
    // `first`: tile 0 (m is still -inf there; afterwards m is finite).
    auto softmax_phase = [&](int t, bool first) __attribute__((always_inline)) {
        const int j0 = t * kKeyTile;
#pragma unroll
        for (int nb = 0; nb < NQ; ++nb) {
        const int qb0 = qw0 + 32 * nb;   // first query row of block nb
        // Mask keys hidden from a query (diagonal tile) or past Tk (ragged tile).
        if ((RAGGED && j0 + kKeyTile > Tk) || (causal && j0 + kKeyTile - 1 > qb0 + qoff)) {
            // Row i of this lane is key j0 + 4*hi + 8*(i/4) + i%4 (+32 in s1);
            // it is visible iff that key <= last, the last key this query sees.
            const int last = (causal ? min(qb0 + col, Tq - 1) + qoff : Tk - 1) - j0 - 4 * hi;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 8 * (i >> 2) + (i & 3);
                if (r > last) s0[nb][i] = -INFINITY;
                if (r + 32 > last) s1[nb][i] = -INFINITY;
            }
        }
        // Online softmax, in log2 units, with the lazy running max m (see
        // kHeadroom).  P is computed and packed with the m in hand; if some p
        // of the wave reached 2 (bit 14 of a bf16 code), the whole wave takes
        // the branch, which raises m to the tile max over both lanes of each
        // query row plus the headroom (so both keep the same m), rescales the
        // accumulators and recomputes P.  Tile 0 takes the branch directly.
        f32x16 e0, e1;
        auto sweep = [&](float m_sub) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                e0[i] = __builtin_fmaf(s0[nb][i], c, -m_sub);
                e1[i] = __builtin_fmaf(s1[nb][i], c, -m_sub);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                e0[i] = __builtin_amdgcn_exp2f(e0[i]);
                e1[i] = __builtin_amdgcn_exp2f(e1[i]);
            }
        };
        // P to bf16, in the operand order of the P V MFMAs.
        auto pack = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bf16x2 p0 =
                    __builtin_convertvector((f32x2){e0[2 * e], e0[2 * e + 1]}, bf16x2);
                const bf16x2 p1 =
                    __builtin_convertvector((f32x2){e1[2 * e], e1[2 * e + 1]}, bf16x2);
                pu[nb][e >> 2][e & 3] = __builtin_bit_cast(uint32_t, p0);
                pu[nb][2 + (e >> 2)][e & 3] = __builtin_bit_cast(uint32_t, p1);
            }
        };
        auto own_max = [&]() __attribute__((always_inline)) {
            float mq[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = 4 * k;
                float m = fmaxf(fmaxf(s0[nb][i], s0[nb][i + 1]), s0[nb][i + 2]);
                m = fmaxf(fmaxf(m, s0[nb][i + 3]), s1[nb][i]);
                m = fmaxf(fmaxf(m, s1[nb][i + 1]), s1[nb][i + 2]);
                mq[k] = fmaxf(m, s1[nb][i + 3]);
            }
            return fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3])) * c;
        };
        // The two-workgroups-per-CU build (128 registers) forms P straight from
        // the scores into the packed operand, two values of each block at a
        // time, so that no fp32 copy of the tile sits beside the scores, which
        // the OR test keeps live; its raise recomputes P the same way.
        auto sweep_pack = [&](float m_sub) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[nb][2 * e], c, -m_sub));
                const float a1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[nb][2 * e + 1], c, -m_sub));
                const float b0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[nb][2 * e], c, -m_sub));
                const float b1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[nb][2 * e + 1], c, -m_sub));
                pu[nb][e >> 2][e & 3] =
                    __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a0, a1}, bf16x2));
                pu[nb][2 + (e >> 2)][e & 3] =
                    __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){b0, b1}, bf16x2));
            }
        };
        auto raise_packed = [&](float m_own) __attribute__((always_inline)) {
            const float m_new = fmaxf(m_run[nb], max_with_partner(m_own) + (float)kHeadroom);
            const float alpha =
                (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[nb] - m_new);
            lsum[nb][0] *= alpha;
            lsum[nb][1] *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) acc[nb][db] *= alpha;
            m_run[nb] = m_new;
            sweep_pack(m_new == -INFINITY ? 0.f : m_new);
        };
        auto raise = [&](float m_own) __attribute__((always_inline)) {
            const float m_new = fmaxf(m_run[nb], max_with_partner(m_own) + (float)kHeadroom);
            const float alpha =
                (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[nb] - m_new);
            lsum[nb][0] *= alpha;   // the two entries a lane may read
            lsum[nb][1] *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) acc[nb][db] *= alpha;
            m_run[nb] = m_new;
            sweep(m_new == -INFINITY ? 0.f : m_new);
        };
        if constexpr (PAIRED) {
            // The same test as below, on P packed by sweep_pack.
            if (first) {
                raise_packed(own_max());
            } else {
                sweep_pack(m_run[nb]);
                uint32_t any = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int j = 0; j < 4; ++j) any |= pu[nb][k][j];
                if (__builtin_amdgcn_ballot_w64((any & 0x40004000u) != 0) != 0)
                    raise_packed(own_max());
            }
        } else if (first) {
            raise(own_max());
            pack();
        } else {
            sweep(m_run[nb]);
            pack();
            uint32_t any = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int j = 0; j < 4; ++j) any |= pu[nb][k][j];
            if (__builtin_amdgcn_ballot_w64((any & 0x40004000u) != 0) != 0) {
                raise(own_max());
                pack();
            }
        }
        }
    };
    // Iteration t of every wave: the MFMA phase of tile t (S(t) from K(t), and
    // P(t-1) V(t-1)), a barrier, the vector phase of tile t, a barrier.  Tile j
    // lives in LDS buffers K[j%4] and V[j%4].  The MFMA phase of tile t also
    // carries the wave's share of the loads of K(t+3) and V(t+2): the leading
    // waves issue theirs in phase 2t, the lagging waves in phase 2t+1.  The
    // target buffers held K(t-1) and V(t-2), last read in phase 2t-1; each
    // wave waits for its loads in its next MFMA phase, so both halves are
    // published by the barrier that ends phase 2t+3.  The vector phase of
    // tile t (phase 2t+1 or 2t+2) reads the first operands of the next MFMA
    // phase, K(t+1) and V(t), published by the end of phase 2t-1.  Near the
    // end the tile index of a load is clamped to the last tile: such a load
    // refills a buffer that is never read again.
    auto loads = [&](int t, LDS_AS char *kw, LDS_AS char *vw) __attribute__((always_inline)) {
        const int tk = min(t + 3, ntiles - 1), tv = min(t + 2, ntiles - 1);
        return PhaseLoads<D, RAGGED>{kload,
                             vload,
                             kw,
                             vw,
                             (const char *)(khead + (int64_t)tk * kKeyTile * D),
                             (const char *)(vhead + (int64_t)tv * kKeyTile * D),
                             Tk - 1 - tk * kKeyTile,
                             Tk - 1 - tv * kKeyTile};
    };
    u32x4 ring[kPrefetch];   // operands of the next MFMA phase's first ops
    // Buffers are named by index: K tile b at lds.k[b], V tile b at byte offset
    // b * kTileBytes from V buffer 0 (a compile-time constant in every read).
    constexpr uint32_t kTB = LdsRing<D>::kTileBytes;
    auto kbuf = [&](int b) __attribute__((always_inline)) { return (LDS_AS char *)lds.k[b]; };
    auto vbuf = [&](int b) __attribute__((always_inline)) { return (LDS_AS char *)lds.v[b]; };
    auto finish = [&](int t, int kn, int vn, bool first) __attribute__((always_inline)) {
        phase_barrier();
        // The first operands of the next MFMA phase: read at the start of the
        // vector phase, or, in the two-workgroups-per-CU build, at its end,
        // so that they are not live beside the scores and P.
        if constexpr (!PAIRED) {
            if (t + 1 < ntiles) preload<D, 0>(kbuf(kn), vn * kTB, off, ring);
            else preload<D, 2>(nullptr, vn * kTB, off, ring);
        }
        softmax_phase(t, first);
        settle<NQ>(pu);
        if constexpr (PAIRED) {
            if (t + 1 < ntiles) preload<D, 0>(kbuf(kn), vn * kTB, off, ring);
            else preload<D, 2>(nullptr, vn * kTB, off, ring);
        }
        phase_barrier();
    };
    // Iteration t: K(t) in buffer kc, V(t-1) in vp; loads into kw, vw; the
    // next phase's K(t+1) in kn, V(t) in vn.
    // With two workgroups per CU, four waves share a SIMD; the ones in an MFMA
    // phase issue first (wave priority 1), so the matrix core is fed as soon
    // as it frees up (about 1 % at T = 4096).
    auto iteration = [&](int t, int kc, int vp, int kw, int vw, int kn, int vn)
                         __attribute__((always_inline)) {
        if constexpr (PAIRED) __builtin_amdgcn_s_setprio(1);
        mfma_phase<D, 0, NQ>(kbuf(kc), vp * kTB, off, qf, pu, s0, s1, acc, lsum, sumsel,
                             loads(t, kbuf(kw), vbuf(vw)), ring);
        if constexpr (PAIRED) __builtin_amdgcn_s_setprio(0);
        finish(t, kn, vn, false);
    };

    // The lagging waves pass one extra barrier: from here on they run one
    // phase behind the leading waves.
    wait_dma_and_barrier();
    preload<D, 1>(kbuf(0), 0, off, ring);
    if (lag) phase_barrier();
    // Tile 0 has no P V yet.
    mfma_phase<D, 1, NQ>(kbuf(0), 0, off, qf, pu, s0, s1, acc, lsum, sumsel,
                         loads(0, kbuf(3), vbuf(2)), ring);
    finish(0, 1, 0, true);
    for (int t = 1; t < ntiles; t += 4) {
        iteration(t, 1, 0, 0, 3, 2, 1);
        if (t + 1 < ntiles) iteration(t + 1, 2, 1, 1, 0, 3, 2);
        if (t + 2 < ntiles) iteration(t + 2, 3, 2, 2, 1, 0, 3);
        if (t + 3 < ntiles) iteration(t + 3, 0, 3, 3, 2, 1, 0);
    }
    // P V of the last tile, then the leading waves pass their extra barrier.
    const int last = (ntiles - 1) % 4;
    const NoLoads none;
    auto pv_last = [&](uint32_t vrel) __attribute__((always_inline)) {
        mfma_phase<D, 2, NQ>(nullptr, vrel, off, qf, pu, s0, s1, acc, lsum, sumsel, none, ring);
    };
    if (last == 0) pv_last(0 * kTB);
    else if (last == 1) pv_last(1 * kTB);
    else if (last == 2) pv_last(2 * kTB);
    else pv_last(3 * kTB);
    if (!lag) phase_barrier();
    // The clamped loads of the last phases must land before the workgroup's
    // LDS is released.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    // Epilogue: O = acc / l, rounded once to bf16; lse = ln 2 * (m + log2 l).
    // The lane index is read again here rather than kept across the loop,
    // where registers are scarcest (two workgroups per CU allow 128).
    const int lane_e = lane_id_opaque();
    const int hi_e = lane_e >> 5;
#pragma unroll
    for (int nb = 0; nb < NQ; ++nb) {
        const int query_e = qw0 + 32 * nb + (lane_e & 31);
        const float l_tot = ((lane_e >> 4) & 1) ? lsum[nb][1] : lsum[nb][0];
        if (query_e < Tq) {
            const float inv = 1.f / l_tot;
            uint16_t *dst = a.o + (q_row0 + query_e) * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = acc[nb][db][4 * g4 + e] * inv;
                    const bf16x4 y = __builtin_convertvector(x, bf16x4);
                    *(bf16x4 *)(dst + 32 * db + 8 * g4 + 4 * hi_e) = y;
                }
            }
            if (hi_e == 0) a.lse[q_row0 + query_e] = (m_run[nb] + log2f(l_tot)) * kLn2;
        }
    }
}

// The item workgroup b of a two-workgroups-per-CU launch runs.  Workgroup b
// goes to XCD b % 8, and workgroups j and j + C of one XCD (j = b / 8, C
// compute units per XCD) start together on one CU and share it to the end,
// as a probe of the hardware's placement showed.  Items come longest first,
// so that second round is taken in reverse: the XCD's j-th longest item
// shares its CU with its (2C - 1 - j)-th, and under the causal mask every CU
// of a two-round grid gets the same number of tiles.  Later rounds go to the
// CUs as they free up and keep the plain order.
__device__ __forceinline__ int paired_item(int b, int nitems, int C) {
    const int x = b & (kQueues - 1), j = b / kQueues;
    if (j < C || j >= 2 * C) return b;
    const int local = (nitems - x + kQueues - 1) / kQueues;   // items of XCD x
    const int m = min(C, local - C);                          // of its second round
    return (2 * C + m - 1 - j) * kQueues + x;
}

// A plain launch: one workgroup per item, item blockIdx.x (reordered as
// above for two workgroups per CU).
template <int D, bool RAGGED, bool PAIRED, int NQ>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(PAIRED ? 4 : 2)))
attn_fwd_bf16_kernel(Bf16Args a) {
    static_assert(!PAIRED || (D <= 64 && !RAGGED), "two workgroups per CU: D <= 64, Tk % 64 == 0");
    static_assert(NQ == 1 || (D <= 64 && !PAIRED), "64 rows per wave: D <= 64, one workgroup per CU");
    __shared__ LdsRing<D> lds;
    lds_poison_all();
    const int item = PAIRED ? paired_item((int)blockIdx.x, a.nitems, a.xcd_cus) : (int)blockIdx.x;
    attn_fwd_bf16_item<D, RAGGED, PAIRED, NQ, false>(a, lds, item);
}

// A persistent launch: each workgroup takes items from the queues until every
// queue is empty.
template <int D, bool RAGGED, bool PAIRED, int NQ>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(PAIRED ? 4 : 2)))
attn_fwd_bf16_persistent_kernel(Bf16Args args) {
    __shared__ LdsRing<D> lds;
    __shared__ int s_item;
    lds_poison_all();

    const int tid = threadIdx.x;
    uint32_t *const queue = args.queue;
    // Thread 0: the queue it starts with (its XCD's, from the XCC_ID hardware
    // register) and the queues found empty.
    const int home = (int)(__builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & (kQueues - 1));
    uint32_t empty = 0;
    for (;;) {
        // The barrier also keeps the next item's loads into LDS behind every
        // wave's last read of the previous item.
        // A ticket below nitems entitles the workgroup to one item, which one
        // of the queues still holds (as many tickets as items are handed out);
        // a later ticket means every item is taken, found with one access.
        if (tid == 0) {
            int it = -1;
            if ((int)atomicAdd(queue + kTicket * kQueueStride, 1u) < args.nitems) {
                for (int t = 0; t < kQueues && it < 0; ++t) {
                    const int x = (home + t) & (kQueues - 1);
                    if ((empty >> x) & 1u) continue;
                    const int len = (args.nitems - x + kQueues - 1) / kQueues;
                    const int k = (int)atomicAdd(queue + x * kQueueStride, 1u);
                    if (k < len) it = x + kQueues * k;
                    else empty |= 1u << x;
                }
            }
            s_item = it;
        }
        __syncthreads();
        const int item = __builtin_amdgcn_readfirstlane(s_item);
        if (item < 0) break;
        // The arguments are read afresh from the kernel-argument segment for
        // every item (through an opaque pointer), so that neither they nor
        // anything derived from them is held in registers across items.
        ArgsPtr ap = (ArgsPtr)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ap));
        attn_fwd_bf16_item<D, RAGGED, PAIRED, NQ, true>(*ap, lds, item);
    }

    // The last workgroup to finish resets the queues.  Every other one has
    // made its last queue access before it counts itself done, so no access
    // to the counters can follow the reset.
    if (tid == 0) {
        __threadfence();
        const uint32_t done = atomicAdd(queue + kDone * kQueueStride, 1u);
        if (done == gridDim.x - 1) {
            for (int x = 0; x < kCounters; ++x) atomicExch(queue + x * kQueueStride, 0u);
        }
    }
}


// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
thread_local char g_last_error[256] = "";

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int validate(const void *q, const void *k, const void *v, const void *out, const void *lse,
             int B, int Hq, int Hkv, int Tq, int Tk, int D, int causal, float scale, size_t elem) {
    if (!q || !k || !v || !out || !lse) return TESSERA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || Tk < 1 || Hq % Hkv != 0) return TESSERA_ERR_SHAPE;
    if (D != 32 && D != 64 && D != 128) return TESSERA_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return TESSERA_ERR_CAUSAL;
    if (causal == 1 && Tq > Tk) return TESSERA_ERR_SHAPE;
    if (!isfinite(scale)) return TESSERA_ERR_SCALE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u) return TESSERA_ERR_ALIGN;
    if ((uintptr_t)lse & 3u) return TESSERA_ERR_ALIGN;
    const size_t qbytes = (size_t)B * Hq * Tq * D * elem;
    const size_t kvbytes = (size_t)B * Hkv * Tk * D * elem;
    const size_t lbytes = (size_t)B * Hq * Tq * sizeof(float);
    if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, k, kvbytes) ||
        overlaps(out, qbytes, v, kvbytes) || overlaps(lse, lbytes, q, qbytes) ||
        overlaps(lse, lbytes, k, kvbytes) || overlaps(lse, lbytes, v, kvbytes) ||
        overlaps(lse, lbytes, out, qbytes))
        return TESSERA_ERR_ALIAS;
    return TESSERA_OK;
}


// ---------------------------------------------------------------------------
// Tile configurations (tessera_attn_tile_config) and the static table of the
// library's picks.
// ---------------------------------------------------------------------------
struct TileRule {
    int D, causal, large, heads_per_workgroup, query_rows_per_wave, workgroups_per_cu, persistent;
};
#include "tile_table.inc"

constexpr int kLargeRowsPerCu = 1024;   // problem-size class boundary of the table
constexpr int kDefaultCus = 256;        // MI355X, when the device cannot be asked

int compute_units() {
    int dev = -1, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        n > 0)
        return n;
    return kDefaultCus;
}

// The table's configuration for these sizes, fitted to them: the largest head
// grouping up to the rule's that divides the GQA group, and one workgroup per
// CU when the key count is not a multiple of the key tile.
tessera_attn_tile_config table_config(int B, int Hq, int Hkv, int Tq, int Tk, int D, int causal) {
    const int64_t rows_per_cu = (int64_t)B * Hq * Tq / compute_units();
    const int large = rows_per_cu >= kLargeRowsPerCu ? 1 : 0;
    tessera_attn_tile_config c = {4, 32, 1, 0};
    for (const TileRule &r : kTileTable) {
        if (r.D == D && r.causal == causal && r.large == large) {
            c = {r.heads_per_workgroup, r.query_rows_per_wave, r.workgroups_per_cu, r.persistent};
            break;
        }
    }
    const int G = Hq / Hkv;
    while (G % c.heads_per_workgroup != 0) c.heads_per_workgroup /= 2;
    if (Tk % kKeyTile != 0) c.workgroups_per_cu = 1;
    return c;
}

// Whether configuration c is one these sizes allow (see the header).
bool config_allowed(const tessera_attn_tile_config &c, int Hq, int Hkv, int Tk, int D) {
    const int hg = c.heads_per_workgroup;
    if ((hg != 1 && hg != 2 && hg != 4) || (Hq / Hkv) % hg != 0) return false;
    if (c.query_rows_per_wave != 32 && c.query_rows_per_wave != 64) return false;
    if (c.workgroups_per_cu != 1 && c.workgroups_per_cu != 2) return false;
    if (c.persistent != 0 && c.persistent != 1) return false;
    if (c.query_rows_per_wave == 64 && (D > 64 || c.workgroups_per_cu == 2)) return false;
    if (c.workgroups_per_cu == 2 && (D > 64 || Tk % kKeyTile != 0 || c.persistent)) return false;
    return true;
}

// ---------------------------------------------------------------------------
// Work queues of persistent launches: kQueueSlots blocks of kQueueWords
// counters per GPU, zero from the library's load on.  A stream keeps one
// block for all its calls: calls on one stream run one after another, so a
// block is never used by two launches at once.  Calls on other streams use
// other blocks; past kQueueSlots streams on one device, and while a stream is
// being captured into a graph (whose replays could overlap), launches run as
// plain grids, which need no counters.
// ---------------------------------------------------------------------------
constexpr int kQueueSlots = 64;
constexpr int kMaxDevices = 64;

}  // namespace

__device__ __align__(128) uint32_t g_work_queues[kQueueSlots * kQueueWords];

namespace {

struct DeviceQueues {
    uint32_t *base = nullptr;            // device address of g_work_queues on this GPU
    int cus = 0;                         // compute units
    int nslots = 0;
    void *stream[kQueueSlots] = {};      // the stream that owns each block
};
std::mutex g_queues_mutex;
DeviceQueues g_queues[kMaxDevices];

// The counter block of `stream` on the current GPU and the GPU's compute-unit
// count, or null when no block is free (or the lookup failed).
uint32_t *queue_block(hipStream_t stream, int *cus) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
        return nullptr;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_queues_mutex);
    DeviceQueues &d = g_queues[dev];
    if (d.base == nullptr) {
        void *p = nullptr;
        int n = 0;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_work_queues)) != hipSuccess || p == nullptr ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 1)
            return nullptr;
        d.base = (uint32_t *)p;
        d.cus = n;
    }
    *cus = d.cus;
    for (int i = 0; i < d.nslots; ++i)
        if (d.stream[i] == (void *)stream) return d.base + (size_t)i * kQueueWords;
    if (d.nslots == kQueueSlots) return nullptr;
    d.stream[d.nslots] = (void *)stream;
    return d.base + (size_t)(d.nslots++) * kQueueWords;
}

// Launches the bf16 build <D, RAGGED, PAIRED, NQ> over `items` work items: as
// a persistent grid (one workgroup per slot the GPU holds at once, items from
// the queues) when asked for and there are more items than slots, else one
// workgroup per item.
template <int D, bool RAGGED, bool PAIRED, int NQ>
int launch_items(Bf16Args a, int64_t items, bool persistent, hipStream_t s) {
    a.nitems = (int)items;
    a.queue = nullptr;
    a.xcd_cus = compute_units() / kQueues;
    if (a.xcd_cus < 1) a.xcd_cus = 1;
    if constexpr (!PAIRED) {
        int cus = 0;
        uint32_t *q = persistent ? queue_block(s, &cus) : nullptr;
        if (q != nullptr) {
            auto *kernel = attn_fwd_bf16_persistent_kernel<D, RAGGED, false, NQ>;
            int per_cu = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)kernel,
                                                             kThreads, 0) == hipSuccess &&
                per_cu > 0 && items > (int64_t)per_cu * cus) {
                a.queue = q;
                return tessera_launch(kernel, dim3((unsigned)(per_cu * cus)), dim3(kThreads), s,
                                      a);
            }
        }
    }
    return tessera_launch(attn_fwd_bf16_kernel<D, RAGGED, PAIRED, NQ>, dim3((unsigned)items),
                          dim3(kThreads), s, a);
}

template <int D>
int launch_d(const Bf16Args &a, int64_t items, bool ragged, const tessera_attn_tile_config &c,
             hipStream_t s) {
    const bool persist = c.persistent != 0;
    if constexpr (D > 64) {
        if (ragged) return launch_items<D, true, false, 1>(a, items, persist, s);
        return launch_items<D, false, false, 1>(a, items, persist, s);
    } else {
        if (c.workgroups_per_cu == 2) return launch_items<D, false, true, 1>(a, items, false, s);
        if (c.query_rows_per_wave == 64) {
            if (ragged) return launch_items<D, true, false, 2>(a, items, persist, s);
            return launch_items<D, false, false, 2>(a, items, persist, s);
        }
        if (ragged) return launch_items<D, true, false, 1>(a, items, persist, s);
        return launch_items<D, false, false, 1>(a, items, persist, s);
    }
}

// The bf16 launch shared by the entry points (arguments already validated,
// configuration allowed for these sizes).
int launch_bf16(const void *q, const void *k, const void *v, void *out, float *lse, int B,
                int Hq, int Hkv, int Tq, int Tk, int D, int causal, float scale,
                const tessera_attn_tile_config &c, void *stream) {
    Bf16Args a;
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.o = (uint16_t *)out;
    a.lse = lse;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Tq = Tq;
    a.Tk = Tk;
    a.qoff = Tk - Tq;
    a.G = Hq / Hkv;
    a.hg = c.heads_per_workgroup;
    a.nqb = kWaves / a.hg;
    a.nslots = a.G / a.hg;
    const int rows_wg = c.query_rows_per_wave * a.nqb;
    a.nqt = (Tq + rows_wg - 1) / rows_wg;
    const int64_t items = (int64_t)a.nqt * B * Hkv * a.nslots;
    if (items > 0x7fffffff) return TESSERA_ERR_TOO_LARGE;
    a.nbh = B * Hkv;
    a.causal = causal;
    a.qmode = scale < 0.f ? 1 : (scale == 0.f ? 2 : 0);
    a.c = scale == 0.f ? 1.0f : (float)(fabs((double)scale) * kLog2e);

    hipStream_t s = (hipStream_t)stream;
    const bool ragged = Tk % kKeyTile != 0;
    if (D == 128) return launch_d<128>(a, items, ragged, c, s);
    if (D == 64) return launch_d<64>(a, items, ragged, c, s);
    return launch_d<32>(a, items, ragged, c, s);
}

}  // namespace

int tessera_validate_fwd(const void *q, const void *k, const void *v, const void *out,
                         const void *lse, int B, int Hq, int Hkv, int Tq, int Tk, int D,
                         int causal, float scale, size_t elem) {
    return validate(q, k, v, out, lse, B, Hq, Hkv, Tq, Tk, D, causal, scale, elem);
}

extern "C" int tessera_attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
                                int B, int Hq, int Hkv, int T, int D, int causal, float scale,
                                void *stream) {
    const int st = validate(q, k, v, out, lse, B, Hq, Hkv, T, T, D, causal, scale, 2);
    if (st != TESSERA_OK) return st;
    return launch_bf16(q, k, v, out, lse, B, Hq, Hkv, T, T, D, causal, scale,
                       table_config(B, Hq, Hkv, T, T, D, causal), stream);
}

extern "C" int tessera_attn_fwd_kv(const void *q, const void *k, const void *v, void *out,
                                   float *lse, int B, int Hq, int Hkv, int Tq, int Tk, int D,
                                   int causal, float scale, void *stream) {
    const int st = validate(q, k, v, out, lse, B, Hq, Hkv, Tq, Tk, D, causal, scale, 2);
    if (st != TESSERA_OK) return st;
    return launch_bf16(q, k, v, out, lse, B, Hq, Hkv, Tq, Tk, D, causal, scale,
                       table_config(B, Hq, Hkv, Tq, Tk, D, causal), stream);
}

extern "C" int tessera_attn_fwd_with_config(const void *q, const void *k, const void *v,
                                            void *out, float *lse, int B, int Hq, int Hkv,
                                            int Tq, int Tk, int D, int causal, float scale,
                                            const tessera_attn_tile_config *config,
                                            void *stream) {
    const int st = validate(q, k, v, out, lse, B, Hq, Hkv, Tq, Tk, D, causal, scale, 2);
    if (st != TESSERA_OK) return st;
    if (!config) return TESSERA_ERR_NULL;
    if (!config_allowed(*config, Hq, Hkv, Tk, D)) return TESSERA_ERR_UNSUPPORTED;
    return launch_bf16(q, k, v, out, lse, B, Hq, Hkv, Tq, Tk, D, causal, scale, *config, stream);
}

extern "C" int tessera_attn_fwd_tile_config(int B, int Hq, int Hkv, int Tq, int Tk, int D,
                                            int causal, tessera_attn_tile_config *config) {
    if (!config) return TESSERA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || Tk < 1 || Hq % Hkv != 0) return TESSERA_ERR_SHAPE;
    if (D != 32 && D != 64 && D != 128) return TESSERA_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return TESSERA_ERR_CAUSAL;
    if (causal == 1 && Tq > Tk) return TESSERA_ERR_SHAPE;
    *config = table_config(B, Hq, Hkv, Tq, Tk, D, causal);
    return TESSERA_OK;
}


extern "C" const char *tessera_attn_status_string(int status) {
    switch (status) {
    case TESSERA_OK: return "ok";
    case TESSERA_ERR_NULL: return "null pointer argument";
    case TESSERA_ERR_SHAPE:
        return "bad shape: B, Hq, Hkv and the row counts must be >= 1, Hq % Hkv == 0, and a "
               "causal call needs no more query rows than key rows";
    case TESSERA_ERR_UNSUPPORTED:
        return "unsupported size: D must be 32, 64 or 128 (RMSNorm: n a multiple of 8, at most "
               "65536; paged decode: (Hq / Hkv) * Tq <= 32, block_size a multiple of 16)";
    case TESSERA_ERR_CAUSAL: return "causal must be 0 or 1";
    case TESSERA_ERR_SCALE: return "scale must be finite";
    case TESSERA_ERR_ALIGN: return "misaligned pointer: q, k, v, out need 16 bytes, lse 4 bytes";
    case TESSERA_ERR_ALIAS: return "out or lse overlaps an input or each other";
    case TESSERA_ERR_TOO_LARGE: return "problem too large for one launch grid";
    case TESSERA_ERR_LAUNCH: return "HIP kernel launch failed";
    case TESSERA_ERR_EPS: return "eps must be finite and non-negative";
    case TESSERA_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case TESSERA_ERR_SCRATCH:
        return "the split partials of this decode exceed the library's fixed scratch buffer "
               "(tessera_paged_decode_scratch_limit bytes); pass a workspace to "
               "tessera_paged_decode instead";
    default: return "unknown status";
    }
}

extern "C" const char *tessera_attn_last_error(void) { return g_last_error; }

// The launch result of every entry point of the library (not exported).
__attribute__((visibility("hidden"))) int tessera_launch_result(hipError_t e) {
    if (e == hipSuccess) return TESSERA_OK;
    snprintf(g_last_error, sizeof g_last_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
    return TESSERA_ERR_LAUNCH;
}

extern "C" int tessera_attn_version(void) { return TESSERA_VERSION; }
