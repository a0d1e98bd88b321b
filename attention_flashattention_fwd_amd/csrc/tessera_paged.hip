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
//   * Split-KV.  A sequence's tokens are cut into splits of L keys; one wave
//     owns one (sequence, KV head, split) unit and computes all query rows of
//     that KV head over its split with an online softmax.  Units are
//     independent one-wave workgroups, so a long sequence spreads over many
//     CUs.  When a sequence has more than one split, each unit writes its
//     normalised partial output and its log2-sum-exp to the workspace, and a
//     second kernel merges them: O = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M).
//   * Each wave streams its keys through its own ring of LDS stages (32 keys
//     of K and of V per stage) with direct global->LDS loads, issued as soon
//     as a stage is free, and no barrier: a wave only ever reads what it
//     loaded itself.  The block table is read once per unit into a register
//     (one entry per lane); the base address of every 16-key half-tile is a
//     scalar taken from it, so a half-tile load is one contiguous 16-row
//     piece of one block.
//   * Both products run on v_mfma_f32_32x32x16_bf16 in the transposed form
//     of the prefill kernel, S^T = K Q^T and O^T = V^T P^T, with the query
//     rows of the KV head as the 32 columns (unused columns hold zero
//     queries and are dropped); the LDS layout, swizzle and operand reads are
//     those of the prefill kernel for a 32-key tile.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "tessera_paged.h"

int tessera_launch_status(void);   // tessera_attn.hip

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
constexpr int kMaxEntries = 64;        // table entries of one split: one per lane
constexpr int kMinSplit = 256;         // keys per split, at least (before rounding)
constexpr int64_t kTargetUnits = 8192;    // (sequence, KV head, split) units aimed for
constexpr uint32_t kBadBits = 0x7fc00000u;    // quiet NaN: marks bad table data
constexpr uint16_t kBadBf16 = 0x7fc0u;

// LDS ring stages per wave: 32 KB of K and V tiles for every head dim, so
// that five one-wave workgroups fit one CU's 160 KB.
template <int D>
constexpr int ring_stages() {
    return D == 128 ? 2 : (D == 64 ? 4 : 8);
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
    float *ws_lse;   // [rows, nsplit] log2-sum-exp of each split
    float *ws_o;     // [rows, nsplit, D] normalised partial outputs
    int Hq, Hkv, G, Tq, M;    // M = G * Tq query rows per KV head
    int bs, max_blocks, num_blocks;
    int nbg;         // B * Hkv
    int nsplit;      // splits of the longest possible sequence
    int L;           // keys per split (a multiple of 32 and of bs)
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
// The s_nop covers the M0-write hazard before the load.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
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

// One wave per (split, sequence, KV head) unit: blockIdx.x = split * B * Hkv
// + sequence * Hkv + KV head.
template <int D>
__global__ void __launch_bounds__(64) paged_decode_kernel(PagedArgs a) {
    constexpr int R = ring_stages<D>();
    constexpr int kRowBytes = 2 * D;
    constexpr int kTileBytes = kTileKeys * kRowBytes;   // one K or V tile
    constexpr int kLoads = kTileBytes / 1024;           // 1 KB loads per tile
    constexpr int kHalfLoads = kLoads / 2;              // ... per 16-key half
    constexpr int kCpr = D / 8;                         // 16-byte chunks per row
    constexpr int kKeysPerLoad = 64 / kCpr;
    static_assert((R - 1) * 2 * kLoads <= 63, "loads in flight exceed the vmcnt range");
    __shared__ __attribute__((aligned(16))) char lds[R][2][kTileBytes];

    const int lane = threadIdx.x;
    const int col = lane & 31, hi = lane >> 5;
    const int s = blockIdx.x / a.nbg;
    const int bg = blockIdx.x - s * a.nbg;
    const int b = bg / a.Hkv;
    const int g = bg - b * a.Hkv;

    // The sequence's length decides how many splits it has; units past them
    // have nothing to do.  A length out of range makes split 0 write NaN.
    const int n = a.lens[b];
    const bool len_ok = n >= 0 && n <= a.max_blocks * a.bs;
    const int nsb = len_ok ? max(1, (n + a.L - 1) / a.L) : 1;
    if (s >= nsb) return;
    const bool direct = nsb == 1;   // the unit writes the final result itself
    const int start = s * a.L;
    const int end = len_ok ? min(start + a.L, n) : start;

    // The table entries of the split, one per lane, checked once.
    const int first = start / a.bs;
    const int count = end > start ? (end - 1) / a.bs - first + 1 : 0;
    int ent = 0;
    if (lane < count) ent = a.table[(int64_t)b * a.max_blocks + first + lane];
    const bool bad =
        !len_ok || __builtin_amdgcn_ballot_w64(lane < count && (ent < 0 || ent >= a.num_blocks)) != 0;
    const int ntiles = bad ? 0 : (end - start + kTileKeys - 1) / kTileKeys;

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

    // Loads tile t of the split into stage `st`.  Each 16-key half lies in one
    // block.  Rows at or past `end` are clamped to the last row that holds a
    // token (a half with none reads the first half's rows): they meet only
    // masked scores, and stay finite so that a zero weight keeps them out.
    auto issue = [&](int t, int st) __attribute__((always_inline)) {
        const int t0 = start + t * kTileKeys;
        const char *kb[2], *vb[2];
        int lastrow[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int th = t0 + 16 * h;
            if (h == 0 || th < end) {
                const int blk = __builtin_amdgcn_readlane(ent, th / a.bs - first);
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

    const int pre = min(R, ntiles);
    for (int t = 0; t < pre; ++t) issue(t, t);

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

    // The visible tokens of this lane's query row: 0 .. kend - 1.
    const int qi = col < a.M ? col % a.Tq : a.Tq - 1;
    const int kend = a.causal ? n - a.Tq + qi + 1 : n;
    const int mask_from = a.causal ? n - a.Tq + 1 : n;   // smallest kend of the unit
    const float c = a.c;
    const bf16x8 sumsel = row_sum_selector(lane);

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
    float m_run = -INFINITY;   // running max of c * s (log2 units)
    f32x4 lsum = f32x4{};      // row sums: entry (lane / 16) % 2 is this lane's

    for (int t = 0; t < ntiles; ++t) {
        const int st = t % R;
        if (t + R <= ntiles) wait_vmcnt<(R - 1) * 2 * kLoads>();
        else wait_vmcnt<0>();
        const LDS_AS char *kt = (const LDS_AS char *)lds[st][0];
        const LDS_AS char *vt = (const LDS_AS char *)lds[st][1];

        f32x16 sc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            sc = mfma32(*(const LDS_AS bf16x8 *)(kt + kread[ks]), qf[ks], sc);

        // Row i of this lane's S^T is key t0 + 8*(i/4) + 4*hi + i%4.
        const int t0 = start + t * kTileKeys;
        if (t0 + kTileKeys > mask_from) {
            const int last = kend - 1 - t0 - 4 * hi;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (8 * (i >> 2) + (i & 3) > last) sc[i] = -INFINITY;
        }

        // Online softmax in log2 units; the accumulators are rescaled only
        // when some row's maximum grew.
        float mt = sc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sc[i]);
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
                const i16x4 up =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(p + 8 * kRowBytes));
                const bf16x8 vop =
                    __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[db] = mfma32(vop, __builtin_bit_cast(bf16x8, pu[step]), acc[db]);
            }
        }
        if (t + R < ntiles) issue(t + R, st);
    }
    // No load may still write this workgroup's LDS when it ends.
    wait_vmcnt<0>();

    if (col >= a.M) return;
    const int64_t row = qrow0 + col;
    const float l = ((lane >> 4) & 1) ? lsum[1] : lsum[0];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse2 = l > 0.f ? m_run + log2f(l) : -INFINITY;
    if (direct) {
        uint16_t *dst = a.o + row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * g4 + e] * inv;
                bf16x4 y = __builtin_convertvector(x, bf16x4);
                if (bad) y = __builtin_bit_cast(bf16x4, u16x4{kBadBf16, kBadBf16, kBadBf16, kBadBf16});
                *(bf16x4 *)(dst + 32 * db + 8 * g4 + 4 * hi) = y;
            }
        }
        if (hi == 0) a.lse[row] = bad ? __uint_as_float(kBadBits) : lse2 * kLn2;
    } else {
        float *dst = a.ws_o + (row * a.nsplit + s) * D;
        if (!bad) {
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
        if (hi == 0) a.ws_lse[row * a.nsplit + s] = bad ? __uint_as_float(kBadBits) : lse2;
    }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Merges the splits of every query row whose sequence has more than one:
// one wave per row, four rows per workgroup.
template <int D>
__global__ void __launch_bounds__(256) paged_combine_kernel(PagedArgs a, int64_t rows) {
    constexpr int kPer = (D + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int b = (int)(row / ((int64_t)a.Hq * a.Tq));
    const int n = a.lens[b];
    if (n < 0 || n > a.max_blocks * a.bs) return;   // split 0 wrote NaN
    const int nsb = max(1, (n + a.L - 1) / a.L);
    if (nsb == 1) return;                           // split 0 wrote the result
    const float *pl = a.ws_lse + row * a.nsplit;
    float mx = -INFINITY;
    bool bad = false;
    for (int s = lane; s < nsb; s += 64) {
        const float x = pl[s];
        bad |= __float_as_uint(x) == kBadBits;
        mx = fmaxf(mx, x);
    }
    uint16_t *dst = a.o + row * D;
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            if (lane + 64 * k < D) dst[lane + 64 * k] = kBadBf16;
        if (lane == 0) a.lse[row] = __uint_as_float(kBadBits);
        return;
    }
    mx = wave_max(mx);
    const float m_use = mx == -INFINITY ? 0.f : mx;
    float o[kPer] = {};
    float wsum = 0.f;
    for (int s = 0; s < nsb; ++s) {
        const float w = __builtin_amdgcn_exp2f(pl[s] - m_use);
        wsum += w;
        const float *src = a.ws_o + (row * a.nsplit + s) * D;
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            if (lane + 64 * k < D) o[k] = __builtin_fmaf(w, src[lane + 64 * k], o[k]);
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        if (lane + 64 * k < D) {
            const __bf16 y = (__bf16)(o[k] * inv);
            dst[lane + 64 * k] = __builtin_bit_cast(uint16_t, y);
        }
    if (lane == 0) a.lse[row] = wsum > 0.f ? (mx + log2f(wsum)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct Plan {
    int L;        // keys per split
    int nsplit;   // splits of a sequence of max_blocks * block_size tokens
};

int64_t gcd64(int64_t x, int64_t y) {
    while (y) {
        const int64_t t = x % y;
        x = y;
        y = t;
    }
    return x;
}

// Splits of L keys, L a multiple of the 32-key tile and of the block size (a
// split starts on a block boundary) and at most 64 blocks long (one table
// entry per lane), sized so that a batch of the longest sequences makes about
// kTargetUnits units (never fewer than kMinSplit keys per split).
Plan make_plan(int B, int Hkv, int bs, int max_blocks) {
    const int64_t cap = (int64_t)max_blocks * bs;
    const int64_t unit = 32 * bs / gcd64(32, bs);
    const int64_t lmax = (kMaxEntries * (int64_t)bs / unit) * unit;
    int64_t L = (cap * B * Hkv + kTargetUnits - 1) / kTargetUnits;
    L = L < kMinSplit ? kMinSplit : L;
    L = (L + unit - 1) / unit * unit;
    L = L > lmax ? lmax : L;
    if (L >= cap) L = (cap + unit - 1) / unit * unit;   // one split holds everything
    Plan p;
    p.L = (int)L;
    p.nsplit = (int)((cap + L - 1) / L);
    return p;
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
    if ((int64_t)max_blocks * block_size > 0x7fffffff) return TESSERA_ERR_TOO_LARGE;
    const Plan p = make_plan(B, Hkv, block_size, max_blocks);
    if ((int64_t)p.nsplit * B * Hkv > 0x7fffffff) return TESSERA_ERR_TOO_LARGE;
    return TESSERA_OK;
}

int64_t workspace_bytes_for(int B, int Hq, int Hkv, int Tq, int D, const Plan &p) {
    if (p.nsplit <= 1) return 0;
    const int64_t cells = (int64_t)B * Hq * Tq * p.nsplit;
    return (cells * 4 + 255) / 256 * 256 + cells * D * 4;
}

}  // namespace

extern "C" long long tessera_paged_decode_workspace(int B, int Hq, int Hkv, int Tq, int D,
                                                    int block_size, int max_blocks) {
    const int st = check_sizes(B, Hq, Hkv, Tq, D, block_size, max_blocks);
    if (st != TESSERA_OK) return -(long long)st;
    return workspace_bytes_for(B, Hq, Hkv, Tq, D, make_plan(B, Hkv, block_size, max_blocks));
}

extern "C" int tessera_paged_decode(const void *q, const void *k_cache, const void *v_cache,
                                    const int *block_table, const int *context_lens, void *out,
                                    float *lse, int B, int Hq, int Hkv, int Tq, int D,
                                    int num_blocks, int block_size, int max_blocks, int causal,
                                    float scale, void *workspace, long long workspace_bytes,
                                    void *stream) {
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
    const Plan p = make_plan(B, Hkv, block_size, max_blocks);
    const int64_t need = workspace_bytes_for(B, Hq, Hkv, Tq, D, p);
    if (need > 0 && (!workspace || workspace_bytes < need)) return TESSERA_ERR_WORKSPACE;
    const size_t rows = (size_t)B * Hq * Tq;
    const size_t qbytes = rows * D * 2, lbytes = rows * 4;
    const size_t cbytes = (size_t)num_blocks * Hkv * block_size * D * 2;
    const size_t tbytes = (size_t)B * max_blocks * 4, nbytes = (size_t)B * 4;
    const size_t wbytes = (size_t)need;
    const void *ins[5] = {q, k_cache, v_cache, block_table, context_lens};
    const size_t insz[5] = {qbytes, cbytes, cbytes, tbytes, nbytes};
    for (int i = 0; i < 5; ++i)
        if (overlaps(out, qbytes, ins[i], insz[i]) || overlaps(lse, lbytes, ins[i], insz[i]) ||
            overlaps(workspace, wbytes, ins[i], insz[i]))
            return TESSERA_ERR_ALIAS;
    if (overlaps(out, qbytes, lse, lbytes) || overlaps(out, qbytes, workspace, wbytes) ||
        overlaps(lse, lbytes, workspace, wbytes))
        return TESSERA_ERR_ALIAS;

    PagedArgs a;
    a.q = (const uint16_t *)q;
    a.kc = (const uint16_t *)k_cache;
    a.vc = (const uint16_t *)v_cache;
    a.table = block_table;
    a.lens = context_lens;
    a.o = (uint16_t *)out;
    a.lse = lse;
    const int64_t cells = (int64_t)rows * p.nsplit;
    a.ws_lse = need > 0 ? (float *)workspace : nullptr;
    a.ws_o = need > 0 ? (float *)((char *)workspace + (cells * 4 + 255) / 256 * 256) : nullptr;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.Tq = Tq;
    a.M = a.G * Tq;
    a.bs = block_size;
    a.max_blocks = max_blocks;
    a.num_blocks = num_blocks;
    a.nbg = B * Hkv;
    a.nsplit = p.nsplit;
    a.L = p.L;
    a.causal = causal;
    a.qmode = scale < 0.f ? 1 : (scale == 0.f ? 2 : 0);
    a.c = scale == 0.f ? 1.0f : (float)(fabs((double)scale) * kLog2e);

    hipStream_t sm = (hipStream_t)stream;
    const dim3 grid((unsigned)((int64_t)p.nsplit * B * Hkv)), blk(64);
    if (D == 128) hipLaunchKernelGGL(paged_decode_kernel<128>, grid, blk, 0, sm, a);
    else if (D == 64) hipLaunchKernelGGL(paged_decode_kernel<64>, grid, blk, 0, sm, a);
    else hipLaunchKernelGGL(paged_decode_kernel<32>, grid, blk, 0, sm, a);
    st = tessera_launch_status();
    if (st != TESSERA_OK || p.nsplit <= 1) return st;
    const int64_t nrows = (int64_t)rows;
    const dim3 cgrid((unsigned)((nrows + 3) / 4)), cblk(256);
    if (D == 128) hipLaunchKernelGGL(paged_combine_kernel<128>, cgrid, cblk, 0, sm, a, nrows);
    else if (D == 64) hipLaunchKernelGGL(paged_combine_kernel<64>, cgrid, cblk, 0, sm, a, nrows);
    else hipLaunchKernelGGL(paged_combine_kernel<32>, cgrid, cblk, 0, sm, a, nrows);
    return tessera_launch_status();
}
