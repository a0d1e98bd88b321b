// tessera_attn_bwd.hip -- gfx950 (MI355X) kernels and C ABI of the attention
// backward pass: dq, dk, dv of the causal grouped-query attention forward for
// an output gradient dO (the fused backward that the page "Tessera: a
// from-scratch distillation and serving stack in one repository", section
// "The kernel set and its torch fallback", lists as missing).
//
// With P the forward's softmax weights, rebuilt from the forward's lse:
//     P_ij  = exp(scale q_i.k_j - lse_i)          dP_ij = dO_i . v_j
//     Delta_i = sum_d dO_id O_id                   dS_ij = P_ij (dP_ij - Delta_i)
//     dq_i = scale sum_j dS_ij k_j    dk_j = scale sum_i dS_ij q_i    dv_j = sum_i P_ij dO_i
// (dk and dv also summed over the query heads of a KV head's group).
//
// Two kernels, each owning what it accumulates, so no atomics and the result
// does not depend on scheduling:
//   * attn_bwd_dq_kernel: a workgroup per query tile (as in the forward); it
//     streams K and V tiles, forms S^T = K Q^T and dP^T = V dO^T on the
//     matrix cores, P and dS on the vector ALUs, and dq^T += K^T dS^T.  It
//     also writes Delta, from the dO and O rows it holds.
//   * attn_bwd_dkdv_kernel (attn_bwd_dkdv_lag_kernel at D = 128, and at
//     D <= 64 on grids of at most two workgroups per CU): a
//     workgroup per 128-key tile of one KV head; it streams the Q and dO
//     tiles of every query head of the group.  Two roles per key block: one
//     wave forms S = Q K^T and P and accumulates dv^T += dO^T P, the other
//     forms dP = dO V^T, takes P from the first through LDS and accumulates
//     dk^T += Q^T dS.
// All use v_mfma_f32_32x32x16_bf16 in the transposed form of the forward:
// the stationary operand (Q and dO, or K and V) sits in registers as the B
// operand, streamed tiles are read from LDS row by row (A operand of the
// score-like products) or through ds_read_b64_tr_b16 (A operand of the
// accumulating products), and the P / dS fragments a lane computes are
// already the B operand of the accumulating products.  Tiles are staged in
// LDS through registers; P and dS are rounded to bf16 for the matrix cores,
// everything else is fp32.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "tessera_attn.h"
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

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.442695040888963407f;
constexpr int kTileRows = 64;    // rows of a streamed tile

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte chunk swizzle of a D-wide bf16 row in LDS, for tiles read both by
// rows (16-byte A-operand reads) and transposed (ds_read_b64_tr_b16).  The LDS
// serves 256 bytes a cycle: 16 lanes of a row read, or 16 lanes of a
// transposed read (32 bytes of each of four consecutive rows).  Row reads stay
// conflict-free when the swizzle permutes the chunks of the rows that share a
// 256-byte window; transposed reads when the four rows' chunk pairs, XORed
// with their swizzles, land apart, so the swizzles of those rows must differ
// above bit 0.  D = 128 (one row per window): rows 4k..4k+3 take 0, 4, 8, 12
// plus k % 4.  D = 64 (two rows per window, even and odd apart): rows 2m and
// 2m+1 take 4 (m % 2) + (m / 2) % 4.  D = 32 (four rows per window): the
// transposed rows already sit in different quarters.  Each is periodic in 16
// rows, so the second 32-row block and the later 16-row steps are fixed
// offsets.
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else if constexpr (D == 64) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    else return (row >> 2) & 3;
}

// A streamed tile: kTileRows rows of D bf16 values, row-major with swizzled
// chunks.
template <int D>
struct Tile {
    static constexpr int kBytes = kTileRows * D * 2;
    static constexpr int kChunks = kTileRows * D / 8;
};

// Per-lane LDS byte offsets of the two A-operand reads of a tile.
//  * row read, block b (rows 32b .. 32b+31), step ks: lane (col, hi) reads 16
//    bytes of row 32b + col, dims 16 ks + 8 hi .. +7.  The swizzle of row
//    col + 32 equals that of row col, so block 1 is a fixed +32 rows.
//  * transposed read (X^T as the A operand, K dimension = rows): for step st
//    and dim block db, lane (grp, s16) reads 8 bytes of rows
//    16 st + 4 hi + s16/4 and that + 8, dims 32 db + 16 (grp & 1) + 4 (s16 & 3)
//    .. +3; after ds_read_b64_tr_b16 it holds rows {4hi..4hi+3, 8+4hi..8+4hi+3}
//    of one dim, the order of a lane's rows in an MFMA result, so a P or dS
//    fragment is the matching B operand as it stands.  st is a fixed offset.
template <int D>
struct TileOffsets {
    uint32_t row[D / 16];
    uint32_t tr[D / 32][2];
    __device__ __forceinline__ explicit TileOffsets(int lane) {
        constexpr int kRowBytes = D * 2;
        const int col = lane & 31, hi = lane >> 5, grp = lane >> 4, s16 = lane & 15;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            row[ks] = col * kRowBytes + (((2 * ks + hi) ^ swz<D>(col)) << 4);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int d = 32 * db + 16 * (grp & 1) + 4 * (s16 & 3);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = 4 * hi + (s16 >> 2) + 8 * h;
                tr[db][h] = r * kRowBytes + (((d >> 3) ^ swz<D>(r)) << 4) + (d & 7) * 2;
            }
        }
    }
};

template <int D>
__device__ __forceinline__ bf16x8 read_row(const LDS_AS char *tile, const TileOffsets<D> &o,
                                           int block, int ks) {
    return *(const LDS_AS bf16x8 *)(tile + o.row[ks] + block * 32 * D * 2);
}

template <int D>
__device__ __forceinline__ bf16x8 read_tr(const LDS_AS char *tile, const TileOffsets<D> &o,
                                          int st, int db) {
    const LDS_AS char *base = tile + st * 16 * D * 2;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(base + o.tr[db][0]));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(base + o.tr[db][1]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Global -> register -> LDS staging of kTileRows rows of one [T, D] head,
// spread over NT threads.  Rows at or past `rows` are written as zeros.
template <int D, int NT>
struct TileStager {
    static constexpr int kPer = (Tile<D>::kChunks + NT - 1) / NT;
    u32x4 r[kPer];
    __device__ __forceinline__ void fetch(const uint16_t *head, int row0, int rows, int tid) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = tid + NT * i;
            const int row = c / (D / 8), ch = c % (D / 8);
            const bool ok = (Tile<D>::kChunks % NT == 0 || c < Tile<D>::kChunks) &&
                            row0 + row < rows;
            r[i] = ok ? *(const u32x4 *)(head + (int64_t)(row0 + row) * D + 8 * ch) : u32x4{};
        }
    }
    __device__ __forceinline__ void store(LDS_AS char *tile, int tid) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = tid + NT * i;
            if (Tile<D>::kChunks % NT != 0 && c >= Tile<D>::kChunks) continue;
            const int row = c / (D / 8), ch = c % (D / 8);
            *(LDS_AS u32x4 *)(tile + row * D * 2 + ((ch ^ swz<D>(row)) << 4)) = r[i];
        }
    }
};

// The B-operand fragment of a stationary [32 rows, D] block: lane (col, hi)
// holds 8 values of row min(row0 + col, rows - 1), dims 16 ks + 8 hi .. +7.
template <int D>
__device__ __forceinline__ void load_fragment(bf16x8 (&f)[D / 16], const uint16_t *head,
                                              int row0, int rows, int lane) {
    const int row = min(row0 + (lane & 31), rows - 1);
    const uint16_t *src = head + (int64_t)row * D + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) f[ks] = *(const bf16x8 *)(src + 16 * ks);
}

// Workgroup barrier that publishes this wave's LDS writes but, unlike
// __syncthreads(), does not wait for its global loads in flight (the next
// tile's rows).  The empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Packs two f32x16 MFMA results (rows 0-31 and 32-63 of a 64-row step
// sequence) into the four bf16 B-operand words per 16-row step.
__device__ __forceinline__ void pack_steps(u32x4 (&out)[4], const f32x16 &a, const f32x16 &b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16x2 p0 = __builtin_convertvector((f32x2){a[2 * e], a[2 * e + 1]}, bf16x2);
        const bf16x2 p1 = __builtin_convertvector((f32x2){b[2 * e], b[2 * e + 1]}, bf16x2);
        out[e >> 2][e & 3] = __builtin_bit_cast(uint32_t, p0);
        out[2 + (e >> 2)][e & 3] = __builtin_bit_cast(uint32_t, p1);
    }
}

// Packs one f32x16 MFMA result (32 rows) into the bf16 B-operand words of its
// two 16-row steps.
__device__ __forceinline__ void pack_half(u32x4 (&out)[2], const f32x16 &a) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16x2 p = __builtin_convertvector((f32x2){a[2 * e], a[2 * e + 1]}, bf16x2);
        out[e >> 2][e & 3] = __builtin_bit_cast(uint32_t, p);
    }
}

// Writes a [D, 32] accumulator (lane: column col of its 32, dims of every
// block) times `mul` as bf16 row `row` of a [rows, D] tensor.
template <int D>
__device__ __forceinline__ void store_rows(uint16_t *dst_row, const f32x16 (&acc)[D / 32],
                                           float mul, int hi) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * g4 + e] * mul;
            *(bf16x4 *)(dst_row + 32 * db + 8 * g4 + 4 * hi) = __builtin_convertvector(x, bf16x4);
        }
    }
}

struct BwdArgs {
    const uint16_t *q, *k, *v, *o, *dout;
    const float *lse;
    uint16_t *dq, *dk, *dv;
    float *delta;
    int Hq, Hkv, T, G;
    int hg, nqb, nslots, nbh, nqt;   // dq kernel work split (as in the forward)
    int dq_waves;
    int nkt;                         // 128-key tiles per head (dk/dv kernel)
    int causal;
    float scale;
    float c;                         // scale * log2(e)
};

// ---------------------------------------------------------------------------
// dq (and Delta): a workgroup of NW waves per query tile of 32 * nqb rows and
// hg query heads of one KV head; wave w takes head w % hg and query block
// w / hg, as in the forward.  Eight waves, two per SIMD (at most 256
// registers each, which D = 128 fits by taking a tile's keys in two halves),
// so that one wave's matrix-core work hides the other's latencies.
// ---------------------------------------------------------------------------
template <int D>
constexpr int kDqWaves = 8;

template <int D, int NW = kDqWaves<D>>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
attn_bwd_dq_kernel(BwdArgs a) {
    constexpr int kDqThreads = 64 * NW;
    __shared__ __attribute__((aligned(16))) char lds_k[2][Tile<D>::kBytes];
    __shared__ __attribute__((aligned(16))) char lds_v[2][Tile<D>::kBytes];
    lds_poison_all();

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5, col = lane & 31;

    const int per_tile = a.nbh * a.nslots;
    const int qt_rev = blockIdx.x / per_tile;
    const int rem = blockIdx.x - qt_rev * per_tile;
    const int qt = a.causal ? (a.nqt - 1 - qt_rev) : qt_rev;
    const int slot = rem / a.nbh;
    const int bh = rem - slot * a.nbh;
    const int b = bh / a.Hkv;
    const int head = (bh - b * a.Hkv) * a.G + slot * a.hg + (w % a.hg);
    const int rows_wg = 32 * a.nqb;
    const int q0 = qt * rows_wg;
    const int qw0 = q0 + 32 * (w / a.hg);
    const int query = qw0 + col;
    const int T = a.T;
    const bool causal = a.causal != 0;

    const int64_t qhead = ((int64_t)b * a.Hq + head) * T;   // row index of (b, head, 0)
    const uint16_t *khead = a.k + (int64_t)bh * T * D;
    const uint16_t *vhead = a.v + (int64_t)bh * T * D;

    const int q_end = min(q0 + rows_wg, T);
    const int ntiles = ((causal ? q_end : T) + kTileRows - 1) / kTileRows;

    TileStager<D, kDqThreads> ks_, vs_;
    ks_.fetch(khead, 0, T, tid);
    vs_.fetch(vhead, 0, T, tid);

    // Stationary fragments, lse and Delta of this lane's query row.
    bf16x8 qf[D / 16], dof[D / 16], of[D / 16];
    load_fragment<D>(qf, a.q + qhead * D, qw0, T, lane);
    load_fragment<D>(dof, a.dout + qhead * D, qw0, T, lane);
    load_fragment<D>(of, a.o + qhead * D, qw0, T, lane);
    float dl = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) dl += (float)dof[ks][e] * (float)of[ks][e];
    }
    dl += __shfl_xor(dl, 32);                    // the other half of the row's dims
    const int qrow = min(query, T - 1);
    const float lse2 = a.lse[qhead + qrow] * kLog2e;
    if (hi == 0 && query < T) a.delta[qhead + query] = dl;

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
    const TileOffsets<D> off(lane);
    const float c = a.c;

    ks_.store((LDS_AS char *)lds_k[0], tid);
    vs_.store((LDS_AS char *)lds_v[0], tid);
    __syncthreads();
    // Tile t sits in buffer t % 2.  The loop below is unrolled by two, so the
    // buffer index is a compile-time constant and each LDS read takes its
    // buffer's base as an immediate offset.
    auto one_tile = [&]<int CUR>(int t) __attribute__((always_inline)) {
        if (t + 1 < ntiles) {
            ks_.fetch(khead, (t + 1) * kTileRows, T, tid);
            vs_.fetch(vhead, (t + 1) * kTileRows, T, tid);
        }
        const LDS_AS char *kt = (const LDS_AS char *)lds_k[CUR];
        const LDS_AS char *vt = (const LDS_AS char *)lds_v[CUR];
        const int j0 = t * kTileRows;
        const bool masked = j0 + kTileRows > T || (causal && j0 + kTileRows - 1 > qw0);
        // The tile's keys in two 32-key halves (S, dP, dS and the dq update of
        // one half at a time), which keeps the registers of a wave within 256.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x16 sh = {}, ph = {};
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                sh = mfma32(read_row<D>(kt, off, h, ks), qf[ks], sh);
                ph = mfma32(read_row<D>(vt, off, h, ks), dof[ks], ph);
            }
            // exponent of P; keys hidden from this query (causal) or past T get -inf
            f32x16 x;
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = __builtin_fmaf(sh[i], c, -lse2);
            if (masked) {
                const int last = (causal ? qrow : T - 1) - j0 - 32 * h - 4 * hi;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (8 * (i >> 2) + (i & 3) > last) x[i] = -INFINITY;
            }
            f32x16 d;   // dS
#pragma unroll
            for (int i = 0; i < 16; ++i) d[i] = __builtin_amdgcn_exp2f(x[i]) * (ph[i] - dl);
            u32x4 dsu[2];
            pack_half(dsu, d);
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    acc[db] = mfma32(read_tr<D>(kt, off, 2 * h + st, db),
                                     __builtin_bit_cast(bf16x8, dsu[st]), acc[db]);
            }
        }
        if (t + 1 < ntiles) {
            ks_.store((LDS_AS char *)lds_k[CUR ^ 1], tid);
            vs_.store((LDS_AS char *)lds_v[CUR ^ 1], tid);
        }
        __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
        one_tile.template operator()<0>(t);
        if (t + 1 < ntiles) one_tile.template operator()<1>(t + 1);
    }
    if (query < T) store_rows<D>(a.dq + (qhead + query) * D, acc, a.scale, hi);
}

// ---------------------------------------------------------------------------
// dk, dv: a workgroup of 8 waves per 128-key tile of one KV head, two per
// SIMD (at most 256 registers each; at D <= 64 two workgroups share a CU).
// Waves w and w + 4 own keys k0 + 32 (w % 4) .. +31: wave w (w < 4) forms S
// and P and accumulates
// dv^T += dO^T P; wave w + 4 forms dP, takes P from wave w through LDS,
// forms dS and accumulates dk^T += Q^T dS.  Each holds one set of
// accumulators and executes half the products, and the two waves of a SIMD
// overlap one's matrix work with the other's vector work.  The workgroup
// loops over the query heads of the group and, for each, over the 64-row
// query tiles that can see these keys, whose Q and dO rows stream through
// LDS shared by all eight waves; each tile is taken in two 32-row halves.
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 8;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKeyTile = 128;
// Waves per SIMD the dk/dv kernel is built for: at D <= 64 a wave fits 128
// registers and the workgroup's LDS (66 KB at D = 64) leaves room for a second
// workgroup per CU, whose waves hide the first's barrier and load waits.
template <int D>
constexpr int kKvWavesPerSimd = D == 128 ? 2 : 4;

template <int D>
__global__ void __launch_bounds__(kKvThreads)
__attribute__((amdgpu_waves_per_eu(kKvWavesPerSimd<D>, kKvWavesPerSimd<D>)))
attn_bwd_dkdv_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) char lds_q[2][Tile<D>::kBytes];
    __shared__ __attribute__((aligned(16))) char lds_d[2][Tile<D>::kBytes];
    __shared__ __attribute__((aligned(16))) float lds_l[2][kTileRows];   // lse * log2 e
    __shared__ __attribute__((aligned(16))) float lds_m[2][kTileRows];   // Delta
    // P of one 32-row half from each dv wave to its dk wave: [half][pair][k][lane]
    // holds the lane's P registers 4k .. 4k+3.
    __shared__ __attribute__((aligned(16))) f32x4 lds_p[2][4][4][64];
    lds_poison_all();

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool dk_wave = w >= 4;   // wave-uniform role
    const int hi = lane >> 5, col = lane & 31;

    // key tile 0 first: under the causal mask it has the most query rows after it
    const int kt_idx = (int)(blockIdx.x / a.nbh);
    const int bh = blockIdx.x - kt_idx * a.nbh;
    const int b = bh / a.Hkv;
    const int hkv = bh - b * a.Hkv;
    const int T = a.T;
    const bool causal = a.causal != 0;
    const int k0 = kt_idx * kKeyTile;
    const int kw0 = k0 + 32 * (w & 3);
    const int key = kw0 + col;

    const uint16_t *khead = a.k + (int64_t)bh * T * D;
    const uint16_t *vhead = a.v + (int64_t)bh * T * D;
    bf16x8 kv[D / 16];   // K (S on the dv waves) or V (dP on the dk waves)
    load_fragment<D>(kv, dk_wave ? vhead : khead, kw0, T, lane);

    f32x16 acc[D / 32];   // dv^T or dk^T of this wave's keys
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
    const TileOffsets<D> off(lane);
    const float c = a.c;

    // the (head, query tile) sequence: heads of the group, tiles from the
    // first that reaches these keys
    const int qt_first = causal ? k0 / kTileRows : 0;
    const int nq = (T + kTileRows - 1) / kTileRows;
    const int per_head = nq - qt_first;
    const int nsteps = a.G * per_head;
    const int64_t head0 = (int64_t)b * a.Hq + (int64_t)hkv * a.G;   // first query head

    TileStager<D, kKvThreads> qs_, ds_;
    float l_in = 0.f, m_in = 0.f;
    // Steps are fetched in order; the (head, query tile) of the next fetch is
    // kept as two counters (a division by per_head would cost tens of
    // instructions per step).
    int f_g = 0, f_qi = 0;
    auto fetch = [&]() __attribute__((always_inline)) {
        const int q0 = (qt_first + f_qi) * kTileRows;
        const int64_t hrow = (head0 + f_g) * T;
        qs_.fetch(a.q + hrow * D, q0, T, tid);
        ds_.fetch(a.dout + hrow * D, q0, T, tid);
        if (tid < kTileRows) {
            const bool ok = q0 + tid < T;
            l_in = ok ? a.lse[hrow + q0 + tid] * kLog2e : INFINITY;   // P = 0 past T
            m_in = ok ? a.delta[hrow + q0 + tid] : 0.f;
        }
        if (++f_qi == per_head) {
            f_qi = 0;
            ++f_g;
        }
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
        qs_.store((LDS_AS char *)lds_q[buf], tid);
        ds_.store((LDS_AS char *)lds_d[buf], tid);
        if (tid < kTileRows) {
            lds_l[buf][tid] = l_in;
            lds_m[buf][tid] = m_in;
        }
    };

    fetch();
    store(0);
    __syncthreads();
    int c_qi = 0;   // query tile of the current step, counted like f_qi
    for (int step = 0; step < nsteps; ++step) {
        const int cur = step & 1;
        if (step + 1 < nsteps) fetch();
        const int q0 = (qt_first + c_qi) * kTileRows;
        if (++c_qi == per_head) c_qi = 0;
        const LDS_AS char *qt = (const LDS_AS char *)lds_q[cur];
        const LDS_AS char *dt = (const LDS_AS char *)lds_d[cur];
        const bool need_mask = causal && q0 < kw0 + 31;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // Lane: key column `key`; register i holds query row
            // q0 + 32 h + 8 (i / 4) + 4 hi + i % 4.  The dv wave forms S
            // (from Q) and P, the dk wave dP (from dO).
            f32x16 sp = {};
            const LDS_AS char *lhs = dk_wave ? dt : qt;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) sp = mfma32(read_row<D>(lhs, off, h, ks), kv[ks], sp);
            f32x4 (&xp)[4][64] = lds_p[h][w & 3];
            if (!dk_wave) {
                // exponent of P; on a step that crosses the diagonal, query
                // rows before this lane's key get -inf (one branch per step, so
                // the other steps run no mask instructions)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 l4 = *(const LDS_AS f32x4 *)&lds_l[cur][32 * h + 8 * j + 4 * hi];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        sp[4 * j + u] = __builtin_fmaf(sp[4 * j + u], c, -l4[u]);
                }
                if (need_mask) {
                    const int first = key - q0 - 32 * h - 4 * hi;   // first visible register row
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (8 * (i >> 2) + (i & 3) < first) sp[i] = -INFINITY;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        sp[4 * j + u] = __builtin_amdgcn_exp2f(sp[4 * j + u]);
                    *(LDS_AS f32x4 *)&xp[j][lane] =
                        f32x4{sp[4 * j], sp[4 * j + 1], sp[4 * j + 2], sp[4 * j + 3]};
                }
            }
            lds_barrier();   // P is in LDS
            if (dk_wave) {
                // dS = P (dP - Delta)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 32 * h + 8 * j + 4 * hi;
                    const f32x4 m4 = *(const LDS_AS f32x4 *)&lds_m[cur][r];
                    const f32x4 p4 = *(const LDS_AS f32x4 *)&xp[j][lane];
#pragma unroll
                    for (int u = 0; u < 4; ++u) sp[4 * j + u] = p4[u] * (sp[4 * j + u] - m4[u]);
                }
            }
            u32x4 xu[2];
            pack_half(xu, sp);
            const LDS_AS char *src = dk_wave ? qt : dt;   // Q^T for dk, dO^T for dv
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    acc[db] = mfma32(read_tr<D>(src, off, 2 * h + st, db),
                                     __builtin_bit_cast(bf16x8, xu[st]), acc[db]);
            }
        }
        if (step + 1 < nsteps) store(cur ^ 1);
        __syncthreads();
    }
    if (key < T) {
        if (dk_wave) store_rows<D>(a.dk + ((int64_t)bh * T + key) * D, acc, a.scale, hi);
        else store_rows<D>(a.dv + ((int64_t)bh * T + key) * D, acc, 1.f, hi);
    }
}

// dk, dv with the hand-over of P one step late (D = 128, and D <= 64 on grids
// too small to give every CU a second workgroup).  The roles are those of
// attn_bwd_dkdv_kernel, but the dk wave forms dS and dk for step s - 1 while
// the dv wave works on step s, so the P it reads was published by the
// barrier that ends every step and no barrier is needed inside one (with one
// workgroup on a CU, nothing else hides those).  Q
// tiles, lse and Delta therefore stay in LDS one step longer (three
// buffers), P is double-buffered by step, and the loop runs one step past
// the last tile for the dk wave.  Same arithmetic, in the same order.
template <int D>
__global__ void __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv_lag_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) char lds_q[3][Tile<D>::kBytes];
    __shared__ __attribute__((aligned(16))) char lds_d[2][Tile<D>::kBytes];
    __shared__ __attribute__((aligned(16))) float lds_l[3][kTileRows];   // lse * log2 e
    __shared__ __attribute__((aligned(16))) float lds_m[3][kTileRows];   // Delta
    // P of step s in [s % 2][half][pair][k][lane] (the lane's P registers 4k .. 4k+3)
    __shared__ __attribute__((aligned(16))) f32x4 lds_p[2][2][4][4][64];
    lds_poison_all();

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool dk_wave = w >= 4;   // wave-uniform role
    const int hi = lane >> 5, col = lane & 31;

    const int kt_idx = (int)(blockIdx.x / a.nbh);
    const int bh = blockIdx.x - kt_idx * a.nbh;
    const int b = bh / a.Hkv;
    const int hkv = bh - b * a.Hkv;
    const int T = a.T;
    const bool causal = a.causal != 0;
    const int k0 = kt_idx * kKeyTile;
    const int kw0 = k0 + 32 * (w & 3);
    const int key = kw0 + col;

    const uint16_t *khead = a.k + (int64_t)bh * T * D;
    const uint16_t *vhead = a.v + (int64_t)bh * T * D;
    bf16x8 kv[D / 16];   // K (S on the dv waves) or V (dP on the dk waves)
    load_fragment<D>(kv, dk_wave ? vhead : khead, kw0, T, lane);

    f32x16 acc[D / 32];   // dv^T or dk^T of this wave's keys
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
    const TileOffsets<D> off(lane);
    const float c = a.c;

    const int qt_first = causal ? k0 / kTileRows : 0;
    const int nq = (T + kTileRows - 1) / kTileRows;
    const int per_head = nq - qt_first;
    const int nsteps = a.G * per_head;
    const int64_t head0 = (int64_t)b * a.Hq + (int64_t)hkv * a.G;

    TileStager<D, kKvThreads> qs_, ds_;
    float l_in = 0.f, m_in = 0.f;
    // Steps are fetched in order (in either role's loop); the (head, query
    // tile) of the next fetch is kept as two counters, not divided out.
    int f_g = 0, f_qi = 0;
    auto fetch = [&]() __attribute__((always_inline)) {
        const int q0 = (qt_first + f_qi) * kTileRows;
        const int64_t hrow = (head0 + f_g) * T;
        qs_.fetch(a.q + hrow * D, q0, T, tid);
        ds_.fetch(a.dout + hrow * D, q0, T, tid);
        if (tid < kTileRows) {
            const bool ok = q0 + tid < T;
            l_in = ok ? a.lse[hrow + q0 + tid] * kLog2e : INFINITY;   // P = 0 past T
            m_in = ok ? a.delta[hrow + q0 + tid] : 0.f;
        }
        if (++f_qi == per_head) {
            f_qi = 0;
            ++f_g;
        }
    };
    // Buffers of step s: Q tile, lse and Delta in [s % 3], dO tile and P in
    // [s % 2].  The step loops below are unrolled by six, so every buffer index
    // is a compile-time constant and each LDS read takes its buffer's base as
    // an immediate offset instead of adding it per read.
    auto store = [&]<int B3, int B2>() __attribute__((always_inline)) {
        qs_.store((LDS_AS char *)lds_q[B3], tid);
        ds_.store((LDS_AS char *)lds_d[B2], tid);
        if (tid < kTileRows) {
            lds_l[B3][tid] = l_in;
            lds_m[B3][tid] = m_in;
        }
    };

    fetch();
    store.template operator()<0, 0>();
    __syncthreads();
    // Each role runs its own loop (registers are allocated per role); both
    // pass the same barriers, one per step, and share the tile staging.
    auto step_end = [&]<int B3, int B2>(int step) __attribute__((always_inline)) {
        if (step + 1 < nsteps) store.template operator()<(B3 + 1) % 3, B2 ^ 1>();
        __syncthreads();
    };
    // Runs step, step + 1, ... up to nsteps (inclusive), six per pass.
    auto run_steps = [&](auto &&one) __attribute__((always_inline)) {
        for (int step = 0; step <= nsteps; step += 6) {
            one.template operator()<0, 0>(step);
            if (step + 1 > nsteps) break;
            one.template operator()<1, 1>(step + 1);
            if (step + 2 > nsteps) break;
            one.template operator()<2, 0>(step + 2);
            if (step + 3 > nsteps) break;
            one.template operator()<0, 1>(step + 3);
            if (step + 4 > nsteps) break;
            one.template operator()<1, 0>(step + 4);
            if (step + 5 > nsteps) break;
            one.template operator()<2, 1>(step + 5);
        }
    };
    if (!dk_wave) {
        int c_qi = 0;   // query tile of the current step, counted like f_qi
        auto dv_step = [&]<int B3, int B2>(int step) __attribute__((always_inline)) {
            if (step + 1 < nsteps) fetch();
            if (step < nsteps) {
                const int q0 = (qt_first + c_qi) * kTileRows;
                if (++c_qi == per_head) c_qi = 0;
                const bool need_mask = causal && q0 < kw0 + 31;
                const LDS_AS char *qt = (const LDS_AS char *)lds_q[B3];
                const LDS_AS char *dt = (const LDS_AS char *)lds_d[B2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    // register i holds query row q0 + 32 h + 8 (i / 4) + 4 hi + i % 4
                    f32x16 sp = {};
#pragma unroll
                    for (int ks = 0; ks < D / 16; ++ks)
                        sp = mfma32(read_row<D>(qt, off, h, ks), kv[ks], sp);
                    f32x4 (&xp)[4][64] = lds_p[B2][h][w & 3];
                    // exponent of P, masked in one branch per step (as above)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const f32x4 l4 =
                            *(const LDS_AS f32x4 *)&lds_l[B3][32 * h + 8 * j + 4 * hi];
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            sp[4 * j + u] = __builtin_fmaf(sp[4 * j + u], c, -l4[u]);
                    }
                    if (need_mask) {
                        const int first = key - q0 - 32 * h - 4 * hi;
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            if (8 * (i >> 2) + (i & 3) < first) sp[i] = -INFINITY;
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            sp[4 * j + u] = __builtin_amdgcn_exp2f(sp[4 * j + u]);
                        *(LDS_AS f32x4 *)&xp[j][lane] =
                            f32x4{sp[4 * j], sp[4 * j + 1], sp[4 * j + 2], sp[4 * j + 3]};
                    }
                    u32x4 xu[2];
                    pack_half(xu, sp);
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
#pragma unroll
                        for (int db = 0; db < D / 32; ++db)
                            acc[db] = mfma32(read_tr<D>(dt, off, 2 * h + st, db),
                                             __builtin_bit_cast(bf16x8, xu[st]), acc[db]);
                    }
                }
            }
            step_end.template operator()<B3, B2>(step);
        };
        run_steps(dv_step);
    } else {
        f32x16 dp[2];   // dP of the step before (both halves)
        auto dk_step = [&]<int B3, int B2>(int step) __attribute__((always_inline)) {
            if (step + 1 < nsteps) fetch();
            if (step > 0) {
                // dS and dk of the step before: its Q tile, Delta and P are still in LDS
                constexpr int P3 = (B3 + 2) % 3, P2 = B2 ^ 1;
                const LDS_AS char *qt = (const LDS_AS char *)lds_q[P3];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f32x4 (&xp)[4][64] = lds_p[P2][h][w & 3];
                    f32x16 ds;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 32 * h + 8 * j + 4 * hi;
                        const f32x4 m4 = *(const LDS_AS f32x4 *)&lds_m[P3][r];
                        const f32x4 p4 = *(const LDS_AS f32x4 *)&xp[j][lane];
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            ds[4 * j + u] = p4[u] * (dp[h][4 * j + u] - m4[u]);
                    }
                    u32x4 xu[2];
                    pack_half(xu, ds);
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
#pragma unroll
                        for (int db = 0; db < D / 32; ++db)
                            acc[db] = mfma32(read_tr<D>(qt, off, 2 * h + st, db),
                                             __builtin_bit_cast(bf16x8, xu[st]), acc[db]);
                    }
                }
            }
            if (step < nsteps) {
                const LDS_AS char *dt = (const LDS_AS char *)lds_d[B2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    dp[h] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < D / 16; ++ks)
                        dp[h] = mfma32(read_row<D>(dt, off, h, ks), kv[ks], dp[h]);
                }
            }
            step_end.template operator()<B3, B2>(step);
        };
        run_steps(dk_step);
    }
    if (key < T) {
        if (dk_wave) store_rows<D>(a.dk + ((int64_t)bh * T + key) * D, acc, a.scale, hi);
        else store_rows<D>(a.dv + ((int64_t)bh * T + key) * D, acc, 1.f, hi);
    }
}

bool overlaps(const void *x, size_t nx, const void *y, size_t ny) {
    const uintptr_t p = (uintptr_t)x, q = (uintptr_t)y;
    return p < q + ny && q < p + nx;
}

// Up to this many dk/dv workgroups per compute unit, D <= 64 runs the
// one-step-late build (one workgroup per CU, no barrier inside a step) rather
// than the two-workgroups-per-CU build: measured on MI355X at D = 64 and 32,
// 256 and 512 workgroups went 9-18 % faster, 1024 and 2048 went 4-16 % slower.
constexpr int kLagGridPerCu = 2;

int bwd_compute_units() {
    int dev = -1, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        n > 0)
        return n;
    return 256;   // MI355X
}

}  // namespace

extern "C" int tessera_attn_bwd(const void *q, const void *k, const void *v, const void *out,
                                const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                float *delta, int B, int Hq, int Hkv, int T, int D, int causal,
                                float scale, void *stream) {
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || !delta)
        return TESSERA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || Hq % Hkv != 0) return TESSERA_ERR_SHAPE;
    if (D != 32 && D != 64 && D != 128) return TESSERA_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return TESSERA_ERR_CAUSAL;
    if (!isfinite(scale)) return TESSERA_ERR_SCALE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout |
         (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15u)
        return TESSERA_ERR_ALIGN;
    if (((uintptr_t)lse | (uintptr_t)delta) & 3u) return TESSERA_ERR_ALIGN;
    const size_t qb = (size_t)B * Hq * T * D * 2, kb = (size_t)B * Hkv * T * D * 2;
    const size_t lb = (size_t)B * Hq * T * 4;
    const void *ins[6] = {q, k, v, out, dout, lse};
    const size_t insz[6] = {qb, kb, kb, qb, qb, lb};
    void *outs[4] = {dq, dk, dv, delta};
    const size_t outsz[4] = {qb, kb, kb, lb};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return TESSERA_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], outsz[i], outs[j], outsz[j])) return TESSERA_ERR_ALIAS;
    }

    BwdArgs a;
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.o = (const uint16_t *)out;
    a.dout = (const uint16_t *)dout;
    a.lse = lse;
    a.dq = (uint16_t *)dq;
    a.dk = (uint16_t *)dk;
    a.dv = (uint16_t *)dv;
    a.delta = delta;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.T = T;
    a.G = Hq / Hkv;
    a.dq_waves = D == 128 ? kDqWaves<128> : kDqWaves<64>;
    a.hg = (a.G % 4 == 0) ? 4 : (a.G % 2 == 0) ? 2 : 1;
    a.nqb = a.dq_waves / a.hg;
    a.nslots = a.G / a.hg;
    a.nbh = B * Hkv;
    a.nqt = (T + 32 * a.nqb - 1) / (32 * a.nqb);
    a.nkt = (T + kKeyTile - 1) / kKeyTile;
    a.causal = causal;
    a.scale = scale;
    a.c = scale * kLog2e;
    const int64_t grid_dq = (int64_t)a.nqt * a.nbh * a.nslots;
    const int64_t grid_kv = (int64_t)a.nkt * a.nbh;
    if (grid_dq > 0x7fffffff || grid_kv > 0x7fffffff) return TESSERA_ERR_TOO_LARGE;

    hipStream_t s = (hipStream_t)stream;
    const dim3 g1((unsigned)grid_dq), b1(64 * a.dq_waves), g2((unsigned)grid_kv), b2(kKvThreads);
    // dq first: it writes the Delta rows the dk/dv kernel reads.
    // dk/dv at D <= 64: the two-workgroups-per-CU build where the grid fills
    // the second slots, else the one-step-late build (see there).
    const bool lag = grid_kv <= kLagGridPerCu * (int64_t)bwd_compute_units();
    int st;
    if (D == 128) {
        st = tessera_launch(attn_bwd_dq_kernel<128>, g1, b1, s, a);
        if (st == TESSERA_OK) st = tessera_launch(attn_bwd_dkdv_lag_kernel<128>, g2, b2, s, a);
    } else if (D == 64) {
        st = tessera_launch(attn_bwd_dq_kernel<64>, g1, b1, s, a);
        if (st == TESSERA_OK)
            st = lag ? tessera_launch(attn_bwd_dkdv_lag_kernel<64>, g2, b2, s, a)
                     : tessera_launch(attn_bwd_dkdv_kernel<64>, g2, b2, s, a);
    } else {
        st = tessera_launch(attn_bwd_dq_kernel<32>, g1, b1, s, a);
        if (st == TESSERA_OK)
            st = lag ? tessera_launch(attn_bwd_dkdv_lag_kernel<32>, g2, b2, s, a)
                     : tessera_launch(attn_bwd_dkdv_kernel<32>, g2, b2, s, a);
    }
    return st;
}
