// tessera_attn_f32.hip -- the fp32 attention forward (tessera_attn_fwd_f32):
// the same operation as the bf16 hot path (page "Tessera: a from-scratch
// distillation and serving stack in one repository", section "The kernel set
// and its torch fallback") with fp32 inputs and outputs, computed on the
// vector ALUs in fp32.  Arguments are validated by the same routine as the
// bf16 entry points (tessera_attn.hip).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "tessera_attn.h"
#include "launch.h"
#include "lds_poison.h"

namespace {

constexpr float kLn2 = 0.693147180559945309f;
constexpr double kLog2e = 1.442695040888963407;

// ---------------------------------------------------------------------------
// fp32 kernel (vector ALUs): 64 query rows per workgroup, four lanes per row,
// each lane owning D/4 consecutive dims; K/V tiles staged in LDS.  The online
// softmax takes keys eight at a time: the eight scores are formed side by
// side (independent dot products and lane exchanges), then one running-max
// update, eight exponentials and one rescale of the accumulator serve them
// all, so the loop is bound by issue rather than by one long dependency chain
// per key.  Exponentials run in log2 units (exp2 of the score times
// scale * log2 e), and lse is converted back to natural log at the end.
// ---------------------------------------------------------------------------
constexpr int kF32Rows = 64;
constexpr int kF32Keys = 64;
constexpr int kF32Block = 8;   // keys per softmax update

template <int D>
__global__ void __launch_bounds__(256)
attn_fwd_f32_kernel(const float *__restrict__ q, const float *__restrict__ k,
                    const float *__restrict__ v, float *__restrict__ out,
                    float *__restrict__ lse, int Hq, int Hkv, int T, int ntiles, int causal,
                    float scale) {
    constexpr int kPer = D / 4;     // dims per lane
    constexpr int kVec = kPer / 4;  // ... as float4
    __shared__ __attribute__((aligned(16))) float sk[kF32Keys * D];
    __shared__ __attribute__((aligned(16))) float sv[kF32Keys * D];
    lds_poison_all();

    const int tid = threadIdx.x;
    const int sub = tid & 3;
    const int tile = blockIdx.x % ntiles;
    const int bh = blockIdx.x / ntiles;   // b * Hq + h
    const int h = bh % Hq;
    const int b = bh / Hq;
    const int i = tile * kF32Rows + (tid >> 2);
    const int64_t kv0 = ((int64_t)b * Hkv + h / (Hq / Hkv)) * T * D;
    const int64_t qrow = ((int64_t)bh * T + min(i, T - 1)) * D;
    const float c2 = scale * (float)kLog2e;   // score -> log2 units

    float4 qr[kVec], acc[kVec];
#pragma unroll
    for (int t = 0; t < kVec; ++t) {
        qr[t] = *(const float4 *)(q + qrow + sub * kPer + 4 * t);
        acc[t] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float m = -INFINITY, l = 0.f;   // m in log2 units

    const int last_q = min(T, tile * kF32Rows + kF32Rows) - 1;
    const int kend = causal ? last_q + 1 : T;
    for (int j0 = 0; j0 < kend; j0 += kF32Keys) {
        __syncthreads();
        for (int e = tid; e < kF32Keys * D / 4; e += 256) {
            const int row = e / (D / 4), c4 = e % (D / 4);
            float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
            if (j0 + row < T) {
                kk = *(const float4 *)(k + kv0 + (int64_t)(j0 + row) * D + 4 * c4);
                vv = *(const float4 *)(v + kv0 + (int64_t)(j0 + row) * D + 4 * c4);
            }
            *(float4 *)(sk + row * D + 4 * c4) = kk;
            *(float4 *)(sv + row * D + 4 * c4) = vv;
        }
        __syncthreads();
        const int jn = min(kF32Keys, kend - j0);
        for (int jb = 0; jb < jn; jb += kF32Block) {
            float x[kF32Block];
#pragma unroll
            for (int u = 0; u < kF32Block; ++u) {
                const float4 *kr = (const float4 *)(sk + (jb + u) * D + sub * kPer);
                float part = 0.f;
#pragma unroll
                for (int t = 0; t < kVec; ++t) {
                    const float4 kk = kr[t];
                    part = fmaf(qr[t].x, kk.x, part);
                    part = fmaf(qr[t].y, kk.y, part);
                    part = fmaf(qr[t].z, kk.z, part);
                    part = fmaf(qr[t].w, kk.w, part);
                }
                x[u] = part;
            }
#pragma unroll
            for (int u = 0; u < kF32Block; ++u) x[u] += __shfl_xor(x[u], 1);
#pragma unroll
            for (int u = 0; u < kF32Block; ++u) x[u] += __shfl_xor(x[u], 2);
            // keys past the tile's last visible key, and (causal) past this row, get -inf
            float mb = m;
#pragma unroll
            for (int u = 0; u < kF32Block; ++u) {
                const int kj = j0 + jb + u;
                x[u] = (kj < kend && !(causal && kj > i)) ? x[u] * c2 : -INFINITY;
                mb = fmaxf(mb, x[u]);
            }
            // a row with no visible key yet keeps l = 0 and acc = 0
            const float mref = mb == -INFINITY ? 0.f : mb;
            const float alpha = __builtin_amdgcn_exp2f(m - mref);
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < kF32Block; ++u) {
                x[u] = __builtin_amdgcn_exp2f(x[u] - mref);
                ps += x[u];
            }
            l = fmaf(l, alpha, ps);
#pragma unroll
            for (int t = 0; t < kVec; ++t) {
                float4 a4 = acc[t];
                a4.x *= alpha;
                a4.y *= alpha;
                a4.z *= alpha;
                a4.w *= alpha;
#pragma unroll
                for (int u = 0; u < kF32Block; ++u) {
                    const float4 vv = *(const float4 *)(sv + (jb + u) * D + sub * kPer + 4 * t);
                    a4.x = fmaf(x[u], vv.x, a4.x);
                    a4.y = fmaf(x[u], vv.y, a4.y);
                    a4.z = fmaf(x[u], vv.z, a4.z);
                    a4.w = fmaf(x[u], vv.w, a4.w);
                }
                acc[t] = a4;
            }
            m = mb;
        }
    }
    if (i < T) {
        const float inv = 1.f / l;
#pragma unroll
        for (int t = 0; t < kVec; ++t) {
            const float4 a4 = acc[t];
            *(float4 *)(out + qrow + sub * kPer + 4 * t) =
                make_float4(a4.x * inv, a4.y * inv, a4.z * inv, a4.w * inv);
        }
        if (sub == 0) lse[(int64_t)bh * T + i] = m * kLn2 + logf(l);
    }
}

}  // namespace

extern "C" int tessera_attn_fwd_f32(const float *q, const float *k, const float *v, float *out,
                                    float *lse, int B, int Hq, int Hkv, int T, int D, int causal,
                                    float scale, void *stream) {
    const int st = tessera_validate_fwd(q, k, v, out, lse, B, Hq, Hkv, T, T, D, causal, scale, 4);
    if (st != TESSERA_OK) return st;
    const int ntiles = (T + kF32Rows - 1) / kF32Rows;
    const int64_t grid = (int64_t)ntiles * B * Hq;
    if (grid > 0x7fffffff) return TESSERA_ERR_TOO_LARGE;
    hipStream_t s = (hipStream_t)stream;
    const dim3 g((unsigned)grid), blk(256);
    if (D == 128)
        return tessera_launch(attn_fwd_f32_kernel<128>, g, blk, s, q, k, v, out, lse, Hq, Hkv, T,
                              ntiles, causal, scale);
    if (D == 64)
        return tessera_launch(attn_fwd_f32_kernel<64>, g, blk, s, q, k, v, out, lse, Hq, Hkv, T,
                              ntiles, causal, scale);
    return tessera_launch(attn_fwd_f32_kernel<32>, g, blk, s, q, k, v, out, lse, Hq, Hkv, T,
                          ntiles, causal, scale);
}
