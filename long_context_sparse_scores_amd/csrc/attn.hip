// Sparse absorbed-MLA attention over the selected latent rows (gfx950).
//
// [TEARDOWN, 刀一 DSA] (clawlihai.cn GLM-5.2 1M architecture teardown): full
// attention runs over only the 2048 selected tokens.  [TEARDOWN, 刀三 MLA]:
// the cache keeps one compressed latent vector per token, shared by all 64
// heads (kv_lora_rank 512; with the 64-dim rope part a row holds 576 bf16).
// In absorbed form each head's query already lives in that latent space, so
//   z_j = sm_scale * <q_h, c_j>   (576 dims),   o_h = softmax(z) . c[:, 0:512].
//
// Work unit: one query (b,t) and a split of its index list.  A workgroup of
// four waves gathers 32 selected rows at a time into LDS (1152 bytes each,
// padded pitch), wave w owns heads 16w..16w+15:
//   S^T (32 rows x 16 heads) = K_rows . Q^T   v_mfma_f32_16x16x32_bf16, q in registers
//   O^T (512 dims x 16 heads) += V^T . P^T    V^T read with ds_read_b64_tr_b16,
//                                             P^T stays in the S^T registers
// Softmax is online in base 2 with a lazily moved reference maximum (the
// accumulators are rescaled only when a tile's maximum exceeds the reference
// by more than 8, so exponentials stay below 2^8).  Splits write unnormalised
// partial outputs plus (max, sum); a combine kernel merges them in split order.
#include "common.h"

namespace dsa {
namespace {

constexpr int kHq = 64;
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRows = 32;                        // gathered rows per tile
constexpr int kPitch = kDqk + 16;                // LDS row pitch in bf16 (1184 bytes)
constexpr int kChunks = kDqk / 8;                // 16-byte chunks per latent row
constexpr int kThreads = 256;
constexpr int kLoads = kRows * kChunks / kThreads;  // 9 chunks per thread per tile
constexpr int kTargetBlocks = 512;
constexpr float kRescaleSlack = 8.0f;            // log2 units

static_assert(kRows * kChunks % kThreads == 0, "tile load must split evenly");

template <bool DIRECT>
__global__ __launch_bounds__(kThreads) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int64_t kv_bstride,
    const int32_t* __restrict__ idx, int T, int L, int k, int rows_per_split, int nsplit, float scale_log2,
    float* __restrict__ part_o, float* __restrict__ part_ml, uint16_t* __restrict__ out, float* __restrict__ lse) {
    const int bt = blockIdx.x / nsplit;
    const int split = blockIdx.x % nsplit;
    const int b = bt / T;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int j0 = split * rows_per_split;
    const int j1 = min(k, j0 + rows_per_split);

    __shared__ __attribute__((aligned(16))) uint16_t tile[kRows * kPitch];
    __shared__ int row_ok[kRows];

    // B operand of S^T: q[head 16w+c][32*ks + 8*g .. +7].
    bf16x8_t qb[kDqk / 32];
    {
        const uint16_t* qh = q + ((int64_t)bt * kHq + 16 * wave + c) * kDqk + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kDqk / 32; ++ks) qb[ks] = *reinterpret_cast<const bf16x8_t*>(qh + 32 * ks);
    }
    f32x4_t o[kDv / 16];
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY;  // reference maximum (log2 units) of head 16w+c
    float lsum = 0.0f;        // this lane's share of the softmax denominator

    const int32_t* sel = idx + (int64_t)bt * k;
    const uint16_t* kvb = kv + (int64_t)b * kv_bstride;
    // transpose-read addressing: lane (g, 4j+q) points at row 4g+j (+16), dims 4q..4q+3 of a 16-dim block
    const int tr_row = 4 * g + ((lane & 15) >> 2);
    const int tr_col = 4 * (lane & 3);

    for (int j = j0; j < j1; j += kRows) {
        __syncthreads();  // the previous tile is no longer read
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int ci = threadIdx.x + kThreads * i;
            const int r = ci / kChunks, cc = ci % kChunks;
            const int jj = j + r;
            const int rid = jj < j1 ? sel[jj] : -1;
            const bool ok = rid >= 0 && rid < L;
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (ok) v = *reinterpret_cast<const u32x4_t*>(kvb + (int64_t)rid * kDqk + 8 * cc);
            *reinterpret_cast<u32x4_t*>(tile + r * kPitch + 8 * cc) = v;
            if (cc == 0) row_ok[r] = ok;
        }
        __syncthreads();

        // S^T tile: rows (rb*16 + 4g + r) x head (16w + c)
        f32x4_t s[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            s[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const uint16_t* arow = tile + (rb * 16 + c) * kPitch + 8 * g;
#pragma unroll
            for (int ks = 0; ks < kDqk / 32; ++ks)
                s[rb] = mfma16x16x32(*reinterpret_cast<const bf16x8_t*>(arow + 32 * ks), qb[ks], s[rb]);
        }
        float x[8];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int rb = e >> 2, r = e & 3;
            const float v = row_ok[rb * 16 + 4 * g + r] ? s[rb][r] * scale_log2 : -INFINITY;
            x[e] = v;
            mx = fmaxf(mx, v);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        if (__ballot(mx > m_ref + kRescaleSlack)) {
            const float m_new = fmaxf(m_ref, mx);
            const float f = (m_new == -INFINITY) ? 1.0f : exp2f(m_ref - m_new);
#pragma unroll
            for (int db = 0; db < kDv / 16; ++db) o[db] *= f;
            lsum *= f;
            m_ref = m_new;
        }
        const float mu = (m_ref == -INFINITY) ? 0.0f : m_ref;
        // P^T operand: k-slot 8g+e holds row (e<4 ? 4g+e : 16+4g+e-4), i.e. this lane's own S^T values.
        bf16x8_t pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint16_t h = f32_to_bf16_rne(exp2f(x[e] - mu));
            lsum += bf16_to_f32(h);
            pb[e] = __builtin_bit_cast(__bf16, h);
        }
        // O^T[dims 16db.. x heads] += V^T[16 dims x 32 rows] . P^T[32 rows x 16 heads]
#pragma unroll
        for (int db = 0; db < kDv / 16; ++db) {
            const bf16x4_t lo = lds_read_tr16(tile + tr_row * kPitch + 16 * db + tr_col);
            const bf16x4_t hi = lds_read_tr16(tile + (16 + tr_row) * kPitch + 16 * db + tr_col);
            const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            o[db] = mfma16x16x32(a, pb, o[db]);
        }
    }

    lsum += __shfl_xor(lsum, 16, kWave);
    lsum += __shfl_xor(lsum, 32, kWave);
    const int head = 16 * wave + c;
    if (DIRECT) {
        const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
        uint16_t* dst = out + ((int64_t)bt * kHq + head) * kDv + 4 * g;
#pragma unroll
        for (int db = 0; db < kDv / 16; ++db) {
            uint32_t lo = (uint32_t)f32_to_bf16_rne(o[db][0] * inv) | ((uint32_t)f32_to_bf16_rne(o[db][1] * inv) << 16);
            uint32_t hi = (uint32_t)f32_to_bf16_rne(o[db][2] * inv) | ((uint32_t)f32_to_bf16_rne(o[db][3] * inv) << 16);
            *reinterpret_cast<uint2*>(dst + 16 * db) = make_uint2(lo, hi);
        }
        if (lse && g == 0)
            lse[(int64_t)bt * kHq + head] = lsum > 0.0f ? (m_ref + log2f(lsum)) * 0.69314718055994531f : -INFINITY;
    } else {
        float* po = part_o + (((int64_t)bt * nsplit + split) * kHq + head) * kDv + 4 * g;
#pragma unroll
        for (int db = 0; db < kDv / 16; ++db) *reinterpret_cast<f32x4_t*>(po + 16 * db) = o[db];
        if (g == 0) {
            float* pm = part_ml + (((int64_t)bt * nsplit + split) * kHq + head) * 2;
            pm[0] = m_ref;
            pm[1] = lsum;
        }
    }
}

// Merge split partials: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, in split order.
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(const float* __restrict__ part_o,
                                                                const float* __restrict__ part_ml, int nsplit,
                                                                uint16_t* __restrict__ out, float* __restrict__ lse) {
    const int bt = blockIdx.x;
    const float* pm = part_ml + (int64_t)bt * nsplit * kHq * 2;
    for (int e = threadIdx.x; e < kHq * kDv / 4; e += kThreads) {
        const int head = e / (kDv / 4);
        const int d4 = e % (kDv / 4);
        float M = -INFINITY;
        for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pm[(s * kHq + head) * 2]);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        float den = 0.0f;
        if (M != -INFINITY) {
            for (int s = 0; s < nsplit; ++s) {
                const float ms = pm[(s * kHq + head) * 2];
                if (ms == -INFINITY) continue;
                const float a = exp2f(ms - M);
                den += a * pm[(s * kHq + head) * 2 + 1];
                const f32x4_t v = *reinterpret_cast<const f32x4_t*>(
                    part_o + (((int64_t)bt * nsplit + s) * kHq + head) * kDv + 4 * d4);
                acc += a * v;
            }
        }
        const float inv = den > 0.0f ? 1.0f / den : 0.0f;
        uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0] * inv) | ((uint32_t)f32_to_bf16_rne(acc[1] * inv) << 16);
        uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2] * inv) | ((uint32_t)f32_to_bf16_rne(acc[3] * inv) << 16);
        *reinterpret_cast<uint2*>(out + ((int64_t)bt * kHq + head) * kDv + 4 * d4) = make_uint2(lo, hi);
        if (lse && d4 == 0)
            lse[(int64_t)bt * kHq + head] = den > 0.0f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
    }
}

struct SplitPlan {
    int nsplit, rows_per_split;
};

SplitPlan plan(int rows, int k) {
    const int tiles = (k + kRows - 1) / kRows;
    int ns = (kTargetBlocks + rows - 1) / rows;
    if (ns > tiles) ns = tiles;
    if (ns < 1) ns = 1;
    const int tiles_per = (tiles + ns - 1) / ns;
    const int rps = tiles_per * kRows;
    return SplitPlan{(k + rps - 1) / rps, rps};
}

}  // namespace

int attn_num_splits(int rows, int k) { return plan(rows, k).nsplit; }

size_t attn_ws_bytes(int rows, int k) {
    const SplitPlan p = plan(rows, k);
    if (p.nsplit == 1) return 0;
    return align_up((size_t)rows * p.nsplit * kHq * (kDv + 2) * sizeof(float), 256);
}

hipError_t launch_attn(const uint16_t* q, const uint16_t* kv, int64_t kv_bstride, const int32_t* idx, int B, int T,
                       int L, int k, float sm_scale, uint16_t* out, float* lse, void* ws, hipStream_t stream) {
    const int rows = B * T;
    const SplitPlan p = plan(rows, k);
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    const unsigned grid = (unsigned)((int64_t)rows * p.nsplit);
    if (p.nsplit == 1) {
        hipLaunchKernelGGL(sparse_mla_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, q, kv, kv_bstride, idx, T,
                           L, k, p.rows_per_split, 1, scale_log2, nullptr, nullptr, out, lse);
        return hipGetLastError();
    }
    float* part_o = reinterpret_cast<float*>(ws);
    float* part_ml = part_o + (size_t)rows * p.nsplit * kHq * kDv;
    hipLaunchKernelGGL(sparse_mla_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, q, kv, kv_bstride, idx, T, L,
                       k, p.rows_per_split, p.nsplit, scale_log2, part_o, part_ml, nullptr, nullptr);
    hipLaunchKernelGGL(attn_combine_kernel, dim3(rows), dim3(kThreads), 0, stream, part_o, part_ml, p.nsplit, out,
                       lse);
    return hipGetLastError();
}

}  // namespace dsa
