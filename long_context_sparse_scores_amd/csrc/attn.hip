// Sparse absorbed-MLA attention over the selected latent rows (gfx950).
//
// [TEARDOWN, 刀一 DSA] (clawlihai.cn GLM-5.2 1M architecture teardown): full
// attention runs over only the 2048 selected tokens.  [TEARDOWN, 刀三 MLA]:
// the cache keeps one compressed latent vector per token, shared by all 64
// heads (kv_lora_rank 512; with the 64-dim rope part a row holds 576 bf16).
// In absorbed form each head's query already lives in that latent space, so
//   z_j = sm_scale * <q_h, c_j>   (576 dims),   o_h = softmax(z) . c[:, 0:512].
//
// Work unit: one query (b,t) and a split of its index list; one 256-thread
// workgroup per CU.  Selected rows are gathered 32 at a time (36 KiB tiles)
// straight from HBM into LDS with direct-to-LDS loads (no registers), four
// tile buffers deep so three tiles are in flight while one is computed.  The
// tile layout XOR-swizzles 16-byte chunks per row to spread operand reads
// over the LDS banks.  Wave w owns heads 16w..16w+15:
//   S^T (32 rows x 16 heads) = K_rows . Q^T   v_mfma_f32_16x16x32_bf16, q in registers
//   O^T (512 dims x 16 heads) += V^T . P^T    V^T read with ds_read_b64_tr_b16,
//                                             P^T stays in the S^T registers
// Softmax is online in base 2 with a lazily moved reference maximum: the
// accumulators are rescaled only when a tile's maximum exceeds the reference
// by more than 32 (so P < 2^32 and the fp32 sums stay far from overflow);
// after the first tile this practically never happens.  Splits write unnormalised
// fp32 partial outputs plus (max, sum); a combine kernel, one block per
// (query, head), merges them in split order.  A query whose list fits one
// split is normalised and written directly.
#include "common.h"

namespace dsa {
namespace {

constexpr int kHq = 64;
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRows = 32;                         // gathered rows per tile
constexpr int kChunks = kDqk / 8;                 // 16-byte chunks per latent row (72)
constexpr int kTileChunks = kRows * kChunks;      // 2304 chunks = 36 KiB per tile
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kLoads = kTileChunks / kThreads;    // 9 direct-to-LDS loads per thread per tile
constexpr int kStages = 4;                        // LDS tile buffers (3 tiles in flight + 1 computing)
constexpr int kMaxSplitRows = 2048;
constexpr int kTargetBlocks = 256;                // one resident block per CU
constexpr int kXcds = 8;                          // MI355X: 8 XCDs, block ids dealt round-robin
constexpr float kRescaleSlack = 32.0f;            // log2 units: P < 2^32, |O| < 2^46 in fp32

static_assert(kTileChunks % kThreads == 0, "tile load must split evenly");

// Tile layout in LDS: row r, 16-byte chunk cc lives at chunk slot r*72 + (cc ^ (r & 7)).
// The XOR spreads the 16 rows read by one MFMA operand over all LDS banks while
// keeping each wave's 64 direct-to-LDS writes (one contiguous KiB) in place.
__device__ __forceinline__ int slot(int r, int cc) { return r * kChunks + (cc ^ (r & 7)); }

// One 16-byte-per-lane direct-to-LDS load: lane l writes LDS bytes [lds + 16 l, lds + 16 l + 16).
// Issued from asm so that the compiler, which cannot tell which tile buffer the
// load fills, does not drain every in-flight load before each LDS read; the
// kernel orders these writes itself with wait_vmem() and lds_barrier().  The
// instruction has no register result and reads its address when issued.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_byte_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_byte_addr) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

__device__ __forceinline__ void gather_tile(const uint16_t* __restrict__ kvb, const int* __restrict__ rows_lds,
                                            int t, int nrows, int L, const uint16_t* tile, int wave, int lane) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(tile));
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int blk = kWaves * i + wave;              // this wave's KiB of the tile
        const int p = 64 * blk + lane;                  // chunk slot written by this lane
        const int r = p / kChunks;
        const int cc = (p % kChunks) ^ (r & 7);         // logical chunk stored in that slot
        const int j = t * kRows + r;
        int rid = j < nrows ? rows_lds[j] : 0;
        rid = (rid >= 0 && rid < L) ? rid : 0;          // masked rows read row 0 (finite) and get P = 0
        lds_dma16(kvb + (int64_t)rid * kDqk + 8 * cc, __builtin_amdgcn_readfirstlane(base + 1024u * blk));
    }
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations
// only.  (__syncthreads() also waits for every outstanding global load,
// which would drain the gather pipeline.)  The asm memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct SoftmaxState {
    f32x4_t o[kDv / 16];  // O^T accumulators: dims 16*db + 4g + r of head 16w + c
    float m_ref;          // reference maximum (log2 units) of head 16w + c
    float lsum;           // this lane's share of the softmax denominator
};

// Per-lane LDS read addresses of one tile (chunk units, relative to the tile),
// split into a lane base plus compile-time offsets.  The swizzle XORs only the
// low three bits of a chunk index, so for chunk = 8m + d it maps to
// 8m + (d ^ (r & 7)): one base per value of d, the 8m part is an immediate.
struct TileAddr {
    int qk[2];  // S^T A operand, row c (+16 per row block): chunks 8m + (4*(ks&1) + g) ^ (c&7)
    int tr[4];  // V^T transpose reads, row tr_row (+16): chunks 8n + (2d + (lane&3)/2) ^ (tr_row&7)
};

__device__ __forceinline__ TileAddr tile_addr(int lane) {
    const int c = lane & 15, g = lane >> 4;
    const int tr_row = 4 * g + ((lane & 15) >> 2);
    TileAddr a;
#pragma unroll
    for (int par = 0; par < 2; ++par) a.qk[par] = c * kChunks + ((4 * par + g) ^ (c & 7));
#pragma unroll
    for (int d = 0; d < 4; ++d) a.tr[d] = tr_row * kChunks + ((2 * d + ((lane & 3) >> 1)) ^ (tr_row & 7));
    return a;
}

// One tile of 32 gathered rows already resident in LDS at `tl`.
__device__ __forceinline__ void attend_tile(const uint16_t* tl, const TileAddr& ad, const int* __restrict__ rows_lds,
                                            int t, int nrows, int L, float scale_log2,
                                            const bf16x8_t (&qb)[kDqk / 32], int lane, SoftmaxState& st) {
    const int g = lane >> 4;
    // S^T tile: rows (rb*16 + 4g + r) x head (16w + c); A operand = row (rb*16 + c), dims 32ks + 8g.
    // Two independent accumulator chains (row blocks) share each q operand; the
    // operand reads run kAhead k-steps ahead of the MFMAs (order pinned below).
    constexpr int kSteps = kDqk / 32;
    constexpr int kAhead = 3;
    f32x4_t s[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    bf16x8_t a[kSteps][2];
    auto load_a = [&](int ks) {
        const uint16_t* p = tl + 8 * (ad.qk[ks & 1] + 8 * (ks >> 1));
        a[ks][0] = *reinterpret_cast<const bf16x8_t*>(p);
        a[ks][1] = *reinterpret_cast<const bf16x8_t*>(p + 8 * 16 * kChunks);
    };
#pragma unroll
    for (int ks = 0; ks < kAhead; ++ks) load_a(ks);
    __builtin_amdgcn_sched_group_barrier(0x0100, 2 * kAhead, 0);
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
        if (ks + kAhead < kSteps) {
            load_a(ks + kAhead);
            __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);
        }
        s[0] = mfma16x16x32(a[ks][0], qb[ks], s[0]);
        s[1] = mfma16x16x32(a[ks][1], qb[ks], s[1]);
        __builtin_amdgcn_sched_group_barrier(0x0008, 2, 0);
    }
    float x[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = t * kRows + (e >> 2) * 16 + 4 * g + (e & 3);
        const int rid = j < nrows ? rows_lds[j] : -1;
        const float v = (rid >= 0 && rid < L) ? s[e >> 2][e & 3] * scale_log2 : -INFINITY;
        x[e] = v;
        mx = fmaxf(mx, v);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    if (__ballot(mx > st.m_ref + kRescaleSlack)) {
        const float m_new = fmaxf(st.m_ref, mx);
        // While the reference is -inf nothing has been accumulated, so only a
        // finite old reference needs the accumulators rescaled.
        const bool scale = st.m_ref != -INFINITY && m_new != st.m_ref;
        if (__ballot(scale)) {
            const float f = scale ? exp2f(st.m_ref - m_new) : 1.0f;
#pragma unroll
            for (int db = 0; db < kDv / 16; ++db) {
                st.o[db] *= f;
                __builtin_amdgcn_sched_barrier(0);  // one 4-register block at a time
            }
            st.lsum *= f;
        }
        st.m_ref = m_new;
    }
    const float mu = (st.m_ref == -INFINITY) ? 0.0f : st.m_ref;
    // P^T operand: k-slot 8g+e holds row (e<4 ? 4g+e : 16+4g+e-4), i.e. this lane's own S^T values.
    bf16x8_t pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint16_t h = f32_to_bf16_rne(exp2f(x[e] - mu));
        st.lsum += bf16_to_f32(h);
        pb[e] = __builtin_bit_cast(__bf16, h);
    }
    // O^T[dims 16db.. x heads] += V^T[16 dims x 32 rows] . P^T[32 rows x 16 heads].
    // Transpose-read addressing: lane (g, 4j+q) points at row 4g+j (+16), dims 4q..4q+3 of the block,
    // i.e. chunk 2db + q/2, byte offset 8*(q&1).
    const int off = 4 * (lane & 1);
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) {
        const uint16_t* p = tl + 8 * (ad.tr[db & 3] + 8 * (db >> 2)) + off;
        const bf16x4_t lo = lds_read_tr16(p);
        const bf16x4_t hi = lds_read_tr16(p + 8 * 16 * kChunks);
        const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        st.o[db] = mfma16x16x32(a, pb, st.o[db]);
    }
}

// One workgroup (one wave per SIMD) fills a CU's LDS, so the scheduler may use
// every register to run operand loads ahead.
template <bool DIRECT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int64_t kv_bstride,
    const int32_t* __restrict__ idx, int rows, int T, int L, int k, int rows_per_split, int nsplit, float scale_log2,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse, uint16_t* __restrict__ out, float* __restrict__ lse) {
    // Blocks are numbered so that every split of query bt lands on XCD bt % 8
    // (consecutive block ids go to consecutive XCDs): the splits' partials and
    // the combine that reads them share one L2.
    const int grp = blockIdx.x / (kXcds * nsplit);
    const int rem = blockIdx.x % (kXcds * nsplit);
    const int split = rem / kXcds;
    const int bt = grp * kXcds + rem % kXcds;
    if (bt >= rows) return;
    const int b = bt / T;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int j0 = split * rows_per_split;
    const int nrows = min(k, j0 + rows_per_split) - j0;
    const int ntiles = (nrows + kRows - 1) / kRows;

    __shared__ __attribute__((aligned(16))) uint16_t tiles[kStages * kTileChunks * 8];
    __shared__ int rows_lds[kMaxSplitRows];

    const int32_t* sel = idx + (int64_t)bt * k + j0;
    for (int j = threadIdx.x; j < nrows; j += kThreads) rows_lds[j] = sel[j];
    __syncthreads();  // rows_lds ready

    // Start the first gathers, then fetch q while they are in flight.
    const uint16_t* kvb = kv + (int64_t)b * kv_bstride;
    const TileAddr ad = tile_addr(lane);
    for (int t = 0; t < kStages - 1 && t < ntiles; ++t)
        gather_tile(kvb, rows_lds, t, nrows, L, tiles + t * (kTileChunks * 8), wave, lane);
    // B operand of S^T: q[head 16w+c][32*ks + 8*g .. +7].
    bf16x8_t qb[kDqk / 32];
    {
        const uint16_t* qh = q + ((int64_t)bt * kHq + 16 * wave + c) * kDqk + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kDqk / 32; ++ks) qb[ks] = *reinterpret_cast<const bf16x8_t*>(qh + 32 * ks);
    }
    SoftmaxState st;
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) st.o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st.m_ref = -INFINITY;
    st.lsum = 0.0f;
    // Consume q here so the compiler's own wait for these loads happens before the
    // tile loop, not inside it where it would also drain later gathers.
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) asm volatile("" ::"v"(qb[ks]));

    for (int t = 0; t < ntiles; ++t) {
        // refill the buffer released at the end of the previous step with tile t+3
        if (t + kStages - 1 < ntiles)
            gather_tile(kvb, rows_lds, t + kStages - 1, nrows, L, tiles + ((t + kStages - 1) % kStages) * (kTileChunks * 8),
                        wave, lane);
        // this thread's loads of tile t are done once at most the loads of the later tiles are outstanding
        const int later = min(ntiles - 1 - t, kStages - 1);
        if (later >= 3) wait_vmem<3 * kLoads>();
        else if (later == 2) wait_vmem<2 * kLoads>();
        else if (later == 1) wait_vmem<kLoads>();
        else wait_vmem<0>();
        lds_barrier();  // every thread's part of tile t is in LDS
        attend_tile(tiles + (t % kStages) * (kTileChunks * 8), ad, rows_lds, t, nrows, L, scale_log2, qb, lane, st);
        lds_barrier();  // nobody reads buffer t % kStages any more
    }

    float lsum = st.lsum;
    const float m_ref = st.m_ref;
    lsum += __shfl_xor(lsum, 16, kWave);
    lsum += __shfl_xor(lsum, 32, kWave);
    const int head = 16 * wave + c;
    const f32x4_t* o = st.o;
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
        // Normalised partial output (bf16) and its log2-sum-exp; an empty split has lse -inf.
        const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
        uint16_t* po = part_o + (((int64_t)bt * nsplit + split) * kHq + head) * kDv + 4 * g;
#pragma unroll
        for (int db = 0; db < kDv / 16; ++db) {
            uint32_t lo = (uint32_t)f32_to_bf16_rne(o[db][0] * inv) | ((uint32_t)f32_to_bf16_rne(o[db][1] * inv) << 16);
            uint32_t hi = (uint32_t)f32_to_bf16_rne(o[db][2] * inv) | ((uint32_t)f32_to_bf16_rne(o[db][3] * inv) << 16);
            *reinterpret_cast<uint2*>(po + 16 * db) = make_uint2(lo, hi);
        }
        if (g == 0) part_lse[((int64_t)bt * nsplit + split) * kHq + head] = lsum > 0.0f ? m_ref + log2f(lsum) : -INFINITY;
    }
}

// Merge the split partials of one (query, head): with lse_s the log2-sum-exp of
// split s, out = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M), in split order.
// One 128-thread block per (query, head), 4 dims per thread; blocks numbered
// like the split kernel so each reads partials from its own XCD's L2.
__global__ __launch_bounds__(128) void attn_combine_kernel(const uint16_t* __restrict__ part_o,
                                                           const float* __restrict__ part_lse, int rows, int nsplit,
                                                           uint16_t* __restrict__ out, float* __restrict__ lse) {
    const int grp = blockIdx.x / (kXcds * kHq);
    const int rem = blockIdx.x % (kXcds * kHq);
    const int head = rem / kXcds;
    const int bt = grp * kXcds + rem % kXcds;
    if (bt >= rows) return;
    const float* pl = part_lse + (int64_t)bt * nsplit * kHq + head;  // split s at pl[s * kHq]
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pl[(int64_t)s * kHq]);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float den = 0.0f;
    if (M != -INFINITY) {
        const uint16_t* po = part_o + ((int64_t)bt * nsplit * kHq + head) * kDv + 4 * threadIdx.x;
        for (int s = 0; s < nsplit; ++s) {
            const float ls = pl[(int64_t)s * kHq];
            if (ls == -INFINITY) continue;
            const float a = exp2f(ls - M);
            den += a;
            const uint2 v = *reinterpret_cast<const uint2*>(po + (int64_t)s * kHq * kDv);
            acc[0] += a * __uint_as_float(v.x << 16);
            acc[1] += a * __uint_as_float(v.x & 0xFFFF0000u);
            acc[2] += a * __uint_as_float(v.y << 16);
            acc[3] += a * __uint_as_float(v.y & 0xFFFF0000u);
        }
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0] * inv) | ((uint32_t)f32_to_bf16_rne(acc[1] * inv) << 16);
    uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2] * inv) | ((uint32_t)f32_to_bf16_rne(acc[3] * inv) << 16);
    *reinterpret_cast<uint2*>(out + ((int64_t)bt * kHq + head) * kDv + 4 * threadIdx.x) = make_uint2(lo, hi);
    if (lse && threadIdx.x == 0)
        lse[(int64_t)bt * kHq + head] = den > 0.0f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
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

static unsigned xcd_grid(int rows, int per_row) {
    return (unsigned)((int64_t)((rows + kXcds - 1) / kXcds) * kXcds * per_row);
}

size_t attn_ws_bytes(int rows, int k) {
    const SplitPlan p = plan(rows, k);
    if (p.nsplit == 1) return 0;
    const size_t n = (size_t)rows * p.nsplit * kHq;
    return align_up(n * kDv * sizeof(uint16_t), 256) + align_up(n * sizeof(float), 256);
}

hipError_t launch_attn(const uint16_t* q, const uint16_t* kv, int64_t kv_bstride, const int32_t* idx, int B, int T,
                       int L, int k, float sm_scale, uint16_t* out, float* lse, void* ws, hipStream_t stream) {
    const int rows = B * T;
    const SplitPlan p = plan(rows, k);
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    if (p.nsplit == 1) {
        hipLaunchKernelGGL(sparse_mla_kernel<true>, dim3(xcd_grid(rows, 1)), dim3(kThreads), 0, stream, q, kv,
                           kv_bstride, idx, rows, T, L, k, p.rows_per_split, 1, scale_log2, nullptr, nullptr, out, lse);
        return hipGetLastError();
    }
    const size_t n = (size_t)rows * p.nsplit * kHq;
    uint16_t* part_o = reinterpret_cast<uint16_t*>(ws);
    float* part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align_up(n * kDv * sizeof(uint16_t), 256));
    hipLaunchKernelGGL(sparse_mla_kernel<false>, dim3(xcd_grid(rows, p.nsplit)), dim3(kThreads), 0, stream, q, kv,
                       kv_bstride, idx, rows, T, L, k, p.rows_per_split, p.nsplit, scale_log2, part_o, part_lse,
                       nullptr, nullptr);
    hipLaunchKernelGGL(attn_combine_kernel, dim3(xcd_grid(rows, kHq)), dim3(128), 0, stream, part_o, part_lse, rows,
                       p.nsplit, out, lse);
    return hipGetLastError();
}

}  // namespace dsa
